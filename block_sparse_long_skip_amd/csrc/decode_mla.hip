// bf16 skip-softmax decode against an MLA latent cache on gfx950:
// d_qk = 576 (512 latent + 64 rope features), values = the first 512 features
// of each key, 64-key tiles, one query token per (batch, head).
//
// Method: BLASST post (seeallochnaya, "BLASST: Dynamic BLocked Attention
// Sparsity via Softmax Thresholding"): key tiles in increasing order, online
// max, a tile dropped whole when its max is far below the running max
// (paragraph beginning "BLASST предлагает"), tile 0 always processed (first
// figure); the post notes the method composes with DeepSeek MLA (paragraph on
// MLA). The running max is global along the cache.
//
// With a latent cache the values are a slice of the keys, so a dropped tile
// saves the exp, the row sums and the P.V MFMAs; the latent bytes are read for
// the scores regardless.
//
// Split along the cache. One workgroup per (batch, KV head, group of 64 query
// heads, split of T consecutive key tiles). The decision for tile j needs the
// running max before j, which for lambda <= 1 is the plain prefix max of the
// tile maxima (a dropped tile never raises it). A split cannot know the maxima
// of the splits before it, so the work runs in two passes plus a merge:
//   pass 0 (speculative): every split runs the ordered tile loop; a split after
//     the first scores tile 0 first (maxima only: it holds the attention sinks),
//     so its running max starts from a lower bound of the exact one that
//     usually equals it. It records every tile max and its own maximum in the
//     workspace and leaves its partial (reference max, row sums, O) there;
//   pass 1 (exact): every split takes the true running max entering it from the
//     maxima of the earlier splits, derives the exact decision of every tile
//     and head from the recorded tile maxima, and writes the mask, the kept
//     counts and the per-tile "some head keeps" flags. The exact rule never
//     keeps a tile the speculative one dropped (its running max is at least as
//     large), so the pass-0 partial is exact unless some tile was kept only
//     speculatively; only those tiles are read again, and their contribution
//     at the partial's reference max is subtracted;
//   merge: a log-sum-exp merge of the partials of each (batch, head).
//
// Workgroup layout (4 waves, 64 heads). Per key tile:
//   * the 64 x 576 tile (72 KB) travels global -> LDS through buffer loads
//     that write LDS directly (no register staging), double-buffered; the next
//     tile's 18 copies per wave go out one per two score MFMA steps of the
//     current tile (issued all at once they stall the wave until the address
//     unit has taken most of them in). The tile is stored in
//     1 KB blocks with the 16-byte chunk index XOR-swizzled by the row (see
//     mla_off) so that both the score operand reads and the transposing value
//     reads hit distinct banks;
//   * wave w = (key half kh = w & 1, head half hh = w >> 1) computes
//     S^T[32 keys][32 heads] = K q^T on v_mfma_f32_32x32x16_bf16, with its
//     heads' queries held in registers;
//   * the per-head tile maxima of the two key halves meet in LDS; every wave
//     then takes the same decision per head, and P^T (bf16) goes to LDS;
//   * if any head keeps the tile, wave w computes output features
//     128w..128w+127 of all 64 heads: O^T += V^T P^T, with V^T read from the
//     key tile by ds_read_b64_tr_b16. The accumulators are rescaled lazily,
//     only when a running max has grown by more than 2^8.
#include <type_traits>
#include <utility>

#include "common.hpp"

namespace blasst {

namespace {
constexpr int BC = 64;
constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int HG = 64;                    // query heads per workgroup
constexpr int KS2 = DQK / 16;             // 36 MFMA steps (32x32x16) over the key features
constexpr int ROWB = DQK * 2;             // 1152 bytes per key row
constexpr int TILEB = BC * ROWB;          // 73728 bytes per tile
constexpr int NCH = TILEB / 16;           // 4608 16-byte chunks per tile
constexpr int DMA_PER_WAVE = NCH / 64 / NW;  // 18 copy instructions per wave per tile
constexpr int CPR = DQK / 64;             // 9 blocks (copy instructions) per block row
static_assert(DMA_PER_WAVE == 2 * CPR && KS2 == 2 * DMA_PER_WAVE,
              "a wave's copies are two block rows, one per two score steps");
constexpr int PP = BC + 8;                // P^T row pitch (bf16): 144 B
constexpr int LIST_MAX = 256;             // most tiles per split
constexpr int TARGET_BLOCKS = 256;        // one workgroup per CU
constexpr float kLazyRescaleLog2 = 8.f;   // rescale once the max grows by 2^8
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit data format, raw access
static_assert(NCH % (64 * NW) == 0, "tile copies split evenly over the waves");
static_assert(DV == 128 * NW, "each wave produces 128 output features");

// LDS layout of a 64 x 576 key tile: 1 KB blocks of 8 rows x 8 chunks of 16
// bytes, block (row / 8, chunk / 8) at 1024 * ((row / 8) * 9 + chunk / 8),
// 128 bytes per row inside a block. One global_load_lds_dwordx4 fills one
// block, so each lane's source offset inside a block is the same for every
// copy. The chunk index inside a block is XOR-ed with mla_f(row): 8 distinct
// values over the even rows (and over the odd rows) of any 16 consecutive
// rows, and a different bit 1 for rows r and r + 2, so the score operand reads
// (16 rows, one chunk) and the transposing value reads (4 rows, 2 chunks) hit
// distinct banks.
__device__ __forceinline__ int mla_f(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int mla_off(int r, int c) {
  return (((r >> 3) * (DQK / 64) + (c >> 3)) << 10) + ((r & 7) << 7) + (((c & 7) ^ mla_f(r)) << 4);
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations
// but not for its copies into the other tile buffer, which stay in flight
// across it (a __syncthreads would wait for them). The memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One block row of a tile into LDS: block cb of the row comes from 128 cb
// bytes further along the key rows. That offset goes in the scalar offset of
// the buffer load: the immediate offset would move the LDS destination too.
template <int CB>
__device__ __forceinline__ void copy_block(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)(lds + 1024 * CB), 16, voff, 128 * CB, 0, 0);
}
template <int... CB>
__device__ __forceinline__ void copy_block_row(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voff,
                                               std::integer_sequence<int, CB...>) {
  (copy_block<CB>(rs, lds, voff), ...);
}

// c + lo + hi of a pair of bf16 values, in one dot-product instruction
__device__ __forceinline__ float add_bf16x2(uint32_t w, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), c, false);
}

// gap of a tile max against a running max, with the conventions of the drop
// rule: -inf for a tile with no visible key, +inf before the first tile
__device__ __forceinline__ float gap_of(float tm, float m) {
  if (tm == kNegInf) return kNegInf;
  if (m == kNegInf) return __builtin_inff();
  return tm - m;
}
}  // namespace

// Workspace of one latent-cache decode call (carved from the caller's buffer).
struct MlaWork {
  float* tmax;     // [B*Hkv][nkt][G]       tile maxima (raw q.k units), heads fastest
  float* smax;     // [B*Hq][nsplit]        maximum of each split's tile maxima
  float* part_o;   // [B*Hq][nsplit][512]   unnormalised partial outputs
  float* part_ml;  // [B*Hq][nsplit][4]     partial (reference max, row sum, row sum of the
                   //                       bf16-rounded p, unused)
  int* part_kept;  // [B*Hq][nsplit]        kept tiles per split (exact decisions)
  uint8_t* anyk;   // [B*Hkv][ngroups][nkt] 1 if some head of the group keeps the tile
  int ngroups, nsplit, T;
};

template <int MODE>
__global__ void __launch_bounds__(NT, 1) decode_mla_split_kernel(DecodeArgs a, MlaWork ws) {
  // the two tile buffers are separate objects so that the compiler can tell
  // the copy into one from the reads of the other (no wait for the copy)
  __shared__ __attribute__((aligned(16))) char Kt0[TILEB];
  __shared__ __attribute__((aligned(16))) char Kt1[TILEB];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[HG * PP];
  __shared__ float tmw[2][2][HG];  // [buffer][key half][head]
  __shared__ float alph[HG];
  __shared__ float lred[2][2][HG];  // [sum kind][key half][head]
  __shared__ int kflag[NW];
  __shared__ uint16_t list[LIST_MAX];  // pass 1: tiles to correct, relative to the split start
  __shared__ uint64_t lmask[LIST_MAX]; // pass 1: heads whose contribution of that tile is removed
  __shared__ float mstart[HG];         // exact running max entering the split
  __shared__ int cntw[NW][HG];
  __shared__ int misw[NW];
  __shared__ int nlist;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int kh = w & 1, hh = w >> 1;

  // logical block = ((split * B*Hkv) + seq) * ngroups + group: the head groups
  // of one (sequence, split) are consecutive, and when the grid is a multiple
  // of 8 consecutive logical blocks share an XCD (blocks are dealt to the XCDs
  // round-robin), so they share the split's latent tiles through its L2
  const int total = (int)gridDim.x;
  int lb = (int)blockIdx.x;
  if ((total & 7) == 0) lb = (lb & 7) * (total >> 3) + (lb >> 3);
  const int gi = lb % ws.ngroups;
  const int rest = lb / ws.ngroups;
  const int nseq = a.B * a.Hkv;
  const int seq = rest % nseq, s = rest / nseq;
  const int b = seq / a.Hkv, kvh = seq % a.Hkv;
  const int G = a.G;
  const int h0 = gi * HG;
  const int nkt = a.nkt;
  const int j0 = s * ws.T, j1 = min(j0 + ws.T, nkt);
  const float c2 = a.scale_log2;
  const float thr = a.thr_raw;
  const int64_t row0 = (int64_t)b * a.Hq + kvh * G + h0;  // (b, head h0 of the group)
  const int nsplit = ws.nsplit;
  const int Nk = a.Nk;
  float* const tmaxp = ws.tmax + (int64_t)seq * nkt * G + h0;  // + j * G + head

  // the score head of this lane: S^T[32 keys][32 heads] per wave, head 32hh + l32
  const int hl = 32 * hh + l32;
  const bool hv = h0 + hl < G;

  // ---- exact decisions (pass 1): true running max entering the split, mask,
  // counts, and whether pass 0 took the same decisions
  float m_init = kNegInf;
  // pass 0 of a split after the first scores tile 0 (which holds the attention
  // sinks) before its own tiles when tiles can be dropped at all: its maxima
  // start the split's running max, a lower bound of the exact one that usually
  // equals it, so the speculative decisions usually are the exact ones
  const int pre = (MODE == 0 && s > 0 && thr != kNegInf) ? 1 : 0;
  int nl = j1 - j0 + pre;
  if constexpr (MODE == 1) {
    const int tn = j1 - j0;
    float* tms = reinterpret_cast<float*>(Kt1);   // [tn][HG] tile maxima of the split
    uint8_t* mk = reinterpret_cast<uint8_t*>(Kt0);  // [HG][LIST_MAX] exact decisions
    uint8_t* tflag = mk + HG * LIST_MAX;             // [tn] some head keeps the tile
    uint64_t* cm = reinterpret_cast<uint64_t*>(Kt1 + 4 * HG * LIST_MAX);  // [tn] heads to correct
    const int hp = lane;  // one head per lane
    const bool hvp = h0 + hp < G;
    // the split's tile maxima into LDS, 16 independent loads per wave at a time
    for (int c = 0; c < tn; c += 16 * NW) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int jj = c + NW * u + w;
        v[u] = (hvp && jj < tn) ? tmaxp[(int64_t)(j0 + jj) * G + hp] : kNegInf;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int jj = c + NW * u + w;
        if (jj < tn) tms[jj * HG + hp] = v[u];
      }
    }
    // maximum of the tile maxima before the split: the split maxima of pass 0
    if (w == 0) {
      float M = kNegInf;
      if (hvp) {
        const float* sm = ws.smax + (row0 + hp) * nsplit;
#pragma unroll 8
        for (int x = 0; x < s; ++x) M = fmaxf(M, sm[x]);
      }
      mstart[hp] = M;
    }
    __syncthreads();
    // wave w takes a quarter of the split; the running maxima entering it
    // follow from the tiles before it (a dropped tile's max is below the
    // running max, so the plain max is the running max over kept tiles)
    const int q0 = (w * tn) / NW, q1 = ((w + 1) * tn) / NW;
    // as pass 0 had it: from tile 0 (splits after the first) and the split's tiles
    float ml = (s > 0 && hvp) ? tmaxp[hp] : kNegInf;
    for (int jj = 0; jj < q0; ++jj) ml = fmaxf(ml, tms[jj * HG + hp]);
    float mt = fmaxf(mstart[hp], ml);  // exact: from tile 0
    int cnt = 0;
    bool mis = false;
    uint8_t* anyrow = ws.anyk + ((int64_t)seq * ws.ngroups + gi) * nkt + j0;
    for (int jj = q0; jj < q1; ++jj) {
      const float tm = tms[jj * HG + hp];
      const int j = j0 + jj;
      const bool kt = hvp && (j == 0 || !(gap_of(tm, mt) < thr));
      const bool kl = hvp && (j == 0 || !(gap_of(tm, ml) < thr));
      mt = fmaxf(mt, tm);
      ml = fmaxf(ml, tm);
      cnt += kt ? 1 : 0;
      mk[hp * LIST_MAX + jj] = kt ? 1 : 0;
      // the exact rule never keeps a tile the speculative one dropped (its
      // running max is at least as large); a tile kept only speculatively has
      // its contribution removed below
      const uint64_t corr = __ballot(kl && !kt);
      mis |= corr != 0;
      const bool any = __ballot(kt) != 0;
      if (lane == 0) {
        tflag[jj] = any ? 1 : 0;
        anyrow[jj] = any ? 1 : 0;
        cm[jj] = corr;
      }
    }
    cntw[w][hp] = cnt;
    const bool wmis = __ballot(mis) != 0;
    if (lane == 0) misw[w] = wmis ? 1 : 0;
    __syncthreads();
    // mask rows of the group's heads, consecutive threads on consecutive tiles
    if (a.mask) {
      for (int idx = t; idx < HG * tn; idx += NT) {
        const int hx = idx / tn, jj = idx - hx * tn;
        if (h0 + hx < G) a.mask[(row0 + hx) * nkt + j0 + jj] = mk[hx * LIST_MAX + jj];
      }
    }
    if (w == 0 && hvp)
      ws.part_kept[(row0 + hp) * nsplit + s] = cntw[0][hp] + cntw[1][hp] + cntw[2][hp] + cntw[3][hp];
    const bool redo = (misw[0] | misw[1] | misw[2] | misw[3]) != 0;
    if (!redo) return;  // the pass-0 partial is already exact
    // list of the tiles to correct, in order, with their head masks
    if (w == 0) {
      int base = 0;
      for (int c0 = 0; c0 < tn; c0 += 64) {
        const uint64_t mk64 = c0 + lane < tn ? cm[c0 + lane] : 0ull;
        const bool f = mk64 != 0ull;
        const uint64_t bits = __ballot(f);
        if (f) {
          const int at = base + __popcll(bits & ((1ull << lane) - 1ull));
          list[at] = (uint16_t)(c0 + lane);
          lmask[at] = mk64;
        }
        base += __popcll(bits);
      }
      if (lane == 0) nlist = base;
    }
    __syncthreads();  // list ready; mk, tms and cm (in the tile buffers) no longer read
    nl = nlist;
  }
  auto tile_of = [&](int idx) __attribute__((always_inline)) -> int {
    if constexpr (MODE == 1) return j0 + __builtin_amdgcn_readfirstlane((int)list[idx]);
    else return idx < pre ? 0 : j0 + idx - pre;
  };

  // ---- queries: q^T as the B operand of v_mfma_f32_32x32x16_bf16, lane
  // supplies q[head hl][16kk + 8h .. +7]; kept in AGPRs (MFMA operands may be AGPRs)
  bf16x8_t qb[KS2];
  {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 +
                         (int64_t)(kvh * G + h0 + (hv ? hl : 0)) * a.qs1;
    u32x4_t v[KS2];
#pragma unroll
    for (int kk = 0; kk < KS2; ++kk) v[kk] = load16(qp + 16 * kk + 8 * h);  // all in flight
#pragma unroll
    for (int kk = 0; kk < KS2; ++kk) {
      u32x4_t x = hv ? v[kk] : (u32x4_t){0u, 0u, 0u, 0u};
      asm volatile("" : "+a"(x));
      qb[kk] = as_bf16x8(x);
    }
  }

  // ---- per-lane LDS offsets
  // score operand (A = K rows): key row 32kh + l32, chunk 2kk + h; kk & 3
  // selects one of four patterns and kk >> 2 the next block (1024 bytes)
  const int kr = 32 * kh + l32;
  int ko[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) ko[x] = mla_off(kr, 2 * x + h);
  // value operand (A = V^T, transposing read), 16-key step ks: lane (group
  // gq = lane/16, j = lane%16) reads key 16ks + 8(gq>>1) + 4hf + j/4 at
  // features 128w + 32db + 16(gq&1) + 4(j&3); db & 1 selects one of two
  // patterns, db >> 1 the next block, ks two block rows (18 KB)
  const int gq = lane >> 4, jq = lane & 15;
  int vo[2][2];
#pragma unroll
  for (int d1 = 0; d1 < 2; ++d1)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 8 * (gq >> 1) + 4 * hf + (jq >> 2);
      const int dv0 = 128 * w + 32 * d1 + 16 * (gq & 1) + 4 * (jq & 3);
      vo[d1][hf] = mla_off(r, dv0 >> 3) + ((dv0 & 7) << 1);
    }

  // ---- tile copies: wave w fills blocks 18w..18w+17 of a tile (block rows
  // 2w and 2w + 1); in block (rb, cb) lane l lands at row 8rb + l/8, physical
  // chunk l%8, so it fetches logical chunk 8cb + ((l%8) ^ mla_f(row)). That
  // offset depends on the lane and on rb & 1 only; the block's own offset is
  // uniform.
  const char* kp = (const char*)((const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1);
  const int64_t rowstride = a.ks2 * 2;  // bytes
  const uint32_t rs32 = (uint32_t)rowstride;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t loff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int rr = lane >> 3;
    loff[par] = (uint32_t)rr * rs32 + ((((lane & 7) ^ mla_f(8 * par + rr))) << 4);
  }
  // Copies go through a buffer resource per (tile, block row): its range ends
  // at the last key of the cache, and the hardware returns zeros for rows
  // past it (their scores are masked below and their values meet p = 0). An
  // empty range (on = false) makes the copies write zeros and read nothing.
  auto copy_rsrc = [&](int j, int r2, bool on) __attribute__((always_inline)) {
    // all uniform; readfirstlane tells the compiler so (no waterfall loop)
    const int row0t = __builtin_amdgcn_readfirstlane(j * BC + 16 * wu + 8 * r2);  // first key
    const int nrec = on ? __builtin_amdgcn_readfirstlane(min(max(Nk - row0t, 0), 8) * (int)rs32) : 0;
    const uint64_t base = (uint64_t)(kp + (int64_t)row0t * rowstride);
    const uint64_t ubase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    return __builtin_amdgcn_make_buffer_rsrc((void*)ubase, (short)0, nrec, kBufferFlags);
  };
  // the whole tile at once (the first tile of the loop)
  auto tile_to_lds = [&](char* tile, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
      copy_block_row(copy_rsrc(j, r2, true), tile + 1024 * (DMA_PER_WAVE * wu + CPR * r2), loff[r2],
                     std::make_integer_sequence<int, CPR>{});
  };

  f32x16_t o[4][2];  // O^T[dv = 128w + 32db + 8(i/4) + 4h + i%4][head 32hb + l32]
  float m = m_init;      // exact running max of head hl (raw units): the decisions
  float m_acc = m_init;  // reference max of the accumulators (lags m by < 2^8 in exp2 units)
  if constexpr (MODE == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][hb][i] = 0.f;
  } else {
    // the correction starts from the pass-0 partial and keeps its reference max
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bool v = h0 + 32 * hb + l32 < G;
      const float* po = ws.part_o + ((row0 + (v ? 32 * hb + l32 : 0)) * nsplit + s) * DV + 128 * w + 4 * h;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4_t x = *(const f32x4_t*)(po + 32 * db + 8 * q4);
          if (!v) x = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][hb][4 * q4 + e] = x[e];
        }
    }
    m_acc = hv ? ws.part_ml[((row0 + hl) * nsplit + s) * 4] : 0.f;
  }
  float lp = 0.f;        // partial row sum over this lane's keys (fp32 p): the lse
  float lq = 0.f;        // the same over the bf16-rounded p that P.V uses: the output
                         // is normalised by it, so rounding a dominant p cancels

  // one key tile; the LDS buffer parity is a compile-time constant so that the
  // compiler can tell the copy into one buffer from the reads of the other
  int idx = 0;
  auto step = [&](auto PAR) __attribute__((always_inline)) {
    constexpr int P = decltype(PAR)::value;
    const int j = tile_of(idx);
    char* kt = P ? Kt1 : Kt0;
    wait_vmem();
    __syncthreads();  // (C) tile idx is in LDS; every wave is done with tile idx-1
    // the next tile's copies into the other buffer (every wave is done with
    // it); after the last tile they write zeros there and read nothing
    const bool nx = idx + 1 < nl;
    const int jn = nx ? tile_of(idx + 1) : j;
    const __amdgpu_buffer_rsrc_t nrs0 = copy_rsrc(jn, 0, nx), nrs1 = copy_rsrc(jn, 1, nx);
    char* const nb = (P ? Kt0 : Kt1) + 1024 * DMA_PER_WAVE * wu;

    // scores S^T[key 32kh + 8(i/4) + 4h + i%4][head hl]: 36 steps on two
    // accumulator chains, each step's K operand read four steps ahead
    f32x16_t s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
    u32x4_t kbuf[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) kbuf[x] = *(const u32x4_t*)(kt + ko[x]);
#pragma unroll
    for (int kk = 0; kk < KS2; ++kk) {
      const u32x4_t cur = kbuf[kk & 3];
      if (kk + 4 < KS2) kbuf[kk & 3] = *(const u32x4_t*)(kt + ko[kk & 3] + 1024 * ((kk + 4) >> 2));
      if ((kk & 1) == 0) {
        // the next tile's copies, one block per two score steps: block c of
        // the wave's 18 is block c % 9 of block row c / 9
        const int c = kk >> 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            c < CPR ? nrs0 : nrs1, (__attribute__((address_space(3))) void*)(nb + 1024 * c), 16,
            loff[c < CPR ? 0 : 1], 128 * (c % CPR), 0, 0);
      }
      if (kk & 1) s1 = mfma32x32x16(as_bf16x8(cur), qb[kk], s1);
      else s0 = mfma32x32x16(as_bf16x8(cur), qb[kk], s0);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x16_t sc = s0 + s1;
    // V^T operand reads of one 16-key step of the P.V product
    auto rdv = [&](int ks, u32x4_t (&va)[4]) __attribute__((always_inline)) {
      const char* vk = kt + 16 * ks * ROWB;  // two block rows
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2_t y0 = ds_read_tr(vk + 1024 * (db >> 1) + vo[db & 1][0]);
        const u32x2_t y1 = ds_read_tr(vk + 1024 * (db >> 1) + vo[db & 1][1]);
        va[db] = (u32x4_t){y0[0], y0[1], y1[0], y1[1]};
      }
    };
    u32x4_t va0[4];  // the first step's, read while the softmax runs
    const int c0 = j * BC;
    if (c0 + BC > Nk) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (c0 + 32 * kh + 8 * (i >> 2) + 4 * h + (i & 3) >= Nk) sc[i] = kNegInf;
    }
    bool keep = false;
    float alpha = 1.f;
    uint32_t pw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if constexpr (MODE == 0) {
      float tm = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tm = fmaxf(tm, sc[i]);
      tm = max_with_lane_xor32(tm);
      if (h == 0) tmw[P][kh][hl] = tm;
      lds_barrier();  // (A) tile maxima of both key halves visible

      const float TM = fmaxf(tmw[P][0][hl], tmw[P][1][hl]);
      rdv(0, va0);
      const bool sink_only = idx < pre;  // tile 0 scored by a later split: max only
      if (sink_only && hv) m = fmaxf(m, TM);
      if (!sink_only && kh == 0 && h == 0 && hv) tmaxp[(int64_t)j * G + hl] = TM;
      keep = !sink_only && hv && (j == 0 || !(gap_of(TM, m) < thr));
      if (keep) {
        // lazy rescale: the accumulators keep their reference max until the
        // running max exceeds it by 2^8 in exp2 units (p then stays <= 256,
        // exact in fp32 and in range for bf16); decisions use the exact max
        m = fmaxf(m, TM);
        if (m_acc == kNegInf) {
          m_acc = m;  // nothing accumulated yet
        } else if ((m - m_acc) * c2 > kLazyRescaleLog2) {
          alpha = fast_exp2((m_acc - m) * c2);
          lp *= alpha;
          lq *= alpha;
          m_acc = m;
        }
        const float mc = m_acc * c2;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float p0 = fast_exp2(fmaf(sc[2 * x], c2, -mc));
          const float p1 = fast_exp2(fmaf(sc[2 * x + 1], c2, -mc));
          lp += p0 + p1;
          pw[x] = pack_bf16x2(p0, p1);
          lq = add_bf16x2(pw[x], lq);
        }
      }
    } else {
      // correction: this tile was kept by pass 0 for the heads in the mask
      // and is dropped by the exact rule; its contribution at the partial's
      // reference max is subtracted (same p, negated)
      rdv(0, va0);
      keep = hv && ((lmask[idx] >> hl) & 1ull) != 0ull;
      if (keep) {
        const float mc = m_acc * c2;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float p0 = -fast_exp2(fmaf(sc[2 * x], c2, -mc));
          const float p1 = -fast_exp2(fmaf(sc[2 * x + 1], c2, -mc));
          lp += p0 + p1;
          pw[x] = pack_bf16x2(p0, p1);
          lq = add_bf16x2(pw[x], lq);
        }
      }
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *(u32x2_t*)&Ps[hl * PP + 32 * kh + 8 * q4 + 4 * h] = (u32x2_t){pw[2 * q4], pw[2 * q4 + 1]};
    if (kh == 0 && h == 0) alph[hl] = alpha;
    const uint64_t kb_ = __ballot(keep), sb_ = __ballot(alpha != 1.f);
    if (lane == 0) kflag[w] = (kb_ ? 1 : 0) | (sb_ ? 2 : 0);
    lds_barrier();  // (B) P^T, rescale factors and flags visible
    const int fl = kflag[0] | kflag[1] | kflag[2] | kflag[3];
    if (fl & 2) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float al = alph[32 * hb + l32];
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db][hb] *= al;
      }
    }
    if (fl & 1) {
      // O^T += V^T P^T over 4 steps of 16 keys: every P^T operand read at
      // once, the V^T operands one step ahead (the first step's before the
      // barrier)
      u32x4_t pb[4][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          pb[ks][hb] = *(const u32x4_t*)&Ps[(32 * hb + l32) * PP + 16 * ks + 8 * h];
      u32x4_t va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) va[db] = va0[db];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4_t van[4];
        if (ks + 1 < 4) rdv(ks + 1, van);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            o[db][hb] = mfma32x32x16(as_bf16x8(va[db]), as_bf16x8(pb[ks][hb]), o[db][hb]);
        if (ks + 1 < 4) {
#pragma unroll
          for (int db = 0; db < 4; ++db) va[db] = van[db];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    ++idx;
  };
  if (nl > 0) tile_to_lds(Kt0, tile_of(0));
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  while (idx < nl) {
    step(even);
    if (idx >= nl) break;
    step(odd);
  }

  // ---- partial of this split: (m, l) per head and the unnormalised O
  const float lsum = sum_with_lane_xor32(lp);
  const float qsum = sum_with_lane_xor32(lq);
  if (h == 0) {
    lred[0][kh][hl] = lsum;
    lred[1][kh][hl] = qsum;
  }
  __syncthreads();
  if (kh == 0 && h == 0 && hv) {
    float* ml = ws.part_ml + ((row0 + hl) * nsplit + s) * 4;
    const float dl = lred[0][0][hl] + lred[0][1][hl];
    const float dq = lred[1][0][hl] + lred[1][1][hl];
    if constexpr (MODE == 0) {
      ml[0] = m_acc;
      ml[1] = dl;
      ml[2] = dq;
      ws.smax[(row0 + hl) * nsplit + s] = m;
    } else {
      ml[1] += dl;  // the removed contributions (negative)
      ml[2] += dq;
    }
  }
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (h0 + 32 * hb + l32 >= G) continue;
    float* po = ws.part_o + ((row0 + 32 * hb + l32) * nsplit + s) * DV + 128 * w + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4_t*)(po + 32 * db + 8 * q4) =
            (f32x4_t){o[db][hb][4 * q4], o[db][hb][4 * q4 + 1], o[db][hb][4 * q4 + 2],
                      o[db][hb][4 * q4 + 3]};
  }
}

// Log-sum-exp merge of the split partials of one (batch, head) per wave, and
// the statistics. 4 rows per block; lane l owns features 8l..8l+7.
__global__ void __launch_bounds__(256) decode_mla_merge_kernel(DecodeArgs a, MlaWork ws) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(row / a.Hq), hq = (int)(row % a.Hq);
  const int kvh = hq / a.G;
  const int nsplit = ws.nsplit;
  const float c2 = a.scale_log2;
  const float* ml = ws.part_ml + row * nsplit * 4;
  // the splits' (m, l, l at the reference max) one per lane, 64 splits at a
  // time; the merged max over the splits that kept something
  float ms = kNegInf;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    if (s < nsplit && ml[4 * s + 1] > 0.f) ms = fmaxf(ms, ml[4 * s]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ms = fmaxf(ms, shfl_xor_f(ms, d));
  // each split's weight 2^((m - ms) c2) (0 for a split that kept nothing),
  // broadcast from its lane; the partial outputs are read with no branch
  // between them, in split order
  float L = 0.f, Lq = 0.f;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    float wgt = 0.f, lw = 0.f, lqw = 0.f;
    if (s < nsplit) {
      const float l = ml[4 * s + 1];
      if (l > 0.f) {
        wgt = fast_exp2((ml[4 * s] - ms) * c2);
        lw = l * wgt;
        lqw = ml[4 * s + 2] * wgt;
      }
    }
    const int cnt = min(64, nsplit - s0);
    const float* po = ws.part_o + (row * nsplit + s0) * DV + 8 * lane;
    auto add = [&](int y, const f32x4_t& v0, const f32x4_t& v1) __attribute__((always_inline)) {
      const float wy = __shfl(wgt, y, 64);
      L += __shfl(lw, y, 64);
      Lq += __shfl(lqw, y, 64);
      acc0 += v0 * wy;
      acc1 += v1 * wy;
    };
    int y = 0;
    for (; y + 4 <= cnt; y += 4) {  // four splits' loads in flight, then their sums
      f32x4_t v[4][2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e][0] = *(const f32x4_t*)(po + (int64_t)(y + e) * DV);
        v[e][1] = *(const f32x4_t*)(po + (int64_t)(y + e) * DV + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) add(y + e, v[e][0], v[e][1]);
    }
    for (; y < cnt; ++y)
      add(y, *(const f32x4_t*)(po + (int64_t)y * DV), *(const f32x4_t*)(po + (int64_t)y * DV + 4));
  }
  const float inv = 1.f / Lq;
  const int64_t ob = b * a.os0 + (int64_t)hq * a.os1 + 8 * lane;
  store_out4(a.out, ob, a.out_f32, acc0[0] * inv, acc0[1] * inv, acc0[2] * inv, acc0[3] * inv);
  store_out4(a.out, ob + 4, a.out_f32, acc1[0] * inv, acc1[1] * inv, acc1[2] * inv, acc1[3] * inv);
  if (a.lse && lane == 0) a.lse[row] = ms * a.scale + logf(L);
  if (a.stats) {
    int kept = 0;
    for (int s = lane; s < nsplit; s += 64) kept += ws.part_kept[row * nsplit + s];
    for (int d = 32; d >= 1; d >>= 1) kept += __shfl_xor(kept, d, 64);
    if (lane == 0) {
      int64_t* st = a.stats + row * 3;
      st[0] = a.nkt;
      st[1] = kept;
    }
    // tiles that some query head of the KV head keeps (any head group): one
    // count per KV head, taken by the wave of its first query head and written
    // to all G rows
    if (hq % a.G == 0) {
      const uint8_t* any0 = ws.anyk + (int64_t)(b * a.Hkv + kvh) * ws.ngroups * a.nkt;
      int cv = 0;
      for (int j = lane; j < a.nkt; j += 64) {
        bool any = false;
        for (int x = 0; x < ws.ngroups; ++x) any |= any0[(int64_t)x * a.nkt + j] != 0;
        cv += any ? 1 : 0;
      }
      for (int d = 32; d >= 1; d >>= 1) cv += __shfl_xor(cv, d, 64);
      for (int x = lane; x < a.G; x += 64) a.stats[(row + x) * 3 + 2] = cv;
    }
  }
}

namespace {
struct MlaPlan {
  int ngroups, nsplit, T;
  size_t off_tmax, off_smax, off_o, off_ml, off_kept, off_any, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

MlaPlan mla_plan(int B, int Hq, int Hkv, int G, int nkt) {
  MlaPlan p;
  p.ngroups = (G + HG - 1) / HG;
  const int64_t units = (int64_t)B * Hkv * p.ngroups;
  int64_t ns = units > 0 ? (TARGET_BLOCKS + units - 1) / units : 1;
  ns = ns < 1 ? 1 : (ns > nkt ? nkt : ns);
  int T = (int)((nkt + ns - 1) / ns);
  if (T > LIST_MAX) T = LIST_MAX;
  p.T = T;
  p.nsplit = (nkt + T - 1) / T;
  const size_t rows = (size_t)B * Hq;
  size_t off = 0;
  p.off_tmax = off;
  off = align256(off + rows * nkt * sizeof(float));
  p.off_smax = off;
  off = align256(off + rows * p.nsplit * sizeof(float));
  p.off_o = off;
  off = align256(off + rows * p.nsplit * DV * sizeof(float));
  p.off_ml = off;
  off = align256(off + rows * p.nsplit * 4 * sizeof(float));
  p.off_kept = off;
  off = align256(off + rows * p.nsplit * sizeof(int));
  p.off_any = off;
  off = align256(off + (size_t)B * Hkv * p.ngroups * nkt);
  p.bytes = off;
  return p;
}
}  // namespace

size_t decode_mla_workspace_bytes(int B, int Hq, int Hkv, int G, int nkt) {
  return mla_plan(B, Hq, Hkv, G, nkt).bytes;
}

hipError_t launch_decode_mla(const DecodeArgs& a, void* workspace, hipStream_t stream) {
  const MlaPlan p = mla_plan(a.B, a.Hq, a.Hkv, a.G, a.nkt);
  char* base = static_cast<char*>(workspace);
  MlaWork ws;
  ws.tmax = reinterpret_cast<float*>(base + p.off_tmax);
  ws.smax = reinterpret_cast<float*>(base + p.off_smax);
  ws.part_o = reinterpret_cast<float*>(base + p.off_o);
  ws.part_ml = reinterpret_cast<float*>(base + p.off_ml);
  ws.part_kept = reinterpret_cast<int*>(base + p.off_kept);
  ws.anyk = reinterpret_cast<uint8_t*>(base + p.off_any);
  ws.ngroups = p.ngroups;
  ws.nsplit = p.nsplit;
  ws.T = p.T;
  const int64_t nblocks = (int64_t)a.B * a.Hkv * p.ngroups * p.nsplit;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_mla_split_kernel<0>, dim3((unsigned)nblocks), dim3(NT), 0, stream, a,
                     ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mla_split_kernel<1>, dim3((unsigned)nblocks), dim3(NT), 0, stream, a,
                     ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.Hq;
  hipLaunchKernelGGL(decode_mla_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, a, ws);
  return hipGetLastError();
}

}  // namespace blasst
