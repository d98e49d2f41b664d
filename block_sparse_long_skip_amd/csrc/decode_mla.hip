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
//   pass 0 (speculative): every split runs the ordered tile loop with a running
//     max that starts at -inf at its first tile, writes every tile max to the
//     workspace, and leaves its partial (m, l, O) there;
//   pass 1 (exact): every split takes the true prefix max at its first tile
//     from the recorded tile maxima, derives the exact decision of every tile
//     and head, writes the mask, the kept counts and the per-tile "some head
//     keeps" flags, and compares with the decisions pass 0 took. Where they
//     agree for every head of the group (always for the first split, and
//     whenever nothing is dropped) the pass-0 partial is already exact. Where
//     they differ the split is recomputed from the true prefix max, visiting
//     only the tiles some head keeps, and its partial is replaced;
//   merge: a log-sum-exp merge of the partials of each (batch, head).
//
// Workgroup layout (4 waves, 64 heads). Per key tile:
//   * the 64 x 576 tile (72 KB) travels global -> LDS with
//     global_load_lds_dwordx4 (no register staging), double-buffered, the next
//     tile's copy issued at the top of the current one. The 16-byte chunk index
//     is XOR-swizzled by the row so that both the score operand reads (16
//     rows, one chunk) and the transposing value reads (4 rows, 2 chunks) hit
//     distinct banks;
//   * wave w = (key half kh = w & 1, head half hh = w >> 1) computes
//     S^T[32 keys][32 heads] = K q^T on v_mfma_f32_16x16x32_bf16, with its
//     heads' queries held in registers;
//   * the per-head tile maxima of the two key halves meet in LDS; every wave
//     then takes the same decision per head, and P^T (bf16) goes to LDS;
//   * if any head keeps the tile, wave w computes output features
//     128w..128w+127 of all 64 heads: O^T += V^T P^T, with V^T read from the
//     key tile by ds_read_b64_tr_b16.
#include <type_traits>

#include "common.hpp"

namespace blasst {

namespace {
constexpr int BC = 64;
constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int HG = 64;                    // query heads per workgroup
constexpr int KS = DQK / 32;              // 18 MFMA steps over the key features
constexpr int ROWB = DQK * 2;             // 1152 bytes per key row
constexpr int TILEB = BC * ROWB;          // 73728 bytes per tile
constexpr int NCH = TILEB / 16;           // 4608 16-byte chunks per tile
constexpr int DMA_PER_WAVE = NCH / 64 / NW;  // 18 copy instructions per wave per tile
constexpr int PP = BC + 8;                // P^T row pitch (bf16): 144 B
constexpr int LIST_MAX = 512;             // most tiles per split
constexpr int TARGET_BLOCKS = 256;        // one workgroup per CU
static_assert(NCH % (64 * NW) == 0, "tile copies split evenly over the waves");
static_assert(DV == 128 * NW, "each wave produces 128 output features");

// XOR on the low 3 bits of the 16-byte chunk index of key row r: 8 distinct
// values over the even rows (and over the odd rows) of any 16 consecutive
// rows, and different high bits for rows r and r+2
__device__ __forceinline__ int mla_f(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int mla_off(int r, int c) { return r * ROWB + ((c ^ mla_f(r)) << 4); }

// Workgroup barrier for LDS data only: waits for this wave's LDS operations
// but not for its copies into the other tile buffer, which stay in flight
// across it (a __syncthreads would wait for them). The memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
  float* tmax;     // [B*Hq][nkt]           tile maxima (raw q.k units)
  float* part_o;   // [B*Hq][nsplit][512]   unnormalised partial outputs
  float* part_ml;  // [B*Hq][nsplit][2]     partial (running max, row sum)
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
  __shared__ float lred[2][HG];
  __shared__ int kflag[NW];
  __shared__ uint16_t list[LIST_MAX];  // kept tiles of the split, relative to its first
  __shared__ int nlist;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
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
  float* const tmaxp = ws.tmax;

  // this lane's two score heads (head half hh, blocks hb = 0, 1)
  int hl[2];
  bool hv[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    hl[hb] = 32 * hh + 16 * hb + n;
    hv[hb] = h0 + hl[hb] < G;
  }

  // ---- exact decisions (pass 1): true prefix max at the split, mask, counts
  float m_init[2] = {kNegInf, kNegInf};
  int nl = j1 - j0;
  if constexpr (MODE == 1) {
    float* pmw = reinterpret_cast<float*>(Ps);  // [NW][HG] maxima of the tiles before the split
    float* smw = pmw + NW * HG;                 // [NW][HG] maxima of each wave's share of the split
    int* cntw = reinterpret_cast<int*>(smw + NW * HG);  // [NW][HG]
    int* misw = cntw + NW * HG;                         // [NW]
    uint8_t* tflag = reinterpret_cast<uint8_t*>(misw + NW);  // [T]
    const int h = lane;
    const bool hvl = h0 + h < G;
    const int64_t row = row0 + h;
    const float* tr = ws.tmax + row * nkt;
    float pmx = kNegInf;
    if (hvl)
      for (int j = (w * j0) / NW; j < ((w + 1) * j0) / NW; ++j) pmx = fmaxf(pmx, tr[j]);
    const int tn = j1 - j0;
    const int q0 = j0 + (w * tn) / NW, q1 = j0 + ((w + 1) * tn) / NW;
    float smx = kNegInf;
    if (hvl)
      for (int j = q0; j < q1; ++j) smx = fmaxf(smx, tr[j]);
    pmw[w * HG + h] = pmx;
    smw[w * HG + h] = smx;
    __syncthreads();
    // running maxima entering this wave's share: exact (from tile 0) and as
    // pass 0 had them (from the split's first tile)
    float mt = fmaxf(fmaxf(pmw[h], pmw[HG + h]), fmaxf(pmw[2 * HG + h], pmw[3 * HG + h]));
    float ml = kNegInf;
    for (int v = 0; v < w; ++v) {
      mt = fmaxf(mt, smw[v * HG + h]);
      ml = fmaxf(ml, smw[v * HG + h]);
    }
    int cnt = 0;
    bool mis = false;
    uint8_t* anyrow = ws.anyk + ((int64_t)seq * ws.ngroups + gi) * nkt;
    for (int j = q0; j < q1; ++j) {
      const float tm = hvl ? tr[j] : kNegInf;
      const bool kt = hvl && (j == 0 || !(gap_of(tm, mt) < thr));
      const bool kl = hvl && (j == 0 || !(gap_of(tm, ml) < thr));
      // a dropped tile's max is below the running max, so the plain max is
      // the running max over kept tiles
      mt = fmaxf(mt, tm);
      ml = fmaxf(ml, tm);
      cnt += kt ? 1 : 0;
      mis |= kt != kl;
      if (a.mask && hvl) a.mask[row * nkt + j] = kt ? 1 : 0;
      const bool any = __ballot(kt) != 0;
      if (lane == 0) {
        tflag[j - j0] = any ? 1 : 0;
        anyrow[j] = any ? 1 : 0;
      }
    }
    cntw[w * HG + h] = cnt;
    const bool wmis = __ballot(mis) != 0;
    if (lane == 0) misw[w] = wmis ? 1 : 0;
    __syncthreads();
    if (w == 0 && hvl)
      ws.part_kept[row * nsplit + s] =
          cntw[h] + cntw[HG + h] + cntw[2 * HG + h] + cntw[3 * HG + h];
    const bool redo = (misw[0] | misw[1] | misw[2] | misw[3]) != 0;
    if (!redo) return;  // the pass-0 partial is exact
    // the score lanes start from the exact prefix max at the split
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int x = hl[hb];
      m_init[hb] = fmaxf(fmaxf(pmw[x], pmw[HG + x]), fmaxf(pmw[2 * HG + x], pmw[3 * HG + x]));
    }
    // list of the tiles some head keeps, in order
    if (w == 0) {
      int base = 0;
      for (int c0 = 0; c0 < tn; c0 += 64) {
        const bool f = c0 + lane < tn && tflag[c0 + lane] != 0;
        const uint64_t bits = __ballot(f);
        if (f) list[base + __popcll(bits & ((1ull << lane) - 1ull))] = (uint16_t)(c0 + lane);
        base += __popcll(bits);
      }
      if (lane == 0) nlist = base;
    }
    __syncthreads();
    nl = nlist;
  }
  auto tile_of = [&](int idx) __attribute__((always_inline)) -> int {
    if constexpr (MODE == 1) return j0 + list[idx];
    else return j0 + idx;
  };

  // ---- queries: q^T as the B operand, lane supplies q[head hl][32kk + 8g .. +7]
  bf16x8_t qb[2][KS];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + (int64_t)(kvh * G + h0 + hl[hb]) * a.qs1;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (hv[hb]) v = load16(qp + 32 * kk + 8 * g);
      asm volatile("" : "+a"(v));  // queries live in AGPRs (MFMA operands may be AGPRs)
      qb[hb][kk] = as_bf16x8(v);
    }
  }

  // ---- per-lane LDS offsets
  // score operand (A = K rows): key row 32kh + 16kb + n, chunk 4kk + g; kk
  // even/odd give two patterns, kk >> 1 adds 128 bytes, kb adds 16 rows
  const int kr = 32 * kh + n;
  const int ko_even = kr * ROWB + (((g ^ mla_f(kr)) & 7) << 4);
  const int ko_odd = kr * ROWB + ((((4 + g) ^ mla_f(kr)) & 7) << 4);
  // value operand (A = V^T, transposing read): lane group g reads keys
  // 32cc + 8g + n/4 (and +4), features 128w + 16db + 4(n&3); cc adds 32 rows,
  // db >> 2 adds 128 bytes
  int vo[4][2];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 8 * g + (n >> 2) + 4 * hf;
      const int c = 16 * w + 2 * d4 + ((n & 3) >> 1);
      vo[d4][hf] = mla_off(r, c) + ((n & 1) << 3);
    }

  // ---- tile copies: wave w issues copies 18w..18w+17; copy q fills LDS chunks
  // 64q..64q+63, lane l chunk p = 64q + l = (row p / 72, physical chunk p % 72),
  // so it fetches the logical chunk the swizzle maps there
  const char* kp = (const char*)((const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1);
  const int64_t rowstride = a.ks2 * 2;  // bytes
  const uint32_t rs32 = (uint32_t)rowstride;
  auto tile_to_lds = [&](char* tile, int j) __attribute__((always_inline)) {
    const int c0 = j * BC;
    const char* tp = kp + (int64_t)c0 * rowstride;
    int ln0 = lane;
    asm volatile("" : "+v"(ln0));
    if (c0 + BC <= Nk) {
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int p = 64 * (DMA_PER_WAVE * w + i) + ln0;
        const int r = p / (DQK / 8), pc = p % (DQK / 8);
        const uint32_t off = (uint32_t)r * rs32 + (uint32_t)((pc ^ mla_f(r)) << 4);
        lds_dma16(tp + off, tile + 1024 * (DMA_PER_WAVE * w + i));
      }
    } else {
      // rows past the end of the cache re-read its last row (masked below);
      // the row index is recomputed here so that nothing of this path is kept
      // live across the tile loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int last = Nk - 1 - c0;
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int r = (64 * (DMA_PER_WAVE * w + i) + ln) / (DQK / 8);
        const int rr = min(r, last);
        lds_dma16(tp + ((uint32_t)rr * rs32 + (uint32_t)((((64 * (DMA_PER_WAVE * w + i) + ln) % (DQK / 8)) ^ mla_f(r)) << 4)), tile + 1024 * (DMA_PER_WAVE * w + i));
      }
    }
  };

  f32x4_t o[8][4];  // O^T[dv = 128w + 16db + 4g + i][head 16hb + n]
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) o[db][hb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m[2] = {m_init[0], m_init[1]};  // running max of the score heads (raw units)
  float lp[2] = {0.f, 0.f};             // partial row sums over this lane's keys

  // one key tile; the LDS buffer parity is a compile-time constant so that the
  // compiler can tell the copy into one buffer from the reads of the other
  int idx = 0;
  auto step = [&](auto PAR) __attribute__((always_inline)) {
    constexpr int P = decltype(PAR)::value;
    const int j = tile_of(idx);
    char* kt = P ? Kt1 : Kt0;
    wait_vmem();
    __syncthreads();  // (C) tile idx is in LDS; every wave is done with tile idx-1
    if (idx + 1 < nl) tile_to_lds(P ? Kt0 : Kt1, tile_of(idx + 1));

    // scores: S^T[key 32kh + 16kb + 4g + i][head hl[hb]]
    f32x4_t sc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) sc[kb][hb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    // the two key-block operands of step kk are read one step ahead; the
    // scheduling fence stops the compiler from hoisting every read of the
    // tile (that would take 144 registers)
    u32x4_t k0 = *(const u32x4_t*)(kt + ko_even);
    u32x4_t k1 = *(const u32x4_t*)(kt + ko_even + 16 * ROWB);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4_t n0 = k0, n1 = k1;
      if (kk + 1 < KS) {
        const int ko = (((kk + 1) & 1) ? ko_odd : ko_even) + 128 * ((kk + 1) >> 1);
        n0 = *(const u32x4_t*)(kt + ko);
        n1 = *(const u32x4_t*)(kt + ko + 16 * ROWB);
      }
      sc[0][0] = mfma16x16x32(as_bf16x8(k0), qb[0][kk], sc[0][0]);
      sc[0][1] = mfma16x16x32(as_bf16x8(k0), qb[1][kk], sc[0][1]);
      sc[1][0] = mfma16x16x32(as_bf16x8(k1), qb[0][kk], sc[1][0]);
      sc[1][1] = mfma16x16x32(as_bf16x8(k1), qb[1][kk], sc[1][1]);
      k0 = n0;
      k1 = n1;
      __builtin_amdgcn_sched_barrier(0);
    }
    const int c0 = j * BC;
    if (c0 + BC > Nk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + 32 * kh + 16 * kb + 4 * g + i >= Nk) sc[kb][0][i] = sc[kb][1][i] = kNegInf;
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float tm = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        tm = fmaxf(tm, fmaxf(fmaxf(sc[kb][hb][0], sc[kb][hb][1]), fmaxf(sc[kb][hb][2], sc[kb][hb][3])));
      tm = fmaxf(tm, shfl_xor_f(tm, 16));
      tm = fmaxf(tm, shfl_xor_f(tm, 32));
      if (g == 0) tmw[P][kh][hl[hb]] = tm;
    }
    lds_barrier();  // (A) tile maxima of both key halves visible

    bool anykeep = false, anyscale = false;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float TM = fmaxf(tmw[P][0][hl[hb]], tmw[P][1][hl[hb]]);
      if constexpr (MODE == 0) {
        if (kh == 0 && g == 0 && hv[hb]) tmaxp[(row0 + hl[hb]) * nkt + j] = TM;
      }
      const bool keep = hv[hb] && (j == 0 || !(gap_of(TM, m[hb]) < thr));
      float alpha = 1.f;
      float p[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (keep) {
        const float m_new = fmaxf(m[hb], TM);
        const float mc = m_new * c2;
        if (m_new != m[hb]) {
          alpha = fast_exp2(m[hb] * c2 - mc);
          lp[hb] *= alpha;
        }
        m[hb] = m_new;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kb][i] = fast_exp2(fmaf(sc[kb][hb][i], c2, -mc));
            lp[hb] += p[kb][i];
          }
      }
      anykeep |= keep;
      anyscale |= alpha != 1.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        *(u32x2_t*)&Ps[hl[hb] * PP + 32 * kh + 16 * kb + 4 * g] =
            (u32x2_t){pack_bf16x2(p[kb][0], p[kb][1]), pack_bf16x2(p[kb][2], p[kb][3])};
      if (kh == 0 && g == 0) alph[hl[hb]] = alpha;
    }
    const uint64_t kb_ = __ballot(anykeep), sb_ = __ballot(anyscale);
    if (lane == 0) kflag[w] = (kb_ ? 1 : 0) | (sb_ ? 2 : 0);
    lds_barrier();  // (B) P^T, rescale factors and flags visible
    const int fl = kflag[0] | kflag[1] | kflag[2] | kflag[3];
    if (fl & 2) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float al = alph[16 * hb + n];
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][hb] *= al;
      }
    }
    if (fl & 1) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x8_t pb[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          pb[hb] = as_bf16x8(*(const u32x4_t*)&Ps[(16 * hb + n) * PP + 32 * cc + 8 * g]);
        const char* vc = kt + cc * 32 * ROWB;
        // value operands read one output block ahead, fenced as above
        u32x2_t y0 = ds_read_tr(vc + vo[0][0]);
        u32x2_t y1 = ds_read_tr(vc + vo[0][1]);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          u32x2_t z0 = y0, z1 = y1;
          if (db + 1 < 8) {
            const int off = ((db + 1) >> 2) * 128;
            z0 = ds_read_tr(vc + off + vo[(db + 1) & 3][0]);
            z1 = ds_read_tr(vc + off + vo[(db + 1) & 3][1]);
          }
          const bf16x8_t va = as_bf16x8((u32x4_t){y0[0], y0[1], y1[0], y1[1]});
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) o[db][hb] = mfma16x16x32(va, pb[hb], o[db][hb]);
          y0 = z0;
          y1 = z1;
          __builtin_amdgcn_sched_barrier(0);
        }
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
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float l = lp[hb];
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    if (g == 0) lred[kh][hl[hb]] = l;
  }
  __syncthreads();
  if (kh == 0 && g == 0) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      if (hv[hb]) {
        float* ml = ws.part_ml + ((row0 + hl[hb]) * nsplit + s) * 2;
        ml[0] = m[hb];
        ml[1] = lred[0][hl[hb]] + lred[1][hl[hb]];
      }
  }
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    if (h0 + 16 * hb + n >= G) continue;
    float* po = ws.part_o + ((row0 + 16 * hb + n) * nsplit + s) * DV + 128 * w + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4_t*)(po + 16 * db) = o[db][hb];
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
  const float* ml = ws.part_ml + row * nsplit * 2;
  float ms = kNegInf;
  for (int s = 0; s < nsplit; ++s)
    if (ml[2 * s + 1] > 0.f) ms = fmaxf(ms, ml[2 * s]);
  float L = 0.f;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float l = ml[2 * s + 1];
    if (!(l > 0.f)) continue;
    const float wgt = fast_exp2((ml[2 * s] - ms) * c2);
    L += l * wgt;
    const float* po = ws.part_o + (row * nsplit + s) * DV + 8 * lane;
    acc0 += *(const f32x4_t*)po * wgt;
    acc1 += *(const f32x4_t*)(po + 4) * wgt;
  }
  const float inv = 1.f / L;
  const int64_t ob = b * a.os0 + (int64_t)hq * a.os1 + 8 * lane;
  store_out4(a.out, ob, a.out_f32, acc0[0] * inv, acc0[1] * inv, acc0[2] * inv, acc0[3] * inv);
  store_out4(a.out, ob + 4, a.out_f32, acc1[0] * inv, acc1[1] * inv, acc1[2] * inv, acc1[3] * inv);
  if (a.lse && lane == 0) a.lse[row] = ms * a.scale + logf(L);
  if (a.stats) {
    // tiles that some query head of the KV head keeps (any head group)
    const uint8_t* any0 = ws.anyk + (int64_t)(b * a.Hkv + kvh) * ws.ngroups * a.nkt;
    int cv = 0;
    for (int j = lane; j < a.nkt; j += 64) {
      bool any = false;
      for (int x = 0; x < ws.ngroups; ++x) any |= any0[(int64_t)x * a.nkt + j] != 0;
      cv += any ? 1 : 0;
    }
    int kept = 0;
    for (int s = lane; s < nsplit; s += 64) kept += ws.part_kept[row * nsplit + s];
    for (int d = 32; d >= 1; d >>= 1) {
      cv += __shfl_xor(cv, d, 64);
      kept += __shfl_xor(kept, d, 64);
    }
    if (lane == 0) {
      int64_t* st = a.stats + row * 3;
      st[0] = a.nkt;
      st[1] = kept;
      st[2] = cv;
    }
  }
}

namespace {
struct MlaPlan {
  int ngroups, nsplit, T;
  size_t off_tmax, off_o, off_ml, off_kept, off_any, bytes;
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
  p.off_o = off;
  off = align256(off + rows * p.nsplit * DV * sizeof(float));
  p.off_ml = off;
  off = align256(off + rows * p.nsplit * 2 * sizeof(float));
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
