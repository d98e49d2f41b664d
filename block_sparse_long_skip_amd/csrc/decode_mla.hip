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
// Layout. One workgroup of 4 waves per (batch, KV head, group of 16 query
// heads); the groups of a sequence are placed on one XCD so that its latent
// tiles are shared through that XCD's L2. Per 64-key tile:
//   * the 64 x 576 tile (72 KB) sits in LDS (double-buffered; the 16-byte
//     chunk index is XOR-swizzled by the row so that both the score operand
//     reads and the transposing value reads hit distinct banks). Tiles are
//     staged through registers two tiles ahead of their use;
//   * wave w scores keys 16w..16w+15 for the 16 heads: S^T = K q^T on
//     v_mfma_f32_16x16x32_bf16 (two accumulator chains over the 18 steps);
//   * the per-head tile maxima of the four waves meet in LDS, every wave then
//     takes the same decision per head, and P^T (bf16) of each wave's 16 keys
//     goes to LDS;
//   * if any head keeps the tile, wave w computes output features
//     128w..128w+127: O^T += V^T P^T, with V^T read straight from the key tile
//     by ds_read_b64_tr_b16.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int BC = 64;
constexpr int DQK = 576;
constexpr int DV = 512;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int HG = 16;                    // query heads per workgroup
constexpr int ROWB = DQK * 2;             // 1152 bytes per key row
constexpr int TILEB = BC * ROWB;          // 73728 bytes per tile
constexpr int NCH = TILEB / 16;           // 4608 16-byte chunks per tile
constexpr int CPT = NCH / NT;             // 18 chunks per thread
constexpr int PP = BC + 8;                // P^T row pitch (bf16): 144 B
static_assert(NCH % NT == 0, "tile chunks split evenly over the workgroup");
static_assert(DV == 128 * NW, "each wave produces 128 output features");

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

// XOR on the low 3 bits of the 16-byte chunk index of key row r: 8 distinct
// values over the even rows (and over the odd rows) of any 16 consecutive
// rows, and different high bits for rows r and r+2
__device__ __forceinline__ int mla_f(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int mla_off(int r, int c) { return r * ROWB + ((c ^ mla_f(r)) << 4); }

__device__ __forceinline__ u32x2_t ds_read_tr(const char* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4_t*)(p)));
}
}  // namespace

__global__ void __launch_bounds__(NT, 1) decode_mla_kernel(DecodeArgs a, int ngroups) {
  __shared__ __attribute__((aligned(16))) char Kt[2][TILEB];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[HG * PP];
  __shared__ float tmw[2][NW][HG];
  __shared__ float lred[NW][HG];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int n = lane & 15;  // head within the group (B/C operand column)
  const int g = lane >> 4;  // 0..3
  // consecutive logical blocks share a sequence; when the grid is a multiple
  // of 8 they are placed on one XCD (blocks are dealt to XCDs round-robin)
  const int total = (int)gridDim.x;
  int lb = (int)blockIdx.x;
  if ((total & 7) == 0) lb = (lb & 7) * (total >> 3) + (lb >> 3);
  const int gi = lb % ngroups;
  const int seq = lb / ngroups;  // (b, kvh)
  const int b = seq / a.Hkv, kvh = seq % a.Hkv;
  const int G = a.G;
  const int h0 = gi * HG;
  const bool hvalid = h0 + n < G;
  const int hq = kvh * G + h0 + n;
  const float c2 = a.scale_log2;

  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + (int64_t)hq * a.qs1;
  const char* kp = (const char*)((const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1);
  const int64_t rowstride = a.ks2 * 2;  // bytes

  // q^T as the B operand: lane supplies q[head n][32kk + 8g .. +7]
  bf16x8_t qb[DQK / 32];
#pragma unroll
  for (int kk = 0; kk < DQK / 32; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (hvalid) v = load16(qp + 32 * kk + 8 * g);
    qb[kk] = as_bf16x8(v);
  }

  // ---- per-lane LDS offsets
  // score operand (A = K rows): key row 16w + n, chunk 4kk + g; kk even/odd
  // give two patterns, kk >> 1 adds 128 bytes
  const int kr = 16 * w + n;
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

  // ---- tile staging: thread t holds chunks t + 256 i (row q/72, chunk q%72)
  auto load_tile = [&](u32x4_t (&r)[CPT], int j) {
    const int c0 = j * BC;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int q = t + NT * i;
      const int row = q / (DQK / 8), ch = q % (DQK / 8);
      const int key = min(c0 + row, a.Nk - 1);  // past the end: clamped, masked below
      r[i] = load16(kp + (int64_t)key * rowstride + ch * 16);
    }
  };
  auto store_tile = [&](char* tile, const u32x4_t (&r)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int q = t + NT * i;
      store16(tile + mla_off(q / (DQK / 8), q % (DQK / 8)), r[i]);
    }
  };

  f32x4_t o[8];  // O^T[dv = 128w + 16db + 4g + i][head n]
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;  // running max of head n (raw units), over kept tiles
  float lp = 0.f;     // this lane's partial row sum
  int kept = 0;
  const int nkt = a.nkt;

  // one key tile: buffer P, staging set `st` receives tile j+2 after handing tile j+1 to LDS
  int j = 0;
  auto step = [&](auto PAR, u32x4_t (&cur)[CPT], u32x4_t (&nxt)[CPT]) {
    constexpr int P = decltype(PAR)::value;
    // tile j is in Kt[P]; cur holds tile j+1 (in flight), nxt holds tile j+2 (in flight)
    // Loads are issued every step (past the last tile they re-read it), so the
    // number of loads in flight is fixed and the wait for `cur` leaves the 18
    // loads of `nxt` outstanding.
    if (j + 1 < nkt) store_tile(Kt[P ^ 1], cur);  // Kt[P^1] was last read before the barrier
    load_tile(cur, min(j + 3, nkt - 1));
    const char* kt = Kt[P];
    // scores of this wave's 16 keys for the 16 heads: two chains over the 18 steps
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DQK / 32; kk += 2) {
      const bf16x8_t k0 = as_bf16x8(*(const u32x4_t*)(kt + ko_even + 128 * (kk >> 1)));
      const bf16x8_t k1 = as_bf16x8(*(const u32x4_t*)(kt + ko_odd + 128 * (kk >> 1)));
      s0 = mfma16x16x32(k0, qb[kk], s0);
      s1 = mfma16x16x32(k1, qb[kk + 1], s1);
    }
    f32x4_t s = s0 + s1;  // S^T[key = 16w + 4g + i][head n]
    const int c0 = j * BC;
    if (c0 + BC > a.Nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c0 + 16 * w + 4 * g + i >= a.Nk) s[i] = kNegInf;
    }
    float tm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    tm = fmaxf(tm, shfl_xor_f(tm, 16));
    tm = fmaxf(tm, shfl_xor_f(tm, 32));
    if (g == 0) tmw[P][w][n] = tm;
    __syncthreads();  // (1) tile maxima visible; tile j+1 in Kt[P^1]
    const float TM = fmaxf(fmaxf(tmw[P][0][n], tmw[P][1][n]), fmaxf(tmw[P][2][n], tmw[P][3][n]));
    float gap;
    if (TM == kNegInf) gap = kNegInf;
    else if (m == kNegInf) gap = __builtin_inff();
    else gap = TM - m;
    const bool keep = hvalid && ((j == 0) || !(gap < a.thr_raw));
    if (a.mask && w == 0 && g == 0 && hvalid) a.mask[((int64_t)b * a.Hq + hq) * nkt + j] = keep ? 1 : 0;
    kept += keep ? 1 : 0;
    if (__any(keep)) {  // the same in every wave: TM and m are replicated
      float p[4] = {0.f, 0.f, 0.f, 0.f};
      if (keep) {
        const float m_new = fmaxf(m, TM);
        const float mc = m_new * c2;
        if (m_new != m) {
          const float alpha = fast_exp2(m * c2 - mc);
          lp *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[db] *= alpha;
        }
        m = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = fast_exp2(fmaf(s[i], c2, -mc));
          lp += p[i];
        }
      }
      *(u32x2_t*)&Ps[n * PP + 16 * w + 4 * g] = (u32x2_t){pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      __syncthreads();  // (2) P^T of all 64 keys visible
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8_t pbv = as_bf16x8(*(const u32x4_t*)&Ps[n * PP + 32 * cc + 8 * g]);
        const char* vt = kt + cc * 32 * ROWB;
        u32x4_t va[8];
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int off = (db >> 2) * 128;
          const u32x2_t y0 = ds_read_tr(vt + off + vo[db & 3][0]);
          const u32x2_t y1 = ds_read_tr(vt + off + vo[db & 3][1]);
          va[db] = (u32x4_t){y0[0], y0[1], y1[0], y1[1]};
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db] = mfma16x16x32(as_bf16x8(va[db]), pbv, o[db]);
      }
    }
    __syncthreads();  // (3) done with Kt[P] and Ps; tile j+1's staging is in LDS
    ++j;
  };

  // prologue: tile 0 into LDS, tiles 1 and 2 in flight
  {
    u32x4_t r0[CPT];
    load_tile(r0, 0);
    store_tile(Kt[0], r0);
  }
  u32x4_t sa[CPT], sb[CPT];
  load_tile(sa, min(1, nkt - 1));
  load_tile(sb, min(2, nkt - 1));
  __syncthreads();
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  while (j < nkt) {
    step(even, sa, sb);
    if (j >= nkt) break;
    step(odd, sb, sa);
  }

  // row sums: lanes (n, g) of every wave hold partials for head n
  lp += shfl_xor_f(lp, 16);
  lp += shfl_xor_f(lp, 32);
  if (g == 0) lred[w][n] = lp;
  __syncthreads();
  const float L = lred[0][n] + lred[1][n] + lred[2][n] + lred[3][n];
  if (hvalid) {
    const float inv = 1.f / L;
    const int64_t ob = b * a.os0 + (int64_t)hq * a.os1;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      store_out4(a.out, ob + 128 * w + 16 * db + 4 * g, a.out_f32, o[db][0] * inv, o[db][1] * inv,
                 o[db][2] * inv, o[db][3] * inv);
    if (w == 0 && g == 0) {
      if (a.lse) a.lse[(int64_t)b * a.Hq + hq] = m * a.scale + logf(L);
      if (a.stats) {
        int64_t* st = a.stats + ((int64_t)b * a.Hq + hq) * 3;
        st[0] = nkt;
        st[1] = kept;
      }
    }
  }
}

// stats[..., 2] for a latent cache: the number of key tiles that at least one
// query head of the KV head keeps, counted from the mask. One block per (b, kvh).
__global__ void __launch_bounds__(256) decode_vtiles_kernel(const uint8_t* mask, int64_t* stats,
                                                            int Hq, int Hkv, int G, int nkt) {
  __shared__ int total;
  const int b = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  int cntv = 0;
  for (int j = threadIdx.x; j < nkt; j += blockDim.x) {
    bool any = false;
    for (int h = 0; h < G; ++h) any |= mask[((int64_t)b * Hq + kvh * G + h) * nkt + j] == 1;
    cntv += any ? 1 : 0;
  }
  atomicAdd(&total, cntv);
  __syncthreads();
  for (int h = threadIdx.x; h < G; h += blockDim.x)
    stats[((int64_t)b * Hq + kvh * G + h) * 3 + 2] = total;
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t stream) {
  const int ngroups = (a.G + HG - 1) / HG;
  const int64_t nblocks = (int64_t)a.B * a.Hkv * ngroups;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_mla_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream, a, ngroups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.stats && a.mask) {
    hipLaunchKernelGGL(decode_vtiles_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, stream,
                       a.mask, a.stats, a.Hq, a.Hkv, a.G, a.nkt);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace blasst
