// bf16 backward of skip-softmax prefill on gfx950, d_qk = d_v = 128, with the
// forward's tile mask (128-row query tiles x 64-key tiles) held fixed.
//
// Method: fine-tuning a model with the skip kernels in place improves its
// quality (BLASST post, "BLASST: Dynamic BLocked Attention Sparsity via
// Softmax Thresholding", paragraph beginning "Все изменения можно делать без
// дообучения"). The keep/drop decisions are piecewise constant in the inputs,
// so the gradient is that of softmax attention over the kept tiles: with
// P = exp(scale q.k - lse) on kept, visible pairs (0 elsewhere),
//   dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO * O),  dS = P (dP - delta),
//   dQ = scale dS K,  dK = scale dS^T Q,
// dK and dV of a KV head summed over the query heads that read it. P is
// recomputed from the forward's lse; only kept tiles are visited.
//
// Kernels:
//   bwd_delta_kernel  delta[row] = dO[row] . O[row] (fp32), into the workspace.
//   bwd_dq_kernel     one workgroup of 4 waves per (batch, query head, query
//                     tile), wave w owning rows 32w..32w+31, laid out like the
//                     forward: S^T = K Q^T and dP^T = V dO^T on MFMA put one
//                     query row in each lane column, dS^T is formed in-lane,
//                     and dQ^T += K^T dS^T reads K^T from the LDS key tile with
//                     the transposing read, the key order inside each MFMA
//                     permuted to match the accumulator layout. The kept key
//                     tiles of the query tile are listed in LDS first; K and V
//                     tiles are double-buffered.
//   bwd_kv_kernel     dV (one launch) and dK (a second launch): one workgroup
//                     of 4 waves per (batch, KV head, pair of key tiles), wave
//                     w owning keys 32w..32w+31 of the pair. S = Q K^T (and for
//                     dK, dP = dO V^T) put one key in each lane column (the K
//                     and V rows of the lane's key live in registers as the B
//                     operands), so P and dS come out of the accumulators
//                     already in the A-operand layout of dV += P^T dO and
//                     dK += dS^T Q; dO and Q are read transposed from 64-row
//                     LDS stages (double-buffered), rows permuted the same way.
//                     The workgroup walks every query head of the KV group and
//                     the query tiles whose mask byte for either key tile is 1.
//                     Splitting dV from dK (S recomputed once more) keeps each
//                     launch within two workgroups per CU.
#include <type_traits>

#include "common.hpp"

namespace blasst {

namespace {
constexpr int D = 128;
constexpr int BR = 128;   // query tile of the forward mask
constexpr int BC = 64;    // key tile of the forward mask
constexpr int NT = 256;
constexpr int KTILE = BC * D * 2;  // 16 KB: 64 rows x 256 B
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit data format, raw access

// XOR applied to the 16-byte chunk index of tile row `row` (depends on row % 16)
__device__ __forceinline__ int swz_f(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
// byte offset of (row, 16-byte chunk c) inside a tile of 256-byte rows
__device__ __forceinline__ int swz(int row, int c) { return row * 256 + ((c ^ swz_f(row)) << 4); }

// Uniform buffer resource over `rows` rows of `rowbytes` bytes starting at p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* p, int rows,
                                                            int64_t rowbytes) {
  const uint64_t tb = (uint64_t)p;
  const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tb >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tb);
  const int nrec = __builtin_amdgcn_readfirstlane((int)((uint32_t)max(rows, 0) * (uint32_t)rowbytes));
  return __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0, nrec, kBufferFlags);
}
}  // namespace

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O): 16 lanes per row, 8 features each
__global__ void __launch_bounds__(NT) bwd_delta_kernel(BackwardArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t row = gid >> 4;
  const int part = (int)(gid & 15);
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Nq;
  float acc = 0.f;
  if (row < nrows) {
    const int64_t bh = row / a.Nq, r = row % a.Nq;
    const int b = (int)(bh / a.Hq), hq = (int)(bh % a.Hq);
    const u32x4_t g = load16((const uint16_t*)a.dout + b * a.dos0 + hq * a.dos1 + r * a.dos2 + 8 * part);
    float o[8];
    const int64_t oo = b * a.os0 + hq * a.os1 + r * a.os2 + 8 * part;
    if (a.out_f32) {
      const f32x4_t x0 = *(const f32x4_t*)((const float*)a.out + oo);
      const f32x4_t x1 = *(const f32x4_t*)((const float*)a.out + oo + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { o[e] = x0[e]; o[4 + e] = x1[e]; }
    } else {
      const u32x4_t x = load16((const uint16_t*)a.out + oo);
#pragma unroll
      for (int e = 0; e < 4; ++e) { o[2 * e] = bf16_lo(x[e]); o[2 * e + 1] = bf16_hi(x[e]); }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(g[e]) * o[2 * e] + bf16_hi(g[e]) * o[2 * e + 1];
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += shfl_xor_f(acc, m);
  if (row < nrows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(NT, 2) bwd_dq_kernel(BackwardArgs a) {
  // K and V tiles of the two buffers, each its own LDS array: the compiler
  // tracks copies into LDS per array, so a read of one buffer does not wait
  // for the copy in flight into the other
  __shared__ __attribute__((aligned(16))) char K0[KTILE];
  __shared__ __attribute__((aligned(16))) char K1[KTILE];
  __shared__ __attribute__((aligned(16))) char V0[KTILE];
  __shared__ __attribute__((aligned(16))) char V1[KTILE];
  char* const Ks[2] = {K0, K1};
  char* const Vs[2] = {V0, V1};
  __shared__ uint16_t tlist[kBackwardMaxTiles];
  __shared__ int wcount[4];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // block -> (query tile, head): heaviest query tiles first; heads of one KV
  // group on one XCD when the head count is a multiple of 8
  const int nbh = a.B * a.Hq;
  const int i = a.nqt - 1 - (int)(blockIdx.x / nbh);
  int bh = (int)(blockIdx.x % nbh);
  if ((nbh & 7) == 0) bh = (bh & 7) * (nbh >> 3) + (bh >> 3);
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / (a.Hq / a.Hkv);

  const int row = i * BR + 32 * w + l32;  // this lane's query row
  const bool valid = row < a.Nq;
  const int qpos = row + (a.Nk - a.Nq);
  const int last_row = min(i * BR + BR - 1, a.Nq - 1);
  const int first_pos = i * BR + (a.Nk - a.Nq);
  const int J = a.causal ? min(a.nkt, (last_row + a.Nk - a.Nq) / BC + 1) : a.nkt;
  const float c2 = a.scale_log2;

  // Q^T and dO^T as B operands: lane supplies row `row`, features 16kk + 8h .. +7
  bf16x8_t qb[D / 16], gb[D / 16];
  {
    // rows past the end load the last row (no branch) and are zeroed
    const int64_t rc = min(row, a.Nq - 1);
    const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + hq * a.qs1 + rc * a.qs2;
    const uint16_t* gp = (const uint16_t*)a.dout + b * a.dos0 + hq * a.dos1 + rc * a.dos2;
    u32x4_t vq[D / 16], vg[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      vq[kk] = load16(qp + 16 * kk + 8 * h);
      vg[kk] = load16(gp + 16 * kk + 8 * h);
    }
    const uint32_t keep = valid ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qb[kk] = as_bf16x8(vq[kk] & keep);
      gb[kk] = as_bf16x8(vg[kk] & keep);
    }
  }
  // the row's lse in exp2 units (+inf for a row that saw nothing or does not
  // exist, so that its P is 0) and its delta
  float lse2 = __builtin_inff(), dlt = 0.f;
  if (valid) {
    const float l = a.lse[(int64_t)bh * a.Nq + row];
    if (l != kNegInf) lse2 = l * kLog2e;
    dlt = a.delta[(int64_t)bh * a.Nq + row];
  }

  // kept key tiles of this query tile, in increasing order
  const uint8_t* mrow = a.mask + ((int64_t)bh * a.nqt + i) * a.nkt;
  int n;
  {
    const int per = (J + NT - 1) / NT;
    const int x0 = min(t * per, J), x1 = min(x0 + per, J);
    int cnt = 0;
    for (int x = x0; x < x1; ++x) cnt += mrow[x] == 1;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wcount[w] = incl;
    __syncthreads();
    int pos = incl - cnt;
    for (int ww = 0; ww < w; ++ww) pos += wcount[ww];
    n = __builtin_amdgcn_readfirstlane(wcount[0] + wcount[1] + wcount[2] + wcount[3]);
    for (int x = x0; x < x1; ++x)
      if (mrow[x] == 1) tlist[pos++] = (uint16_t)x;
    __syncthreads();
  }

  // tile copies: wave w fills rows 16w..16w+15, 4 rows per instruction
  const int sub = lane >> 4, pch = lane & 15;
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int trow = 16 * w + 4 * r + sub;
    const int ch = pch ^ swz_f(trow);
    koff[r] = (uint32_t)(((int64_t)trow * a.ks2 + ch * 8) * 2);
    voff[r] = (uint32_t)(((int64_t)trow * a.vs2 + ch * 8) * 2);
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const char* kp = (const char*)((const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1);
  const char* vp = (const char*)((const uint16_t*)a.v + b * a.vs0 + kvh * a.vs1);
  auto tile_to_lds = [&](char* tile, const char* base, const uint32_t (&off)[4], int64_t stride,
                         int c0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (int64_t)c0 * stride * 2, min(a.Nk - c0, BC), stride * 2);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + (16 * wu + 4 * r) * 256), 16, off[r],
          0, 0, 0);
  };
  auto tile_at = [&](int x) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane((int)tlist[x]);
  };
  // operand reads: key row 32kb + l32, chunk 2kk + h (kb = 1 is +8192 bytes)
  int kro[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kro[kk] = swz(l32, 2 * kk + h);
  // transposing reads of a key tile as K^T: lane group g16 = lane/16 reads keys
  // 16c + 4h + jj/4 and +8 (key chunk c is +4096 bytes), features dv0..dv0+3
  const int g16 = lane >> 4, jj = lane & 15;
  int tro[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dv0 = 32 * db + 16 * (g16 & 1) + 4 * (jj & 3);
    const int r0 = 4 * h + (jj >> 2);
    tro[db][0] = swz(r0, dv0 >> 3) + ((dv0 & 7) << 1);
    tro[db][1] = swz(r0 + 8, dv0 >> 3) + ((dv0 & 7) << 1);
  }

  // S^T = K Q^T and dP^T = V dO^T for the 32-key half of a key tile (K at kt,
  // V at vt in LDS; Q^T, dO^T in registers); each step's two operands are read
  // two steps ahead (a three-deep register ring)
  auto scores2 = [&](const char* kt, const char* vt, f32x16_t& s, f32x16_t& dp)
      __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
    u32x4_t xk[3], xv[3];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      xk[kk] = *(const u32x4_t*)(kt + kro[kk]);
      xv[kk] = *(const u32x4_t*)(vt + kro[kk]);
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + 2 < D / 16) {
        xk[(kk + 2) % 3] = *(const u32x4_t*)(kt + kro[kk + 2]);
        xv[(kk + 2) % 3] = *(const u32x4_t*)(vt + kro[kk + 2]);
      }
      s = mfma32x32x16(as_bf16x8(xk[kk % 3]), qb[kk], s);
      dp = mfma32x32x16(as_bf16x8(xv[kk % 3]), gb[kk], dp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16_t dqa[4];  // dQ^T[d = 32db + 8(r/4) + 4h + r%4][row], unscaled
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

  if (n > 0) {
    tile_to_lds(Ks[0], kp, koff, a.ks2, tile_at(0) * BC);
    tile_to_lds(Vs[0], vp, voff, a.vs2, tile_at(0) * BC);
  }
  auto step = [&](auto PAR, int idx) __attribute__((always_inline)) {
    constexpr int P = decltype(PAR)::value;
    wait_vmem();
    __syncthreads();  // tile idx is in LDS; every wave is done with tile idx-1
    if (idx + 1 < n) {
      const int cn = tile_at(idx + 1) * BC;
      tile_to_lds(Ks[P ^ 1], kp, koff, a.ks2, cn);
      tile_to_lds(Vs[P ^ 1], vp, voff, a.vs2, cn);
    }
    const int c0 = tile_at(idx) * BC;
    const bool edge = (c0 + BC > a.Nk) || (a.causal && c0 + BC - 1 > first_pos);
    const char* kt = Ks[P];
    const char* vt = Vs[P];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T and dP^T for keys 32kb..32kb+31 (V tile at the same offset in Vs)
      f32x16_t s, dp;
      scores2(kt + 8192 * kb, vt + 8192 * kb, s, dp);
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = c0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (col >= a.Nk || (a.causal && col > qpos)) s[r] = kNegInf;
        }
      }
      // dS^T (bf16) in the B-operand layout of key chunk c = 2kb + cl: keys
      // 16c + 8(e/4) + 4h + e%4
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        // this chunk's K^T reads first, so the dS math covers their latency
        const int c = 2 * kb + cl;
        u32x4_t ka[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const u32x2_t y0 = ds_read_tr(kt + 4096 * c + tro[db][0]);
          const u32x2_t y1 = ds_read_tr(kt + 4096 * c + tro[db][1]);
          ka[db] = (u32x4_t){y0[0], y0[1], y1[0], y1[1]};
        }
        __builtin_amdgcn_sched_barrier(0);
        uint32_t pw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int r = 8 * cl + 2 * e2;
          const float p0 = fast_exp2(fmaf(s[r], c2, -lse2));
          const float p1 = fast_exp2(fmaf(s[r + 1], c2, -lse2));
          pw[e2] = pack_bf16x2(p0 * (dp[r] - dlt), p1 * (dp[r + 1] - dlt));
        }
        const bf16x8_t pb = as_bf16x8((u32x4_t){pw[0], pw[1], pw[2], pw[3]});
        // dQ^T += K^T dS^T over this 16-key chunk: 4 independent output blocks
#pragma unroll
        for (int db = 0; db < 4; ++db) dqa[db] = mfma32x32x16(as_bf16x8(ka[db]), pb, dqa[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  for (int idx = 0; idx < n; idx += 2) {
    step(even, idx);
    if (idx + 1 < n) step(odd, idx + 1);
  }

  if (valid) {
    float* dqp = a.dq + b * a.qs0 + hq * a.qs1 + (int64_t)row * a.qs2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *(f32x4_t*)(dqp + 32 * db + 8 * qd + 4 * h) =
            (f32x4_t){a.scale * dqa[db][4 * qd], a.scale * dqa[db][4 * qd + 1],
                      a.scale * dqa[db][4 * qd + 2], a.scale * dqa[db][4 * qd + 3]};
  }
}

// ---------------------------------------------------------------------------
// dV (DK = false) or dK (DK = true) of two consecutive key tiles (128 keys),
// in separate launches so that each fits two workgroups per CU. dV recomputes
// S; dK recomputes S and dP. Wave w owns keys 32w .. 32w+31 of the pair (key
// tile w / 2) over every query row, so each 64-row stage of Q, dO, lse and
// delta copied into LDS (double-buffered) serves 128 keys and no partial sums
// are exchanged. The workgroup visits the query tiles that keep either key
// tile; a wave whose key tile a query tile drops skips it.
template <bool DK>
__global__ void __launch_bounds__(NT, 2) bwd_kv_kernel(BackwardArgs a) {
  constexpr int SR = 64;             // query rows per LDS stage
  constexpr int STILE = SR * D * 2;  // 16 KB
  __shared__ __attribute__((aligned(16))) char Qs[2][STILE];
  __shared__ __attribute__((aligned(16))) char Gs[2][STILE];  // dO
  __shared__ __attribute__((aligned(16))) float LD[2][2][SR];  // [buffer][lse, delta][row]
  __shared__ uint16_t ilist[kBackwardMaxTiles];  // (query tile << 2) | keeps of the two key tiles
  __shared__ int wcount[4];
  static_assert((kBackwardMaxTiles << 2) <= 65536, "a list entry holds the query tile in 14 bits");

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int kt = w >> 1, kh = w & 1;  // key tile of the pair, key half

  // block -> (key-tile pair, (batch, KV head)): low key tiles (most query
  // tiles when causal) first
  const int nbk = a.B * a.Hkv;
  const int jp = (int)(blockIdx.x / nbk);
  const int bk = (int)(blockIdx.x % nbk);
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int j = 2 * jp + kt;  // this wave's key tile
  const int c0 = j * BC;
  const int key = c0 + 32 * kh + l32;  // this lane's key (MFMA column)
  const bool kvalid = key < a.Nk;
  const float c2 = a.scale_log2;

  // K (and for dK, V) rows of the lane's key as B operands: features
  // 16kk + 8h .. +7; keys past the end load the last key and are zeroed
  bf16x8_t kb[D / 16], vb[DK ? D / 16 : 1];
  {
    const int64_t kc = min(key, a.Nk - 1);
    const uint16_t* kp = (const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1 + kc * a.ks2;
    const uint16_t* vp = (const uint16_t*)a.v + b * a.vs0 + kvh * a.vs1 + kc * a.vs2;
    const uint32_t keep = kvalid ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kb[kk] = as_bf16x8(load16(kp + 16 * kk + 8 * h) & keep);
      if constexpr (DK) vb[kk] = as_bf16x8(load16(vp + 16 * kk + 8 * h) & keep);
    }
  }

  // A-operand reads (rows as MFMA rows): row base + l32, chunk 2kk + h
  int aro[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) aro[kk] = swz(l32, 2 * kk + h);
  // transposing reads (rows as the MFMA k index, permuted like the
  // accumulator rows): lane group g16 reads rows 16c + 4h + jj/4 and +8,
  // features d0..d0+3 of output block db
  const int g16 = lane >> 4, jj = lane & 15;
  int tro[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d0 = 32 * db + 16 * (g16 & 1) + 4 * (jj & 3);
    const int r0 = 4 * h + (jj >> 2);
    tro[db][0] = swz(r0, d0 >> 3) + ((d0 & 7) << 1);
    tro[db][1] = swz(r0 + 8, d0 >> 3) + ((d0 & 7) << 1);
  }
  // stage copies of 64 rows: wave w fills rows 16w..16w+15, instruction r
  // (0..3) rows 16w + 4r + lane/16
  const int sub = lane >> 4, pch = lane & 15;
  uint32_t qoff[4], goff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int trow = 16 * w + 4 * r + sub;
    const int ch = pch ^ swz_f(trow);
    qoff[r] = (uint32_t)(((int64_t)trow * a.qs2 + ch * 8) * 2);
    goff[r] = (uint32_t)(((int64_t)trow * a.dos2 + ch * 8) * 2);
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto stage_to_lds = [&](char* tile, const char* base, const uint32_t* off, int64_t stride,
                          int r0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (int64_t)r0 * stride * 2, min(a.Nq - r0, SR), stride * 2);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + (16 * wu + 4 * r) * 256), 16, off[r],
          0, 0, 0);
  };
  // lse (and for dK, delta) of 64 rows: wave 0 copies 256 bytes each
  auto rows_to_lds = [&](float (&dst)[2][SR], const float* lse_row, const float* dl_row, int r0)
      __attribute__((always_inline)) {
    if (wu == 0) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc((const char*)(lse_row + r0), min(a.Nq - r0, SR), 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rl, (__attribute__((address_space(3))) void*)(&dst[0][0]), 4, 4 * lane, 0, 0, 0);
      if constexpr (DK) {
        const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char*)(dl_row + r0), min(a.Nq - r0, SR), 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rd, (__attribute__((address_space(3))) void*)(&dst[1][0]), 4, 4 * lane, 0, 0, 0);
      }
    }
  };

  f32x16_t acc[4];  // dK or dV[key 8(r/4) + 4h + r%4 of the wave's 32][d = 32db + l32]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const bool second = 2 * jp + 1 < a.nkt;  // the pair has a second key tile
  for (int g = 0; g < G; ++g) {
    const int hq = kvh * G + g;
    const int64_t bh = (int64_t)b * a.Hq + hq;
    // query tiles that keep either key tile, in increasing order
    const uint8_t* mcol = a.mask + bh * a.nqt * a.nkt + 2 * jp;
    auto keeps = [&](int x) __attribute__((always_inline)) -> int {
      const uint8_t* m = mcol + (int64_t)x * a.nkt;
      return (m[0] == 1 ? 1 : 0) | (second && m[1] == 1 ? 2 : 0);
    };
    int n;
    {
      const int per = (a.nqt + NT - 1) / NT;
      const int x0 = min(t * per, a.nqt), x1 = min(x0 + per, a.nqt);
      int cnt = 0;
      for (int x = x0; x < x1; ++x) cnt += keeps(x) != 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      __syncthreads();  // the previous head's list and stages are no longer read
      if (lane == 63) wcount[w] = incl;
      __syncthreads();
      int pos = incl - cnt;
      for (int ww = 0; ww < w; ++ww) pos += wcount[ww];
      n = __builtin_amdgcn_readfirstlane(wcount[0] + wcount[1] + wcount[2] + wcount[3]);
      for (int x = x0; x < x1; ++x) {
        const int kp = keeps(x);
        if (kp) ilist[pos++] = (uint16_t)((x << 2) | kp);
      }
      __syncthreads();
    }
    const char* qp = (const char*)((const uint16_t*)a.q + b * a.qs0 + hq * a.qs1);
    const char* gp = (const char*)((const uint16_t*)a.dout + b * a.dos0 + hq * a.dos1);
    const float* lse_row = a.lse + bh * a.Nq;
    const float* dl_row = a.delta + bh * a.Nq;
    // stage x: rows SR (x & 1) .. of the (x / 2)-th listed query tile
    const int nst = 2 * n;
    auto entry = [&](int x) __attribute__((always_inline)) -> int {
      return __builtin_amdgcn_readfirstlane((int)ilist[x >> 1]);
    };
    if (nst > 0) {
      const int r0 = (entry(0) >> 2) * BR;
      stage_to_lds(Qs[0], qp, qoff, a.qs2, r0);
      stage_to_lds(Gs[0], gp, goff, a.dos2, r0);
      rows_to_lds(LD[0], lse_row, dl_row, r0);
    }
    auto step = [&](auto PAR, int x) __attribute__((always_inline)) {
      constexpr int P = decltype(PAR)::value;
      wait_vmem();
      __syncthreads();  // stage x is in LDS; every wave is done with x-1
      if (x + 1 < nst) {
        const int rn = (entry(x + 1) >> 2) * BR + SR * ((x + 1) & 1);
        stage_to_lds(Qs[P ^ 1], qp, qoff, a.qs2, rn);
        stage_to_lds(Gs[P ^ 1], gp, goff, a.dos2, rn);
        rows_to_lds(LD[P ^ 1], lse_row, dl_row, rn);
      }
      const int e = entry(x);
      if (!((e >> kt) & 1)) return;  // this query tile drops the wave's key tile
      const int r0 = (e >> 2) * BR + SR * (x & 1);
      const bool edge = (r0 + SR > a.Nq) || (c0 + BC > a.Nk) ||
                        (a.causal && c0 + BC - 1 > r0 + (a.Nk - a.Nq));
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int rb = 32 * sb;  // first row of the 32-row block in the stage
        const char* qt = Qs[P] + rb * 256;
        const char* gt = Gs[P] + rb * 256;
        // S[row][key] = Q K^T (and dP[row][key] = dO V^T)
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
        // operands read two steps ahead (a three-deep register ring)
        u32x4_t xq[3], xg[3];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          xq[kk] = *(const u32x4_t*)(qt + aro[kk]);
          if constexpr (DK) xg[kk] = *(const u32x4_t*)(gt + aro[kk]);
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk + 2 < D / 16) {
            xq[(kk + 2) % 3] = *(const u32x4_t*)(qt + aro[kk + 2]);
            if constexpr (DK) xg[(kk + 2) % 3] = *(const u32x4_t*)(gt + aro[kk + 2]);
          }
          s = mfma32x32x16(as_bf16x8(xq[kk % 3]), kb[kk], s);
          if constexpr (DK) dp = mfma32x32x16(as_bf16x8(xg[kk % 3]), vb[kk], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qrow = r0 + rb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (qrow >= a.Nq || !kvalid || (a.causal && key > qrow + (a.Nk - a.Nq))) s[r] = kNegInf;
          }
        }
        // per 16-row step ks (accumulator rows 8ks .. 8ks+7 of this lane,
        // query rows rb + 8(r/4) + 4h + r%4): P (dV) or dS (dK) in bf16 as
        // the A operand, then dV += P^T dO or dK += dS^T Q
        const char* bt = DK ? qt : gt;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // this step's transposing reads first, so the P or dS math covers them
          u32x2_t ya[4][2];
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            ya[db][0] = ds_read_tr(bt + 4096 * ks + tro[db][0]);
            ya[db][1] = ds_read_tr(bt + 4096 * ks + tro[db][1]);
          }
          __builtin_amdgcn_sched_barrier(0);
          uint32_t pw[4];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int q4 = 2 * ks + q;
            const f32x4_t x4 = *(const f32x4_t*)&LD[P][0][rb + 8 * q4 + 4 * h];
            f32x4_t y4 = {0.f, 0.f, 0.f, 0.f};
            if constexpr (DK) y4 = *(const f32x4_t*)&LD[P][1][rb + 8 * q4 + 4 * h];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              const int r = 4 * q4 + 2 * e2;
              const float l0 = x4[2 * e2] == kNegInf ? __builtin_inff() : x4[2 * e2] * kLog2e;
              const float l1 = x4[2 * e2 + 1] == kNegInf ? __builtin_inff() : x4[2 * e2 + 1] * kLog2e;
              const float p0 = fast_exp2(fmaf(s[r], c2, -l0));
              const float p1 = fast_exp2(fmaf(s[r + 1], c2, -l1));
              if constexpr (DK)
                pw[2 * q + e2] = pack_bf16x2(p0 * (dp[r] - y4[2 * e2]), p1 * (dp[r + 1] - y4[2 * e2 + 1]));
              else
                pw[2 * q + e2] = pack_bf16x2(p0, p1);
            }
          }
          const u32x4_t pa = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
          for (int db = 0; db < 4; ++db)
            acc[db] = mfma32x32x16(
                as_bf16x8(pa),
                as_bf16x8((u32x4_t){ya[db][0][0], ya[db][0][1], ya[db][1][0], ya[db][1][1]}), acc[db]);
        }
      }
    };
    const std::integral_constant<int, 0> even;
    const std::integral_constant<int, 1> odd;
    for (int x = 0; x < nst; x += 2) {
      step(even, x);
      if (x + 1 < nst) step(odd, x + 1);
    }
  }

  float* dst = DK ? a.dk + b * a.ks0 + kvh * a.ks1 : a.dv + b * a.vs0 + kvh * a.vs1;
  const int64_t ds2 = DK ? a.ks2 : a.vs2;
  const float mul = DK ? a.scale : 1.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = c0 + 32 * kh + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kr < a.Nk) dst[(int64_t)kr * ds2 + 32 * db + l32] = mul * acc[db][r];
    }
}

hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Nq;
  if (rows > 0) {
    const int64_t nb = (rows * 16 + NT - 1) / NT;
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)nb), dim3(NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((int64_t)a.B * a.Hq * a.nqt)), dim3(NT), 0,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nkv = (int64_t)a.B * a.Hkv * ((a.nkt + 1) / 2);  // key-tile pairs
  if (nkv > 0) {
    bwd_kv_kernel<false><<<dim3((unsigned)nkv), dim3(NT), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_kv_kernel<true><<<dim3((unsigned)nkv), dim3(NT), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace blasst
