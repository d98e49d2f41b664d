// bf16 skip-softmax decode on gfx950: one query token per (batch, head)
// against a contiguous KV cache with separate values, 64-key tiles (the latent
// cache kernel lives in decode_mla.hip).
//
// Method: BLASST post (seeallochnaya, "BLASST: Dynamic BLocked Attention
// Sparsity via Softmax Thresholding"): key tiles in increasing order, online
// max, a tile dropped whole when its max is far below the running max and its
// V never read (paragraph beginning "BLASST предлагает"), tile 0 always
// processed (first figure). For decode the running max is global along the
// cache: tile 0 is the cache's first tile and the decision for tile j uses the
// max over all tiles before j.
//
// decode_gqa_kernel (separate V, d = 128, up to 16 query heads per KV head):
//   one workgroup of 4 waves per (batch, KV head). The waves split the keys:
//   in round r wave w takes tile 4r + w.
//   * K is loaded from HBM straight into the 16x16x32 MFMA operand layout
//     (16-byte loads), one round ahead; scores S^T = K q^T put the group's
//     query heads in the MFMA columns.
//   * The per-head tile maxima of a round meet in LDS, so each wave decides
//     its tile against the exact prefix max of every earlier tile.
//   * V is loaded only when some head of the group keeps the tile. Its P.V is
//     done one round later, so the load has a whole round to land: the V rows
//     go to the wave's own LDS slice and O^T += V^T P^T reads them back
//     transposed (ds_read_b64_tr_b16). The online-softmax rescale of the
//     output is deferred in the same order, so the arithmetic is unchanged.
//   * Each wave keeps its own (m, l, O) partial; a log-sum-exp merge across
//     the waves ends the kernel.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int BC = 64;
constexpr int D = 128;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int SLICE = BC * D * 2;  // 16 KB: one V tile, 64 rows x 256 B


// 16-byte chunk c of row r of a 64 x 256 B tile, chunk index XOR-swizzled by the row
__device__ __forceinline__ int vswz(int r, int c) {
  return r * 256 + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4);
}
}  // namespace

__global__ void __launch_bounds__(NT, 1) decode_gqa_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char Vs[NW][SLICE];
  __shared__ float tmx[2][NW][16];
  __shared__ int cnt[NW][17];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int n = lane & 15;  // head within the group (B/C operand column)
  const int g = lane >> 4;  // 0..3
  const int bk = blockIdx.x;
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int G = a.G;
  const bool hvalid = n < G;
  const int hq = kvh * G + n;
  const int nkt = a.nkt;
  const float c2 = a.scale_log2;

  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + (int64_t)hq * a.qs1;
  const uint16_t* kp = (const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1;
  const uint16_t* vp = (const uint16_t*)a.v + b * a.vs0 + kvh * a.vs1;

  bf16x8_t qb[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (hvalid) v = load16(qp + 32 * kk + 8 * g);
    qb[kk] = as_bf16x8(v);
  }

  // K tile j in the A-operand layout: kr[kb][kk] = K[16kb + n][32kk + 8g .. +7]
  // (rows past the end of the cache are clamped to its last row; their scores
  // are masked to -inf)
  auto load_k = [&](u32x4_t (&kr)[4][D / 32], int j) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(j * BC + 16 * kb + n, a.Nk - 1);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        kr[kb][kk] = load16(kp + (int64_t)key * a.ks2 + 32 * kk + 8 * g);
    }
  };
  // V tile j, row-major: lane holds rows 16g + i (i = 0..15), chunk n
  auto load_v = [&](u32x4_t (&vr)[16], int j) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = min(j * BC + 16 * g + i, a.Nk - 1);
      vr[i] = load16(vp + (int64_t)key * a.vs2 + 8 * n);
    }
  };
  char* vs = Vs[w];
  // O^T += V^T P^T with V^T read transposed from the wave's slice: key chunk cc,
  // feature block db; lane group g reads keys 32cc + 4g + (n>>2) (and +16),
  // features 16db + 4(n&3)
  auto pv = [&](f32x4_t (&o)[D / 16], const bf16x8_t (&pb)[2]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4_t va[D / 16];
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int r0 = 32 * cc + 4 * g + (n >> 2);
        const int dv0 = 16 * db + 4 * (n & 3);
        const int inb = (dv0 & 7) << 1;
        const u32x2_t y0 = ds_read_tr(vs + vswz(r0, dv0 >> 3) + inb);
        const u32x2_t y1 = ds_read_tr(vs + vswz(r0 + 16, dv0 >> 3) + inb);
        va[db] = (u32x4_t){y0[0], y0[1], y1[0], y1[1]};
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db] = mfma16x16x32(as_bf16x8(va[db]), pb[cc], o[db]);
    }
  };

  f32x4_t o[D / 16];  // O^T[dv = 16db + 4g + i][head n], relative to mw
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float Mg = kNegInf;  // global running max of head n over all tiles decided so far
  float mw = kNegInf;  // this wave's accumulation max for head n
  float lw = 0.f;      // this lane's partial row sum
  int kept = 0, vtiles = 0;
  // the previous round's P.V, deferred
  bool pend = false;
  float alpha_p = 1.f;
  bf16x8_t pb_p[2];
  u32x4_t vr[16];
  const int nrounds = (nkt + NW - 1) / NW;

  u32x4_t ka[4][D / 32], kn_[4][D / 32];
  load_k(ka, min(w, nkt - 1));

  int r = 0;
  // one round; kc holds this round's K tile, kn receives the next round's
  auto round = [&](u32x4_t (&kc)[4][D / 32], u32x4_t (&kn)[4][D / 32]) {
    const int j = r * NW + w;
    const bool active = j < nkt;
    const int c0 = j * BC;
    load_k(kn, min(j + NW, nkt - 1));  // every round, so the wait for kc stays precise
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) s[kb] = mfma16x16x32(as_bf16x8(kc[kb][kk]), qb[kk], s[kb]);
    }
    if (c0 + BC > a.Nk) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + 16 * kb + 4 * g + i >= a.Nk) s[kb][i] = kNegInf;
    }
    float tm = kNegInf;
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        tm = fmaxf(tm, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
      tm = fmaxf(tm, shfl_xor_f(tm, 16));
      tm = fmaxf(tm, shfl_xor_f(tm, 32));
    }
    if (g == 0) tmx[r & 1][w][n] = tm;
    __syncthreads();
    float pre = Mg, Mnew = Mg;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const float v = tmx[r & 1][x][n];
      if (x < w) pre = fmaxf(pre, v);
      Mnew = fmaxf(Mnew, v);
    }
    Mg = Mnew;

    // the previous round's P.V (its V had this whole round to land)
    if (pend) {
#pragma unroll
      for (int i = 0; i < 16; ++i) store16(vs + vswz(16 * g + i, n), vr[i]);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db] *= alpha_p;
      pv(o, pb_p);
      pend = false;
    }
    if (active) {
      float gap;
      if (tm == kNegInf) gap = kNegInf;
      else if (pre == kNegInf) gap = __builtin_inff();
      else gap = tm - pre;
      const bool keep = hvalid && ((j == 0) || !(gap < a.thr_raw));
      if (a.mask && g == 0 && hvalid) a.mask[((int64_t)b * a.Hq + hq) * nkt + j] = keep ? 1 : 0;
      kept += keep ? 1 : 0;
      if (__any(keep)) {
        ++vtiles;
        load_v(vr, j);  // V only for a tile some head keeps
        // P_j against this wave's accumulation max; the output rescale is
        // applied together with the deferred P.V
        float mc = 0.f;
        alpha_p = 1.f;
        if (keep) {
          const float m_new = fmaxf(mw, tm);
          mc = m_new * c2;
          alpha_p = fast_exp2(mw * c2 - mc);
          mw = m_new;
          lw *= alpha_p;
        }
        // P^T in the B-operand layout of chunk cc: keys 32cc + 16(e/4) + 4g + e%4
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          uint32_t pw[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float p0 = 0.f, p1 = 0.f;
            if (keep) {
              p0 = fast_exp2(fmaf(s[2 * cc + (e >> 2)][e & 3], c2, -mc));
              p1 = fast_exp2(fmaf(s[2 * cc + (e >> 2)][(e & 3) + 1], c2, -mc));
            }
            lw += p0 + p1;
            pw[e >> 1] = pack_bf16x2(p0, p1);
          }
          pb_p[cc] = as_bf16x8((u32x4_t){pw[0], pw[1], pw[2], pw[3]});
        }
        pend = true;
      }
    }
    ++r;
  };
  while (r < nrounds) {
    round(ka, kn_);
    if (r >= nrounds) break;
    round(kn_, ka);
  }
  if (pend) {
#pragma unroll
    for (int i = 0; i < 16; ++i) store16(vs + vswz(16 * g + i, n), vr[i]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] *= alpha_p;
    pv(o, pb_p);
  }

  // log-sum-exp merge of the waves' partials
  lw += shfl_xor_f(lw, 16);
  lw += shfl_xor_f(lw, 32);
  __syncthreads();
  float* part = reinterpret_cast<float*>(vs);  // [D][16] outputs, then m[16], l[16]
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(16 * db + 4 * g + i) * 16 + n] = o[db][i];
  if (g == 0) {
    part[D * 16 + n] = mw;
    part[D * 16 + 16 + n] = lw;
    cnt[w][n] = kept;
    if (n == 0) cnt[w][16] = vtiles;
  }
  __syncthreads();
  for (int idx = t; idx < G * D; idx += NT) {
    const int hn = idx / D, dv = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int x = 0; x < NW; ++x) M = fmaxf(M, reinterpret_cast<const float*>(Vs[x])[D * 16 + hn]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const float* px = reinterpret_cast<const float*>(Vs[x]);
      const float wgt = fast_exp2((px[D * 16 + hn] - M) * c2);
      L += px[D * 16 + 16 + hn] * wgt;
      acc += px[dv * 16 + hn] * wgt;
    }
    const int hh = kvh * G + hn;
    store_out1(a.out, b * a.os0 + (int64_t)hh * a.os1 + dv, a.out_f32, acc / L);
    if (dv == 0) {
      if (a.lse) a.lse[(int64_t)b * a.Hq + hh] = M * a.scale + logf(L);
      if (a.stats) {
        int kt = 0, vl = 0;
        for (int x = 0; x < NW; ++x) { kt += cnt[x][hn]; vl += cnt[x][16]; }
        int64_t* st = a.stats + ((int64_t)b * a.Hq + hh) * 3;
        st[0] = nkt;
        st[1] = kt;
        st[2] = vl;
      }
    }
  }
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t stream) {
  const int64_t nblocks = (int64_t)a.B * a.Hkv;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_gqa_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
