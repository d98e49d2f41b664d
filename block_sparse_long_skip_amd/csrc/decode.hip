// bf16 skip-softmax decode on gfx950: one query token per (batch, head)
// against a contiguous KV cache with separate values, 64-key tiles (the latent
// cache kernel lives in decode_mla.hip).
//
// Method: BLASST post (seeallochnaya, "BLASST: Dynamic BLocked Attention
// Sparsity via Softmax Thresholding"): key tiles in increasing order, online
// max, a tile dropped whole when its max is far below the running max and its
// V never read (paragraph beginning "BLASST предлагает"), tile 0 always
// processed (first figure); composes with DeepSeek MLA (paragraph on MLA).
// For decode the running max is global along the cache: tile 0 is the cache's
// first tile and the decision for tile j uses the max over all tiles before j.
//
// decode_gqa_kernel (separate V, d = 128, up to 16 query heads per KV head):
//   one workgroup of 8 waves per (batch, KV head). The waves split the keys:
//   in round r wave w takes tile 8r + w. Scores S^T = K q^T come from one
//   16x16x32 MFMA chain per 16 keys, with K loaded straight from HBM into the
//   MFMA operand layout (16-byte loads). The per-head tile maxima of a round
//   are exchanged through LDS, so each wave decides its tile against the exact
//   prefix max of every earlier tile. V is loaded only when some head of the
//   group keeps the tile, transposed into the wave's own LDS slice, and
//   O^T += V^T P^T runs on MFMA. Each wave keeps its own (m, l, O) partial;
//   a log-sum-exp merge across the 8 waves ends the kernel.
//
#include "common.hpp"

namespace blasst {

namespace {
constexpr int BC = 64;
// GQA
constexpr int GD = 128;
constexpr int GNW = 8;
constexpr int GNT = GNW * 64;
constexpr int GVP = BC + 8;  // V^T slice pitch (bf16): 144 B rows
}  // namespace

__global__ void __launch_bounds__(GNT) decode_gqa_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Vt[GNW][GD * GVP];
  __shared__ float tmx[2][GNW][16];
  __shared__ int cnt[GNW][17];

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

  const uint16_t* qp = (const uint16_t*)a.q + b * a.qs0 + (int64_t)hq * a.qs1;
  const uint16_t* kp = (const uint16_t*)a.k + b * a.ks0 + kvh * a.ks1;
  const uint16_t* vp = (const uint16_t*)a.v + b * a.vs0 + kvh * a.vs1;

  bf16x8_t qb[GD / 32];
#pragma unroll
  for (int kk = 0; kk < GD / 32; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (hvalid) v = load16(qp + 32 * kk + 8 * g);
    qb[kk] = as_bf16x8(v);
  }

  f32x4_t o[GD / 16];  // O^T[dv = 16db + 4g + i][head n]
#pragma unroll
  for (int db = 0; db < GD / 16; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float Mg = kNegInf;  // global running max of head n over all tiles decided so far
  float mw = kNegInf;  // this wave's accumulation max for head n
  float lw = 0.f;      // this lane's partial row sum
  int kept = 0, vtiles = 0;
  uint16_t* vt = Vt[w];
  const int nrounds = (a.nkt + GNW - 1) / GNW;

  for (int r = 0; r < nrounds; ++r) {
    const int j = r * GNW + w;
    const bool active = j < a.nkt;
    const int c0 = j * BC;
    f32x4_t s[4];
    float tm = kNegInf;
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        const int key = c0 + 16 * kb + (lane & 15);
        u32x4_t kr[GD / 32];
#pragma unroll
        for (int kk = 0; kk < GD / 32; ++kk) {
          kr[kk] = (u32x4_t){0u, 0u, 0u, 0u};
          if (key < a.Nk) kr[kk] = load16(kp + (int64_t)key * a.ks2 + 32 * kk + 8 * g);
        }
#pragma unroll
        for (int kk = 0; kk < GD / 32; ++kk) s[kb] = mfma16x16x32(as_bf16x8(kr[kk]), qb[kk], s[kb]);
      }
      if (c0 + BC > a.Nk) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c0 + 16 * kb + 4 * g + i >= a.Nk) s[kb][i] = kNegInf;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tm = fmaxf(tm, s[kb][i]);
      tm = fmaxf(tm, shfl_xor_f(tm, 16));
      tm = fmaxf(tm, shfl_xor_f(tm, 32));
    }
    if (g == 0) tmx[r & 1][w][n] = tm;
    __syncthreads();
    float pre = Mg, Mnew = Mg;
#pragma unroll
    for (int x = 0; x < GNW; ++x) {
      const float v = tmx[r & 1][x][n];
      if (x < w) pre = fmaxf(pre, v);
      Mnew = fmaxf(Mnew, v);
    }
    Mg = Mnew;

    if (active) {
      float gap;
      if (tm == kNegInf) gap = kNegInf;
      else if (pre == kNegInf) gap = __builtin_inff();
      else gap = tm - pre;
      const bool keep = hvalid && ((j == 0) || !(gap < a.thr_raw));
      if (a.mask && g == 0 && hvalid) a.mask[((int64_t)b * a.Hq + hq) * a.nkt + j] = keep ? 1 : 0;
      kept += keep ? 1 : 0;
      if (__any(keep)) {
        ++vtiles;
        // V tile (only now): lane loads keys 16g'+i (i = 0..15) of dv chunk (lane&15)
        {
          const int cd = (lane & 15) * 8, kg = 16 * (lane >> 4);
          u32x4_t vr[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = c0 + kg + i;
            vr[i] = (u32x4_t){0u, 0u, 0u, 0u};
            if (key < a.Nk) vr[i] = load16(vp + (int64_t)key * a.vs2 + cd);
          }
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            u32x4_t lo0 = {pack_lo16(vr[0][p], vr[1][p]), pack_lo16(vr[2][p], vr[3][p]),
                           pack_lo16(vr[4][p], vr[5][p]), pack_lo16(vr[6][p], vr[7][p])};
            u32x4_t lo1 = {pack_lo16(vr[8][p], vr[9][p]), pack_lo16(vr[10][p], vr[11][p]),
                           pack_lo16(vr[12][p], vr[13][p]), pack_lo16(vr[14][p], vr[15][p])};
            u32x4_t hi0 = {pack_hi16(vr[0][p], vr[1][p]), pack_hi16(vr[2][p], vr[3][p]),
                           pack_hi16(vr[4][p], vr[5][p]), pack_hi16(vr[6][p], vr[7][p])};
            u32x4_t hi1 = {pack_hi16(vr[8][p], vr[9][p]), pack_hi16(vr[10][p], vr[11][p]),
                           pack_hi16(vr[12][p], vr[13][p]), pack_hi16(vr[14][p], vr[15][p])};
            store16(&vt[(cd + 2 * p) * GVP + kg], lo0);
            store16(&vt[(cd + 2 * p) * GVP + kg + 8], lo1);
            store16(&vt[(cd + 2 * p + 1) * GVP + kg], hi0);
            store16(&vt[(cd + 2 * p + 1) * GVP + kg + 8], hi1);
          }
        }
        float mc = 0.f;
        if (keep) {
          const float m_new = fmaxf(mw, tm);
          mc = m_new * a.scale_log2;
          const float alpha = fast_exp2(mw * a.scale_log2 - mc);
          mw = m_new;
          lw *= alpha;
#pragma unroll
          for (int db = 0; db < GD / 16; ++db) o[db] *= alpha;
        }
        // P^T in the B-operand layout of chunk cc: keys 32cc + 16(e/4) + 4g + e%4
        bf16x8_t pb[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          uint32_t pw[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float p0 = 0.f, p1 = 0.f;
            if (keep) {
              p0 = fast_exp2(fmaf(s[2 * cc + (e >> 2)][e & 3], a.scale_log2, -mc));
              p1 = fast_exp2(fmaf(s[2 * cc + (e >> 2)][(e & 3) + 1], a.scale_log2, -mc));
            }
            lw += p0 + p1;
            pw[e >> 1] = pack_bf16x2(p0, p1);
          }
          pb[cc] = as_bf16x8((u32x4_t){pw[0], pw[1], pw[2], pw[3]});
        }
        __threadfence_block();  // this wave's V^T slice is written
#pragma unroll
        for (int db = 0; db < GD / 16; ++db) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const uint16_t* row = &vt[(16 * db + (lane & 15)) * GVP + 32 * cc + 4 * g];
            u32x2_t x0 = *(const u32x2_t*)row;
            u32x2_t x1 = *(const u32x2_t*)(row + 16);
            o[db] = mfma16x16x32(as_bf16x8((u32x4_t){x0[0], x0[1], x1[0], x1[1]}), pb[cc], o[db]);
          }
        }
        __threadfence_block();  // reads done before the next round rewrites the slice
      }
    }
  }

  // log-sum-exp merge of the 8 waves' partials
  lw += shfl_xor_f(lw, 16);
  lw += shfl_xor_f(lw, 32);
  __syncthreads();
  float* part = reinterpret_cast<float*>(vt);  // [GD][16] outputs, then m[16], l[16]
#pragma unroll
  for (int db = 0; db < GD / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(16 * db + 4 * g + i) * 16 + n] = o[db][i];
  if (g == 0) {
    part[GD * 16 + n] = mw;
    part[GD * 16 + 16 + n] = lw;
    cnt[w][n] = kept;
    if (n == 0) cnt[w][16] = vtiles;
  }
  __syncthreads();
  for (int idx = t; idx < G * GD; idx += GNT) {
    const int hn = idx / GD, dv = idx % GD;
    float M = kNegInf;
#pragma unroll
    for (int x = 0; x < GNW; ++x) M = fmaxf(M, reinterpret_cast<const float*>(Vt[x])[GD * 16 + hn]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int x = 0; x < GNW; ++x) {
      const float* px = reinterpret_cast<const float*>(Vt[x]);
      const float wgt = fast_exp2((px[GD * 16 + hn] - M) * a.scale_log2);
      L += px[GD * 16 + 16 + hn] * wgt;
      acc += px[dv * 16 + hn] * wgt;
    }
    const int hh = kvh * G + hn;
    store_out1(a.out, b * a.os0 + (int64_t)hh * a.os1 + dv, a.out_f32, acc / L);
    if (dv == 0) {
      if (a.lse) a.lse[(int64_t)b * a.Hq + hh] = M * a.scale + logf(L);
      if (a.stats) {
        int kt = 0, vl = 0;
        for (int x = 0; x < GNW; ++x) { kt += cnt[x][hn]; vl += cnt[x][16]; }
        int64_t* st = a.stats + ((int64_t)b * a.Hq + hh) * 3;
        st[0] = a.nkt;
        st[1] = kt;
        st[2] = vl;
      }
    }
  }
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t stream) {
  const int64_t nblocks = (int64_t)a.B * a.Hkv;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_gqa_kernel, dim3((unsigned)nblocks), dim3(GNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
