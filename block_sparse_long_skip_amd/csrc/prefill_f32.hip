// fp32 skip-softmax prefill, d_qk = d_v = 64, 64x64 tiles (gfx950, VALU).
//
// Method: BLASST post (seeallochnaya, "BLASST: Dynamic BLocked Attention
// Sparsity via Softmax Thresholding"): key tiles visited left to right
// (paragraph "В чём идея"), online max with rescale (paragraph on
// FlashAttention 1), a tile dropped whole when its max is far below the running
// max, its V never read (paragraph beginning "BLASST предлагает"), tile 0
// always processed (first figure).
//
// One workgroup of 256 threads per (batch, query head, query tile). Lane l of
// every wave owns query row l of the tile; wave w owns key columns
// [16w, 16w+16) of each key tile. Each wave therefore sees every row, so the
// tile vote is a plain wave ballot; the four waves share the running max (the
// row max of a tile is combined through LDS) and keep separate partial row
// sums and outputs, summed once at the end.
//
// Scores q.k are accumulated in fp64 and the running max is kept in fp64, so
// large logits (strongly peaked attention) lose no precision before the
// exponent; P.V and the row sums accumulate in fp32.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int D = 64;
constexpr int BR = 64;
constexpr int BC = 64;
constexpr int NT = 256;
}  // namespace

__global__ void __launch_bounds__(NT) prefill_f32_kernel(PrefillArgs a) {
  __shared__ float smem[2 * BC * D];
  __shared__ double red[4][BR];
  float (*Ks)[D] = reinterpret_cast<float (*)[D]>(smem);
  float (*Vs)[D] = reinterpret_cast<float (*)[D]>(smem + BC * D);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int nbh = a.B * a.Hq;
  // heaviest (last) query tiles first under causal masking
  const int i = a.nqt - 1 - (int)(blockIdx.x / nbh);
  const int bh = (int)(blockIdx.x % nbh);
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / (a.Hq / a.Hkv);

  const float* qp = (const float*)a.q + b * a.qs0 + hq * a.qs1;
  const float* kp = (const float*)a.k + b * a.ks0 + kvh * a.ks1;
  const float* vp = (const float*)a.v + b * a.vs0 + kvh * a.vs1;

  const int row = i * BR + lane;
  const bool valid = row < a.Nq;
  const int qpos = row + (a.Nk - a.Nq);  // key position of this query
  // last visited key tile: the tile holding the largest visible key of the tile's last row
  const int last_row = min(i * BR + BR - 1, a.Nq - 1);
  const int J = a.causal ? min(a.nkt, (last_row + a.Nk - a.Nq) / BC + 1) : a.nkt;

  float q[D];
  if (valid) {
    const f32x4_t* q4 = (const f32x4_t*)(qp + (int64_t)row * a.qs2);
#pragma unroll
    for (int x = 0; x < D / 4; ++x) {
      f32x4_t v = q4[x];
      q[4 * x] = v[0]; q[4 * x + 1] = v[1]; q[4 * x + 2] = v[2]; q[4 * x + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int x = 0; x < D; ++x) q[x] = 0.f;
  }

  float o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) o[x] = 0.f;
  double m = -__builtin_inf();
  float l = 0.f;
  int kept = 0;
  uint8_t* mrow = a.mask ? a.mask + ((int64_t)bh * a.nqt + i) * a.nkt : nullptr;

  for (int j = 0; j < J; ++j) {
    const int c0 = j * BC;
    __syncthreads();  // previous tile's LDS reads are done
    // K tile -> LDS: 64 rows x 16 float4, 4 per thread, zero past Nk
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int idx = t + r * NT;
      const int kr = idx >> 4, kc = (idx & 15) * 4;
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (c0 + kr < a.Nk) v = *(const f32x4_t*)(kp + (int64_t)(c0 + kr) * a.ks2 + kc);
      *(f32x4_t*)&Ks[kr][kc] = v;
    }
    __syncthreads();

    double s[16];
    double pm = -__builtin_inf();
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) {
      const int col = c0 + 16 * w + cc;
      double acc = 0.0;
#pragma unroll
      for (int x = 0; x < D; x += 4) {
        f32x4_t kv = *(const f32x4_t*)&Ks[16 * w + cc][x];
        acc = fma((double)q[x], (double)kv[0], acc);
        acc = fma((double)q[x + 1], (double)kv[1], acc);
        acc = fma((double)q[x + 2], (double)kv[2], acc);
        acc = fma((double)q[x + 3], (double)kv[3], acc);
      }
      const bool vis = col < a.Nk && (!a.causal || col <= qpos);
      s[cc] = vis ? acc : -__builtin_inf();
      pm = fmax(pm, s[cc]);
    }
    red[w][lane] = pm;
    __syncthreads();
    const double mt = fmax(fmax(red[0][lane], red[1][lane]), fmax(red[2][lane], red[3][lane]));

    // tile vote: drop only if every valid row's gap is below the threshold
    double gap;
    if (mt == -__builtin_inf()) gap = -__builtin_inf();
    else if (m == -__builtin_inf()) gap = __builtin_inf();
    else gap = mt - m;
    const bool lane_keep = valid && !(gap < (double)a.thr_raw);
    const bool keep = (j == 0) || __any(lane_keep);

    if (keep) {
      // V is read only for kept tiles
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int idx = t + r * NT;
        const int vr = idx >> 4, vc = (idx & 15) * 4;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (c0 + vr < a.Nk) v = *(const f32x4_t*)(vp + (int64_t)(c0 + vr) * a.vs2 + vc);
        *(f32x4_t*)&Vs[vr][vc] = v;
      }
      __syncthreads();
      const double m_new = fmax(m, mt);
      const double mref = (m_new == -__builtin_inf()) ? 0.0 : m_new;
      const double sl2 = (double)a.scale * 1.4426950408889634;
      const float alpha = fast_exp2((float)((m - mref) * sl2));
      l *= alpha;
#pragma unroll
      for (int x = 0; x < D; ++x) o[x] *= alpha;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const float p = fast_exp2((float)((s[cc] - mref) * sl2));
        l += p;
#pragma unroll
        for (int x = 0; x < D; x += 4) {
          f32x4_t vv = *(const f32x4_t*)&Vs[16 * w + cc][x];
          o[x] = fmaf(p, vv[0], o[x]);
          o[x + 1] = fmaf(p, vv[1], o[x + 1]);
          o[x + 2] = fmaf(p, vv[2], o[x + 2]);
          o[x + 3] = fmaf(p, vv[3], o[x + 3]);
        }
      }
      m = m_new;
      ++kept;
    }
    if (mrow && t == 0) mrow[j] = keep ? 1 : 0;
  }
  if (mrow) {
    for (int j = J + t; j < a.nkt; j += NT) mrow[j] = 2;
  }

  // combine the four waves' partial sums (same running max in every wave)
  __syncthreads();
  __syncthreads();
  float* acc = smem;  // reuse LDS: [64 rows][D + 1], padded against bank conflicts
  red[w][lane] = (double)l;
  for (int src = 1; src < 4; ++src) {
    if (w == src) {
#pragma unroll
      for (int x = 0; x < D; ++x) acc[lane * (D + 1) + x] = o[x];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int x = 0; x < D; ++x) o[x] += acc[lane * (D + 1) + x];
    }
    __syncthreads();
  }
  if (w == 0) {
    const double lt = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    if (valid) {
      const float inv = (float)(1.0 / lt);
      float* op = (float*)a.out + b * a.os0 + hq * a.os1 + (int64_t)row * a.os2;
#pragma unroll
      for (int x = 0; x < D; x += 4) {
        f32x4_t v = {o[x] * inv, o[x + 1] * inv, o[x + 2] * inv, o[x + 3] * inv};
        *(f32x4_t*)(op + x) = v;
      }
      if (a.lse) a.lse[(int64_t)bh * a.Nq + row] = (float)(m * (double)a.scale + log(lt));
    }
    if (a.stats && lane == 0) {
      atomicAdd((unsigned long long*)&a.stats[2 * bh], (unsigned long long)J);
      atomicAdd((unsigned long long*)&a.stats[2 * bh + 1], (unsigned long long)kept);
    }
  }
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t nblocks = (int64_t)a.B * a.Hq * a.nqt;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_f32_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
