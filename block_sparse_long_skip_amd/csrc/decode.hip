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
//
// Few sequences (batch x KV heads below half the CU count): one workgroup per
// (batch, KV head) would leave most CUs idle, so the cache is split along its
// length over workgroups, with exact decisions and no speculation:
//   pass 1 (scores): each split computes S^T = K q^T for its tiles (the K
//     bytes, read once) and stores the fp32 scores, every tile max and the
//     split's maximum in the workspace (64 G floats per tile against the
//     tile's 16 KB of K);
//   pass 2 (accumulate): each split starts its running max from the maxima of
//     the earlier splits, which is the exact prefix max at its first tile, and
//     runs the same round loop on the stored scores: exact decisions, V read
//     only for kept tiles, P.V, a log-sum-exp merge of its waves; its partial
//     (m, l, O) goes to the workspace;
//   merge: a log-sum-exp merge of the split partials of each (batch, head).
#include "common.hpp"

namespace blasst {

namespace {
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
constexpr int BC = 64;
constexpr int D = 128;
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int SLICE = BC * D * 2;  // 16 KB: one V tile, 64 rows x 256 B
constexpr int kGqaSplitBlocks = 256;  // workgroups a split decode aims for


// 16-byte chunk c of row r of a 64 x 256 B tile, chunk index XOR-swizzled by the row
__device__ __forceinline__ int vswz(int r, int c) {
  return r * 256 + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4);
}
}  // namespace

// Workspace of a split decode (carved from the caller's buffer).
struct GqaSplit {
  float* sc;       // [units][nkt][G][64]  scores (raw q.k units), lane order (kb, g, i)
  float* smax;     // [units][nsplit][G]   maximum of each split's tile maxima
  float* part_o;   // [B*Hq][nsplit][128]  the split's output (normalised by its l)
  float* part_ml;  // [B*Hq][nsplit][2]    the split's (max, row sum); l = 0: nothing kept
  int* part_kept;  // [B*Hq][nsplit]       kept tiles
  int* part_vt;    // [units][nsplit]      V tiles read
  int nsplit, T;
};

// MODE 0: the whole cache per workgroup; 1: split, scores only; 2: split,
// exact decisions and accumulation on the stored scores
template <int MODE>
__global__ void __launch_bounds__(NT, 1) decode_gqa_kernel(DecodeArgs a, GqaSplit sp) {
  __shared__ __attribute__((aligned(16))) char Vs[NW][SLICE];
  __shared__ float tmx[2][NW][16];
  __shared__ int cnt[NW][17];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int n = lane & 15;  // head within the group (B/C operand column)
  const int g = lane >> 4;  // 0..3
  const int units = a.B * a.Hkv;
  const int unit = MODE == 0 ? (int)blockIdx.x : (int)blockIdx.x % units;
  const int split = MODE == 0 ? 0 : (int)blockIdx.x / units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int G = a.G;
  const bool hvalid = n < G;
  const int hq = kvh * G + n;
  const int nkt = a.nkt;
  const float c2 = a.scale_log2;
  const int j0 = MODE == 0 ? 0 : split * sp.T;             // this workgroup's tiles
  const int j1 = MODE == 0 ? nkt : min(j0 + sp.T, nkt);
  // stored scores of (tile j, head n): 64 floats, this lane's 16 at (kb, g)
  auto sc_at = [&](int j) { return sp.sc + (((int64_t)unit * nkt + j) * G + n) * 64 + 4 * g; };

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
  const int nrounds = (j1 - j0 + NW - 1) / NW;

  if constexpr (MODE == 2) {
    // the exact running max entering the split: the maxima of the earlier splits
    if (hvalid)
      for (int x = 0; x < split; ++x) Mg = fmaxf(Mg, sp.smax[((int64_t)unit * sp.nsplit + x) * G + n]);
  }
  float smx = kNegInf;  // pass 1: this lane's maximum over its tiles

  u32x4_t ka[4][D / 32], kn_[4][D / 32];
  if constexpr (MODE != 2) load_k(ka, min(j0 + w, j1 - 1));
  // pass 2 reads the stored scores one round ahead instead of K
  f32x4_t sa[4], sn_[4];
  auto load_s = [&](f32x4_t (&sr)[4], int j) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sr[kb] = hvalid ? *(const f32x4_t*)(sc_at(j) + 16 * kb) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
  };
  if constexpr (MODE == 2) load_s(sa, min(j0 + w, j1 - 1));

  int r = 0;
  // one round; kc / scs hold this round's K tile / stored scores, kn / snx
  // receive the next round's
  auto round = [&](u32x4_t (&kc)[4][D / 32], u32x4_t (&kn)[4][D / 32], f32x4_t (&scs)[4],
                   f32x4_t (&snx)[4]) {
    const int j = j0 + r * NW + w;
    const bool active = j < j1;
    const int c0 = j * BC;
    f32x4_t s[4];
    if constexpr (MODE != 2) {
      load_k(kn, min(j + NW, j1 - 1));  // every round, so the wait for kc stays precise
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          s[kb] = mfma16x16x32(as_bf16x8(kc[kb][kk]), qb[kk], s[kb]);
      }
      if (c0 + BC > a.Nk) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c0 + 16 * kb + 4 * g + i >= a.Nk) s[kb][i] = kNegInf;
      }
    } else {
      load_s(snx, min(j + NW, j1 - 1));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = scs[kb];
    }
    float tm = kNegInf;
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        tm = fmaxf(tm, fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3])));
      tm = fmaxf(tm, shfl_xor_f(tm, 16));
      tm = fmaxf(tm, shfl_xor_f(tm, 32));
    }
    if constexpr (MODE == 1) {
      // scores only: store this tile's scores, keep the split's maximum
      if (active && hvalid) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) *(f32x4_t*)(sc_at(j) + 16 * kb) = s[kb];
        smx = fmaxf(smx, tm);
      }
      ++r;
      return;
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
    round(ka, kn_, sa, sn_);
    if (r >= nrounds) break;
    round(kn_, ka, sn_, sa);
  }
  if constexpr (MODE == 1) {
    // the split's maximum per head: over the lanes of a head, then the waves
    if (g == 0) tmx[0][w][n] = smx;
    __syncthreads();
    if (w == 0 && g == 0 && hvalid)
      sp.smax[((int64_t)unit * sp.nsplit + split) * G + n] =
          fmaxf(fmaxf(tmx[0][0][n], tmx[0][1][n]), fmaxf(tmx[0][2][n], tmx[0][3][n]));
    return;
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
    if (M != kNegInf) {  // (a split may keep nothing for a head)
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const float* px = reinterpret_cast<const float*>(Vs[x]);
        const float wgt = fast_exp2((px[D * 16 + hn] - M) * c2);
        L += px[D * 16 + 16 + hn] * wgt;
        acc += px[dv * 16 + hn] * wgt;
      }
    }
    const int hh = kvh * G + hn;
    if constexpr (MODE == 2) {
      const int64_t prow = ((int64_t)b * a.Hq + hh) * sp.nsplit + split;
      sp.part_o[prow * D + dv] = L > 0.f ? acc / L : 0.f;
      if (dv == 0) {
        sp.part_ml[2 * prow] = M;
        sp.part_ml[2 * prow + 1] = L;
        int kt = 0, vl = 0;
        for (int x = 0; x < NW; ++x) { kt += cnt[x][hn]; vl += cnt[x][16]; }
        sp.part_kept[prow] = kt;
        if (hn == 0) sp.part_vt[(int64_t)unit * sp.nsplit + split] = vl;
      }
      continue;
    }
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

// Log-sum-exp merge of the split partials of one (batch, head) per wave, and
// the statistics. 4 rows per block; lane l owns features 2l and 2l + 1.
__global__ void __launch_bounds__(256) decode_gqa_merge_kernel(DecodeArgs a, GqaSplit sp) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(row / a.Hq), hq = (int)(row % a.Hq);
  const int unit = b * a.Hkv + hq / a.G;
  const float c2 = a.scale_log2;
  const float* ml = sp.part_ml + row * sp.nsplit * 2;
  // the splits' (m, l) one per lane, 64 splits at a time; the merged max over
  // the splits that kept something
  float ms = kNegInf;
  for (int x0 = 0; x0 < sp.nsplit; x0 += 64) {
    const int x = x0 + lane;
    if (x < sp.nsplit && ml[2 * x + 1] > 0.f) ms = fmaxf(ms, ml[2 * x]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ms = fmaxf(ms, shfl_xor_f(ms, d));
  // each split's weight l 2^((m - ms) c2) (0 for a split that kept nothing,
  // whose partial output is 0), broadcast from its lane; the partial outputs
  // are read with no branch between them, in split order
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int x0 = 0; x0 < sp.nsplit; x0 += 64) {
    const int x = x0 + lane;
    float wl = 0.f;
    if (x < sp.nsplit) {
      const float l = ml[2 * x + 1];
      if (l > 0.f) wl = l * fast_exp2((ml[2 * x] - ms) * c2);
    }
    const int cnt = min(64, sp.nsplit - x0);
    const float* po = sp.part_o + (row * sp.nsplit + x0) * D + 2 * lane;
    int y = 0;
    for (; y + 8 <= cnt; y += 8) {  // eight loads in flight, then their sums
      f32x2_t v[8];
      float wy[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wy[e] = __shfl(wl, y + e, 64);
        v[e] = *(const f32x2_t*)(po + (int64_t)(y + e) * D);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        L += wy[e];
        o0 += v[e][0] * wy[e];
        o1 += v[e][1] * wy[e];
      }
    }
    for (; y < cnt; ++y) {
      const float wy = __shfl(wl, y, 64);
      const f32x2_t v = *(const f32x2_t*)(po + (int64_t)y * D);
      L += wy;
      o0 += v[0] * wy;
      o1 += v[1] * wy;
    }
  }
  const int64_t ob = b * a.os0 + (int64_t)hq * a.os1 + 2 * lane;
  store_out1(a.out, ob, a.out_f32, o0 / L);
  store_out1(a.out, ob + 1, a.out_f32, o1 / L);
  if (a.lse && lane == 0) a.lse[row] = ms * a.scale + logf(L);
  if (a.stats) {
    int kept = 0, vt = 0;
    for (int x = lane; x < sp.nsplit; x += 64) {
      kept += sp.part_kept[row * sp.nsplit + x];
      vt += sp.part_vt[(int64_t)unit * sp.nsplit + x];
    }
    for (int d = 32; d >= 1; d >>= 1) {
      kept += __shfl_xor(kept, d, 64);
      vt += __shfl_xor(vt, d, 64);
    }
    if (lane == 0) {
      int64_t* st = a.stats + row * 3;
      st[0] = a.nkt;
      st[1] = kept;
      st[2] = vt;
    }
  }
}

namespace {
struct GqaPlan {
  int nsplit, T;  // nsplit = 1: one workgroup per (batch, KV head), no workspace
  size_t off_sc, off_smax, off_o, off_ml, off_kept, off_vt, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split the cache when the (batch, KV head) pairs fill less than half of the
// 256 CUs: about one workgroup per CU in total, whole rounds of 4 tiles per
// split.
GqaPlan gqa_plan(int B, int Hq, int Hkv, int G, int nkt) {
  GqaPlan p{};
  const int64_t units = (int64_t)B * Hkv;
  p.nsplit = 1;
  p.T = nkt;
  if (units > 0 && units < 128) {
    const int64_t want = (kGqaSplitBlocks + units - 1) / units;
    int T = (int)((nkt + want - 1) / want);
    T = (T + NW - 1) / NW * NW;
    const int ns = (nkt + T - 1) / T;
    if (ns > 1) {
      p.nsplit = ns;
      p.T = T;
    }
  }
  if (p.nsplit == 1) return p;
  const size_t rows = (size_t)B * Hq;
  size_t off = 0;
  p.off_sc = off;
  off = align256(off + (size_t)units * nkt * G * 64 * sizeof(float));
  p.off_smax = off;
  off = align256(off + (size_t)units * p.nsplit * G * sizeof(float));
  p.off_o = off;
  off = align256(off + rows * p.nsplit * D * sizeof(float));
  p.off_ml = off;
  off = align256(off + rows * p.nsplit * 2 * sizeof(float));
  p.off_kept = off;
  off = align256(off + rows * p.nsplit * sizeof(int));
  p.off_vt = off;
  off = align256(off + (size_t)units * p.nsplit * sizeof(int));
  p.bytes = off;
  return p;
}
}  // namespace

size_t decode_gqa_workspace_bytes(int B, int Hq, int Hkv, int G, int nkt) {
  return gqa_plan(B, Hq, Hkv, G, nkt).bytes;
}

hipError_t launch_decode_gqa(const DecodeArgs& a, void* workspace, hipStream_t stream) {
  const int64_t units = (int64_t)a.B * a.Hkv;
  if (units == 0) return hipSuccess;
  const GqaPlan p = gqa_plan(a.B, a.Hq, a.Hkv, a.G, a.nkt);
  GqaSplit sp{};
  sp.nsplit = p.nsplit;
  sp.T = p.T;
  if (p.nsplit == 1) {
    hipLaunchKernelGGL(decode_gqa_kernel<0>, dim3((unsigned)units), dim3(NT), 0, stream, a, sp);
    return hipGetLastError();
  }
  char* base = static_cast<char*>(workspace);
  sp.sc = reinterpret_cast<float*>(base + p.off_sc);
  sp.smax = reinterpret_cast<float*>(base + p.off_smax);
  sp.part_o = reinterpret_cast<float*>(base + p.off_o);
  sp.part_ml = reinterpret_cast<float*>(base + p.off_ml);
  sp.part_kept = reinterpret_cast<int*>(base + p.off_kept);
  sp.part_vt = reinterpret_cast<int*>(base + p.off_vt);
  const unsigned nb = (unsigned)(units * p.nsplit);
  hipLaunchKernelGGL(decode_gqa_kernel<1>, dim3(nb), dim3(NT), 0, stream, a, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_gqa_kernel<2>, dim3(nb), dim3(NT), 0, stream, a, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.Hq;
  hipLaunchKernelGGL(decode_gqa_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, a, sp);
  return hipGetLastError();
}

}  // namespace blasst
