// Two-pass skip-softmax prefill on gfx950: an MXFP4 max pre-pass fixes the
// tile map, then exact attention runs over the kept tiles.
//
// Method: a reply in the digg thread "BLASST wins Best Paper at MLSys 2026 ..."
// suggests recomputing q.k in 4-bit only to find the maxima (the first pass
// needs no exponentials), fixing the sparsity map from them, and then gathering
// the kept blocks for the real computation. Here "4-bit" is MXFP4 from the OCP
// Microscaling Formats (MX) Specification v1.0 (FP4 E2M1 elements, one E8M0
// power-of-two scale per 32 consecutive features), the element format gfx950's
// scaled matrix instructions take natively. The map is the skip rule on those
// scores; the second pass is the block-sparse prefill kernel with lambda = 0
// and the kept tiles as its set (launched by the C ABI).
//
//   mx_quantize_fp4_kernel  one thread per block of 32 features: the block's
//                           shared exponent floor(log2 max|x|) - 2 (clamped to
//                           [-127, 127]), each element x / 2^shared rounded to
//                           E2M1 (nearest, ties to the even code, clamped at 6),
//                           the sign copied; 16 code bytes and one scale byte.
//   twopass_map_kernel      one workgroup of 4 waves per (batch, query head,
//                           128-row query tile), wave w owning rows 32w..32w+31.
//                           S^T = K Q^T per 64-key tile on two scaled
//                           32x32x64 FP4 MFMAs per 32-key half (lane = query
//                           row, as in the bf16 prefill), K codes loaded from
//                           global memory one tile ahead. The running max of a
//                           row is the prefix max of all earlier tile maxima (a
//                           dropped tile cannot raise it when lambda <= 1), so
//                           waves sweep independently and only OR their votes
//                           into an LDS byte per tile; the map row is written
//                           after one barrier.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int NT = 256;
constexpr int BR = 128;  // query tile
constexpr int BC = 64;   // key tile
constexpr int ROWB = 64; // code bytes per row (d = 128)
constexpr int TPS = 4;   // key tiles per LDS stage of the map kernel
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// E2M1 code (magnitude index 0..7) of a >= 0: nearest of 0, .5, 1, 1.5, 2, 3,
// 4, 6, ties to the even code, values above 6 clamped. The spacing is 0.5
// below 2, 1 in [2, 4) and 2 above; rint rounds half to even and the
// products by powers of two are exact.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  const float inv = a >= 4.f ? 0.5f : (a >= 2.f ? 1.f : 2.f);
  const float q = fminf(rintf(a * inv) * (1.f / inv), 6.f);
  return q < 2.f ? (uint32_t)(q * 2.f) : (q < 4.f ? 4u + (uint32_t)(q - 2.f) : (q < 6.f ? 6u : 7u));
}

// floor(log2 a) for finite a > 0, subnormals included
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t bits = __float_as_uint(a);
  const int ef = (int)(bits >> 23);
  return ef != 0 ? ef - 127 : (31 - __clz((int)bits)) - 149;
}

// chunk swizzle of key row r in the LDS stage
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 3; }

__device__ __forceinline__ i32x8_t operand(const u32x4_t& v) {
  return (i32x8_t){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}

// D += A B with FP4 operands (first 16 bytes of each lane's 32) and E8M0
// scales taken from byte 0 of sa / sb.
__device__ __forceinline__ f32x16_t mfma_fp4(const i32x8_t& a, int sa, const i32x8_t& b, int sb,
                                             const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
}  // namespace

__global__ void __launch_bounds__(NT) mx_quantize_fp4_kernel(MxQuantArgs a) {
  const int nb = a.d >> 5;
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t nrows = (int64_t)a.d0 * a.d1 * a.n;
  if (gid >= nrows * nb) return;
  const int64_t row = gid / nb;
  const int blk = (int)(gid % nb);
  const int64_t i01 = row / a.n;
  const int64_t pos = row % a.n;
  const int64_t i0 = i01 / a.d1, i1 = i01 % a.d1;
  const uint16_t* src = (const uint16_t*)a.x + i0 * a.s0 + i1 * a.s1 + pos * a.s2 + 32 * blk;
  u32x4_t w[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = load16(src + 8 * c);
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[c][e])), fabsf(bf16_hi(w[c][e]))));
  const int shared = amax == 0.f ? -127 : min(max(floor_log2(amax) - 2, -127), 127);
  const float mul = __uint_as_float((uint32_t)(127 - shared) << 23);  // 2^-shared, a normal float
  u32x4_t packed;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = w[c][e];  // features 8c + 2e (low half) and 8c + 2e + 1
      const uint32_t lo = e2m1_code(fabsf(bf16_lo(x)) * mul) | ((x >> 12) & 8u);
      const uint32_t hi = e2m1_code(fabsf(bf16_hi(x)) * mul) | ((x >> 28) & 8u);
      word |= (lo | (hi << 4)) << (8 * e);
    }
    packed[c] = word;
  }
  store16(a.codes + row * (a.d >> 1) + 16 * blk, packed);
  a.scales[row * nb + blk] = (uint8_t)(shared + 127);
}

__global__ void __launch_bounds__(NT) twopass_map_kernel(TwoPassMapArgs a) {
  // K codes and scales of TPS consecutive key tiles per stage, two stages.
  // Codes of key r (64 bytes, four 16-byte chunks) sit at r * 64 with chunk c
  // stored at position c ^ swz(r), so the 16-byte operand reads of 8
  // consecutive keys fall in distinct banks.
  __shared__ __attribute__((aligned(16))) char kbuf[2][TPS][BC * ROWB];
  __shared__ __attribute__((aligned(16))) uint32_t sbuf[2][TPS][BC];
  __shared__ uint8_t flag[kPrefillMaxSetTiles];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // block -> (query tile, head), as in the bf16 prefill: heaviest query tiles
  // first, heads of one KV group on one XCD when the head count allows
  const int nbh = a.B * a.Hq;
  const int i = a.nqt - 1 - (int)(blockIdx.x / nbh);
  int bh = (int)(blockIdx.x % nbh);
  if ((nbh & 7) == 0) bh = (bh & 7) * (nbh >> 3) + (bh >> 3);
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / (a.Hq / a.Hkv);

  const int row = i * BR + 32 * w + l32;
  const bool valid = row < a.Nq;
  const int qpos = row + (a.Nk - a.Nq);
  const int last_row = min(i * BR + BR - 1, a.Nq - 1);
  const int first_pos = i * BR + (a.Nk - a.Nq);
  const int J = a.causal ? min(a.nkt, (last_row + a.Nk - a.Nq) / BC + 1) : a.nkt;
  const int nstage = (J + TPS - 1) / TPS;

  for (int x = t; x < J; x += NT) flag[x] = 0;

  // Q^T as the B operand: lane (row, h) supplies features 64kk + 32h .. +31,
  // i.e. code bytes 32kk + 16h .. +15, with the scale of feature block 2kk + h
  const int64_t qrow = (int64_t)bh * a.Nq + min(row, a.Nq - 1);
  const uint8_t* qp = a.qc + qrow * ROWB;
  const i32x8_t qb0 = operand(load16(qp + 16 * h));
  const i32x8_t qb1 = operand(load16(qp + 32 + 16 * h));
  const uint32_t qsw = *(const uint32_t*)(a.qs + qrow * 4);
  const int qs0 = (int)((qsw >> (8 * h)) & 0xffu);
  const int qs1 = (int)((qsw >> (16 + 8 * h)) & 0xffu);

  const int64_t kbase = (int64_t)(b * a.Hkv + kvh) * a.Nk;
  const uint8_t* kc = a.kc + kbase * ROWB;
  const uint8_t* ks = a.ks + kbase * 4;

  // Copies of stage st into buffer st & 1: wave w moves the codes of keys
  // 16w .. 16w + 15 of each tile (lane -> key 16w + lane / 4, physical chunk
  // lane % 4, fetching the logical chunk stored there); wave (tile % 4) moves
  // that tile's 64 scale words. Keys past Nk repeat the last key.
  const int ckey = 16 * w + (lane >> 2);
  const int cchunk = (lane & 3) ^ swz_k(ckey);
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int buf = st & 1;
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int j = st * TPS + u;
      if (j < J) {
        const int key = min(j * BC + ckey, a.Nk - 1);
        lds_dma16(kc + (int64_t)key * ROWB + 16 * cchunk, &kbuf[buf][u][w * 1024]);
        if (w == (u & 3)) {
          const int skey = min(j * BC + lane, a.Nk - 1);
          __builtin_amdgcn_global_load_lds(ks + (int64_t)skey * 4,
                                           (__attribute__((address_space(3))) void*)&sbuf[buf][u][0],
                                           4, 0, 0);
        }
      }
    }
  };

  // operand reads of key half kb: key 32kb + l32, logical chunks h and 2 + h
  int aoff[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = 32 * kb + l32;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) aoff[kb][kk] = key * ROWB + 16 * ((2 * kk + h) ^ swz_k(key));
  }

  // S^T of tile u of the stage in buffer buf: keys 32kb + 8(r/4) + 4h + r%4
  // of the tile in register r of s[kb], this lane's row in its column
  auto scores = [&](int buf, int u, f32x16_t (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t sw = sbuf[buf][u][32 * kb + l32];
      const int ks0 = (int)((sw >> (8 * h)) & 0xffu);
      const int ks1 = (int)((sw >> (16 + 8 * h)) & 0xffu);
      const u32x4_t k0 = *(const u32x4_t*)&kbuf[buf][u][aoff[kb][0]];
      const u32x4_t k1 = *(const u32x4_t*)&kbuf[buf][u][aoff[kb][1]];
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      acc = mfma_fp4(operand(k0), ks0, qb0, qs0, acc);
      s[kb] = mfma_fp4(operand(k1), ks1, qb1, qs1, acc);
    }
  };

  float m = kNegInf;  // prefix max of this row's tile maxima (raw q.k units)
  // tile j: row max over visible keys, the row's vote, the workgroup flag
  auto decide = [&](int j, f32x16_t (&s)[2]) __attribute__((always_inline)) {
    const int c0 = j * BC;
    if (c0 + BC > a.Nk || (a.causal && c0 + BC - 1 > first_pos)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = c0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (col >= a.Nk || (a.causal && col > qpos)) s[kb][r] = kNegInf;
        }
    }
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(fmaxf(mt, s[0][r]), s[1][r]);
    mt = max_with_lane_xor32(mt);
    // keep unless the gap is below the threshold; a row with no visible key
    // has gap -inf, and a row with no running max yet has gap +inf (mt - m
    // is +inf when m = -inf and mt is finite; no NaN can arise)
    const float gap = mt == kNegInf ? kNegInf : mt - m;
    const bool keep = valid && !(gap < a.thr_raw);
    if (__ballot(keep) != 0ull && lane == 0) flag[j] = 1;
    m = fmaxf(m, mt);
  };

  issue(0);
  for (int st = 0; st < nstage; ++st) {
    wait_vmem();
    __syncthreads();  // stage st landed; every wave is done with stage st - 1
    if (st + 1 < nstage) issue(st + 1);
    const int buf = st & 1;
    const int j0 = st * TPS;
    // the next tile's MFMAs are issued before this tile's reduction
    f32x16_t sa[2], sb[2];
    scores(buf, 0, sa);
#pragma unroll
    for (int u = 0; u < TPS; u += 2) {
      if (j0 + u >= J) break;
      if (j0 + u + 1 < J) scores(buf, u + 1, sb);
      decide(j0 + u, sa);
      if (j0 + u + 1 >= J) break;
      if (u + 2 < TPS && j0 + u + 2 < J) scores(buf, u + 2, sa);
      decide(j0 + u + 1, sb);
    }
  }
  __syncthreads();

  // the map row: tile 0 always kept, tiles past the causal bound not visited
  uint8_t* mrow = a.map + ((int64_t)bh * a.nqt + i) * a.nkt;
  int kept = 0;
  for (int x = t; x < a.nkt; x += NT) {
    const uint8_t v = x >= J ? 2 : ((x == 0 || flag[x]) ? 1 : 0);
    mrow[x] = v;
    kept += v == 1;
  }
  if (a.stats) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kept += __shfl_xor(kept, o, 64);
    if (lane == 0) {
      atomicAdd((unsigned long long*)&a.stats[2 * bh + 1], (unsigned long long)kept);
      if (w == 0) atomicAdd((unsigned long long*)&a.stats[2 * bh], (unsigned long long)J);
    }
  }
}

hipError_t launch_mx_quantize_fp4(const MxQuantArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.d0 * a.d1 * a.n * (a.d >> 5);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_fp4_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_twopass_map(const TwoPassMapArgs& a, hipStream_t stream) {
  const int64_t nblocks = (int64_t)a.B * a.Hq * a.nqt;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(twopass_map_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
