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
//                           pair of 128-row query tiles), waves 0-1 on the
//                           first tile and 2-3 on the second, each wave owning
//                           64 rows as two 32-row blocks that share every K
//                           operand read. S^T = K Q^T per 64-key tile on two
//                           scaled 32x32x64 FP4 MFMAs per 32-key half and row
//                           block (lane = query row, as in the bf16 prefill);
//                           K codes and scales are staged in LDS four tiles at
//                           a time, double-buffered. The running max of a row
//                           is the prefix max of all earlier tile maxima (a
//                           dropped tile cannot raise it when lambda <= 1), so
//                           waves sweep independently and only OR their votes
//                           into a bit per tile; the map rows are written after
//                           one barrier.
#include <type_traits>

#include "common.hpp"

namespace blasst {

namespace {
constexpr int NT = 256;
constexpr int BR = 128;  // query tile
constexpr int BC = 64;   // key tile
constexpr int ROWB = 64; // code bytes per row (d = 128)
constexpr int TPS = 4;   // key tiles per LDS stage of the map kernel
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit data format, raw access
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
  // K codes and scales of TPS consecutive key tiles per stage, two stages,
  // each buffer its own LDS array (copies into LDS are tracked per array, so
  // reading one stage does not wait for the copy in flight into the other).
  // Codes of key r (64 bytes, four 16-byte chunks) sit at r * 64 with chunk c
  // stored at position c ^ swz(r), so the 16-byte operand reads of 8
  // consecutive keys fall in distinct banks.
  __shared__ __attribute__((aligned(16))) char kbuf0[TPS][BC * ROWB];
  __shared__ __attribute__((aligned(16))) char kbuf1[TPS][BC * ROWB];
  __shared__ __attribute__((aligned(16))) uint32_t sbuf0[TPS][BC];
  __shared__ __attribute__((aligned(16))) uint32_t sbuf1[TPS][BC];
  // keep flags of the pair's two query tiles, one bit per key tile
  __shared__ uint32_t flagw[2][kPrefillMaxSetTiles / 32];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: the wave's tile and bounds are scalars
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // block -> (query-tile pair, batch, head): units of one (batch, KV head,
  // pair of consecutive query tiles), heaviest pairs first, the G query heads
  // of a unit in G consecutive slots of one XCD (block x runs on XCD x % 8, as
  // its slot x / 8 there); blocks past the last unit return at once
  const int G = a.Hq / a.Hkv;
  const int ngrp = a.B * a.Hkv;
  const int npair = (a.nqt + 1) >> 1;
  const int slot = (int)(blockIdx.x >> 3);
  const int64_t u = (int64_t)(slot / G) * 8 + (blockIdx.x & 7);
  if (u >= (int64_t)ngrp * npair) return;
  const int ip = npair - 1 - (int)(u / ngrp);
  const int grp = (int)(u % ngrp);
  const int b = grp / a.Hkv, kvh = grp % a.Hkv;
  const int hq = kvh * G + slot % G;
  const int bh = b * a.Hq + hq;

  // key tiles visited by query tile qt (all of them when not causal)
  auto visited = [&](int qt) -> int {
    const int last_row = min(qt * BR + BR - 1, a.Nq - 1);
    return a.causal ? min(a.nkt, (last_row + a.Nk - a.Nq) / BC + 1) : a.nkt;
  };
  const int i0 = 2 * ip;                      // the pair's first query tile
  const bool two = i0 + 1 < a.nqt;            // the pair has a second tile
  const int Jt0 = visited(i0);
  const int Jt1 = two ? visited(i0 + 1) : 0;
  const int Jwg = max(Jt0, Jt1);
  const int nstage = (Jwg + TPS - 1) / TPS;

  // this wave: query tile i0 + w / 2, rows 64 (w % 2) .. +63 of it as two
  // 32-row blocks rb, one row per lane column in each
  const int tw = w >> 1;
  const int qi = i0 + tw;
  const bool tile_ok = tw == 0 || two;
  const int Jw = tw == 0 ? Jt0 : Jt1;        // 0 for a missing second tile
  const int first_pos = qi * BR + (a.Nk - a.Nq);
  int row[2], qpos[2];
  bool valid[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    row[rb] = qi * BR + 64 * (w & 1) + 32 * rb + l32;
    valid[rb] = tile_ok && row[rb] < a.Nq;
    qpos[rb] = row[rb] + (a.Nk - a.Nq);
  }

  for (int x = t; x < 2 * (kPrefillMaxSetTiles / 32); x += NT) (&flagw[0][0])[x] = 0u;

  // Q^T as the B operand: lane (row, h) supplies features 64kk + 32h .. +31,
  // i.e. code bytes 32kk + 16h .. +15, with the scale of feature block 2kk + h
  i32x8_t qb0[2], qb1[2];
  int qs0[2], qs1[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t qrow = (int64_t)bh * a.Nq + min(row[rb], a.Nq - 1);
    const uint8_t* qp = a.qc + qrow * ROWB;
    qb0[rb] = operand(load16(qp + 16 * h));
    qb1[rb] = operand(load16(qp + 32 + 16 * h));
    const uint32_t qsw = *(const uint32_t*)(a.qs + qrow * 4);
    qs0[rb] = (int)((qsw >> (8 * h)) & 0xffu);
    qs1[rb] = (int)((qsw >> (16 + 8 * h)) & 0xffu);
  }

  const int64_t kbase = (int64_t)(b * a.Hkv + kvh) * a.Nk;
  const uint8_t* kc = a.kc + kbase * ROWB;
  const uint8_t* ks = a.ks + kbase * 4;

  // Copies of stage st into the buffers of parity st & 1, through a buffer
  // resource per tile whose size stops at Nk (keys past it read as zero codes
  // and are masked in the reduction): wave w moves the codes of keys 16w ..
  // 16w + 15 of each tile (lane -> key 16w + lane / 4, physical chunk lane % 4,
  // fetching the logical chunk stored there); wave (tile % 4) moves that
  // tile's 64 scale words.
  const int ckey = 16 * w + (lane >> 2);
  const int cchunk = (lane & 3) ^ swz_k(ckey);
  const uint32_t kvoff = (uint32_t)(ckey * ROWB + 16 * cchunk);
  const int wu = w;
  // one buffer resource over this KV head's codes and one over its scales;
  // the tile offset goes into the per-lane offset, so the range check covers it
  auto rsrc = [&](const uint8_t* p, int bytes) __attribute__((always_inline)) {
    const uint64_t tb = (uint64_t)p;
    const uint64_t ub =
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tb >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tb);
    return __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
  };
  const __amdgpu_buffer_rsrc_t krs = rsrc(kc, a.Nk * ROWB);
  const __amdgpu_buffer_rsrc_t srs = rsrc(ks, a.Nk * 4);
  auto kbuf_of = [&](auto PAR) -> char (&)[TPS][BC * ROWB] {
    if constexpr (decltype(PAR)::value) return kbuf1; else return kbuf0;
  };
  auto sbuf_of = [&](auto PAR) -> uint32_t (&)[TPS][BC] {
    if constexpr (decltype(PAR)::value) return sbuf1; else return sbuf0;
  };
  auto issue = [&](auto PAR, int st) __attribute__((always_inline)) {
    char (&kbuf)[TPS][BC * ROWB] = kbuf_of(PAR);
    uint32_t (&sbuf)[TPS][BC] = sbuf_of(PAR);
#pragma unroll
    for (int uu = 0; uu < TPS; ++uu) {
      const int j = st * TPS + uu;
      if (j < Jwg) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            krs, (__attribute__((address_space(3))) void*)&kbuf[uu][wu * 1024], 16,
            kvoff + (uint32_t)(j * BC * ROWB), 0, 0, 0);
        if (wu == (uu & 3))
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              srs, (__attribute__((address_space(3))) void*)&sbuf[uu][0], 4,
              (uint32_t)(4 * lane + j * BC * 4), 0, 0, 0);
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

  // S^T of tile uu of a stage for both row blocks: keys 32kb + 8(r/4) + 4h +
  // r%4 of the tile in register r of s[rb][kb], the lane's row of block rb in
  // its column; each K operand read feeds both row blocks
  auto scores = [&](const char (&kbuf)[TPS][BC * ROWB], const uint32_t (&sbuf)[TPS][BC], int uu,
                    f32x16_t (&s)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t sw = sbuf[uu][32 * kb + l32];
      const int ks0 = (int)((sw >> (8 * h)) & 0xffu);
      const int ks1 = (int)((sw >> (16 + 8 * h)) & 0xffu);
      const u32x4_t k0 = *(const u32x4_t*)&kbuf[uu][aoff[kb][0]];
      const u32x4_t k1 = *(const u32x4_t*)&kbuf[uu][aoff[kb][1]];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        acc = mfma_fp4(operand(k0), ks0, qb0[rb], qs0[rb], acc);
        s[rb][kb] = mfma_fp4(operand(k1), ks1, qb1[rb], qs1[rb], acc);
      }
    }
  };

  float m[2] = {kNegInf, kNegInf};  // prefix max of each row's tile maxima (raw q.k units)
  // tile j: row max over visible keys, the rows' votes, the tile's flag bit
  auto decide = [&](int j, f32x16_t (&s)[2][2]) __attribute__((always_inline)) {
    const int c0 = j * BC;
    if (c0 + BC > a.Nk || (a.causal && c0 + BC - 1 > first_pos)) {
      // key c0 + cc + 4h of register r (cc = 32kb + 8(r/4) + r%4) is masked
      // past the sequence or after the row's position: cc > lim, one per-lane
      // bound per row block against immediate offsets
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        int lim = a.Nk - 1 - c0;
        if (a.causal) lim = min(lim, qpos[rb] - c0);
        lim -= 4 * h;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[rb][kb][r] = kNegInf;
      }
    }
    bool keep = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(fmaxf(mt, s[rb][0][r]), s[rb][1][r]);
      mt = max_with_lane_xor32(mt);
      // keep unless the gap is below the threshold; a row with no visible key
      // has gap -inf, and a row with no running max yet has gap +inf (mt - m
      // is +inf when m = -inf and mt is finite; no NaN can arise)
      const float gap = mt == kNegInf ? kNegInf : mt - m[rb];
      keep |= valid[rb] && !(gap < a.thr_raw);
      m[rb] = fmaxf(m[rb], mt);
    }
    if (__ballot(keep) != 0ull && lane == 0) atomicOr(&flagw[tw][j >> 5], 1u << (j & 31));
  };

  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
  auto stage = [&](auto PAR, int st) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();  // stage st landed; every wave is done with stage st - 1
    if (st + 1 < nstage) {
      if constexpr (decltype(PAR)::value) issue(even, st + 1); else issue(odd, st + 1);
    }
    const char (&kbuf)[TPS][BC * ROWB] = kbuf_of(PAR);
    const uint32_t (&sbuf)[TPS][BC] = sbuf_of(PAR);
    const int j0 = st * TPS;
#pragma unroll
    for (int uu = 0; uu < TPS; ++uu) {
      if (j0 + uu >= Jw) break;  // past this wave's query tile (uniform)
      f32x16_t sc[2][2];
      scores(kbuf, sbuf, uu, sc);
      decide(j0 + uu, sc);
      // one tile's scores live at a time; the other waves on the SIMD (four
      // per SIMD at this register count) overlap one wave's reduction with
      // another's MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  issue(even, 0);
  for (int st = 0; st < nstage; st += 2) {
    stage(even, st);
    if (st + 1 < nstage) stage(odd, st + 1);
  }
  __syncthreads();

  // the map rows: tile 0 always kept, tiles past the causal bound not visited
  int kept = 0;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if (tt == 1 && !two) break;
    const int Jt = tt == 0 ? Jt0 : Jt1;
    uint8_t* mrow = a.map + ((int64_t)bh * a.nqt + i0 + tt) * a.nkt;
    for (int x = t; x < a.nkt; x += NT) {
      const uint8_t v =
          x >= Jt ? 2 : ((x == 0 || ((flagw[tt][x >> 5] >> (x & 31)) & 1u)) ? 1 : 0);
      mrow[x] = v;
      kept += v == 1;
    }
  }
  if (a.stats) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kept += __shfl_xor(kept, o, 64);
    if (lane == 0) {
      atomicAdd((unsigned long long*)&a.stats[2 * bh + 1], (unsigned long long)kept);
      if (w == 0) atomicAdd((unsigned long long*)&a.stats[2 * bh], (unsigned long long)(Jt0 + Jt1));
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
  // units of one (batch, KV head, query-tile pair): whole rounds of 8 units
  // (one per XCD), G blocks per unit
  const int64_t units = (int64_t)a.B * a.Hkv * ((a.nqt + 1) / 2);
  const int64_t nblocks = (units + 7) / 8 * 8 * (a.Hq / a.Hkv);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(twopass_map_kernel, dim3((unsigned)nblocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace blasst
