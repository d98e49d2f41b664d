// Device helpers shared by the gfx950 kernels of libblasst.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blasst {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Longest block-set row (key tiles of one query tile) the block-sparse prefill
// lists in LDS.
constexpr int kPrefillMaxSetTiles = 6144;

// Bytes of the per-GPU scratch array the allocation-free decode uses in place
// of a caller's workspace (64 MiB: the batch-16 latent decode over 32768 keys
// with 128 query heads needs about 37 MB).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// Arguments of every prefill kernel (element strides; last dim contiguous).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  uint8_t* mask;   // nullable [B,Hq,nqt,nkt]
  float* lse;      // nullable [B,Hq,Nq]
  int64_t* stats;  // nullable [B,Hq,2], zeroed by the launcher
  // nullable block set [B,Hq,nqt,nkt] (element strides bms0..bms2, key tiles
  // contiguous; a zero stride broadcasts): nonzero = the block may be attended
  const uint8_t* block_mask;
  int64_t bms0, bms1, bms2;
  int B, Hq, Hkv, Nq, Nk;
  int nqt, nkt;
  int causal;
  int out_f32;  // 1: out is float32, 0: out is bfloat16
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  float scale;      // softmax scale applied to q.k
  float scale_log2; // scale * log2(e)
  float thr_raw;    // ln(lambda) / scale: the drop threshold in raw q.k units
};

// Longest list of kept tiles (key tiles of a query tile, or query tiles of a
// key tile) the backward kernels hold in LDS.
constexpr int kBackwardMaxTiles = 6144;

// Arguments of the backward kernels (element strides; last dim contiguous).
// The gradients dq, dk, dv are float32 with the element strides of q, k, v;
// dout has the strides of out.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;    // forward output, bf16 or float32 (out_f32)
  const void* dout;   // bf16
  const float* lse;   // [B,Hq,Nq] forward lse
  const uint8_t* mask;  // [B,Hq,nqt,nkt] forward mask, 1 = kept
  float* dq;
  float* dk;
  float* dv;
  float* delta;       // workspace [B,Hq,Nq]
  int B, Hq, Hkv, Nq, Nk;
  int nqt, nkt;
  int causal;
  int out_f32;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2, dos0, dos1, dos2;
  float scale, scale_log2;
};

// Arguments of the MXFP4 quantizer: x [d0, d1, n, d] bf16 with element
// strides s0..s2 (features contiguous) -> codes [d0 * d1 * n][d / 2] (two
// elements per byte, the even one in the low nibble) and scales
// [d0 * d1 * n][d / 32] (E8M0), both contiguous.
struct MxQuantArgs {
  const void* x;
  uint8_t* codes;
  uint8_t* scales;
  int d0, d1, n, d;
  int64_t s0, s1, s2;
};

// Arguments of the two-pass map kernel (d = 128: 64 code bytes and 4 scale
// bytes per row, rows ordered as (batch, head, position)).
struct TwoPassMapArgs {
  const uint8_t* qc;   // [B * Hq * Nq][64]
  const uint8_t* qs;   // [B * Hq * Nq][4]
  const uint8_t* kc;   // [B * Hkv * Nk][64]
  const uint8_t* ks;   // [B * Hkv * Nk][4]
  uint8_t* map;        // [B, Hq, nqt, nkt]: 0 dropped, 1 kept, 2 not visited
  int64_t* stats;      // nullable [B, Hq, 2], zeroed by the launcher
  int B, Hq, Hkv, Nq, Nk;
  int nqt, nkt;
  int causal;
  float thr_raw;       // ln(lambda) / scale
};

// Arguments of the decode kernels.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;  // null for a latent (MLA) cache
  void* out;
  uint8_t* mask;   // nullable [B,Hq,nkt]
  float* lse;      // nullable [B,Hq]
  int64_t* stats;  // nullable [B,Hq,3]
  int B, Hq, Hkv, Nk, G;
  int nkt;
  int out_f32;  // 1: out is float32, 0: out is bfloat16
  int64_t qs0, qs1, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1;
  float scale, scale_log2, thr_raw;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> one dword of two bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Low halves of two dwords -> (lo(a), lo(b)); high halves -> (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b,
                                                 const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Lane l and lane l^32 exchange values (gfx950 v_permlane32_swap). Either
// order of the returned pair holds {own, partner}; callers only combine them
// with commutative operations.
__device__ __forceinline__ float max_with_lane_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_lane_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Store 4 consecutive output features as bf16 (8 bytes) or float32 (16 bytes).
__device__ __forceinline__ void store_out4(void* out, int64_t elem_off, bool f32, float a,
                                           float b, float c, float d) {
  if (f32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + elem_off) = (f32x4_t){a, b, c, d};
  } else {
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + elem_off) =
        (u32x2_t){pack_bf16x2(a, b), pack_bf16x2(c, d)};
  }
}
__device__ __forceinline__ void store_out1(void* out, int64_t elem_off, bool f32, float a) {
  if (f32) static_cast<float*>(out)[elem_off] = a;
  else static_cast<uint16_t*>(out)[elem_off] = (uint16_t)(pack_bf16x2(a, 0.f) & 0xffffu);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void store16(void* p, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives element i%4 of the 4-element rows addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
__device__ __forceinline__ u32x2_t ds_read_tr(const char* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4_t*)(p)));
}

// global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at lds_base + 16 l; lds_base must be the same in every lane.
__device__ __forceinline__ void lds_dma16(const void* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   0);
}

// wait for this wave's outstanding global memory operations, including the
// copies into LDS
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__global__ void zero_i64_kernel(int64_t* p, int64_t n);

}  // namespace blasst
