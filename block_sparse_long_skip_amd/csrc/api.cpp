// libblasst C ABI: argument validation and kernel dispatch.
//
// Every argument is checked before the first HIP call, so a rejected call
// launches nothing and leaves every output untouched. No C++ exception crosses
// the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/blasst.h"
#include "common.hpp"

// Scratch of the allocation-free decode (blasst_attn_decode_noalloc): one
// array per GPU, in the library's device code, alive until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so it is
// never passed to a kernel or a copy: its device address on the current GPU
// comes from hipGetSymbolAddress, once per device (scratch_address below), and
// that address is what the kernels get.
static __device__ __align__(256) char scratch[blasst::kNoAllocScratchBytes];

namespace blasst {
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_gqa(const DecodeArgs& a, void* workspace, hipStream_t stream);
hipError_t launch_decode_mla(const DecodeArgs& a, void* workspace, hipStream_t stream);
hipError_t launch_backward_bf16(const BackwardArgs& a, hipStream_t stream);
hipError_t launch_mx_quantize_fp4(const MxQuantArgs& a, hipStream_t stream);
hipError_t launch_twopass_map(const TwoPassMapArgs& a, hipStream_t stream);
size_t decode_mla_workspace_bytes(int B, int Hq, int Hkv, int G, int nkt);
size_t decode_gqa_workspace_bytes(int B, int Hq, int Hkv, int G, int nkt);

__global__ void zero_i64_kernel(int64_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
}  // namespace blasst

namespace {

thread_local char g_last_error[512] = "";

blasst_status_t fail(blasst_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
blasst_status_t fail(blasst_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

blasst_status_t ok() {
  g_last_error[0] = '\0';
  return BLASST_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A tensor pointer may be NULL exactly when the tensor has no elements.
bool missing(const void* p, int64_t elements) { return p == nullptr && elements > 0; }
int64_t count(int64_t a, int64_t b, int64_t c) {
  return (a > 0 && b > 0 && c > 0) ? a * b * c : 0;
}

bool strides_aligned(const int64_t* s, int n, int elem) {
  for (int i = 0; i < n; ++i)
    if (((s[i] * elem) & 15) != 0) return false;
  return true;
}

blasst_status_t check_dtypes(blasst_dtype_t in, blasst_dtype_t out) {
  if (in != BLASST_FP32 && in != BLASST_BF16) return fail(BLASST_E_DTYPE, "unknown dtype %d", (int)in);
  if (out != BLASST_FP32 && out != BLASST_BF16)
    return fail(BLASST_E_DTYPE, "unknown out_dtype %d", (int)out);
  if (in == BLASST_FP32 && out != BLASST_FP32)
    return fail(BLASST_E_DTYPE, "float32 inputs write float32 outputs");
  return BLASST_OK;
}

blasst_status_t check_lambda_scale(float lambda, float scale) {
  if (std::isnan(lambda) || lambda < 0.f || lambda > 1.f)
    return fail(BLASST_E_LAMBDA, "lambda must lie in [0, 1], got %g", (double)lambda);
  if (!std::isfinite(scale)) return fail(BLASST_E_ARG, "scale must be finite");
  return BLASST_OK;
}

// ln(lambda) / scale, the threshold in raw q.k units (-inf for lambda = 0).
float raw_threshold(float lambda, float scale) {
  if (lambda == 0.f) return -INFINITY;
  return (float)(std::log((double)lambda) / (double)scale);
}

blasst_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BLASST_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

blasst_status_t zero_stats(int64_t* stats, int64_t n, hipStream_t st) {
  if (!stats || n == 0) return BLASST_OK;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(blasst::zero_i64_kernel, dim3(blocks), dim3(256), 0, st, stats, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BLASST_E_HIP, "stats zero fill: %s", hipGetErrorString(e));
  return BLASST_OK;
}

// Both prefill entry points (masked: block-sparse mode with block_mask).
// Validates a prefill call and fills its kernel arguments; launches nothing.
blasst_status_t prepare_prefill(const void* q, const void* k, const void* v, bool masked,
                                const uint8_t* block_mask, const int64_t* block_mask_stride,
                                void* out, uint8_t* mask_out, float* lse_out, int64_t* stats_out,
                                const blasst_shape_t* shape, blasst_dtype_t dtype,
                                blasst_dtype_t out_dtype, float lambda, float scale, int causal,
                                int br, int bc, blasst::PrefillArgs* args, bool* use_f32) {
  blasst_status_t st0;
  if (!shape) return fail(BLASST_E_NULL, "shape is NULL");
  {
    const blasst_shape_t& z = *shape;
    const int64_t nq_el = count(z.batch, z.heads_q, z.len_q), nk_el = count(z.batch, z.heads_kv, z.len_kv);
    if (missing(q, nq_el) || missing(out, nq_el) || missing(k, nk_el) || missing(v, nk_el))
      return fail(BLASST_E_NULL, "q, k, v and out are required");
    if (masked && (!block_mask_stride || missing(block_mask, nq_el)))
      return fail(BLASST_E_NULL, "block_mask and block_mask_stride are required");
  }
  st0 = check_dtypes(dtype, out_dtype);
  if (st0 != BLASST_OK) return st0;
  const blasst_shape_t& s = *shape;
  if (s.batch < 0 || s.heads_q < 1 || s.heads_kv < 1 || s.len_q < 0 || s.len_kv < 1 ||
      s.d_qk < 1 || s.d_v < 1)
    return fail(BLASST_E_SHAPE, "sizes out of range (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d dv=%d)",
                s.batch, s.heads_q, s.heads_kv, s.len_q, s.len_kv, s.d_qk, s.d_v);
  if (s.heads_q % s.heads_kv != 0)
    return fail(BLASST_E_SHAPE, "heads_q (%d) must be a multiple of heads_kv (%d)", s.heads_q,
                s.heads_kv);
  if (causal && s.len_q > s.len_kv)
    return fail(BLASST_E_SHAPE, "causal prefill needs len_q <= len_kv (%d > %d)", s.len_q,
                s.len_kv);
  if (br < 1 || bc < 1) return fail(BLASST_E_SHAPE, "tile sizes must be positive");
  blasst_status_t st = check_lambda_scale(lambda, scale);
  if (st != BLASST_OK) return st;
  const int elem = dtype == BLASST_FP32 ? 4 : 2;
  const int oelem = out_dtype == BLASST_FP32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(BLASST_E_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (!strides_aligned(s.q_stride, 3, elem) || !strides_aligned(s.k_stride, 3, elem) ||
      !strides_aligned(s.v_stride, 3, elem) || !strides_aligned(s.o_stride, 3, oelem))
    return fail(BLASST_E_ALIGN, "every stride times the element size must be a multiple of 16");
  const bool f32 = dtype == BLASST_FP32 && s.d_qk == 64 && s.d_v == 64 && br == 64 && bc == 64;
  const bool b16 = dtype == BLASST_BF16 && s.d_qk == 128 && s.d_v == 128 && br == 128 && bc == 64;
  if (!f32 && !b16)
    return fail(BLASST_E_UNSUPPORTED,
                "no prefill kernel for dtype=%d d_qk=%d d_v=%d br=%d bc=%d (supported: fp32 "
                "64/64 64x64, bf16 128/128 128x64)",
                (int)dtype, s.d_qk, s.d_v, br, bc);
  // the bf16 kernel addresses a 64-row tile with 32-bit per-lane byte offsets
  if (b16 && (s.k_stride[2] < s.d_qk || s.v_stride[2] < s.d_v))
    return fail(BLASST_E_SHAPE, "key/value rows overlap (position stride below the row length)");
  if (b16 && (s.k_stride[2] > (1 << 24) || s.v_stride[2] > (1 << 24)))
    return fail(BLASST_E_UNSUPPORTED, "bf16 prefill needs key/value position strides <= 2^24 elements");
  const int64_t nqt = ((int64_t)s.len_q + br - 1) / br;
  const int64_t nkt = ((int64_t)s.len_kv + bc - 1) / bc;
  // the bf16 kernel pads its grid to whole rounds of 8 (KV head, query tile) units
  if ((int64_t)s.batch * s.heads_q * nqt + 8LL * (s.heads_q / s.heads_kv) > 0x7fffffffLL)
    return fail(BLASST_E_UNSUPPORTED, "grid too large");
  if (masked) {
    if (!b16)
      return fail(BLASST_E_UNSUPPORTED, "block-sparse prefill needs bf16 inputs, d = 128, 128x64 tiles");
    if (block_mask_stride[0] < 0 || block_mask_stride[1] < 0 || block_mask_stride[2] < 0)
      return fail(BLASST_E_SHAPE, "block_mask strides must be >= 0");
    if (nkt > blasst::kPrefillMaxSetTiles)
      return fail(BLASST_E_UNSUPPORTED, "block-sparse prefill supports at most %d key tiles (got %lld)",
                  blasst::kPrefillMaxSetTiles, (long long)nkt);
  }

  const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)s.d_qk));
  blasst::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.mask = mask_out; a.lse = lse_out; a.stats = stats_out;
  a.block_mask = block_mask;
  a.bms0 = masked ? block_mask_stride[0] : 0;
  a.bms1 = masked ? block_mask_stride[1] : 0;
  a.bms2 = masked ? block_mask_stride[2] : 0;
  a.B = s.batch; a.Hq = s.heads_q; a.Hkv = s.heads_kv; a.Nq = s.len_q; a.Nk = s.len_kv;
  a.nqt = (int)nqt; a.nkt = (int)nkt; a.causal = causal ? 1 : 0;
  a.out_f32 = out_dtype == BLASST_FP32 ? 1 : 0;
  a.qs0 = s.q_stride[0]; a.qs1 = s.q_stride[1]; a.qs2 = s.q_stride[2];
  a.ks0 = s.k_stride[0]; a.ks1 = s.k_stride[1]; a.ks2 = s.k_stride[2];
  a.vs0 = s.v_stride[0]; a.vs1 = s.v_stride[1]; a.vs2 = s.v_stride[2];
  a.os0 = s.o_stride[0]; a.os1 = s.o_stride[1]; a.os2 = s.o_stride[2];
  a.scale = sc;
  a.scale_log2 = sc * blasst::kLog2e;
  a.thr_raw = raw_threshold(lambda, sc);
  *args = a;
  *use_f32 = f32;
  return BLASST_OK;
}

blasst_status_t run_prefill(const void* q, const void* k, const void* v, bool masked,
                            const uint8_t* block_mask, const int64_t* block_mask_stride,
                            void* out, uint8_t* mask_out, float* lse_out, int64_t* stats_out,
                            const blasst_shape_t* shape, blasst_dtype_t dtype,
                            blasst_dtype_t out_dtype, float lambda, float scale, int causal,
                            int br, int bc, void* stream) {
  blasst::PrefillArgs a;
  bool f32 = false;
  blasst_status_t st = prepare_prefill(q, k, v, masked, block_mask, block_mask_stride, out, mask_out,
                                       lse_out, stats_out, shape, dtype, out_dtype, lambda, scale,
                                       causal, br, bc, &a, &f32);
  if (st != BLASST_OK) return st;
  const blasst_shape_t& s = *shape;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  st = zero_stats(stats_out, (int64_t)s.batch * s.heads_q * 2, hs);
  if (st != BLASST_OK) return st;
  if (s.batch == 0 || s.len_q == 0) return ok();
  const hipError_t e = f32 ? blasst::launch_prefill_f32(a, hs) : blasst::launch_prefill_bf16(a, hs);
  return hip_status(e, "prefill launch");
}

}  // namespace

extern "C" {

int blasst_version(void) { return BLASST_VERSION; }

const char* blasst_last_error(void) { return g_last_error; }

const char* blasst_status_string(blasst_status_t s) {
  switch (s) {
    case BLASST_OK: return "BLASST_OK";
    case BLASST_E_NULL: return "BLASST_E_NULL: a required pointer is NULL";
    case BLASST_E_SHAPE: return "BLASST_E_SHAPE: invalid sizes";
    case BLASST_E_DTYPE: return "BLASST_E_DTYPE: unknown dtype";
    case BLASST_E_LAMBDA: return "BLASST_E_LAMBDA: lambda outside [0, 1] or NaN";
    case BLASST_E_ALIGN: return "BLASST_E_ALIGN: pointer or stride not 16-byte aligned";
    case BLASST_E_UNSUPPORTED: return "BLASST_E_UNSUPPORTED: no kernel for this combination";
    case BLASST_E_ARG: return "BLASST_E_ARG: invalid scalar argument";
    case BLASST_E_HIP: return "BLASST_E_HIP: HIP runtime error";
    case BLASST_E_WORKSPACE: return "BLASST_E_WORKSPACE: workspace missing, too small or misaligned";
  }
  return "BLASST: unknown status";
}

blasst_status_t blasst_attn_prefill(const void* q, const void* k, const void* v, void* out,
                                    uint8_t* mask_out, float* lse_out, int64_t* stats_out,
                                    const blasst_shape_t* shape, blasst_dtype_t dtype,
                                    blasst_dtype_t out_dtype, float lambda, float scale,
                                    int causal, int br, int bc, void* stream) {
  return run_prefill(q, k, v, false, nullptr, nullptr, out, mask_out, lse_out, stats_out, shape, dtype,
                     out_dtype, lambda, scale, causal, br, bc, stream);
}

blasst_status_t blasst_attn_prefill_masked(const void* q, const void* k, const void* v,
                                           const uint8_t* block_mask,
                                           const int64_t block_mask_stride[3], void* out,
                                           uint8_t* mask_out, float* lse_out,
                                           int64_t* stats_out, const blasst_shape_t* shape,
                                           blasst_dtype_t dtype, blasst_dtype_t out_dtype,
                                           float lambda, float scale, int causal, int br, int bc,
                                           void* stream) {
  return run_prefill(q, k, v, true, block_mask, block_mask_stride, out, mask_out, lse_out, stats_out,
                     shape, dtype, out_dtype, lambda, scale, causal, br, bc, stream);
}

}  // extern "C"

namespace {

enum class DecodeKernel { kGqa, kLatent };

// Validation shared by the decode entry point and its workspace query.
blasst_status_t check_decode(const blasst_shape_t& s, blasst_dtype_t dtype, bool has_v, int bc,
                             DecodeKernel* kind) {
  if (s.batch < 0 || s.heads_q < 1 || s.heads_kv < 1 || s.len_kv < 1 || s.d_qk < 1 || s.d_v < 1)
    return fail(BLASST_E_SHAPE, "sizes out of range (B=%d Hq=%d Hkv=%d Nk=%d d=%d dv=%d)",
                s.batch, s.heads_q, s.heads_kv, s.len_kv, s.d_qk, s.d_v);
  if (s.len_q != 1) return fail(BLASST_E_SHAPE, "decode needs len_q == 1 (got %d)", s.len_q);
  if (s.heads_q % s.heads_kv != 0)
    return fail(BLASST_E_SHAPE, "heads_q (%d) must be a multiple of heads_kv (%d)", s.heads_q,
                s.heads_kv);
  if (!has_v && s.d_v >= s.d_qk)
    return fail(BLASST_E_SHAPE, "a latent cache (v_cache NULL) needs d_v < d_qk");
  if (bc < 1) return fail(BLASST_E_SHAPE, "tile size must be positive");
  const int G = s.heads_q / s.heads_kv;
  const bool gqa = dtype == BLASST_BF16 && has_v && s.d_qk == 128 && s.d_v == 128 && bc == 64 &&
                   G <= 16;
  const bool mla = dtype == BLASST_BF16 && !has_v && s.d_qk == 576 && s.d_v == 512 && bc == 64;
  if (!gqa && !mla)
    return fail(BLASST_E_UNSUPPORTED,
                "no decode kernel for dtype=%d d_qk=%d d_v=%d bc=%d G=%d v_cache=%s (supported: "
                "bf16 128/128 bc=64 G<=16; bf16 latent 576/512 bc=64)",
                (int)dtype, s.d_qk, s.d_v, bc, G, has_v ? "set" : "NULL");
  *kind = gqa ? DecodeKernel::kGqa : DecodeKernel::kLatent;
  return BLASST_OK;
}

size_t decode_workspace(const blasst_shape_t& s, DecodeKernel kind, int bc) {
  if (s.batch == 0) return 0;
  const int nkt = (s.len_kv + bc - 1) / bc;
  if (kind == DecodeKernel::kGqa)
    return blasst::decode_gqa_workspace_bytes(s.batch, s.heads_q, s.heads_kv,
                                              s.heads_q / s.heads_kv, nkt);
  return blasst::decode_mla_workspace_bytes(s.batch, s.heads_q, s.heads_kv,
                                            s.heads_q / s.heads_kv, nkt);
}

// Validates a decode call and fills its kernel arguments, the kernel kind and
// the scratch bytes it needs; launches nothing.
blasst_status_t prepare_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                               uint8_t* mask_out, float* lse_out, int64_t* stats_out,
                               const blasst_shape_t* shape, blasst_dtype_t dtype,
                               blasst_dtype_t out_dtype, float lambda, float scale, int bc,
                               blasst::DecodeArgs* args, DecodeKernel* kind_out, size_t* need) {
  if (!shape) return fail(BLASST_E_NULL, "shape is NULL");
  if (missing(q, count(shape->batch, shape->heads_q, 1)) ||
      missing(out, count(shape->batch, shape->heads_q, 1)) ||
      missing(k_cache, count(shape->batch, shape->heads_kv, shape->len_kv)))
    return fail(BLASST_E_NULL, "q, k_cache and out are required");
  blasst_status_t st = check_dtypes(dtype, out_dtype);
  if (st != BLASST_OK) return st;
  const blasst_shape_t& s = *shape;
  DecodeKernel kind;
  st = check_decode(s, dtype, v_cache != nullptr, bc, &kind);
  if (st != BLASST_OK) return st;
  st = check_lambda_scale(lambda, scale);
  if (st != BLASST_OK) return st;
  const int elem = dtype == BLASST_FP32 ? 4 : 2;
  const int oelem = out_dtype == BLASST_FP32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(k_cache) || (v_cache && !aligned16(v_cache)) || !aligned16(out))
    return fail(BLASST_E_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!strides_aligned(s.q_stride, 2, elem) || !strides_aligned(s.k_stride, 3, elem) ||
      (v_cache && !strides_aligned(s.v_stride, 3, elem)) || !strides_aligned(s.o_stride, 2, oelem))
    return fail(BLASST_E_ALIGN, "every stride times the element size must be a multiple of 16");
  if (kind == DecodeKernel::kLatent && s.k_stride[2] < s.d_qk)
    return fail(BLASST_E_SHAPE, "latent cache rows overlap (k_stride[2] = %lld < d_qk = %d)",
                (long long)s.k_stride[2], s.d_qk);
  if (kind == DecodeKernel::kLatent && s.k_stride[2] * 2 * 64 > (int64_t)INT32_MAX)
    return fail(BLASST_E_UNSUPPORTED, "latent cache row stride too large (%lld elements)",
                (long long)s.k_stride[2]);
  const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)s.d_qk));
  blasst::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.out = out;
  a.mask = mask_out; a.lse = lse_out; a.stats = stats_out;
  a.B = s.batch; a.Hq = s.heads_q; a.Hkv = s.heads_kv; a.Nk = s.len_kv;
  a.G = s.heads_q / s.heads_kv;
  a.nkt = (s.len_kv + bc - 1) / bc;
  a.out_f32 = out_dtype == BLASST_FP32 ? 1 : 0;
  a.qs0 = s.q_stride[0]; a.qs1 = s.q_stride[1];
  a.ks0 = s.k_stride[0]; a.ks1 = s.k_stride[1]; a.ks2 = s.k_stride[2];
  a.vs0 = s.v_stride[0]; a.vs1 = s.v_stride[1]; a.vs2 = s.v_stride[2];
  a.os0 = s.o_stride[0]; a.os1 = s.o_stride[1];
  a.scale = sc;
  a.scale_log2 = sc * blasst::kLog2e;
  a.thr_raw = raw_threshold(lambda, sc);
  *args = a;
  *kind_out = kind;
  *need = decode_workspace(s, kind, bc);
  return BLASST_OK;
}

blasst_status_t launch_decode(const blasst::DecodeArgs& a, DecodeKernel kind, void* workspace,
                              hipStream_t hs) {
  if (a.B == 0) return ok();
  const hipError_t e = kind == DecodeKernel::kGqa ? blasst::launch_decode_gqa(a, workspace, hs)
                                                  : blasst::launch_decode_mla(a, workspace, hs);
  return hip_status(e, "decode launch");
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

blasst_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BLASST_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BLASST_E_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(BLASST_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BLASST_OK;
}

}  // namespace

extern "C" {

blasst_status_t blasst_decode_workspace_size(const blasst_shape_t* shape, blasst_dtype_t dtype,
                                             int has_v_cache, int bc, size_t* bytes) {
  if (!shape || !bytes) return fail(BLASST_E_NULL, "shape and bytes are required");
  blasst_status_t st = check_dtypes(dtype, dtype);
  if (st != BLASST_OK) return st;
  DecodeKernel kind;
  st = check_decode(*shape, dtype, has_v_cache != 0, bc, &kind);
  if (st != BLASST_OK) return st;
  *bytes = decode_workspace(*shape, kind, bc);
  return ok();
}

size_t blasst_attn_decode_workspace_size(const blasst_shape_t* shape, blasst_dtype_t dtype,
                                         int bc) {
  // The cache kind follows from the sizes: only a latent cache has d_v < d_qk.
  size_t bytes = 0;
  if (!shape) {
    fail(BLASST_E_NULL, "shape is NULL");
    return SIZE_MAX;
  }
  const int has_v = shape->d_v < shape->d_qk ? 0 : 1;
  if (blasst_decode_workspace_size(shape, dtype, has_v, bc, &bytes) != BLASST_OK) return SIZE_MAX;
  return bytes;
}

blasst_status_t blasst_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                   void* out, uint8_t* mask_out, float* lse_out,
                                   int64_t* stats_out, const blasst_shape_t* shape,
                                   blasst_dtype_t dtype, blasst_dtype_t out_dtype, float lambda,
                                   float scale, int bc, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  blasst::DecodeArgs a;
  DecodeKernel kind;
  size_t need = 0;
  blasst_status_t st = prepare_decode(q, k_cache, v_cache, out, mask_out, lse_out, stats_out, shape,
                                      dtype, out_dtype, lambda, scale, bc, &a, &kind, &need);
  if (st != BLASST_OK) return st;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(BLASST_E_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need,
                  workspace ? workspace_bytes : (size_t)0, workspace);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(BLASST_E_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return launch_decode(a, kind, workspace, reinterpret_cast<hipStream_t>(stream));
}

blasst_status_t blasst_attn_decode_noalloc(const void* q, const void* k_cache,
                                           const void* v_cache, void* out, uint8_t* mask_out,
                                           float* lse_out, int64_t* stats_out,
                                           const blasst_shape_t* shape, blasst_dtype_t dtype,
                                           blasst_dtype_t out_dtype, float lambda, float scale,
                                           int bc, void* stream) {
  blasst::DecodeArgs a;
  DecodeKernel kind;
  size_t need = 0;
  blasst_status_t st = prepare_decode(q, k_cache, v_cache, out, mask_out, lse_out, stats_out, shape,
                                      dtype, out_dtype, lambda, scale, bc, &a, &kind, &need);
  if (st != BLASST_OK) return st;
  if (need > blasst::kNoAllocScratchBytes)
    return fail(BLASST_E_UNSUPPORTED,
                "this shape needs %zu bytes of scratch; the allocation-free decode holds %zu "
                "(use blasst_attn_decode with a workspace)",
                need, (size_t)blasst::kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != BLASST_OK) return st;
  }
  return launch_decode(a, kind, ws, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Validation shared by the backward entry point and its workspace query.
blasst_status_t check_backward(const blasst_shape_t& s, blasst_dtype_t dtype, int causal, int br,
                               int bc) {
  if (s.batch < 0 || s.heads_q < 1 || s.heads_kv < 1 || s.len_q < 0 || s.len_kv < 1 ||
      s.d_qk < 1 || s.d_v < 1)
    return fail(BLASST_E_SHAPE, "sizes out of range (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d dv=%d)",
                s.batch, s.heads_q, s.heads_kv, s.len_q, s.len_kv, s.d_qk, s.d_v);
  if (s.heads_q % s.heads_kv != 0)
    return fail(BLASST_E_SHAPE, "heads_q (%d) must be a multiple of heads_kv (%d)", s.heads_q,
                s.heads_kv);
  if (causal && s.len_q > s.len_kv)
    return fail(BLASST_E_SHAPE, "causal prefill needs len_q <= len_kv (%d > %d)", s.len_q,
                s.len_kv);
  if (br < 1 || bc < 1) return fail(BLASST_E_SHAPE, "tile sizes must be positive");
  if (dtype != BLASST_FP32 && dtype != BLASST_BF16)
    return fail(BLASST_E_DTYPE, "unknown dtype %d", (int)dtype);
  if (dtype != BLASST_BF16 || s.d_qk != 128 || s.d_v != 128 || br != 128 || bc != 64)
    return fail(BLASST_E_UNSUPPORTED,
                "no backward kernel for dtype=%d d_qk=%d d_v=%d br=%d bc=%d (supported: bf16 "
                "128/128 128x64)",
                (int)dtype, s.d_qk, s.d_v, br, bc);
  const int64_t nqt = ((int64_t)s.len_q + br - 1) / br;
  const int64_t nkt = ((int64_t)s.len_kv + bc - 1) / bc;
  if (nqt > blasst::kBackwardMaxTiles || nkt > blasst::kBackwardMaxTiles)
    return fail(BLASST_E_UNSUPPORTED, "backward supports at most %d query and key tiles",
                blasst::kBackwardMaxTiles);
  if ((int64_t)s.batch * s.heads_q * nqt > 0x7fffffffLL ||
      (int64_t)s.batch * s.heads_kv * nkt > 0x7fffffffLL)
    return fail(BLASST_E_UNSUPPORTED, "grid too large");
  if (s.k_stride[2] < s.d_qk || s.v_stride[2] < s.d_v || s.q_stride[2] < s.d_qk ||
      s.o_stride[2] < s.d_v)
    return fail(BLASST_E_SHAPE, "rows overlap (position stride below the row length)");
  if (s.k_stride[2] > (1 << 24) || s.v_stride[2] > (1 << 24) || s.q_stride[2] > (1 << 24) ||
      s.o_stride[2] > (1 << 24))
    return fail(BLASST_E_UNSUPPORTED, "backward needs position strides <= 2^24 elements");
  return BLASST_OK;
}

size_t backward_workspace(const blasst_shape_t& s) {
  const size_t n = (size_t)s.batch * s.heads_q * s.len_q * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

blasst_status_t blasst_prefill_backward_workspace_size(const blasst_shape_t* shape,
                                                       blasst_dtype_t dtype, int causal, int br,
                                                       int bc, size_t* bytes) {
  if (!shape || !bytes) return fail(BLASST_E_NULL, "shape and bytes are required");
  const blasst_status_t st = check_backward(*shape, dtype, causal, br, bc);
  if (st != BLASST_OK) return st;
  *bytes = backward_workspace(*shape);
  return ok();
}

blasst_status_t blasst_attn_prefill_backward(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, const uint8_t* mask, float* dq, float* dk, float* dv,
    const blasst_shape_t* shape, blasst_dtype_t dtype, blasst_dtype_t out_dtype, float scale,
    int causal, int br, int bc, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape) return fail(BLASST_E_NULL, "shape is NULL");
  {
    const int64_t nq_el = count(shape->batch, shape->heads_q, shape->len_q);
    const int64_t nk_el = count(shape->batch, shape->heads_kv, shape->len_kv);
    if (missing(q, nq_el) || missing(out, nq_el) || missing(dout, nq_el) || missing(lse, nq_el) ||
        missing(mask, nq_el) || missing(dq, nq_el) || missing(k, nk_el) || missing(v, nk_el) ||
        missing(dk, nk_el) || missing(dv, nk_el))
      return fail(BLASST_E_NULL, "q, k, v, out, dout, lse, mask, dq, dk and dv are required");
  }
  const blasst_shape_t& s = *shape;
  blasst_status_t st = check_backward(s, dtype, causal, br, bc);
  if (st != BLASST_OK) return st;
  if (out_dtype != BLASST_FP32 && out_dtype != BLASST_BF16)
    return fail(BLASST_E_DTYPE, "unknown out_dtype %d", (int)out_dtype);
  if (!std::isfinite(scale)) return fail(BLASST_E_ARG, "scale must be finite");
  const int oelem = out_dtype == BLASST_FP32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(BLASST_E_ALIGN, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (!strides_aligned(s.q_stride, 3, 2) || !strides_aligned(s.k_stride, 3, 2) ||
      !strides_aligned(s.v_stride, 3, 2) || !strides_aligned(s.o_stride, 3, 2) ||
      !strides_aligned(s.o_stride, 3, oelem))
    return fail(BLASST_E_ALIGN, "every stride times the element size must be a multiple of 16");
  const size_t need = backward_workspace(s);
  if (need > 0) {
    if (!workspace) return fail(BLASST_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
      return fail(BLASST_E_WORKSPACE, "workspace of %zu bytes is smaller than %zu", workspace_bytes,
                  need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(BLASST_E_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)s.d_qk));
  blasst::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse; a.mask = mask;
  a.dq = dq; a.dk = dk; a.dv = dv; a.delta = static_cast<float*>(workspace);
  a.B = s.batch; a.Hq = s.heads_q; a.Hkv = s.heads_kv; a.Nq = s.len_q; a.Nk = s.len_kv;
  a.nqt = (s.len_q + br - 1) / br; a.nkt = (s.len_kv + bc - 1) / bc;
  a.causal = causal ? 1 : 0;
  a.out_f32 = out_dtype == BLASST_FP32 ? 1 : 0;
  a.qs0 = s.q_stride[0]; a.qs1 = s.q_stride[1]; a.qs2 = s.q_stride[2];
  a.ks0 = s.k_stride[0]; a.ks1 = s.k_stride[1]; a.ks2 = s.k_stride[2];
  a.vs0 = s.v_stride[0]; a.vs1 = s.v_stride[1]; a.vs2 = s.v_stride[2];
  a.os0 = s.o_stride[0]; a.os1 = s.o_stride[1]; a.os2 = s.o_stride[2];
  a.dos0 = s.o_stride[0]; a.dos1 = s.o_stride[1]; a.dos2 = s.o_stride[2];
  a.scale = sc;
  a.scale_log2 = sc * blasst::kLog2e;
  if (s.batch == 0) return ok();
  return hip_status(blasst::launch_backward_bf16(a, reinterpret_cast<hipStream_t>(stream)),
                    "backward launch");
}

}  // extern "C"

namespace {

// Byte offsets of the two-pass workspace segments, each 256-byte aligned.
struct TwoPassLayout {
  size_t qc, qs, kc, ks, map, total;
};

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

TwoPassLayout twopass_layout(const blasst_shape_t& s, int br, int bc) {
  const size_t qrows = (size_t)s.batch * s.heads_q * s.len_q;
  const size_t krows = (size_t)s.batch * s.heads_kv * s.len_kv;
  const size_t nqt = ((size_t)s.len_q + br - 1) / br, nkt = ((size_t)s.len_kv + bc - 1) / bc;
  TwoPassLayout L;
  L.qc = 0;
  L.qs = L.qc + align256(qrows * (s.d_qk / 2));
  L.kc = L.qs + align256(qrows * (s.d_qk / 32));
  L.ks = L.kc + align256(krows * (s.d_qk / 2));
  L.map = L.ks + align256(krows * (s.d_qk / 32));
  L.total = L.map + align256((size_t)s.batch * s.heads_q * nqt * nkt);
  return L;
}

// The two-pass call supports exactly the block-sparse prefill's configuration.
blasst_status_t check_twopass(const blasst_shape_t& s, blasst_dtype_t dtype, int causal, int br,
                              int bc) {
  if (s.batch < 0 || s.heads_q < 1 || s.heads_kv < 1 || s.len_q < 0 || s.len_kv < 1 ||
      s.d_qk < 1 || s.d_v < 1)
    return fail(BLASST_E_SHAPE, "sizes out of range (B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d dv=%d)",
                s.batch, s.heads_q, s.heads_kv, s.len_q, s.len_kv, s.d_qk, s.d_v);
  if (dtype != BLASST_FP32 && dtype != BLASST_BF16)
    return fail(BLASST_E_DTYPE, "unknown dtype %d", (int)dtype);
  if (dtype != BLASST_BF16 || s.d_qk != 128 || s.d_v != 128 || br != 128 || bc != 64)
    return fail(BLASST_E_UNSUPPORTED,
                "no two-pass kernel for dtype=%d d_qk=%d d_v=%d br=%d bc=%d (supported: bf16 "
                "128/128 128x64)",
                (int)dtype, s.d_qk, s.d_v, br, bc);
  (void)causal;
  return BLASST_OK;
}

blasst_status_t check_workspace(const void* ws, size_t bytes, size_t need) {
  if (need == 0) return BLASST_OK;
  if (!ws) return fail(BLASST_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (bytes < need)
    return fail(BLASST_E_WORKSPACE, "workspace of %zu bytes is smaller than %zu", bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(BLASST_E_WORKSPACE, "workspace must be 256-byte aligned");
  return BLASST_OK;
}

blasst::MxQuantArgs quant_args(const void* x, const int64_t* stride, int d0, int d1, int n, int d,
                               uint8_t* codes, uint8_t* scales) {
  blasst::MxQuantArgs a;
  a.x = x; a.codes = codes; a.scales = scales;
  a.d0 = d0; a.d1 = d1; a.n = n; a.d = d;
  a.s0 = stride[0]; a.s1 = stride[1]; a.s2 = stride[2];
  return a;
}

}  // namespace

extern "C" {

blasst_status_t blasst_quantize_mxfp4(const void* x, const int64_t x_stride[3], int32_t d0,
                                      int32_t d1, int32_t n, int32_t d, blasst_dtype_t dtype,
                                      uint8_t* codes, uint8_t* scales, void* stream) {
  const int64_t nrows = count(d0, d1, n);
  if (!x_stride || missing(x, nrows) || missing(codes, nrows) || missing(scales, nrows))
    return fail(BLASST_E_NULL, "x, x_stride, codes and scales are required");
  if (d0 < 0 || d1 < 0 || n < 0 || d < 32 || d % 32 != 0)
    return fail(BLASST_E_SHAPE, "need d0, d1, n >= 0 and d a positive multiple of 32 (got %d %d %d %d)",
                d0, d1, n, d);
  if (dtype != BLASST_BF16) return fail(BLASST_E_DTYPE, "MXFP4 quantization takes bf16 input");
  if (!aligned16(x) || !aligned16(codes)) return fail(BLASST_E_ALIGN, "x and codes must be 16-byte aligned");
  if (!strides_aligned(x_stride, 3, 2))
    return fail(BLASST_E_ALIGN, "every stride times the element size must be a multiple of 16");
  if ((int64_t)d0 * d1 * n * (d / 32) > 0x7fffffffLL * 256LL)
    return fail(BLASST_E_UNSUPPORTED, "grid too large");
  const blasst::MxQuantArgs a = quant_args(x, x_stride, d0, d1, n, d, codes, scales);
  return hip_status(blasst::launch_mx_quantize_fp4(a, reinterpret_cast<hipStream_t>(stream)),
                    "MXFP4 quantize launch");
}

blasst_status_t blasst_prefill_twopass_workspace_size(const blasst_shape_t* shape,
                                                      blasst_dtype_t dtype, int causal, int br,
                                                      int bc, size_t* bytes) {
  if (!shape || !bytes) return fail(BLASST_E_NULL, "shape and bytes are required");
  const blasst_status_t st = check_twopass(*shape, dtype, causal, br, bc);
  if (st != BLASST_OK) return st;
  *bytes = twopass_layout(*shape, br, bc).total;
  return ok();
}

blasst_status_t blasst_attn_prefill_twopass(const void* q, const void* k, const void* v,
                                            void* out, uint8_t* mask_out, float* lse_out,
                                            int64_t* stats_out, const blasst_shape_t* shape,
                                            blasst_dtype_t dtype, blasst_dtype_t out_dtype,
                                            float lambda, float scale, int causal, int br, int bc,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  if (!shape) return fail(BLASST_E_NULL, "shape is NULL");
  const blasst_shape_t& s = *shape;
  blasst_status_t st = check_twopass(s, dtype, causal, br, bc);
  if (st != BLASST_OK) return st;
  const TwoPassLayout L = twopass_layout(s, br, bc);
  st = check_workspace(workspace, workspace_bytes, L.total);
  if (st != BLASST_OK) return st;
  // the second pass is the block-sparse prefill over the map; validating it
  // first covers every pointer, stride and size rule of the inputs and outputs
  char* ws = static_cast<char*>(workspace);
  uint8_t* map = mask_out ? mask_out : (ws ? reinterpret_cast<uint8_t*>(ws + L.map) : nullptr);
  const int nqt = (s.len_q + br - 1) / br, nkt = (s.len_kv + bc - 1) / bc;
  const int64_t map_stride[3] = {(int64_t)s.heads_q * nqt * nkt, (int64_t)nqt * nkt, nkt};
  blasst::PrefillArgs a2;
  bool f32 = false;
  st = prepare_prefill(q, k, v, true, map, map_stride, out, nullptr, lse_out, nullptr, shape,
                       dtype, out_dtype, lambda, scale, causal, br, bc, &a2, &f32);
  if (st != BLASST_OK) return st;
  a2.thr_raw = raw_threshold(0.f, a2.scale);  // exact softmax over the kept tiles

  blasst::TwoPassMapArgs m;
  m.qc = reinterpret_cast<const uint8_t*>(ws + L.qc);
  m.qs = reinterpret_cast<const uint8_t*>(ws + L.qs);
  m.kc = reinterpret_cast<const uint8_t*>(ws + L.kc);
  m.ks = reinterpret_cast<const uint8_t*>(ws + L.ks);
  m.map = map;
  m.stats = stats_out;
  m.B = s.batch; m.Hq = s.heads_q; m.Hkv = s.heads_kv; m.Nq = s.len_q; m.Nk = s.len_kv;
  m.nqt = nqt; m.nkt = nkt; m.causal = causal ? 1 : 0;
  m.thr_raw = raw_threshold(lambda, a2.scale);

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  st = zero_stats(stats_out, (int64_t)s.batch * s.heads_q * 2, hs);
  if (st != BLASST_OK) return st;
  if (s.batch == 0 || s.len_q == 0) return ok();
  hipError_t e = blasst::launch_mx_quantize_fp4(
      quant_args(q, s.q_stride, s.batch, s.heads_q, s.len_q, s.d_qk, reinterpret_cast<uint8_t*>(ws + L.qc),
                 reinterpret_cast<uint8_t*>(ws + L.qs)), hs);
  if (e == hipSuccess)
    e = blasst::launch_mx_quantize_fp4(
        quant_args(k, s.k_stride, s.batch, s.heads_kv, s.len_kv, s.d_qk,
                   reinterpret_cast<uint8_t*>(ws + L.kc), reinterpret_cast<uint8_t*>(ws + L.ks)), hs);
  if (e == hipSuccess) e = blasst::launch_twopass_map(m, hs);
  if (e == hipSuccess) e = blasst::launch_prefill_bf16(a2, hs);
  return hip_status(e, "two-pass prefill launch");
}

}  // extern "C"
