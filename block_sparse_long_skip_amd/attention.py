"""Thin ctypes binding over libblasst (include/blasst.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libblasst.so. PyTorch provides device memory (output tensors are
allocated with ``torch.empty`` on the input's device) and the stream
(``torch.cuda.current_stream()``). There is no CPU fallback: if the library
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblasst.so")

BLASST_FP32 = 0
BLASST_BF16 = 1

STATUS = {
    0: "BLASST_OK", 1: "BLASST_E_NULL", 2: "BLASST_E_SHAPE", 3: "BLASST_E_DTYPE",
    4: "BLASST_E_LAMBDA", 5: "BLASST_E_ALIGN", 6: "BLASST_E_UNSUPPORTED", 7: "BLASST_E_ARG",
    8: "BLASST_E_HIP", 9: "BLASST_E_WORKSPACE",
}

# Every symbol include/blasst.h declares.
EXPORTED = ("blasst_attn_prefill", "blasst_attn_prefill_masked", "blasst_attn_prefill_backward",
            "blasst_prefill_backward_workspace_size", "blasst_quantize_mxfp4",
            "blasst_attn_prefill_twopass", "blasst_prefill_twopass_workspace_size",
            "blasst_attn_decode", "blasst_attn_decode_noalloc", "blasst_attn_decode_workspace_size",
            "blasst_decode_workspace_size", "blasst_status_string", "blasst_last_error",
            "blasst_version")


class Shape(ctypes.Structure):
    """blasst_shape_t."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("len_q", ctypes.c_int32), ("len_kv", ctypes.c_int32), ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
    ]


class BlasstError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libblasst.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_long_skip_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i64p, u8p, fp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.blasst_attn_prefill.restype = ctypes.c_int
    lib.blasst_attn_prefill.argtypes = [vp, vp, vp, vp, u8p, fp, i64p, ctypes.POINTER(Shape),
                                        ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        vp]
    lib.blasst_attn_prefill_masked.restype = ctypes.c_int
    lib.blasst_attn_prefill_masked.argtypes = [vp, vp, vp, u8p, ctypes.POINTER(ctypes.c_int64), vp,
                                               u8p, fp, i64p, ctypes.POINTER(Shape),
                                               ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                               ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, vp]
    lib.blasst_attn_prefill_backward.restype = ctypes.c_int
    lib.blasst_attn_prefill_backward.argtypes = [vp, vp, vp, vp, vp, fp, u8p, fp, fp, fp,
                                                 ctypes.POINTER(Shape), ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t,
                                                 vp]
    lib.blasst_prefill_backward_workspace_size.restype = ctypes.c_int
    lib.blasst_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int,
                                                           ctypes.c_int, ctypes.c_int,
                                                           ctypes.c_int,
                                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.blasst_quantize_mxfp4.restype = ctypes.c_int
    lib.blasst_quantize_mxfp4.argtypes = [vp, ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int, u8p, u8p, vp]
    lib.blasst_attn_prefill_twopass.restype = ctypes.c_int
    lib.blasst_attn_prefill_twopass.argtypes = [vp, vp, vp, vp, u8p, fp, i64p, ctypes.POINTER(Shape),
                                                ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.blasst_prefill_twopass_workspace_size.restype = ctypes.c_int
    lib.blasst_prefill_twopass_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int,
                                                          ctypes.c_int, ctypes.c_int,
                                                          ctypes.c_int,
                                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.blasst_attn_decode.restype = ctypes.c_int
    lib.blasst_attn_decode.argtypes = [vp, vp, vp, vp, u8p, fp, i64p, ctypes.POINTER(Shape),
                                       ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.blasst_decode_workspace_size.restype = ctypes.c_int
    lib.blasst_decode_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.blasst_attn_decode_noalloc.restype = ctypes.c_int
    lib.blasst_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, u8p, fp, i64p, ctypes.POINTER(Shape),
                                               ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                               ctypes.c_float, ctypes.c_int, vp]
    lib.blasst_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.blasst_attn_decode_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int,
                                                      ctypes.c_int]
    lib.blasst_status_string.restype = ctypes.c_char_p
    lib.blasst_status_string.argtypes = [ctypes.c_int]
    lib.blasst_last_error.restype = ctypes.c_char_p
    lib.blasst_last_error.argtypes = []
    lib.blasst_version.restype = ctypes.c_int
    lib.blasst_version.argtypes = []
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        detail = load_library().blasst_last_error().decode(errors="replace")
        raise BlasstError(status, detail)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return BLASST_FP32
    if dt == torch.bfloat16:
        return BLASST_BF16
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _strides3(t: torch.Tensor):
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    s = t.stride()
    return (s[0], s[1], s[2]) if t.dim() == 4 else (s[0], s[1], 0)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _require_device(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libblasst runs on the GPU only: every tensor must be on a HIP device")


@dataclass
class AttnResult:
    out: torch.Tensor
    mask: Optional[torch.Tensor]
    lse: Optional[torch.Tensor]
    stats: Optional[torch.Tensor]

    @property
    def skip_fraction(self) -> float:
        """Dropped / visited key tiles over the whole call (needs stats)."""
        st = self.stats.double()
        visited = st[..., 0].sum().item()
        return 0.0 if visited == 0 else 1.0 - st[..., 1].sum().item() / visited


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: float, causal: bool = True,
            br: Optional[int] = None, bc: int = 64, scale: Optional[float] = None,
            out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
            want_mask: bool = True, want_lse: bool = True,
            want_stats: bool = True) -> AttnResult:
    """Skip-softmax prefill. q [B,Hq,Nq,d], k [B,Hkv,Nk,d], v [B,Hkv,Nk,dv] on one GPU.

    out_dtype defaults to the input dtype; bfloat16 inputs may ask for float32."""
    lib = load_library()
    _require_device(q, k, v, out)
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    if br is None:
        br = 64 if q.dtype == torch.float32 else 128
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, Nq, dv), dtype=out_dtype or q.dtype, device=dev)
    nqt, nkt = -(-Nq // br), -(-Nk // bc)
    mask = torch.empty((B, Hq, nqt, nkt), dtype=torch.uint8, device=dev) if want_mask else None
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev) if want_lse else None
    stats = torch.empty((B, Hq, 2), dtype=torch.int64, device=dev) if want_stats else None
    sh = Shape(B, Hq, Hkv, Nq, Nk, d, dv, _strides3(q), _strides3(k), _strides3(v), _strides3(out))
    st = lib.blasst_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(mask), _ptr(lse),
                                 _ptr(stats), ctypes.byref(sh), _dtype_code(q.dtype),
                                 _dtype_code(out.dtype), float(lam),
                                 float(scale) if scale else 0.0, int(bool(causal)), int(br),
                                 int(bc), _stream(dev))
    _check(st)
    return AttnResult(out, mask, lse, stats)


def prefill_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                   lam: float, causal: bool = True, br: int = 128, bc: int = 64,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None, want_mask: bool = True,
                   want_lse: bool = True, want_stats: bool = True) -> AttnResult:
    """Block-sparse skip-softmax prefill: attention restricted to the blocks that
    ``block_mask`` (bool or uint8, broadcastable to [B, Hq, ceil(Nq/br),
    ceil(Nk/bc)], on the GPU) marks; the skip rule runs inside the set."""
    lib = load_library()
    _require_device(q, k, v, out, block_mask)
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    dev = q.device
    nqt, nkt = -(-Nq // br), -(-Nk // bc)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if block_mask.dtype != torch.uint8:
        raise TypeError("block_mask must be bool or uint8")
    bm = block_mask.expand(B, Hq, nqt, nkt)
    if bm.stride(3) != 1:
        bm = bm.contiguous()
    if out is None:
        out = torch.empty((B, Hq, Nq, dv), dtype=out_dtype or q.dtype, device=dev)
    mask = torch.empty((B, Hq, nqt, nkt), dtype=torch.uint8, device=dev) if want_mask else None
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev) if want_lse else None
    stats = torch.empty((B, Hq, 2), dtype=torch.int64, device=dev) if want_stats else None
    sh = Shape(B, Hq, Hkv, Nq, Nk, d, dv, _strides3(q), _strides3(k), _strides3(v), _strides3(out))
    bms = (ctypes.c_int64 * 3)(bm.stride(0), bm.stride(1), bm.stride(2))
    st = lib.blasst_attn_prefill_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(bm), bms, _ptr(out),
                                        _ptr(mask), _ptr(lse), _ptr(stats), ctypes.byref(sh),
                                        _dtype_code(q.dtype), _dtype_code(out.dtype), float(lam),
                                        float(scale) if scale else 0.0, int(bool(causal)),
                                        int(br), int(bc), _stream(dev))
    _check(st)
    return AttnResult(out, mask, lse, stats)


def prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                     dout: torch.Tensor, lse: torch.Tensor, mask: torch.Tensor,
                     causal: bool = True, br: int = 128, bc: int = 64,
                     scale: Optional[float] = None,
                     workspace: Optional[torch.Tensor] = None) -> tuple:
    """Gradients (dq, dk, dv), float32, of a bf16 skip-softmax prefill with its
    tile mask held fixed. out, lse and mask are the forward's outputs; dout is
    the gradient of the loss with respect to out (bf16)."""
    lib = load_library()
    _require_device(q, k, v, out, dout, lse, mask)
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv_ = k.shape[1], k.shape[2], v.shape[3]
    dev = q.device
    if dout.dtype != torch.bfloat16:
        raise TypeError("dout must be bfloat16")
    if dout.stride() != out.stride():
        dout, out = dout.contiguous(), out.contiguous()
    lse = lse.contiguous()
    mask = mask.contiguous()
    dq = torch.empty_strided(q.shape, q.stride(), dtype=torch.float32, device=dev)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=torch.float32, device=dev)
    dv = torch.empty_strided(v.shape, v.stride(), dtype=torch.float32, device=dev)
    sh = Shape(B, Hq, Hkv, Nq, Nk, d, dv_, _strides3(q), _strides3(k), _strides3(v),
               _strides3(out))
    n = ctypes.c_size_t(0)
    _check(lib.blasst_prefill_backward_workspace_size(ctypes.byref(sh), _dtype_code(q.dtype),
                                                      int(bool(causal)), int(br), int(bc),
                                                      ctypes.byref(n)))
    if workspace is None:
        workspace = _workspace(n.value, dev)
    st = lib.blasst_attn_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(mask), _ptr(dq),
        _ptr(dk), _ptr(dv), ctypes.byref(sh), _dtype_code(q.dtype), _dtype_code(out.dtype),
        float(scale) if scale else 0.0, int(bool(causal)), int(br), int(bc), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return dq, dk, dv


def quantize_mxfp4(x: torch.Tensor) -> tuple:
    """MXFP4 codes and E8M0 scales of a bf16 [d0, d1, n, d] tensor (features
    contiguous): codes uint8 [d0, d1, n, d / 2] (two per byte, the even
    feature in the low nibble), scales uint8 [d0, d1, n, d / 32]."""
    lib = load_library()
    _require_device(x)
    d0, d1, n, d = x.shape
    codes = torch.empty((d0, d1, n, d // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((d0, d1, n, max(d // 32, 0)), dtype=torch.uint8, device=x.device)
    xs = (ctypes.c_int64 * 3)(*_strides3(x))
    _check(lib.blasst_quantize_mxfp4(_ptr(x), xs, d0, d1, n, d, _dtype_code(x.dtype), _ptr(codes),
                                     _ptr(scales), _stream(x.device)))
    return codes, scales


def prefill_twopass_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int = 128,
                                   dv: int = 128, causal: bool = True, br: int = 128,
                                   bc: int = 64, dtype: torch.dtype = torch.bfloat16) -> int:
    """Bytes of device workspace blasst_attn_prefill_twopass needs."""
    lib = load_library()
    z = (0, 0, 0)
    sh = Shape(B, Hq, Hkv, Nq, Nk, d, dv, z, z, z, z)
    n = ctypes.c_size_t(0)
    _check(lib.blasst_prefill_twopass_workspace_size(ctypes.byref(sh), _dtype_code(dtype),
                                                     int(bool(causal)), int(br), int(bc),
                                                     ctypes.byref(n)))
    return n.value


def prefill_twopass(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lam: float,
                    causal: bool = True, br: int = 128, bc: int = 64,
                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, want_mask: bool = True,
                    want_lse: bool = True, want_stats: bool = True,
                    workspace: Optional[torch.Tensor] = None) -> AttnResult:
    """Two-pass prefill: the tile map from the skip rule on MXFP4 scores, then
    exact attention over the kept tiles. ``mask`` of the result is that map."""
    lib = load_library()
    _require_device(q, k, v, out, workspace)
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, Nq, dv), dtype=out_dtype or q.dtype, device=dev)
    nqt, nkt = -(-Nq // br), -(-Nk // bc)
    mask = torch.empty((B, Hq, nqt, nkt), dtype=torch.uint8, device=dev) if want_mask else None
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev) if want_lse else None
    stats = torch.empty((B, Hq, 2), dtype=torch.int64, device=dev) if want_stats else None
    sh = Shape(B, Hq, Hkv, Nq, Nk, d, dv, _strides3(q), _strides3(k), _strides3(v), _strides3(out))
    n = ctypes.c_size_t(0)
    _check(lib.blasst_prefill_twopass_workspace_size(ctypes.byref(sh), _dtype_code(q.dtype),
                                                     int(bool(causal)), int(br), int(bc),
                                                     ctypes.byref(n)))
    if workspace is None:
        workspace = _workspace(n.value, dev)
    st = lib.blasst_attn_prefill_twopass(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(mask), _ptr(lse), _ptr(stats), ctypes.byref(sh),
        _dtype_code(q.dtype), _dtype_code(out.dtype), float(lam), float(scale) if scale else 0.0,
        int(bool(causal)), int(br), int(bc), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return AttnResult(out, mask, lse, stats)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor], lam: float,
           bc: int = 64, scale: Optional[float] = None, dv: Optional[int] = None,
           out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
           want_mask: bool = True, want_lse: bool = True, want_stats: bool = True,
           workspace: Optional[torch.Tensor] = None) -> AttnResult:
    """Skip-softmax decode. q [B,Hq,d]; k_cache [B,Hkv,Nk,d]; v_cache [B,Hkv,Nk,dv] or
    None for a latent cache whose values are k_cache[..., :dv]. `workspace` is a
    uint8 device tensor of at least decode_workspace_size(...) bytes; when None
    one is allocated through torch's caching allocator."""
    lib = load_library()
    _require_device(q, k_cache, v_cache, out)
    B, Hq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if v_cache is not None:
        dv = v_cache.shape[3]
    elif dv is None:
        raise ValueError("dv is required for a latent cache")
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=out_dtype or q.dtype, device=dev)
    nkt = -(-Nk // bc)
    mask = torch.empty((B, Hq, nkt), dtype=torch.uint8, device=dev) if want_mask else None
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_lse else None
    stats = torch.empty((B, Hq, 3), dtype=torch.int64, device=dev) if want_stats else None
    vs = _strides3(v_cache) if v_cache is not None else (0, 0, 0)
    sh = Shape(B, Hq, Hkv, 1, Nk, d, dv, _strides3(q), _strides3(k_cache), vs, _strides3(out))
    nbytes = ctypes.c_size_t(0)
    _check(lib.blasst_decode_workspace_size(ctypes.byref(sh), _dtype_code(q.dtype),
                                            int(v_cache is not None), int(bc),
                                            ctypes.byref(nbytes)))
    if workspace is None and nbytes.value > 0:
        workspace = _workspace(nbytes.value, dev)
    if workspace is not None:
        _require_device(workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.blasst_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(mask),
                                _ptr(lse), _ptr(stats), ctypes.byref(sh), _dtype_code(q.dtype),
                                _dtype_code(out.dtype), float(lam),
                                float(scale) if scale else 0.0, int(bc), _ptr(workspace),
                                ws_bytes, _stream(dev))
    _check(st)
    return AttnResult(out, mask, lse, stats)


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                   lam: float, bc: int = 64, scale: Optional[float] = None,
                   dv: Optional[int] = None, out: Optional[torch.Tensor] = None,
                   mask: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   stats: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None) -> AttnResult:
    """blasst_attn_decode_noalloc: the decode with the library's per-GPU static
    scratch in place of a workspace. Outputs the caller passes are written in
    place (nothing is allocated then); missing ones are allocated here with
    torch.empty before the call, as in decode(). Calls on one GPU must not overlap."""
    lib = load_library()
    _require_device(q, k_cache, v_cache, out, mask, lse, stats)
    B, Hq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if v_cache is not None:
        dv = v_cache.shape[3]
    elif dv is None:
        raise ValueError("dv is required for a latent cache")
    dev = q.device
    nkt = -(-Nk // bc)
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=out_dtype or q.dtype, device=dev)
    for t, shp, dt in ((mask, (B, Hq, nkt), torch.uint8), (lse, (B, Hq), torch.float32),
                       (stats, (B, Hq, 3), torch.int64)):
        if t is not None and (tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous()):
            raise ValueError(f"output of shape {tuple(t.shape)} {t.dtype}: expected a contiguous "
                             f"{shp} {dt}")
    vs = _strides3(v_cache) if v_cache is not None else (0, 0, 0)
    sh = Shape(B, Hq, Hkv, 1, Nk, d, dv, _strides3(q), _strides3(k_cache), vs, _strides3(out))
    st = lib.blasst_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                        _ptr(mask), _ptr(lse), _ptr(stats), ctypes.byref(sh),
                                        _dtype_code(q.dtype), _dtype_code(out.dtype), float(lam),
                                        float(scale) if scale else 0.0, int(bc), _stream(dev))
    _check(st)
    return AttnResult(out, mask, lse, stats)


def decode_workspace_size(B: int, Hq: int, Hkv: int, Nk: int, d: int, dv: int,
                          latent: bool, dtype: torch.dtype = torch.bfloat16,
                          bc: int = 64) -> int:
    """Bytes of device workspace blasst_attn_decode needs (0 if none)."""
    lib = load_library()
    z = (0, 0, 0)
    sh = Shape(B, Hq, Hkv, 1, Nk, d, dv, z, z, z, z)
    nbytes = ctypes.c_size_t(0)
    _check(lib.blasst_decode_workspace_size(ctypes.byref(sh), _dtype_code(dtype),
                                            int(not latent), int(bc), ctypes.byref(nbytes)))
    return nbytes.value


def _workspace(nbytes: int, dev: torch.device) -> torch.Tensor:
    # torch's caching allocator hands out 512-byte aligned blocks; the library
    # needs 256
    t = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    assert t.data_ptr() % 256 == 0
    return t


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


__all__ = ["prefill", "prefill_masked", "prefill_backward", "quantize_mxfp4",
           "prefill_twopass", "prefill_twopass_workspace_size", "decode", "decode_noalloc",
           "decode_workspace_size", "load_library", "Shape", "BlasstError", "AttnResult",
           "EXPORTED", "LIB_PATH", "STATUS"]
