"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (so these
calls never reach the device). Pointers here are fake, 16-byte-aligned
addresses: every case below fails validation before anything is launched."""
import ctypes
import math
import os
import re

import pytest

from block_sparse_long_skip_amd import attention as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blasst.h")

pytestmark = pytest.mark.skipif(not os.path.exists(A.LIB_PATH),
                                reason="libblasst.so not built (python -m block_sparse_long_skip_amd.build)")

P = 0x10000  # fake aligned device addresses, never dereferenced
BF16, FP32 = A.BLASST_BF16, A.BLASST_FP32


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(blasst_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = A.load_library()
    declared = _header_functions()
    assert set(declared) == set(A.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.blasst_version() == 230


def test_status_strings():
    lib = A.load_library()
    for code, name in A.STATUS.items():
        assert lib.blasst_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.blasst_status_string(99)


def _shape(B=1, Hq=4, Hkv=2, Nq=256, Nk=256, d=128, dv=128, elem=2):
    def st(n, dd):
        return (Hq * n * dd, n * dd, dd)
    return A.Shape(B, Hq, Hkv, Nq, Nk, d, dv, st(Nq, d), (Hkv * Nk * d, Nk * d, d),
                   (Hkv * Nk * dv, Nk * dv, dv), st(Nq, dv))


def _prefill(sh, q=P, k=P, v=P, out=P, dtype=BF16, lam=1e-3, scale=0.0, causal=1, br=128, bc=64,
             shape_ptr=True, out_dtype=None):
    lib = A.load_library()
    return lib.blasst_attn_prefill(q, k, v, out, None, None, None,
                                   ctypes.byref(sh) if shape_ptr else None, dtype,
                                   dtype if out_dtype is None else out_dtype, lam, scale,
                                   causal, br, bc, None)


def _decode(sh, q=P, k=P, v=P, out=P, mask=None, stats=None, dtype=BF16, lam=1e-3, bc=64,
            out_dtype=None, ws=None, ws_bytes=0):
    lib = A.load_library()
    return lib.blasst_attn_decode(q, k, v, out, mask, None, stats, ctypes.byref(sh), dtype,
                                  dtype if out_dtype is None else out_dtype, lam, 0.0, bc, ws,
                                  ws_bytes, None)


def _ws_size(sh, has_v, dtype=BF16, bc=64):
    n = ctypes.c_size_t(12345)
    st = A.load_library().blasst_decode_workspace_size(ctypes.byref(sh), dtype, int(has_v), bc,
                                                        ctypes.byref(n))
    return st, n.value


def _err():
    return A.load_library().blasst_last_error().decode()


@pytest.mark.parametrize("case,expect", [
    ("null_shape", 1), ("null_q", 1), ("null_v", 1), ("bad_dtype", 3), ("heads", 2),
    ("causal_nq_gt_nk", 2), ("neg_len", 2), ("lam_neg", 4), ("lam_gt1", 4), ("lam_nan", 4),
    ("scale_inf", 7), ("misaligned_ptr", 5), ("misaligned_stride", 5), ("bad_d", 6),
    ("bad_tile", 6), ("f32_wrong_d", 6), ("zero_tile", 2), ("f32_in_bf16_out", 3),
    ("bad_out_dtype", 3), ("overlapping_kv_rows", 2),
])
def test_prefill_validation(case, expect):
    sh = _shape()
    kw = {}
    if case == "null_shape":
        kw["shape_ptr"] = False
    elif case == "null_q":
        kw["q"] = None
    elif case == "null_v":
        kw["v"] = None
    elif case == "bad_dtype":
        kw["dtype"] = 5
    elif case == "heads":
        sh.heads_q = 3
    elif case == "causal_nq_gt_nk":
        sh.len_q, sh.len_kv = 300, 200
    elif case == "neg_len":
        sh.len_q = -1
    elif case == "lam_neg":
        kw["lam"] = -0.1
    elif case == "lam_gt1":
        kw["lam"] = 1.5
    elif case == "lam_nan":
        kw["lam"] = math.nan
    elif case == "scale_inf":
        kw["scale"] = math.inf
    elif case == "misaligned_ptr":
        kw["k"] = P + 8
    elif case == "misaligned_stride":
        sh.q_stride[2] = 100  # 200 bytes, not a multiple of 16
    elif case == "bad_d":
        sh.d_qk = sh.d_v = 96
    elif case == "bad_tile":
        kw["br"] = 64
    elif case == "f32_wrong_d":
        kw["dtype"], kw["br"] = FP32, 64
    elif case == "zero_tile":
        kw["bc"] = 0
    elif case == "f32_in_bf16_out":
        kw["dtype"], kw["out_dtype"], kw["br"] = FP32, BF16, 64
        sh.d_qk = sh.d_v = 64
    elif case == "bad_out_dtype":
        kw["out_dtype"] = 9
    elif case == "overlapping_kv_rows":
        sh.k_stride[2] = 64
    assert _prefill(sh, **kw) == expect, _err()
    assert _err() != ""


def _prefill_masked(sh, bm=P, bms=(0, 0, 4), dtype=BF16, br=128, bc=64, lam=1e-3, q=P):
    lib = A.load_library()
    strides = None if bms is None else (ctypes.c_int64 * 3)(*bms)
    return lib.blasst_attn_prefill_masked(q, P, P, bm, strides, P, None, None, None,
                                          ctypes.byref(sh), dtype, dtype, lam, 0.0, 1, br, bc,
                                          None)


@pytest.mark.parametrize("case,expect", [
    ("null_block_mask", 1), ("null_strides", 1), ("negative_stride", 2), ("f32", 6),
    ("too_many_key_tiles", 6), ("bad_tile", 6), ("null_q", 1), ("lam", 4),
])
def test_prefill_masked_validation(case, expect):
    sh = _shape()
    kw = {}
    if case == "null_block_mask":
        kw["bm"] = None
    elif case == "null_strides":
        kw["bms"] = None
    elif case == "negative_stride":
        kw["bms"] = (0, -4, 4)
    elif case == "f32":
        sh = _shape(d=64, dv=64)
        kw["dtype"], kw["br"] = FP32, 64
    elif case == "too_many_key_tiles":
        sh = _shape(Nq=128, Nk=6144 * 64 + 1)
    elif case == "bad_tile":
        kw["br"] = 64
    elif case == "null_q":
        kw["q"] = None
    elif case == "lam":
        kw["lam"] = -1.0
    assert _prefill_masked(sh, **kw) == expect, _err()
    assert _err() != ""


def _backward(sh, dtype=BF16, br=128, bc=64, ws=P, ws_bytes=1 << 30, q=P, lse=P, scale=0.0,
              out_dtype=None, causal=1):
    lib = A.load_library()
    return lib.blasst_attn_prefill_backward(q, P, P, P, P, lse, P, P, P, P, ctypes.byref(sh), dtype,
                                            dtype if out_dtype is None else out_dtype, scale,
                                            causal, br, bc, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_q", 1), ("null_lse", 1), ("f32", 6), ("bad_d", 6), ("bad_tile", 6), ("heads", 2),
    ("causal_nq_gt_nk", 2), ("no_workspace", 9), ("small_workspace", 9),
    ("misaligned_workspace", 9), ("scale_inf", 7), ("misaligned_stride", 5),
    ("overlapping_rows", 2), ("too_many_tiles", 6), ("bad_out_dtype", 3),
])
def test_prefill_backward_validation(case, expect):
    sh = _shape()
    kw = {}
    if case == "null_q":
        kw["q"] = None
    elif case == "null_lse":
        kw["lse"] = None
    elif case == "f32":
        sh = _shape(d=64, dv=64)
        kw["dtype"], kw["br"] = FP32, 64
    elif case == "bad_d":
        sh.d_qk = sh.d_v = 96
    elif case == "bad_tile":
        kw["bc"] = 128
    elif case == "heads":
        sh.heads_q = 3
    elif case == "causal_nq_gt_nk":
        sh.len_q, sh.len_kv = 300, 200
    elif case == "no_workspace":
        kw["ws"] = None
    elif case == "small_workspace":
        kw["ws_bytes"] = 16
    elif case == "misaligned_workspace":
        kw["ws"] = P + 16
    elif case == "scale_inf":
        kw["scale"] = math.inf
    elif case == "misaligned_stride":
        sh.q_stride[1] += 4  # 8 bytes, not a multiple of 16
    elif case == "overlapping_rows":
        sh.k_stride[2] = 64
    elif case == "too_many_tiles":
        sh = _shape(Nq=128, Nk=6144 * 64 + 1)
    elif case == "bad_out_dtype":
        kw["out_dtype"] = 7
    assert _backward(sh, **kw) == expect, _err()
    assert _err() != ""


def test_prefill_backward_workspace_size():
    lib = A.load_library()
    n = ctypes.c_size_t(7)
    sh = _shape(B=2, Hq=4, Hkv=2, Nq=300, Nk=700)
    assert lib.blasst_prefill_backward_workspace_size(ctypes.byref(sh), BF16, 1, 128, 64,
                                                      ctypes.byref(n)) == 0, _err()
    assert n.value >= 2 * 4 * 300 * 4 and n.value % 256 == 0
    assert lib.blasst_prefill_backward_workspace_size(ctypes.byref(sh), FP32, 1, 128, 64,
                                                      ctypes.byref(n)) == 6


def _twopass(sh, dtype=BF16, br=128, bc=64, ws=P, ws_bytes=1 << 30, q=P, mask=P, lam=1e-3,
             scale=0.0, out_dtype=None, causal=1):
    lib = A.load_library()
    return lib.blasst_attn_prefill_twopass(q, P, P, P, mask, P, P, ctypes.byref(sh), dtype,
                                           dtype if out_dtype is None else out_dtype, lam, scale,
                                           causal, br, bc, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_q", 1), ("f32", 6), ("bad_d", 6), ("bad_tile", 6), ("heads", 2), ("causal_nq_gt_nk", 2),
    ("no_workspace", 9), ("no_workspace_no_mask", 9), ("small_workspace", 9),
    ("misaligned_workspace", 9), ("lam", 4), ("scale_inf", 7), ("misaligned_stride", 5),
    ("too_many_key_tiles", 6), ("bad_out_dtype", 3), ("null_shape", 1),
])
def test_prefill_twopass_validation(case, expect):
    sh = _shape()
    kw = {}
    if case == "null_q":
        kw["q"] = None
    elif case == "f32":
        sh = _shape(d=64, dv=64)
        kw["dtype"], kw["br"] = FP32, 64
    elif case == "bad_d":
        sh.d_qk = sh.d_v = 96
    elif case == "bad_tile":
        kw["bc"] = 128
    elif case == "heads":
        sh.heads_q = 3
    elif case == "causal_nq_gt_nk":
        sh.len_q, sh.len_kv = 300, 200
    elif case == "no_workspace":
        kw["ws"] = None
    elif case == "no_workspace_no_mask":
        kw["ws"], kw["mask"] = None, None
    elif case == "small_workspace":
        kw["ws_bytes"] = 16
    elif case == "misaligned_workspace":
        kw["ws"] = P + 16
    elif case == "lam":
        kw["lam"] = 1.5
    elif case == "scale_inf":
        kw["scale"] = math.inf
    elif case == "misaligned_stride":
        sh.q_stride[1] += 4
    elif case == "too_many_key_tiles":
        sh = _shape(Nq=128, Nk=6144 * 64 + 1)
    elif case == "bad_out_dtype":
        kw["out_dtype"] = 7
    if case == "null_shape":
        lib = A.load_library()
        st = lib.blasst_attn_prefill_twopass(P, P, P, P, P, P, P, None, BF16, BF16, 1e-3, 0.0, 1,
                                             128, 64, P, 1 << 30, None)
        assert st == expect, _err()
    else:
        assert _twopass(sh, **kw) == expect, _err()
    assert _err() != ""


def test_prefill_twopass_workspace_size():
    lib = A.load_library()
    n = ctypes.c_size_t(7)
    sh = _shape(B=2, Hq=4, Hkv=2, Nq=300, Nk=700)
    assert lib.blasst_prefill_twopass_workspace_size(ctypes.byref(sh), BF16, 1, 128, 64,
                                                     ctypes.byref(n)) == 0, _err()
    need = (2 * 4 * 300 * (64 + 4) + 2 * 2 * 700 * (64 + 4) + 2 * 4 * 3 * 11)
    assert need <= n.value <= need + 5 * 256 and n.value % 256 == 0
    assert lib.blasst_prefill_twopass_workspace_size(ctypes.byref(sh), BF16, 1, 64, 64,
                                                     ctypes.byref(n)) == 6


@pytest.mark.parametrize("case,expect", [
    ("null_x", 1), ("null_codes", 1), ("d_not_multiple", 2), ("d_zero", 2), ("negative_n", 2),
    ("f32", 3), ("misaligned_x", 5), ("misaligned_codes", 5), ("misaligned_stride", 5),
])
def test_quantize_mxfp4_validation(case, expect):
    lib = A.load_library()
    x, codes, d, n, dtype = P, P, 128, 10, BF16
    stride = [4 * 10 * 128, 10 * 128, 128]
    if case == "null_x":
        x = None
    elif case == "null_codes":
        codes = None
    elif case == "d_not_multiple":
        d = 48
    elif case == "d_zero":
        d = 0
    elif case == "negative_n":
        n = -1
    elif case == "f32":
        dtype = FP32
    elif case == "misaligned_x":
        x = P + 2
    elif case == "misaligned_codes":
        codes = P + 8
    elif case == "misaligned_stride":
        stride[2] = 132
    st = lib.blasst_quantize_mxfp4(x, (ctypes.c_int64 * 3)(*stride), 1, 4, n, d, dtype, codes, P,
                                   None)
    assert st == expect, _err()
    assert _err() != ""


@pytest.mark.parametrize("case,expect", [
    ("len_q", 2), ("latent_dv", 2), ("gqa_too_many_heads", 6), ("bad_bc", 6),
    ("null_k", 1), ("lam", 4), ("f32", 6), ("mla_no_workspace", 9),
    ("mla_small_workspace", 9), ("mla_misaligned_workspace", 9), ("mla_overlapping_rows", 2),
])
def test_decode_validation(case, expect):
    sh = _shape(Hq=8, Hkv=2, Nq=1, Nk=1000)
    kw = {}
    if case == "len_q":
        sh.len_q = 2
    elif case == "latent_dv":
        kw["v"] = None
        sh.d_v = sh.d_qk
    elif case == "gqa_too_many_heads":
        sh.heads_q, sh.heads_kv = 64, 2
    elif case == "bad_bc":
        kw["bc"] = 128
    elif case.startswith("mla_"):
        sh = _shape(Hq=32, Hkv=1, Nq=1, Nk=1000, d=576, dv=512)
        kw["v"], kw["stats"], kw["mask"] = None, P, P
        need = _ws_size(sh, False)[1]
        if case == "mla_small_workspace":
            kw["ws"], kw["ws_bytes"] = P, need - 1
        elif case == "mla_misaligned_workspace":
            kw["ws"], kw["ws_bytes"] = P + 16, need
        elif case == "mla_overlapping_rows":
            kw["ws"], kw["ws_bytes"] = P, need
            sh.k_stride[2] = 512
    elif case == "null_k":
        kw["k"] = None
    elif case == "lam":
        kw["lam"] = 2.0
    elif case == "f32":
        kw["dtype"] = FP32
    assert _decode(sh, **kw) == expect, _err()


def test_decode_workspace_size():
    """GQA decode over enough (batch, KV head) pairs needs no workspace; fewer
    pairs split the cache and need one for the scores, maxima and partials; a
    latent cache needs one that grows with the cache length and the batch, and
    the query validates like the call."""
    st, n = _ws_size(_shape(B=32, Hq=32, Hkv=8, Nq=1, Nk=65536), True)
    assert (st, n) == (0, 0)
    st, n = _ws_size(_shape(B=1, Hq=32, Hkv=8, Nq=1, Nk=65536), True)
    # at least the stored scores: 64 floats per (KV head, tile, query head)
    assert st == 0 and n >= 8 * 1024 * 4 * 64 * 4 and n % 256 == 0
    st, n = _ws_size(_shape(Hq=8, Hkv=2, Nq=1, Nk=64), True)
    assert (st, n) == (0, 0)  # a single tile: nothing to split
    sizes = []
    for B, Nk in [(1, 1000), (1, 64000), (4, 64000)]:
        st, n = _ws_size(_shape(B=B, Hq=128, Hkv=1, Nq=1, Nk=Nk, d=576, dv=512), False)
        assert st == 0 and n > 0 and n % 256 == 0, _err()
        # at least the tile maxima and one partial output row per (batch, head)
        assert n >= B * 128 * (4 * -(-Nk // 64) + 4 * 512)
        sizes.append(n)
    assert sizes[0] < sizes[1] < sizes[2]
    st, _ = _ws_size(_shape(B=0, Hq=128, Hkv=1, Nq=1, Nk=64, d=576, dv=512), False)
    assert st == 0
    assert _ws_size(_shape(Hq=8, Hkv=2, Nq=2, Nk=1000), True)[0] == 2
    assert _ws_size(_shape(Hq=8, Hkv=2, Nq=1, Nk=1000, d=96, dv=96), True)[0] == 6
    lib = A.load_library()
    sh = _shape(Hq=8, Hkv=2, Nq=1, Nk=1000)
    assert lib.blasst_decode_workspace_size(ctypes.byref(sh), BF16, 1, 64, None) == 1


def test_attn_decode_workspace_size_contract_form():
    """blasst_attn_decode_workspace_size(shape, dtype, bc) takes the cache kind
    from the sizes and returns the same bytes as the status-returning query;
    SIZE_MAX, with the reason in blasst_last_error, for anything with no kernel."""
    lib = A.load_library()
    size_max = ctypes.c_size_t(-1).value
    for sh, has_v in [(_shape(Hq=8, Hkv=2, Nq=1, Nk=1000), True),
                      (_shape(B=32, Hq=32, Hkv=8, Nq=1, Nk=4096), True),
                      (_shape(B=3, Hq=128, Hkv=1, Nq=1, Nk=9000, d=576, dv=512), False),
                      (_shape(B=1, Hq=20, Hkv=2, Nq=1, Nk=300, d=576, dv=512), False)]:
        st, n = _ws_size(sh, has_v)
        assert st == 0
        assert lib.blasst_attn_decode_workspace_size(ctypes.byref(sh), BF16, 64) == n
    bad = [(_shape(Hq=8, Hkv=2, Nq=2, Nk=1000), BF16, 64),            # len_q != 1
           (_shape(Hq=8, Hkv=2, Nq=1, Nk=1000, d=96, dv=96), BF16, 64),  # no kernel
           (_shape(Hq=8, Hkv=2, Nq=1, Nk=1000), FP32, 64),            # no fp32 decode
           (_shape(Hq=8, Hkv=2, Nq=1, Nk=1000), BF16, 32)]            # tile size
    for sh, dt, bc in bad:
        assert lib.blasst_attn_decode_workspace_size(ctypes.byref(sh), dt, bc) == size_max
        assert _err() != ""
    assert lib.blasst_attn_decode_workspace_size(None, BF16, 64) == size_max


def test_binding_has_no_cpu_fallback():
    """The Python binding refuses CPU tensors instead of computing anything."""
    import torch
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(Exception):
        A.prefill(q, q, q, 0.0)


def test_empty_calls_accept_null_tensors():
    """A tensor pointer may be NULL when the tensor has no elements; such calls
    succeed (no query rows and no statistics: nothing to launch)."""
    lib = A.load_library()
    sh = _shape(B=0)
    assert lib.blasst_attn_prefill(None, None, None, None, None, None, None, ctypes.byref(sh), BF16,
                                   BF16, 1e-3, 0.0, 1, 128, 64, None) == 0, _err()
    bms = (ctypes.c_int64 * 3)(0, 0, 0)
    assert lib.blasst_attn_prefill_masked(None, None, None, None, bms, None, None, None, None,
                                          ctypes.byref(sh), BF16, BF16, 1e-3, 0.0, 1, 128, 64,
                                          None) == 0, _err()
    assert lib.blasst_attn_prefill_twopass(None, None, None, None, None, None, None, ctypes.byref(sh),
                                           BF16, BF16, 1e-3, 0.0, 1, 128, 64, None, 0, None) == 0, _err()
    assert lib.blasst_attn_prefill_backward(None, None, None, None, None, None, None, None, None, None,
                                            ctypes.byref(sh), BF16, BF16, 0.0, 1, 128, 64, None, 0,
                                            None) == 0, _err()
    # decode: a NULL v_cache selects the latent layout, so an empty GQA call
    # passes some V pointer and an empty latent call passes none
    shd = _shape(B=0, Hq=8, Hkv=2, Nq=1, Nk=1000)
    assert lib.blasst_attn_decode(None, None, P, None, None, None, None, ctypes.byref(shd), BF16,
                                  BF16, 1e-3, 0.0, 64, None, 0, None) == 0, _err()
    shl = _shape(B=0, Hq=128, Hkv=1, Nq=1, Nk=1000, d=576, dv=512)
    assert lib.blasst_attn_decode(None, None, None, None, None, None, None, ctypes.byref(shl), BF16,
                                  BF16, 1e-3, 0.0, 64, None, 0, None) == 0, _err()
    assert lib.blasst_quantize_mxfp4(None, (ctypes.c_int64 * 3)(0, 0, 128), 1, 4, 0, 128, BF16, None,
                                     None, None) == 0, _err()
    # no query rows but a key range: q and out may be NULL, k and v may not
    sh = _shape(Nq=0)
    assert lib.blasst_attn_prefill(None, P, P, None, None, None, None, ctypes.byref(sh), BF16, BF16,
                                   1e-3, 0.0, 1, 128, 64, None) == 0, _err()
    assert lib.blasst_attn_prefill(None, None, P, None, None, None, None, ctypes.byref(sh), BF16,
                                   BF16, 1e-3, 0.0, 1, 128, 64, None) == 1
    # a block-sparse call still needs its strides
    assert lib.blasst_attn_prefill_masked(None, P, P, None, None, None, None, None, None,
                                          ctypes.byref(sh), BF16, BF16, 1e-3, 0.0, 1, 128, 64,
                                          None) == 1
