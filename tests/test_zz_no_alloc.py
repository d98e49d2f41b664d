"""The allocation-free decode (blasst_attn_decode_noalloc) against the
workspace decode (blasst_attn_decode), through the C ABI.

Both run the same kernels with the same plan, so every output must agree bit
for bit. Two calls in a row on the one static scratch array, the second with
a smaller input, show that nothing carries over between calls; a latent-cache
shape larger than the array is refused before any launch, and a GQA shape
(which needs no scratch) runs too.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_sparse_long_skip_amd import attention as A
from block_sparse_long_skip_amd import synth
from parity import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    A.load_library()
    yield
    torch.cuda.synchronize()


def _inputs(w):
    inp = synth.make_inputs(w)
    q, k = to_device(inp.q, w), to_device(inp.k, w)
    v = to_device(inp.v, w) if inp.v is not None else None
    return q, k, v


def _outputs(w, out_dtype):
    nkt = synth.n_tiles(w.Nk, w.bc)
    return (torch.full((w.B, w.Hq, w.dv), 3.0, dtype=out_dtype, device="cuda"),
            torch.full((w.B, w.Hq, nkt), 9, dtype=torch.uint8, device="cuda"),
            torch.full((w.B, w.Hq), 5.0, dtype=torch.float32, device="cuda"),
            torch.full((w.B, w.Hq, 3), -7, dtype=torch.int64, device="cuda"))


def _same(ref, out, mask, lse, stats):
    assert torch.equal(ref.out.view(torch.int16) if ref.out.dtype == torch.bfloat16 else ref.out,
                       out.view(torch.int16) if out.dtype == torch.bfloat16 else out)
    assert torch.equal(ref.mask, mask)
    assert torch.equal(ref.lse, lse)
    assert torch.equal(ref.stats, stats)


def test_noalloc_matches_workspace_decode_twice_smaller_second():
    big = synth.WORKLOADS[5].with_gain(6.0)   # batch 16, 128 heads, 32768 latent keys
    small = synth.small_workload("decode_mla", d=576, dv=512, dtype="bf16", bc=64, gain=6.0,
                                 seed=58, window=64, B=2, Hq=128, Hkv=1, Nk=5000)
    assert (A.decode_workspace_size(small.B, small.Hq, 1, small.Nk, 576, 512, latent=True)
            < A.decode_workspace_size(big.B, big.Hq, 1, big.Nk, 576, 512, latent=True)
            <= 64 << 20)
    for w, lam, od in ((big, 1e-2, torch.bfloat16), (small, 1e-3, torch.float32)):
        q, k, _ = _inputs(w)
        ref = A.decode(q, k, None, lam, dv=512, out_dtype=od)
        out, mask, lse, stats = _outputs(w, od)
        A.decode_noalloc(q, k, None, lam, dv=512, out=out, mask=mask, lse=lse, stats=stats)
        torch.cuda.synchronize()
        _same(ref, out, mask, lse, stats)
        assert (mask == 0).any(), "the case must drop tiles"
        print(f"{w.name}: bit-identical to the workspace decode, "
              f"{int((mask == 0).sum())} tiles dropped")


def test_noalloc_gqa_and_null_outputs():
    w = synth.small_workload("decode", d=128, dtype="bf16", bc=64, gain=6.0, seed=46,
                             window=64, B=2, Hq=8, Hkv=2, Nk=3000)
    q, k, v = _inputs(w)
    ref = A.decode(q, k, v, 1e-2)
    out, mask, lse, stats = _outputs(w, torch.bfloat16)
    A.decode_noalloc(q, k, v, 1e-2, out=out, mask=mask, lse=lse, stats=stats)
    torch.cuda.synchronize()
    _same(ref, out, mask, lse, stats)
    # optional outputs may be NULL
    out2 = torch.empty_like(out)
    A.decode_noalloc(q, k, v, 1e-2, out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), ref.out.view(torch.int16))


def test_noalloc_refuses_a_shape_beyond_the_scratch():
    """Batch 64 over 65536 latent keys needs more than the 64 MiB array: the
    call is refused before any launch and its output is left untouched."""
    lib = A.load_library()
    B, Hq, Nk = 64, 128, 65536
    need = A.decode_workspace_size(B, Hq, 1, Nk, 576, 512, latent=True)
    assert need > 64 << 20
    q = torch.zeros((B, Hq, 576), dtype=torch.bfloat16, device="cuda")
    # one cache shared by the whole batch (batch stride 0): every address the
    # shape describes lies inside this tensor, whether or not a kernel runs
    k = torch.zeros((1, 1, Nk, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, Hq, 512), 2.0, dtype=torch.bfloat16, device="cuda")
    sh = A.Shape(B, Hq, 1, 1, Nk, 576, 512, (Hq * 576, 576, 0), (0, 0, 576),
                 (0, 0, 0), (Hq * 512, 512, 0))
    st = lib.blasst_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), None, out.data_ptr(), None,
                                        None, None, ctypes.byref(sh), A.BLASST_BF16,
                                        A.BLASST_BF16, ctypes.c_float(1e-3), ctypes.c_float(0.0),
                                        64, None)
    assert st == 6, lib.blasst_last_error()
    assert b"scratch" in lib.blasst_last_error()
    torch.cuda.synchronize()
    assert (out == 2.0).all()
