"""Guard canaries around every output, through the C ABI.

Each output lives inside a larger device buffer filled with 0xFF (NaN in bf16
and fp32, -1 in int64, 255 in the uint8 mask, which holds only 0, 1 and 2):
4 KiB of guard before and after it, and the row-major outputs (out, dq, dk, dv)
as strided views whose rows are padded by 16 poisoned elements. After the call
every guard and padding byte must still be 0xFF, the output itself must hold
no poison, and it must equal, bit for bit, the result of the same call into
plain contiguous tensors.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

from block_sparse_long_skip_amd import attention as A
from block_sparse_long_skip_amd import synth
from parity import to_device

pytestmark = pytest.mark.gpu

GUARD = 4096
PAD = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    A.load_library()
    yield
    torch.cuda.synchronize()


class Guarded:
    """A view of `shape` at GUARD bytes into a 0xFF-filled byte buffer; with
    pad the last dimension's rows carry PAD more poisoned elements."""

    def __init__(self, shape, dtype, pad=False):
        self.shape = tuple(shape)
        self.dtype = dtype
        full = list(shape)
        if pad:
            full[-1] += PAD
        n = int(np.prod(full)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD + n + GUARD,), 0xFF, dtype=torch.uint8, device="cuda")
        self.full = self.buf[GUARD:GUARD + n].view(dtype).view(full)
        self.t = self.full[..., :shape[-1]] if pad else self.full
        self.pad = pad

    def check(self, label):
        b = self.buf.cpu().numpy()
        assert (b[:GUARD] == 0xFF).all(), f"{label}: guard before the output was written"
        assert (b[-GUARD:] == 0xFF).all(), f"{label}: guard after the output was written"
        if self.pad:
            tail = self.full[..., self.shape[-1]:].contiguous().view(torch.uint8).cpu().numpy()
            assert (tail == 0xFF).all(), f"{label}: row padding was written"
        body = self.t.contiguous().view(torch.uint8).cpu().numpy()
        el = self.t.element_size()
        poisoned = (body.reshape(-1, el) == 0xFF).all(axis=1)
        assert not poisoned.any(), f"{label}: {int(poisoned.sum())} elements left unwritten"


def _same(a, b, label):
    a, b = a.contiguous(), b.contiguous()
    assert a.dtype == b.dtype and a.shape == b.shape, label
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{label}: bits differ"


def _shape(q, k, v, o, d, dv, decode=False):
    Bq, Hq = q.shape[0], q.shape[1]
    Nq = 1 if decode else q.shape[2]
    vs = A._strides3(v) if v is not None else (0, 0, 0)
    return A.Shape(Bq, Hq, k.shape[1], Nq, k.shape[2], d, dv, A._strides3(q), A._strides3(k), vs,
                   A._strides3(o))


def _check_status(st):
    assert st == 0, A.load_library().blasst_last_error().decode()


@pytest.mark.parametrize("kind", ["bf16_to_bf16", "bf16_to_fp32", "fp32", "masked", "twopass"])
def test_prefill_outputs_guarded(kind):
    lib = A.load_library()
    f32 = kind == "fp32"
    d, br = (64, 64) if f32 else (128, 128)
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=300, Nk=700, d=d,
                             dtype="fp32" if f32 else "bf16", br=br, bc=64, seed=61, gain=6.0,
                             window=32)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    od = torch.float32 if kind in ("bf16_to_fp32", "fp32") else torch.bfloat16
    lam = 1e-2
    sel = synth.block_set(w, 0.4, seed=5) if kind == "masked" else None
    bm = torch.from_numpy(sel).cuda() if sel is not None else None
    if kind == "masked":
        ref = A.prefill_masked(q, k, v, bm, lam, out_dtype=od)
    elif kind == "twopass":
        ref = A.prefill_twopass(q, k, v, lam, out_dtype=od)
    else:
        ref = A.prefill(q, k, v, lam, br=br, out_dtype=od)
    nqt, nkt = synth.n_tiles(w.Nq, br), synth.n_tiles(w.Nk, 64)
    out = Guarded((w.B, w.Hq, w.Nq, w.dv), od, pad=True)
    mask = Guarded((w.B, w.Hq, nqt, nkt), torch.uint8)
    lse = Guarded((w.B, w.Hq, w.Nq), torch.float32)
    stats = Guarded((w.B, w.Hq, 2), torch.int64)
    sh = _shape(q, k, v, out.t, w.d, w.dv)
    dt, odt = A._dtype_code(q.dtype), A._dtype_code(od)
    stream = A._stream(q.device)
    if kind == "masked":
        bms = (ctypes.c_int64 * 3)(bm.stride(0), bm.stride(1), bm.stride(2))
        st = lib.blasst_attn_prefill_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), bm.data_ptr(),
                                            bms, out.t.data_ptr(), mask.t.data_ptr(),
                                            lse.t.data_ptr(), stats.t.data_ptr(), ctypes.byref(sh),
                                            dt, odt, lam, 0.0, 1, br, 64, stream)
    elif kind == "twopass":
        n = A.prefill_twopass_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        st = lib.blasst_attn_prefill_twopass(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             out.t.data_ptr(), mask.t.data_ptr(), lse.t.data_ptr(),
                                             stats.t.data_ptr(), ctypes.byref(sh), dt, odt, lam, 0.0,
                                             1, br, 64, ws.data_ptr(), n, stream)
    else:
        st = lib.blasst_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.t.data_ptr(),
                                     mask.t.data_ptr(), lse.t.data_ptr(), stats.t.data_ptr(),
                                     ctypes.byref(sh), dt, odt, lam, 0.0, 1, br, 64, stream)
    _check_status(st)
    torch.cuda.synchronize()
    for g, r, name in ((out, ref.out, "out"), (mask, ref.mask, "mask"), (lse, ref.lse, "lse"),
                       (stats, ref.stats, "stats")):
        g.check(f"{kind} {name}")
        _same(g.t, r, f"{kind} {name}")
    assert (ref.mask == 0).any(), "the case must drop tiles"


@pytest.mark.parametrize("latent", [False, True])
def test_decode_outputs_guarded(latent):
    lib = A.load_library()
    if latent:
        w = synth.small_workload("decode_mla", d=576, dv=512, dtype="bf16", bc=64, gain=6.0,
                                 seed=62, window=64, B=2, Hq=64, Hkv=1, Nk=3000)
    else:
        w = synth.small_workload("decode", d=128, dtype="bf16", bc=64, gain=6.0, seed=63,
                                 window=64, B=3, Hq=8, Hkv=2, Nk=2000)
    inp = synth.make_inputs(w)
    q, k = to_device(inp.q, w), to_device(inp.k, w)
    v = to_device(inp.v, w) if inp.v is not None else None
    lam = 1e-2
    ref = A.decode(q, k, v, lam, dv=w.dv)
    nkt = synth.n_tiles(w.Nk, 64)
    out = Guarded((w.B, w.Hq, w.dv), torch.bfloat16, pad=True)
    mask = Guarded((w.B, w.Hq, nkt), torch.uint8)
    lse = Guarded((w.B, w.Hq), torch.float32)
    stats = Guarded((w.B, w.Hq, 3), torch.int64)
    sh = _shape(q, k, v, out.t, w.d, w.dv, decode=True)
    n = A.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.dv, latent=latent)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    st = lib.blasst_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr() if v is not None else None,
                                out.t.data_ptr(), mask.t.data_ptr(), lse.t.data_ptr(),
                                stats.t.data_ptr(), ctypes.byref(sh), A.BLASST_BF16, A.BLASST_BF16,
                                lam, 0.0, 64, ws.data_ptr(), n, A._stream(q.device))
    _check_status(st)
    torch.cuda.synchronize()
    for g, r, name in ((out, ref.out, "out"), (mask, ref.mask, "mask"), (lse, ref.lse, "lse"),
                       (stats, ref.stats, "stats")):
        g.check(f"decode latent={latent} {name}")
        _same(g.t, r, f"decode latent={latent} {name}")
    assert (ref.mask == 0).any(), "the case must drop tiles"


def test_backward_outputs_guarded():
    """dq, dk and dv take the element strides of q, k and v: padded inputs give
    padded gradients, whose padding must stay poisoned."""
    lib = A.load_library()
    w = synth.small_workload("prefill", B=1, Hq=4, Hkv=2, Nq=300, Nk=500, d=128, dtype="bf16",
                             br=128, bc=64, seed=64, gain=6.0, window=32)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    fwd = A.prefill(q, k, v, 1e-2)
    g = np.random.default_rng(3).standard_normal((w.B, w.Hq, w.Nq, w.dv)).astype(np.float32)
    dout = torch.from_numpy(g).to(torch.bfloat16).cuda()
    ref = A.prefill_backward(q, k, v, fwd.out, dout, fwd.lse, fwd.mask)
    # padded copies of the inputs (same values) and gradients with their strides
    qp, kp, vp = (Guarded(x.shape, torch.bfloat16, pad=True) for x in (q, k, v))
    for gp, x in ((qp, q), (kp, k), (vp, v)):
        gp.t.copy_(x)
    dq, dk, dv = (Guarded(x.shape, torch.float32, pad=True) for x in (q, k, v))
    assert dq.t.stride() == qp.t.stride() and dk.t.stride() == kp.t.stride()
    sh = _shape(qp.t, kp.t, vp.t, fwd.out, w.d, w.dv)
    n = ctypes.c_size_t(0)
    _check_status(lib.blasst_prefill_backward_workspace_size(ctypes.byref(sh), A.BLASST_BF16, 1,
                                                             128, 64, ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    st = lib.blasst_attn_prefill_backward(
        qp.t.data_ptr(), kp.t.data_ptr(), vp.t.data_ptr(), fwd.out.data_ptr(), dout.data_ptr(),
        fwd.lse.data_ptr(), fwd.mask.data_ptr(), dq.t.data_ptr(), dk.t.data_ptr(),
        dv.t.data_ptr(), ctypes.byref(sh), A.BLASST_BF16, A.BLASST_BF16, 0.0, 1, 128, 64,
        ws.data_ptr(), n.value, A._stream(q.device))
    _check_status(st)
    torch.cuda.synchronize()
    for gp, r, name in ((dq, ref[0], "dq"), (dk, ref[1], "dk"), (dv, ref[2], "dv")):
        gp.check(f"backward {name}")
        _same(gp.t, r, f"backward {name}")
    for gp in (qp, kp, vp):
        gp.check("backward input (read only)")
