"""GPU parity of the prefill backward (dq, dk, dv with the forward's mask held
fixed) against the oracle's gradients, through the C ABI.

Every input of the GPU backward comes from the generator or the oracle: the
mask, lse and output of the forward are the oracle's (the output rounded to the
type the call stores), so both sides differentiate the same function and no
oracle input comes from the GPU.

For a call whose forward output is stored in bf16, delta = rowsum(dout * out)
is taken from that stored output on both sides (the oracle's output, rounded).

Bar, element by element: the kernels round P and dS to bf16 before their
products and accumulate in fp32. With u = 2^-8, the unit roundoff of bf16
(8 significand bits, nearest even), that rounding moves each product of an
element by at most u times its absolute value, so by at most u M in total,
where M is the sum of the absolute values of the products the element is made
of (M = scale |dS| |k| for dq, scale |dS|^T |q| for dk, |P|^T |dout| for dv,
from the oracle). A second u M covers the fp32 arithmetic that forms P and dS
before the rounding (the exponential, dP - delta): |err| <= 2u M +
1e-5 (1 + max|ref|), the last term for the fp32 accumulation of dP and delta,
which cancel where one key dominates a row. A tensor-wide bound would not do: dq = scale sum_j dS_j k_j
with sum_j dS_j = 0, so it cancels heavily when the keys share a large
component (the planted direction at gain 6).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_skip_amd import attention as A
from block_sparse_long_skip_amd import synth
from parity import to_device

pytestmark = pytest.mark.gpu

U = 2.0 ** -8  # bf16 unit roundoff


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    A.load_library()
    yield
    torch.cuda.synchronize()


def _dout(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.f32_to_bf16_bits(x)


def _check(name, got, ref, mag, label):
    got = got.double().cpu().numpy() if isinstance(got, torch.Tensor) else got
    err = np.abs(got - ref)
    bound = 2 * U * mag + 1e-5 * (1.0 + np.abs(ref).max())
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    msg = (f"{label} {name}: max_abs={err.max():.3e} max(err/bound)={(err / bound).max():.3f} "
           f"at {worst}: err={err[worst]:.3e} bound={bound[worst]:.3e} "
           f"rms_rel={np.sqrt((err ** 2).mean() / max((ref ** 2).mean(), 1e-300)):.2e}")
    print(msg)
    assert np.isfinite(got).all(), msg
    assert (err <= bound).all(), msg


def _dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.cuda() if dtype is None else t.to(dtype).cuda()


def _backward(w, inp, fwd, g_np, out="fp32", rows=None, scale=None):
    """GPU backward with the oracle's forward (mask, lse, out) as its inputs.
    rows: optional (mask, lse, out) arrays for the whole call (sampled runs)."""
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    mask, lse, o = rows if rows is not None else (fwd.mask, fwd.lse, fwd.out)
    od = torch.float32 if out == "fp32" else torch.bfloat16
    g = torch.from_numpy(g_np).view(torch.bfloat16).cuda()
    dq, dk, dv = A.prefill_backward(q, k, v, _dev(o, torch.float32).to(od), g,
                                    _dev(lse, torch.float32), _dev(mask), causal=w.causal,
                                    scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


SHAPES = [
    dict(B=1, Hq=2, Hkv=1, Nq=300, Nk=300, causal=True),
    dict(B=2, Hq=4, Hkv=2, Nq=130, Nk=333, causal=True),
    dict(B=1, Hq=2, Hkv=2, Nq=200, Nk=129, causal=False),
    dict(B=1, Hq=1, Hkv=1, Nq=1, Nk=1, causal=True),
    # eight query heads per KV head, an odd key-tile count and a ragged last query tile
    dict(B=1, Hq=8, Hkv=1, Nq=200, Nk=520, causal=True),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("lam,gain,out", [(0.0, 1.0, "fp32"), (1e-2, 6.0, "fp32"),
                                          (1e-3, 1.0, "bf16")])
def test_prefill_backward_small(shape, lam, gain, out):
    w = synth.small_workload("prefill", d=128, dtype="bf16", br=128, bc=64, gain=gain, seed=51,
                             window=32, **shape)
    inp = synth.make_inputs(w)
    qf, kf, vf = (synth.to_float(x, w) for x in (inp.q, inp.k, inp.v))
    fwd = oracle.prefill(qf, kf, vf, lam, w.causal, 128, 64)
    g_np = _dout(np.random.default_rng(5), (w.B, w.Hq, w.Nq, w.dv))
    dq, dk, dv = _backward(w, inp, fwd, g_np, out)
    # delta is taken from the output as stored (rounded to bf16 for a bf16 call)
    o_stored = fwd.out if out == "fp32" else synth.bf16_bits_to_f32(
        synth.f32_to_bf16_bits(fwd.out.astype(np.float32))).astype(np.float64)
    rq, rk, rv, mq, mk, mv = oracle.prefill_backward(qf, kf, vf, synth.to_float(g_np, w), fwd.mask,
                                                     w.causal, 128, 64, magnitudes=True,
                                                     out=o_stored)
    label = f"{shape} lam={lam} g={gain} out={out} dropped={(fwd.mask == 0).sum()}"
    _check("dq", dq, rq, mq, label)
    _check("dk", dk, rk, mk, label)
    _check("dv", dv, rv, mv, label)



@pytest.mark.parametrize("scale", [0.05, 0.2])
def test_prefill_backward_explicit_scale(scale):
    """A softmax scale other than 1/sqrt(d): the forward (oracle) and the
    backward both use it; dq and dk carry it as a factor."""
    w = synth.small_workload("prefill", B=1, Hq=4, Hkv=2, Nq=300, Nk=520, d=128, dtype="bf16",
                             br=128, bc=64, gain=6.0, seed=58, window=32)
    inp = synth.make_inputs(w)
    qf, kf, vf = (synth.to_float(x, w) for x in (inp.q, inp.k, inp.v))
    fwd = oracle.prefill(qf, kf, vf, 1e-2, True, 128, 64, scale=scale)
    assert (fwd.mask == 0).any()
    g_np = _dout(np.random.default_rng(8), (w.B, w.Hq, w.Nq, w.dv))
    dq, dk, dv = _backward(w, inp, fwd, g_np, scale=scale)
    rq, rk, rv, mq, mk, mv = oracle.prefill_backward(qf, kf, vf, synth.to_float(g_np, w), fwd.mask,
                                                     True, 128, 64, scale=scale, magnitudes=True)
    _check("dq", dq, rq, mq, f"scale={scale}")
    _check("dk", dk, rk, mk, f"scale={scale}")
    _check("dv", dv, rv, mv, f"scale={scale}")

def test_prefill_backward_block_sparse():
    """A block-sparse forward (the oracle's) whose set leaves the first query
    tile with no key and drops tiles inside the set: rows that saw nothing and
    tiles outside the set get no gradient."""
    w = synth.small_workload("prefill", B=1, Hq=2, Hkv=1, Nq=300, Nk=700, d=128, dtype="bf16",
                             br=128, bc=64, gain=6.0, seed=53, window=32)
    sel = synth.block_set(w, 0.3, seed=4)
    sel[:, :, 0, :] = 0
    inp = synth.make_inputs(w)
    qf, kf, vf = (synth.to_float(x, w) for x in (inp.q, inp.k, inp.v))
    fwd = oracle.prefill_masked(qf, kf, vf, sel, 1e-2, True, 128, 64)
    assert (fwd.lse == -np.inf).any() and (fwd.mask == 0).any()
    g_np = _dout(np.random.default_rng(6), (w.B, w.Hq, w.Nq, w.dv))
    dq, dk, dv = _backward(w, inp, fwd, g_np)
    rq, rk, rv, mq, mk, mv = oracle.prefill_backward(qf, kf, vf, synth.to_float(g_np, w), fwd.mask,
                                                     True, 128, 64, magnitudes=True)
    _check("dq", dq, rq, mq, "block-sparse")
    _check("dk", dk, rk, mk, "block-sparse")
    _check("dv", dv, rv, mv, "block-sparse")
    assert (dq.cpu().numpy()[fwd.lse == -np.inf] == 0).all()


@pytest.mark.parametrize("lam,gain", [(1e-3, 1.0), (1e-2, 6.0)])
def test_prefill_backward_llama8b_n32768(lam, gain):
    """The benchmark's configuration (Llama-3.1-8B layer, N = 32768), whole call
    on the GPU, checked on two sub-problems the oracle can run: dq of the first
    three query tiles (square causal rows [0, R) see only keys [0, R)) and dk,
    dv of the keys of the last query tile (only its rows see them), for the
    query heads of KV head 0. The other rows get an all-kept mask and zero
    out/lse; no checked gradient depends on them."""
    w = synth.WORKLOADS[2].with_gain(gain)
    inp = synth.make_inputs(w)
    G = w.Hq // w.Hkv
    f = lambda x: synth.to_float(x, w)
    R = 3 * 128
    r0 = w.Nq - 128
    qp, kp, vp = f(inp.q[:, :G, :R]), f(inp.k[:, :1, :R]), f(inp.v[:, :1, :R])
    pre = oracle.prefill(qp, kp, vp, lam, True, 128, 64)
    qs, ks, vs = f(inp.q[:, :G, r0:]), f(inp.k[:, :1]), f(inp.v[:, :1])
    suf = oracle.prefill(qs, ks, vs, lam, True, 128, 64)
    nqt, nkt = synth.n_tiles(w.Nq, 128), synth.n_tiles(w.Nk, 64)
    mask = np.ones((w.B, w.Hq, nqt, nkt), np.uint8)
    lse = np.zeros((w.B, w.Hq, w.Nq), np.float32)
    out = np.zeros((w.B, w.Hq, w.Nq, w.dv), np.float32)
    mask[:, :G, :3, :R // 64] = pre.mask
    mask[:, :G, :3, R // 64:] = 2
    lse[:, :G, :R], out[:, :G, :R] = pre.lse, pre.out
    mask[:, :G, -1:] = suf.mask
    lse[:, :G, r0:], out[:, :G, r0:] = suf.lse, suf.out
    g_np = _dout(np.random.default_rng(7), (w.B, w.Hq, w.Nq, w.dv))
    dq, dk, dv = _backward(w, inp, None, g_np, "fp32", rows=(mask, lse, out))
    rq, _, _, mq, _, _ = oracle.prefill_backward(qp, kp, vp, f(g_np[:, :G, :R]), pre.mask, True,
                                                 128, 64, magnitudes=True)
    _check("dq prefix", dq[:, :G, :R], rq, mq, f"lam={lam} g={gain}")
    _, rk, rv, _, mk, mv = oracle.prefill_backward(qs, ks, vs, f(g_np[:, :G, r0:]), suf.mask, True,
                                                   128, 64, magnitudes=True)
    _check("dk suffix", dk[:, :1, r0:], rk[:, :, r0:], mk[:, :, r0:], f"lam={lam} g={gain}")
    _check("dv suffix", dv[:, :1, r0:], rv[:, :, r0:], mv[:, :, r0:], f"lam={lam} g={gain}")


def test_prefill_backward_strided_layout_matches_contiguous():
    """[B, N, H, d] storage of q, k, v, out and dout gives the same gradient bits
    as [B, H, N, d] (a layout property of the GPU path; the forward's mask, lse
    and out feed both calls)."""
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=257, Nk=400, d=128, dtype="bf16",
                             br=128, bc=64, gain=6.0, seed=57, window=32, causal=True)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    fwd = A.prefill(q, k, v, 1e-2)
    g = torch.from_numpy(_dout(np.random.default_rng(8), (w.B, w.Hq, w.Nq, w.dv))).view(
        torch.bfloat16).cuda()
    ref = A.prefill_backward(q, k, v, fwd.out, g, fwd.lse, fwd.mask)
    il = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)
    qs, ks, vs, os_, gs = (il(x) for x in (q, k, v, fwd.out, g))
    assert qs.stride(2) == w.Hq * w.d and os_.stride() == gs.stride()
    got = A.prefill_backward(qs, ks, vs, os_, gs, fwd.lse, fwd.mask)
    torch.cuda.synchronize()
    assert got[0].stride() == qs.stride() and got[1].stride() == ks.stride()
    for r, x in zip(ref, got):
        assert torch.equal(r, x)
