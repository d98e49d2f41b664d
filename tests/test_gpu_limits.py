"""GPU tests at the limits of the supported sizes, through the C ABI.

* Empty calls: no query rows (B = 1, Nq = 0) and no batch (B = 0) succeed with
  NULL pointers for the empty tensors; the backward of a call with no query
  rows gives zero dK and dV.
* The longest key range the tile lists hold: one 128-row query tile against
  6144 key tiles (393216 keys), for the block-sparse prefill, the two-pass
  prefill (its map kernel flags every key tile in LDS) and the backward (the
  dQ kernel lists every kept key tile in LDS), each against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_skip_amd import attention as A
from block_sparse_long_skip_amd import synth
from parity import Tally, prefill_masked_tile_parity, prefill_twopass_tile_parity, to_device

pytestmark = pytest.mark.gpu

MAX_TILES = 6144


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    A.load_library()
    yield
    torch.cuda.synchronize()


def test_empty_calls():
    w = synth.small_workload("prefill", B=1, Hq=2, Hkv=1, Nq=128, Nk=200, seed=71)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    q0 = q[:, :, :0]  # no query rows (torch gives it a NULL data pointer)
    for fn in (lambda: A.prefill(q0, k, v, 1e-2),
               lambda: A.prefill_masked(q0, k, v, torch.ones((1, 1, 1, 4), dtype=torch.bool,
                                                             device="cuda"), 1e-2),
               lambda: A.prefill_twopass(q0, k, v, 1e-2)):
        r = fn()
        torch.cuda.synchronize()
        assert r.out.shape[2] == 0 and r.lse.shape[2] == 0
        assert (r.stats == 0).all()
    # no batch: every tensor empty, statistics empty
    qb, kb, vb = (x[:0] for x in (q, k, v))
    r = A.prefill(qb, kb, vb, 1e-2)
    torch.cuda.synchronize()
    assert r.out.shape[0] == 0
    # backward with no query rows: dK and dV are zero (no row reads any key)
    g0 = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16, device="cuda")[:, :, :0]
    o0 = torch.zeros((1, 2, 8, 128), dtype=torch.float32, device="cuda")[:, :, :0]
    lse0 = torch.zeros((1, 2, 8), dtype=torch.float32, device="cuda")[:, :, :0]
    m0 = torch.zeros((1, 2, 1, 4), dtype=torch.uint8, device="cuda")[:, :, :0]
    dq, dk, dv = A.prefill_backward(q0, k, v, o0, g0, lse0, m0)
    torch.cuda.synchronize()
    assert dq.numel() == 0
    assert (dk == 0).all() and (dv == 0).all()


def _longest():
    """One query tile against 6144 key tiles, planted so that tiles drop."""
    return synth.small_workload("prefill", B=1, Hq=1, Hkv=1, Nq=128, Nk=MAX_TILES * 64, d=128,
                                dtype="bf16", br=128, bc=64, gain=6.0, seed=72, window=32,
                                causal=True)


def test_block_sparse_longest_key_range():
    w = _longest()
    inp = synth.make_inputs(w)
    sel = synth.block_set(w, 0.1, seed=5)
    sel[..., -1] = 1  # the last key tile, at the end of the list
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    r = A.prefill_masked(q, k, v, torch.from_numpy(sel).cuda(), 1e-2, causal=True,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    tally = Tally()
    prefill_masked_tile_parity(r, inp, w, 1e-2, sel, 0, 0, 0, tally)
    m = r.mask.cpu().numpy()
    assert ((m != 2) == (sel != 0)).all() and m[0, 0, 0, -1] != 2
    tally.check(w.dtype, "block-sparse, 6144 key tiles")


def test_twopass_longest_key_range():
    w = _longest()
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    r = A.prefill_twopass(q, k, v, 1e-2, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tally = Tally()
    prefill_twopass_tile_parity(r, inp, w, 1e-2, 0, 0, 0, tally)
    m = r.mask.cpu().numpy()
    assert (m == 0).any() and (m != 2).all()
    assert int(r.stats[0, 0, 0]) == MAX_TILES
    tally.check(w.dtype, "two-pass, 6144 key tiles")


def test_backward_longest_key_range():
    """dQ lists every kept key tile of the query tile in LDS; dK and dV of every
    key against the oracle too (one query tile: the oracle runs it in full)."""
    w = _longest()
    inp = synth.make_inputs(w)
    qf, kf, vf = (synth.to_float(x, w) for x in (inp.q, inp.k, inp.v))
    fwd = oracle.prefill(qf, kf, vf, 1e-2, True, 128, 64)
    assert (fwd.mask == 0).any()
    g = np.random.default_rng(9).standard_normal((1, 1, 128, 128)).astype(np.float32)
    g_bits = synth.f32_to_bf16_bits(g)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    dq, dk, dv = A.prefill_backward(
        q, k, v, torch.from_numpy(fwd.out).float().cuda(),
        torch.from_numpy(g_bits).view(torch.bfloat16).cuda(),
        torch.from_numpy(fwd.lse).float().cuda(), torch.from_numpy(fwd.mask).cuda())
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(qf, kf, vf, synth.to_float(g_bits, w), fwd.mask, True, 128, 64,
                                  magnitudes=True, out=fwd.out.astype(np.float32).astype(np.float64))
    for name, got, rg, mg in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3], ref[3:]):
        e = np.abs(got.double().cpu().numpy() - rg)
        bound = 2 * 2.0 ** -8 * mg + 1e-5 * (1.0 + np.abs(rg).max())
        worst = float((e / bound).max())
        print(f"{name}: max_abs={e.max():.3e} worst/bound={worst:.3f}")
        assert worst <= 1.0, name
