"""GPU parity: every HIP kernel against the CPU oracle, through the C ABI.

Small cases span several tiles with ragged tails and run the whole oracle;
the full-size workloads (Llama-3.1-8B-shaped prefill at N=32768, Qwen2.5-7B-
shaped prefill at N=131072, batch-32 GQA decode over 65536 keys, batch-16 MLA
decode over 32768 latent keys) run the kernel in the launch configuration the
benchmark times and compare sampled query tiles / rows with the oracle.
The supplementary gain (planted boosts scaled by g) makes dropped tiles appear;
at gain 1 the workloads as specified drop nothing.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_skip_amd import attention as A
from block_sparse_long_skip_amd import synth
from parity import (Tally, check_mask_row, decode_row_parity, from_device,
                    prefill_masked_tile_parity, prefill_tile_parity, sample_qtiles, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    A.load_library()
    yield
    torch.cuda.synchronize()


OUT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _prefill(inp, w, lam, out="native", **kw):
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    od = OUT.get(out)
    r = A.prefill(q, k, v, lam, causal=w.causal, br=w.br, bc=w.bc, out_dtype=od, **kw)
    torch.cuda.synchronize()
    return r


def _decode(inp, w, lam, out="native", workspace=None, scale=None):
    q, k = to_device(inp.q, w), to_device(inp.k, w)
    v = to_device(inp.v, w) if inp.v is not None else None
    r = A.decode(q, k, v, lam, bc=w.bc, dv=w.dv, out_dtype=OUT.get(out), workspace=workspace,
                 scale=scale)
    torch.cuda.synchronize()
    return r


def _check_prefill_full(w, lam, label, out="native", scale=None):
    inp = synth.make_inputs(w)
    res = _prefill(inp, w, lam, out, scale=scale)
    tally = Tally()
    nqt = synth.n_tiles(w.Nq, w.br)
    stats_mask = res.mask.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hq):
            for i in range(nqt):
                prefill_tile_parity(res, inp, w, lam, b, h, i, tally, scale=scale)
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 0], (stats_mask != 2).sum(axis=(2, 3)))
    assert np.array_equal(st[..., 1], (stats_mask == 1).sum(axis=(2, 3)))
    _check_tally(tally, w, label, res.out.dtype == torch.bfloat16)
    return res


def _check_tally(tally, w, label, out_bf16):
    """The bar of the parity helpers; at gain 1 (the workloads as specified)
    bf16 outputs must also meet the plain bar against the unrounded oracle."""
    tally.check(w.dtype, label, out_bf16=out_bf16)
    if out_bf16 and w.gain == 1.0:
        tally.check(w.dtype, label + " (unrounded reference)", out_bf16=True, strict=True)


# ----------------------------------------------------------------------------- prefill fp32

@pytest.mark.parametrize("gain", [1.0, 6.0])
@pytest.mark.parametrize("lam", [0.0, 1e-3, 1e-2])
def test_prefill_fp32_n1024(lam, gain):
    w = synth.WORKLOADS[1].with_gain(gain)
    res = _check_prefill_full(w, lam, f"fp32 n1024 lam={lam} g={gain}")
    if gain == 6.0 and lam > 0:
        assert res.skip_fraction > 0.0


@pytest.mark.parametrize("shape", [
    dict(B=2, Hq=4, Hkv=2, Nq=200, Nk=200, causal=True),
    dict(B=1, Hq=2, Hkv=1, Nq=70, Nk=333, causal=True),    # bottom-right alignment
    dict(B=1, Hq=3, Hkv=3, Nq=129, Nk=65, causal=False),
    dict(B=1, Hq=1, Hkv=1, Nq=1, Nk=130, causal=True),
])
@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-2, 6.0), (1.0, 6.0)])
def test_prefill_fp32_ragged(shape, lam, gain):
    w = synth.small_workload("prefill", d=64, dtype="fp32", br=64, bc=64, gain=gain, seed=21,
                             **shape)
    _check_prefill_full(w, lam, f"fp32 {shape} lam={lam}")


# ----------------------------------------------------------------------------- prefill bf16

@pytest.mark.parametrize("shape", [
    dict(B=1, Hq=2, Hkv=1, Nq=300, Nk=300, causal=True),
    dict(B=2, Hq=4, Hkv=2, Nq=130, Nk=333, causal=True),
    dict(B=1, Hq=2, Hkv=2, Nq=200, Nk=129, causal=False),
    dict(B=1, Hq=1, Hkv=1, Nq=128, Nk=128, causal=True),
    dict(B=1, Hq=1, Hkv=1, Nq=5, Nk=64, causal=True),
    dict(B=1, Hq=1, Hkv=1, Nq=1, Nk=1, causal=True),
    # several query tiles with ragged key ranges (bottom-right causal) and a
    # non-causal shape with drops in every query tile
    dict(B=1, Hq=2, Hkv=1, Nq=384, Nk=1000, causal=True),
    dict(B=1, Hq=1, Hkv=1, Nq=512, Nk=700, causal=False),
])
@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-3, 1.0), (1e-2, 6.0), (1.0, 6.0)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_prefill_bf16_small(shape, lam, gain, out):
    w = synth.small_workload("prefill", d=128, dtype="bf16", br=128, bc=64, gain=gain, seed=33,
                             window=32, **shape)
    _check_prefill_full(w, lam, f"bf16 {shape} lam={lam} g={gain}", out)


def _prefill_sampled(cfg, lam, gain, heads, per_head, seed, out="bf16"):
    w = (synth.WORKLOADS[cfg] if isinstance(cfg, int) else cfg).with_gain(gain)
    inp = synth.make_inputs(w)
    res = _prefill(inp, w, lam, out)
    tally = Tally()
    kv_cache = {}
    for (h, i) in sample_qtiles(w, heads, per_head, seed):
        kvh = h // w.G
        if kvh not in kv_cache:
            kv_cache = {kvh: (synth.to_float(inp.k[0, kvh], w), synth.to_float(inp.v[0, kvh], w))}
        kf, vf = kv_cache[kvh]
        prefill_tile_parity(res, inp, w, lam, 0, h, i, tally, kf=kf, vf=vf)
    # whole-call invariants on the GPU mask
    m = res.mask.cpu().numpy()
    nqt, nkt = m.shape[2], m.shape[3]
    assert (m[..., 0] == 1).all()
    last_vis = (np.minimum((np.arange(nqt) + 1) * w.br, w.Nq) - 1 + w.Nk - w.Nq) // w.bc
    assert ((m == 2) == (np.arange(nkt)[None, :] > last_vis[:, None])[None, None]).all()
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=(2, 3)))
    _check_tally(tally, w, f"workload {cfg} lam={lam} g={gain}", out == "bf16")
    return res


@pytest.mark.parametrize("lam,gain,out", [(0.0, 1.0, "bf16"), (1e-4, 1.0, "bf16"),
                                          (1e-3, 1.0, "bf16"), (1e-2, 1.0, "bf16"),
                                          (1e-3, 6.0, "bf16"), (1e-2, 6.0, "bf16"),
                                          (1e-2, 6.0, "fp32")])
def test_prefill_llama8b_n32768(lam, gain, out):
    res = _prefill_sampled(2, lam, gain, heads=[0, 5, 31], per_head=3, seed=2, out=out)
    if gain == 1.0:
        assert res.skip_fraction == 0.0  # the as-specified planting is too weak to drop tiles
    else:
        assert res.skip_fraction > 0.05


@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-3, 1.0), (1e-3, 8.0)])
def test_prefill_qwen7b_n131072(lam, gain):
    _prefill_sampled(4, lam, gain, heads=[0, 27], per_head=1, seed=4)


@pytest.mark.parametrize("lam", [1e-3, 1e-2])
def test_prefill_qwen7b_n131072_low_needles(lam):
    """The benchmark's skip-regime input: the 131072-long layer with every KV
    head at 0.1% needles and gain 8, where most tiles hold no planted key."""
    w = synth.WORKLOADS[4].scaled(needle_rate=0.001, needle_rate_range=None)
    res = _prefill_sampled(w, lam, 8.0, heads=[0, 13, 27], per_head=1, seed=5)
    assert res.skip_fraction > 0.5


# ----------------------------------------------------------------------------- decode

def _check_decode(w, lam, pairs=None, out="bf16", scale=None):
    inp = synth.make_inputs(w)
    res = _decode(inp, w, lam, out, scale=scale)
    tally = Tally()
    if pairs is None:
        pairs = [(b, kvh) for b in range(w.B) for kvh in range(w.Hkv)]
    for (b, kvh) in pairs:
        kf = synth.to_float(inp.k[b, kvh], w)
        vf = kf[:, :w.dv] if inp.v is None else synth.to_float(inp.v[b, kvh], w)
        for hq in range(kvh * w.G, (kvh + 1) * w.G):
            decode_row_parity(res, synth.to_float(inp.q[b, hq], w), kf, vf, lam, w.bc, b, hq, tally,
                              scale=scale)
    m = res.mask.cpu().numpy()
    st = res.stats.cpu().numpy()
    nkt = m.shape[2]
    assert (st[..., 0] == nkt).all() and (m[..., 0] == 1).all()
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=2))
    for b in range(w.B):
        for kvh in range(w.Hkv):
            grp = m[b, kvh * w.G:(kvh + 1) * w.G]
            assert (st[b, kvh * w.G:(kvh + 1) * w.G, 2] == (grp == 1).any(axis=0).sum()).all()
    _check_tally(tally, w, f"decode {w.name} lam={lam} g={w.gain}", out == "bf16")
    return res


@pytest.mark.parametrize("shape", [
    dict(B=2, Hq=8, Hkv=2, Nk=1000),
    dict(B=1, Hq=16, Hkv=1, Nk=777),
    dict(B=3, Hq=3, Hkv=3, Nk=64),
    dict(B=1, Hq=5, Hkv=1, Nk=1),
    dict(B=2, Hq=4, Hkv=1, Nk=4100),
])
@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-3, 6.0), (1e-2, 6.0), (1.0, 6.0)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_decode_gqa_small(shape, lam, gain, out):
    w = synth.small_workload("decode", d=128, dtype="bf16", bc=64, gain=gain, seed=44,
                             window=64, **shape)
    _check_decode(w, lam, out=out)


@pytest.mark.parametrize("lam,gain,out", [(0.0, 1.0, "bf16"), (1e-3, 1.0, "bf16"),
                                          (1e-2, 6.0, "bf16"), (1e-2, 6.0, "fp32")])
def test_decode_gqa_b32_n65536(lam, gain, out):
    w = synth.WORKLOADS[3].with_gain(gain)
    res = _check_decode(w, lam, pairs=[(0, 0), (7, 3), (31, 7)], out=out)
    if gain > 1:
        assert res.skip_fraction > 0.3


@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-3, 1.0), (1e-3, 6.0), (1e-2, 6.0)])
def test_decode_gqa_b1_n65536_split(lam, gain):
    """One sequence with 8 KV heads fills 8 of the 256 CUs with one workgroup
    per (batch, KV head), so the cache is split along its length: scores and
    tile maxima first, then exact decisions and P.V per split, then a
    log-sum-exp merge. Every (KV head, query head) row against the oracle."""
    w = synth.WORKLOADS[3].scaled(B=1).with_gain(gain)
    assert A.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.dv, latent=False) > 0
    res = _check_decode(w, lam, out="fp32")
    if gain > 1 and lam > 0:
        assert res.skip_fraction > 0.3


@pytest.mark.parametrize("lam,gain", [(1e-3, 1.0), (1e-2, 6.0)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_decode_gqa_split_many_splits(lam, gain, out):
    """One sequence with one KV head over 300 key tiles: the split plan makes
    75 splits of 4 tiles, so the merge walks a second chunk of split partials
    and a remainder of its eight-at-a-time loop. Every row against the oracle."""
    w = synth.small_workload("decode", B=1, Hq=4, Hkv=1, Nk=300 * 64, d=128, dtype="bf16", bc=64,
                             gain=gain, seed=57, window=64)
    assert A.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.dv, latent=False) > 0
    _check_decode(w, lam, out=out)


# The latent-cache kernel splits the cache over workgroups (one split per
# tile at these sizes, a few tiles per split at the larger ones) and redoes the
# splits whose speculative decisions differ from the exact ones; two head
# groups (G = 128), a partial group (G = 100) and several KV heads are covered.
@pytest.mark.parametrize("shape", [
    dict(B=2, Hq=32, Hkv=1, Nk=1000),
    dict(B=1, Hq=20, Hkv=2, Nk=300),
    dict(B=1, Hq=16, Hkv=1, Nk=64),
    dict(B=1, Hq=128, Hkv=1, Nk=2000),
    dict(B=1, Hq=100, Hkv=1, Nk=5000),
    dict(B=3, Hq=128, Hkv=2, Nk=9000),
])
@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-3, 6.0), (1e-2, 6.0), (1.0, 6.0)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_decode_mla_small(shape, lam, gain, out):
    w = synth.small_workload("decode_mla", d=576, dv=512, dtype="bf16", bc=64, gain=gain,
                             seed=55, window=64, **shape)
    _check_decode(w, lam, out=out)


@pytest.mark.parametrize("lam,gain,out", [(0.0, 1.0, "bf16"), (1e-2, 1.0, "bf16"),
                                          (1e-2, 6.0, "bf16"), (1e-2, 6.0, "fp32")])
def test_decode_mla_b16_n32768(lam, gain, out):
    w = synth.WORKLOADS[5].with_gain(gain)
    _check_decode(w, lam, pairs=[(0, 0), (15, 0)], out=out)


@pytest.mark.parametrize("cfg,lam", [(3, 1e-2), (5, 1e-2)])
def test_decode_whole_call_gain6(cfg, lam):
    """Every (batch, head) row of the batch-32 GQA decode and of the batch-16
    latent decode at gain 6 against the oracle: the whole mask (exact outside
    the near-threshold band), every output row and lse, and the statistics."""
    from parity import check_mask_row, oracle_decode_all
    w = synth.WORKLOADS[cfg].with_gain(6.0)
    inp = synth.make_inputs(w)
    res = _decode(inp, w, lam, "fp32")
    del inp
    ref_out, ref_lse, ref_mask, ref_gap = oracle_decode_all(w, lam)
    gm = res.mask.cpu().numpy()
    tally = Tally()
    flipped_rows = []
    for b in range(w.B):
        for hq in range(w.Hq):
            if check_mask_row(gm[b, hq], ref_mask[b, hq], ref_gap[b, hq], lam, tally,
                              f"b{b} h{hq}").any():
                flipped_rows.append((b, hq))
    keep = np.ones((w.B, w.Hq), bool)
    for (b, hq) in flipped_rows:  # compared in the sampled tests against the GPU's own mask
        keep[b, hq] = False
    got = res.out.double().cpu().numpy()
    got_lse = res.lse.double().cpu().numpy()
    tally.add(got[keep], ref_out[keep], got_lse[keep] - ref_lse[keep])
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 1], (gm == 1).sum(axis=2))
    groups = gm.reshape(w.B, w.Hkv, w.G, -1)
    assert np.array_equal(st[..., 2].reshape(w.B, w.Hkv, w.G),
                          np.repeat((groups == 1).any(axis=2).sum(axis=2)[..., None], w.G, 2))
    assert res.skip_fraction > 0.25
    tally.check(w.dtype, f"decode {w.name} whole call lam={lam} g=6 "
                f"({len(flipped_rows)} rows with band flips)")


def test_decode_mla_split_count_invariance():
    """The latent decode splits the cache over workgroups with a split length T
    chosen from the batch: a 32768-key sequence runs with T = 4 at batch 1,
    64 at batch 16, 128 at batch 32 and 256 at batch 64. The same sequence
    (the cache shared by the whole batch through a zero batch stride, its query
    at batch index 0) must give the same mask and statistics bit for bit at
    every T. Outputs differ in rounding only (each split rounds its
    probabilities to bf16 against its own reference max), so each T's output
    and lse are held to the bar against the oracle."""
    w = synth.WORKLOADS[5].with_gain(6.0)
    u = synth.unit_direction(w)
    k1 = to_device(synth.k_slice(w, 0, 0, u), w).view(1, 1, w.Nk, w.d)
    q1 = to_device(np.stack([synth.q_slice(w, 0, h, u) for h in range(w.Hq)]).reshape(w.Hq, w.d), w)
    lam = 1e-2
    results = {}
    for B in (1, 16, 32, 64):
        q = torch.randn((B, w.Hq, w.d), dtype=torch.float32, device="cuda").to(torch.bfloat16)
        q[0] = q1
        k = k1.expand(B, 1, w.Nk, w.d)  # batch stride 0 (batch 1 keeps its own)
        assert B == 1 or k.stride(0) == 0
        r = A.decode(q, k, None, lam, dv=w.dv, out_dtype=torch.float32)
        torch.cuda.synchronize()
        results[B] = (r.out[0].double().cpu().numpy(), r.mask[0].cpu().numpy(),
                      r.stats[0].cpu().numpy(), r.lse[0].double().cpu().numpy())
        del q, k, r
    ref_mask, ref_stats = results[1][1], results[1][2]
    for B, (_, m, st_, _) in results.items():
        assert np.array_equal(m, ref_mask), f"mask differs at batch {B}"
        assert np.array_equal(st_, ref_stats), f"statistics differ at batch {B}"
    assert (ref_mask == 0).any()
    kf = synth.to_float(synth.k_slice(w, 0, 0, u), w)
    rows = [oracle.blasst_rows(synth.to_float(synth.q_slice(w, 0, hq, u), w), kf, kf[:, :w.dv],
                               lam, w.bc, np.ones((1, w.Nk), bool), 1.0 / math.sqrt(w.d))
            for hq in range(w.Hq)]
    for B, (o, m, _, l_) in results.items():
        tally = Tally()
        for hq, t in enumerate(rows):
            flips = check_mask_row(m[hq], t.mask, t.gap, lam, tally, f"B{B} h{hq}")
            if not flips.any():
                tally.add(o[hq], t.out[0], np.array([l_[hq] - t.lse[0]]))
        tally.check(w.dtype, f"latent decode, sequence inside batch {B}")


def test_decode_mla_workspace_reuse():
    """The workspace carries nothing between calls: a call after another shape
    has used (and left garbage in) the same buffer gives the same bits."""
    w1 = synth.small_workload("decode_mla", d=576, dv=512, dtype="bf16", bc=64, gain=6.0,
                              seed=56, window=64, B=2, Hq=64, Hkv=1, Nk=3000)
    w2 = synth.small_workload("decode_mla", d=576, dv=512, dtype="bf16", bc=64, gain=1.0,
                              seed=57, window=64, B=1, Hq=128, Hkv=1, Nk=5000)
    n = max(A.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nk, 576, 512, latent=True)
            for w in (w1, w2))
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    i1, i2 = synth.make_inputs(w1), synth.make_inputs(w2)
    r1 = _decode(i1, w1, 1e-2, "fp32", workspace=ws)
    first = [x.clone() for x in (r1.out, r1.mask, r1.lse, r1.stats)]
    _decode(i2, w2, 1e-3, "fp32", workspace=ws)
    r3 = _decode(i1, w1, 1e-2, "fp32", workspace=ws)
    for a_, b_ in zip(first, (r3.out, r3.mask, r3.lse, r3.stats)):
        assert torch.equal(a_, b_)


# ----------------------------------------------------------------------------- block-sparse prefill

def _prefill_masked(inp, w, bm, lam, out="native"):
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    if isinstance(bm, np.ndarray):
        bm = torch.from_numpy(bm).cuda()
    r = A.prefill_masked(q, k, v, bm, lam, causal=w.causal, br=w.br, bc=w.bc,
                         out_dtype=OUT.get(out))
    torch.cuda.synchronize()
    return r


def _check_masked_full(w, sel, lam, label, out="native"):
    inp = synth.make_inputs(w)
    res = _prefill_masked(inp, w, sel, lam, out)
    tally = Tally()
    nqt = synth.n_tiles(w.Nq, w.br)
    for b in range(w.B):
        for h in range(w.Hq):
            for i in range(nqt):
                prefill_masked_tile_parity(res, inp, w, lam, sel, b, h, i, tally)
    m = res.mask.cpu().numpy()
    assert (m[sel == 0] == 2).all(), "blocks outside the set must be reported not visited"
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 0], (m != 2).sum(axis=(2, 3)))
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=(2, 3)))
    tally.check(w.dtype, label, out_bf16=res.out.dtype == torch.bfloat16)
    return res


MASKED_SHAPES = [
    dict(B=1, Hq=2, Hkv=1, Nq=300, Nk=700, causal=True),
    dict(B=2, Hq=2, Hkv=2, Nq=256, Nk=256, causal=True),
    dict(B=1, Hq=2, Hkv=1, Nq=200, Nk=333, causal=False),
]
# (density, sink, local): CRISP-shaped sets, a set with rows that see nothing
# (no sink, no local window), and the full set
MASKED_SETS = [(0.3, True, 2), (0.2, False, 0), (1.0, True, 0)]


@pytest.mark.parametrize("shape", MASKED_SHAPES)
@pytest.mark.parametrize("bset", MASKED_SETS, ids=lambda x: f"d{x[0]}_sink{int(x[1])}_loc{x[2]}")
@pytest.mark.parametrize("lam,gain", [(0.0, 1.0), (1e-2, 6.0), (1.0, 6.0)])
def test_prefill_masked_small(shape, bset, lam, gain):
    w = synth.small_workload("prefill", d=128, dtype="bf16", br=128, bc=64, gain=gain, seed=41,
                             window=32, **shape)
    density, sink, local = bset
    sel = synth.block_set(w, density, sink=sink, local=local, seed=1)
    _check_masked_full(w, sel, lam, f"masked {shape} set={bset} lam={lam} g={gain}", "fp32")


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_prefill_masked_edge_sets(out):
    """An empty set (every row zero, lse -inf, every block not visited), a set
    holding only the tail tile past the last row's diagonal, and a set whose
    only block is the ragged last key tile."""
    w = synth.small_workload("prefill", B=1, Hq=2, Hkv=1, Nq=130, Nk=333, seed=43, gain=6.0)
    inp = synth.make_inputs(w)
    nqt, nkt = synth.n_tiles(w.Nq, w.br), synth.n_tiles(w.Nk, w.bc)
    empty = np.zeros((1, 2, nqt, nkt), np.uint8)
    r = _prefill_masked(inp, w, empty, 1e-2, out)
    assert (r.out == 0).all() and (r.lse == -math.inf).all() and (r.mask == 2).all()
    assert (r.stats == 0).all()
    last = empty.copy()
    last[..., nkt - 1] = 1  # causal: only the last query rows reach it
    _check_masked_full(w, last, 1e-2, f"masked last-tile-only out={out}", out)
    _check_masked_full(w.scaled(causal=False), last, 1e-2, f"masked tail non-causal out={out}", out)


@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_prefill_masked_first_tile_is_the_diagonal(out):
    """Each query tile's set holds only the key tile of its last row's causal
    limit, with Nk - Nq = 133 (not a multiple of 32): inside a wave, rows whose
    limit falls before that tile see nothing while the others start their
    running max there, so one wave mixes rows that rescale with rows that have
    no reference max (they must come out as zeros with lse -inf)."""
    w = synth.small_workload("prefill", B=1, Hq=2, Hkv=1, Nq=200, Nk=333, seed=47, gain=6.0,
                             window=32)
    nqt, nkt = synth.n_tiles(w.Nq, w.br), synth.n_tiles(w.Nk, w.bc)
    sel = np.zeros((1, 2, nqt, nkt), np.uint8)
    for i in range(nqt):
        last = min((i + 1) * w.br, w.Nq) - 1
        sel[..., i, (last + w.Nk - w.Nq) // w.bc] = 1
    res = _check_masked_full(w, sel, 1e-2, f"masked diagonal-first out={out}", out)
    lse = res.lse.cpu().numpy()
    assert np.isneginf(lse).any() and np.isfinite(lse).any()
    assert torch.isfinite(res.out.float()).all()


def test_prefill_masked_full_set_matches_prefill():
    """With every block selected the block-sparse path is the plain kernel, bit for bit."""
    w = synth.WORKLOADS[2].scaled(Nq=2048, Nk=3000, Hq=8, Hkv=2).with_gain(6.0)
    inp = synth.make_inputs(w)
    nqt, nkt = synth.n_tiles(w.Nq, w.br), synth.n_tiles(w.Nk, w.bc)
    ones = torch.ones((1, 1, 1, nkt), dtype=torch.bool, device="cuda")  # broadcast set
    for lam in (0.0, 1e-3, 1e-2):
        ref = _prefill(inp, w, lam)
        got = _prefill_masked(inp, w, ones, lam)
        assert torch.equal(ref.out.view(torch.int16), got.out.view(torch.int16))
        assert torch.equal(ref.lse, got.lse)
        assert torch.equal(ref.mask, got.mask)
        assert torch.equal(ref.stats, got.stats)


def test_prefill_masked_broadcast_matches_expanded():
    """A set shared over batch and heads (zero strides) equals the expanded copy."""
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=400, Nk=900, seed=45, gain=6.0)
    inp = synth.make_inputs(w)
    sel = synth.block_set(w, 0.3, seed=2)[:1, :1]
    shared = torch.from_numpy(sel).cuda()
    a = _prefill_masked(inp, w, shared, 1e-2)
    b = _prefill_masked(inp, w, shared.expand(2, 4, -1, -1).contiguous(), 1e-2)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.mask, b.mask) and torch.equal(a.stats, b.stats)


@pytest.mark.parametrize("lam,gain,density", [(0.0, 1.0, 0.1), (1e-3, 6.0, 0.1), (1e-2, 6.0, 0.25)])
def test_prefill_masked_llama8b_n32768(lam, gain, density):
    """The benchmark's block-sparse configuration: sampled query tiles against
    the oracle, whole-call invariants on the GPU mask."""
    w = synth.WORKLOADS[2].with_gain(gain)
    inp = synth.make_inputs(w)
    sel = synth.block_set(w, density, seed=3)
    res = _prefill_masked(inp, w, sel, lam, "bf16")
    tally = Tally()
    kv_cache = {}
    for (h, i) in sample_qtiles(w, [0, 9, 31], 3, seed=4):
        kvh = h // w.G
        if kvh not in kv_cache:
            kv_cache = {kvh: (synth.to_float(inp.k[0, kvh], w), synth.to_float(inp.v[0, kvh], w))}
        kf, vf = kv_cache[kvh]
        prefill_masked_tile_parity(res, inp, w, lam, sel, 0, h, i, tally, kf=kf, vf=vf)
    m = res.mask.cpu().numpy()
    nqt, nkt = m.shape[2], m.shape[3]
    last_vis = (np.minimum((np.arange(nqt) + 1) * w.br, w.Nq) - 1 + w.Nk - w.Nq) // w.bc
    reach = np.arange(nkt)[None, :] <= last_vis[:, None]
    assert ((m != 2) == ((sel[0] != 0) & reach[None])).all()
    assert (m[..., 0] == 1).all(), "the sink tile is selected and first: always kept"
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=(2, 3)))
    tally.check(w.dtype, f"masked llama8b lam={lam} g={gain} density={density}", out_bf16=True)


# ----------------------------------------------------------------------------- behaviour

def test_rejected_call_leaves_outputs_untouched():
    w = synth.small_workload("prefill", Nq=200, Nk=200, seed=3)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    out = torch.full((1, w.Hq, 200, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.BlasstError) as e:
        A.prefill(q, k, v, 1.5, out=out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_bitwise_repeatable_and_lambda_nesting():
    w = synth.WORKLOADS[2].scaled(Nq=4096, Nk=4096).with_gain(6.0)
    inp = synth.make_inputs(w)
    prev = None
    for lam in (0.0, 1e-4, 1e-3, 1e-2, 0.1, 1.0):
        r1 = _prefill(inp, w, lam)
        r2 = _prefill(inp, w, lam)
        assert torch.equal(r1.out.view(torch.int16), r2.out.view(torch.int16))
        assert torch.equal(r1.mask, r2.mask)
        kept = (r1.mask == 1).cpu().numpy()
        if prev is not None:
            assert not (kept & ~prev).any()
        prev = kept


def test_strided_layout_matches_contiguous():
    """[B, N, H, d] storage (heads interleaved) gives the same bits as [B, H, N, d]."""
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=257, Nk=257, seed=9, gain=6.0)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    ref = A.prefill(q, k, v, 1e-2)
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert qs.stride(2) == w.Hq * w.d
    got = A.prefill(qs, ks, vs, 1e-2)
    torch.cuda.synchronize()
    assert torch.equal(ref.out.view(torch.int16), got.out.view(torch.int16))
    assert torch.equal(ref.mask, got.mask)


# ----------------------------------------------------------------------------- explicit scale

# Every entry point takes a softmax scale (<= 0 means 1/sqrt(d_qk)); a sharper
# and a flatter scale than the default, with drops, on each kernel.
@pytest.mark.parametrize("scale", [0.05, 0.2])
def test_prefill_bf16_explicit_scale(scale):
    w = synth.small_workload("prefill", d=128, dtype="bf16", br=128, bc=64, gain=6.0, seed=34,
                             window=32, B=1, Hq=2, Hkv=1, Nq=300, Nk=700, causal=True)
    _check_prefill_full(w, 1e-2, f"bf16 scale={scale}", scale=scale)


@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_prefill_fp32_explicit_scale(scale):
    w = synth.small_workload("prefill", d=64, dtype="fp32", br=64, bc=64, gain=6.0, seed=35,
                             window=32, B=1, Hq=2, Hkv=1, Nq=200, Nk=333, causal=True)
    _check_prefill_full(w, 1e-2, f"fp32 scale={scale}", scale=scale)


@pytest.mark.parametrize("scale", [0.03, 0.2])
def test_decode_gqa_explicit_scale(scale):
    w = synth.small_workload("decode", d=128, dtype="bf16", bc=64, gain=6.0, seed=56,
                             window=64, B=2, Hq=8, Hkv=2, Nk=1000)
    _check_decode(w, 1e-2, scale=scale)


@pytest.mark.parametrize("scale", [0.02, 0.1])
def test_decode_mla_explicit_scale(scale):
    w = synth.small_workload("decode_mla", d=576, dv=512, dtype="bf16", bc=64, gain=6.0, seed=57,
                             window=64, B=1, Hq=128, Hkv=1, Nk=2000)
    _check_decode(w, 1e-2, scale=scale)
