"""GPU parity of the two-pass prefill (MXFP4 max pre-pass, then exact attention
over the kept tiles) and of the MXFP4 quantizer, through the C ABI.

Bar:
  * MXFP4 codes and scales: bit for bit equal to the oracle's quantization
    (integer results of a definition with one rounding rule);
  * the map: the skip rule on the scores of the dequantized q and k, bit-exact
    except tiles whose oracle gap lies within the near-threshold band of
    ln(lambda) (the 4-bit products are exact and their sums exact in float32,
    so only the rounding of the final gap can differ);
  * out and lse: exact attention over the kept tiles, to the bf16-input bar of
    the one-pass prefill.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_skip_amd import attention as A
from block_sparse_long_skip_amd import synth
from parity import Tally, mxfp4_values, prefill_twopass_tile_parity, sample_qtiles, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    A.load_library()
    yield
    torch.cuda.synchronize()


OUT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _packed(codes: np.ndarray) -> np.ndarray:
    """One code per element -> two per byte, the even feature in the low nibble."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _mx_inputs(rng, shape):
    """bf16 values over many binades: per-block powers of two from 2^-133 to
    2^120, exact E2M1 midpoints at the block's scale, zero blocks, negative
    zeros and bf16 subnormals."""
    x = rng.standard_normal(shape).astype(np.float64)
    nb = shape[-1] // 32
    blk = x.reshape(*shape[:-1], nb, 32)
    e = rng.integers(-133, 121, size=blk.shape[:-1])
    blk *= np.ldexp(1.0, e)[..., None]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    tie = rng.random(blk.shape[:-1]) < 0.25
    te = rng.integers(-30, 30, size=blk.shape[:-1])
    tv = rng.choice(mids, size=blk.shape) * rng.choice([-1.0, 1.0], size=blk.shape)
    tv[..., 0] = 4.0
    blk[tie] = (tv * np.ldexp(1.0, te)[..., None])[tie]
    blk[rng.random(blk.shape[:-1]) < 0.05] = 0.0
    x = blk.reshape(shape)
    x[rng.random(shape) < 0.02] = -0.0
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    return bits, synth.bf16_bits_to_f32(bits).astype(np.float64)


def _on_device(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def test_quantize_mxfp4_bit_exact():
    rng = np.random.default_rng(51)
    bits, vals = _mx_inputs(rng, (2, 3, 77, 128))
    assert (np.abs(vals[vals != 0]) < 2.0 ** -126).any(), "fixture must hold bf16 subnormals"
    codes, scales = A.quantize_mxfp4(_on_device(bits))
    rc, rs = oracle.mx_quantize_fp4(vals)
    assert np.array_equal(codes.cpu().numpy(), _packed(rc))
    assert np.array_equal(scales.cpu().numpy(), rs)
    # a strided [B, N, H, d] view quantizes like its contiguous copy
    t = _on_device(bits).permute(0, 2, 1, 3)
    codes, scales = A.quantize_mxfp4(t)
    rc, rs = oracle.mx_quantize_fp4(vals.transpose(0, 2, 1, 3))
    assert np.array_equal(codes.cpu().numpy(), _packed(rc))
    assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("d", [32, 96, 576])
def test_quantize_mxfp4_other_widths(d):
    rng = np.random.default_rng(52 + d)
    bits, vals = _mx_inputs(rng, (1, 2, 33, d))
    codes, scales = A.quantize_mxfp4(_on_device(bits))
    rc, rs = oracle.mx_quantize_fp4(vals)
    assert np.array_equal(codes.cpu().numpy(), _packed(rc))
    assert np.array_equal(scales.cpu().numpy(), rs)


def _twopass(inp, w, lam, out="native", **kw):
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    r = A.prefill_twopass(q, k, v, lam, causal=w.causal, br=w.br, bc=w.bc, out_dtype=OUT.get(out),
                          **kw)
    torch.cuda.synchronize()
    return r


def _check_full(w, lam, label, out="fp32"):
    inp = synth.make_inputs(w)
    res = _twopass(inp, w, lam, out)
    tally = Tally()
    for b in range(w.B):
        for h in range(w.Hq):
            kvh = h // w.G
            kd = mxfp4_values(synth.to_float(inp.k[b, kvh], w))
            for i in range(synth.n_tiles(w.Nq, w.br)):
                prefill_twopass_tile_parity(res, inp, w, lam, b, h, i, tally, kd=kd)
    m = res.mask.cpu().numpy()
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 0], (m != 2).sum(axis=(2, 3)))
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=(2, 3)))
    tally.check(w.dtype, label, out_bf16=res.out.dtype == torch.bfloat16)
    return res


SHAPES = [
    dict(B=1, Hq=2, Hkv=1, Nq=300, Nk=300, causal=True),
    dict(B=2, Hq=4, Hkv=2, Nq=130, Nk=333, causal=True),
    dict(B=1, Hq=2, Hkv=2, Nq=200, Nk=129, causal=False),
    dict(B=1, Hq=1, Hkv=1, Nq=5, Nk=64, causal=True),
    dict(B=1, Hq=1, Hkv=1, Nq=1, Nk=1, causal=True),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("lam,gain,out", [(0.0, 1.0, "fp32"), (1e-3, 1.0, "bf16"),
                                          (1e-2, 6.0, "fp32"), (1.0, 6.0, "fp32")])
def test_prefill_twopass_small(shape, lam, gain, out):
    w = synth.small_workload("prefill", d=128, dtype="bf16", br=128, bc=64, gain=gain, seed=61,
                             window=32, **shape)
    _check_full(w, lam, f"twopass {shape} lam={lam} g={gain}", out)


def test_prefill_twopass_drops_and_differs_from_one_pass():
    """On planted inputs the 4-bit map drops tiles, and its decisions are not
    all the exact ones (the variant is an approximation of the rule); the
    one-pass mask stays the exact rule's."""
    w = synth.small_workload("prefill", B=1, Hq=4, Hkv=1, Nq=1024, Nk=2048, d=128, dtype="bf16",
                             br=128, bc=64, gain=6.0, seed=62, window=32, causal=True)
    res = _check_full(w, 1e-2, "twopass planted lam=1e-2 g=6")
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    one = A.prefill(q, k, v, 1e-2, causal=True)
    m2, m1 = res.mask.cpu().numpy(), one.mask.cpu().numpy()
    assert (m2 == 0).any()
    assert np.array_equal(m1 == 2, m2 == 2)
    print(f"map tiles differing from the exact rule: {int((m1 != m2).sum())} of {int((m1 != 2).sum())}")


def test_prefill_twopass_on_grid_matches_one_pass():
    """q and k exactly representable in MXFP4 (and bf16): the pre-pass sees the
    exact scores, so the map is the one-pass mask."""
    rng = np.random.default_rng(63)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def grid(shape, positive, e0, e1):
        x = rng.choice(mags, size=shape)
        if not positive:
            x = x * rng.choice([-1.0, 1.0], size=shape)
        blk = x.reshape(*shape[:-1], shape[-1] // 32, 32)
        blk[..., 0] = 4.0
        pw = np.ldexp(1.0, rng.integers(e0, e1, size=blk.shape[:-1]))
        return (blk * pw[..., None]).reshape(shape)

    # every fourth key tile aligned with the (positive) queries, the others small
    B, Hq, Hkv, Nq, Nk = 1, 2, 1, 384, 1000
    q = grid((B, Hq, Nq, 128), True, -2, 0)
    k = grid((B, Hkv, Nk, 128), False, -4, -2)
    aligned = (np.arange(Nk) // 64) % 4 == 0
    k[:, :, aligned] = grid((B, Hkv, int(aligned.sum()), 128), True, -2, 0)
    v = rng.standard_normal((B, Hkv, Nk, 128))
    assert np.array_equal(mxfp4_values(q), q) and np.array_equal(mxfp4_values(k), k)
    tq, tk, tv = (_on_device(synth.f32_to_bf16_bits(x.astype(np.float32))) for x in (q, k, v))
    vv = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v.astype(np.float32))).astype(np.float64)
    for lam in (1e-3, 1e-1):
        two = A.prefill_twopass(tq, tk, tv, lam, causal=True, out_dtype=torch.float32)
        one = A.prefill(tq, tk, tv, lam, causal=True, out_dtype=torch.float32)
        ref = oracle.prefill(q, k, vv, lam, True, 128, 64)
        assert (ref.mask == 0).any(), "fixture must drop tiles"
        near = np.abs(ref.gap - math.log(lam)) <= 1e-3
        for got in (two.mask.cpu().numpy(), one.mask.cpu().numpy()):
            assert ((got == ref.mask) | near).all()
        d = (two.out - one.out).abs().max().item()
        assert d <= 1e-2, d


@pytest.mark.parametrize("lam,gain,out", [(1e-3, 1.0, "bf16"), (1e-2, 6.0, "bf16"),
                                          (1e-3, 6.0, "fp32")])
def test_prefill_twopass_llama8b_n32768(lam, gain, out):
    """The benchmark's two-pass configuration: sampled query tiles against the
    oracle, whole-call invariants on the map."""
    w = synth.WORKLOADS[2].with_gain(gain)
    inp = synth.make_inputs(w)
    res = _twopass(inp, w, lam, out)
    tally = Tally()
    cache = {}
    for (h, i) in sample_qtiles(w, [0, 13, 31], 3, seed=6):
        kvh = h // w.G
        if kvh not in cache:
            kf, vf = synth.to_float(inp.k[0, kvh], w), synth.to_float(inp.v[0, kvh], w)
            cache = {kvh: (kf, vf, mxfp4_values(kf))}
        kf, vf, kd = cache[kvh]
        prefill_twopass_tile_parity(res, inp, w, lam, 0, h, i, tally, kf=kf, vf=vf, kd=kd)
    m = res.mask.cpu().numpy()
    nqt, nkt = m.shape[2], m.shape[3]
    assert (m[..., 0] == 1).all()
    last_vis = (np.minimum((np.arange(nqt) + 1) * w.br, w.Nq) - 1 + w.Nk - w.Nq) // w.bc
    assert ((m == 2) == (np.arange(nkt)[None, :] > last_vis[:, None])[None, None]).all()
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=(2, 3)))
    tally.check(w.dtype, f"twopass llama8b lam={lam} g={gain}", out_bf16=out == "bf16")
    if gain > 1.0:
        assert res.skip_fraction > 0.05


def test_prefill_twopass_qwen7b_n131072_low_needles():
    """The benchmark's skip-regime two-pass call: the 131072-long layer (28 query
    heads on 4 KV heads, so seven query heads share each map-kernel unit) with
    every KV head at 0.1% needles, gain 8, lambda 1e-3. Sampled query tiles of
    heads in three KV groups against the oracle, and whole-call invariants on
    the map, which must drop most tiles."""
    w = synth.WORKLOADS[4].scaled(needle_rate=0.001, needle_rate_range=None).with_gain(8.0)
    inp = synth.make_inputs(w)
    res = _twopass(inp, w, 1e-3, "bf16")
    tally = Tally()
    cache = {}
    for (h, i) in sample_qtiles(w, [0, 13, 27], 1, seed=7):
        kvh = h // w.G
        if kvh not in cache:
            kf, vf = synth.to_float(inp.k[0, kvh], w), synth.to_float(inp.v[0, kvh], w)
            cache = {kvh: (kf, vf, mxfp4_values(kf))}
        kf, vf, kd = cache[kvh]
        prefill_twopass_tile_parity(res, inp, w, 1e-3, 0, h, i, tally, kf=kf, vf=vf, kd=kd)
    m = res.mask.cpu().numpy()
    nqt, nkt = m.shape[2], m.shape[3]
    assert (m[..., 0] == 1).all()
    last_vis = (np.minimum((np.arange(nqt) + 1) * w.br, w.Nq) - 1 + w.Nk - w.Nq) // w.bc
    assert ((m == 2) == (np.arange(nkt)[None, :] > last_vis[:, None])[None, None]).all()
    st = res.stats.cpu().numpy()
    assert np.array_equal(st[..., 0], (m != 2).sum(axis=(2, 3)))
    assert np.array_equal(st[..., 1], (m == 1).sum(axis=(2, 3)))
    tally.check(w.dtype, "twopass qwen7b low needles lam=1e-3 g=8", out_bf16=True)
    assert res.skip_fraction > 0.5


def test_prefill_twopass_map_in_workspace_matches():
    """Without mask_out the map lives in the workspace; out, lse and statistics
    are the same bits as with it."""
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=300, Nk=700, d=128, dtype="bf16",
                             br=128, bc=64, gain=6.0, seed=64, window=32, causal=True)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    ref = A.prefill_twopass(q, k, v, 1e-2, causal=True)
    got = A.prefill_twopass(q, k, v, 1e-2, causal=True, want_mask=False)
    torch.cuda.synchronize()
    assert got.mask is None
    assert torch.equal(ref.out.view(torch.int16), got.out.view(torch.int16))
    assert torch.equal(ref.lse, got.lse)
    assert torch.equal(ref.stats, got.stats)


def test_prefill_twopass_strided_layout_matches_contiguous():
    """[B, N, H, d] storage (heads interleaved) gives the same bits as [B, H, N, d]."""
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=257, Nk=400, d=128, dtype="bf16",
                             br=128, bc=64, gain=6.0, seed=65, window=32, causal=True)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    ref = A.prefill_twopass(q, k, v, 1e-2, causal=True)
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert qs.stride(2) == w.Hq * w.d
    got = A.prefill_twopass(qs, ks, vs, 1e-2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(ref.out.view(torch.int16), got.out.view(torch.int16))
    assert torch.equal(ref.mask, got.mask)
    assert torch.equal(ref.stats, got.stats)


def test_prefill_twopass_rejected_call_leaves_outputs_untouched():
    w = synth.small_workload("prefill", Nq=200, Nk=200, seed=66)
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    out = torch.full((1, w.Hq, 200, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.BlasstError) as e:
        A.prefill_twopass(q, k, v, 1.5, out=out)
    assert e.value.status == 4
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(A.BlasstError) as e:
        A.prefill_twopass(q, k, v, 1e-2, out=out, workspace=small)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert (out == 7.0).all()
