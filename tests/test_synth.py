"""Input generator checks (no GPU): determinism, slice regeneration, bf16 rounding."""
import numpy as np
import torch

from block_sparse_long_skip_amd import synth


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    x = x.astype(np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_regenerate_exactly():
    w = synth.small_workload("prefill", B=2, Hq=4, Hkv=2, Nq=77, Nk=77, d=128, window=16, seed=3)
    inp = synth.make_inputs(w, threads=4)
    u = synth.unit_direction(w)
    assert np.array_equal(inp.k[1, 1], synth.k_slice(w, 1, 1, u))
    assert np.array_equal(inp.q[0, 3], synth.q_slice(w, 0, 3, u))
    assert np.array_equal(inp.v[1, 0], synth.v_slice(w, 1, 0))
    again = synth.make_inputs(w, threads=1)
    for a, b in ((inp.q, again.q), (inp.k, again.k), (inp.v, again.v)):
        assert np.array_equal(a, b)


def test_planting_recipe():
    w = synth.small_workload("decode", B=1, Hq=4, Hkv=2, Nk=4000, d=64, dtype="fp32",
                             needle_rate=0.01, window=256, seed=5, gain=2.0)
    u = synth.unit_direction(w)
    assert abs(np.linalg.norm(u) - 1) < 1e-6
    pos = synth.needle_positions(w, 0, 1)
    assert len(pos) == 40 and pos.min() >= 4 and len(np.unique(pos)) == 40
    k = synth.k_slice(w, 0, 1, u)
    proj = k @ u
    # sinks and needles carry +4g along u, the last 256 keys +2g, the rest none
    base = np.ones(w.Nk, bool)
    base[:4] = False
    base[pos] = False
    base[-256:] = False
    assert abs(proj[base].mean()) < 0.1
    assert abs(proj[:4].mean() - 8.0) < 1.5
    assert abs(proj[pos[pos < w.Nk - 256]].mean() - 8.0) < 0.6


def test_workload_table():
    w2 = synth.WORKLOADS[2]
    assert (w2.B, w2.Hq, w2.Hkv, w2.Nq, w2.d, w2.br, w2.bc) == (1, 32, 8, 32768, 128, 128, 64)
    assert synth.dense_equivalent_flops(w2) == 2 * 256 * 32 * (32768 * 32769 // 2)
    w4 = synth.WORKLOADS[4]
    r = synth.needle_rates(w4)
    assert r.shape == (4,) and (r >= 0.001).all() and (r <= 0.05).all()
    w5 = synth.WORKLOADS[5]
    assert w5.v_is_k_slice and (w5.d, w5.dv, w5.Hq, w5.Hkv) == (576, 512, 128, 1)
