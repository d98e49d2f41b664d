"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the
algorithmic work counted for the roofline, and the rule that counter traffic
is reported only for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_long_skip_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_algorithmic_flops_of_the_bench_layer():
    """Causal N = 32768 with 128 x 64 tiles: query tile i sees 2(i + 1) key tiles,
    so each head visits sum_i 2(i + 1) = 256 * 257 tiles; every visited tile
    costs 2 Br Bc d for QK^T and a kept one another 2 Br Bc dv for P.V."""
    w = synth.WORKLOADS[2]
    per_head = 256 * 257
    stats = torch.zeros((w.B, w.Hq, 2), dtype=torch.int64)
    stats[..., 0] = per_head
    stats[..., 1] = per_head
    flops, visited, kept = bench.prefill_algorithmic_flops(w, stats)
    assert visited == kept == w.Hq * per_head == 2_105_344
    assert flops == 2.0 * 128 * 64 * (128 + 128) * 2_105_344
    # a dropped tile keeps its QK^T cost and loses its P.V cost
    stats[0, 0, 1] -= 10
    flops2, _, kept2 = bench.prefill_algorithmic_flops(w, stats)
    assert kept2 == kept - 10
    assert flops - flops2 == 2.0 * 128 * 64 * 128 * 10


def test_traffic_only_for_the_measured_source():
    path = os.path.join(bench.PROFILE_DIR, "prefill_bf16_llama8b_n32768.pmc.json")
    with open(path) as f:
        sha = json.load(f)["kernel_source_sha"]
    got, _ = bench.read_traffic("prefill_bf16_llama8b_n32768", sha)
    assert got is not None and got > 0
    other, why = bench.read_traffic("prefill_bf16_llama8b_n32768", "0" * len(sha))
    assert other is None and "changed" in why
    none, why = bench.read_traffic("no_such_kernel", sha)
    assert none is None


def test_source_hash_follows_the_text():
    a = bench.source_sha(bench.PREFILL_SOURCES)
    assert a == bench.source_sha(bench.PREFILL_SOURCES)
    assert a != bench.source_sha(bench.PREFILL_SOURCES[:1])


def test_headline_is_the_largest_prefill_layer():
    """The bench line's workload is the 131072-long Qwen2.5-7B-shaped prefill
    (28/4 heads): 1024 query tiles per head, tile i sees 2(i + 1) key tiles,
    so 28 * 1024 * 1025 = 29,388,800 visited tiles at lambda = 0."""
    w = synth.WORKLOADS[bench.HEADLINE_CFG]
    assert (w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.causal) == (131072, 131072, 28, 4, 128, True)
    assert w.Hq * sum(2 * (i + 1) for i in range(w.Nq // w.br)) == 29_388_800
    assert w.Nq * w.Nk >= max(x.Nq * x.Nk for x in synth.WORKLOADS.values() if x.kind == "prefill")
    low = bench.skip_regime_workload(w)
    assert (synth.needle_rates(low) == bench.SKIP_NEEDLE_RATE).all()
    assert (low.Nq, low.Hq, low.seed) == (w.Nq, w.Hq, w.seed)
