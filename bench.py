#!/usr/bin/env python3
"""Benchmark: BLASST skip-softmax attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one skip-softmax prefill call (the whole hot path: QK^T on MFMA, the
per-tile drop vote, V loads and P.V for kept tiles, the output, lse, the tile
mask and the statistics) over the Qwen2.5-7B-shaped long prefill layer, the
largest workload that runs on one GPU: causal, B=1, 28 query / 4 KV heads,
N=131072, d=128, bf16, 128x64 tiles, lambda=1e-3, seeded synthetic inputs
already resident in HBM. The line printed on stdout carries:

  value        dense-equivalent TFLOP/s = 2 (d + dv) B Hq P / t, where P is the
               number of visible (query, key) pairs (causal: N(N+1)/2); the
               same numerator is used for every lambda
  roofline     the prefill kernel against the bf16 MFMA peak (2.5 PFLOP/s):
               algorithmic FLOPs per launch (2 Br Bc d per visited tile for
               QK^T plus 2 Br Bc dv per kept tile for P.V) / mean launch time
               from HIP events on the launch stream; HBM traffic per launch
               from rocprofv3 counters when the committed counter summary
               matches the current kernel source
  lambda_sweep the headline layer at every lambda at gain 1 (the workload as
               specified, nothing is dropped) and at the supplementary gain 8:
               TFLOP/s, skip fraction (overall and per KV head with its needle
               rate) and speed-up over lambda = 0
  skip_regime  the same shape with every KV head at 0.1% needles, gain 8
               (supplementary): one-pass and two-pass against lambda = 0
  prefill_llama8b_n32768
               the Llama-3.1-8B-shaped layer (N=32768, 32/8 heads) the same way,
               at gains 1 and 6
  block_sparse_prefill
               the Llama-shaped layer restricted to seeded block sets shaped like
               those of block-sparse prefill methods (sink tile, local window,
               vertical columns, scattered blocks) at densities 0.1 and 0.25:
               algorithmic TFLOP/s of the selected work and speed-up over dense
               lambda = 0
  prefill_backward
               dq, dk, dv of the Llama-shaped layer with the forward's mask held
               fixed: algorithmic TFLOP/s (5 products per kept tile)
  prefill_twopass
               the two-pass variant on the Llama-shaped layer (MXFP4 max
               pre-pass, then exact attention over the kept tiles): time against
               the one-pass call, the pre-pass share, agreement of its map with
               the exact rule's mask, and FP4 TFLOP/s of the pre-pass
  decode       the batch-32 GQA decode over 65536 keys, the same layer for one
               sequence (cache split over workgroups) and the batch-16 MLA
               decode over 32768 latent keys: GB/s of the bytes actually read
               (K always, V only for tiles some head keeps) against 8 TB/s
  cpu_baseline the CPU oracle timed on a bounded sample of query tiles of the
               headline layer (a reported baseline, not a target)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense FP4 MFMA
PEAK_HBM_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
PREFILL_SOURCES = ["block_sparse_long_skip_amd/csrc/prefill_bf16.hip",
                   "block_sparse_long_skip_amd/csrc/common.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--lam", type=float, default=1e-3, help="headline lambda")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-masked", action="store_true", help="skip the block-sparse prefill leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward leg")
    ap.add_argument("--no-twopass", action="store_true", help="skip the two-pass prefill leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget")
    ap.add_argument("--only", choices=["prefill", "prefill_masked", "backward", "twopass",
                                       "twopass_skip", "decode_gqa", "decode_gqa_b1", "decode_mla",
                                       "copy"],
                    help="launch only this kernel --steps times (for rocprofv3 counter passes)")
    ap.add_argument("--workload", choices=["qwen7b", "llama8b"], default="qwen7b",
                    help="prefill layer of --only prefill: the 131072-long Qwen2.5-7B shape or "
                         "the 32768-long Llama-3.1-8B shape")
    return ap.parse_args()


# --------------------------------------------------------------------------- helpers

def to_device(x, w):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if w.dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def time_calls(fn, steps, warmup):
    """Run fn() warmup times, then time `steps` calls with HIP events on the current
    stream. Returns (mean ms per call from events, wall ms per step, last result,
    median ms per call)."""
    import torch
    res = None
    for _ in range(warmup):
        res = fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        starts[s].record()
        res = fn()
        ends[s].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    ev = sum(per) / steps
    med = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return ev, wall, res, med


def prefill_algorithmic_flops(w, stats):
    st = stats.double()
    visited = st[..., 0].sum().item()
    kept = st[..., 1].sum().item()
    return 2.0 * w.br * w.bc * (w.d * visited + w.dv * kept), visited, kept


def read_traffic(kind: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"{kind}.pmc.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != sha:
        return None, "kernel changed since the counters were taken"
    return d.get("hbm_bytes_per_launch"), os.path.relpath(path, os.path.dirname(PROFILE_DIR))


# --------------------------------------------------------------------------- legs

HEADLINE_CFG = 4  # the largest single-GPU workload: the Qwen2.5-7B-shaped 131072-long prefill
SKIP_NEEDLE_RATE = 0.001  # low end of that workload's per-head needle-rate range


def skip_regime_workload(w):
    """The headline shape with every KV head at the low end of its needle-rate
    range (0.1%): a supplementary input, not one of the listed workloads, where
    most tiles hold no planted key and the pages' 50-60% skip regime is reached."""
    from dataclasses import replace
    return replace(w, name=w.name + "_needles0.1pct", needle_rate=SKIP_NEEDLE_RATE,
                   needle_rate_range=None)


def per_group_skip(w, stats):
    """Skip fraction per KV head (its query heads pooled), with its needle rate."""
    from block_sparse_long_skip_amd import synth
    st = stats.double().cpu()
    rates = synth.needle_rates(w)
    out = []
    for g in range(w.Hkv):
        vis = st[:, g * w.G:(g + 1) * w.G, 0].sum().item()
        kept = st[:, g * w.G:(g + 1) * w.G, 1].sum().item()
        out.append(dict(kv_head=g, needle_rate=round(float(rates[g]), 5),
                        skip_fraction=round(1.0 - kept / max(vis, 1.0), 4)))
    return out


def prefill_row(w, lam, gain, ms, res, dense, base_ms):
    alg, visited, kept = prefill_algorithmic_flops(w, res.stats)
    atf = alg / (ms * 1e-3) / 1e12
    return dict(gain=gain, lam=lam, ms=round(ms, 4), tflops=round(dense / (ms * 1e-3) / 1e12, 2),
                algorithmic_tflops=round(atf, 2), frac_mfma=round(atf / PEAK_BF16_TFLOPS, 4),
                skip_fraction=round(res.skip_fraction, 4),
                speedup_vs_lam0=round(base_ms / ms, 3) if base_ms else None)


def bench_prefill(args, cid, kind, gains, skip_regime=False):
    """One causal prefill workload: the headline lambda at gain 1 timed over
    --steps calls (value, roofline), then a lambda sweep at each listed gain
    (and, with skip_regime, on the low-needle variant, one-pass and two-pass)."""
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    w = synth.WORKLOADS[cid]
    log(f"[bench] generating {w.name} (gain 1)")
    inp = synth.make_inputs(w)
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    del inp
    dense = synth.dense_equivalent_flops(w)

    def call(lam, q_=q, k_=k, v_=v):
        return A.prefill(q_, k_, v_, lam, causal=True, br=w.br, bc=w.bc)

    log(f"[bench] timing {w.name} lambda={args.lam} steps={args.steps} warmup={args.warmup}")
    ev_ms, wall_ms, res, med_ms = time_calls(lambda: call(args.lam), args.steps, args.warmup)
    alg, visited, kept = prefill_algorithmic_flops(w, res.stats)
    value = dense / (ev_ms * 1e-3) / 1e12
    achieved = alg / (ev_ms * 1e-3) / 1e12
    sha = source_sha(PREFILL_SOURCES)
    traffic, tnote = read_traffic(f"prefill_bf16_{kind}", sha)
    out = dict(workload=w.name, value=value, ms_per_step=ev_ms, median_ms=med_ms,
               wall_ms_per_step=wall_ms, skip_fraction=1.0 - kept / visited,
               visited_tiles=int(visited), kept_tiles=int(kept),
               roofline=dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                             unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                             traffic=traffic, traffic_note=tnote,
                             algorithmic_flops_per_launch=alg,
                             kernel="prefill_bf16_kernel<false>", kernel_source_sha=sha))
    log(f"[bench]   {w.name}: {ev_ms:.3f} ms (median {med_ms:.3f}), {value:.1f} dense-equivalent "
        f"TFLOP/s, {achieved / PEAK_BF16_TFLOPS:.3f} of the bf16 peak")
    sweep = []
    reps = max(3, args.steps // 2)
    if not args.no_sweep:
        for gain in gains:
            if gain != 1.0:
                log(f"[bench] generating {w.name} gain {gain}")
                gi = synth.make_inputs(w.with_gain(gain))
                q2, k2, v2 = (to_device(x, w) for x in (gi.q, gi.k, gi.v))
                del gi
            else:
                q2, k2, v2 = q, k, v
            base = None
            for lam in w.lambdas + ((1e-2,) if gain != 1.0 and 1e-2 not in w.lambdas else ()):
                ms, _, r, _ = time_calls(lambda: call(lam, q2, k2, v2), reps, args.warmup)
                base = ms if lam == 0.0 else base
                row = prefill_row(w, lam, gain, ms, r, dense, base)
                if w.Hkv > 1 and lam > 0:
                    row["per_kv_head"] = per_group_skip(w.with_gain(gain), r.stats)
                sweep.append(row)
                log(f"[bench]   gain {gain} lam {lam}: {ms:.3f} ms, skip {r.skip_fraction:.3f}")
            del q2, k2, v2
            torch.cuda.empty_cache()
    out["sweep"] = sweep
    if skip_regime and not args.no_sweep:
        out["skip_regime"] = bench_skip_regime(args, w, dense, reps)
    del q, k, v, res
    torch.cuda.empty_cache()
    return out, w


def bench_skip_regime(args, w, dense, reps):
    """The low-needle variant of the workload at gain 8: one-pass at every
    lambda, and the two-pass variant (MXFP4 max pre-pass, then exact attention
    over the kept tiles) beside it."""
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    ws_ = skip_regime_workload(w).with_gain(8.0)
    log(f"[bench] generating {ws_.name} gain 8 (skip regime)")
    gi = synth.make_inputs(ws_)
    q, k, v = (to_device(x, ws_) for x in (gi.q, gi.k, gi.v))
    del gi
    wsp = torch.empty(A.prefill_twopass_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk),
                      dtype=torch.uint8, device="cuda")
    rows, base = [], None
    for lam in (0.0, 1e-3, 1e-2):
        ms, _, r, _ = time_calls(lambda: A.prefill(q, k, v, lam, causal=True), reps, args.warmup)
        base = ms if lam == 0.0 else base
        row = prefill_row(ws_, lam, 8.0, ms, r, dense, base)
        if lam > 0:
            tms, _, tr, _ = time_calls(lambda: A.prefill_twopass(q, k, v, lam, causal=True,
                                                                 workspace=wsp), reps, args.warmup)
            vis = r.mask != 2
            row["twopass"] = dict(ms=round(tms, 4), speedup_vs_lam0=round(base / tms, 3),
                                  speedup_vs_one_pass=round(ms / tms, 3),
                                  skip_fraction=round(tr.skip_fraction, 4),
                                  map_agreement=round(((tr.mask == r.mask) & vis).sum().item()
                                                      / max(vis.sum().item(), 1), 5))
            del tr, vis
        rows.append(row)
        log(f"[bench]   skip regime lam {lam}: {ms:.3f} ms, skip {r.skip_fraction:.3f}"
            + (f", two-pass {row['twopass']['ms']:.3f} ms" if "twopass" in row else ""))
        del r
    del q, k, v, wsp
    torch.cuda.empty_cache()
    return dict(workload=ws_.name, needle_rate=SKIP_NEEDLE_RATE, gain=8.0,
                note="supplementary input (not a listed workload): every KV head at the low end "
                     "of the needle-rate range", rows=rows)


def bench_prefill_masked(args, dense_ms):
    """Block-sparse prefill on the same layer: CRISP-shaped block sets (sink tile,
    a 2-tile local window at the diagonal, per-head vertical columns and scattered
    blocks) of two densities, at lambda 0 and the headline lambda. Reports the
    algorithmic TFLOP/s of the selected work against the MFMA peak and the
    speed-up over the dense causal call at lambda 0."""
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    w = synth.WORKLOADS[2]
    rows = []
    for gain in (1.0, 6.0):
        log(f"[bench] generating {w.name} gain {gain} for block-sparse prefill")
        inp = synth.make_inputs(w.with_gain(gain))
        q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
        del inp
        for density in (0.1, 0.25):
            bm = torch.from_numpy(synth.block_set(w, density, seed=3)).cuda()
            for lam in (0.0, args.lam):
                # ~1 ms calls: warm up for tens of milliseconds so the clocks settle
                ms, _, r, _ = time_calls(lambda: A.prefill_masked(q, k, v, bm, lam, causal=True,
                                                               br=w.br, bc=w.bc),
                                      max(3, args.steps // 2), max(args.warmup, 30))
                alg, visited, kept = prefill_algorithmic_flops(w, r.stats)
                tf = alg / (ms * 1e-3) / 1e12
                rows.append(dict(gain=gain, density=density, lam=lam, ms=round(ms, 4),
                                 algorithmic_tflops=round(tf, 2),
                                 frac_mfma=round(tf / PEAK_BF16_TFLOPS, 4),
                                 visited_tiles=int(visited), kept_tiles=int(kept),
                                 skip_fraction=round(r.skip_fraction, 4),
                                 speedup_vs_dense_lam0=round(dense_ms / ms, 3)))
                log(f"[bench]   masked gain {gain} density {density} lam {lam}: {ms:.3f} ms "
                    f"{tf:.0f} TFLOP/s, visited {int(visited)} kept {int(kept)}")
            del bm
        del q, k, v
        torch.cuda.empty_cache()
    return rows


def bench_twopass(args):
    """Two-pass prefill on the bench layer (MXFP4 max pre-pass, then exact
    attention over the kept tiles) against the one-pass call at the same lambda.
    Pass 2 is timed alone as the block-sparse call over the map at lambda 0; the
    rest of the call (MXFP4 quantization of q and k and the map kernel) is the
    pre-pass, priced at 2 Br Bc d FP4 FLOPs per visited tile against the FP4 peak."""
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    w = synth.WORKLOADS[2]
    ws = torch.empty(A.prefill_twopass_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk),
                     dtype=torch.uint8, device="cuda")
    rows = []
    for gain, lams in ((1.0, (args.lam,)), (6.0, (1e-3, 1e-2, 1e-1))):
        log(f"[bench] generating {w.name} gain {gain} for the two-pass prefill")
        inp = synth.make_inputs(w.with_gain(gain))
        q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
        del inp
        for lam in lams:
            steps, warm = max(3, args.steps // 2), max(args.warmup, 5)
            one_ms, _, one, _ = time_calls(lambda: A.prefill(q, k, v, lam, causal=True), steps, warm)
            two_ms, _, two, _ = time_calls(lambda: A.prefill_twopass(q, k, v, lam, causal=True,
                                                                  workspace=ws), steps, warm)
            kept = two.mask == 1
            p2_ms, _, _, _ = time_calls(lambda: A.prefill_masked(q, k, v, kept, 0.0, causal=True,
                                                              want_mask=False, want_stats=False),
                                     steps, warm)
            pre_ms = max(two_ms - p2_ms, 1e-6)
            visited = (two.mask != 2)
            n_vis = int(visited.sum().item())
            agree = int(((two.mask == one.mask) & visited).sum().item())
            fp4_tf = 2.0 * w.br * w.bc * w.d * n_vis / (pre_ms * 1e-3) / 1e12
            dev = (two.out.float() - one.out.float()).abs().max().item()
            rows.append(dict(gain=gain, lam=lam, ms=round(two_ms, 4), one_pass_ms=round(one_ms, 4),
                             speedup_vs_one_pass=round(one_ms / two_ms, 3),
                             prepass_ms=round(pre_ms, 4), pass2_ms=round(p2_ms, 4),
                             skip_fraction=round(two.skip_fraction, 4),
                             one_pass_skip_fraction=round(one.skip_fraction, 4),
                             map_agreement=round(agree / max(n_vis, 1), 5),
                             max_abs_out_vs_one_pass=round(dev, 5),
                             prepass_fp4_tflops=round(fp4_tf, 1),
                             prepass_frac_fp4=round(fp4_tf / PEAK_FP4_TFLOPS, 4)))
            log(f"[bench]   twopass gain {gain} lam {lam}: {two_ms:.3f} ms (pre {pre_ms:.3f} + "
                f"pass2 {p2_ms:.3f}) vs one-pass {one_ms:.3f} ms; skip {two.skip_fraction:.3f} "
                f"(one-pass {one.skip_fraction:.3f}), map agreement {agree / max(n_vis, 1):.4f}")
            del one, two, kept, visited
        del q, k, v
        torch.cuda.empty_cache()
    return rows


def backward_inputs(w, lam, gain):
    """Forward on the GPU (its mask, lse and bf16 output feed the backward) and a
    seeded bf16 dout."""
    import numpy as np
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    inp = synth.make_inputs(w.with_gain(gain))
    q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
    del inp
    fwd = A.prefill(q, k, v, lam, causal=True, br=w.br, bc=w.bc)
    g = np.random.default_rng(7).standard_normal((w.B, w.Hq, w.Nq, w.dv)).astype(np.float32)
    dout = torch.from_numpy(g).to(torch.bfloat16).cuda()
    return q, k, v, fwd, dout


def bench_backward(args):
    """The prefill backward (dq, dk, dv with the forward's mask held fixed) on the
    bench layer: algorithmic TFLOP/s = 5 products of 2 Br Bc d FLOPs per kept
    tile (S recomputed, dP, dV, dK, dQ) over the call time."""
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    w = synth.WORKLOADS[2]
    rows = []
    for gain, lam in ((1.0, args.lam), (6.0, 1e-2)):
        log(f"[bench] backward inputs gain {gain} lam {lam}")
        q, k, v, fwd, dout = backward_inputs(w, lam, gain)
        ws = torch.empty(max(1, w.B * w.Hq * w.Nq * 4), dtype=torch.uint8, device="cuda")
        call = lambda: A.prefill_backward(q, k, v, fwd.out, dout, fwd.lse, fwd.mask, causal=True,
                                          workspace=ws)
        ms, _, _, _ = time_calls(call, max(3, args.steps // 4), max(args.warmup, 2))
        kept = fwd.stats[..., 1].double().sum().item()
        flops = 5 * 2.0 * w.br * w.bc * w.d * kept
        dense = 2.5 * synth.dense_equivalent_flops(w)  # 5 products of 2 d FLOPs per visible pair
        tf = flops / (ms * 1e-3) / 1e12
        rows.append(dict(gain=gain, lam=lam, ms=round(ms, 4), kept_tiles=int(kept),
                         skip_fraction=round(fwd.skip_fraction, 4),
                         algorithmic_tflops=round(tf, 2), frac_mfma=round(tf / PEAK_BF16_TFLOPS, 4),
                         dense_equiv_tflops=round(dense / (ms * 1e-3) / 1e12, 2)))
        log(f"[bench]   backward gain {gain} lam {lam}: {ms:.3f} ms {tf:.0f} TFLOP/s "
            f"skip {fwd.skip_fraction:.3f}")
        del q, k, v, fwd, dout, ws
        torch.cuda.empty_cache()
    return rows


def bench_decode(args):
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth

    results = {}
    # Every timed call follows a read of this 1 GiB buffer, which evicts the cache
    # from L2 and MALL. A read, not a fill: a fill leaves about 300 MB of dirty
    # lines there, and writing them back (≈40 µs) would be charged to the decode.
    flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
    # the batch-32 GQA decode, the same layer for a single sequence (its cache
    # split over workgroups), and the batch-16 MLA decode
    for w, kind in ((synth.WORKLOADS[3], "decode_gqa_b32_n65536"),
                    (synth.WORKLOADS[3].scaled(B=1), "decode_gqa_b1_n65536"),
                    (synth.WORKLOADS[5], "decode_mla_b16_n32768")):
        rows = []
        for gain in (1.0, 6.0):
            log(f"[bench] generating {w.name} gain {gain}")
            inp = synth.make_inputs(w.with_gain(gain))
            q, k = to_device(inp.q, w), to_device(inp.k, w)
            v = to_device(inp.v, w) if inp.v is not None else None
            del inp
            nws = A.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.dv, latent=v is None,
                                          bc=w.bc)
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
            for lam in w.lambdas:
                times = []
                res = None
                # three untimed calls first: the GPU sat idle while the host generated
                # the inputs, and the first calls after that run at a lower clock
                nwarm = 3
                for it in range(nwarm + max(3, args.steps // 2)):
                    torch.sum(flush)
                    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s.record()
                    res = A.decode(q, k, v, lam, bc=w.bc, dv=w.dv, workspace=ws)
                    e.record()
                    torch.cuda.synchronize()
                    if it >= nwarm:
                        times.append(s.elapsed_time(e))
                ms = sum(times) / len(times)
                st = res.stats.double()
                G = w.G
                vtiles = st[:, ::G, 2].sum().item()  # per (batch, KV head)
                kbytes = w.B * w.Hkv * w.Nk * w.d * 2
                vbytes = vtiles * w.bc * w.dv * 2 if v is not None else 0
                qo = w.B * w.Hq * (w.d + w.dv) * 2
                byt = kbytes + vbytes + qo
                gbs = byt / (ms * 1e-3) / 1e9
                rows.append(dict(gain=gain, lam=lam, ms=round(ms, 4), gbs=round(gbs, 1),
                                 frac_hbm=round(gbs / PEAK_HBM_GBS, 4),
                                 bytes_read=int(byt), skip_fraction=round(res.skip_fraction, 4),
                                 v_tiles_read_fraction=(round(vtiles / (w.B * w.Hkv * res.mask.shape[2]), 4)
                                                        if v is not None else None)))
                log(f"[bench]   {kind} gain {gain} lam {lam}: {ms:.3f} ms {gbs:.0f} GB/s "
                    f"skip {res.skip_fraction:.3f}")
            del q, k, v, ws
            torch.cuda.empty_cache()
        results[kind] = rows
    del flush
    return results


def cpu_baseline(args, w):
    """The oracle, as it stands, on a time-bounded sample of query tiles (head 0,
    tiles drawn at random), at the headline lambda; dense-equivalent TFLOP/s."""
    import numpy as np
    import oracle
    from block_sparse_long_skip_amd import synth

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads") or 0) for d in threadpool_info()) or None
    except Exception:  # noqa: BLE001
        pass
    cores = threads or len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                             cpu_model)
    except OSError:
        pass
    u = synth.unit_direction(w)
    kf = synth.to_float(synth.k_slice(w, 0, 0, u), w)
    vf = synth.to_float(synth.v_slice(w, 0, 0), w)
    qh = synth.to_float(synth.q_slice(w, 0, 0, u), w)
    nqt = synth.n_tiles(w.Nq, w.br)
    order = np.random.default_rng(12345).permutation(nqt)
    flops, done, t0 = 0.0, [], time.perf_counter()
    scale = 1.0 / math.sqrt(w.d)
    for i in order:
        r0, r1 = i * w.br, min((i + 1) * w.br, w.Nq)
        vis = oracle.visible(w.Nq, w.Nk, True, r0, r1 - r0)
        oracle.blasst_rows(qh[r0:r1], kf, vf, args.lam, w.bc, vis, scale)
        flops += 2.0 * (w.d + w.dv) * float(vis.sum())
        done.append(int(i))
        if time.perf_counter() - t0 > args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{len(done)} of {nqt} query tiles of head 0 of {w.name} (random order, "
                       f"seed 12345), lambda={args.lam}, float64 NumPy, {dt:.1f} s",
                seconds=round(dt, 2), cpu_model=cpu_model)


def only(args):
    """Launch a single kernel `steps` times (used under rocprofv3 counter passes)."""
    import torch
    from block_sparse_long_skip_amd import attention as A
    from block_sparse_long_skip_amd import synth
    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x {args.steps}")
        return
    if args.only in ("twopass", "twopass_skip"):
        # the Llama-shaped layer at gain 6, lambda 1e-2; or the headline layer's
        # low-needle input at gain 8, lambda 1e-3 (the skip regime)
        if args.only == "twopass":
            w, gain, lam = synth.WORKLOADS[2], 6.0, 1e-2
        else:
            w, gain, lam = skip_regime_workload(synth.WORKLOADS[HEADLINE_CFG]), 8.0, 1e-3
        inp = synth.make_inputs(w.with_gain(gain))
        q, k, v = (to_device(x, w) for x in (inp.q, inp.k, inp.v))
        del inp
        ws = torch.empty(A.prefill_twopass_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk),
                         dtype=torch.uint8, device="cuda")
        for _ in range(args.steps):
            A.prefill_twopass(q, k, v, lam, causal=True, workspace=ws)
        torch.cuda.synchronize()
        log(f"[bench] launched two-pass ({w.name}, gain {gain}, lambda {lam}) x {args.steps}")
        return
    if args.only == "backward":
        w = synth.WORKLOADS[2]
        q, k, v, fwd, dout = backward_inputs(w, args.lam, 1.0)
        for _ in range(args.steps):
            A.prefill_backward(q, k, v, fwd.out, dout, fwd.lse, fwd.mask, causal=True)
        torch.cuda.synchronize()
        log(f"[bench] launched backward x {args.steps}")
        return
    cid = {"prefill": {"qwen7b": 4, "llama8b": 2}[args.workload], "prefill_masked": 2,
           "decode_gqa": 3, "decode_gqa_b1": 3, "decode_mla": 5}[args.only]
    w = synth.WORKLOADS[cid]
    if args.only == "decode_gqa_b1":
        w = w.scaled(B=1)  # one sequence: the cache is split over workgroups
    inp = synth.make_inputs(w)
    q, k = to_device(inp.q, w), to_device(inp.k, w)
    v = to_device(inp.v, w) if inp.v is not None else None
    ws = None
    if w.kind != "prefill":
        nws = A.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.dv, latent=v is None,
                                      bc=w.bc)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    if args.only == "prefill":
        # the headline leg's own timing loop, so a kernel trace of this run and
        # the HIP-event mean it prints cover the same launches
        ms, _, res, med = time_calls(lambda: A.prefill(q, k, v, args.lam, causal=True, br=w.br,
                                                       bc=w.bc), args.steps, args.warmup)
        alg, _, _ = prefill_algorithmic_flops(w, res.stats)
        print(json.dumps(dict(workload=w.name, lam=args.lam, warmup=args.warmup,
                              steps=args.steps, event_mean_ms=round(ms, 4),
                              event_median_ms=round(med, 4),
                              algorithmic_flops_per_launch=alg,
                              frac=round(alg / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))),
              flush=True)
        return
    bm = torch.from_numpy(synth.block_set(w, 0.1, seed=3)).cuda() if args.only == "prefill_masked" else None
    for _ in range(args.steps):
        if bm is not None:
            A.prefill_masked(q, k, v, bm, args.lam, causal=True, br=w.br, bc=w.bc, want_stats=False)
        elif w.kind == "prefill":
            A.prefill(q, k, v, args.lam, causal=True, br=w.br, bc=w.bc, want_stats=False)
        else:
            A.decode(q, k, v, args.lam, bc=w.bc, dv=w.dv, want_stats=False, workspace=ws)
    torch.cuda.synchronize()
    log(f"[bench] launched {args.only} x {args.steps}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single MI355X; sharding is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from block_sparse_long_skip_amd import attention as A
    A.load_library()
    if args.only:
        only(args)
        return
    t_start = time.perf_counter()
    pre, w = bench_prefill(args, HEADLINE_CFG, "qwen7b_n131072", gains=(1.0, 8.0), skip_regime=True)
    llama, _ = bench_prefill(args, 2, "llama8b_n32768", gains=(1.0, 6.0))
    dense_ms = next((x["ms"] for x in llama["sweep"] if x["gain"] == 1.0 and x["lam"] == 0.0), None)
    masked = None if args.no_masked or dense_ms is None else bench_prefill_masked(args, dense_ms)
    backward = None if args.no_backward else bench_backward(args)
    twopass = None if args.no_twopass else bench_twopass(args)
    decode = None if args.no_decode else bench_decode(args)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, w)
    line = {
        "metric": "dense-equiv attention TFLOP/s + decode KV GB/s vs roofline, skip fraction per λ",
        "value": round(pre["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded planted sinks/needles/recent window, gain 1)",
        "config": {"workload": "prefill_qwen7b_n131072: causal B=1 Hq=28 Hkv=4 N=131072 d=128 "
                               "bf16 128x64 tiles", "lambda": args.lam, "gain": 1.0,
                   "out_dtype": "bf16", "skip_fraction": round(pre["skip_fraction"], 4),
                   "median_ms": round(pre["median_ms"], 4)},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "lambda_sweep": pre["sweep"],
        "skip_regime": pre.get("skip_regime"),
        "prefill_llama8b_n32768": {k_: llama[k_] for k_ in ("value", "ms_per_step", "median_ms",
                                                           "roofline", "sweep")},
        "block_sparse_prefill": masked,
        "prefill_backward": backward,
        "prefill_twopass": twopass,
        "decode": decode,
        "wall_s": round(time.perf_counter() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
