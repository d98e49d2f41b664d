"""Pins for the CPU oracle (no GPU).

Each ``pin_*`` function checks the oracle against something other than
itself: hand-derived fixtures under tests/golden, torch's CPU
scaled_dot_product_attention in float64, the closed form implied by the
prefix-max invariant, and a from-definition brute force. The mutation tests
at the bottom plant plausible mistakes in a copy of the oracle's source and
check that at least one pin catches each of them.
"""
import importlib.util
import json
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_skip_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f(x):
    return float(x) if not isinstance(x, str) else float(x.replace("inf", "inf"))


def _rand_case(rng, B, Hq, Hkv, Nq, Nk, d, dv, plant=0.0):
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, dv))
    if plant:
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        q += plant * u
        idx = rng.choice(Nk, size=max(1, Nk // 12), replace=False)
        k[:, :, idx] += plant * u
        k[:, :, 0] += plant * u
    return q, k, v


def _sdpa(q, k, v, causal, scale, attn_mask=None):
    """torch CPU float64 reference for one head or a batch of heads."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    return torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, is_causal=causal and attn_mask is None, scale=scale).numpy()


# --------------------------------------------------------------------------- pins

def pin_hand_example(orc):
    g = _load("hand_example.json")
    sh = g["shape"]
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for case in g["cases"]:
        lam = math.exp(case["log_lambda"]) if case["log_lambda"] != "-inf" else 0.0
        r = orc.prefill(q, k, v, lam, sh["causal"], sh["br"], sh["bc"], scale=sh["scale"])
        assert r.mask[0, 0, 0].tolist() == case["mask"]
        assert np.allclose(r.gap[0, 0, 0], [_f(x) for x in case["gap"]], rtol=0, atol=1e-12)
        ks = np.array(case["out_terms"]["kept_scores"])
        kv = np.array(case["out_terms"]["kept_values"])
        # closed form: softmax over the kept keys only
        want_out = float((np.exp(ks) * kv).sum() / np.exp(ks).sum())
        want_lse = float(np.log(np.exp(ks).sum()))
        assert abs(r.out[0, 0, 0, 0] - want_out) < 1e-12
        assert abs(r.lse[0, 0, 0] - want_lse) < 1e-12
    # the first case's closed form to ten digits: (1 + 3e) / (1 + e)
    assert abs((1 + 3 * math.e) / (1 + math.e) - 2.4621171573) < 1e-10


def pin_row_aggregation(orc):
    g = _load("row_aggregation.json")
    sh = g["shape"]
    q = np.array(g["q"])[None, None]
    for case in g["cases"]:
        k = np.array(case["k"])[None, None]
        v = np.arange(sh["Nk"], dtype=np.float64).reshape(1, 1, sh["Nk"], 1)
        r = orc.prefill(q, k, v, g["lambda"], sh["causal"], sh["br"], sh["bc"], scale=sh["scale"])
        assert r.mask[0, 0, 0].tolist() == case["mask"], case["derivation"]
        assert np.allclose(r.gap[0, 0, 0], [_f(x) for x in case["gap"]])


def pin_tie(orc):
    g = _load("tie.json")
    q = np.array(g["q"])[None, None]
    for case in g["cases"]:
        k = np.array(case["k"])[None, None]
        v = np.array(case["v"])[None, None]
        r = orc.prefill(q, k, v, g["lambda"], False, 1, 1, scale=1.0)
        assert r.mask[0, 0, 0].tolist() == case["mask"], case["derivation"]
        if "out" in case:
            assert abs(r.out[0, 0, 0, 0] - case["out"]) < 1e-12


def pin_causal_visibility(orc):
    g = _load("causal_visibility.json")
    sh = g["shape"]
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, sh["Nq"], 1))
    k = rng.standard_normal((1, 1, sh["Nk"], 1))
    v = rng.standard_normal((1, 1, sh["Nk"], 1))
    r = orc.prefill(q, k, v, 0.0, True, sh["br"], sh["bc"], scale=1.0)
    assert r.mask[0, 0].tolist() == g["expect"]["mask_lambda0"]


def pin_lambda0_sdpa(orc):
    """lambda = 0 drops nothing: equals textbook softmax attention (torch SDPA, float64)."""
    rng = np.random.default_rng(1)
    for (B, Hq, Hkv, N, d, dv, br, bc, causal) in [
        (1, 2, 2, 37, 8, 8, 8, 4, True),
        (2, 4, 2, 53, 16, 12, 16, 8, True),   # GQA, dv != d, ragged
        (1, 6, 3, 40, 4, 4, 5, 7, False),
        (1, 3, 1, 129, 8, 8, 128, 64, True),  # the bf16 kernel's tiling, ragged tail
    ]:
        q, k, v = _rand_case(rng, B, Hq, Hkv, N, N, d, dv)
        sc = 1.0 / math.sqrt(d)
        r = orc.prefill(q, k, v, 0.0, causal, br, bc)
        G = Hq // Hkv
        kk = np.repeat(k, G, axis=1)  # q head h reads kv head h // G
        vv = np.repeat(v, G, axis=1)
        ref = _sdpa(q, kk, vv, causal, sc)
        assert np.abs(r.out - ref).max() < 1e-12
        # lse against logsumexp of the visible scores
        s = sc * np.einsum("bhqd,bhkd->bhqk", q, kk)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
        assert np.abs(r.lse - ref_lse).max() < 1e-12
        assert (r.mask[r.mask != 2] == 1).all()


def pin_bottom_right_causal(orc):
    """Causal with Nq < Nk equals the last Nq rows of the square causal problem."""
    rng = np.random.default_rng(2)
    Nk, Nq, d = 45, 13, 8
    qfull, k, v = _rand_case(rng, 1, 1, 1, Nk, Nk, d, d)
    ref = _sdpa(qfull, k, v, True, 1.0 / math.sqrt(d))[:, :, Nk - Nq:]
    r = orc.prefill(qfull[:, :, Nk - Nq:], k, v, 0.0, True, 4, 8)
    assert np.abs(r.out - ref).max() < 1e-12


def pin_masked_sdpa(orc):
    """lambda > 0: the output is softmax attention restricted to the kept tiles."""
    rng = np.random.default_rng(3)
    n_skipped = 0
    for (B, Hq, Hkv, Nq, Nk, d, br, bc, causal, lam) in [
        (1, 2, 1, 70, 70, 16, 8, 4, True, 1e-2),
        (1, 2, 2, 33, 90, 8, 4, 8, True, 1e-1),
        (2, 2, 1, 25, 64, 8, 5, 3, False, 1e-3),
    ]:
        q, k, v = _rand_case(rng, B, Hq, Hkv, Nq, Nk, d, d, plant=6.0)
        sc = 1.0 / math.sqrt(d)
        r = orc.prefill(q, k, v, lam, causal, br, bc)
        n_skipped += int((r.mask == 0).sum())
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                keep = orc.expand_tile_mask(r.mask[b, h], br, bc, Nq, Nk)
                r_idx = np.arange(Nq)[:, None] + (Nk - Nq)
                vis = (np.arange(Nk)[None, :] <= r_idx) if causal else np.ones((Nq, Nk), bool)
                am = keep & vis
                ref = _sdpa(q[b, h][None], k[b, h // G][None], v[b, h // G][None], False, sc,
                            attn_mask=am[None])
                assert np.abs(r.out[b, h] - ref[0]).max() < 1e-12
    assert n_skipped > 0, "fixture must exercise dropped tiles"


def pin_masked_dense_attention(orc):
    """Softmax restricted to a set of (query, key) pairs, the reference the GPU
    parity checks fall back to on near-threshold flips: the tile-to-pair
    expansion against a hand-built fixture, then the restricted softmax
    against torch SDPA (float64) with the same boolean mask, and its lse
    against torch.logsumexp of the allowed scores."""
    g = _load("tile_expansion.json")
    sh = g["shape"]
    el = orc.expand_tile_mask(np.array(g["tile_mask"], np.uint8), sh["br"], sh["bc"], sh["Nq"],
                              sh["Nk"])
    assert el.tolist() == g["expect"], g["derivation"]
    rng = np.random.default_rng(23)
    for (Nq, Nk, d, dv, causal) in [(9, 9, 4, 3, True), (6, 17, 8, 8, True), (11, 5, 4, 6, False)]:
        q, k, v = (rng.standard_normal((n, m)) * 2.0 for n, m in ((Nq, d), (Nk, d), (Nk, dv)))
        keep = rng.random((Nq, Nk)) < 0.5
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq) if causal \
            else np.ones((Nq, Nk), bool)
        keep[np.arange(Nq), np.arange(Nq) + (Nk - Nq) if causal else 0] = True  # a pair per row
        sc = 0.7
        out, lse = orc.masked_dense_attention(q, k, v, keep, causal, sc)
        am = keep & vis
        ref = _sdpa(q[None], k[None], v[None], False, sc, attn_mask=am[None])[0]
        assert np.abs(out - ref).max() < 1e-12
        s = np.where(am, sc * (q @ k.T), -np.inf)
        assert np.abs(lse - torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()).max() < 1e-12


def _prefix_max_closed_form(q, k, lam, causal, br, bc, scale):
    """mask[i,j] = j==0 or max_r (tilemax[r,j] - max_{t<j} tilemax[r,t]) >= thr, from dense S."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    thr = -np.inf if lam == 0 else np.log(lam)
    nqt, nkt = -(-Nq // br), -(-Nk // bc)
    out = np.full((B, Hq, nqt, nkt), 2, dtype=np.uint8)
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, h] @ k[b, h // G].T
            if causal:
                s = np.where(np.arange(Nk)[None] <= np.arange(Nq)[:, None] + Nk - Nq, s, -np.inf)
            # pad to whole tiles with -inf, then per-(row, tile) maxima
            sp = np.full((nqt * br, nkt * bc), -np.inf)
            sp[:Nq, :Nk] = s
            tm = sp.reshape(nqt, br, nkt, bc).max(axis=3)  # [nqt, br, nkt]
            pm = np.maximum.accumulate(tm, axis=2)
            prev = np.concatenate([np.full((nqt, br, 1), -np.inf), pm[:, :, :-1]], axis=2)
            with np.errstate(invalid="ignore"):
                gap = np.where(tm == -np.inf, -np.inf, np.where(prev == -np.inf, np.inf, tm - prev))
            g = gap.max(axis=1)  # over rows (padding rows are all -inf)
            visited = (tm > -np.inf).any(axis=1)
            keep = (np.arange(nkt)[None] == 0) | ~(g < thr)
            out[b, h] = np.where(visited, keep.astype(np.uint8), 2)
    return out


def pin_closed_form_mask(orc):
    rng = np.random.default_rng(4)
    for (Hq, Hkv, Nq, Nk, d, br, bc, causal) in [
        (2, 1, 96, 96, 8, 16, 8, True), (2, 2, 40, 77, 4, 8, 5, True), (3, 3, 31, 50, 8, 6, 4, False),
    ]:
        q, k, v = _rand_case(rng, 1, Hq, Hkv, Nq, Nk, d, d, plant=5.0)
        for lam in (0.0, 1e-4, 1e-2, 0.2, 1.0):
            r = orc.prefill(q, k, v, lam, causal, br, bc)
            cf = _prefix_max_closed_form(q, k, lam, causal, br, bc, 1 / math.sqrt(d))
            assert (r.mask == cf).all(), (lam, causal)


def _brute(q, k, v, lam, causal, br, bc, scale, sel=None):
    """Pure-Python loops straight from the definition, no incremental state.

    The running max before tile j is recomputed from scratch as the max score
    over the tiles kept so far; the output is a plain softmax over kept keys.
    ``sel`` (optional [nQt][nKt] booleans) restricts attention to a block set:
    a pair is visible only inside a selected block, and a row that sees no key
    gets a zero output and lse -inf. Returns (mask, out, lse).
    """
    Nq, d = len(q), len(q[0])
    Nk = len(k)
    thr = -math.inf if lam == 0 else math.log(lam)
    nqt, nkt = -(-Nq // br), -(-Nk // bc)

    def score(r, c):
        return scale * sum(q[r][x] * k[c][x] for x in range(d))

    def vis(r, c):
        if sel is not None and not sel[r // br][c // bc]:
            return False
        return (not causal) or c <= r + Nk - Nq

    mask = [[2] * nkt for _ in range(nqt)]
    out = [[0.0] * len(v[0]) for _ in range(Nq)]
    lse = [-math.inf] * Nq
    for i in range(nqt):
        rows = range(i * br, min((i + 1) * br, Nq))
        kept = []
        for j in range(nkt):
            cols = range(j * bc, min((j + 1) * bc, Nk))
            if not any(vis(r, c) for r in rows for c in cols):
                continue
            gaps = []
            for r in rows:
                vals = [score(r, c) for c in cols if vis(r, c)]
                if not vals:
                    gaps.append(-math.inf)
                    continue
                prev = [score(r, c) for t in kept for c in range(t * bc, min((t + 1) * bc, Nk))
                        if vis(r, c)]
                gaps.append(math.inf if not prev else max(vals) - max(prev))
            g = max(gaps)
            if j == 0 or not (g < thr):
                kept.append(j)
                mask[i][j] = 1
            else:
                mask[i][j] = 0
        for r in rows:
            cs = [c for t in kept for c in range(t * bc, min((t + 1) * bc, Nk)) if vis(r, c)]
            if not cs:
                continue
            mx = max(score(r, c) for c in cs)
            w = [math.exp(score(r, c) - mx) for c in cs]
            den = sum(w)
            lse[r] = mx + math.log(den)
            for x in range(len(v[0])):
                out[r][x] = sum(wi * v[c][x] for wi, c in zip(w, cs)) / den
    return mask, out, lse


def pin_brute_force(orc):
    rng = np.random.default_rng(5)
    for trial in range(24):
        Nq = int(rng.integers(1, 13))
        Nk = int(rng.integers(Nq, 17))
        d = int(rng.choice([1, 2, 4]))
        br = int(rng.choice([1, 2, 4]))
        bc = int(rng.choice([1, 2, 4]))
        causal = bool(rng.integers(0, 2))
        lam = float(rng.choice([0.0, 1e-3, 0.05, 0.3, 1.0]))
        q, k, v = _rand_case(rng, 1, 1, 1, Nq, Nk, d, 2, plant=float(rng.choice([0.0, 3.0])))
        sc = 1.0 / math.sqrt(d)
        r = orc.prefill(q, k, v, lam, causal, br, bc)
        bm, bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), lam, causal, br,
                            bc, sc)
        assert r.mask[0, 0].tolist() == bm, trial
        assert np.abs(r.out[0, 0] - np.array(bo)).max() < 1e-12, trial
        assert np.abs(r.lse[0, 0] - np.array(bl)).max() < 1e-12, trial


def pin_decode_sdpa(orc):
    """Decode at lambda 0 (plain GQA and MLA latent layout) equals softmax attention."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, Nk, d = 2, 8, 2, 150, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    r = orc.decode(q, k, v, 0.0, 64)
    G = Hq // Hkv
    ref = _sdpa(q[:, :, None], np.repeat(k, G, 1), np.repeat(v, G, 1), False, 1 / math.sqrt(d))
    assert np.abs(r.out - ref[:, :, 0]).max() < 1e-12
    # MLA: one latent head, V = first dv columns of K
    km = rng.standard_normal((B, 1, Nk, 24))
    qm = rng.standard_normal((B, 4, 24))
    rm = orc.decode(qm, km, None, 0.0, 64, dv=16)
    refm = _sdpa(qm[:, :, None], np.repeat(km, 4, 1), np.repeat(km[..., :16], 4, 1), False,
                 1 / math.sqrt(24))
    assert np.abs(rm.out - refm[:, :, 0]).max() < 1e-12


def _random_block_set(rng, B, Hq, nqt, nkt, density):
    """Random block set with the cases that matter forced in: tile 0 left out of
    some query tiles, and one query tile with an empty set."""
    sel = rng.random((B, Hq, nqt, nkt)) < density
    sel[..., 0, 0] = False
    if nqt > 1:
        sel[0, 0, 1] = False
    return sel.astype(np.uint8)


def _block_pairs(sel_row, causal, br, bc, Nq, Nk):
    """[Nq, Nk] booleans: causal visibility and block-set membership, from scratch."""
    r = np.arange(Nq)[:, None]
    c = np.arange(Nk)[None, :]
    ok = np.asarray(sel_row, dtype=bool)[r // br, c // bc]
    if causal:
        ok = ok & (c <= r + Nk - Nq)
    return ok


def pin_block_sparse_sdpa(orc):
    """lambda = 0 inside a block set: softmax attention over the set's keys
    (torch float64 with the block mask), zero rows and lse -inf where a row
    sees no key, and every block outside the set reported not visited."""
    rng = np.random.default_rng(12)
    for (B, Hq, Hkv, Nq, Nk, d, br, bc, causal) in [
        (1, 2, 1, 40, 70, 8, 8, 8, True), (2, 2, 2, 33, 50, 4, 5, 7, False),
        (1, 3, 1, 20, 20, 4, 4, 4, True),
    ]:
        q, k, v = _rand_case(rng, B, Hq, Hkv, Nq, Nk, d, d, plant=4.0)
        nqt, nkt = -(-Nq // br), -(-Nk // bc)
        sel = _random_block_set(rng, B, Hq, nqt, nkt, 0.5)
        sc = 1.0 / math.sqrt(d)
        r = orc.prefill_masked(q, k, v, sel, 0.0, causal, br, bc)
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                ok = _block_pairs(sel[b, h], causal, br, bc, Nq, Nk)
                seen = ok.any(axis=1)
                assert (r.out[b, h][~seen] == 0).all() and (r.lse[b, h][~seen] == -np.inf).all()
                ref = _sdpa(q[b, h][seen][None], k[b, h // G][None], v[b, h // G][None], False, sc,
                            attn_mask=ok[seen][None])[0]
                assert np.abs(r.out[b, h][seen] - ref).max() < 1e-12
                s = sc * q[b, h][seen] @ k[b, h // G].T
                s = np.where(ok[seen], s, -np.inf)
                mx = s.max(axis=1)
                lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
                assert np.abs(r.lse[b, h][seen] - lse).max() < 1e-12
                # visited = in the set and with at least one causally visible pair
                for i in range(nqt):
                    for j in range(nkt):
                        blk = ok[i * br:(i + 1) * br, j * bc:(j + 1) * bc]
                        assert (r.mask[b, h, i, j] == 2) == (not blk.any())
        assert (r.mask == 1).sum() == (r.mask != 2).sum(), "lambda 0 drops nothing"
        assert (r.stats[..., 0] == (r.mask != 2).sum(axis=(2, 3))).all()


def pin_block_sparse_kept(orc):
    """lambda > 0 inside a block set: the output is softmax attention over the
    set's blocks that the returned mask keeps, and the first tile of the set
    that a query tile visits is kept."""
    rng = np.random.default_rng(13)
    n_dropped = 0
    for (B, Hq, Hkv, Nq, Nk, d, br, bc, causal, lam) in [
        (1, 2, 1, 64, 96, 8, 8, 4, True, 1e-2), (1, 2, 2, 30, 80, 8, 6, 5, False, 1e-1),
    ]:
        q, k, v = _rand_case(rng, B, Hq, Hkv, Nq, Nk, d, d, plant=6.0)
        nqt, nkt = -(-Nq // br), -(-Nk // bc)
        sel = _random_block_set(rng, B, Hq, nqt, nkt, 0.7)
        sc = 1.0 / math.sqrt(d)
        r = orc.prefill_masked(q, k, v, sel, lam, causal, br, bc)
        n_dropped += int((r.mask == 0).sum())
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                assert (r.mask[b, h][sel[b, h] == 0] == 2).all()
                for i in range(nqt):
                    vis_t = np.nonzero(r.mask[b, h, i] != 2)[0]
                    if len(vis_t):
                        assert r.mask[b, h, i, vis_t[0]] == 1
                keep = orc.expand_tile_mask(r.mask[b, h], br, bc, Nq, Nk)
                ok = _block_pairs(sel[b, h], causal, br, bc, Nq, Nk) & keep
                seen = ok.any(axis=1)
                ref = _sdpa(q[b, h][seen][None], k[b, h // G][None], v[b, h // G][None], False, sc,
                            attn_mask=ok[seen][None])[0]
                assert np.abs(r.out[b, h][seen] - ref).max() < 1e-12
    assert n_dropped > 0, "fixture must exercise dropped tiles"


def pin_block_sparse_full_set(orc):
    """A block set that holds every block gives the plain skip-softmax prefill."""
    rng = np.random.default_rng(14)
    q, k, v = _rand_case(rng, 1, 2, 1, 45, 60, 8, 8, plant=6.0)
    sel = np.ones((1, 1, 6, 8), dtype=np.uint8)  # broadcast over heads
    for lam in (0.0, 1e-2):
        rp = orc.prefill(q, k, v, lam, True, 8, 8)
        rm = orc.prefill_masked(q, k, v, sel, lam, True, 8, 8)
        assert np.array_equal(rp.mask, rm.mask)
        assert np.abs(rp.out - rm.out).max() == 0 and np.abs(rp.lse - rm.lse).max() == 0


def pin_block_sparse_brute(orc):
    rng = np.random.default_rng(15)
    for trial in range(24):
        Nq = int(rng.integers(1, 11))
        Nk = int(rng.integers(Nq, 15))
        d = int(rng.choice([1, 2, 4]))
        br = int(rng.choice([1, 2, 3]))
        bc = int(rng.choice([1, 2, 4]))
        causal = bool(rng.integers(0, 2))
        lam = float(rng.choice([0.0, 1e-3, 0.05, 0.3, 1.0]))
        q, k, v = _rand_case(rng, 1, 1, 1, Nq, Nk, d, 2, plant=float(rng.choice([0.0, 3.0])))
        nqt, nkt = -(-Nq // br), -(-Nk // bc)
        sel = (rng.random((nqt, nkt)) < 0.6).astype(np.uint8)
        sc = 1.0 / math.sqrt(d)
        r = orc.prefill_masked(q, k, v, sel, lam, causal, br, bc)
        bm, bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), lam, causal, br,
                            bc, sc, sel=sel.tolist())
        assert r.mask[0, 0].tolist() == bm, trial
        assert np.abs(r.out[0, 0] - np.array(bo)).max() < 1e-12, trial
        assert np.array_equal(r.lse[0, 0] == -np.inf, np.array(bl) == -np.inf), trial
        fin = np.isfinite(np.array(bl))
        assert np.abs(r.lse[0, 0][fin] - np.array(bl)[fin]).max(initial=0) < 1e-12, trial
        assert r.stats[0, 0].tolist() == [int((r.mask[0, 0] != 2).sum()), int((r.mask[0, 0] == 1).sum())]


def _allowed(mask_row, causal, br, bc, Nq, Nk):
    """[Nq, Nk] booleans from a tile mask row (1 = kept) and causality, from scratch."""
    r = np.arange(Nq)[:, None]
    c = np.arange(Nk)[None, :]
    ok = (np.asarray(mask_row) == 1)[r // br, c // bc]
    if causal:
        ok = ok & (c <= r + Nk - Nq)
    return ok


def _bwd_case(rng, orc, B, Hq, Hkv, Nq, Nk, d, br, bc, causal, lam, empty_rows=False):
    q, k, v = _rand_case(rng, B, Hq, Hkv, Nq, Nk, d, d, plant=5.0)
    dout = rng.standard_normal((B, Hq, Nq, d))
    mask = orc.prefill(q, k, v, lam, causal, br, bc).mask.copy()
    if empty_rows:  # a block-sparse forward whose first query tile saw nothing
        mask[:, :, 0, :] = np.where(mask[:, :, 0, :] == 2, 2, 0)
    return q, k, v, dout, mask


def pin_backward_autograd(orc):
    """Gradients equal torch autograd (CPU, float64) of softmax attention over the
    allowed elements, the loss being sum(dout * out)."""
    rng = np.random.default_rng(16)
    n_dropped = 0
    for (B, Hq, Hkv, Nq, Nk, d, br, bc, causal, lam, empty) in [
        (1, 4, 2, 40, 70, 8, 8, 8, True, 1e-2, False),
        (2, 2, 1, 33, 50, 4, 5, 7, False, 1e-1, False),
        (1, 2, 2, 24, 24, 4, 8, 4, True, 0.0, True),
    ]:
        q, k, v, dout, mask = _bwd_case(rng, orc, B, Hq, Hkv, Nq, Nk, d, br, bc, causal, lam, empty)
        n_dropped += int((mask == 0).sum())
        sc = 1.0 / math.sqrt(d)
        dq, dk, dv = orc.prefill_backward(q, k, v, dout, mask, causal, br, bc)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        loss = torch.zeros((), dtype=torch.float64)
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                ok = _allowed(mask[b, h], causal, br, bc, Nq, Nk)
                rows = ok.any(axis=1)
                okt = torch.from_numpy(ok[rows])
                s_ = sc * tq[b, h][torch.from_numpy(rows)] @ tk[b, h // G].T
                p_ = torch.softmax(s_.masked_fill(~okt, -math.inf), dim=-1)
                o_ = p_ @ tv[b, h // G]
                loss = loss + (o_ * torch.from_numpy(dout[b, h][rows])).sum()
        loss.backward()
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.abs(got - ref.numpy()).max() < 1e-12
        if empty:
            assert (dq[:, :, :br] == 0).all()
    assert n_dropped > 0, "fixture must exercise dropped tiles"


def pin_backward_finite_difference(orc):
    """Central differences of sum(dout * out) with the mask held fixed; the
    forward here is a plain loop over the allowed keys."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, Nq, Nk, d, br, bc = 1, 2, 1, 5, 7, 3, 2, 3
    q, k, v, dout, mask = _bwd_case(rng, orc, B, Hq, Hkv, Nq, Nk, d, br, bc, True, 0.3)
    sc = 1.0 / math.sqrt(d)

    def loss(q_, k_, v_):
        total = 0.0
        for h in range(Hq):
            ok = _allowed(mask[0, h], True, br, bc, Nq, Nk)
            for r in range(Nq):
                cs = [c for c in range(Nk) if ok[r, c]]
                if not cs:
                    continue
                sco = [sc * float(q_[0, h, r] @ k_[0, 0, c]) for c in cs]
                mx = max(sco)
                w = [math.exp(x - mx) for x in sco]
                for x in range(d):
                    o = sum(wi * v_[0, 0, c, x] for wi, c in zip(w, cs)) / sum(w)
                    total += dout[0, h, r, x] * o
        return total

    dq, dk, dv = orc.prefill_backward(q, k, v, dout, mask, True, br, bc)
    hstep = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + hstep
            lp = loss(q, k, v)
            arr[idx] = keep - hstep
            lm = loss(q, k, v)
            arr[idx] = keep
            assert abs((lp - lm) / (2 * hstep) - grad[idx]) < 1e-6, idx


def pin_mxfp4_golden(orc):
    """Hand-derived MXFP4 blocks (tests/golden/mxfp4_blocks.json)."""
    for blk in _load("mxfp4_blocks.json")["blocks"]:
        codes, scales = orc.mx_quantize_fp4(np.array([blk["values"]]))
        assert codes[0].tolist() == blk["codes"], blk["derivation"]
        assert int(scales[0, 0]) == blk["scale"], blk["derivation"]


def _mx_brute(x):
    """One MXFP4 block by exhaustive search: the shared exponent found by
    stepping powers of two, each element the nearest of the 8 magnitudes times
    2^shared (ties to the even code), sign copied."""
    amax = max(abs(v) for v in x)
    if amax == 0:
        e = -127
    else:
        e = 0
        while 2.0 ** (e + 1) <= amax:
            e += 1
        while 2.0 ** e > amax:
            e -= 1
        e = min(max(e - 2, -127), 127)
    X = 2.0 ** e
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = []
    for v in x:
        dist = [abs(abs(v) - m * X) for m in mags]
        best = min(dist)
        cands = [c for c in range(8) if dist[c] == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        codes.append(c | (8 if math.copysign(1.0, v) < 0 else 0))
    return codes, e + 127


def pin_mxfp4_brute_force(orc):
    """Random blocks over many binades, with planted exact ties, against the
    exhaustive search; the dequantized values lie within half a spacing."""
    rng = np.random.default_rng(21)
    grid_mid = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0]
    for trial in range(300):
        e = int(rng.integers(-140, 120))
        x = rng.standard_normal(32) * 2.0 ** e
        if trial % 3 == 0:   # exact midpoints of the grid at the block's scale
            amax_e = int(rng.integers(-20, 20))
            x = np.array([rng.choice(grid_mid) * rng.choice([-1, 1]) for _ in range(32)]) * 2.0 ** amax_e
            x[0] = 4.0 * 2.0 ** amax_e
        if trial % 7 == 0:
            x[rng.integers(0, 32, 5)] = 0.0
        codes, scales = orc.mx_quantize_fp4(x[None])
        bc, bs = _mx_brute(x.tolist())
        assert codes[0].tolist() == bc, trial
        assert int(scales[0, 0]) == bs, trial
    # a row of several blocks quantizes block by block
    x = rng.standard_normal((3, 128)) * np.repeat(2.0 ** rng.integers(-8, 8, (3, 4)), 32, axis=1)
    codes, scales = orc.mx_quantize_fp4(x)
    for r in range(3):
        for blk in range(4):
            bc, bs = _mx_brute(x[r, 32 * blk:32 * blk + 32].tolist())
            assert codes[r, 32 * blk:32 * blk + 32].tolist() == bc
            assert int(scales[r, blk]) == bs
    deq = orc.mx_dequantize_fp4(codes, scales)
    X = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(x) / X   # in [0, 8): half the E2M1 spacing, or the clamp above 6
    half = np.select([a >= 6, a >= 4, a >= 2], [a - 6, 1.0, 0.5], 0.25)
    assert (np.abs(deq - x) <= half * X * (1 + 1e-12)).all()


def _on_grid(rng, shape):
    """Values that MXFP4 represents exactly: each block of 32 holds a magnitude
    4 or 6 times its power of two, so the block's shared exponent is that power."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = rng.choice(mags, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    blk = x.reshape(*shape[:-1], shape[-1] // 32, 32)
    blk[..., 0] = rng.choice([4.0, -6.0], size=blk.shape[:-1])
    pw = 2.0 ** rng.integers(-3, 2, size=blk.shape[:-1])
    return (blk * pw[..., None]).reshape(shape)


def pin_twopass_on_grid(orc):
    """When q and k are exactly MXFP4-representable, the pre-pass sees the exact
    scores, so the two-pass result is the one-pass result."""
    rng = np.random.default_rng(22)
    for (Hq, Hkv, Nq, Nk, br, bc, causal) in [(2, 1, 40, 70, 8, 8, True), (2, 2, 33, 50, 5, 7, False)]:
        q = _on_grid(rng, (1, Hq, Nq, 32))
        k = _on_grid(rng, (1, Hkv, Nk, 32))
        k[:, :, ::9] = np.abs(k[:, :, ::9])  # some keys align with positive queries
        q = np.abs(q) * np.where(rng.random(q.shape) < 0.8, 1.0, -1.0)
        v = rng.standard_normal((1, Hkv, Nk, 8))
        assert np.array_equal(orc.mx_dequantize_fp4(*orc.mx_quantize_fp4(q)), q)
        n_dropped = 0
        for lam in (0.0, 1e-2, 0.3):
            r1 = orc.prefill(q, k, v, lam, causal, br, bc)
            r2 = orc.prefill_twopass(q, k, v, lam, causal, br, bc)
            assert np.array_equal(r1.mask, r2.mask)
            assert np.array_equal(r1.stats, r2.stats)
            assert np.abs(r1.out - r2.out).max() < 1e-12
            assert np.abs(r1.lse - r2.lse).max() < 1e-12
            n_dropped += int((r1.mask == 0).sum())
        assert n_dropped > 0, "fixture must exercise dropped tiles"


def pin_twopass_map_and_output(orc):
    """The map is the closed-form prefix-max rule on the dequantized scores
    (differing from the exact scores' map on this fixture), and the output is
    softmax over the kept tiles (torch SDPA, float64, element mask)."""
    rng = np.random.default_rng(23)
    n_diff = n_dropped = 0
    for (Hq, Hkv, Nq, Nk, br, bc, causal) in [(2, 1, 64, 96, 16, 8, True), (1, 1, 30, 45, 7, 5, False)]:
        q, k, v = _rand_case(rng, 1, Hq, Hkv, Nq, Nk, 64, 16, plant=4.0)
        qd = orc.mx_dequantize_fp4(*orc.mx_quantize_fp4(q))
        kd = orc.mx_dequantize_fp4(*orc.mx_quantize_fp4(k))
        sc = 1 / math.sqrt(64)
        for lam in (1e-2, 0.1, 0.3):
            r = orc.prefill_twopass(q, k, v, lam, causal, br, bc)
            assert (r.mask == _prefix_max_closed_form(qd, kd, lam, causal, br, bc, sc)).all()
            exact = _prefix_max_closed_form(q, k, lam, causal, br, bc, sc)
            n_diff += int((exact != r.mask).sum())
            n_dropped += int((r.mask == 0).sum())
            G = Hq // Hkv
            for h in range(Hq):
                keep = orc.expand_tile_mask(r.mask[0, h], br, bc, Nq, Nk)
                allowed = keep & orc.visible(Nq, Nk, causal)
                ref = _sdpa(q[0, h][None], k[0, h // G][None], v[0, h // G][None], False, sc,
                            np.where(allowed, 0.0, -np.inf)[None])[0]
                assert np.abs(r.out[0, h] - ref).max() < 1e-12
            assert (r.stats[..., 1] == (r.mask == 1).sum(axis=(2, 3))).all()
    assert n_diff > 0, "fixture must make the 4-bit map differ from the exact one"
    assert n_dropped > 0


PINS = [pin_hand_example, pin_row_aggregation, pin_tie, pin_causal_visibility,
        pin_lambda0_sdpa, pin_bottom_right_causal, pin_masked_sdpa, pin_masked_dense_attention,
        pin_closed_form_mask,
        pin_brute_force, pin_decode_sdpa, pin_block_sparse_sdpa, pin_block_sparse_kept,
        pin_block_sparse_full_set, pin_block_sparse_brute, pin_backward_autograd,
        pin_backward_finite_difference, pin_mxfp4_golden, pin_mxfp4_brute_force,
        pin_twopass_on_grid, pin_twopass_map_and_output]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)


# --------------------------------------------------------------------------- invariants

def test_threshold_domain():
    assert oracle.threshold(0.0) == -math.inf
    assert oracle.threshold(1.0) == 0.0
    assert abs(oracle.threshold(1e-3) - math.log(1e-3)) < 1e-15
    for bad in (-1e-9, 1.0000001, float("nan"), 2.0):
        with pytest.raises(ValueError):
            oracle.threshold(bad)


def test_prefix_max_invariant_and_nesting():
    """For lambda <= 1 a dropped tile can never raise the running max, so the
    running max on entry to tile j is the plain prefix max; kept sets are nested
    in lambda and tile 0 is always kept."""
    rng = np.random.default_rng(7)
    q, k, v = _rand_case(rng, 1, 2, 1, 64, 200, 8, 8, plant=6.0)
    lams = [0.0, 1e-6, 1e-4, 1e-3, 1e-2, 0.1, 1.0]
    prev_kept = None
    fracs = []
    for lam in lams:
        kept_all = []
        for h in range(2):
            for i in range(4):
                t = oracle.prefill_tile(q, k, v, 0, h, i, lam, True, 16, 8)
                vis_t = t.mask != 2
                pm = np.maximum.accumulate(t.tile_max, axis=0)
                prev = np.vstack([np.full((1, pm.shape[1]), -np.inf), pm[:-1]])
                assert np.array_equal(t.m_before[vis_t], prev[vis_t])
                assert t.mask[0] == 1
                kept_all.append(t.mask == 1)
        kept = np.concatenate(kept_all)
        if prev_kept is not None:
            assert not (kept & ~prev_kept).any(), "kept sets must be nested in lambda"
        prev_kept = kept
        fracs.append(1 - kept.sum() / len(kept))
    assert all(a <= b for a, b in zip(fracs, fracs[1:]))
    assert fracs[-1] > 0.2


def test_stats_consistency():
    rng = np.random.default_rng(8)
    q, k, v = _rand_case(rng, 2, 4, 2, 50, 50, 8, 8, plant=6.0)
    r = oracle.prefill(q, k, v, 1e-2, True, 8, 8)
    assert (r.stats[..., 0] == (r.mask != 2).sum(axis=(2, 3))).all()
    assert (r.stats[..., 1] == (r.mask == 1).sum(axis=(2, 3))).all()
    qd = rng.standard_normal((2, 4, 8)) + 3
    rd = oracle.decode(qd, k, v, 1e-2, 8)
    G = 2
    for b in range(2):
        for h in range(4):
            grp = rd.mask[b, (h // G) * G:(h // G + 1) * G]
            assert rd.stats[b, h, 2] == (grp == 1).any(axis=0).sum()


def test_decode_equals_prefill_with_one_row():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, Nk, d = 1, 4, 2, 70, 8
    q = rng.standard_normal((B, Hq, d)) + 2.0
    k, v = rng.standard_normal((B, Hkv, Nk, d)), rng.standard_normal((B, Hkv, Nk, d))
    k[:, :, ::9] += 3.0
    for lam in (0.0, 1e-2, 0.5):
        rd = oracle.decode(q, k, v, lam, 8)
        rp = oracle.prefill(q[:, :, None], k, v, lam, False, 1, 8)
        assert np.array_equal(rd.mask, rp.mask[:, :, 0])
        assert np.abs(rd.out - rp.out[:, :, 0]).max() == 0


def test_generator_workload_skips_only_with_gain():
    """The workloads as specified plant boosts too weak to cross ln(lambda); the
    supplementary gain makes dropped tiles appear (recorded in the design notes)."""
    w = synth.small_workload("prefill", Hq=1, Hkv=1, Nq=256, Nk=1024, d=64, dtype="fp32",
                             br=64, bc=64, seed=11, window=0)
    for gain, expect_skip in ((1.0, False), (6.0, True)):
        inp = synth.make_inputs(w.with_gain(gain))
        q, k, v = (synth.to_float(x, w) for x in (inp.q, inp.k, inp.v))
        r = oracle.prefill(q, k, v, 1e-2, True, 64, 64)
        assert bool((r.mask == 0).any()) == expect_skip


# --------------------------------------------------------------------------- mutation tests

_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "blasst_oracle.py")).read()

MUTATIONS = {
    "any_row_instead_of_all_rows": ("g = g_r.max() if rows else -np.inf", "g = g_r.min() if rows else -np.inf"),
    "non_strict_threshold": ("keep = (j == 0) or not (g < thr)", "keep = (j == 0) or not (g <= thr)"),
    "dropped_rescale_of_l": ("l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    "dropped_rescale_of_o": ("o = alpha[:, None] * o + p @ v[c0:c1]", "o = o + p @ v[c0:c1]"),
    "gqa_modulo_mapping": ("kvh = hq // (Hq // hkv)\n    nk = k.shape[2]", "kvh = hq % hkv\n    nk = k.shape[2]"),
    "top_left_causal": ("return c <= r + (nk - nq)", "return c <= r"),
    "gap_sign_flipped": ("np.where(m == -np.inf, np.inf, mt - m)", "np.where(m == -np.inf, np.inf, m - mt)"),
    "missing_scale": ("s = scale * (q @ k.T)\n    s = np.where(vis", "s = (q @ k.T)\n    s = np.where(vis"),
    "running_max_not_updated": ("        m = m_new\n", "        m = np.maximum(m, 0 * m_new)\n"),
    "first_tile_not_forced": ("keep = (j == 0) or not (g < thr)", "keep = not (g < thr) and j >= 0"),
    "threshold_log10": ("math.log(lam)", "math.log10(lam)"),
    "block_set_ignored": ("vis = visible(nq, nk, causal, row0, len(q_rows)) & in_set[None, :]",
                          "vis = visible(nq, nk, causal, row0, len(q_rows))"),
    "block_set_wrong_query_tile": ("v[b, kvh], sel[b, hq, i], lam,", "v[b, kvh], sel[b, hq, 0], lam,"),
    "block_set_expanded_by_rows": ("np.repeat(np.asarray(sel_row) != 0, bc)[:nk]",
                                   "np.repeat(np.asarray(sel_row) != 0, len(q_rows))[:nk]"),
    "block_set_wrong_row_offset": ("causal, nq, r0, bc, scale)", "causal, nq, 0, bc, scale)"),
    "empty_rows_not_zeroed": ("np.where(seen[:, None], r.out, 0.0)", "r.out"),
    "bwd_dq_missing_scale": ("dq[b, hq] = scale * (ds @ k[b, kvh])", "dq[b, hq] = (ds @ k[b, kvh])"),
    "bwd_delta_dropped": ("ds = p * (dp - delta)", "ds = p * dp"),
    "bwd_dk_not_summed_over_group": ("dk[b, kvh] += scale * (ds.T @ q[b, hq])",
                                     "dk[b, kvh] = scale * (ds.T @ q[b, hq])"),
    "bwd_mask_ignored": ("allowed = vis & expand_tile_mask(mask[b, hq], br, bc, nq, nk)", "allowed = vis"),
    "bwd_unnormalised_p": ("p = np.where(live, e / np.where(live, den, 1.0), 0.0)",
                           "p = np.where(live, e, 0.0)"),
    "bwd_dk_uses_dp": ("dk[b, kvh] += scale * (ds.T @ q[b, hq])", "dk[b, kvh] += scale * (dp.T @ q[b, hq])"),
    "mx_scale_exponent_off_by_one": ("ex - 1 - E2M1_EMAX, -E8M0_BIAS)", "ex - E2M1_EMAX, -E8M0_BIAS)"),
    "mx_round_half_up": ("np.rint(a / ulp) * ulp", "np.floor(a / ulp + 0.5) * ulp"),
    "mx_no_clamp": ("np.minimum(np.rint(a / ulp) * ulp, E2M1_MAX)", "np.rint(a / ulp) * ulp"),
    "mx_sign_dropped": ("code |= (np.signbit(blk).astype(np.uint8) << 3)", "code |= 0"),
    "twopass_decides_on_exact_scores": ("pre = prefill_tile(qd, kd, v,", "pre = prefill_tile(q, k, v,"),
    "tile_expansion_transposed": ("el = np.repeat(np.repeat(kept, br, axis=0), bc, axis=1)",
                                  "el = np.repeat(np.repeat(kept, bc, axis=0), br, axis=1)"),
    "restricted_softmax_keep_ignored": ("allowed = keep & visible(q.shape[0], k.shape[0], causal)",
                                        "allowed = visible(q.shape[0], k.shape[0], causal)"),
    "restricted_softmax_lse_without_max": ("(mx + np.log(den))[:, 0]", "(np.log(den))[:, 0]"),
    "twopass_pass2_over_visible": ("pre.mask == MASK_KEPT, 0.0,", "pre.mask != MASK_NOT_VISITED, 0.0,"),
}


def _mutant(old, new):
    assert old in _SRC, f"mutation anchor missing: {old!r}"
    src = _SRC.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    sys.modules["oracle_mutant"] = mod
    exec(compile(src, "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTATIONS[name]
    mut = _mutant(old, new)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except Exception:  # noqa: BLE001 - any failure means the pin caught it
            caught.append(pin.__name__)
    # "first tile not forced" is benign: tile 0 always has gap +inf, so the
    # convention already keeps it. Every other mutation must be caught.
    if name == "first_tile_not_forced":
        assert caught == []
    else:
        assert caught, f"no pin caught mutation {name}"


def test_backward_magnitudes_bound_the_gradients():
    """The error-scale tensors the backward parity bar uses are sums of absolute
    products, so they bound the gradients themselves (triangle inequality)."""
    rng = np.random.default_rng(18)
    q, k, v, dout, mask = _bwd_case(rng, oracle, 1, 4, 2, 40, 70, 8, 8, 8, True, 1e-2)
    dq, dk, dv, mq, mk, mv = oracle.prefill_backward(q, k, v, dout, mask, True, 8, 8, magnitudes=True)
    plain = oracle.prefill_backward(q, k, v, dout, mask, True, 8, 8)
    for g, m, p in ((dq, mq, plain[0]), (dk, mk, plain[1]), (dv, mv, plain[2])):
        assert np.array_equal(g, p)
        assert (np.abs(g) <= m * (1 + 1e-12) + 1e-300).all()
        assert (m > 0).any()


def test_backward_stored_output_only_changes_delta():
    """Passing the exact output as the stored one changes nothing; a perturbed
    stored output moves dq and dk (through delta) but not dv."""
    rng = np.random.default_rng(19)
    q, k, v, dout, mask = _bwd_case(rng, oracle, 1, 2, 1, 24, 40, 4, 8, 8, True, 1e-2)
    ref = oracle.prefill_backward(q, k, v, dout, mask, True, 8, 8)
    o = oracle.masked_dense_attention  # exact output per head
    out = np.zeros(dout.shape)
    for h in range(2):
        keep = _allowed(mask[0, h], True, 8, 8, 24, 40)
        out[0, h] = o(q[0, h], k[0, 0], v[0, 0], keep, False)[0]
    same = oracle.prefill_backward(q, k, v, dout, mask, True, 8, 8, out=out)
    for a_, b_ in zip(ref, same):
        assert np.abs(a_ - b_).max() < 1e-12
    moved = oracle.prefill_backward(q, k, v, dout, mask, True, 8, 8, out=out * 1.01)
    assert np.abs(moved[0] - ref[0]).max() > 1e-6 and np.abs(moved[1] - ref[1]).max() > 1e-6
    assert np.abs(moved[2] - ref[2]).max() == 0
