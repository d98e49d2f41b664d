"""Shared parity helpers for the GPU tests: GPU result vs the CPU oracle.

Bar (element by element, on the same seeded inputs):
  * the kept-tile mask matches exactly, except key tiles whose oracle max-gap
    lies within BAND of ln(lambda); those flips are logged, and the rows of a
    query tile touched by a flip are compared with softmax attention restricted
    to the GPU's own mask (so the output check stays exact in meaning);
  * arithmetic of bf16-input kernels (float32 outputs): max-abs <= 1e-2 and
    mean-abs <= 1e-3 against the float64 oracle; fp32 kernels: 1e-5;
  * bf16 outputs: the kernel rounds its fp32 result to bf16 (nearest even),
    so it is compared with the oracle's output rounded the same way: max-abs
    <= 1e-2 plus half a bf16 spacing at each of the two values (one ulp inside
    a binade: two values within 1e-2 can round to neighbours one ulp apart),
    mean-abs <= 1e-3 unchanged;
  * strict=True (the workloads as specified, gain 1): bf16 outputs against the
    unrounded float64 oracle with the plain 1e-2 / 1e-3 bar, no ulp allowance;
  * lse: 2e-3 (bf16 inputs) / 1e-5 (fp32) absolute; stats: exact.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from block_sparse_long_skip_amd import synth

BAND = 1e-3
TOL = {"bf16": dict(max_abs=1e-2, mean_abs=1e-3, lse=2e-3),
       "fp32": dict(max_abs=1e-5, mean_abs=1e-5, lse=1e-5)}
BF16_BITS = 8  # significand bits of bfloat16, the implicit one included


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), as float64. Written from
    the format: keep 8 significant bits of the binary significand. np.frexp gives
    x = m 2^e with 0.5 <= |m| < 1, so m 2^8 is an integer after rounding and
    np.rint rounds half to even. (Subnormal bf16 values do not arise here.)"""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, BF16_BITS)), e - BF16_BITS)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (x already a bf16 value; 0 at 0)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - BF16_BITS))


def to_device(x: np.ndarray, w: synth.Workload) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if w.dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def from_device(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@dataclass
class Tally:
    """Aggregate of one parity check (every compared element)."""
    got: list = field(default_factory=list)
    ref: list = field(default_factory=list)
    lse_err: list = field(default_factory=list)
    tiles: int = 0
    flips: int = 0
    band: int = 0
    notes: list = field(default_factory=list)

    def add(self, got: np.ndarray, ref: np.ndarray, lse_err: np.ndarray):
        """got: GPU output values (float64); ref: the oracle's float64 values."""
        # lse -inf on both sides (a row that sees no key) is a match
        lse_err = np.where(np.isnan(lse_err), np.inf, lse_err)
        self.got.append(np.asarray(got, np.float64).ravel())
        self.ref.append(np.asarray(ref, np.float64).ravel())
        self.lse_err.append(np.abs(lse_err).ravel())

    def check(self, dtype: str, label: str = "", out_bf16: bool = False, strict: bool = False):
        """dtype: input type ("bf16"/"fp32"); out_bf16: outputs were stored as
        bf16; strict: no rounding of the reference for bf16 outputs."""
        tol = TOL[dtype]
        g = np.concatenate(self.got) if self.got else np.zeros(1)
        r = np.concatenate(self.ref) if self.ref else np.zeros(1)
        le = np.concatenate(self.lse_err) if self.lse_err else np.zeros(1)
        rounded = out_bf16 and not strict
        if rounded:
            r = round_bf16(r)
        e = np.abs(g - r)
        # |rne(g') - rne(r)| <= |g - g'| + |g' - r| + |r - rne(r)| for the kernel's
        # fp32 value g' behind its bf16 output g: half a spacing at each end
        bound = tol["max_abs"] + (0.5 * (ulp_bf16(r) + ulp_bf16(g)) if rounded else 0.0)
        msg = (f"{label}: max_abs={e.max():.3e} mean_abs={e.mean():.3e} lse_max={le.max():.3e} "
               f"excess_over_bound={np.max(e - bound):.3e} "
               f"tiles={self.tiles} flips={self.flips} near_threshold={self.band} "
               f"out={'bf16' if out_bf16 else 'fp32'}"
               f"{' vs rne-bf16(oracle)' if rounded else ''}")
        print(msg, *self.notes[:10], sep="\n  ")
        assert np.isfinite(e).all(), msg
        assert (e <= bound).all(), msg
        assert e.mean() <= tol["mean_abs"], msg
        assert le.max() <= tol["lse"], msg
        return msg


def _thr(lam: float) -> float:
    return -math.inf if lam == 0 else math.log(lam)


def check_mask_row(gpu_row: np.ndarray, orc_row: np.ndarray, gap_row: np.ndarray, lam: float,
                   tally: Tally, where: str) -> np.ndarray:
    """Exact mask match outside the near-threshold band. Returns the flip positions."""
    thr = _thr(lam)
    visited = orc_row != oracle.MASK_NOT_VISITED
    assert np.array_equal(gpu_row == oracle.MASK_NOT_VISITED, ~visited), f"{where}: visited set"
    assert set(np.unique(gpu_row)).issubset({0, 1, 2}), f"{where}: mask values"
    first = np.nonzero(visited)[0]
    if len(first):
        assert gpu_row[first[0]] == oracle.MASK_KEPT, f"{where}: first visited tile must be kept"
    near = visited & (np.abs(gap_row - thr) <= BAND) if math.isfinite(thr) else np.zeros_like(visited)
    tally.band += int(near.sum())
    flips = visited & (gpu_row != orc_row)
    bad = flips & ~near
    assert not bad.any(), (f"{where}: mask differs outside the band at tiles {np.nonzero(bad)[0][:8]}"
                           f" gaps {gap_row[bad][:8]} thr {thr}")
    tally.tiles += int(visited.sum())
    if flips.any():
        tally.flips += int(flips.sum())
        tally.notes.append(f"{where}: flipped tiles {np.nonzero(flips)[0].tolist()} "
                           f"gaps {gap_row[flips].tolist()} thr {thr}")
    return flips


def masked_reference(q_rows, k, v, keep_el, scale):
    """Softmax over the kept keys only, via the oracle's dense routine (visibility
    already folded into keep_el)."""
    return oracle.masked_dense_attention(q_rows, k, v, keep_el, False, scale)


def prefill_tile_parity(res, inp, w: synth.Workload, lam: float, b: int, h: int, i: int,
                        tally: Tally, qf=None, kf=None, vf=None, scale=None):
    """Compare one (b, h, query tile i) of a GPU prefill result with the oracle
    (softmax scale 1/sqrt(d) unless given)."""
    G = w.Hq // w.Hkv
    kvh = h // G
    r0, r1 = i * w.br, min((i + 1) * w.br, w.Nq)
    q = qf if qf is not None else synth.to_float(inp.q[b, h, r0:r1], w)
    k = kf if kf is not None else synth.to_float(inp.k[b, kvh], w)
    v = vf if vf is not None else synth.to_float(inp.v[b, kvh], w)
    scale = 1.0 / math.sqrt(w.d) if scale is None else scale
    vis = oracle.visible(w.Nq, w.Nk, w.causal, r0, r1 - r0)
    t = oracle.blasst_rows(q, k, v, lam, w.bc, vis, scale)
    gpu_mask = res.mask[b, h, i].cpu().numpy()
    flips = check_mask_row(gpu_mask, t.mask, t.gap, lam, tally, f"b{b} h{h} qtile{i}")
    ref_out, ref_lse = t.out, t.lse
    if flips.any():
        keep_el = oracle.expand_tile_mask(gpu_mask[None, :], r1 - r0, w.bc, r1 - r0, w.Nk) & vis
        ref_out, ref_lse = masked_reference(q, k, v, keep_el, scale)
    got = from_device(res.out[b, h, r0:r1])
    got_lse = res.lse[b, h, r0:r1].cpu().numpy().astype(np.float64)
    tally.add(got, ref_out, got_lse - ref_lse)
    return t


def lse_diff(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """got - ref, with 0 where both are -inf (NaN where only one is, which fails)."""
    both = (got == -np.inf) & (ref == -np.inf)
    with np.errstate(invalid="ignore"):
        d = got - ref
    d = np.where(both, 0.0, d)
    return np.where(np.isinf(d), np.nan, d)


def prefill_masked_tile_parity(res, inp, w: synth.Workload, lam: float, sel: np.ndarray, b: int,
                               h: int, i: int, tally: Tally, kf=None, vf=None):
    """Compare one (b, h, query tile i) of a GPU block-sparse prefill with the
    oracle's block_sparse_rows; sel is the block set [B, Hq, nQt, nKt]."""
    kvh = h // (w.Hq // w.Hkv)
    r0, r1 = i * w.br, min((i + 1) * w.br, w.Nq)
    q = synth.to_float(inp.q[b, h, r0:r1], w)
    k = kf if kf is not None else synth.to_float(inp.k[b, kvh], w)
    v = vf if vf is not None else synth.to_float(inp.v[b, kvh], w)
    scale = 1.0 / math.sqrt(w.d)
    t = oracle.block_sparse_rows(q, k, v, sel[b, h, i], lam, w.causal, w.Nq, r0, w.bc, scale)
    gpu_mask = res.mask[b, h, i].cpu().numpy()
    flips = check_mask_row(gpu_mask, t.mask, t.gap, lam, tally, f"b{b} h{h} qtile{i}")
    ref_out, ref_lse = t.out, t.lse
    if flips.any():
        # same routine on the GPU's own kept set: the set narrowed to its kept tiles
        kept = (gpu_mask == oracle.MASK_KEPT).astype(np.uint8)
        t2 = oracle.block_sparse_rows(q, k, v, kept, 0.0, w.causal, w.Nq, r0, w.bc, scale)
        ref_out, ref_lse = t2.out, t2.lse
    got = from_device(res.out[b, h, r0:r1])
    got_lse = res.lse[b, h, r0:r1].cpu().numpy().astype(np.float64)
    tally.add(got, ref_out, lse_diff(got_lse, ref_lse))
    return t


def mxfp4_values(x: np.ndarray) -> np.ndarray:
    """The oracle's MXFP4 round trip of float values (blocks of 32 along the last axis)."""
    return oracle.mx_dequantize_fp4(*oracle.mx_quantize_fp4(x))


def prefill_twopass_tile_parity(res, inp, w: synth.Workload, lam: float, b: int, h: int, i: int,
                                tally: Tally, kf=None, vf=None, kd=None):
    """Compare one (b, h, query tile i) of a GPU two-pass prefill with the oracle:
    the map against the skip rule on the MXFP4-dequantized q and k (whose gaps
    define the near-threshold band), the output against exact attention over the
    kept tiles (the GPU's own kept tiles where the map flipped inside the band).
    kd: the dequantized keys of the head, when the caller caches them."""
    kvh = h // (w.Hq // w.Hkv)
    r0, r1 = i * w.br, min((i + 1) * w.br, w.Nq)
    q = synth.to_float(inp.q[b, h, r0:r1], w)
    k = kf if kf is not None else synth.to_float(inp.k[b, kvh], w)
    v = vf if vf is not None else synth.to_float(inp.v[b, kvh], w)
    kd = kd if kd is not None else mxfp4_values(k)
    scale = 1.0 / math.sqrt(w.d)
    vis = oracle.visible(w.Nq, w.Nk, w.causal, r0, r1 - r0)
    pre = oracle.blasst_rows(mxfp4_values(q), kd, v, lam, w.bc, vis, scale)
    gpu_mask = res.mask[b, h, i].cpu().numpy()
    flips = check_mask_row(gpu_mask, pre.mask, pre.gap, lam, tally, f"b{b} h{h} qtile{i}")
    kept = gpu_mask if flips.any() else pre.mask
    t = oracle.block_sparse_rows(q, k, v, (kept == oracle.MASK_KEPT).astype(np.uint8), 0.0,
                                 w.causal, w.Nq, r0, w.bc, scale)
    got = from_device(res.out[b, h, r0:r1])
    got_lse = res.lse[b, h, r0:r1].cpu().numpy().astype(np.float64)
    tally.add(got, t.out, lse_diff(got_lse, t.lse))
    return pre


def decode_row_parity(res, q64, k64, v64, lam: float, bc: int, b: int, hq: int, tally: Tally,
                      scale=None):
    """Compare one (b, hq) decode row. q64 [d]; k64 [Nk,d]; v64 [Nk,dv] (float64);
    softmax scale 1/sqrt(d) unless given."""
    nk = k64.shape[0]
    scale = 1.0 / math.sqrt(q64.shape[0]) if scale is None else scale
    t = oracle.blasst_rows(q64[None], k64, v64, lam, bc, np.ones((1, nk), bool), scale)
    gpu_mask = res.mask[b, hq].cpu().numpy()
    flips = check_mask_row(gpu_mask, t.mask, t.gap, lam, tally, f"b{b} h{hq}")
    ref_out, ref_lse = t.out[0], t.lse[0]
    if flips.any():
        keep_el = oracle.expand_tile_mask(gpu_mask[None, :], 1, bc, 1, nk)
        o, l_ = masked_reference(q64[None], k64, v64, keep_el, scale)
        ref_out, ref_lse = o[0], l_[0]
    got = from_device(res.out[b, hq])
    tally.add(got, ref_out, np.array([float(res.lse[b, hq]) - ref_lse]))
    return t


def sample_qtiles(w: synth.Workload, heads, per_head: int, seed: int):
    """Query tiles {0, 1, middle, last} plus random ones, for each listed head."""
    nqt = synth.n_tiles(w.Nq, w.br)
    rng = np.random.default_rng(seed)
    out = []
    for h in heads:
        base = sorted({0, min(1, nqt - 1), nqt // 2, nqt - 1})
        extra = rng.choice(nqt, size=min(per_head, nqt), replace=False).tolist()
        out += [(h, i) for i in sorted(set(base + extra))]
    return out


def _decode_group_rows(job):
    """Oracle decode rows of one (batch, KV head) of a generated workload (run in
    a worker process: the slices are regenerated there from the seed)."""
    w, b, kvh, lam, scale = job
    u = synth.unit_direction(w)
    kf = synth.to_float(synth.k_slice(w, b, kvh, u), w)
    vf = kf[:, :w.dv] if w.v_is_k_slice else synth.to_float(synth.v_slice(w, b, kvh), w)
    rows = []
    for hq in range(kvh * w.G, (kvh + 1) * w.G):
        q = synth.to_float(synth.q_slice(w, b, hq, u), w).reshape(-1)
        t = oracle.blasst_rows(q[None], kf, vf, lam, w.bc, np.ones((1, w.Nk), bool), scale)
        rows.append((hq, t.out[0], t.lse[0], t.mask, t.gap))
    return b, kvh, rows


def oracle_decode_all(w: synth.Workload, lam: float, workers: int = 8, scale=None):
    """The oracle over every (batch, head) row of a decode workload, in worker
    processes (spawned: the GPU process is never forked). Returns out, lse,
    mask, gap arrays shaped like the GPU call's."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    scale = 1.0 / math.sqrt(w.d) if scale is None else scale
    nkt = synth.n_tiles(w.Nk, w.bc)
    out = np.zeros((w.B, w.Hq, w.dv))
    lse = np.zeros((w.B, w.Hq))
    mask = np.zeros((w.B, w.Hq, nkt), np.uint8)
    gap = np.zeros((w.B, w.Hq, nkt))
    jobs = [(w, b, kvh, lam, scale) for b in range(w.B) for kvh in range(w.Hkv)]
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        for b, kvh, rows in ex.map(_decode_group_rows, jobs):
            for hq, o, l_, m, g in rows:
                out[b, hq], lse[b, hq], mask[b, hq], gap[b, hq] = o, l_, m, g
    return out, lse, mask, gap
