"""Seeded synthetic attention inputs with planted structure.

This module only *makes inputs*. It holds none of the attention arithmetic, so
both the CPU oracle (via the tests) and the GPU path can use it without sharing
any of the method's code.

The structure planted here stands in for what the pages describe long-context
attention as attending to: attention sinks on the first tokens and a recent
local window (the CRISP write-up on rit.work, "Что сделали"), plus a sprinkle
of "needle" keys for retrieval (same page, "Что показали"). A shared unit
direction ``u`` in ``R^d`` is added to the planted keys (``+4g u`` for sinks and
needles, ``+2g u`` for the recent window) and to every query (``+g u``); ``g``
is the gain, 1 for the workloads as specified. V is never planted.

Randomness: every tensor slice has its own ``numpy`` PCG64 stream, keyed by
``SeedSequence([seed, tag, b, h])``. Any (batch, head) slice can therefore be
regenerated on its own (the oracle samples heads of the large workloads), and
slices can be drawn in parallel threads. Values are drawn as float32
N(0, 1). bf16 workloads are rounded to bfloat16 with round-to-nearest-even and
stored as raw ``uint16`` bit patterns, which is the exact storage format the
GPU reads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

# Stream tags for SeedSequence([seed, tag, ...]).
_TAG_U, _TAG_Q, _TAG_K, _TAG_V, _TAG_NEEDLE, _TAG_RATE = 0, 1, 2, 3, 4, 5

SINK_TOKENS = 4
SINK_BOOST = 4.0
NEEDLE_BOOST = 4.0
WINDOW_BOOST = 2.0
QUERY_BOOST = 1.0


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, tiling, threshold sweep and generator knobs."""

    name: str
    kind: str  # "prefill" | "decode" | "decode_mla"
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dv: int
    dtype: str  # "fp32" | "bf16"
    causal: bool
    br: int
    bc: int
    lambdas: tuple
    seed: int
    needle_rate: float = 0.02
    # per-KV-head needle rate drawn uniformly from this range when set
    needle_rate_range: Optional[tuple] = None
    window: int = 0
    gain: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def v_is_k_slice(self) -> bool:
        return self.kind == "decode_mla"

    def with_gain(self, g: float) -> "Workload":
        return replace(self, gain=float(g))

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads the method is measured on. Shapes follow the model layers
# the pages name (Llama-3.1-8B and Qwen2.5-7B attention layers for prefill, a
# DeepSeek-style MLA latent cache for decode).
WORKLOADS = {
    1: Workload("prefill_f32_n1024", "prefill", 1, 1, 1, 1024, 1024, 64, 64, "fp32",
                True, 64, 64, (0.0, 1e-3, 1e-2), 1000, needle_rate=0.02, window=0),
    2: Workload("prefill_llama8b_n32768", "prefill", 1, 32, 8, 32768, 32768, 128, 128,
                "bf16", True, 128, 64, (0.0, 1e-4, 1e-3, 1e-2), 2000,
                needle_rate=0.02, window=256),
    3: Workload("decode_gqa_b32_n65536", "decode", 32, 32, 8, 1, 65536, 128, 128, "bf16",
                False, 1, 64, (0.0, 1e-3, 1e-2), 3000, needle_rate=0.005, window=256),
    4: Workload("prefill_qwen7b_n131072", "prefill", 1, 28, 4, 131072, 131072, 128, 128,
                "bf16", True, 128, 64, (0.0, 1e-3), 4000, needle_rate_range=(0.001, 0.05),
                window=256),
    5: Workload("decode_mla_b16_n32768", "decode_mla", 16, 128, 1, 1, 32768, 576, 512,
                "bf16", False, 1, 64, (0.0, 1e-3, 1e-2), 5000, needle_rate=0.02,
                window=256),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def unit_direction(w: Workload) -> np.ndarray:
    u = _rng(w.seed, _TAG_U).standard_normal(w.d, dtype=np.float64)
    return (u / np.linalg.norm(u)).astype(np.float32)


def needle_rates(w: Workload) -> np.ndarray:
    """Needle rate for each KV head (one value per head, shared across the batch)."""
    if w.needle_rate_range is None:
        return np.full(w.Hkv, w.needle_rate, dtype=np.float64)
    lo, hi = w.needle_rate_range
    return _rng(w.seed, _TAG_RATE).uniform(lo, hi, size=w.Hkv)


def needle_positions(w: Workload, b: int, h: int) -> np.ndarray:
    """Sorted needle key positions in [SINK_TOKENS, Nk) for (batch b, kv head h)."""
    lo = min(SINK_TOKENS, w.Nk)
    pool = w.Nk - lo
    n = int(round(needle_rates(w)[h] * w.Nk))
    n = max(0, min(n, pool))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    pos = _rng(w.seed, _TAG_NEEDLE, b, h).choice(pool, size=n, replace=False) + lo
    return np.sort(pos.astype(np.int64))


def _store(x: np.ndarray, w: Workload) -> np.ndarray:
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else x.astype(np.float32, copy=False)


def k_slice(w: Workload, b: int, h: int, u: Optional[np.ndarray] = None) -> np.ndarray:
    """Keys of (batch b, kv head h): [Nk, d], in storage format (uint16 bf16 bits or float32)."""
    if u is None:
        u = unit_direction(w)
    g = np.float32(w.gain)
    k = _rng(w.seed, _TAG_K, b, h).standard_normal((w.Nk, w.d), dtype=np.float32)
    ns = min(SINK_TOKENS, w.Nk)
    k[:ns] += np.float32(SINK_BOOST) * g * u
    k[needle_positions(w, b, h)] += np.float32(NEEDLE_BOOST) * g * u
    if w.window > 0:
        k[max(0, w.Nk - w.window):] += np.float32(WINDOW_BOOST) * g * u
    return _store(k, w)


def v_slice(w: Workload, b: int, h: int) -> np.ndarray:
    """Values of (batch b, kv head h): [Nk, dv]."""
    v = _rng(w.seed, _TAG_V, b, h).standard_normal((w.Nk, w.dv), dtype=np.float32)
    return _store(v, w)


def q_slice(w: Workload, b: int, h: int, u: Optional[np.ndarray] = None) -> np.ndarray:
    """Queries of (batch b, q head h): [Nq, d]."""
    if u is None:
        u = unit_direction(w)
    q = _rng(w.seed, _TAG_Q, b, h).standard_normal((w.Nq, w.d), dtype=np.float32)
    q += np.float32(QUERY_BOOST * w.gain) * u
    return _store(q, w)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(out: np.ndarray, fn, nb: int, nh: int, threads: Optional[int]) -> None:
    def job(bh):
        b, h = divmod(bh, nh)
        out[b, h] = fn(b, h)

    n = threads or _threads()
    if n == 1 or nb * nh == 1:
        for bh in range(nb * nh):
            job(bh)
        return
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(job, range(nb * nh)))


@dataclass
class Inputs:
    w: Workload
    q: np.ndarray  # prefill [B,Hq,Nq,d]; decode [B,Hq,d]
    k: np.ndarray  # [B,Hkv,Nk,d]
    v: Optional[np.ndarray]  # [B,Hkv,Nk,dv] or None when V is a slice of K
    meta: dict = field(default_factory=dict)


def make_inputs(w: Workload, threads: Optional[int] = None) -> Inputs:
    """Draw the whole workload. Arrays are uint16 (bf16 bits) or float32."""
    st = np.uint16 if w.dtype == "bf16" else np.float32
    u = unit_direction(w)
    q = np.empty((w.B, w.Hq, w.Nq, w.d), dtype=st)
    k = np.empty((w.B, w.Hkv, w.Nk, w.d), dtype=st)
    _fill(q, lambda b, h: q_slice(w, b, h, u), w.B, w.Hq, threads)
    _fill(k, lambda b, h: k_slice(w, b, h, u), w.B, w.Hkv, threads)
    v = None
    if not w.v_is_k_slice:
        v = np.empty((w.B, w.Hkv, w.Nk, w.dv), dtype=st)
        _fill(v, lambda b, h: v_slice(w, b, h), w.B, w.Hkv, threads)
    if w.kind != "prefill":
        q = q.reshape(w.B, w.Hq, w.d)
    return Inputs(w, q, k, v, {"u": u, "needle_rates": needle_rates(w)})


def to_float(x: np.ndarray, w: Workload) -> np.ndarray:
    """Storage format -> float64 values (exact)."""
    if w.dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def small_workload(kind: str = "prefill", *, B=1, Hq=2, Hkv=1, Nq=200, Nk=200, d=128,
                   dv=None, dtype="bf16", causal=True, br=None, bc=64, seed=7,
                   gain=1.0, needle_rate=0.02, window=0,
                   lambdas: Sequence[float] = (0.0, 1e-3, 1e-2)) -> Workload:
    """A test-sized workload with the same generator (ragged sizes welcome)."""
    if dv is None:
        dv = 512 if kind == "decode_mla" else d
    if br is None:
        br = 1 if kind != "prefill" else (64 if dtype == "fp32" else 128)
    if kind != "prefill":
        Nq = 1
        causal = False
    return Workload(f"{kind}_small_{seed}", kind, B, Hq, Hkv, Nq, Nk, d, dv, dtype, causal,
                    br, bc, tuple(lambdas), seed, needle_rate=needle_rate, window=window,
                    gain=gain)


def block_set(w: Workload, density: float, *, local: int = 2, sink: bool = True,
              seed: int = 0) -> np.ndarray:
    """A seeded block set [B, Hq, nQt, nKt] (uint8, 1 = block selected) for
    block-sparse prefill, shaped like the sets block-sparse prefill methods
    select (CRISP write-up on rit.work, "Что сделали"): the first key tile
    (attention sinks) when ``sink``, the ``local`` key tiles ending at each
    query tile's causal diagonal (recent window), a per-head set of "vertical"
    key-tile columns selected for every query tile, and scattered blocks. The
    vertical columns and the scattered blocks each take about ``density / 2``
    of the tiles. Blocks past the diagonal are drawn too (a kernel must ignore
    them)."""
    nqt, nkt = n_tiles(w.Nq, w.br), n_tiles(w.Nk, w.bc)
    out = np.zeros((w.B, w.Hq, nqt, nkt), dtype=np.uint8)
    last = (np.minimum((np.arange(nqt) + 1) * w.br, w.Nq) - 1 + (w.Nk - w.Nq if w.causal else 0))
    diag = np.minimum(last // w.bc, nkt - 1) if w.causal else np.full(nqt, nkt - 1)
    cols = np.arange(nkt)[None, :]
    for b in range(w.B):
        for h in range(w.Hq):
            rng = _rng(w.seed, 6, seed, b, h)
            vertical = rng.random(nkt) < density / 2
            scattered = rng.random((nqt, nkt)) < density / 2
            sel = vertical[None, :] | scattered
            sel |= (cols > diag[:, None] - local) & (cols <= diag[:, None])
            if sink:
                sel[:, 0] = True
            out[b, h] = sel
    return out


def dense_equivalent_flops(w: Workload) -> float:
    """2*(d+dv) FLOPs per visible (query, key) pair, summed over batch and heads."""
    if w.kind == "prefill" and w.causal:
        # query i sits at Nk-Nq+i and sees keys 0..Nk-Nq+i
        off = w.Nk - w.Nq
        pairs = w.Nq * (off + 1) + w.Nq * (w.Nq - 1) // 2
    else:
        pairs = w.Nq * w.Nk
    return 2.0 * (w.d + w.dv) * w.B * w.Hq * pairs


def n_tiles(n: int, t: int) -> int:
    return (n + t - 1) // t


__all__ = [
    "Workload", "WORKLOADS", "Inputs", "make_inputs", "small_workload", "q_slice", "k_slice",
    "v_slice", "unit_direction", "needle_positions", "needle_rates", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "to_float", "dense_equivalent_flops", "n_tiles", "block_set",
]


if __name__ == "__main__":  # pragma: no cover - quick timing aid
    import time
    for cid in (1, 2):
        t0 = time.time()
        inp = make_inputs(WORKLOADS[cid])
        print(cid, inp.q.shape, inp.k.shape, f"{time.time() - t0:.2f}s")
