"""Plain CPU oracle for BLASST skip-softmax attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke entry and
the benchmark's CPU-baseline leg may import this module. The GPU path neither
imports it nor shares any code with it, and this module imports nothing from
the GPU path.

What is computed (sources are the BLASST explainer post "BLASST: Dynamic
BLocked Attention Sparsity via Softmax Thresholding" on the seeallochnaya
Telegram channel, called "the BLASST post" below, and the digg.com thread
"BLASST wins Best Paper at MLSys 2026 ...", called "the digg thread"):

* Attention is computed block by block along the keys, in increasing key
  order, with the usual max-subtracted (shift-invariant) softmax
  (BLASST post, paragraph "В чём идея").
* The maximum is tracked online: a running per-row maximum is compared with
  each new block's maximum, and earlier partial sums are rescaled when it
  grows; after the last block the result is exact (BLASST post, paragraph on
  the online trick of FlashAttention 1).
* BLASST: when a block's maximum is far below the maximum of the blocks
  before it, the whole block is dropped, and its V rows take no part in the
  result (BLASST post, paragraph beginning "BLASST предлагает"). The first block
  is always processed (BLASST post, first figure). The test is a single scalar
  threshold on the online softmax statistics, reusing the running max (digg
  thread, the authors' posts).

Readings taken where the pages are silent (each one is listed in the design
notes of the repository):

* thr = ln(lambda) in the natural-log units of the scaled logits
  s = scale * q.k; lambda = 0 means thr = -inf (nothing dropped); lambda must
  lie in [0, 1].
* A tile's gap is the maximum over its valid rows of (row max in the tile
  minus the row's running max), so a tile is dropped only when *every* row is
  below the threshold; the comparison is strict (a tie keeps the tile).
* A row with no visible key in the tile votes "drop" (gap -inf); a row whose
  running max is still -inf votes "keep" (gap +inf).
* Causal masking is bottom-right aligned: query i sits at key position
  Nk - Nq + i. Tiles with no visible (row, key) pair at all are "not visited"
  (mask value 2) and are not counted as dropped.
* GQA: query head h reads key/value head h // (Hq / Hkv).
* Decode is the same rule with one query row per (batch, head); tile 0 is
  the global first key tile and the running max is global along the keys.
* Block-sparse mode: a (query, key) pair is visible when causality allows it
  and its (query tile, key tile) block is in the caller's set; the skip rule
  then runs over the set's tiles only, so "tile 0" is the first tile of the
  set that the query tile visits. Rows that see nothing output zero, lse -inf.
* Two-pass variant (a reply in the digg thread): the tile map comes from the
  skip rule on scores of MXFP4-quantized q and k (OCP MX v1.0), then exact
  attention runs over the kept tiles; see the section at the end.

Arithmetic is float64 throughout; inputs are whatever float values the caller
passes (bf16 workloads pass the exact bf16 values, widened).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

MASK_SKIPPED = 0
MASK_KEPT = 1
MASK_NOT_VISITED = 2


def threshold(lam: float) -> float:
    """thr = ln(lambda), with ln(0) = -inf. lambda must be in [0, 1]."""
    lam = float(lam)
    if not (0.0 <= lam <= 1.0):
        raise ValueError(f"lambda must lie in [0, 1], got {lam!r}")
    return -math.inf if lam == 0.0 else math.log(lam)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def visible(nq: int, nk: int, causal: bool, row0: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """Boolean [rows, nk]: may query (row0 + r) see key c? Bottom-right causal alignment."""
    if rows is None:
        rows = nq - row0
    r = np.arange(row0, row0 + rows)[:, None]
    c = np.arange(nk)[None, :]
    if not causal:
        return np.ones((rows, nk), dtype=bool)
    return c <= r + (nk - nq)


@dataclass
class TileRowResult:
    out: np.ndarray       # [rows, dv]
    lse: np.ndarray       # [rows]
    mask: np.ndarray      # [nKt] uint8: 0 dropped, 1 kept, 2 not visited
    gap: np.ndarray       # [nKt] float64 tile max-gap (nan where not visited)
    m_before: np.ndarray  # [nKt, rows] running max on entry to each tile (-inf before tile 0)
    tile_max: np.ndarray  # [nKt, rows] row max inside each tile (-inf where none visible)


def blasst_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, lam: float, bc: int,
                vis: np.ndarray, scale: float) -> TileRowResult:
    """The ordered skip rule for one block of query rows against one key/value head.

    q: [rows, d] query rows that form one query tile; k: [Nk, d]; v: [Nk, dv];
    vis: [rows, Nk] visibility. Key tiles are visited left to right.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows, nk = vis.shape
    dv = v.shape[1]
    thr = threshold(lam)
    nkt = -(-nk // bc)

    # scores of this query tile against every key, masked entries at -inf
    s = scale * (q @ k.T)
    s = np.where(vis, s, -np.inf)

    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    o = np.zeros((rows, dv))
    mask = np.full(nkt, MASK_NOT_VISITED, dtype=np.uint8)
    gap = np.full(nkt, np.nan)
    m_before = np.full((nkt, rows), -np.inf)
    tile_max = np.full((nkt, rows), -np.inf)

    for j in range(nkt):
        c0, c1 = j * bc, min((j + 1) * bc, nk)
        if not vis[:, c0:c1].any():
            continue  # no visible (row, key) pair: the tile is not visited
        st = s[:, c0:c1]
        mt = st.max(axis=1)
        m_before[j] = m
        tile_max[j] = mt
        # per-row gap with the infinity conventions, then the tile's max-gap
        with np.errstate(invalid="ignore"):  # mt - m is discarded where either is -inf
            g_r = np.where(mt == -np.inf, -np.inf, np.where(m == -np.inf, np.inf, mt - m))
        g = g_r.max() if rows else -np.inf
        gap[j] = g
        keep = (j == 0) or not (g < thr)
        if not keep:
            mask[j] = MASK_SKIPPED
            continue
        mask[j] = MASK_KEPT
        m_new = np.maximum(m, mt)
        # a row that has seen no key yet keeps empty sums (reference 0 instead of -inf)
        m_ref = np.where(m_new == -np.inf, 0.0, m_new)
        alpha = np.exp(m - m_ref)        # 0 where m was -inf
        p = np.exp(st - m_ref[:, None])  # 0 where masked
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[c0:c1]
        m = m_new

    with np.errstate(divide="ignore", invalid="ignore"):
        out = o / l[:, None]
        lse = m + np.log(l)
    return TileRowResult(out, lse, mask, gap, m_before, tile_max)


@dataclass
class OracleResult:
    out: np.ndarray    # prefill [B,Hq,Nq,dv] / decode [B,Hq,dv]
    lse: np.ndarray    # prefill [B,Hq,Nq] / decode [B,Hq]
    mask: np.ndarray   # prefill [B,Hq,nQt,nKt] / decode [B,Hq,nKt]
    gap: np.ndarray    # same shape as mask
    stats: np.ndarray  # prefill [B,Hq,2] = (visited, kept); decode [B,Hq,3] adds V tiles loaded


def prefill_tile(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, hq: int, i: int,
                 lam: float, causal: bool, br: int, bc: int,
                 scale: Optional[float] = None) -> TileRowResult:
    """One (batch b, query head hq, query tile i) of a prefill call.

    q: [B,Hq,Nq,d]; k: [B,Hkv,Nk,d]; v: [B,Hkv,Nk,dv].
    """
    B, Hq, nq, d = q.shape
    hkv = k.shape[1]
    if Hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    kvh = hq // (Hq // hkv)
    nk = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    r0, r1 = i * br, min((i + 1) * br, nq)
    vis = visible(nq, nk, causal, r0, r1 - r0)
    return blasst_rows(q[b, hq, r0:r1], k[b, kvh], v[b, kvh], lam, bc, vis, scale)


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, lam: float, causal: bool,
            br: int, bc: int, scale: Optional[float] = None) -> OracleResult:
    """Whole prefill call: every (b, hq, query tile) independently."""
    B, Hq, nq, d = q.shape
    nk, dv = k.shape[2], v.shape[3]
    if causal and nq > nk:
        raise ValueError("causal prefill needs Nq <= Nk")
    nqt, nkt = -(-nq // br), -(-nk // bc)
    out = np.zeros((B, Hq, nq, dv))
    lse = np.zeros((B, Hq, nq))
    mask = np.full((B, Hq, nqt, nkt), MASK_NOT_VISITED, dtype=np.uint8)
    gap = np.full((B, Hq, nqt, nkt), np.nan)
    stats = np.zeros((B, Hq, 2), dtype=np.int64)
    for b in range(B):
        for hq in range(Hq):
            for i in range(nqt):
                r = prefill_tile(q, k, v, b, hq, i, lam, causal, br, bc, scale)
                r0 = i * br
                out[b, hq, r0:r0 + r.out.shape[0]] = r.out
                lse[b, hq, r0:r0 + r.out.shape[0]] = r.lse
                mask[b, hq, i] = r.mask
                gap[b, hq, i] = r.gap
            stats[b, hq, 0] = int((mask[b, hq] != MASK_NOT_VISITED).sum())
            stats[b, hq, 1] = int((mask[b, hq] == MASK_KEPT).sum())
    return OracleResult(out, lse, mask, gap, stats)


def block_sparse_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, sel_row: np.ndarray,
                      lam: float, causal: bool, nq: int, row0: int, bc: int,
                      scale: float) -> TileRowResult:
    """One query tile of block-sparse prefill against one key/value head.

    q_rows: [rows, d], the queries row0 .. row0+rows-1 of a call with nq
    queries; k: [Nk, d]; v: [Nk, dv]; sel_row: [nKt], this query tile's row of
    the block set (nonzero = may attend). A (query, key) pair is visible when
    the causal rule allows it and its key tile is in the set; the skip rule then
    runs on that visibility, so tiles outside the set are "not visited" and the
    first tile of the set that has a visible pair is kept (its rows have no
    running max yet, so their gap is +inf). A row that sees no key outputs zero
    with lse = -inf.
    """
    nk = k.shape[0]
    in_set = np.repeat(np.asarray(sel_row) != 0, bc)[:nk]
    vis = visible(nq, nk, causal, row0, len(q_rows)) & in_set[None, :]
    r = blasst_rows(q_rows, k, v, lam, bc, vis, scale)
    seen = vis.any(axis=1)
    r.out = np.where(seen[:, None], r.out, 0.0)
    r.lse = np.where(seen, r.lse, -np.inf)
    return r


def prefill_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_mask: np.ndarray,
                   lam: float, causal: bool, br: int, bc: int,
                   scale: Optional[float] = None) -> OracleResult:
    """Prefill restricted to a caller-given set of (query tile, key tile) blocks.

    Ordinary softmax attention computed only inside selected blocks is the
    last stage of block-sparse prefill methods (the CRISP summary on rit.work,
    section "Что сделали", last paragraph); block-sparse masks are one of the
    mask kinds of the LongCA-bench post on denisavetisyan.com (section "Сад
    Внимания: LongCA-bench и Стандартизация Оценки"). Each query tile runs
    block_sparse_rows on its row of the set.

    block_mask: [B, Hq, nQt, nKt], broadcastable from the left; nonzero marks
    a block the query tile may attend.
    """
    B, Hq, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    dv = v.shape[3]
    if Hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and nq > nk:
        raise ValueError("causal prefill needs Nq <= Nk")
    if scale is None:
        scale = default_scale(d)
    nqt, nkt = -(-nq // br), -(-nk // bc)
    sel = np.broadcast_to(np.asarray(block_mask), (B, Hq, nqt, nkt))
    out = np.zeros((B, Hq, nq, dv))
    lse = np.full((B, Hq, nq), -np.inf)
    mask = np.full((B, Hq, nqt, nkt), MASK_NOT_VISITED, dtype=np.uint8)
    gap = np.full((B, Hq, nqt, nkt), np.nan)
    stats = np.zeros((B, Hq, 2), dtype=np.int64)
    for b in range(B):
        for hq in range(Hq):
            kvh = hq // (Hq // hkv)
            for i in range(nqt):
                r0, r1 = i * br, min((i + 1) * br, nq)
                r = block_sparse_rows(q[b, hq, r0:r1], k[b, kvh], v[b, kvh], sel[b, hq, i], lam,
                                      causal, nq, r0, bc, scale)
                out[b, hq, r0:r1] = r.out
                lse[b, hq, r0:r1] = r.lse
                mask[b, hq, i] = r.mask
                gap[b, hq, i] = r.gap
            stats[b, hq, 0] = int((mask[b, hq] != MASK_NOT_VISITED).sum())
            stats[b, hq, 1] = int((mask[b, hq] == MASK_KEPT).sum())
    return OracleResult(out, lse, mask, gap, stats)


def prefill_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                     mask: np.ndarray, causal: bool, br: int, bc: int,
                     scale: Optional[float] = None, magnitudes: bool = False,
                     out: Optional[np.ndarray] = None) -> tuple:
    """Gradients of a skip-softmax prefill with its tile mask held fixed.

    Fine-tuning a model with the skip kernels in place improves its quality
    (BLASST post, paragraph beginning "Все изменения можно делать без
    дообучения"). The keep/drop decisions are a piecewise-constant function of
    the inputs, so almost everywhere the gradient is that of softmax attention
    over the kept tiles, the mask being a constant.

    q [B,Hq,Nq,d], k [B,Hkv,Nk,d], v [B,Hkv,Nk,dv], dout [B,Hq,Nq,dv];
    mask [B,Hq,nQt,nKt] as returned by the forward (1 = kept; 0 and 2 take no
    part). Per query head, with A = causal visibility AND the expanded kept
    tiles:
        S = scale q k^T (-inf outside A);  P = row softmax of S over A (a row
        with no allowed key has P = 0);  O = P v
        dv = P^T dout;  dP = dout v^T;  delta = rowsum(dout * O)
        dS = P * (dP - delta);  dq = scale dS k;  dk = scale dS^T q
    and dk, dv of a KV head are the sums over the query heads that read it.
    out, if given, is the stored forward output [B,Hq,Nq,dv] that delta is taken
    from (an implementation saves the output in the type it was written in);
    by default delta uses the exact output P v.
    Returns (dq, dk, dv) in float64; with magnitudes=True also the sums of the
    absolute values of the products each element is made of (scale |dS| |k|,
    scale |dS|^T |q|, |P|^T |dout|), the scale of a rounding-error bound.
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, Hq, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    if Hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = default_scale(d)
    G = Hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    vis = visible(nq, nk, causal)
    for b in range(B):
        for hq in range(Hq):
            kvh = hq // G
            allowed = vis & expand_tile_mask(mask[b, hq], br, bc, nq, nk)
            s = np.where(allowed, scale * (q[b, hq] @ k[b, kvh].T), -np.inf)
            mx = s.max(axis=1, keepdims=True)
            live = np.isfinite(mx)
            e = np.exp(s - np.where(live, mx, 0.0))
            den = e.sum(axis=1, keepdims=True)
            p = np.where(live, e / np.where(live, den, 1.0), 0.0)
            o = p @ v[b, kvh]
            dv[b, kvh] += p.T @ dout[b, hq]
            dp = dout[b, hq] @ v[b, kvh].T
            if out is not None:
                o = np.asarray(out[b, hq], dtype=np.float64)
            delta = (dout[b, hq] * o).sum(axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, hq] = scale * (ds @ k[b, kvh])
            dk[b, kvh] += scale * (ds.T @ q[b, hq])
            if magnitudes:
                mq[b, hq] = scale * (np.abs(ds) @ np.abs(k[b, kvh]))
                mk[b, kvh] += scale * (np.abs(ds).T @ np.abs(q[b, hq]))
                mv[b, kvh] += p.T @ np.abs(dout[b, hq])
    if magnitudes:
        return dq, dk, dv, mq, mk, mv
    return dq, dk, dv


def decode_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, hq: int,
               lam: float, bc: int, scale: Optional[float] = None) -> TileRowResult:
    """One (batch b, query head hq) decode row: a single query that sees every key.

    q: [B,Hq,d]; k: [B,Hkv,Nk,d]; v: [B,Hkv,Nk,dv] (for an MLA latent cache pass
    ``k[..., :dv]``).
    """
    B, Hq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    kvh = hq // (Hq // hkv)
    if scale is None:
        scale = default_scale(d)
    return blasst_rows(q[b, hq][None, :], k[b, kvh], v[b, kvh], lam, bc,
                       np.ones((1, nk), dtype=bool), scale)


def decode(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray], lam: float, bc: int,
           scale: Optional[float] = None, dv: Optional[int] = None) -> OracleResult:
    """Whole decode call. With ``v`` None the values are ``k[..., :dv]`` (MLA)."""
    B, Hq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    G = Hq // hkv
    if v is None:
        if dv is None:
            raise ValueError("dv is required when V is a slice of K")
        v = k[..., :dv]
    dv = v.shape[3]
    nkt = -(-nk // bc)
    out = np.zeros((B, Hq, dv))
    lse = np.zeros((B, Hq))
    mask = np.zeros((B, Hq, nkt), dtype=np.uint8)
    gap = np.zeros((B, Hq, nkt))
    stats = np.zeros((B, Hq, 3), dtype=np.int64)
    for b in range(B):
        for hq in range(Hq):
            r = decode_row(q, k, v, b, hq, lam, bc, scale)
            out[b, hq] = r.out[0]
            lse[b, hq] = r.lse[0]
            mask[b, hq] = r.mask
            gap[b, hq] = r.gap
        for g0 in range(0, Hq, G):
            # a V tile is fetched for a KV head when any query head that reads it keeps it
            loaded = int((mask[b, g0:g0 + G] == MASK_KEPT).any(axis=0).sum())
            stats[b, g0:g0 + G, 2] = loaded
        stats[b, :, 0] = nkt
        stats[b, :, 1] = (mask[b] == MASK_KEPT).sum(axis=1)
    return OracleResult(out, lse, mask, gap, stats)


def expand_tile_mask(mask_row: np.ndarray, br: int, bc: int, nq: int, nk: int) -> np.ndarray:
    """[nQt, nKt] tile mask -> [nq, nk] boolean 'kept' per (query, key) pair."""
    kept = (np.asarray(mask_row) == MASK_KEPT)
    el = np.repeat(np.repeat(kept, br, axis=0), bc, axis=1)
    return el[:nq, :nk]


def masked_dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray,
                           causal: bool, scale: Optional[float] = None) -> tuple:
    """Softmax attention restricted to the kept keys (numerator and denominator).

    One head: q [Nq,d], k [Nk,d], v [Nk,dv], keep [Nq,Nk] boolean. Returns (out, lse).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    if scale is None:
        scale = default_scale(q.shape[1])
    s = scale * (q @ k.T)
    allowed = keep & visible(q.shape[0], k.shape[0], causal)
    s = np.where(allowed, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p @ v) / den, (mx + np.log(den))[:, 0]


# --------------------------------------------------------------------------- two-pass variant
#
# The digg thread suggests a cheaper first pass (one commenter's reply to the
# authors): recompute q.k in 4-bit precision only to find the maxima (no
# exponentials are needed there), fix the sparsity map from them, then gather
# the kept blocks and compute attention over them. Readings taken:
# * "4-bit" is MXFP4 from the OCP Microscaling Formats (MX) Specification
#   v1.0: FP4 E2M1 elements, one E8M0 power-of-two scale per block of 32
#   consecutive elements along the feature axis (here d_qk).
# * The map is the skip rule itself (blasst_rows) run on the scores of the
#   dequantized q and k, with the same scale and tiles.
# * The second pass is exact softmax attention over the kept tiles only:
#   block-sparse prefill with lambda = 0 and the kept tiles as the set.

MX_BLOCK = 32
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # code & 7 -> magnitude
E2M1_EMAX = 2          # exponent of the largest normal, 6 = 1.5 * 2^2
E2M1_MAX = 6.0
E8M0_BIAS = 127


def round_to_e2m1(a: np.ndarray) -> np.ndarray:
    """Nearest FP4 E2M1 magnitude to a >= 0, ties to the even code, larger
    values clamped to the largest normal (6).

    The spacing of E2M1 is 0.5 below 2 (subnormal 0.5 included), 1 in [2, 4)
    and 2 in [4, 8); np.rint rounds half to even.
    """
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)                       # a = f * 2^ex with f in [0.5, 1)
    e = np.clip(ex - 1, 0, E2M1_EMAX)         # binade exponent; below 1 the subnormal spacing
    ulp = np.ldexp(0.5, e)                    # 2^(e - 1): one mantissa bit
    return np.minimum(np.rint(a / ulp) * ulp, E2M1_MAX)


def mx_quantize_fp4(x: np.ndarray) -> tuple:
    """MXFP4 quantization along the last axis (OCP MX v1.0, conversion of a
    block of scalar floats to an MX block).

    Per block of 32: shared exponent = floor(log2(max |x|)) - emax_elem,
    clamped to the E8M0 range [-127, 127] (an all-zero block takes -127);
    each element is x / 2^shared rounded to E2M1 (round_to_e2m1), the sign
    copied from x. Returns (codes uint8 [..., d] with sign in bit 3 and the
    magnitude index in bits 0-2, scales uint8 [..., d / 32] = shared + 127).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % MX_BLOCK:
        raise ValueError("the feature size must be a multiple of 32")
    blk = x.reshape(*x.shape[:-1], d // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)
    shared = np.where(amax > 0, ex - 1 - E2M1_EMAX, -E8M0_BIAS)
    shared = np.clip(shared, -E8M0_BIAS, E8M0_BIAS)
    mag = round_to_e2m1(np.abs(blk) / np.ldexp(1.0, shared)[..., None])
    code = np.searchsorted(E2M1_MAGNITUDES, mag).astype(np.uint8)
    code |= (np.signbit(blk).astype(np.uint8) << 3)
    return code.reshape(x.shape), (shared + E8M0_BIAS).astype(np.uint8)


def mx_dequantize_fp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of MXFP4 codes: sign * E2M1 magnitude * 2^(scale - 127)."""
    codes = np.asarray(codes)
    mag = E2M1_MAGNITUDES[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    x = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - E8M0_BIAS)
    return sign * mag * np.repeat(x, MX_BLOCK, axis=-1)


def twopass_tile(q: np.ndarray, k: np.ndarray, v: np.ndarray, qd: np.ndarray, kd: np.ndarray,
                 b: int, hq: int, i: int, lam: float, causal: bool, br: int, bc: int,
                 scale: Optional[float] = None) -> tuple:
    """One (batch, query head, query tile) of the two-pass variant.

    qd, kd: the MXFP4-dequantized q and k. Returns (pre, r): pre is the skip
    rule on the dequantized scores (its mask and gaps are the pass-1 map); r is
    exact attention of q, k, v over pre's kept tiles.
    """
    B, Hq, nq, d = q.shape
    kvh = hq // (Hq // k.shape[1])
    if scale is None:
        scale = default_scale(d)
    pre = prefill_tile(qd, kd, v, b, hq, i, lam, causal, br, bc, scale)
    r0, r1 = i * br, min((i + 1) * br, nq)
    r = block_sparse_rows(q[b, hq, r0:r1], k[b, kvh], v[b, kvh], pre.mask == MASK_KEPT, 0.0,
                          causal, nq, r0, bc, scale)
    return pre, r


def prefill_twopass(q: np.ndarray, k: np.ndarray, v: np.ndarray, lam: float, causal: bool,
                    br: int, bc: int, scale: Optional[float] = None) -> OracleResult:
    """Whole two-pass prefill call. mask, gap and stats are the pass-1 map's
    (gap on the dequantized scores); out and lse are the exact attention over
    the kept tiles."""
    B, Hq, nq, d = q.shape
    nk, dv = k.shape[2], v.shape[3]
    if causal and nq > nk:
        raise ValueError("causal prefill needs Nq <= Nk")
    qd = mx_dequantize_fp4(*mx_quantize_fp4(q))
    kd = mx_dequantize_fp4(*mx_quantize_fp4(k))
    nqt, nkt = -(-nq // br), -(-nk // bc)
    out = np.zeros((B, Hq, nq, dv))
    lse = np.full((B, Hq, nq), -np.inf)
    mask = np.full((B, Hq, nqt, nkt), MASK_NOT_VISITED, dtype=np.uint8)
    gap = np.full((B, Hq, nqt, nkt), np.nan)
    stats = np.zeros((B, Hq, 2), dtype=np.int64)
    for b in range(B):
        for hq in range(Hq):
            for i in range(nqt):
                pre, r = twopass_tile(q, k, v, qd, kd, b, hq, i, lam, causal, br, bc, scale)
                r0 = i * br
                out[b, hq, r0:r0 + r.out.shape[0]] = r.out
                lse[b, hq, r0:r0 + r.out.shape[0]] = r.lse
                mask[b, hq, i] = pre.mask
                gap[b, hq, i] = pre.gap
            stats[b, hq, 0] = int((mask[b, hq] != MASK_NOT_VISITED).sum())
            stats[b, hq, 1] = int((mask[b, hq] == MASK_KEPT).sum())
    return OracleResult(out, lse, mask, gap, stats)


__all__ = [
    "threshold", "default_scale", "visible", "blasst_rows", "prefill_tile", "prefill",
    "block_sparse_rows", "prefill_masked", "prefill_backward",
    "round_to_e2m1", "mx_quantize_fp4", "mx_dequantize_fp4", "twopass_tile", "prefill_twopass",
    "MX_BLOCK", "E2M1_MAGNITUDES",
    "decode_row", "decode", "expand_tile_mask", "masked_dense_attention",
    "OracleResult", "TileRowResult", "MASK_SKIPPED", "MASK_KEPT", "MASK_NOT_VISITED",
]
