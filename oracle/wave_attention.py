"""Masked softmax attention of one wave tick, in numpy float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Plain definition, no
blocking of any reduction: every output row is softmax over a fully
materialised score row with the wave mask applied as -inf.

Citations name pages of "Wave Forcing: Towards Speed-of-Light Streaming Video
Generation":
  [summary]   the structured summary page (picx.dev), section "Methodology";
  [full text] the full-text page (paperpeel.com), with section / equation.

Readings of points the pages leave open:
  * the store chunk is stage S of the tick and is an active chunk like the
    others; the wave mask 1[j >= s] therefore gives every denoising stage the
    live store, and the store sees only itself among live chunks;
  * the anchor is the oldest history chunk: same pages, same attention;
  * per-stage history budgets are expressed as hist_first[s], the first
    history chunk stage s may see (0 = all);
  * softmax scale is a parameter (1/sqrt(D) in every workload);
  * rows of inactive chunks are neither queries nor keys.
"""
from __future__ import annotations

import concurrent.futures
import os
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

Segment = Tuple[str, int]  # ("hist", c) or ("live", j)


# ----------------------------------------------------------------------------
# number decoding
# ----------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns; float arrays are taken at their value."""
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# tick composition and the wave mask
# ----------------------------------------------------------------------------
def tick_members(k: int, S: int, n_chunks: Optional[int] = None) -> Dict[int, int]:
    """Chunk index held by each stage slot at tick k.

    [summary] Methodology 1: at tick k the denoising inputs are
    Z_k^(0), Z_{k-1}^(1), ..., Z_{k-S+1}^(S-1) (stage s holds chunk k-s) and the
    store adds B_{k-S} at s = S. Chunks that do not exist yet (index < 0) or no
    longer exist (index >= n_chunks) leave their slot empty (fill / drain).
    """
    out = {}
    for s in range(S + 1):
        c = k - s
        if c < 0:
            continue
        if n_chunks is not None and c >= n_chunks:
            continue
        out[s] = c
    return out


def active_mask_for_tick(k: int, S: int, n_chunks: Optional[int] = None) -> int:
    """Bitmask of occupied stage slots at tick k (bit s = stage s, bit S = store)."""
    m = 0
    for s in tick_members(k, S, n_chunks):
        m |= 1 << s
    return m


def _active(active_mask: int, S: int) -> List[int]:
    return [s for s in range(S + 1) if (active_mask >> s) & 1]


def wave_mask(S: int, active_mask: int) -> np.ndarray:
    """M_WF over stage slots 0..S (store = S).

    [summary] "Introduction and Theoretical Foundation" / [full text] Eq. (4):
    chunk at stage s may read live K/V of the chunk at stage j exactly when
    j >= s, both in the active set. Entry [s, j]; False outside the active set.
    """
    act = set(_active(active_mask, S))
    m = np.zeros((S + 1, S + 1), dtype=bool)
    for s in range(S + 1):
        for j in range(S + 1):
            m[s, j] = (s in act) and (j in act) and (j >= s)
    return m


def context_segments(s: int, S: int, active_mask: int, n_hist: int,
                     hist_first: int = 0) -> List[Segment]:
    """Ordered layer context of the query chunk at stage s.

    [summary] Methodology 1 / [full text] Eq. (5) and Appendix B.3: anchor, then
    bounded clean history (oldest first), then the live store, then the live
    denoising chunks j >= s in increasing j (self first). The anchor is history
    chunk 0. For the store itself (s = S) the live part is the store alone.
    """
    segs: List[Segment] = [("hist", c) for c in range(hist_first, n_hist)]
    m = wave_mask(S, active_mask)
    if m[s, S]:
        segs.append(("live", S))
    for j in range(s, S):
        if m[s, j]:
            segs.append(("live", j))
    return segs


def key_axis_labels(S: int, n_hist: int) -> List[Segment]:
    """Segments of the oracle's single key axis: all history, then live S, 0..S-1.

    Restricted by the mask of stage s this is exactly the Eq. (5) order.
    """
    return [("hist", c) for c in range(n_hist)] + [("live", S)] + \
        [("live", j) for j in range(S)]


def token_mask(s: int, S: int, active_mask: int, n_hist: int, T: int,
               hist_first: int = 0) -> np.ndarray:
    """Visibility of every key on the key axis for a query in chunk s (bool, length
    (n_hist + S + 1) * T): history chunk c visible iff c >= hist_first, live
    chunk j visible iff M_WF[s, j]."""
    m = wave_mask(S, active_mask)
    vis = []
    for kind, idx in key_axis_labels(S, n_hist):
        if kind == "hist":
            ok = (idx >= hist_first) and bool((active_mask >> s) & 1)
        else:
            ok = bool(m[s, idx])
        vis.append(np.full(T, ok, dtype=bool))
    return np.concatenate(vis) if vis else np.zeros(0, dtype=bool)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _key_matrix(live: np.ndarray, hist: np.ndarray, h: int, S: int) -> np.ndarray:
    """Stack K (or V) of head h along the key axis of key_axis_labels()."""
    n_hist = hist.shape[0]
    parts = [hist[c, :, h, :] for c in range(n_hist)]
    parts.append(live[S, :, h, :])
    parts.extend(live[j, :, h, :] for j in range(S))
    return np.concatenate(parts, axis=0)


def _hf(hist_first: Optional[Sequence[int]], s: int) -> int:
    return 0 if hist_first is None else int(hist_first[s])


def attention_tick(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   hist_k: np.ndarray, hist_v: np.ndarray, S: int, active_mask: int,
                   scale: float, hist_first: Optional[Sequence[int]] = None,
                   stages: Optional[Iterable[int]] = None,
                   heads: Optional[Iterable[int]] = None,
                   rows: Optional[np.ndarray] = None,
                   threads: Optional[int] = None,
                   row_group: int = 512) -> Dict[int, np.ndarray]:
    """Outputs of one tick: {stage s: O_s float64 [len(rows)][len(heads)][D]}.

    q, k, v: live chunks [S+1][T][H][D]; hist_k, hist_v: [n_hist][T][H][D] in
    logical (oldest-first) order; uint16 = bf16 bits, float = values.

    For each active stage s and head h (heads are independent, run on a thread
    pool): Sc = scale * Q K^T over the whole key axis, Sc = -inf where the
    materialised token mask is False, m = rowmax, P = exp(Sc - m), l = sum P,
    O = (P V) / l. Query rows are processed `row_group` at a time only to bound
    memory; each row's result does not depend on the grouping.
    """
    T = q.shape[1]
    H = q.shape[2]
    n_hist = hist_k.shape[0]
    act = _active(active_mask, S)
    stages = act if stages is None else [s for s in stages if s in act]
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(T) if rows is None else np.asarray(rows)

    D = q.shape[3]
    masks = {s: token_mask(s, S, active_mask, n_hist, T, _hf(hist_first, s)) for s in stages}
    out = {s: np.zeros((len(rows), len(heads), D), dtype=np.float64) for s in stages}

    def one_head(hi: int) -> None:
        h = heads[hi]
        K = as_f64(_key_matrix(k, hist_k, h, S))
        V = as_f64(_key_matrix(v, hist_v, h, S))
        for s in stages:
            for r0 in range(0, len(rows), row_group):
                rr = rows[r0:r0 + row_group]
                Q = as_f64(q[s, rr, h, :])
                sc = (Q @ K.T) * scale
                mask2d = np.tile(masks[s], (len(rr), 1))      # materialised mask
                sc = np.where(mask2d, sc, -np.inf)
                m = sc.max(axis=1, keepdims=True)
                p = np.exp(sc - m)
                l = p.sum(axis=1, keepdims=True)
                out[s][r0:r0 + len(rr), hi, :] = (p @ V) / l

    # Heads run on a thread pool only when each head is heavy; for a few sampled
    # rows the matrix products' own threads are faster than nesting pools.
    nthreads = threads or (min(len(heads), len(os.sched_getaffinity(0)))
                           if len(rows) >= 1024 else 1)
    if nthreads <= 1 or len(heads) == 1:
        for hi in range(len(heads)):
            one_head(hi)
    else:
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one_head, range(len(heads))))
    return out


def attention_tick_paged(q, k, v, store, hist_pages: Sequence[Sequence[int]], S: int,
                         active_mask: int, scale: float, **kw) -> Dict[int, np.ndarray]:
    """Same as attention_tick with the history read from a dict page store through
    per-chunk page lists ([full text] §4.2 / Appendix B.3: history lives in pages)."""
    T = q.shape[1]
    hk, hv = store.gather(hist_pages, T)
    return attention_tick(q, k, v, hk, hv, S, active_mask, scale, **kw)


def attention_tick_fully_paged(q, store, hist_pages: Sequence[Sequence[int]],
                               live_pages: Sequence[Optional[Sequence[int]]], S: int,
                               active_mask: int, scale: float, **kw) -> Dict[int, np.ndarray]:
    """Same as attention_tick with every K/V segment read from the page store: the
    history through hist_pages and live slot j through live_pages[j] (None for a
    slot that is not active). [full text] Appendix B.8, Eq. (13): the K/V arrays
    hold the anchor, the bounded history, the live store and the denoising chunks."""
    T, H, D = q.shape[1], q.shape[2], q.shape[3]
    hk, hv = store.gather(hist_pages, T)
    lk = np.zeros((S + 1, T, H, D), np.uint16)
    lv = np.zeros_like(lk)
    for j in range(S + 1):
        if (active_mask >> j) & 1:
            if live_pages[j] is None:
                raise ValueError(f"active slot {j} has no pages")
            kk, vv = store.gather([live_pages[j]], T)
            lk[j], lv[j] = kk[0], vv[0]
    return attention_tick(q, lk, lv, hk, hv, S, active_mask, scale, **kw)


# ----------------------------------------------------------------------------
# key counts and useful FLOPs
# ----------------------------------------------------------------------------
def keys_per_stage(S: int, active_mask: int, n_hist: int, T: int,
                   hist_first: Optional[Sequence[int]] = None) -> Dict[int, int]:
    """Number of visible keys per active stage, counted from the token mask."""
    return {s: int(token_mask(s, S, active_mask, n_hist, T, _hf(hist_first, s)).sum())
            for s in _active(active_mask, S)}


def useful_flops(S: int, active_mask: int, n_hist: int, T: int, H: int, D: int,
                 hist_first: Optional[Sequence[int]] = None) -> int:
    """Mask-true (query, key) pairs x 4*D flops x H heads (Q K^T plus P V; no
    exponentials counted). Counted from the materialised token mask."""
    pairs = sum(T * n for n in keys_per_stage(S, active_mask, n_hist, T, hist_first).values())
    return 4 * D * H * pairs
