"""8-bit (e4m3) keys and queries for the FP8 attention tier.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). numpy, with the
quantisation decisions taken in float32 exactly as stated below.

The pages name K/V quantisation as a way to shrink K/V payloads and an 8-bit
attention backend (SageAttention) for local computation ([full text] §4.3,
§5 "Compute configurations"), and measure FP8 K/V collectives at about half
the bf16 time (Appendix C.5, Table 8; C.6). They give neither the 8-bit
format nor the quantisation granularity. Readings taken here:
  * format: e4m3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    no infinities; largest finite value 448; exponent field 0 holds the
    subnormals m * 2^-9);
  * what is 8-bit: Q and K, the operands of Q.K^T (the SageAttention-like
    tier); P and V stay 16-bit, since e4m3 P would carry ~6 % per-element error;
  * scales: one float32 scale per (64-token tile, head) for K and per (query
    row, head) for Q: amax = max |x| over the group (float32, exact for bf16
    inputs), scale = amax / 448, inv = 448 / amax (both float32 divisions;
    inv = scale = 0 for an all-zero group, and for a group with amax below
    2^-100, TINY_AMAX), code = e4m3 of float32(x * inv)
    rounded to nearest, ties to even; the value a code stands for is
    decode(code) * scale;
  * scores are the products of the dequantised Q and K; everything after the
    scores is the bf16 tier's plain masked softmax attention.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

E4M3_MAX = 448.0
# Groups of queries or keys whose amax lies below 2^-100 are stored as zero
# (scale 0, zero codes). Below about 2^-119, 448 / amax would exceed the largest
# float32, and between the two the scale amax / 448 would fall among float32's
# subnormals; the values such a group carries are below 2^-100 in any case.
TINY_AMAX = 2.0 ** -100
# The exponent of a power-of-two value scale is an E8M0 byte (e + 127), so
# e >= -127; tiles with amax below 448 * 2^-128 take e = -127 and are still
# scaled exactly (their codes are e4m3 of v * 2^127, below 448).
E8M0_MIN = -127


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3 codes -> float64 values (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float values (|x| <= 464) -> e4m3 codes, rounded to nearest, ties to even
    (each value is taken exactly as given; callers pass float32 results)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > 464.0) or np.any(np.isnan(x)):
        raise ValueError("value outside the e4m3 range")
    sign = np.signbit(x)
    a = np.abs(x)
    # quantum of the binade holding a (subnormal quantum 2^-9 below 2^-6)
    _, ex = np.frexp(a)                     # a = f * 2^ex, 0.5 <= f < 1
    ex = np.maximum(ex, -5)                 # 2^-6 and below: fixed quantum
    q = np.ldexp(1.0, ex - 4)               # 3 mantissa bits -> 4 significant bits
    r = np.round(a / q) * q                 # ties to even
    r = np.minimum(r, E4M3_MAX)             # 464 / q would be 448 + half a quantum
    # code from the rounded value
    codes = np.zeros(a.shape, dtype=np.int64)
    nz = r > 0
    _, e2 = np.frexp(r[nz])
    ee = e2 - 1 + 7                         # biased exponent of r = 1.m * 2^(e2-1)
    sub = ee <= 0
    mant = np.where(sub, np.round(r[nz] / 2.0 ** -9),
                    np.round((r[nz] / np.exp2(e2 - 1.0) - 1.0) * 8.0))
    codes[nz] = np.where(sub, mant, (ee << 3) | mant.astype(np.int64))
    codes = codes | np.where(sign, 0x80, 0)  # negative values keep their sign, zero too
    return codes.astype(np.uint8)


def quantize_groups(x: np.ndarray, axes) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise x (values; bf16 bit patterns must be decoded first) with one
    scale per group, reducing over `axes` (the other axes index the groups).
    Returns (codes uint8 like x, scales float32 with the reduced axes kept as 1).
    A group whose amax is below TINY_AMAX is stored as all-zero (scale 0, zero
    codes), as a group of zeros is."""
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=axes, keepdims=True).astype(np.float32)
    big = amax >= np.float32(TINY_AMAX)
    safe = np.where(big, amax, np.float32(1))
    scale = np.where(big, amax / np.float32(E4M3_MAX), np.float32(0)).astype(np.float32)
    inv = np.where(big, np.float32(E4M3_MAX) / safe, np.float32(0)).astype(np.float32)
    y = (xf * inv).astype(np.float32)       # float32 product, rounded once
    return e4m3_encode(y), scale


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * scale.astype(np.float64)


def quantize_k_tiles(k_bits_or_vals: np.ndarray, tile: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Keys [T][H][D] of one chunk -> (codes [T][H][D], scales [ceil(T/tile)][H]):
    one scale per (64-token tile, head); tokens past T do not exist (a short
    last tile takes its amax over its own tokens)."""
    from .wave_attention import as_f64

    k = as_f64(k_bits_or_vals).astype(np.float32)
    T, H, D = k.shape
    nt = -(-T // tile)
    codes = np.zeros((T, H, D), np.uint8)
    scales = np.zeros((nt, H), np.float32)
    for t in range(nt):
        blk = k[t * tile:(t + 1) * tile]                      # [n][H][D]
        c, s = quantize_groups(blk, axes=(0, 2))              # scale per head
        codes[t * tile:(t + 1) * tile] = c
        scales[t] = s[0, :, 0]
    return codes, scales


def quantize_q_rows(q_bits_or_vals: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Queries [..., D] -> (codes, scales [...]): one scale per (row, head)."""
    from .wave_attention import as_f64

    q = as_f64(q_bits_or_vals).astype(np.float32)
    c, s = quantize_groups(q, axes=-1)
    return c, s[..., 0]


class Fp8PageStore:
    """Page id -> (K codes uint8 [P][H][D], K scales float32 [P/64][H], V bf16
    bits uint16 [P][H][D]): the history pages of the 8-bit tier. A chunk's keys
    are quantised per (64-token tile, head) of the chunk (quantize_k_tiles), so
    P must be a multiple of 64 and every scale covers 64 tokens of one page;
    unused slots of the last page hold zero codes, and a scale slot past the
    chunk's last tile holds 0."""

    def __init__(self, P: int, H: int, D: int, tile: int = 64):
        if P % tile:
            raise ValueError("page size must be a multiple of the scale tile")
        self.P, self.H, self.D, self.tile = P, H, D, tile
        self.pages = {}

    def write_chunk(self, ids, k_bits, v_bits) -> None:
        T = k_bits.shape[0]
        P, tile = self.P, self.tile
        if len(ids) != -(-T // P):
            raise ValueError("wrong number of page ids for the chunk")
        codes, scales = quantize_k_tiles(k_bits, tile)
        for n, pid in enumerate(ids):
            kc = np.zeros((P, self.H, self.D), np.uint8)
            ks = np.zeros((P // tile, self.H), np.float32)
            vb = np.zeros((P, self.H, self.D), np.uint16)
            t0, t1 = n * P, min(T, (n + 1) * P)
            kc[:t1 - t0] = codes[t0:t1]
            vb[:t1 - t0] = v_bits[t0:t1]
            nt = -(-(t1 - t0) // tile)
            ks[:nt] = scales[t0 // tile:t0 // tile + nt]
            self.pages[int(pid)] = (kc, ks, vb)

    def drop(self, ids) -> None:
        for pid in ids:
            self.pages.pop(int(pid), None)

    def gather(self, page_lists, T: int):
        """Dequantised K (float64) and V bits (uint16), [n][T][H][D], read token by
        token through the per-chunk page lists."""
        n = len(page_lists)
        K = np.zeros((n, T, self.H, self.D), np.float64)
        V = np.zeros((n, T, self.H, self.D), np.uint16)
        for c, ids in enumerate(page_lists):
            for t in range(T):
                kc, ks, vb = self.pages[int(ids[t // self.P])]
                slot = t % self.P
                K[c, t] = e4m3_decode(kc[slot]) * ks[slot // self.tile][:, None].astype(np.float64)
                V[c, t] = vb[slot]
        return K, V


def attention_tick_fp8(q_bits, store: "Fp8PageStore", hist_pages, live_pages, S: int,
                       active_mask: int, scale: float, **kw):
    """One tick of the 8-bit tier, every key read through the 8-bit pages
    (the fully paged context of the bf16 tier): each query row is quantised
    with its own scale (quantize_q_rows), keys and values are the pages'
    dequantised values, and the attention itself is the plain masked softmax
    of attention_tick over those values."""
    from .wave_attention import attention_tick

    T, H, D = q_bits.shape[1], q_bits.shape[2], q_bits.shape[3]
    rows = kw.get("rows")
    if rows is None:
        qc, qs = quantize_q_rows(q_bits)
        qv = e4m3_decode(qc) * qs[..., None].astype(np.float64)
    else:  # each row is quantised on its own: only the requested rows are needed
        rows = np.asarray(rows)
        qc, qs = quantize_q_rows(q_bits[:, rows])
        qv = np.zeros(q_bits.shape, np.float64)
        qv[:, rows] = e4m3_decode(qc) * qs[..., None].astype(np.float64)
    hk, hv = store.gather(hist_pages, T)
    lk = np.zeros((S + 1, T, H, D), np.float64)
    lv = np.zeros((S + 1, T, H, D), hv.dtype)   # bf16 bits, or dequantised values
    for j in range(S + 1):
        if (active_mask >> j) & 1:
            if live_pages[j] is None:
                raise ValueError(f"active slot {j} has no pages")
            kk, vv = store.gather([live_pages[j]], T)
            lk[j], lv[j] = kk[0], vv[0]
    from .wave_attention import as_f64
    return attention_tick(qv, lk, as_f64(lv), hk, as_f64(hv), S, active_mask, scale, **kw)


# ----------------------------------------------------------------------------
# 8-bit values (the tier where V is e4m3 too)
# ----------------------------------------------------------------------------
# Reading: V is quantised per (64-token tile, head) with a
# power-of-two scale 2^e, e the smallest integer with amax <= 448 * 2^e (so the
# scale is an 8-bit exponent and the codes are e4m3 of v * 2^-e, a product
# that is exact in float32), e = 0 for an all-zero tile. P is rounded to e4m3
# (the device keeps every P at most 448) for the P.V product; that rounding
# depends on the device's running reference, so the tick is checked against the
# exact attention of the dequantised values: element by element within the
# worst-case bound p_error_bound() gives, and per (stage, head) in the rel-L2
# sense within kv8_l2_allowance() of the RMS term p_rounding_rms() gives.


def pow2_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (amax > 0), else 0.
    amax = f * 2^E with 0.5 <= f < 1 and 448 = 0.875 * 2^9, so e = E - 9 when
    f <= 0.875 and E - 8 otherwise; -127 is the smallest exponent the E8M0
    scale byte holds."""
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)
    e = np.maximum(np.where(f <= 0.875, E - 9, E - 8), E8M0_MIN)
    return np.where(amax > 0, e, 0).astype(np.int64)


def quantize_v_tiles(v_bits_or_vals: np.ndarray, tile: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Values [T][H][D] of one chunk -> (codes [T][H][D], exponents [ceil(T/tile)][H]):
    codes = e4m3 of v * 2^-e per (64-token tile, head)."""
    from .wave_attention import as_f64

    v = as_f64(v_bits_or_vals).astype(np.float32)
    T, H, D = v.shape
    nt = -(-T // tile)
    codes = np.zeros((T, H, D), np.uint8)
    exps = np.zeros((nt, H), np.int64)
    for t in range(nt):
        blk = v[t * tile:(t + 1) * tile]
        amax = np.abs(blk).max(axis=(0, 2)).astype(np.float32)       # [H]
        e = pow2_exponent(amax)
        exps[t] = e
        y = blk.astype(np.float64) * np.exp2(-e)[None, :, None]        # exact (power of two)
        codes[t * tile:(t + 1) * tile] = e4m3_encode(y)
    return codes, exps


class Fp8KvPageStore(Fp8PageStore):
    """The 8-bit page store with V in e4m3 as well: page id -> (K codes, K scales,
    V codes uint8 [P][H][D], V exponents int [P/64][H])."""

    def write_chunk(self, ids, k_bits, v_bits) -> None:
        T = k_bits.shape[0]
        P, tile = self.P, self.tile
        if len(ids) != -(-T // P):
            raise ValueError("wrong number of page ids for the chunk")
        kc_all, ks_all = quantize_k_tiles(k_bits, tile)
        vc_all, ve_all = quantize_v_tiles(v_bits, tile)
        for n, pid in enumerate(ids):
            kc = np.zeros((P, self.H, self.D), np.uint8)
            ks = np.zeros((P // tile, self.H), np.float32)
            vc = np.zeros((P, self.H, self.D), np.uint8)
            ve = np.zeros((P // tile, self.H), np.int64)
            t0, t1 = n * P, min(T, (n + 1) * P)
            kc[:t1 - t0] = kc_all[t0:t1]
            vc[:t1 - t0] = vc_all[t0:t1]
            nt = -(-(t1 - t0) // tile)
            ks[:nt] = ks_all[t0 // tile:t0 // tile + nt]
            ve[:nt] = ve_all[t0 // tile:t0 // tile + nt]
            self.pages[int(pid)] = (kc, ks, vc, ve)

    def gather(self, page_lists, T: int):
        """Dequantised K and V (float64), [n][T][H][D]."""
        n = len(page_lists)
        K = np.zeros((n, T, self.H, self.D), np.float64)
        V = np.zeros((n, T, self.H, self.D), np.float64)
        for c, ids in enumerate(page_lists):
            for t in range(T):
                kc, ks, vc, ve = self.pages[int(ids[t // self.P])]
                slot = t % self.P
                K[c, t] = e4m3_decode(kc[slot]) * ks[slot // self.tile][:, None].astype(np.float64)
                V[c, t] = e4m3_decode(vc[slot]) * np.exp2(ve[slot // self.tile])[:, None]
        return K, V


def attention_tick_fp8kv(q_bits, store: "Fp8KvPageStore", hist_pages, live_pages, S: int,
                         active_mask: int, scale: float, **kw):
    """The tick of the 8-bit K/V tier over the dequantised Q, K and V (exact
    softmax, float64): what the device approximates up to its e4m3 rounding of
    P, bounded by p_error_bound()."""
    return attention_tick_fp8(q_bits, store, hist_pages, live_pages, S, active_mask, scale, **kw)


def _p_rounding_inputs(q_bits, store: "Fp8KvPageStore", hist_pages, live_pages, S: int,
                       active_mask: int, scale: float, stages, heads, rows):
    """For each requested (stage, head): the exact softmax weights P of the
    dequantised tick relative to each row's max (max P = 1) over the stage's
    visible keys, and those keys' dequantised values. Yields (s, hi, P, V)."""
    from .wave_attention import _active, token_mask, _key_matrix

    T, H, D = q_bits.shape[1], q_bits.shape[2], q_bits.shape[3]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    qc, qs = quantize_q_rows(q_bits[:, rows])     # each row is quantised on its own
    qv = e4m3_decode(qc) * qs[..., None].astype(np.float64)
    hk, hv = store.gather(hist_pages, T)
    lk = np.zeros((S + 1, T, H, D))
    lv = np.zeros((S + 1, T, H, D))
    for j in range(S + 1):
        if (active_mask >> j) & 1:
            kk, vv = store.gather([live_pages[j]], T)
            lk[j], lv[j] = kk[0], vv[0]
    act = _active(active_mask, S)
    stages = act if stages is None else [s for s in stages if s in act]
    heads = list(range(H)) if heads is None else list(heads)
    n_hist = hk.shape[0]
    for s in stages:
        m = token_mask(s, S, active_mask, n_hist, T, 0)
        for hi, h in enumerate(heads):
            K = _key_matrix(lk, hk, h, S)[m]
            V = _key_matrix(lv, hv, h, S)[m]                               # [keys][D]
            sc = (qv[s, :, h, :] @ K.T) * scale
            yield s, hi, np.exp(sc - sc.max(axis=1, keepdims=True)), V


def _p_rounding_weights(p: np.ndarray) -> np.ndarray:
    """Largest change of each P (relative to its row's max) when the device
    rounds it to e4m3 at a reference at or below the row max: the device holds
    P * 2^a with a >= 0 (its reference is a below the max) and every such value
    at most 448, inside e4m3's range; a normal e4m3 value (at least 2^-6) is
    within half a quantum, 2^-4 of itself, of the value it rounds, a subnormal
    one within 2^-10 absolutely, i.e. 2^-10 * 2^-a <= 2^-10 relative to the max."""
    return np.maximum(2.0 ** -4 * p, 2.0 ** -10)


def p_error_bound(q_bits, store: "Fp8KvPageStore", hist_pages, live_pages, S: int,
                  active_mask: int, scale: float, stages=None, heads=None, rows=None):
    """Per (stage, row, head) worst-case bound on |O_device - O_exact| from
    rounding P to e4m3 alone, for any reference the device may take at or below
    the row max with every P at most 448 (_p_rounding_weights): each P moves by
    at most w(P) = max(2^-4 P, 2^-10), so the output, a P-weighted mean with the
    exact sum of P as divisor, moves by at most sum(w(P) |v|) / sum(P) in every
    channel. Returns {stage: [rows][heads]} (the worst channel of each row).

    The bound assumes every rounding errs the same way; for near-uniform rows
    over thousands of keys it exceeds the outputs themselves, so on its own it
    cannot tell a wrong output from a right one there (p_rounding_rms can)."""
    return p_rounding_terms(q_bits, store, hist_pages, live_pages, S, active_mask, scale,
                            stages, heads, rows)[0]


# Rel-L2 criterion of the 8-bit K/V tick (per stage and head). The device
# output differs from the exact attention of the dequantised values by
#   E = sum_k d_k v_k / sum_k P_k   (d_k: the e4m3 rounding error of P_k)
# plus bf16 output rounding. Over the many (row, channel) elements of one
# (stage, head) the roundings of different P act as independent errors of
# mean near zero, so the squared norm of E concentrates near
#   sum_rows sum_d sum_k var(d_k) v_kd^2 / (sum_k P_k)^2 .
# Rounding to nearest gives |d_k| <= w(P_k) (_p_rounding_weights), hence
# var(d_k) <= w(P_k)^2: R^2 = sum_rows sum_d sum_k w(P_k)^2 v_kd^2 / L^2 bounds
# that expectation (for a uniformly placed value within its quantum, var =
# quantum^2 / 12 <= w^2 / 3, so R is at least 1.7x the expected norm), and the
# criterion allows twice R. What is not independent — the small bias of
# rounding values spread over a binade (at most ~(quantum / value)^2 / 12 <=
# 2^-8 / 12 relative) and the bf16 rounding of the output (at most 2^-9
# relative) — is a fraction of the output itself: 2^-8 of its norm covers both.
# When one key dominates a row, E is that key's rounding error alone, at most
# w(P) |v|, which the same 2 R covers with room to spare.
KV8_RMS_FACTOR = 2.0
KV8_REL_SLACK = 2.0 ** -8


def p_rounding_rms(q_bits, store: "Fp8KvPageStore", hist_pages, live_pages, S: int,
                   active_mask: int, scale: float, stages=None, heads=None, rows=None):
    """R per (stage, head) over the given rows (see the criterion above):
    sqrt(sum over rows and channels of sum_k w(P_k)^2 v_kd^2 / (sum_k P_k)^2).
    Returns {stage: [heads]}."""
    return p_rounding_terms(q_bits, store, hist_pages, live_pages, S, active_mask, scale,
                            stages, heads, rows)[1]


def p_rounding_terms(q_bits, store: "Fp8KvPageStore", hist_pages, live_pages, S: int,
                     active_mask: int, scale: float, stages=None, heads=None, rows=None):
    """(p_error_bound(...), p_rounding_rms(...)) from one pass over the tick."""
    T, H = q_bits.shape[1], q_bits.shape[2]
    n_rows = T if rows is None else len(rows)
    n_heads = H if heads is None else len(list(heads))
    bound, rms = {}, {}
    for s, hi, p, V in _p_rounding_inputs(q_bits, store, hist_pages, live_pages, S, active_mask,
                                         scale, stages, heads, rows):
        if s not in bound:
            bound[s] = np.zeros((n_rows, n_heads))
            rms[s] = np.zeros(n_heads)
        w = _p_rounding_weights(p)
        L = p.sum(axis=1, keepdims=True)
        bound[s][:, hi] = ((w @ np.abs(V)) / L).max(axis=1)
        rms[s][hi] = np.sqrt(float((((w * w) @ (V * V)) / (L * L)).sum()))
    return bound, rms


def kv8_l2_allowance(rms: float, exact_norm: float) -> float:
    """The largest ||O_device - O_exact|| (Frobenius norm over one stage and head)
    the 8-bit K/V tick may show: KV8_RMS_FACTOR * R + KV8_REL_SLACK * ||O_exact||."""
    return KV8_RMS_FACTOR * rms + KV8_REL_SLACK * exact_norm
