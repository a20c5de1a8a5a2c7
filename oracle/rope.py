"""Rotary position embedding of a chunk's keys, and the anchor's re-rotation.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Plain numpy float64.

Citations name pages of "Wave Forcing: Towards Speed-of-Light Streaming Video
Generation": [summary] = the structured summary page, [full text] = the
full-text page, with section.

What the pages fix:
  * K/V are published after the QKV projection and RoPE, so the attention pages
    hold rotated keys ([summary] Methodology 3; [full text] Appendix B.1);
  * the two K/V arrays hold the anchor, the bounded history, the live store and
    at most S denoising chunks ([full text] Appendix B.8, Eq. (13)): live chunks
    are paged too;
  * the first clean chunk is a persistent anchor whose unrotated key is kept so
    that RoPE can be applied again when the bounded window shifts; every other
    page keeps the rotated keys it was written with ([full text] Appendix B.3).

Readings where the pages are silent:
  * rotary form: channel pair (2i, 2i+1) of a head vector is turned by the
    angle a = coordinate * frequency: (x0, x1) -> (x0 cos a - x1 sin a,
    x0 sin a + x1 cos a);
  * axes: a chunk is a latent grid of F frames x R rows x C columns with tokens
    in row-major (frame, row, column) order; the head dim is cut into three
    contiguous channel groups of d_f, d_r, d_c channels (each even), turned by
    the frame, row and column coordinate; pair i of a group of d channels has
    frequency theta^(-2i/d), theta = 10000. Default split: d_r = d_c =
    2*floor(D/6), d_f = D - 2*d_r (44/42/42 at D = 128, 24/20/20 at D = 64);
  * frame coordinates are absolute in the video: a chunk starting at latent
    frame f0 has frame coordinates f0 .. f0 + F - 1;
  * after a window shift the anchor takes the F frames just before the oldest
    retained non-anchor chunk.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

DEFAULT_THETA = 10000.0


def default_split(D: int) -> Tuple[int, int, int]:
    """Channels per axis (frame, row, column) for head dim D."""
    d_rc = 2 * (D // 6)
    return D - 2 * d_rc, d_rc, d_rc


def token_coords(T: int, grid: Sequence[int], frame0: int) -> np.ndarray:
    """int64 [T][3]: (frame, row, column) of each token of a chunk whose latent
    grid is grid = (F, R, C) with F*R*C = T, first frame at frame0."""
    F, R, C = (int(g) for g in grid)
    if F * R * C != T:
        raise ValueError(f"grid {grid} does not hold {T} tokens")
    t = np.arange(T, dtype=np.int64)
    return np.stack([frame0 + t // (R * C), (t // C) % R, t % C], axis=1)


def pair_axis_and_frequency(D: int, split: Sequence[int], theta: float
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """For each of the D/2 channel pairs: the axis (0 frame, 1 row, 2 column) whose
    coordinate turns it, and its frequency theta^(-2i/d) (i = pair index within
    the axis group of d channels)."""
    if sum(split) != D or any(d < 0 or d % 2 for d in split):
        raise ValueError(f"split {split} is not three even parts of {D}")
    axis, freq = [], []
    for a, d in enumerate(split):
        for i in range(d // 2):
            axis.append(a)
            freq.append(float(theta) ** (-2.0 * i / d))
    return np.array(axis, dtype=np.int64), np.array(freq, dtype=np.float64)


def rope_angles(T: int, D: int, grid: Sequence[int], frame0: int,
                split: Optional[Sequence[int]] = None, theta: float = DEFAULT_THETA) -> np.ndarray:
    """float64 [T][D/2]: the angle of every channel pair of every token."""
    split = default_split(D) if split is None else tuple(split)
    axis, freq = pair_axis_and_frequency(D, split, theta)
    coords = token_coords(T, grid, frame0).astype(np.float64)
    return coords[:, axis] * freq[None, :]


def rope(x, grid: Sequence[int], frame0: int, split: Optional[Sequence[int]] = None,
         theta: float = DEFAULT_THETA) -> np.ndarray:
    """Rotated keys, float64 [T][H][D]; x is [T][H][D] (uint16 = bf16 bits, or
    values). Every head of a token gets the same rotation."""
    from .wave_attention import as_f64

    v = as_f64(x)
    T, H, D = v.shape
    ang = rope_angles(T, D, grid, frame0, split, theta)[:, None, :]   # [T][1][D/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def anchor_frame0(oldest_retained_chunk: int, frames_per_chunk: int) -> int:
    """First frame of the anchor after a window shift: the F frames just before
    the oldest retained non-anchor chunk (chunk c covers frames c*F ..)."""
    return (int(oldest_retained_chunk) - 1) * int(frames_per_chunk)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), rounded once to nearest, ties to even
    (no intermediate rounding to float32). Magnitudes past the bf16 range
    become +-inf, as in an IEEE conversion."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    out[~fin] = x[~fin]
    xf = x[fin]
    _, e = np.frexp(xf)               # xf = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)           # below 2^-126: fixed quantum 2^-133 (subnormals)
    quantum = np.ldexp(1.0, e - 8)    # 8 significant bits
    out[fin] = np.round(xf / quantum) * quantum   # np.round: ties to even
    f32 = out.astype(np.float32)      # exact: every rounded value is a float32
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
