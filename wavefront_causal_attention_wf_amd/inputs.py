"""Seeded synthetic inputs for the wave-tick attention path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic, so the CPU oracle (tests only) and the HIP path can both be
fed from it without sharing any computation.

Shapes and value distributions follow the workloads stated for the method:
post-RoPE Q/K/V of one DiT self-attention layer, one chunk of 3 latent frames
x 30 x 52 = 4680 tokens, Wan-1.3B-like 12 heads x 128 or 14B-like 40 heads x
128, bf16 values ~ N(0, 0.5^2). The pages' own efficiency runs use dummy
(random) DiT weights, so random activations stand in for real attention inputs.

Layouts (all C-contiguous):
  live q/k/v : [S+1][T][H][D]   chunk slot s = stage s, slot S = store chunk
  history k/v: [n_hist][T][H][D] oldest chunk first (logical order)
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class TickConfig:
    """One wave-tick workload (a single DiT layer's self-attention)."""

    name: str
    S: int            # denoising stages; chunk slot S is the store chunk
    T: int            # tokens per chunk
    H: int            # heads
    D: int            # head dim
    P: int            # tokens per page
    n_hist: int       # clean history chunks resident in pages
    num_pages: int    # pages in the K pool (and in the V pool)
    std: float        # standard deviation of Q/K/V
    bf16_inputs: bool  # False: fp32 draws (the tiny case); True: bf16 values
    page_order: str   # "identity" or "permutation"
    seed: int = 0         # tensor seed
    seed_pages: int = 1   # free-list permutation seed
    ticks: int = 1        # >1 only for the streaming rollout
    window: int = 0       # rolling history window (rollout); 0 -> n_hist

    @property
    def ppc(self) -> int:
        return -(-self.T // self.P)

    @property
    def history_window(self) -> int:
        return self.window if self.window else self.n_hist


CONFIGS = {
    # Small case the oracle finishes in well under a second.
    "tiny": TickConfig("tiny", S=2, T=64, H=2, D=64, P=16, n_hist=2, num_pages=8,
                       std=1.0, bf16_inputs=False, page_order="identity", seed=0),
    # Wan-1.3B-like single layer, 4-step wavefront (width 5 incl. store).
    "wan13_4step": TickConfig("wan13_4step", S=4, T=4680, H=12, D=128, P=64, n_hist=3,
                              num_pages=4096, std=0.5, bf16_inputs=True,
                              page_order="permutation"),
    # Wan-1.3B-like single layer, 5-step wavefront (width 6), 6 history chunks.
    "wan13_5step": TickConfig("wan13_5step", S=5, T=4680, H=12, D=128, P=64, n_hist=6,
                              num_pages=8192, std=0.5, bf16_inputs=True,
                              page_order="permutation"),
    # 14B-like single layer (40 heads), 4-step wavefront.
    "wan14b_4step": TickConfig("wan14b_4step", S=4, T=4680, H=40, D=128, P=64, n_hist=3,
                               num_pages=4096, std=0.5, bf16_inputs=True,
                               page_order="permutation"),
    # 120 consecutive ticks at the Wan-1.3B-like shape, rolling window of 3.
    "rollout120": TickConfig("rollout120", S=4, T=4680, H=12, D=128, P=64, n_hist=3,
                             num_pages=4096, std=0.5, bf16_inputs=True,
                             page_order="permutation", ticks=120, window=3),
}


# Latent grid of one chunk (frames, rows, columns): 3 latent frames of a 60 x 104
# latent patchified 2 x 2, i.e. 30 x 52 tokens per frame, 4680 tokens per chunk.
WAN_CHUNK_GRID = (3, 30, 52)


def chunk_grid(T: int) -> tuple:
    """Latent grid of a T-token chunk: the Wan chunk grid at T = 4680, else T
    frames of a single token (a grid only the rotary embedding reads)."""
    if T == 4680:
        return WAN_CHUNK_GRID
    return (T, 1, 1)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return the uint16 bits.

    Input preparation only: the draws are finite, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def initial_free_order(cfg: TickConfig) -> np.ndarray:
    """Initial order of the page free list: identity, or a seeded permutation."""
    if cfg.page_order == "identity":
        return np.arange(cfg.num_pages, dtype=np.int32)
    rng = np.random.default_rng(cfg.seed_pages)
    return rng.permutation(cfg.num_pages).astype(np.int32)


@dataclasses.dataclass
class TickInputs:
    """Host copies of one tick's inputs.

    *_f32 hold the raw fp32 draws (only for the tiny fp32 case); *_bits hold the
    bf16 bit patterns the GPU path consumes (uint16, same layout).
    """

    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    hist_k_bits: np.ndarray
    hist_v_bits: np.ndarray
    q_f32: Optional[np.ndarray] = None
    k_f32: Optional[np.ndarray] = None
    v_f32: Optional[np.ndarray] = None
    hist_k_f32: Optional[np.ndarray] = None
    hist_v_f32: Optional[np.ndarray] = None


def draw_tick(cfg: TickConfig, seed: Optional[int] = None, n_hist: Optional[int] = None,
              T: Optional[int] = None) -> TickInputs:
    """Draw one tick's Q/K/V (live chunks) and history K/V.

    numpy PCG64 seeded with `seed` (default cfg.seed); draws in the order live q,
    live k, live v, history k, history v, each float32 N(0, std^2).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    S, H, D = cfg.S, cfg.H, cfg.D
    T = cfg.T if T is None else T
    nh = cfg.n_hist if n_hist is None else n_hist
    live = (S + 1, T, H, D)
    hist = (nh, T, H, D)

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if cfg.std != 1.0:
            x *= np.float32(cfg.std)
        return x

    q, k, v = draw(live), draw(live), draw(live)
    hk, hv = draw(hist), draw(hist)
    out = TickInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v),
                     f32_to_bf16_bits(hk), f32_to_bf16_bits(hv))
    if not cfg.bf16_inputs:
        out.q_f32, out.k_f32, out.v_f32, out.hist_k_f32, out.hist_v_f32 = q, k, v, hk, hv
    return out


def draw_live(cfg: TickConfig, seed: int) -> tuple:
    """Draw only the live q, k, v of one rollout tick (bf16 bits)."""
    rng = np.random.default_rng(seed)
    shape = (cfg.S + 1, cfg.T, cfg.H, cfg.D)
    out = []
    for _ in range(3):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.float32(cfg.std)
        out.append(f32_to_bf16_bits(x))
    return tuple(out)


def rollout_seed(k: int) -> int:
    """Seed of rollout tick k's live Q/K/V."""
    return 1000 + k


def draw_live_torch(cfg: TickConfig, seed: int, device, T: Optional[int] = None):
    """Live q, k, v of one tick drawn on the device with torch's seeded generator:
    bf16 [S+1][T][H][D] ~ N(0, std^2) (normal in fp32, then rounded to bf16).

    Used where hundreds of ticks are needed (streaming rollout, timing); any
    oracle check on these inputs reads host copies of the same tensors.
    """
    import torch

    T = cfg.T if T is None else T
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (cfg.S + 1, T, cfg.H, cfg.D)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(cfg.std)
        out.append(x.to(torch.bfloat16))
    return tuple(out)


def to_device_bf16(bits: np.ndarray, device):
    """uint16 bf16 bit patterns -> torch bfloat16 tensor on `device` (bit copy)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_tensor_bits(t) -> np.ndarray:
    """torch bfloat16 tensor -> host uint16 bit patterns (bit copy)."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
