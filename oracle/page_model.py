"""Dict-based page store and FIFO free-list model of the paged clean K/V history.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix ([full text] §4.2, Appendix B.3 and B.8, Eq. (13)):
  * clean history K/V lives in fixed-capacity pages, so storage does not grow
    with video length;
  * the store chunk's K/V is written straight into its final page slots;
  * after the tick the live store page is promoted to retained history (no
    second broadcast), and the bounded window drops the oldest chunk; the
    first clean chunk may be kept as a persistent anchor.

Readings where the pages are silent:
  * a page holds P consecutive tokens of one chunk, all heads: [P][H][D]; a
    chunk owns ceil(T/P) whole pages and the slots past token T-1 of its last
    page are zero, so page contents are fully determined;
  * the free list is FIFO: allocation pops from the front, eviction appends the
    evicted chunk's page ids, in page order, at the back;
  * eviction removes history index 0, or index 1 when the anchor is pinned.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class PageModelError(Exception):
    """Raised with a code name: 'EINVAL', 'ENOMEM' or 'ESTATE'."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


class PageStore:
    """Page id -> (K page, V page), each uint16 [P][H][D] (bf16 bits)."""

    def __init__(self, P: int, H: int, D: int):
        self.P, self.H, self.D = P, H, D
        self.pages: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    def write_chunk(self, ids: Sequence[int], k_tokens: np.ndarray, v_tokens: np.ndarray) -> None:
        """Token t of the chunk goes to slot t % P of page ids[t // P]; unused slots
        of the last page are zero."""
        T = k_tokens.shape[0]
        P = self.P
        if len(ids) != -(-T // P):
            raise PageModelError("EINVAL", "wrong number of page ids for the chunk")
        for pid in ids:
            self.pages[int(pid)] = (np.zeros((P, self.H, self.D), np.uint16),
                                    np.zeros((P, self.H, self.D), np.uint16))
        for t in range(T):
            kp, vp = self.pages[int(ids[t // P])]
            kp[t % P] = k_tokens[t]
            vp[t % P] = v_tokens[t]

    def drop(self, ids: Sequence[int]) -> None:
        """Forget pages returned to the free list (their device bytes are unspecified)."""
        for pid in ids:
            self.pages.pop(int(pid), None)

    def gather(self, page_lists: Sequence[Sequence[int]], T: int) -> Tuple[np.ndarray, np.ndarray]:
        """Logical history K, V [n][T][H][D] (uint16) read token by token through the
        per-chunk page lists."""
        n = len(page_lists)
        K = np.zeros((n, T, self.H, self.D), np.uint16)
        V = np.zeros_like(K)
        for c, ids in enumerate(page_lists):
            for t in range(T):
                kp, vp = self.pages[int(ids[t // self.P])]
                K[c, t] = kp[t % self.P]
                V[c, t] = vp[t % self.P]
        return K, V


class FifoPageModel:
    """Free list + rolling history window of a single request's attention pages."""

    def __init__(self, num_pages: int, page_size: int, chunk_tokens: int, window_chunks: int,
                 pin_anchor: bool = False, initial_free_order: Optional[Sequence[int]] = None):
        if num_pages <= 0 or page_size <= 0 or chunk_tokens <= 0 or window_chunks <= 0:
            raise PageModelError("EINVAL", "sizes must be positive")
        if pin_anchor and window_chunks < 2:
            raise PageModelError("EINVAL", "a pinned anchor needs a window of at least 2")
        order = list(range(num_pages)) if initial_free_order is None else [int(x) for x in initial_free_order]
        if sorted(order) != list(range(num_pages)):
            raise PageModelError("EINVAL", "initial free order must be a permutation")
        self.num_pages = num_pages
        self.P = page_size
        self.T = chunk_tokens
        self.window = window_chunks
        self.pin_anchor = bool(pin_anchor)
        self.ppc = -(-chunk_tokens // page_size)
        self.free = collections.deque(order)
        self.history: List[List[int]] = []
        self.live: Optional[List[int]] = None

    def alloc_chunk(self) -> List[int]:
        """Pages for the store chunk about to be written (the live store)."""
        if self.live is not None:
            raise PageModelError("ESTATE", "a live chunk is already allocated")
        if len(self.free) < self.ppc:
            raise PageModelError("ENOMEM", "free list exhausted")
        self.live = [self.free.popleft() for _ in range(self.ppc)]
        return list(self.live)

    def commit(self) -> List[int]:
        """Promote the live store chunk to history; evict when over the window.
        Returns the evicted page ids (empty if none)."""
        if self.live is None:
            raise PageModelError("ESTATE", "commit without a live chunk")
        self.history.append(self.live)
        self.live = None
        evicted: List[int] = []
        if len(self.history) > self.window:
            idx = 1 if self.pin_anchor else 0
            evicted = self.history.pop(idx)
            self.free.extend(evicted)
        return evicted

    def export(self) -> List[List[int]]:
        """History page lists, oldest chunk first."""
        return [list(c) for c in self.history]

    def num_free(self) -> int:
        return len(self.free)
