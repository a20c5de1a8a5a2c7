"""Brute-force wave-tick attention in pure Python (tiny shapes only).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Independent of wave_attention.py: no mask matrix, no page store, no numpy
arithmetic. For each query it lists the visible keys directly from the rule
([summary] "Introduction and Theoretical Foundation": a chunk sees itself in
full, cached clean history, and live chunks at cleaner stages j >= s, never
later noisier ones; [full text] Appendix B.3: the store sees anchor, retained
history and itself) and forms sum_i e^{z_i} v_i / sum_i e^{z_i} with math.fsum.
"""
from __future__ import annotations

import math
import struct
from typing import Dict, List, Optional, Sequence

import numpy as np


def _val(x) -> float:
    """A bf16 bit pattern (numpy uint16 scalar) or a float, as a Python float."""
    if isinstance(x, np.uint16):
        return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]
    return float(x)


def _to_lists(a: np.ndarray):
    if a.dtype == np.uint16:
        flat = [_val(np.uint16(b)) for b in a.reshape(-1).tolist()]
        return np.array(flat, dtype=object).reshape(a.shape).tolist()
    return a.astype(float).tolist()


def brute_force_tick(q, k, v, hist_k, hist_v, S: int, active_mask: int, scale: float,
                     hist_first: Optional[Sequence[int]] = None) -> Dict[int, List]:
    """{stage s: nested list [T][H][D]} for every active stage."""
    Q, K, V = _to_lists(q), _to_lists(k), _to_lists(v)
    HK, HV = _to_lists(hist_k), _to_lists(hist_v)
    T, H, D = len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    n_hist = len(HK)
    live_stages = [s for s in range(S + 1) if (active_mask >> s) & 1]
    out: Dict[int, List] = {}
    for s in live_stages:
        first = 0 if hist_first is None else hist_first[s]
        # visible (key vector, value vector) sources, by the rule
        sources = []
        for c in range(first, n_hist):
            sources.append((HK[c], HV[c]))
        if s == S:
            sources.append((K[S], V[S]))              # the store sees only itself live
        else:
            if S in live_stages:
                sources.append((K[S], V[S]))          # live store is cleaner than any stage
            for j in live_stages:
                if s <= j < S:
                    sources.append((K[j], V[j]))      # itself and cleaner chunks
        res = []
        for t in range(T):
            per_head = []
            for h in range(H):
                qv = Q[s][t][h]
                zs, vs = [], []
                for (kc, vc) in sources:
                    for u in range(T):
                        zs.append(scale * math.fsum(qv[d] * kc[u][h][d] for d in range(D)))
                        vs.append(vc[u][h])
                zmax = max(zs)
                w = [math.exp(z - zmax) for z in zs]
                den = math.fsum(w)
                per_head.append([math.fsum(w[i] * vs[i][d] for i in range(len(w))) / den
                                 for d in range(D)])
            res.append(per_head)
        out[s] = res
    return out
