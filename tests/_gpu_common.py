"""Shared set-up for the GPU parity tests: one tick on the device through the
C ABI, and the same tick in the CPU oracle, fed from the same seeded inputs."""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import oracle
from wavefront_causal_attention_wf_amd import inputs
from wavefront_causal_attention_wf_amd import wfattn

DEV = "cuda:0"
ATOL = 2e-2        # max-abs bound on bf16 outputs
REL_L2 = 5e-3      # rel-L2 bound, checked per (stage, head)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Tick:
    S: int
    T: int
    H: int
    D: int
    P: int
    n_hist: int
    num_pages: int
    scale: float
    active_mask: int
    hist_first: Optional[Sequence[int]]
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    o: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    hist_pages: torch.Tensor
    hist_ids: np.ndarray
    store: oracle.PageStore


def setup_tick(S, T, H, D, P, n_hist, num_pages, *, seed=0, page_seed=1, qscale=1.0, std=0.5,
               active_mask=None, hist_first=None, poison_pool=True, order=None,
               tick_inputs: Optional[inputs.TickInputs] = None) -> Tick:
    """Draw inputs, write the history through wf_store_paged into a (NaN-poisoned)
    pool using the C page table, mirror every step in the oracle's page model."""
    cfg = inputs.TickConfig("t", S=S, T=T, H=H, D=D, P=P, n_hist=n_hist, num_pages=num_pages,
                            std=std, bf16_inputs=True, page_order="permutation", seed=seed,
                            seed_pages=page_seed)
    x = tick_inputs or inputs.draw_tick(cfg)
    q_bits = x.q_bits
    if qscale != 1.0:
        q_bits = inputs.f32_to_bf16_bits(
            oracle.decode_bf16(x.q_bits).astype(np.float32) * np.float32(qscale))
    if order is None:
        order = inputs.initial_free_order(cfg)
    window = max(n_hist, 1)
    pt = wfattn.PageTable(num_pages, P, T, window, initial_free_order=order)
    model = oracle.FifoPageModel(num_pages, P, T, window, initial_free_order=order)
    store = oracle.PageStore(P, H, D)
    fill = float("nan") if poison_pool else 0.0
    k_pool = torch.full((num_pages, P, H, D), fill, dtype=torch.bfloat16, device=DEV)
    v_pool = torch.full((num_pages, P, H, D), fill, dtype=torch.bfloat16, device=DEV)
    hk = inputs.to_device_bf16(x.hist_k_bits, DEV)
    hv = inputs.to_device_bf16(x.hist_v_bits, DEV)
    for c in range(n_hist):
        ids = pt.alloc_chunk()
        ids_m = model.alloc_chunk()
        assert list(ids) == ids_m
        wfattn.wf_store_paged(hk[c], hv[c], k_pool, v_pool, torch.from_numpy(ids).to(DEV))
        store.write_chunk(ids_m, x.hist_k_bits[c], x.hist_v_bits[c])
        pt.commit()
        model.commit()
    hist = pt.export()
    assert hist.tolist() == model.export()
    hist_dev = torch.from_numpy(np.ascontiguousarray(hist)).to(DEV)
    q = inputs.to_device_bf16(q_bits, DEV)
    k = inputs.to_device_bf16(x.k_bits, DEV)
    v = inputs.to_device_bf16(x.v_bits, DEV)
    o = torch.full_like(q, float("nan"))
    mask = (1 << (S + 1)) - 1 if active_mask is None else active_mask
    return Tick(S, T, H, D, P, n_hist, num_pages, 1.0 / np.sqrt(D), mask, hist_first,
                q_bits, x.k_bits, x.v_bits, q, k, v, o, k_pool, v_pool, hist_dev,
                np.asarray(hist), store)


def workspace_for(t: Tick) -> Optional[torch.Tensor]:
    """A workspace of the size wf_tick_workspace_bytes asks for this tick
    (None where the tick takes none)."""
    nb = wfattn.workspace_bytes(t.S, t.active_mask, t.T, t.H, t.D, t.n_hist, t.hist_first, t.P,
                                t.num_pages)
    return None if nb == 0 else torch.empty(nb, dtype=torch.uint8, device=DEV)


def run_tick(t: Tick, q=None, k=None, v=None, o=None, hist_pages=None, k_pool=None,
             v_pool=None, workspace=None) -> torch.Tensor:
    o = t.o if o is None else o
    wfattn.wf_attn_tick(t.q if q is None else q, t.k if k is None else k,
                        t.v if v is None else v, o, t.S, t.active_mask, t.scale,
                        t.k_pool if k_pool is None else k_pool,
                        t.v_pool if v_pool is None else v_pool,
                        t.hist_pages if hist_pages is None else hist_pages, t.hist_first,
                        workspace=workspace)
    torch.cuda.synchronize()
    return o


def oracle_tick(t: Tick, stages=None, heads=None, rows=None) -> Dict[int, np.ndarray]:
    return oracle.attention_tick_paged(t.q_bits, t.k_bits, t.v_bits, t.store,
                                       t.hist_ids.tolist(), t.S, t.active_mask, t.scale,
                                       hist_first=t.hist_first, stages=stages, heads=heads,
                                       rows=rows)


def compare(got_o: torch.Tensor, want: Dict[int, np.ndarray], heads=None, rows=None,
            atol=ATOL, rel=REL_L2, label="") -> float:
    """Per (stage, head): max-abs <= atol and rel-L2 <= rel. Returns the worst rel-L2."""
    if rows is not None:  # select the sampled rows on the device before the copy
        idx = torch.as_tensor(np.asarray(rows), dtype=torch.long, device=got_o.device)
        got_o = got_o.index_select(1, idx)
    g = got_o.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for s, w in want.items():
        H = w.shape[1]
        hs = list(range(H)) if heads is None else list(heads)
        gs = g[s][:, hs, :]
        assert np.isfinite(gs).all(), f"{label} stage {s}: non-finite outputs"
        for hi in range(len(hs)):
            d = gs[:, hi] - w[:, hi]
            mx = np.abs(d).max()
            r = np.linalg.norm(d) / max(np.linalg.norm(w[:, hi]), 1e-30)
            worst = max(worst, r)
            assert mx <= atol, f"{label} stage {s} head {hs[hi]}: max-abs {mx:.3e}"
            assert r <= rel, f"{label} stage {s} head {hs[hi]}: rel-L2 {r:.3e}"
    return worst
