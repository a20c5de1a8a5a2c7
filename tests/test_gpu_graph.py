"""The tick's launches captured in a HIP graph and replayed (callers that
capture their serving loop): wf_attn_tick with a caller workspace (the
run-time pool's counters are cleared by a small kernel in the same stream,
so the capture holds no memset) and the store chunk's page write fused into
the launch. Every replay, with the program's own eager work (poisoning the
outputs and the store pages) and synchronisations between replays, must equal
the eager launch bit for bit; the eager launch is within the parity bar of
the oracle on sampled rows."""
import numpy as np
import pytest
import torch

from _gpu_common import DEV, compare, oracle_tick, say, setup_tick, workspace_for
from wavefront_causal_attention_wf_amd import wfattn

pytestmark = pytest.mark.gpu

REPLAYS = 4


def free_store_pages(t, n: int) -> torch.Tensor:
    """n page ids that hold no history page of the tick."""
    used = set(int(p) for p in t.hist_ids.reshape(-1))
    free = [p for p in range(t.num_pages) if p not in used][:n]
    assert len(free) == n
    return torch.tensor(free, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("S,T,H,P,n_hist", [
    (4, 1100, 4, 64, 3),    # pool items, tail items, packed lists
    (5, 1460, 40, 64, 2),   # launches over head ranges, each with its pool
])
def test_tick_replays_in_a_graph(S, T, H, P, n_hist):
    say(f"[graph] S={S} T={T} H={H} P={P} n_hist={n_hist}")
    ppc = -(-T // P)
    t = setup_tick(S, T, H, 128, P, n_hist, (n_hist + 2) * ppc + 8, seed=61)
    ws = workspace_for(t)
    assert ws is not None
    sp = free_store_pages(t, ppc)
    o = torch.full_like(t.q, float("nan"))

    def launch():
        wfattn.wf_attn_tick(t.q, t.k, t.v, o, t.S, t.active_mask, t.scale, t.k_pool, t.v_pool,
                            t.hist_pages, store_pages=sp, workspace=ws)

    launch()  # eager: plans the launch (cached by shape) before the capture
    torch.cuda.synchronize()
    o_ref = o.clone()
    k_ref, v_ref = t.k_pool[sp.long()].clone(), t.v_pool[sp.long()].clone()
    rows = np.array(sorted({0, 31, 32, 255, 256, T // 2, T - 73, T - 1}))
    worst = compare(o_ref, oracle_tick(t, rows=rows), rows=rows, label="eager")
    say(f"  eager launch: worst rel-L2 vs oracle {worst:.2e}")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        o.fill_(float("nan"))
        t.k_pool[sp.long()] = float("nan")
        t.v_pool[sp.long()] = float("nan")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}: outputs"
        assert torch.equal(t.k_pool[sp.long()].view(torch.int16), k_ref.view(torch.int16)), \
            f"replay {r}: K pages"
        assert torch.equal(t.v_pool[sp.long()].view(torch.int16), v_ref.view(torch.int16)), \
            f"replay {r}: V pages"
    say(f"  {REPLAYS} replays bit-identical to the eager launch (outputs and store pages)")
    del g
