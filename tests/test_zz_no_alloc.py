"""wf_attn_tick_noalloc (the run-time pool in the library's own per-GPU array,
no allocation by the call) against wf_attn_tick with a caller workspace of the
same size: two calls in a row, the second with a smaller tick (the array keeps
the first call's states and counters), each bit for bit equal to the other
entry point's launch and within the parity bar of the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

from _gpu_common import compare, oracle_tick, run_tick, say, setup_tick
from wavefront_causal_attention_wf_amd import wfattn

pytestmark = pytest.mark.gpu

# (S, T, H, P, n_hist): the 4-step steady tick's shape, then a smaller tick
CALLS = [(4, 4680, 12, 64, 3), (2, 600, 2, 64, 1)]


def sample_rows(T: int, seed: int) -> np.ndarray:
    fixed = [0, 31, 32, 255, 256, T // 2, T - 73, T - 33, T - 1]
    rnd = np.random.default_rng(seed).choice(T, 8, replace=False)
    return np.array(sorted({r for r in fixed + list(rnd) if 0 <= r < T}))


def test_noalloc_two_calls_second_smaller():
    for i, (S, T, H, P, n_hist) in enumerate(CALLS):
        say(f"no-alloc call {i}: S={S} T={T} H={H} P={P} n_hist={n_hist}")
        t = setup_tick(S, T, H, 128, P, n_hist, (n_hist + 2) * -(-T // P) + 8, seed=40 + i)
        full = wfattn.workspace_bytes(S, t.active_mask, T, H, 128, n_hist, None, P, t.num_pages)
        nb = min(full, wfattn.NOALLOC_SCRATCH_BYTES)
        assert nb > 0
        ws = torch.empty(nb, dtype=torch.uint8, device=t.q.device)
        d = wfattn.make_tick_desc(S, t.active_mask, T, H, 128, t.scale, t.q, t.k, t.v, t.o,
                                  t.k_pool, t.v_pool, t.num_pages, P, t.hist_pages, n_hist,
                                  None, workspace=ws)
        n_pool = int(np.sum(wfattn.tick_work_order(d, 0)[:, 0] == -1))
        say(f"  scratch bytes {nb} (full pool {full}), pool items {n_pool}")
        assert n_pool > 0
        o_na = torch.full_like(t.q, float("nan"))
        wfattn.wf_attn_tick_noalloc(t.q, t.k, t.v, o_na, S, t.active_mask, t.scale, t.k_pool,
                                    t.v_pool, t.hist_pages, scratch_bytes=nb)
        torch.cuda.synchronize()
        o_ws = run_tick(t, o=torch.full_like(t.q, float("nan")), workspace=ws)
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), f"call {i}"
        rows = sample_rows(T, seed=i)
        worst = compare(o_na, oracle_tick(t, rows=rows), rows=rows, label=f"no-alloc call {i}")
        say(f"  bit-identical to wf_attn_tick with a workspace; worst rel-L2 vs oracle {worst:.2e}")
        del t, ws, o_na, o_ws
        torch.cuda.empty_cache()


def test_noalloc_head_split_tick():
    """A tick that runs as two launches over head ranges (240 (stage, head)
    groups), each with its own pool in the same array: bit for bit equal to
    wf_attn_tick with a caller workspace of the same size, and within the
    parity bar of the oracle on sampled rows."""
    S, T, H, P, n_hist = 5, 1460, 40, 64, 2
    say(f"no-alloc head split: S={S} T={T} H={H} P={P} n_hist={n_hist}")
    t = setup_tick(S, T, H, 128, P, n_hist, (n_hist + 2) * -(-T // P) + 8, seed=47)
    full = wfattn.workspace_bytes(S, t.active_mask, T, H, 128, n_hist, None, P, t.num_pages)
    nb = min(full, wfattn.NOALLOC_SCRATCH_BYTES)
    ws = torch.empty(nb, dtype=torch.uint8, device=t.q.device)
    d = wfattn.make_tick_desc(S, t.active_mask, T, H, 128, t.scale, t.q, t.k, t.v, t.o,
                              t.k_pool, t.v_pool, t.num_pages, P, t.hist_pages, n_hist,
                              None, workspace=ws)
    order = wfattn.tick_work_order(d, 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert len(set(order[order[:, 0] >= 0, 0].tolist())) > cus   # more than one launch
    assert int(np.sum(order[:, 0] == -1)) > 0
    o_na = torch.full_like(t.q, float("nan"))
    wfattn.wf_attn_tick_noalloc(t.q, t.k, t.v, o_na, S, t.active_mask, t.scale, t.k_pool,
                                t.v_pool, t.hist_pages, scratch_bytes=nb)
    torch.cuda.synchronize()
    o_ws = run_tick(t, o=torch.full_like(t.q, float("nan")), workspace=ws)
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
    rows = sample_rows(T, seed=5)
    worst = compare(o_na, oracle_tick(t, rows=rows), rows=rows, label="no-alloc head split")
    say(f"  bit-identical to wf_attn_tick with a workspace; worst rel-L2 vs oracle {worst:.2e}")


def test_noalloc_replays_in_a_graph():
    """The allocation-free call captured in a HIP graph and replayed, with the
    program's own eager work (poisoned outputs, a tick of another shape through
    the same array) and synchronisations between replays: every replay equal
    bit for bit to the eager call, which equals wf_attn_tick with a caller
    workspace of the same size."""
    S, T, H, P, n_hist = 4, 1100, 4, 64, 3
    say(f"no-alloc graph: S={S} T={T} H={H} P={P} n_hist={n_hist}")
    t = setup_tick(S, T, H, 128, P, n_hist, (n_hist + 2) * -(-T // P) + 8, seed=48)
    full = wfattn.workspace_bytes(S, t.active_mask, T, H, 128, n_hist, None, P, t.num_pages)
    nb = min(full, wfattn.NOALLOC_SCRATCH_BYTES)
    assert nb > 0
    o = torch.full_like(t.q, float("nan"))

    def launch():
        wfattn.wf_attn_tick_noalloc(t.q, t.k, t.v, o, S, t.active_mask, t.scale, t.k_pool,
                                    t.v_pool, t.hist_pages, scratch_bytes=nb)

    launch()  # eager: takes the array's address and plans the launch before the capture
    torch.cuda.synchronize()
    o_ref = o.clone()
    ws = torch.empty(nb, dtype=torch.uint8, device=t.q.device)
    o_ws = run_tick(t, o=torch.full_like(t.q, float("nan")), workspace=ws)
    assert torch.equal(o_ref.view(torch.int16), o_ws.view(torch.int16))
    other = setup_tick(2, 600, 2, 128, 64, 1, 3 * 10 + 8, seed=49)
    o_other = torch.full_like(other.q, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    for r in range(4):
        o.fill_(float("nan"))
        # another tick through the same array between replays (its counters and
        # states are left there; the replay must clear what it needs)
        wfattn.wf_attn_tick_noalloc(other.q, other.k, other.v, o_other, other.S,
                                    other.active_mask, other.scale, other.k_pool, other.v_pool,
                                    other.hist_pages, scratch_bytes=wfattn.NOALLOC_SCRATCH_BYTES)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}"
    say("  4 replays bit-identical to the eager call")
    del g


def test_noalloc_8bit_tick():
    """An 8-bit K/V tick (every chunk through e4m3 pages; tail items and the
    run-time pool as the bf16 tick takes them): the allocation-free call bit
    for bit equal to wf_attn_tick with a caller workspace of the same size."""
    S, T, H, P, n_hist = 4, 1100, 4, 64, 3
    D = 128
    say(f"no-alloc 8-bit K/V: S={S} T={T} H={H} P={P} n_hist={n_hist}")
    ppc = -(-T // P)
    num_pages = (n_hist + S + 1) * ppc + 3
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(50)
    k_pool = torch.zeros((num_pages, P, H, D), dtype=torch.uint8, device=dev)
    k_scale = torch.zeros((num_pages, P // 64, H), dtype=torch.float32, device=dev)
    v_pool = torch.zeros((num_pages, P // 64, H, D, 64), dtype=torch.uint8, device=dev)
    v_exp = torch.zeros((num_pages, P // 64, H), dtype=torch.uint8, device=dev)
    ids = torch.randperm(num_pages, generator=torch.Generator().manual_seed(51))[
        :(n_hist + S + 1) * ppc].to(torch.int32).to(dev)
    hist = ids[:n_hist * ppc].view(n_hist, ppc)
    live = ids[n_hist * ppc:].view(S + 1, ppc)
    kv = (torch.randn((n_hist + S + 1, T, H, D), generator=gen, device=dev) * 0.5).to(torch.bfloat16)
    vv = (torch.randn((n_hist + S + 1, T, H, D), generator=gen, device=dev) * 0.5).to(torch.bfloat16)
    wfattn.wf_store_paged_fp8_chunks(kv, vv, k_pool, k_scale, v_pool, ids.view(-1, ppc),
                                     v_exp=v_exp)
    q = (torch.randn((S + 1, T, H, D), generator=gen, device=dev) * 0.5).to(torch.bfloat16)
    mask = (1 << (S + 1)) - 1
    scale = 1.0 / float(np.sqrt(D))
    nb = wfattn.workspace_bytes(S, mask, T, H, D, n_hist, None, P, num_pages, k8=True, v8=True)
    assert 0 < nb <= wfattn.NOALLOC_SCRATCH_BYTES
    o_na = torch.full_like(q, float("nan"))
    wfattn.wf_attn_tick_noalloc(q, None, None, o_na, S, mask, scale, k_pool, v_pool, hist,
                                live_pages=live, k_scale=k_scale, v_exp=v_exp, scratch_bytes=nb)
    torch.cuda.synchronize()
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    o_ws = torch.full_like(q, float("nan"))
    wfattn.wf_attn_tick(q, None, None, o_ws, S, mask, scale, k_pool, v_pool, hist,
                        live_pages=live, k_scale=k_scale, v_exp=v_exp, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o_na.float()).all()
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
    say("  bit-identical to wf_attn_tick with a workspace")
