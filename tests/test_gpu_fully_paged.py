"""GPU: the fully paged tick — every key of every slot's context read through
pages ([full text] Appendix B.8, Eq. (13)) — and the producer flow that fills
those pages with rotated keys, including the anchor's re-rotation when the
window shifts ([full text] Appendix B.3).

* Small ticks: live K/V copied into pages; the paged launch must give the same
  bits as the launch that reads live K/V from k and v (same arithmetic, same
  key order), and match the oracle's fully paged attention. Pages of inactive
  slots are NaN-poisoned and must not be read.
* Streaming rollout at the Wan-1.3B-like shape with a pinned anchor: each tick
  the producer call rotates and pages every live chunk at its own frames, the
  store chunk goes to freshly allocated pages, the anchor's keys are rotated
  again after each window shift, and attention reads everything through pages.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_common import DEV, compare, say, setup_tick, run_tick
from test_gpu_rope import check_k_pages
from wavefront_causal_attention_wf_amd import inputs, wfattn

pytestmark = pytest.mark.gpu

bits = inputs.bf16_tensor_bits


@pytest.mark.parametrize("S,T,H,D,P,n_hist,mask", [
    (4, 200, 2, 128, 64, 2, 0b11111),
    (4, 200, 2, 128, 16, 2, 0b11111),     # pages not a multiple of 64: per-lane path
    (3, 130, 2, 64, 64, 1, 0b1011),       # slot 2 inactive
    (2, 64, 2, 64, 16, 0, 0b111),         # no history
    (4, 70, 3, 128, 64, 3, 0b10110),      # stage 0 and stage 3 inactive
])
def test_paged_live_equals_contiguous_and_oracle(S, T, H, D, P, n_hist, mask):
    say(f"fully paged S={S} T={T} H={H} D={D} P={P} n_hist={n_hist} mask={mask:b}")
    ppc = -(-T // P)
    num_pages = (n_hist + S + 2) * ppc + 3
    order = np.random.default_rng(T + S).permutation(num_pages).astype(np.int32)
    t = setup_tick(S, T, H, D, P, n_hist, num_pages, seed=S * 100 + T, active_mask=mask,
                   order=order)
    # live slot j -> the next ppc ids of the free order; inactive slots point at
    # the last, never written (NaN) pages
    nan_ids = order[-ppc:]
    live = np.empty((S + 1, ppc), np.int32)
    live_lists = []
    for j in range(S + 1):
        if (mask >> j) & 1:
            ids = order[(n_hist + j) * ppc:(n_hist + j + 1) * ppc]
            wfattn.wf_store_paged(t.k[j], t.v[j], t.k_pool, t.v_pool, torch.from_numpy(ids).to(DEV))
            t.store.write_chunk(ids, t.k_bits[j], t.v_bits[j])
            live[j] = ids
            live_lists.append(ids.tolist())
        else:
            live[j] = nan_ids
            live_lists.append(None)
    o_contig = run_tick(t).clone()
    o_paged = torch.full_like(t.q, float("nan"))
    wfattn.wf_attn_tick(t.q, None, None, o_paged, S, mask, t.scale, t.k_pool, t.v_pool,
                        t.hist_pages, t.hist_first, live_pages=torch.from_numpy(live).to(DEV))
    torch.cuda.synchronize()
    act = [s for s in range(S + 1) if (mask >> s) & 1]
    for s in act:
        assert np.array_equal(bits(o_paged[s]), bits(o_contig[s])), f"stage {s}"
    want = oracle.attention_tick_fully_paged(t.q_bits, t.store, t.hist_ids.tolist(), live_lists,
                                             S, mask, t.scale)
    worst = compare(o_paged, want, label="fully paged")
    say(f"  bit-identical to the contiguous launch; worst rel-L2 vs oracle {worst:.2e}")


def test_paged_live_head_split_equals_contiguous():
    """240 (stage, head) groups: both launches run as launches over head ranges;
    reading the live chunks through pages gives the bits of reading them from
    k and v (whose parity against the oracle the attention tests check)."""
    S, T, H, D, P, n_hist = 5, 1460, 40, 128, 64, 2
    mask = (1 << (S + 1)) - 1
    say(f"fully paged, head split: S={S} T={T} H={H} n_hist={n_hist}")
    ppc = -(-T // P)
    num_pages = (n_hist + S + 2) * ppc + 3
    order = np.random.default_rng(T + H).permutation(num_pages).astype(np.int32)
    t = setup_tick(S, T, H, D, P, n_hist, num_pages, seed=S * 100 + T + H, order=order)
    live = np.stack([order[(n_hist + j) * ppc:(n_hist + j + 1) * ppc] for j in range(S + 1)])
    for j in range(S + 1):
        wfattn.wf_store_paged(t.k[j], t.v[j], t.k_pool, t.v_pool, torch.from_numpy(live[j]).to(DEV))
    o_contig = run_tick(t).clone()
    o_paged = torch.full_like(t.q, float("nan"))
    wfattn.wf_attn_tick(t.q, None, None, o_paged, S, mask, t.scale, t.k_pool, t.v_pool,
                        t.hist_pages, t.hist_first, live_pages=torch.from_numpy(live).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o_paged.view(torch.int16), o_contig.view(torch.int16))
    say("  bit-identical to the contiguous launch")


def test_fully_paged_rollout_with_anchor():
    """12 ticks from an empty history, S = 4, T = 4680 (3 x 30 x 52 latent grid),
    12 heads x 128, window 3 with the anchor pinned; pre-rotation K and V drawn
    per tick, Q taken as already rotated. Chunk c covers latent frames 3c..3c+2.
    Every launch passes a workspace (run-time pool), as the bench does."""
    cfg = inputs.CONFIGS["wan13_4step"]
    S, T, H, D, P = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P
    grid = inputs.chunk_grid(T)
    F = grid[0]
    split = oracle.default_split(D)
    ppc = cfg.ppc
    window, ticks = 3, 12
    n_fifo = cfg.num_pages
    n_pool = n_fifo + S * ppc                        # + fixed pages of the S denoising slots
    order = inputs.initial_free_order(cfg)
    pt = wfattn.PageTable(n_fifo, P, T, window, pin_anchor=True, initial_free_order=order)
    model = oracle.FifoPageModel(n_fifo, P, T, window, pin_anchor=True, initial_free_order=order)
    store = oracle.PageStore(P, H, D)
    k_pool = torch.full((n_pool, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.full_like(k_pool, float("nan"))
    slot_ids = [np.arange(n_fifo + j * ppc, n_fifo + (j + 1) * ppc, dtype=np.int32) for j in range(S)]
    hist_chunks = []          # video chunk index of each history entry (oldest first)
    anchor = None             # (ids, K before rotation: device + host bits, V bits)
    scale = 1.0 / np.sqrt(D)
    live_dev = torch.empty((S + 1, ppc), dtype=torch.int32, device=DEV)
    # the bench's workspace: part of each tick through the run-time pool
    nb = wfattn.workspace_bytes(S, (1 << (S + 1)) - 1, T, H, D, window, None, P, n_pool,
                                live_paged=True)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    for k in range(ticks):
        mask = oracle.active_mask_for_tick(k, S)
        q, kk, vv = inputs.draw_live_torch(cfg, inputs.rollout_seed(k), DEV)
        qb, kb, vb = bits(q), bits(kk), bits(vv)
        live_lists = [None] * (S + 1)
        live = np.zeros((S + 1, ppc), np.int32)
        store_ids = None
        for j in range(S + 1):
            if not (mask >> j) & 1:
                continue
            c = k - j                                 # video chunk held by slot j
            if j < S:
                ids = slot_ids[j]
            else:
                ids = pt.alloc_chunk()
                assert ids.tolist() == model.alloc_chunk()
                store_ids = ids
            wfattn.wf_rope_store_paged(kk[j], vv[j], k_pool, v_pool, torch.from_numpy(ids).to(DEV),
                                       grid, F * c, split)
            rot = oracle.round_to_bf16_bits(oracle.rope(kb[j], grid, F * c, split))
            store.write_chunk(ids, rot, vb[j])
            live[j] = ids
            live_lists[j] = ids.tolist()
        hist = pt.export()
        assert hist.tolist() == model.export()
        live_dev.copy_(torch.from_numpy(live))
        o = torch.full_like(q, float("nan"))
        wfattn.wf_attn_tick(q, None, None, o, S, mask, scale, k_pool, v_pool,
                            torch.from_numpy(np.ascontiguousarray(hist)).to(DEV),
                            live_pages=live_dev, workspace=ws)
        torch.cuda.synchronize()
        rows = np.array(sorted({0, 63, 64, 2339, T - 9, T - 8, T - 1}
                               | set(np.random.default_rng(k).choice(T, 6, replace=False))))
        heads = None if k in (0, S, S + 2, ticks - 1) else [0]
        want = oracle.attention_tick_fully_paged(qb, store, model.export(), live_lists, S, mask,
                                                 scale, rows=rows, heads=heads)
        worst = compare(o, want, rows=rows, heads=heads, label=f"tick {k}")
        if store_ids is not None:
            if k in (S, S + 3):
                check_k_pages(bits(k_pool), store_ids, kb[S], grid, F * (k - S), split)
            ev = pt.commit()
            ev_m = model.commit()
            assert ev.tolist() == ev_m
            store.drop(ev_m)
            hist_chunks.append(k - S)
            if anchor is None:                        # the first clean chunk is the anchor
                anchor = (store_ids, kk[S].clone(), kb[S].copy(), vb[S].copy())
            if ev_m:                                  # window shift: index 1 left
                hist_chunks.pop(1)
                f0 = oracle.anchor_frame0(hist_chunks[1], F)
                a_ids, a_kdev, a_kbits, a_vbits = anchor
                wfattn.wf_rope_store_paged(a_kdev, None, k_pool, None,
                                           torch.from_numpy(a_ids).to(DEV), grid, f0, split)
                store.write_chunk(a_ids, oracle.round_to_bf16_bits(
                    oracle.rope(a_kbits, grid, f0, split)), a_vbits)
                torch.cuda.synchronize()
                if k == S + 4:
                    check_k_pages(bits(k_pool), a_ids, a_kbits, grid, f0, split)
                say(f"  tick {k}: window shift, anchor moved to frames {f0}..{f0 + F - 1}")
        say(f"[fully paged rollout] tick {k}: mask {mask:#x}, history chunks {hist_chunks}, "
            f"worst rel-L2 {worst:.2e} ({'all heads' if heads is None else 'head 0'})")
    assert anchor is not None and len(hist_chunks) == window and hist_chunks[0] == 0
