"""Parity at the full workload sizes, in the launch configuration the bench
times, and over a 120-tick streaming rollout.

The full-size ticks use the bench's own input recipe (history chunks and live
q/k/v drawn on the device by the seeded generator, history written through
wf_store_paged into NaN-poisoned pools); the oracle reads host copies of the
same generator output and builds its own page store from its own page model.
Outputs are compared on sampled query rows (every stage and head), chosen to
cover tile edges and the ragged last query tile, and on every row of every
stage and head for the bench's 4-step tick and for the rollout's fill ticks
and its last tick.
"""
import numpy as np
import pytest
import torch

import oracle
from wavefront_causal_attention_wf_amd import inputs, wfattn

from _gpu_common import DEV, compare, say

pytestmark = pytest.mark.gpu

bits = inputs.bf16_tensor_bits


def sample_rows(T: int, seed: int, n_random: int = 18) -> np.ndarray:
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, T // 2, T - 73, T - 72, T - 33, T - 2, T - 1]
    rnd = np.random.default_rng(seed).choice(T, n_random, replace=False)
    return np.array(sorted({r for r in fixed + list(rnd) if 0 <= r < T}))


class MirroredPages:
    """C page table + device pools, every step mirrored in the oracle's page
    model and dict page store (which never reads the device pools)."""

    def __init__(self, cfg, window: int, pin_anchor: bool = False):
        order = inputs.initial_free_order(cfg)
        self.cfg = cfg
        self.pt = wfattn.PageTable(cfg.num_pages, cfg.P, cfg.T, window, pin_anchor=pin_anchor,
                                   initial_free_order=order)
        self.model = oracle.FifoPageModel(cfg.num_pages, cfg.P, cfg.T, window,
                                          pin_anchor=pin_anchor, initial_free_order=order)
        self.store = oracle.PageStore(cfg.P, cfg.H, cfg.D)
        shape = (cfg.num_pages, cfg.P, cfg.H, cfg.D)
        self.k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        self.v_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        self.live_ids = None

    def store_chunk(self, k_chunk: torch.Tensor, v_chunk: torch.Tensor,
                    write: bool = True) -> np.ndarray:
        """Allocate the store chunk's pages (C table and oracle model) and record
        its K/V in the oracle store; write them to the device pools unless the
        tick's attention launch does it (write=False, store_pages)."""
        ids = self.pt.alloc_chunk()
        ids_m = self.model.alloc_chunk()
        assert ids.tolist() == ids_m
        if write:
            wfattn.wf_store_paged(k_chunk, v_chunk, self.k_pool, self.v_pool,
                                  torch.from_numpy(ids).to(DEV))
        self.store.write_chunk(ids_m, bits(k_chunk), bits(v_chunk))
        self.live_ids = ids_m
        return ids

    def check_pages(self, ids) -> None:
        """Device pool pages == the oracle store's pages, bit for bit."""
        idx = torch.as_tensor(list(ids), device=DEV, dtype=torch.long)
        got_k = bits(self.k_pool.index_select(0, idx))
        got_v = bits(self.v_pool.index_select(0, idx))
        for n, pid in enumerate(ids):
            want_k, want_v = self.store.pages[int(pid)]
            assert np.array_equal(got_k[n], want_k), f"K page {pid}"
            assert np.array_equal(got_v[n], want_v), f"V page {pid}"

    def commit(self) -> None:
        ev = self.pt.commit()
        ev_m = self.model.commit()
        assert ev.tolist() == ev_m
        self.store.drop(ev_m)
        self.live_ids = None
        self.check_tables()

    def check_tables(self) -> None:
        assert self.pt.export().tolist() == self.model.export()
        assert self.pt.num_free() == self.model.num_free()

    def hist_device(self) -> torch.Tensor:
        h = self.pt.export()
        return torch.from_numpy(np.ascontiguousarray(h)).to(DEV)


def workspace(cfg) -> torch.Tensor:
    """The workspace the bench passes: wf_tick_workspace_bytes of the
    configuration's full-width tick (ticks of other shapes use what fits)."""
    nb = wfattn.workspace_bytes(cfg.S, (1 << (cfg.S + 1)) - 1, cfg.T, cfg.H, cfg.D,
                                max(cfg.n_hist, 1), None, cfg.P, cfg.num_pages)
    assert nb > 0, cfg.name
    return torch.empty(nb, dtype=torch.uint8, device=DEV)


def run_tick(cfg, pages: MirroredPages, q, k, v, mask: int, store_ids=None,
             ws=None) -> torch.Tensor:
    """One tick; with store_ids the same launch writes the store chunk's pages;
    with ws part of the work goes through the run-time pool."""
    o = torch.full_like(q, float("nan"))
    wfattn.wf_attn_tick(q, k, v, o, cfg.S, mask, 1.0 / np.sqrt(cfg.D), pages.k_pool,
                        pages.v_pool, pages.hist_device(),
                        store_pages=None if store_ids is None else torch.from_numpy(store_ids).to(DEV),
                        workspace=ws)
    torch.cuda.synchronize()
    return o


def oracle_rows(cfg, pages: MirroredPages, q, k, v, mask: int, rows, heads=None):
    return oracle.attention_tick_paged(bits(q), bits(k), bits(v), pages.store,
                                       pages.model.export(), cfg.S, mask, 1.0 / np.sqrt(cfg.D),
                                       rows=rows, heads=heads)


@pytest.mark.parametrize("name,pool", [("wan13_4step", True), ("wan13_4step", False),
                                       ("wan13_5step", True), ("wan13_5step", False),
                                       ("wan14b_4step", True), ("wan14b_4step", False)])
def test_full_size_tick_sampled_rows(name, pool):
    """One steady tick exactly as the bench sets it up: n_hist history chunks
    (generator seeds 2000 + c) stored through the page table, live inputs from
    the rollout seed of tick 0, all S+1 slots active; with the bench's
    workspace (run-time pool) and without. (The 14B-like tick's 200 groups
    run as launches over head ranges.)"""
    cfg = inputs.CONFIGS[name]
    say(f"[full-size] {name}: S={cfg.S} T={cfg.T} H={cfg.H} n_hist={cfg.n_hist} pool={pool}")
    pages = MirroredPages(cfg, cfg.n_hist)
    for c in range(cfg.n_hist):
        hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, DEV)
        ids = pages.store_chunk(hk[0], hv[0])
        pages.check_pages(ids)
        pages.commit()
        del hk, hv
    q, k, v = inputs.draw_live_torch(cfg, inputs.rollout_seed(0), DEV)
    mask = (1 << (cfg.S + 1)) - 1
    o = run_tick(cfg, pages, q, k, v, mask, ws=workspace(cfg) if pool else None)
    assert torch.isfinite(o.float()).all()
    rows = sample_rows(cfg.T, seed=len(name))
    want = oracle_rows(cfg, pages, q, k, v, mask, rows)
    worst = compare(o, want, rows=rows, label=name)
    say(f"[full-size] {name}: worst rel-L2 {worst:.2e} over {len(rows)} rows x {cfg.H} heads")


def _bench_tick(cfg):
    pages = MirroredPages(cfg, cfg.n_hist)
    for c in range(cfg.n_hist):
        hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, DEV)
        ids = pages.store_chunk(hk[0], hv[0])
        pages.check_pages(ids)
        pages.commit()
        del hk, hv
    q, k, v = inputs.draw_live_torch(cfg, inputs.rollout_seed(0), DEV)
    return pages, q, k, v


def test_full_size_4step_every_row_every_head():
    """The bench's 4-step tick with its store write fused into the launch and
    the bench's workspace (the timed configuration): every row of every stage
    and head against the oracle, and the store chunk's pages bit for bit."""
    cfg = inputs.CONFIGS["wan13_4step"]
    say(f"[full-size, all rows] S={cfg.S} T={cfg.T} H={cfg.H} n_hist={cfg.n_hist}")
    pages, q, k, v = _bench_tick(cfg)
    mask = (1 << (cfg.S + 1)) - 1
    ids = pages.store_chunk(k[cfg.S], v[cfg.S], write=False)
    o = run_tick(cfg, pages, q, k, v, mask, store_ids=ids, ws=workspace(cfg))
    pages.check_pages(ids)
    pages.store.drop(ids)          # the store chunk's pages are not history yet
    want = oracle_rows(cfg, pages, q, k, v, mask, None)
    worst = compare(o, want, label="wan13_4step all rows")
    say(f"[full-size, all rows] worst rel-L2 {worst:.2e} over {cfg.T} rows x {cfg.H} heads")


def test_full_size_4step_peaked_sampled_rows():
    """The 4-step tick with Q x 16: scores of std 4 over 18,720-37,440 keys,
    so each row is dominated by a few keys ([full text] Eq. (4): where the
    mask matters most). Sampled rows of every stage and head."""
    cfg = inputs.CONFIGS["wan13_4step"]
    say(f"[full-size, peaked] S={cfg.S} T={cfg.T} H={cfg.H}, Q x 16")
    pages, q, k, v = _bench_tick(cfg)
    q = q * 16.0                   # exact in bf16 (a power of two)
    mask = (1 << (cfg.S + 1)) - 1
    o = run_tick(cfg, pages, q, k, v, mask, ws=workspace(cfg))
    rows = sample_rows(cfg.T, seed=16)
    want = oracle_rows(cfg, pages, q, k, v, mask, rows)
    worst = compare(o, want, rows=rows, label="wan13_4step q*16")
    say(f"[full-size, peaked] worst rel-L2 {worst:.2e} over {len(rows)} rows x {cfg.H} heads")


ROLLOUT_KEY_TICKS = (0, 1, 2, 3, 119)


@pytest.fixture(scope="module")
def rollout120():
    """120 ticks of a streaming rollout from an empty history (pipeline fill:
    stages activate one per tick and the store joins at tick S), window 3,
    4096-page permuted pool (pages are recycled about every 55 chunks).

    Every tick: page ids, evictions and exported tables equal the oracle model;
    the stored chunk's pool pages equal the oracle store bit for bit; every
    output is finite; head 0 matches the oracle on sampled rows. On a spread of
    ticks (fill, first eviction, recycled pages, last) every head matches on
    sampled rows. Odd ticks write the store chunk with wf_store_paged before the
    attention launch, even ticks let the attention launch write it
    (store_pages); every tick passes the bench's workspace (run-time pool). Returns host copies of the key ticks' inputs, outputs and
    history pages, which the tests below compare in full."""
    cfg = inputs.CONFIGS["rollout120"]
    S = cfg.S
    pages = MirroredPages(cfg, cfg.window)
    check_at = {0, 1, S - 1, S, S + 1, S + 3, S + 4, 40, 61, 90, cfg.ticks - 1}
    kept = {}
    ws = workspace(cfg)
    for t in range(cfg.ticks):
        mask = oracle.active_mask_for_tick(t, S)
        q, k, v = inputs.draw_live_torch(cfg, inputs.rollout_seed(t), DEV)
        store_on = bool((mask >> S) & 1)
        fused = store_on and t % 2 == 0
        if store_on:
            ids = pages.store_chunk(k[S], v[S], write=not fused)
            if not fused:
                pages.check_pages(ids)
        pages.check_tables()
        o = run_tick(cfg, pages, q, k, v, mask, store_ids=ids if fused else None, ws=ws)
        if fused:
            pages.check_pages(ids)
        for s in range(S + 1):
            if (mask >> s) & 1:
                assert torch.isfinite(o[s].float()).all(), f"tick {t} stage {s}"
        rows0 = sample_rows(cfg.T, seed=10_000 + t, n_random=4)
        want = oracle_rows(cfg, pages, q, k, v, mask, rows0, heads=[0])
        worst0 = compare(o, want, heads=[0], rows=rows0, label=f"tick {t} head 0")
        if t in check_at:
            rows = sample_rows(cfg.T, seed=t, n_random=6)
            want = oracle_rows(cfg, pages, q, k, v, mask, rows)
            worst = compare(o, want, rows=rows, label=f"tick {t}")
            say(f"[rollout] tick {t}: mask {mask:#x}, history "
                f"{len(pages.model.export())} chunks, worst rel-L2 {worst:.2e} (all heads, "
                f"sampled rows), {worst0:.2e} (head 0)")
        if t in ROLLOUT_KEY_TICKS:
            hist = pages.model.export()
            kept[t] = dict(q=bits(q), k=bits(k), v=bits(v), o=o.float().cpu().numpy(), mask=mask,
                           hist=hist, pages={p: pages.store.pages[p] for c in hist for p in c})
        if store_on:
            pages.commit()
        del q, k, v, o
    # every page still resident matches the oracle store
    resident = [p for c in pages.model.export() for p in c]
    pages.check_pages(resident)
    assert pages.pt.num_free() == cfg.num_pages - cfg.window * cfg.ppc
    return kept


def test_streaming_rollout_120_ticks(rollout120):
    assert sorted(rollout120) == list(ROLLOUT_KEY_TICKS)


@pytest.mark.parametrize("t", ROLLOUT_KEY_TICKS)
def test_rollout_key_tick_every_row_every_head(rollout120, t):
    """Ticks 0-3 (pipeline fill: one, two, three, four active stages, no store
    yet) and the last tick (full width, three history chunks on recycled
    pages): every row of every active stage and head against the oracle
    ([full text] Appendix B.6: the same outputs at every tick)."""
    cfg = inputs.CONFIGS["rollout120"]
    r = rollout120[t]
    store = oracle.PageStore(cfg.P, cfg.H, cfg.D)
    store.pages.update(r["pages"])
    want = oracle.attention_tick_paged(r["q"], r["k"], r["v"], store, r["hist"], cfg.S,
                                       r["mask"], 1.0 / np.sqrt(cfg.D))
    worst = compare(torch.from_numpy(r["o"]), want, label=f"tick {t} all rows")
    say(f"[rollout] tick {t}: every row of {len(want)} stages x {cfg.H} heads, "
        f"worst rel-L2 {worst:.2e}")
