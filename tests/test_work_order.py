"""Host checks of the attention launch's work order (wf_tick_work_order, the
plan wf_attn_tick launches): every (slot, head, query tile) of the active slots
is computed by exactly one block, blocks past an XCD's list exit, and the
packed order keeps the XCDs even and their CUs busy to the end in a
list-scheduling model (one workgroup per CU; a freed CU takes the XCD's next
workgroup)."""
import heapq

import numpy as np
import pytest

from wavefront_causal_attention_wf_amd import inputs

wf = pytest.importorskip("wavefront_causal_attention_wf_amd.wfattn")

FAKE = 1 << 20  # never dereferenced: the call is host only


def desc(S, mask, T, H, n_hist, hist_first=None, num_pages=8192):
    return wf.make_tick_desc(S, mask, T, H, 128, 0.088, FAKE, FAKE, FAKE, FAKE,
                             FAKE if n_hist else None, FAKE if n_hist else None,
                             num_pages if n_hist else 0, 64 if n_hist else 0,
                             FAKE if n_hist else None, n_hist, hist_first)


def keys_of(S, mask, n_hist, hist_first, s):
    hf = 0 if hist_first is None else hist_first[s]
    n = (n_hist - hf) + ((mask >> S) & 1)
    n += sum(1 for j in range(s, S) if (mask >> j) & 1)
    return n


CASES = [
    ("wan13_4step", 4, 0b11111, 4680, 12, 3, None),
    ("wan13_5step", 5, 0b111111, 4680, 12, 6, None),
    ("wan14b_4step", 4, 0b11111, 4680, 40, 3, None),        # 200 groups: launches of fewer heads
    ("fill", 4, 0b00111, 4680, 12, 0, None),                 # fill tick, no store yet
    ("budgets", 4, 0b11111, 4680, 12, 3, [0, 1, 1, 2, 3]),   # per-slot history budgets
    ("small", 2, 0b101, 700, 3, 1, None),
    ("plain", 7, 0xFF, 200, 40, 1, None),                    # 320 groups: plain order
    ("tail1", 7, 0xFF, 96, 40, 1, None),                     # one query tile: all tail items
]


def with_workspace(d, nbytes=None):
    """The descriptor with a (never dereferenced) workspace of nbytes, by
    default the size wf_tick_workspace_bytes asks for."""
    d.workspace = FAKE
    d.workspace_bytes = wf.tick_workspace_bytes(d) if nbytes is None else nbytes
    return d


@pytest.mark.parametrize("name,S,mask,T,H,n_hist,hf", CASES)
@pytest.mark.parametrize("cus,ws", [(32, False), (0, False), (32, True)])
def test_every_row_once(name, S, mask, T, H, n_hist, hf, cus, ws):
    """Every query row of every active (slot, head) is computed by exactly one
    item, in rows of whole query tiles or (tail items) 32-row slices; with a
    workspace, some of them by the run-time pool (block -1, listed last)."""
    d = desc(S, mask, T, H, n_hist, hf)
    order = wf.tick_work_order(with_workspace(d) if ws else d, cus)
    assert order.shape[1] == 6
    cover = {(s, h): np.zeros(T, np.int32) for s in range(S + 1) if (mask >> s) & 1
             for h in range(H)}
    for blk, item, s, h, q0, n in order:
        assert (int(s), int(h)) in cover, (s, h)
        assert 0 <= q0 and n > 0 and q0 + n <= T
        cover[(int(s), int(h))][q0:q0 + n] += 1
    for key, c in cover.items():
        assert np.all(c == 1), (key, int(c.min()), int(c.max()))
    listed = order[order[:, 0] >= 0]
    assert np.all(np.diff(listed[:, 0]) >= 0)  # rows grouped by block, launch order
    assert np.all(order[len(listed):, 0] == -1)


def items_of(order):
    """{(block, item): [(slot, head, first row, rows), ...]} in launch order."""
    out = {}
    for blk, item, s, h, q0, n in order:
        out.setdefault((int(blk), int(item)), []).append((int(s), int(h), int(q0), int(n)))
    return out


def makespan(order, S, mask, n_hist, hf, T, cus):
    """Modelled CU efficiency (block b on XCD b % 8, item length = key tiles of
    the slot whose context it walks, the one with the most keys): one block per
    CU running its list (packed order), or one item per block taken by the
    XCD's next free CU in launch order."""
    tps = -(-T // 64)
    w = lambda s: keys_of(S, mask, n_hist, hf, s) * tps
    items = items_of(order)
    iw = {k: max(w(s) for s, _, _, _ in rows) for k, rows in items.items()}
    total = sum(iw.values())
    blocks = sorted({b for b, _ in items})
    if len(blocks) < len(items):       # lists per block
        worst = max(sum(v for (b, _), v in iw.items() if b == blk) for blk in blocks)
    else:
        worst = 0
        for x in range(8):
            t = [0] * cus
            heapq.heapify(t)
            for (b, _), v in iw.items():
                if b % 8 == x:
                    heapq.heappush(t, heapq.heappop(t) + v)
            worst = max(worst, max(t))
    return total / (8 * cus * worst), worst
# lowest modelled efficiency accepted: the fill tick's workgroups are 1-3 key
# chunks long and an XCD has 5.25 chunks of work per CU (tail items merge each
# head's three 72-row last tiles into items of 3 and 1 chunks), so 6 is the
# best makespan (87.5 %)
FLOOR = {"wan13_4step": 0.95, "wan13_5step": 0.95, "fill": 0.875, "budgets": 0.95}


@pytest.mark.parametrize("name,S,mask,T,H,n_hist,hf", CASES[:2] + CASES[3:5])
def test_packed_order_keeps_cus_busy(name, S, mask, T, H, n_hist, hf):
    packed = wf.tick_work_order(desc(S, mask, T, H, n_hist, hf), 32)
    eff, span = makespan(packed, S, mask, n_hist, hf, T, 32)
    # whole groups per XCD, heaviest first (the order without packing), for reference
    _, span_groups = makespan(wf.tick_work_order(desc(S, mask, T, H, n_hist, hf), 0), S, mask,
                              n_hist, hf, T, 32)
    assert eff >= FLOOR[name], eff
    assert span <= span_groups
    # XCD loads within 2 % of each other
    tps = -(-T // 64)
    iw = {k: max(keys_of(S, mask, n_hist, hf, s) * tps for s, _, _, _ in rows)
          for k, rows in items_of(packed).items()}
    loads = [sum(v for (b, _), v in iw.items() if b % 8 == x) for x in range(8)]
    assert max(loads) <= 1.02 * min(loads), loads


def test_work_order_errors():
    n = __import__("ctypes").c_int64()
    d = desc(4, 0b11111, 4680, 12, 3)
    out = np.empty(6, np.int32)
    st = wf.library().wf_tick_work_order(__import__("ctypes").byref(d), 32,
                                         out.ctypes.data_as(wf._i32p), out.size,
                                         __import__("ctypes").byref(n))
    assert st == -1  # capacity too small
    assert wf.library().wf_tick_work_order(__import__("ctypes").byref(d), 32, None, 0, None) == -1


def test_tail_items_merge_last_query_tiles():
    """At T = 4680 each slot's last query tile holds 72 rows (three 32-row
    slices, the last with 8): the five slots' 15 slices of a head become two
    tail items of up to eight slices; each walks the context of its first
    slice's slot, which holds every other slice's slot's context."""
    S, mask, T, H, n_hist = 4, 0b11111, 4680, 12, 3
    order = wf.tick_work_order(desc(S, mask, T, H, n_hist), 32)
    items = items_of(order)
    tail = {k: rows for k, rows in items.items() if any(q0 >= 18 * 256 for _, _, q0, _ in rows)}
    assert all(q0 >= 18 * 256 for rows in tail.values() for _, _, q0, _ in rows)
    assert len(tail) == 2 * H
    for rows in tail.values():
        assert len({h for _, h, _, _ in rows}) == 1
        assert sum(-(-n // 32) for _, _, _, n in rows) <= 8          # slices of one item
        walk = max(keys_of(S, mask, n_hist, None, s) for s, _, _, _ in rows)
        assert walk == keys_of(S, mask, n_hist, None, rows[0][0])    # first slice's slot
    # ordinary items are whole 256-row tiles
    for k, rows in items.items():
        if k not in tail:
            assert len(rows) == 1 and rows[0][2] % 256 == 0 and rows[0][3] == 256


@pytest.mark.parametrize("hf,expect_tail", [(None, True), ([0, 1, 1, 2, 3], False)])
def test_tail_items_need_nested_contexts(hf, expect_tail):
    """Different history budgets break the nesting: no tail items then."""
    order = wf.tick_work_order(desc(4, 0b11111, 4680, 12, 3, hf), 32)
    has_tail = any(n < 256 and q0 % 256 != 0 for _, _, _, _, q0, n in order)
    assert has_tail == expect_tail


def test_plain_order_when_tables_overflow():
    """8 slots x 40 heads = 320 (stage, head) groups exceed the XCD tables (and
    200-row tiles are too full for tail items): one item per block, blocks in
    stage-major order (heaviest stage first), head, then query tile — the order
    the kernel decodes when no table is used."""
    S, mask, T, H = 7, 0xFF, 200, 40
    order = wf.tick_work_order(desc(S, mask, T, H, 1), 32)
    ntq = -(-T // 256)
    assert len(order) == (S + 1) * H * ntq
    assert np.array_equal(order[:, 0], np.arange(len(order)))      # one item per block
    assert np.all(order[:, 1] == 0)
    stages = [s for s in range(S + 1)]
    stages.sort(key=lambda s: -keys_of(S, mask, 1, None, s))        # heaviest first (stable)
    want = [(s, h, 256 * q) for s in stages for h in range(H) for q in range(ntq)]
    assert [(int(r[2]), int(r[3]), int(r[4])) for r in order] == want


@pytest.mark.parametrize("ws", [False, True])
def test_head_split_launches(ws):
    """200 (stage, head) groups of the 14B-like tick are more than one packed
    plan holds, and one item per block would leave 15 items per CU to the
    dispatcher: the tick runs as launches over head ranges of ceil(H / n)
    heads, each a packed plan of one block per CU (blocks numbered on across
    the launches), each launch's items of its own heads only."""
    S, mask, T, H, n_hist = 4, 0b11111, 4680, 40, 3
    d = desc(S, mask, T, H, n_hist)
    order = wf.tick_work_order(with_workspace(d) if ws else d, 32)
    listed = order[order[:, 0] >= 0]
    n_blocks = int(listed[:, 0].max()) + 1
    assert n_blocks % 256 == 0 and n_blocks // 256 >= 2
    n = n_blocks // 256
    hp = -(-H // n)
    ranges = []
    for launch in range(n):
        rows = listed[(listed[:, 0] >= 256 * launch) & (listed[:, 0] < 256 * (launch + 1))]
        heads = sorted(set(rows[:, 3].tolist()))
        assert heads == list(range(heads[0], heads[0] + len(heads)))
        ranges.append((heads[0], len(heads)))
        eff, _ = makespan(rows, S, mask, n_hist, None, T, 32)
        assert eff >= 0.95, (launch, eff)
    assert ranges == [(i * hp, min(hp, H - i * hp)) for i in range(n)]
    pool = order[order[:, 0] == -1]
    assert (len(pool) > 0) == ws
    assert np.all(np.diff(pool[:, 1]) == 1)
    # pool items follow the launches: heads of each launch's range in turn
    assert np.all(np.diff(pool[:, 3] // hp) >= 0)


STATE_BYTES = 256 * (128 + 2) * 4   # one piece's partial state, D = 128


@pytest.mark.parametrize("name,S,mask,T,H,n_hist,hf", CASES[:2] + CASES[3:6])
def test_run_time_pool(name, S, mask, T, H, n_hist, hf):
    """The pool holds whole query tiles of the heaviest slot (the one with the
    most keys), at most 128, about 8 % of the tick's key tiles, spread over
    heads; the workspace holds 1 KB of counters and one partial state per
    chunk of that slot's walk for each item."""
    d = with_workspace(desc(S, mask, T, H, n_hist, hf))
    order = wf.tick_work_order(d, 32)
    pool = order[order[:, 0] == -1]
    keys = {s: keys_of(S, mask, n_hist, hf, s) for s in range(S + 1) if (mask >> s) & 1}
    heavy = max(keys, key=lambda s: keys[s])
    assert 0 < len(pool) <= 128
    assert np.array_equal(pool[:, 1], np.arange(len(pool)))
    assert np.all(pool[:, 2] == heavy)
    assert np.all(pool[:, 4] % 256 == 0)
    assert d.workspace_bytes == 1024 + len(pool) * keys[heavy] * STATE_BYTES
    # share of the work: pool tiles x walk length over all tiles' walks
    tps = -(-T // 64)
    all_w = sum(-(-T // 32) * 32 / 256 * keys[s] for s in keys) * H   # in query-tile walks
    share = len(pool) * keys[heavy] / all_w
    assert len(pool) == 128 or 0.06 <= share <= 0.10, share
    heads = np.bincount(pool[:, 3], minlength=H)
    assert heads.max() - heads.min() <= 1          # one tile per head in turn


def test_pool_follows_workspace_size():
    """A smaller workspace holds fewer pool items; one below a single item's
    states, or none at all, gives no pool (and the same lists as without)."""
    S, mask, T, H, n_hist = 4, 0b11111, 4680, 12, 3
    full = wf.tick_workspace_bytes(desc(S, mask, T, H, n_hist))
    per_item = 8 * STATE_BYTES
    n_full = (full - 1024) // per_item
    assert full == 1024 + n_full * per_item and n_full > 5
    for n in (5, 1):
        order = wf.tick_work_order(with_workspace(desc(S, mask, T, H, n_hist), 1024 + n * per_item + 100), 32)
        assert int(np.sum(order[:, 0] == -1)) == n
    plain = wf.tick_work_order(desc(S, mask, T, H, n_hist), 32)
    for nbytes in (0, 1024 + per_item - 1):
        order = wf.tick_work_order(with_workspace(desc(S, mask, T, H, n_hist), nbytes), 32)
        assert np.array_equal(order, plain)


def test_no_pool_where_it_does_not_apply():
    """Pages that are not whole 64-key tiles (per-lane page lookups) take no
    workspace."""
    S, mask, T, H, n_hist = 4, 0b11111, 4680, 12, 3
    d = desc(S, mask, T, H, n_hist)
    d.P = 48
    assert wf.tick_workspace_bytes(d) == 0


@pytest.mark.parametrize("v8", [False, True])
@pytest.mark.parametrize("S,mask,T,H,n_hist", [(4, 0b11111, 4680, 12, 3), (4, 0b11111, 4680, 40, 3),
                                               (2, 0b111, 300, 2, 1)])
def test_8bit_ticks_plan_like_bf16(S, mask, T, H, n_hist, v8):
    """The 8-bit tiers (every chunk through pages) take the same work order as
    the bf16 tick of the same shape: tail items, the run-time pool with the
    same workspace, launches over head ranges; every row once."""
    def d8(ws):
        d = desc(S, mask, T, H, n_hist)
        d.k_format = wf.K_E4M3
        d.k_scale = FAKE
        d.live_pages = FAKE
        if v8:
            d.v_format = wf.V_E4M3
            d.v_exp = FAKE
        return with_workspace(d) if ws else d
    ref = desc(S, mask, T, H, n_hist)
    ref.live_pages = FAKE
    for ws in (False, True):
        d = d8(ws)
        want = with_workspace(ref) if ws else ref
        assert d.workspace_bytes == want.workspace_bytes
        order = wf.tick_work_order(d, 32)
        assert np.array_equal(order, wf.tick_work_order(want, 32))
        cover = {(s, h): np.zeros(T, np.int32) for s in range(S + 1) if (mask >> s) & 1
                 for h in range(H)}
        for blk, item, s, h, q0, n in order:
            cover[(int(s), int(h))][q0:q0 + n] += 1
        assert all(np.all(c == 1) for c in cover.values())
        assert (int(np.sum(order[:, 0] == -1)) > 0) == (ws and d.workspace_bytes > 0)
    assert d8(True).workspace_bytes > 0


def test_pool_takes_ragged_last_tiles_without_tail_items():
    """Last query tiles of more than half a workgroup (180 rows at T = 1460)
    are not tail items; the pool then starts with them (rows past T are never
    a piece's output)."""
    d = with_workspace(desc(4, 0b11111, 1460, 3, 2))
    pool = wf.tick_work_order(d, 32)
    pool = pool[pool[:, 0] == -1]
    assert len(pool) >= 3
    assert np.all(pool[:3, 4] == 1280) and np.all(pool[:3, 5] == 180)
    assert sorted(pool[:3, 3].tolist()) == [0, 1, 2]


def _random_shapes(n, seed, large=False):
    """Seeded tick shapes across the planner's regimes: packed lists, tail
    items, head splits, plain order, fill/drain masks, history budgets."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        S = int(rng.integers(3 if large else 0, 8))
        mask = int(rng.integers(1, 1 << (S + 1)))
        if large and rng.random() < 0.6:
            mask = (1 << (S + 1)) - 1
        T = int(rng.choice([1460, 2048, 4680] if large else
                           [1, 64, 96, 200, 256, 300, 700, 1024, 1460, 2048, 4680]))
        H = int(rng.choice([12, 24, 40] if large else [1, 2, 3, 12, 24, 40]))
        n_hist = int(rng.integers(0, 4))
        if n_hist + S + 1 > 32:
            n_hist = 0
        hf = None
        if n_hist and rng.random() < 0.3:
            hf = [int(rng.integers(0, n_hist + 1)) for _ in range(S + 1)]
        out.append((S, mask, T, H, n_hist, hf))
    return out


@pytest.mark.parametrize("S,mask,T,H,n_hist,hf",
                         _random_shapes(40, 2026) + _random_shapes(40, 7, large=True))
def test_random_shapes_every_row_once(S, mask, T, H, n_hist, hf):
    """Every row of every active (slot, head) exactly once, with and without a
    workspace (also one a third of the size asked for, which holds fewer pool
    items), and for parts with 24 or 38 CUs per XCD; launches over head ranges
    cover disjoint, contiguous ranges."""
    for cus, ws in ((32, False), (32, True), (32, "third"), (24, True), (38, False)):
        d = desc(S, mask, T, H, n_hist, hf)
        if ws:
            d = with_workspace(d)
            if d.workspace_bytes == 0:
                continue
            if ws == "third":
                d.workspace_bytes = 1024 + (d.workspace_bytes - 1024) // 3
        order = wf.tick_work_order(d, cus)
        cover = {(s, h): np.zeros(T, np.int32) for s in range(S + 1) if (mask >> s) & 1
                 for h in range(H)}
        for blk, item, s, h, q0, n in order:
            assert (int(s), int(h)) in cover, (s, h)
            assert 0 <= q0 and n > 0 and q0 + n <= T
            cover[(int(s), int(h))][q0:q0 + n] += 1
        for key, c in cover.items():
            assert np.all(c == 1), (key, ws, int(c.min()), int(c.max()))
        listed = order[order[:, 0] >= 0]
        assert np.all(np.diff(listed[:, 0]) >= 0)
        assert np.all(order[len(listed):, 0] == -1)
        n_blocks = int(listed[:, 0].max()) + 1 if len(listed) else 0
        if cus == 32 and n_blocks > 256 and n_blocks % 256 == 0 and \
                len(set(listed[:, 0].tolist())) == n_blocks:
            # packed launches of one block per CU: each covers a contiguous head range
            ranges = []
            for launch in range(n_blocks // 256):
                rows = listed[(listed[:, 0] >= 256 * launch) & (listed[:, 0] < 256 * (launch + 1))]
                heads = sorted(set(rows[:, 3].tolist()))
                assert heads == list(range(heads[0], heads[0] + len(heads)))
                ranges.append(heads)
            flat = [h for r in ranges for h in r]
            assert flat == sorted(flat) and len(flat) == len(set(flat))
