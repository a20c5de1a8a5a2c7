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
    ("wan14b_4step", 4, 0b11111, 4680, 40, 3, None),        # too large to pack: whole groups
    ("fill", 4, 0b00111, 4680, 12, 0, None),                 # fill tick, no store yet
    ("budgets", 4, 0b11111, 4680, 12, 3, [0, 1, 1, 2, 3]),   # per-slot history budgets
    ("small", 2, 0b101, 700, 3, 1, None),
    ("plain", 7, 0xFF, 96, 40, 1, None),                     # 320 groups: plain order
]


@pytest.mark.parametrize("name,S,mask,T,H,n_hist,hf", CASES)
@pytest.mark.parametrize("cus", [32, 0])
def test_every_tile_once(name, S, mask, T, H, n_hist, hf, cus):
    order = wf.tick_work_order(desc(S, mask, T, H, n_hist, hf), cus)
    ntq = -(-T // 256)
    want = {(s, h, q) for s in range(S + 1) if (mask >> s) & 1 for h in range(H)
            for q in range(ntq)}
    got = [tuple(int(v) for v in r[1:]) for r in order]
    assert len(got) == len(set(got)), "a tile is computed twice"
    assert set(got) == want
    assert np.all(np.diff(order[:, 0]) >= 0)  # rows grouped by block, launch order


def makespan(order, S, mask, n_hist, hf, T, cus):
    """Modelled CU efficiency (block b on XCD b % 8, item length = key tiles):
    one block per CU running its list (packed order), or one item per block
    taken by the XCD's next free CU in launch order."""
    tps = -(-T // 64)
    w = lambda s: keys_of(S, mask, n_hist, hf, s) * tps
    total = sum(w(s) for _, s, _, _ in order)
    blocks = order[:, 0]
    worst = 0
    if len(np.unique(blocks)) < len(blocks):       # lists per block
        for blk in np.unique(blocks):
            worst = max(worst, sum(w(s) for _, s, _, _ in order[blocks == blk]))
    else:
        for x in range(8):
            t = [0] * cus
            heapq.heapify(t)
            for _, s, _, _ in order[blocks % 8 == x]:
                heapq.heappush(t, heapq.heappop(t) + w(s))
            worst = max(worst, max(t))
    return total / (8 * cus * worst)
# lowest modelled efficiency accepted: the fill tick's workgroups are 1-3 key
# chunks long and an XCD has 5.3 chunks of work per CU, so 6 is the best
# makespan (89 %)
FLOOR = {"wan13_4step": 0.95, "wan13_5step": 0.95, "fill": 0.89, "budgets": 0.95}


@pytest.mark.parametrize("name,S,mask,T,H,n_hist,hf", CASES[:2] + CASES[3:5])
def test_packed_order_keeps_cus_busy(name, S, mask, T, H, n_hist, hf):
    packed = wf.tick_work_order(desc(S, mask, T, H, n_hist, hf), 32)
    eff = makespan(packed, S, mask, n_hist, hf, T, 32)
    # whole groups per XCD, heaviest first (the order without packing), for reference
    eff_groups = makespan(wf.tick_work_order(desc(S, mask, T, H, n_hist, hf), 0), S, mask, n_hist,
                          hf, T, 32)
    assert eff >= FLOOR[name], eff
    assert eff >= eff_groups
    # XCD loads within 2 % of each other
    tps = -(-T // 64)
    loads = [sum(keys_of(S, mask, n_hist, hf, s) * tps for _, s, _, _ in packed[packed[:, 0] % 8 == x])
             for x in range(8)]
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


def test_plain_order_when_tables_overflow():
    """8 slots x 40 heads = 320 (stage, head) groups exceed the XCD tables: one
    item per block, blocks in stage-major order (heaviest stage first), head,
    then query tile — the order the kernel decodes when no table is used."""
    S, mask, T, H = 7, 0xFF, 96, 40
    order = wf.tick_work_order(desc(S, mask, T, H, 1), 32)
    ntq = -(-T // 256)
    assert len(order) == (S + 1) * H * ntq
    assert np.array_equal(order[:, 0], np.arange(len(order)))      # one item per block
    stages = [s for s in range(S + 1)]
    stages.sort(key=lambda s: -keys_of(S, mask, 1, None, s))        # heaviest first (stable)
    want = [(s, h, q) for s in stages for h in range(H) for q in range(ntq)]
    assert [tuple(int(v) for v in r[1:]) for r in order] == want
