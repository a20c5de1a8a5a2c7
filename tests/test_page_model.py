"""Pins of the oracle's page store and FIFO window model (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle.page_model import PageModelError
from wavefront_causal_attention_wf_amd import inputs


@pytest.mark.parametrize("pin", [False, True])
@pytest.mark.parametrize("W", [2, 3, 5])
def test_window_closed_form(pin, W):
    """After k commits the history holds chunks max(0, k-W) .. k-1 (with a pinned
    anchor: chunk 0 plus the last W-1), each chunk keeps the pages it was given,
    and free = N - ppc * (chunks resident)."""
    N, P, T = 97, 16, 37
    ppc = 3
    order = np.random.default_rng(W).permutation(N)
    m = oracle.FifoPageModel(N, P, T, W, pin_anchor=pin, initial_free_order=order)
    assert m.ppc == ppc
    given = {}
    for k in range(1, 40):
        ids = m.alloc_chunk()
        given[k - 1] = ids
        assert m.num_free() == N - ppc * (len(m.history) + 1)
        m.commit()
        if pin and k > W:
            want = [0] + list(range(k - W + 1, k))
        else:
            want = list(range(max(0, k - W), k))
        assert m.export() == [given[c] for c in want]
        assert m.num_free() == N - ppc * len(want)
        flat = [p for c in m.export() for p in c]
        assert len(set(flat)) == len(flat)
    # before any eviction the pages come straight off the initial order
    m2 = oracle.FifoPageModel(N, P, T, W, initial_free_order=order)
    for _ in range(W):
        m2.alloc_chunk()
        m2.commit()
    assert [p for c in m2.export() for p in c] == list(order[: W * ppc])


def test_identity_order_gives_iota_table():
    m = oracle.FifoPageModel(8, 16, 64, 2)
    for _ in range(2):
        m.alloc_chunk()
        m.commit()
    assert m.export() == [[0, 1, 2, 3], [4, 5, 6, 7]]


def test_eviction_recycles_fifo():
    m = oracle.FifoPageModel(6, 16, 32, 1)
    a = m.alloc_chunk()
    assert m.commit() == []
    b = m.alloc_chunk()
    assert m.commit() == a            # oldest chunk goes back to the tail
    assert list(m.free) == [4, 5, 0, 1]
    c = m.alloc_chunk()
    assert c == [4, 5] and b == [2, 3]


def test_errors():
    m = oracle.FifoPageModel(4, 16, 32, 2)
    with pytest.raises(PageModelError) as e:
        m.commit()
    assert e.value.code == "ESTATE"
    m.alloc_chunk()
    with pytest.raises(PageModelError) as e:
        m.alloc_chunk()
    assert e.value.code == "ESTATE"
    m.commit()
    m.alloc_chunk()
    m.commit()
    with pytest.raises(PageModelError) as e:
        m.alloc_chunk()            # both chunks resident, window not exceeded
    assert e.value.code == "ENOMEM"
    with pytest.raises(PageModelError):
        oracle.FifoPageModel(4, 16, 32, 1, pin_anchor=True)
    with pytest.raises(PageModelError):
        oracle.FifoPageModel(4, 16, 32, 2, initial_free_order=[0, 1, 1, 2])


def test_store_and_gather_round_trip_with_zero_tail():
    P, H, D, T = 16, 2, 8, 37
    rng = np.random.default_rng(0)
    k = inputs.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    v = inputs.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    s = oracle.PageStore(P, H, D)
    ids = [7, 2, 5]
    s.write_chunk(ids, k, v)
    # page contents: consecutive tokens, last page zero past token T-1
    assert np.array_equal(s.pages[7][0], k[0:16])
    assert np.array_equal(s.pages[2][1], v[16:32])
    assert np.array_equal(s.pages[5][0][:5], k[32:37])
    assert not s.pages[5][0][5:].any() and not s.pages[5][1][5:].any()
    K, V = s.gather([ids], T)
    assert np.array_equal(K[0], k) and np.array_equal(V[0], v)
    with pytest.raises(PageModelError):
        s.write_chunk([1, 2], k, v)


def test_rollout_schedule_history_lengths():
    """Rollout starting from empty history (full text Appendix B.6: the first tick
    starts with empty history): history 0, 1, 2, then stays at the window."""
    c = inputs.CONFIGS["rollout120"]
    m = oracle.FifoPageModel(c.num_pages, c.P, c.T, c.window,
                             initial_free_order=inputs.initial_free_order(c))
    lengths = []
    for _ in range(c.ticks):
        lengths.append(len(m.export()))
        m.alloc_chunk()
        m.commit()
    assert lengths[:5] == [0, 1, 2, 3, 3] and set(lengths[3:]) == {3}
    assert m.num_free() == c.num_pages - 3 * c.ppc
