"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test ties an oracle function to something the pages or mathematics fix:
hand-written tables from the pages' rules (tests/golden), closed forms the
pages state (fan-out counts, round count, per-rank key counts), brute force on
tiny inputs, a library attention routine for the dense special cases, and
invariances (perturbing masked chunks, relabelling pages).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import page_model
from wavefront_causal_attention_wf_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _rand(rng, shape, bf16=True, scale=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    return inputs.f32_to_bf16_bits(x) if bf16 else x


def _case(seed, S, T, H, D, n_hist, bf16=True, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = _rand(rng, (S + 1, T, H, D), bf16, qscale)
    k = _rand(rng, (S + 1, T, H, D), bf16)
    v = _rand(rng, (S + 1, T, H, D), bf16)
    hk = _rand(rng, (n_hist, T, H, D), bf16)
    hv = _rand(rng, (n_hist, T, H, D), bf16)
    return q, k, v, hk, hv


def _sdpa64(Q, K, V, scale):
    """Dense attention by torch's library routine, float64 on the CPU."""
    q = torch.from_numpy(np.ascontiguousarray(Q))[None]
    k = torch.from_numpy(np.ascontiguousarray(K))[None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0].numpy()


# ---------------------------------------------------------------------------
# tables and closed forms from the pages
# ---------------------------------------------------------------------------
def test_wave_mask_matches_hand_table():
    want = np.array([[int(x) for x in r] for r in _read_table("wave_mask_S4.txt")], bool)
    got = oracle.wave_mask(4, 0b11111)
    assert got.shape == (5, 5)
    assert (got == want).all()


def test_tick_members_match_hand_table():
    for row in _read_table("tick_sets_S4.txt"):
        k = int(row[0])
        want = {s: int(c) for s, c in enumerate(row[1:]) if c != "-"}
        assert oracle.tick_members(k, 4, n_chunks=8) == want, k


@pytest.mark.parametrize("S", range(1, 8))
def test_fanout_counts(S):
    """Full text Appendix B.8: among denoising stages a chunk's live K/V goes to the
    j noisier ranks, S(S-1)/2 payload destinations per layer; the store adds S."""
    m = oracle.wave_mask(S, (1 << (S + 1)) - 1)
    denoise_edges = sum(1 for s in range(S) for j in range(S) if j != s and m[s, j])
    store_edges = sum(1 for s in range(S) if m[s, S])
    assert denoise_edges == S * (S - 1) // 2
    assert store_edges == S
    for j in range(S):  # rank j feeds exactly j noisier ranks
        assert sum(1 for s in range(S) if s != j and m[s, j]) == j


@pytest.mark.parametrize("S,N", [(1, 1), (2, 5), (4, 8), (5, 100)])
def test_round_count(S, N):
    """Full text Appendix B.3: N_chunk + S rounds including fill and drain."""
    busy = [k for k in range(N + 3 * S + 5) if oracle.active_mask_for_tick(k, S, N)]
    assert busy == list(range(N + S))


@pytest.mark.parametrize("S,n_hist,T", [(4, 3, 4680), (5, 6, 4680), (2, 2, 64), (1, 0, 7)])
def test_keys_per_stage_closed_form(S, n_hist, T):
    """Summary page, Methodology 3: rank s reads N_s = N_prefix + (S - s) N_C keys,
    N_prefix = history + live store, N_C = one chunk; the store reads history + itself."""
    got = oracle.keys_per_stage(S, (1 << (S + 1)) - 1, n_hist, T)
    n_prefix = n_hist * T + T
    for s in range(S):
        assert got[s] == n_prefix + (S - s) * T
    assert got[S] == n_hist * T + T
    # cleaner ranks read fewer keys
    assert all(got[s] > got[s + 1] for s in range(S))


def test_useful_flops_closed_form():
    for name in ("tiny", "wan13_4step", "wan13_5step", "wan14b_4step"):
        c = inputs.CONFIGS[name]
        S, C = c.S, c.n_hist
        want = 4 * c.D * c.H * c.T ** 2 * ((S + 1) * C + (S + 1) * (S + 2) // 2)
        got = oracle.useful_flops(S, (1 << (S + 1)) - 1, C, c.T, c.H, c.D)
        assert got == want
    f1 = oracle.useful_flops(4, 0b11111, 3, 4680, 12, 128)
    assert abs(f1 / 1e12 - 4.037) < 1e-3
    # a partial tick counts only active stages and the history they see
    f = oracle.useful_flops(4, 0b10011, 3, 100, 2, 64, hist_first=[1, 0, 0, 0, 2])
    pairs = 100 * ((2 + 1 + 2) * 100 + (3 + 1 + 1) * 100 + (1 + 1) * 100)
    assert f == 4 * 64 * 2 * pairs


def test_context_order_eq5():
    """Eq. (5): anchor/history oldest first, live store, self, then cleaner j in
    increasing order."""
    segs = oracle.context_segments(1, 4, 0b11111, 3)
    assert segs == [("hist", 0), ("hist", 1), ("hist", 2), ("live", 4), ("live", 1),
                    ("live", 2), ("live", 3)]
    assert oracle.context_segments(4, 4, 0b11111, 3) == [("hist", 0), ("hist", 1),
                                                       ("hist", 2), ("live", 4)]
    # fill tick: store slot empty, only stages 0 and 1 present
    assert oracle.context_segments(0, 4, 0b00011, 0) == [("live", 0), ("live", 1)]


# ---------------------------------------------------------------------------
# brute force (C1)
# ---------------------------------------------------------------------------
def _brute_cases():
    rng = np.random.default_rng(123)
    cases = []
    for i, (S, T) in enumerate([(0, 1), (1, 7), (2, 16), (3, 5), (2, 1), (5, 3), (1, 16)]):
        n_hist = int(rng.integers(0, 4))
        mask = int(rng.integers(1, 1 << (S + 1)))
        hf = [int(rng.integers(0, n_hist + 1)) for _ in range(S + 1)]
        cases.append((i, S, T, n_hist, mask, hf))
    return cases


@pytest.mark.parametrize("i,S,T,n_hist,mask,hf", _brute_cases())
def test_oracle_matches_brute_force(i, S, T, n_hist, mask, hf):
    H, D, P = 2, 8, 16
    q, k, v, hk, hv = _case(1000 + i, S, T, H, D, n_hist)
    # history goes through the dict page store with scattered page ids
    store = oracle.PageStore(P, H, D)
    ppc = -(-T // P)
    ids = np.random.default_rng(i).permutation(64)[: n_hist * ppc].reshape(n_hist, ppc)
    for c in range(n_hist):
        store.write_chunk(ids[c], hk[c], hv[c])
    scale = 1.0 / np.sqrt(D)
    got = oracle.attention_tick_paged(q, k, v, store, ids.tolist(), S, mask, scale, hist_first=hf)
    want = oracle.brute_force_tick(q, k, v, hk, hv, S, mask, scale, hist_first=hf)
    assert set(got) == set(want) == {s for s in range(S + 1) if (mask >> s) & 1}
    for s in got:
        w = np.array(want[s])
        err = np.abs(got[s] - w).max() / max(np.abs(w).max(), 1e-300)
        assert err <= 1e-12, (s, err)


def test_brute_force_fp32_tiny_config_stage_sample():
    """The tiny workload itself (fp32 inputs), one head, brute force vs oracle."""
    c = inputs.CONFIGS["tiny"]
    x = inputs.draw_tick(c)
    T = 16  # first 16 tokens of each chunk keep the pure-Python sum fast
    sl = (slice(None), slice(0, T), slice(0, 1))
    q, k, v = x.q_f32[sl], x.k_f32[sl], x.v_f32[sl]
    hk, hv = x.hist_k_f32[sl], x.hist_v_f32[sl]
    got = oracle.attention_tick(q, k, v, hk, hv, c.S, 0b111, 1 / 8)
    want = oracle.brute_force_tick(q, k, v, hk, hv, c.S, 0b111, 1 / 8)
    for s in got:
        assert np.abs(got[s] - np.array(want[s])).max() <= 1e-12


# ---------------------------------------------------------------------------
# invariances and special cases (C2-C6)
# ---------------------------------------------------------------------------
def test_perturbing_noisier_chunks_leaves_output_bitwise_unchanged():
    S, T, H, D, nh = 4, 24, 2, 16, 2
    q, k, v, hk, hv = _case(7, S, T, H, D, nh)
    mask = (1 << (S + 1)) - 1
    base = oracle.attention_tick(q, k, v, hk, hv, S, mask, 0.25)
    rng = np.random.default_rng(8)
    for s in range(S + 1):
        k2, v2 = k.copy(), v.copy()
        for j in range(s):  # noisier chunks j < s
            k2[j] = _rand(rng, (T, H, D))
            v2[j] = _rand(rng, (T, H, D))
        got = oracle.attention_tick(q, k2, v2, hk, hv, S, mask, 0.25, stages=[s])
        assert np.array_equal(got[s], base[s]), s
        # positive controls: a visible live chunk, and history, both matter
        for j in range(s, S + 1):
            k3 = k.copy()
            k3[j] = _rand(rng, (T, H, D))
            assert not np.array_equal(oracle.attention_tick(q, k3, v, hk, hv, S, mask, 0.25,
                                                            stages=[s])[s], base[s])
        hk3 = hk.copy()
        hk3[0] = _rand(rng, (T, H, D))
        assert not np.array_equal(oracle.attention_tick(q, k, v, hk3, hv, S, mask, 0.25,
                                                        stages=[s])[s], base[s])


@pytest.mark.parametrize("n_hist", [0, 1, 3])
def test_S0_reduces_to_dense_attention(n_hist):
    """With no denoising stage the tick is just the store: dense attention over
    history + itself."""
    T, H, D = 33, 3, 16
    q, k, v, hk, hv = _case(11, 0, T, H, D, n_hist)
    got = oracle.attention_tick(q, k, v, hk, hv, 0, 0b1, 0.3)[0]
    for h in range(H):
        K = np.concatenate([oracle.decode_bf16(hk[c, :, h]) for c in range(n_hist)] +
                           [oracle.decode_bf16(k[0, :, h])])
        V = np.concatenate([oracle.decode_bf16(hv[c, :, h]) for c in range(n_hist)] +
                           [oracle.decode_bf16(v[0, :, h])])
        want = _sdpa64(oracle.decode_bf16(q[0, :, h]), K, V, 0.3)
        assert np.abs(got[:, h] - want).max() <= 1e-12


@pytest.mark.parametrize("qscale", [1.0, 8.0])
def test_concatenated_context_equals_masked_paged(qscale):
    """Full text Appendix B.6: attention over the ordered context of Eq. (5), however
    it is delivered, is the same function. Concatenate the context of each stage
    (history gathered from pages, then live store, self, cleaner chunks) and run
    unmasked dense attention by a library routine."""
    S, T, H, D, nh, P = 3, 40, 2, 32, 2, 16
    q, k, v, hk, hv = _case(21, S, T, H, D, nh, qscale=qscale)
    ppc = -(-T // P)
    ids = np.random.default_rng(5).permutation(32)[: nh * ppc].reshape(nh, ppc)
    store = oracle.PageStore(P, H, D)
    for c in range(nh):
        store.write_chunk(ids[c], hk[c], hv[c])
    mask = 0b1111
    scale = 1 / np.sqrt(D)
    got = oracle.attention_tick_paged(q, k, v, store, ids.tolist(), S, mask, scale)
    for s in range(S + 1):
        segs = oracle.context_segments(s, S, mask, nh)
        for h in range(H):
            ks, vs = [], []
            for kind, idx in segs:
                if kind == "hist":
                    kp = np.concatenate([store.pages[int(p)][0] for p in ids[idx]])[:T, h]
                    vp = np.concatenate([store.pages[int(p)][1] for p in ids[idx]])[:T, h]
                else:
                    kp, vp = k[idx, :, h], v[idx, :, h]
                ks.append(oracle.decode_bf16(kp))
                vs.append(oracle.decode_bf16(vp))
            want = _sdpa64(oracle.decode_bf16(q[s, :, h]), np.concatenate(ks), np.concatenate(vs),
                           scale)
            assert np.abs(got[s][:, h] - want).max() <= 1e-12 * max(1, np.abs(want).max())


def test_special_cases():
    S, T, H, D, nh = 2, 20, 2, 16, 2
    q, k, v, hk, hv = _case(31, S, T, H, D, nh)
    mask = 0b111
    # stage 0 sees every key: dense attention over all of them
    o0 = oracle.attention_tick(q, k, v, hk, hv, S, mask, 0.2, stages=[0])[0]
    for h in range(H):
        K = np.concatenate([oracle.decode_bf16(hk[c, :, h]) for c in range(nh)] +
                           [oracle.decode_bf16(k[j, :, h]) for j in range(S + 1)])
        V = np.concatenate([oracle.decode_bf16(hv[c, :, h]) for c in range(nh)] +
                           [oracle.decode_bf16(v[j, :, h]) for j in range(S + 1)])
        assert np.abs(o0[:, h] - _sdpa64(oracle.decode_bf16(q[0, :, h]), K, V, 0.2)).max() <= 1e-12
    # constant V -> constant O
    c = inputs.f32_to_bf16_bits(np.full((1,), 0.375, np.float32))[0]
    vc = np.full_like(v, c)
    hvc = np.full_like(hv, c)
    oc = oracle.attention_tick(q, k, vc, hk, hvc, S, mask, 0.2)
    for s in oc:
        assert np.abs(oc[s] - 0.375).max() <= 1e-15
    # T = 1, no history: the store's output is its own V
    q1, k1, v1, hk1, hv1 = _case(32, S, 1, H, D, 0)
    o1 = oracle.attention_tick(q1, k1, v1, hk1, hv1, S, mask, 0.2)
    assert np.array_equal(o1[S][0], oracle.decode_bf16(v1[S, 0]))
    # hist_first = n_hist hides history for that stage only
    oh = oracle.attention_tick(q, k, v, hk, hv, S, mask, 0.2, hist_first=[0, nh, 0])
    o_none = oracle.attention_tick(q, k, v, hk[:0], hv[:0], S, mask, 0.2, stages=[1])
    base = oracle.attention_tick(q, k, v, hk, hv, S, mask, 0.2)
    assert np.array_equal(oh[1], o_none[1])
    assert np.array_equal(oh[0], base[0]) and np.array_equal(oh[2], base[2])


def test_store_ignores_every_denoising_chunk():
    S, T, H, D, nh = 3, 12, 2, 8, 1
    q, k, v, hk, hv = _case(41, S, T, H, D, nh)
    base = oracle.attention_tick(q, k, v, hk, hv, S, 0b1111, 0.3, stages=[S])
    rng = np.random.default_rng(42)
    k2, v2 = k.copy(), v.copy()
    k2[:S] = _rand(rng, (S, T, H, D))
    v2[:S] = _rand(rng, (S, T, H, D))
    got = oracle.attention_tick(q, k2, v2, hk, hv, S, 0b1111, 0.3, stages=[S])
    assert np.array_equal(got[S], base[S])


def test_page_relabelling_is_invisible():
    """The result depends on the logical order of history only, not on which
    physical pages hold it."""
    S, T, H, D, nh, P = 2, 37, 2, 16, 3, 16
    q, k, v, hk, hv = _case(51, S, T, H, D, nh)
    ppc = -(-T // P)
    outs = []
    for seed in (0, 1):
        ids = np.random.default_rng(seed).permutation(40)[: nh * ppc].reshape(nh, ppc)
        store = oracle.PageStore(P, H, D)
        for c in range(nh):
            store.write_chunk(ids[c], hk[c], hv[c])
        outs.append(oracle.attention_tick_paged(q, k, v, store, ids.tolist(), S, 0b111, 0.25))
    for s in outs[0]:
        assert np.array_equal(outs[0][s], outs[1][s])


def test_inactive_stages_are_neither_queries_nor_keys():
    S, T, H, D = 3, 10, 1, 8
    q, k, v, hk, hv = _case(61, S, T, H, D, 1)
    mask = 0b1010  # stages 1 and 3 (store) present
    got = oracle.attention_tick(q, k, v, hk, hv, S, mask, 0.3)
    assert set(got) == {1, 3}
    k2, v2 = k.copy(), v.copy()
    k2[2] = 0
    v2[2] = 12345
    k2[0] = 0
    got2 = oracle.attention_tick(q, k2, v2, hk, hv, S, mask, 0.3)
    for s in got:
        assert np.array_equal(got[s], got2[s])


def test_mask_count_matches_flops():
    S, nh, T = 3, 2, 9
    mask = 0b1111
    for s in range(S + 1):
        tm = oracle.token_mask(s, S, mask, nh, T)
        assert tm.sum() == (nh + 1 + (S - s if s < S else 0)) * T


def test_bf16_decode_exact():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 65280.0, 1e-38], np.float32)
    bits = inputs.f32_to_bf16_bits(vals)
    dec = oracle.decode_bf16(bits)
    assert dec[0] == 0.0 and dec[1] == 1.0 and dec[2] == -2.5 and dec[3] == 3.140625
    assert dec[4] == 65280.0
    # decoding is exact: re-encoding the decoded value returns the same bits
    assert np.array_equal(inputs.f32_to_bf16_bits(dec.astype(np.float32)), bits)
