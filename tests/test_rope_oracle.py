"""Pins of the oracle's rotary embedding, bf16 rounding and fully paged context.

Each check ties the oracle to something other than itself: hand-worked values
of the rotation (the convention and the axis split), a frequency ladder in
closed form, the defining invariants of a rotary embedding (norms kept, scores
depend only on coordinate differences, rotations compose), a library bf16
conversion, hand-derived rounding ties, and the contiguous-context attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_hand_worked_token():
    """D = 6 split (2, 2, 2): one pair per axis, each with frequency 1, so the
    angles are the coordinates themselves. Token 23 of a 2 x 3 x 4 grid starting
    at frame 5 sits at frame 6, row 2, column 3."""
    grid, f0 = (2, 3, 4), 5
    x = np.zeros((24, 1, 6))
    x[23, 0] = [1.0, 0.0, 0.0, 1.0, 1.0, 1.0]
    got = oracle.rope(x, grid, f0, split=(2, 2, 2))[23, 0]
    c3, s3 = math.cos(3), math.sin(3)
    want = [math.cos(6), math.sin(6), -math.sin(2), math.cos(2), c3 - s3, s3 + c3]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # every other token of that chunk had zero input and stays zero
    assert not oracle.rope(x, grid, f0, split=(2, 2, 2))[:23].any()


def test_frequency_ladder():
    """All 8 channels on the frame axis with theta = 16: pair i has frequency
    16^(-i/4) = 2^-i, so at frame 8 the angles are 8, 4, 2, 1."""
    x = np.zeros((1, 1, 8))
    x[0, 0, 0::2] = 1.0
    got = oracle.rope(x, (1, 1, 1), 8, split=(8, 0, 0), theta=16.0)[0, 0]
    want = []
    for a in (8.0, 4.0, 2.0, 1.0):
        want += [math.cos(a), math.sin(a)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    ax, fr = oracle.pair_axis_and_frequency(8, (8, 0, 0), 16.0)
    assert ax.tolist() == [0, 0, 0, 0] and np.allclose(fr, [1, 0.5, 0.25, 0.125], rtol=1e-15)


def test_default_split_and_group_order():
    assert oracle.default_split(128) == (44, 42, 42)
    assert oracle.default_split(64) == (24, 20, 20)
    ax, fr = oracle.pair_axis_and_frequency(128, (44, 42, 42), 10000.0)
    assert ax.tolist() == [0] * 22 + [1] * 21 + [2] * 21
    # each group restarts its ladder at frequency 1
    assert fr[0] == fr[22] == fr[43] == 1.0
    assert math.isclose(fr[1], 10000.0 ** (-2 / 44), rel_tol=1e-15)
    assert math.isclose(fr[23], 10000.0 ** (-2 / 42), rel_tol=1e-15)


def test_token_coordinates():
    c = oracle.token_coords(4680, (3, 30, 52), 12)
    assert c[0].tolist() == [12, 0, 0]
    assert c[51].tolist() == [12, 0, 51]
    assert c[52].tolist() == [12, 1, 0]
    assert c[1560].tolist() == [13, 0, 0]
    assert c[4679].tolist() == [14, 29, 51]
    with pytest.raises(ValueError):
        oracle.token_coords(4680, (3, 30, 51), 0)


def test_norms_are_kept():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(60, 3, 64))
    y = oracle.rope(x, (5, 3, 4), 7)
    pairs_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    pairs_out = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(pairs_in, pairs_out, rtol=1e-13, atol=0)


def test_scores_depend_only_on_coordinate_differences():
    """q.k after rotation is unchanged when both chunks move by the same number of
    frames (a reflection or a wrong sign in one component would break this)."""
    rng = np.random.default_rng(1)
    q = rng.normal(size=(48, 2, 128))
    k = rng.normal(size=(48, 2, 128))
    grid = (4, 3, 4)
    s1 = np.einsum("thd,uhd->htu", oracle.rope(q, grid, 3), oracle.rope(k, grid, 0))
    s2 = np.einsum("thd,uhd->htu", oracle.rope(q, grid, 3 + 41), oracle.rope(k, grid, 41))
    assert np.allclose(s1, s2, rtol=0, atol=1e-10)
    # and it does change with the frame difference
    s3 = np.einsum("thd,uhd->htu", oracle.rope(q, grid, 4), oracle.rope(k, grid, 0))
    assert not np.allclose(s1, s3, atol=1e-3)


def test_rotations_compose_and_invert_on_the_frame_axis():
    """With one row and one column per frame only the frame axis turns, and
    R(b) R(a) = R(a + b), R(-a) R(a) = identity, R(0) = identity."""
    rng = np.random.default_rng(2)
    x = rng.normal(size=(6, 2, 64))
    grid = (6, 1, 1)
    # token t sits at frame f0 + t: turned by 10 + t, then by 25 + t
    twice = oracle.rope(oracle.rope(x, grid, 10), grid, 25)
    direct = np.stack([oracle.rope(x[t:t + 1], (1, 1, 1), 35 + 2 * t)[0] for t in range(6)])
    assert np.allclose(twice, direct, rtol=0, atol=1e-12)
    one = x[:1]
    back = oracle.rope(oracle.rope(one, (1, 1, 1), 9), (1, 1, 1), -9)
    assert np.allclose(back, one, rtol=0, atol=1e-14)
    assert np.array_equal(oracle.rope(one, (1, 1, 1), 0), one)


def test_anchor_rerotation():
    """After a shift the anchor's keys are its unrotated keys turned at the new
    frames, which equals turning its old rotated keys by the frame difference."""
    assert oracle.anchor_frame0(5, 3) == 12
    assert oracle.anchor_frame0(1, 3) == 0   # before any shift: frames 0..2
    rng = np.random.default_rng(3)
    k = rng.normal(size=(1, 4, 64))
    new = oracle.rope(k, (1, 1, 1), oracle.anchor_frame0(7, 3))
    via_old = oracle.rope(oracle.rope(k, (1, 1, 1), 0), (1, 1, 1), 18)
    assert np.allclose(new, via_old, rtol=0, atol=1e-12)


def test_round_to_bf16_ties_and_single_rounding():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2.0 ** -8: 0x3F80,            # tie -> even (1.0)
        one + 3 * 2.0 ** -8: 0x3F82,        # tie -> even (1 + 2^-6)
        one + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # above the tie: rounded once, up
        -(one + 2.0 ** -8): 0xBF80,
        2.0 ** -130: 0x0008,                # bf16 subnormal, exact
        0.0: 0x0000,
        float("inf"): 0x7F80,
    }
    got = oracle.round_to_bf16_bits(np.array(list(cases.keys())))
    assert got.tolist() == list(cases.values())
    # float32 first would round the 2^-30 case to the tie and then down to 1.0
    f32_first = torch.tensor([one + 2.0 ** -8 + 2.0 ** -30], dtype=torch.float32).to(torch.bfloat16)
    assert int(f32_first.view(torch.int16).item()) & 0xFFFF == 0x3F80


def test_round_to_bf16_matches_library_on_float32_values():
    """For float32-exact inputs one rounding step is all there is, so torch's
    float32 -> bfloat16 conversion (nearest, ties to even) must agree."""
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.normal(scale=s, size=20000) for s in (1e-3, 1.0, 300.0)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_fully_paged_context_equals_contiguous():
    """Attention over a context read entirely through (permuted) pages equals the
    same attention over contiguous live chunks."""
    rng = np.random.default_rng(5)
    S, T, H, D, P = 2, 40, 2, 16, 16
    ppc = -(-T // P)
    to_bits = lambda a: oracle.round_to_bf16_bits(a)
    q = to_bits(rng.normal(size=(S + 1, T, H, D)))
    k = to_bits(rng.normal(size=(S + 1, T, H, D)))
    v = to_bits(rng.normal(size=(S + 1, T, H, D)))
    hk = to_bits(rng.normal(size=(2, T, H, D)))
    hv = to_bits(rng.normal(size=(2, T, H, D)))
    ids = rng.permutation(40)
    store = oracle.PageStore(P, H, D)
    hist_pages = [ids[c * ppc:(c + 1) * ppc].tolist() for c in range(2)]
    for c in range(2):
        store.write_chunk(hist_pages[c], hk[c], hv[c])
    live_pages = [ids[(2 + j) * ppc:(3 + j) * ppc].tolist() for j in range(S + 1)]
    for j in range(S + 1):
        store.write_chunk(live_pages[j], k[j], v[j])
    mask = 0b111
    want = oracle.attention_tick(q, k, v, hk, hv, S, mask, 0.25)
    got = oracle.attention_tick_fully_paged(q, store, hist_pages, live_pages, S, mask, 0.25)
    for s in want:
        assert np.array_equal(got[s], want[s])
    # an inactive slot needs no pages
    got2 = oracle.attention_tick_fully_paged(q, store, hist_pages, [live_pages[0], None, live_pages[2]],
                                            S, 0b101, 0.25)
    want2 = oracle.attention_tick(q, k, v, hk, hv, S, 0b101, 0.25)
    for s in want2:
        assert np.array_equal(got2[s], want2[s])
