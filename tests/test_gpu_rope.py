"""GPU: wf_rope_store_paged against the oracle's rotary embedding and page store.

V pages are compared bit for bit. K is rotated in fp32 on the device and in
float64 by the oracle; each stored key must lie within half a bf16 unit in the
last place (of the exact value) plus the fp32 error bound of the angle, the
sine and cosine and the two products, and almost all of them must equal the
oracle's correctly rounded bits. Page tails are zero; pages outside the chunk
keep their NaN poison.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu_common import DEV, say
from wavefront_causal_attention_wf_amd import inputs, wfattn

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0


def _bits(t):
    return inputs.bf16_tensor_bits(t)


def _draw(rng, shape):
    return inputs.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(0.5))


def _ulp_bf16(x):
    """Spacing of bf16 values around |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def check_k_pages(kp_bits, ids, k_pre_bits, grid, frame0, split, theta=10000.0, T=None):
    """Stored rotated keys vs the oracle, token by token through the page ids."""
    T = k_pre_bits.shape[0] if T is None else T
    H, D = k_pre_bits.shape[1], k_pre_bits.shape[2]
    P = kp_bits.shape[1]
    exact = oracle.rope(k_pre_bits, grid, frame0, split, theta)           # float64
    want_bits = oracle.round_to_bf16_bits(exact)
    tok = np.arange(T)
    got_bits = kp_bits[np.asarray(ids)[tok // P], tok % P]               # [T][H][D]
    got = oracle.decode_bf16(got_bits)
    x = oracle.decode_bf16(k_pre_bits)
    mag = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])                     # |x0| + |x1| per pair
    mag = np.repeat(mag, 2, axis=-1)
    theta_max = np.abs(oracle.rope_angles(T, D, grid, frame0, split, theta)).max()
    # fp32: angle (2 roundings), sin/cos (a few ulp), two products and a sum
    delta = mag * 2.0 ** -21 * (4.0 + theta_max)
    bound = 0.5 * _ulp_bf16(np.abs(exact) + delta) + delta
    err = np.abs(got - exact)
    assert (err <= bound).all(), f"worst excess {(err - bound).max():.3e}"
    same = (got_bits == want_bits).mean()
    assert same >= 0.99, f"only {same:.4f} of keys equal the correctly rounded value"
    return same


CASES = [
    # T, grid, H, D, P, N, frame0, split
    (64, (1, 8, 8), 2, 64, 16, 8, 0, None),
    (37, (1, 1, 37), 3, 64, 16, 10, 5, (24, 20, 20)),
    (100, (4, 5, 5), 1, 128, 48, 5, 1000, (64, 32, 32)),
    (60, (3, 4, 5), 2, 128, 64, 3, 12, (128, 0, 0)),
    (4680, (3, 30, 52), 12, 128, 64, 200, 396, None),
]


@pytest.mark.parametrize("T,grid,H,D,P,N,frame0,split", CASES)
def test_rope_store_matches_oracle(T, grid, H, D, P, N, frame0, split):
    say(f"rope store T={T} grid={grid} H={H} D={D} P={P} frame0={frame0} split={split}")
    split = oracle.default_split(D) if split is None else split
    rng = np.random.default_rng(T + 7 * H)
    k = _draw(rng, (T, H, D))
    v = _draw(rng, (T, H, D))
    ppc = -(-T // P)
    ids = rng.permutation(N)[:ppc].astype(np.int32)
    kp = torch.full((N, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    wfattn.wf_rope_store_paged(inputs.to_device_bf16(k, DEV), inputs.to_device_bf16(v, DEV), kp,
                               vp, torch.from_numpy(ids).to(DEV), grid, frame0, split)
    torch.cuda.synchronize()
    kb, vb = _bits(kp), _bits(vp)
    same = check_k_pages(kb, ids, k, grid, frame0, split)
    # V pages and the zero tails: bit-exact against the oracle store
    store = oracle.PageStore(P, H, D)
    store.write_chunk(ids, k, v)
    for pid in range(N):
        if pid in store.pages:
            assert np.array_equal(vb[pid], store.pages[pid][1]), pid
            n_valid = T - P * int(np.where(ids == pid)[0][0])
            if n_valid < P:
                assert (kb[pid, n_valid:] == 0).all(), pid
        else:
            assert (kb[pid] == NAN_BITS).all() and (vb[pid] == NAN_BITS).all(), pid
    say(f"  {same:.5f} of keys equal the correctly rounded value")


def test_rope_k_only_rewrite_keeps_v():
    """The anchor's re-rotation: K rewritten at new frames from the unrotated keys,
    V pages untouched."""
    say("rope K-only rewrite")
    T, grid, H, D, P, N = 4680, (3, 30, 52), 4, 128, 64, 100
    rng = np.random.default_rng(11)
    k = _draw(rng, (T, H, D))
    v = _draw(rng, (T, H, D))
    ids = rng.permutation(N)[:-(-T // P)].astype(np.int32)
    kp = torch.full((N, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    ids_d = torch.from_numpy(ids).to(DEV)
    kd = inputs.to_device_bf16(k, DEV)
    wfattn.wf_rope_store_paged(kd, inputs.to_device_bf16(v, DEV), kp, vp, ids_d, grid, 0)
    torch.cuda.synchronize()
    v_before = _bits(vp)
    new_f0 = oracle.anchor_frame0(9, 3)
    wfattn.wf_rope_store_paged(kd, None, kp, None, ids_d, grid, new_f0)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(vp), v_before)
    check_k_pages(_bits(kp), ids, k, grid, new_f0, oracle.default_split(D))


@pytest.mark.parametrize("n,T,grid,H,D,P,frame0,step", [
    (3, 100, (4, 5, 5), 2, 128, 48, 40, -4),      # ragged pages, frames descending
    (2, 64, (1, 8, 8), 3, 64, 16, 0, 1),          # heads not a multiple of four
    (5, 4680, (3, 30, 52), 12, 128, 64, 12, -3),  # a 4-step tick's live chunks
])
def test_rope_store_chunks_equals_one_call_per_chunk(n, T, grid, H, D, P, frame0, step):
    """wf_rope_store_paged_chunks (n chunks, one launch, chunk c at first frame
    frame0 + c * step) leaves every pool byte as n wf_rope_store_paged calls
    do, so its pages are the oracle's as well; the first chunk's keys are also
    checked against the oracle directly."""
    say(f"rope store chunks n={n} T={T} grid={grid} H={H} D={D} P={P} frame0={frame0} step={step}")
    rng = np.random.default_rng(T + n)
    ppc = -(-T // P)
    num_pages = n * ppc + 5
    k_bits = _draw(rng, (n, T, H, D))
    v_bits = _draw(rng, (n, T, H, D))
    k = inputs.to_device_bf16(k_bits, DEV)
    v = inputs.to_device_bf16(v_bits, DEV)
    ids = rng.permutation(num_pages)[:n * ppc].astype(np.int32).reshape(n, ppc)
    ids_dev = torch.from_numpy(ids).to(DEV)
    pools = [torch.full((num_pages, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
             for _ in range(4)]
    wfattn.wf_rope_store_paged_chunks(k, v, pools[0], pools[1], ids_dev, grid, frame0, step)
    for c in range(n):
        wfattn.wf_rope_store_paged(k[c], v[c], pools[2], pools[3], ids_dev[c], grid,
                                   frame0 + c * step)
    torch.cuda.synchronize()
    assert torch.equal(pools[0].view(torch.int16), pools[2].view(torch.int16)), "K pages"
    assert torch.equal(pools[1].view(torch.int16), pools[3].view(torch.int16)), "V pages"
    split = wfattn.default_rope_split(D)
    same = check_k_pages(_bits(pools[0]), ids[0], k_bits[0], grid, frame0, tuple(split))
    say(f"  equal to per-chunk calls; chunk 0 keys correctly rounded: {same:.4f}")
