"""GPU: wf_store_paged / wf_gather_paged are bit-exact against the oracle's dict
page store, including zero-filled page tails and untouched foreign pages."""
import numpy as np
import pytest
import torch

import oracle
from _gpu_common import DEV, say
from wavefront_causal_attention_wf_amd import inputs, wfattn

pytestmark = pytest.mark.gpu


def _bits(t):
    return inputs.bf16_tensor_bits(t)


@pytest.mark.parametrize("T,H,D,P,N", [(64, 2, 64, 16, 8), (37, 3, 64, 16, 10),
                                       (4680, 12, 128, 64, 200), (100, 1, 128, 48, 5)])
def test_store_paged_bit_exact(T, H, D, P, N):
    say(f"store T={T} H={H} D={D} P={P} N={N}")
    rng = np.random.default_rng(T + H)
    k = inputs.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    v = inputs.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    ppc = -(-T // P)
    ids = rng.permutation(N)[:ppc].astype(np.int32)
    kp = torch.full((N, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vp = torch.full((N, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    wfattn.wf_store_paged(inputs.to_device_bf16(k, DEV), inputs.to_device_bf16(v, DEV), kp, vp,
                          torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    store = oracle.PageStore(P, H, D)
    store.write_chunk(ids, k, v)
    kb, vb = _bits(kp), _bits(vp)
    for pid in range(N):
        if pid in store.pages:
            assert np.array_equal(kb[pid], store.pages[pid][0]), pid
            assert np.array_equal(vb[pid], store.pages[pid][1]), pid
        else:  # pages not in the chunk keep their NaN poison
            assert (kb[pid] == 0x7FC0).all() and (vb[pid] == 0x7FC0).all(), pid
    # gather back: equals the oracle's token-by-token gather
    kd = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=DEV)
    vd = torch.empty_like(kd)
    wfattn.wf_gather_paged(kp, vp, torch.from_numpy(ids[None]).to(DEV), kd, vd)
    torch.cuda.synchronize()
    K, V = store.gather([ids], T)
    assert np.array_equal(_bits(kd), K) and np.array_equal(_bits(vd), V)


def test_gather_several_chunks():
    say("gather several chunks")
    T, H, D, P, N, n = 150, 2, 64, 32, 40, 3
    rng = np.random.default_rng(5)
    ppc = -(-T // P)
    ids = rng.permutation(N)[: n * ppc].reshape(n, ppc).astype(np.int32)
    kp = torch.full((N, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    store = oracle.PageStore(P, H, D)
    for c in range(n):
        k = inputs.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
        v = inputs.f32_to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
        wfattn.wf_store_paged(inputs.to_device_bf16(k, DEV), inputs.to_device_bf16(v, DEV), kp,
                              vp, torch.from_numpy(ids[c]).to(DEV))
        store.write_chunk(ids[c], k, v)
    kd = torch.empty((n, T, H, D), dtype=torch.bfloat16, device=DEV)
    vd = torch.empty_like(kd)
    wfattn.wf_gather_paged(kp, vp, torch.from_numpy(ids).to(DEV), kd, vd)
    torch.cuda.synchronize()
    K, V = store.gather(ids.tolist(), T)
    assert np.array_equal(_bits(kd), K) and np.array_equal(_bits(vd), V)


def test_check_pages_mode_rejects_bad_ids(monkeypatch):
    say("WF_CHECK_PAGES")
    monkeypatch.setenv("WF_CHECK_PAGES", "1")
    T, H, D, P, N = 32, 1, 64, 16, 4
    k = torch.zeros((T, H, D), dtype=torch.bfloat16, device=DEV)
    kp = torch.zeros((N, P, H, D), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    bad = torch.tensor([1, 4], dtype=torch.int32, device=DEV)
    with pytest.raises(wfattn.WfError) as e:
        wfattn.wf_store_paged(k, k, kp, vp, bad)
    assert e.value.name == "WF_EINVAL"
    good = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    wfattn.wf_store_paged(k, k, kp, vp, good)
    torch.cuda.synchronize()


@pytest.mark.parametrize("S,T,H,D,P,n_hist", [(2, 100, 2, 64, 16, 1), (4, 4680, 12, 128, 64, 3),
                                              (3, 70, 3, 128, 64, 0),
                                              (5, 1460, 40, 128, 64, 2)])  # two head launches
def test_store_fused_into_attention_launch(S, T, H, D, P, n_hist):
    """wf_attn_tick with store_pages: the pages equal the oracle store bit for bit
    (zero tails, other pages untouched) and the outputs equal those of the
    separate wf_store_paged + wf_attn_tick sequence bit for bit."""
    from _gpu_common import setup_tick, run_tick
    say(f"fused store S={S} T={T} H={H} D={D} P={P} n_hist={n_hist}")
    ppc = -(-T // P)
    num_pages = (n_hist + 2) * ppc + 5
    order = np.random.default_rng(T).permutation(num_pages).astype(np.int32)
    t = setup_tick(S, T, H, D, P, n_hist, num_pages, seed=T + S, order=order)
    ids = order[n_hist * ppc:(n_hist + 1) * ppc]
    before = _bits(t.k_pool), _bits(t.v_pool)
    o_sep = run_tick(t).clone()
    o = torch.full_like(t.q, float("nan"))
    wfattn.wf_attn_tick(t.q, t.k, t.v, o, S, t.active_mask, t.scale, t.k_pool, t.v_pool,
                        t.hist_pages, store_pages=torch.from_numpy(ids).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_sep.view(torch.int16))
    t.store.write_chunk(ids, t.k_bits[S], t.v_bits[S])
    kb, vb = _bits(t.k_pool), _bits(t.v_pool)
    for pid in range(num_pages):
        if pid in ids:
            assert np.array_equal(kb[pid], t.store.pages[int(pid)][0]), pid
            assert np.array_equal(vb[pid], t.store.pages[int(pid)][1]), pid
        else:  # history pages and free pages are not touched
            assert np.array_equal(kb[pid], before[0][pid]) and np.array_equal(vb[pid], before[1][pid]), pid
