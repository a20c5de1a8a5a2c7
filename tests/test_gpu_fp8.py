"""GPU: the 8-bit tier — e4m3 key pages with per-(64-token tile, head) scales
written by wf_store_paged_fp8, and the tick whose Q.K^T runs on the e4m3 MFMA
([full text] §4.3: K/V quantisation and an 8-bit attention backend;
Appendix C.5 Table 8 and C.6: FP8 K/V).

* The producer's pages (codes, scales, V) must equal the oracle's 8-bit page
  store bit for bit: both take every decision (amax, the two fp32 quotients,
  the fp32 product, rounding to nearest even) in the same precision.
* The tick must match the oracle's attention over the dequantised values
  within the bf16 tier's tolerance: the only extra rounding on the device is
  the fp32 accumulation of exact e4m3 products and two fp32 scale products.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from _gpu_common import DEV, compare, say
from test_gpu_fullsize import sample_rows
from wavefront_causal_attention_wf_amd import inputs, wfattn

pytestmark = pytest.mark.gpu

bits = inputs.bf16_tensor_bits


class Fp8Pages:
    """Device pools of the 8-bit tier (codes poisoned with NaN codes 0xFF, scales
    and V with NaN) and the oracle's 8-bit page store, written side by side."""

    def __init__(self, num_pages, P, H, D):
        self.P, self.H, self.D = P, H, D
        self.k_pool = torch.full((num_pages, P, H, D), 0xFF, dtype=torch.uint8, device=DEV)
        self.k_scale = torch.full((num_pages, P // 64, H), float("nan"), dtype=torch.float32,
                                  device=DEV)
        self.v_pool = torch.full((num_pages, P, H, D), float("nan"), dtype=torch.bfloat16,
                                 device=DEV)
        self.store = ofp8.Fp8PageStore(P, H, D)

    def write(self, ids, k_chunk: torch.Tensor, v_chunk: torch.Tensor, k_bits=None, v_bits=None):
        wfattn.wf_store_paged_fp8(k_chunk, v_chunk, self.k_pool, self.k_scale, self.v_pool,
                                  torch.from_numpy(np.asarray(ids, np.int32)).to(DEV))
        self.store.write_chunk(list(ids), bits(k_chunk) if k_bits is None else k_bits,
                               bits(v_chunk) if v_bits is None else v_bits)

    def check(self, ids):
        """Device pages of `ids` == the oracle's pages, bit for bit."""
        torch.cuda.synchronize()
        idx = torch.as_tensor(np.asarray(ids), dtype=torch.long, device=DEV)
        kc = self.k_pool.index_select(0, idx).cpu().numpy()
        ks = self.k_scale.index_select(0, idx).cpu().numpy()
        vb = bits(self.v_pool.index_select(0, idx))
        for n, pid in enumerate(ids):
            wk, ws, wv = self.store.pages[int(pid)]
            bad = kc[n] != wk
            if bad.any():
                signed_zero = np.all(((kc[n][bad] | wk[bad]) & 0x7F) == 0)
                raise AssertionError(f"page {pid}: {int(bad.sum())} codes differ "
                                     f"(only signed zeros: {bool(signed_zero)}); first "
                                     f"{kc[n][bad][:4]} vs {wk[bad][:4]}")
            assert np.array_equal(ks[n].view(np.uint32), ws.view(np.uint32)), f"page {pid} scales"
            assert np.array_equal(vb[n], wv), f"page {pid} V"


@pytest.mark.parametrize("T,H,D,P", [
    (200, 2, 128, 64),      # ragged last page
    (150, 3, 64, 128),      # two scale tiles per page, the last page's second one empty
    (64, 1, 128, 64),       # one full page
    (4680, 12, 128, 64),    # the Wan-1.3B-like chunk
])
def test_store_fp8_matches_oracle_bits(T, H, D, P):
    say(f"store fp8 T={T} H={H} D={D} P={P}")
    ppc = -(-T // P)
    num_pages = ppc + 5
    cfg = inputs.TickConfig("s", S=0, T=T, H=H, D=D, P=P, n_hist=0, num_pages=num_pages,
                            std=0.5, bf16_inputs=True, page_order="permutation")
    k, v, _ = inputs.draw_live_torch(cfg, 77 + T, DEV)
    k[0, 3] = 0.0                                   # a zero row inside a tile
    pg = Fp8Pages(num_pages, P, H, D)
    ids = np.random.default_rng(T).permutation(num_pages)[:ppc].astype(np.int32)
    pg.write(ids, k[0], v[0])
    pg.check(ids)
    # pages outside the chunk are untouched
    others = sorted(set(range(num_pages)) - set(ids.tolist()))
    torch.cuda.synchronize()
    idx = torch.as_tensor(others, dtype=torch.long, device=DEV)
    assert bool((pg.k_pool.index_select(0, idx) == 0xFF).all())
    assert bool(torch.isnan(pg.k_scale.index_select(0, idx)).all())


@pytest.mark.parametrize("v8", [False, True])
def test_store_fp8_tiny_tiles(v8):
    """Tiles whose amax lies far below 1: keys under 2^-100 are stored as zero
    (scale 0), values take the least exponent -127 when smaller than 448 *
    2^-128. bf16 inputs around 2^-120 (normal) and 1e-38 (subnormal)."""
    say(f"store fp8 tiny tiles, 8-bit values {v8}")
    T, H, D, P = 256, 2, 128, 64
    cfg = inputs.TickConfig("s", S=0, T=T, H=H, D=D, P=P, n_hist=0, num_pages=8, std=0.5,
                            bf16_inputs=True, page_order="identity")
    k, v, _ = inputs.draw_live_torch(cfg, 5, DEV)
    k, v = k[0].clone(), v[0].clone()
    k[0:64, 0] *= 2.0 ** -120            # normal bf16, far below 2^-100
    k[64:128, 1] *= 1e-38                # subnormal bf16
    k[128:192, 0] *= 2.0 ** -99          # just above the threshold: a normal tile
    v[0:64, 1] *= 2.0 ** -120
    v[128:192, 0] *= 1e-38
    ids = np.array([5, 2, 7, 0], np.int32)
    pg = Fp8KvPages(8, P, H, D) if v8 else Fp8Pages(8, P, H, D)
    pg.write(ids, k, v)
    pg.check(ids)
    torch.cuda.synchronize()
    assert float(pg.k_scale[5, 0, 0]) == 0.0 and float(pg.k_scale[2, 0, 1]) == 0.0
    assert float(pg.k_scale[7, 0, 0]) > 0.0
    if v8:
        assert int(pg.v_exp[5, 0, 1]) == 0 and int(pg.v_exp[7, 0, 0]) == 0   # e = -127


def workspace8(S, mask, T, H, P, n_hist, num_pages, v8=False):
    """The workspace wf_tick_workspace_bytes asks for an 8-bit tick (run-time
    pool), or None where it takes none."""
    nb = wfattn.workspace_bytes(S, mask, T, H, 128, n_hist, None, P, num_pages, k8=True, v8=v8)
    return torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None


def _fp8_tick(S, T, H, P, n_hist, mask, seed, q_gain=1.0, ws=False):
    D = 128
    cfg = inputs.TickConfig("f8", S=S, T=T, H=H, D=D, P=P, n_hist=n_hist, num_pages=1,
                            std=0.5, bf16_inputs=True, page_order="identity", seed=seed)
    x = inputs.draw_tick(cfg)
    q_bits = x.q_bits
    if q_gain != 1.0:
        q_bits = inputs.f32_to_bf16_bits(oracle.decode_bf16(q_bits).astype(np.float32)
                                         * np.float32(q_gain))
    ppc = -(-T // P)
    num_pages = (n_hist + S + 2) * ppc + 3
    order = np.random.default_rng(seed + 5).permutation(num_pages).astype(np.int32)
    pg = Fp8Pages(num_pages, P, H, D)
    hist = order[:n_hist * ppc].reshape(n_hist, ppc) if n_hist else np.zeros((0, ppc), np.int32)
    for c in range(n_hist):
        pg.write(hist[c], inputs.to_device_bf16(x.hist_k_bits[c], DEV),
                 inputs.to_device_bf16(x.hist_v_bits[c], DEV), x.hist_k_bits[c], x.hist_v_bits[c])
    nan_ids = order[-ppc:]                    # never written: inactive slots point here
    live = np.empty((S + 1, ppc), np.int32)
    live_lists = []
    for j in range(S + 1):
        if (mask >> j) & 1:
            ids = order[(n_hist + j) * ppc:(n_hist + j + 1) * ppc]
            pg.write(ids, inputs.to_device_bf16(x.k_bits[j], DEV),
                     inputs.to_device_bf16(x.v_bits[j], DEV), x.k_bits[j], x.v_bits[j])
            live[j] = ids
            live_lists.append(ids.tolist())
        else:
            live[j] = nan_ids
            live_lists.append(None)
    q = inputs.to_device_bf16(q_bits, DEV)
    o = torch.full_like(q, float("nan"))
    scale = 1.0 / np.sqrt(D)
    work = workspace8(S, mask, T, H, P, n_hist, num_pages) if ws else None
    wfattn.wf_attn_tick(q, None, None, o, S, mask, scale, pg.k_pool, pg.v_pool,
                        torch.from_numpy(np.ascontiguousarray(hist)).to(DEV) if n_hist else None,
                        live_pages=torch.from_numpy(live).to(DEV), k_scale=pg.k_scale,
                        workspace=work)
    torch.cuda.synchronize()
    return pg, q_bits, hist, live_lists, o, scale


@pytest.mark.parametrize("ws", [False, True])   # with a workspace: the run-time pool
@pytest.mark.parametrize("S,T,H,P,n_hist,mask,q_gain", [
    (4, 200, 2, 64, 2, 0b11111, 1.0),
    (3, 130, 2, 128, 1, 0b1011, 1.0),     # slot 2 inactive, two scale tiles per page
    (2, 64, 2, 64, 0, 0b111, 1.0),        # no history, one tile per chunk (tail items)
    (4, 70, 3, 64, 3, 0b10110, 1.0),      # stages 0 and 3 inactive, ragged tiles (tail items)
    (2, 300, 2, 64, 1, 0b111, 4.0),       # peaked softmax: the running max is raised
    (4, 1100, 4, 64, 3, 0b11111, 1.0),    # 8-chunk walks, 76-row last tiles: lists, tail items, pool
])
def test_fp8_tick_matches_oracle(S, T, H, P, n_hist, mask, q_gain, ws):
    say(f"fp8 tick S={S} T={T} H={H} P={P} n_hist={n_hist} mask={mask:b} q_gain={q_gain} ws={ws}")
    pg, q_bits, hist, live_lists, o, scale = _fp8_tick(S, T, H, P, n_hist, mask,
                                                       seed=S * 31 + T, q_gain=q_gain, ws=ws)
    for ids in list(hist) + [l for l in live_lists if l is not None]:
        pg.check(list(ids))
    want = ofp8.attention_tick_fp8(q_bits, pg.store, hist.tolist(), live_lists, S, mask, scale)
    worst = compare(o, want, label="fp8 tick")
    # rows of inactive slots are left untouched
    for s in range(S + 1):
        if not (mask >> s) & 1:
            assert torch.isnan(o[s].float()).all()
    say(f"  worst rel-L2 {worst:.2e}")


# wan13_4step runs the packed per-CU work order; wan14b_4step (H = 40) has too
# many items for it and runs whole (stage, head) groups dealt to XCDs
FULL_SIZE = ["wan13_4step", "wan14b_4step"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_fp8_tick_full_size_sampled_rows(name):
    """Full-size 4-step ticks in the 8-bit tier, as the bench times them:
    three history chunks and five live chunks in 8-bit pages, sampled rows of
    every stage and head against the oracle."""
    cfg = inputs.CONFIGS[name]
    say(f"[full-size fp8] S={cfg.S} T={cfg.T} H={cfg.H} n_hist={cfg.n_hist}")
    ppc = cfg.ppc
    pg = Fp8Pages(cfg.num_pages, cfg.P, cfg.H, cfg.D)
    order = inputs.initial_free_order(cfg)
    hist = order[:cfg.n_hist * ppc].reshape(cfg.n_hist, ppc)
    for c in range(cfg.n_hist):
        hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, DEV)
        pg.write(hist[c], hk[0], hv[0])
        del hk, hv
    q, k, v = inputs.draw_live_torch(cfg, inputs.rollout_seed(0), DEV)
    live = order[cfg.n_hist * ppc:(cfg.n_hist + cfg.S + 1) * ppc].reshape(cfg.S + 1, ppc)
    for j in range(cfg.S + 1):
        pg.write(live[j], k[j], v[j])
    pg.check(list(hist[0]) + list(live[cfg.S]))
    mask = (1 << (cfg.S + 1)) - 1
    o = torch.full_like(q, float("nan"))
    scale = 1.0 / np.sqrt(cfg.D)
    wfattn.wf_attn_tick(q, None, None, o, cfg.S, mask, scale, pg.k_pool, pg.v_pool,
                        torch.from_numpy(np.ascontiguousarray(hist)).to(DEV),
                        live_pages=torch.from_numpy(np.ascontiguousarray(live)).to(DEV),
                        k_scale=pg.k_scale,
                        workspace=workspace8(cfg.S, mask, cfg.T, cfg.H, cfg.P, cfg.n_hist,
                                             cfg.num_pages))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    rows = sample_rows(cfg.T, seed=8)
    want = ofp8.attention_tick_fp8(bits(q), pg.store, hist.tolist(), live.tolist(), cfg.S, mask,
                                   scale, rows=rows)
    worst = compare(o, want, rows=rows, label="fp8 full size")
    say(f"[full-size fp8] worst rel-L2 {worst:.2e} over {len(rows)} rows x {cfg.H} heads")


# ---------------------------------------------------------------------------
# 8-bit values too (v_format = E4M3)
# ---------------------------------------------------------------------------
def v8_token_of_column():
    """Token (0..63) stored at byte 32*g + j of a transposed 8-bit V row."""
    return np.array([32 * (j // 16) + 16 * ((j // 8) % 2) + 8 * g + j % 8
                     for g in range(2) for j in range(32)])


class Fp8KvPages:
    """Device pools of the 8-bit K/V tier, poisoned, and the oracle's store."""

    def __init__(self, num_pages, P, H, D):
        self.P, self.H, self.D = P, H, D
        self.k_pool = torch.full((num_pages, P, H, D), 0xFF, dtype=torch.uint8, device=DEV)
        self.k_scale = torch.full((num_pages, P // 64, H), float("nan"), dtype=torch.float32,
                                  device=DEV)
        self.v_pool = torch.full((num_pages, P // 64, H, D, 64), 0xFF, dtype=torch.uint8,
                                 device=DEV)
        self.v_exp = torch.full((num_pages, P // 64, H), 0xFF, dtype=torch.uint8, device=DEV)
        self.store = ofp8.Fp8KvPageStore(P, H, D)

    def write(self, ids, k_chunk, v_chunk, k_bits=None, v_bits=None):
        wfattn.wf_store_paged_fp8(k_chunk, v_chunk, self.k_pool, self.k_scale, self.v_pool,
                                  torch.from_numpy(np.asarray(ids, np.int32)).to(DEV),
                                  v_exp=self.v_exp)
        self.store.write_chunk(list(ids), bits(k_chunk) if k_bits is None else k_bits,
                               bits(v_chunk) if v_bits is None else v_bits)

    def check(self, ids):
        torch.cuda.synchronize()
        idx = torch.as_tensor(np.asarray(ids), dtype=torch.long, device=DEV)
        kc = self.k_pool.index_select(0, idx).cpu().numpy()
        ks = self.k_scale.index_select(0, idx).cpu().numpy()
        vt = self.v_pool.index_select(0, idx).cpu().numpy()      # [n][P/64][H][D][64]
        ve = self.v_exp.index_select(0, idx).cpu().numpy()
        tok = v8_token_of_column()
        for n, pid in enumerate(ids):
            wk, ws, wv, we = self.store.pages[int(pid)]
            assert np.array_equal(kc[n], wk), f"page {pid} key codes"
            assert np.array_equal(ks[n].view(np.uint32), ws.view(np.uint32)), f"page {pid} scales"
            # logical value codes [P][H][D] from the transposed tiles
            logical = np.zeros_like(wv)
            for sub in range(self.P // 64):
                rows = vt[n, sub]                                  # [H][D][64]
                logical[sub * 64 + tok] = rows.transpose(2, 0, 1)
            bad = logical != wv
            assert not bad.any(), f"page {pid}: {int(bad.sum())} value codes differ"
            assert np.array_equal(ve[n].astype(np.int64), we + 127), f"page {pid} exponents"


def _fp8kv_tick(S, T, H, P, n_hist, mask, seed, q_zero=False, ws=False):
    D = 128
    cfg = inputs.TickConfig("f8kv", S=S, T=T, H=H, D=D, P=P, n_hist=n_hist, num_pages=1,
                            std=0.5, bf16_inputs=True, page_order="identity", seed=seed)
    x = inputs.draw_tick(cfg)
    q_bits = np.zeros_like(x.q_bits) if q_zero else x.q_bits
    ppc = -(-T // P)
    num_pages = (n_hist + S + 2) * ppc + 3
    order = np.random.default_rng(seed + 9).permutation(num_pages).astype(np.int32)
    pg = Fp8KvPages(num_pages, P, H, D)
    hist = order[:n_hist * ppc].reshape(n_hist, ppc) if n_hist else np.zeros((0, ppc), np.int32)
    for c in range(n_hist):
        pg.write(hist[c], inputs.to_device_bf16(x.hist_k_bits[c], DEV),
                 inputs.to_device_bf16(x.hist_v_bits[c], DEV), x.hist_k_bits[c], x.hist_v_bits[c])
    nan_ids = order[-ppc:]
    live = np.empty((S + 1, ppc), np.int32)
    live_lists = []
    for j in range(S + 1):
        if (mask >> j) & 1:
            ids = order[(n_hist + j) * ppc:(n_hist + j + 1) * ppc]
            pg.write(ids, inputs.to_device_bf16(x.k_bits[j], DEV),
                     inputs.to_device_bf16(x.v_bits[j], DEV), x.k_bits[j], x.v_bits[j])
            live[j] = ids
            live_lists.append(ids.tolist())
        else:
            live[j] = nan_ids
            live_lists.append(None)
    q = inputs.to_device_bf16(q_bits, DEV)
    o = torch.full_like(q, float("nan"))
    scale = 1.0 / np.sqrt(D)
    work = workspace8(S, mask, T, H, P, n_hist, num_pages, v8=True) if ws else None
    wfattn.wf_attn_tick(q, None, None, o, S, mask, scale, pg.k_pool, pg.v_pool,
                        torch.from_numpy(np.ascontiguousarray(hist)).to(DEV) if n_hist else None,
                        live_pages=torch.from_numpy(live).to(DEV), k_scale=pg.k_scale,
                        v_exp=pg.v_exp, workspace=work)
    torch.cuda.synchronize()
    return pg, q_bits, hist, live_lists, o, scale


def compare_kv8(o, want, bound, rms, rows=None, label=""):
    """The two checks of the 8-bit K/V tick against the exact attention of the
    dequantised values:
      * element by element, |device - exact| <= the worst-case e4m3-P bound +
        the bf16 output rounding and fp32 slack (2^-8 |exact| + 2e-3);
      * per (stage, head), ||device - exact|| <= kv8_l2_allowance(R, ||exact||),
        R from the statistics of the e4m3 rounding of P (p_rounding_rms). At the
        workload's size the first check alone would accept an all-zero output;
        this one rejects it, a wrong value exponent and a wrong token order.
    Returns the worst ratios (element, rel-L2) of error to allowance."""
    if rows is not None:
        o = o.index_select(1, torch.as_tensor(np.asarray(rows), dtype=torch.long, device=o.device))
    g = o.float().cpu().numpy().astype(np.float64)
    worst_el, worst_l2 = 0.0, 0.0
    for s, w in want.items():
        d = np.abs(g[s] - w)
        lim = bound[s][:, :, None] + 2.0 ** -8 * np.abs(w) + 2e-3
        assert np.isfinite(g[s]).all(), f"{label} stage {s}: non-finite outputs"
        assert np.all(d <= lim), f"{label} stage {s}: max excess {float((d - lim).max()):.3e}"
        worst_el = max(worst_el, float((d / lim).max()))
        for h in range(w.shape[1]):
            err = float(np.linalg.norm(g[s][:, h] - w[:, h]))
            allow = ofp8.kv8_l2_allowance(float(rms[s][h]), float(np.linalg.norm(w[:, h])))
            assert err <= allow, (f"{label} stage {s} head {h}: ||error|| {err:.3e} > "
                                  f"allowance {allow:.3e} (rel-L2 {err / np.linalg.norm(w[:, h]):.3e})")
            worst_l2 = max(worst_l2, err / allow)
    return worst_el, worst_l2


@pytest.mark.parametrize("T,H,P", [(200, 2, 64), (150, 3, 128), (4680, 12, 64)])
def test_store_fp8kv_matches_oracle_bits(T, H, P):
    say(f"store fp8 K/V T={T} H={H} P={P}")
    ppc = -(-T // P)
    num_pages = ppc + 3
    cfg = inputs.TickConfig("s", S=0, T=T, H=H, D=128, P=P, n_hist=0, num_pages=num_pages,
                            std=0.5, bf16_inputs=True, page_order="permutation")
    k, v, _ = inputs.draw_live_torch(cfg, 99 + T, DEV)
    v[0, 5] = 0.0
    pg = Fp8KvPages(num_pages, P, H, 128)
    ids = np.random.default_rng(T + 1).permutation(num_pages)[:ppc].astype(np.int32)
    pg.write(ids, k[0], v[0])
    pg.check(ids)


@pytest.mark.parametrize("S,T,H,P,n_hist,mask,ws", [
    (4, 200, 2, 64, 2, 0b11111, False),
    (3, 130, 2, 128, 1, 0b1011, False),
    (4, 1100, 4, 64, 3, 0b11111, True),    # tail items and the run-time pool's merges
])
def test_fp8kv_tick_exact_p(S, T, H, P, n_hist, mask, ws):
    """Zero queries make every score 0 and every P exactly 1 (an e4m3 value), so
    the output is the mean of the dequantised values: the bf16 tier's bounds."""
    say(f"fp8 K/V tick, P = 1: S={S} T={T} H={H} P={P} ws={ws}")
    pg, q_bits, hist, live_lists, o, scale = _fp8kv_tick(S, T, H, P, n_hist, mask, seed=T,
                                                         q_zero=True, ws=ws)
    want = ofp8.attention_tick_fp8kv(q_bits, pg.store, hist.tolist(), live_lists, S, mask, scale)
    compare(o, want, label="fp8 K/V, P = 1")


@pytest.mark.parametrize("S,T,H,P,n_hist,mask,ws", [
    (4, 200, 2, 64, 2, 0b11111, False),
    (3, 130, 2, 128, 1, 0b1011, False),
    (4, 70, 3, 64, 3, 0b10110, False),     # tail items
    (4, 70, 3, 64, 3, 0b10110, True),
    (4, 1100, 4, 64, 3, 0b11111, True),    # lists, tail items, the run-time pool
])
def test_fp8kv_tick_within_p_bound(S, T, H, P, n_hist, mask, ws):
    say(f"fp8 K/V tick S={S} T={T} H={H} P={P} n_hist={n_hist} mask={mask:b} ws={ws}")
    pg, q_bits, hist, live_lists, o, scale = _fp8kv_tick(S, T, H, P, n_hist, mask, seed=T + 7,
                                                         ws=ws)
    for ids in list(hist) + [l for l in live_lists if l is not None]:
        pg.check(list(ids))
    want = ofp8.attention_tick_fp8kv(q_bits, pg.store, hist.tolist(), live_lists, S, mask, scale)
    bound, rms = ofp8.p_rounding_terms(q_bits, pg.store, hist.tolist(), live_lists, S, mask,
                                       scale)
    r_el, r_l2 = compare_kv8(o, want, bound, rms, label="fp8 K/V")
    say(f"  worst error / allowance: element {r_el:.3f}, rel-L2 {r_l2:.3f}")


@pytest.mark.parametrize("name", FULL_SIZE)
def test_fp8kv_tick_full_size_sampled_rows(name):
    cfg = inputs.CONFIGS[name]
    say(f"[full-size fp8 K/V] S={cfg.S} T={cfg.T} H={cfg.H} n_hist={cfg.n_hist}")
    ppc = cfg.ppc
    pg = Fp8KvPages(cfg.num_pages, cfg.P, cfg.H, cfg.D)
    order = inputs.initial_free_order(cfg)
    hist = order[:cfg.n_hist * ppc].reshape(cfg.n_hist, ppc)
    for c in range(cfg.n_hist):
        hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, DEV)
        pg.write(hist[c], hk[0], hv[0])
        del hk, hv
    q, k, v = inputs.draw_live_torch(cfg, inputs.rollout_seed(0), DEV)
    live = order[cfg.n_hist * ppc:(cfg.n_hist + cfg.S + 1) * ppc].reshape(cfg.S + 1, ppc)
    for j in range(cfg.S + 1):
        pg.write(live[j], k[j], v[j])
    pg.check(list(hist[0][:4]) + list(live[cfg.S][-4:]))
    mask = (1 << (cfg.S + 1)) - 1
    o = torch.full_like(q, float("nan"))
    scale = 1.0 / np.sqrt(cfg.D)
    wfattn.wf_attn_tick(q, None, None, o, cfg.S, mask, scale, pg.k_pool, pg.v_pool,
                        torch.from_numpy(np.ascontiguousarray(hist)).to(DEV),
                        live_pages=torch.from_numpy(np.ascontiguousarray(live)).to(DEV),
                        k_scale=pg.k_scale, v_exp=pg.v_exp,
                        workspace=workspace8(cfg.S, mask, cfg.T, cfg.H, cfg.P, cfg.n_hist,
                                             cfg.num_pages, v8=True))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    rows = sample_rows(cfg.T, seed=9, n_random=8)
    qb = bits(q)
    want = ofp8.attention_tick_fp8kv(qb, pg.store, hist.tolist(), live.tolist(), cfg.S, mask,
                                     scale, rows=rows)
    bound, rms = ofp8.p_rounding_terms(qb, pg.store, hist.tolist(), live.tolist(), cfg.S, mask,
                                       scale, rows=rows)
    r_el, r_l2 = compare_kv8(o, want, bound, rms, rows=rows, label="fp8 K/V full size")
    say(f"[full-size fp8 K/V] worst error / allowance: element {r_el:.3f}, rel-L2 {r_l2:.3f} "
        f"over {len(rows)} rows")


@pytest.mark.parametrize("n,T,H,D,P,v8", [
    (3, 200, 2, 128, 64, False),    # ragged last page
    (2, 150, 3, 64, 128, False),    # two scale tiles per page, the last one empty
    (5, 4680, 12, 128, 64, False),  # a 4-step tick's live chunks
    (3, 200, 2, 128, 64, True),     # 8-bit values (D = 128, as the attention reads them)
    (2, 150, 3, 128, 128, True),
    (5, 4680, 12, 128, 64, True),
])
def test_store_fp8_chunks_equals_one_call_per_chunk(n, T, H, D, P, v8):
    """wf_store_paged_fp8_chunks (n chunks, one launch) leaves every pool byte
    as n wf_store_paged_fp8 calls do (pools poisoned alike beforehand), so its
    pages are the oracle's as well."""
    say(f"store fp8 chunks n={n} T={T} H={H} D={D} P={P} v8={v8}")
    ppc = -(-T // P)
    num_pages = n * ppc + 7
    cfg = inputs.TickConfig("s", S=n - 1, T=T, H=H, D=D, P=P, n_hist=0, num_pages=num_pages,
                            std=0.5, bf16_inputs=True, page_order="permutation")
    _, k, v = inputs.draw_live_torch(cfg, 91 + T, DEV)
    ids = torch.from_numpy(np.random.default_rng(T).permutation(num_pages)[:n * ppc]
                           .astype(np.int32).reshape(n, ppc)).to(DEV)

    def pools():
        kp = torch.full((num_pages, P, H, D), 0xFF, dtype=torch.uint8, device=DEV)
        ks = torch.full((num_pages, P // 64, H), float("nan"), dtype=torch.float32, device=DEV)
        if v8:
            vp = torch.full((num_pages, P // 64, H, D, 64), 0xFF, dtype=torch.uint8, device=DEV)
            ve = torch.full((num_pages, P // 64, H), 0xFF, dtype=torch.uint8, device=DEV)
        else:
            vp = torch.full((num_pages, P, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
            ve = None
        return kp, ks, vp, ve

    a, b = pools(), pools()
    wfattn.wf_store_paged_fp8_chunks(k, v, a[0], a[1], a[2], ids, v_exp=a[3])
    for c in range(n):
        wfattn.wf_store_paged_fp8(k[c], v[c], b[0], b[1], b[2], ids[c], v_exp=b[3])
    torch.cuda.synchronize()
    for x, y, name in zip(a, b, ("k_pool", "k_scale", "v_pool", "v_exp")):
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), name
