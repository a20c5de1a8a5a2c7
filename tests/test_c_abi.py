"""Host-side checks of the C-ABI library (no GPU needed): the shared library
loads and exports every function include/wf_attn.h declares; the C page table
matches the oracle's FIFO window model call for call, also under AddressSanitizer
and UBSan; argument validation rejects bad calls before touching the device;
the useful-FLOP count equals the oracle's mask count."""
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle.page_model import PageModelError
from wavefront_causal_attention_wf_amd import build_lib, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wf_attn.h")

CODES = {"EINVAL": -1, "ENOMEM": -2, "EHIP": -3, "EUNSUPPORTED": -4, "ESTATE": -5}


def _wfattn():
    if not os.path.exists(build_lib.LIB_PATH):
        build_lib.build()
    from wavefront_causal_attention_wf_amd import wfattn
    return wfattn


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(wf_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_header_function():
    wf = _wfattn()
    names = header_functions()
    assert len(names) >= 13, names
    lib = wf.library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in wf_attn.h but not exported"
    assert sorted(wf.EXPORTED_SYMBOLS) == names
    declared = int(re.search(r"#define WF_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert wf.abi_version() == declared
    nm = subprocess.run(["nm", "-D", "--defined-only", build_lib.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (wf_[a-z0-9_]+)$", nm, flags=re.M))
    assert exported == set(names)


def test_descriptor_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of wf_tick_desc and wf_rope_desc have the C layout:
    size and every field offset, as a host compiler lays out the header."""
    wf = _wfattn()
    structs = {"wf_tick_desc": wf.WfTickDesc, "wf_rope_desc": wf.WfRopeDesc}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "wf_attn.h"', "int main() {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True,
                   capture_output=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        cname, field, val = line.split()
        got[(cname, field)] = int(val)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == __import__("ctypes").sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


# ---------------------------------------------------------------------------
# page table: C vs oracle model
# ---------------------------------------------------------------------------
def _schedule(wf, N, P, T, W, pin, order, ticks):
    c = wf.PageTable(N, P, T, W, pin_anchor=pin, initial_free_order=order)
    m = oracle.FifoPageModel(N, P, T, W, pin_anchor=pin, initial_free_order=order)
    assert c.ppc == m.ppc
    for k in range(ticks):
        assert c.alloc_chunk().tolist() == m.alloc_chunk()
        assert c.num_free() == m.num_free()
        assert c.commit().tolist() == m.commit()
        assert c.export().tolist() == m.export()
        assert c.num_free() == m.num_free()
    c.close()


@pytest.mark.parametrize("pin", [False, True])
def test_page_table_matches_model_rollout(pin):
    """120-tick rollout at the 4680-token, 64-token-page shape (74 pages per
    chunk, the last one ragged), window 3, permuted pool of 4096 pages."""
    wf = _wfattn()
    cfg = inputs.CONFIGS["wan13_4step"]
    order = inputs.initial_free_order(cfg)
    _schedule(wf, cfg.num_pages, cfg.P, cfg.T, 3, pin, order, 120)


@pytest.mark.parametrize("N,P,T,W", [(12, 16, 64, 2), (9, 16, 40, 2), (64, 16, 17, 5), (4, 4, 4, 1)])
def test_page_table_matches_model_small(N, P, T, W):
    wf = _wfattn()
    order = np.random.default_rng(N * 31 + W).permutation(N)
    _schedule(wf, N, P, T, W, False, order, 30)
    if W >= 2:
        _schedule(wf, N, P, T, W, True, None, 30)


def test_page_table_errors_leave_state_unchanged():
    wf = _wfattn()
    for bad in [(0, 16, 64, 2), (8, 0, 64, 2), (8, 16, 0, 2), (8, 16, 64, 0)]:
        with pytest.raises(wf.WfError) as e:
            wf.PageTable(*bad)
        assert e.value.status == CODES["EINVAL"]
    with pytest.raises(wf.WfError) as e:
        wf.PageTable(8, 16, 64, 1, pin_anchor=True)
    assert e.value.status == CODES["EINVAL"]
    with pytest.raises(wf.WfError) as e:
        wf.PageTable(4, 16, 64, 2, initial_free_order=[0, 1, 1, 3])
    assert e.value.status == CODES["EINVAL"]
    with pytest.raises(wf.WfError) as e:
        wf.PageTable(4, 16, 64, 2, initial_free_order=[0, 1, 2, 4])
    assert e.value.status == CODES["EINVAL"]

    pt = wf.PageTable(10, 16, 40, 2)  # 3 pages per chunk
    with pytest.raises(wf.WfError) as e:
        pt.commit()
    assert e.value.status == CODES["ESTATE"]
    ids = pt.alloc_chunk()
    with pytest.raises(wf.WfError) as e:
        pt.alloc_chunk()
    assert e.value.status == CODES["ESTATE"]
    assert pt.num_free() == 7
    pt.commit()
    pt.alloc_chunk()
    pt.commit()
    pt.alloc_chunk()
    before = (pt.export().tolist(), pt.num_free())
    pt.commit()  # evicts the first chunk
    assert pt.export().tolist()[0] != ids.tolist()
    pt.alloc_chunk()
    pt.commit()
    # 10 pages, window 2: 6 resident, 4 free; one more live chunk leaves 1
    pt.alloc_chunk()
    assert pt.num_free() == 1
    pt.commit()
    assert pt.num_free() == 4
    del before

    small = wf.PageTable(5, 16, 40, 2)  # room for one chunk, then ENOMEM
    small.alloc_chunk()
    small.commit()
    state = (small.export().tolist(), small.num_free())
    with pytest.raises(wf.WfError) as e:
        small.alloc_chunk()
    assert e.value.status == CODES["ENOMEM"]
    assert (small.export().tolist(), small.num_free()) == state
    assert "free pages" in wf.last_error()


def _driver_script(N, P, T, W, pin, order, ticks, caps):
    lines = [f"create {N} {P} {T} {W} {int(pin)} {1 if order is not None else 0}"
             + ("" if order is None else " " + " ".join(str(int(x)) for x in order)), "ppc"]
    for k in range(ticks):
        cap_a, cap_c, cap_e = caps(k)
        lines += [f"alloc {cap_a}", "free", f"commit {cap_c}", f"export {cap_e}", "free"]
    return "\n".join(lines) + "\n"


def _model_replay(N, P, T, W, pin, order, ticks, caps):
    """Expected driver output, from the oracle model and the documented error rules."""
    out = []
    try:
        m = oracle.FifoPageModel(N, P, T, W, pin_anchor=pin, initial_free_order=order)
        out.append("create 0")
    except PageModelError as e:
        return [f"create {CODES[e.code]}"]
    out.append(f"ppc 0 {m.ppc}")
    for k in range(ticks):
        cap_a, cap_c, cap_e = caps(k)
        if cap_a < m.ppc:
            out.append(f"alloc {CODES['EINVAL']}")
        else:
            try:
                ids = m.alloc_chunk()
                out.append("alloc 0 " + " ".join(map(str, ids)))
            except PageModelError as e:
                out.append(f"alloc {CODES[e.code]}")
        out.append(f"free 0 {m.num_free()}")
        will_evict = m.live is not None and len(m.history) + 1 > m.window
        if m.live is None:
            out.append(f"commit {CODES['ESTATE']} -1")
        elif will_evict and 0 < cap_c < m.ppc:
            out.append(f"commit {CODES['EINVAL']} -1")
        else:
            ev = m.commit()
            shown = " " + " ".join(map(str, ev)) if (cap_c > 0 and ev) else ""
            out.append(f"commit 0 {len(ev)}{shown}")
        need = len(m.history) * m.ppc
        if need > 0 and cap_e < need:
            out.append(f"export {CODES['EINVAL']} -1")
        else:
            flat = [p for c in m.export() for p in c]
            out.append(f"export 0 {len(m.history)}" + ("".join(f" {p}" for p in flat)))
        out.append(f"free 0 {m.num_free()}")
    return out


def test_page_table_under_sanitizers(tmp_path):
    """The page table built with g++ -fsanitize=address,undefined, driven through
    a long schedule with interleaved error calls; output equals the model's."""
    exe = str(tmp_path / "page_table_driver")
    try:
        build_lib.build_host_page_table_test(exe)
    except RuntimeError as e:
        pytest.skip(f"sanitizer build unavailable: {e}")
    cases = [
        (4096, 64, 4680, 3, False, inputs.initial_free_order(inputs.CONFIGS["wan13_4step"]), 60,
         lambda k: (74, 74, 4 * 74)),
        (4096, 64, 4680, 3, True, None, 60, lambda k: (74, 74 if k % 3 else 0, 4 * 74)),
        (10, 16, 40, 2, False, np.random.default_rng(3).permutation(10), 40,
         lambda k: (3 if k % 5 else 2, 3 if k % 7 else 1, 6 if k % 4 else 3)),
        (5, 16, 40, 2, True, None, 12, lambda k: (3, 3, 9)),
    ]
    for N, P, T, W, pin, order, ticks, caps in cases:
        script = _driver_script(N, P, T, W, pin, order, ticks, caps)
        res = subprocess.run([exe], input=script, capture_output=True, text=True, timeout=120)
        assert res.returncode == 0, res.stderr[-2000:]
        got = res.stdout.strip().splitlines()
        want = _model_replay(N, P, T, W, pin, order, ticks, caps)
        assert got == want


# ---------------------------------------------------------------------------
# validation (returns before any device work) and the FLOP count
# ---------------------------------------------------------------------------
def _desc(wf, **kw):
    a = dict(S=4, active_mask=0x1F, T=4680, H=12, D=128, scale=1.0 / np.sqrt(128), q=None, k=None,
             v=None, o=None, k_pool=None, v_pool=None, num_pages=4096, P=64, hist_pages=None,
             n_hist=0)
    a.update(kw)
    return wf.make_tick_desc(a["S"], a["active_mask"], a["T"], a["H"], a["D"], a["scale"], a["q"],
                             a["k"], a["v"], a["o"], a["k_pool"], a["v_pool"], a["num_pages"],
                             a["P"], a["hist_pages"], a["n_hist"])


@pytest.mark.parametrize("kw,code", [
    (dict(S=8, active_mask=1), "EINVAL"),
    (dict(S=-1, active_mask=0), "EINVAL"),
    (dict(S=2, active_mask=0x10), "EINVAL"),
    (dict(T=-1), "EINVAL"),
    (dict(H=0), "EINVAL"),
    (dict(D=96), "EUNSUPPORTED"),
    (dict(scale=0.0), "EINVAL"),
    (dict(scale=float("inf")), "EINVAL"),
    (dict(n_hist=-1), "EINVAL"),
    (dict(n_hist=28), "EUNSUPPORTED"),
])
def test_tick_validation(kw, code):
    wf = _wfattn()
    d = _desc(wf, **kw)
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES[code]
    with pytest.raises(wf.WfError) as e:
        wf.tick_useful_flops_desc(d)
    assert e.value.status == CODES[code]


def test_tick_validation_pointers_and_pool():
    wf = _wfattn()
    # missing tensors for a non-empty tick
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_tick_desc(_desc(wf), stream=0)
    assert e.value.status == CODES["EINVAL"]
    fake = 1 << 20  # never dereferenced: validation fails first
    base = dict(q=fake, k=fake, v=fake, o=fake)
    with pytest.raises(wf.WfError) as e:  # misaligned q
        wf.wf_attn_tick_desc(_desc(wf, **{**base, "q": fake + 2}), stream=0)
    assert e.value.status == CODES["EINVAL"]
    with pytest.raises(wf.WfError) as e:  # history without pools
        wf.wf_attn_tick_desc(_desc(wf, **base, n_hist=3), stream=0)
    assert e.value.status == CODES["EINVAL"]
    pools = dict(k_pool=fake, v_pool=fake, hist_pages=fake)
    with pytest.raises(wf.WfError) as e:  # page size not a multiple of 16
        wf.wf_attn_tick_desc(_desc(wf, **base, **pools, n_hist=3, P=40), stream=0)
    assert e.value.status == CODES["EINVAL"]
    with pytest.raises(wf.WfError) as e:  # pool too small for the history
        wf.wf_attn_tick_desc(_desc(wf, **base, **pools, n_hist=3, num_pages=100), stream=0)
    assert e.value.status == CODES["EINVAL"]
    with pytest.raises(wf.WfError) as e:  # page table larger than the LDS budget
        wf.wf_attn_tick_desc(_desc(wf, **base, **pools, n_hist=3, P=16, T=60000,
                                   num_pages=40000), stream=0)
    assert e.value.status == CODES["EUNSUPPORTED"]
    with pytest.raises(wf.WfError) as e:  # tile-source table larger than the LDS budget
        wf.wf_attn_tick_desc(_desc(wf, **base, **pools, n_hist=25, num_pages=2000), stream=0)
    assert e.value.status == CODES["EUNSUPPORTED"]
    assert "tiles" in wf.last_error()
    # empty ticks are accepted without touching the device
    wf.wf_attn_tick_desc(_desc(wf, T=0), stream=0)
    wf.wf_attn_tick_desc(_desc(wf, active_mask=0), stream=0)


def test_store_gather_validation():
    wf = _wfattn()
    lib = wf.library()
    fake = 1 << 20
    # NULL sources, bad sizes, misalignment: all rejected on the host
    assert lib.wf_store_paged(None, fake, fake, fake, fake, 64, 2, 64, 8, 16, None) == CODES["EINVAL"]
    assert lib.wf_store_paged(fake, fake, fake, fake, fake, 64, 1, 4, 8, 16, None) == CODES["EINVAL"]
    assert lib.wf_store_paged(fake, fake, fake, fake, fake, -1, 2, 64, 8, 16, None) == CODES["EINVAL"]
    assert lib.wf_store_paged(fake + 2, fake, fake, fake, fake, 64, 2, 64, 8, 16, None) == CODES["EINVAL"]
    assert lib.wf_store_paged(fake, fake, fake, fake, fake, 64, 2, 64, 2, 16, None) == CODES["EINVAL"]
    assert lib.wf_gather_paged(fake, fake, None, 1, fake, fake, 64, 2, 64, 8, 16, None) == CODES["EINVAL"]
    assert lib.wf_gather_paged(fake, fake, fake, -1, fake, fake, 64, 2, 64, 8, 16, None) == CODES["EINVAL"]
    # zero-size calls are no-ops
    assert lib.wf_store_paged(None, None, None, None, None, 0, 2, 64, 8, 16, None) == 0
    assert lib.wf_gather_paged(None, None, None, 3, None, None, 0, 2, 64, 8, 16, None) == 0


def test_tick_validation_live_pages():
    """A fully paged tick needs the pools but not k and v; the page-id budget of
    the non-64-multiple page path counts the live slots' pages too."""
    wf = _wfattn()
    fake = 1 << 20
    d = _desc(wf, q=fake, o=fake)
    d.live_pages = fake
    with pytest.raises(wf.WfError) as e:  # no pools
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES["EINVAL"]
    d = _desc(wf, q=fake, o=fake, k_pool=fake, v_pool=fake, num_pages=50)
    d.live_pages = fake
    with pytest.raises(wf.WfError) as e:  # a chunk needs 74 pages, the pool has 50
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES["EINVAL"]
    d = _desc(wf, q=fake, o=fake, k_pool=fake, v_pool=fake, P=16, T=9000, num_pages=40000,
              hist_pages=fake, n_hist=3)
    d.live_pages = fake
    # (3 + 5) * 563 page ids > 4096 (3 * 563 alone would fit)
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES["EUNSUPPORTED"]
    assert "page table" in wf.last_error()
    # the fused store excludes paged live slots and needs the store slot active
    d = _desc(wf, q=fake, k=fake, v=fake, o=fake, k_pool=fake, v_pool=fake)
    d.live_pages = fake
    d.store_pages = fake
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES["EINVAL"]
    d = _desc(wf, q=fake, k=fake, v=fake, o=fake, k_pool=fake, v_pool=fake, active_mask=0x0F)
    d.store_pages = fake
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES["EINVAL"]
    # without live_pages k and v are still required
    d = _desc(wf, q=fake, o=fake, k_pool=fake, v_pool=fake)
    with pytest.raises(wf.WfError) as e:
        wf.wf_attn_tick_desc(d, stream=0)
    assert e.value.status == CODES["EINVAL"]


def test_rope_store_validation():
    wf = _wfattn()
    lib = wf.library()
    fake = 1 << 20

    def call(T=4680, H=12, D=128, num_pages=4096, P=64, grid=(3, 30, 52), frame0=0,
             split=(44, 42, 42), theta=10000.0, k=fake, v=fake, kp=fake, vp=fake, ids=fake,
             null_desc=False):
        r = None if null_desc else wf.make_rope_desc(grid, frame0, split, theta, D)
        return lib.wf_rope_store_paged(k, v, kp, vp, ids, T, H, D, num_pages, P,
                                       None if r is None else __import__("ctypes").byref(r), None)

    E, U = CODES["EINVAL"], CODES["EUNSUPPORTED"]
    assert call(null_desc=True) == E
    assert call(grid=(3, 30, 51)) == E          # does not hold T tokens
    assert call(grid=(0, 30, 52)) == E
    assert call(frame0=-1) == E
    assert call(frame0=(1 << 24) - 2) == E      # frame coordinates past 2^24
    assert call(split=(43, 43, 42)) == E        # odd parts
    assert call(split=(44, 42, 40)) == E        # sum != D
    assert call(theta=0.0) == E
    assert call(theta=float("nan")) == E
    assert call(D=96, split=(32, 32, 32)) == U
    assert call(k=None) == E
    assert call(v=None) == E                    # v_src without v_pool or the reverse
    assert call(kp=fake + 8) == E               # misaligned
    assert call(num_pages=10) == E              # the chunk needs 74 pages
    assert call(T=0, grid=(1, 1, 1)) == 0       # empty chunk: no-op


@pytest.mark.parametrize("name", ["tiny", "wan13_4step", "wan13_5step", "wan14b_4step"])
def test_useful_flops_matches_oracle(name):
    wf = _wfattn()
    c = inputs.CONFIGS[name]
    full = (1 << (c.S + 1)) - 1
    for mask in {full, full & ~1, 1 << c.S, full >> 1, 0b101 & full}:
        got = wf.wf_tick_useful_flops(c.S, mask, c.T, c.H, c.D, c.n_hist, P=c.P,
                                      num_pages=c.num_pages)
        want = oracle.useful_flops(c.S, mask, c.n_hist, c.T, c.H, c.D)
        assert got == want, (name, mask)
    if name == "wan13_4step":
        assert abs(wf.wf_tick_useful_flops(c.S, full, c.T, c.H, c.D, c.n_hist, P=c.P,
                                           num_pages=c.num_pages) - 4.037e12) < 1e9


def test_tick_validation_fp8_keys():
    """The 8-bit tier: k_format and v_format must be known; e4m3 keys need D =
    128, P a multiple of 64, live_pages, k_scale (4-byte aligned) and no fused
    store; e4m3 values need e4m3 keys and v_exp."""
    wf = _wfattn()
    fake = 1 << 20

    def desc(**kw):
        base = dict(q=fake, o=fake, k_pool=fake, v_pool=fake)
        live = kw.pop("live", True)
        fmt = kw.pop("k_format", wf.K_E4M3)
        scale = kw.pop("k_scale", fake)
        store = kw.pop("store", False)
        d = _desc(wf, **{**base, **kw})
        if live:
            d.live_pages = fake
        if store:
            d.store_pages = fake
        d.k_format = fmt
        d.k_scale = scale
        return d

    def desc_v(v_format, k_format=None, v_exp=fake):
        d = desc() if k_format is None else desc(k_format=k_format)
        d.v_format = v_format
        d.v_exp = v_exp
        return d

    for d, code in ((desc_v(2), "EINVAL"),                        # unknown value format
                    (desc_v(1, k_format=0), "EINVAL"),            # 8-bit values need 8-bit keys
                    (desc_v(1, v_exp=None), "EINVAL")):           # 8-bit values need v_exp
        with pytest.raises(wf.WfError) as e:
            wf.wf_attn_tick_desc(d, stream=0)
        assert e.value.status == CODES[code], wf.last_error()
    for d, code in ((desc(k_format=2), "EINVAL"),
                    (desc(D=64), "EUNSUPPORTED"),
                    (desc(P=16), "EINVAL"),
                    (desc(live=False, k=fake, v=fake), "EINVAL"),
                    (desc(store=True, k=fake, v=fake), "EINVAL"),
                    (desc(k_scale=None), "EINVAL"),
                    (desc(k_scale=fake + 2), "EINVAL")):
        with pytest.raises(wf.WfError) as e:
            wf.wf_attn_tick_desc(d, stream=0)
        assert e.value.status == CODES[code], wf.last_error()
    wf.wf_attn_tick_desc(desc(T=0), stream=0)  # empty tick: no-op


def test_store_fp8_validation():
    wf = _wfattn()
    lib = wf.library()
    fake = 1 << 20

    def call(T=4680, H=12, D=128, num_pages=4096, P=64, k=fake, v=fake, kp=fake, ks=fake,
             vp=fake, ids=fake):
        return lib.wf_store_paged_fp8(k, v, kp, ks, vp, None, ids, T, H, D, num_pages, P, None)

    E, U = CODES["EINVAL"], CODES["EUNSUPPORTED"]
    assert call(P=96) == E                      # scale tiles of 64 tokens must tile a page
    assert call(P=0) == E
    assert call(T=-1) == E
    assert call(D=96) == U
    assert call(ks=None) == E
    assert call(ids=None) == E
    assert call(ks=fake + 2) == E               # scales not 4-byte aligned
    assert call(kp=fake + 8) == E               # codes not 16-byte aligned
    assert call(num_pages=10) == E              # the chunk needs 74 pages
    assert call(T=0, k=None, v=None, kp=None, ks=None, vp=None, ids=None) == 0


# ---------------------------------------------------------------------------
# The Python binding refuses, before any library call, arguments whose element
# type, layout or shape do not match what the call reads and writes (the
# library trusts sizes and device page ids). CPU tensors suffice: every check
# here runs before the check that tensors live on the GPU, which is tested last.
# ---------------------------------------------------------------------------
def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _ids(*shape, dtype=None):
    return torch.zeros(shape, dtype=dtype or torch.int32)


def test_binding_rejects_bad_store_and_gather_arguments():
    wf = _wfattn()
    T, H, D, P, N = 100, 2, 64, 16, 20
    ppc = -(-T // P)
    k, kp = _bf(T, H, D), _bf(N, P, H, D)
    cases = [
        (TypeError, lambda: wf.wf_store_paged(k, k, kp, kp, _ids(ppc, dtype=torch.int64))),
        (ValueError, lambda: wf.wf_store_paged(k, k, kp, kp, _ids(ppc + 1))),
        (ValueError, lambda: wf.wf_store_paged(k, k, kp, kp, _ids(ppc, 1))),
        (ValueError, lambda: wf.wf_store_paged(k, k, kp, kp, _ids(2 * ppc)[::2])),
        (ValueError, lambda: wf.wf_store_paged(k, k, _bf(N, P, H, 2 * D), _bf(N, P, H, 2 * D),
                                               _ids(ppc))),                       # pool's D
        (ValueError, lambda: wf.wf_store_paged(k, k, _bf(N, P, H + 1, D), _bf(N, P, H + 1, D),
                                               _ids(ppc))),                       # pool's H
        (ValueError, lambda: wf.wf_store_paged(k, _bf(T + 1, H, D), kp, kp, _ids(ppc))),
        (ValueError, lambda: wf.wf_store_paged(k, k, kp, _bf(N + 1, P, H, D), _ids(ppc))),
        (TypeError, lambda: wf.wf_store_paged(k.float(), k, kp, kp, _ids(ppc))),
        (ValueError, lambda: wf.wf_store_paged(k, k, kp, kp, _ids(ppc))),         # on the CPU
        (ValueError, lambda: wf.wf_gather_paged(kp, kp, _ids(ppc), _bf(1, T, H, D),
                                                _bf(1, T, H, D))),               # ids not [n][ppc]
        (TypeError, lambda: wf.wf_gather_paged(kp, kp, _ids(1, ppc, dtype=torch.int64),
                                               _bf(1, T, H, D), _bf(1, T, H, D))),
        (ValueError, lambda: wf.wf_gather_paged(kp, kp, _ids(1, ppc), _bf(1, T, H, D),
                                                _bf(2, T, H, D))),
        (ValueError, lambda: wf.wf_rope_store_paged(k, k, kp, None, _ids(ppc), (T, 1, 1), 0)),
        (TypeError, lambda: wf.wf_rope_store_paged(k, None, kp, None,
                                                   _ids(ppc, dtype=torch.int64), (T, 1, 1), 0)),
        (ValueError, lambda: wf.wf_rope_store_paged(k, None, _bf(N, P, H, D + 2), None,
                                                    _ids(ppc), (T, 1, 1), 0)),
    ]
    for exc, call in cases:
        with pytest.raises(exc):
            call()


def test_binding_rejects_bad_fp8_store_arguments():
    wf = _wfattn()
    T, H, D, P, N = 100, 2, 128, 64, 6
    ppc = -(-T // P)
    k = _bf(T, H, D)
    kc = torch.zeros((N, P, H, D), dtype=torch.uint8)
    ks = torch.zeros((N, P // 64, H), dtype=torch.float32)
    vb = _bf(N, P, H, D)
    v8 = torch.zeros((N, P // 64, H, D, 64), dtype=torch.uint8)
    ve = torch.zeros((N, P // 64, H), dtype=torch.uint8)
    cases = [
        (TypeError, lambda: wf.wf_store_paged_fp8(k, k, vb, ks, vb, _ids(ppc))),   # K not uint8
        (TypeError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks.double(), vb, _ids(ppc))),
        (ValueError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks[:, :, :1].contiguous(), vb,
                                                   _ids(ppc))),
        (TypeError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, v8, _ids(ppc))),   # 8-bit V, no v_exp
        (TypeError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, vb, _ids(ppc), v_exp=ve)),
        (ValueError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, v8[:, :, :, :64].contiguous(),
                                                   _ids(ppc), v_exp=ve)),          # V layout
        (ValueError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, v8, _ids(ppc),
                                                   v_exp=ve[:, :, :1].contiguous())),
        (TypeError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, vb, _ids(ppc, dtype=torch.int64))),
        (ValueError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, vb, _ids(ppc + 1))),
        (ValueError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, vb, _ids(ppc))),  # on the CPU
        (ValueError, lambda: wf.wf_store_paged_fp8(k, k, kc, ks, v8, _ids(ppc), v_exp=ve)),
    ]
    for exc, call in cases:
        with pytest.raises(exc):
            call()


def test_binding_rejects_bad_tick_arguments():
    wf = _wfattn()
    S, T, H, D, P, N, nh = 2, 100, 2, 64, 16, 40, 2
    ppc = -(-T // P)
    q = _bf(S + 1, T, H, D)
    kp = _bf(N, P, H, D)
    hist = _ids(nh, ppc)

    def tick(**kw):
        args = dict(q=q, k=q, v=q, o=q, S=S, active_mask=0b111, scale=0.125, k_pool=kp,
                    v_pool=kp, hist_pages=hist)
        args.update(kw)
        wf.wf_attn_tick(**args)

    cases = [
        (ValueError, dict(S=S + 1)),                                   # q not [S+1][T][H][D]
        (ValueError, dict(o=_bf(S + 1, T, H, D + 64))),
        (ValueError, dict(k=_bf(S + 1, T + 1, H, D))),
        (TypeError, dict(v=q.float())),
        (TypeError, dict(hist_pages=_ids(nh, ppc, dtype=torch.int64))),   # int64 page ids
        (ValueError, dict(hist_pages=_ids(nh, ppc + 1))),
        (ValueError, dict(hist_pages=_ids(nh * ppc))),                  # flat, not [n][ppc]
        (ValueError, dict(hist_pages=_ids(nh, 2 * ppc)[:, ::2])),       # not contiguous
        (ValueError, dict(k_pool=_bf(N, P, H, 2 * D), v_pool=_bf(N, P, H, 2 * D))),  # pool's D
        (ValueError, dict(v_pool=_bf(N, P, H + 1, D))),                 # pool's H
        (ValueError, dict(k_pool=None)),
        (TypeError, dict(store_pages=_ids(ppc, dtype=torch.int64))),
        (ValueError, dict(store_pages=_ids(ppc - 1))),
        (ValueError, dict(k=None, v=None, live_pages=_ids(S, ppc))),    # not [S+1][ppc]
        (TypeError, dict(k=None, v=None, live_pages=_ids(S + 1, ppc),
                         k_scale=torch.zeros((N, 1, H)))),             # 8-bit keys, bf16 pool
        (ValueError, dict()),                                           # right, but on the CPU
    ]
    for exc, kw in cases:
        with pytest.raises(exc):
            tick(**kw)


def test_tick_validation_workspace():
    """A workspace must be 256-byte aligned with workspace_bytes >= 0 (bytes
    without a pointer are ignored); wf_tick_workspace_bytes validates like the
    launch and refuses a NULL result pointer."""
    import ctypes
    wf = _wfattn()
    fake = 1 << 20

    def desc(ws, nb):
        d = _desc(wf, q=fake, k=fake, v=fake, o=fake)
        d.workspace = ws
        d.workspace_bytes = nb
        return d

    for d in (desc(fake + 128, 1 << 20), desc(fake, -1)):
        with pytest.raises(wf.WfError) as e:
            wf.wf_attn_tick_desc(d, stream=0)
        assert e.value.status == CODES["EINVAL"], wf.last_error()
    assert wf.library().wf_tick_workspace_bytes(ctypes.byref(desc(None, 0)), None) == CODES["EINVAL"]
    bad = desc(None, 0)
    bad.H = 0
    with pytest.raises(wf.WfError):
        wf.tick_workspace_bytes(bad)
    assert wf.tick_workspace_bytes(desc(None, 0)) >= 0


def test_noalloc_validation():
    """wf_attn_tick_noalloc refuses a workspace pointer and workspace_bytes
    outside [0, WF_NOALLOC_SCRATCH_BYTES] before touching the device."""
    import ctypes
    wf = _wfattn()
    fake = 1 << 20
    declared = re.search(r"#define WF_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", open(HEADER).read())
    assert int(declared.group(1)) << int(declared.group(2)) == wf.NOALLOC_SCRATCH_BYTES
    for ws, nb in ((fake, 1 << 20), (None, wf.NOALLOC_SCRATCH_BYTES + 1), (None, -1)):
        d = _desc(wf, q=fake, k=fake, v=fake, o=fake)
        d.workspace = ws
        d.workspace_bytes = nb
        assert wf.library().wf_attn_tick_noalloc(ctypes.byref(d), None) == CODES["EINVAL"]
        assert "wf_attn_tick_noalloc" in wf.last_error()
