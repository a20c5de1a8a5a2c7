#!/usr/bin/env python3
"""Throughput of the wave-tick hot path on one MI355X.

One step = one steady-state tick of the streaming rollout at the Wan-1.3B-like
4-step shape (S = 4: five 4680-token chunks incl. the store, 12 heads x 128,
bf16, 3 clean history chunks in 64-token pages of a 4096-page pool):
  page-table alloc of the store chunk's pages (host) -> page ids to the device
  -> history table to the device -> wf_attn_tick (all five query chunks and
  the store chunk's page write, one launch) -> commit (promote the store
  chunk, evict the oldest history chunk, host).
Inputs are resident in HBM before the timed region (seeded device RNG).

Prints one JSON line. `value` = useful TFLOP/s of the whole step (mask-true
query-key pairs x 4*D flops x H); `roofline` = the attention kernel alone,
timed with HIP events on its launch stream; `cpu_baseline` = the fp64 CPU
oracle on a bounded sample of the same tick. Also reported: the same tick with
a separate store launch, the store and rotary-store kernels' bandwidth, the
fully paged flow (every live chunk rotated into pages, attention reading the
whole context through pages), the 8-bit tiers, the 5-step and 14B-like ticks
(`configs`) and the 120-tick streaming rollout timed whole (`rollout120`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# 8-bit tier: Q.K^T (half the useful flops) on fp8 MFMA, P.V on bf16 MFMA, so
# the time floor is F/2 / 5000 + F/2 / 2500 and the blended peak 3333 TFLOP/s.
PEAK_FP8_TIER_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Bandwidth kernels are timed over this many distinct source chunks and page
# sets, launched in turn: at the 1.3B shape the sources alone take 24 x 28.75 MB
# = 690 MB, well above the 256 MB last-level cache, so each launch reads its
# inputs from HBM rather than from the cache the previous launches filled.
ROTATION = 24

# HBM traffic of the attention kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes (scaled by a plain-copy calibration), recorded with a hash of the
# kernel's sources and build flags; reported only while that hash still matches.
COUNTERS_FILE = os.path.join(ROOT, "profiles", "wf_attn_tick_wan13_4step_counters.md")


def attn_kernel_hash() -> str:
    """sha256 of the attention kernel's sources (comments and whitespace removed)
    and the build flags."""
    import hashlib
    import re

    from wavefront_causal_attention_wf_amd import build_lib

    h = hashlib.sha256()
    paths = [os.path.join(build_lib.CSRC, "wf_attn.hip"), os.path.join(build_lib.CSRC, "wf_internal.h"),
             os.path.join(build_lib.INCLUDE, "wf_attn.h")]
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    h.update(" ".join(build_lib.HIP_FLAGS).encode())
    return h.hexdigest()


def recorded_traffic(config_name: str):
    """(bytes per launch, note) from the committed counter summary, or (None, why)."""
    if config_name != "wan13_4step":
        return None, "counters recorded for wan13_4step only"
    try:
        text = open(COUNTERS_FILE).read()
    except OSError:
        return None, "no counter summary"
    vals = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0] in ("kernel_sha256", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    if vals.get("kernel_sha256") != attn_kernel_hash():
        return None, "kernel changed since the counters were taken"
    return int(vals["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


PEAK_CLOCK_MHZ = 2400.0     # the clock the MFMA peaks are quoted at


def power_window(step, seconds: float = 1.5, sync=None) -> dict:
    """Socket power and GFX clocks while `step` (one tick) runs back to back
    for `seconds`: the amdsmi GPU metrics table (the first GPU it lists, the
    only one on a one-GPU machine), read every 0.1 s after the first 0.4 s.
    Reading it changes nothing on the GPU. Returns the medians over the
    samples (per XCD for the clocks; entries outside 100-5000 MHz, which the
    table uses for absent XCDs, are dropped), or an error note where the
    library or the metrics are not available. `sync` waits for the device
    (torch.cuda.synchronize unless given)."""
    import threading

    if sync is None:
        import torch

        sync = torch.cuda.synchronize
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # no amdsmi, no driver access: report, do not fail the bench
        return {"error": f"amdsmi unavailable: {str(e)[:160]}"}
    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(0.4)
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            except Exception:
                break
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 100 <= c <= 5000]
            pw = m.get("current_socket_power")
            if isinstance(pw, (int, float)) and clks:
                samples.append((float(pw), clks))
            time.sleep(0.1)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    ticks = 0
    while time.perf_counter() - t0 < seconds:
        step()
        ticks += 1
    sync()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not samples:
        return {"error": "no power or clock samples from the GPU metrics table"}
    n_xcd = min(len(c) for _, c in samples)
    per_xcd = [float(np.median([c[i] for _, c in samples])) for i in range(n_xcd)]
    return {"source": "amdsmi GPU metrics, sampled while the tick ran back to back",
            "ticks": ticks, "samples": len(samples),
            "socket_power_w": float(np.median([p for p, _ in samples])),
            "gfx_clk_mhz_per_xcd": per_xcd,
            "gfx_clk_mhz_mean": round(float(np.mean(per_xcd)), 1)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="wan13_4step",
                    choices=["wan13_4step", "wan13_5step", "wan14b_4step"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0,
                    help="approximate CPU seconds for the oracle sample")
    ap.add_argument("--rotate", type=int, default=4, help="distinct live-input sets cycled")
    ap.add_argument("--kernel-hash", action="store_true",
                    help="print the attention kernel's source hash (recorded with its counters)")
    ap.add_argument("--mode", default="tick",
                    choices=["tick", "attn", "store", "rope", "paged", "copy", "fp8", "fp8kv",
                             "store8"],
                    help="tick: the full hot path (default, prints the JSON line); attn / "
                         "store / rope / fp8 (8-bit tier attention) / store8 (8-bit tier "
                         "producer write): only that kernel, --steps launches (for profilers); "
                         "paged: --steps ticks of the fully paged flow; copy: a plain 1 GiB "
                         "device copy (calibrates HBM byte counters)")
    return ap.parse_args()


def tick_workspace(cfg, dev, live_paged: bool = False):
    """The attention launch's workspace (run-time pool) for the configuration's
    full-width tick, or None where the tick takes none."""
    import torch

    from wavefront_causal_attention_wf_amd import wfattn

    nb = wfattn.workspace_bytes(cfg.S, (1 << (cfg.S + 1)) - 1, cfg.T, cfg.H, cfg.D,
                                max(cfg.n_hist, 1), None, cfg.P, cfg.num_pages,
                                live_paged=live_paged)
    return torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None


class Rollout:
    """Device state of a steady-state rollout: pools, page table, live inputs."""

    def __init__(self, cfg, rotate: int, dev, fused: bool = True):
        import torch

        from wavefront_causal_attention_wf_amd import inputs, wfattn

        self.torch, self.wf, self.cfg, self.dev = torch, wfattn, cfg, dev
        self.fused = fused
        S, T, H, D, P = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P
        self.order = inputs.initial_free_order(cfg)
        self.pt = wfattn.PageTable(cfg.num_pages, P, T, cfg.n_hist,
                                   initial_free_order=self.order)
        self.k_pool = torch.zeros((cfg.num_pages, P, H, D), dtype=torch.bfloat16, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.ppc = self.pt.ppc
        # ring of pinned host slots for the per-step page-id uploads
        self.nslot = 8
        self.ids_host = torch.empty((self.nslot, self.ppc), dtype=torch.int32, pin_memory=True)
        self.hist_host = torch.empty((self.nslot, cfg.n_hist * self.ppc), dtype=torch.int32,
                                     pin_memory=True)
        self.ids_dev = torch.empty((self.nslot, self.ppc), dtype=torch.int32, device=dev)
        self.hist_dev = torch.empty((self.nslot, cfg.n_hist, self.ppc), dtype=torch.int32,
                                    device=dev)
        self.slot_ev = [None] * self.nslot
        self.step_i = 0
        # history: n_hist clean chunks written through the store path
        for c in range(cfg.n_hist):
            hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, dev)
            ids = torch.from_numpy(self.pt.alloc_chunk()).to(dev)
            wfattn.wf_store_paged(hk[0], hv[0], self.k_pool, self.v_pool, ids)
            self.pt.commit()
        self.live = [inputs.draw_live_torch(cfg, inputs.rollout_seed(i), dev)
                     for i in range(rotate)]
        self.o = torch.empty_like(self.live[0][0])
        self.scale = 1.0 / float(np.sqrt(D))
        self.mask = (1 << (S + 1)) - 1
        self.ws = tick_workspace(cfg, dev)
        torch.cuda.synchronize()

    def step(self, attn_events=None):
        torch, wf, cfg = self.torch, self.wf, self.cfg
        slot = self.step_i % self.nslot
        if self.slot_ev[slot] is not None:
            self.slot_ev[slot].synchronize()
        q, k, v = self.live[self.step_i % len(self.live)]
        self.step_i += 1
        S = cfg.S
        ids = self.pt.alloc_chunk()
        self.ids_host[slot].numpy()[:] = ids
        self.ids_dev[slot].copy_(self.ids_host[slot], non_blocking=True)
        if not self.fused:
            wf.wf_store_paged(k[S], v[S], self.k_pool, self.v_pool, self.ids_dev[slot])
        hist = self.pt.export()
        self.hist_host[slot].numpy()[:] = hist.reshape(-1)
        self.hist_dev[slot].view(-1).copy_(self.hist_host[slot], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.slot_ev[slot] = ev
        if attn_events is not None:
            attn_events[0].record()
        wf.wf_attn_tick(q, k, v, self.o, S, self.mask, self.scale, self.k_pool, self.v_pool,
                        self.hist_dev[slot],
                        store_pages=self.ids_dev[slot] if self.fused else None,
                        workspace=self.ws)
        if attn_events is not None:
            attn_events[1].record()
        self.pt.commit()


def separate_store_step(cfg, dev, steps: int = 10, warmup: int = 3) -> dict:
    """The same tick with the store chunk written by its own wf_store_paged launch
    before the attention launch (two launches per tick)."""
    import torch

    ro = Rollout(cfg, 2, dev, fused=False)
    for _ in range(warmup):
        ro.step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        ro.step(ev[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    attn = float(np.mean([x.elapsed_time(y) for x, y in ev]))
    return {"flow": "wf_store_paged + wf_attn_tick (two launches)", "ms_per_step": round(ms, 4),
            "attn_kernel_ms_mean": round(attn, 4)}


def graph_time_ms(fn, rotation: int, launches: int) -> float:
    """Mean device time per launch of fn(0), fn(1), ... (fn(i) launches one
    kernel on the current stream): `launches` launches captured once in a HIP
    graph and replayed, HIP events around the replays, so the host's per-call
    cost (argument checks, ctypes) does not pace launches of ~10 us."""
    import torch

    for i in range(rotation):  # warm, and nothing lazy left for the capture
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * launches)
    del g
    return ms


def store_bandwidth(cfg, dev, launches: int = 96, rotation: int = ROTATION) -> dict:
    """wf_store_paged and wf_gather_paged alone (graph_time_ms).

    cold: rotating over `rotation` distinct source chunks and page sets (the
    sources alone exceed the 256 MB last-level cache); warm: one chunk and page set
    repeated; copy: a plain device-to-device copy of the store's byte count (the
    achievable ceiling for a read+write stream of that size)."""
    import torch

    from wavefront_causal_attention_wf_amd import inputs, wfattn

    T, H, D, P = cfg.T, cfg.H, cfg.D, cfg.P
    ppc = cfg.ppc
    pool_pages = max(cfg.num_pages, rotation * ppc)
    kp = torch.zeros((pool_pages, P, H, D), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    srcs = [inputs.draw_live_torch(cfg, 3000 + i, dev, T=T)[0] for i in range(rotation)]
    ksrc = [x[0].clone() for x in srcs]
    vsrc = [x[1].clone() for x in srcs]
    del srcs
    order = torch.from_numpy(inputs.initial_free_order(
        inputs.TickConfig("rot", S=0, T=T, H=H, D=D, P=P, n_hist=0, num_pages=pool_pages,
                          std=0.5, bf16_inputs=True, page_order="permutation")))
    ids = [order[i * ppc:(i + 1) * ppc].to(torch.int32).to(dev) for i in range(rotation)]
    kd = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=dev)
    vd = torch.empty_like(kd)

    def timed(fn) -> float:
        return graph_time_ms(fn, rotation, launches)

    store_cold = timed(lambda i: wfattn.wf_store_paged(ksrc[i % rotation], vsrc[i % rotation],
                                                       kp, vp, ids[i % rotation]))
    store_warm = timed(lambda i: wfattn.wf_store_paged(ksrc[0], vsrc[0], kp, vp, ids[0]))
    gather_cold = timed(lambda i: wfattn.wf_gather_paged(kp, vp, ids[i % rotation].view(1, ppc),
                                                         kd, vd))
    # a tick's S+1 chunks out of their pages in one launch (page sets rotated)
    n = cfg.S + 1
    ids_n = [torch.stack([ids[(i * n + c) % rotation] for c in range(n)]) for i in range(rotation)]
    kd_n = torch.empty((n, T, H, D), dtype=torch.bfloat16, device=dev)
    vd_n = torch.empty_like(kd_n)
    gather_n = graph_time_ms(lambda i: wfattn.wf_gather_paged(kp, vp, ids_n[i % rotation], kd_n, vd_n),
                             rotation, launches // 4)
    nbytes = 2 * (T * H * D * 2) + 2 * (ppc * P * H * D * 2)   # read K,V + write whole pages
    gbytes = 4 * (T * H * D * 2)   # read the K,V tokens from their pages + write them
    # a copy of nbytes / 2 bytes moves nbytes (read + write)
    csrc = [torch.empty(nbytes // 4, dtype=torch.int16, device=dev) for _ in range(rotation)]
    cdst = [torch.empty_like(x) for x in csrc]
    copy_cold = timed(lambda i: cdst[i % rotation].copy_(csrc[i % rotation]))

    def rate(nb, ms):
        return round(nb / (ms * 1e-3) / 1e9, 1)

    return {"kernel": "wf_store_paged", "us_mean": round(store_cold * 1e3, 2),
            "bytes": nbytes, "gb_per_s": rate(nbytes, store_cold),
            "frac_hbm_peak": round(rate(nbytes, store_cold) / PEAK_HBM_GBS, 4),
            "rotation": rotation,
            "warm_us_mean": round(store_warm * 1e3, 2), "warm_gb_per_s": rate(nbytes, store_warm),
            "copy_same_bytes_us": round(copy_cold * 1e3, 2),
            "copy_same_bytes_gb_per_s": rate(nbytes, copy_cold),
            "gather": {"kernel": "wf_gather_paged", "us_mean": round(gather_cold * 1e3, 2),
                       "bytes": gbytes, "gb_per_s": rate(gbytes, gather_cold),
                       "frac_hbm_peak": round(rate(gbytes, gather_cold) / PEAK_HBM_GBS, 4),
                       "tick_chunks": {
                           "kernel": f"wf_gather_paged ({n} chunks, one launch)",
                           "us_mean": round(gather_n * 1e3, 2), "bytes": n * gbytes,
                           "gb_per_s": rate(n * gbytes, gather_n),
                           "frac_hbm_peak": round(rate(n * gbytes, gather_n) / PEAK_HBM_GBS, 4)}}}


def rope_store_bandwidth(cfg, dev, launches: int = 96, rotation: int = ROTATION) -> dict:
    """wf_rope_store_paged alone (graph_time_ms), inputs rotated over
    `rotation` ticks and page sets like the store measurement: reads K and V of
    one chunk, rotates K, writes the chunk's whole pages of K and V; and
    wf_rope_store_paged_chunks of a tick's S+1 live chunks in one launch (the
    fully paged tick's producer write)."""
    import torch

    from wavefront_causal_attention_wf_amd import inputs, wfattn

    S, T, H, D, P = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P
    n = S + 1
    ppc = cfg.ppc
    grid = inputs.chunk_grid(T)
    pool_pages = max(cfg.num_pages, rotation * n * ppc)
    kp = torch.zeros((pool_pages, P, H, D), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    srcs = [inputs.draw_live_torch(cfg, 3100 + i, dev, T=T)[1:3] for i in range(rotation)]
    ids = [torch.arange(i * n * ppc, (i + 1) * n * ppc, dtype=torch.int32, device=dev).view(n, ppc)
           for i in range(rotation)]

    def launch(i):
        k, v = srcs[i % rotation]
        wfattn.wf_rope_store_paged(k[0], v[0], kp, vp, ids[i % rotation][0], grid, 3 * (100 + i))

    def tick(i):
        k, v = srcs[i % rotation]
        wfattn.wf_rope_store_paged_chunks(k, v, kp, vp, ids[i % rotation], grid,
                                          grid[0] * (100 + i + S), -grid[0])

    def rate(ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"us_mean": round(ms * 1e3, 2), "bytes": nbytes, "gb_per_s": round(gbs, 1),
                "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}

    nbytes = 2 * (T * H * D * 2) + 2 * (ppc * P * H * D * 2)
    out = {"kernel": "wf_rope_store_paged", **rate(graph_time_ms(launch, rotation, launches), nbytes),
           "rotation": rotation, "grid": list(grid)}
    out["tick_chunks"] = {"kernel": f"wf_rope_store_paged_chunks ({n} chunks, one launch)",
                          **rate(graph_time_ms(tick, rotation, launches // 4), n * nbytes)}
    del srcs, kp, vp
    torch.cuda.empty_cache()
    return out


class FullyPagedRollout:
    """Steady ticks of the fully paged flow: every live chunk's K/V is rotated and
    written into pages by wf_rope_store_paged (denoising slots into fixed pages,
    the store chunk into freshly allocated FIFO pages), then wf_attn_tick reads
    the whole context through pages, then the store chunk is promoted."""

    def __init__(self, cfg, dev, rotate: int = 2):
        import torch

        from wavefront_causal_attention_wf_amd import inputs, wfattn

        self.torch, self.wf, self.cfg, self.dev = torch, wfattn, cfg, dev
        S, T, H, D, P = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P
        self.ppc = ppc = cfg.ppc
        self.grid = inputs.chunk_grid(T)
        n_fifo = cfg.num_pages
        self.pt = wfattn.PageTable(n_fifo, P, T, cfg.n_hist,
                                   initial_free_order=inputs.initial_free_order(cfg))
        self.k_pool = torch.zeros((n_fifo + S * ppc, P, H, D), dtype=torch.bfloat16, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.slot_ids = [torch.arange(n_fifo + j * ppc, n_fifo + (j + 1) * ppc, dtype=torch.int32,
                                      device=dev) for j in range(S)]
        self.chunk = 0   # video chunk index of the next store chunk
        for c in range(cfg.n_hist):
            hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, dev)
            ids = torch.from_numpy(self.pt.alloc_chunk()).to(dev)
            wfattn.wf_rope_store_paged(hk[0], hv[0], self.k_pool, self.v_pool, ids, self.grid,
                                       3 * self.chunk)
            self.pt.commit()
            self.chunk += 1
        self.live = [inputs.draw_live_torch(cfg, inputs.rollout_seed(i), dev) for i in range(rotate)]
        self.o = torch.empty_like(self.live[0][0])
        self.live_dev = torch.empty((S + 1, ppc), dtype=torch.int32, device=dev)
        # ring of pinned host slots for the per-tick page-id uploads
        self.nslot = 8
        self.ids_host = torch.empty((self.nslot, ppc), dtype=torch.int32, pin_memory=True)
        self.hist_host = torch.empty((self.nslot, cfg.n_hist, ppc), dtype=torch.int32,
                                     pin_memory=True)
        self.slot_ev = [None] * self.nslot
        self.hist_dev = torch.empty((cfg.n_hist, ppc), dtype=torch.int32, device=dev)
        for j in range(S):
            self.live_dev[j].copy_(self.slot_ids[j])
        self.scale = 1.0 / float(np.sqrt(D))
        self.mask = (1 << (S + 1)) - 1
        self.i = 0
        self.ws = tick_workspace(cfg, dev, live_paged=True)
        torch.cuda.synchronize()

    def step(self, attn_events=None):
        torch, wf, cfg = self.torch, self.wf, self.cfg
        S, F = cfg.S, self.grid[0]
        q, k, v = self.live[self.i % len(self.live)]
        slot = self.i % self.nslot
        self.i += 1
        if self.slot_ev[slot] is not None:   # that slot's uploads have been consumed
            self.slot_ev[slot].synchronize()
        self.ids_host[slot].numpy()[:] = self.pt.alloc_chunk()
        self.live_dev[S].copy_(self.ids_host[slot], non_blocking=True)
        c_store = self.chunk
        # slot j holds video chunk c_store + S - j: every live chunk in one launch
        wf.wf_rope_store_paged_chunks(k, v, self.k_pool, self.v_pool, self.live_dev, self.grid,
                                      F * (c_store + S), -F)
        self.hist_host[slot].numpy()[:] = self.pt.export()
        self.hist_dev.copy_(self.hist_host[slot], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.slot_ev[slot] = ev
        if attn_events is not None:
            attn_events[0].record()
        wf.wf_attn_tick(q, None, None, self.o, S, self.mask, self.scale, self.k_pool,
                        self.v_pool, self.hist_dev, live_pages=self.live_dev,
                        workspace=self.ws)
        if attn_events is not None:
            attn_events[1].record()
        self.pt.commit()
        self.chunk += 1


def fully_paged(cfg, dev, steps: int = 10, warmup: int = 3) -> dict:
    import torch

    from wavefront_causal_attention_wf_amd import wfattn

    ro = FullyPagedRollout(cfg, dev)
    flops = wfattn.wf_tick_useful_flops(cfg.S, ro.mask, cfg.T, cfg.H, cfg.D, cfg.n_hist, P=cfg.P,
                                        num_pages=cfg.num_pages)
    for _ in range(warmup):
        ro.step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        ro.step(ev[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    attn = float(np.mean([x.elapsed_time(y) for x, y in ev]))
    return {"flow": f"wf_rope_store_paged_chunks ({cfg.S + 1} live chunks, one launch) + "
                    "wf_attn_tick with "
                    "live_pages (whole context through pages) + commit",
            "ms_per_tick": round(ms, 4), "ticks_per_s": round(1e3 / ms, 2),
            "useful_tflop_per_s": round(flops / (ms * 1e-3) / 1e12, 2),
            "attn_kernel_ms_mean": round(attn, 4),
            "attn_tflop_per_s": round(flops / (attn * 1e-3) / 1e12, 2),
            "attn_frac_bf16_peak": round(flops / (attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


class Fp8Tick:
    """The 8-bit tier at the same shape, fully paged: history and live chunks in
    e4m3 key pages (+ scales) and bf16 value pages written by wf_store_paged_fp8,
    the tick's attention reading every key through them; with v8, e4m3 value
    pages (transposed tiles + exponents) as well."""

    def __init__(self, cfg, dev, v8: bool = False):
        import torch

        from wavefront_causal_attention_wf_amd import inputs, wfattn

        self.torch, self.wf, self.cfg = torch, wfattn, cfg
        S, T, H, D, P = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P
        self.ppc = ppc = cfg.ppc
        n = (cfg.n_hist + S + 1) * ppc
        order = torch.from_numpy(inputs.initial_free_order(cfg)[:n].copy()).to(dev)
        self.hist = order[:cfg.n_hist * ppc].view(cfg.n_hist, ppc)
        self.live = order[cfg.n_hist * ppc:].view(S + 1, ppc)
        self.k_pool = torch.zeros((cfg.num_pages, P, H, D), dtype=torch.uint8, device=dev)
        self.k_scale = torch.zeros((cfg.num_pages, P // 64, H), dtype=torch.float32, device=dev)
        if v8:
            self.v_pool = torch.zeros((cfg.num_pages, P // 64, H, D, 64), dtype=torch.uint8,
                                      device=dev)
            self.v_exp = torch.zeros((cfg.num_pages, P // 64, H), dtype=torch.uint8, device=dev)
        else:
            self.v_pool = torch.zeros((cfg.num_pages, P, H, D), dtype=torch.bfloat16, device=dev)
            self.v_exp = None
        for c in range(cfg.n_hist):
            hk, hv, _ = inputs.draw_live_torch(cfg, 2000 + c, dev)
            wfattn.wf_store_paged_fp8(hk[0], hv[0], self.k_pool, self.k_scale, self.v_pool,
                                      self.hist[c], v_exp=self.v_exp)
            del hk, hv
        self.q, self.k, self.v = inputs.draw_live_torch(cfg, inputs.rollout_seed(0), dev)
        self.store_live()
        self.o = torch.empty_like(self.q)
        self.scale = 1.0 / float(np.sqrt(D))
        self.mask = (1 << (S + 1)) - 1
        # the run-time pool's workspace, as the bf16 tick takes it
        nb = wfattn.workspace_bytes(S, self.mask, T, H, D, cfg.n_hist, None, P, cfg.num_pages,
                                    k8=True, v8=v8)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        torch.cuda.synchronize()

    def store_live(self):
        # every live chunk's producer write, one launch
        self.wf.wf_store_paged_fp8_chunks(self.k, self.v, self.k_pool, self.k_scale, self.v_pool,
                                          self.live, v_exp=self.v_exp)

    def attn(self):
        self.wf.wf_attn_tick(self.q, None, None, self.o, self.cfg.S, self.mask, self.scale,
                             self.k_pool, self.v_pool, self.hist, live_pages=self.live,
                             k_scale=self.k_scale, v_exp=self.v_exp, workspace=self.ws)


def fp8_tier(cfg, dev, launches: int = 20, warmup: int = 3, v8: bool = False) -> dict:
    """8-bit tier: attention launches alone, and the tick with every live chunk's
    producer write (one wf_store_paged_fp8_chunks launch + the attention). v8: values in
    e4m3 too (P.V on the fp8 MFMA: all useful flops at the fp8 peak)."""
    import torch

    from wavefront_causal_attention_wf_amd import wfattn

    ft = Fp8Tick(cfg, dev, v8)
    flops = wfattn.wf_tick_useful_flops(cfg.S, ft.mask, cfg.T, cfg.H, cfg.D, cfg.n_hist, P=cfg.P,
                                        num_pages=cfg.num_pages)
    for _ in range(warmup):
        ft.attn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        ft.attn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / launches
    a.record()
    for _ in range(launches):
        ft.store_live()
        ft.attn()
    b.record()
    torch.cuda.synchronize()
    ms_tick = a.elapsed_time(b) / launches
    tf = flops / (ms * 1e-3) / 1e12
    if v8:
        return {"tier": "e4m3 Q, K and V (per-row / per-(64-token tile, head) fp32 scales for Q "
                        "and K, power-of-two per-(tile, head) scales for V), e4m3 P; Q.K^T and "
                        "P.V on fp8 MFMA; every key and value through pages",
                "attn_kernel_ms_mean": round(ms, 4), "useful_tflop_per_s": round(tf, 2),
                "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "tick_with_producer_writes_ms": round(ms_tick, 4),
                "tick_flow": f"wf_store_paged_fp8_chunks with v_exp ({cfg.S + 1} live chunks, "
                             "one launch) + wf_attn_tick"}
    return {"tier": "e4m3 Q and K (per-row / per-(64-token tile, head) fp32 scales), Q.K^T on "
                    "fp8 MFMA, bf16 P.V; every key through pages",
            "attn_kernel_ms_mean": round(ms, 4), "useful_tflop_per_s": round(tf, 2),
            "frac_blended_peak": round(tf / PEAK_FP8_TIER_TFLOPS, 4),
            "blended_peak_tflop_per_s": round(PEAK_FP8_TIER_TFLOPS, 1),
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "tick_with_producer_writes_ms": round(ms_tick, 4),
            "tick_flow": f"wf_store_paged_fp8_chunks ({cfg.S + 1} live chunks, one launch) + "
                         "wf_attn_tick"}


def store_fp8_bandwidth(cfg, dev, launches: int = 96, rotation: int = ROTATION) -> dict:
    """The 8-bit tier's producer writes, rotating over `rotation` source ticks
    and page sets so that they do not sit in the last-level cache:
    wf_store_paged_fp8 of one chunk (K quantised, V copied), and
    wf_store_paged_fp8_chunks of a tick's S+1 live chunks in one launch, with V
    copied and with V quantised (v_exp) — the tick's producer write."""
    import torch

    from wavefront_causal_attention_wf_amd import inputs, wfattn

    S, T, H, D, P, ppc = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P, cfg.ppc
    n = S + 1
    srcs = [inputs.draw_live_torch(cfg, 3000 + i, dev, T=T)[1:3] for i in range(rotation)]
    pages = rotation * n * ppc
    k_pool = torch.zeros((pages, P, H, D), dtype=torch.uint8, device=dev)
    k_scale = torch.zeros((pages, P // 64, H), dtype=torch.float32, device=dev)
    v_pool = torch.zeros((pages, P, H, D), dtype=torch.bfloat16, device=dev)
    v8_pool = torch.zeros((pages, P // 64, H, D, 64), dtype=torch.uint8, device=dev)
    v_exp = torch.zeros((pages, P // 64, H), dtype=torch.uint8, device=dev)
    ids = [torch.arange(i * n * ppc, (i + 1) * n * ppc, dtype=torch.int32, device=dev).view(n, ppc)
           for i in range(rotation)]

    def one(i):
        k, v = srcs[i % rotation]
        wfattn.wf_store_paged_fp8(k[0], v[0], k_pool, k_scale, v_pool, ids[(i * 3) % rotation][0])

    def tick(i):
        k, v = srcs[i % rotation]
        wfattn.wf_store_paged_fp8_chunks(k, v, k_pool, k_scale, v_pool, ids[(i * 3) % rotation])

    def tick_v8(i):
        k, v = srcs[i % rotation]
        wfattn.wf_store_paged_fp8_chunks(k, v, k_pool, k_scale, v8_pool, ids[(i * 3) % rotation],
                                         v_exp=v_exp)

    def rate(ms, nbytes):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"us_mean": round(ms * 1e3, 2), "bytes": nbytes, "gb_per_s": round(gbs, 1),
                "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}

    # per chunk: K and V read (bf16), codes + bf16 V written, one scale per (tile, head)
    chunk = 2 * (T * H * D * 2) + ppc * P * H * D * 3 + ppc * (P // 64) * H * 4
    # 8-bit values: codes for V too, one exponent byte per (tile, head)
    chunk8 = 2 * (T * H * D * 2) + ppc * P * H * D * 2 + ppc * (P // 64) * H * 5
    # headline: the tick's producer write (its live chunks, one launch)
    out = {"kernel": f"wf_store_paged_fp8_chunks ({n} live chunks of a tick, one launch)",
           **rate(graph_time_ms(tick, rotation, launches // 4), n * chunk), "rotation": rotation}
    out["one_chunk"] = {"kernel": "wf_store_paged_fp8 (one chunk per launch)",
                        **rate(graph_time_ms(one, rotation, launches), chunk)}
    out["tick_chunks_v8"] = {"kernel": f"wf_store_paged_fp8_chunks with v_exp ({n} chunks)",
                             **rate(graph_time_ms(tick_v8, rotation, launches // 4), n * chunk8)}
    del srcs, k_pool, k_scale, v_pool, v8_pool, v_exp
    torch.cuda.empty_cache()
    return out


def other_config(name: str, dev, steps: int = 10, warmup: int = 3) -> dict:
    """Steady ticks of another full-size configuration, timed like the main one
    (the attention launch with the store chunk's page write, HIP events)."""
    import torch

    from wavefront_causal_attention_wf_amd import inputs, wfattn

    cfg = inputs.CONFIGS[name]
    ro = Rollout(cfg, 2, dev)
    flops = wfattn.wf_tick_useful_flops(cfg.S, ro.mask, cfg.T, cfg.H, cfg.D, cfg.n_hist, P=cfg.P,
                                        num_pages=cfg.num_pages)
    for _ in range(warmup):
        ro.step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        ro.step(ev[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    attn = float(np.mean([x.elapsed_time(y) for x, y in ev]))
    tf = flops / (attn * 1e-3) / 1e12
    del ro
    torch.cuda.empty_cache()
    return {"workload": f"{name}: S={cfg.S} (width {cfg.S + 1}), T={cfg.T}, H={cfg.H}, "
                        f"D={cfg.D}, {cfg.n_hist} history chunks in P={cfg.P} pages of a "
                        f"{cfg.num_pages}-page pool",
            "useful_tflop_per_tick": round(flops / 1e12, 4), "ms_per_step": round(ms, 4),
            "ticks_per_s": round(1e3 / ms, 2), "attn_kernel_ms_mean": round(attn, 4),
            "useful_tflop_per_s": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def active_slots(t: int, S: int) -> int:
    """Occupied slots at rollout tick t from an empty start ([summary]
    Methodology 1: stage s holds chunk t - s, the store chunk t - S; a slot is
    occupied once its chunk exists)."""
    return (1 << (min(t, S) + 1)) - 1


def rollout120(dev, warmup: int = 1) -> dict:
    """The 120-tick streaming rollout at the 1.3B 4-step shape, timed whole.

    Every tick's live Q/K/V (fresh seeded N(0, 0.5^2) draws) is generated on
    the device before the timed region (120 x 3 x 71.9 MB = 25.9 GB). From an
    empty history the stages fill one per tick and the store joins at tick S;
    each tick with the store: alloc (host page table) -> its page ids to the
    device -> the history table to the device -> wf_attn_tick (all occupied
    query chunks plus the store chunk's page write, one launch) -> commit
    (promotion, eviction of the oldest chunk beyond the 3-chunk window, host).
    `warmup` whole rollouts run first on a separate page table."""
    import torch

    from wavefront_causal_attention_wf_amd import inputs, wfattn

    cfg = inputs.CONFIGS["rollout120"]
    S, T, H, D, P = cfg.S, cfg.T, cfg.H, cfg.D, cfg.P
    ticks = cfg.ticks
    live = [inputs.draw_live_torch(cfg, inputs.rollout_seed(t), dev) for t in range(ticks)]
    k_pool = torch.zeros((cfg.num_pages, P, H, D), dtype=torch.bfloat16, device=dev)
    v_pool = torch.zeros_like(k_pool)
    o = torch.empty_like(live[0][0])
    ws = tick_workspace(cfg, dev)
    ppc = cfg.ppc
    nslot = 8
    ids_host = torch.empty((nslot, ppc), dtype=torch.int32, pin_memory=True)
    hist_host = torch.empty((nslot, cfg.window * ppc), dtype=torch.int32, pin_memory=True)
    ids_dev = torch.empty((nslot, ppc), dtype=torch.int32, device=dev)
    hist_dev = torch.empty((nslot, cfg.window * ppc), dtype=torch.int32, device=dev)
    scale = 1.0 / float(np.sqrt(D))
    flops = []
    n_hist = 0
    for t in range(ticks):
        flops.append(wfattn.wf_tick_useful_flops(S, active_slots(t, S), T, H, D, n_hist, P=P,
                                                 num_pages=cfg.num_pages))
        if t >= S:
            n_hist = min(n_hist + 1, cfg.window)
    torch.cuda.synchronize()

    def run(events=None):
        pt = wfattn.PageTable(cfg.num_pages, P, T, cfg.window,
                              initial_free_order=inputs.initial_free_order(cfg))
        slot_ev = [None] * nslot
        for t in range(ticks):
            slot = t % nslot
            if slot_ev[slot] is not None:
                slot_ev[slot].synchronize()
            if events is not None:
                events[t].record()
            q, k, v = live[t]
            mask = active_slots(t, S)
            store = None
            if t >= S:
                ids_host[slot].numpy()[:] = pt.alloc_chunk()
                ids_dev[slot].copy_(ids_host[slot], non_blocking=True)
                store = ids_dev[slot]
            hist = pt.export()
            nh = hist.shape[0]
            hd = None
            if nh:
                hist_host[slot].numpy()[:nh * ppc] = hist.reshape(-1)
                hd = hist_dev[slot][:nh * ppc].view(nh, ppc)
                hd.copy_(hist_host[slot][:nh * ppc].view(nh, ppc), non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            slot_ev[slot] = ev
            wfattn.wf_attn_tick(q, k, v, o, S, mask, scale, k_pool, v_pool, hd,
                                store_pages=store, workspace=ws)
            if t >= S:
                pt.commit()
        if events is not None:
            events[ticks].record()
        pt.close()

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(ticks + 1)]
    wall0 = time.perf_counter()
    run(events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tick_ms = np.array([events[t].elapsed_time(events[t + 1]) for t in range(ticks)])
    total_ms = events[0].elapsed_time(events[ticks])
    flops = np.array(flops)

    def part(lo: int) -> dict:
        ms = float(tick_ms[lo:].sum())
        return {"ticks": ticks - lo, "ms": round(ms, 3), "ticks_per_s": round((ticks - lo) * 1e3 / ms, 2),
                "useful_tflop_per_s": round(float(flops[lo:].sum()) / (ms * 1e-3) / 1e12, 2),
                "tick_ms_p50": round(float(np.median(tick_ms[lo:])), 4)}

    out = {"workload": f"rollout120: {ticks} consecutive ticks from an empty history, S={S}, "
                       f"T={T}, H={H}, D={D}, window {cfg.window} chunks, {cfg.num_pages}-page "
                       f"FIFO pool, fresh Q/K/V per tick (pre-generated on the device)",
           "ticks_per_s": round(ticks * 1e3 / total_ms, 2), "total_ms": round(total_ms, 3),
           "wall_ms": round(wall * 1e3, 3),
           "useful_tflop_per_s": round(float(flops.sum()) / (total_ms * 1e-3) / 1e12, 2),
           "ticks_3_to_119": part(3),
           "full_width_ticks_7_to_119": part(S + cfg.window)}
    del live, k_pool, v_pool, o, ws
    torch.cuda.empty_cache()
    return out


def profile_mode(args, cfg, dev) -> None:
    """Launch-only loops for profilers (no JSON line)."""
    import torch

    from wavefront_causal_attention_wf_amd import wfattn

    if args.mode == "copy":
        n = 1 << 29  # 2^29 bf16 = 1 GiB
        x = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
        y = torch.empty_like(x)
        for _ in range(args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        log(f"copy: {args.steps} x 1 GiB read + 1 GiB write")
        return
    if args.mode == "store":
        r = store_bandwidth(cfg, dev, launches=args.steps)
        log(f"store: {r}")
        return
    if args.mode == "rope":
        r = rope_store_bandwidth(cfg, dev, launches=args.steps)
        log(f"rope store: {r}")
        return
    if args.mode == "paged":
        r = fully_paged(cfg, dev, steps=args.steps)
        log(f"fully paged: {r}")
        return
    if args.mode in ("fp8", "fp8kv"):
        ft = Fp8Tick(cfg, dev, v8=args.mode == "fp8kv")
        for _ in range(args.steps):
            ft.attn()
        torch.cuda.synchronize()
        log(f"fp8 attn: {args.steps} launches")
        return
    if args.mode == "store8":
        r = store_fp8_bandwidth(cfg, dev, launches=args.steps)
        log(f"fp8 store: {r}")
        return
    ro = Rollout(cfg, 1, dev)
    q, k, v = ro.live[0]
    hist = torch.from_numpy(ro.pt.export().copy()).to(dev)
    # the launch the tick times: attention plus the store chunk's page write
    store_ids = torch.from_numpy(ro.pt.alloc_chunk()).to(dev)
    mask = (1 << (cfg.S + 1)) - 1
    for _ in range(args.steps):
        wfattn.wf_attn_tick(q, k, v, ro.o, cfg.S, mask, ro.scale, ro.k_pool, ro.v_pool, hist,
                            store_pages=store_ids, workspace=ro.ws)
    torch.cuda.synchronize()
    log(f"attn: {args.steps} launches (with the fused store)")


def cpu_baseline(cfg, budget_s: float) -> dict:
    """fp64 oracle on a bounded sample of one steady tick: all stages, heads
    0..n-1, every query row; n grows while the budget allows."""
    import oracle
    from wavefront_causal_attention_wf_amd import inputs

    cores = len(os.sched_getaffinity(0))
    x = inputs.draw_tick(cfg)
    model = oracle.FifoPageModel(cfg.num_pages, cfg.P, cfg.T, cfg.n_hist,
                                 initial_free_order=inputs.initial_free_order(cfg))
    store = oracle.PageStore(cfg.P, cfg.H, cfg.D)
    for c in range(cfg.n_hist):
        store.write_chunk(model.alloc_chunk(), x.hist_k_bits[c], x.hist_v_bits[c])
        model.commit()
    hist = model.export()
    mask = (1 << (cfg.S + 1)) - 1
    per_head = oracle.useful_flops(cfg.S, mask, cfg.n_hist, cfg.T, 1, cfg.D)
    done_flops, spent, heads = 0, 0.0, 0
    while heads < cfg.H:
        t0 = time.perf_counter()
        oracle.attention_tick_paged(x.q_bits, x.k_bits, x.v_bits, store, hist, cfg.S, mask,
                                    1.0 / np.sqrt(cfg.D), heads=[heads])
        dt = time.perf_counter() - t0
        spent += dt
        done_flops += per_head
        heads += 1
        log(f"oracle head {heads - 1}: {dt:.1f} s")
        if spent + dt > budget_s:
            break
    return {"value": done_flops / spent / 1e12, "unit": "TFLOP/s (useful)", "cores": cores,
            "kind": "oracle",
            "sample": f"one full tick of {cfg.name} (all {cfg.S + 1} query chunks, all "
                      f"{cfg.T} rows) restricted to heads 0..{heads - 1} of {cfg.H}; "
                      f"{done_flops / 1e9:.1f} GFLOP useful in {spent:.1f} s, numpy float64, "
                      f"heads run one at a time (BLAS threads = {cores})"}


def main():
    args = parse()
    if args.kernel_hash:
        print(attn_kernel_hash())
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1 "
                                   "(the tick is not sharded across GPUs)"}))
        sys.exit(2)
    import torch

    from wavefront_causal_attention_wf_amd import inputs, wfattn

    cfg = inputs.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"config {cfg.name}: S={cfg.S} T={cfg.T} H={cfg.H} D={cfg.D} P={cfg.P} "
        f"n_hist={cfg.n_hist} pool={cfg.num_pages}")
    if args.mode != "tick":
        profile_mode(args, cfg, dev)
        return
    ro = Rollout(cfg, args.rotate, dev)
    # The other sections run first: they keep the GPU busy for several seconds, so
    # the main tick below is timed at the clock the chip holds under sustained
    # load rather than while it is still rising from idle (ticks right after an
    # idle GPU run up to 25 % slower for the first ~25 ticks).
    extra = {}

    def section(key, fn, *args):
        """A secondary measurement; a Python-level failure there is recorded
        in its place rather than costing the run its main line."""
        try:
            extra[key] = fn(*args)
        except Exception as e:  # noqa: BLE001 - reported in the JSON line
            extra[key] = {"error": f"{type(e).__name__}: {str(e)[:300]}"}
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        log(f"{key}: {extra[key]}")

    section("store", store_bandwidth, cfg, dev)
    section("separate_store_step", separate_store_step, cfg, dev)
    section("rope_store", rope_store_bandwidth, cfg, dev)
    section("fully_paged", fully_paged, cfg, dev)
    section("fp8_tier", fp8_tier, cfg, dev)
    section("fp8kv_tier", lambda c, d: fp8_tier(c, d, v8=True), cfg, dev)
    section("store_fp8", store_fp8_bandwidth, cfg, dev)
    if cfg.name == "wan13_4step":
        configs = {}
        for name in ("wan13_5step", "wan14b_4step"):
            try:
                configs[name] = other_config(name, dev)
            except Exception as e:  # noqa: BLE001
                configs[name] = {"error": f"{type(e).__name__}: {str(e)[:300]}"}
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
            log(f"{name}: {configs[name]}")
        extra["configs"] = configs
        section("rollout120", rollout120, dev)
    # the power and clocks the chip holds under this tick (the MFMA peaks are
    # quoted at 2.4 GHz; under sustained MFMA load the board's power limit sets
    # the clock)
    power = power_window(ro.step)
    log(f"power: {power}")
    mask = (1 << (cfg.S + 1)) - 1
    flops = wfattn.wf_tick_useful_flops(cfg.S, mask, cfg.T, cfg.H, cfg.D, cfg.n_hist, P=cfg.P,
                                        num_pages=cfg.num_pages)
    for _ in range(args.warmup):
        ro.step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        ro.step(ev[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    attn_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}); "
        f"attn kernel mean {attn_ms.mean():.3f} ms p10 {np.percentile(attn_ms, 10):.3f} "
        f"p90 {np.percentile(attn_ms, 90):.3f}")

    traffic, traffic_note = recorded_traffic(cfg.name)
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flops / (attn_ms.mean() * 1e-3) / 1e12
    out = {
        "metric": "wave-attn TFLOP/s (useful) + ticks/s, % bf16 MFMA peak, 1\u00d7MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 0.5^2) bf16 Q/K/V, seeded page permutation)",
        "config": {"workload": f"{cfg.name}: one steady wave tick, S={cfg.S} (width "
                               f"{cfg.S + 1} incl. store), T={cfg.T}, H={cfg.H}, D={cfg.D}, "
                               f"{cfg.n_hist} history chunks in P={cfg.P} pages of a "
                               f"{cfg.num_pages}-page pool",
                   "global_batch": 1, "seq_len": cfg.T * (cfg.S + 1), "parallelism": "none"},
        "ticks_per_s": round(1e3 / ms_step, 2),
        "useful_tflop_per_tick": round(flops / 1e12, 4),
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "kernel": "wf_attn_tick",
                     "kernel_ms_mean": round(float(attn_ms.mean()), 4)},
    }
    if "gfx_clk_mhz_mean" in power:  # the fraction of the peak at the clock held
        held = PEAK_BF16_TFLOPS * power["gfx_clk_mhz_mean"] / PEAK_CLOCK_MHZ
        power["bf16_peak_at_held_clock_tflops"] = round(held, 1)
        power["frac_of_peak_at_held_clock"] = round(achieved / held, 4)
    out["power"] = power
    out.update(extra)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
