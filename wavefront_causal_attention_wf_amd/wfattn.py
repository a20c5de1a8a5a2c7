"""Thin Python binding over libwfattn.so (include/wf_attn.h).

Argument marshalling only: tensors are passed as device pointers
(`tensor.data_ptr()`), the stream is torch's current HIP stream unless one is
given, and every step of the computation runs in the library's HIP kernels.
There is no fallback: importing this module raises if the library has not
been built, and every non-OK status raises WfError with the library's text.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from .build_lib import LIB_PATH

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first "
                      "(python -m wavefront_causal_attention_wf_amd.build_lib)")

_lib = ctypes.CDLL(LIB_PATH)

WF_OK = 0
STATUS_NAMES = {0: "WF_OK", -1: "WF_EINVAL", -2: "WF_ENOMEM", -3: "WF_EHIP",
                -4: "WF_EUNSUPPORTED", -5: "WF_ESTATE"}
MAX_STAGES = 8
MAX_SEGMENTS = 32

_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)


class WfError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.wf_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class WfTickDesc(ctypes.Structure):
    """Mirror of wf_tick_desc."""
    _fields_ = [("S", _i32), ("active_mask", _u32), ("T", _i32), ("H", _i32), ("D", _i32),
                ("scale", ctypes.c_float),
                ("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp),
                ("k_pool", _vp), ("v_pool", _vp), ("num_pages", _i32), ("P", _i32),
                ("hist_pages", _vp), ("n_hist", _i32), ("hist_first", _i32 * MAX_STAGES),
                ("live_pages", _vp), ("store_pages", _vp),
                ("k_format", _i32), ("k_scale", _vp), ("v_format", _i32), ("v_exp", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_int64)]


K_BF16 = 0
K_E4M3 = 1
V_BF16 = 0
V_E4M3 = 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # WF_NOALLOC_SCRATCH_BYTES


class WfRopeDesc(ctypes.Structure):
    """Mirror of wf_rope_desc."""
    _fields_ = [("grid", _i32 * 3), ("frame0", _i32), ("split", _i32 * 3),
                ("theta", ctypes.c_float)]


_lib.wf_last_error.restype = ctypes.c_char_p
_lib.wf_last_error.argtypes = []
_lib.wf_abi_version.restype = _i32
_lib.wf_page_table_create.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32p, ctypes.POINTER(_vp)]
_lib.wf_page_table_destroy.argtypes = [_vp]
_lib.wf_page_table_destroy.restype = None
_lib.wf_page_table_pages_per_chunk.argtypes = [_vp, _i32p]
_lib.wf_page_table_alloc_chunk.argtypes = [_vp, _i32p, _i32]
_lib.wf_page_table_commit.argtypes = [_vp, _i32p, _i32, _i32p]
_lib.wf_page_table_export.argtypes = [_vp, _i32p, _i32, _i32p]
_lib.wf_page_table_num_free.argtypes = [_vp, _i32p]
_lib.wf_store_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]
_lib.wf_gather_paged.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]
_lib.wf_rope_store_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                     ctypes.POINTER(WfRopeDesc), _vp]
_lib.wf_rope_store_paged_chunks.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                            _i32, ctypes.POINTER(WfRopeDesc), _i32, _vp]
_lib.wf_store_paged_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _vp]
_lib.wf_store_paged_fp8_chunks.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                            _i32, _i32, _i32, _vp]
_lib.wf_attn_tick.argtypes = [ctypes.POINTER(WfTickDesc), _vp]
_lib.wf_attn_tick_noalloc.argtypes = [ctypes.POINTER(WfTickDesc), _vp]
_lib.wf_tick_useful_flops.argtypes = [ctypes.POINTER(WfTickDesc), ctypes.POINTER(ctypes.c_double)]
_lib.wf_tick_work_order.argtypes = [ctypes.POINTER(WfTickDesc), _i32, _i32p, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_int64)]
_lib.wf_tick_workspace_bytes.argtypes = [ctypes.POINTER(WfTickDesc), ctypes.POINTER(ctypes.c_int64)]
for _f in ("wf_page_table_create", "wf_page_table_pages_per_chunk", "wf_page_table_alloc_chunk",
           "wf_page_table_commit", "wf_page_table_export", "wf_page_table_num_free",
           "wf_store_paged", "wf_gather_paged", "wf_rope_store_paged", "wf_store_paged_fp8",
           "wf_store_paged_fp8_chunks", "wf_rope_store_paged_chunks",
           "wf_attn_tick", "wf_tick_useful_flops", "wf_tick_work_order",
           "wf_tick_workspace_bytes", "wf_attn_tick_noalloc"):
    getattr(_lib, _f).restype = _i32

EXPORTED_SYMBOLS = ("wf_last_error", "wf_abi_version", "wf_page_table_create",
                    "wf_page_table_destroy", "wf_page_table_pages_per_chunk",
                    "wf_page_table_alloc_chunk", "wf_page_table_commit", "wf_page_table_export",
                    "wf_page_table_num_free", "wf_store_paged", "wf_gather_paged",
                    "wf_rope_store_paged", "wf_rope_store_paged_chunks", "wf_store_paged_fp8",
                    "wf_store_paged_fp8_chunks", "wf_attn_tick",
                    "wf_tick_useful_flops", "wf_tick_work_order", "wf_tick_workspace_bytes",
                    "wf_attn_tick_noalloc")


def _check(status: int, where: str) -> None:
    if status != WF_OK:
        raise WfError(status, where)


def abi_version() -> int:
    return int(_lib.wf_abi_version())


def library():
    """The loaded ctypes library (for tests that call symbols directly)."""
    return _lib


def last_error() -> str:
    """Text of the calling thread's last failed call."""
    return _lib.wf_last_error().decode(errors="replace")


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor (anything with data_ptr()), an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# Argument checks. The library trusts sizes and page ids it is given (device
# page ids are range-checked only with WF_CHECK_PAGES=1), so the binding
# refuses, before any call, tensors whose element type, layout or shape do not
# match what the call reads and writes: dtype and contiguity first, then
# shapes, then that every tensor is on the GPU.
def _check_bf16(name, t):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 bit patterns (bfloat16/int16/uint16), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_typed(name, t, dtype_name: str):
    if str(t.dtype) != "torch." + dtype_name:
        raise TypeError(f"{name} must be a {dtype_name} tensor, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_shape(name, t, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_ids(name, t, shape) -> None:
    """Page ids: a contiguous int32 tensor of exactly `shape`."""
    if t is None or not hasattr(t, "data_ptr"):
        raise TypeError(f"{name} must be an int32 tensor on the GPU")
    _check_typed(name, t, "int32")
    _check_shape(name, t, shape)


def _check_on_gpu(**tensors) -> None:
    devs = set()
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU, got {t.device}")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(map(str, devs))}")


def _pages_per_chunk(T: int, P: int) -> int:
    if P <= 0:
        raise ValueError(f"page size P = {P} must be positive")
    return -(-T // P)


# ---------------------------------------------------------------------------
# page table (host)
# ---------------------------------------------------------------------------
class PageTable:
    """wf_page_table_*: FIFO free list + rolling history window (host state)."""

    def __init__(self, num_pages: int, page_size: int, chunk_tokens: int, window_chunks: int,
                 pin_anchor: bool = False, initial_free_order: Optional[Sequence[int]] = None):
        self._h = _vp()
        order_p = None
        if initial_free_order is not None:
            self._order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            order_p = self._order.ctypes.data_as(_i32p)
        _check(_lib.wf_page_table_create(num_pages, page_size, chunk_tokens, window_chunks,
                                         int(bool(pin_anchor)), order_p, ctypes.byref(self._h)),
               "wf_page_table_create")
        n = _i32()
        _check(_lib.wf_page_table_pages_per_chunk(self._h, ctypes.byref(n)),
               "wf_page_table_pages_per_chunk")
        self.ppc = n.value
        self.window = window_chunks

    def close(self) -> None:
        if self._h:
            _lib.wf_page_table_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_chunk(self) -> np.ndarray:
        out = np.empty(self.ppc, np.int32)
        _check(_lib.wf_page_table_alloc_chunk(self._h, out.ctypes.data_as(_i32p), self.ppc),
               "wf_page_table_alloc_chunk")
        return out

    def commit(self) -> np.ndarray:
        ev = np.empty(self.ppc, np.int32)
        n = _i32()
        _check(_lib.wf_page_table_commit(self._h, ev.ctypes.data_as(_i32p), self.ppc,
                                         ctypes.byref(n)), "wf_page_table_commit")
        return ev[: n.value].copy()

    def export(self, out: Optional[np.ndarray] = None) -> np.ndarray:
        """History page lists [n_hist][ppc], oldest first (int32)."""
        cap = (self.window + 1) * self.ppc
        buf = np.empty(cap, np.int32) if out is None else out
        n = _i32()
        _check(_lib.wf_page_table_export(self._h, buf.ctypes.data_as(_i32p), buf.size,
                                         ctypes.byref(n)), "wf_page_table_export")
        return buf[: n.value * self.ppc].reshape(n.value, self.ppc)

    def num_free(self) -> int:
        n = _i32()
        _check(_lib.wf_page_table_num_free(self._h, ctypes.byref(n)), "wf_page_table_num_free")
        return n.value


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------
def wf_store_paged(k_src, v_src, k_pool, v_pool, page_ids, stream=None) -> None:
    """Scatter one chunk's K/V [T][H][D] into pool pages [num_pages][P][H][D]."""
    for n, t in (("k_src", k_src), ("v_src", v_src), ("k_pool", k_pool), ("v_pool", v_pool)):
        _check_bf16(n, t)
    if k_src.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("k_src must be [T][H][D] and k_pool [num_pages][P][H][D]")
    T, H, D = k_src.shape
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    _check_shape("v_src", v_src, k_src.shape)
    _check_shape("k_pool", k_pool, (num_pages, P, H, D))
    _check_shape("v_pool", v_pool, k_pool.shape)
    _check_ids("page_ids", page_ids, (_pages_per_chunk(T, P),))
    _check_on_gpu(k_src=k_src, v_src=v_src, k_pool=k_pool, v_pool=v_pool, page_ids=page_ids)
    _check(_lib.wf_store_paged(_ptr(k_src), _ptr(v_src), _ptr(k_pool), _ptr(v_pool),
                               _ptr(page_ids), T, H, D, num_pages, P, _stream(stream)),
           "wf_store_paged")


def wf_gather_paged(k_pool, v_pool, page_ids, k_dst, v_dst, stream=None) -> None:
    """Copy n chunks out of pool pages into contiguous [n][T][H][D]."""
    for n, t in (("k_pool", k_pool), ("v_pool", v_pool), ("k_dst", k_dst), ("v_dst", v_dst)):
        _check_bf16(n, t)
    if k_dst.dim() != 4 or k_pool.dim() != 4:
        raise ValueError("k_dst must be [n][T][H][D] and k_pool [num_pages][P][H][D]")
    n_chunks, T, H, D = k_dst.shape
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    _check_shape("v_dst", v_dst, k_dst.shape)
    _check_shape("k_pool", k_pool, (num_pages, P, H, D))
    _check_shape("v_pool", v_pool, k_pool.shape)
    _check_ids("page_ids", page_ids, (n_chunks, _pages_per_chunk(T, P)))
    _check_on_gpu(k_pool=k_pool, v_pool=v_pool, page_ids=page_ids, k_dst=k_dst, v_dst=v_dst)
    _check(_lib.wf_gather_paged(_ptr(k_pool), _ptr(v_pool), _ptr(page_ids), n_chunks,
                                _ptr(k_dst), _ptr(v_dst), T, H, D, num_pages, P,
                                _stream(stream)), "wf_gather_paged")


def wf_store_paged_fp8(k_src, v_src, k_pool, k_scale, v_pool, page_ids, stream=None,
                       v_exp=None) -> None:
    """One chunk's K/V [T][H][D] (bf16) into the 8-bit tier's pages: K as e4m3
    codes in k_pool (uint8 [num_pages][P][H][D]) with fp32 scales in k_scale
    ([num_pages][P/64][H]); V copied into v_pool (bf16 [num_pages][P][H][D]),
    or with v_exp (uint8 [num_pages][P/64][H]) quantised into v_pool (uint8
    [num_pages][P/64][H][D][64], transposed tiles)."""
    _store_fp8(k_src, v_src, k_pool, k_scale, v_pool, page_ids, stream, v_exp, chunks=False)


def wf_store_paged_fp8_chunks(k_src, v_src, k_pool, k_scale, v_pool, page_ids, stream=None,
                              v_exp=None) -> None:
    """n chunks [n][T][H][D] in one launch, page_ids int32 [n][ceil(T/P)]; each
    chunk as wf_store_paged_fp8 writes it."""
    _store_fp8(k_src, v_src, k_pool, k_scale, v_pool, page_ids, stream, v_exp, chunks=True)


def _store_fp8(k_src, v_src, k_pool, k_scale, v_pool, page_ids, stream, v_exp, chunks):
    for n, t in (("k_src", k_src), ("v_src", v_src)):
        _check_bf16(n, t)
    _check_typed("k_pool", k_pool, "uint8")
    _check_typed("k_scale", k_scale, "float32")
    if v_exp is None:
        _check_bf16("v_pool", v_pool)
    else:
        _check_typed("v_pool", v_pool, "uint8")
        _check_typed("v_exp", v_exp, "uint8")
    if k_src.dim() != (4 if chunks else 3) or k_pool.dim() != 4:
        raise ValueError(f"k_src must be {'[n][T][H][D]' if chunks else '[T][H][D]'} and k_pool "
                         "[num_pages][P][H][D]")
    n_chunks = k_src.shape[0] if chunks else 1
    T, H, D = k_src.shape[-3:]
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    _check_shape("v_src", v_src, k_src.shape)
    _check_shape("k_pool", k_pool, (num_pages, P, H, D))
    _check_shape("k_scale", k_scale, (num_pages, P // 64, H))
    if v_exp is None:
        _check_shape("v_pool", v_pool, (num_pages, P, H, D))
    else:
        _check_shape("v_pool", v_pool, (num_pages, P // 64, H, D, 64))
        _check_shape("v_exp", v_exp, (num_pages, P // 64, H))
    ppc = _pages_per_chunk(T, P)
    _check_ids("page_ids", page_ids, (n_chunks, ppc) if chunks else (ppc,))
    _check_on_gpu(k_src=k_src, v_src=v_src, k_pool=k_pool, k_scale=k_scale, v_pool=v_pool,
                  v_exp=v_exp, page_ids=page_ids)
    if chunks:
        _check(_lib.wf_store_paged_fp8_chunks(_ptr(k_src), _ptr(v_src), n_chunks, _ptr(k_pool),
                                              _ptr(k_scale), _ptr(v_pool), _ptr(v_exp),
                                              _ptr(page_ids), T, H, D, num_pages, P,
                                              _stream(stream)), "wf_store_paged_fp8_chunks")
    else:
        _check(_lib.wf_store_paged_fp8(_ptr(k_src), _ptr(v_src), _ptr(k_pool), _ptr(k_scale),
                                       _ptr(v_pool), _ptr(v_exp), _ptr(page_ids), T, H, D,
                                       num_pages, P, _stream(stream)), "wf_store_paged_fp8")


def default_rope_split(D: int):
    """Channels per axis (frame, row, column): rows and columns 2*floor(D/6) each."""
    d_rc = 2 * (D // 6)
    return (D - 2 * d_rc, d_rc, d_rc)


def make_rope_desc(grid: Sequence[int], frame0: int, split: Optional[Sequence[int]] = None,
                   theta: float = 10000.0, D: int = 128) -> WfRopeDesc:
    r = WfRopeDesc()
    for i in range(3):
        r.grid[i] = int(grid[i])
    r.frame0 = int(frame0)
    sp = default_rope_split(D) if split is None else split
    for i in range(3):
        r.split[i] = int(sp[i])
    r.theta = float(theta)
    return r


def wf_rope_store_paged(k_src, v_src, k_pool, v_pool, page_ids, grid: Sequence[int],
                        frame0: int, split: Optional[Sequence[int]] = None,
                        theta: float = 10000.0, stream=None) -> None:
    """Rotate one chunk's keys [T][H][D] (latent grid `grid`, first frame `frame0`)
    and write them, with V copied, into pool pages; v_src = v_pool = None rewrites
    K only (the anchor's re-rotation)."""
    _check_bf16("k_src", k_src)
    _check_bf16("k_pool", k_pool)
    if (v_src is None) != (v_pool is None):
        raise ValueError("v_src and v_pool are given together (or both None: K only)")
    if v_src is not None:
        _check_bf16("v_src", v_src)
        _check_bf16("v_pool", v_pool)
    if k_src.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("k_src must be [T][H][D] and k_pool [num_pages][P][H][D]")
    T, H, D = k_src.shape
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    _check_shape("k_pool", k_pool, (num_pages, P, H, D))
    if v_src is not None:
        _check_shape("v_src", v_src, k_src.shape)
        _check_shape("v_pool", v_pool, k_pool.shape)
    _check_ids("page_ids", page_ids, (_pages_per_chunk(T, P),))
    _check_on_gpu(k_src=k_src, v_src=v_src, k_pool=k_pool, v_pool=v_pool, page_ids=page_ids)
    r = make_rope_desc(grid, frame0, split, theta, D)
    _check(_lib.wf_rope_store_paged(_ptr(k_src), _ptr(v_src), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(page_ids), T, H, D, num_pages, P, ctypes.byref(r),
                                    _stream(stream)), "wf_rope_store_paged")


def wf_rope_store_paged_chunks(k_src, v_src, k_pool, v_pool, page_ids, grid: Sequence[int],
                               frame0: int, frame_step: int,
                               split: Optional[Sequence[int]] = None, theta: float = 10000.0,
                               stream=None) -> None:
    """n chunks [n][T][H][D] in one launch, page_ids int32 [n][ceil(T/P)];
    chunk c as wf_rope_store_paged writes it at first frame frame0 + c *
    frame_step."""
    _check_bf16("k_src", k_src)
    _check_bf16("k_pool", k_pool)
    if (v_src is None) != (v_pool is None):
        raise ValueError("v_src and v_pool are given together (or both None: K only)")
    if v_src is not None:
        _check_bf16("v_src", v_src)
        _check_bf16("v_pool", v_pool)
    if k_src.dim() != 4 or k_pool.dim() != 4:
        raise ValueError("k_src must be [n][T][H][D] and k_pool [num_pages][P][H][D]")
    n, T, H, D = k_src.shape
    num_pages, P = k_pool.shape[0], k_pool.shape[1]
    _check_shape("k_pool", k_pool, (num_pages, P, H, D))
    if v_src is not None:
        _check_shape("v_src", v_src, k_src.shape)
        _check_shape("v_pool", v_pool, k_pool.shape)
    _check_ids("page_ids", page_ids, (n, _pages_per_chunk(T, P)))
    _check_on_gpu(k_src=k_src, v_src=v_src, k_pool=k_pool, v_pool=v_pool, page_ids=page_ids)
    r = make_rope_desc(grid, frame0, split, theta, D)
    _check(_lib.wf_rope_store_paged_chunks(_ptr(k_src), _ptr(v_src), n, _ptr(k_pool),
                                           _ptr(v_pool), _ptr(page_ids), T, H, D, num_pages, P,
                                           ctypes.byref(r), int(frame_step), _stream(stream)),
           "wf_rope_store_paged_chunks")


def make_tick_desc(S: int, active_mask: int, T: int, H: int, D: int, scale: float,
                   q=None, k=None, v=None, o=None, k_pool=None, v_pool=None,
                   num_pages: int = 0, P: int = 0, hist_pages=None, n_hist: int = 0,
                   hist_first: Optional[Sequence[int]] = None,
                   live_pages=None, store_pages=None, k_scale=None,
                   v_exp=None, workspace=None) -> WfTickDesc:
    d = WfTickDesc()
    d.S, d.active_mask, d.T, d.H, d.D, d.scale = S, active_mask, T, H, D, scale
    d.q, d.k, d.v, d.o = _ptr(q), _ptr(k), _ptr(v), _ptr(o)
    d.k_pool, d.v_pool = _ptr(k_pool), _ptr(v_pool)
    d.num_pages, d.P = num_pages, P
    d.hist_pages, d.n_hist = _ptr(hist_pages), n_hist
    hf = [0] * MAX_STAGES if hist_first is None else list(hist_first) + [0] * (MAX_STAGES - len(hist_first))
    for i in range(MAX_STAGES):
        d.hist_first[i] = int(hf[i])
    d.live_pages = _ptr(live_pages)
    d.store_pages = _ptr(store_pages)
    d.k_format = K_BF16 if k_scale is None else K_E4M3
    d.k_scale = _ptr(k_scale)
    d.v_format = V_BF16 if v_exp is None else V_E4M3
    d.v_exp = _ptr(v_exp)
    d.workspace = _ptr(workspace)
    d.workspace_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    return d


def wf_attn_tick(q, k, v, o, S: int, active_mask: int, scale: float, k_pool=None, v_pool=None,
                 hist_pages=None, hist_first: Optional[Sequence[int]] = None,
                 stream=None, live_pages=None, store_pages=None, k_scale=None,
                 v_exp=None, workspace=None) -> None:
    """wf_attn_tick; arguments as tick_desc."""
    d = tick_desc(q, k, v, o, S, active_mask, scale, k_pool, v_pool, hist_pages, hist_first,
                  live_pages, store_pages, k_scale, v_exp, workspace)
    _check(_lib.wf_attn_tick(ctypes.byref(d), _stream(stream)), "wf_attn_tick")


def wf_attn_tick_noalloc(q, k, v, o, S: int, active_mask: int, scale: float, k_pool=None,
                         v_pool=None, hist_pages=None, hist_first: Optional[Sequence[int]] = None,
                         stream=None, live_pages=None, store_pages=None, k_scale=None,
                         v_exp=None, scratch_bytes: int = 0) -> None:
    """wf_attn_tick_noalloc: as wf_attn_tick, the run-time pool in the
    library's own per-GPU array, of which it may use scratch_bytes (at most
    WF_NOALLOC_SCRATCH_BYTES)."""
    d = tick_desc(q, k, v, o, S, active_mask, scale, k_pool, v_pool, hist_pages, hist_first,
                  live_pages, store_pages, k_scale, v_exp, None)
    d.workspace_bytes = int(scratch_bytes)
    _check(_lib.wf_attn_tick_noalloc(ctypes.byref(d), _stream(stream)), "wf_attn_tick_noalloc")


def tick_desc(q, k, v, o, S: int, active_mask: int, scale: float, k_pool=None, v_pool=None,
              hist_pages=None, hist_first: Optional[Sequence[int]] = None, live_pages=None,
              store_pages=None, k_scale=None, v_exp=None, workspace=None) -> WfTickDesc:
    """Checked descriptor of one tick: q, k, v, o [S+1][T][H][D]; pools [num_pages][P][H][D];
    hist_pages int32 [n_hist][ceil(T/P)] on the device; live_pages (optional)
    int32 [S+1][ceil(T/P)] on the device: live K/V read from those pages (k and
    v may then be None); store_pages (optional) int32 [ceil(T/P)] on the device:
    the same launch writes the store chunk's K/V into those pages. k_scale
    (optional, float32 [num_pages][P/64][H]): the 8-bit tier — k_pool holds
    e4m3 codes (uint8) as written by wf_store_paged_fp8, live_pages required.
    v_exp (optional, uint8 [num_pages][P/64][H], with k_scale): 8-bit values —
    v_pool holds the transposed e4m3 tiles written by wf_store_paged_fp8.
    workspace (optional, contiguous device tensor of workspace_bytes(...)
    bytes, 256-byte aligned): part of the work is handed out at run time to
    free CUs (launches sharing a workspace must not overlap)."""
    live = (("k", k), ("v", v)) if live_pages is None else ()
    for n, t in (("q", q), ("o", o)) + live:
        _check_bf16(n, t)
    if q.dim() != 4 or q.shape[0] != S + 1:
        raise ValueError(f"q must be [S+1][T][H][D] with S + 1 = {S + 1}, got {tuple(q.shape)}")
    _, T, H, D = q.shape
    for n, t in (("o", o),) + live:
        _check_shape(n, t, q.shape)
    n_hist, num_pages, P = 0, 0, 0
    if hist_pages is not None and hist_pages.numel() > 0:
        if hist_pages.dim() != 2:
            raise ValueError("hist_pages must be [n_hist][ceil(T/P)]")
        n_hist = hist_pages.shape[0]
    pooled = n_hist > 0 or live_pages is not None or store_pages is not None
    if pooled:
        if k_pool is None or v_pool is None:
            raise ValueError("history, live_pages or store_pages need k_pool and v_pool")
        if k_scale is None:
            _check_bf16("k_pool", k_pool)
        else:
            _check_typed("k_pool", k_pool, "uint8")
            _check_typed("k_scale", k_scale, "float32")
        if v_exp is None:
            _check_bf16("v_pool", v_pool)
        else:
            _check_typed("v_pool", v_pool, "uint8")
            _check_typed("v_exp", v_exp, "uint8")
        if k_pool.dim() != 4:
            raise ValueError("k_pool must be [num_pages][P][H][D]")
        num_pages, P = k_pool.shape[0], k_pool.shape[1]
        ppc = _pages_per_chunk(T, P)
        _check_shape("k_pool", k_pool, (num_pages, P, H, D))
        if v_exp is None:
            _check_shape("v_pool", v_pool, (num_pages, P, H, D))
        else:
            _check_shape("v_pool", v_pool, (num_pages, P // 64, H, D, 64))
            _check_shape("v_exp", v_exp, (num_pages, P // 64, H))
        if k_scale is not None:
            _check_shape("k_scale", k_scale, (num_pages, P // 64, H))
        if n_hist:
            _check_ids("hist_pages", hist_pages, (n_hist, ppc))
        if live_pages is not None:
            _check_ids("live_pages", live_pages, (S + 1, ppc))
        if store_pages is not None:
            _check_ids("store_pages", store_pages, (ppc,))
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _check_on_gpu(q=q, o=o, k=k if live_pages is None else None,
                  v=v if live_pages is None else None,
                  k_pool=k_pool if pooled else None, v_pool=v_pool if pooled else None,
                  hist_pages=hist_pages if n_hist else None, live_pages=live_pages,
                  store_pages=store_pages, k_scale=k_scale, v_exp=v_exp, workspace=workspace)
    return make_tick_desc(S, active_mask, T, H, D, scale, q, k, v, o,
                          k_pool if pooled else None, v_pool if pooled else None, num_pages, P,
                          hist_pages if n_hist else None, n_hist, hist_first, live_pages,
                          store_pages, k_scale, v_exp, workspace)


def wf_attn_tick_desc(desc: WfTickDesc, stream=None) -> None:
    """Raw call with a prepared descriptor (used by the bench and the error tests)."""
    _check(_lib.wf_attn_tick(ctypes.byref(desc), _stream(stream)), "wf_attn_tick")


def wf_tick_useful_flops(S: int, active_mask: int, T: int, H: int, D: int, n_hist: int = 0,
                         hist_first: Optional[Sequence[int]] = None, P: int = 16,
                         num_pages: int = 0) -> float:
    """Useful FLOPs the library counts for a tick (host only; no device pointers needed
    beyond non-NULL placeholders)."""
    fake = 16  # aligned non-NULL placeholder: nothing is dereferenced by this call
    d = make_tick_desc(S, active_mask, T, H, D, 1.0, fake, fake, fake, fake,
                       fake if n_hist else None, fake if n_hist else None,
                       max(num_pages, n_hist * -(-T // P)) if n_hist else 0, P if n_hist else 0,
                       fake if n_hist else None, n_hist, hist_first)
    return tick_useful_flops_desc(d)


def tick_useful_flops_desc(desc: WfTickDesc) -> float:
    out = ctypes.c_double()
    _check(_lib.wf_tick_useful_flops(ctypes.byref(desc), ctypes.byref(out)),
           "wf_tick_useful_flops")
    return out.value


def tick_work_order(desc: WfTickDesc, cus_per_xcd: int = 0) -> np.ndarray:
    """Host-only plan of wf_attn_tick: int32 [n_rows][6] = (block, item, slot,
    head, first query row, rows) in launch order, a block's items in the order
    it runs them (a tail item has one row per slot it serves)."""
    n = ctypes.c_int64()
    _check(_lib.wf_tick_work_order(ctypes.byref(desc), cus_per_xcd, None, 0, ctypes.byref(n)),
           "wf_tick_work_order")
    out = np.empty(6 * n.value, np.int32)
    _check(_lib.wf_tick_work_order(ctypes.byref(desc), cus_per_xcd, out.ctypes.data_as(_i32p),
                                   out.size, ctypes.byref(n)), "wf_tick_work_order")
    return out.reshape(n.value, 6)


def tick_workspace_bytes(desc: WfTickDesc) -> int:
    """wf_tick_workspace_bytes: workspace size for the full run-time pool (0: none)."""
    out = ctypes.c_int64()
    _check(_lib.wf_tick_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)),
           "wf_tick_workspace_bytes")
    return out.value


def workspace_bytes(S: int, active_mask: int, T: int, H: int, D: int, n_hist: int = 0,
                    hist_first: Optional[Sequence[int]] = None, P: int = 64,
                    num_pages: int = 0, live_paged: bool = False, k8: bool = False,
                    v8: bool = False) -> int:
    """Workspace bytes wf_attn_tick would use for a tick of this shape: bf16
    keys, or (k8) 8-bit keys, with (v8) 8-bit values too; the 8-bit tiers read
    every live chunk through pages."""
    fake = 16
    live_paged = live_paged or k8
    d = make_tick_desc(S, active_mask, T, H, D, 1.0, fake, fake, fake, fake,
                       fake if (n_hist or live_paged) else None, fake if (n_hist or live_paged) else None,
                       max(num_pages, (n_hist + S + 1) * -(-T // P)) if (n_hist or live_paged) else 0,
                       P if (n_hist or live_paged) else 0, fake if n_hist else None, n_hist,
                       hist_first, fake if live_paged else None,
                       k_scale=fake if k8 else None, v_exp=fake if (k8 and v8) else None)
    return tick_workspace_bytes(d)
