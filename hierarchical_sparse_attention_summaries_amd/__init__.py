"""Python binding of libhga (HGA routed attention on MI355X).

Argument marshalling only: every step runs in the HIP kernels of libhga.so,
called through its C ABI (include/hga.h). PyTorch supplies device memory and
the current stream. There is no fallback: if the library is missing this
module raises at import time.

    cm, gm = build_summaries(K, chunk, group)
    chunk_idx, group_idx = route(Q, cm, gm, T, chunk, group, k_chunk, k_group)
    O, lse = attend(Q, K, V, group_idx, group)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["HGAError", "lib", "summary_counts", "build_summaries", "update_summaries",
           "route", "attend", "route_workspace_bytes", "attend_workspace_bytes", "Shape",
           "Layout", "build_summaries_ex", "update_summaries_ex", "route_ex", "attend_ex",
           "route_fresh_ex", "decode_step_ex", "decode_step_one_launch",
           "decode_step_one_launch_cus", "workspace_check", "workspace_reset", "attend_staged", "decode_step_noalloc",
           "LIB_PATH", "WORKSPACE_ZERO_BYTES"]

# The library is libhga.so beside this file; HGA_LIB may name another build of
# it (the phase-stamp build, libhga_phases.so, for bench.py --phases).
LIB_PATH = os.environ.get("HGA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libhga.so")

F32, BF16 = 0, 1
_STATUS = {0: "HGA_OK", -1: "HGA_ERR_NULL", -2: "HGA_ERR_SHAPE", -3: "HGA_ERR_DTYPE",
           -4: "HGA_ERR_LAYOUT", -5: "HGA_ERR_PARAM", -6: "HGA_ERR_WORKSPACE",
           -7: "HGA_ERR_HIP", -8: "HGA_ERR_UNSUPPORTED", -9: "HGA_ERR_TIMEOUT"}
ERR_TIMEOUT = -9


class HGAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib.hga_status_str(status).decode() if _lib is not None else ""
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({text})")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("q_heads", ctypes.c_int64),
                ("kv_heads", ctypes.c_int64), ("n_queries", ctypes.c_int64),
                ("seq_len", ctypes.c_int64), ("head_dim", ctypes.c_int64)]


class _KvLayoutC(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


class Layout:
    """Ragged and/or paged K/V. seq_lens: int32 [B] device tensor of keys per
    sequence (None: every sequence holds the full capacity). block_table: int32
    [B, max_pages] device tensor of page ids (None: dense [B, Hkv, T, D] K/V);
    with pages, K and V are pools [n_pages, Hkv, page_tokens, D]."""

    def __init__(self, seq_lens=None, block_table=None, page_tokens=0, n_pages=0):
        for t, n in ((seq_lens, "seq_lens"), (block_table, "block_table")):
            if t is not None and (not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous()):
                raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
        self.seq_lens, self.block_table = seq_lens, block_table
        self.page_tokens, self.n_pages = page_tokens, n_pages

    @property
    def paged(self):
        return self.block_table is not None

    def c(self):
        bt = self.block_table
        return _KvLayoutC(1 if self.paged else 0, self.page_tokens,
                          bt.shape[1] if self.paged else 0, self.n_pages,
                          bt.data_ptr() if self.paged else None,
                          self.seq_lens.data_ptr() if self.seq_lens is not None else None)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libhga.so not built at {LIB_PATH}; run "
                          "`python hierarchical_sparse_attention_summaries_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    P = ctypes.POINTER
    sig = {
        "hga_abi_version": (ctypes.c_int, []),
        "hga_workspace_zero_bytes": (ctypes.c_size_t, []),
        "hga_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "hga_summary_counts": (ctypes.c_int, [i64, i32, i32, P(i64), P(i64)]),
        "hga_build_summaries": (ctypes.c_int, [vp, i32, i64, i64, i64, i64, i32, i32, vp, vp, vp]),
        "hga_update_summaries": (ctypes.c_int, [vp, i32, i64, i64, i64, i64, i32, i32, i64, i64,
                                                vp, vp, vp]),
        "hga_route_workspace_size": (ctypes.c_int, [P(Shape), i32, i32, i32, i32, P(sz)]),
        "hga_route": (ctypes.c_int, [P(Shape), vp, i32, vp, vp, i32, i32, i32, i32, f32, vp, vp,
                                     vp, sz, vp]),
        "hga_attend_workspace_size": (ctypes.c_int, [P(Shape), i32, i32, P(sz)]),
        "hga_attend": (ctypes.c_int, [P(Shape), vp, vp, vp, i32, vp, i32, i32, f32, vp, vp, vp,
                                      sz, vp]),
        "hga_build_summaries_ex": (ctypes.c_int, [vp, i32, P(_KvLayoutC), i64, i64, i64, i64, i32,
                                                  i32, vp, vp, vp]),
        "hga_update_summaries_ex": (ctypes.c_int, [vp, i32, P(_KvLayoutC), i64, i64, i64, i64, i32,
                                                   i32, i64, vp, vp, vp]),
        "hga_route_ex": (ctypes.c_int, [P(Shape), P(_KvLayoutC), vp, i32, vp, vp, i32, i32, i32, i32,
                                        f32, vp, vp, vp, sz, vp]),
        "hga_attend_ex": (ctypes.c_int, [P(Shape), P(_KvLayoutC), vp, vp, vp, i32, vp, i32, i32, f32,
                                         vp, vp, vp, sz, vp]),
        "hga_route_fresh_ex": (ctypes.c_int, [P(Shape), P(_KvLayoutC), vp, vp, i32, vp, vp, i32, i32,
                                              i32, i32, f32, vp, vp, vp, sz, vp]),
        "hga_decode_step_workspace_size": (ctypes.c_int, [P(Shape), i32, i32, i32, i32, P(sz)]),
        "hga_attend_staged_sizes": (ctypes.c_int, [P(Shape), i32, i32, P(i64), P(sz)]),
        "hga_attend_staged": (ctypes.c_int, [P(Shape), vp, vp, vp, i32, vp, i32, i32, f32, vp, vp,
                                             vp, vp, i64, vp, sz, vp]),
        "hga_decode_step_one_launch": (ctypes.c_int, [P(Shape), i32, i32, i32, i32, i32, P(i32)]),
        "hga_decode_step_one_launch_cus": (ctypes.c_int, [P(Shape), i32, i32, i32, i32, i32, i32,
                                                          P(i32)]),
        "hga_workspace_check": (ctypes.c_int, [vp, sz, vp]),
        "hga_decode_step_noalloc": (ctypes.c_int, [P(Shape), P(_KvLayoutC), vp, vp, vp, i32, vp,
                                                   vp, i32, i32, i32, i32, f32, vp, vp, vp, vp,
                                                   i32, vp]),
        "hga_workspace_reset": (ctypes.c_int, [vp, sz, vp]),
        "hga_decode_step_ex": (ctypes.c_int, [P(Shape), P(_KvLayoutC), vp, vp, vp, i32, vp, vp, i32,
                                              i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = _load()
# Bytes at the start of every workspace that must be zero before its first use
# (every call leaves them at zero).
WORKSPACE_ZERO_BYTES = int(_lib.hga_workspace_zero_bytes())


def lib():
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise HGAError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _need(t: torch.Tensor, name: str, ndim: int, host_ok: bool = False):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda and not (host_ok and t.is_pinned()):
        raise ValueError(f"{name} must be on a GPU" + (" or pinned host memory" if host_ok else ""))


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# Zero-initialised workspaces, one per (device, stream, role), grown on demand.
# The library leaves their zero region at zero after each call. Calls that
# share a workspace must not overlap; calls on one stream never do, so a
# workspace of its own per stream keeps calls on different streams apart.
_ws_lock = threading.Lock()
_ws: dict = {}


def _workspace(device: torch.device, role: str, nbytes: int) -> torch.Tensor:
    key = (device.index, torch.cuda.current_stream(device).cuda_stream, role)
    with _ws_lock:
        buf = _ws.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            _ws[key] = buf
        return buf


def summary_counts(seq_len: int, chunk: int, group: int):
    nc, ng = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.hga_summary_counts(seq_len, chunk, group, ctypes.byref(nc), ctypes.byref(ng)),
           "hga_summary_counts")
    return nc.value, ng.value


def _gpu_of(t: torch.Tensor) -> torch.device:
    return t.device if t.is_cuda else torch.device("cuda", torch.cuda.current_device())


def build_summaries(K: torch.Tensor, chunk: int, group: int, chunk_mean=None, group_mean=None):
    """Mean key per chunk and per group. K [B, Hkv, T, D] -> ([B,Hkv,n_c,D], [B,Hkv,n_g,D]) f32.
    K may be a pinned host tensor (read in place); the summaries live on the GPU."""
    _need(K, "K", 4, host_ok=True)
    B, H, T, D = K.shape
    n_c, n_g = summary_counts(T, chunk, group)
    dev = _gpu_of(K)
    if chunk_mean is None:
        chunk_mean = torch.empty((B, H, n_c, D), dtype=torch.float32, device=dev)
    if group_mean is None:
        group_mean = torch.empty((B, H, n_g, D), dtype=torch.float32, device=dev)
    _need(chunk_mean, "chunk_mean", 4)
    _need(group_mean, "group_mean", 4)
    if tuple(chunk_mean.shape) != (B, H, n_c, D) or tuple(group_mean.shape) != (B, H, n_g, D) \
            or chunk_mean.dtype != torch.float32 or group_mean.dtype != torch.float32:
        raise ValueError("summary buffers must be float32 [B, Hkv, n, D]")
    _check(_lib.hga_build_summaries(_ptr(K), _dtype_code(K), B, H, T, D, chunk, group,
                                    _ptr(chunk_mean), _ptr(group_mean), _stream(dev)),
           "hga_build_summaries")
    return chunk_mean, group_mean


def update_summaries(K: torch.Tensor, chunk: int, group: int, t_begin: int, t_end: int,
                     chunk_mean: torch.Tensor, group_mean: torch.Tensor):
    """Recompute the summaries of the chunks (and their groups) touching [t_begin, t_end)."""
    _need(K, "K", 4, host_ok=True)
    _need(chunk_mean, "chunk_mean", 4)
    _need(group_mean, "group_mean", 4)
    B, H, T, D = K.shape
    n_c, n_g = summary_counts(T, chunk, group)
    if tuple(chunk_mean.shape) != (B, H, n_c, D) or tuple(group_mean.shape) != (B, H, n_g, D):
        raise ValueError("summary buffers do not match K")
    _check(_lib.hga_update_summaries(_ptr(K), _dtype_code(K), B, H, T, D, chunk, group, t_begin,
                                     t_end, _ptr(chunk_mean), _ptr(group_mean),
                                     _stream(chunk_mean.device)),
           "hga_update_summaries")


def _shape(Q: torch.Tensor, Hkv: int, T: int) -> Shape:
    B, Hq, Nq, D = Q.shape
    return Shape(B, Hq, Hkv, Nq, T, D)


def route_workspace_bytes(shape: Shape, chunk, group, k_chunk, k_group) -> int:
    n = ctypes.c_size_t()
    _check(_lib.hga_route_workspace_size(ctypes.byref(shape), chunk, group, k_chunk, k_group,
                                         ctypes.byref(n)), "hga_route_workspace_size")
    return n.value


def attend_workspace_bytes(shape: Shape, group, k_group) -> int:
    n = ctypes.c_size_t()
    _check(_lib.hga_attend_workspace_size(ctypes.byref(shape), group, k_group, ctypes.byref(n)),
           "hga_attend_workspace_size")
    return n.value


def route(Q: torch.Tensor, chunk_mean: torch.Tensor, group_mean: torch.Tensor, seq_len: int,
          chunk: int, group: int, k_chunk: int, k_group: int, scale: float = 0.0,
          want_chunks: bool = True, chunk_idx=None, group_idx=None, workspace=None):
    """Two-level routing. Returns (chunk_idx [B,Hq,Nq,k_chunk+2] or None, group_idx [B,Hq,Nq,k_group])."""
    _need(Q, "Q", 4)
    _need(chunk_mean, "chunk_mean", 4)
    _need(group_mean, "group_mean", 4)
    B, Hq, Nq, D = Q.shape
    Hkv = chunk_mean.shape[1]
    n_c, n_g = summary_counts(seq_len, chunk, group)
    if tuple(chunk_mean.shape) != (B, Hkv, n_c, D) or tuple(group_mean.shape) != (B, Hkv, n_g, D):
        raise ValueError("summary shapes do not match Q / seq_len")
    shape = _shape(Q, Hkv, seq_len)
    nbytes = route_workspace_bytes(shape, chunk, group, k_chunk, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "route", nbytes)
    if want_chunks and chunk_idx is None:
        chunk_idx = torch.empty((B, Hq, Nq, k_chunk + 2), dtype=torch.int32, device=Q.device)
    if group_idx is None:
        group_idx = torch.empty((B, Hq, Nq, k_group), dtype=torch.int32, device=Q.device)
    _check(_lib.hga_route(ctypes.byref(shape), _ptr(Q), _dtype_code(Q), _ptr(chunk_mean),
                          _ptr(group_mean), chunk, group, k_chunk, k_group, float(scale),
                          _ptr(chunk_idx), _ptr(group_idx), _ptr(ws), ws.numel(),
                          _stream(Q.device)), "hga_route")
    return chunk_idx, group_idx


def attend(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, group_idx: torch.Tensor, group: int,
           scale: float = 0.0, want_lse: bool = True, out=None, lse=None, workspace=None):
    """Exact attention over the routed groups. Returns (O like Q, lse [B,Hq,Nq] f32 or None).
    K and V may be pinned host tensors (read in place over the host link)."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, host_ok=True)
    _need(V, "V", 4, host_ok=True)
    _need(group_idx, "group_idx", 4)
    if group_idx.dtype != torch.int32:
        raise TypeError("group_idx must be int32")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share one dtype")
    B, Hq, Nq, D = Q.shape
    Hkv, T = K.shape[1], K.shape[2]
    if tuple(K.shape) != (B, Hkv, T, D) or tuple(V.shape) != tuple(K.shape):
        raise ValueError("K/V shapes do not match Q")
    k_group = group_idx.shape[3]
    if tuple(group_idx.shape[:3]) != (B, Hq, Nq):
        raise ValueError("group_idx must be [B, Hq, Nq, k_group]")
    shape = _shape(Q, Hkv, T)
    nbytes = attend_workspace_bytes(shape, group, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "attend", nbytes)
    if out is None:
        out = torch.empty_like(Q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=Q.device)
    _check(_lib.hga_attend(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q),
                           _ptr(group_idx), k_group, group, float(scale), _ptr(out),
                           _ptr(lse if want_lse else None), _ptr(ws), ws.numel(),
                           _stream(Q.device)), "hga_attend")
    return out, (lse if want_lse else None)


# ---------------------------------------------------------------- ragged / paged
def _kv_dims(K, layout, batch, seq_len):
    """(B, Hkv, T, D) of a dense cache or of a page pool under `layout`."""
    if layout is not None and layout.paged:
        _, H, page, D = K.shape
        B = layout.block_table.shape[0]
        T = seq_len if seq_len is not None else layout.block_table.shape[1] * page
        if page != layout.page_tokens:
            raise ValueError("page pool's third dim must equal layout.page_tokens")
        return B, H, T, D
    B, H, T, D = K.shape
    return B, H, T, D


def _lay(layout):
    return ctypes.byref(layout.c()) if layout is not None else None


def build_summaries_ex(K, chunk, group, layout=None, seq_len=None, chunk_mean=None,
                       group_mean=None):
    """build_summaries over a ragged and/or paged cache (see Layout)."""
    _need(K, "K", 4, host_ok=True)
    B, H, T, D = _kv_dims(K, layout, None, seq_len)
    n_c, n_g = summary_counts(T, chunk, group)
    dev = _gpu_of(K)
    if chunk_mean is None:
        chunk_mean = torch.zeros((B, H, n_c, D), dtype=torch.float32, device=dev)
    if group_mean is None:
        group_mean = torch.zeros((B, H, n_g, D), dtype=torch.float32, device=dev)
    _check(_lib.hga_build_summaries_ex(_ptr(K), _dtype_code(K), _lay(layout), B, H, T, D, chunk,
                                       group, _ptr(chunk_mean), _ptr(group_mean), _stream(dev)),
           "hga_build_summaries_ex")
    return chunk_mean, group_mean


def update_summaries_ex(K, chunk, group, newest, chunk_mean, group_mean, layout=None,
                        seq_len=None):
    """Refresh the chunks holding each sequence's newest `newest` keys."""
    _need(K, "K", 4, host_ok=True)
    B, H, T, D = _kv_dims(K, layout, None, seq_len)
    _check(_lib.hga_update_summaries_ex(_ptr(K), _dtype_code(K), _lay(layout), B, H, T, D, chunk,
                                        group, newest, _ptr(chunk_mean), _ptr(group_mean),
                                        _stream(chunk_mean.device)), "hga_update_summaries_ex")


def route_ex(Q, chunk_mean, group_mean, seq_len, chunk, group, k_chunk, k_group, layout=None,
             scale=0.0, want_chunks=True, chunk_idx=None, group_idx=None, workspace=None):
    """route with per-sequence lengths (layout.seq_lens); seq_len is the capacity T."""
    _need(Q, "Q", 4)
    B, Hq, Nq, D = Q.shape
    Hkv = chunk_mean.shape[1]
    shape = _shape(Q, Hkv, seq_len)
    nbytes = route_workspace_bytes(shape, chunk, group, k_chunk, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "route", nbytes)
    if want_chunks and chunk_idx is None:
        chunk_idx = torch.empty((B, Hq, Nq, k_chunk + 2), dtype=torch.int32, device=Q.device)
    if group_idx is None:
        group_idx = torch.empty((B, Hq, Nq, k_group), dtype=torch.int32, device=Q.device)
    _check(_lib.hga_route_ex(ctypes.byref(shape), _lay(layout), _ptr(Q), _dtype_code(Q),
                             _ptr(chunk_mean), _ptr(group_mean), chunk, group, k_chunk, k_group,
                             float(scale), _ptr(chunk_idx), _ptr(group_idx), _ptr(ws), ws.numel(),
                             _stream(Q.device)), "hga_route_ex")
    return chunk_idx, group_idx


def attend_ex(Q, K, V, group_idx, group, layout=None, seq_len=None, scale=0.0, want_lse=True,
              out=None, lse=None, workspace=None):
    """attend over a ragged and/or paged cache (see Layout)."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, host_ok=True)
    _need(V, "V", 4, host_ok=True)
    _need(group_idx, "group_idx", 4)
    B, Hq, Nq, D = Q.shape
    Bk, Hkv, T, Dk = _kv_dims(K, layout, None, seq_len)
    if (Bk, Dk) != (B, D) or tuple(V.shape) != tuple(K.shape):
        raise ValueError("K/V do not match Q")
    k_group = group_idx.shape[3]
    shape = _shape(Q, Hkv, T)
    nbytes = attend_workspace_bytes(shape, group, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "attend", nbytes)
    if out is None:
        out = torch.empty_like(Q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=Q.device)
    _check(_lib.hga_attend_ex(ctypes.byref(shape), _lay(layout), _ptr(Q), _ptr(K), _ptr(V),
                              _dtype_code(Q), _ptr(group_idx), k_group, group, float(scale),
                              _ptr(out), _ptr(lse if want_lse else None), _ptr(ws), ws.numel(),
                              _stream(Q.device)), "hga_attend_ex")
    return out, (lse if want_lse else None)


def route_fresh_ex(Q, K, chunk_mean, group_mean, seq_len, chunk, group, k_chunk, k_group,
                   layout=None, scale=0.0, want_chunks=True, chunk_idx=None, group_idx=None,
                   workspace=None):
    """Decode step of steps 1-2: refresh the summaries of each sequence's newest
    Nq keys from K, then route (one launch for small batches)."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, host_ok=True)
    B, Hq, Nq, D = Q.shape
    Hkv = chunk_mean.shape[1]
    shape = _shape(Q, Hkv, seq_len)
    nbytes = route_workspace_bytes(shape, chunk, group, k_chunk, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "route", nbytes)
    if want_chunks and chunk_idx is None:
        chunk_idx = torch.empty((B, Hq, Nq, k_chunk + 2), dtype=torch.int32, device=Q.device)
    if group_idx is None:
        group_idx = torch.empty((B, Hq, Nq, k_group), dtype=torch.int32, device=Q.device)
    _check(_lib.hga_route_fresh_ex(ctypes.byref(shape), _lay(layout), _ptr(Q), _ptr(K),
                                   _dtype_code(Q), _ptr(chunk_mean), _ptr(group_mean), chunk, group,
                                   k_chunk, k_group, float(scale), _ptr(chunk_idx), _ptr(group_idx),
                                   _ptr(ws), ws.numel(), _stream(Q.device)), "hga_route_fresh_ex")
    return chunk_idx, group_idx


def decode_step_workspace_bytes(shape: Shape, chunk, group, k_chunk, k_group) -> int:
    n = ctypes.c_size_t()
    _check(_lib.hga_decode_step_workspace_size(ctypes.byref(shape), chunk, group, k_chunk,
                                               k_group, ctypes.byref(n)),
           "hga_decode_step_workspace_size")
    return n.value


def decode_step_one_launch(shape: Shape, dtype: str, chunk, group, k_chunk, k_group) -> bool:
    """Whether decode_step_ex runs these arguments as a single kernel launch."""
    one = ctypes.c_int32()
    code = {"f32": F32, "bf16": BF16}[dtype]
    _check(_lib.hga_decode_step_one_launch(ctypes.byref(shape), code, chunk, group, k_chunk,
                                           k_group, ctypes.byref(one)),
           "hga_decode_step_one_launch")
    return bool(one.value)


def decode_step_one_launch_cus(shape: Shape, dtype: str, chunk, group, k_chunk, k_group,
                               compute_units: int) -> bool:
    """The same decision for a device of `compute_units` CUs (no device needed)."""
    one = ctypes.c_int32()
    code = {"f32": F32, "bf16": BF16}[dtype]
    _check(_lib.hga_decode_step_one_launch_cus(ctypes.byref(shape), code, chunk, group, k_chunk,
                                               k_group, compute_units, ctypes.byref(one)),
           "hga_decode_step_one_launch_cus")
    return bool(one.value)


def workspace_check(workspace: torch.Tensor):
    """Synchronises the current stream and raises HGAError(HGA_ERR_TIMEOUT) if
    a bounded wait of a one-launch decode step on this workspace gave up (its
    rows are NaN; the workspace stays flagged until workspace_reset)."""
    _check(_lib.hga_workspace_check(_ptr(workspace), workspace.numel(),
                                    _stream(workspace.device)), "hga_workspace_check")


def workspace_reset(workspace: torch.Tensor):
    """Zeroes the workspace's zero region (status word included), in stream order."""
    _check(_lib.hga_workspace_reset(_ptr(workspace), workspace.numel(),
                                    _stream(workspace.device)), "hga_workspace_reset")


def decode_step_ex(Q, K, V, chunk_mean, group_mean, seq_len, chunk, group, k_chunk, k_group,
                   layout=None, scale=0.0, want_chunks=True, want_lse=True, chunk_idx=None,
                   group_idx=None, out=None, lse=None, workspace=None, check=False):
    """One decode step: refresh the summaries of each sequence's newest Nq keys
    from K, route, and attend (one launch for small batches). Returns
    (O, lse, chunk_idx, group_idx). With check=True the call synchronises and
    raises HGAError(HGA_ERR_TIMEOUT) if a bounded wait gave up (see
    workspace_check)."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, host_ok=True)
    _need(V, "V", 4, host_ok=True)
    B, Hq, Nq, D = Q.shape
    Hkv = chunk_mean.shape[1]
    if tuple(V.shape) != tuple(K.shape):
        raise ValueError("K and V differ in shape")
    shape = _shape(Q, Hkv, seq_len)
    nbytes = decode_step_workspace_bytes(shape, chunk, group, k_chunk, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "decode", nbytes)
    if want_chunks and chunk_idx is None:
        chunk_idx = torch.empty((B, Hq, Nq, k_chunk + 2), dtype=torch.int32, device=Q.device)
    if group_idx is None:
        group_idx = torch.empty((B, Hq, Nq, k_group), dtype=torch.int32, device=Q.device)
    if out is None:
        out = torch.empty_like(Q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=Q.device)
    _check(_lib.hga_decode_step_ex(ctypes.byref(shape), _lay(layout), _ptr(Q), _ptr(K), _ptr(V),
                                   _dtype_code(Q), _ptr(chunk_mean), _ptr(group_mean), chunk,
                                   group, k_chunk, k_group, float(scale),
                                   _ptr(chunk_idx if want_chunks else None), _ptr(group_idx),
                                   _ptr(out), _ptr(lse if want_lse else None), _ptr(ws),
                                   ws.numel(), _stream(Q.device)), "hga_decode_step_ex")
    if check:
        workspace_check(ws)
    return out, (lse if want_lse else None), chunk_idx, group_idx


def decode_step_noalloc(Q, K, V, chunk_mean, group_mean, seq_len, chunk, group, k_chunk,
                        k_group, layout=None, scale=0.0, want_chunks=True, want_lse=True,
                        chunk_idx=None, group_idx=None, out=None, lse=None, reset=False):
    """decode_step_ex whose scratch is the library's fixed per-device array (no
    workspace; the library call allocates nothing; outputs given as out=,
    lse=, group_idx=, chunk_idx= are used as they are). reset=True clears the
    array's zero region first (after NaN rows from a wait that gave up).
    Returns (O, lse, chunk_idx, group_idx)."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, host_ok=True)
    _need(V, "V", 4, host_ok=True)
    B, Hq, Nq, D = Q.shape
    Hkv = chunk_mean.shape[1]
    if tuple(V.shape) != tuple(K.shape):
        raise ValueError("K and V differ in shape")
    shape = _shape(Q, Hkv, seq_len)
    if want_chunks and chunk_idx is None:
        chunk_idx = torch.empty((B, Hq, Nq, k_chunk + 2), dtype=torch.int32, device=Q.device)
    if group_idx is None:
        group_idx = torch.empty((B, Hq, Nq, k_group), dtype=torch.int32, device=Q.device)
    if out is None:
        out = torch.empty_like(Q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=Q.device)
    _check(_lib.hga_decode_step_noalloc(ctypes.byref(shape), _lay(layout), _ptr(Q), _ptr(K),
                                        _ptr(V), _dtype_code(Q), _ptr(chunk_mean),
                                        _ptr(group_mean), chunk, group, k_chunk, k_group,
                                        float(scale), _ptr(chunk_idx if want_chunks else None),
                                        _ptr(group_idx), _ptr(out),
                                        _ptr(lse if want_lse else None), 1 if reset else 0,
                                        _stream(Q.device)), "hga_decode_step_noalloc")
    return out, (lse if want_lse else None), chunk_idx, group_idx


def attend_staged_sizes(shape: Shape, group, k_group):
    pages, nbytes = ctypes.c_int64(), ctypes.c_size_t()
    _check(_lib.hga_attend_staged_sizes(ctypes.byref(shape), group, k_group, ctypes.byref(pages),
                                        ctypes.byref(nbytes)), "hga_attend_staged_sizes")
    return pages.value, nbytes.value


def attend_staged(Q, K, V, group_idx, group, scale=0.0, want_lse=True, out=None, lse=None,
                  pools=None, workspace=None):
    """attend for slowly read K/V (e.g. pinned host memory): each (sequence, KV
    head)'s distinct routed groups are copied once into a device pool, then
    attention reads the pool. Same results as attend."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, host_ok=True)
    _need(V, "V", 4, host_ok=True)
    _need(group_idx, "group_idx", 4)
    B, Hq, Nq, D = Q.shape
    Bk, Hkv, T, Dk = K.shape
    if (Bk, Dk) != (B, D) or tuple(V.shape) != tuple(K.shape):
        raise ValueError("K/V do not match Q")
    k_group = group_idx.shape[3]
    shape = _shape(Q, Hkv, T)
    pages, nbytes = attend_staged_sizes(shape, group, k_group)
    ws = workspace if workspace is not None else _workspace(Q.device, "staged", nbytes)
    if pools is None:
        kp = _workspace(Q.device, "pool_k", pages * group * D * Q.element_size())
        vp = _workspace(Q.device, "pool_v", pages * group * D * Q.element_size())
    else:
        kp, vp = pools
    if out is None:
        out = torch.empty_like(Q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=Q.device)
    _check(_lib.hga_attend_staged(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q),
                                  _ptr(group_idx), k_group, group, float(scale), _ptr(out),
                                  _ptr(lse if want_lse else None), _ptr(kp), _ptr(vp), pages,
                                  _ptr(ws), ws.numel(), _stream(Q.device)), "hga_attend_staged")
    return out, (lse if want_lse else None)

