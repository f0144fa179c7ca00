"""Thin ctypes binding of libheadcast.so (include/headcast.h).

Argument marshalling only: every step runs in the library's HIP kernels. Device
memory is torch tensors (their data_ptr), streams are torch's current HIP stream.
The functions keep the C names. Loading fails loudly when the library is missing.

One layer of an autoregressive rollout (tensors [tokens][H][d] bf16 on the GPU):

    desc = make_desc(geometry)                       # or LayerDesc(...) by hand
    labels, stats = hc_classify_heads(desc, hc_default_classify_params(), q, k_hist,
                                      v_hist, n_hist_frames, k_cur, v_cur)  # once
    buf = hc_build_head_buffers(desc, labels, k_hist, v_hist, n_hist_frames)
    ws = routed_workspace(buf)                       # serves every later fill state
    for each denoising step of the block:
        out = hc_routed_attention(buf, q, k_cur, v_cur, workspace=ws)
    hc_append_chunk(buf, k_cur, v_cur)               # the finished block enters the ring
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# HEADCAST_LIBRARY selects another build of the same library (the host-sanitizer build
# of the CPU tests); either way a missing file is an error, never a fallback.
LIB_PATH = os.environ.get("HEADCAST_LIBRARY") or os.path.join(HERE, "libheadcast.so")

SINK, DUMMY, SPATIAL, GLOBAL = 0, 1, 2, 3
HC_BF16, HC_F32 = 0, 1
HC_VARIANT_DUMMY_PREVIOUS, HC_VARIANT_SPATIAL_CELLS, HC_VARIANT_SPATIAL_OWN_LAUNCH = 1, 2, 4
KERNEL_KINDS = ("dense", "merge", "spatial", "copy", "stats", "fp32")


class HCError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frame_h", ctypes.c_int32), ("frame_w", ctypes.c_int32),
                ("chunk_frames", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("variant", ctypes.c_int32)]


class ClassifyParams(ctypes.Structure):
    _fields_ = [("theta_sink", ctypes.c_float), ("theta_dummy", ctypes.c_float),
                ("theta_spatial", ctypes.c_float), ("theta_score", ctypes.c_float),
                ("gamma", ctypes.c_float), ("percentile", ctypes.c_float),
                ("proxy_grid_h", ctypes.c_int32), ("proxy_grid_w", ctypes.c_int32),
                ("sink_proxy_includes_current", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SIGS = {
    "hc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hc_last_error": (ctypes.c_char_p, []),
    "hc_default_classify_params": (ctypes.c_int, [ctypes.POINTER(ClassifyParams)]),
    "hc_head_buffers_bytes": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, ctypes.POINTER(_SZ)]),
    "hc_build_head_buffers": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _P, _P, _I32, _P, _SZ,
                                             ctypes.POINTER(_P), _P]),
    "hc_build_head_buffers_at": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _P, _P, _I32, _I64, _P, _SZ,
                                                ctypes.POINTER(_P), _P]),
    "hc_plan_head_buffers": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _P, _I64, ctypes.POINTER(_P)]),
    "hc_append_chunk": (ctypes.c_int, [_P, _P, _P, _P]),
    "hc_buffers_state": (ctypes.c_int, [_P, ctypes.POINTER(_I64)]),
    "hc_free_head_buffers": (ctypes.c_int, [_P]),
    "hc_routed_workspace_bytes": (ctypes.c_int, [_P, ctypes.POINTER(_SZ)]),
    "hc_routed_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _SZ, _P]),
    "hc_routed_attention_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "hc_classify_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(LayerDesc),
                                                   ctypes.POINTER(ClassifyParams), _I32,
                                                   ctypes.POINTER(_SZ)]),
    "hc_classify_heads": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(ClassifyParams),
                                         _P, _P, _P, _I32, _P, _P, _P, _SZ, _P, _P, _P]),
    "hc_reduce_statistics": (ctypes.c_int, [_P, _I64, _I32, ctypes.c_double, ctypes.c_double, _P]),
    "hc_decide": (_I32, [ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                         ctypes.POINTER(ClassifyParams)]),
    "hc_debug_slot_table": (ctypes.c_int, [_P, _P]),
    "hc_debug_head_region": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                                            ctypes.POINTER(_I64)]),
    "hc_debug_gather_origins": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _I32, _I32, _P, _P]),
    "hc_debug_routed_plan": (ctypes.c_int, [_P, _P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "hc_debug_dense_queues": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(_I32)]),
    "hc_debug_spatial_plan": (ctypes.c_int, [_P, _P]),
    "hc_timing_enable": (ctypes.c_int, [_I32]),
    "hc_timing_read": (ctypes.c_int, [_P, _P]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def lib():
    """The loaded library; raises if it was not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with head_routed_sparse_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise HCError(status, lib().hc_last_error().decode())


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _elem(desc):
    """torch dtype of a layer's tensors."""
    import torch
    return torch.bfloat16 if desc.dtype == HC_BF16 else torch.float32


def _dev(t, name, dtype=None, numel=0):
    """Device pointer of a tensor the kernels read or write: a contiguous GPU tensor of
    the layer's dtype with at least `numel` elements (the C ABI sees only the pointer,
    so these are checked here, before any call)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise HCError(7, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise HCError(2, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise HCError(3, f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() < numel:
        raise HCError(2, f"{name} has {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _block_numel(desc):
    """Elements of one block's [C*S][H][d] tensor."""
    return desc.chunk_frames * desc.frame_h * desc.frame_w * desc.num_heads * desc.head_dim


def make_desc(geom, variant: int = 0) -> LayerDesc:
    """LayerDesc from an object with the Geometry fields (see inputs.Geometry)."""
    return LayerDesc(geom.num_heads, geom.head_dim, geom.frame_h, geom.frame_w,
                     geom.chunk_frames, geom.window_frames, geom.grid_h, geom.grid_w,
                     float(geom.softmax_scale), HC_BF16 if geom.dtype == "bf16" else HC_F32, int(variant))


def hc_default_classify_params(**overrides) -> ClassifyParams:
    p = ClassifyParams()
    _check(lib().hc_default_classify_params(ctypes.byref(p)))
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


def _labels_arr(labels):
    return np.ascontiguousarray(np.asarray(labels, dtype=np.int32))


def hc_head_buffers_bytes(desc: LayerDesc, labels) -> int:
    n = _SZ()
    lab = _labels_arr(labels)
    _check(lib().hc_head_buffers_bytes(ctypes.byref(desc), lab.ctypes.data_as(_P), ctypes.byref(n)))
    return n.value


class HeadBuffers:
    """Host handle of the per-head buffers plus the device tensor they live in."""

    def __init__(self, handle, memory, desc):
        self.handle = handle
        self.memory = memory
        self.desc = desc

    def __del__(self):
        if self.handle and _lib is not None:
            _lib.hc_free_head_buffers(self.handle)
            self.handle = None


def hc_build_head_buffers(desc: LayerDesc, labels, k_hist, v_hist, n_hist_frames: int,
                          memory=None, stream=None) -> HeadBuffers:
    import torch
    lab = _labels_arr(labels)
    nbytes = hc_head_buffers_bytes(desc, lab)
    hist = int(n_hist_frames) * desc.frame_h * desc.frame_w * desc.num_heads * desc.head_dim
    kp = _dev(k_hist, "k_hist", _elem(desc), hist)
    vp = _dev(v_hist, "v_hist", _elem(desc), hist)
    if memory is None:
        memory = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    mp = _dev(memory, "memory", torch.uint8)
    h = _P()
    _check(lib().hc_build_head_buffers(ctypes.byref(desc), lab.ctypes.data_as(_P), kp, vp,
                                       int(n_hist_frames), mp, memory.numel(), ctypes.byref(h),
                                       _stream(stream)))
    return HeadBuffers(h, memory, desc)


def hc_build_head_buffers_at(desc: LayerDesc, labels, k_hist, v_hist, n_hist_frames: int, next_block: int,
                             memory=None, stream=None) -> HeadBuffers:
    """Buffers of a rollout resumed with `next_block` as the next block to append; the
    history tensors hold the window's blocks in logical order (sink block first)."""
    import torch
    lab = _labels_arr(labels)
    nbytes = hc_head_buffers_bytes(desc, lab)
    hist = int(n_hist_frames) * desc.frame_h * desc.frame_w * desc.num_heads * desc.head_dim
    kp = _dev(k_hist, "k_hist", _elem(desc), hist)
    vp = _dev(v_hist, "v_hist", _elem(desc), hist)
    if memory is None:
        memory = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    mp = _dev(memory, "memory", torch.uint8)
    h = _P()
    _check(lib().hc_build_head_buffers_at(ctypes.byref(desc), lab.ctypes.data_as(_P), kp, vp,
                                          int(n_hist_frames), int(next_block), mp, memory.numel(),
                                          ctypes.byref(h), _stream(stream)))
    return HeadBuffers(h, memory, desc)


def hc_plan_head_buffers(desc: LayerDesc, labels, next_block: int) -> HeadBuffers:
    lab = _labels_arr(labels)
    h = _P()
    _check(lib().hc_plan_head_buffers(ctypes.byref(desc), lab.ctypes.data_as(_P), int(next_block),
                                      ctypes.byref(h)))
    return HeadBuffers(h, None, desc)


def hc_append_chunk(buffers: HeadBuffers, k_chunk, v_chunk, stream=None):
    d, n = buffers.desc, _block_numel(buffers.desc)
    _check(lib().hc_append_chunk(buffers.handle, _dev(k_chunk, "k_chunk", _elem(d), n),
                                 _dev(v_chunk, "v_chunk", _elem(d), n), _stream(stream)))


def hc_buffers_state(buffers: HeadBuffers) -> int:
    n = _I64()
    _check(lib().hc_buffers_state(buffers.handle, ctypes.byref(n)))
    return n.value


def hc_routed_workspace_bytes(buffers: HeadBuffers) -> int:
    n = _SZ()
    _check(lib().hc_routed_workspace_bytes(buffers.handle, ctypes.byref(n)))
    return n.value


def routed_workspace(buffers: HeadBuffers):
    import torch
    return torch.empty(max(hc_routed_workspace_bytes(buffers), 16), dtype=torch.uint8, device="cuda")


def hc_routed_attention(buffers: HeadBuffers, q, k_cur, v_cur, out=None, workspace=None, stream=None):
    import torch
    d, n = buffers.desc, _block_numel(buffers.desc)
    qp = _dev(q, "q", _elem(d), n)
    kp = _dev(k_cur, "k_cur", _elem(d), n)
    vp = _dev(v_cur, "v_cur", _elem(d), n)
    if out is None:
        out = torch.empty_like(q)
    op = _dev(out, "out", _elem(d), n)
    if workspace is None:
        workspace = routed_workspace(buffers)
    wp = _dev(workspace, "workspace", torch.uint8)
    _check(lib().hc_routed_attention(buffers.handle, qp, kp, vp, op, wp, workspace.numel(), _stream(stream)))
    return out


def hc_routed_attention_noalloc(buffers: HeadBuffers, q, k_cur, v_cur, out=None, stream=None):
    """The routed step with the library's own scratch for partial results (no
    workspace argument, no allocation in the library)."""
    import torch
    d, n = buffers.desc, _block_numel(buffers.desc)
    qp = _dev(q, "q", _elem(d), n)
    kp = _dev(k_cur, "k_cur", _elem(d), n)
    vp = _dev(v_cur, "v_cur", _elem(d), n)
    if out is None:
        out = torch.empty_like(q)
    op = _dev(out, "out", _elem(d), n)
    _check(lib().hc_routed_attention_noalloc(buffers.handle, qp, kp, vp, op, _stream(stream)))
    return out


def hc_classify_workspace_bytes(desc: LayerDesc, params: ClassifyParams, n_hist_frames: int) -> int:
    n = _SZ()
    _check(lib().hc_classify_workspace_bytes(ctypes.byref(desc), ctypes.byref(params),
                                             int(n_hist_frames), ctypes.byref(n)))
    return n.value


def hc_classify_heads(desc: LayerDesc, params: ClassifyParams, q, k_hist, v_hist, n_hist_frames,
                      k_cur, v_cur, workspace=None, stream=None):
    """Returns (labels int32 [H], stats float64 [H][6])."""
    import torch
    n = _block_numel(desc)
    hist = int(n_hist_frames) * desc.frame_h * desc.frame_w * desc.num_heads * desc.head_dim
    ptrs = [_dev(q, "q", _elem(desc), n), _dev(k_hist, "k_hist", _elem(desc), hist),
            _dev(v_hist, "v_hist", _elem(desc), hist), _dev(k_cur, "k_cur", _elem(desc), n),
            _dev(v_cur, "v_cur", _elem(desc), n)]
    if workspace is None:
        workspace = torch.empty(hc_classify_workspace_bytes(desc, params, n_hist_frames),
                                dtype=torch.uint8, device="cuda")
    wp = _dev(workspace, "workspace", torch.uint8)
    H = desc.num_heads
    labels = np.zeros(H, np.int32)
    stats = np.zeros((H, 6), np.float64)
    _check(lib().hc_classify_heads(ctypes.byref(desc), ctypes.byref(params), ptrs[0], ptrs[1], ptrs[2],
                                   int(n_hist_frames), ptrs[3], ptrs[4], wp, workspace.numel(),
                                   labels.ctypes.data_as(_P), stats.ctypes.data_as(_P), _stream(stream)))
    return labels, stats


def hc_reduce_statistics(per_token: np.ndarray, head_dim: int, gamma: float, percentile: float = 5.0):
    a = np.ascontiguousarray(per_token, dtype=np.float32)
    out = np.zeros(6, np.float64)
    _check(lib().hc_reduce_statistics(a.ctypes.data_as(_P), a.shape[0], head_dim, gamma, percentile,
                                      out.ctypes.data_as(_P)))
    return out


def hc_decide(cos_sink, cos_dummy, cos_spatial, score, params: ClassifyParams = None) -> int:
    return int(lib().hc_decide(cos_sink, cos_dummy, cos_spatial, score,
                               ctypes.byref(params) if params is not None else None))


def hc_debug_slot_table(buffers: HeadBuffers) -> np.ndarray:
    d = buffers.desc
    t = np.zeros((d.num_heads, d.window_frames - d.chunk_frames), np.int32)
    _check(lib().hc_debug_slot_table(buffers.handle, t.ctypes.data_as(_P)))
    return t


def hc_debug_head_region(buffers: HeadBuffers, head: int):
    k, v, r = _I64(), _I64(), _I64()
    _check(lib().hc_debug_head_region(buffers.handle, head, ctypes.byref(k), ctypes.byref(v), ctypes.byref(r)))
    return k.value, v.value, r.value


def hc_debug_gather_origins(desc: LayerDesc, grid_h: int, grid_w: int, stream=None):
    import torch
    out = torch.empty((desc.frame_h * desc.frame_w, 2), dtype=torch.int32, device="cuda")
    _check(lib().hc_debug_gather_origins(ctypes.byref(desc), grid_h, grid_w, _ptr(out), _stream(stream)))
    return out


def hc_debug_routed_plan(buffers: HeadBuffers):
    n, items = _I32(), _I32()
    _check(lib().hc_debug_routed_plan(buffers.handle, None, 0, ctypes.byref(n), ctypes.byref(items)))
    e = np.zeros((n.value, 8), np.int32)
    _check(lib().hc_debug_routed_plan(buffers.handle, e.ctypes.data_as(_P), n.value, ctypes.byref(n),
                                      ctypes.byref(items)))
    return e, items.value


def hc_debug_dense_queues(buffers: HeadBuffers):
    """XCD queues of the routed call's dense launch: a list of 8 lists of (first, count)
    runs, and the longest queue."""
    runs = np.zeros((8, 16, 2), np.int32)
    n = np.zeros(8, np.int32)
    ln = _I32()
    _check(lib().hc_debug_dense_queues(buffers.handle, runs.ctypes.data_as(_P), n.ctypes.data_as(_P),
                                       ctypes.byref(ln)))
    return [[tuple(int(v) for v in runs[x, r]) for r in range(n[x])] for x in range(8)], ln.value


def hc_debug_spatial_plan(buffers: HeadBuffers):
    """(tile rows, tile columns, frame parts, partial slots, Spatial tiles in the dense
    launch) of the routed call."""
    p = np.zeros(5, np.int32)
    _check(lib().hc_debug_spatial_plan(buffers.handle, p.ctypes.data_as(_P)))
    return tuple(int(x) for x in p)


def hc_timing_enable(on: bool = True):
    _check(lib().hc_timing_enable(1 if on else 0))


def hc_timing_read():
    """Per kernel kind: (total ms, launches); synchronises the recorded events."""
    ms = np.zeros(6, np.float64)
    cnt = np.zeros(6, np.int64)
    _check(lib().hc_timing_read(ms.ctypes.data_as(_P), cnt.ctypes.data_as(_P)))
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_KINDS)}
