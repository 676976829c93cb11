"""ctypes binding of libnomas_attn.so (include/nomas_attn.h).

Argument marshalling only: every computation runs in the library.  Function
names match the C ABI.  Tensors are torch tensors used as device memory; the
stream argument defaults to torch's current stream on the tensor's device.
"""
from __future__ import annotations

import ctypes as C
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libnomas_attn.so")
HEADER = os.path.join(ROOT, "include", "nomas_attn.h")

MAX_ACTIONS = 32
HEAD_DIM = 128

OK, ERR_INVALID_ARGUMENT, ERR_LAYOUT, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_STALE_PLAN, \
    ERR_ALIGNMENT, ERR_HIP = range(8)
TEXT_QUERY = {"R": 0, "K": 1, "H": 2}
PLAN_HOST_ONLY = 1
PLAN_GRAD_F32 = 2
PLAN_KV_HEAD_MAJOR = 4
TILE_EMPTY, TILE_FULL, TILE_PARTIAL = 0, 1, 2


class nomas_action(C.Structure):
    _fields_ = [("n_tokens", C.c_int32), ("frame_lo", C.c_int32), ("frame_hi", C.c_int32)]


class nomas_segment(C.Structure):
    _fields_ = [("video", C.c_int32), ("index", C.c_int32), ("n_frames", C.c_int32),
                ("tokens_per_frame", C.c_int32), ("n_head", C.c_int32),
                ("n_actions", C.c_int32), ("n_pad", C.c_int32), ("reserved", C.c_int32),
                ("actions", nomas_action * MAX_ACTIONS)]


class nomas_layout(C.Structure):
    _fields_ = [("n_segments", C.c_int32), ("segments", C.POINTER(nomas_segment))]


class nomas_plan_opts(C.Structure):
    _fields_ = [("num_heads", C.c_int32), ("head_dim", C.c_int32), ("block_q", C.c_int32),
                ("block_k", C.c_int32), ("text_query_mode", C.c_int32), ("flags", C.c_int32),
                ("window_segments", C.c_int32), ("video_keep_percent", C.c_int32)]


class nomas_plan_info(C.Structure):
    _fields_ = [("n_queries", C.c_int64), ("n_keys", C.c_int64), ("n_cached_keys", C.c_int64),
                ("n_q_tiles", C.c_int64), ("n_k_tiles", C.c_int64),
                ("n_empty_tiles", C.c_int64), ("n_full_tiles", C.c_int64),
                ("n_partial_tiles", C.c_int64), ("unmasked_pairs", C.c_int64),
                ("executed_pairs", C.c_int64), ("effective_flop", C.c_double),
                ("block_q", C.c_int32), ("block_k", C.c_int32), ("num_heads", C.c_int32),
                ("text_query_mode", C.c_int32), ("sparse_list_entries", C.c_int64),
                ("video_keep_percent", C.c_int32), ("window_segments", C.c_int32)]


class nomas_camera_plan_info(C.Structure):
    _fields_ = [("n_queries", C.c_int64), ("n_video_queries", C.c_int64),
                ("n_camera_tokens", C.c_int64), ("visible_pairs", C.c_int64),
                ("effective_flop", C.c_double), ("algorithmic_bytes", C.c_double),
                ("num_heads", C.c_int32), ("radius_frames", C.c_int32)]


class NomasError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


_lib = None


def load():
    """Load the shared library; raise if it is not built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m segment_causal_masked_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    sig = {
        "nomas_attn_plan": [C.POINTER(nomas_layout), C.POINTER(nomas_layout), P,
                            C.POINTER(nomas_plan_opts), C.POINTER(P)],
        "nomas_plan_get_info": [P, C.POINTER(nomas_plan_info)],
        "nomas_plan_export_classes": [P, P, SZ],
        "nomas_plan_destroy": [P],
        "nomas_attn_fwd_workspace_size": [P, C.POINTER(SZ)],
        "nomas_attn_fwd": [P, P, P, I64, P, P, I64, P, I64, P, F32, P, SZ, P],
        "nomas_attn_fwd_noalloc": [P, P, P, I64, P, P, I64, P, I64, P, F32, P],
        "nomas_attn_bwd_workspace_size": [P, C.POINTER(SZ)],
        "nomas_action_latent_window": [I64, I64, I64, C.POINTER(I32), C.POINTER(I32)],
        "nomas_attn_bwd": [P, P, P, P, P, P, P, I64, I64, P, P, P, F32, P, SZ, P],
        "nomas_kvcache_create": [I32, I32, I64, P, P, C.POINTER(P)],
        "nomas_kvcache_append": [P, C.POINTER(nomas_segment), P, P, I64, P],
        "nomas_kvcache_truncate": [P, I32],
        "nomas_kvcache_reset": [P],
        "nomas_kvcache_len": [P, C.POINTER(I64), C.POINTER(I32)],
        "nomas_kvcache_destroy": [P],
        "nomas_kvcache_int8_create": [I32, I32, I64, P, P, P, P, C.POINTER(P)],
        "nomas_kvcache_int8_append": [P, C.POINTER(nomas_segment), P, P, I64, P],
        "nomas_kvcache_int8_expand": [P, P, P],
        "nomas_kvcache_int8_truncate": [P, I32],
        "nomas_kvcache_adopt": [P, C.POINTER(nomas_segment), I32],
        "nomas_kvcache_int8_adopt": [P, C.POINTER(nomas_segment), I32],
        "nomas_kvcache_int8_len": [P, C.POINTER(I64), C.POINTER(I32)],
        "nomas_kvcache_int8_destroy": [P],
        "nomas_camera_attn_plan": [C.POINTER(nomas_layout), I32, I32, I32, C.POINTER(P)],
        "nomas_camera_plan_get_info": [P, C.POINTER(nomas_camera_plan_info)],
        "nomas_camera_plan_export_ranges": [P, P, SZ],
        "nomas_camera_plan_destroy": [P],
        "nomas_camera_attn_fwd": [P, P, I64, P, P, I64, P, I64, F32, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I32
    lib.nomas_status_string.argtypes = [I32]
    lib.nomas_status_string.restype = C.c_char_p
    lib.nomas_last_error.argtypes = []
    lib.nomas_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def header_functions():
    """Names of the functions include/nomas_attn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nomas_\w+)\s*\(", text)))


def _check(status, where):
    if status != OK:
        lib = load()
        raise NomasError(status, where, lib.nomas_last_error().decode())


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def to_c_segment(s) -> nomas_segment:
    """Any record with video/index/n_frames/tokens_per_frame/n_head/actions/n_pad."""
    c = nomas_segment()
    c.video, c.index = int(s.video), int(s.index)
    c.n_frames, c.tokens_per_frame = int(s.n_frames), int(s.tokens_per_frame)
    c.n_head, c.n_pad = int(s.n_head), int(getattr(s, "n_pad", 0))
    acts = list(s.actions)
    c.n_actions = len(acts)
    for i, (n, lo, hi) in enumerate(acts[:MAX_ACTIONS]):
        c.actions[i].n_tokens, c.actions[i].frame_lo, c.actions[i].frame_hi = int(n), int(lo), int(hi)
    return c


class _Layout:
    """Keeps the ctypes segment array alive with the layout that points to it."""

    def __init__(self, segments):
        segments = list(segments)
        self.arr = (nomas_segment * max(1, len(segments)))()
        for i, s in enumerate(segments):
            self.arr[i] = to_c_segment(s)
        self.c = nomas_layout(len(segments), C.cast(self.arr, C.POINTER(nomas_segment)))


def _stream_ptr(stream, tensor=None):
    if stream is not None:
        return C.c_void_p(int(stream))
    import torch
    dev = tensor.device if tensor is not None else None
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _token_stride(t, name, heads):
    if t is None:
        return 0
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [tokens, {heads}, {HEAD_DIM}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
        raise ValueError(f"{name} must have contiguous heads x dims")
    return t.stride(0)


def _head_stride(t, name, heads):
    """Head stride of a head-major [heads, rows, 128] tensor with contiguous rows."""
    if t is None:
        return 0
    if t.dim() != 3 or t.shape[0] != heads or t.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [{heads}, rows, {HEAD_DIM}] (head-major plan), got {tuple(t.shape)}")
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != HEAD_DIM):
        raise ValueError(f"{name} must have contiguous rows of {HEAD_DIM}")
    return t.stride(0)


def _kv_stride(plan, t, name):
    """The kv_stride argument for new-token K / V (or dK / dV) of this plan."""
    if plan.kv_head_major:
        return _head_stride(t, name, plan.heads)
    return _token_stride(t, name, plan.heads)


# ----------------------------------------------------------------------------
# objects
# ----------------------------------------------------------------------------

class Plan:
    def __init__(self, handle, heads, grad_f32=False, kv_head_major=False):
        self.handle = C.c_void_p(handle)
        self.heads = heads
        self.grad_f32 = grad_f32
        self.kv_head_major = kv_head_major

    def info(self) -> nomas_plan_info:
        return nomas_plan_get_info(self)

    def __del__(self):
        if getattr(self, "handle", None) and self.handle.value and _lib is not None:
            _lib.nomas_plan_destroy(self.handle)
            self.handle = C.c_void_p(0)


class KVCacheInt8:
    """INT8 cache handle plus the caller-owned storage: codes [H][capacity][128]
    and exponents [H][capacity], int8."""

    def __init__(self, handle, k_codes, v_codes, k_exp, v_exp, heads, capacity):
        self.handle = C.c_void_p(handle)
        self.k_codes, self.v_codes, self.k_exp, self.v_exp = k_codes, v_codes, k_exp, v_exp
        self.heads, self.capacity = heads, capacity

    def __del__(self):
        if getattr(self, "handle", None) and self.handle.value and _lib is not None:
            _lib.nomas_kvcache_int8_destroy(self.handle)
            self.handle = C.c_void_p(0)


class CameraPlan:
    def __init__(self, handle, heads):
        self.handle = C.c_void_p(handle)
        self.heads = heads

    def info(self) -> nomas_camera_plan_info:
        return nomas_camera_plan_get_info(self)

    def __del__(self):
        if getattr(self, "handle", None) and self.handle.value and _lib is not None:
            _lib.nomas_camera_plan_destroy(self.handle)
            self.handle = C.c_void_p(0)


class KVCache:
    """Cache handle plus the caller-owned K/V storage ([H][capacity][128] bf16)."""

    def __init__(self, handle, k_buf, v_buf, heads, capacity):
        self.handle = C.c_void_p(handle)
        self.k_buf, self.v_buf = k_buf, v_buf
        self.heads, self.capacity = heads, capacity

    def __del__(self):
        if getattr(self, "handle", None) and self.handle.value and _lib is not None:
            _lib.nomas_kvcache_destroy(self.handle)
            self.handle = C.c_void_p(0)


# ----------------------------------------------------------------------------
# the ABI, function by function
# ----------------------------------------------------------------------------

def nomas_attn_plan(q_layout, kv_layout, cache=None, *, heads=16, mode="R", host_only=False,
                    block_q=0, block_k=0, window=0, video_keep_percent=0, grad_f32=False,
                    kv_head_major=False) -> Plan:
    lib = load()
    ql, kl = _Layout(q_layout), _Layout(kv_layout)
    flags = ((PLAN_HOST_ONLY if host_only else 0) | (PLAN_GRAD_F32 if grad_f32 else 0) |
             (PLAN_KV_HEAD_MAJOR if kv_head_major else 0))
    opts = nomas_plan_opts(heads, HEAD_DIM, block_q, block_k, TEXT_QUERY[mode], flags, window,
                           video_keep_percent)
    out = C.c_void_p()
    _check(lib.nomas_attn_plan(C.byref(ql.c), C.byref(kl.c),
                               cache.handle if cache is not None else None,
                               C.byref(opts), C.byref(out)), "nomas_attn_plan")
    return Plan(out.value, heads, grad_f32, kv_head_major)


def nomas_plan_get_info(plan) -> nomas_plan_info:
    info = nomas_plan_info()
    _check(load().nomas_plan_get_info(plan.handle, C.byref(info)), "nomas_plan_get_info")
    return info


def nomas_plan_export_classes(plan):
    import numpy as np
    info = nomas_plan_get_info(plan)
    buf = np.zeros((info.n_q_tiles, info.n_k_tiles), np.uint8)
    _check(load().nomas_plan_export_classes(plan.handle, buf.ctypes.data_as(C.c_void_p),
                                            buf.size), "nomas_plan_export_classes")
    return buf


def nomas_attn_fwd_workspace_size(plan) -> int:
    n = C.c_size_t()
    _check(load().nomas_attn_fwd_workspace_size(plan.handle, C.byref(n)), "nomas_attn_fwd_workspace_size")
    return n.value


def nomas_attn_fwd(plan, cache, q, k_new, v_new, o, lse=None, scale=HEAD_DIM ** -0.5,
                   workspace=None, stream=None):
    h = plan.heads
    qs = _token_stride(q, "q", h)
    os_ = _token_stride(o, "o", h)
    ks = _kv_stride(plan, k_new, "k_new")
    vs = _kv_stride(plan, v_new, "v_new")
    if k_new is not None and v_new is not None and ks != vs:
        raise ValueError("k_new and v_new must share a stride")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().nomas_attn_fwd(plan.handle, cache.handle if cache is not None else None,
                                 _ptr(q), qs, _ptr(k_new), _ptr(v_new), ks, _ptr(o), os_,
                                 _ptr(lse), float(scale), _ptr(workspace), ws_bytes,
                                 _stream_ptr(stream, q)), "nomas_attn_fwd")


def nomas_attn_fwd_noalloc(plan, cache, q, k_new, v_new, o, lse=None, scale=HEAD_DIM ** -0.5,
                           stream=None):
    h = plan.heads
    qs = _token_stride(q, "q", h)
    os_ = _token_stride(o, "o", h)
    ks = _kv_stride(plan, k_new, "k_new")
    vs = _kv_stride(plan, v_new, "v_new")
    if k_new is not None and v_new is not None and ks != vs:
        raise ValueError("k_new and v_new must share a stride")
    _check(load().nomas_attn_fwd_noalloc(plan.handle, cache.handle if cache is not None else None,
                                         _ptr(q), qs, _ptr(k_new), _ptr(v_new), ks, _ptr(o), os_,
                                         _ptr(lse), float(scale), _stream_ptr(stream, q)),
           "nomas_attn_fwd_noalloc")


def nomas_attn_bwd_workspace_size(plan) -> int:
    n = C.c_size_t()
    _check(load().nomas_attn_bwd_workspace_size(plan.handle, C.byref(n)), "nomas_attn_bwd_workspace_size")
    return n.value


def nomas_attn_bwd(plan, q, k, v, o, d_o, lse, dq, dk, dv, scale=HEAD_DIM ** -0.5,
                   workspace=None, stream=None):
    h = plan.heads
    qs = _token_stride(q, "q", h)
    for name, t in (("o", o), ("d_o", d_o), ("dq", dq)):
        if _token_stride(t, name, h) != qs:
            raise ValueError(f"{name} must share q's token stride")
    ks = _kv_stride(plan, k, "k")
    for name, t in (("v", v), ("dk", dk), ("dv", dv)):
        if _kv_stride(plan, t, name) != ks:
            raise ValueError(f"{name} must share k's stride")
    want = "torch.float32" if plan.grad_f32 else "torch.bfloat16"
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None and str(t.dtype) != want:
            raise ValueError(f"{name} must be {want} for this plan")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().nomas_attn_bwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o),
                                 _ptr(lse), qs, ks, _ptr(dq), _ptr(dk), _ptr(dv), float(scale),
                                 _ptr(workspace), ws_bytes, _stream_ptr(stream, q)),
           "nomas_attn_bwd")


def nomas_action_latent_window(first, end, n_pixel_frames):
    """(frame_lo, frame_hi) in latent frames of an action over pixel frames
    [first, end) of a segment of n_pixel_frames frames."""
    lo, hi = C.c_int32(), C.c_int32()
    _check(load().nomas_action_latent_window(int(first), int(end), int(n_pixel_frames),
                                             C.byref(lo), C.byref(hi)), "nomas_action_latent_window")
    return lo.value, hi.value


def nomas_kvcache_create(heads, capacity, k_buf, v_buf) -> KVCache:
    for name, t in (("k_buf", k_buf), ("v_buf", v_buf)):
        if tuple(t.shape) != (heads, capacity, HEAD_DIM) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{heads}, {capacity}, {HEAD_DIM}] tensor")
    out = C.c_void_p()
    _check(load().nomas_kvcache_create(heads, HEAD_DIM, capacity, _ptr(k_buf), _ptr(v_buf),
                                       C.byref(out)), "nomas_kvcache_create")
    return KVCache(out.value, k_buf, v_buf, heads, capacity)


def nomas_kvcache_append(cache, segment, k_new, v_new, stream=None):
    ks = _token_stride(k_new, "k_new", cache.heads)
    if _token_stride(v_new, "v_new", cache.heads) != ks:
        raise ValueError("k_new and v_new must share a token stride")
    seg = to_c_segment(segment)
    _check(load().nomas_kvcache_append(cache.handle, C.byref(seg), _ptr(k_new), _ptr(v_new), ks,
                                       _stream_ptr(stream, k_new)), "nomas_kvcache_append")


def nomas_kvcache_truncate(cache, n_segments):
    _check(load().nomas_kvcache_truncate(cache.handle, n_segments), "nomas_kvcache_truncate")


def nomas_kvcache_adopt(cache, segments):
    lay = _Layout(segments)
    _check(load().nomas_kvcache_adopt(cache.handle, lay.c.segments, lay.c.n_segments),
           "nomas_kvcache_adopt")


def nomas_kvcache_reset(cache):
    _check(load().nomas_kvcache_reset(cache.handle), "nomas_kvcache_reset")


def nomas_kvcache_len(cache):
    n, s = C.c_int64(), C.c_int32()
    _check(load().nomas_kvcache_len(cache.handle, C.byref(n), C.byref(s)), "nomas_kvcache_len")
    return n.value, s.value


def nomas_kvcache_int8_create(heads, capacity, device="cuda", buffers=None) -> KVCacheInt8:
    """Allocates the int8 storage (torch tensors) and creates the handle;
    buffers=(k_codes, v_codes, k_exp, v_exp) uses existing storage instead."""
    import torch
    if buffers is None:
        kc = torch.zeros((heads, capacity, HEAD_DIM), dtype=torch.int8, device=device)
        vc = torch.zeros_like(kc)
        ke = torch.zeros((heads, capacity), dtype=torch.int8, device=device)
        ve = torch.zeros_like(ke)
    else:
        kc, vc, ke, ve = buffers
        for t, shape in ((kc, (heads, capacity, HEAD_DIM)), (vc, (heads, capacity, HEAD_DIM)),
                         (ke, (heads, capacity)), (ve, (heads, capacity))):
            if tuple(t.shape) != shape or not t.is_contiguous() or str(t.dtype) != "torch.int8":
                raise ValueError(f"INT8 cache buffers must be contiguous int8 {shape}")
    out = C.c_void_p()
    _check(load().nomas_kvcache_int8_create(heads, HEAD_DIM, capacity, _ptr(kc), _ptr(vc), _ptr(ke),
                                            _ptr(ve), C.byref(out)), "nomas_kvcache_int8_create")
    return KVCacheInt8(out.value, kc, vc, ke, ve, heads, capacity)


def nomas_kvcache_int8_append(cache, segment, k_new, v_new, stream=None):
    ks = _token_stride(k_new, "k_new", cache.heads)
    if _token_stride(v_new, "v_new", cache.heads) != ks:
        raise ValueError("k_new and v_new must share a token stride")
    seg = to_c_segment(segment)
    _check(load().nomas_kvcache_int8_append(cache.handle, C.byref(seg), _ptr(k_new), _ptr(v_new), ks,
                                            _stream_ptr(stream, k_new)), "nomas_kvcache_int8_append")


def nomas_kvcache_int8_expand(cache, dst, stream=None):
    _check(load().nomas_kvcache_int8_expand(cache.handle, dst.handle, _stream_ptr(stream, dst.k_buf)),
           "nomas_kvcache_int8_expand")


def nomas_kvcache_int8_truncate(cache, n_segments):
    _check(load().nomas_kvcache_int8_truncate(cache.handle, n_segments), "nomas_kvcache_int8_truncate")


def nomas_kvcache_int8_adopt(cache, segments):
    lay = _Layout(segments)
    _check(load().nomas_kvcache_int8_adopt(cache.handle, lay.c.segments, lay.c.n_segments),
           "nomas_kvcache_int8_adopt")


def nomas_kvcache_int8_len(cache):
    n, s = C.c_int64(), C.c_int32()
    _check(load().nomas_kvcache_int8_len(cache.handle, C.byref(n), C.byref(s)), "nomas_kvcache_int8_len")
    return n.value, s.value


def nomas_kvcache_int8_destroy(cache):
    if cache.handle.value:
        _check(load().nomas_kvcache_int8_destroy(cache.handle), "nomas_kvcache_int8_destroy")
        cache.handle = C.c_void_p(0)


def nomas_camera_attn_plan(q_layout, *, heads=16, radius=-1, host_only=False) -> CameraPlan:
    ql = _Layout(q_layout)
    out = C.c_void_p()
    _check(load().nomas_camera_attn_plan(C.byref(ql.c), heads, radius,
                                         PLAN_HOST_ONLY if host_only else 0, C.byref(out)),
           "nomas_camera_attn_plan")
    return CameraPlan(out.value, heads)


def nomas_camera_plan_get_info(plan) -> nomas_camera_plan_info:
    info = nomas_camera_plan_info()
    _check(load().nomas_camera_plan_get_info(plan.handle, C.byref(info)), "nomas_camera_plan_get_info")
    return info


def nomas_camera_plan_export_ranges(plan):
    import numpy as np
    info = nomas_camera_plan_get_info(plan)
    buf = np.zeros((info.n_queries, 2), np.int32)
    _check(load().nomas_camera_plan_export_ranges(plan.handle, buf.ctypes.data_as(C.c_void_p),
                                                  buf.size), "nomas_camera_plan_export_ranges")
    return buf


def nomas_camera_plan_destroy(plan):
    if plan.handle.value:
        _check(load().nomas_camera_plan_destroy(plan.handle), "nomas_camera_plan_destroy")
        plan.handle = C.c_void_p(0)


def nomas_camera_attn_fwd(plan, q, k_cam, v_cam, o, scale=HEAD_DIM ** -0.5, stream=None):
    h = plan.heads
    qs = _token_stride(q, "q", h)
    os_ = _token_stride(o, "o", h)
    cs = _token_stride(k_cam, "k_cam", h)
    if v_cam is not None and _token_stride(v_cam, "v_cam", h) != cs:
        raise ValueError("k_cam and v_cam must share a token stride")
    _check(load().nomas_camera_attn_fwd(plan.handle, _ptr(q), qs, _ptr(k_cam), _ptr(v_cam), cs,
                                        _ptr(o), os_, float(scale), _stream_ptr(stream, q)),
           "nomas_camera_attn_fwd")


def nomas_status_string(status) -> str:
    return load().nomas_status_string(status).decode()


def nomas_last_error() -> str:
    return load().nomas_last_error().decode()


def nomas_plan_destroy(plan):
    if plan.handle.value:
        _check(load().nomas_plan_destroy(plan.handle), "nomas_plan_destroy")
        plan.handle = C.c_void_p(0)


def nomas_kvcache_destroy(cache):
    if cache.handle.value:
        _check(load().nomas_kvcache_destroy(cache.handle), "nomas_kvcache_destroy")
        cache.handle = C.c_void_p(0)
