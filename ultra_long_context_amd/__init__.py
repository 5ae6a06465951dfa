"""Python binding of the MI355X Hierarchical Sparse Attention (HSA) forward.

Thin ctypes layer over ``libhsa.so`` (C ABI declared in ``include/hsa.h``).  It
only marshals arguments: shapes come from the tensors, device memory and the
HIP stream come from PyTorch, and every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is not built,
every call raises.

The step computed is the HSA forward of "Every Token Counts: Generalizing 16M
Ultra-Long Context in LLMs" (agent-atlas explainer, "How It Works
(Technically)", Steps 1-4).
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = ["HsaError", "HsaShape", "forward", "forward_noalloc", "retrieve_topk", "chunk_attend_blend", "chunk_landmarks",
           "backward", "backward_workspace_size", "workspace_size", "new_workspace", "library_path", "load_library", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhsa.so")
_lib = None
_lock = threading.Lock()

HSA_FLAG_QK_L2NORM = 0x1
DTYPE_F32, DTYPE_BF16 = 0, 1
CHUNK = 64
MAX_TOP_K = 64

EXPORTED_SYMBOLS = ("hsa_workspace_size", "hsa_workspace_init", "hsa_retrieve_topk",
                    "hsa_chunk_attend_blend", "hsa_forward", "hsa_forward_profiled", "hsa_forward_noalloc",
                    "hsa_chunk_landmarks", "hsa_backward_workspace_size", "hsa_backward",
                    "hsa_backward_profiled",
                    "hsa_status_string", "hsa_version")

# kernel stages (hsa_stage_t)
STAGES = ("scan", "merge", "bucket", "attend", "combine")

_STATUS = {0: "HSA_OK", 1: "HSA_ERR_NULL_POINTER", 2: "HSA_ERR_BAD_SHAPE", 3: "HSA_ERR_UNSUPPORTED",
           4: "HSA_ERR_WORKSPACE_TOO_SMALL", 5: "HSA_ERR_DEVICE", 6: "HSA_ERR_MISALIGNED",
           7: "HSA_ERR_SCRATCH_TOO_SMALL"}
STATIC_SCRATCH_BYTES = 16 << 20   # HSA_STATIC_SCRATCH_BYTES (hsa_forward_noalloc)


class HsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _load().hsa_status_string(status).decode() if _lib is not None else ""
        super().__init__("%s failed: %s (%s)" % (where, _STATUS.get(status, status), msg))


class HsaShape(ctypes.Structure):
    """Mirror of hsa_shape_t."""
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int64),
                ("q_pos0", ctypes.c_int64), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ret_scale", ctypes.c_float),
                ("attn_scale", ctypes.c_float), ("flags", ctypes.c_uint32), ("dtype", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libhsa.so (raises if it has not been built)."""
    return _load()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError("HSA HIP library not built: %s is missing "
                                   "(run __graft_entry__.build() or ultra_long_context_amd/build.py)"
                                   % _LIB_PATH)
            lib = ctypes.CDLL(_LIB_PATH)
            vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
            shp = ctypes.POINTER(HsaShape)
            lib.hsa_workspace_size.argtypes = [shp, ctypes.POINTER(sz)]
            lib.hsa_workspace_size.restype = st
            lib.hsa_workspace_init.argtypes = [vp, sz, vp]
            lib.hsa_workspace_init.restype = st
            lib.hsa_retrieve_topk.argtypes = [shp, vp, vp, vp, vp, vp, sz, vp]
            lib.hsa_retrieve_topk.restype = st
            lib.hsa_chunk_attend_blend.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
            lib.hsa_chunk_attend_blend.restype = st
            lib.hsa_forward.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
            lib.hsa_forward.restype = st
            lib.hsa_forward_profiled.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                 ctypes.POINTER(vp)]
            lib.hsa_forward_profiled.restype = st
            lib.hsa_forward_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.hsa_forward_noalloc.restype = st
            lib.hsa_chunk_landmarks.argtypes = [shp, vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
            lib.hsa_chunk_landmarks.restype = st
            lib.hsa_backward_workspace_size.argtypes = [shp, ctypes.POINTER(sz)]
            lib.hsa_backward_workspace_size.restype = st
            lib.hsa_backward.argtypes = [shp] + [vp] * 13 + [vp, sz, vp]
            lib.hsa_backward.restype = st
            lib.hsa_backward_profiled.argtypes = [shp] + [vp] * 13 + [vp, sz, vp, ctypes.POINTER(vp)]
            lib.hsa_backward_profiled.restype = st
            lib.hsa_status_string.argtypes = [st]
            lib.hsa_status_string.restype = ctypes.c_char_p
            lib.hsa_version.restype = ctypes.c_int32
            _lib = lib
    return _lib


def make_shape(*, batch, q_len, kv_len, q_pos0, n_q_heads, n_kv_heads, head_dim, top_k,
               dtype, qk_norm=True, ret_scale=None, attn_scale=None) -> HsaShape:
    return HsaShape(batch=batch, q_len=q_len, kv_len=kv_len, q_pos0=q_pos0, n_q_heads=n_q_heads,
                    n_kv_heads=n_kv_heads, head_dim=head_dim, top_k=top_k,
                    ret_scale=0.0 if ret_scale is None else float(ret_scale),
                    attn_scale=0.0 if attn_scale is None else float(attn_scale),
                    flags=HSA_FLAG_QK_L2NORM if qk_norm else 0, dtype=dtype)


def workspace_size(shape: HsaShape) -> int:
    n = ctypes.c_size_t(0)
    st = _load().hsa_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if st:
        raise HsaError(st, "hsa_workspace_size")
    return int(n.value)


def backward_workspace_size(shape: HsaShape) -> int:
    n = ctypes.c_size_t(0)
    st = _load().hsa_backward_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if st:
        raise HsaError(st, "hsa_backward_workspace_size")
    return int(n.value)


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------
_ws_cache = {}


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError("HSA tensors must be bfloat16 or float32, got %s" % t.dtype)


def _check(t, name, ndim, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %s" % (name, ndim, tuple(t.shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def new_workspace(nbytes: int, device):
    """Allocate a workspace tensor and zero its counter region (hsa_workspace_init)."""
    ws = _torch().empty(max(int(nbytes), 16384), dtype=_torch().uint8, device=device)
    st = _load().hsa_workspace_init(_ptr(ws), ws.numel(), _stream(device))
    if st:
        raise HsaError(st, "hsa_workspace_init")
    return ws


def _cache_key(device):
    """Workspaces are cached per (device, stream): calls on different streams
    may overlap on the GPU, and the library requires each of them to have its
    own workspace (arrival counters and partial buffers)."""
    torch = _torch()
    index = device.index if device.index is not None else torch.cuda.current_device()
    return index, torch.cuda.current_stream(device).cuda_stream


def _workspace(shape, device, workspace=None):
    """The caller's workspace (which must have been initialised once), or a
    cached one per (device, stream), grown as needed.  A replaced workspace
    was only ever used on the same stream, so torch's stream-ordered allocator
    hands its memory out again only after that stream's earlier work."""
    need = workspace_size(shape)
    if workspace is not None:
        return workspace, need
    key = _cache_key(device)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = new_workspace(need, device)
        _ws_cache[key] = ws
    return ws, need


def _after_failure(status, ws, device, where):
    """A call that failed on the device (HSA_ERR_DEVICE) may have left the
    workspace's arrival counters non-zero; they are zeroed again
    (hsa_workspace_init on the same stream) before the error is raised, so the
    next call with this workspace starts clean.  Argument errors launch
    nothing and leave the workspace as it was."""
    if status == 5:
        _load().hsa_workspace_init(_ptr(ws), ws.numel(), _stream(device))
    raise HsaError(status, where)


def _event_handle(ev) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (created on first record)."""
    if ev.cuda_event == 0:
        ev.record()
    return ev.cuda_event


def _stage_array(stage_events):
    evs = (ctypes.c_void_p * (2 * len(STAGES)))()
    for name, (e0, e1) in stage_events.items():
        s = STAGES.index(name)
        evs[2 * s] = _event_handle(e0)
        evs[2 * s + 1] = _event_handle(e1)
    return evs


def forward(q_ret, landmarks, q_attn, k, v, *, q_pos0: int, top_k: int, qk_norm: bool = True,
            ret_scale: float | None = None, attn_scale: float | None = None,
            return_topk: bool = False, out=None, workspace=None, stage_events=None):
    """HSA forward (Steps 1-4).

    q_ret [B, Lq, Hkv, d], landmarks [B, Hkv, Lkv//64, d], q_attn [B, Lq, Hq, d],
    k, v [B, Hkv, Lkv, d]; all bf16 or all fp32, contiguous, on one GPU.
    Returns out [B, Lq, Hq, d] (and topk_idx int32, topk_score fp32
    [B, Lq, Hkv, K] if return_topk).  Runs on the current stream.

    stage_events: optional {stage name: (start, end) torch.cuda.Event} with
    names from STAGES; the library records them around that stage's kernels
    (hsa_forward_profiled).
    """
    torch = _torch()
    for t, n in ((q_ret, "q_ret"), (landmarks, "landmarks"), (q_attn, "q_attn"), (k, "k"), (v, "v")):
        _check(t, n, 4, q_ret.dtype)
    B, Lq, Hkv, d = q_ret.shape
    Hq = q_attn.shape[2]
    Lkv = k.shape[2]
    if (tuple(landmarks.shape) != (B, Hkv, Lkv // CHUNK, d) or tuple(q_attn.shape) != (B, Lq, Hq, d)
            or tuple(k.shape) != (B, Hkv, Lkv, d) or tuple(v.shape) != tuple(k.shape)):
        raise ValueError("inconsistent HSA input shapes")
    shape = make_shape(batch=B, q_len=Lq, kv_len=Lkv, q_pos0=q_pos0, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, top_k=top_k, dtype=_dtype_code(q_ret), qk_norm=qk_norm,
                       ret_scale=ret_scale, attn_scale=attn_scale)
    dev = q_ret.device
    ws, need = _workspace(shape, dev, workspace)
    if out is None:
        out = torch.empty_like(q_attn)
    else:
        _check(out, "out", 4, q_attn.dtype)
    idx = score = None
    if return_topk:
        idx = torch.empty((B, Lq, Hkv, top_k), dtype=torch.int32, device=dev)
        score = torch.empty((B, Lq, Hkv, top_k), dtype=torch.float32, device=dev)
    args = (ctypes.byref(shape), _ptr(q_ret), _ptr(landmarks), _ptr(q_attn), _ptr(k), _ptr(v),
            _ptr(out), _ptr(idx), _ptr(score), _ptr(ws), ws.numel(), _stream(dev))
    if stage_events is None:
        st = _load().hsa_forward(*args)
        if st:
            _after_failure(st, ws, dev, "hsa_forward")
    else:
        st = _load().hsa_forward_profiled(*args, _stage_array(stage_events))
        if st:
            _after_failure(st, ws, dev, "hsa_forward_profiled")
    return (out, idx, score) if return_topk else out


def forward_noalloc(q_ret, landmarks, q_attn, k, v, out, *, q_pos0: int, top_k: int,
                    qk_norm: bool = True, ret_scale: float | None = None,
                    attn_scale: float | None = None, topk=None):
    """hsa_forward_noalloc: the forward with the library's static scratch as its
    workspace (no workspace argument; shapes needing more than
    STATIC_SCRATCH_BYTES raise HSA_ERR_SCRATCH_TOO_SMALL).  `out` (and `topk`,
    an optional (topk_idx, topk_score) pair) are caller-provided, so this
    wrapper allocates nothing either.  Calls that overlap on one GPU race."""
    torch = _torch()
    for t, n in ((q_ret, "q_ret"), (landmarks, "landmarks"), (q_attn, "q_attn"), (k, "k"), (v, "v")):
        _check(t, n, 4, q_ret.dtype)
    _check(out, "out", 4, q_attn.dtype)
    B, Lq, Hkv, d = q_ret.shape
    Hq, Lkv = q_attn.shape[2], k.shape[2]
    if (tuple(landmarks.shape) != (B, Hkv, Lkv // CHUNK, d) or tuple(q_attn.shape) != (B, Lq, Hq, d)
            or tuple(k.shape) != (B, Hkv, Lkv, d) or tuple(v.shape) != tuple(k.shape)
            or out.shape != q_attn.shape):
        raise ValueError("inconsistent HSA input shapes")
    idx = score = None
    if topk is not None:
        idx, score = topk
        _check(idx, "topk_idx", 4, torch.int32)
        _check(score, "topk_score", 4, torch.float32)
        if tuple(idx.shape) != (B, Lq, Hkv, top_k) or score.shape != idx.shape:
            raise ValueError("topk must be (topk_idx, topk_score) of shape [B, Lq, Hkv, K]")
    shape = make_shape(batch=B, q_len=Lq, kv_len=Lkv, q_pos0=q_pos0, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, top_k=top_k, dtype=_dtype_code(q_ret), qk_norm=qk_norm,
                       ret_scale=ret_scale, attn_scale=attn_scale)
    st = _load().hsa_forward_noalloc(ctypes.byref(shape), _ptr(q_ret), _ptr(landmarks), _ptr(q_attn),
                                     _ptr(k), _ptr(v), _ptr(out), _ptr(idx), _ptr(score),
                                     _stream(q_ret.device))
    if st:
        raise HsaError(st, "hsa_forward_noalloc")
    return out


def retrieve_topk(q_ret, landmarks, *, q_pos0: int, top_k: int, kv_len: int | None = None,
                  ret_scale: float | None = None, out=None, workspace=None):
    """Steps 1-2: returns (topk_idx int32, topk_score fp32), each [B, Lq, Hkv, K]."""
    torch = _torch()
    _check(q_ret, "q_ret", 4)
    _check(landmarks, "landmarks", 4, q_ret.dtype)
    B, Lq, Hkv, d = q_ret.shape
    if tuple(landmarks.shape[:2]) != (B, Hkv) or landmarks.shape[3] != d:
        raise ValueError("landmarks must be [B, Hkv, Nc, d]")
    Lkv = landmarks.shape[2] * CHUNK if kv_len is None else int(kv_len)
    if Lkv // CHUNK != landmarks.shape[2]:
        raise ValueError("kv_len // 64 must equal the number of landmarks")
    shape = make_shape(batch=B, q_len=Lq, kv_len=Lkv, q_pos0=q_pos0, n_q_heads=Hkv,
                       n_kv_heads=Hkv, head_dim=d, top_k=top_k, dtype=_dtype_code(q_ret),
                       ret_scale=ret_scale)
    dev = q_ret.device
    ws, _ = _workspace(shape, dev, workspace)
    if out is None:
        idx = torch.empty((B, Lq, Hkv, top_k), dtype=torch.int32, device=dev)
        score = torch.empty((B, Lq, Hkv, top_k), dtype=torch.float32, device=dev)
    else:
        idx, score = out
        _check(idx, "topk_idx", 4, torch.int32)
        _check(score, "topk_score", 4, torch.float32)
        if tuple(idx.shape) != (B, Lq, Hkv, top_k) or score.shape != idx.shape:
            raise ValueError("out must be (topk_idx, topk_score) of shape [B, Lq, Hkv, K]")
    st = _load().hsa_retrieve_topk(ctypes.byref(shape), _ptr(q_ret), _ptr(landmarks), _ptr(idx),
                                   _ptr(score), _ptr(ws), ws.numel(), _stream(dev))
    if st:
        _after_failure(st, ws, dev, "hsa_retrieve_topk")
    return idx, score


def chunk_attend_blend(q_attn, k, v, topk_idx, topk_score, *, qk_norm: bool = True,
                       attn_scale: float | None = None, out=None, workspace=None):
    """Steps 3-4 for a given selection [B, Lq, Hkv, K] (int32 indices, fp32 scores)."""
    torch = _torch()
    _check(q_attn, "q_attn", 4)
    _check(k, "k", 4, q_attn.dtype)
    _check(v, "v", 4, q_attn.dtype)
    _check(topk_idx, "topk_idx", 4, torch.int32)
    _check(topk_score, "topk_score", 4, torch.float32)
    B, Lq, Hq, d = q_attn.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    K = topk_idx.shape[3]
    if tuple(topk_idx.shape) != (B, Lq, Hkv, K) or topk_score.shape != topk_idx.shape:
        raise ValueError("selection must be [B, Lq, Hkv, K]")
    if tuple(k.shape) != (B, Hkv, Lkv, d) or v.shape != k.shape:
        raise ValueError("k, v must be [B, Hkv, Lkv, d]")
    # A given selection is used as is (q_pos0 plays no role here).
    shape = make_shape(batch=B, q_len=Lq, kv_len=Lkv, q_pos0=0, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, top_k=K, dtype=_dtype_code(q_attn), qk_norm=qk_norm,
                       attn_scale=attn_scale)
    dev = q_attn.device
    ws, _ = _workspace(shape, dev, workspace)
    if out is None:
        out = torch.empty_like(q_attn)
    st = _load().hsa_chunk_attend_blend(ctypes.byref(shape), _ptr(q_attn), _ptr(k), _ptr(v),
                                        _ptr(topk_idx), _ptr(topk_score), _ptr(out), _ptr(ws),
                                        ws.numel(), _stream(dev))
    if st:
        _after_failure(st, ws, dev, "hsa_chunk_attend_blend")
    return out


def chunk_landmarks(k, *, chunk_begin: int = 0, chunk_end: int | None = None, out=None):
    """Chunk-mean landmarks of chunks [chunk_begin, chunk_end) (all complete
    chunks by default) for k [B, Hkv, Lkv, d]; writes and returns
    out [B, Hkv, Lkv // 64, d] (allocated if None; chunks outside the range are
    left as they are)."""
    torch = _torch()
    _check(k, "k", 4)
    B, Hkv, Lkv, d = k.shape
    nc = Lkv // CHUNK
    c1 = nc if chunk_end is None else int(chunk_end)
    if out is None:
        out = torch.empty((B, Hkv, nc, d), dtype=k.dtype, device=k.device)
    else:
        _check(out, "out", 4, k.dtype)
        if tuple(out.shape) != (B, Hkv, nc, d):
            raise ValueError("out must be [B, Hkv, Lkv // 64, d]")
    shape = make_shape(batch=B, q_len=1, kv_len=Lkv, q_pos0=0, n_q_heads=Hkv, n_kv_heads=Hkv,
                       head_dim=d, top_k=1, dtype=_dtype_code(k))
    st = _load().hsa_chunk_landmarks(ctypes.byref(shape), _ptr(k), _ptr(out), int(chunk_begin), c1,
                                     _stream(k.device))
    if st:
        raise HsaError(st, "hsa_chunk_landmarks")
    return out


_bwd_ws_cache = {}


def backward(q_ret, landmarks, q_attn, k, v, topk_idx, topk_score, dout, *, qk_norm: bool = True,
             ret_scale: float | None = None, attn_scale: float | None = None, out=None,
             workspace=None, stage_events=None):
    """Gradients of sum(out * dout) for the HSA output computed from the given
    selection (Steps 2-4; the selection itself carries no gradient).

    Inputs as for forward / chunk_attend_blend (bf16), dout [B, Lq, Hq, d] bf16.
    Returns (dq_ret, dlandmarks, dq_attn, dk, dv), fp32, shaped like their
    inputs; `out` may supply them.  workspace: a uint8 GPU tensor of at least
    backward_workspace_size() bytes (cached per device and stream if None).  stage_events:
    as for forward (stages "bucket", "attend", "combine"; hsa_backward_profiled).
    """
    torch = _torch()
    for t, n in ((q_ret, "q_ret"), (landmarks, "landmarks"), (q_attn, "q_attn"), (k, "k"), (v, "v"),
                 (dout, "dout")):
        _check(t, n, 4, torch.bfloat16)
    _check(topk_idx, "topk_idx", 4, torch.int32)
    _check(topk_score, "topk_score", 4, torch.float32)
    B, Lq, Hkv, d = q_ret.shape
    Hq, Lkv, K = q_attn.shape[2], k.shape[2], topk_idx.shape[3]
    if (tuple(landmarks.shape) != (B, Hkv, Lkv // CHUNK, d) or tuple(q_attn.shape) != (B, Lq, Hq, d)
            or tuple(k.shape) != (B, Hkv, Lkv, d) or v.shape != k.shape or dout.shape != q_attn.shape
            or tuple(topk_idx.shape) != (B, Lq, Hkv, K) or topk_score.shape != topk_idx.shape):
        raise ValueError("inconsistent HSA backward shapes")
    shape = make_shape(batch=B, q_len=Lq, kv_len=Lkv, q_pos0=0, n_q_heads=Hq, n_kv_heads=Hkv,
                       head_dim=d, top_k=K, dtype=DTYPE_BF16, qk_norm=qk_norm, ret_scale=ret_scale,
                       attn_scale=attn_scale)
    dev = q_ret.device
    need = backward_workspace_size(shape)
    if workspace is None:
        key = _cache_key(dev)
        workspace = _bwd_ws_cache.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            _bwd_ws_cache[key] = workspace
    if out is None:
        f = dict(dtype=torch.float32, device=dev)
        out = (torch.empty(q_ret.shape, **f), torch.empty(landmarks.shape, **f),
               torch.empty(q_attn.shape, **f), torch.empty(k.shape, **f), torch.empty(v.shape, **f))
    names = ("dq_ret", "dlandmarks", "dq_attn", "dk", "dv")
    for t, n, ref in zip(out, names, (q_ret, landmarks, q_attn, k, v)):
        _check(t, n, 4, torch.float32)
        if t.shape != ref.shape:
            raise ValueError("%s must have shape %s" % (n, tuple(ref.shape)))
    args = (ctypes.byref(shape), _ptr(q_ret), _ptr(landmarks), _ptr(q_attn), _ptr(k), _ptr(v),
            _ptr(topk_idx), _ptr(topk_score), _ptr(dout), *[_ptr(t) for t in out], _ptr(workspace),
            workspace.numel(), _stream(dev))
    if stage_events is None:
        st = _load().hsa_backward(*args)
        if st:
            raise HsaError(st, "hsa_backward")
    else:
        st = _load().hsa_backward_profiled(*args, _stage_array(stage_events))
        if st:
            raise HsaError(st, "hsa_backward_profiled")
    return out
