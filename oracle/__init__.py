"""ctypes wrapper of the fp64 CPU oracle (``oracle/hsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``.  The HIP library never imports, links or
calls anything here, and this package imports nothing from the library.

Arrays are the stored bits of the inputs (``float32``, or ``uint16`` holding
bf16); the C code widens them exactly to fp64.  Shapes (dense, row-major):
  q_ret [B, Lq, Hkv, d], landmarks [B, Hkv, Nc, d], q_attn [B, Lq, Hq, d],
  k, v [B, Hkv, Lkv, d], with Nc = Lkv // 64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hsa_oracle.c")
_LIB = os.path.join(_HERE, "libhsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.hsa_oracle_forward.restype = i32
        lib.hsa_oracle_forward.argtypes = [i64] * 8 + [dbl, dbl, i32, i32] + [vp] * 5 + [vp, i64] + [vp] * 4
        lib.hsa_oracle_attend_blend.restype = i32
        lib.hsa_oracle_attend_blend.argtypes = [i64] * 7 + [dbl, i32, i32] + [vp] * 5 + [vp, i64, vp, vp]
        lib.hsa_oracle_raw_scores.restype = i64
        lib.hsa_oracle_raw_scores.argtypes = [i64] * 6 + [i32, vp, vp, i64, i64, vp]
        lib.hsa_oracle_backward.restype = i32
        lib.hsa_oracle_backward.argtypes = [i64] * 7 + [dbl, dbl, i32, i32] + [vp] * 13
        lib.hsa_oracle_chunk_landmarks.restype = i32
        lib.hsa_oracle_chunk_landmarks.argtypes = [i64] * 4 + [i32, vp, i64, i64, vp]
        lib.hsa_oracle_max_threads.restype = i32
        lib.hsa_oracle_set_threads.argtypes = [i32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _is_bf16(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("oracle inputs must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _rows_arg(rows, B, Lq):
    if rows is None:
        return None, B * Lq
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= B * Lq):
        raise ValueError("row id out of range")
    return r, r.size


def default_scale(d: int) -> float:
    """1/sqrt(d): the scaled-dot-product normaliser of Steps 2 and 3."""
    return 1.0 / math.sqrt(d)


def forward(q_ret, landmarks, q_attn, k, v, *, q_pos0: int, top_k: int, qk_norm: bool = True,
            ret_scale: float | None = None, attn_scale: float | None = None, rows=None,
            with_output: bool = True):
    """Selection and output for the listed flat rows (b*Lq + r); all rows if None.

    Returns (topk_idx int32 [n,Hkv,K], topk_score f64 [n,Hkv,K],
             weights f64 [n,Hkv,K], out f64 [n,Hq,d] or None).
    """
    arrs = [np.ascontiguousarray(a) for a in (q_ret, landmarks, q_attn, k, v)]
    bf = _is_bf16(arrs[0])
    for a in arrs:
        if _is_bf16(a) != bf:
            raise TypeError("mixed input dtypes")
    B, Lq, Hkv, d = arrs[0].shape
    Hq = arrs[2].shape[2]
    Lkv = arrs[3].shape[2]
    if arrs[1].shape != (B, Hkv, Lkv // 64, d):
        raise ValueError("landmarks must be [B, Hkv, Lkv//64, d]")
    rs = default_scale(d) if ret_scale is None else float(ret_scale)
    as_ = default_scale(d) if attn_scale is None else float(attn_scale)
    r_arr, n = _rows_arg(rows, B, Lq)
    idx = np.empty((n, Hkv, top_k), np.int32)
    score = np.empty((n, Hkv, top_k), np.float64)
    w = np.empty((n, Hkv, top_k), np.float64)
    out = np.empty((n, Hq, d), np.float64) if with_output else None
    st = _load().hsa_oracle_forward(
        B, Lq, int(q_pos0), Lkv, Hq, Hkv, d, int(top_k), rs, as_, int(bool(qk_norm)), bf,
        *[_ptr(a) for a in arrs], None if r_arr is None else _ptr(r_arr), n,
        _ptr(idx), _ptr(score), _ptr(w), None if out is None else _ptr(out))
    if st != 0:
        raise RuntimeError("hsa_oracle_forward failed with status %d" % st)
    return idx, score, w, out


def attend_blend(q_attn, k, v, topk_idx, topk_score, *, qk_norm: bool = True,
                 attn_scale: float | None = None, rows=None):
    """Steps 3-4 for a given selection.  topk_idx/topk_score are [n, Hkv, K]
    for the listed rows (all rows if None).  Returns (weights, out)."""
    arrs = [np.ascontiguousarray(a) for a in (q_attn, k, v)]
    bf = _is_bf16(arrs[0])
    B, Lq, Hq, d = arrs[0].shape
    Hkv, Lkv = arrs[1].shape[1], arrs[1].shape[2]
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    sc = np.ascontiguousarray(topk_score, dtype=np.float64)
    K = idx.shape[-1]
    r_arr, n = _rows_arg(rows, B, Lq)
    if idx.shape != (n, Hkv, K) or sc.shape != idx.shape:
        raise ValueError("selection must be [n_rows, Hkv, K]")
    as_ = default_scale(d) if attn_scale is None else float(attn_scale)
    w = np.empty((n, Hkv, K), np.float64)
    out = np.empty((n, Hq, d), np.float64)
    st = _load().hsa_oracle_attend_blend(
        B, Lq, Lkv, Hq, Hkv, d, K, as_, int(bool(qk_norm)), bf, *[_ptr(a) for a in arrs],
        _ptr(idx), _ptr(sc), None if r_arr is None else _ptr(r_arr), n, _ptr(w), _ptr(out))
    if st != 0:
        raise RuntimeError("hsa_oracle_attend_blend failed with status %d" % st)
    return w, out


def raw_scores(q_ret, landmarks, *, q_pos0: int, kv_len: int, flat_row: int, g: int):
    """fp64 raw retrieval scores of every chunk for one (row, kv head); NaN where
    the chunk is not eligible.  Returns (raw [Nc], n_eligible)."""
    q = np.ascontiguousarray(q_ret)
    lm = np.ascontiguousarray(landmarks)
    B, Lq, Hkv, d = q.shape
    nc = kv_len // 64
    raw = np.empty(nc, np.float64)
    n = _load().hsa_oracle_raw_scores(B, Lq, int(q_pos0), int(kv_len), Hkv, d, _is_bf16(q),
                                      _ptr(q), _ptr(lm), int(flat_row), int(g), _ptr(raw))
    if n < 0:
        raise ValueError("bad arguments")
    return raw, int(n)


def backward(q_ret, landmarks, q_attn, k, v, dout, topk_idx, topk_score, *, qk_norm: bool = True,
             ret_scale: float | None = None, attn_scale: float | None = None):
    """Gradients of sum(out * dout) for a given selection topk_idx / topk_score
    [B, Lq, Hkv, K] (scores are the s of Step 4).  All arrays in the stored
    dtype (dout too).  Returns fp64 (dq_ret, dlandmarks, dq_attn, dk, dv)."""
    arrs = [np.ascontiguousarray(a) for a in (q_ret, landmarks, q_attn, k, v, dout)]
    bf = _is_bf16(arrs[0])
    for a in arrs:
        if _is_bf16(a) != bf:
            raise TypeError("mixed input dtypes")
    B, Lq, Hkv, d = arrs[0].shape
    Hq = arrs[2].shape[2]
    Lkv = arrs[3].shape[2]
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    sc = np.ascontiguousarray(topk_score, dtype=np.float64)
    K = idx.shape[-1]
    if idx.shape != (B, Lq, Hkv, K) or sc.shape != idx.shape or arrs[5].shape != arrs[2].shape:
        raise ValueError("selection must be [B, Lq, Hkv, K] and dout like q_attn")
    rs = default_scale(d) if ret_scale is None else float(ret_scale)
    as_ = default_scale(d) if attn_scale is None else float(attn_scale)
    outs = [np.empty(a.shape, np.float64) for a in (arrs[0], arrs[1], arrs[2], arrs[3], arrs[4])]
    st = _load().hsa_oracle_backward(B, Lq, Lkv, Hq, Hkv, d, K, rs, as_, int(bool(qk_norm)), bf,
                                     *[_ptr(a) for a in arrs], _ptr(idx), _ptr(sc),
                                     *[_ptr(o) for o in outs])
    if st != 0:
        raise RuntimeError("hsa_oracle_backward failed with status %d" % st)
    return tuple(outs)


def chunk_landmarks(k, *, chunk_begin: int = 0, chunk_end: int | None = None):
    """fp64 landmarks (chunk means of the keys) of chunks [chunk_begin, chunk_end)
    for k [B, Hkv, Lkv, d].  Returns [B, Hkv, chunk_end - chunk_begin, d]."""
    kk = np.ascontiguousarray(k)
    B, Hkv, Lkv, d = kk.shape
    c1 = Lkv // 64 if chunk_end is None else int(chunk_end)
    out = np.empty((B, Hkv, max(0, c1 - int(chunk_begin)), d), np.float64)
    st = _load().hsa_oracle_chunk_landmarks(B, Hkv, Lkv, d, _is_bf16(kk), _ptr(kk), int(chunk_begin), c1,
                                            _ptr(out))
    if st != 0:
        raise ValueError("hsa_oracle_chunk_landmarks: bad arguments")
    return out


def max_threads() -> int:
    return int(_load().hsa_oracle_max_threads())


def set_threads(n: int) -> None:
    _load().hsa_oracle_set_threads(int(n))
