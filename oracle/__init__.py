"""fp64 CPU oracle of the MoBA forward pass (ctypes wrapper of moba_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with the
GPU path (the HIP library under block_sparse_long_moba_amd/csrc) and is never a
fallback for it.

All functions take host numpy arrays in the packed variable-length layout
q[T][Hq][d], k/v[T][Hkv][d] (float32, or uint16 holding bf16 bit patterns) and
cu_seqlens[S+1] (int32). Results are float64. The arithmetic and the readings of
the pages it follows are documented in moba_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moba_oracle.c")
# MOBA_ORACLE_LIBRARY names a prebuilt copy (the sanitizer build); it is loaded as is
_PREBUILT = os.environ.get("MOBA_ORACLE_LIBRARY")
_LIB = _PREBUILT or os.path.join(_HERE, "libmoba_oracle.so")
_lib = None

SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                  "-fno-sanitize-recover=undefined"]


def build_sanitized(out_dir: str) -> str:
    """The oracle with AddressSanitizer and UndefinedBehaviorSanitizer (clang,
    the runtime the sanitized HIP library uses), into out_dir."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libmoba_oracle.so")
    subprocess.check_call(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp",
                           "-fPIC", "-shared", "-Wall", "-Wextra"] + SANITIZE_FLAGS +
                          ["-o", lib, _SRC, "-lm"])
    return lib


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if _PREBUILT:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        p, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_block_first.argtypes = [p, i32, i32, p]
        lib.oracle_block_first.restype = i64
        lib.oracle_meanpool.argtypes = [p, i32, i64, i32, i32, p, i32, i32, p]
        lib.oracle_select.argtypes = [p, i32, p, i64, i32, i32, i32, p, i32, i32, i32,
                                      p, i64, p, p, p, i32]
        lib.oracle_attend.argtypes = [p, p, p, i32, i64, i32, i32, i32, p, i32, i32, i32,
                                      p, p, i64, dbl, p, p]
        lib.oracle_moba.argtypes = [p, p, p, i32, i64, i32, i32, i32, p, i32, i32, i32, dbl,
                                    p, i64, p, p, p, p]
        lib.oracle_select_window.argtypes = [p, i32, i32, i64, i32, i32, i32, p, i64, p]
        lib.oracle_minmaxpool.argtypes = [p, i32, i64, i32, i32, p, i32, i32, p, p]
        lib.oracle_select_pooled.argtypes = [p, i32, p, p, p, i64, i32, i32, i32, p, i32, i32,
                                             i32, i32, i32, p, i64, p, p]
        lib.oracle_attend_bwd.argtypes = [p, p, p, p, i32, i64, i32, i32, i32, p, i32, i32, i32,
                                          p, dbl, p, p, p]
        lib.oracle_attend_bwd_dq_rows.argtypes = [p, p, p, p, i32, i64, i32, i32, i32, p, i32,
                                                  i32, i32, p, p, i64, dbl, p]
        lib.oracle_dense_causal.argtypes = [p, p, p, i32, i64, i32, i32, i32, p, i32, p, i64,
                                            dbl, p, p]
        for f in (lib.oracle_meanpool, lib.oracle_select, lib.oracle_attend, lib.oracle_moba,
                  lib.oracle_dense_causal):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_inputs(*arrs):
    dt = None
    for a in arrs:
        assert a.flags.c_contiguous, "oracle inputs must be C-contiguous"
        assert a.dtype in (np.float32, np.uint16), "fp32 or bf16 bit patterns"
        dt = a.dtype if dt is None else dt
        assert a.dtype == dt, "q, k, v must share one dtype"
    return int(dt == np.uint16)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.size


def _cu(cu_seqlens):
    return np.ascontiguousarray(cu_seqlens, dtype=np.int32)


def block_first(cu_seqlens, block_size):
    """first[s] = global index of sequence s's first block; first[S] = total."""
    cu = _cu(cu_seqlens)
    S = cu.size - 1
    first = np.zeros(S + 1, dtype=np.int64)
    _load().oracle_block_first(_ptr(cu), S, block_size, _ptr(first))
    return first


def meanpool(k, cu_seqlens, block_size):
    """K-bar[total_blocks][Hkv][d] (float64)."""
    bf = _check_inputs(k)
    cu = _cu(cu_seqlens)
    T, Hkv, d = k.shape
    nb = int(block_first(cu, block_size)[-1])
    kbar = np.zeros((max(nb, 1), Hkv, d), dtype=np.float64)
    _load().oracle_meanpool(_ptr(k), bf, T, Hkv, d, _ptr(cu), cu.size - 1, block_size, _ptr(kbar))
    return kbar[:nb]


def select(q, kbar, cu_seqlens, block_size, topk, rows=None, want_scores=False):
    """Block selection. Returns (sel[n][Hq][topk] int32, near_tie[n][Hq] bool,
    scores[n][Hq][max_blocks] or None)."""
    bf = _check_inputs(q)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = kbar.shape[1]
    kb = np.ascontiguousarray(kbar, dtype=np.float64)
    r, n = _rows(rows)
    n = T if r is None else n
    sel = np.zeros((n, Hq, topk), dtype=np.int32)
    tie = np.zeros((n, Hq), dtype=np.uint8)
    max_blocks = int(max(1, np.max((np.diff(cu) + block_size - 1) // block_size, initial=1)))
    scores = np.zeros((n, Hq, max_blocks), dtype=np.float64) if want_scores else None
    _load().oracle_select(_ptr(q), bf, _ptr(kb), T, Hq, Hkv, d, _ptr(cu), cu.size - 1,
                          block_size, topk, _ptr(r), n, _ptr(sel), _ptr(tie), _ptr(scores),
                          max_blocks)
    return sel, tie.astype(bool), scores


def select_window(cu_seqlens, block_size, topk, n_sink, num_q_heads, rows=None, total_tokens=None):
    """Fixed gate (sliding window, optionally with n_sink initial blocks):
    sel[n][Hq][topk] int32."""
    cu = _cu(cu_seqlens)
    T = int(cu[-1]) if total_tokens is None else int(total_tokens)
    r, n = _rows(rows)
    n = T if r is None else n
    assert 0 <= n_sink < topk
    sel = np.zeros((n, num_q_heads, topk), dtype=np.int32)
    _load().oracle_select_window(_ptr(cu), cu.size - 1, block_size, T, num_q_heads, topk, n_sink,
                                 _ptr(r), n, _ptr(sel))
    return sel


def minmaxpool(k, cu_seqlens, block_size):
    """(K-max, K-min)[total_blocks][Hkv][d] (float64): elementwise max / min
    over each block's rows."""
    bf = _check_inputs(k)
    cu = _cu(cu_seqlens)
    T, Hkv, d = k.shape
    nb = int(block_first(cu, block_size)[-1])
    kmax = np.zeros((max(nb, 1), Hkv, d), dtype=np.float64)
    kmin = np.zeros((max(nb, 1), Hkv, d), dtype=np.float64)
    _load().oracle_minmaxpool(_ptr(k), bf, T, Hkv, d, _ptr(cu), cu.size - 1, block_size,
                              _ptr(kmax), _ptr(kmin))
    return kmax[:nb], kmin[:nb]


def select_pooled(q, kbar, kmax, kmin, cu_seqlens, block_size, topk, extra_max, extra_min,
                  rows=None):
    """Gate with extra blocks from max- and min-pooled keys:
    (sel[n][Hq][topk] int32, near_tie[n][Hq] bool)."""
    bf = _check_inputs(q)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = kbar.shape[1]
    assert topk - extra_max - extra_min >= 1 and extra_max >= 0 and extra_min >= 0
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (kbar, kmax, kmin)]
    r, n = _rows(rows)
    n = T if r is None else n
    sel = np.zeros((n, Hq, topk), dtype=np.int32)
    tie = np.zeros((n, Hq), dtype=np.uint8)
    _load().oracle_select_pooled(_ptr(q), bf, _ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]), T, Hq,
                                 Hkv, d, _ptr(cu), cu.size - 1, block_size, topk, extra_max,
                                 extra_min, _ptr(r), n, _ptr(sel), _ptr(tie))
    return sel, tie.astype(bool)


def attend(q, k, v, cu_seqlens, block_size, topk, sel, scale=None, rows=None):
    """Attention over the union of the selected blocks: (out[n][Hq][d], lse[n][Hq])."""
    bf = _check_inputs(q, k, v)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, n = _rows(rows)
    n = T if r is None else n
    s = np.ascontiguousarray(sel, dtype=np.int32)
    assert s.shape == (n, Hq, topk)
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    _load().oracle_attend(_ptr(q), _ptr(k), _ptr(v), bf, T, Hq, Hkv, d, _ptr(cu), cu.size - 1,
                          block_size, topk, _ptr(s), _ptr(r), n, scale, _ptr(out), _ptr(lse))
    return out, lse


def attend_bwd(q, k, v, dout, cu_seqlens, block_size, topk, sel, scale=None):
    """Gradients of the attention over a selection, all rows:
    (dq[T][Hq][d], dk[T][Hkv][d], dv[T][Hkv][d]) in float64."""
    bf = _check_inputs(q, k, v)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    s = np.ascontiguousarray(sel, dtype=np.int32)
    assert s.shape == (T, Hq, topk)
    go = np.ascontiguousarray(dout, dtype=np.float64)
    assert go.shape == (T, Hq, d)
    dq = np.zeros((T, Hq, d))
    dk = np.zeros((T, Hkv, d))
    dv = np.zeros((T, Hkv, d))
    _load().oracle_attend_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(go), bf, T, Hq, Hkv, d, _ptr(cu),
                              cu.size - 1, block_size, topk, _ptr(s), scale, _ptr(dq), _ptr(dk),
                              _ptr(dv))
    return dq, dk, dv


def attend_bwd_dq_rows(q, k, v, dout_rows, cu_seqlens, block_size, topk, sel_rows, rows,
                       scale=None):
    """dq of the listed rows only (all heads), float64 [n][Hq][d]; dout_rows and
    sel_rows hold those rows."""
    bf = _check_inputs(q, k, v)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    n = r.size
    s = np.ascontiguousarray(sel_rows, dtype=np.int32)
    assert s.shape == (n, Hq, topk)
    go = np.ascontiguousarray(dout_rows, dtype=np.float64)
    assert go.shape == (n, Hq, d)
    dq = np.zeros((n, Hq, d))
    _load().oracle_attend_bwd_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(go), bf, T, Hq, Hkv, d,
                                      _ptr(cu), cu.size - 1, block_size, topk, _ptr(s), _ptr(r), n,
                                      scale, _ptr(dq))
    return dq


def moba(q, k, v, cu_seqlens, block_size, topk, scale=None, rows=None):
    """Whole forward pass: (out[n][Hq][d], lse[n][Hq], sel[n][Hq][topk], near_tie[n][Hq])."""
    bf = _check_inputs(q, k, v)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, n = _rows(rows)
    n = T if r is None else n
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    sel = np.zeros((n, Hq, topk), dtype=np.int32)
    tie = np.zeros((n, Hq), dtype=np.uint8)
    _load().oracle_moba(_ptr(q), _ptr(k), _ptr(v), bf, T, Hq, Hkv, d, _ptr(cu), cu.size - 1,
                        block_size, topk, scale, _ptr(r), n, _ptr(out), _ptr(lse), _ptr(sel),
                        _ptr(tie))
    return out, lse, sel, tie.astype(bool)


def dense_causal(q, k, v, cu_seqlens, scale=None, rows=None):
    """Dense causal attention per sequence: (out[n][Hq][d], lse[n][Hq])."""
    bf = _check_inputs(q, k, v)
    cu = _cu(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    r, n = _rows(rows)
    n = T if r is None else n
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    _load().oracle_dense_causal(_ptr(q), _ptr(k), _ptr(v), bf, T, Hq, Hkv, d, _ptr(cu),
                                cu.size - 1, _ptr(r), n, scale, _ptr(out), _ptr(lse))
    return out, lse
