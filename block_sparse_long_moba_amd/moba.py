"""Thin ctypes binding of libmoba.so (include/moba.h): argument marshalling only.

Every step of the forward pass runs in the HIP library; this module only turns
torch tensors (device memory) and the current HIP stream into the C ABI's
pointers and sizes, and raises on a non-success status. There is no fallback:
if the library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# MOBA_LIBRARY names another build of the same library (e.g. the sanitizer build)
LIB_PATH = os.environ.get("MOBA_LIBRARY") or os.path.join(HERE, "libmoba.so")

DTYPE_FP32, DTYPE_BF16 = 0, 1
STATUS = {0: "MOBA_SUCCESS", 1: "MOBA_ERROR_INVALID_VALUE", 2: "MOBA_ERROR_UNSUPPORTED",
          3: "MOBA_ERROR_WORKSPACE_TOO_SMALL", 4: "MOBA_ERROR_HIP"}

# Every entry point include/moba.h declares.
EXPORTS = ["moba_status_string", "moba_last_error", "moba_workspace_status", "moba_plan",
           "moba_fwd_workspace_size",
           "moba_seqtable", "moba_meanpool", "moba_gate", "moba_minmaxpool", "moba_gate_window",
           "moba_gate_pooled", "moba_dispatch", "moba_attn_fwd", "moba_attn_fwd_diag",
           "moba_attn_fwd_hist", "moba_merge", "moba_attn_prep", "moba_attn_fwd_own_merge",
           "moba_fwd_ex", "moba_fwd_gated",
           "moba_fwd_strided", "moba_fwd", "moba_fwd_noalloc",
           "moba_decode_workspace_size", "moba_decode_prepare", "moba_decode",
           "moba_bwd_plan", "moba_bwd_workspace_size", "moba_bwd", "moba_bwd_delta",
           "moba_attn_bwd_dq", "moba_attn_bwd_dq_sum", "moba_attn_bwd_dkdv",
           "moba_dense_causal_workspace_size", "moba_dense_causal_fwd"]

GATE_MEAN, GATE_WINDOW, GATE_POOLED = 0, 1, 2


class MobaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("total_tokens", ctypes.c_int64), ("num_seqs", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Gate(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("extra_max", ctypes.c_int32), ("extra_min", ctypes.c_int32)]


def gate_mean() -> Gate:
    return Gate(GATE_MEAN, 0, 0, 0)


def gate_window(n_sink=0) -> Gate:
    return Gate(GATE_WINDOW, int(n_sink), 0, 0)


def gate_pooled(extra_max=1, extra_min=1) -> Gate:
    return Gate(GATE_POOLED, 0, int(extra_max), int(extra_min))


class Strides(ctypes.Structure):
    """Element strides (row, head) of q, k, v and out (moba_strides_t)."""
    _fields_ = [(n, ctypes.c_int64) for n in ("q_token", "q_head", "k_token", "k_head",
                                               "v_token", "v_head", "out_token", "out_head")]


class Layout(ctypes.Structure):
    _fields_ = [("num_blocks_bound", ctypes.c_int64), ("padded_tokens", ctypes.c_int64),
                ("kv_heads_per_pass", ctypes.c_int32), ("q_heads_per_pass", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("table_offset", ctypes.c_size_t), ("kbar_offset", ctypes.c_size_t),
                ("vt_offset", ctypes.c_size_t), ("idx_offset", ctypes.c_size_t),
                ("bins_offset", ctypes.c_size_t), ("items_offset", ctypes.c_size_t),
                ("part_o_offset", ctypes.c_size_t), ("part_lse_offset", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """Load libmoba.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError("libmoba.so not built: run __graft_entry__.build() or "
                          "python -m block_sparse_long_moba_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I32, I64, F, Z = (ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int32,
                                ctypes.c_int64, ctypes.c_float, ctypes.c_size_t)
        LP = ctypes.POINTER(Layout)
        sig = {
            "moba_status_string": ([I32], ctypes.c_char_p),
            "moba_last_error": ([], ctypes.c_char_p),
            "moba_workspace_status": ([I32, P, P], I32),
            "moba_plan": ([S, I32, I32, I32, LP], I32),
            "moba_fwd_workspace_size": ([S, I32, I32, I32], Z),
            "moba_seqtable": ([P, S, I32, LP, P, P], I32),
            "moba_meanpool": ([P, S, I32, LP, P, P], I32),
            "moba_gate": ([P, S, I32, I32, LP, P, I32, P], I32),
            "moba_minmaxpool": ([P, S, I32, LP, P, P], I32),
            "moba_gate_window": ([S, I32, I32, I32, LP, P, I32, P], I32),
            "moba_gate_pooled": ([P, S, I32, I32, I32, I32, LP, P, I32, P], I32),
            "moba_dispatch": ([S, I32, I32, LP, P, I32, P], I32),
            "moba_attn_fwd": ([P, P, P, S, I32, I32, F, LP, P, I32, P], I32),
            "moba_attn_fwd_diag": ([P, P, P, S, I32, I32, F, LP, P, I32, P], I32),
            "moba_attn_fwd_hist": ([P, P, S, I32, I32, F, LP, P, I32, P], I32),
            "moba_merge": ([S, I32, I32, LP, P, I32, P, P, P], I32),
            "moba_attn_prep": ([P, P, S, I32, I32, LP, P, I32, P], I32),
            "moba_attn_fwd_own_merge": ([P, P, S, I32, I32, F, LP, P, I32, P, P, P], I32),
            "moba_fwd_ex": ([P, P, P, P, S, I32, I32, F, P, P, P, Z, P], I32),
            "moba_fwd_gated": ([P, P, P, P, S, I32, I32, ctypes.POINTER(Gate), F, P, P, P, Z,
                                P], I32),
            "moba_fwd_strided": ([P, P, P, P, S, ctypes.POINTER(Strides), I32, I32,
                                  ctypes.POINTER(Gate), F, P, P, P, Z, P], I32),
            "moba_fwd": ([P, P, P, P, S, I32, I32, P, P, P], I32),
            "moba_fwd_noalloc": ([P, P, P, P, S, I32, I32, F, P, P, P], I32),
            "moba_decode_workspace_size": ([S, I32, I32], Z),
            "moba_decode_prepare": ([P, P, S, I32, I32, P, Z, P], I32),
            "moba_decode": ([P, P, P, S, I32, I32, F, P, P, P, Z, P], I32),
            "moba_bwd_plan": ([S, I32, I32, I32, LP], I32),
            "moba_bwd_workspace_size": ([S, I32, I32, I32], Z),
            "moba_bwd": ([P, P, P, P, P, P, P, S, I32, I32, ctypes.POINTER(Gate), F, P, P, P, P,
                          Z, P], I32),
            "moba_bwd_delta": ([P, P, S, I32, I32, LP, P, P], I32),
            "moba_attn_bwd_dq": ([P, P, P, P, P, S, I32, I32, F, LP, P, I32, I32, P], I32),
            "moba_attn_bwd_dq_sum": ([S, I32, I32, LP, P, I32, P, P], I32),
            "moba_attn_bwd_dkdv": ([P, P, P, P, P, S, I32, I32, F, LP, P, I32, P, P, P], I32),
            "moba_dense_causal_workspace_size": ([S], Z),
            "moba_dense_causal_fwd": ([P, P, P, P, S, F, P, P, P, Z, P], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise MobaError(status, lib().moba_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(total_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim=128, dtype="bf16",
               max_seqlen=0) -> Shape:
    dt = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}[dtype] if isinstance(dtype, str) else int(dtype)
    return Shape(int(total_tokens), int(num_seqs), int(max_seqlen), int(num_q_heads),
                 int(num_kv_heads), int(head_dim), dt)


def shape_of(q, k, cu_seqlens, max_seqlen=0) -> Shape:
    import torch
    T, Hq, d = q.shape
    dt = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_FP32}[q.dtype]
    return Shape(T, cu_seqlens.numel() - 1, int(max_seqlen), Hq, k.shape[1], d, dt)


def moba_workspace_status(num_seqs, workspace, stream=None):
    """Raises MobaError if the device-side input check of the last call that
    built a block table in `workspace` failed (synchronises the stream)."""
    _check(lib().moba_workspace_status(int(num_seqs), _ptr(workspace), _stream(stream)))


def moba_plan(shape: Shape, block_size: int, topk: int, kv_heads_per_pass: int = 0) -> Layout:
    lay = Layout()
    _check(lib().moba_plan(ctypes.byref(shape), block_size, topk, kv_heads_per_pass,
                           ctypes.byref(lay)))
    return lay


def moba_fwd_workspace_size(shape: Shape, block_size: int, topk: int,
                            kv_heads_per_pass: int = 0) -> int:
    return lib().moba_fwd_workspace_size(ctypes.byref(shape), block_size, topk, kv_heads_per_pass)


def moba_seqtable(cu_seqlens, shape, block_size, layout, workspace, stream=None):
    _check(lib().moba_seqtable(_ptr(cu_seqlens), ctypes.byref(shape), block_size,
                               ctypes.byref(layout), _ptr(workspace), _stream(stream)))


def moba_meanpool(k, shape, block_size, layout, workspace, stream=None):
    _check(lib().moba_meanpool(_ptr(k), ctypes.byref(shape), block_size, ctypes.byref(layout),
                               _ptr(workspace), _stream(stream)))


def moba_gate(q, shape, block_size, topk, layout, workspace, kv_head_begin=0, stream=None):
    _check(lib().moba_gate(_ptr(q), ctypes.byref(shape), block_size, topk, ctypes.byref(layout),
                           _ptr(workspace), kv_head_begin, _stream(stream)))


def moba_minmaxpool(k, shape, block_size, layout, workspace, stream=None):
    _check(lib().moba_minmaxpool(_ptr(k), ctypes.byref(shape), block_size, ctypes.byref(layout),
                                 _ptr(workspace), _stream(stream)))


def moba_gate_window(shape, block_size, topk, n_sink, layout, workspace, kv_head_begin=0,
                     stream=None):
    _check(lib().moba_gate_window(ctypes.byref(shape), block_size, topk, n_sink,
                                  ctypes.byref(layout), _ptr(workspace), kv_head_begin,
                                  _stream(stream)))


def moba_gate_pooled(q, shape, block_size, topk, extra_max, extra_min, layout, workspace,
                     kv_head_begin=0, stream=None):
    _check(lib().moba_gate_pooled(_ptr(q), ctypes.byref(shape), block_size, topk, extra_max,
                                  extra_min, ctypes.byref(layout), _ptr(workspace),
                                  kv_head_begin, _stream(stream)))


def moba_dispatch(shape, block_size, topk, layout, workspace, kv_head_begin=0, stream=None):
    _check(lib().moba_dispatch(ctypes.byref(shape), block_size, topk, ctypes.byref(layout),
                               _ptr(workspace), kv_head_begin, _stream(stream)))


def moba_attn_fwd(q, k, v, shape, block_size, topk, layout, workspace, kv_head_begin=0,
                  softmax_scale=0.0, stream=None):
    _check(lib().moba_attn_fwd(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(shape), block_size, topk,
                               softmax_scale, ctypes.byref(layout), _ptr(workspace),
                               kv_head_begin, _stream(stream)))


def moba_attn_fwd_diag(q, k, v, shape, block_size, topk, layout, workspace, kv_head_begin=0,
                       softmax_scale=0.0, stream=None):
    _check(lib().moba_attn_fwd_diag(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(shape), block_size,
                                    topk, softmax_scale, ctypes.byref(layout), _ptr(workspace),
                                    kv_head_begin, _stream(stream)))


def moba_attn_fwd_hist(q, k, shape, block_size, topk, layout, workspace, kv_head_begin=0,
                       softmax_scale=0.0, stream=None):
    _check(lib().moba_attn_fwd_hist(_ptr(q), _ptr(k), ctypes.byref(shape), block_size, topk,
                                    softmax_scale, ctypes.byref(layout), _ptr(workspace),
                                    kv_head_begin, _stream(stream)))


def moba_merge(shape, block_size, topk, layout, workspace, out, lse=None, kv_head_begin=0,
               stream=None):
    _check(lib().moba_merge(ctypes.byref(shape), block_size, topk, ctypes.byref(layout),
                            _ptr(workspace), kv_head_begin, _ptr(out), _ptr(lse),
                            _stream(stream)))


def moba_attn_prep(k, v, shape, block_size, topk, layout, workspace, kv_head_begin=0,
                   stream=None):
    _check(lib().moba_attn_prep(_ptr(k), _ptr(v), ctypes.byref(shape), block_size, topk,
                                ctypes.byref(layout), _ptr(workspace), kv_head_begin,
                                _stream(stream)))


def moba_attn_fwd_own_merge(q, k, shape, block_size, topk, layout, workspace, out, lse=None,
                            kv_head_begin=0, softmax_scale=0.0, stream=None):
    _check(lib().moba_attn_fwd_own_merge(_ptr(q), _ptr(k), ctypes.byref(shape), block_size, topk,
                                         softmax_scale, ctypes.byref(layout), _ptr(workspace),
                                         kv_head_begin, _ptr(out), _ptr(lse), _stream(stream)))


def _contiguous(**tensors):
    """The entry points without strides read [T][H][d] tensors packed row by row."""
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous (moba_fwd_strided takes strided tensors)"
                             % name)


def strides_of(q, k, v, out) -> Strides:
    """Strides of [T][H][d] tensors whose last dimension is contiguous."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("%s: a [T][H][d] tensor with contiguous d is required" % name)
    return Strides(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                   out.stride(0), out.stride(1))


def _outputs(q, out, lse, want_lse=True):
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    return out, lse


def moba_fwd(q, k, v, cu_seqlens, block_size, topk, out=None, lse=None, max_seqlen=0,
             stream=None):
    """MoBA forward pass; returns (out [T][Hq][d], lse [Hq][T])."""
    _contiguous(q=q, k=k, v=v, out=out)
    out, lse = _outputs(q, out, lse)
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    _check(lib().moba_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), ctypes.byref(sh),
                          block_size, topk, _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


NOALLOC_WORKSPACE_BYTES = 256 << 20  # MOBA_NOALLOC_WORKSPACE_BYTES of include/moba.h


def moba_fwd_noalloc(q, k, v, cu_seqlens, block_size, topk, out=None, lse=None,
                     softmax_scale=0.0, max_seqlen=0, stream=None):
    """MoBA forward pass on the library's static workspace (no allocation in
    the library; out and lse are allocated here only when not given)."""
    _contiguous(q=q, k=k, v=v, out=out)
    out, lse = _outputs(q, out, lse)
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    _check(lib().moba_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), ctypes.byref(sh),
                                  block_size, topk, softmax_scale, _ptr(out), _ptr(lse),
                                  _stream(stream)))
    return out, lse


def moba_fwd_ex(q, k, v, cu_seqlens, block_size, topk, workspace, out=None, lse=None,
                softmax_scale=0.0, max_seqlen=0, stream=None):
    """MoBA forward pass with a caller-provided workspace (uint8 device tensor)."""
    _contiguous(q=q, k=k, v=v, out=out)
    out, lse = _outputs(q, out, lse)
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    _check(lib().moba_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), ctypes.byref(sh),
                             block_size, topk, softmax_scale, _ptr(out), _ptr(lse),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)))
    return out, lse


def moba_fwd_gated(q, k, v, cu_seqlens, block_size, topk, gate, workspace, out=None, lse=None,
                   softmax_scale=0.0, max_seqlen=0, stream=None):
    """Forward pass with a gate variant (Gate) and a caller-provided workspace."""
    _contiguous(q=q, k=k, v=v, out=out)
    out, lse = _outputs(q, out, lse)
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    _check(lib().moba_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), ctypes.byref(sh),
                                block_size, topk, ctypes.byref(gate), softmax_scale, _ptr(out),
                                _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def moba_fwd_strided(q, k, v, cu_seqlens, block_size, topk, workspace, gate=None, out=None,
                     lse=None, softmax_scale=0.0, max_seqlen=0, stream=None):
    """Forward pass over [T][H][d] tensors with any row and head strides (the
    last dimension contiguous), e.g. views of one fused qkv tensor; gate None
    is the mean gate. Returns (out, lse); a given out keeps its strides."""
    out, lse = _outputs(q, out, lse)
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    st = strides_of(q, k, v, out)
    _check(lib().moba_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), ctypes.byref(sh),
                                  ctypes.byref(st), block_size, topk,
                                  None if gate is None else ctypes.byref(gate), softmax_scale,
                                  _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def moba_decode_workspace_size(cache_shape: Shape, block_size: int, topk: int) -> int:
    return lib().moba_decode_workspace_size(ctypes.byref(cache_shape), block_size, topk)


def moba_decode_prepare(k_cache, cu_seqlens, cache_shape, block_size, topk, workspace,
                        stream=None):
    _check(lib().moba_decode_prepare(_ptr(k_cache), _ptr(cu_seqlens), ctypes.byref(cache_shape),
                                     block_size, topk, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def moba_decode(q, k_cache, v_cache, cache_shape, block_size, topk, workspace, out=None,
                lse=None, softmax_scale=0.0, stream=None):
    """One query per sequence (q [S][Hq][d]) over the cache; returns (out, lse [Hq][S])."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    _check(lib().moba_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(cache_shape),
                             block_size, topk, softmax_scale, _ptr(out), _ptr(lse),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)))
    return out, lse


def moba_bwd_plan(shape: Shape, block_size: int, topk: int, kv_heads_per_pass: int = 0) -> Layout:
    lay = Layout()
    _check(lib().moba_bwd_plan(ctypes.byref(shape), block_size, topk, kv_heads_per_pass,
                               ctypes.byref(lay)))
    return lay


def moba_bwd_workspace_size(shape: Shape, block_size: int, topk: int,
                            kv_heads_per_pass: int = 0) -> int:
    return lib().moba_bwd_workspace_size(ctypes.byref(shape), block_size, topk, kv_heads_per_pass)


def moba_bwd(q, k, v, out, lse, dout, cu_seqlens, block_size, topk, workspace, gate=None,
             dq=None, dk=None, dv=None, softmax_scale=0.0, max_seqlen=0, stream=None):
    """Gradients (dq, dk, dv) of the forward pass that wrote out and lse."""
    import torch
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    _check(lib().moba_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                          _ptr(cu_seqlens), ctypes.byref(sh), block_size, topk,
                          None if gate is None else ctypes.byref(gate), softmax_scale, _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def moba_bwd_delta(out, dout, shape, block_size, topk, layout, workspace, stream=None):
    _check(lib().moba_bwd_delta(_ptr(out), _ptr(dout), ctypes.byref(shape), block_size, topk,
                                ctypes.byref(layout), _ptr(workspace), _stream(stream)))


def moba_attn_bwd_dq(q, k, v, dout, lse, shape, block_size, topk, layout, workspace,
                     kv_head_begin=0, which=3, softmax_scale=0.0, stream=None):
    _check(lib().moba_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                  ctypes.byref(shape), block_size, topk, softmax_scale,
                                  ctypes.byref(layout), _ptr(workspace), kv_head_begin, which,
                                  _stream(stream)))


def moba_attn_bwd_dq_sum(shape, block_size, topk, layout, workspace, dq, kv_head_begin=0,
                         stream=None):
    _check(lib().moba_attn_bwd_dq_sum(ctypes.byref(shape), block_size, topk,
                                      ctypes.byref(layout), _ptr(workspace), kv_head_begin,
                                      _ptr(dq), _stream(stream)))


def moba_attn_bwd_dkdv(q, k, v, dout, lse, shape, block_size, topk, layout, workspace, dk, dv,
                       kv_head_begin=0, softmax_scale=0.0, stream=None):
    _check(lib().moba_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                    ctypes.byref(shape), block_size, topk, softmax_scale,
                                    ctypes.byref(layout), _ptr(workspace), kv_head_begin,
                                    _ptr(dk), _ptr(dv), _stream(stream)))


def moba_dense_causal_workspace_size(shape: Shape) -> int:
    return lib().moba_dense_causal_workspace_size(ctypes.byref(shape))


def moba_dense_causal_fwd(q, k, v, cu_seqlens, out=None, lse=None, softmax_scale=0.0,
                          workspace=None, max_seqlen=0, stream=None):
    """Dense causal attention per sequence; returns (out, lse)."""
    out, lse = _outputs(q, out, lse)
    sh = shape_of(q, k, cu_seqlens, max_seqlen)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moba_dense_causal_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                       ctypes.byref(sh), softmax_scale, _ptr(out), _ptr(lse),
                                       _ptr(workspace), nbytes, _stream(stream)))
    return out, lse


def _autograd_function():
    """torch.autograd.Function over moba_fwd_gated and moba_bwd (built on first
    use so that importing this module does not import torch)."""
    import torch

    class MobaAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, cu_seqlens, block_size, topk, gate, softmax_scale, max_seqlen):
            gate = gate_mean() if gate is None else gate
            sh = shape_of(q, k, cu_seqlens, max_seqlen)
            # the largest pass (a divisor of Hkv) whose workspace fits the limit
            P = sh.num_kv_heads
            limit = int(float(os.environ.get("MOBA_WORKSPACE_LIMIT_GIB", "48")) * (1 << 30))
            while P > 1 and moba_fwd_workspace_size(sh, block_size, topk, P) > limit:
                P -= 1
            ws = torch.empty(moba_fwd_workspace_size(sh, block_size, topk, P), dtype=torch.uint8,
                             device=q.device)
            out, lse = moba_fwd_gated(q, k, v, cu_seqlens, block_size, topk, gate, ws,
                                      softmax_scale=softmax_scale, max_seqlen=max_seqlen)
            ctx.save_for_backward(q, k, v, cu_seqlens, out, lse)
            ctx.args = (block_size, topk, gate, softmax_scale, max_seqlen)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, cu_seqlens, out, lse = ctx.saved_tensors
            block_size, topk, gate, softmax_scale, max_seqlen = ctx.args
            sh = shape_of(q, k, cu_seqlens, max_seqlen)
            limit = int(float(os.environ.get("MOBA_WORKSPACE_LIMIT_GIB", "48")) * (1 << 30))
            P = sh.num_kv_heads
            while P > 1 and moba_bwd_workspace_size(sh, block_size, topk, P) > limit:
                P -= 1
            ws = torch.empty(moba_bwd_workspace_size(sh, block_size, topk, P), dtype=torch.uint8,
                             device=q.device)
            dq, dk, dv = moba_bwd(q, k, v, out, lse, dout.contiguous(), cu_seqlens, block_size,
                                  topk, ws, gate=gate, softmax_scale=softmax_scale,
                                  max_seqlen=max_seqlen)
            return dq, dk, dv, None, None, None, None, None, None

    return MobaAttention


_MobaAttention = None


def moba_attention(q, k, v, cu_seqlens, block_size, topk, gate=None, softmax_scale=0.0,
                   max_seqlen=0):
    """Differentiable MoBA attention (bf16 for gradients): out = moba_fwd_gated(...),
    and autograd calls moba_bwd for dq, dk, dv. The workspaces are allocated
    per call (a pass size that fits MOBA_WORKSPACE_LIMIT_GIB, default 48)."""
    global _MobaAttention
    if _MobaAttention is None:
        _MobaAttention = _autograd_function()
    return _MobaAttention.apply(q, k, v, cu_seqlens, block_size, topk, gate, softmax_scale,
                                max_seqlen)
