"""Attention with per-head learnable sinks for MI355X (gfx950): Python binding.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn_sink.so`` (built from ``csrc/`` by ``build.py``), reached
through the C ABI of ``include/attn_sink.h``.  PyTorch provides device memory
and the current HIP stream.  There is no fallback: if the shared library is
missing, ``load()`` raises.

The operation (sink softmax of "Unlocking Agentic RL Training for GPT-OSS",
euno.news, sub-sections 带汇聚的注意力 / 数学公式 / 反向传播):
    o_i   = sum_j P_ij v_j,  P_ij = exp(s_ij) / (sum_j' exp(s_ij') + exp(S_h))
    lse_i = log(sum_j exp(s_ij) + exp(S_h))
    dS_h  = -sum_i P_sink_i <dO_i, o_i>
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["load", "fwd", "fwd_decode", "fwd_decode_workspace_bytes", "merge", "bwd", "bwd_workspace_bytes",
           "Shape", "AttnSinkError", "sink_attention", "timing_enable", "timing_read", "LIB_PATH"]

# ATTN_SINK_LIBRARY may point at another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("ATTN_SINK_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libattn_sink.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1


class Shape(ctypes.Structure):
    """Mirror of attn_sink_shape."""
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("num_heads_q", ctypes.c_int),
        ("num_heads_kv", ctypes.c_int),
        ("num_seqs", ctypes.c_int),
        ("total_q", ctypes.c_int),
        ("total_k", ctypes.c_int),
        ("max_seqlen_q", ctypes.c_int),
        ("max_seqlen_k", ctypes.c_int),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int),
        ("window", ctypes.c_int),
    ]


class AttnSinkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib().attn_sink_status_string(status).decode()} (status {status})")


_LIB = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the shared library (raises if it is not built) and declare its symbols."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m attention_learnable_sinks_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sp, st = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int
    lib.attn_sink_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_sink_fwd.restype = st
    lib.attn_sink_fwd_decode.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_sink_fwd_decode.restype = st
    lib.attn_sink_fwd_decode_workspace_bytes.argtypes = [sp]
    lib.attn_sink_fwd_decode_workspace_bytes.restype = ctypes.c_size_t
    ci = ctypes.c_int
    lib.attn_sink_merge.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp]
    lib.attn_sink_merge.restype = st
    lib.attn_sink_bwd_workspace_bytes.argtypes = [sp]
    lib.attn_sink_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_sink_bwd.argtypes = [sp] + [vp] * 12 + [ctypes.c_size_t, vp]
    lib.attn_sink_bwd.restype = st
    lib.attn_sink_status_string.argtypes = [st]
    lib.attn_sink_status_string.restype = ctypes.c_char_p
    lib.attn_sink_timing_enable.argtypes = [ctypes.c_int]
    lib.attn_sink_timing_enable.restype = st
    lib.attn_sink_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.attn_sink_timing_read.restype = ctypes.c_int
    if path is None:
        _LIB = lib
    return lib


def _lib():
    return load()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def make_shape(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
               max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float, causal: bool, window: int) -> Shape:
    if q.dtype == torch.bfloat16:
        dt = BF16
    elif q.dtype == torch.float32:
        dt = FP32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return Shape(dtype=dt, head_dim=q.shape[2], num_heads_q=q.shape[1], num_heads_kv=k.shape[1],
                 num_seqs=cu_seqlens_q.numel() - 1, total_q=q.shape[0], total_k=k.shape[0],
                 max_seqlen_q=int(max_seqlen_q), max_seqlen_k=int(max_seqlen_k),
                 cu_seqlens_q=cu_seqlens_q.data_ptr(), cu_seqlens_k=cu_seqlens_k.data_ptr(),
                 softmax_scale=float(softmax_scale), causal=int(bool(causal)), window=int(window))


def _check_tensors(q, k, v, sinks, cu_q, cu_k):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 3-d device tensor [T, H, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype or v.shape != k.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q, k, v must share dtype and head dim; k and v must match")
    if sinks.dtype != torch.float32 or sinks.numel() != q.shape[1] or not sinks.is_cuda or not sinks.is_contiguous():
        raise ValueError("sinks must be a contiguous float32 device tensor [Hq]")
    for name, cu in (("cu_seqlens_q", cu_q), ("cu_seqlens_k", cu_k)):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_cuda or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor [num_seqs + 1]")


def fwd(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
        softmax_scale=None, causal=True, window=0, out=None, lse=None):
    """Forward.  q [Tq, Hq, 64], k/v [Tk, Hkv, 64] (bf16 or fp32), sinks [Hq] fp32,
    cu_seqlens int32 on the device.  Returns (o [Tq, Hq, 64], lse [Hq, Tq] fp32)."""
    cu_seqlens_k = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
    _check_tensors(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k)
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if cu_seqlens_q.numel() > 1 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if cu_seqlens_k.numel() > 1 else 0
    if softmax_scale is None:
        softmax_scale = q.shape[2] ** -0.5
    shape = make_shape(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal, window)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device) if lse is None else lse
    st = _lib().attn_sink_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o), _ptr(lse),
                              _stream(q.device))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_fwd")
    return o, lse


def fwd_decode_workspace_bytes(shape: Shape) -> int:
    return int(_lib().attn_sink_fwd_decode_workspace_bytes(ctypes.byref(shape)))


def fwd_decode(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, max_seqlen_k=None,
               softmax_scale=None, causal=True, window=0, workspace=None, out=None, lse=None):
    """Forward for a few new rows per sequence against a long key range (decoding
    step or short chunk against a KV cache), split over keys.  Same arguments and
    results as fwd(); needs (Hq / Hkv) * max_seqlen_q <= 32.  `workspace` (uint8
    device tensor of at least fwd_decode_workspace_bytes bytes) is allocated here
    when not given."""
    _check_tensors(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k)
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if cu_seqlens_q.numel() > 1 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if cu_seqlens_k.numel() > 1 else 0
    if softmax_scale is None:
        softmax_scale = q.shape[2] ** -0.5
    shape = make_shape(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal, window)
    if workspace is None:
        workspace = torch.empty(max(fwd_decode_workspace_bytes(shape), 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device) if lse is None else lse
    st = _lib().attn_sink_fwd_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o),
                                     _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(q.device))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_fwd_decode")
    return o, lse


def merge(o_parts, lse_parts, sinks, out=None, lse=None):
    """Merge per-shard attention partials (each from fwd() with sinks = -inf over one
    key shard) into sink attention, the sink counted once.  o_parts [P, Tq, Hq, 64]
    (bf16 or fp32), lse_parts [P, Hq, Tq] fp32, sinks [Hq] fp32, all contiguous on the
    device.  Returns (o [Tq, Hq, 64], lse [Hq, Tq])."""
    if o_parts.dim() != 4 or not o_parts.is_contiguous() or not o_parts.is_cuda:
        raise ValueError("o_parts must be a contiguous 4-d device tensor [P, Tq, Hq, d]")
    p, tq, hq, d = o_parts.shape
    if lse_parts.shape != (p, hq, tq) or lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be a contiguous float32 tensor [P, Hq, Tq]")
    if sinks.dtype != torch.float32 or sinks.numel() != hq or not sinks.is_contiguous():
        raise ValueError("sinks must be a contiguous float32 tensor [Hq]")
    if o_parts.dtype == torch.bfloat16:
        dt = BF16
    elif o_parts.dtype == torch.float32:
        dt = FP32
    else:
        raise TypeError(f"unsupported dtype {o_parts.dtype}")
    o = torch.empty(tq, hq, d, dtype=o_parts.dtype, device=o_parts.device) if out is None else out
    lse = torch.empty(hq, tq, dtype=torch.float32, device=o_parts.device) if lse is None else lse
    st = _lib().attn_sink_merge(dt, d, hq, tq, p, _ptr(o_parts), _ptr(lse_parts), _ptr(sinks), _ptr(o), _ptr(lse),
                                _stream(o_parts.device))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_merge")
    return o, lse


def bwd_workspace_bytes(shape: Shape) -> int:
    return int(_lib().attn_sink_bwd_workspace_bytes(ctypes.byref(shape)))


def bwd(q, k, v, sinks, o, lse, dout, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
        softmax_scale=None, causal=True, window=0, workspace=None, dq=None, dk=None, dv=None, dsinks=None):
    """Backward.  Returns (dq, dk, dv, dsinks).  `workspace` (uint8 device tensor of at
    least bwd_workspace_bytes bytes) is allocated here when not given."""
    cu_seqlens_k = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
    _check_tensors(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k)
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if cu_seqlens_q.numel() > 1 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if cu_seqlens_k.numel() > 1 else 0
    if softmax_scale is None:
        softmax_scale = q.shape[2] ** -0.5
    shape = make_shape(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal, window)
    need = bwd_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dsinks = torch.empty_like(sinks) if dsinks is None else dsinks
    st = _lib().attn_sink_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o), _ptr(lse),
                              _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_bwd")
    return dq, dk, dv, dsinks


def timing_enable(enable: bool = True) -> None:
    st = _lib().attn_sink_timing_enable(int(enable))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_timing_enable")


def timing_read() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded since timing_enable(True)."""
    n = 8
    names = (ctypes.c_char_p * n)()
    cnt = (ctypes.c_int * n)()
    ms = (ctypes.c_double * n)()
    k = _lib().attn_sink_timing_read(names, cnt, ms, n)
    if k < 0:
        raise RuntimeError("attn_sink_timing_read failed")
    return {names[i].decode(): (cnt[i], ms[i]) for i in range(min(k, n))}


class _SinkAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, sinks, cu_q, cu_k, max_q, max_k, scale, causal, window):
        o, lse = fwd(q, k, v, sinks, cu_q, cu_k, max_q, max_k, scale, causal, window)
        ctx.save_for_backward(q, k, v, sinks, o, lse, cu_q, cu_k)
        ctx.args = (max_q, max_k, scale, causal, window)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, sinks, o, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, scale, causal, window = ctx.args
        dq, dk, dv, ds = bwd(q, k, v, sinks, o, lse, do.contiguous(), cu_q, cu_k, max_q, max_k, scale, causal, window)
        return dq, dk, dv, ds, None, None, None, None, None, None, None


def sink_attention(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                   softmax_scale=None, causal=True, window=0):
    """Differentiable sink attention (autograd wrapper over fwd/bwd)."""
    cu_seqlens_k = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item())
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item())
    if softmax_scale is None:
        softmax_scale = q.shape[2] ** -0.5
    return _SinkAttentionFn.apply(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                                  softmax_scale, causal, window)
