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

__all__ = ["load", "fwd", "fwd_decode", "fwd_decode_noalloc", "fwd_decode_workspace_bytes", "merge", "bwd", "bwd_workspace_bytes",
           "Shape", "AttnSinkError", "sink_attention", "timing_enable", "timing_read", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_sink.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
DECODE_SCRATCH_BYTES = 64 << 20  # ATTN_SINK_DECODE_SCRATCH_BYTES
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
    lib.attn_sink_fwd_decode_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_sink_fwd_decode_noalloc.restype = st
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


def _check_buf(name, t, shape, dtype, device):
    """A tensor the kernels read or write: exactly `shape`, `dtype`, contiguous, on `device`."""
    if not isinstance(t, torch.Tensor) or t.device != device or tuple(t.shape) != tuple(shape) or \
            t.dtype != dtype or not t.is_contiguous():
        got = (tuple(t.shape), t.dtype, t.device, t.is_contiguous()) if isinstance(t, torch.Tensor) else type(t)
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}; got {got}")


def _check_workspace(t, need, device):
    if not isinstance(t, torch.Tensor) or t.device != device or t.dtype != torch.uint8 or t.dim() != 1 or \
            not t.is_contiguous() or t.numel() < need:
        raise ValueError(f"workspace must be a contiguous 1-d uint8 tensor of at least {need} bytes on {device}")


def _check_tensors(q, k, v, sinks, cu_q, cu_k, device_type="cuda"):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or not t.is_contiguous() or t.device.type != device_type:
            raise ValueError(f"{name} must be a contiguous 3-d device tensor [T, H, d]")
    dev = q.device
    if k.dtype != q.dtype or v.dtype != q.dtype or v.shape != k.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q, k, v must share dtype and head dim; k and v must match")
    if k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on one device")
    _check_buf("sinks", sinks, (q.shape[1],), torch.float32, dev)
    for name, cu in (("cu_seqlens_q", cu_q), ("cu_seqlens_k", cu_k)):
        if not isinstance(cu, torch.Tensor) or cu.dtype != torch.int32 or cu.dim() != 1 or cu.device != dev or \
                not cu.is_contiguous() or cu.numel() < 1:
            raise ValueError(f"{name} must be a contiguous int32 tensor [num_seqs + 1] on {dev}")
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length (num_seqs + 1)")


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
    _check_buf("out", o, q.shape, q.dtype, q.device)
    _check_buf("lse", lse, (q.shape[1], q.shape[0]), torch.float32, q.device)
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
    need = fwd_decode_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device) if lse is None else lse
    _check_buf("out", o, q.shape, q.dtype, q.device)
    _check_buf("lse", lse, (q.shape[1], q.shape[0]), torch.float32, q.device)
    st = _lib().attn_sink_fwd_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o),
                                     _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(q.device))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_fwd_decode")
    return o, lse


def fwd_decode_noalloc(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, max_seqlen_k=None,
                       softmax_scale=None, causal=True, window=0, out=None, lse=None):
    """fwd_decode() in the library's fixed per-GPU scratch (no workspace, no
    allocation in the call itself; out= and lse= make the whole call allocation-free).
    Calls that overlap on one GPU race on that scratch."""
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
    _check_buf("out", o, q.shape, q.dtype, q.device)
    _check_buf("lse", lse, (q.shape[1], q.shape[0]), torch.float32, q.device)
    st = _lib().attn_sink_fwd_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o),
                                             _ptr(lse), _stream(q.device))
    if st != OK:
        raise AttnSinkError(st, "attn_sink_fwd_decode_noalloc")
    return o, lse


def merge(o_parts, lse_parts, sinks, out=None, lse=None):
    """Merge per-shard attention partials (each from fwd() with sinks = -inf over one
    key shard) into sink attention, the sink counted once.  o_parts [P, Tq, Hq, 64]
    (bf16 or fp32), lse_parts [P, Hq, Tq] fp32, sinks [Hq] fp32, all contiguous on the
    device.  Returns (o [Tq, Hq, 64], lse [Hq, Tq])."""
    if not isinstance(o_parts, torch.Tensor) or o_parts.dim() != 4 or not o_parts.is_contiguous() or \
            not o_parts.is_cuda:
        raise ValueError("o_parts must be a contiguous 4-d device tensor [P, Tq, Hq, d]")
    p, tq, hq, d = o_parts.shape
    dev = o_parts.device
    _check_buf("lse_parts", lse_parts, (p, hq, tq), torch.float32, dev)
    _check_buf("sinks", sinks, (hq,), torch.float32, dev)
    if o_parts.dtype == torch.bfloat16:
        dt = BF16
    elif o_parts.dtype == torch.float32:
        dt = FP32
    else:
        raise TypeError(f"unsupported dtype {o_parts.dtype}")
    o = torch.empty(tq, hq, d, dtype=o_parts.dtype, device=dev) if out is None else out
    lse = torch.empty(hq, tq, dtype=torch.float32, device=dev) if lse is None else lse
    _check_buf("out", o, (tq, hq, d), o_parts.dtype, dev)
    _check_buf("lse", lse, (hq, tq), torch.float32, dev)
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
        _check_buf(name, t, q.shape, q.dtype, q.device)
    _check_buf("lse", lse, (q.shape[1], q.shape[0]), torch.float32, q.device)
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
    _check_workspace(workspace, need, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dsinks = torch.empty_like(sinks) if dsinks is None else dsinks
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v), ("dsinks", dsinks, sinks)):
        _check_buf(name, t, ref.shape, ref.dtype, q.device)
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
