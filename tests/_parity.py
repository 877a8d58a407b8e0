"""Helpers for GPU-vs-oracle parity tests: run the HIP path through the binding,
run the oracle on the same host values, compare normwise.

Metric (per tensor): max |x - x_ref| / max |x_ref| over the compared entries.
Tolerances: 2e-2 when the tensors are bfloat16, 1e-5 when they are float32.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"bf16": 2e-2, "fp32": 1e-5}


def dtype_name(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "fp32"


def to_dev(inp: dict, dev="cuda") -> dict:
    out = dict(inp)
    for k in ("q", "k", "v", "dout", "sinks", "cu_seqlens"):
        if inp.get(k) is not None:
            out[k] = inp[k].to(dev).contiguous()
    return out


def gpu_fwd_bwd(als, inp: dict, dout=None, with_bwd=True) -> dict:
    """Forward (+ backward) on the GPU; returns host float64 numpy arrays."""
    d = to_dev(inp)
    cu = d["cu_seqlens"]
    o, lse = als.fwd(d["q"], d["k"], d["v"], d["sinks"], cu, cu, inp["max_seqlen"], inp["max_seqlen"],
                     inp["softmax_scale"], inp["causal"], inp["window"])
    res = dict(o=o, lse=lse)
    if with_bwd:
        do = d["dout"] if dout is None else dout.to("cuda").contiguous()
        dq, dk, dv, ds = als.bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, do, cu, cu, inp["max_seqlen"],
                                 inp["max_seqlen"], inp["softmax_scale"], inp["causal"], inp["window"])
        res.update(dq=dq, dk=dk, dv=dv, dsinks=ds)
    torch.cuda.synchronize()
    return {k: v.detach().float().cpu().numpy().astype(np.float64) for k, v in res.items()}


def oracle_bwd(inp: dict, **kw) -> dict:
    return oracle.sink_attention_backward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["dout"],
                                          inp["cu_seqlens"], inp["cu_seqlens"], inp["softmax_scale"],
                                          inp["causal"], inp["window"], **kw)


def relerr(x: np.ndarray, ref: np.ndarray) -> float:
    """Normwise relative error over entries where ref is not NaN (the oracle marks
    entries it did not compute with NaN)."""
    m = ~np.isnan(ref)
    assert m.any(), "nothing to compare"
    r, g = ref[m], x[m]
    finite = np.isfinite(r)
    # -inf lse (rows with no mass at all) must match exactly
    assert np.array_equal(g[~finite], r[~finite]), "non-finite reference entries differ"
    r, g = r[finite], g[finite]
    assert np.all(np.isfinite(g)), "non-finite GPU values"
    if r.size == 0:
        return 0.0
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))


def compare(gpu: dict, ref: dict, keys, tol: float, label: str = "") -> dict:
    errs = {}
    for k in keys:
        errs[k] = relerr(gpu[k], ref[k])
    print(f"[parity] {label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    return errs
