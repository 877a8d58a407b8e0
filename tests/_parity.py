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


def sink_terms(inp: dict, ref: dict) -> np.ndarray:
    """sum_i |P_sink_i D_i| per head, from the oracle's own O and LSE: the size of the
    terms whose sum is dS_h (its condition scale: dS_h can cancel to a small fraction
    of it, where float32 arithmetic on the terms leaves an error of a few units of
    roundoff times this sum)."""
    sinks = inp["sinks"].double().numpy()
    dout = inp["dout"].double().numpy()
    with np.errstate(invalid="ignore"):
        ps = np.exp(sinks[:, None] - ref["lse"])                 # [Hq, T]
        d = np.einsum("thc,thc->ht", dout, ref["o"])             # [Hq, T]
        return np.nansum(np.abs(ps * d), axis=1)


def compare_dsinks_per_head(gpu: dict, ref: dict, heads, tol: float, label: str = "", terms=None,
                            roundoff: float = 0.0) -> np.ndarray:
    """dS_h head by head (a head whose reference is small is not hidden behind the
    largest one, as it is normwise): |dS_h - ref| <= tol |ref| + roundoff sum_i
    |P_sink_i D_i|.  With roundoff = 0 (the default) this is the plain per-head
    relative error |dS_h - ref| / |ref| <= tol."""
    heads = list(heads)
    g, r = gpu["dsinks"][heads], ref["dsinks"][heads]
    assert np.all(np.isfinite(r)) and np.all(np.isfinite(g))
    t = np.zeros(len(heads)) if terms is None else np.asarray(terms)[heads]
    errs = np.abs(g - r) / np.maximum(np.abs(r), 1e-30)
    bound = tol + roundoff * t / np.maximum(np.abs(r), 1e-30)
    cond = t / np.maximum(np.abs(r), 1e-30)
    print(f"[parity] {label} dS_h per head (rel. error, condition sum|terms|/|dS_h|): " +
          " ".join(f"{h}:{e:.1e}" + (f"/{c:.0f}" if terms is not None else "") for h, e, c in zip(heads, errs, cond)),
          flush=True)
    bad = {int(h): float(e) for h, e, b in zip(heads, errs, bound) if not e <= b}
    assert not bad, f"{label}: dS_h over tolerance {tol} for heads {bad}"
    return errs
