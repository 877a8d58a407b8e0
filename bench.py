"""Benchmark: sink-attention forward + backward on the GPT-OSS-20B attention shape.

One step = attn_sink_fwd + attn_sink_bwd over one batch (B=1, Hq=64, Hkv=8,
d=64, N=4096, causal, bf16, synthetic inputs resident in HBM).  Prints one JSON
line: whole-job TFLOP/s (algorithmic: 4d FLOP forward + 10d FLOP backward per
visible (query, key) pair per query head), the roofline of the dominant
kernel (per-launch durations from HIP events recorded by the library on the
launch stream over the timed region), and the CPU oracle timed on a bounded
sample of the same workload.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector and MFMA)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Sources of the training kernels (forward, backward) and of the decoding-step kernels:
# a counter summary is valid only for the digest of the sources of its kernel.
KERNEL_SOURCES = ["attention_learnable_sinks_amd/csrc/common.h", "attention_learnable_sinks_amd/csrc/fwd.hip",
                  "attention_learnable_sinks_amd/csrc/bwd.hip"]
DECODE_SOURCES = ["attention_learnable_sinks_amd/csrc/common.h", "attention_learnable_sinks_amd/csrc/decode.hip"]


def _code_only(text: str) -> str:
    """Source text without comments, blank lines or trailing blanks: an edit to a
    comment leaves the kernel, and the digest, unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def source_digest(paths=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(DECODE_SOURCES if "decode" in kernel else KERNEL_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_sclk(workload: str, kernel: str):
    """Core clock (GHz) the kernel ran at in the committed counter run (an upper bound:
    the busy counter includes some cycles outside the kernel), or None when there is none
    or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    digest, clocks = None, {}
    for line in open(path):
        parts = line.split()
        if line.startswith("kernel_source_digest") and len(parts) > 1:
            digest = parts[1]
        elif line.startswith("sclk_ghz") and len(parts) == 3:
            clocks[parts[1]] = float(parts[2])
    if digest != source_digest(KERNEL_SOURCES):
        return None
    short = kernel.replace("attn_sink_", "")  # attn_sink_bwd_dkdv_kernel -> bwd_dkdv_kernel
    for name, ghz in clocks.items():
        if short in name and "DF16bLi64" in name:
            return ghz
    return None


def count_pairs(seqlens, causal: bool, window: int) -> int:
    """Visible (query, key) pairs per query head: the work unit of the FLOP count."""
    total = 0
    for n in seqlens:
        for i in range(n):
            hi = i + 1 if causal else n
            lo = max(0, i - window + 1) if window > 0 else 0
            total += max(0, hi - lo)
    return total


def cpu_baseline(inp: dict, workload, pairs: int, budget_s: float = 12.0, gpu_out=None):
    """Time the float64 oracle on whole kv groups of the same inputs until about
    `budget_s` seconds have been spent; report the algorithmic rate of that sample.
    If GPU outputs are given, also report their normwise error on the sample."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    # The oracle's threads: one per core this process may run on, at most the host
    # share the GPU's jobs are given (OMP_NUM_THREADS where it is set).
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = max(1, min(threads, int(os.environ["OMP_NUM_THREADS"])))
    limiter = threadpool_limits(limits=threads)
    group = workload.num_heads_q // workload.num_heads_kv
    done, t_total, errs = 0, 0.0, {}
    for g in range(workload.num_heads_kv):
        heads = list(range(g * group, (g + 1) * group))
        t0 = time.perf_counter()
        ref = oracle.sink_attention_backward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["dout"],
                                             inp["cu_seqlens"], inp["cu_seqlens"], inp["softmax_scale"],
                                             inp["causal"], inp["window"], heads=heads)
        t_total += time.perf_counter() - t0
        done += 1
        if gpu_out is not None:
            for name in ("o", "lse", "dq", "dk", "dv", "dsinks"):
                r = ref[name]
                if name in ("dk", "dv"):
                    r = r[:, g:g + 1]
                    x = gpu_out[name][:, g:g + 1]
                else:
                    x = gpu_out[name]
                m = ~np.isnan(r)
                e = float(np.max(np.abs(x[m] - r[m])) / np.max(np.abs(r[m])))
                errs[name] = max(errs.get(name, 0.0), e)
        if t_total >= budget_s:
            break
    limiter.restore_original_limits()
    d = workload.head_dim
    flop = pairs * group * done * 4 * d + pairs * group * done * 10 * d
    return dict(value=round(flop / t_total / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{workload.name}: kv groups 0..{done - 1} ({done * group} of {workload.num_heads_q} query "
                       f"heads), forward+backward, float64 numpy with {threads} BLAS threads, {t_total:.1f} s",
                affinity_cores=len(os.sched_getaffinity(0))), errs


def decode_bench(als, torch, dev, steps: int, warmup: int) -> dict:
    """Time the decoding-step forward (attn_sink_fwd_decode) on the rollout decoding
    workload, each layer kind, with the training forward kernel on the same inputs
    beside it.  Algorithmic bytes per call: the K and V rows every sequence's new rows
    can see (whole cache, or the window), Q, and O + LSE written once."""
    from workloads import DECODE_WORKLOADS, make_decode_inputs

    w = DECODE_WORKLOADS["decode_rollout"]
    res = {"workload": w.name, "source_digest": source_digest(DECODE_SOURCES),
           "num_seqs": len(w.cache_lens), "new_rows": w.new_rows,
           "cache_keys": int(sum(w.cache_lens)), "num_heads_q": w.num_heads_q, "num_heads_kv": w.num_heads_kv,
           "layers": []}
    for layer in range(len(w.layers)):
        inp = make_decode_inputs(w, layer)
        d = {k: inp[k].to(dev).contiguous() for k in ("q", "k", "v", "sinks", "cu_seqlens_q", "cu_seqlens_k")}
        args = (d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"], d["cu_seqlens_k"], inp["max_seqlen_q"],
                inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"], inp["window"])
        shape = als.make_shape(d["q"], d["k"], d["cu_seqlens_q"], d["cu_seqlens_k"], inp["max_seqlen_q"],
                               inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"], inp["window"])
        ws = torch.empty(als.fwd_decode_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        o = torch.empty_like(d["q"])
        lse = torch.empty(w.num_heads_q, d["q"].shape[0], dtype=torch.float32, device=dev)
        timings = {}
        for name, call in (("decode", lambda: als.fwd_decode(*args, workspace=ws, out=o, lse=lse)),
                           ("fwd", lambda: als.fwd(*args, out=o, lse=lse))):
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            als.timing_enable(True)
            t0 = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            kern = als.timing_read()
            als.timing_enable(False)
            timings[name] = ((t1 - t0) * 1e3 / steps, {k: v[1] / v[0] for k, v in kern.items()})
        window, rows = inp["window"], w.new_rows
        keys = sum(min(n, window + rows - 1) if window > 0 else n for n in w.cache_lens)
        elem = 2 if w.dtype == "bf16" else 4
        tq = d["q"].shape[0]
        hd = w.head_dim
        byts = 2 * keys * w.num_heads_kv * hd * elem + 2 * tq * w.num_heads_q * hd * elem + tq * w.num_heads_q * 4
        dec_ms = sum(timings["decode"][1].values())
        part_ms = timings["decode"][1].get("attn_sink_decode_partial_kernel", float("nan"))
        kv_part = 2 * keys * w.num_heads_kv * hd * elem + tq * w.num_heads_q * hd * elem  # partial kernel: K, V, Q
        part_gbs = kv_part / (part_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(part_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(part_gbs / PEAK_HBM_GBS, 4),
                    traffic=read_traffic(w.name, "attn_sink_decode_partial_kernel") if window == 0 else None,
                    kernel="attn_sink_decode_partial_kernel", launch_ms=round(part_ms, 5),
                    algorithmic_bytes=int(kv_part))
        res["layers"].append({
            "window": int(window), "visible_keys": int(keys), "algorithmic_bytes": int(byts),
            "us_per_call": round(timings["decode"][0] * 1e3, 2),
            "kernels_us": {k: round(v * 1e3, 2) for k, v in timings["decode"][1].items()},
            "gbs": round(byts / (dec_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm": round(byts / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "partial_kernel_frac_of_hbm": round(kv_part / (part_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "fwd_kernel_us": round(sum(timings["fwd"][1].values()) * 1e3, 2),
            "roofline": roof,
        })
        del ws, o, lse, d
    return res


class Step:
    """One fwd+bwd step of a workload layer on the device: inputs, outputs and the
    backward workspace allocated once, outside any timed region."""

    def __init__(self, als, torch, dev, w, layer):
        from workloads import make_inputs

        self.als, self.w = als, w
        inp = make_inputs(w, layer=layer)
        self.inp = inp
        d = {k: inp[k].to(dev).contiguous() for k in ("q", "k", "v", "dout", "sinks", "cu_seqlens")}
        self.d = d
        cu = d["cu_seqlens"]
        self.mx, self.scale = inp["max_seqlen"], inp["softmax_scale"]
        self.causal, self.window = inp["causal"], inp["window"]
        shape = als.make_shape(d["q"], d["k"], cu, cu, self.mx, self.mx, self.scale, self.causal, self.window)
        self.ws = torch.empty(max(als.bwd_workspace_bytes(shape), 1), dtype=torch.uint8, device=dev)
        self.o = torch.empty_like(d["q"])
        self.lse = torch.empty(w.num_heads_q, w.total, dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        self.dsk = torch.empty_like(d["sinks"])
        self.pairs = count_pairs(w.seqlens, self.causal, self.window)

    def __call__(self):
        d, cu, a = self.d, self.d["cu_seqlens"], self.als
        a.fwd(d["q"], d["k"], d["v"], d["sinks"], cu, cu, self.mx, self.mx, self.scale, self.causal, self.window,
              out=self.o, lse=self.lse)
        a.bwd(d["q"], d["k"], d["v"], d["sinks"], self.o, self.lse, d["dout"], cu, cu, self.mx, self.mx, self.scale,
              self.causal, self.window, workspace=self.ws, dq=self.dq, dk=self.dk, dv=self.dv, dsinks=self.dsk)

    def host_outputs(self):
        import numpy as np
        return {k: t.float().cpu().numpy().astype(np.float64) for k, t in
                dict(o=self.o, lse=self.lse, dq=self.dq, dk=self.dk, dv=self.dv, dsinks=self.dsk).items()}


def kernel_events(als, torch, step, n):
    """Average ms per launch of each library kernel over n steps (HIP events that the
    library records on the launch stream), and the wall time per step."""
    als.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = als.timing_read()
    als.timing_enable(False)
    return {k: v[1] / v[0] for k, v in kern.items()}, (t1 - t0) * 1e3 / n


def figures(w, step, per, workload_name):
    """Forward / backward figures and the dominant kernel's roofline from per-launch
    kernel durations (ms).  Algorithmic work: 4d FLOP forward and 10d backward per
    visible (query, key) pair and query head; per kernel, the forward runs 2 GEMMs
    (4d), the dQ kernel 3 (S, dP, dQ: 6d) and the dK/dV kernel 4 (S, dP, dV, dK: 8d).
    Algorithmic bytes: each operand moved once."""
    hd, hq, hkv, t_tok = w.head_dim, w.num_heads_q, w.num_heads_kv, w.total
    pairs = step.pairs
    fwd_flop, bwd_flop = 4 * hd * pairs * hq, 10 * hd * pairs * hq
    elem = 2 if w.dtype == "bf16" else 4
    mfma_peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    qb, kb = t_tok * hq * hd * elem, t_tok * hkv * hd * elem  # one [T, Hq, d] / [T, Hkv, d] tensor
    rows = t_tok * hq * 4                                       # one fp32 value per row and head
    kern_bytes = {
        "attn_sink_fwd_kernel": qb + 2 * kb + qb + rows,                    # Q, K, V -> O, LSE
        "attn_sink_bwd_dq_kernel": 3 * qb + 2 * kb + rows + qb + 2 * rows,  # Q, O, dO, K, V, LSE -> dQ, rows
        "attn_sink_bwd_dkdv_kernel": 2 * qb + 2 * kb + 2 * rows + 2 * kb,   # Q, dO, K, V, rows -> dK, dV
        "attn_sink_bwd_finish_kernel": 2 * kb,
    }
    gemm_d = {"attn_sink_fwd_kernel": 4, "attn_sink_bwd_dq_kernel": 6, "attn_sink_bwd_dkdv_kernel": 8}
    fwd_ms = per.get("attn_sink_fwd_kernel", float("nan"))
    bwd_ms = sum(v for k, v in per.items() if k != "attn_sink_fwd_kernel")
    fwd_bytes = kern_bytes["attn_sink_fwd_kernel"]
    bwd_bytes = 3 * qb + 2 * kb + rows + qb + 2 * kb + rows  # Q K V O dO LSE -> dQ dK dV, plus D

    def leg(flop, byts, ms):
        tf = flop / (ms * 1e-3) / 1e12
        gbs = byts / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "tflops": round(tf, 3), "frac_of_peak": round(tf / mfma_peak, 4),
                "algorithmic_gbs": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4)}

    dom = max(per, key=per.get)
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte where the two peaks meet
    flop = gemm_d.get(dom, 0) * hd * pairs * hq
    byts = kern_bytes.get(dom, 0)
    if flop > 0 and flop / max(byts, 1) >= ridge:
        work, unit, bound, peak = flop / 1e12, "TFLOP/s", "mfma", mfma_peak
    else:
        work, unit, bound, peak = byts / 1e9, "GB/s", "hbm", PEAK_HBM_GBS
    achieved = work / (per[dom] * 1e-3)
    roofline = dict(bound=bound, achieved=round(achieved, 3), peak=peak, unit=unit, frac=round(achieved / peak, 4),
                    traffic=read_traffic(workload_name, dom), kernel=dom, launch_ms=round(per[dom], 5),
                    flop_per_byte=round(flop / max(byts, 1), 1))
    return {"fwd": leg(fwd_flop, fwd_bytes, fwd_ms), "bwd": leg(bwd_flop, bwd_bytes, bwd_ms),
            "fwd_bwd_tflops": round((fwd_flop + bwd_flop) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 3),
            "kernels_ms_per_launch": {k: round(v, 5) for k, v in per.items()},
            "roofline": roofline}, fwd_flop, bwd_flop


# The other workload layers, measured in the same run (their parity is the GPU tests'):
# (name, layer) in the order they are reported.
OTHER_CONFIGS = [("tiny", 0), ("window_16k", 0), ("varlen", 0), ("varlen", 1), ("long_20k", 0), ("d128_4k", 0)]


def config_bench(als, torch, dev, steps: int, warmup: int) -> dict:
    """Per-workload fwd / bwd figures from the library's per-kernel events (a warm-up,
    then `steps` steps with events); each layer's buffers are freed before the next."""
    from workloads import WORKLOADS

    out = {}
    for name, layer in OTHER_CONFIGS:
        w = WORKLOADS[name]
        key = f"{name}:{layer}" if len(w.layers) > 1 else name
        step = Step(als, torch, dev, w, layer)
        n = steps if step.pairs * w.num_heads_q < 5e10 else max(3, steps // 4)  # long layers: fewer steps
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        per, _ = kernel_events(als, torch, step, n)
        fig, _, _ = figures(w, step, per, key.replace(":", "_layer"))
        fig.update(steps=n, dtype=w.dtype, seqlens=len(w.seqlens), total=w.total, heads=[w.num_heads_q, w.num_heads_kv],
                   head_dim=w.head_dim, window=int(step.window), causal=bool(step.causal))
        out[key] = fig
        del step
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU takes some 30-50 steps (tens of ms) after a pause to settle at its working
    # clock; fewer warm-up steps measure the ramp.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gptoss_4k")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (for counter calibration)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decoding-step leg")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workload layers")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps, each after rewriting a 512 MiB buffer (L2 and MALL flushed), timed apart")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library is a single-GPU kernel library "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_learnable_sinks_amd as als
    from workloads import WORKLOADS

    als.load()
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    step = Step(als, torch, dev, w, args.layer)
    causal, window, scale = step.causal, step.window, step.scale

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Steps with the library's per-kernel HIP events recorded on the launch stream: the
    # per-launch durations of the roofline.  The event records add about 25 us of queue
    # markers per step, so `value` comes from the next, uninstrumented pass.  At least
    # 40 steps, so the GPU has settled before that pass even with a short warm-up.
    n_ev = max(args.steps, 40)
    per, ms_ev = kernel_events(als, torch, step, n_ev)
    # The K timed steps, uninstrumented: `value` and ms_per_step.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    host = None if args.no_cpu else step.host_outputs()

    # Cold-cache steps: a 512 MiB write between steps evicts L2 and the MALL; only the
    # library's kernels are timed (HIP events around each launch).
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        als.timing_enable(True)
        for _ in range(args.cold_steps):
            flush.fill_(1)
            step()
        torch.cuda.synchronize()
        kc = als.timing_read()
        als.timing_enable(False)
        del flush
        per_c = {k: v[1] / v[0] for k, v in kc.items()}
        cold = {"fwd_ms": round(per_c.get("attn_sink_fwd_kernel", float("nan")), 5),
                "bwd_ms": round(sum(v for k, v in per_c.items() if k != "attn_sink_fwd_kernel"), 5),
                "steps": args.cold_steps}

    # committed profiles are named per layer for workloads with several layer calls
    wname = f"{args.workload}_layer{args.layer}" if len(w.layers) > 1 else args.workload
    fig, fwd_flop, bwd_flop = figures(w, step, per, wname)
    ms = (t1 - t0) * 1e3 / args.steps
    value = (fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12
    roofline = fig["roofline"]
    dom = roofline["kernel"]
    # The same against the clock the kernel actually ran at (CUs x 4096 bf16 FLOP per clock x
    # the core clock from the committed counter run, an upper bound, so this fraction is a
    # lower bound).
    sclk = read_sclk(wname, dom) if roofline["bound"] == "mfma" and w.dtype == "bf16" else None
    if sclk is not None:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        adj = cus * 4096 * sclk * 1e9 / 1e12
        roofline.update(sclk_ghz=sclk, clock_adjusted_peak=round(adj, 1),
                        frac_of_clock_adjusted_peak=round(roofline["achieved"] / adj, 4))
    inp = step.inp
    del step
    torch.cuda.empty_cache()

    configs = None if args.no_configs else config_bench(als, torch, dev, max(args.steps, 10), max(args.warmup, 5))
    dec = None if args.no_decode else decode_bench(als, torch, dev, max(args.steps, 10), max(args.warmup, 2))

    cpu, errs = None, {}
    if not args.no_cpu:
        cpu, errs = cpu_baseline(inp, w, count_pairs(w.seqlens, causal, window), args.cpu_budget, host)

    out = {
        "metric": "attention fwd+bwd TFLOP/s and % bf16 MFMA peak, GPT-OSS-20B shape",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_with_kernel_events": round(ms_ev, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": len(w.seqlens), "seqlens": list(w.seqlens)[:8],
                   "num_heads_q": w.num_heads_q, "num_heads_kv": w.num_heads_kv, "head_dim": w.head_dim,
                   "causal": bool(causal), "window": int(window), "softmax_scale": scale},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": fig["fwd"],
        "bwd": fig["bwd"],
        "cold_cache": cold,
        "configs": configs,
        "decode": dec,
        "kernels_ms_per_launch": fig["kernels_ms_per_launch"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity_on_cpu_sample": {k: float(f"{v:.3e}") for k, v in errs.items()} or None,
        "kernel_source_digest": source_digest(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
