"""The training forward and backward and the decoding forward captured in a HIP graph
(torch.cuda.CUDAGraph): every replay must give bitwise the eager results.

With max_seqlen, the outputs and the workspace passed in, no entry point allocates,
sets memory or synchronises inside a call, so the calls are capturable; the kernels
overwrite every output, so a replay depends on its inputs alone.  Before each replay
the outputs are poisoned with NaN and the program runs eager work of its own and
synchronises, so that a replay which left anything to an earlier run would show."""

import pytest
import torch

from _parity import to_dev
from workloads import decode_case, random_case

pytestmark = pytest.mark.gpu


def _replays_match(run, outs, label, replays=3):
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()  # warm-up off the capture stream, as torch asks
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(replays):
        for t in outs:
            t.fill_(float("nan"))
        x = torch.randn(512, 512, device="cuda")
        assert torch.isfinite((x @ x).sum()).item()  # eager work and a synchronisation
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t, e), f"{label}: replay {rep}, output {i}"


@pytest.mark.parametrize("window", [0, 50])
def test_training_step_in_a_graph(gpu_lib, window):
    """Forward and backward in one graph: per-head tiles (no window, the dK/dV head
    splits and the finish kernel's partial sums) and head-packed tiles (window 50)."""
    inp = random_case([300, 77, 190], 16, 2, 64, "bf16", seed=71 + window, window=window)
    d = to_dev(inp)
    cu, n, sc = d["cu_seqlens"], inp["max_seqlen"], inp["softmax_scale"]
    print(f"[case] graph training step window {window}", flush=True)
    q, k, v, s, do = d["q"], d["k"], d["v"], d["sinks"], d["dout"]
    o, lse = torch.empty_like(q), torch.empty(q.shape[1], q.shape[0], device="cuda")
    dq, dk, dv, ds = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(s)
    shape = gpu_lib.make_shape(q, k, cu, cu, n, n, sc, True, window)
    ws = torch.empty(max(gpu_lib.bwd_workspace_bytes(shape), 1), dtype=torch.uint8, device="cuda")

    def run():
        gpu_lib.fwd(q, k, v, s, cu, cu, n, n, sc, True, window, out=o, lse=lse)
        gpu_lib.bwd(q, k, v, s, o, lse, do, cu, cu, n, n, sc, True, window, workspace=ws, dq=dq, dk=dk, dv=dv,
                    dsinks=ds)

    _replays_match(run, [o, lse, dq, dk, dv, ds], f"training window {window}")


@pytest.mark.parametrize("noalloc", [False, True])
def test_decoding_step_in_a_graph(gpu_lib, noalloc):
    """The decoding forward (multi-chunk caches: partial and merge kernels) in a graph,
    with a caller workspace and in the library's fixed scratch."""
    inp = decode_case([3000, 1200, 64], 1, 64, 8, 64, "bf16", seed=73)
    d = {k: inp[k].cuda().contiguous() for k in ("q", "k", "v", "sinks", "cu_seqlens_q", "cu_seqlens_k")}
    print(f"[case] graph decoding step noalloc={noalloc}", flush=True)
    args = (d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"], d["cu_seqlens_k"], inp["max_seqlen_q"],
            inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"], inp["window"])
    o, lse = torch.empty_like(d["q"]), torch.empty(d["q"].shape[1], d["q"].shape[0], device="cuda")
    shape = gpu_lib.make_shape(d["q"], d["k"], d["cu_seqlens_q"], d["cu_seqlens_k"], inp["max_seqlen_q"],
                               inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"], inp["window"])
    ws = torch.empty(max(gpu_lib.fwd_decode_workspace_bytes(shape), 1), dtype=torch.uint8, device="cuda")

    def run():
        if noalloc:
            gpu_lib.fwd_decode_noalloc(*args, out=o, lse=lse)
        else:
            gpu_lib.fwd_decode(*args, workspace=ws, out=o, lse=lse)

    _replays_match(run, [o, lse], f"decoding noalloc={noalloc}")
