"""The C ABI from several host threads at once: the library keeps no per-call state
outside the caller's buffers, so forward and backward calls issued concurrently from
two threads, each on a stream of its own (default priority), give bitwise the results
of the same calls made one after the other.  The second round runs with the timing
records on, so that their lock is exercised while both threads launch."""

import threading

import pytest
import torch

from _parity import to_dev
from workloads import random_case

pytestmark = pytest.mark.gpu


def _case(seed, window):
    inp = random_case([260, 97], 16, 2, 64, "bf16", seed=seed, window=window)
    d = to_dev(inp)
    q = d["q"]
    bufs = dict(o=torch.empty_like(q), lse=torch.empty(q.shape[1], q.shape[0], device="cuda"),
                dq=torch.empty_like(q), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
                ds=torch.empty_like(d["sinks"]))
    return inp, d, bufs


def _step(als, inp, d, b):
    cu, n, sc, w = d["cu_seqlens"], inp["max_seqlen"], inp["softmax_scale"], inp["window"]
    als.fwd(d["q"], d["k"], d["v"], d["sinks"], cu, cu, n, n, sc, True, w, out=b["o"], lse=b["lse"])
    als.bwd(d["q"], d["k"], d["v"], d["sinks"], b["o"], b["lse"], d["dout"], cu, cu, n, n, sc, True, w,
            dq=b["dq"], dk=b["dk"], dv=b["dv"], dsinks=b["ds"])


@pytest.mark.parametrize("timing", [False, True])
def test_two_threads_match_serial_calls(gpu_lib, timing):
    cases = [_case(81, 0), _case(82, 40)]
    print(f"[case] two host threads, timing records {timing}", flush=True)
    for inp, d, b in cases:
        _step(gpu_lib, inp, d, b)
    torch.cuda.synchronize()
    ref = [{k: t.clone() for k, t in b.items()} for _, _, b in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(i):
        try:
            inp, d, b = cases[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(5):
                    _step(gpu_lib, inp, d, b)
            streams[i].synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(repr(e))

    for _, _, b in cases:
        for t in b.values():
            t.fill_(float("nan"))
    torch.cuda.synchronize()
    gpu_lib.timing_enable(timing)
    try:
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    finally:
        gpu_lib.timing_enable(False)
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (_, _, b) in enumerate(cases):
        for k, t in b.items():
            assert torch.equal(t, ref[i][k]), f"thread {i}: {k}"
    if timing:
        recs = gpu_lib.timing_read()
        assert recs.get("attn_sink_fwd_kernel", (0,))[0] >= 10  # both threads' launches were recorded
