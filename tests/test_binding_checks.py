"""Host-only checks of the Python binding's argument validation: the binding is the
only layer that sees tensor shapes, dtypes and devices, so every tensor handed to
the C ABI (inputs, caller-provided outputs and workspaces) must be checked there
before its pointer reaches a kernel."""

import pytest
import torch

import attention_learnable_sinks_amd as als


def _inputs(tq=10, tk=10, hq=4, hkv=2, d=64, dtype=torch.bfloat16):
    q = torch.zeros(tq, hq, d, dtype=dtype)
    k = torch.zeros(tk, hkv, d, dtype=dtype)
    v = torch.zeros(tk, hkv, d, dtype=dtype)
    s = torch.zeros(hq)
    cu = torch.tensor([0, tq], dtype=torch.int32)
    return q, k, v, s, cu


def test_host_tensors_are_rejected_before_any_call():
    q, k, v, s, cu = _inputs()
    with pytest.raises(ValueError):
        als.fwd(q, k, v, s, cu, cu, 10, 10, 0.125, True, 0)
    with pytest.raises(ValueError):
        als.bwd(q, k, v, s, q, torch.zeros(4, 10), q, cu, cu, 10, 10, 0.125, True, 0)
    with pytest.raises(ValueError):
        als.fwd_decode(q, k, v, s, cu, cu, 10, 10, 0.125, True, 0)
    with pytest.raises(ValueError):
        als.merge(q[None], torch.zeros(1, 4, 10), s)


def test_input_set_checks():
    q, k, v, s, cu = _inputs()
    als._check_tensors(q, k, v, s, cu, cu, device_type="cpu")  # well-formed
    bad = [
        dict(cu_k=torch.tensor([0, 5, 10], dtype=torch.int32)),     # cu lengths differ
        dict(cu_q=torch.tensor([0, 10], dtype=torch.int64)),        # cu dtype
        dict(sinks=torch.zeros(3)),                                 # sinks [Hq]
        dict(sinks=torch.zeros(4, dtype=torch.float64)),
        dict(v=torch.zeros(10, 2, 64)),                             # dtype mismatch
        dict(k=torch.zeros(10, 2, 32, dtype=torch.bfloat16)),       # head dim mismatch
        dict(q=torch.zeros(10, 64, 4, dtype=torch.bfloat16).transpose(1, 2)),  # not contiguous
        dict(q=torch.zeros(10, 256, dtype=torch.bfloat16)),         # not 3-d
    ]
    for kw in bad:
        args = dict(q=q, k=k, v=v, sinks=s, cu_q=cu, cu_k=cu)
        args.update(kw)
        with pytest.raises(ValueError):
            als._check_tensors(args["q"], args["k"], args["v"], args["sinks"], args["cu_q"], args["cu_k"],
                               device_type="cpu")


def test_output_and_workspace_buffers_are_size_checked():
    dev = torch.device("cpu")
    als._check_buf("out", torch.zeros(10, 4, 64), (10, 4, 64), torch.float32, dev)
    for t in (torch.zeros(9, 4, 64), torch.zeros(10, 4, 64, dtype=torch.bfloat16),
              torch.zeros(10, 64, 4).transpose(1, 2), torch.zeros(10 * 4 * 64), None):
        with pytest.raises(ValueError):
            als._check_buf("out", t, (10, 4, 64), torch.float32, dev)
    als._check_workspace(torch.zeros(100, dtype=torch.uint8), 100, dev)
    for t in (torch.zeros(99, dtype=torch.uint8), torch.zeros(100, dtype=torch.int8),
              torch.zeros(10, 10, dtype=torch.uint8), None):
        with pytest.raises(ValueError):
            als._check_workspace(t, 100, dev)
