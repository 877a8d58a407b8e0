"""attn_sink_fwd_decode_noalloc: the decoding forward in the library's fixed
per-GPU scratch, for callers that cannot allocate.  Through the C ABI it must give
bitwise what attn_sink_fwd_decode gives with a caller-provided workspace (same
kernels, same layout), on two calls in a row, the second with a smaller input
(the scratch then holds the first call's partials)."""

import ctypes

import pytest
import torch

from workloads import decode_case

pytestmark = pytest.mark.gpu


def _dev(inp):
    return {k: inp[k].cuda().contiguous() for k in ("q", "k", "v", "sinks", "cu_seqlens_q", "cu_seqlens_k")}


def _shape(als, inp, d):
    return als.make_shape(d["q"], d["k"], d["cu_seqlens_q"], d["cu_seqlens_k"], inp["max_seqlen_q"],
                          inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"], inp["window"])


def test_noalloc_decode_equals_the_workspace_entry_point(gpu_lib):
    lib = gpu_lib.load()
    st = torch.cuda.current_stream().cuda_stream
    cases = [("first, multi-chunk", decode_case([3000, 12000, 50, 7000], 2, 64, 8, 64, "bf16", seed=61)),
             ("second, smaller", decode_case([1500, 300], 1, 64, 8, 64, "bf16", seed=62))]
    sizes = []
    for label, inp in cases:
        print(f"[case] noalloc decode: {label}", flush=True)
        d = _dev(inp)
        shape = _shape(gpu_lib, inp, d)
        need = gpu_lib.fwd_decode_workspace_bytes(shape)
        assert 0 < need <= gpu_lib.DECODE_SCRATCH_BYTES
        sizes.append(need)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ref = torch.full_like(d["q"], float("nan"))
        lse_ref = torch.full((d["q"].shape[1], d["q"].shape[0]), float("nan"), device="cuda")
        assert lib.attn_sink_fwd_decode(ctypes.byref(shape), d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                        d["sinks"].data_ptr(), o_ref.data_ptr(), lse_ref.data_ptr(), ws.data_ptr(),
                                        need, st) == gpu_lib.OK
        o = torch.full_like(d["q"], float("nan"))
        lse = torch.full((d["q"].shape[1], d["q"].shape[0]), float("nan"), device="cuda")
        assert lib.attn_sink_fwd_decode_noalloc(ctypes.byref(shape), d["q"].data_ptr(), d["k"].data_ptr(),
                                                d["v"].data_ptr(), d["sinks"].data_ptr(), o.data_ptr(),
                                                lse.data_ptr(), st) == gpu_lib.OK
        torch.cuda.synchronize()
        assert not torch.isnan(o_ref.float()).any() and not torch.isnan(lse_ref).any()
        assert torch.equal(o, o_ref), label
        assert torch.equal(lse, lse_ref), label
    assert sizes[1] < sizes[0]
