"""GPU parity of the decoding-step forward (attn_sink_fwd_decode) against the CPU
oracle, element by element.

The cases cover what the split-K organisation can get wrong: caches shorter than
one 64-key tile, ragged last tiles, enough keys for many splits (so the merge
combines partials of different maxima and empty splits), new rows that see no key
at all, sequences without new rows, every column count from 1 to 32 of the
(query head x new row) block (G = 1, 3, 8, 32), kv head counts that split into
workgroups of 1, 2, 4, 6 or 8 heads, sequences finished in one chunk beside
sequences merged from many, windows that cut a tile, non-causal rows, and sinks at
-inf and far above every score.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import DECODE_WORKLOADS, decode_case, make_decode_inputs
from _parity import TOL, compare

pytestmark = pytest.mark.gpu

KEYS = ("cu_seqlens_q", "cu_seqlens_k", "q", "k", "v", "sinks")


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _dev(inp):
    return {k: inp[k].cuda().contiguous() for k in KEYS}


def _decode(als, inp, workspace=None):
    d = _dev(inp)
    o, lse = als.fwd_decode(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                            inp["max_seqlen_q"], inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"],
                            inp["window"], workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def _fwd(als, inp):
    d = _dev(inp)
    o, lse = als.fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"], d["cu_seqlens_k"], inp["max_seqlen_q"],
                     inp["max_seqlen_k"], inp["softmax_scale"], inp["causal"], inp["window"])
    torch.cuda.synchronize()
    return o, lse


def _oracle(inp, **kw):
    return oracle.sink_attention_forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens_q"],
                                         inp["cu_seqlens_k"], inp["softmax_scale"], inp["causal"], inp["window"],
                                         **kw)


def _check(als, inp, label, tol=None):
    tol = TOL["bf16" if inp["q"].dtype == torch.bfloat16 else "fp32"] if tol is None else tol
    print(f"[case] decode {label}", flush=True)
    o, lse = _decode(als, inp)
    ro, rlse = _oracle(inp)
    return compare(dict(o=_np(o), lse=_np(lse)), dict(o=ro, lse=rlse), ("o", "lse"), tol, f"decode {label}")


CASES = [
    # cache lengths, new rows (per sequence or one count), hq, hkv, causal, window
    ([1, 63, 64, 65, 700, 3001], 1, 64, 8, True, 0),
    ([1, 63, 64, 65, 700, 3001], 1, 64, 8, True, 128),
    ([5, 130, 2000], [1, 4, 2], 64, 8, True, 0),
    ([3, 130, 2000], 4, 64, 8, True, 37),
    ([400, 1000], 32, 8, 8, True, 0),
    ([400, 1000], 10, 24, 8, True, 50),
    ([900, 77], 1, 32, 1, True, 0),
    ([600, 1500], 3, 16, 2, False, 0),
    ([600, 1500], 3, 16, 2, False, 100),
    ([0, 50, 10], [2, 2, 0], 8, 2, True, 0),
    ([20000], 2, 64, 8, True, 0),
    ([300, 5000, 2], 2, 24, 12, True, 0),
    ([4000, 90], 5, 6, 2, True, 300),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-c{int(c[4])}-w{c[5]}" for c in CASES])
def test_decode_against_oracle(gpu_lib, case, dtype):
    cache, rows, hq, hkv, causal, window = case
    inp = decode_case(cache, rows, hq, hkv, 64, dtype, seed=sum(cache) + hq, causal=causal, window=window)
    _check(gpu_lib, inp, f"{case} {dtype}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_agrees_with_the_forward_kernel(gpu_lib, dtype):
    """Same function as attn_sink_fwd, and both normalise by the float32 sum of the
    probabilities before they are rounded for the P.V product: equal up to rounding
    order.  fp32: 1e-5 normwise.  bf16: LSE to 1e-6 normwise, and O within one bf16
    unit in the last place of its largest element (at most 2^-7 normwise: the two
    kernels round P under different running maxima, so an output element may land on
    either side of a rounding boundary)."""
    for window in (0, 128):
        inp = decode_case([70, 4000, 9000], 4, 64, 8, 64, dtype, seed=21, window=window)
        a_o, a_lse = _decode(gpu_lib, inp)
        b_o, b_lse = _fwd(gpu_lib, inp)
        a, b = dict(o=_np(a_o), lse=_np(a_lse)), dict(o=_np(b_o), lse=_np(b_lse))
        if dtype == "fp32":
            compare(a, b, ("o", "lse"), 1e-5, f"decode vs fwd {dtype} w{window}")
            continue
        compare(a, b, ("lse",), 1e-6, f"decode vs fwd lse {dtype} w{window}")
        top = np.max(np.abs(b["o"]))
        ulp_top = 2.0 ** (np.floor(np.log2(top)) - 7)  # bf16 spacing at the largest |O|
        diff = np.max(np.abs(a["o"] - b["o"]))
        print(f"[decode vs fwd] w{window}: max |diff| = {diff / ulp_top:.2f} bf16 ulp of max|O| "
              f"({diff / top:.2e} normwise); {np.mean(a['o'] == b['o']):.3f} of elements equal", flush=True)
        assert diff <= ulp_top, (diff, ulp_top)


def test_decode_is_repeatable(gpu_lib):
    inp = decode_case([3000, 12000, 50], 2, 64, 8, 64, "bf16", seed=22)
    a = _decode(gpu_lib, inp)
    b = _decode(gpu_lib, inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_is_batch_invariant(gpu_lib):
    """A sequence's outputs are bitwise the same whether it is decoded alone, first or
    last in a batch, or beside caches of other lengths (the key chunking depends on
    the sequence alone), for full and windowed layers."""
    for window in (0, 128):
        big = decode_case([5000, 70, 12000, 2100], [1, 3, 2, 4], 64, 8, 64, "bf16", seed=27, window=window)
        o_all, lse_all = _decode(gpu_lib, big)
        cq, ck = big["cu_seqlens_q"].tolist(), big["cu_seqlens_k"].tolist()
        for b in (0, 2, 3):
            one = dict(big)
            one["q"] = big["q"][cq[b]:cq[b + 1]].contiguous()
            one["k"] = big["k"][ck[b]:ck[b + 1]].contiguous()
            one["v"] = big["v"][ck[b]:ck[b + 1]].contiguous()
            one["cu_seqlens_q"] = torch.tensor([0, cq[b + 1] - cq[b]], dtype=torch.int32)
            one["cu_seqlens_k"] = torch.tensor([0, ck[b + 1] - ck[b]], dtype=torch.int32)
            one["max_seqlen_q"], one["max_seqlen_k"] = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
            o1, lse1 = _decode(gpu_lib, one)
            assert torch.equal(o1, o_all[cq[b]:cq[b + 1]]), (window, b)
            assert torch.equal(lse1, lse_all[:, cq[b]:cq[b + 1]]), (window, b)


def test_decode_minus_inf_sink(gpu_lib):
    """S_h = -inf: standard attention; a row without visible keys then has o = 0, lse = -inf."""
    inp = decode_case([0, 300, 5000], [1, 2, 3], 16, 4, 64, "fp32", seed=23)
    inp["sinks"] = torch.full((16,), float("-inf"))
    _check(gpu_lib, inp, "S_h=-inf")
    o, lse = _decode(gpu_lib, inp)
    assert torch.all(lse[:, 0].cpu() == float("-inf")) and torch.all(o[0].cpu() == 0)


def test_decode_large_sink_absorbs_everything(gpu_lib):
    inp = decode_case([700, 5000], 2, 8, 2, 64, "fp32", seed=24)
    inp["sinks"] = torch.tensor([30.0, 60.0] * 4)
    o, lse = _decode(gpu_lib, inp)
    assert float(o.abs().max()) < 1e-8
    np.testing.assert_allclose(_np(lse), np.array([[30.0], [60.0]] * 4) * np.ones((1, 4)), rtol=1e-6)


def test_decode_workspace_reuse(gpu_lib):
    """One workspace serves a large call and then a smaller one; the second result
    equals a call with a fresh workspace."""
    big = decode_case([16000, 9000], 4, 64, 8, 64, "bf16", seed=25)
    small = decode_case([700, 80, 3000], 1, 64, 8, 64, "bf16", seed=26)
    d = _dev(big)
    shape = gpu_lib.make_shape(d["q"], d["k"], d["cu_seqlens_q"], d["cu_seqlens_k"], big["max_seqlen_q"],
                               big["max_seqlen_k"], 0.125, True, 0)
    ws = torch.empty(gpu_lib.fwd_decode_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    _decode(gpu_lib, big, workspace=ws)
    a = _decode(gpu_lib, small, workspace=ws)
    b = _decode(gpu_lib, small)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("layer", [0, 1], ids=["full", "window128"])
def test_decode_rollout_full_size(gpu_lib, layer):
    """The benchmarked decoding step (64 sequences, caches of 1k-16k keys, one new
    row, 64 query / 8 kv heads), every output element against the oracle."""
    inp = make_decode_inputs(DECODE_WORKLOADS["decode_rollout"], layer)
    _check(gpu_lib, inp, f"rollout layer {layer}")
