"""Sequence (context) parallelism on one GPU: the keys are cut into shards, each
shard is attended with the sink switched off (attn_sink_fwd, S_h = -inf), and
attn_sink_merge combines the partials, adding the sink once.  The merged output
must equal the oracle's sink attention over all the keys; the backward, run per
shard with the merged O and LSE, must give the full gradients (dq summed over the
shards, dk / dv per shard, dsinks as the shards' sum less n - 1 times a call with
no keys).  The shards stand in for
devices: what crosses devices in a real run (the partials, dq, dsinks) is exactly
what these tests combine."""

import numpy as np
import pytest
import torch

import oracle
from workloads import random_case
from _parity import TOL, compare

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _shard_bounds(n, g):
    """Cut n keys into g contiguous shards of unequal sizes (the last may be empty)."""
    cuts = sorted({0, n} | {int(n * f) for f in (0.17, 0.5, 0.93)[: g - 1]})
    while len(cuts) < g + 1:
        cuts.append(n)
    return list(zip(cuts[:-1], cuts[1:]))


def _split_keys(inp, g):
    """Per shard: (k_s, v_s, cu_k_s) holding each sequence's keys of that shard."""
    cu = inp["cu_seqlens"].tolist()
    out = []
    for s in range(g):
        ks, vs, cuk = [], [], [0]
        for b in range(len(cu) - 1):
            n = cu[b + 1] - cu[b]
            lo, hi = _shard_bounds(n, g)[s]
            ks.append(inp["k"][cu[b] + lo:cu[b] + hi])
            vs.append(inp["v"][cu[b] + lo:cu[b] + hi])
            cuk.append(cuk[-1] + hi - lo)
        out.append((torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), torch.tensor(cuk, dtype=torch.int32)))
    return out


def _sharded_forward(als, inp, g):
    dev = lambda t: t.cuda().contiguous()
    q, sinks, cuq = dev(inp["q"]), dev(inp["sinks"]), dev(inp["cu_seqlens"])
    off = torch.full_like(sinks, float("-inf"))
    o_parts, lse_parts = [], []
    for k_s, v_s, cuk in _split_keys(inp, g):
        maxk = int((cuk[1:] - cuk[:-1]).max())
        o_s, lse_s = als.fwd(q, dev(k_s), dev(v_s), off, cuq, dev(cuk), inp["max_seqlen"], maxk,
                             inp["softmax_scale"], False, 0)
        o_parts.append(o_s)
        lse_parts.append(lse_s)
    o, lse = als.merge(torch.stack(o_parts).contiguous(), torch.stack(lse_parts).contiguous(), sinks)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shards", [1, 2, 4])
def test_sharded_forward_equals_full_attention(gpu_lib, dtype, shards):
    inp = random_case([300, 77, 513], 8, 2, 64, dtype, seed=31 + shards, causal=False, scale=0.125)
    o, lse = _sharded_forward(gpu_lib, inp, shards)
    ro, rlse = oracle.sink_attention_forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                             inp["cu_seqlens"], 0.125, False, 0)
    compare(dict(o=_np(o), lse=_np(lse)), dict(o=ro, lse=rlse), ("o", "lse"), TOL[dtype],
            f"sharded fwd {shards} shards {dtype}")


def test_merge_of_one_part_adds_only_the_sink(gpu_lib):
    """One part: lse = logaddexp(lse_1, S_h) and o = o_1 * sigmoid(lse_1 - S_h), the
    closed form of appending the sink to a finished softmax."""
    torch.manual_seed(3)
    tq, hq = 50, 4
    o1 = torch.randn(1, tq, hq, 64)
    l1 = torch.randn(1, hq, tq) * 3
    l1[0, 1, 7] = float("-inf")  # a row that saw no key
    s = torch.tensor([0.5, -2.0, float("-inf"), 4.0])
    o, lse = gpu_lib.merge(o1.cuda(), l1.cuda(), s.cuda())
    ref_lse = np.logaddexp(_np(l1[0]), _np(s)[:, None])
    w = np.exp(_np(l1[0]) - ref_lse)  # [hq, tq]
    ref_o = _np(o1[0]) * w.T[:, :, None]
    np.testing.assert_allclose(_np(lse), ref_lse, rtol=0, atol=1e-5)
    np.testing.assert_allclose(_np(o), ref_o, rtol=1e-5, atol=1e-5)
    assert float(lse[1, 7]) == -2.0 and torch.all(o[7, 1] == 0)  # only the sink: o = 0, lse = S_h


def test_merge_with_no_mass_anywhere(gpu_lib):
    """Every part -inf and the sink -inf: o = 0, lse = -inf (no division by zero)."""
    o1 = torch.randn(3, 5, 2, 64).cuda()
    l1 = torch.full((3, 2, 5), float("-inf")).cuda()
    o, lse = gpu_lib.merge(o1, l1, torch.full((2,), float("-inf")).cuda())
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_sharded_causal_ring_equals_full_attention(gpu_lib):
    """One causal sequence of G equal shards, as a ring would visit them: for shard s,
    its own rows see it causally (diagonal block, N_q = N_k), later rows see all of
    it, earlier rows none of it."""
    for dtype in ("fp32", "bf16"):
        n, g, hq, hkv = 384, 3, 8, 2
        L = n // g
        inp = random_case([n], hq, hkv, 64, dtype, seed=40, causal=True, scale=0.125)
        q, k, v = (inp[x].cuda().contiguous() for x in ("q", "k", "v"))
        sinks = inp["sinks"].cuda()
        off = torch.full_like(sinks, float("-inf"))
        one = lambda m: torch.tensor([0, m], dtype=torch.int32, device="cuda")
        o_parts = torch.zeros(g, n, hq, 64, dtype=q.dtype, device="cuda")
        lse_parts = torch.full((g, hq, n), float("-inf"), device="cuda")
        for s in range(g):
            ks, vs = k[s * L:(s + 1) * L].contiguous(), v[s * L:(s + 1) * L].contiguous()
            qd = q[s * L:(s + 1) * L].contiguous()
            od, ld = gpu_lib.fwd(qd, ks, vs, off, one(L), one(L), L, L, 0.125, True, 0)
            o_parts[s, s * L:(s + 1) * L] = od
            lse_parts[s, :, s * L:(s + 1) * L] = ld
            if s + 1 < g:
                qo = q[(s + 1) * L:].contiguous()
                oo, lo = gpu_lib.fwd(qo, ks, vs, off, one(n - (s + 1) * L), one(L), n - (s + 1) * L, L, 0.125,
                                     False, 0)
                o_parts[s, (s + 1) * L:] = oo
                lse_parts[s, :, (s + 1) * L:] = lo
        o, lse = gpu_lib.merge(o_parts, lse_parts, sinks)
        torch.cuda.synchronize()
        ro, rlse = oracle.sink_attention_forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                                 inp["cu_seqlens"], 0.125, True, 0)
        compare(dict(o=_np(o), lse=_np(lse)), dict(o=ro, lse=rlse), ("o", "lse"), TOL[dtype],
                f"causal ring {g} shards {dtype}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sharded_backward_equals_full_gradients(gpu_lib, dtype):
    """Per-shard attn_sink_bwd with the merged o, lse: dq summed over the shards,
    dk / dv from each shard.  dsinks: each call returns its shard's part of
    -sum_i P_sink_i sum_j P_ij dP_ij plus the key-independent term
    -sum_i P_sink_i D_i (1 - P_sink_i) (D_i = <dO_i, O_i>), which a call with no keys
    returns alone; so dS_h = sum over the shards - (shards - 1) x that call."""
    shards = 3
    inp = random_case([300, 77, 513], 8, 2, 64, dtype, seed=50, causal=False, scale=0.125)
    o, lse = _sharded_forward(gpu_lib, inp, shards)
    dev = lambda t: t.cuda().contiguous()
    q, sinks, cuq, do = dev(inp["q"]), dev(inp["sinks"]), dev(inp["cu_seqlens"]), dev(inp["dout"])
    dq = torch.zeros(q.shape, dtype=torch.float64)
    dk_parts, dv_parts, ds = [], [], []
    split = _split_keys(inp, shards)
    for k_s, v_s, cuk in split:
        maxk = int((cuk[1:] - cuk[:-1]).max())
        dq_s, dk_s, dv_s, ds_s = gpu_lib.bwd(q, dev(k_s), dev(v_s), sinks, o, lse, do, cuq, dev(cuk),
                                             inp["max_seqlen"], maxk, 0.125, False, 0)
        dq += dq_s.double().cpu()
        dk_parts.append(dk_s.double().cpu())
        dv_parts.append(dv_s.double().cpu())
        ds.append(ds_s)
    none = torch.zeros(0, inp["k"].shape[1], 64, dtype=q.dtype, device="cuda")
    cu0 = torch.zeros_like(cuq)
    ds_none = gpu_lib.bwd(q, none, none, sinks, o, lse, do, cuq, cu0, inp["max_seqlen"], 0, 0.125, False, 0)[3]
    dsinks = sum(x.double() for x in ds) - (shards - 1) * ds_none.double()
    full = gpu_lib.bwd(q, dev(inp["k"]), dev(inp["v"]), sinks, o, lse, do, cuq, cuq, inp["max_seqlen"],
                       inp["max_seqlen"], 0.125, False, 0)[3]
    torch.cuda.synchronize()
    torch.testing.assert_close(dsinks.float(), full, rtol=1e-5, atol=1e-6)  # as one call over all keys
    # reassemble dk / dv in the packed order of the full key tensor
    cu = inp["cu_seqlens"].tolist()
    dk = torch.zeros(inp["k"].shape, dtype=torch.float64)
    dv = torch.zeros(inp["v"].shape, dtype=torch.float64)
    for s, (_, _, cuk) in enumerate(split):
        cuk = cuk.tolist()
        for b in range(len(cu) - 1):
            lo, hi = _shard_bounds(cu[b + 1] - cu[b], shards)[s]
            dk[cu[b] + lo:cu[b] + hi] = dk_parts[s][cuk[b]:cuk[b + 1]]
            dv[cu[b] + lo:cu[b] + hi] = dv_parts[s][cuk[b]:cuk[b + 1]]
    ref = oracle.sink_attention_backward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["dout"],
                                         inp["cu_seqlens"], inp["cu_seqlens"], 0.125, False, 0)
    got = dict(dq=dq.numpy(), dk=dk.numpy(), dv=dv.numpy(), dsinks=_np(dsinks))
    compare(got, ref, ("dq", "dk", "dv", "dsinks"), TOL[dtype], f"sharded bwd {dtype}")


def test_merge_is_repeatable(gpu_lib):
    o1 = torch.randn(5, 200, 8, 64, dtype=torch.bfloat16).cuda()
    l1 = (torch.randn(5, 8, 200) * 4).cuda()
    s = torch.randn(8).cuda()
    a = gpu_lib.merge(o1, l1, s)
    b = gpu_lib.merge(o1, l1, s)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
