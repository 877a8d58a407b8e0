"""GPU parity at head dim 128 (the kernels are templated on the head dim; a 128-wide
row is stored as two 64-column LDS tile blocks).  Every path is checked against
the oracle, element by element: training forward and backward (several tiles,
ragged tails, GQA, causal / window / non-causal, unequal query and key lengths),
the full-size 4k causal workload (one kv group), the decoding forward, and the
sharded forward with the sink-aware merge."""

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, decode_case, make_inputs, random_case
from _parity import TOL, compare, gpu_fwd_bwd, oracle_bwd

pytestmark = pytest.mark.gpu
ALL = ("o", "lse", "dq", "dk", "dv", "dsinks")
SCALE = 128 ** -0.5

CASES = [
    # seqlens, hq, hkv, causal, window
    ([300], 8, 2, True, 0),
    ([1, 77, 300, 0, 129], 4, 1, True, 0),
    ([333, 64, 200], 4, 4, True, 37),
    ([257], 4, 2, False, 0),
    ([190, 450], 4, 4, False, 100),
    ([300], 8, 2, True, 64),  # one sequence, window: head-packed forward tiles
    ([200, 77, 345], 16, 2, True, 50),  # 8 query heads per kv head, window: packed dK/dV tiles too
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}-c{int(c[3])}-w{c[4]}" for c in CASES])
def test_d128_small(gpu_lib, case, dtype):
    seqlens, hq, hkv, causal, window = case
    inp = random_case(seqlens, hq, hkv, 128, dtype, seed=sum(seqlens) + 128, causal=causal, window=window,
                      scale=SCALE)
    print(f"[case] d128 {case} {dtype}", flush=True)
    gpu = gpu_fwd_bwd(gpu_lib, inp)
    compare(gpu, oracle_bwd(inp), ALL, TOL[dtype], f"d128 {case} {dtype}")


def test_d128_unequal_lengths_bottom_right(gpu_lib):
    torch.manual_seed(6)
    lq, lk = [100, 7, 130], [160, 3, 130]
    hq, hkv = 4, 2
    for dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        q = torch.randn(sum(lq), hq, 128).to(dtype)
        k = torch.randn(sum(lk), hkv, 128).to(dtype)
        v = torch.randn(sum(lk), hkv, 128).to(dtype)
        do = torch.randn(sum(lq), hq, 128).to(dtype)
        s = torch.randn(hq)
        cq = torch.tensor(np.cumsum([0] + lq), dtype=torch.int32)
        ck = torch.tensor(np.cumsum([0] + lk), dtype=torch.int32)
        o, lse = gpu_lib.fwd(q.cuda(), k.cuda(), v.cuda(), s.cuda(), cq.cuda(), ck.cuda(), max(lq), max(lk),
                             SCALE, True, 40)
        dq, dk, dv, ds = gpu_lib.bwd(q.cuda(), k.cuda(), v.cuda(), s.cuda(), o, lse, do.cuda(), cq.cuda(),
                                     ck.cuda(), max(lq), max(lk), SCALE, True, 40)
        ref = oracle.sink_attention_backward(q, k, v, s, do, cq, ck, SCALE, True, 40)
        gpu = {n: t.float().cpu().numpy().astype(np.float64)
               for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, dsinks=ds).items()}
        compare(gpu, ref, ALL, tol, f"d128 unequal lengths {dtype}")


def test_d128_4k_group0(gpu_lib):
    """4k causal, 32 query / 8 kv heads of 128: every output of kv group 0."""
    inp = make_inputs(WORKLOADS["d128_4k"])
    print("[case] d128_4k", flush=True)
    gpu = gpu_fwd_bwd(gpu_lib, inp)
    ref = oracle_bwd(inp, heads=range(4))
    for key in ("dk", "dv"):
        ref[key][:, 1:] = np.nan
    compare(gpu, ref, ALL, TOL["bf16"], "d128_4k group 0")


def test_d128_repeatable(gpu_lib):
    inp = random_case([700, 300], 8, 2, 128, "bf16", seed=9, scale=SCALE)
    a = gpu_fwd_bwd(gpu_lib, inp)
    b = gpu_fwd_bwd(gpu_lib, inp)
    for key in ALL:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_d128_decode(gpu_lib, dtype):
    for window in (0, 128):
        inp = decode_case([1, 65, 3001, 20000], [1, 2, 4, 1], 32, 8, 128, dtype, seed=11, window=window,
                          scale=SCALE)
        d = {k: inp[k].cuda().contiguous() for k in ("q", "k", "v", "sinks", "cu_seqlens_q", "cu_seqlens_k")}
        o, lse = gpu_lib.fwd_decode(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens_q"], d["cu_seqlens_k"],
                                    inp["max_seqlen_q"], inp["max_seqlen_k"], SCALE, True, window)
        torch.cuda.synchronize()
        ro, rlse = oracle.sink_attention_forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens_q"],
                                                 inp["cu_seqlens_k"], SCALE, True, window)
        got = dict(o=o.float().cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))
        compare(got, dict(o=ro, lse=rlse), ("o", "lse"), TOL[dtype], f"d128 decode {dtype} w{window}")


def test_d128_sharded_merge(gpu_lib):
    """Keys cut into 3 shards, each attended with the sink off, merged with the sink."""
    inp = random_case([300, 513], 8, 2, 128, "fp32", seed=12, causal=False, scale=SCALE)
    cu = inp["cu_seqlens"].tolist()
    q, sinks, cuq = inp["q"].cuda(), inp["sinks"].cuda(), inp["cu_seqlens"].cuda()
    off = torch.full_like(sinks, float("-inf"))
    o_parts, lse_parts = [], []
    for lo_f, hi_f in ((0.0, 0.3), (0.3, 0.8), (0.8, 1.0)):
        ks, vs, cuk = [], [], [0]
        for b in range(len(cu) - 1):
            n = cu[b + 1] - cu[b]
            lo, hi = int(n * lo_f), int(n * hi_f)
            ks.append(inp["k"][cu[b] + lo:cu[b] + hi])
            vs.append(inp["v"][cu[b] + lo:cu[b] + hi])
            cuk.append(cuk[-1] + hi - lo)
        cuk = torch.tensor(cuk, dtype=torch.int32)
        o_s, l_s = gpu_lib.fwd(q, torch.cat(ks).contiguous().cuda(), torch.cat(vs).contiguous().cuda(), off, cuq,
                               cuk.cuda(), inp["max_seqlen"], int((cuk[1:] - cuk[:-1]).max()), SCALE, False, 0)
        o_parts.append(o_s)
        lse_parts.append(l_s)
    o, lse = gpu_lib.merge(torch.stack(o_parts).contiguous(), torch.stack(lse_parts).contiguous(), sinks)
    torch.cuda.synchronize()
    ro, rlse = oracle.sink_attention_forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                             inp["cu_seqlens"], SCALE, False, 0)
    got = dict(o=o.cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))
    compare(got, dict(o=ro, lse=rlse), ("o", "lse"), TOL["fp32"], "d128 sharded merge")
