"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases compare every output element; they span several query and key
tiles (forward tiles of 128 queries x 64 keys, backward tiles of 64 queries x
128 keys) and end in ragged tails.  The five workload configurations run at
full size in the launch configuration the benchmark times; there the oracle
computes whole kv groups (every row of their query heads, every key of their kv
head) exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, random_case
from _parity import TOL, compare, compare_dsinks_per_head, gpu_fwd_bwd, oracle_bwd, sink_terms, to_dev

pytestmark = pytest.mark.gpu
ALL = ("o", "lse", "dq", "dk", "dv", "dsinks")


def _full_case(als, inp, label, tol=None):
    tol = TOL["bf16" if inp["q"].dtype == torch.bfloat16 else "fp32"] if tol is None else tol
    print(f"[case] {label}", flush=True)
    gpu = gpu_fwd_bwd(als, inp)
    ref = oracle_bwd(inp)
    return compare(gpu, ref, ALL, tol, label)


# ----------------------------------------------------------------------------- small, every element
def test_tiny_fp32(gpu_lib):
    inp = make_inputs(WORKLOADS["tiny"])
    _full_case(gpu_lib, inp, "tiny fp32")


SMALL = [
    # seqlens, hq, hkv, causal, window, sink distribution
    ([300], 8, 2, True, 0, ("normal",)),
    ([1, 77, 300, 0, 129], 4, 1, True, 0, ("normal",)),
    ([333, 64, 200], 8, 8, True, 37, ("uniform", -2.0, 4.0)),
    ([257], 4, 2, False, 0, ("normal",)),
    ([190, 450], 4, 4, False, 100, ("uniform", -2.0, 8.0)),
    ([513], 16, 2, True, 128, ("normal",)),
    ([300], 16, 1, True, 0, ("normal",)),  # one kv head: dK/dV over 16 head splits
    ([200, 77, 345], 16, 2, True, 50, ("uniform", -2.0, 8.0)),  # 8 heads per kv head: packed window tiles
    ([300, 45], 16, 2, True, 1, ("uniform", -2.0, 8.0)),  # window 1: every row sees its own key only
    ([260, 3], 4, 2, True, 65, ("normal",)),  # window one key past a 64-key tile
    ([300, 45], 16, 2, False, 60, ("uniform", -2.0, 8.0)),  # packed tiles, window without causal mask
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-{c[1]}x{c[2]}-c{int(c[3])}-w{c[4]}" for c in SMALL])
def test_small_ragged(gpu_lib, case, dtype):
    seqlens, hq, hkv, causal, window, dist = case
    inp = random_case(seqlens, hq, hkv, 64, dtype, seed=sum(seqlens) + hq, causal=causal, window=window,
                      sink_dist=dist, scale=0.125)
    _full_case(gpu_lib, inp, f"small {case} {dtype}")


def test_unequal_lengths_bottom_right(gpu_lib):
    """N_q != N_k per sequence: causal and window align the last query with the last key."""
    torch.manual_seed(5)
    lq, lk = [100, 7, 130, 0], [160, 3, 130, 50]
    hq, hkv = 4, 2
    for dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        for window in (0, 40):
            q = torch.randn(sum(lq), hq, 64).to(dtype)
            k = torch.randn(sum(lk), hkv, 64).to(dtype)
            v = torch.randn(sum(lk), hkv, 64).to(dtype)
            do = torch.randn(sum(lq), hq, 64).to(dtype)
            s = torch.randn(hq)
            cq = torch.tensor(np.cumsum([0] + lq), dtype=torch.int32)
            ck = torch.tensor(np.cumsum([0] + lk), dtype=torch.int32)
            o, lse = gpu_lib.fwd(q.cuda(), k.cuda(), v.cuda(), s.cuda(), cq.cuda(), ck.cuda(), max(lq), max(lk),
                                 0.125, True, window)
            dq, dk, dv, ds = gpu_lib.bwd(q.cuda(), k.cuda(), v.cuda(), s.cuda(), o, lse, do.cuda(), cq.cuda(),
                                         ck.cuda(), max(lq), max(lk), 0.125, True, window)
            ref = oracle.sink_attention_backward(q, k, v, s, do, cq, ck, 0.125, True, window)
            gpu = {n: t.float().cpu().numpy().astype(np.float64)
                   for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, dsinks=ds).items()}
            compare(gpu, ref, ALL, tol, f"unequal lengths {dtype} w{window}")


# ----------------------------------------------------------------------------- special cases
def test_minus_inf_sink_is_standard_attention(gpu_lib):
    inp = random_case([200, 131], 4, 2, 64, "fp32", seed=11)
    inp["sinks"] = torch.full((4,), float("-inf"))
    gpu = gpu_fwd_bwd(gpu_lib, inp)
    ref = oracle_bwd(inp)
    compare(gpu, ref, ("o", "lse", "dq", "dk", "dv"), 1e-5, "S_h=-inf")
    assert np.all(gpu["dsinks"] == 0.0)
    # and against torch's own attention for one head (float32, CPU)
    q, k, v = inp["q"][:200, 0], inp["k"][:200, 0], inp["v"][:200, 0]
    std = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True,
                                                           scale=0.125)[0]
    assert np.max(np.abs(gpu["o"][:200, 0] - std.numpy())) < 1e-5


def test_large_sink_absorbs_everything(gpu_lib):
    inp = random_case([300], 2, 1, 64, "fp32", seed=12)
    inp["sinks"] = torch.tensor([30.0, 60.0])
    gpu = gpu_fwd_bwd(gpu_lib, inp)
    assert np.max(np.abs(gpu["o"])) < 1e-8
    np.testing.assert_allclose(gpu["lse"], np.array([[30.0], [60.0]]) * np.ones((1, 300)), rtol=1e-6)
    ref = oracle_bwd(inp)
    compare(gpu, ref, ("lse", "dsinks"), 1e-5, "S_h=30,60")


def test_constant_v(gpu_lib):
    inp = random_case([260], 4, 2, 64, "fp32", seed=13)
    c = torch.randn(64)
    inp["v"] = c.expand(260, 2, 64).contiguous()
    gpu = gpu_fwd_bwd(gpu_lib, inp, with_bwd=False)
    p_sink = np.exp(inp["sinks"].numpy()[:, None] - gpu["lse"])
    np.testing.assert_allclose(gpu["o"], ((1 - p_sink).T)[:, :, None] * c.numpy(), atol=1e-5)


def test_window_at_least_n_equals_causal(gpu_lib):
    inp = random_case([400], 8, 2, 64, "bf16", seed=14)
    a = gpu_fwd_bwd(gpu_lib, inp)
    inp["window"] = 400
    b = gpu_fwd_bwd(gpu_lib, inp)
    for key in ("o", "lse"):
        assert np.array_equal(a[key], b[key]), key
    # dS_h: the window run's dQ tiles pack the query heads of a kv head, so its
    # partials group the rows differently: the same sum up to fp32 rounding order.
    np.testing.assert_allclose(a["dsinks"], b["dsinks"], rtol=1e-5, atol=1e-7)
    for key in ("dq", "dk", "dv"):
        assert np.max(np.abs(a[key] - b[key])) <= 1e-2 * np.max(np.abs(a[key])), key


def test_varlen_equals_separate_calls(gpu_lib):
    lens = [130, 0, 257, 64]
    inp = random_case(lens, 8, 2, 64, "bf16", seed=15, window=50)
    packed = gpu_fwd_bwd(gpu_lib, inp)
    cu = np.cumsum([0] + lens)
    ds = np.zeros(8)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        a, e = cu[b], cu[b + 1]
        one = dict(inp, q=inp["q"][a:e], k=inp["k"][a:e], v=inp["v"][a:e], dout=inp["dout"][a:e],
                   cu_seqlens=torch.tensor([0, n], dtype=torch.int32), max_seqlen=n)
        g = gpu_fwd_bwd(gpu_lib, one)
        assert np.array_equal(g["o"], packed["o"][a:e])
        assert np.array_equal(g["lse"], packed["lse"][:, a:e])
        for key in ("dq", "dk", "dv"):
            assert np.max(np.abs(g[key] - packed[key][a:e])) <= 1e-2 * max(1e-30, np.max(np.abs(packed[key][a:e])))
        ds += g["dsinks"]
    np.testing.assert_allclose(ds, packed["dsinks"], rtol=1e-4, atol=1e-5)


def test_gqa_equals_duplicated_kv(gpu_lib):
    inp = random_case([300], 8, 2, 64, "fp32", seed=16)
    a = gpu_fwd_bwd(gpu_lib, inp)
    dup = dict(inp, k=inp["k"].repeat_interleave(4, dim=1).contiguous(),
               v=inp["v"].repeat_interleave(4, dim=1).contiguous())
    b = gpu_fwd_bwd(gpu_lib, dup)
    for key in ("o", "lse", "dq", "dsinks"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-5, atol=1e-5)
    for key in ("dk", "dv"):
        np.testing.assert_allclose(a[key], b[key].reshape(300, 2, 4, 64).sum(2), rtol=1e-4, atol=1e-5)


def test_repeatability(gpu_lib):
    """Every output is bitwise repeatable (no atomics; fixed reduction orders)."""
    inp = random_case([700, 333], 8, 2, 64, "bf16", seed=17)
    runs = [gpu_fwd_bwd(gpu_lib, inp) for _ in range(3)]
    for r in runs[1:]:
        for key in ALL:
            assert np.array_equal(r[key], runs[0][key]), key


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_running_max_raised_mid_row(gpu_lib, dtype):
    """Key norms ramp up 40x along the sequence, so the scores of a row grow by far
    more than 64 (log2 units) from its first key tiles to its last: the forward must
    raise its running max and rescale O several times within one row.

    Tolerance: scores reach |s| ~ 150 here, and a float32 score carries an absolute
    error of about |s| * 2^-24 * sqrt(64) ~ 7e-5, which is the relative error it
    puts into exp(s); float32 is therefore held to 2e-4 instead of 1e-5 (bf16, whose
    bar comes from rounding P to 8 bits, keeps its usual one)."""
    inp = random_case([700, 190], 4, 2, 64, dtype, seed=21)
    ramp = torch.cat([torch.linspace(1.0, 40.0, 700), torch.linspace(1.0, 40.0, 190)])
    inp["k"] = (inp["k"].float() * ramp[:, None, None]).to(inp["k"].dtype)
    s_max = float((inp["q"].float() @ inp["k"].float().reshape(-1, 64).T).abs().max()) * 0.125
    print(f"[case] growing scores {dtype}: max |s| = {s_max:.1f}", flush=True)
    _full_case(gpu_lib, inp, f"growing scores {dtype}", tol=2e-4 if dtype == "fp32" else None)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("hq,hkv,causal", [(16, 2, True), (16, 1, True), (8, 4, True), (16, 2, False)])
def test_head_packed_tiles_bitwise(gpu_lib, dtype, hq, hkv, causal):
    """Window layers run on forward and dQ tiles that pack the query heads of a kv
    head (rows = positions x heads); layers without a window run on per-head tiles.
    A row's arithmetic depends only on its own scores, with key tiles at the same
    absolute key positions, so (1) a window of at least n keys (packed) gives
    bitwise the per-head causal / full O, LSE and dQ, and dS_h up to the rounding
    order of its partials, and (2) a sequence alone gives bitwise the rows it gets
    inside a ragged batch.  dK and dV sum over (head, row); with 8 query heads per kv
    head the bf16 window backward packs its query tiles too, which changes that
    order, so there they agree to one rounding of the element type (bitwise
    otherwise)."""
    n, m, window = 300, 77, 70
    inp = random_case([n, m], hq, hkv, 64, dtype, seed=hq + hkv + int(causal), causal=causal, window=window)
    d = to_dev(inp)
    sc = inp["softmax_scale"]
    print(f"[case] head-packed {dtype} {hq}x{hkv} causal={causal}", flush=True)
    cu2 = torch.tensor([0, n, n + m], dtype=torch.int32, device="cuda")
    cu1 = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    q, k, v = d["q"][:n].contiguous(), d["k"][:n].contiguous(), d["v"][:n].contiguous()
    o_wide, lse_wide = gpu_lib.fwd(q, k, v, d["sinks"], cu1, cu1, n, n, sc, causal, n + 5)
    o_none, lse_none = gpu_lib.fwd(q, k, v, d["sinks"], cu1, cu1, n, n, sc, causal, 0)
    do = d["dout"][:n].contiguous()
    g_wide = gpu_lib.bwd(q, k, v, d["sinks"], o_none, lse_none, do, cu1, cu1, n, n, sc, causal, n + 5)
    g_none = gpu_lib.bwd(q, k, v, d["sinks"], o_none, lse_none, do, cu1, cu1, n, n, sc, causal, 0)
    o2, lse2 = gpu_lib.fwd(d["q"], d["k"], d["v"], d["sinks"], cu2, cu2, n, n, sc, causal, window)
    o1, lse1 = gpu_lib.fwd(q, k, v, d["sinks"], cu1, cu1, n, n, sc, causal, window)
    torch.cuda.synchronize()
    assert torch.equal(o_wide, o_none) and torch.equal(lse_wide, lse_none)
    assert torch.equal(g_wide[0], g_none[0]), "dq"
    for name, x, y in zip(("dk", "dv"), g_wide[1:3], g_none[1:3]):
        if dtype == "bf16" and hq == 8 * hkv:
            ymax = y.float().abs().max().item()
            ulp = 2.0 ** (np.floor(np.log2(ymax)) - 7)  # one bf16 ulp at the tensor's largest magnitude
            assert (x.float() - y.float()).abs().max().item() <= ulp, name
        else:
            assert torch.equal(x, y), name
    # dS_h = -sum_i P_sink,i D_i over the head's rows; packed tiles group those rows
    # into other partials, so the two agree up to the order of a float32 sum of n
    # terms.  Either order lies within (n-1) u sum_i |P_sink,i D_i| of the exact sum
    # (u = 2^-24), so the two within twice that.  The terms cancel, so the bar is set
    # by their absolute sum, not by |dS_h|.
    o64 = o_none.double().cpu()
    dd = (o64 * do.double().cpu()).sum(-1)  # D_i = dO_i . O_i, [n, hq]
    psink = torch.exp(d["sinks"].double().cpu()[None, :] - lse_none.double().cpu().T)  # [n, hq]
    bound = 2 * (n - 1) * 2.0**-24 * (psink * dd).abs().sum(0)
    diff = (g_wide[3].double() - g_none[3].double()).abs().cpu()
    assert bool((diff <= bound).all()), f"dS_h {diff.tolist()} vs {bound.tolist()}"
    assert torch.equal(o1, o2[:n]) and torch.equal(lse1, lse2[:, :n])
    ref = oracle_bwd(inp)
    compare({"o": o2.float().cpu().numpy().astype(np.float64), "lse": lse2.cpu().numpy().astype(np.float64)},
            ref, ("o", "lse"), TOL[dtype], f"head-packed {dtype} {hq}x{hkv}")


@pytest.mark.parametrize("window", [0, 50])
def test_rows_alone_match_the_full_forward_bitwise(gpu_lib, window):
    """Inference-style calls -- one decode row against its whole prefix, or a chunk
    of rows -- give bitwise the same O, LSE and dQ rows as the full training call.
    Bottom-right alignment plus key tiles at absolute key positions make a row's
    arithmetic independent of the other rows it is computed with; the key ramp makes
    some rows raise their running max mid-sequence, which must not leak into others."""
    n = 300
    inp = random_case([n], 8, 2, 64, "bf16", seed=23, window=window)
    ramp = torch.linspace(1.0, 30.0, n)
    inp["k"] = (inp["k"].float() * ramp[:, None, None]).to(torch.bfloat16)
    d = to_dev(inp)
    sc = inp["softmax_scale"]
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    o_full, lse_full = gpu_lib.fwd(d["q"], d["k"], d["v"], d["sinks"], cu, cu, n, n, sc, True, window)
    dq_full = gpu_lib.bwd(d["q"], d["k"], d["v"], d["sinks"], o_full, lse_full, d["dout"], cu, cu, n, n, sc,
                          True, window)[0]
    for r0, r1 in [(299, 300), (0, 1), (131, 132), (64, 101), (200, 300)]:
        print(f"[case] rows {r0}..{r1} window {window}", flush=True)
        cq = torch.tensor([0, r1 - r0], dtype=torch.int32, device="cuda")
        ck = torch.tensor([0, r1], dtype=torch.int32, device="cuda")
        q, k, v = d["q"][r0:r1].contiguous(), d["k"][:r1].contiguous(), d["v"][:r1].contiguous()
        o, lse = gpu_lib.fwd(q, k, v, d["sinks"], cq, ck, r1 - r0, r1, sc, True, window)
        dq = gpu_lib.bwd(q, k, v, d["sinks"], o, lse, d["dout"][r0:r1].contiguous(), cq, ck, r1 - r0, r1, sc,
                         True, window)[0]
        torch.cuda.synchronize()
        assert torch.equal(o, o_full[r0:r1]), (r0, r1, "o")
        assert torch.equal(lse, lse_full[:, r0:r1]), (r0, r1, "lse")
        assert torch.equal(dq, dq_full[r0:r1]), (r0, r1, "dq")


def test_autograd_wrapper(gpu_lib):
    inp = to_dev(random_case([150, 90], 4, 2, 64, "fp32", seed=18))
    q, k, v, s = (inp[n].clone().requires_grad_(True) for n in ("q", "k", "v", "sinks"))
    o = gpu_lib.sink_attention(q, k, v, s, inp["cu_seqlens"], softmax_scale=0.125)
    (o * inp["dout"]).sum().backward()
    ref = oracle.sink_attention_backward(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["sinks"].cpu(),
                                         inp["dout"].cpu(), [0, 150, 240], [0, 150, 240], 0.125, True, 0)
    for name, t in (("dq", q.grad), ("dk", k.grad), ("dv", v.grad), ("dsinks", s.grad)):
        from _parity import relerr
        assert relerr(t.double().cpu().numpy(), ref[name]) < 1e-5, name


def test_empty_batch_rows(gpu_lib):
    """All sequences empty: nothing to compute, the sink gradient is 0."""
    q = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    s = torch.randn(4, device="cuda")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, lse = gpu_lib.fwd(q, k, k, s, cu, cu, 0, 0, 0.125, True, 0)
    dq, dk, dv, ds = gpu_lib.bwd(q, k, k, s, o, lse, q, cu, cu, 0, 0, 0.125, True, 0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.all(ds == 0)


# ----------------------------------------------------------------------------- full-size workloads
def _groups_full(als, inp, groups, label):
    """Every output of whole kv groups at full size: O, LSE and dQ of their query
    heads on every row, dK and dV of their kv heads on every key, and dS_h head by
    head."""
    hq, hkv = inp["q"].shape[1], inp["k"].shape[1]
    G = hq // hkv
    heads = [g * G + j for g in groups for j in range(G)]
    print(f"[case] {label} groups {list(groups)}", flush=True)
    gpu = gpu_fwd_bwd(als, inp)
    ref = oracle_bwd(inp, heads=heads)
    other = [g for g in range(hkv) if g not in groups]
    for key in ("dk", "dv"):
        ref[key][:, other] = np.nan
    compare(gpu, ref, ALL, TOL["bf16"], f"{label} groups {list(groups)}")
    compare_dsinks_per_head(gpu, ref, heads, TOL["bf16"], label, terms=sink_terms(inp, ref))


def test_gptoss_4k_group0(gpu_lib):
    """4k causal GPT-OSS shape: every output of kv group 0 (8 query heads)."""
    _groups_full(gpu_lib, make_inputs(WORKLOADS["gptoss_4k"]), [0], "gptoss_4k")


def test_window_16k_groups(gpu_lib):
    _groups_full(gpu_lib, make_inputs(WORKLOADS["window_16k"]), [0, 7], "window_16k")


@pytest.mark.timeout(900)
def test_long_20k_group1(gpu_lib):
    """Long rollout (20,480 rows, sinks U[-2, 8]): kv group 1, whose query heads have
    sinks 7.31, 3.69, 7.82, 4.06, 6.68, -1.77, 7.72 and 5.58, so the sink's share
    dominates many rows.  That is the regime which stresses LSE and dS_h."""
    _groups_full(gpu_lib, make_inputs(WORKLOADS["long_20k"]), [1], "long_20k")


@pytest.mark.timeout(900)
def test_varlen_full_layer_group7(gpu_lib):
    """Ragged 8-sequence batch, full causal layer: kv group 7, the group with the
    widest sink spread of this layer (2.78 down to -2.52)."""
    _groups_full(gpu_lib, make_inputs(WORKLOADS["varlen"], layer=0), [7], "varlen full")


def test_varlen_window_layer_group(gpu_lib):
    _groups_full(gpu_lib, make_inputs(WORKLOADS["varlen"], layer=1), [1], "varlen window")


# ----------------------------------------------------------------------------- backward in isolation
def _bwd_on_oracle_forward(als, inp, heads=None):
    """attn_sink_bwd fed the oracle's O (rounded once to the element type) and LSE
    (float32) in place of the GPU forward's.  Rows of heads the oracle left out
    (NaN) take the GPU forward's values, so every head's inputs are finite."""
    d = to_dev(inp)
    cu = d["cu_seqlens"]
    n, sc = inp["max_seqlen"], inp["softmax_scale"]
    ref = oracle_bwd(inp, heads=heads)
    o_gpu, lse_gpu = als.fwd(d["q"], d["k"], d["v"], d["sinks"], cu, cu, n, n, sc, inp["causal"], inp["window"])
    o_ref = torch.from_numpy(ref["o"]).to(d["q"].dtype).cuda()
    lse_ref = torch.from_numpy(ref["lse"]).float().cuda()
    o = torch.where(torch.isnan(o_ref.float()), o_gpu, o_ref).contiguous()
    lse = torch.where(torch.isnan(lse_ref), lse_gpu, lse_ref).contiguous()
    dq, dk, dv, ds = als.bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, d["dout"], cu, cu, n, n, sc,
                             inp["causal"], inp["window"])
    torch.cuda.synchronize()
    gpu = {k: t.float().cpu().numpy().astype(np.float64) for k, t in dict(dq=dq, dk=dk, dv=dv, dsinks=ds).items()}
    return gpu, ref


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("window", [0, 70])
def test_backward_on_the_oracle_forward(gpu_lib, dtype, window):
    """The backward alone, on the oracle's forward outputs: a backward error cannot
    hide behind (or be caused by) an error of the GPU forward.  This is the kernel
    counterpart of freezing the attention layers to isolate a fault ([Keryc]
    "Practical tips for teams who want to reproduce or extend this")."""
    inp = random_case([300, 129, 64], 8, 2, 64, dtype, seed=31 + window, causal=True, window=window,
                      sink_dist=("uniform", -2.0, 8.0))
    print(f"[case] backward on the oracle's forward {dtype} w{window}", flush=True)
    gpu, ref = _bwd_on_oracle_forward(gpu_lib, inp)
    compare(gpu, ref, ("dq", "dk", "dv", "dsinks"), TOL[dtype], f"bwd on oracle fwd {dtype} w{window}")
    # float32: 1e-5 of |dS_h| plus float32 roundoff (1e-6, about 16 units) of the terms
    # dS_h sums, since a head's terms can cancel to a small fraction of their size.
    compare_dsinks_per_head(gpu, ref, range(8), TOL[dtype], f"bwd on oracle fwd {dtype} w{window}",
                            terms=sink_terms(inp, ref), roundoff=1e-6 if dtype == "fp32" else 0.0)


def test_backward_on_the_oracle_forward_4k_group0(gpu_lib):
    inp = make_inputs(WORKLOADS["gptoss_4k"])
    print("[case] backward on the oracle's forward, gptoss_4k group 0", flush=True)
    gpu, ref = _bwd_on_oracle_forward(gpu_lib, inp, heads=range(8))
    for key in ("dk", "dv"):
        ref[key][:, 1:] = np.nan
    compare(gpu, ref, ("dq", "dk", "dv", "dsinks"), TOL["bf16"], "bwd on oracle fwd gptoss_4k group 0")
    compare_dsinks_per_head(gpu, ref, range(8), TOL["bf16"], "bwd on oracle fwd gptoss_4k group 0",
                            terms=sink_terms(inp, ref))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("window", [0, 50])
def test_rows_past_a_sequence_are_never_read(gpu_lib, dtype, window):
    """Tiles that straddle a sequence's end must see zeros, not the rows that follow it
    in memory: with the next sequence's Q, K, V and dO set to NaN, the first
    sequence's O, LSE and dQ equal those of a call on it alone, bitwise, and its dK and
    dV agree to the rounding of the head-split partials (the split count depends on
    the batch); a masked product 0 x NaN would otherwise poison them."""
    n0, n1 = 100, 77  # the first sequence ends inside a 64- and a 128-row tile
    inp = random_case([n0, n1], 8, 2, 64, dtype, seed=41 + window, window=window)
    for key in ("q", "k", "v", "dout"):
        inp[key][n0:] = float("nan")
    print(f"[case] rows past a sequence {dtype} w{window}", flush=True)
    both = gpu_fwd_bwd(gpu_lib, inp)
    one = dict(inp, q=inp["q"][:n0], k=inp["k"][:n0], v=inp["v"][:n0], dout=inp["dout"][:n0],
               cu_seqlens=torch.tensor([0, n0], dtype=torch.int32), max_seqlen=n0)
    alone = gpu_fwd_bwd(gpu_lib, one)
    assert np.all(np.isfinite(alone["o"])) and np.all(np.isfinite(alone["dk"]))
    assert np.array_equal(both["o"][:n0], alone["o"])
    assert np.array_equal(both["lse"][:, :n0], alone["lse"])
    assert np.array_equal(both["dq"][:n0], alone["dq"])
    for key in ("dk", "dv"):
        assert np.all(np.isfinite(both[key][:n0])), key
        err = np.max(np.abs(both[key][:n0] - alone[key])) / np.max(np.abs(alone[key]))
        assert err <= TOL[dtype], (key, err)
