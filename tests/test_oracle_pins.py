"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties the oracle to something fixed outside it: a hand-derived worked
example, a library routine (torch SDPA, scipy logsumexp, torch autograd), a
closed form, an invariant the pages state, or finite differences.  The last
block plants mistakes in a copy of the oracle and checks that a pin catches
each one.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import sink_attention as sa
from workloads import WORKLOADS, random_case, varlen_lengths

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _fwd(q, k, v, s, cu, scale, causal=True, window=0):
    return oracle.sink_attention_forward(q, k, v, s, cu, cu, scale, causal, window)


def _bwd(q, k, v, s, do, cu, scale, causal=True, window=0):
    return oracle.sink_attention_backward(q, k, v, s, do, cu, cu, scale, causal, window)


# ---------------------------------------------------------------- worked example
def _ev(x):
    """Evaluate a fixture entry: a float or an expression of rationals times ln2/ln3/ln4/ln6/ln8."""
    if not isinstance(x, str):
        return float(x)
    total = 0.0
    for term in x.replace("-", "+-").split("+"):
        term = term.strip()
        if not term:
            continue
        coef, _, log = term.partition("*") if "*" in term else (term, "", "")
        if coef.startswith("ln") or coef.startswith("-ln"):
            coef, log = ("-1" if coef.startswith("-") else "1"), coef.lstrip("-")
        val = float(Fraction(coef))
        if log:
            val *= math.log(int(log[2:]))
        total += val
    return total


def _evarr(a):
    return np.array([[_ev(x) for x in row] for row in a]) if isinstance(a[0], list) else np.array([_ev(x) for x in a])


@pytest.fixture(scope="module")
def golden():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


def test_golden_worked_example_causal(golden):
    inp, exp = golden["inputs"], golden["expected_causal"]
    q = _evarr(inp["q"])[:, None, :]
    k = _evarr(inp["k"])[:, None, :]
    v = _evarr(inp["v"])[:, None, :]
    do = _evarr(inp["dout"])[:, None, :]
    s = np.array([_ev(inp["sink"])])
    cu = [0, 2]
    o, lse = _fwd(q, k, v, s, cu, inp["softmax_scale"], True, 0)
    np.testing.assert_allclose(o[:, 0], _evarr(exp["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], _evarr(exp["lse"]), rtol=0, atol=1e-12)
    g = _bwd(q, k, v, s, do, cu, inp["softmax_scale"], True, 0)
    np.testing.assert_allclose(g["dq"][:, 0], _evarr(exp["dq"]), atol=1e-12)
    np.testing.assert_allclose(g["dk"][:, 0], _evarr(exp["dk"]), atol=1e-12)
    np.testing.assert_allclose(g["dv"][:, 0], _evarr(exp["dv"]), atol=1e-12)
    np.testing.assert_allclose(g["dsinks"], [exp["dsink"]], atol=1e-12)


def test_golden_worked_example_window(golden):
    inp, exp = golden["inputs"], golden["expected_window1"]
    q = _evarr(inp["q"])[:, None, :]
    k = _evarr(inp["k"])[:, None, :]
    v = _evarr(inp["v"])[:, None, :]
    s = np.array([_ev(inp["sink"])])
    o, lse = _fwd(q, k, v, s, [0, 2], 1.0, True, 1)
    np.testing.assert_allclose(o[:, 0], _evarr(exp["o"]), atol=1e-12)
    np.testing.assert_allclose(lse[0], _evarr(exp["lse"]), atol=1e-12)


# ---------------------------------------------------------------- invariants / closed forms
MASKS = [(True, 0), (True, 3), (False, 0), (False, 4)]


@pytest.mark.parametrize("causal,window", MASKS)
def test_probabilities_plus_sink_sum_to_one(causal, window):
    """With V = identity the output row is the content probabilities, so
    sum_j P_ij + P_sink_i = 1 can be read from the public outputs."""
    rng = np.random.default_rng(1)
    n, hq, hkv = 9, 4, 2
    d = n
    q, k = _rand(rng, n, hq, d), _rand(rng, n, hkv, d)
    v = np.broadcast_to(np.eye(n)[:, None, :], (n, hkv, n)).copy()
    sinks = rng.standard_normal(hq) * 2
    o, lse = _fwd(q, k, v, sinks, [0, n], 0.3, causal, window)
    total = o.sum(axis=2).T + np.exp(sinks[:, None] - lse)
    np.testing.assert_allclose(total, 1.0, atol=1e-13)


def _masked_scores(q, k, scale, causal, window):
    n_q, n_k = q.shape[0], k.shape[0]
    s = scale * q @ k.T
    vis = np.ones((n_q, n_k), bool)
    for i in range(n_q):
        for j in range(n_k):
            ii = i + n_k - n_q
            if causal and j > ii:
                vis[i, j] = False
            if window > 0 and j <= ii - window:
                vis[i, j] = False
    return s, vis


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 5), (False, 0)])
def test_minus_inf_sink_is_standard_attention(causal, window):
    """S_h = -inf removes the sink: torch's scaled_dot_product_attention (fp64, CPU)."""
    rng = np.random.default_rng(2)
    n, hq, hkv, d, scale = 17, 4, 2, 8, 0.35
    q, k, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    sinks = np.full(hq, -np.inf)
    o, lse = _fwd(q, k, v, sinks, [0, n], scale, causal, window)
    for h in range(hq):
        g = h // (hq // hkv)
        s, vis = _masked_scores(q[:, h], k[:, g], scale, causal, window)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[:, h])[None], torch.tensor(k[:, g])[None], torch.tensor(v[:, g])[None],
            attn_mask=torch.tensor(vis)[None], scale=scale)[0].numpy()
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)
        np.testing.assert_allclose(lse[h], logsumexp(np.where(vis, s, -np.inf), axis=1), atol=1e-12)
    # a very negative finite sink is the same to double precision
    o2, _ = _fwd(q, k, v, np.full(hq, -60.0), [0, n], scale, causal, window)
    np.testing.assert_allclose(o2, o, atol=1e-12)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 4), (False, 0)])
def test_closed_form_against_standard_attention(causal, window):
    """Appending one column to the softmax: LSE = logaddexp(LSE_std, S_h) and
    O = O_std * sigmoid(LSE_std - S_h), with O_std from torch SDPA."""
    rng = np.random.default_rng(3)
    n, hq, hkv, d, scale = 13, 2, 1, 6, 0.5
    q, k, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    sinks = rng.uniform(-2, 4, hq)
    o, lse = _fwd(q, k, v, sinks, [0, n], scale, causal, window)
    for h in range(hq):
        s, vis = _masked_scores(q[:, h], k[:, 0], scale, causal, window)
        lse_std = logsumexp(np.where(vis, s, -np.inf), axis=1)
        o_std = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[:, h])[None], torch.tensor(k[:, 0])[None], torch.tensor(v[:, 0])[None],
            attn_mask=torch.tensor(vis)[None], scale=scale)[0].numpy()
        np.testing.assert_allclose(lse[h], np.logaddexp(lse_std, sinks[h]), atol=1e-12)
        sig = 1.0 / (1.0 + np.exp(-(lse_std - sinks[h])))
        np.testing.assert_allclose(o[:, h], o_std * sig[:, None], atol=1e-12)


def test_sink_never_multiplies_v():
    """Constant V rows c: O_i = (1 - P_sink_i) c."""
    rng = np.random.default_rng(4)
    n, d = 11, 5
    q, k = _rand(rng, n, 2, d), _rand(rng, n, 1, d)
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (n, 1, d)).copy()
    sinks = np.array([0.7, -1.3])
    o, lse = _fwd(q, k, v, sinks, [0, n], 0.4)
    p_sink = np.exp(sinks[:, None] - lse)
    np.testing.assert_allclose(o, ((1 - p_sink).T)[:, :, None] * c, atol=1e-13)


def test_single_key_row():
    """Causal row 0 sees one key: O_0 = sigmoid(s_00 - S_h) v_0, LSE_0 = logaddexp(s_00, S_h)."""
    rng = np.random.default_rng(5)
    n, d, scale = 6, 7, 0.6
    q, k, v = _rand(rng, n, 1, d), _rand(rng, n, 1, d), _rand(rng, n, 1, d)
    sink = np.array([1.1])
    o, lse = _fwd(q, k, v, sink, [0, n], scale)
    s00 = scale * float(np.dot(q[0, 0], k[0, 0]))
    np.testing.assert_allclose(o[0, 0], v[0, 0] / (1 + math.exp(sink[0] - s00)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.logaddexp(s00, sink[0]), atol=1e-14)


def test_window_one_is_a_single_key_per_row():
    """Window 1 (causal): every row sees its own key only, so with p_i = sigmoid(s_ii - S_h)
    the forward is O_i = p_i v_i, LSE_i = logaddexp(s_ii, S_h), and the chain rule through
    the two-entry softmax [s_ii, S_h] gives dS_ii = p_i (1 - p_i) <dO_i, v_i>,
    dq_i = scale dS_ii k_i, dk_i = scale sum_h dS_ii q_i (over the kv head's query heads),
    dv_i = sum_h p_i dO_i and dS_h = -sum_i (1 - p_i) p_i <dO_i, v_i>."""
    rng = np.random.default_rng(17)
    lens, hq, hkv, d, scale = [5, 3], 4, 2, 6, 0.4
    n, g = sum(lens), hq // hkv
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d), _rand(rng, n, hq, d)
    sinks = rng.standard_normal(hq)
    r = _bwd(q, k, v, sinks, do, cu, scale, True, 1)
    kh, vh = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)  # [n, hq, d]
    s = scale * np.einsum("nhd,nhd->nh", q, kh)
    p = 1.0 / (1.0 + np.exp(sinks[None, :] - s))
    dp = np.einsum("nhd,nhd->nh", do, vh)
    ds = p * (1 - p) * dp
    np.testing.assert_allclose(r["o"], p[..., None] * vh, atol=1e-13)
    np.testing.assert_allclose(r["lse"], np.logaddexp(s, sinks[None, :]).T, atol=1e-13)
    np.testing.assert_allclose(r["dq"], scale * ds[..., None] * kh, atol=1e-13)
    dk = (scale * ds[..., None] * q).reshape(n, hkv, g, d).sum(2)
    dv = (p[..., None] * do).reshape(n, hkv, g, d).sum(2)
    np.testing.assert_allclose(r["dk"], dk, atol=1e-13)
    np.testing.assert_allclose(r["dv"], dv, atol=1e-13)
    np.testing.assert_allclose(r["dsinks"], -((1 - p) * p * dp).sum(0), atol=1e-13)


def test_empty_row_and_empty_sequence():
    """A sequence of length 0 writes nothing; a row with no visible key (N_q > N_k,
    causal) has O = 0 and LSE = S_h; with S_h = -inf it has LSE = -inf."""
    rng = np.random.default_rng(6)
    d = 4
    q, k, v = _rand(rng, 5, 1, d), _rand(rng, 3, 1, d), _rand(rng, 3, 1, d)
    cu_q, cu_k = [0, 0, 5], [0, 0, 3]
    o, lse = oracle.sink_attention_forward(q, k, v, np.array([0.5]), cu_q, cu_k, 1.0, True, 0)
    # n_q = 5, n_k = 3, bottom-right: rows 0, 1 see no key
    np.testing.assert_allclose(o[:2, 0], 0.0)
    np.testing.assert_allclose(lse[0, :2], 0.5)
    assert np.all(np.isfinite(o[2:]))
    o, lse = oracle.sink_attention_forward(q, k, v, np.array([-np.inf]), cu_q, cu_k, 1.0, True, 0)
    np.testing.assert_allclose(o[:2, 0], 0.0)
    assert np.all(lse[0, :2] == -np.inf)
    g = oracle.sink_attention_backward(q, k, v, np.array([-np.inf]), q, cu_q, cu_k, 1.0, True, 0)
    assert np.all(np.isfinite(g["dq"])) and np.isfinite(g["dsinks"][0])
    np.testing.assert_allclose(g["dq"][:2], 0.0)


# ---------------------------------------------------------------- backward
def _loss(q, k, v, s, do, cu, scale, causal, window):
    o, _ = _fwd(q, k, v, s, cu, scale, causal, window)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 3), (False, 0)])
def test_backward_matches_central_differences(causal, window):
    rng = np.random.default_rng(7)
    n, hq, hkv, d, scale = 6, 2, 1, 4, 0.7
    q, k, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    do = _rand(rng, n, hq, d)
    sinks = np.array([0.3, -0.8])
    cu = [0, n]
    g = _bwd(q, k, v, sinks, do, cu, scale, causal, window)
    eps = 1e-6
    for name, x, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"]), ("s", sinks, g["dsinks"])):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, sinks, do, cu, scale, causal, window)
            x[idx] = old - eps
            lm = _loss(q, k, v, sinks, do, cu, scale, causal, window)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - grad)) / np.max(np.abs(fd))
        assert err < 1e-6, (name, err)


def test_literal_sink_gradient_reading_disagrees_with_finite_differences():
    """The printed sink-gradient equation has dL/dS_ij as its inner factor; read
    literally (the score gradient dS_ij) it does not match the true derivative,
    read with dL/dP_ij it does.  Documents the reading the oracle takes."""
    rng = np.random.default_rng(8)
    n, d, scale = 5, 3, 1.0
    q, k, v, do = _rand(rng, n, 1, d), _rand(rng, n, 1, d), _rand(rng, n, 1, d), _rand(rng, n, 1, d)
    s = np.array([0.2])
    cu = [0, n]
    eps = 1e-6
    fd = (_loss(q, k, v, s + eps, do, cu, scale, True, 0) - _loss(q, k, v, s - eps, do, cu, scale, True, 0)) / (2 * eps)
    g = _bwd(q, k, v, s, do, cu, scale, True, 0)
    assert abs(g["dsinks"][0] - fd) < 1e-7
    # literal reading: -sum_i P_sink_i sum_j P_ij dS_ij
    o, lse = _fwd(q, k, v, s, cu, scale)
    sc, vis = _masked_scores(q[:, 0], k[:, 0], scale, True, 0)
    p = np.where(vis, np.exp(sc - lse[0][:, None]), 0.0)
    dp = do[:, 0] @ v[:, 0].T
    dd = np.sum(do[:, 0] * o[:, 0], axis=1)
    ds = p * (dp - dd[:, None])
    literal = -np.sum(np.exp(s[0] - lse[0]) * np.sum(p * ds, axis=1))
    assert abs(literal - fd) > 1e-3


def test_autograd_through_concat_softmax_slice():
    """torch autograd (fp64) through the pages' pseudo-code: append the sink column,
    softmax over N_k+1, drop the last column, multiply by V."""
    rng = np.random.default_rng(9)
    n, hq, hkv, d, scale = 10, 4, 2, 6, 0.45
    window = 4
    q, k, v, do = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d), _rand(rng, n, hq, d)
    sinks = rng.standard_normal(hq)
    tq, tk, tv, ts = (torch.tensor(x, requires_grad=True) for x in (q, k, v, sinks))
    outs = []
    for h in range(hq):
        g = h // (hq // hkv)
        scores = tq[:, h] @ tk[:, g].T * scale
        _, vis = _masked_scores(q[:, h], k[:, g], scale, True, window)
        scores = scores.masked_fill(~torch.tensor(vis), float("-inf"))
        combined = torch.cat([scores, ts[h].expand(n, 1)], dim=-1)
        probs = torch.softmax(combined, dim=-1)
        outs.append(probs[:, :-1] @ tv[:, g])
    out = torch.stack(outs, dim=1)
    (out * torch.tensor(do)).sum().backward()
    g = _bwd(q, k, v, sinks, do, [0, n], scale, True, window)
    np.testing.assert_allclose(g["o"], out.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dsinks"], ts.grad.numpy(), atol=1e-12)


def test_constant_keys_tie_dq_to_sink_gradient():
    """All keys equal to c: sum_j dS_ij = P_sink_i D_i, so sum_i dq_i = -scale * dsink * c."""
    rng = np.random.default_rng(10)
    n, d, scale = 12, 5, 0.8
    c = rng.standard_normal(d)
    q, v, do = _rand(rng, n, 1, d), _rand(rng, n, 1, d), _rand(rng, n, 1, d)
    k = np.broadcast_to(c, (n, 1, d)).copy()
    g = _bwd(q, k, v, np.array([0.4]), do, [0, n], scale, True, 0)
    np.testing.assert_allclose(g["dq"][:, 0].sum(axis=0), -scale * g["dsinks"][0] * c, atol=1e-12)


# ---------------------------------------------------------------- structure: GQA, varlen, window
def test_gqa_equals_duplicated_kv():
    rng = np.random.default_rng(11)
    n, hq, hkv, d = 9, 6, 2, 4
    q, k, v, do = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d), _rand(rng, n, hq, d)
    sinks = rng.standard_normal(hq)
    kd, vd = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
    g1 = _bwd(q, k, v, sinks, do, [0, n], 0.5, True, 3)
    g2 = _bwd(q, kd, vd, sinks, do, [0, n], 0.5, True, 3)
    np.testing.assert_allclose(g1["o"], g2["o"], atol=1e-13)
    np.testing.assert_allclose(g1["dq"], g2["dq"], atol=1e-13)
    np.testing.assert_allclose(g1["dsinks"], g2["dsinks"], atol=1e-13)
    np.testing.assert_allclose(g1["dk"], g2["dk"].reshape(n, hkv, hq // hkv, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(g1["dv"], g2["dv"].reshape(n, hkv, hq // hkv, d).sum(2), atol=1e-13)


def test_varlen_equals_separate_calls():
    rng = np.random.default_rng(12)
    lens = [5, 0, 9, 1, 7]
    t, hq, hkv, d = sum(lens), 4, 2, 3
    q, k, v, do = _rand(rng, t, hq, d), _rand(rng, t, hkv, d), _rand(rng, t, hkv, d), _rand(rng, t, hq, d)
    sinks = rng.standard_normal(hq)
    cu = [0] + list(np.cumsum(lens))
    g = _bwd(q, k, v, sinks, do, cu, 0.6, True, 4)
    ds = np.zeros(hq)
    for b in range(len(lens)):
        a, e = cu[b], cu[b + 1]
        gb = _bwd(q[a:e], k[a:e], v[a:e], sinks, do[a:e], [0, e - a], 0.6, True, 4)
        for key in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(g[key][a:e], gb[key], atol=1e-13)
        np.testing.assert_allclose(g["lse"][:, a:e], gb["lse"], atol=1e-13)
        ds += gb["dsinks"]
    np.testing.assert_allclose(g["dsinks"], ds, atol=1e-13)


def test_window_at_least_n_is_full_causal():
    rng = np.random.default_rng(13)
    n = 14
    q, k, v, do = _rand(rng, n, 2, 3), _rand(rng, n, 1, 3), _rand(rng, n, 1, 3), _rand(rng, n, 2, 3)
    s = rng.standard_normal(2)
    a = _bwd(q, k, v, s, do, [0, n], 0.5, True, 0)
    b = _bwd(q, k, v, s, do, [0, n], 0.5, True, n)
    for key in ("o", "lse", "dq", "dk", "dv", "dsinks"):
        np.testing.assert_allclose(a[key], b[key], atol=0)


def test_row_blocking_does_not_change_results(monkeypatch):
    rng = np.random.default_rng(14)
    n = 40
    q, k, v, do = _rand(rng, n, 2, 3), _rand(rng, n, 1, 3), _rand(rng, n, 1, 3), _rand(rng, n, 2, 3)
    s = rng.standard_normal(2)
    ref = _bwd(q, k, v, s, do, [0, n], 0.5, True, 7)
    monkeypatch.setattr(sa, "ROW_BLOCK", 3)
    got = _bwd(q, k, v, s, do, [0, n], 0.5, True, 7)
    for key in ("o", "lse", "dq", "dk", "dv", "dsinks"):
        np.testing.assert_allclose(got[key], ref[key], atol=1e-13)


def test_sampled_backward_keeps_full_values():
    rng = np.random.default_rng(15)
    n = 20
    q, k, v, do = _rand(rng, n, 4, 3), _rand(rng, n, 2, 3), _rand(rng, n, 2, 3), _rand(rng, n, 4, 3)
    s = rng.standard_normal(4)
    full = _bwd(q, k, v, s, do, [0, n], 0.5, True, 0)
    part = oracle.sink_attention_backward(q, k, v, s, do, [0, n], [0, n], 0.5, True, 0,
                                          heads=[2, 3], q_rows=[0, 7, 19])
    rows = [0, 7, 19]
    np.testing.assert_allclose(part["dq"][rows][:, 2:], full["dq"][rows][:, 2:], atol=1e-13)
    np.testing.assert_allclose(part["o"][rows][:, 2:], full["o"][rows][:, 2:], atol=1e-13)
    np.testing.assert_allclose(part["lse"][2:, rows], full["lse"][2:, rows], atol=1e-13)
    assert np.all(np.isnan(part["dq"][1])) and np.all(np.isnan(part["dsinks"]))
    assert np.all(np.isnan(part["dk"]))
    part = oracle.sink_attention_backward(q, k, v, s, do, [0, n], [0, n], 0.5, True, 0,
                                          heads=[2, 3], k_rows=[1, 18])
    np.testing.assert_allclose(part["dk"][[1, 18], 1], full["dk"][[1, 18], 1], atol=1e-13)
    np.testing.assert_allclose(part["dv"][[1, 18], 1], full["dv"][[1, 18], 1], atol=1e-13)
    np.testing.assert_allclose(part["dsinks"][2:], full["dsinks"][2:], atol=1e-13)
    assert np.all(np.isnan(part["dk"][2])) and np.all(np.isnan(part["dsinks"][:2]))
    o, lse = oracle.sink_attention_forward(q, k, v, s, [0, n], [0, n], 0.5, True, 0, heads=[1], q_rows=rows)
    np.testing.assert_allclose(o[rows, 1], full["o"][rows, 1], atol=1e-13)
    np.testing.assert_allclose(lse[1, rows], full["lse"][1, rows], atol=1e-13)


@pytest.mark.parametrize("n,causal,window", [(1, True, 0), (37, True, 0), (37, True, 5), (37, False, 0), (37, False, 6)])
def test_visible_pairs_brute_force(n, causal, window):
    _, vis = _masked_scores(np.zeros((n, 1)), np.zeros((n, 1)), 1.0, causal, window)
    assert oracle.visible_pairs([0, n], [0, n], causal, window) == int(vis.sum())


def test_visible_pairs_closed_forms():
    assert oracle.visible_pairs([0, 4096], [0, 4096], True, 0) == 4096 * 4097 // 2
    assert oracle.visible_pairs([0, 16384], [0, 16384], True, 128) == sum(min(i + 1, 128) for i in range(16384))


def test_workload_table():
    assert varlen_lengths(0) == (14090, 10808, 8875, 5168, 5752, 1653, 2179, 1277)
    assert WORKLOADS["varlen"].total == 49802
    inp = random_case([5, 3], 4, 2, 8, "bf16", seed=1)
    assert inp["q"].dtype == torch.bfloat16 and inp["q"].shape == (8, 4, 8)
    assert inp["cu_seqlens"].tolist() == [0, 5, 8]


# ---------------------------------------------------------------- planted mistakes
# Each mutation plants one plausible mistake in a private copy of the oracle's
# source; at least one pin above must then fail.
MUTATIONS = [
    ("sink dropped from the normaliser", "+ np.exp(sink - m0)", "+ 0.0 * np.exp(sink - m0)"),
    ("sink scaled like a score", "m = np.maximum(s.max(axis=1, initial=-np.inf), sink)",
     "sink = 0.5 * sink\n    m = np.maximum(s.max(axis=1, initial=-np.inf), sink)"),
    ("interleaved GQA map", "g = h // group", "g = h % hkv"),
    ("sink gradient sign", "dsinks[h] += -np.sum", "dsinks[h] += np.sum"),
    ("causal mask off by one", "vis &= j <= i", "vis &= j < i"),
    ("window mask off by one", "vis &= j > i - window", "vis &= j >= i - window"),
    ("top-left instead of bottom-right alignment", "+ (n_k - n_q)", "+ 0 * (n_k - n_q)"),
    ("dropped D term in dS", "ds = p * (dp - dd[:, None])", "ds = p * dp"),
    ("dk without the softmax scale", "+= softmax_scale * (ds[:, keep].T @ qr)", "+= (ds[:, keep].T @ qr)"),
    ("dv from dS instead of P", "+= p[:, keep].T @ dor", "+= ds[:, keep].T @ dor"),
    ("wrong operand in dq", "softmax_scale * (ds @ kb)", "softmax_scale * (ds @ vb)"),
]


def _pins(golden_data):
    return [
        lambda: test_golden_worked_example_causal(golden_data),
        lambda: test_golden_worked_example_window(golden_data),
        lambda: [test_probabilities_plus_sink_sum_to_one(c, w) for c, w in MASKS],
        lambda: test_minus_inf_sink_is_standard_attention(True, 5),
        lambda: test_closed_form_against_standard_attention(True, 4),
        test_sink_never_multiplies_v,
        test_single_key_row,
        test_empty_row_and_empty_sequence,
        lambda: test_backward_matches_central_differences(True, 3),
        test_autograd_through_concat_softmax_slice,
        test_gqa_equals_duplicated_kv,
    ]


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(label, old, new, monkeypatch, golden):
    import types
    src = open(sa.__file__).read()
    assert src.count(old) >= 1, label
    mutant = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mutant.__dict__)
    monkeypatch.setattr(oracle, "sink_attention_forward", mutant.sink_attention_forward)
    monkeypatch.setattr(oracle, "sink_attention_backward", mutant.sink_attention_backward)
    caught = []
    for pin in _pins(golden):
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin)
    assert caught, f"no pin caught: {label}"
