"""Plain float64 CPU reference of attention with per-head learnable sinks.

TEST INFRASTRUCTURE ONLY: used by the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``; never by the library it checks.

Sources. The method is defined on these pages (cited by title and section):

* [Unlocking] "解锁 GPT-OSS 的 Agentic RL 训练：实用回顾" (Unlocking Agentic RL Training
  for GPT-OSS: a practical retrospective), euno.news, section "FlashAttention V3 中的
  注意力汇聚支持" (attention-sink support in FlashAttention V3), with the sub-sections
  标准注意力 (standard attention), 带汇聚的注意力 (attention with sinks), 数学公式
  (formulas) and 反向传播 (backward pass).  This page is the authority.
* [Treinamento] "Treinamento de RL Agêntico para modelos GPT-OSS: lições práticas do
  LinkedIn com MoE e FlashAttention", section "Desafio 3: Attention Sinks no
  FlashAttention": the same concat/softmax/slice description.
* [Keryc] keryc.com, "GPT-OSS enables agentic RL training: key fixes", section
  "2) Attention sinks": the sink joins the normaliser but never multiplies V.

What is computed, for every sequence b and query head h, with kv head
g = h // (Hq // Hkv) (GQA: the pages are silent; contiguous groups are taken):

    s_ij      = scale * <q_i, k_j>                         [Unlocking, 标准注意力]
    the per-head sink logit S_h joins each score row as one extra column, the
    softmax runs over the N_k + 1 entries, and the extra column is dropped before
    the product with V                                     [Unlocking, 带汇聚的注意力]
    P_ij      = exp(s_ij) / (sum_j' exp(s_ij') + exp(S_h))   [Unlocking, 数学公式, 1st eq.]
    P_sink_i  = exp(S_h)  / (same denominator)             [Unlocking, 数学公式, 2nd eq.]
    O_i       = sum_j P_ij v_j                             [Keryc, 2): sink not in output]
    LSE_i     = log(sum_j exp(s_ij) + exp(S_h))            (natural log, sink included)

Masks (the pages show none): key j is visible to query i when
(not causal or j <= i + off) and (window <= 0 or j > i + off - window), where
off = N_k - N_q aligns the last query with the last key.  Masked scores leave the
row before the sink is appended; the sink is visible to every row.

Backward (the pages give only the sink gradient; the rest is the chain rule
through the softmax over the combined row, whose sink column receives zero
upstream gradient because it is sliced off before the product with V):

    dP_ij = <dO_i, v_j>,   D_i = sum_j P_ij dP_ij  (= <dO_i, O_i>)
    dS_ij = P_ij (dP_ij - D_i)
    dq_i  = scale * sum_j dS_ij k_j
    dk_j  = scale * sum_{h in g} sum_i dS_ij q_i
    dv_j  = sum_{h in g} sum_i P_ij dO_i
    dS_h  = - sum_i P_sink_i D_i                           [Unlocking, 反向传播]

The printed sink-gradient equation names the inner factor as the derivative of
the loss with respect to the score; only the derivative with respect to the
probability (dP_ij) makes it the true gradient, so that is the reading taken
here.  Finite differences in the test suite pin it.

Degenerate rows: if S_h = -inf and no key is visible, the row has no mass at all;
this oracle returns O = 0, LSE = -inf, P_sink = 0 for it.

No blocking beyond splitting query rows into blocks (for memory); each block sees
the whole key range its rows can see, so the arithmetic is the definition above.
"""

from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def visible_mask(rows, cols, n_q: int, n_k: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: True where local query rows[a] sees local key cols[b]."""
    i = np.asarray(rows, dtype=np.int64)[:, None] + (n_k - n_q)
    j = np.asarray(cols, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= j > i - window
    return vis


def _key_range(r0: int, r1: int, n_q: int, n_k: int, causal: bool, window: int):
    """Half-open key range [lo, hi) that contains every key some row in [r0, r1) can see."""
    off = n_k - n_q
    lo, hi = 0, n_k
    if causal:
        hi = min(n_k, max(0, (r1 - 1) + off + 1))
    if window > 0:
        lo = max(0, min(n_k, r0 + off - window + 1))
    return lo, max(lo, hi)


def _sink_softmax(s: np.ndarray, vis: np.ndarray, sink: float):
    """Softmax of each row of `s` with the sink logit appended as one more column.

    Returns (P over the key columns, P_sink per row, LSE per row).  Columns with
    vis == False are excluded (probability 0).  [Unlocking, 数学公式]
    """
    s = np.where(vis, s, -np.inf)
    m = np.maximum(s.max(axis=1, initial=-np.inf), sink)      # max over the N_k+1 entries
    alive = np.isfinite(m)                                    # False only if sink = -inf and no key
    m0 = np.where(alive, m, 0.0)
    z = np.exp(s - m0[:, None]).sum(axis=1) + np.exp(sink - m0)
    lse = np.where(alive, m0 + np.log(np.where(alive, z, 1.0)), -np.inf)
    lse0 = np.where(alive, lse, 0.0)
    p = np.where(vis & alive[:, None], np.exp(s - lse0[:, None]), 0.0)
    p_sink = np.where(alive, np.exp(sink - lse0), 0.0)
    return p, p_sink, lse


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: upcast exactly (bf16/fp32 -> fp32 -> fp64)
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _seqs(cu_q, cu_k):
    cu_q = [int(x) for x in np.asarray(cu_q).ravel()]
    cu_k = [int(x) for x in np.asarray(cu_k).ravel()]
    assert len(cu_q) == len(cu_k) and len(cu_q) >= 1
    return [(cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]) for b in range(len(cu_q) - 1)]


def _row_blocks(rows):
    """Split a sorted array of local query rows into blocks of at most ROW_BLOCK rows."""
    return [rows[a:a + ROW_BLOCK] for a in range(0, len(rows), ROW_BLOCK)]


def _local_rows(sel, a, e):
    """Local row indices of sequence [a, e) kept by the global selection `sel` (None = all)."""
    if sel is None:
        return np.arange(e - a)
    sel = np.asarray(sel, dtype=np.int64)
    return np.sort(sel[(sel >= a) & (sel < e)]) - a


def sink_attention_forward(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, softmax_scale,
                           causal=True, window=0, heads=None, q_rows=None):
    """Forward of sink attention over a packed (varlen) batch.

    q [total_q, Hq, d], k/v [total_k, Hkv, d], sinks [Hq] (natural-log units, not
    multiplied by softmax_scale), cu_seqlens_* [num_seqs+1].
    Returns (o [total_q, Hq, d], lse [Hq, total_q]) in float64.  `heads` and
    `q_rows` (global query indices) restrict what is computed; the rest is NaN.
    Each kept row is computed against every key it can see.
    """
    q, k, v, sinks = _as64(q), _as64(k), _as64(v), _as64(sinks)
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    heads = range(hq) if heads is None else heads
    o = np.full((total_q, hq, v.shape[2]), np.nan)
    lse = np.full((hq, total_q), np.nan)
    for (q0, q1, k0, k1) in _seqs(cu_seqlens_q, cu_seqlens_k):
        n_q, n_k = q1 - q0, k1 - k0
        for h in heads:
            g = h // group
            sink = float(sinks[h])
            for rows in _row_blocks(_local_rows(q_rows, q0, q1)):
                lo, hi = _key_range(rows[0], rows[-1] + 1, n_q, n_k, causal, window)
                cols = np.arange(lo, hi)
                s = softmax_scale * (q[q0 + rows, h] @ k[k0 + lo:k0 + hi, g].T)   # Q K^T / sqrt(d)
                p, _, lse[h, q0 + rows] = _sink_softmax(
                    s, visible_mask(rows, cols, n_q, n_k, causal, window), sink)
                o[q0 + rows, h] = p @ v[k0 + lo:k0 + hi, g]                    # sink never multiplies V
    return o, lse


def sink_attention_backward(q, k, v, sinks, do, cu_seqlens_q, cu_seqlens_k, softmax_scale,
                            causal=True, window=0, heads=None, q_rows=None, k_rows=None):
    """Gradients of L = sum(dO * O) with respect to q, k, v and the sinks.

    The forward is recomputed here in float64 (nothing is taken from elsewhere).
    Each block of query rows sees its whole visible key range, so its softmax
    statistics, O, D and dS are complete within the block.

    Sampling, for large inputs, never changes a kept value:
      * `heads`: only these query heads; dk/dv then hold only their contributions.
      * `q_rows` (global query indices): only these rows are computed; o, lse and
        dq are kept for them, while dk, dv and dsinks (sums over all rows) are NaN.
      * `k_rows` (global key indices): dk/dv are kept only for these keys.
    Returns dict(dq, dk, dv, dsinks, o, lse), float64.
    """
    q, k, v, sinks, do = _as64(q), _as64(k), _as64(v), _as64(sinks), _as64(do)
    total_q, hq, d = q.shape
    total_k, hkv, _ = k.shape
    group = hq // hkv
    heads = list(range(hq)) if heads is None else list(heads)
    dq = np.full_like(q, np.nan)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = np.full(hq, np.nan)
    o = np.full_like(q, np.nan)
    lse = np.full((hq, total_q), np.nan)
    k_keep = np.ones(total_k, bool)
    if k_rows is not None:
        k_keep[:] = False
        k_keep[np.asarray(k_rows, dtype=np.int64)] = True
    for h in heads:
        dsinks[h] = 0.0
    for (q0, q1, k0, k1) in _seqs(cu_seqlens_q, cu_seqlens_k):
        n_q, n_k = q1 - q0, k1 - k0
        for h in heads:
            g = h // group
            sink = float(sinks[h])
            for rows in _row_blocks(_local_rows(q_rows, q0, q1)):
                lo, hi = _key_range(rows[0], rows[-1] + 1, n_q, n_k, causal, window)
                cols = np.arange(lo, hi)
                qr, dor = q[q0 + rows, h], do[q0 + rows, h]
                kb, vb = k[k0 + lo:k0 + hi, g], v[k0 + lo:k0 + hi, g]
                s = softmax_scale * (qr @ kb.T)
                p, p_sink, lse_r = _sink_softmax(s, visible_mask(rows, cols, n_q, n_k, causal, window), sink)
                o_r = p @ vb
                o[q0 + rows, h], lse[h, q0 + rows] = o_r, lse_r
                dd = np.einsum("id,id->i", dor, o_r)          # D_i = <dO_i, O_i>
                dsinks[h] += -np.sum(p_sink * dd)             # dS_h = -sum_i P_sink_i D_i
                dp = dor @ vb.T                               # dP_ij = <dO_i, v_j>
                ds = p * (dp - dd[:, None])                   # dS_ij = P_ij (dP_ij - D_i)
                dq[q0 + rows, h] = softmax_scale * (ds @ kb)
                keep = k_keep[k0 + lo:k0 + hi]
                if keep.any():
                    dk[k0 + lo:k0 + hi, g][keep] += softmax_scale * (ds[:, keep].T @ qr)
                    dv[k0 + lo:k0 + hi, g][keep] += p[:, keep].T @ dor
    if q_rows is not None:
        dk[:] = np.nan
        dv[:] = np.nan
        dsinks[:] = np.nan
    dk[~k_keep] = np.nan
    dv[~k_keep] = np.nan
    return dict(dq=dq, dk=dk, dv=dv, dsinks=dsinks, o=o, lse=lse)


def visible_pairs(cu_seqlens_q, cu_seqlens_k, causal=True, window=0) -> int:
    """Number of visible (query, key) pairs per query head, counted row by row."""
    total = 0
    for (q0, q1, k0, k1) in _seqs(cu_seqlens_q, cu_seqlens_k):
        n_q, n_k = q1 - q0, k1 - k0
        i = np.arange(n_q, dtype=np.int64) + (n_k - n_q)
        hi = np.minimum(n_k, i + 1) if causal else np.full(n_q, n_k)
        lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(n_q, np.int64)
        total += int(np.maximum(0, hi - np.minimum(hi, lo)).sum())
    return total
