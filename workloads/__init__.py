"""Seeded synthetic inputs for sink attention, shared by the tests, the benchmark and smoke.

This module holds no part of the attention arithmetic: it only draws random
tensors (and rounds them once to the storage dtype), so both the HIP path and
the CPU oracle can be fed the very same values.

The shapes follow the GPT-OSS layer shape (64 query heads, 8 KV heads, head
dim 64, sliding window 128) and the sequence lengths the pages describe for
agentic RL rollouts (responses up to 16k tokens after a prompt); the pages run
RL benchmarks that are not reproduced here, so these synthetic tensors stand in
for them.

Draw order for one layer: q, k, v, sinks, dout (all float32 from one
``torch.Generator('cpu')``), then each is rounded to the storage dtype.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple            # per-sequence lengths (N_q = N_k)
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    dtype: str                # "bf16" or "fp32"
    seed: int
    layers: tuple             # ((causal, window, sink_dist), ...); one attention call each
    softmax_scale: float = 0.125

    @property
    def total(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> List[int]:
        return [0] + list(np.cumsum(self.seqlens).astype(int).tolist())


def varlen_lengths(seed: int = 0, n: int = 8, low: int = 1024, high: int = 16384) -> tuple:
    """Lengths of the packed batch: uniform integers in [low, high] from numpy's default_rng."""
    return tuple(int(x) for x in np.random.default_rng(seed).integers(low, high, size=n, endpoint=True))


# sink distributions: ("normal",) N(0,1); ("uniform", a, b) U[a, b]
WORKLOADS = {
    "tiny": Workload("tiny", (64,), 2, 1, 64, "fp32", 0, ((True, 0, ("normal",)),)),
    "gptoss_4k": Workload("gptoss_4k", (4096,), 64, 8, 64, "bf16", 1, ((True, 0, ("normal",)),)),
    "window_16k": Workload("window_16k", (16384,), 64, 8, 64, "bf16", 2,
                           ((True, 128, ("uniform", -2.0, 4.0)),)),
    "varlen": Workload("varlen", varlen_lengths(0), 64, 8, 64, "bf16", 3,
                       ((True, 0, ("normal",)), (True, 128, ("normal",)))),
    "long_20k": Workload("long_20k", (20480,), 64, 8, 64, "bf16", 4,
                         ((True, 0, ("uniform", -2.0, 8.0)),)),
    # head dim 128 at the same width (32 query heads x 128 = 64 x 64), 4k causal
    "d128_4k": Workload("d128_4k", (4096,), 32, 8, 128, "bf16", 7, ((True, 0, ("normal",)),),
                        softmax_scale=128 ** -0.5),
}


def _draw_sinks(gen: torch.Generator, n: int, dist) -> torch.Tensor:
    if dist[0] == "normal":
        return torch.randn(n, generator=gen, dtype=torch.float32)
    if dist[0] == "uniform":
        a, b = dist[1], dist[2]
        return torch.rand(n, generator=gen, dtype=torch.float32) * (b - a) + a
    raise ValueError(dist)


def make_inputs(w: Workload, layer: int = 0, seed: Optional[int] = None,
                with_dout: bool = True) -> dict:
    """Host tensors for one layer call of workload `w`.

    q [T, Hq, d], k/v [T, Hkv, d], dout [T, Hq, d] in the storage dtype; sinks
    [Hq] float32.  Every layer of a workload shares q/k/v/dout and gets its own
    sink vector (drawn in layer order after dout).
    """
    gen = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    t, hq, hkv, d = w.total, w.num_heads_q, w.num_heads_kv, w.head_dim
    q = torch.randn(t, hq, d, generator=gen, dtype=torch.float32)
    k = torch.randn(t, hkv, d, generator=gen, dtype=torch.float32)
    v = torch.randn(t, hkv, d, generator=gen, dtype=torch.float32)
    sinks = [_draw_sinks(gen, hq, lay[2]) for lay in w.layers]
    dout = torch.randn(t, hq, d, generator=gen, dtype=torch.float32) if with_dout else None
    store = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    causal, window, _ = w.layers[layer]
    return dict(q=q.to(store), k=k.to(store), v=v.to(store),
                dout=None if dout is None else dout.to(store),
                sinks=sinks[layer].contiguous(),
                cu_seqlens=torch.tensor(w.cu_seqlens, dtype=torch.int32),
                causal=causal, window=window, softmax_scale=w.softmax_scale,
                max_seqlen=int(max(w.seqlens)) if len(w.seqlens) else 0)


def random_case(seqlens, hq, hkv, d=64, dtype="bf16", seed=0, causal=True, window=0,
                sink_dist=("normal",), scale=None) -> dict:
    """Small ad-hoc case (tests): same draw order as make_inputs."""
    w = Workload("case", tuple(seqlens), hq, hkv, d, dtype, seed, ((causal, window, sink_dist),),
                 softmax_scale=(1.0 / np.sqrt(d)) if scale is None else scale)
    return make_inputs(w)


# ----------------------------------------------------------------------------- decoding steps
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decoding step of a rollout batch: each sequence brings `new_rows` query
    rows and attends to its whole KV cache (the cache includes the new rows' keys,
    which sit at its end)."""
    name: str
    cache_lens: tuple         # keys per sequence
    new_rows: int             # query rows per sequence
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    dtype: str
    seed: int
    layers: tuple             # ((causal, window, sink_dist), ...)
    softmax_scale: float = 0.125


# A rollout batch mid-generation: 64 sequences whose caches hold prompt + response
# so far (uniform in [1024, 16384], the same range as the packed training batch),
# one new token each; GPT-OSS alternates full and 128-key sliding-window layers.
DECODE_WORKLOADS = {
    "decode_rollout": DecodeWorkload("decode_rollout", varlen_lengths(5, n=64), 1, 64, 8, 64, "bf16", 6,
                                     ((True, 0, ("normal",)), (True, 128, ("normal",)))),
}


def make_decode_inputs(w: DecodeWorkload, layer: int = 0, seed: Optional[int] = None,
                       new_rows=None) -> dict:
    """Host tensors for one layer call of a decoding step.  Draw order: q, k, v,
    then one sink vector per layer (float32 from one torch.Generator('cpu')).
    `new_rows` (one count per sequence) overrides w.new_rows."""
    gen = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    nb = len(w.cache_lens)
    rows = [w.new_rows] * nb if new_rows is None else list(new_rows)
    tq, tk, hq, hkv, d = int(sum(rows)), int(sum(w.cache_lens)), w.num_heads_q, w.num_heads_kv, w.head_dim
    q = torch.randn(tq, hq, d, generator=gen, dtype=torch.float32)
    k = torch.randn(tk, hkv, d, generator=gen, dtype=torch.float32)
    v = torch.randn(tk, hkv, d, generator=gen, dtype=torch.float32)
    sinks = [_draw_sinks(gen, hq, lay[2]) for lay in w.layers]
    store = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    causal, window, _ = w.layers[layer]
    return dict(q=q.to(store), k=k.to(store), v=v.to(store), sinks=sinks[layer].contiguous(),
                cu_seqlens_q=torch.tensor([0] + np.cumsum(rows).astype(int).tolist(), dtype=torch.int32),
                cu_seqlens_k=torch.tensor([0] + np.cumsum(w.cache_lens).astype(int).tolist(), dtype=torch.int32),
                causal=causal, window=window, softmax_scale=w.softmax_scale,
                max_seqlen_q=int(max(rows)) if rows else 0,
                max_seqlen_k=int(max(w.cache_lens)) if nb else 0)


def decode_case(cache_lens, new_rows, hq, hkv, d=64, dtype="bf16", seed=0, causal=True, window=0,
                sink_dist=("normal",), scale=0.125) -> dict:
    """Small ad-hoc decoding step (tests); `new_rows` is an int or one count per sequence."""
    rows = [new_rows] * len(cache_lens) if isinstance(new_rows, int) else list(new_rows)
    w = DecodeWorkload("case", tuple(cache_lens), max(rows) if rows else 0, hq, hkv, d, dtype, seed,
                       ((causal, window, sink_dist),), softmax_scale=scale)
    return make_decode_inputs(w, new_rows=rows)
