"""Seeded synthetic inputs for the sparse decode step.

This module only draws inputs: key/value caches, context lengths and the
per-head query sequence.  It holds none of the method's arithmetic, and it is
the one module that both the HIP path's callers and the CPU oracle's callers
share.  Every draw comes from a ``torch.Generator`` seeded from
(seed, layer, tensor tag); the same call on the same device returns the same
bytes.  Generation on a GPU and on the CPU use different engines, so a test
that compares the two sides always hands the oracle the exact bytes the GPU
consumed.

Recipe (the pages run real Qwen3-8B / Qwen3-32B decoding on long
chain-of-thought benchmarks; those weights and datasets are not used, and
these draws stand in for them with the same shapes):
  * K, V ~ N(0, 1) per element, drawn in fp32; for each (sequence, KV head) a
    set of distinct "heavy" token positions, uniform over the sequence, has its
    K row (not V) multiplied by a factor; then rounded to bf16
    (round-to-nearest-even) or kept fp32.
  * queries follow an AR(1) process per (sequence, query head, coordinate):
    q_s = a * q_{s-1} + sigma * eps, q_0 ~ N(0, sigma^2 / (1 - a^2)).
  * ragged context lengths are uniform integers in a closed range.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_TAG_K, _TAG_V, _TAG_HEAVY, _TAG_Q, _TAG_LEN, _TAG_MISC = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    t_cap: int
    kv_dtype: str                      # "bf16" or "f32"
    window: int
    lam: float
    top_c: int
    heavy_count: Optional[int] = None  # fixed count per (sequence, KV head) ...
    heavy_frac: Optional[float] = None  # ... or a fraction of the sequence length
    heavy_factor: float = 3.0
    seq_len_range: Optional[Tuple[int, int]] = None  # ragged lengths, inclusive
    history_steps: int = 0             # queries drawn before the first decode step
    recent: int = 0                    # newest tokens attended beside the selection (asp_cfg.recent)
    ar_a: float = 0.9
    ar_sigma: float = 0.3
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny case that the oracle finishes in well under a second.
TINY = Workload("tiny", layers=1, batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, t_cap=512,
                kv_dtype="f32", window=8, lam=1e-2, top_c=64, heavy_count=8, heavy_factor=4.0,
                history_steps=64)
# One Qwen3-8B-shaped decoder layer at 32k context (GQA group 4).
Q8B_LAYER = Workload("qwen3-8b-layer", layers=1, batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     t_cap=32768, kv_dtype="bf16", window=16, lam=1e-2, top_c=2048,
                     heavy_frac=0.01, heavy_factor=3.0, history_steps=16)
# Qwen3-8B-shaped stack: 36 layers, batch 32, 16k context.
Q8B_STACK = Workload("qwen3-8b-stack", layers=36, batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     t_cap=16384, kv_dtype="bf16", window=16, lam=1e-2, top_c=2048,
                     heavy_frac=0.01, heavy_factor=3.0, history_steps=16)
# Qwen3-32B-shaped: 64 layers, batch 16, 64 query heads on 8 KV heads (group 8).
Q32B = Workload("qwen3-32b", layers=64, batch=16, n_q_heads=64, n_kv_heads=8, head_dim=128,
                t_cap=32768, kv_dtype="bf16", window=16, lam=1e-2, top_c=2048,
                heavy_frac=0.01, heavy_factor=3.0, history_steps=16)
# Long-CoT ragged stress: batch 64, lengths uniform in [8192, 131072].
RAGGED = Workload("ragged-long-cot", layers=1, batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                  t_cap=131072, kv_dtype="bf16", window=16, lam=1e-2, top_c=2048,
                  heavy_frac=0.01, heavy_factor=3.0, seq_len_range=(8192, 131072), history_steps=32)

CONFIGS = {w.name: w for w in (TINY, Q8B_LAYER, Q8B_STACK, Q32B, RAGGED)}


def _gen(device, seed: int, layer: int, tag: int, sub: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000003 + layer) * 131 + tag) * 1000033 + sub)
    return g


def torch_kv_dtype(wl: Workload) -> torch.dtype:
    return torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32


def make_seq_lens(wl: Workload, device="cpu") -> torch.Tensor:
    """Context length per sequence (int32, [B])."""
    if wl.seq_len_range is None:
        return torch.full((wl.batch,), wl.t_cap, dtype=torch.int32, device=device)
    lo, hi = wl.seq_len_range
    g = _gen("cpu", wl.seed, 0, _TAG_LEN)
    lens = torch.randint(lo, hi + 1, (wl.batch,), generator=g, dtype=torch.int64)
    return lens.to(torch.int32).to(device)


def heavy_count(wl: Workload, t: int) -> int:
    if wl.heavy_count is not None:
        return min(wl.heavy_count, t)
    if wl.heavy_frac is not None:
        return min(int(round(wl.heavy_frac * t)), t)
    return 0


def make_kv(wl: Workload, seq_lens: torch.Tensor, layer: int = 0, device="cpu"):
    """K and V caches [B][Hkv][T_cap][D] in the workload's dtype, on ``device``.

    Rows at or past a sequence's length are drawn too (they are never read by a
    correct implementation).  Generation runs one sequence at a time to bound
    the fp32 staging memory.
    """
    B, Hkv, T, D = wl.batch, wl.n_kv_heads, wl.t_cap, wl.head_dim
    dt = torch_kv_dtype(wl)
    k = torch.empty((B, Hkv, T, D), dtype=dt, device=device)
    v = torch.empty((B, Hkv, T, D), dtype=dt, device=device)
    lens = seq_lens.to("cpu").tolist()
    for b in range(B):
        gk = _gen(device, wl.seed, layer, _TAG_K, b)
        gv = _gen(device, wl.seed, layer, _TAG_V, b)
        kb = torch.randn((Hkv, T, D), generator=gk, dtype=torch.float32, device=device)
        vb = torch.randn((Hkv, T, D), generator=gv, dtype=torch.float32, device=device)
        tb = int(lens[b])
        nh = heavy_count(wl, tb)
        if nh > 0:
            # heavy rows drawn on the host (a permutation there needs no
            # device sort) and scaled where the cache lives
            gh = _gen("cpu", wl.seed, layer, _TAG_HEAVY, b)
            for g in range(Hkv):
                pos = torch.randperm(tb, generator=gh)[:nh].to(device)
                kb[g, pos, :] *= wl.heavy_factor
        k[b].copy_(kb.to(dt))
        v[b].copy_(vb.to(dt))
        del kb, vb
    return k, v


def make_queries(wl: Workload, n_steps: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """AR(1) query sequence [n_steps][B][Hq][D] fp32 (row s is q_s)."""
    B, Hq, D = wl.batch, wl.n_q_heads, wl.head_dim
    g = _gen(device, wl.seed, layer, _TAG_Q)
    eps = torch.randn((n_steps, B, Hq, D), generator=g, dtype=torch.float32, device=device)
    a, sig = wl.ar_a, wl.ar_sigma
    q = torch.empty_like(eps)
    q[0] = eps[0] * (sig / (1.0 - a * a) ** 0.5)
    for s in range(1, n_steps):
        q[s] = a * q[s - 1] + sig * eps[s]
    return q


def empty_history(wl: Workload, device="cpu"):
    """An empty query ring: (q_hist[B][Hq][W][D] zeros, newest[B] = W-1, len[B] = 0)."""
    B, Hq, W, D = wl.batch, wl.n_q_heads, wl.window, wl.head_dim
    q_hist = torch.zeros((B, Hq, W, D), dtype=torch.float32, device=device)
    newest = torch.full((B,), W - 1, dtype=torch.int32, device=device)
    length = torch.zeros((B,), dtype=torch.int32, device=device)
    return q_hist, newest, length


def uniform_ints(n: int, lo: int, hi: int, seed: int, device="cpu") -> torch.Tensor:
    """Seeded uniform int32 draws in [lo, hi] (for randomized small test shapes)."""
    g = _gen("cpu", seed, 0, _TAG_MISC)
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).to(torch.int32).to(device)


def randn(shape, seed: int, sub: int = 0, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """Seeded standard-normal draws (for randomized small test inputs)."""
    g = _gen(device, seed, 0, _TAG_MISC, sub)
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(dtype)
