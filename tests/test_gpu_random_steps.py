"""Seeded random shapes through the pipelined asp_step (GPU required): the
bootstrap and four pipelined steps, on one stream and on two streams with a
context, equal bit for bit the same schedule built from the individual entry
points (whose stages the oracle checks elsewhere), for shapes drawn like those
of test_gpu_random_shapes: group, head_dim, K/V dtype, t_cap, C, window, a ring
that is or is not full when the steps start, ragged lengths including 0 and
t_cap, sometimes the newest-token window.
"""
import os

import numpy as np
import pytest
import torch

from query_aware_sparse_amd import workload as wk
from test_gpu_step import DEV, Problem, _manual_run, _step_run

pytestmark = pytest.mark.gpu
N_CASES = int(os.environ.get("ASP_RANDOM_STEPS", "32"))  # more cases: set the variable


def draw(seed: int):
    r = np.random.default_rng(2000 + seed)
    B = int(r.integers(1, 5))
    Hkv = int(r.integers(1, 3))
    G = int(r.choice([1, 2, 4, 8]))
    D = int(r.choice([64, 128]))
    T_cap = int(r.choice([r.integers(16, 700), r.integers(700, 4000), 512 * int(r.integers(1, 7))]))
    C = int(r.choice([1, r.integers(1, T_cap + 1), T_cap]))
    W = int(r.choice([4, 8, 16, 32]))
    lens = r.integers(0, T_cap + 1, size=B)
    lens[0] = T_cap
    if B > 1:
        lens[-1] = int(r.choice([0, 1, lens[-1]]))
    wl = wk.TINY.replace(name="random-%d" % seed, batch=B, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D,
                         t_cap=T_cap, kv_dtype=str(r.choice(["bf16", "f32"])), window=W, top_c=C,
                         history_steps=int(r.integers(1, W + 3)), heavy_count=min(8, T_cap),
                         recent=int(r.choice([0, 0, r.integers(1, T_cap + 1)])), seed=seed)
    return wl, [int(x) for x in lens]


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_step_modes_bit_identical_to_entry_points(seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl, lens = draw(seed)
    n = 5
    runs = {}
    for mode in ("manual", "one_stream", "two_streams"):
        p = Problem(wl, kv_device=DEV, n_steps=n, lens=lens)
        p.fill_history()
        torch.cuda.synchronize()
        runs[mode] = _manual_run(p, n) if mode == "manual" else _step_run(p, mode, n)
    for mode in ("one_stream", "two_streams"):
        for s in range(n):
            for a, b in zip(runs["manual"][s], runs[mode][s]):
                np.testing.assert_array_equal(a, b, err_msg="%s step %d (%s, lens %s)" % (mode, s, wl, lens))
