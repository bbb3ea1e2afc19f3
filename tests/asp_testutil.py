"""Helpers shared by the GPU parity tests: device checks, dtype conversions and
the staged end-to-end comparison against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kv_np(t: torch.Tensor) -> np.ndarray:
    """Host copy of a K/V tensor as the oracle takes it (fp32, or bf16 bits as uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def dims_for(A, B, Hq, Hkv, D, T_cap, kv):
    return A.Dims(B, Hq, Hkv, D, T_cap, A.KV_BF16 if kv == "bf16" else A.KV_F32)


def assert_pred_close(gpu: np.ndarray, orc: np.ndarray, rel: float = 1e-4):
    """Predicted queries: max-abs error per (b, h) within rel * max|q_orc|."""
    B, Hq, D = orc.shape
    err = np.abs(gpu.astype(np.float64) - orc).max(axis=2)
    ref = np.abs(orc).max(axis=2)
    bad = ~(err <= rel * np.maximum(ref, 1e-30))  # a NaN on either side counts as a mismatch
    assert not bad.any(), "predictor mismatch at %s: err %s ref %s" % (np.argwhere(bad)[:5], err[bad][:5], ref[bad][:5])


def assert_selection_within_gap(idx_gpu, n_gpu, s_orc, seq_lens, C, rel_gap=1e-5):
    """End-to-end selection check: the GPU set has size C_eff, and every index in
    the symmetric difference with the oracle's own top-C (computed on fp64
    scores) lies within rel_gap * max|score| of the oracle's C_eff-th score."""
    import oracle
    idx_o, n_o = oracle.select(s_orc, seq_lens, C)
    B, Hkv, _ = s_orc.shape
    for b in range(B):
        T = int(seq_lens[b])
        for g in range(Hkv):
            ce = min(C, T)
            assert n_gpu[b, g] == ce
            sg = set(idx_gpu[b, g, :ce].tolist())
            so = set(idx_o[b, g, :ce].tolist())
            assert len(sg) == ce and all(0 <= i < T for i in sg)
            assert (idx_gpu[b, g, ce:] == -1).all()
            if sg == so:
                continue
            row = s_orc[b, g, :T]
            thr = np.sort(row)[::-1][ce - 1]
            tol = rel_gap * np.abs(row).max()
            for i in sg ^ so:
                assert abs(row[i] - thr) <= tol, (b, g, i, row[i], thr, tol)
