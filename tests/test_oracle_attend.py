"""Pins for the oracle's sparse decode attention (runs on the CPU).

Decode attention over only the selected tokens (reproduction card, "Layout"
and "Key finding"; research-map summary, "Approach").  Pinned against
PyTorch's scaled_dot_product_attention in fp64 when every token is selected,
and against exact special cases.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def sdpa_dense(q, k, v, T):
    """Library dense decode attention, fp64: q[B][Hq][D], k/v[B][Hkv][T][D]."""
    B, Hq, D = q.shape
    G = Hq // k.shape[1]
    kk = torch.from_numpy(np.repeat(k[:, :, :T], G, axis=1))
    vv = torch.from_numpy(np.repeat(v[:, :, :T], G, axis=1))
    qq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    return F.scaled_dot_product_attention(qq, kk, vv)[:, :, 0, :].numpy()


@pytest.mark.parametrize("kv", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 4])
def test_full_selection_equals_dense_attention(orc, kv, G):
    r = np.random.default_rng(G + 10)
    B, Hkv, T, D = 2, 2, 96, 64
    Hq = G * Hkv
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    k = r.standard_normal((B, Hkv, T, D)).astype(np.float32) * 2
    v = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    if kv == "bf16":
        kin, vin = bf16_bits(k), bf16_bits(v)
        kd, vd = bf16_values(kin), bf16_values(vin)
    else:
        kin, vin = k, v
        kd, vd = k.astype(np.float64), v.astype(np.float64)
    idx = np.tile(np.arange(T, dtype=np.int32), (B, Hkv, 1))
    n_sel = np.full((B, Hkv), T, np.int32)
    out = orc.attend(q, kin, vin, idx, n_sel)
    ref = sdpa_dense(q, kd, vd, T)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value_row(orc):
    r = np.random.default_rng(3)
    q = r.standard_normal((1, 2, 64)).astype(np.float32)
    k = r.standard_normal((1, 1, 20, 64)).astype(np.float32)
    v = r.standard_normal((1, 1, 20, 64)).astype(np.float32)
    idx = np.full((1, 1, 4), -1, np.int32)
    idx[0, 0, 0] = 13
    out = orc.attend(q, k, v, idx, np.array([[1]], np.int32))
    np.testing.assert_array_equal(out[0, 0], v[0, 0, 13])
    np.testing.assert_array_equal(out[0, 1], v[0, 0, 13])


def test_zero_query_averages_selected_values(orc):
    r = np.random.default_rng(4)
    q = np.zeros((1, 1, 64), np.float32)
    k = r.standard_normal((1, 1, 30, 64)).astype(np.float32)
    v = r.standard_normal((1, 1, 30, 64)).astype(np.float32)
    sel = np.array([2, 3, 11, 17, 29], np.int32)
    out = orc.attend(q, k, v, sel.reshape(1, 1, -1), np.array([[5]], np.int32))
    np.testing.assert_allclose(out[0, 0], v[0, 0, sel].astype(np.float64).mean(axis=0), rtol=1e-14, atol=1e-15)


def test_order_of_selected_indices_does_not_matter(orc):
    r = np.random.default_rng(5)
    q = r.standard_normal((1, 4, 64)).astype(np.float32)
    k = r.standard_normal((1, 1, 200, 64)).astype(np.float32)
    v = r.standard_normal((1, 1, 200, 64)).astype(np.float32)
    sel = np.sort(r.choice(200, 40, replace=False)).astype(np.int32)
    a = orc.attend(q, k, v, sel.reshape(1, 1, -1), np.array([[40]], np.int32))
    b = orc.attend(q, k, v, r.permutation(sel).astype(np.int32).reshape(1, 1, -1), np.array([[40]], np.int32))
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_subset_equals_dense_attention_on_the_gathered_rows(orc):
    # Attention over a selected subset is dense attention over those rows alone.
    r = np.random.default_rng(6)
    B, Hkv, G, T, D = 1, 1, 2, 300, 128
    q = r.standard_normal((B, Hkv * G, D)).astype(np.float32)
    k = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = r.standard_normal((B, Hkv, T, D)).astype(np.float32)
    sel = np.sort(r.choice(T, 64, replace=False)).astype(np.int32)
    out = orc.attend(q, k, v, sel.reshape(1, 1, -1), np.array([[64]], np.int32))
    ref = sdpa_dense(q, k[:, :, sel].astype(np.float64), v[:, :, sel].astype(np.float64), 64)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_empty_selection_gives_zero_and_bad_index_raises(orc):
    q = np.ones((1, 1, 64), np.float32)
    k = np.ones((1, 1, 4, 64), np.float32)
    idx = np.full((1, 1, 2), -1, np.int32)
    out = orc.attend(q, k, k, idx, np.array([[0]], np.int32))
    assert not out.any()
    idx[0, 0, 0] = 4
    with pytest.raises(IndexError):
        orc.attend(q, k, k, idx, np.array([[1]], np.int32))
