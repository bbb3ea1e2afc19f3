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


# ---- the union with the newest tokens (the library's optional recent window)

def test_recent_window_alone_is_dense_attention_over_the_tail(orc):
    # No selection: the newest r tokens of each sequence, i.e. dense attention
    # over rows [T - r, T).
    r_ = np.random.default_rng(7)
    B, Hkv, G, T_cap, D = 2, 2, 2, 200, 64
    q = r_.standard_normal((B, Hkv * G, D)).astype(np.float32)
    k = r_.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    v = r_.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    lens, recent = np.array([150, 40], np.int32), 50
    idx = np.full((B, Hkv, 8), -1, np.int32)
    out = orc.attend_with_recent(q, k, v, idx, np.zeros((B, Hkv), np.int32), lens, recent)
    for b in range(B):
        T = int(lens[b]); lo = max(T - recent, 0)
        ref = sdpa_dense(q[b:b + 1], k[b:b + 1, :, lo:T].astype(np.float64), v[b:b + 1, :, lo:T].astype(np.float64),
                         T - lo)
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=1e-12, atol=1e-13)


def test_recent_window_counts_a_selected_token_once(orc):
    # The selection overlaps the window (and repeats an index): the union is
    # attended with each token once, the same as dense attention over it.
    r_ = np.random.default_rng(8)
    B, Hkv, G, T_cap, D = 1, 1, 4, 300, 64
    q = r_.standard_normal((B, G, D)).astype(np.float32)
    k = r_.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    v = r_.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    T, recent = 250, 20
    sel = np.array([[[3, 17, 235, 240, 240, 249, -1, 400]]], np.int32)   # 235.. in the window; -1, 400 skipped
    out = orc.attend_with_recent(q, k, v, sel, np.array([[8]], np.int32), np.array([T], np.int32), recent)
    union = np.array(sorted({3, 17} | set(range(T - recent, T))))
    ref = sdpa_dense(q, k[:, :, union].astype(np.float64), v[:, :, union].astype(np.float64), len(union))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_recent_window_longer_than_the_sequence_and_zero_recent(orc):
    r_ = np.random.default_rng(9)
    q = r_.standard_normal((1, 2, 64)).astype(np.float32)
    k = r_.standard_normal((1, 1, 64, 64)).astype(np.float32)
    sel = np.array([[[5, 9, -1]]], np.int32)
    n = np.array([[2]], np.int32)
    # recent = 0 is the plain selection
    np.testing.assert_array_equal(orc.attend_with_recent(q, k, k, sel, n, np.array([30], np.int32), 0),
                                  orc.attend(q, k, k, sel, n))
    # recent past the length covers the whole sequence: dense over [0, T)
    out = orc.attend_with_recent(q, k, k, sel, n, np.array([30], np.int32), 1000)
    ref = sdpa_dense(q, k[:, :, :30].astype(np.float64), k[:, :, :30].astype(np.float64), 30)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
