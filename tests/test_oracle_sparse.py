"""Pins of the oracle's indexer, top-k selection and sparse attention (CPU)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as att
from oracle import sparse
from workloads import bf16_bits_to_f64, randn_bf16


def _fraction_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    if fr == 0:
        return np.float32(0.0)
    d = np.float32(float(fr))            # candidate (possibly double-rounded)
    # neighbours of the candidate in float32
    lo = np.nextafter(d, np.float32(-np.inf))
    hi = np.nextafter(d, np.float32(np.inf))
    best = min((lo, d, hi), key=lambda c: (abs(Fraction(float(c)) - fr),
                                             int(np.asarray(c).view(np.uint32)) & 1))
    return np.float32(best)


def test_indexer_scores_are_exact_dot_rounded_once_then_relu():
    rng = np.random.default_rng(0)
    q = bf16_bits_to_f64(randn_bf16(rng, (128,)))
    k = bf16_bits_to_f64(randn_bf16(rng, (400, 128)))
    s = sparse.indexer_scores(q, k, 400)
    assert s.dtype == np.float32
    for j in range(400):
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k[j]))
        want = max(_fraction_to_f32(exact), np.float32(0.0))
        assert s[j] == want, j
    # seq_len cuts the scan
    assert sparse.indexer_scores(q, k, 17).shape == (17,)


def _brute_topk(scores, k):
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    sel = sorted(order[:min(k, len(scores))])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_topk_against_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    k = int(rng.integers(1, 70))
    # few distinct values -> many ties, including zeros
    scores = rng.integers(0, 5, size=n).astype(np.float32)
    got = sparse.topk_select(scores, k)
    assert list(got) == _brute_topk(scores, k)
    keff = min(k, n)
    sel = got[:keff]
    assert np.all(np.diff(sel) > 0)
    uns = np.setdiff1d(np.arange(n), sel)
    if len(uns) and keff:
        assert scores[sel].min() >= scores[uns].max()
        # at the boundary value, every selected index precedes every unselected one
        t = scores[sel].min()
        if np.any(scores[uns] == t):
            assert sel[scores[sel] == t].max() < uns[scores[uns] == t].min()


def test_short_context_selects_everything():
    s = np.array([3.0, 0.0, 1.0], dtype=np.float32)
    assert list(sparse.topk_select(s, 5)) == [0, 1, 2, -1, -1]


def test_full_selection_reduces_to_dense_mqa():
    """k >= L: sparse attention over all rows equals dense MQA decode over the
    latent rows (K = latent, V = its first Dv dims)."""
    rng = np.random.default_rng(3)
    B, H, L, Dqk, Dv, Di = 2, 4, 50, 24, 16, 8
    q = rng.standard_normal((B, H, Dqk))
    lat = rng.standard_normal((B, L, Dqk))
    qi = rng.standard_normal((B, Di))
    ki = rng.standard_normal((B, L, Di))
    seq = np.array([50, 31])
    idx, out = sparse.topk_sparse_decode(q, lat, qi, ki, seq, top_k=64, scale=0.3, Dv=Dv)
    dense = att.decode(q, lat[:, None], lat[:, None, :, :Dv], seq, 0.3, None)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-14)
    assert list(idx[1][:31]) == list(range(31)) and np.all(idx[1][31:] == -1)


def test_selection_equals_minus_inf_mask():
    """[attention] DSA ③: adding a -inf mask to unselected scores then softmax
    equals attending to the selected rows only."""
    rng = np.random.default_rng(4)
    L, D = 40, 12
    q = rng.standard_normal(D)
    lat = rng.standard_normal((L, D))
    idx = np.array([1, 5, 6, 20, 39])
    got = sparse.sparse_attention_one(q, lat, np.concatenate([idx, [-1, -1]]), 0.5, 8)
    s = lat @ q * 0.5
    mask = np.full(L, -np.inf)
    mask[idx] = 0.0
    p = att.softmax(s + mask)
    assert np.allclose(got, p @ lat[:, :8], rtol=1e-13)


def test_relu_zeroes_negative_scores():
    q = np.ones(4)
    k = np.array([[1, 1, 1, 1], [-1, -1, -1, -1], [0.5, -0.5, 0, 0]], dtype=np.float64)
    assert list(sparse.indexer_scores(q, k, 3)) == [4.0, 0.0, 0.0]


def test_dense_mla_decode_equals_unabsorbed_multihead_attention():
    """The absorbed (MQA) form equals multi-head attention with per-head keys
    W_UK[h] c_j plus the shared rope key, and values W_UV[h] c_j: scores
    q_h . k_hj = (W_UK[h]^T q_h) . c_j + q_h^R . k_j^R (matrix associativity),
    and sum_j p_j W_UV[h] c_j = W_UV[h] (sum_j p_j c_j)."""
    rng = np.random.default_rng(21)
    B, H, L, dc, dR, dh = 2, 3, 17, 8, 4, 6
    c = rng.standard_normal((B, L, dc))
    kR = rng.standard_normal((B, L, dR))
    W_UK = rng.standard_normal((H, dh, dc))
    W_UV = rng.standard_normal((H, dh, dc))
    qn = rng.standard_normal((B, H, dh))
    qR = rng.standard_normal((B, H, dR))
    seq = np.array([17, 9])
    scale = 0.37
    # unabsorbed: per-head keys [W_UK c ; k^R] and values W_UV c (MHA, Hkv = H)
    K = np.concatenate([np.einsum("hdc,blc->bhld", W_UK, c), np.broadcast_to(kR[:, None], (B, H, L, dR))], -1)
    V = np.einsum("hdc,blc->bhld", W_UV, c)
    qfull = np.concatenate([qn, qR], -1)
    mha = att.decode(qfull, K, V, seq, scale, None)
    # absorbed: q~ = [W_UK^T q ; q^R] against latent rows [c ; k^R], then W_UV
    qa = np.concatenate([np.einsum("hdc,bhd->bhc", W_UK, qn), qR], -1)
    lat = np.concatenate([c, kR], -1)
    o_lat = sparse.mla_dense_decode(qa, lat, seq, scale, Dv=dc)
    absorbed = np.einsum("hdc,bhc->bhd", W_UV, o_lat)
    assert np.allclose(absorbed, mha, rtol=1e-11, atol=1e-12)
    # and it is the sparse path with every row selected
    for b in range(B):
        for h in range(H):
            one = sparse.sparse_attention_one(qa[b, h], lat[b], np.arange(seq[b]), scale, dc)
            assert np.array_equal(one, o_lat[b, h])



def test_weighted_indexer_pins():
    """[稀疏注意力] DSA ①: I_s = sum_j w_j ReLU(q_j . k_s).
    * one head with weight 1 is the single-head indexer (exactly, before its
      float32 rounding);
    * two heads q_0 = e_1, q_1 = -e_1 with weights (1, 2) give the closed form
      k_1 for k_1 >= 0 and -2 k_1 for k_1 < 0 (ReLU per head, then weights;
      summing before the ReLU would give max(0, -k_1) instead);
    * linear in the weights, and a head whose dots are all negative adds
      nothing whatever its weight."""
    rng = np.random.default_rng(5)
    L, D = 200, 16
    k = rng.standard_normal((L, D))
    q = rng.standard_normal((1, D))
    one = sparse.weighted_indexer_scores(q, np.array([1.0]), k, L)
    assert np.array_equal(one.astype(np.float32), sparse.indexer_scores(q[0], k, L))
    q2 = np.zeros((2, D))
    q2[0, 1], q2[1, 1] = 1.0, -1.0
    got = sparse.weighted_indexer_scores(q2, np.array([1.0, 2.0]), k, L)
    want = np.where(k[:, 1] >= 0, k[:, 1], -2.0 * k[:, 1])
    assert np.array_equal(got, want)
    qh = rng.standard_normal((3, D))
    w1, w2 = rng.standard_normal(3), rng.standard_normal(3)
    s12 = sparse.weighted_indexer_scores(qh, w1 + w2, k, L)
    assert np.allclose(s12, sparse.weighted_indexer_scores(qh, w1, k, L)
                       + sparse.weighted_indexer_scores(qh, w2, k, L), rtol=1e-12, atol=1e-12)
    kpos = np.abs(k)
    qneg = np.vstack([qh[:1], -np.abs(rng.standard_normal((1, D)))])   # head 1: all dots < 0
    a = sparse.weighted_indexer_scores(qneg, np.array([0.7, 123.0]), kpos, L)
    b = sparse.weighted_indexer_scores(qneg[:1], np.array([0.7]), kpos, L)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)   # (the product's summation order may differ)


def test_topk_select_exact_matches_sorting():
    """Exact-score top-k: the k largest by value, ties to the lower index."""
    s = np.array([3.0, -1.0, 3.0, 7.5, 0.0, 3.0, -2.0])
    assert list(sparse.topk_select_exact(s, 3)) == [0, 2, 3]
    assert list(sparse.topk_select_exact(s, 4)) == [0, 2, 3, 5]
    assert list(sparse.topk_select_exact(s[:2], 4)) == [0, 1, -1, -1]
    rng = np.random.default_rng(6)
    v = rng.standard_normal(1000)
    sel = sparse.topk_select_exact(v, 100)
    assert set(sel) == set(np.argsort(-v)[:100])


def test_sparse_attention_heads_equals_one_head_at_a_time_and_sdpa():
    """The grouped form equals sparse_attention_one per head and torch's
    scaled_dot_product_attention (float64, CPU) on the selected rows, with
    the first Dv columns as values."""
    import torch
    rng = np.random.default_rng(90)
    H, L, Dqk, Dv = 6, 200, 40, 24
    q = rng.standard_normal((H, Dqk))
    lat = rng.standard_normal((L, Dqk))
    idx = np.array(sorted(rng.choice(L, 50, replace=False)) + [-1, -1])
    got = sparse.sparse_attention_heads(q, lat, idx, 0.3, Dv)
    for h in range(H):
        assert np.allclose(got[h], sparse.sparse_attention_one(q[h], lat, idx, 0.3, Dv),
                           rtol=1e-13, atol=1e-15)
    rows = torch.from_numpy(lat[idx[idx >= 0]])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], rows[None, None].expand(1, H, -1, -1),
        rows[None, None, :, :Dv].expand(1, H, -1, -1), scale=0.3).numpy()[0, :, 0]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)
