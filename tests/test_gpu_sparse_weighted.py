"""GPU parity of topk_sparse_decode_weighted (multi-head weighted indexer,
through the C ABI) against the fp64 oracle.

The device sums each head's dot product and the weighted sum over the heads
in fp32, then re-scores in fp64 every key whose fp32 score lies within its
rounding bound of the k-th one, so its index set must equal the exact top-k
(ties to the lower index).  Checked, per row: the set has the right size and
form; it is valid within the rounding bound
    min over selected j of (e_j + eps_j) >= max over unselected i of (e_i - eps_i)
with e the exact scores and eps_j a bound on the fp32 scores' error for key j
(an fp32 sum of n terms errs by at most gamma_n = n u / (1 - n u) times the
sum of their magnitudes, u = 2^-24: 128 exact products per head, then the
ReLU (1-Lipschitz) and the weighted sum over H_I heads; a factor 2 kept as
slack); and it equals the oracle's exact top-k.  The attention output is
compared with the oracle's attention over the selected set."""
import math

import numpy as np
import pytest

from helpers import assert_close, from_dev, to_dev
from oracle import sparse as osp
from workloads import (SPARSE_128K, bf16_bits_to_f64, bf16_tensor_to_f64, device_randn_bf16,
                       f32_to_bf16_bits, sparse_inputs_host)

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(192)


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def _exact_and_bound(qi, w, ki, L):
    """Exact scores e [L] and the device error bound eps [L] (fp64)."""
    k = ki[:L]
    dots = k @ qi.T                                   # [L, H_I]
    mags = np.abs(k) @ np.abs(qi).T                   # sum_d |q_hd k_d|
    e = np.maximum(dots, 0.0) @ w
    H_I = qi.shape[0]
    eps = _gamma(qi.shape[1] + 2) * (mags @ np.abs(w)) + _gamma(H_I + 8) * (np.maximum(dots, 0.0) @ np.abs(w))
    return e, 2.0 * eps + 1e-30


def _check_selection(sel, e, eps, k, L, what):
    keff = min(k, L)
    assert np.all(sel[keff:] == -1), f"{what}: padding"
    s = sel[:keff]
    assert np.all(np.diff(s) > 0) and s[0] >= 0 and s[-1] < L, f"{what}: not ascending in range"
    if keff == L:
        return
    mask = np.zeros(L, dtype=bool)
    mask[s] = True
    lo = np.min(e[mask] + eps[mask])
    hi = np.max(e[~mask] - eps[~mask])
    assert lo >= hi, f"{what}: selection not valid within the rounding bound ({lo} < {hi})"
    exact = osp.topk_select_exact(e, k)
    if not np.array_equal(sel, exact):
        diff = np.setxor1d(exact[:keff], s)
        raise AssertionError(f"{what}: {len(diff)} indices differ from the exact top-k: {diff[:8]}")


def _run(m, d, qi_bits, w, top_k, heads=None):
    import torch
    B, H, _ = d["q"].shape
    L_all = d["seq_lens"]
    print(f"[case] weighted sparse B={B} H={H} H_I={qi_bits.shape[1]} S_max={d['latent'].shape[1]} "
          f"lens={list(L_all)} k={top_k}", flush=True)
    idx, out = m.topk_sparse_decode_weighted(
        to_dev(d["q"]), to_dev(d["latent"]), to_dev(qi_bits),
        torch.from_numpy(w.astype(np.float32)).cuda(), to_dev(d["k_index"]),
        torch.from_numpy(L_all).cuda(), top_k, SCALE)
    torch.cuda.synchronize()
    gidx, got = idx.cpu().numpy(), from_dev(out)
    qf, lat = bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["latent"])
    qif, kif = bf16_bits_to_f64(qi_bits), bf16_bits_to_f64(d["k_index"])
    for b in range(B):
        L = int(L_all[b])
        e, eps = _exact_and_bound(qif[b], w[b].astype(np.float32).astype(np.float64), kif[b], L)
        _check_selection(gidx[b], e, eps, top_k, L, f"batch {b}")
        print(f"[parity] batch {b}: index set equals the exact top-k", flush=True)
        for h in (range(H) if heads is None else heads):
            ref = osp.sparse_attention_one(qf[b, h], lat[b], gidx[b], SCALE, 512)
            assert_close(got[b, h], ref, f"weighted sparse out (b={b}, h={h})")
    return gidx


def _weights(rng, B, H_I, sign=None):
    w = rng.standard_normal((B, H_I)).astype(np.float32) / 8
    if sign == "neg":
        w = -np.abs(w)
    return w


@pytest.mark.parametrize("H_I", [64, 16, 32, 48])
def test_weighted_sparse_parity(m, H_I):
    from workloads import randn_bf16
    rng = np.random.default_rng(90 + H_I)
    d = sparse_inputs_host(2, 16, 3000, 576, 128, 91, [3000, 1500])
    qi = randn_bf16(rng, (2, H_I, 128))
    _run(m, d, qi, _weights(rng, 2, H_I), 256)


def test_weighted_sparse_negative_weights_and_short_rows(m):
    """All weights negative: every score <= 0 and the order-preserving keys of
    negative values decide; a context shorter than k selects everything."""
    from workloads import randn_bf16
    rng = np.random.default_rng(92)
    d = sparse_inputs_host(3, 16, 2500, 576, 128, 93, [2500, 300, 2001])
    qi = randn_bf16(rng, (3, 64, 128))
    gidx = _run(m, d, qi, _weights(rng, 3, 64, "neg"), 512)
    assert list(gidx[1][:300]) == list(range(300)) and np.all(gidx[1][300:] == -1)


def test_weighted_sparse_ties_take_lower_indices(m):
    """Identical key rows give identical fp32 scores: the lowest k indices."""
    from workloads import randn_bf16
    rng = np.random.default_rng(94)
    d = sparse_inputs_host(1, 16, 3000, 576, 128, 95, [3000])
    d["k_index"][0, :] = d["k_index"][0, 0]
    qi = randn_bf16(rng, (1, 64, 128))
    gidx = _run(m, d, qi, _weights(rng, 1, 64), 700)
    assert list(gidx[0]) == list(range(700))


def test_weighted_sparse_band_reaches_below_the_threshold_bin(m):
    """16 heads all along dim 0 (q_h = e_0) with weights 1/16: key s scores
    max(k_s[0], 0) exactly, in fp32 too.  k-1 keys score 4, the k-th score is
    exactly 1.0 (the lowest value of its first-digit bin), 100 keys score
    1 - 2^-8 (the bin below), the rest 0; one key with |k| = 256 (its dim 1)
    widens the re-scored band to about +-2^-6, so the band reaches into the
    bin below and its keys there come from the row itself.  Row 1 has two
    keys at exactly 1.0: the lower index wins."""
    rng = np.random.default_rng(96)
    B, S, k = 2, 3000, 256
    d = sparse_inputs_host(B, 16, S, 576, 128, 97, [S, S])
    ki = np.zeros((B, S, 128), dtype=np.float32)
    ki[:, :, 0] = -1.0
    for b in range(B):
        perm = rng.permutation(S)
        n_t = 1 + b                                  # keys at exactly 1.0
        ki[b, perm[:k - 1], 0] = 4.0
        ki[b, perm[k - 1:k - 1 + n_t], 0] = 1.0
        ki[b, perm[k - 1 + n_t:k - 1 + n_t + 100], 0] = 1.0 - 2.0 ** -8
        ki[b, perm[-1], 1] = 256.0                   # score 0, largest norm
    d["k_index"] = f32_to_bf16_bits(ki)
    qi = np.zeros((B, 16, 128), dtype=np.float32)
    qi[:, :, 0] = 1.0
    w = np.full((B, 16), 1.0 / 16, dtype=np.float32)
    gidx = _run(m, d, f32_to_bf16_bits(qi), w, k)
    for b in range(B):
        e = np.maximum(ki[b, :, 0].astype(np.float64), 0.0)
        assert np.array_equal(gidx[b], osp.topk_select_exact(e, k))


def test_weighted_sparse_full_size_128k(m):
    """B=4, L=128K, H=128, H_I=64, k=2048: every row's index set equals the
    exact top-k, attention of every head against the oracle."""
    import torch
    cfg = SPARSE_128K
    B, H, S, k, H_I = cfg.B, cfg.H, cfg.S_max, cfg.top_k, 64
    print(f"[case] weighted sparse full size B={B} H={H} S={S} k={k} H_I={H_I}", flush=True)
    q = device_randn_bf16((B, H, cfg.Dqk), cfg.seed * 10 + 7)
    lat = device_randn_bf16((B, S, cfg.Dqk), cfg.seed * 10 + 8)
    qi = device_randn_bf16((B, H_I, cfg.D_idx), cfg.seed * 10 + 9)
    ki = device_randn_bf16((B, S, cfg.D_idx), cfg.seed * 10 + 10)
    w = _weights(np.random.default_rng(cfg.seed), B, H_I)
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    idx, out = m.topk_sparse_decode_weighted(q, lat, qi, torch.from_numpy(w).cuda(), ki, lens, k,
                                             cfg.scale)
    torch.cuda.synchronize()
    gidx, got = idx.cpu().numpy(), from_dev(out)
    qf, qif = bf16_tensor_to_f64(q), bf16_tensor_to_f64(qi)
    for b in range(B):
        e, eps = _exact_and_bound(qif[b], w[b].astype(np.float64), bf16_tensor_to_f64(ki[b]), S)
        _check_selection(gidx[b], e, eps, k, S, f"full-size batch {b}")
        print(f"[parity] full-size batch {b}: index set equals the exact top-k", flush=True)
        rows = bf16_tensor_to_f64(lat[b][torch.from_numpy(gidx[b].astype(np.int64)).cuda()])
        ref = osp.sparse_attention_heads(qf[b], rows, np.arange(k), cfg.scale, cfg.Dv)
        assert_close(got[b], ref, f"weighted full-size every head (b={b})")
