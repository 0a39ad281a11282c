"""GPU parity of qsa_sparse_decode (through the C ABI) against the fp64 QSA
oracle.

The block keys are formed in fp32 (mean, L2 norm, RoPE) and enter the score
product as hi + lo bf16 terms; scores are fp32 sums.  The device then
re-scores in fp64 (block key rebuilt in fp64) every block whose fp32 score
lies within its rounding bound of the 512th, so its block set must equal the
exact top 512 (ties to the lower block).  A bound per block j on the fp32
scores' error,
    eps_j = 2^-13 * sum_h sum_d |q_hd| |bk_jd| + gamma_72 * score_j,
about four times the sum of the worst cases of the steps (fp32 sums of 128
squares and 256 MFMA products, the split's 2^-17, fp32 sin/cos), gives a
second, independent check.  Checked: the token list is the expansion of a
block set plus the exact tail, the set has the right size,
    min over selected (e + eps) >= max over unselected (e - eps),
and the set equals the oracle's exact top 512; the attention output is
compared with the oracle's attention over the device's tokens."""
import math

import numpy as np
import pytest

from helpers import assert_close, from_dev, to_dev
from oracle import attention as oatt
from oracle import qsa as oqsa
from oracle import rope as orope
from workloads import (QSA_128K, ROPE_PLAIN, bf16_bits_to_f64, bf16_tensor_to_f64,
                       device_randn_bf16, randn_bf16, rope_settings)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def _check_tokens(tok, qi, ki, L, rope_p, what):
    """The device's token list for one batch row: valid within the rounding
    bound and equal to the exact top 512 blocks (plus the tail)."""
    nb = L // 4
    bk = oqsa.block_keys(ki, L, rope_p)
    e = oqsa.block_scores(qi, bk)
    eps = 2.0 ** -13 * (np.abs(bk) @ np.abs(qi).T).sum(axis=1) + _gamma(72) * e + 1e-30
    c = min(512, nb)
    t = tok[tok >= 0]
    assert np.all(tok[len(t):] == -1), f"{what}: padding"
    assert len(t) == 4 * c + L % 4, f"{what}: {len(t)} tokens"
    assert list(t[4 * c:]) == list(range(4 * nb, L)), f"{what}: tail"
    blocks = t[:4 * c].reshape(c, 4) if c else np.zeros((0, 4), dtype=np.int64)
    assert np.all(blocks == blocks[:, :1] + np.arange(4)) and np.all(blocks[:, 0] % 4 == 0), \
        f"{what}: block expansion"
    sel = blocks[:, 0] // 4
    assert np.all(np.diff(sel) > 0) and (c == 0 or (sel[0] >= 0 and sel[-1] < nb)), f"{what}: order"
    if c == nb:
        return
    mask = np.zeros(nb, dtype=bool)
    mask[sel] = True
    lo, hi = np.min(e[mask] + eps[mask]), np.max(e[~mask] - eps[~mask])
    assert lo >= hi, f"{what}: block set not valid within the rounding bound ({lo} < {hi})"
    exact = oqsa.select_tokens(e, L, 512)
    if not np.array_equal(tok, exact):
        ex = exact[exact >= 0][:4 * c:4] // 4
        diff = np.setxor1d(ex, sel)
        raise AssertionError(f"{what}: {len(diff)} blocks differ from the exact top 512: {diff[:8]}")


def _run(m, B, Hq, Hkv, S, lens, H_I, seed, rope_p, plant=None):
    import torch
    rng = np.random.default_rng(seed)
    D = 128
    q, kc, vc = randn_bf16(rng, (B, Hq, D)), randn_bf16(rng, (B, Hkv, S, D)), randn_bf16(rng, (B, Hkv, S, D))
    qi, ki = randn_bf16(rng, (B, H_I, 128)), randn_bf16(rng, (B, S, 128))
    if plant is not None:
        plant(qi, ki)
    lens = np.asarray(lens, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    print(f"[case] qsa B={B} Hq={Hq} Hkv={Hkv} S={S} lens={list(lens)} H_I={H_I}", flush=True)
    tok, out = m.qsa_sparse_decode(to_dev(q), to_dev(kc), to_dev(vc), to_dev(qi), to_dev(ki),
                                   torch.from_numpy(lens).cuda(), scale, block_rope=rope_p)
    torch.cuda.synchronize()
    gtok, got = tok.cpu().numpy(), from_dev(out)
    qf, kf, vf = bf16_bits_to_f64(q), bf16_bits_to_f64(kc), bf16_bits_to_f64(vc)
    qif, kif = bf16_bits_to_f64(qi), bf16_bits_to_f64(ki)
    for b in range(B):
        L = int(lens[b])
        _check_tokens(gtok[b], qif[b], kif[b], L, rope_p, f"batch {b}")
        print(f"[parity] batch {b}: block set equals the exact top 512", flush=True)
        t = gtok[b][gtok[b] >= 0]
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            ref = oatt.attend(qf[b, h], kf[b, kv][t], vf[b, kv][t], scale)
            assert_close(got[b, h], ref, f"qsa out (b={b}, h={h})")
    return gtok, got


ROPE64 = rope_settings(ROPE_PLAIN, base=1e4, rotary_dim=64)


@pytest.mark.parametrize("H_I", [64, 16, 32, 48])
def test_qsa_parity(m, H_I):
    _run(m, 2, 16, 2, 5000, [5000, 2999], H_I, 100 + H_I, ROPE64)


def test_qsa_short_contexts_and_full_budget(m):
    """L < 4 (tail only), L = 100 (every block), L = 2049 (512 blocks + 1:
    every token), L = 2052 (513 blocks: one left out)."""
    import torch
    gtok, got = _run(m, 4, 8, 1, 2100, [3, 100, 2049, 2052], 64, 105, ROPE64)
    assert list(gtok[0][:4]) == [0, 1, 2, -1]
    assert list(gtok[2][gtok[2] >= 0]) == list(range(2049))


def test_qsa_needle_block_and_no_rope(m):
    """A block whose keys point along an indexer head's query is selected
    even in a long context; block keys without RoPE."""
    def plant(qi, ki):
        ki[0, 4 * 1000:4 * 1000 + 4] = qi[0, 0]
    gtok, _ = _run(m, 1, 16, 4, 8000, [8000], 64, 106, None, plant=plant)
    assert 4000 in set(gtok[0])


def test_qsa_gqa_groups(m):
    """g = 1 (MHA), g = 16 (one kv head), g = 5 (a partial head tile)."""
    _run(m, 1, 4, 4, 3000, [3000], 16, 107, ROPE64)
    _run(m, 1, 16, 1, 3000, [2999], 16, 108, ROPE64)
    _run(m, 2, 10, 2, 3000, [3000, 1234], 16, 109, ROPE64)


def test_qsa_long_rows_take_the_two_kernel_select(m):
    """More than 16384 blocks per row (S_max = 132000): the chunk and row
    select kernels with the band re-scoring."""
    _run(m, 1, 8, 1, 132000, [132000], 64, 110, ROPE64)


def test_qsa_full_size_128k(m):
    """B=4, L=128K, Hq=32, Hkv=4, 64 indexer heads: every row's block set
    equals the exact top 512, every head against the oracle."""
    import torch
    cfg = QSA_128K
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    print(f"[case] qsa full size B={B} S={S}", flush=True)
    q = device_randn_bf16((B, Hq, D), cfg.seed * 10 + 1)
    kc = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 2)
    vc = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 3)
    qi = device_randn_bf16((B, cfg.H_I, cfg.D_idx), cfg.seed * 10 + 4)
    ki = device_randn_bf16((B, S, cfg.D_idx), cfg.seed * 10 + 5)
    tok, out = m.qsa_sparse_decode(q, kc, vc, qi, ki, torch.from_numpy(cfg.seq_lens()).cuda(),
                                   cfg.scale, block_rope=cfg.block_rope())
    torch.cuda.synchronize()
    gtok, got = tok.cpu().numpy(), from_dev(out)
    qf, qif = bf16_tensor_to_f64(q), bf16_tensor_to_f64(qi)
    for b in range(B):
        _check_tokens(gtok[b], qif[b], bf16_tensor_to_f64(ki[b]), S, cfg.block_rope(),
                           f"full-size batch {b}")
        print(f"[parity] full-size batch {b}: block set equals the exact top 512", flush=True)
        t = gtok[b][gtok[b] >= 0]
        tt = torch.from_numpy(t.astype(np.int64)).cuda()
        g = Hq // Hkv
        for kv in range(Hkv):
            ref = oatt.decode_group(qf[b, kv * g:(kv + 1) * g], bf16_tensor_to_f64(kc[b, kv][tt]),
                                    bf16_tensor_to_f64(vc[b, kv][tt]), len(t), cfg.scale, None)
            assert_close(got[b, kv * g:(kv + 1) * g], ref, f"qsa full size (b={b}, kv={kv})")
