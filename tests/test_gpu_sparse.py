"""GPU parity of topk_sparse_decode (through the C ABI) against the fp64 oracle:
index sets bit-exact, attention outputs within tolerance."""
import math

import numpy as np
import pytest

from helpers import KERNEL_ATOL, KERNEL_RTOL, Guarded, assert_close, from_dev, to_dev
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


def _run(m, d, top_k, heads=None):
    import torch
    B, H, _ = d["q"].shape
    print(f"[case] sparse B={B} H={H} S_max={d['latent'].shape[1]} lens={list(d['seq_lens'])} "
          f"k={top_k}", flush=True)
    idx, out = m.topk_sparse_decode(to_dev(d["q"]), to_dev(d["latent"]), to_dev(d["q_index"]),
                                    to_dev(d["k_index"]), torch.from_numpy(d["seq_lens"]).cuda(),
                                    top_k, SCALE)
    torch.cuda.synchronize()
    ridx, rout = osp.topk_sparse_decode(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["latent"]),
                                        bf16_bits_to_f64(d["q_index"]),
                                        bf16_bits_to_f64(d["k_index"]), d["seq_lens"], top_k,
                                        SCALE, 512, heads=heads)
    gidx = idx.cpu().numpy()
    for b in range(B):
        if not np.array_equal(gidx[b], ridx[b]):
            diff = np.setxor1d(gidx[b][gidx[b] >= 0], ridx[b][ridx[b] >= 0])
            raise AssertionError(f"batch {b}: index sets differ at {diff[:10]}")
    got = from_dev(out)
    if heads is not None:
        got, rout = got[:, heads], rout[:, heads]
    assert_close(got, rout, "sparse out")
    return gidx


def test_sparse_small(m):
    d = sparse_inputs_host(2, 16, 3000, 576, 128, 41, [3000, 1500])
    _run(m, d, 256)


def test_sparse_odd_capacity(m):
    """S_max not a multiple of 4 (score rows are padded internally)."""
    d = sparse_inputs_host(3, 16, 3001, 576, 128, 46, [3001, 2999, 1])
    _run(m, d, 129)


def test_sparse_short_context_and_full_selection(m):
    d = sparse_inputs_host(2, 32, 600, 576, 128, 42, [100, 600])
    idx = _run(m, d, 512)
    assert list(idx[0][:100]) == list(range(100)) and np.all(idx[0][100:] == -1)


def test_sparse_ties_and_relu_zeros(m):
    """Few distinct scores (rows repeat), most of them ReLU zeros: the lower
    index must win every tie."""
    rng = np.random.default_rng(43)
    d = sparse_inputs_host(2, 16, 4000, 576, 128, 43, [4000, 3999])
    base = d["k_index"][:, :8].copy()
    reps = rng.integers(0, 8, size=(2, 4000))
    d["k_index"] = np.stack([base[b][reps[b]] for b in range(2)])
    _run(m, d, 700)
    # all-negative dot products except a few: zeros dominate the selection
    d2 = sparse_inputs_host(1, 16, 5000, 576, 128, 44, [5000])
    qi = np.zeros((1, 128), np.float32)
    qi[0, 0] = 1.0
    ki = -np.abs(bf16_bits_to_f64(d2["k_index"]).astype(np.float32))
    ki[0, ::97, 0] = 1.5
    d2["q_index"] = f32_to_bf16_bits(qi)
    d2["k_index"] = f32_to_bf16_bits(ki)
    _run(m, d2, 300)


def test_sparse_large_threshold_bin(m):
    """More than 8192 equal scores in the threshold bin: the multi-pass path."""
    d = sparse_inputs_host(1, 16, 20000, 576, 128, 45, [20000])
    d["k_index"][0, :] = d["k_index"][0, 0]
    d["q_index"][0] = d["k_index"][0, 0]      # every score equals |k_0|^2 > 0
    _run(m, d, 2048)


@pytest.mark.parametrize("n_eq", [12000, 12400])
def test_sparse_threshold_bin_at_lds_capacity(m, n_eq):
    """n_eq equal top scores (|k_0|^2 ~ 128, the other scores ~ N(0, 128)):
    the threshold bin just inside (12000) and just past (12400) the 12288
    entries the row workgroup holds in LDS; the lowest 2048 indices win."""
    d = sparse_inputs_host(1, 16, 16000, 576, 128, 47, [16000])
    d["k_index"][0, :n_eq] = d["k_index"][0, 0]
    d["q_index"][0] = d["k_index"][0, 0]
    idx = _run(m, d, 2048)
    assert list(idx[0]) == list(range(2048))


def test_sparse_overflow_and_lds_rows_in_one_call(m):
    """Row 0: 20000 equal top scores (the finish kernel's overflow path);
    row 1: ordinary scores (its LDS path); row 2 shorter than k (every index).
    Each row takes its own path in the same launch."""
    d = sparse_inputs_host(3, 16, 24000, 576, 128, 48, [24000, 23001, 1500])
    d["k_index"][0, :20000] = d["k_index"][0, 0]
    d["q_index"][0] = d["k_index"][0, 0]
    idx = _run(m, d, 2048)
    assert list(idx[0]) == list(range(2048))
    assert list(idx[2][:1500]) == list(range(1500)) and np.all(idx[2][1500:] == -1)


def test_sparse_long_rows_take_the_two_kernel_select(m):
    """Rows longer than 16384 keys are selected by the chunk and row kernels
    (shorter ones by one kernel per row): row 0 with 20000 equal top scores
    (the row kernel's overflow path), row 1 ordinary, row 2 shorter than k."""
    d = sparse_inputs_host(3, 16, 40000, 576, 128, 49, [40000, 39001, 1500])
    d["k_index"][0, :20000] = d["k_index"][0, 0]
    d["q_index"][0] = d["k_index"][0, 0]
    idx = _run(m, d, 2048)
    assert list(idx[0]) == list(range(2048))
    assert list(idx[2][:1500]) == list(range(1500)) and np.all(idx[2][1500:] == -1)


def test_sparse_full_size_128k(m):
    import torch
    cfg = SPARSE_128K
    B, H, S, k = cfg.B, cfg.H, cfg.S_max, cfg.top_k
    print(f"[case] sparse full size B={B} H={H} S={S} k={k}", flush=True)
    q = device_randn_bf16((B, H, cfg.Dqk), cfg.seed * 10 + 1)
    lat = device_randn_bf16((B, S, cfg.Dqk), cfg.seed * 10 + 2)
    qi = device_randn_bf16((B, cfg.D_idx), cfg.seed * 10 + 3)
    ki = device_randn_bf16((B, S, cfg.D_idx), cfg.seed * 10 + 4)
    lens = torch.from_numpy(cfg.seq_lens()).cuda()
    out_g = Guarded((B, H, cfg.Dv), torch.bfloat16, seed=5)
    idx_g = Guarded((B, k), torch.int32, seed=6)
    ws = Guarded((m.topk_sparse_decode_workspace_size(B, H, S, k),), torch.uint8, seed=7)
    idx, out = m.topk_sparse_decode(q, lat, qi, ki, lens, k, cfg.scale, topk_idx=idx_g.view,
                                    out=out_g.view, workspace=ws.view)
    torch.cuda.synchronize()
    first_idx, first_out = idx.clone(), out.clone()
    m.topk_sparse_decode(q, lat, qi, ki, lens, k, cfg.scale, topk_idx=idx_g.view,
                         out=out_g.view, workspace=ws.view)
    torch.cuda.synchronize()
    assert torch.equal(first_idx, idx) and torch.equal(first_out, out), "two identical calls differ"
    gidx = idx.cpu().numpy()
    got = from_dev(out)
    qf, qif = bf16_tensor_to_f64(q), bf16_tensor_to_f64(qi)
    for b in range(B):
        kib = bf16_tensor_to_f64(ki[b])
        ridx = osp.topk_select(osp.indexer_scores(qif[b], kib, S), k)
        assert np.array_equal(gidx[b], ridx), f"batch {b}: index sets differ"
        rows = bf16_tensor_to_f64(lat[b][torch.from_numpy(ridx.astype(np.int64)).cuda()])
        ref = osp.sparse_attention_heads(qf[b], rows, np.arange(k), cfg.scale, cfg.Dv)
        assert_close(got[b], ref, f"full-size every head (b={b})")
        assert_close(got[b], ref, f"full-size every head (b={b}) kernel precision",
                     atol=KERNEL_ATOL, rtol=KERNEL_RTOL)
    out_g.check("out")
    idx_g.check("topk_idx")
    ws.check("workspace")


def test_sparse_largest_cache(m):
    """The largest latent cache the ABI accepts: 1,864,135 rows of 1152 bytes
    (2^31 - 128 bytes), every row a candidate.  The gather's byte offsets of
    the last rows sit at the 32-bit limit and the select runs over 456 key
    chunks; index set bit-exact and every head against the oracle."""
    import torch
    B, H, S, k = 1, 16, 1864135, 2048
    print(f"[case] sparse largest cache B={B} H={H} S={S} k={k}", flush=True)
    q = device_randn_bf16((B, H, 576), 81)
    lat = device_randn_bf16((B, S, 576), 82)
    qi = device_randn_bf16((B, 128), 83)
    ki = device_randn_bf16((B, S, 128), 84)
    lens = torch.tensor([S], dtype=torch.int32).cuda()
    idx, out = m.topk_sparse_decode(q, lat, qi, ki, lens, k, SCALE)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()[0]
    ridx = osp.topk_select(osp.indexer_scores(bf16_tensor_to_f64(qi)[0], bf16_tensor_to_f64(ki[0]), S), k)
    assert np.array_equal(gidx, ridx), "index sets differ"
    assert ridx.max() > S - 200000, "the selection reaches the last rows"
    rows = bf16_tensor_to_f64(lat[0][torch.from_numpy(ridx.astype(np.int64)).cuda()])
    ref = osp.sparse_attention_heads(bf16_tensor_to_f64(q)[0], rows, np.arange(k), SCALE, 512)
    assert_close(from_dev(out)[0], ref, "largest cache, every head")
    assert_close(from_dev(out)[0], ref, "largest cache, kernel precision", atol=KERNEL_ATOL,
                 rtol=KERNEL_RTOL)
