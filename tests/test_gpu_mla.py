"""GPU parity of mla_decode (dense absorbed-MLA decode, through the C ABI)
against the fp64 oracle: every head attends to all latent rows < seq_lens[b]."""
import math

import numpy as np
import pytest

from helpers import KERNEL_ATOL, KERNEL_RTOL, assert_close, from_dev, to_dev
from oracle import sparse as osp
from workloads import (SPARSE_128K, bf16_bits_to_f64, bf16_tensor_to_f64, device_randn_bf16,
                       sparse_inputs_host)

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(192)


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _run(m, q_bits, lat_bits, lens, scale=SCALE, heads=None):
    import torch
    B, H, _ = q_bits.shape
    lens = np.asarray(lens, dtype=np.int32)
    print(f"[case] mla B={B} H={H} S_max={lat_bits.shape[1]} lens={list(lens)}", flush=True)
    out = m.mla_decode(to_dev(q_bits), to_dev(lat_bits), torch.from_numpy(lens).cuda(), scale)
    torch.cuda.synchronize()
    ref = osp.mla_dense_decode(bf16_bits_to_f64(q_bits), bf16_bits_to_f64(lat_bits), lens, scale,
                               512, heads=heads)
    got = from_dev(out)
    if heads is not None:
        got, ref = got[:, heads], ref[:, heads]
    assert_close(got, ref, "mla out")
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-2, rel


def _peaky(q_bits):
    """q scaled by 4 (exact in bf16): scores spread ~7 units, a few rows dominate."""
    return (q_bits.astype(np.uint32) + (2 << 7)).astype(np.uint16)


def test_mla_small_ragged(m):
    d = sparse_inputs_host(2, 16, 3000, 576, 128, 51, [3000, 1500])
    _run(m, d["q"], d["latent"], d["seq_lens"])


def test_mla_single_row_and_partial_subchunks(m):
    """L = 1 (the output is that row's first 512 values), L = 33 and a length
    that ends inside a sub-chunk of the last row range."""
    d = sparse_inputs_host(3, 64, 5000, 576, 128, 52, [5000, 1, 33])
    _run(m, d["q"], d["latent"], d["seq_lens"])
    d = sparse_inputs_host(1, 16, 777, 576, 128, 53, [777])
    _run(m, d["q"], d["latent"], d["seq_lens"])


def test_mla_peaky_two_head_groups(m):
    """128 heads (two workgroups share every row range), a sharp softmax."""
    d = sparse_inputs_host(1, 128, 20000, 576, 128, 54, [20000])
    _run(m, _peaky(d["q"]), d["latent"], d["seq_lens"], heads=[0, 1, 31, 63, 64, 100, 127])


def test_mla_heads_not_a_multiple_of_64(m):
    """48 heads: the last wave of the head group has no heads and only copies."""
    d = sparse_inputs_host(2, 48, 9000, 576, 128, 55, [8999, 4097])
    _run(m, _peaky(d["q"]), d["latent"], d["seq_lens"])


def test_mla_score_jump_takes_the_rescaling_path(m):
    """A row far into a row range whose score for head 0 is ~480 (base 2) above
    the range's first sub-chunk: the workgroup recomputes with rescaling."""
    d = sparse_inputs_host(1, 16, 6000, 576, 128, 57, [6000])
    d["latent"][0, 4164] = (d["q"][0, 0].astype(np.uint32) + (3 << 7)).astype(np.uint16)   # 8 q
    _run(m, d["q"], d["latent"], d["seq_lens"])


def test_mla_matches_full_selection_sparse(m):
    """Dense decode = top-k sparse decode with every row selected (k = L)."""
    import torch
    d = sparse_inputs_host(2, 32, 2048, 576, 128, 56, [2048, 2048])
    lens = torch.from_numpy(d["seq_lens"]).cuda()
    q, lat = to_dev(d["q"]), to_dev(d["latent"])
    dense = from_dev(m.mla_decode(q, lat, lens, SCALE))
    _, sp = m.topk_sparse_decode(q, lat, to_dev(d["q_index"]), to_dev(d["k_index"]), lens, 2048,
                                 SCALE)
    torch.cuda.synchronize()
    assert_close(dense, from_dev(sp), "dense vs full-selection sparse")


def test_mla_full_size_128k(m):
    """B=4, L=128K, H=128 (the 576-dim latent cache of the sparse workload),
    every head against the oracle."""
    import torch
    cfg = SPARSE_128K
    B, H, S = cfg.B, cfg.H, cfg.S_max
    print(f"[case] mla full size B={B} H={H} S={S}", flush=True)
    q = device_randn_bf16((B, H, cfg.Dqk), cfg.seed * 10 + 5)
    lat = device_randn_bf16((B, S, cfg.Dqk), cfg.seed * 10 + 6)
    lens_np = np.array([S, S - 1, 65537, 1000], dtype=np.int32)
    out = m.mla_decode(q, lat, torch.from_numpy(lens_np).cuda(), cfg.scale)
    torch.cuda.synchronize()
    got = from_dev(out)
    qf = bf16_tensor_to_f64(q)
    for b in range(B):
        latb = bf16_tensor_to_f64(lat[b, :lens_np[b]])
        ref = osp.sparse_attention_heads(qf[b], latb, np.arange(lens_np[b]), cfg.scale, cfg.Dv)
        assert_close(got[b], ref, f"full-size every head (b={b})")
        assert_close(got[b], ref, f"full-size every head (b={b}) kernel precision",
                     atol=KERNEL_ATOL, rtol=KERNEL_RTOL)
        rel = np.linalg.norm(got[b] - ref) / np.linalg.norm(ref)
        assert rel < 1e-2, (b, rel)


def test_mla_largest_cache(m):
    """The largest latent cache the ABI accepts: 1,864,135 rows of 1152 bytes
    (2^31 - 128 bytes), every row attended (the last 32-row step holds 7
    rows); the copies of the last rows sit at the 32-bit offset limit.  Every
    head against the oracle."""
    import torch
    B, H, S = 1, 16, 1864135
    print(f"[case] mla largest cache B={B} H={H} S={S}", flush=True)
    q = device_randn_bf16((B, H, 576), 91)
    lat = device_randn_bf16((B, S, 576), 92)
    out = m.mla_decode(q, lat, torch.tensor([S], dtype=torch.int32).cuda(), SCALE)
    torch.cuda.synchronize()
    ref = osp.sparse_attention_heads(bf16_tensor_to_f64(q)[0], bf16_tensor_to_f64(lat[0]),
                                     np.arange(S), SCALE, 512)
    assert_close(from_dev(out)[0], ref, "mla largest cache, every head")
    assert_close(from_dev(out)[0], ref, "mla largest cache, kernel precision", atol=KERNEL_ATOL,
                 rtol=KERNEL_RTOL)

