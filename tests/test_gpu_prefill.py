"""GPU parity of gqa_prefill_causal (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest

from helpers import assert_close, from_dev, to_dev
from oracle import attention as oatt
from workloads import (PREFILL_8K, ROPE_NONE, ROPE_NTK, ROPE_PI, ROPE_PLAIN, ROPE_YARN, TINY,
                       bf16_bits_to_f64, bf16_tensor_to_f64, device_randn_bf16,
                       prefill_inputs_host, rope_settings, tiny_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


@pytest.mark.parametrize("n_kv", TINY.n_kv_options)
def test_prefill_tiny_config(m, n_kv):
    """B=2, T=10, C=64, 8 heads of dim 8, RoPE base 1e4 at positions 0..9."""
    import torch
    d = tiny_inputs(n_kv)
    print(f"[case] tiny n_kv={n_kv}", flush=True)
    out = m.gqa_prefill_causal(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), TINY.scale,
                               rope=TINY.rope())
    torch.cuda.synchronize()
    ref = oatt.prefill_causal(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["k"]),
                              bf16_bits_to_f64(d["v"]), TINY.scale, TINY.rope())
    got = from_dev(out)
    assert got.shape == (2, 8, 10, 8)
    assert_close(got, ref, f"tiny n_kv={n_kv}")
    # merged heads give the page demo's output shape (B, T, C)
    assert got.transpose(0, 2, 1, 3).reshape(2, 10, 64).shape == (2, 10, 64)


CASES = [
    # (B, T, Hq, Hkv, D, rope)
    (2, 300, 8, 2, 128, rope_settings(ROPE_NTK, base=1e6, factor=4.0)),
    (1, 129, 4, 4, 128, rope_settings(ROPE_PLAIN, base=1e4)),            # MHA, ragged tail
    (1, 200, 8, 1, 128, rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=64)),
    (2, 65, 6, 2, 64, rope_settings(ROPE_PI, base=1e4, factor=2.0)),
    (1, 100, 4, 2, 32, rope_settings(ROPE_PLAIN, base=1e4)),
    (1, 70, 2, 1, 16, None),
    (1, 1, 4, 2, 128, rope_settings(ROPE_PLAIN, base=1e4)),              # T = 1
    (1, 64, 2, 2, 128, rope_settings(ROPE_PLAIN, base=1e4, rotary_dim=64)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}Hq{c[2]}Hkv{c[3]}D{c[4]}" for c in CASES])
def test_prefill_parity(m, case):
    import torch
    B, T, Hq, Hkv, D, rope = case
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=31)
    scale = 1 / math.sqrt(D)
    print(f"[case] prefill {case[:5]} rope={rope and rope['scaling']}", flush=True)
    out = m.gqa_prefill_causal(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), scale, rope=rope)
    torch.cuda.synchronize()
    ref = oatt.prefill_causal(bf16_bits_to_f64(p["q"]), bf16_bits_to_f64(p["k"]),
                              bf16_bits_to_f64(p["v"]), scale,
                              rope if rope is not None else rope_settings(ROPE_NONE))
    assert_close(from_dev(out), ref, f"prefill {case[:5]}")


def test_prefill_structured_and_gqa_equals_repeated_mha(m):
    import torch
    B, T, Hq, Hkv, D = 1, 260, 8, 2, 128
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=32)
    rope = rope_settings(ROPE_NTK, base=1e6, factor=4.0)
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    vf = bf16_bits_to_f64(p["v"])
    # V == 1 -> 1
    o = m.gqa_prefill_causal(q, k, torch.ones_like(v), 0.09, rope=rope)
    torch.cuda.synchronize()
    assert_close(from_dev(o), np.ones((B, Hq, T, D)), "V=1")
    # q == 0 -> prefix means of V; row 0 == v_0
    o = from_dev(m.gqa_prefill_causal(torch.zeros_like(q), k, v, 0.09, rope=rope))
    pm = np.cumsum(vf, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    assert_close(o, np.repeat(pm, Hq // Hkv, axis=1), "q=0 prefix mean")
    o = from_dev(m.gqa_prefill_causal(q, k, v, 0.09, rope=rope))
    assert_close(o[:, :, 0], np.repeat(vf[:, :, 0], Hq // Hkv, axis=1), "row 0")
    # GQA == MHA over repeated K/V, bit for bit
    g = Hq // Hkv
    o1 = m.gqa_prefill_causal(q, k, v, 0.09, rope=rope)
    o2 = m.gqa_prefill_causal(q, k.repeat_interleave(g, dim=1).contiguous(),
                              v.repeat_interleave(g, dim=1).contiguous(), 0.09, rope=rope)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_prefill_full_size_8k_sampled_rows(m):
    """T=8192, 32 q heads, 8 kv heads, NTK s=4 base 1e6: sampled output rows."""
    import torch
    cfg = PREFILL_8K
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    print(f"[case] prefill full size T={T}", flush=True)
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 3)
    out = m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope())
    torch.cuda.synchronize()
    got = from_dev(out)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(3)
    samples = [(0, 0), (5, 1), (31, T - 1), (17, 4095), (8, 127), (9, 128)]
    samples += [(int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(10)]
    kf = bf16_tensor_to_f64(k)
    vf = bf16_tensor_to_f64(v)
    qf = bf16_tensor_to_f64(q)
    for h, i in samples:
        kv = h // (Hq // Hkv)
        ref = oatt.prefill_causal(qf[:, h:h + 1, :i + 1], kf[:, kv:kv + 1, :i + 1],
                                  vf[:, kv:kv + 1, :i + 1], cfg.scale, cfg.rope(), rows=[i])
        assert_close(got[:, h, i], ref[:, 0, i], f"full-size row (h={h}, i={i})")


# ---------------------------------------------------------------------------
# gqa_prefill_window: the band mask (row i sees keys i-w+1 .. i)
# ---------------------------------------------------------------------------

WINDOW_CASES = [
    # (B, T, Hq, Hkv, D, window)
    (1, 300, 8, 2, 128, 1),      # each row sees only itself
    (2, 517, 8, 2, 128, 5),      # narrow band: most rows' windows inside one tile
    (1, 400, 4, 4, 128, 64),     # one tile wide
    (1, 400, 4, 1, 128, 65),
    (1, 700, 8, 2, 128, 200),    # band spans several tiles, ragged tail
    (2, 333, 6, 2, 64, 100),     # head dim 64
    (1, 100, 4, 2, 32, 7),
    (1, 150, 4, 2, 128, 150),    # window = T: plain causal
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[f"B{c[0]}T{c[1]}Hq{c[2]}D{c[4]}w{c[5]}"
                                                    for c in WINDOW_CASES])
def test_prefill_window_parity(m, case):
    import torch
    B, T, Hq, Hkv, D, w = case
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=37)
    rope = rope_settings(ROPE_NTK, base=1e6, factor=4.0)
    scale = 1 / math.sqrt(D)
    print(f"[case] prefill window B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} w={w}", flush=True)
    out = m.gqa_prefill_causal(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), scale, rope=rope,
                               window=w)
    torch.cuda.synchronize()
    ref = oatt.prefill_causal(bf16_bits_to_f64(p["q"]), bf16_bits_to_f64(p["k"]),
                              bf16_bits_to_f64(p["v"]), scale, rope, window=w)
    got = from_dev(out)
    assert np.all(np.isfinite(got))
    assert_close(got, ref, f"prefill window {case}")


def test_prefill_window_full_size_8k_sampled_rows(m):
    """The 8K prefill with a 4096-token window: sampled rows, including rows
    whose window starts mid-tile and the first rows that lose early keys."""
    import torch
    cfg = PREFILL_8K
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    w = 4096
    print(f"[case] prefill window full size T={T} w={w}", flush=True)
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 3)
    out = m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), window=w)
    torch.cuda.synchronize()
    got = from_dev(out)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(5)
    samples = [(0, 0), (3, 4095), (4, 4096), (31, T - 1), (7, 5000), (12, 4097 + 63)]
    samples += [(int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(8)]
    kf, vf, qf = bf16_tensor_to_f64(k), bf16_tensor_to_f64(v), bf16_tensor_to_f64(q)
    for h, i in samples:
        kv = h // (Hq // Hkv)
        ref = oatt.prefill_causal(qf[:, h:h + 1, :i + 1], kf[:, kv:kv + 1, :i + 1],
                                  vf[:, kv:kv + 1, :i + 1], cfg.scale, cfg.rope(), rows=[i],
                                  window=w)
        assert_close(got[:, h, i], ref[:, 0, i], f"window full-size row (h={h}, i={i})")
