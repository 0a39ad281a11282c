"""GPU parity of Dynamic NTK RoPE (s = max(1, L_cur / L_train) per call) in
every entry point that rotates, through the C ABI, against the fp64 oracle."""
import math

import numpy as np
import pytest

from helpers import ATOL, RTOL, assert_close, check_every_head, from_dev, to_dev
from oracle import attention as oatt
from oracle import rope as orope
from workloads import (DECODE_32K_YARN, ROPE_DYNAMIC_NTK, ROPE_PLAIN, bf16_bits_to_f64,
                       bf16_tensor_to_f64, decode_inputs_host, device_randn_bf16,
                       prefill_inputs_host, randn_bf16, rope_settings)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _dyn(L_train, base=5e5, **kw):
    return rope_settings(ROPE_DYNAMIC_NTK, base=base, original_max_position=L_train, **kw)


def _bf16_ulp(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7)


def _fails_tolerance(got, ref):
    return np.max(np.abs(got - ref) / (ATOL + RTOL * np.abs(ref))) > 1.0


@pytest.mark.parametrize("D", [128, 64])
def test_dynamic_ntk_decode(m, D):
    """Contexts below, at, just past and far past L_train = 512: each q is
    rotated with its own sequence's s."""
    import torch
    B, Hq, Hkv, S = 4, 16, 2, 900
    lens = np.array([100, 512, 513, 900], dtype=np.int32)
    rope = _dyn(512)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 81, lens)
    print(f"[case] dynamic NTK decode D={D} lens={list(lens)}", flush=True)
    # q = 1 on every dim makes the rotation visible in every score
    q = np.full((B, Hq, D), 0x3F80, dtype=np.uint16)
    q[:, ::2] = d["q"][:, ::2]
    out = m.gqa_decode(to_dev(q), to_dev(d["k"]), to_dev(d["v"]), torch.from_numpy(lens).cuda(),
                       1.0 / math.sqrt(D), q_rope=rope)
    torch.cuda.synchronize()
    got = from_dev(out)
    qf, kf, vf = bf16_bits_to_f64(q), bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"])
    ref = oatt.decode(qf, kf, vf, lens, 1.0 / math.sqrt(D), rope)
    assert_close(got, ref, f"dynamic NTK decode D={D}")
    # the long context's result is not plain RoPE's
    plain = oatt.decode(qf[3:], kf[3:], vf[3:], lens[3:], 1.0 / math.sqrt(D),
                        rope_settings(ROPE_PLAIN, base=5e5))
    assert _fails_tolerance(got[3:], plain)


def test_dynamic_ntk_decode_append(m):
    """The appended key is rotated at L-1 with s(L); the query likewise."""
    import torch
    B, Hq, Hkv, D, S = 3, 16, 2, 128, 800
    lens = np.array([200, 512, 800], dtype=np.int32)
    rope = _dyn(256)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 82, lens)
    rng = np.random.default_rng(83)
    kn, vn = randn_bf16(rng, (B, Hkv, D)), randn_bf16(rng, (B, Hkv, D))
    print(f"[case] dynamic NTK append lens={list(lens)}", flush=True)
    kc, vc = to_dev(d["k"]), to_dev(d["v"])
    out = m.gqa_decode_append(to_dev(d["q"]), to_dev(kn), to_dev(vn), kc, vc,
                              torch.from_numpy(lens).cuda(), 0.09, q_rope=rope)
    torch.cuda.synchronize()
    k0, v0 = bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"])
    ref, kref, _ = oatt.decode_append(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(kn),
                                      bf16_bits_to_f64(vn), k0, v0, lens, 0.09, rope)
    assert_close(from_dev(out), ref, "dynamic NTK append")
    kg = from_dev(kc)
    for b, L in enumerate(lens):
        r = int(L) - 1
        assert np.all(np.abs(kg[b, :, r] - kref[b, :, r]) <= _bf16_ulp(kref[b, :, r])), b


def test_dynamic_ntk_rolling_window(m):
    """A rolling buffer far shorter than the sequence: s from the absolute
    length, not from the buffer size."""
    import torch
    B, Hq, Hkv, D, S = 2, 8, 2, 128, 96
    lens = np.array([150, 2000], dtype=np.int32)
    rope = _dyn(128)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 84, np.minimum(lens, S))
    rng = np.random.default_rng(85)
    kn, vn = randn_bf16(rng, (B, Hkv, D)), randn_bf16(rng, (B, Hkv, D))
    print(f"[case] dynamic NTK rolling lens={list(lens)}", flush=True)
    kc, vc = to_dev(d["k"]), to_dev(d["v"])
    out = m.gqa_decode_window(to_dev(d["q"]), kc, vc, torch.from_numpy(lens).cuda(), 0.09,
                              rolling=True, k_new=to_dev(kn), v_new=to_dev(vn), q_rope=rope)
    torch.cuda.synchronize()
    k0, v0 = bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"])
    kref, vref = oatt.append_rows_window(k0, v0, bf16_bits_to_f64(kn), bf16_bits_to_f64(vn),
                                         lens, rope, rolling=True)
    ref = oatt.decode_window(bf16_bits_to_f64(d["q"]), kref, vref, lens, 0.09, rope, rolling=True)
    assert_close(from_dev(out), ref, "dynamic NTK rolling")


@pytest.mark.parametrize("T", [200, 700])
def test_dynamic_ntk_prefill(m, T):
    """Prefill of T tokens uses s = max(1, T / 256): 1 at T = 200, 2.73 at 700."""
    import torch
    B, Hq, Hkv, D = 1, 4, 2, 128
    rope = _dyn(256, base=1e4)
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=86)
    print(f"[case] dynamic NTK prefill T={T}", flush=True)
    out = m.gqa_prefill_causal(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), 0.09, rope=rope)
    torch.cuda.synchronize()
    ref = oatt.prefill_causal(bf16_bits_to_f64(p["q"]), bf16_bits_to_f64(p["k"]),
                              bf16_bits_to_f64(p["v"]), 0.09, rope)
    assert_close(from_dev(out), ref, f"dynamic NTK prefill T={T}")


def test_dynamic_ntk_rope_apply(m):
    """rope_apply takes L_cur from the setting's current_len."""
    import torch
    rng = np.random.default_rng(87)
    n_tok, H, D = 300, 4, 128
    x = randn_bf16(rng, (n_tok, H, D))
    pos = rng.integers(0, 20000, size=n_tok).astype(np.int32)
    for cur in (3000, 20000):
        rope = _dyn(4096, current_len=cur)
        print(f"[case] dynamic NTK rope_apply current_len={cur}", flush=True)
        out = m.rope_apply(to_dev(x), torch.from_numpy(pos).cuda(), rope)
        torch.cuda.synchronize()
        ref = orope.rotate_rows(bf16_bits_to_f64(x), pos, rope)
        assert_close(from_dev(out), ref, f"dynamic NTK rope_apply {cur}")


def test_dynamic_ntk_decode_full_size_32k(m):
    """The 32K decode workload (ragged 16K-32K contexts) with Dynamic NTK
    from L_train = 8192 (s between 2 and 4 per sequence), every head."""
    import torch
    cfg = DECODE_32K_YARN
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    lens = cfg.seq_lens()
    rope = _dyn(8192, base=cfg.base)
    print(f"[case] dynamic NTK full size B={B} S_max={S}", flush=True)
    q = device_randn_bf16((B, Hq, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 3)
    out = m.gqa_decode(q, k, v, torch.from_numpy(lens).cuda(), cfg.scale, q_rope=rope)
    torch.cuda.synchronize()
    check_every_head(from_dev(out), q, k, v, lens, cfg.scale, rope, Hq, Hkv, "dynamic NTK full size")
