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


# whole 128-row query tiles: the first, the two either side of row 4095/4096,
# one in the middle and the last (every head, every row of each)
FULL_TILES = [0, 31, 32, 45, 63]


def _prefill_full(m, window, k2=0):
    import torch
    from helpers import Guarded
    cfg = PREFILL_8K
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    print(f"[case] prefill full size T={T} window={window} q x{2 ** k2}", flush=True)
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 10 + 1) * float(2 ** k2)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 3)
    out = Guarded((B, Hq, T, D), torch.bfloat16, seed=3)
    ws = Guarded((m.gqa_prefill_workspace_size(B, Hkv, T, D, cfg.rope()),), torch.uint8, seed=4)
    m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), out=out.view, workspace=ws.view,
                         window=window)
    out.check("prefill out")
    ws.check("prefill workspace")
    first = out.view.clone()
    m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), out=out.view, workspace=ws.view,
                         window=window)
    torch.cuda.synchronize()
    assert torch.equal(first, out.view), "two identical calls differ"
    got = from_dev(out.view)
    assert np.all(np.isfinite(got))
    rows = [r for t in FULL_TILES for r in range(128 * t, 128 * (t + 1))]
    ref = oatt.prefill_causal(bf16_tensor_to_f64(q), bf16_tensor_to_f64(k), bf16_tensor_to_f64(v),
                              cfg.scale, cfg.rope(), rows=rows, window=window)
    assert_close(got[:, :, rows], ref[:, :, rows], f"prefill full size w={window} x{2 ** k2}")


def test_prefill_window_largest_context(m):
    """The longest prompt the ABI accepts for D = 128 (2^23 - 1 tokens: a kv
    head's K rows are 2^31 - 256 bytes) through a 256-token window: the
    first and last query tiles (the last holds 127 rows) and a tile at row
    2^22 against the oracle.  The oracle rotates at positions 0 .. n-1 of
    the slice it is given; with a window the outputs of a slice starting at
    p0 depend only on position differences (the RoPE identity its CPU tests
    pin), so a slice of the window's rows before the checked ones stands in
    for the whole prompt."""
    import torch
    B, Hq, Hkv, D, T, w = 1, 2, 1, 128, (1 << 23) - 1, 256
    rope = rope_settings(ROPE_NTK, base=1.0e6, factor=4.0)
    scale = 1.0 / math.sqrt(D)
    print(f"[case] prefill largest context T={T} window={w}", flush=True)
    q = device_randn_bf16((B, Hq, T, D), 61)
    k = device_randn_bf16((B, Hkv, T, D), 62)
    v = device_randn_bf16((B, Hkv, T, D), 63)
    out = m.gqa_prefill_causal(q, k, v, scale, rope=rope, window=w)
    torch.cuda.synchronize()
    for r0, r1 in ((0, 128), (1 << 22, (1 << 22) + 128), (T - 127, T)):
        s0 = max(0, r0 - (w - 1))
        sl = slice(s0, r1)
        ref = oatt.prefill_causal(bf16_tensor_to_f64(q[:, :, sl]), bf16_tensor_to_f64(k[:, :, sl]),
                                  bf16_tensor_to_f64(v[:, :, sl]), scale, rope,
                                  rows=range(r0 - s0, r1 - s0), window=w)
        got = from_dev(out[:, :, r0:r1])
        assert_close(got, ref[:, :, r0 - s0:r1 - s0], f"largest context rows {r0}..{r1 - 1}")


def _exp_shift(bits, e):
    """bf16 values times 2^e, exactly (the exponent field moved; zeros kept)."""
    out = bits.astype(np.int32)
    nz = (bits & 0x7FFF) != 0
    out[nz] += e << 7
    return out.astype(np.uint16)


@pytest.mark.parametrize("fp16_scores", [False, True])
def test_prefill_v_at_the_fp16_range_edges(m, fp16_scores):
    """V enters the P.V product as fp16: values near the top of fp16's range
    (|v| up to ~4e4 < 65504) stay exact, so in units of 2^13 the output meets
    the usual tolerance; values near 2^-20 (fp16 subnormals) lose at most
    2^-25 each, so the output errs by at most 2^-25 absolute: checked in
    units of 2^-20 (a flush to zero would miss by ~1)."""
    import torch
    B, T, Hq, Hkv, D = 1, 260, 8, 2, 128
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=33)
    rope = rope_settings(ROPE_NTK, base=1e6, factor=4.0)
    scale = 1 / math.sqrt(D)
    qf, kf = bf16_bits_to_f64(p["q"]), bf16_bits_to_f64(p["k"])
    for e in (13, -20):
        vb = _exp_shift(p["v"], e)
        vf = bf16_bits_to_f64(vb)
        assert np.max(np.abs(vf)) < 65504.0
        print(f"[case] prefill V x 2^{e} fp16_scores={fp16_scores}", flush=True)
        out = m.gqa_prefill_causal(to_dev(p["q"]), to_dev(p["k"]), to_dev(vb), scale, rope=rope,
                                   fp16_scores=fp16_scores)
        torch.cuda.synchronize()
        ref = oatt.prefill_causal(qf, kf, vf, scale, rope)
        got = from_dev(out)
        if e > 0:   # the path is linear in V: in units of 2^e the usual tolerance holds
            assert_close(got * 2.0 ** -e, ref * 2.0 ** -e, f"V x 2^{e} (in units of 2^{e})")
        else:
            err = np.abs(got - ref) * 2.0 ** 20
            bound = 2.0 ** -5 + 1e-2 * np.abs(ref) * 2.0 ** 20
            assert np.all(err <= bound), f"V x 2^{e}: max err/bound {np.max(err / bound):.3f}"


def test_prefill_full_size_8k_whole_tiles(m):
    """T=8192, 32 q heads, 8 kv heads, NTK s=4 base 1e6: every head over five
    whole query tiles; guarded output and workspace; two calls bitwise equal."""
    _prefill_full(m, 0)


def test_prefill_full_size_8k_peaked(m):
    """The same with q x 8 (a sharp softmax)."""
    _prefill_full(m, 0, 3)


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


def test_prefill_window_full_size_8k_whole_tiles(m):
    """The 8K prefill with a 4096-token window over the same whole tiles
    (tile 32 holds the first rows that lose early keys)."""
    _prefill_full(m, 4096)
