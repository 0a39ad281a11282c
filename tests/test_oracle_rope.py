"""Pins of the oracle's RoPE against what the pages fix (CPU only)."""
import cmath
import math

import numpy as np
import pytest

from oracle import rope
from workloads import (ROPE_DYNAMIC_NTK, ROPE_NTK, ROPE_PI, ROPE_PLAIN, ROPE_YARN,
                       DECODE_32K_YARN, PREFILL_8K, rope_settings)

SETTINGS = {
    "plain_1e4": rope_settings(ROPE_PLAIN, base=1e4),
    "plain_5e5": rope_settings(ROPE_PLAIN, base=5e5),
    "pi_s4": rope_settings(ROPE_PI, base=1e4, factor=4.0),
    "ntk_s4": rope_settings(ROPE_NTK, base=1e6, factor=4.0),
    "yarn_s4": rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=8192),
    "yarn_s8_1e4": rope_settings(ROPE_YARN, base=1e4, factor=8.0, original_max_position=4096),
}


def _amp(p):
    return rope.yarn_mscale(p["factor"]) if p["scaling"] == ROPE_YARN and p["yarn_mscale"] else 1.0


@pytest.mark.parametrize("name", sorted(SETTINGS))
def test_relative_position_identity(name):
    """[transformer架构] §1.1: R_m^T R_n = R_{n-m}, so scores depend only on n - m."""
    p = SETTINGS[name]
    rng = np.random.default_rng(7)
    D = 128
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    amp = _amp(p)
    for m, n in [(0, 0), (3, 11), (4095, 17), (100, 31000)]:
        ref = rope.rotate_rows(q[None], [m], p)[0] @ rope.rotate_rows(k[None], [n], p)[0]
        # q^T R_{n-m} k, scaled by amp^2 (amp once inside the rotation of k, once here)
        rel = amp * (q @ rope.rotate_rows(k[None], [n - m], p)[0])
        assert abs(ref - rel) <= 1e-9 * (1 + abs(ref))
        for delta in (1, 137, 4095, 24000):
            sh = (rope.rotate_rows(q[None], [m + delta], p)[0]
                  @ rope.rotate_rows(k[None], [n + delta], p)[0])
            assert abs(sh - ref) <= 1e-9 * (1 + abs(ref)), (m, n, delta)


@pytest.mark.parametrize("name", sorted(SETTINGS))
def test_norm_and_position_zero(name):
    p = SETTINGS[name]
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 64))
    amp = _amp(p)
    y = rope.rotate_rows(x, [0, 1, 2, 1000, 32767], p)
    assert np.allclose(np.linalg.norm(y, axis=-1), amp * np.linalg.norm(x, axis=-1), rtol=1e-12)
    assert np.allclose(y[0], amp * x[0], rtol=0, atol=1e-14)


def test_complex_multiply_form_and_page_matrix():
    """Each pair is (x_2i + j x_2i+1) e^{j m theta_i}; equivalently the page's
    2x2 matrix [[cos, -sin], [sin, cos]] acting on the column (x_2i, x_2i+1)."""
    rng = np.random.default_rng(11)
    D, base = 16, 10000.0
    p = rope_settings(ROPE_PLAIN, base=base)
    x = rng.standard_normal(D)
    for m in (0, 1, 5, 77):
        y = rope.rotate_rows(x[None], [m], p)[0]
        for i in range(D // 2):
            th = base ** (-2.0 * i / D)
            z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * m * th)
            assert abs(y[2 * i] - z.real) < 1e-12 and abs(y[2 * i + 1] - z.imag) < 1e-12
            R = np.array([[math.cos(m * th), -math.sin(m * th)],
                          [math.sin(m * th), math.cos(m * th)]])
            assert np.allclose(R @ x[2 * i:2 * i + 2], y[2 * i:2 * i + 2], atol=1e-12)


def test_rotary_dim_subslice_leaves_rest():
    p = rope_settings(ROPE_PLAIN, base=1e4, rotary_dim=8)
    x = np.random.default_rng(0).standard_normal((3, 2, 24))
    y = rope.rotate_rows(x, [0, 5, 9], p)
    assert np.array_equal(y[..., 8:], x[..., 8:])
    assert not np.allclose(y[1:, :, :8], x[1:, :, :8])


def test_first_pair_turns_one_radian_per_position():
    """theta_0 = base^0 = 1 for every base: pair 0 turns by m radians."""
    for base in (1e4, 5e5, 1e6):
        p = rope_settings(ROPE_PLAIN, base=base)
        y = rope.rotate_rows(np.eye(1, 128)[None][0], [3], p)[0]
        assert abs(math.atan2(y[1], y[0]) - 3.0) < 1e-12


@pytest.mark.parametrize("kind", [ROPE_PI, ROPE_NTK, ROPE_YARN])
def test_factor_one_reduces_to_plain(kind):
    base = 5e5
    p = rope_settings(kind, base=base, factor=1.0, original_max_position=8192)
    x = np.random.default_rng(1).standard_normal((4, 2, 128))
    pos = [0, 9, 4095, 30000]
    assert np.allclose(rope.rotate_rows(x, pos, p),
                       rope.rotate_rows(x, pos, rope_settings(ROPE_PLAIN, base=base)),
                       rtol=0, atol=1e-12)


def test_ntk_closed_forms():
    """[transformer架构] §1.2 ②: b' = b s^(d/(d-2)); high dims are compressed like
    PI, low dims are unchanged -- exactly theta'_0 = theta_0 and
    theta'_{d/2-1} = theta_{d/2-1} / s."""
    d, s = PREFILL_8K.D, PREFILL_8K.ntk_factor
    bp = rope.ntk_base(PREFILL_8K.base, s, d)
    assert abs(bp - 4088994.243248622) < 1e-6
    th = rope.base_frequencies(d, PREFILL_8K.base)
    thp = rope.base_frequencies(d, bp)
    assert thp[0] == th[0] == 1.0
    assert abs(thp[-1] / (th[-1] / s) - 1.0) < 1e-12
    # intermediate dims are compressed by s^(2i/(d-2)), strictly between 1 and s
    ratio = th / thp
    assert np.all(np.diff(ratio) > 0) and ratio[0] == 1.0


def test_yarn_bands_reduce_to_pi_and_plain():
    """[transformer架构] §1.2 ③(a): gamma = 0 (r <= alpha) keeps PI's theta/s,
    gamma = 1 (r > beta) keeps theta; (b): sqrt(1/t) = 0.1 ln s + 1."""
    cfg = DECODE_32K_YARN
    p = cfg.rope()
    d, s = cfg.D, p["factor"]
    th = rope.base_frequencies(d, p["base"])
    r = p["original_max_position"] * th / (2 * math.pi)
    g = rope.yarn_ramp(r, 1.0, 32.0)
    ty = rope.yarn_frequencies(d, p["base"], s, p["original_max_position"], 1.0, 32.0)
    hi = np.where(r > 32.0)[0]
    lo = np.where(r <= 1.0)[0]
    mid = np.where((r > 1.0) & (r <= 32.0))[0]
    # band indices for base 5e5, L_train 8192, d = 128
    assert list(hi) == list(range(0, 19))
    assert list(mid) == list(range(19, 35))
    assert list(lo) == list(range(35, 64))
    assert np.all(g[hi] == 1.0) and np.all(g[lo] == 0.0)
    assert np.all((g[mid] > 0) & (g[mid] < 1))
    assert np.array_equal(ty[hi], th[hi])
    assert np.allclose(ty[lo], th[lo] / s, rtol=1e-15)
    # middle band lies between PI and the unscaled frequency
    assert np.all((ty[mid] > th[mid] / s) & (ty[mid] < th[mid]))
    # temperature
    ms = rope.yarn_mscale(4.0)
    assert abs(ms - 1.1386294361119891) < 1e-15
    assert abs(ms * ms - 1.29648) < 1e-5
    # the whole rotation: pairs in the low band equal PI's rotation times mscale,
    # pairs in the high band equal the plain rotation times mscale
    x = np.random.default_rng(5).standard_normal((3, 1, d))
    pos = [1, 1000, 32767]
    yy = rope.rotate_rows(x, pos, p) / ms
    ypi = rope.rotate_rows(x, pos, rope_settings(ROPE_PI, base=p["base"], factor=s))
    ypl = rope.rotate_rows(x, pos, rope_settings(ROPE_PLAIN, base=p["base"]))
    for i in lo:
        assert np.allclose(yy[..., 2 * i:2 * i + 2], ypi[..., 2 * i:2 * i + 2], atol=1e-12)
    for i in hi:
        assert np.allclose(yy[..., 2 * i:2 * i + 2], ypl[..., 2 * i:2 * i + 2], atol=1e-12)


def test_yarn_ramp_reading_values():
    """The linear middle band (a reading: the page gives no formula)."""
    assert rope.yarn_ramp(1.0, 1.0, 32.0) == 0.0
    assert rope.yarn_ramp(32.0, 1.0, 32.0) == 1.0
    assert abs(rope.yarn_ramp(16.5, 1.0, 32.0) - 0.5) < 1e-15
    th = rope.base_frequencies(128, 5e5)
    r19 = 8192 * th[19] / (2 * math.pi)
    assert abs(rope.yarn_ramp(r19, 1.0, 32.0) - (r19 - 1.0) / 31.0) < 1e-15


def test_dynamic_ntk_factor_and_reductions():
    """[transformer架构] §1.2 ④: s = max(1, L_cur / L_train), then the NTK
    formula.  A sequence no longer than L_train keeps the original
    frequencies (s = 1); at 3 L_train the frequencies are NTK's with s = 3; at
    1.5 L_train the lowest frequency is exactly PI-compressed by 1.5 and the
    highest is unchanged."""
    assert rope.dynamic_ntk_factor(100, 4096) == 1.0
    assert rope.dynamic_ntk_factor(4096, 4096) == 1.0
    assert rope.dynamic_ntk_factor(8192, 4096) == 2.0
    assert rope.dynamic_ntk_factor(6144, 4096) == 1.5
    d, base, L_train = 128, 5e5, 4096
    dyn = rope_settings(ROPE_DYNAMIC_NTK, base=base, original_max_position=L_train)
    plain = rope.frequencies_and_scales(rope_settings(ROPE_PLAIN, base=base), d)
    for L in (1, 2000, 4096):
        got = rope.frequencies_and_scales(rope.with_length(dyn, L), d)
        assert np.array_equal(got[0], plain[0]) and got[1:] == (1.0, 1.0)
    ntk3 = rope.frequencies_and_scales(rope_settings(ROPE_NTK, base=base, factor=3.0), d)
    got = rope.frequencies_and_scales(rope.with_length(dyn, 3 * L_train), d)
    assert np.array_equal(got[0], ntk3[0])
    th = rope.frequencies_and_scales(rope.with_length(dyn, 6144), d)[0]
    assert th[0] == 1.0
    assert abs(th[-1] / (base ** (-(d - 2) / d) / 1.5) - 1.0) < 1e-12
    # the length is part of the call: without it the setting is refused
    with pytest.raises(ValueError):
        rope.frequencies_and_scales(dyn, d)
    # other settings pass through with_length unchanged
    p = rope_settings(ROPE_NTK, base=base, factor=2.0)
    assert rope.with_length(p, 99) is p and rope.with_length(None, 5) is None
