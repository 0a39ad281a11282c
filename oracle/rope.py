"""RoPE and its long-context frequency scalings, in float64.

Test infrastructure only (see the package docstring).

Readings where the pages leave a step open:

* A pair is two adjacent dims (2i, 2i+1): the pages split the d dims into d/2
  two-dimensional subspaces without saying which dims pair up.
* The frequency index runs over i = 0 .. rotary_dim/2 - 1 with d = rotary_dim.
* YaRN's middle band is the linear ramp gamma(r) = (r - alpha)/(beta - alpha),
  continuous with 0 at r = alpha and 1 at r = beta.  (parity unpinned: the page
  only says "linear transition".)
* The YaRN temperature multiplies both cos and sin by 0.1 ln s + 1.
* Dynamic NTK's current length L_cur is the length of the sequence at the
  call, the token being processed included: T for a prefill of T tokens,
  seq_lens[b] for a decode step (whose new token sits at seq_lens[b]-1), and
  an explicit ``current_len`` for a plain rotation of given positions.  Every
  rotation a call performs uses that call's s (keys cached by earlier calls
  keep the s they were rotated with).
"""
from __future__ import annotations

import math

import numpy as np

NONE, PLAIN, PI, NTK, YARN, DYNAMIC_NTK = 0, 1, 2, 3, 4, 5


def base_frequencies(rotary_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i = 0 .. d/2-1.

    [transformer架构] §1.1 RoPE 原理, the rotation R(m, theta_i) and its theta_i.
    """
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / rotary_dim)


def ntk_base(base: float, s: float, rotary_dim: int) -> float:
    """b' = b * s^(d/(d-2)).  [transformer架构] §1.2 ② NTK-aware scaling."""
    return float(base) * float(s) ** (rotary_dim / (rotary_dim - 2.0))


def dynamic_ntk_factor(L_cur: int, L_train: int) -> float:
    """s = max(1, L_cur / L_train), recomputed for every call.

    [transformer架构] §1.2 ④ Dynamic NTK: the factor follows the current
    sequence length and is then put into the NTK formula (§1.2 ②); a
    sequence no longer than L_train keeps the original frequencies (s = 1).
    """
    return max(1.0, float(L_cur) / float(L_train))


def with_length(p, L_cur: int):
    """The setting a call with current sequence length L_cur uses: Dynamic
    NTK settings get ``current_len = L_cur``; every other setting (and None)
    is returned as it is."""
    if p is None or int(p["scaling"]) != DYNAMIC_NTK:
        return p
    q = dict(p)
    q["current_len"] = int(L_cur)
    return q


def yarn_ramp(r, alpha: float, beta: float) -> np.ndarray:
    """gamma(r): 0 for r <= alpha, 1 for r > beta, linear in between.

    [transformer架构] §1.2 ③(a), the three-band table (NTK-by-parts).
    """
    r = np.asarray(r, dtype=np.float64)
    mid = (r - alpha) / (beta - alpha)
    return np.where(r > beta, 1.0, np.where(r <= alpha, 0.0, mid))


def yarn_frequencies(rotary_dim: int, base: float, s: float, L_train: int,
                     alpha: float, beta: float) -> np.ndarray:
    """theta^YaRN_i = (1 - gamma(r_i)) theta_i / s + gamma(r_i) theta_i,
    with r_i = L_train theta_i / (2 pi).

    [transformer架构] §1.2 ③(a), r_i and the effective-frequency equation.
    """
    theta = base_frequencies(rotary_dim, base)
    r = L_train * theta / (2.0 * math.pi)
    gamma = yarn_ramp(r, alpha, beta)
    return (1.0 - gamma) * theta / s + gamma * theta


def yarn_mscale(s: float) -> float:
    """sqrt(1/t) = 0.1 ln s + 1.  [transformer架构] §1.2 ③(b) attention temperature."""
    return 0.1 * math.log(s) + 1.0


def effective_rotary_dim(p: dict, head_dim: int) -> int:
    return int(p["rotary_dim"]) if int(p.get("rotary_dim", 0)) else int(head_dim)


def frequencies_and_scales(p: dict, rotary_dim: int):
    """Return (theta[d/2], position_scale, amplitude) for a RoPE setting.

    position_scale multiplies m (PI: m/s); amplitude multiplies cos and sin
    (YaRN temperature).
    """
    kind = int(p["scaling"])
    base = float(p["base"])
    s = float(p.get("factor", 1.0))
    if kind == PLAIN:
        return base_frequencies(rotary_dim, base), 1.0, 1.0
    if kind == PI:
        # [transformer架构] §1.2 ① Position Interpolation: theta unchanged, m -> m/s.
        return base_frequencies(rotary_dim, base), 1.0 / s, 1.0
    if kind == NTK:
        # [transformer架构] §1.2 ②: theta'_i = (b')^(-2i/d).
        return base_frequencies(rotary_dim, ntk_base(base, s, rotary_dim)), 1.0, 1.0
    if kind == DYNAMIC_NTK:
        # [transformer架构] §1.2 ④: s from the call's length, then §1.2 ②.
        L_cur = int(p["current_len"])
        if L_cur < 1:
            raise ValueError("Dynamic NTK needs the call's current length (current_len >= 1)")
        s_dyn = dynamic_ntk_factor(L_cur, int(p["original_max_position"]))
        return base_frequencies(rotary_dim, ntk_base(base, s_dyn, rotary_dim)), 1.0, 1.0
    if kind == YARN:
        theta = yarn_frequencies(rotary_dim, base, s, int(p["original_max_position"]),
                                 float(p["yarn_alpha"]), float(p["yarn_beta"]))
        amp = yarn_mscale(s) if int(p.get("yarn_mscale", 1)) else 1.0
        return theta, 1.0, amp
    raise ValueError(f"unknown RoPE scaling kind {kind}")


def cos_sin(positions, p: dict, rotary_dim: int):
    """cos(m theta_i) and sin(m theta_i) for each position, scaled by the
    amplitude; shapes [n_pos, d/2]."""
    theta, pscale, amp = frequencies_and_scales(p, rotary_dim)
    m = np.asarray(positions, dtype=np.float64) * pscale
    ang = m[:, None] * theta[None, :]
    return amp * np.cos(ang), amp * np.sin(ang)


def rotate_rows(x, positions, p: dict):
    """Apply R(m, theta_i) to the adjacent pairs (x_2i, x_2i+1) of the first
    rotary_dim dims of every row; the remaining dims pass through unchanged.

    x: [n_pos, ..., D] (float64), positions: [n_pos]; returns a new array.

    [transformer架构] §1.1 RoPE 原理: the 2x2 rotation [[cos, -sin], [sin, cos]]
    acting on each pair.  The same section fixes that V is never rotated, so
    callers pass Q and K only.
    """
    x = np.asarray(x, dtype=np.float64)
    if int(p["scaling"]) == NONE:
        return x.copy()
    D = x.shape[-1]
    rd = effective_rotary_dim(p, D)
    c, s = cos_sin(positions, p, rd)                  # [n_pos, rd/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (rd // 2,)
    c = c.reshape(shape)
    s = s.reshape(shape)
    out = x.copy()
    xe = x[..., 0:rd:2]
    xo = x[..., 1:rd:2]
    out[..., 0:rd:2] = xe * c - xo * s
    out[..., 1:rd:2] = xe * s + xo * c
    return out
