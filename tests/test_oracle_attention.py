"""Pins of the oracle's dense attention (prefill and decode), CPU only."""
import math

import numpy as np
import pytest
import torch

from conftest import golden_rows
from oracle import attention as att
from oracle import rope
from workloads import (ROPE_DYNAMIC_NTK, ROPE_NONE, ROPE_NTK, ROPE_PLAIN, ROPE_YARN, TINY, rope_settings,
                       tiny_inputs)

NO_ROPE = rope_settings(ROPE_NONE)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_softmax_rows_sum_to_one():
    s = _rand((50, 300), 0) * np.array([[1.0], [30.0], [300.0], [1e-3], [700.0]] * 10)
    p = att.softmax(s)
    assert np.all(np.abs(p.sum(-1) - 1.0) < 1e-12)
    assert np.all(p >= 0)
    assert np.allclose(att.softmax(s + 123.0), p, rtol=1e-12, atol=1e-15)


def test_two_key_closed_form():
    """Two visible keys: weights are the logistic of the score gap."""
    rng = np.random.default_rng(1)
    q, k0, k1, v0, v1 = (rng.standard_normal(16) for _ in range(5))
    scale = 0.25
    w0 = 1.0 / (1.0 + math.exp(scale * (q @ k1 - q @ k0)))
    out = att.attend(q, np.stack([k0, k1]), np.stack([v0, v1]), scale)
    assert np.allclose(out, w0 * v0 + (1 - w0) * v1, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("hkv", [8, 2, 1])
def test_gqa_equals_mha_on_repeated_kv(hkv):
    """[注意力变体与MoE] "MQA 与 GQA": GQA is MHA after repeating each K/V head
    g times along the head axis (repeat_interleave)."""
    B, Hq, T, D = 2, 8, 9, 16
    q, k, v = _rand((B, Hq, T, D), 1), _rand((B, hkv, T, D), 2), _rand((B, hkv, T, D), 3)
    g = Hq // hkv
    out = att.causal_attention(q, k, v, 0.3)
    ref = att.causal_attention(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.3)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)
    # decode too
    L = np.array([9, 4])
    od = att.decode(q[:, :, 0], k, v, L, 0.3, None)
    rd = att.decode(q[:, :, 0], np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), L, 0.3, None)
    assert np.allclose(od, rd, rtol=1e-13, atol=1e-14)


def test_mqa_every_head_reads_kv_head_zero():
    B, Hq, T, D = 1, 4, 6, 8
    q, k, v = _rand((B, Hq, T, D), 4), _rand((B, 1, T, D), 5), _rand((B, 1, T, D), 6)
    out = att.causal_attention(q, k, v, 0.5)
    for h in range(Hq):
        one = att.causal_attention(q[:, h:h + 1], k, v, 0.5)
        assert np.allclose(out[:, h], one[:, 0])


def test_matches_torch_sdpa_library_routine():
    """Causal GQA attention equals torch's scaled_dot_product_attention (CPU,
    float64, is_causal, enable_gqa) -- an independent library routine."""
    B, Hq, Hkv, T, D = 2, 8, 2, 37, 32
    q, k, v = _rand((B, Hq, T, D), 7), _rand((B, Hkv, T, D), 8), _rand((B, Hkv, T, D), 9)
    scale = 1 / math.sqrt(D)
    ours = att.causal_attention(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=True, scale=scale, enable_gqa=True).numpy()
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_structured_invariants():
    B, Hq, Hkv, T, D = 1, 4, 2, 12, 16
    q, k, v = _rand((B, Hq, T, D), 10), _rand((B, Hkv, T, D), 11), _rand((B, Hkv, T, D), 12)
    out = att.causal_attention(q, k, v, 0.7)
    # row 0 sees only key 0
    for h in range(Hq):
        assert np.allclose(out[0, h, 0], v[0, h // 2, 0], rtol=1e-14)
    # q = 0: uniform weights -> prefix means
    z = att.causal_attention(np.zeros_like(q), k, v, 0.7)
    pm = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    for h in range(Hq):
        assert np.allclose(z[0, h], pm[0, h // 2], rtol=1e-13, atol=1e-14)
    # V == 1 -> output 1
    ones = att.causal_attention(q, k, np.ones_like(v), 0.7)
    assert np.allclose(ones, 1.0, rtol=1e-14)
    # planted needle: one key aligned with a large q dominates
    qn = np.zeros((1, 1, T, D)); qn[0, 0, -1, 0] = 40.0
    kn = np.zeros((1, 1, T, D)); kn[0, 0, 5, 0] = 1.0
    vn = _rand((1, 1, T, D), 13)
    o = att.causal_attention(qn, kn, vn, 1.0, rows=[T - 1])
    assert np.allclose(o[0, 0, -1], vn[0, 0, 5], atol=1e-15 + 1e-12)


def test_decode_of_last_token_equals_prefill_last_row():
    """Decode against a cache of rope(K) reproduces prefill's last row."""
    B, Hq, Hkv, T, D = 2, 8, 2, 23, 32
    q, k, v = _rand((B, Hq, T, D), 14), _rand((B, Hkv, T, D), 15), _rand((B, Hkv, T, D), 16)
    p = rope_settings(ROPE_YARN, base=1e4, factor=4.0, original_max_position=8)
    pre = att.prefill_causal(q, k, v, 0.2, p, rows=[T - 1])
    kc = rope.rotate_rows(k.transpose(2, 0, 1, 3), np.arange(T), p).transpose(1, 2, 0, 3)
    dec = att.decode(q[:, :, T - 1], kc, v, np.array([T, T]), 0.2, p)
    assert np.allclose(dec, pre[:, :, T - 1], rtol=1e-12, atol=1e-13)
    # a shorter context sees only its prefix: seq_len 7 decode == prefill row 6
    pre6 = att.prefill_causal(q, k, v, 0.2, p, rows=[6])
    dec6 = att.decode(q[:, :, 6], kc, v, np.array([7, 7]), 0.2, p)
    assert np.allclose(dec6, pre6[:, :, 6], rtol=1e-12, atol=1e-13)


def test_round_bf16_is_the_nearest_bf16_value_ties_to_even():
    """Against brute force over explicit bf16 grids (8 significant bits:
    2^(e-1) (1 + j/128) in the binade [2^(e-1), 2^e); spacing 2^-133 below
    2^-126): random values of both signs round to the nearest grid value,
    exact halfway points to the neighbour with even j, grid values to
    themselves; normal results are float32 values with zero low 16 bits;
    below 2^-125 the grid is every multiple of 2^-133."""
    rng = np.random.default_rng(33)
    for e in (-3, 0, 1, 7, 100, -125):
        lo = 2.0 ** (e - 1)
        grid = lo * (1.0 + np.arange(129) / 128.0)
        x = lo * (1.0 + rng.random(4000))
        want = grid[np.argmin(np.abs(x[:, None] - grid[None, :]), axis=1)]
        for sgn in (1.0, -1.0):
            assert np.array_equal(att.round_bf16(sgn * x), sgn * want), e
        half = lo * (1.0 + (2 * np.arange(128) + 1) / 256.0)      # between j and j + 1
        j = np.arange(128)
        even = np.where(j % 2 == 0, grid[j], grid[j + 1])
        assert np.array_equal(att.round_bf16(half), even), e
        assert np.array_equal(att.round_bf16(grid), grid), e
        bits = att.round_bf16(x).astype(np.float32).view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), e
    sub = 2.0 ** -133 * np.arange(0, 257)          # spacing 2^-133 up to 2^-125 (subnormals and the first binade)
    xs = sub[:-1] + 2.0 ** -133 * rng.random(256)
    want = sub[np.argmin(np.abs(xs[:, None] - sub[None, :]), axis=1)]
    assert np.array_equal(att.round_bf16(xs), want)
    assert att.round_bf16(0.0) == 0.0


def test_decode_append_builds_the_prefill_cache():
    """Appending tokens one at a time (rotated key and value written at the
    token's position, then decode) reproduces every prefill row up to the
    bf16 rounding of the cached keys, and the cache it leaves holds
    round_bf16(rope(K)) and V; rows past the new token stay as they were.
    A wrong write position, a missing rotation or a rotation at the wrong
    position moves rows by far more than that rounding (O(0.1) here)."""
    B, Hq, Hkv, T, D = 2, 8, 2, 12, 32
    q, k, v = _rand((B, Hq, T, D), 24), _rand((B, Hkv, T, D), 25), _rand((B, Hkv, T, D), 26)
    p = rope_settings(ROPE_YARN, base=1e4, factor=4.0, original_max_position=8)
    pre = att.prefill_causal(q, k, v, 0.3, p)
    S_max = T + 5
    junk_k, junk_v = _rand((B, Hkv, S_max, D), 27), _rand((B, Hkv, S_max, D), 28)
    kc, vc = junk_k.copy(), junk_v.copy()
    for t in range(T):
        lens = np.array([t + 1] * B)
        out, kc, vc = att.decode_append(q[:, :, t], k[:, :, t], v[:, :, t], kc, vc, lens, 0.3, p)
        assert np.allclose(out, pre[:, :, t], rtol=0, atol=2e-2), t
    krot = rope.rotate_rows(k.transpose(2, 0, 1, 3), np.arange(T), p).transpose(1, 2, 0, 3)
    assert np.array_equal(kc[:, :, :T], att.round_bf16(krot))
    assert np.allclose(kc[:, :, :T], krot, rtol=2.0 ** -8, atol=0)   # half a bf16 unit
    assert np.array_equal(vc[:, :, :T], v)
    assert np.array_equal(kc[:, :, T:], junk_k[:, :, T:])
    assert np.array_equal(vc[:, :, T:], junk_v[:, :, T:])
    # without RoPE a (bf16) key is stored as given
    kb = att.round_bf16(k[:, :, 3])
    kc2, vc2 = att.append_rows(junk_k, junk_v, kb, v[:, :, 3], np.array([5, 9]), None)
    assert np.array_equal(kc2[0, :, 4], kb[0]) and np.array_equal(kc2[1, :, 8], kb[1])
    assert np.array_equal(vc2[0, :, 4], v[0, :, 3]) and np.array_equal(vc2[1, :, 8], v[1, :, 3])


def test_sliding_window_decode_pins():
    """Window 1 attends only to the new token itself (output = its value);
    window 2 is the two-key logistic; a window at least as long as the
    context is plain decode; and the last row of the pages' band-masked
    attention (softmax(QK^T scale + M) V with M = 0 for i-w+1 <= j <= i,
    -inf elsewhere) equals the windowed decode."""
    B, Hq, Hkv, S, D = 2, 4, 2, 40, 16
    q, k, v = _rand((B, Hq, D), 51), _rand((B, Hkv, S, D), 52), _rand((B, Hkv, S, D), 53)
    lens = np.array([40, 23])
    p = rope_settings(ROPE_PLAIN, base=1e4)
    o1 = att.decode_window(q, k, v, lens, 0.3, p, window=1)
    for b in range(B):
        for h in range(Hq):
            assert np.allclose(o1[b, h], v[b, h // 2, lens[b] - 1], rtol=0, atol=1e-15)
    o2 = att.decode_window(q, k, v, lens, 0.3, None, window=2)
    for b in range(B):
        for h in range(Hq):
            L, kv = lens[b], h // 2
            d = 0.3 * (q[b, h] @ k[b, kv, L - 1] - q[b, h] @ k[b, kv, L - 2])
            w_new = 1.0 / (1.0 + math.exp(-d))
            ref = w_new * v[b, kv, L - 1] + (1 - w_new) * v[b, kv, L - 2]
            assert np.allclose(o2[b, h], ref, rtol=1e-13, atol=1e-14)
    assert np.allclose(att.decode_window(q, k, v, lens, 0.3, p, window=64),
                       att.decode(q, k, v, lens, 0.3, p), rtol=0, atol=0)
    w = 7
    ow = att.decode_window(q, k, v, lens, 0.3, p, window=w)
    for b in range(B):
        L = lens[b]
        i = L - 1
        qr = rope.rotate_rows(q[b], np.full(Hq, i), p)
        for h in range(Hq):
            s_ = 0.3 * k[b, h // 2, :L] @ qr[h]
            M = np.where((np.arange(L) >= i - w + 1) & (np.arange(L) <= i), 0.0, -np.inf)
            a = np.exp(s_ + M - np.max(s_ + M))
            assert np.allclose(ow[b, h], (a / a.sum()) @ v[b, h // 2, :L], rtol=1e-12, atol=1e-13)


def test_sliding_window_prefill_pins():
    """Every row of the windowed prefill equals the pages' band-masked
    softmax(QK^T scale + M)V written out as a full matrix; window 1 gives
    out_i = v_i; a window of T or more is plain causal prefill; the last row
    equals the windowed decode of the last token over a cache of rope(K)."""
    B, Hq, Hkv, T, D = 1, 4, 2, 19, 16
    q, k, v = _rand((B, Hq, T, D), 81), _rand((B, Hkv, T, D), 82), _rand((B, Hkv, T, D), 83)
    p = rope_settings(ROPE_YARN, base=1e4, factor=4.0, original_max_position=8)
    w = 5
    got = att.prefill_causal(q, k, v, 0.3, p, window=w)
    qr = rope.rotate_rows(q.transpose(2, 0, 1, 3), np.arange(T), p).transpose(1, 2, 0, 3)
    kr = rope.rotate_rows(k.transpose(2, 0, 1, 3), np.arange(T), p).transpose(1, 2, 0, 3)
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    M = np.where((j >= i - w + 1) & (j <= i), 0.0, -np.inf)
    for h in range(Hq):
        S_ = 0.3 * qr[0, h] @ kr[0, h // 2].T + M
        A = np.exp(S_ - S_.max(1, keepdims=True))
        A /= A.sum(1, keepdims=True)
        assert np.allclose(got[0, h], A @ v[0, h // 2], rtol=1e-12, atol=1e-13)
    one = att.prefill_causal(q, k, v, 0.3, p, window=1)
    assert np.allclose(one, np.repeat(v, Hq // Hkv, axis=1), rtol=0, atol=1e-15)
    assert np.array_equal(att.prefill_causal(q, k, v, 0.3, p, window=T),
                          att.prefill_causal(q, k, v, 0.3, p))
    dec = att.decode_window(q[:, :, T - 1], kr, v, np.array([T]), 0.3, p, window=w)
    assert np.allclose(dec, got[:, :, T - 1], rtol=1e-12, atol=1e-13)


def test_rolling_buffer_equals_linear_cache_with_its_window():
    """Writing position t to slot t mod S of a rolling buffer and attending
    to every filled slot is the linear cache with window S, for contexts
    shorter and longer than the buffer (older positions overwritten)."""
    B, Hq, Hkv, D, S = 3, 4, 1, 16, 16
    lens = np.array([5, 16, 53])
    Lmax = int(lens.max())
    kpos, vpos = _rand((B, Hkv, Lmax, D), 61), _rand((B, Hkv, Lmax, D), 62)
    q = _rand((B, Hq, D), 63)
    p = rope_settings(ROPE_YARN, base=1e4, factor=4.0, original_max_position=8)
    roll_k, roll_v = _rand((B, Hkv, S, D), 64), _rand((B, Hkv, S, D), 65)   # junk in unwritten slots
    for b in range(B):
        for t in range(lens[b]):
            roll_k[b, :, t % S], roll_v[b, :, t % S] = kpos[b, :, t], vpos[b, :, t]
    a = att.decode_window(q, roll_k, roll_v, lens, 0.25, p, rolling=True)
    lin = att.decode_window(q, kpos, vpos, lens, 0.25, p, window=S)
    assert np.allclose(a, lin, rtol=1e-13, atol=1e-14)
    # a window shorter than the buffer: the band's slots wrap around the
    # buffer's end for L = 53 (positions 44..52 of w = 9 sit in slots 12..15
    # and 0..4), and the result is still the linear cache's window
    for w in (1, 5, 9, S):
        a = att.decode_window(q, roll_k, roll_v, lens, 0.25, p, window=w, rolling=True)
        lin = att.decode_window(q, kpos, vpos, lens, 0.25, p, window=w)
        assert np.allclose(a, lin, rtol=1e-13, atol=1e-14)
    assert sorted(att.window_rows(53, S, 9, rolling=True)) == [0, 1, 2, 3, 4, 12, 13, 14, 15]
    with pytest.raises(ValueError):
        att.window_rows(53, S, S + 1, rolling=True)
    # the append step writes slot (L-1) mod S (rolling) or row L-1 (linear)
    kn, vn = _rand((B, Hkv, D), 66), _rand((B, Hkv, D), 67)
    kr, vr = att.append_rows_window(roll_k, roll_v, kn, vn, lens, p, rolling=True)
    for b in range(B):
        slot = (lens[b] - 1) % S
        assert np.array_equal(vr[b, :, slot], vn[b])
        assert np.array_equal(kr[b, :, slot],
                              att.round_bf16(rope.rotate_rows(kn[b], np.full(Hkv, lens[b] - 1), p)))
        others = [r for r in range(S) if r != slot]
        assert np.array_equal(kr[b, :, others], roll_k[b, :, others])


def test_tiny_demo_shapes_and_param_counts():
    """[注意力变体与MoE] "MQA 与 GQA": the demo's printed output shape and K/V
    parameter counts for n_kv_head = 8, 2, 1."""
    for n_kv, ob, ot, oc, params in golden_rows("tiny_attention_demo.txt"):
        d = tiny_inputs(int(n_kv))
        y = att.projected_attention(d["x"], d["wq"], d["wk"], d["wv"], TINY.n_head, int(n_kv))
        assert y.shape == (int(ob), int(ot), int(oc))
        assert d["wk"].size + d["wv"].size == int(params)
        # the element-by-element definition equals the oracle's vectorised,
        # head-mapped causal attention on the projected and split heads
        x = d["x"].astype(np.float64)
        hd = TINY.head_dim

        def split(w, n):
            return (x @ w.astype(np.float64)).reshape(2, 10, n, hd).transpose(0, 2, 1, 3)

        o2 = att.causal_attention(split(d["wq"], 8), split(d["wk"], int(n_kv)),
                                  split(d["wv"], int(n_kv)), 1 / math.sqrt(hd))
        assert np.allclose(o2.transpose(0, 2, 1, 3).reshape(2, 10, 64), y, rtol=1e-12, atol=1e-13)


def test_decode_group_equals_per_head_decode_and_sdpa():
    """decode_group (the g heads of one kv head at once) equals decode_one per
    head, and torch's scaled_dot_product_attention (CPU float64) on the
    rotated query rows -- an independent library routine."""
    n, L, D = 8, 57, 32
    qr, K, V = _rand((n, D), 81), _rand((70, D), 82), _rand((70, D), 83)
    p = rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=16)
    got = att.decode_group(qr, K, V, L, 0.2, p)
    for h in range(n):
        assert np.allclose(got[h], att.decode_one(qr[h], K, V, L, 0.2, p), rtol=1e-13, atol=1e-15)
    qrot = rope.rotate_rows(qr[None], np.array([L - 1]), p)[0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qrot)[None, :, None], torch.from_numpy(K[:L])[None, None].expand(1, n, L, D),
        torch.from_numpy(V[:L])[None, None].expand(1, n, L, D), scale=0.2).numpy()[0, :, 0]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_prefill_rope_is_relative():
    """Shifting every position by the same amount leaves prefill unchanged
    (RoPE scores depend only on n - m)."""
    B, Hq, Hkv, T, D = 1, 2, 1, 8, 16
    q, k, v = _rand((B, Hq, T, D), 17), _rand((B, Hkv, T, D), 18), _rand((B, Hkv, T, D), 19)
    p = rope_settings(ROPE_PLAIN, base=1e4)
    out = att.prefill_causal(q, k, v, 0.25, p)
    sh = 1000
    qr = rope.rotate_rows(q.transpose(2, 0, 1, 3), np.arange(T) + sh, p).transpose(1, 2, 0, 3)
    kr = rope.rotate_rows(k.transpose(2, 0, 1, 3), np.arange(T) + sh, p).transpose(1, 2, 0, 3)
    assert np.allclose(att.causal_attention(qr, kr, v, 0.25), out, rtol=1e-10, atol=1e-12)


def test_dynamic_ntk_uses_each_calls_length():
    """Dynamic NTK ([transformer架构] §1.2 ④) in the attention steps: a decode
    step rotates q (and an appended key) with s from its own sequence's
    length, a prefill with s from T.  Sequences no longer than L_train match
    plain RoPE, longer ones match NTK at s = L / L_train."""
    B, Hq, Hkv, S_max, D, L_train = 3, 4, 2, 24, 16, 8
    q, kc, vc = _rand((B, Hq, D), 61), _rand((B, Hkv, S_max, D), 62), _rand((B, Hkv, S_max, D), 63)
    dyn = rope_settings(ROPE_DYNAMIC_NTK, base=1e4, original_max_position=L_train)
    lens = np.array([5, 8, 20])
    got = att.decode(q, kc, vc, lens, 0.3, dyn)
    plain = att.decode(q, kc, vc, lens, 0.3, rope_settings(ROPE_PLAIN, base=1e4))
    ntk = att.decode(q, kc, vc, lens, 0.3, rope_settings(ROPE_NTK, base=1e4, factor=2.5))
    assert np.array_equal(got[:2], plain[:2]) and np.array_equal(got[2], ntk[2])
    assert not np.allclose(got[2], plain[2])
    # windowed decode and the appended key follow the same rule
    gw = att.decode_window(q, kc, vc, lens, 0.3, dyn, window=4)
    nw = att.decode_window(q, kc, vc, lens, 0.3, rope_settings(ROPE_NTK, base=1e4, factor=2.5),
                           window=4)
    assert np.array_equal(gw[2], nw[2])
    kn, vn = _rand((B, Hkv, D), 64), _rand((B, Hkv, D), 65)
    k1, _ = att.append_rows(kc, vc, kn, vn, lens, dyn)
    k2, _ = att.append_rows(kc, vc, kn, vn, lens, rope_settings(ROPE_NTK, base=1e4, factor=2.5))
    k3, _ = att.append_rows(kc, vc, kn, vn, lens, rope_settings(ROPE_PLAIN, base=1e4))
    assert np.array_equal(k1[2], k2[2]) and np.array_equal(k1[:2], k3[:2])
    # prefill: s from T
    T = 20
    qp, kp, vp = _rand((1, Hq, T, D), 66), _rand((1, Hkv, T, D), 67), _rand((1, Hkv, T, D), 68)
    pd = att.prefill_causal(qp, kp, vp, 0.3, dyn)
    pn = att.prefill_causal(qp, kp, vp, 0.3, rope_settings(ROPE_NTK, base=1e4, factor=2.5))
    assert np.array_equal(pd, pn)
    ps = att.prefill_causal(qp[:, :, :6], kp[:, :, :6], vp[:, :, :6], 0.3, dyn)
    pp = att.prefill_causal(qp[:, :, :6], kp[:, :, :6], vp[:, :, :6], 0.3,
                            rope_settings(ROPE_PLAIN, base=1e4))
    assert np.array_equal(ps, pp)


def _band_sink_mask(T, w, s):
    """The StreamingLLM mask written from its description: row i keeps the
    band i-w+1 <= j <= i ([transformer架构] §2.5.1) and the first s columns
    (§2.5.4), never a column past the diagonal."""
    m = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            m[i, j] = j <= i and (i - w + 1 <= j or j < s)
    return m


@pytest.mark.parametrize("w,s", [(5, 2), (1, 1), (8, 3), (3, 9)])
def test_sink_window_equals_sdpa_with_the_page_mask(w, s):
    """Prefill with s sink tokens and a window of w equals torch's
    scaled_dot_product_attention (CPU, float64) given the band-plus-first-s-
    columns boolean mask -- an independent routine fed the mask itself."""
    B, Hq, Hkv, T, D = 1, 4, 2, 23, 16
    q, k, v = _rand((B, Hq, T, D), 91), _rand((B, Hkv, T, D), 92), _rand((B, Hkv, T, D), 93)
    ours = att.causal_attention(q, k, v, 0.3, window=w, sinks=s)
    mask = torch.from_numpy(_band_sink_mask(T, w, s))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.3,
        enable_gqa=True).numpy()
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_sink_window_reductions_and_closed_form():
    """s = 0 is the plain sliding window; s + w > i sees every earlier key
    (plain causal); w = 1, s = 1 leaves two keys, 0 and i: the logistic of
    their score gap."""
    B, Hq, Hkv, T, D = 1, 2, 1, 30, 8
    q, k, v = _rand((B, Hq, T, D), 94), _rand((B, Hkv, T, D), 95), _rand((B, Hkv, T, D), 96)
    assert np.array_equal(att.causal_attention(q, k, v, 0.4, window=6, sinks=0),
                          att.causal_attention(q, k, v, 0.4, window=6))
    full = att.causal_attention(q, k, v, 0.4)
    big = att.causal_attention(q, k, v, 0.4, window=20, sinks=10)
    assert np.allclose(big, full, rtol=1e-14, atol=1e-15)
    two = att.causal_attention(q, k, v, 0.4, window=1, sinks=1)
    for i in range(1, T):
        w0 = 1.0 / (1.0 + math.exp(0.4 * (q[0, 0, i] @ k[0, 0, i] - q[0, 0, i] @ k[0, 0, 0])))
        assert np.allclose(two[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, i], rtol=1e-12)
    assert np.allclose(two[0, :, 0], v[0, 0, 0][None])
    assert list(att.visible_keys(9, 3, 2)) == [0, 1, 7, 8, 9]
    assert list(att.visible_keys(4, 3, 4)) == [0, 1, 2, 3, 4]


def test_sink_decode_equals_prefill_rows_and_rolling_sinks():
    """Decode with sinks over a cache of rope(K) reproduces prefill rows; a
    rolling buffer whose first s slots keep the sinks equals the linear cache
    with sinks and a window of S_max - s, and its written slot skips the
    sink slots."""
    B, Hq, Hkv, T, D = 1, 4, 2, 40, 16
    q, k, v = _rand((B, Hq, T, D), 97), _rand((B, Hkv, T, D), 98), _rand((B, Hkv, T, D), 99)
    p = rope_settings(ROPE_PLAIN, base=1e4)
    w, s = 7, 3
    kc = rope.rotate_rows(k.transpose(2, 0, 1, 3), np.arange(T), p).transpose(1, 2, 0, 3)
    for L in (2, 5, 11, 40):
        pre = att.prefill_causal(q, k, v, 0.3, p, rows=[L - 1], window=w, sinks=s)
        dec = att.decode_window(q[:, :, L - 1], kc, v, np.array([L]), 0.3, p, window=w, sinks=s)
        assert np.allclose(dec, pre[:, :, L - 1], rtol=1e-12, atol=1e-13)
    # rolling buffer of S_max = 10 slots, 3 of them sinks: fill it token by token
    # (the write stores the rotated keys as bf16, so the linear cache to match
    # holds them rounded too)
    S_max = 10
    kcb = att.round_bf16(kc)
    rk = np.zeros((B, Hkv, S_max, D))
    rv = np.zeros((B, Hkv, S_max, D))
    for t in range(T):
        rk, rv = att.append_rows_window(rk, rv, k[:, :, t], v[:, :, t], np.array([t + 1]), p,
                                        rolling=True, sinks=s)
        slot = att.sink_slot(t, S_max, s)
        assert slot == (t if t < s else s + (t - s) % (S_max - s))
        dec_r = att.decode_window(q[:, :, t], rk, rv, np.array([t + 1]), 0.3, p, rolling=True,
                                  sinks=s)
        dec_l = att.decode_window(q[:, :, t], kcb, v, np.array([t + 1]), 0.3, p, window=S_max - s,
                                  sinks=s)
        assert np.allclose(dec_r, dec_l, rtol=1e-12, atol=1e-13)
        # windows shorter than the ring of 7 slots (wrapping around it as t grows)
        for wr in (1, 4, 6):
            dec_r = att.decode_window(q[:, :, t], rk, rv, np.array([t + 1]), 0.3, p, window=wr,
                                      rolling=True, sinks=s)
            dec_l = att.decode_window(q[:, :, t], kcb, v, np.array([t + 1]), 0.3, p, window=wr,
                                      sinks=s)
            assert np.allclose(dec_r, dec_l, rtol=1e-12, atol=1e-13)
    for j in range(s):   # the sink slots still hold positions 0..s-1
        assert np.array_equal(rk[:, :, j], kcb[:, :, j]) and np.array_equal(rv[:, :, j], v[:, :, j])
