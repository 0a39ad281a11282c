"""Dense grouped-query attention (prefill and single-token decode), float64.

Test infrastructure only (see the package docstring).

Readings where the pages leave a step open:

* q head h reads kv head floor(h / g), g = n_head / n_kv_head: the pages'
  GQA code repeats each K/V head g times along the head axis
  (repeat_interleave / expand+reshape), which gives exactly this map.
* Prefill positions are 0 .. T-1 and row i sees keys j <= i (the pages mask
  the strict upper triangle with -inf).
* A decode step's new token has already been appended to the cache:
  seq_lens[b] rows are visible and the query sits at position seq_lens[b]-1
  (the pages' decode concatenates the new key to the past keys before
  attending).
* Cached keys are stored after RoPE, so decode rotates only q.
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum, over the last axis.

    [注意力变体与MoE] "MQA 与 GQA", attention(): s.softmax(-1).
    """
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q_vec, K, V, scale: float) -> np.ndarray:
    """One query row against the visible keys: softmax(scale * K q) @ V.

    [注意力变体与MoE] "MQA 与 GQA", attention(): s = q k^T / sqrt(hd), softmax,
    then the weighted sum of V.
    """
    s = (np.asarray(K, dtype=np.float64) @ np.asarray(q_vec, dtype=np.float64)) * scale
    return softmax(s) @ np.asarray(V, dtype=np.float64)


def kv_head_of(h: int, n_head: int, n_kv_head: int) -> int:
    """The kv head that q head h reads.

    [注意力变体与MoE] "MQA 与 GQA": k.repeat_interleave(g, dim=1), g = n_head //
    n_kv_head; [attention] GQA code: unsqueeze(2).expand(...).reshape(...).
    """
    return h // (n_head // n_kv_head)


def causal_attention(q, k, v, scale: float, rows=None, heads=None, window: int = 0) -> np.ndarray:
    """Causal GQA attention on already-rotated inputs.

    q: [B, Hq, T, D]; k: [B, Hkv, T, D]; v: [B, Hkv, T, Dv].  Row i attends to
    keys 0..i, or with a sliding window w > 0 to keys i-w+1..i.
    ``rows``/``heads`` restrict the computation to a sample; the result then
    holds NaN elsewhere.

    [注意力变体与MoE] "MQA 与 GQA", attention(): masked_fill(triu(1), -inf);
    [transformer架构] §2.5.1: the band mask (0 for i-w+1 <= j <= i).
    """
    B, Hq, T, _ = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("n_head must be a multiple of n_kv_head")
    rows = range(T) if rows is None else rows
    heads = range(Hq) if heads is None else heads
    out = np.full((B, Hq, T, v.shape[-1]), np.nan)
    for b in range(B):
        for h in heads:
            kv = kv_head_of(h, Hq, Hkv)
            for i in rows:
                j0 = max(0, i - window + 1) if window else 0
                out[b, h, i] = attend(q[b, h, i], k[b, kv, j0:i + 1], v[b, kv, j0:i + 1], scale)
    return out


def prefill_causal(q, k, v, scale: float, rope_p: dict, rows=None, heads=None,
                   window: int = 0) -> np.ndarray:
    """RoPE on Q and K at positions 0..T-1, then causal GQA attention (with a
    sliding window when window > 0).

    [transformer架构] §1.1 (rotate Q and K, not V) and §1.2 (scalings);
    attention as in :func:`causal_attention`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    T = q.shape[2]
    pos = np.arange(T)
    rope_p = _rope.with_length(rope_p, T)
    # rotate along the position axis: move T first
    qr = _rope.rotate_rows(q.transpose(2, 0, 1, 3), pos, rope_p).transpose(1, 2, 0, 3)
    kr = _rope.rotate_rows(k.transpose(2, 0, 1, 3), pos, rope_p).transpose(1, 2, 0, 3)
    return causal_attention(qr, kr, v, scale, rows=rows, heads=heads, window=window)


def decode_one(q_vec, K, V, seq_len: int, scale: float, rope_p) -> np.ndarray:
    """One (batch, q head) decode output: q rotated at position seq_len-1
    attends to the first seq_len rows of its kv head's cache."""
    qv = np.asarray(q_vec, dtype=np.float64)[None, :]
    if rope_p is not None:
        qv = _rope.rotate_rows(qv, np.array([seq_len - 1]), _rope.with_length(rope_p, seq_len))
    return attend(qv[0], K[:seq_len], V[:seq_len], scale)


def decode(q, k_cache, v_cache, seq_lens, scale: float, rope_p, pairs=None) -> np.ndarray:
    """Single-token GQA decode over a post-RoPE cache.

    q: [B, Hq, D]; k_cache: [B, Hkv, S_max, D]; v_cache: [B, Hkv, S_max, Dv];
    seq_lens: [B].  ``pairs`` restricts to a list of (b, h); other outputs NaN.

    [注意力变体与MoE] "生成时的瓶颈" (new token's q against all cached K/V) and
    [注意力机制进化史] "解码中的KV Cache" (the new key/value are concatenated to
    the past ones before attending).
    """
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("n_head must be a multiple of n_kv_head")
    out = np.full((B, Hq, v_cache.shape[-1]), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        kv = kv_head_of(h, Hq, Hkv)
        out[b, h] = decode_one(q[b, h], k_cache[b, kv], v_cache[b, kv], int(seq_lens[b]),
                               scale, rope_p)
    return out


def append_rows(k_cache, v_cache, k_new, v_new, seq_lens, rope_p):
    """The decode step's cache write: the new token's key, rotated at its
    position seq_lens[b]-1, and its value go into row seq_lens[b]-1 of every
    kv head; returns new (float64) copies of the caches.

    [注意力机制进化史] "解码中的KV Cache" (the new key and value are
    concatenated to the past ones); [transformer架构] §1.1 (the key is
    rotated at its own position, the value is not).  Keys are cached after
    RoPE, as in :func:`decode`.
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    for b in range(kc.shape[0]):
        pos = int(seq_lens[b]) - 1
        kr = k_new[b]
        if rope_p is not None:
            kr = _rope.rotate_rows(k_new[b][None], np.array([pos]),
                                   _rope.with_length(rope_p, pos + 1))[0]
        kc[b, :, pos] = kr
        vc[b, :, pos] = v_new[b]
    return kc, vc


def decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float, rope_p,
                  pairs=None):
    """One decode step with its cache write: :func:`append_rows`, then
    :func:`decode` over the updated caches.  Returns (out, k_cache', v_cache')."""
    kc, vc = append_rows(k_cache, v_cache, k_new, v_new, seq_lens, rope_p)
    return decode(q, kc, vc, seq_lens, scale, rope_p, pairs=pairs), kc, vc


def window_rows(seq_len: int, S_max: int, window: int = 0, rolling: bool = False):
    """Cache rows the new token (position seq_len-1) attends to.

    Sliding window ([transformer架构] §2.5.1): query i sees keys j with
    i - w + 1 <= j <= i.  Linear cache: position p is row p (window 0 = no
    window).  Rolling buffer ([transformer架构] §2.5.2): position t lives in
    slot t mod S_max, so the buffer holds the last S_max positions and the
    window is the buffer (window must be 0).
    """
    L = int(seq_len)
    if rolling:
        if window:
            raise ValueError("a rolling buffer's window is its size")
        positions = np.arange(max(0, L - S_max), L)
        return positions % S_max
    w = int(window) if window else L
    return np.arange(max(0, L - w), L)


def decode_window(q, k_cache, v_cache, seq_lens, scale: float, rope_p, window: int = 0,
                  rolling: bool = False, pairs=None) -> np.ndarray:
    """Single-token decode over the rows of :func:`window_rows`; q rotated at
    its absolute position seq_lens[b]-1 (keys are cached after RoPE, so a
    rolling buffer needs no re-rotation)."""
    B, Hq, _ = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    out = np.full((B, Hq, v_cache.shape[-1]), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        kv = kv_head_of(h, Hq, Hkv)
        L = int(seq_lens[b])
        rows = window_rows(L, S_max, window, rolling)
        qv = np.asarray(q[b, h], dtype=np.float64)[None, :]
        if rope_p is not None:
            qv = _rope.rotate_rows(qv, np.array([L - 1]), _rope.with_length(rope_p, L))
        out[b, h] = attend(qv[0], np.asarray(k_cache[b, kv], np.float64)[rows],
                           np.asarray(v_cache[b, kv], np.float64)[rows], scale)
    return out


def append_rows_window(k_cache, v_cache, k_new, v_new, seq_lens, rope_p, rolling: bool = False):
    """:func:`append_rows` for either cache: the new token (position
    seq_lens[b]-1) goes to row seq_lens[b]-1 of a linear cache, or to slot
    (seq_lens[b]-1) mod S_max of a rolling buffer ([transformer架构] §2.5.2:
    the oldest entry is overwritten)."""
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    S_max = kc.shape[2]
    for b in range(kc.shape[0]):
        pos = int(seq_lens[b]) - 1
        row = pos % S_max if rolling else pos
        kr = np.asarray(k_new[b], dtype=np.float64)
        if rope_p is not None:
            kr = _rope.rotate_rows(kr[None], np.array([pos]), _rope.with_length(rope_p, pos + 1))[0]
        kc[b, :, row] = kr
        vc[b, :, row] = np.asarray(v_new[b], dtype=np.float64)
    return kc, vc


def page_attention(x, Wq, Wk, Wv, n_head: int, n_kv_head: int) -> np.ndarray:
    """The pages' whole GQA attention function (projection, head split, K/V
    repeated g times along the head axis, causal softmax, heads merged), with
    no RoPE.  Output [B, T, C].

    [注意力变体与MoE] "MQA 与 GQA", attention(x, Wq, Wk, Wv, n_head, n_kv_head).
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    hd = C // n_head
    q = (x @ np.asarray(Wq, np.float64)).reshape(B, T, n_head, hd).transpose(0, 2, 1, 3)
    k = (x @ np.asarray(Wk, np.float64)).reshape(B, T, n_kv_head, hd).transpose(0, 2, 1, 3)
    v = (x @ np.asarray(Wv, np.float64)).reshape(B, T, n_kv_head, hd).transpose(0, 2, 1, 3)
    g = n_head // n_kv_head
    k = np.repeat(k, g, axis=1)
    v = np.repeat(v, g, axis=1)
    s = (q @ k.transpose(0, 1, 3, 2)) / np.sqrt(hd)
    s = np.where(np.triu(np.ones((T, T), dtype=bool), 1), -np.inf, s)
    y = softmax(s) @ v
    return y.transpose(0, 2, 1, 3).reshape(B, T, C)
