"""Dense grouped-query attention (prefill and single-token decode), float64.

Test infrastructure only (see the package docstring).

Readings where the pages leave a step open:

* q head h reads kv head floor(h / g), g = n_head / n_kv_head: the pages'
  GQA code repeats each K/V head g times along the head axis, copies of one
  head side by side, which gives exactly this map.
* Prefill positions are 0 .. T-1 and row i sees keys j <= i (the pages mask
  the strict upper triangle with -inf).
* A decode step's new token has already been appended to the cache:
  seq_lens[b] rows are visible and the query sits at position seq_lens[b]-1
  (the pages' decode concatenates the new key to the past keys before
  attending).
* Cached keys are stored after RoPE, so decode rotates only q.
* The cache holds bf16, so a decode step that writes its new key attends
  over the key as cached: the rotated key rounded to the nearest bf16 value
  (ties to even), not the unrounded rotation (the pages' decode attends
  over the cache after the new row is concatenated to it).
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope


def round_bf16(x) -> np.ndarray:
    """The nearest bfloat16 value of each element, as float64.

    bfloat16 keeps float32's sign and 8-bit exponent and 7 stored fraction
    bits, i.e. 8 significant bits: in the binade [2^(e-1), 2^e) its values
    are 2^(e-8) apart.  Round to nearest, ties to the even neighbour (the
    one whose last significant bit is 0).  Below bfloat16's smallest normal
    value 2^-126 the spacing stays 2^-133 (its subnormals).  Finite
    results only (no overflow handling: the cached keys are far inside the
    range).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    e = np.maximum(e, -125)                  # subnormal spacing 2^-133
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)   # rint: half to even


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum, over the last axis.

    [注意力变体与MoE] "MQA 与 GQA" (softmax over the key axis).
    """
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q_vec, K, V, scale: float) -> np.ndarray:
    """One query row against the visible keys: softmax(scale * K q) @ V.

    [注意力变体与MoE] "MQA 与 GQA": scores q.k divided by sqrt(hd), softmax,
    then the weighted sum of V.
    """
    s = (np.asarray(K, dtype=np.float64) @ np.asarray(q_vec, dtype=np.float64)) * scale
    return softmax(s) @ np.asarray(V, dtype=np.float64)


def kv_head_of(h: int, n_head: int, n_kv_head: int) -> int:
    """The kv head that q head h reads.

    [注意力变体与MoE] "MQA 与 GQA" and [attention] GQA: each K/V head is
    repeated g = n_head / n_kv_head times along the head axis, consecutive
    copies next to each other, so q head h meets copy h of that expanded axis,
    which is kv head floor(h / g).
    """
    return h // (n_head // n_kv_head)


def visible_keys(i: int, window: int = 0, sinks: int = 0) -> np.ndarray:
    """Key positions query i attends to: 0..i (causal); with a sliding window
    w > 0 only i-w+1..i; with s sink tokens beside a window also 0..s-1 (each
    position once).

    [transformer架构] §2.5.1 (the band mask); [attention] "Slide Window
    Attention (SWA)", 修复方案 1. StreamingLLM: the effective context is the
    first s tokens followed by the sliding window; [transformer架构] §2.5.4
    (StreamingLLM's mask: the band plus the first k columns kept).  Reading:
    the window is the band of §2.5.1 (w keys ending at i), so s = 0 is the
    plain sliding window.
    """
    if not window:
        return np.arange(i + 1)
    lo = max(0, i - window + 1)
    head = np.arange(min(sinks, lo))
    return np.concatenate([head, np.arange(lo, i + 1)]).astype(np.int64)


def causal_attention(q, k, v, scale: float, rows=None, heads=None, window: int = 0,
                     sinks: int = 0) -> np.ndarray:
    """Causal GQA attention on already-rotated inputs.

    q: [B, Hq, T, D]; k: [B, Hkv, T, D]; v: [B, Hkv, T, Dv].  Row i attends to
    keys 0..i, or with a sliding window w > 0 to keys i-w+1..i, plus keys
    0..s-1 with s sink tokens (:func:`visible_keys`).
    ``rows``/``heads`` restrict the computation to a sample; the result then
    holds NaN elsewhere.

    [注意力变体与MoE] "MQA 与 GQA" (the scores above the diagonal are masked
    to -inf); [transformer架构] §2.5.1: the band mask (0 for i-w+1 <= j <= i).
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
                js = visible_keys(i, window, sinks)
                out[b, h, i] = attend(q[b, h, i], k[b, kv, js], v[b, kv, js], scale)
    return out


def prefill_causal(q, k, v, scale: float, rope_p: dict, rows=None, heads=None,
                   window: int = 0, sinks: int = 0) -> np.ndarray:
    """RoPE on Q and K at positions 0..T-1, then causal GQA attention (with a
    sliding window when window > 0, and sink tokens beside it when sinks > 0).

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
    return causal_attention(qr, kr, v, scale, rows=rows, heads=heads, window=window, sinks=sinks)


def decode_one(q_vec, K, V, seq_len: int, scale: float, rope_p) -> np.ndarray:
    """One (batch, q head) decode output: q rotated at position seq_len-1
    attends to the first seq_len rows of its kv head's cache."""
    qv = np.asarray(q_vec, dtype=np.float64)[None, :]
    if rope_p is not None:
        qv = _rope.rotate_rows(qv, np.array([seq_len - 1]), _rope.with_length(rope_p, seq_len))
    return attend(qv[0], K[:seq_len], V[:seq_len], scale)


def decode_group(q_rows, K, V, seq_len: int, scale: float, rope_p) -> np.ndarray:
    """The decode outputs of several query heads that read one kv head: each
    row of q_rows [n, D] is rotated at position seq_len-1 and attends to the
    first seq_len rows of K and V, exactly as :func:`decode_one` does for one
    head (the scores of all rows form one [n, seq_len] product).  Returns
    [n, Dv].

    [注意力变体与MoE] "MQA 与 GQA": the g heads of a group share their K/V
    head, so they see the same keys; [注意力变体与MoE] "生成时的瓶颈" for the
    decode step itself.
    """
    qv = np.asarray(q_rows, dtype=np.float64)
    if rope_p is not None:
        qv = _rope.rotate_rows(qv[None], np.array([seq_len - 1]),
                               _rope.with_length(rope_p, seq_len))[0]
    K = np.asarray(K, dtype=np.float64)[:seq_len]
    V = np.asarray(V, dtype=np.float64)[:seq_len]
    return softmax((qv @ K.T) * scale) @ V


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
    position seq_lens[b]-1 and rounded to bf16 as the cache stores it
    (:func:`round_bf16`), and its value (bf16 already) go into row
    seq_lens[b]-1 of every kv head; returns new (float64) copies of the
    caches.

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
        kc[b, :, pos] = round_bf16(kr)
        vc[b, :, pos] = v_new[b]
    return kc, vc


def decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float, rope_p,
                  pairs=None):
    """One decode step with its cache write: :func:`append_rows`, then
    :func:`decode` over the updated caches.  Returns (out, k_cache', v_cache')."""
    kc, vc = append_rows(k_cache, v_cache, k_new, v_new, seq_lens, rope_p)
    return decode(q, kc, vc, seq_lens, scale, rope_p, pairs=pairs), kc, vc


def sink_slot(t: int, S_max: int, sinks: int = 0) -> int:
    """Slot of position t in a rolling buffer of S_max slots whose first
    `sinks` slots keep positions 0..sinks-1 for good: later positions cycle
    through the other S_max - sinks slots, overwriting the oldest.

    [transformer架构] §2.5.2 (the rolling buffer, position t in slot t mod w)
    with [attention] "Slide Window Attention (SWA)", 修复方案 1 (StreamingLLM
    keeps the sink tokens' KV cache); sinks = 0 is slot t mod S_max.
    """
    t = int(t)
    return t if t < sinks else sinks + (t - sinks) % (S_max - sinks)


def window_rows(seq_len: int, S_max: int, window: int = 0, rolling: bool = False,
                sinks: int = 0):
    """Cache rows the new token (position seq_len-1) attends to.

    Sliding window ([transformer架构] §2.5.1): query i sees keys j with
    i - w + 1 <= j <= i; with s sink tokens also j < s (:func:`visible_keys`).
    Linear cache: position p is row p (window 0 = no window).  Rolling
    buffer ([transformer架构] §2.5.2): position t lives in slot
    :func:`sink_slot`, so the buffer holds the sinks and the last
    S_max - s positions (its ring).  Window 0 attends to all of them (the
    buffer is the window); a window w of at most the ring's S_max - s slots
    attends to the slots of the visible positions, all still in the buffer
    (reading: §2.5.2 sizes the buffer to the window; a smaller window over
    a larger buffer keeps the §2.5.1 band, whose slots may wrap around the
    buffer's end).
    """
    L = int(seq_len)
    if rolling:
        if not 0 <= sinks < S_max:
            raise ValueError("the sinks must leave a ring of at least one slot")
        ring = S_max - sinks
        if not 0 <= window <= ring:
            raise ValueError("a rolling buffer's window must fit its ring of S_max - sinks slots")
        if window:
            positions = visible_keys(L - 1, int(window), sinks)
        else:
            positions = np.concatenate([np.arange(min(sinks, L)),
                                        np.arange(max(sinks, L - ring), L)]).astype(np.int64)
        return np.array([sink_slot(t, S_max, sinks) for t in positions], dtype=np.int64)
    return visible_keys(L - 1, int(window), sinks)


def decode_window(q, k_cache, v_cache, seq_lens, scale: float, rope_p, window: int = 0,
                  rolling: bool = False, pairs=None, sinks: int = 0) -> np.ndarray:
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
        rows = window_rows(L, S_max, window, rolling, sinks)
        qv = np.asarray(q[b, h], dtype=np.float64)[None, :]
        if rope_p is not None:
            qv = _rope.rotate_rows(qv, np.array([L - 1]), _rope.with_length(rope_p, L))
        out[b, h] = attend(qv[0], np.asarray(k_cache[b, kv], np.float64)[rows],
                           np.asarray(v_cache[b, kv], np.float64)[rows], scale)
    return out


def append_rows_window(k_cache, v_cache, k_new, v_new, seq_lens, rope_p, rolling: bool = False,
                       sinks: int = 0):
    """:func:`append_rows` for either cache: the new token (position
    seq_lens[b]-1) goes to row seq_lens[b]-1 of a linear cache, or to slot
    :func:`sink_slot` of a rolling buffer ([transformer架构] §2.5.2: the
    oldest entry is overwritten; sink slots never are)."""
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    S_max = kc.shape[2]
    for b in range(kc.shape[0]):
        pos = int(seq_lens[b]) - 1
        row = sink_slot(pos, S_max, sinks) if rolling else pos
        kr = np.asarray(k_new[b], dtype=np.float64)
        if rope_p is not None:
            kr = _rope.rotate_rows(kr[None], np.array([pos]), _rope.with_length(rope_p, pos + 1))[0]
        kc[b, :, row] = round_bf16(kr)
        vc[b, :, row] = np.asarray(v_new[b], dtype=np.float64)
    return kc, vc


def projected_attention(x, Wq, Wk, Wv, n_head: int, n_kv_head: int) -> np.ndarray:
    """Causal GQA self-attention of a hidden-state sequence, no RoPE, written
    from the definition one output element group at a time.  Output [B, T, C].

    x is [B, T, C] and the projections map C to n_head (Wq) or n_kv_head (Wk,
    Wv) heads of width hd = C / n_head.  For batch b, query position i and
    query head h (columns h*hd .. (h+1)*hd - 1 of the output): the query is
    x[b, i] projected by head h's columns of Wq; it is compared with the keys
    of positions j = 0 .. i, each x[b, j] projected by the columns of kv head
    floor(h / g) of Wk (g = n_head / n_kv_head); the scores are divided by
    sqrt(hd), normalised by softmax, and weight the same positions' values
    (the same kv head's columns of Wv).

    [注意力变体与MoE] "MQA 与 GQA" (the attention function there takes x, the
    three projections and the two head counts; its output keeps x's shape).
    """
    x = np.asarray(x, dtype=np.float64)
    Wq, Wk, Wv = (np.asarray(w, dtype=np.float64) for w in (Wq, Wk, Wv))
    B, T, C = x.shape
    if C % n_head or n_head % n_kv_head:
        raise ValueError("C must split into n_head heads and n_head into n_kv_head groups")
    hd = C // n_head
    g = n_head // n_kv_head
    y = np.zeros((B, T, n_head * hd))
    for b in range(B):
        for h in range(n_head):
            kv = h // g
            cq = slice(h * hd, (h + 1) * hd)
            ckv = slice(kv * hd, (kv + 1) * hd)
            for i in range(T):
                qi = x[b, i] @ Wq[:, cq]
                keys = np.array([x[b, j] @ Wk[:, ckv] for j in range(i + 1)])
                vals = np.array([x[b, j] @ Wv[:, ckv] for j in range(i + 1)])
                y[b, i, cq] = softmax(keys @ qi / np.sqrt(hd)) @ vals
    return y
