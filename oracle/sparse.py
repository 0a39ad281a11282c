"""DSA-style top-k sparse decode over an MLA latent cache, float64.

Test infrastructure only (see the package docstring).

The chain is o = Attn(q, KV[TopK(ReLU(K_I . q_I))]) ([稀疏注意力] "改进一：DSA",
the selection-chain figure), with the single-head, unweighted indexer.

Readings where the pages leave a step open:

* Indexer precision: a score is the exact dot product of the bf16 inputs,
  rounded once to float32, then ReLU.  The float64 dot below is exact for
  these inputs in all but vanishingly rare exponent spreads (each product of
  two bf16 values has 16 significant bits; 128 of them fit in float64's 53
  unless their magnitudes span more than ~30 binades).  Selection compares
  the float32 scores.
* Ties (including the ReLU zeros) go to the lower index; k_eff = min(k, L);
  the selected indices are returned in ascending order and padded with -1.
* Attention over the selected rows equals the pages' -inf index mask followed
  by softmax ([attention] DSA ③ Token-wise Mask), so the oracle attends to the
  gathered rows directly.
* The query is given already absorbed into the latent space (weight
  absorption, [attention] "乘法结合律" 的变换) with its RoPE part already
  rotated; V is the first Dv dims of each latent row.
* The multi-head weighted indexer (the page's formula with H_I heads and
  per-head weights) is kept exact here (float64 dots, ReLU, weighted sum);
  the selection is made on those values, ties to the lower index.  A device
  that sums in float32 can only be checked for a selection that is valid
  within its own rounding bound (see the GPU tests).
"""
from __future__ import annotations

import numpy as np

from .attention import softmax


def indexer_scores(q_index, k_index, seq_len: int) -> np.ndarray:
    """score_j = ReLU(q_I . k_I,j) for j < seq_len, as float32.

    [transformer架构] §2.2(1) Lightning Indexer (one head, weight 1) and
    [稀疏注意力] DSA chain ReLU(K_I . q_I).
    """
    k = np.asarray(k_index, dtype=np.float64)[:seq_len]
    s = (k @ np.asarray(q_index, dtype=np.float64)).astype(np.float32)
    return np.maximum(s, np.float32(0.0))


def topk_select(scores, k: int) -> np.ndarray:
    """Indices of the min(k, len) largest scores, ties to the lower index,
    ascending, padded with -1 to length k.

    [transformer架构] §2.2(2) Top-k 稀疏选择; [attention] DSA ① (Top-K of the
    indexer scores).
    """
    scores = np.asarray(scores, dtype=np.float32)
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores.astype(np.float64)))
    keff = min(k, n)
    sel = np.sort(order[:keff]).astype(np.int32)
    out = np.full(k, -1, dtype=np.int32)
    out[:keff] = sel
    return out


def weighted_indexer_scores(q_index, w_index, k_index, seq_len: int) -> np.ndarray:
    """I_s = sum_j w_j * ReLU(q_j . k_s) over the H_I indexer heads j, for
    s < seq_len, in float64.

    [稀疏注意力] DSA ① Lightning Indexer: H_I query heads q_j (64 on the
    page), one key k_s shared by all heads, a learned weight w_j per head, ReLU
    in place of softmax, summed over the heads.

    q_index: [H_I, D_idx]; w_index: [H_I]; k_index: [L, D_idx].
    """
    k = np.asarray(k_index, dtype=np.float64)[:seq_len]
    dots = k @ np.asarray(q_index, dtype=np.float64).T          # [L, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w_index, dtype=np.float64)


def topk_select_exact(scores, k: int) -> np.ndarray:
    """:func:`topk_select` on float64 scores (no rounding to float32)."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))
    keff = min(k, n)
    out = np.full(k, -1, dtype=np.int32)
    out[:keff] = np.sort(order[:keff]).astype(np.int32)
    return out


def sparse_attention_one(q_vec, latent, idx, scale: float, Dv: int) -> np.ndarray:
    """softmax(scale * q . c_j) over the selected rows j, times c_j[:Dv].

    [attention] DSA ② MQA 等价变换 (every head reads the one latent row) and
    ③ (unselected rows are -inf before the softmax).
    """
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    rows = np.asarray(latent, dtype=np.float64)[idx]
    p = softmax((rows @ np.asarray(q_vec, dtype=np.float64)) * scale)
    return p @ rows[:, :Dv]


def sparse_attention_heads(q_rows, latent, idx, scale: float, Dv: int) -> np.ndarray:
    """:func:`sparse_attention_one` for several heads at once (q_rows [H, Dqk]):
    every head reads the same selected latent rows, so the scores of all heads
    form one [rows, H] product and each head's softmax runs over the rows.
    Returns [H, Dv].

    [attention] DSA ② (the heads share the one latent row) and ③.
    """
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    rows = np.asarray(latent, dtype=np.float64)[idx]
    s = (rows @ np.asarray(q_rows, dtype=np.float64).T) * scale      # [rows, H]
    p = softmax(s.T)                                                 # [H, rows]
    return p @ rows[:, :Dv]


def topk_sparse_decode(q, latent, q_index, k_index, seq_lens, top_k: int, scale: float,
                       Dv: int, batches=None, heads=None):
    """Whole chain per batch row.  Returns (topk_idx [B, k] int32, out [B, H, Dv]).

    ``batches``/``heads`` restrict the attention output to a sample (NaN
    elsewhere); indices are computed for every selected batch row.
    """
    B, H, _ = q.shape
    batches = range(B) if batches is None else batches
    heads = range(H) if heads is None else heads
    idx = np.full((B, top_k), -1, dtype=np.int32)
    out = np.full((B, H, Dv), np.nan)
    for b in batches:
        s = indexer_scores(q_index[b], k_index[b], int(seq_lens[b]))
        idx[b] = topk_select(s, top_k)
        for h in heads:
            out[b, h] = sparse_attention_one(q[b, h], latent[b], idx[b], scale, Dv)
    return idx, out


def mla_dense_decode(q, latent, seq_lens, scale: float, Dv: int, heads=None) -> np.ndarray:
    """Dense absorbed-MLA decode: every head attends to all seq_lens[b] latent
    rows (no selection), scores over the full row, values its first Dv dims.

    [attention] DSA ② (the MQA form of absorbed MLA: every head reads the one
    shared latent row) without the indexer and top-k steps; equivalently
    :func:`sparse_attention_one` with every row selected.
    """
    B, H, _ = q.shape
    heads = range(H) if heads is None else heads
    out = np.full((B, H, Dv), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        for h in heads:
            out[b, h] = sparse_attention_one(q[b, h], latent[b], np.arange(L), scale, Dv)
    return out

