"""QSA: micro-block selection, then standard sparse GQA over the selected
tokens, float64.

Test infrastructure only (see the package docstring).

The chain follows [attention] Qwen Sparse Attention (QSA) ①-④: the visible
prefix is cut into 4-token micro-blocks, each complete block is summarised by
one block key (the mean of its keys, normalised, rotated at the block's first
position), the indexer heads score the block keys with ReLU and the scores
are summed over the heads, the top 512 blocks are expanded back to their 4
tokens each, the incomplete tail block (0-3 tokens) is appended
unconditionally, and standard GQA attention runs over that token set with
the full-precision cached K and V.

Readings where the pages leave a step open:

* The keys pooled into block keys are the indexer keys (one shared head of
  D_idx dims per token), cached before RoPE: the pooled mean would otherwise
  mix rotations, and the page rotates the block key itself.
* "Normalise" is the L2 normalisation of the mean to unit length (no learned
  parameters are given); a zero mean stays zero.
* RoPE acts on the first rotary_dim dims of the block key at the position of
  the block's first token, 4 j for block j (positions from 0), with the
  scaling settings of the RoPE module; the indexer query heads are supplied
  already rotated at the query's position.
* The block score is the unweighted sum over the indexer heads of
  ReLU(q_h . block_key), as in the page's pseudo-code.
* Top-k over blocks: the 512 largest scores, ties to the lower block index,
  fewer if there are fewer complete blocks; the token list is ascending
  (selected blocks, then the tail) and padded with -1 to 4 * 512 + 3.
* The final attention is the page's Softmax(Q K_sparse^T / sqrt(d_k)) V_sparse
  per query head over the token list, with the head's GQA kv head; the scale
  is an argument, the query is supplied already rotated (the cached keys are
  post-RoPE).
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope
from .attention import attend, kv_head_of
from .sparse import topk_select_exact

BLOCK = 4


def block_keys(k_index, seq_len: int, rope_p) -> np.ndarray:
    """Block key of every complete 4-token block of the first seq_len keys:
    mean, L2-normalised, rotated at the block's first position.

    [attention] QSA ① (group every 4 tokens, mean-pool the keys of a block,
    normalise, RoPE at the block's first position).  Returns [seq_len // 4, D].
    """
    k = np.asarray(k_index, dtype=np.float64)
    nb = seq_len // BLOCK
    mean = k[:BLOCK * nb].reshape(nb, BLOCK, k.shape[1]).mean(axis=1)
    norm = np.linalg.norm(mean, axis=1, keepdims=True)
    unit = np.divide(mean, norm, out=np.zeros_like(mean), where=norm > 0)
    if rope_p is None or nb == 0:
        return unit
    return _rope.rotate_rows(unit, BLOCK * np.arange(nb), rope_p)


def block_scores(q_heads, bkeys) -> np.ndarray:
    """sum over indexer heads h of ReLU(q_h . block_key_j).

    [attention] QSA ① scores (the DSA Lightning Indexer's ReLU multi-head
    scoring applied to blocks instead of tokens, no softmax).
    """
    dots = np.asarray(bkeys, dtype=np.float64) @ np.asarray(q_heads, dtype=np.float64).T
    return np.maximum(dots, 0.0).sum(axis=1)


def select_tokens(scores, seq_len: int, n_blocks: int = 512) -> np.ndarray:
    """Top n_blocks block indices expanded to their 4 tokens, then the tail
    tokens 4 * (seq_len // 4) .. seq_len - 1; ascending, -1 padded to
    4 * n_blocks + 3.

    [attention] QSA ② (Expand & Assembly: lossless expansion of the selected
    blocks, unconditional tail).
    """
    nb = seq_len // BLOCK
    out = np.full(BLOCK * n_blocks + BLOCK - 1, -1, dtype=np.int32)
    toks = []
    if nb > 0:
        sel = topk_select_exact(scores, n_blocks)
        sel = sel[sel >= 0]
        toks = (BLOCK * sel[:, None] + np.arange(BLOCK)[None, :]).reshape(-1).tolist()
    toks += list(range(BLOCK * nb, seq_len))
    out[:len(toks)] = toks
    return out


def qsa_decode(q, k_cache, v_cache, q_index, k_index, seq_lens, scale: float, rope_p,
               n_blocks: int = 512, pairs=None):
    """Whole chain per batch row.  Returns (token_idx [B, 4 n_blocks + 3],
    out [B, Hq, D]); ``pairs`` restricts the attention to (b, h) pairs.

    q [B, Hq, D] (rotated), k_cache/v_cache [B, Hkv, S_max, D] (keys
    post-RoPE), q_index [B, H_I, D_idx] (rotated), k_index [B, S_max, D_idx]
    (pre-RoPE); [attention] QSA ③-④ for the attention over the tokens.
    """
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[1]
    tok = np.full((B, BLOCK * n_blocks + BLOCK - 1), -1, dtype=np.int32)
    out = np.full((B, Hq, v_cache.shape[-1]), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        bk = block_keys(k_index[b], L, rope_p)
        tok[b] = select_tokens(block_scores(q_index[b], bk), L, n_blocks)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        kv = kv_head_of(h, Hq, Hkv)
        t = tok[b][tok[b] >= 0]
        out[b, h] = attend(np.asarray(q[b, h], dtype=np.float64),
                           np.asarray(k_cache[b, kv], dtype=np.float64)[t],
                           np.asarray(v_cache[b, kv], dtype=np.float64)[t], scale)
    return tok, out
