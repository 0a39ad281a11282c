"""Pins of the QSA oracle ([attention] Qwen Sparse Attention ①-④) against
what the page fixes: the 4-token micro-block, the 512-block budget that
expands to 2048 tokens, the unconditional tail (at most 2051 tokens), the
ReLU multi-head sum, the block key's RoPE at the block start, and the whole
chain reducing to dense GQA decode when every block is selected."""
import numpy as np
import pytest

from oracle import attention as att
from oracle import qsa
from oracle import rope
from workloads import ROPE_NONE, ROPE_PLAIN, rope_settings


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("L", [0 + 1, 2, 3, 4, 7, 8, 4 * 600 + 3, 4 * 600])
def test_expand_and_tail(L):
    """Blocks expand to their 4 tokens, the tail (L mod 4 tokens) is always
    there, the list is ascending, at most 4*512 + 3 = 2051 long."""
    nb = L // 4
    scores = np.arange(nb, dtype=np.float64)[::-1]        # block 0 best
    tok = qsa.select_tokens(scores, L, 512)
    assert tok.shape == (2051,)
    t = tok[tok >= 0]
    assert np.all(np.diff(t) > 0) and np.all(tok[len(t):] == -1)
    n_sel = min(nb, 512)
    assert len(t) == 4 * n_sel + L % 4
    assert list(t[:4 * n_sel]) == list(range(4 * n_sel))   # the best blocks are the first ones
    assert list(t[4 * n_sel:]) == list(range(4 * nb, L))
    if nb >= 512:
        assert len(t) <= 2051 and 4 * 512 == 2048          # the page's budget: 2048 / 4 = 512 blocks


def test_block_key_mean_norm_and_rope_position():
    """A block of four copies of k has block key R(4j) k/|k|; scaling a
    block's keys by c > 0 leaves its key unchanged; a mixed block's key is
    the normalised mean; without RoPE block j is just that."""
    D = 16
    p = rope_settings(ROPE_PLAIN, base=100.0, rotary_dim=8)
    k = _rand((12, D), 1)
    k[4:8] = k[5]                                          # block 1: four copies
    bk = qsa.block_keys(k, 12, p)
    want = rope.rotate_rows((k[5] / np.linalg.norm(k[5]))[None], np.array([4]), p)[0]
    assert np.allclose(bk[1], want, rtol=1e-13, atol=1e-15)
    k2 = k.copy()
    k2[8:12] *= 7.5
    assert np.allclose(qsa.block_keys(k2, 12, p)[2], bk[2], rtol=1e-13, atol=1e-15)
    m0 = k[0:4].mean(axis=0)
    assert np.allclose(qsa.block_keys(k, 12, None)[0], m0 / np.linalg.norm(m0), rtol=1e-14)
    assert np.allclose(np.linalg.norm(bk, axis=1), 1.0)   # rotation keeps the unit length
    assert qsa.block_keys(k, 3, p).shape == (0, D)         # no complete block


def test_scores_relu_per_head_and_relative_position():
    """Two heads q and -q: the score of a block key b is |q . b| (ReLU per
    head, then the sum; summing first would give 0).  With RoPE, a query
    rotated at position m scores block j through m - 4j only."""
    D = 16
    q = _rand((1, D), 2)
    b = _rand((5, D), 3)
    got = qsa.block_scores(np.vstack([q, -q]), b)
    assert np.allclose(got, np.abs(b @ q[0]), rtol=1e-14)
    p = rope_settings(ROPE_PLAIN, base=100.0)
    k = _rand((40, D), 4)
    qh = _rand((3, D), 5)
    s1 = qsa.block_scores(rope.rotate_rows(qh, np.array([30] * 3), p), qsa.block_keys(k, 40, p))
    # shift the query by 8 and the keys by two blocks: block j+2 now sits where block j was
    k_shift = np.vstack([_rand((8, D), 6), k])[:48]
    s2 = qsa.block_scores(rope.rotate_rows(qh, np.array([38] * 3), p), qsa.block_keys(k_shift, 48, p))
    assert np.allclose(s2[2:12], s1[:10], rtol=1e-12, atol=1e-12)


def test_needle_block_is_selected():
    """The block whose keys point along the (rotated-back) query ranks first."""
    D, L = 32, 4000
    p = rope_settings(ROPE_PLAIN, base=1e4)
    k = _rand((L, D), 7) * 0.3
    qv = _rand((1, D), 8)
    j = 517
    k[4 * j:4 * j + 4] = qv[0]
    qh = rope.rotate_rows(qv, np.array([4 * j]), p)       # query at the block's position
    s = qsa.block_scores(qh, qsa.block_keys(k, L, p))
    assert int(np.argmax(s)) == j
    tok = qsa.select_tokens(s, L, 1)
    assert list(tok[tok >= 0]) == [4 * j, 4 * j + 1, 4 * j + 2, 4 * j + 3]


@pytest.mark.parametrize("L", [37, 40, 2])
def test_all_blocks_selected_is_dense_decode(L):
    """With a budget of at least L/4 blocks every token is attended (complete
    blocks plus the tail): the chain equals dense GQA decode."""
    B, Hq, Hkv, S, D, HI = 1, 8, 2, 48, 16, 3
    q, kc, vc = _rand((B, Hq, D), 9), _rand((B, Hkv, S, D), 10), _rand((B, Hkv, S, D), 11)
    qi, ki = _rand((B, HI, 8), 12), _rand((B, S, 8), 13)
    lens = np.array([L])
    tok, out = qsa.qsa_decode(q, kc, vc, qi, ki, lens, 0.3, rope_settings(ROPE_PLAIN, base=1e4),
                              n_blocks=12)
    assert list(tok[0][tok[0] >= 0]) == list(range(L))
    dense = att.decode(q, kc, vc, lens, 0.3, rope_settings(ROPE_NONE))
    assert np.allclose(out, dense, rtol=1e-13, atol=1e-14)
