"""GPU parity of rope_apply (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

from helpers import assert_close, from_dev, to_dev
from oracle import rope as orope
from workloads import (ROPE_NONE, ROPE_NTK, ROPE_PI, ROPE_PLAIN, ROPE_YARN, bf16_bits_to_f64,
                       randn_bf16, rope_settings)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


SETTINGS = [
    rope_settings(ROPE_PLAIN, base=1e4),
    rope_settings(ROPE_PI, base=1e4, factor=4.0),
    rope_settings(ROPE_NTK, base=1e6, factor=4.0),
    rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=8192),
    rope_settings(ROPE_YARN, base=1e4, factor=8.0, original_max_position=2048, yarn_mscale=0),
]


@pytest.mark.parametrize("k", range(len(SETTINGS)))
def test_rope_apply_parity(m, k):
    import torch
    p = SETTINGS[k]
    rng = np.random.default_rng(k)
    n_tok, H, D = 300, 4, 128
    x = randn_bf16(rng, (n_tok, H, D))
    pos = rng.integers(0, 40000, size=n_tok).astype(np.int32)
    pos[:3] = [0, 1, 32767]
    print(f"[case] rope kind={p['scaling']} n_tok={n_tok}", flush=True)
    out = m.rope_apply(to_dev(x), torch.from_numpy(pos).cuda(), p)
    torch.cuda.synchronize()
    ref = orope.rotate_rows(bf16_bits_to_f64(x), pos, p)
    assert_close(from_dev(out), ref, f"rope kind {p['scaling']}")


def test_rope_strided_bhtd_inplace_and_subslice(m):
    import torch
    rng = np.random.default_rng(5)
    H, T, D = 3, 50, 64
    x = randn_bf16(rng, (H, T, D))
    xd = to_dev(x)
    view = xd.permute(1, 0, 2)          # [T, H, D] with strides (D, T*D, 1)
    pos = torch.arange(T, dtype=torch.int32, device="cuda") + 7
    p = rope_settings(ROPE_PLAIN, base=1e4, rotary_dim=32)
    m.rope_apply(view, pos, p, out=view)  # in place
    torch.cuda.synchronize()
    ref = orope.rotate_rows(bf16_bits_to_f64(x).transpose(1, 0, 2), np.arange(T) + 7, p)
    got = from_dev(xd).transpose(1, 0, 2)
    assert_close(got, ref, "strided in place")
    assert np.array_equal(got[..., 32:], bf16_bits_to_f64(x).transpose(1, 0, 2)[..., 32:])


def test_rope_mla_rope_slice_out_of_place(m):
    """Rotate only the 64 decoupled-RoPE dims at offset 512 of 576-wide rows."""
    import torch
    rng = np.random.default_rng(6)
    n_tok = 100
    x = randn_bf16(rng, (n_tok, 1, 576))
    xd = to_dev(x)
    out = torch.zeros_like(xd)
    pos = torch.arange(n_tok, dtype=torch.int32, device="cuda") * 1000
    p = rope_settings(ROPE_YARN, base=1e4, factor=40.0, original_max_position=4096)
    m.rope_apply(xd[:, :, 512:], pos, p, out=out[:, :, 512:])
    torch.cuda.synchronize()
    ref = orope.rotate_rows(bf16_bits_to_f64(x)[:, :, 512:], np.arange(n_tok) * 1000, p)
    assert_close(from_dev(out)[:, :, 512:], ref, "mla slice")
    assert np.all(from_dev(out)[:, :, :512] == 0)


def test_rope_none_copies(m):
    import torch
    rng = np.random.default_rng(8)
    x = randn_bf16(rng, (10, 2, 16))
    pos = torch.zeros(10, dtype=torch.int32, device="cuda")
    out = m.rope_apply(to_dev(x), pos, rope_settings(ROPE_NONE))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), bf16_bits_to_f64(x))


@pytest.mark.parametrize("H,n_tok", [(160, 33), (24, 41)])
def test_rope_many_heads_and_ragged_token_groups(m, H, n_tok):
    """Rows wider than one pass of the block (160 heads x 16 chunks > 2048
    chunks: several passes after the cos/sin table), and token groups that do
    not divide the token count (24 heads: 5 tokens per block)."""
    import torch
    rng = np.random.default_rng(H + n_tok)
    D = 128
    x = randn_bf16(rng, (n_tok, H, D))
    pos = rng.integers(0, 70000, size=n_tok).astype(np.int32)
    p = rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=8192, rotary_dim=96)
    print(f"[case] rope H={H} n_tok={n_tok}", flush=True)
    out = m.rope_apply(to_dev(x), torch.from_numpy(pos).cuda(), p)
    torch.cuda.synchronize()
    ref = orope.rotate_rows(bf16_bits_to_f64(x), pos, p)
    got = from_dev(out)
    assert_close(got, ref, f"rope H={H}")
    assert np.array_equal(got[..., 96:], bf16_bits_to_f64(x)[..., 96:])
