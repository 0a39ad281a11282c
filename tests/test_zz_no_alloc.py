"""gqa_decode_noalloc (the decode entry point for callers that cannot
allocate) through the C ABI: two calls in a row on one device, the second
with a smaller input, each bitwise equal to gqa_decode's output on the same
inputs (the same kernels over the same work split, states in the static
scratch instead of a workspace) and within tolerance of the fp64 oracle."""
import math

import numpy as np
import pytest

from helpers import assert_close, from_dev, to_dev
from oracle import attention as oatt
from workloads import ROPE_YARN, bf16_bits_to_f64, decode_inputs_host, rope_settings

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _call_abi(m, q, k, v, sl, scale, rope, out):
    import torch
    B, Hq, D = q.shape
    _, Hkv, S, _ = k.shape
    st = m.lib().gqa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), B, Hq,
                                    Hkv, D, S, float(scale), m.rope_params(rope), out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, m.lib().gqa_status_string(st)


def test_noalloc_decode_two_calls_match_gqa_decode(m):
    import torch
    rope = rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=256)
    cases = [(4, 32, 4, 128, 3000, [3000, 2500, 1777, 9], 401),   # larger first
             (2, 8, 2, 64, 700, [700, 33], 402)]                     # then a smaller one
    for B, Hq, Hkv, D, S, lens, seed in cases:
        print(f"[case] noalloc decode B={B} Hq={Hq} Hkv={Hkv} D={D} S={S} lens={lens}", flush=True)
        d = decode_inputs_host(B, Hq, Hkv, D, S, seed, lens)
        q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
        sl = torch.from_numpy(d["seq_lens"]).cuda()
        scale = 1 / math.sqrt(D)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        _call_abi(m, q, k, v, sl, scale, rope, out)
        ref_dev = m.gqa_decode(q, k, v, sl, scale, q_rope=rope)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_dev), "gqa_decode_noalloc differs from gqa_decode"
        ref = oatt.decode(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["k"]),
                          bf16_bits_to_f64(d["v"]), d["seq_lens"], scale, rope)
        assert_close(from_dev(out), ref, f"noalloc decode B={B} D={D}")


def test_noalloc_decode_rejects_states_beyond_the_scratch(m):
    import torch
    q = torch.zeros((4096, 64, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1, 1, 16), dtype=torch.bfloat16, device="cuda")   # never read
    sl = torch.ones(4096, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    st = m.lib().gqa_decode_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), sl.data_ptr(), 4096,
                                    64, 8, 128, 64, 0.1, None, out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == m.ERR_WORKSPACE_TOO_SMALL
