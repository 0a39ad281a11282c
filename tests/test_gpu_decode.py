"""GPU parity of gqa_decode (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest

from helpers import assert_close, check_every_head, from_dev, to_dev
from oracle import attention as oatt
from workloads import (DECODE_4K, DECODE_32K_YARN, ROPE_PLAIN, ROPE_YARN, bf16_bits_to_f64,
                       bf16_tensor_to_f64, decode_inputs_host, device_randn_bf16, rope_settings)

pytestmark = pytest.mark.gpu


def assert_split_agree(a, b, what):
    """Two work splits of one decode agree to one bf16 rounding step of the
    larger output (2^-7 of its magnitude) plus 2e-5 for the fp32 summation
    order."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 2e-5
    err = np.abs(a - b)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (what, worst, float(err[worst]), float(bound[worst]))


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _run_case(m, B, Hq, Hkv, D, S_max, seq_lens, rope, seed, n_parts=None, scale=None):
    import torch
    d = decode_inputs_host(B, Hq, Hkv, D, S_max, seed, seq_lens)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    print(f"[case] B={B} Hq={Hq} Hkv={Hkv} D={D} S_max={S_max} lens={list(seq_lens)} "
          f"rope={rope and rope['scaling']} parts={n_parts} seed={seed}", flush=True)
    out = m.gqa_decode(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]),
                       torch.from_numpy(d["seq_lens"]).cuda(), scale, q_rope=rope,
                       n_parts=n_parts)
    torch.cuda.synchronize()
    ref = oatt.decode(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"]),
                      d["seq_lens"], scale, rope)
    return from_dev(out), ref


CASES = [
    # (B, Hq, Hkv, D, S_max, seq_lens)
    (3, 16, 2, 128, 700, [700, 333, 1]),      # GQA g=8, ragged, a one-row context
    (2, 8, 8, 128, 257, [257, 31]),           # MHA
    (2, 16, 1, 128, 300, [300, 64]),          # MQA g=16
    (1, 32, 1, 128, 200, [130]),              # g=32 (two head blocks)
    (1, 64, 1, 128, 96, [96]),                # g=64 (four head blocks)
    (2, 8, 2, 64, 333, [333, 65]),            # head dim 64
    (2, 12, 4, 128, 129, [129, 33]),          # g=3: partial head block
    # more than 64 sequences: the row space and a range's first context are
    # found by the chunked prefix passes (64 sequences per pass)
    (100, 8, 2, 128, 200, [int(x) for x in np.random.default_rng(15).integers(1, 201, 100)]),
    (130, 8, 1, 64, 96, [int(x) for x in np.random.default_rng(16).integers(1, 97, 130)]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}D{c[3]}" for c in CASES])
def test_decode_parity_small(m, case):
    B, Hq, Hkv, D, S, lens = case
    rope = rope_settings(ROPE_PLAIN, base=500000.0)
    got, ref = _run_case(m, B, Hq, Hkv, D, S, np.array(lens, dtype=np.int32), rope, seed=11)
    assert_close(got, ref, f"decode {case[:5]}")
    if B > 64:   # and with few, long ranges (groups that span many sequences)
        for parts in (1, 7):
            got, ref = _run_case(m, B, Hq, Hkv, D, S, np.array(lens, dtype=np.int32), rope, seed=11,
                                 n_parts=parts)
            assert_close(got, ref, f"decode {case[:5]} parts={parts}")


def test_decode_yarn_and_split_independence(m):
    """The output does not depend on how the rows are cut into work ranges,
    including ranges that span several contexts or hold a single row."""
    rope = rope_settings(ROPE_YARN, base=500000.0, factor=4.0, original_max_position=64)
    lens = np.array([1000, 777, 64, 65], dtype=np.int32)
    outs = []
    for parts in (None, 1, 2, 7, 64, 1000, 5000, 20000):
        got, ref = _run_case(m, 4, 16, 2, 128, 1000, lens, rope, seed=12, n_parts=parts)
        assert_close(got, ref, f"yarn parts={parts}")
        outs.append(got)
    # every split computes the same fp32 sums in another order (differences
    # ~1e-6) and rounds them to bf16 once, so two splits differ by at most one
    # bf16 step of the larger value (2^-7 of it) plus that order difference
    for parts, o in zip((1, 2, 7, 64, 1000, 5000, 20000), outs[1:]):
        assert_split_agree(o, outs[0], f"parts={parts}")


def test_decode_calls_on_two_streams_run_concurrently_and_agree(m):
    """The library keeps no mutable state: two decodes with disjoint buffers
    on two streams (default priority), issued back to back many times, give
    the results of the same calls made one at a time on one stream."""
    import torch
    rope = rope_settings(ROPE_YARN, base=500000.0, factor=4.0, original_max_position=64)
    cases = []
    for seed, lens in ((21, [900, 17, 512]), (22, [64, 1000, 333])):
        h = decode_inputs_host(3, 16, 2, 128, 1000, seed, lens)
        d = [to_dev(h[key]) for key in ("q", "k", "v")]
        cases.append((d, torch.tensor(lens, dtype=torch.int32).cuda()))
    print("[case] decode on two streams", flush=True)
    ref = []
    for (q, k, v), lens in cases:
        ref.append(m.gqa_decode(q, k, v, lens, 0.088, q_rope=rope))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in ref]
    ws = [torch.empty(m.gqa_decode_workspace_size(3, 16, 2, 128, 1000), dtype=torch.uint8,
                      device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(20):
        for i, (((q, k, v), lens), st) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(st):
                m.gqa_decode(q, k, v, lens, 0.088, q_rope=rope, out=outs[i], workspace=ws[i],
                             stream=st)
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o, r)


def test_decode_no_rope_and_gqa_equals_repeated_mha(m):
    """GQA on the GPU equals an MHA run over K/V materialised with each head
    repeated g times (repeat_interleave): bit for bit when the whole row
    space is one group range (n_parts=1) and every context holds a multiple
    of four 32-row tiles (250 and 100 rows: 8 and 4 tiles, the last ragged),
    so each head's tiles go to the same waves and states in both runs;
    within rounding for the default work split (whose range boundaries
    depend on the total row count)."""
    import torch
    B, Hq, Hkv, D, S = 2, 16, 4, 128, 300
    d = decode_inputs_host(B, Hq, Hkv, D, S, 13, [250, 100])
    sl = torch.from_numpy(d["seq_lens"]).cuda()
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    g = Hq // Hkv
    kr = k.repeat_interleave(g, dim=1).contiguous()
    vr = v.repeat_interleave(g, dim=1).contiguous()
    o1 = m.gqa_decode(q, k, v, sl, 0.1, n_parts=1)
    o2 = m.gqa_decode(q, kr, vr, sl, 0.1, n_parts=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    o3 = m.gqa_decode(q, kr, vr, sl, 0.1)
    torch.cuda.synchronize()
    assert_split_agree(from_dev(o3), from_dev(o1), "default split vs one range")
    ref = oatt.decode(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"]),
                      d["seq_lens"], 0.1, None)
    assert_close(from_dev(o1), ref, "no-rope")


def test_decode_structured_cases(m):
    """V == 1 gives 1; q == 0 gives the mean of the visible V rows; a planted
    needle key dominates (outputs of magnitude ~1, where the tolerance bites)."""
    import torch
    B, Hq, Hkv, D, S = 2, 8, 1, 128, 2000
    lens = np.array([2000, 1500], dtype=np.int32)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 14, lens)
    sl = torch.from_numpy(lens).cuda()
    k, v = to_dev(d["k"]), to_dev(d["v"])
    ones = torch.ones_like(v)
    o = m.gqa_decode(to_dev(d["q"]), k, ones, sl, 0.09)
    torch.cuda.synchronize()
    assert_close(from_dev(o), np.ones((B, Hq, D)), "V=1")
    qz = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    o = m.gqa_decode(qz, k, v, sl, 0.09)
    vf = bf16_bits_to_f64(d["v"])
    ref = np.stack([np.repeat(vf[b, 0, :lens[b]].mean(0)[None], Hq, 0) for b in range(B)])
    assert_close(from_dev(o), ref, "q=0 mean")
    # needle: row 777 of batch 0 equals q (scaled up), every other key ~N(0,1)
    q = d["q"].copy()
    kk = d["k"].copy()
    kk[0, 0, 777] = q[0, 0]
    qf = bf16_bits_to_f64(q)
    o = m.gqa_decode(to_dev(q), to_dev(kk), v, sl, 0.5)
    ref = oatt.decode(qf, bf16_bits_to_f64(kk), vf, lens, 0.5, None)
    assert_close(from_dev(o), ref, "needle")
    assert np.abs(ref[0, 0] - vf[0, 0, 777]).max() < 1e-3


def _full_size(m, cfg, k2=0):
    """The workload at full size with guarded output and workspace, run twice
    (bitwise equal); every head against the oracle.  k2 > 0 multiplies q by
    2^k2 on the device (exact in bf16): a sharp softmax."""
    import torch
    from helpers import Guarded
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    lens = cfg.seq_lens()
    print(f"[case] full size B={B} Hq={Hq} Hkv={Hkv} S_max={S} lens={list(lens)} q x{2 ** k2}",
          flush=True)
    q = device_randn_bf16((B, Hq, D), cfg.seed * 10 + 1) * float(2 ** k2)
    k = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 3)
    sl = torch.from_numpy(lens).cuda()
    out = Guarded((B, Hq, D), torch.bfloat16, seed=1)
    ws = Guarded((m.gqa_decode_workspace_size(B, Hq, Hkv, D, S),), torch.uint8, seed=2)
    m.gqa_decode(q, k, v, sl, cfg.scale, q_rope=cfg.rope(), out=out.view, workspace=ws.view)
    out.check("out")
    ws.check("workspace")
    first = out.view.clone()
    m.gqa_decode(q, k, v, sl, cfg.scale, q_rope=cfg.rope(), out=out.view, workspace=ws.view)
    torch.cuda.synchronize()
    assert torch.equal(first, out.view), "two identical calls differ"
    got = from_dev(out.view)
    check_every_head(got, q, k, v, lens, cfg.scale, cfg.rope(), Hq, Hkv, "full size")


def test_decode_full_size_4k(m):
    _full_size(m, DECODE_4K)


def test_decode_full_size_32k_yarn_ragged(m):
    _full_size(m, DECODE_32K_YARN)


@pytest.mark.parametrize("k2", [2, 3])
def test_decode_full_size_peaked(m, k2):
    """Both decode workloads with q x 4 and x 8: outputs O(1), every head."""
    _full_size(m, DECODE_4K, k2)
    _full_size(m, DECODE_32K_YARN, k2)


def test_decode_largest_cache(m):
    """The largest cache the ABI accepts for D = 128: 2^23 - 1 rows per kv
    head (2^31 - 256 bytes of K and of V), every row attended (the last tile
    holds 31 rows), q rotated at position 2^23 - 2.  Byte offsets of the last
    tiles and of the prefetch past them sit at the 32-bit limit; every head
    against the oracle."""
    import torch
    B, Hq, Hkv, D, S = 1, 8, 1, 128, (1 << 23) - 1
    print(f"[case] largest cache B={B} Hq={Hq} Hkv={Hkv} D={D} S_max={S}", flush=True)
    q = device_randn_bf16((B, Hq, D), 71)
    k = device_randn_bf16((B, Hkv, S, D), 72)
    v = device_randn_bf16((B, Hkv, S, D), 73)
    lens = np.array([S], dtype=np.int32)
    rope = rope_settings(ROPE_PLAIN, base=500000.0)
    out = m.gqa_decode(q, k, v, torch.from_numpy(lens).cuda(), 1.0 / math.sqrt(D), q_rope=rope)
    torch.cuda.synchronize()
    check_every_head(from_dev(out), q, k, v, lens, 1.0 / math.sqrt(D), rope, Hq, Hkv,
                     "largest cache")


# ---------------------------------------------------------------------------
# gqa_decode_append: the decode step with its cache write fused
# ---------------------------------------------------------------------------

def _bf16_ulp(x):
    """One bf16 unit in the last place at the magnitude of x (x != 0)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7)


def _check_written_rows(m, kc_dev, vc_dev, k0, v0, kref, kn, vn, lens):
    """Row L-1 of every kv head holds the rotated new key (within one bf16
    unit of the fp64 rotation: the kernel rotates in fp32) and exactly the
    new value; every other row is untouched."""
    kg, vg = from_dev(kc_dev), from_dev(vc_dev)
    for b, L in enumerate(lens):
        r = int(L) - 1
        err = np.abs(kg[b, :, r] - kref[b, :, r])
        assert np.all(err <= _bf16_ulp(kref[b, :, r]) + 1e-30), f"written key row b={b}"
        assert np.array_equal(vg[b, :, r], bf16_bits_to_f64(vn)[b]), f"written value row b={b}"
        kg[b, :, r] = k0[b, :, r]
        vg[b, :, r] = v0[b, :, r]
    assert np.array_equal(kg, k0) and np.array_equal(vg, v0), "rows other than L-1 changed"


APPEND_CASES = [
    # (B, Hq, Hkv, D, S_max, seq_lens, rope)
    (3, 16, 2, 128, 700, [700, 333, 1], "yarn"),    # new row: last of the cache, mid tile, alone
    (4, 8, 8, 128, 130, [32, 33, 64, 65], "plain"),  # new row at both ends of a 32-row tile
    (2, 16, 1, 128, 300, [300, 97], "none"),        # MQA, key stored as given
    (2, 8, 2, 64, 200, [200, 17], "yarn"),          # head dim 64
    (2, 12, 4, 128, 129, [129, 2], "plain"),        # g=3
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}D{c[3]}{c[6]}"
                                                    for c in APPEND_CASES])
def test_decode_append_parity(m, case):
    import torch
    from workloads import ROPE_NONE, randn_bf16
    B, Hq, Hkv, D, S, lens, kind = case
    rope = {"yarn": rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=64),
            "plain": rope_settings(ROPE_PLAIN, base=1e4),
            "none": rope_settings(ROPE_NONE)}[kind]
    lens = np.array(lens, dtype=np.int32)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 31, lens)
    rng = np.random.default_rng(32)
    kn, vn = randn_bf16(rng, (B, Hkv, D)), randn_bf16(rng, (B, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    print(f"[case] append B={B} Hq={Hq} Hkv={Hkv} D={D} lens={list(lens)} rope={kind}", flush=True)
    kc, vc = to_dev(d["k"]), to_dev(d["v"])
    out = m.gqa_decode_append(to_dev(d["q"]), to_dev(kn), to_dev(vn), kc, vc,
                              torch.from_numpy(lens).cuda(), scale, q_rope=rope)
    torch.cuda.synchronize()
    k0, v0 = bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"])
    ref, kref, _ = oatt.decode_append(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(kn),
                                      bf16_bits_to_f64(vn), k0, v0, lens, scale,
                                      None if kind == "none" else rope)
    assert_close(from_dev(out), ref, f"append {case}")
    _check_written_rows(m, kc, vc, k0, v0, kref, kn, vn, lens)


def test_decode_append_then_decode_matches(m):
    """After an append the caches hold the new row: a plain decode over them
    gives the append step's output."""
    import torch
    from workloads import randn_bf16
    B, Hq, Hkv, D, S = 2, 16, 2, 128, 400
    lens = np.array([400, 123], dtype=np.int32)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 41, lens)
    rng = np.random.default_rng(42)
    kn, vn = randn_bf16(rng, (B, Hkv, D)), randn_bf16(rng, (B, Hkv, D))
    rope = rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=64)
    sl = torch.from_numpy(lens).cuda()
    kc, vc, q = to_dev(d["k"]), to_dev(d["v"]), to_dev(d["q"])
    print("[case] append then decode", flush=True)
    o1 = m.gqa_decode_append(q, to_dev(kn), to_dev(vn), kc, vc, sl, 0.1, q_rope=rope)
    o2 = m.gqa_decode(q, kc, vc, sl, 0.1, q_rope=rope)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_decode_append_full_size_32k_yarn_ragged(m):
    import torch
    cfg = DECODE_32K_YARN
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    lens = cfg.seq_lens()
    print(f"[case] append full size B={B} S_max={S}", flush=True)
    q = device_randn_bf16((B, Hq, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 3)
    kn = device_randn_bf16((B, Hkv, D), cfg.seed * 10 + 4)
    vn = device_randn_bf16((B, Hkv, D), cfg.seed * 10 + 5)
    k0, v0 = k.clone(), v.clone()
    sl = torch.from_numpy(lens).cuda()
    out = m.gqa_decode_append(q, kn, vn, k, v, sl, cfg.scale, q_rope=cfg.rope())
    torch.cuda.synchronize()
    # every row but L-1 untouched (compared on the device)
    rows = torch.from_numpy(lens.astype(np.int64) - 1).cuda()
    bi = torch.arange(B, device="cuda")
    k0[bi, :, rows] = k[bi, :, rows]
    v0[bi, :, rows] = v[bi, :, rows]
    assert torch.equal(k0, k) and torch.equal(v0, v)
    assert torch.equal(v[bi, :, rows], vn)
    got = from_dev(out)
    qf, knf, vnf = bf16_tensor_to_f64(q), bf16_tensor_to_f64(kn), bf16_tensor_to_f64(vn)
    g = Hq // Hkv
    for b in range(B):
        L = int(lens[b])
        for kv in range(Hkv):
            kb = bf16_tensor_to_f64(k0[b, kv, :L])      # rows < L-1 as they were
            vb = bf16_tensor_to_f64(v0[b, kv, :L])
            kc, vc = oatt.append_rows(kb[None, None], vb[None, None], knf[b, kv][None, None],
                                      vnf[b, kv][None, None], np.array([L]), cfg.rope())
            ref = oatt.decode_group(qf[b, kv * g:(kv + 1) * g], kc[0, 0], vc[0, 0], L, cfg.scale,
                                    cfg.rope())
            assert_close(got[b, kv * g:(kv + 1) * g], ref, f"append full size (b={b}, kv={kv}, L={L})")
            kw = bf16_tensor_to_f64(k[b, kv, L - 1])
            assert np.all(np.abs(kw - kc[0, 0, L - 1]) <= _bf16_ulp(kc[0, 0, L - 1]))


# ---------------------------------------------------------------------------
# gqa_decode_window: sliding window over a linear cache, rolling buffer
# ---------------------------------------------------------------------------

WINDOW_CASES = [
    # (B, Hq, Hkv, D, S_max, seq_lens, window, rolling, append)
    (3, 16, 2, 128, 700, [700, 333, 9], 64, 0, False),     # window < L and a context shorter than it
    (2, 8, 8, 128, 300, [300, 200], 1, 0, False),          # window 1: the token itself
    (2, 16, 1, 128, 300, [300, 97], 33, 0, True),          # MQA, append, window crossing a tile
    (2, 8, 2, 64, 200, [200, 17], 100, 0, True),           # head dim 64
    (4, 16, 2, 128, 64, [5, 64, 65, 300], 0, 1, False),    # rolling: short, exactly full, wrapped
    (3, 16, 2, 128, 96, [96, 150, 1000], 0, 1, True),      # rolling with the write (slot (L-1) mod S)
    (2, 12, 4, 64, 50, [31, 77], 0, 1, True),              # rolling, g=3, head dim 64
    # rolling with a window shorter than the buffer: all filled slots (5),
    # a band inside the buffer (30) and bands wrapping around its end (65, 70)
    (4, 16, 2, 128, 64, [5, 30, 65, 70], 24, 1, False),
    # ... with the write: the new token's slot is in the wrapped part (130, 100)
    (4, 16, 2, 128, 96, [96, 130, 1010, 100], 40, 1, True),
    (2, 12, 4, 64, 50, [31, 102], 10, 1, True),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[f"B{c[0]}Hq{c[1]}D{c[3]}w{c[6]}r{c[7]}a{int(c[8])}"
                                                    for c in WINDOW_CASES])
def test_decode_window_parity(m, case):
    import torch
    from workloads import randn_bf16
    B, Hq, Hkv, D, S, lens, window, rolling, append = case
    lens = np.array(lens, dtype=np.int32)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 71, np.minimum(lens, S))
    rng = np.random.default_rng(72)
    kn, vn = randn_bf16(rng, (B, Hkv, D)), randn_bf16(rng, (B, Hkv, D))
    rope = rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=64)
    scale = 1.0 / math.sqrt(D)
    print(f"[case] window B={B} Hq={Hq} Hkv={Hkv} D={D} S={S} lens={list(lens)} w={window} "
          f"rolling={rolling} append={append}", flush=True)
    kc, vc = to_dev(d["k"]), to_dev(d["v"])
    out = m.gqa_decode_window(to_dev(d["q"]), kc, vc, torch.from_numpy(lens).cuda(), scale,
                              window=window, rolling=bool(rolling),
                              k_new=to_dev(kn) if append else None,
                              v_new=to_dev(vn) if append else None, q_rope=rope)
    torch.cuda.synchronize()
    k0, v0 = bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"])
    kref, vref = k0, v0
    if append:
        kref, vref = oatt.append_rows_window(k0, v0, bf16_bits_to_f64(kn), bf16_bits_to_f64(vn),
                                             lens, rope, rolling=bool(rolling))
    ref = oatt.decode_window(bf16_bits_to_f64(d["q"]), kref, vref, lens, scale, rope,
                             window=window, rolling=bool(rolling))
    assert_close(from_dev(out), ref, f"window {case}")
    kg, vg = from_dev(kc), from_dev(vc)
    if append:
        for b, L in enumerate(lens):
            r = (int(L) - 1) % S if rolling else int(L) - 1
            assert np.all(np.abs(kg[b, :, r] - kref[b, :, r]) <= _bf16_ulp(kref[b, :, r])), b
            assert np.array_equal(vg[b, :, r], vref[b, :, r]), b
            kg[b, :, r], vg[b, :, r] = k0[b, :, r], v0[b, :, r]
    assert np.array_equal(kg, k0) and np.array_equal(vg, v0), "rows other than the new one changed"


@pytest.mark.parametrize("mode", ["window4096", "rolling4096", "rolling8192w4096"])
def test_decode_window_full_size_32k(m, mode):
    """The 32K workload (ragged 16K-32K contexts, YaRN) with a 4096-token
    sliding window over its linear cache, as a 4096-slot rolling buffer
    (contexts far longer than the buffer), and as an 8192-slot rolling buffer
    with a 4096-token window (wrapping around the buffer's end for about half
    of the contexts), every head against the oracle."""
    import torch
    cfg = DECODE_32K_YARN
    B, Hq, Hkv, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.D
    lens = cfg.seq_lens()
    S, window, rolling = {"window4096": (cfg.S_max, 4096, False), "rolling4096": (4096, 0, True),
                          "rolling8192w4096": (8192, 4096, True)}[mode]
    print(f"[case] window full size {mode}", flush=True)
    q = device_randn_bf16((B, Hq, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 3)
    sl = torch.from_numpy(lens).cuda()
    out = m.gqa_decode_window(q, k, v, sl, cfg.scale, window=window, rolling=rolling,
                              q_rope=cfg.rope())
    torch.cuda.synchronize()
    got = from_dev(out)
    qf = bf16_tensor_to_f64(q)
    g = Hq // Hkv
    from oracle import rope as orope
    for b in range(B):
        L = int(lens[b])
        rows = torch.from_numpy(oatt.window_rows(L, S, window, rolling)).cuda()
        qv = orope.rotate_rows(qf[b][None], np.array([L - 1]), cfg.rope())[0]
        for kv in range(Hkv):
            kb = bf16_tensor_to_f64(k[b, kv][rows])
            vb = bf16_tensor_to_f64(v[b, kv][rows])
            ref = oatt.decode_group(qv[kv * g:(kv + 1) * g], kb, vb, len(rows), cfg.scale, None)
            assert_close(got[b, kv * g:(kv + 1) * g], ref, f"{mode} (b={b}, kv={kv}, L={L})")
