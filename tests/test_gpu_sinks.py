"""GPU parity of StreamingLLM sink tokens beside the sliding window
([attention] "Slide Window Attention (SWA)", 修复方案 1; [transformer架构]
§2.5.4: the band mask plus the first k columns): gqa_decode_sink_window over
a linear cache and over a rolling buffer whose first slots keep the sinks,
and gqa_prefill_sink_window, against the fp64 oracle; plus the fp16-score
prefill option on the workloads whose scores spread by about one unit."""
import math

import numpy as np
import pytest

from helpers import Guarded, assert_close, from_dev, to_dev
from oracle import attention as oatt
from oracle import rope as orope
from workloads import (DECODE_32K_YARN, PREFILL_8K, ROPE_NTK, ROPE_YARN, bf16_bits_to_f64,
                       bf16_tensor_to_f64, decode_inputs_host, device_randn_bf16,
                       prefill_inputs_host, randn_bf16, rope_settings)

pytestmark = pytest.mark.gpu
YARN = rope_settings(ROPE_YARN, base=5e5, factor=4.0, original_max_position=64)
NTK = rope_settings(ROPE_NTK, base=1e6, factor=4.0)


@pytest.fixture(scope="module")
def m():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def _bf16_ulp(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7)


DECODE_CASES = [
    # (B, Hq, Hkv, D, S_max, seq_lens, sinks, window, rolling, append)
    (3, 16, 2, 128, 700, [700, 333, 9], 4, 64, 0, False),    # a context shorter than the band
    (2, 8, 8, 128, 300, [300, 200], 1, 1, 0, False),         # two keys: the sink and the token
    (2, 16, 1, 128, 300, [300, 97], 33, 40, 0, True),        # sinks past one tile, append
    (2, 8, 2, 64, 200, [200, 17], 4, 100, 0, True),          # head dim 64
    (2, 12, 4, 128, 300, [300, 70], 64, 64, 0, False),       # two tiles of sinks, g=3
    (2, 16, 2, 128, 2000, [2000, 1999], 4, 1500, 0, True),   # long band, pieces cross the sink end
    (4, 16, 2, 128, 64, [5, 64, 65, 300], 4, 0, 1, False),   # rolling: short, full, wrapped
    (3, 16, 2, 128, 96, [96, 150, 1000], 4, 0, 1, True),     # rolling write skips the sink slots
    (2, 12, 4, 64, 50, [31, 77], 10, 0, 1, True),            # rolling, g=3, head dim 64
    # rolling with a window shorter than the ring: every filled slot (5), a
    # band inside the ring (40, 300), a band wrapping around the buffer's end
    # (65: the first segment is the sinks and slot 4)
    (4, 16, 2, 128, 64, [5, 40, 65, 300], 4, 24, 1, False),
    (3, 16, 2, 128, 96, [96, 130, 1000], 4, 40, 1, True),    # the write lands in the wrapped part (130)
    (2, 12, 4, 64, 50, [31, 102], 10, 20, 1, True),
    # ~128K attended rows: a workgroup's four waves share ranges of 16+ tiles,
    # and context starts (two tiles of sinks, then the band) fall inside them
    (4, 8, 4, 128, 10000, [10000, 9000, 8300, 9999], 40, 8192, 0, True),
    (4, 8, 4, 128, 8192, [20000, 9000, 8192, 12345], 40, 0, 1, True),
    # the same with a 4096-token window: 20000 and 9000 wrap (first segments
    # of 3696 and 848 rows), 8192 and 12345 do not
    (4, 8, 4, 128, 8192, [20000, 9000, 8192, 12345], 40, 4096, 1, True),
    # more than 64 sequences (the chunked prefix passes), sinks, window and the write
    (80, 8, 2, 128, 300, [int(x) for x in np.random.default_rng(17).integers(1, 301, 80)], 4, 100, 0, True),
]


@pytest.mark.parametrize("case", DECODE_CASES,
                         ids=[f"B{c[0]}D{c[3]}s{c[6]}w{c[7]}r{c[8]}a{int(c[9])}" for c in DECODE_CASES])
def test_decode_sink_window_parity(m, case):
    import torch
    B, Hq, Hkv, D, S, lens, sinks, window, rolling, append = case
    lens = np.array(lens, dtype=np.int32)
    d = decode_inputs_host(B, Hq, Hkv, D, S, 301, np.minimum(lens, S))
    rng = np.random.default_rng(302)
    kn, vn = randn_bf16(rng, (B, Hkv, D)), randn_bf16(rng, (B, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    print(f"[case] decode sinks={sinks} w={window} rolling={rolling} append={append} "
          f"B={B} Hq={Hq} Hkv={Hkv} D={D} S={S} lens={list(lens)}", flush=True)
    kc, vc = to_dev(d["k"]), to_dev(d["v"])
    out = m.gqa_decode_window(to_dev(d["q"]), kc, vc, torch.from_numpy(lens).cuda(), scale,
                              window=window, rolling=bool(rolling), sinks=sinks,
                              k_new=to_dev(kn) if append else None,
                              v_new=to_dev(vn) if append else None, q_rope=YARN)
    torch.cuda.synchronize()
    k0, v0 = bf16_bits_to_f64(d["k"]), bf16_bits_to_f64(d["v"])
    kref, vref = k0, v0
    if append:
        kref, vref = oatt.append_rows_window(k0, v0, bf16_bits_to_f64(kn), bf16_bits_to_f64(vn),
                                             lens, YARN, rolling=bool(rolling), sinks=sinks)
    ref = oatt.decode_window(bf16_bits_to_f64(d["q"]), kref, vref, lens, scale, YARN,
                             window=window, rolling=bool(rolling), sinks=sinks)
    assert_close(from_dev(out), ref, f"sink decode {case}")
    kg, vg = from_dev(kc), from_dev(vc)
    if append:
        for b, L in enumerate(lens):
            r = oatt.sink_slot(int(L) - 1, S, sinks) if rolling else int(L) - 1
            assert np.all(np.abs(kg[b, :, r] - kref[b, :, r]) <= _bf16_ulp(kref[b, :, r])), b
            assert np.array_equal(vg[b, :, r], vref[b, :, r]), b
            kg[b, :, r], vg[b, :, r] = k0[b, :, r], v0[b, :, r]
    assert np.array_equal(kg, k0) and np.array_equal(vg, v0), "rows other than the new one changed"


def test_decode_sink_window_equals_window_when_no_sinks(m):
    """sinks = 0 through the sink entry point is bitwise the window entry point."""
    import torch
    d = decode_inputs_host(2, 16, 2, 128, 900, 303, [900, 450])
    sl = torch.from_numpy(d["seq_lens"]).cuda()
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    a = m.gqa_decode_window(q, k, v, sl, 0.1, window=300, q_rope=YARN)
    lib = m.lib()
    b = torch.empty_like(a)
    ws = torch.empty(m.gqa_decode_workspace_size(2, 16, 2, 128, 900), dtype=torch.uint8,
                     device="cuda")
    st = lib.gqa_decode_sink_window(q.data_ptr(), None, None, k.data_ptr(), v.data_ptr(),
                                    sl.data_ptr(), 2, 16, 2, 128, 900, 0, 300, 0, 0.1,
                                    m.rope_params(YARN), b.data_ptr(), ws.data_ptr(), ws.numel(),
                                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(a, b)


def test_decode_sink_window_full_size_32k(m):
    """The 32K workload (ragged 16K-32K contexts, YaRN) with 4 sink tokens
    and a 4096-token window: every head, guarded output, two calls equal."""
    import torch
    cfg = DECODE_32K_YARN
    B, Hq, Hkv, D, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.S_max
    lens = cfg.seq_lens()
    sinks, window = 4, 4096
    print(f"[case] sink decode full size s={sinks} w={window}", flush=True)
    q = device_randn_bf16((B, Hq, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, S, D), cfg.seed * 10 + 3)
    sl = torch.from_numpy(lens).cuda()
    out = Guarded((B, Hq, D), torch.bfloat16, seed=11)
    m.gqa_decode_window(q, k, v, sl, cfg.scale, window=window, sinks=sinks, q_rope=cfg.rope(),
                        out=out.view)
    out.check("sink decode out")
    first = out.view.clone()
    m.gqa_decode_window(q, k, v, sl, cfg.scale, window=window, sinks=sinks, q_rope=cfg.rope(),
                        out=out.view)
    torch.cuda.synchronize()
    assert torch.equal(first, out.view)
    got = from_dev(out.view)
    qf = bf16_tensor_to_f64(q)
    g = Hq // Hkv
    for b in range(B):
        L = int(lens[b])
        rows = oatt.window_rows(L, S, window, False, sinks)
        assert len(rows) == sinks + window
        rt = torch.from_numpy(rows).cuda()
        qv = orope.rotate_rows(qf[b][None], np.array([L - 1]), cfg.rope())[0]
        for kv in range(Hkv):
            ref = oatt.decode_group(qv[kv * g:(kv + 1) * g], bf16_tensor_to_f64(k[b, kv][rt]),
                                    bf16_tensor_to_f64(v[b, kv][rt]), len(rows), cfg.scale, None)
            assert_close(got[b, kv * g:(kv + 1) * g], ref, f"sink decode full size (b={b}, kv={kv})")


PREFILL_CASES = [
    # (B, T, Hq, Hkv, D, sinks, window)
    (1, 300, 8, 2, 128, 4, 64),       # later query tiles take a separate sink tile
    (2, 517, 8, 2, 128, 1, 5),        # narrow band
    (1, 400, 4, 4, 128, 70, 64),      # sinks over two tiles
    (1, 700, 8, 2, 128, 4, 200),      # band over several tiles, ragged tail
    (2, 333, 6, 2, 64, 3, 100),       # head dim 64
    (1, 100, 4, 2, 32, 2, 7),         # head dim 32
    (1, 150, 4, 2, 128, 200, 16),     # sinks past T: plain causal
    (1, 257, 4, 1, 128, 64, 64),      # sinks end at a tile edge
]


@pytest.mark.parametrize("case", PREFILL_CASES,
                         ids=[f"B{c[0]}T{c[1]}D{c[4]}s{c[5]}w{c[6]}" for c in PREFILL_CASES])
def test_prefill_sink_window_parity(m, case):
    import torch
    B, T, Hq, Hkv, D, sinks, w = case
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=311)
    scale = 1 / math.sqrt(D)
    print(f"[case] prefill sinks={sinks} w={w} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    out = m.gqa_prefill_causal(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), scale, rope=NTK,
                               window=w, sinks=sinks)
    torch.cuda.synchronize()
    ref = oatt.prefill_causal(bf16_bits_to_f64(p["q"]), bf16_bits_to_f64(p["k"]),
                              bf16_bits_to_f64(p["v"]), scale, NTK, window=w, sinks=sinks)
    got = from_dev(out)
    assert np.all(np.isfinite(got))
    assert_close(got, ref, f"prefill sinks {case}")


def test_prefill_sink_window_full_size_8k(m):
    """The 8K prefill with 4 sinks and a 4096 window: every head over five
    whole query tiles (the first, either side of row 4095/4096, a middle one
    and the last)."""
    import torch
    cfg = PREFILL_8K
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    print(f"[case] prefill sinks full size T={T}", flush=True)
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 3)
    out = m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), window=4096, sinks=4)
    torch.cuda.synchronize()
    got = from_dev(out)
    rows = [r for t in (0, 31, 32, 45, 63) for r in range(128 * t, 128 * (t + 1))]
    ref = oatt.prefill_causal(bf16_tensor_to_f64(q), bf16_tensor_to_f64(k), bf16_tensor_to_f64(v),
                              cfg.scale, cfg.rope(), rows=rows, window=4096, sinks=4)
    assert_close(got[:, :, rows], ref[:, :, rows], "prefill sinks full size")


FP16_CASES = [
    # (B, T, Hq, Hkv, D, sinks, window)
    (2, 300, 8, 2, 128, 0, 0),
    (1, 129, 4, 4, 128, 0, 0),
    (2, 65, 6, 2, 64, 0, 0),
    (1, 700, 8, 2, 128, 0, 200),
    (1, 300, 8, 2, 128, 4, 64),
]


@pytest.mark.parametrize("case", FP16_CASES,
                         ids=[f"B{c[0]}T{c[1]}D{c[4]}s{c[5]}w{c[6]}" for c in FP16_CASES])
def test_prefill_fp16_scores_parity(m, case):
    """gqa_prefill_fp16 on N(0,1) inputs with scale 1/sqrt(d) (scores spread
    by about one unit, the regime its precision note covers)."""
    import torch
    B, T, Hq, Hkv, D, sinks, w = case
    p = prefill_inputs_host(B, T, Hq, Hkv, D, seed=321)
    scale = 1 / math.sqrt(D)
    print(f"[case] prefill fp16 scores {case}", flush=True)
    out = m.gqa_prefill_causal(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), scale, rope=NTK,
                               window=w, sinks=sinks, fp16_scores=True)
    torch.cuda.synchronize()
    ref = oatt.prefill_causal(bf16_bits_to_f64(p["q"]), bf16_bits_to_f64(p["k"]),
                              bf16_bits_to_f64(p["v"]), scale, NTK, window=w, sinks=sinks)
    assert_close(from_dev(out), ref, f"prefill fp16 {case}")


def test_prefill_fp16_scores_full_size_8k(m):
    """The 8K prefill workload through gqa_prefill_fp16: every head over five
    whole query tiles."""
    import torch
    cfg = PREFILL_8K
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    print(f"[case] prefill fp16 full size T={T}", flush=True)
    q = device_randn_bf16((B, Hq, T, D), cfg.seed * 10 + 1)
    k = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 2)
    v = device_randn_bf16((B, Hkv, T, D), cfg.seed * 10 + 3)
    out = m.gqa_prefill_causal(q, k, v, cfg.scale, rope=cfg.rope(), fp16_scores=True)
    torch.cuda.synchronize()
    got = from_dev(out)
    rows = [r for t in (0, 31, 32, 45, 63) for r in range(128 * t, 128 * (t + 1))]
    ref = oatt.prefill_causal(bf16_tensor_to_f64(q), bf16_tensor_to_f64(k), bf16_tensor_to_f64(v),
                              cfg.scale, cfg.rope(), rows=rows)
    assert_close(got[:, :, rows], ref[:, :, rows], "prefill fp16 full size")
