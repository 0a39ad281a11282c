"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, golden_rows

HEADER = os.path.join(ROOT, "include", "gqa_attn.h")


@pytest.fixture(scope="module")
def m():
    import mqa_kv_cache_amd
    return mqa_kv_cache_amd


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("rope_apply", "gqa_decode", "gqa_prefill_causal", "topk_sparse_decode", "mla_decode",
                 "kv_bytes_per_token", "mla_kv_bytes_per_token", "gqa_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(m):
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(m.EXPORTED) == declared_functions()


def test_status_strings(m):
    lib = m.lib()
    for code in range(5):
        assert lib.gqa_status_string(code)
    assert lib.gqa_status_string(99) == b"unknown status"


def test_kv_bytes_closed_forms(m):
    for _, layers, kv, hd, bpe, kib, gib in golden_rows("kv_bytes_llama2_70b.txt"):
        assert m.kv_bytes_per_token(int(layers), int(kv), int(hd), int(bpe)) == int(kib) * 1024
    for L, h, hd, dc, dr, bpe, mha_kib, mla_kib, ratio, mla_b in golden_rows("kv_bytes_mla_v3.txt"):
        assert m.mla_kv_bytes_per_token(int(L), int(dc), int(dr), int(bpe)) == int(mla_b)
        assert m.kv_bytes_per_token(int(L), int(h), int(hd), int(bpe)) == int(mha_kib) * 1024
    for layers, kv, hd, bpe, tokens, total in golden_rows("kv_bytes_llama2_7b.txt"):
        assert m.kv_bytes_per_token(int(layers), int(kv), int(hd), int(bpe)) * int(tokens) == int(total)
    assert m.kv_bytes_per_token(-1, 8, 128, 2) == -1
    assert m.kv_bytes_per_token(2**31 - 1, 2**31 - 1, 2**31 - 1, 2) == -1
    assert m.mla_kv_bytes_per_token(61, -1, 64, 2) == -1


P = 0x10000       # aligned fake device pointer: never dereferenced (validation fails first)
MIS = 0x10002     # misaligned


def _rope(m, **kw):
    return m.rope_params(dict(kw))


def _decode(m, q=P, k=P, v=P, sl=P, B=2, Hq=16, Hkv=2, D=128, S=64, scale=0.1, rope=None,
            out=P, ws=P, wsn=1 << 30):
    return m.lib().gqa_decode(q, k, v, sl, B, Hq, Hkv, D, S, scale, rope, out, ws, wsn, None)


def test_decode_validation(m):
    assert _decode(m, Hq=15, Hkv=2) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, B=0) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, D=96) == m.ERR_UNSUPPORTED
    assert _decode(m, Hq=128, Hkv=1) == m.ERR_UNSUPPORTED       # g > 64
    assert _decode(m, q=0) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, k=MIS) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, ws=P + 16) == m.ERR_INVALID_ARGUMENT      # workspace not 256-aligned
    assert _decode(m, scale=float("nan")) == m.ERR_INVALID_ARGUMENT
    need = m.gqa_decode_workspace_size(2, 16, 2, 128, 64)
    assert need > 0
    assert _decode(m, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert _decode(m, wsn=need - 1, rope=_rope(m, scaling=m.ROPE_PLAIN, base=1e4, factor=2.0)) \
        == m.ERR_INVALID_ARGUMENT
    assert _decode(m, wsn=0, rope=_rope(m, scaling=m.ROPE_YARN, base=1e4, factor=4.0,
                                        original_max_position=8192, yarn_alpha=32.0,
                                        yarn_beta=1.0)) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, wsn=0, rope=_rope(m, scaling=m.ROPE_PI, base=1e4, factor=0.5)) \
        == m.ERR_INVALID_ARGUMENT
    assert _decode(m, wsn=0, rope=_rope(m, scaling=m.ROPE_PLAIN, base=1e4, rotary_dim=7)) \
        == m.ERR_INVALID_ARGUMENT
    assert _decode(m, wsn=0, rope=_rope(m, scaling=m.ROPE_PLAIN, base=1e4, rotary_dim=12)) \
        == m.ERR_UNSUPPORTED
    assert _decode(m, wsn=0, rope=_rope(m, scaling=9, base=1e4)) == m.ERR_INVALID_ARGUMENT
    assert m.gqa_decode_workspace_size(2, 15, 2, 128, 64) == 0
    # a context's K or V rows must fit 32-bit byte offsets: 2^23 rows of 256 B
    # are 2^31 bytes (rejected); one row fewer is the largest cache accepted
    assert _decode(m, S=1 << 23, wsn=0) == m.ERR_UNSUPPORTED
    assert _decode(m, S=(1 << 23) - 1, wsn=0) == m.ERR_WORKSPACE_TOO_SMALL
    assert _decode(m, D=64, S=1 << 24, wsn=0) == m.ERR_UNSUPPORTED
    assert _decode(m, D=64, S=(1 << 24) - 1, wsn=0) == m.ERR_WORKSPACE_TOO_SMALL
    lib = m.lib()
    assert lib.gqa_decode_parts(P, P, P, P, 2, 16, 2, 128, 64, 0.1, None, P, P, 1 << 30, -3,
                                None) == m.ERR_INVALID_ARGUMENT   # negative part count
    assert lib.gqa_decode_parts(P, P, P, P, 2, 16, 2, 128, 64, 0.1, None, P, P, 1 << 30,
                                (1 << 20) + 1, None) == m.ERR_INVALID_ARGUMENT
    assert m.gqa_decode_workspace_size(2, 16, 2, 128, 64, 5000) > m.gqa_decode_workspace_size(2, 16, 2, 128, 64, 10)
    assert lib.gqa_decode_combine(P, 2, 16, 2, 128, 64, P, 1, 0, P, None) == m.ERR_WORKSPACE_TOO_SMALL


def test_decode_append_validation(m):
    lib = m.lib()

    def app(q=P, kn=P, vn=P, k=P, v=P, sl=P, B=2, Hq=16, Hkv=2, D=128, S=64, scale=0.1, rope=None,
            out=P, ws=P, wsn=1 << 30):
        return lib.gqa_decode_append(q, kn, vn, k, v, sl, B, Hq, Hkv, D, S, scale, rope, out, ws,
                                     wsn, None)
    assert app(kn=0) == m.ERR_INVALID_ARGUMENT
    assert app(vn=0) == m.ERR_INVALID_ARGUMENT
    assert app(kn=MIS) == m.ERR_INVALID_ARGUMENT
    assert app(vn=MIS) == m.ERR_INVALID_ARGUMENT
    assert app(out=0) == m.ERR_INVALID_ARGUMENT
    assert app(out=MIS) == m.ERR_INVALID_ARGUMENT
    assert app(Hq=15) == m.ERR_INVALID_ARGUMENT
    assert app(D=96) == m.ERR_UNSUPPORTED
    assert app(ws=P + 16) == m.ERR_INVALID_ARGUMENT
    assert app(scale=float("inf")) == m.ERR_INVALID_ARGUMENT
    need = m.gqa_decode_workspace_size(2, 16, 2, 128, 64)
    assert app(wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert app(wsn=0, rope=_rope(m, scaling=m.ROPE_PLAIN, base=1e4, rotary_dim=7)) \
        == m.ERR_INVALID_ARGUMENT


def test_decode_window_validation(m):
    lib = m.lib()

    def win(kn=0, vn=0, window=0, rolling=0, wsn=1 << 30):
        return lib.gqa_decode_window(P, kn, vn, P, P, P, 2, 16, 2, 128, 64, window, rolling, 0.1,
                                     None, P, P, wsn, None)
    assert win(window=-1) == m.ERR_INVALID_ARGUMENT
    assert win(rolling=2) == m.ERR_INVALID_ARGUMENT
    assert win(rolling=1, window=65) == m.ERR_INVALID_ARGUMENT   # a window past the buffer
    assert win(kn=P) == m.ERR_INVALID_ARGUMENT                   # k_new without v_new
    assert win(kn=P, vn=MIS) == m.ERR_INVALID_ARGUMENT
    need = m.gqa_decode_workspace_size(2, 16, 2, 128, 64)
    assert win(window=5, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert win(rolling=1, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    # a window up to the buffer's size passes the argument checks
    assert win(rolling=1, window=8, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert win(rolling=1, window=64, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL


def test_prefill_validation(m):
    lib = m.lib()

    def call(B=1, T=16, Hq=8, Hkv=2, D=128, rope=None, ws=P, wsn=0, q=P):
        return lib.gqa_prefill_causal(q, P, P, B, T, Hq, Hkv, D, 0.1, rope, P, ws, wsn, None)

    assert call(Hq=7) == m.ERR_INVALID_ARGUMENT
    assert call(T=0) == m.ERR_INVALID_ARGUMENT
    assert call(D=96) == m.ERR_UNSUPPORTED
    assert call(q=MIS) == m.ERR_INVALID_ARGUMENT
    r = _rope(m, scaling=m.ROPE_NTK, base=1e6, factor=4.0)
    need = m.gqa_prefill_workspace_size(1, 2, 16, 128, r.contents)
    assert need == 3 * (2 * 64 * 128 * 2)      # K hi and lo rows + fp16 V^T tiles, T padded to 64
    assert call(rope=r, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert call(rope=r, ws=None, wsn=need) == m.ERR_INVALID_ARGUMENT
    assert m.gqa_prefill_workspace_size(1, 2, 16, 128, None) == need
    # a head's rows must fit 32-bit byte offsets: 2^23 tokens of 256 B are
    # rejected, one fewer is the longest prompt accepted
    assert call(T=1 << 23) == m.ERR_UNSUPPORTED
    assert call(T=(1 << 23) - 1) == m.ERR_WORKSPACE_TOO_SMALL


def test_prefill_window_validation(m):
    lib = m.lib()
    assert lib.gqa_prefill_window(P, P, P, 1, 64, 8, 2, 128, -1, 0.1, None, P, P, 1 << 30,
                                  None) == m.ERR_INVALID_ARGUMENT
    assert lib.gqa_prefill_window(P, P, P, 1, 64, 8, 2, 96, 16, 0.1, None, P, P, 1 << 30,
                                  None) == m.ERR_UNSUPPORTED
    assert lib.gqa_prefill_window(P, P, P, 1, 64, 8, 2, 128, 16, 0.1, None, P, P, 1,
                                  None) == m.ERR_WORKSPACE_TOO_SMALL


def test_decode_noalloc_validation(m):
    """The no-allocation decode validates like gqa_decode and rejects shapes
    whose states exceed its 16 MiB static scratch before touching a device."""
    lib = m.lib()

    def call(B=2, Hq=16, Hkv=2, D=128, S=64, q=P, out=P):
        return lib.gqa_decode_noalloc(q, P, P, P, B, Hq, Hkv, D, S, 0.1, None, out, None)
    assert call(Hq=15) == m.ERR_INVALID_ARGUMENT
    assert call(D=96) == m.ERR_UNSUPPORTED
    assert call(q=None) == m.ERR_INVALID_ARGUMENT
    assert call(out=MIS) == m.ERR_INVALID_ARGUMENT
    # 4096 sequences x 8 kv heads: (1024 + 32768) slots x 8 heads x 128 x 4 B > 16 MiB
    assert m.gqa_decode_workspace_size(4096, 64, 8, 128, 64) > (16 << 20)
    assert call(B=4096, Hq=64, Hkv=8) == m.ERR_WORKSPACE_TOO_SMALL


def test_sink_window_validation(m):
    """StreamingLLM entry points: negative sinks, a rolling buffer with no
    ring slot left, and the usual shape/workspace checks."""
    lib = m.lib()

    def dec(sinks=4, window=64, rolling=0, wsn=1 << 30):
        return lib.gqa_decode_sink_window(P, 0, 0, P, P, P, 2, 16, 2, 128, 64, sinks, window,
                                          rolling, 0.1, None, P, P, wsn, None)
    assert dec(sinks=-1) == m.ERR_INVALID_ARGUMENT
    assert dec(window=-1) == m.ERR_INVALID_ARGUMENT
    assert dec(rolling=1, window=0, sinks=64) == m.ERR_INVALID_ARGUMENT   # no ring slot left
    assert dec(rolling=1, window=61) == m.ERR_INVALID_ARGUMENT   # past the ring of 64 - 4 slots
    need = m.gqa_decode_workspace_size(2, 16, 2, 128, 64)
    assert dec(wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert dec(rolling=1, window=0, sinks=63, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert dec(rolling=1, window=60, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert dec(rolling=1, window=1, sinks=63, wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    for fn in (lib.gqa_prefill_sink_window, lib.gqa_prefill_fp16):
        assert fn(P, P, P, 1, 64, 8, 2, 128, -1, 16, 0.1, None, P, P, 1 << 30,
                  None) == m.ERR_INVALID_ARGUMENT
        assert fn(P, P, P, 1, 64, 8, 2, 128, 4, -1, 0.1, None, P, P, 1 << 30,
                  None) == m.ERR_INVALID_ARGUMENT
        assert fn(P, P, P, 1, 64, 7, 2, 128, 4, 16, 0.1, None, P, P, 1 << 30,
                  None) == m.ERR_INVALID_ARGUMENT
        assert fn(P, P, P, 1, 64, 8, 2, 96, 4, 16, 0.1, None, P, P, 1 << 30,
                  None) == m.ERR_UNSUPPORTED
        assert fn(P, P, P, 1, 64, 8, 2, 128, 4, 16, 0.1, None, P, P, 1,
                  None) == m.ERR_WORKSPACE_TOO_SMALL


def test_sparse_validation(m):
    lib = m.lib()

    def call(B=2, H=128, Dqk=576, Dv=512, Di=128, S=4096, k=2048, wsn=0, idx=P):
        return lib.topk_sparse_decode(P, P, P, P, P, B, H, Dqk, Dv, Di, S, k, 0.07, idx, P, P,
                                      wsn, None)

    assert call(k=0) == m.ERR_INVALID_ARGUMENT
    assert call(k=5000, S=4096) == m.ERR_INVALID_ARGUMENT
    assert call(k=8192, S=100000) == m.ERR_UNSUPPORTED
    assert call(Dqk=512) == m.ERR_UNSUPPORTED
    assert call(H=100) == m.ERR_UNSUPPORTED
    assert call(idx=MIS) == m.ERR_INVALID_ARGUMENT
    need = m.topk_sparse_decode_workspace_size(2, 128, 4096, 2048)
    assert need > 0
    assert call(wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    # a row's latent bytes (1152 per row) must fit 32-bit byte offsets
    assert call(S=1864136) == m.ERR_UNSUPPORTED            # 2,147,484,672 bytes
    assert call(S=1864135) == m.ERR_WORKSPACE_TOO_SMALL    # 2,147,483,520 bytes: the largest


def test_sparse_weighted_validation(m):
    lib = m.lib()
    need = m.topk_sparse_decode_workspace_size(2, 128, 4096, 2048)

    def call(HI=64, w=P, wsn=need, H=128, k=2048):
        return lib.topk_sparse_decode_weighted(P, P, P, w, P, P, 2, H, HI, 576, 512, 128, 4096, k,
                                               0.07, P, P, P, wsn, None)

    assert call(HI=0) == m.ERR_INVALID_ARGUMENT
    assert call(HI=24) == m.ERR_UNSUPPORTED
    assert call(HI=128) == m.ERR_UNSUPPORTED
    assert call(w=None) == m.ERR_INVALID_ARGUMENT
    assert call(w=P + 2) == m.ERR_INVALID_ARGUMENT
    assert call(k=0) == m.ERR_INVALID_ARGUMENT
    assert call(H=100) == m.ERR_UNSUPPORTED
    assert call(wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL


def test_qsa_validation(m):
    lib = m.lib()
    need = m.qsa_sparse_decode_workspace_size(2, 32, 4096)
    assert need > 0

    def call(Hq=32, Hkv=4, D=128, HI=64, Di=128, S=4096, scale=0.08, rope=None, wsn=need, tok=P):
        return lib.qsa_sparse_decode(P, P, P, P, P, P, 2, Hq, Hkv, D, HI, Di, S, scale, rope, tok, P,
                                     P, wsn, None)

    assert call(Hq=30) == m.ERR_INVALID_ARGUMENT
    assert call(D=64) == m.ERR_UNSUPPORTED
    assert call(Di=64) == m.ERR_UNSUPPORTED
    assert call(Hq=64, Hkv=2) == m.ERR_UNSUPPORTED     # g = 32 > 16
    assert call(HI=24) == m.ERR_UNSUPPORTED
    assert call(HI=0) == m.ERR_INVALID_ARGUMENT
    assert call(scale=float("nan")) == m.ERR_INVALID_ARGUMENT
    assert call(tok=MIS) == m.ERR_INVALID_ARGUMENT
    assert call(wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    dyn = _rope(m, scaling=m.ROPE_DYNAMIC_NTK, base=1e4, original_max_position=100)
    assert call(rope=dyn) == m.ERR_UNSUPPORTED
    bad = _rope(m, scaling=m.ROPE_PLAIN, base=0.5)
    assert call(rope=bad) == m.ERR_INVALID_ARGUMENT


def test_mla_validation(m):
    lib = m.lib()

    def call(B=2, H=128, Dqk=576, Dv=512, S=4096, scale=0.07, wsn=0, q=P, out=P, ws=P):
        return lib.mla_decode(q, P, P, B, H, Dqk, Dv, S, scale, out, ws, wsn, None)

    need = m.mla_decode_workspace_size(2, 128, 4096)
    assert need > 0
    assert call(B=0, wsn=need) == m.ERR_INVALID_ARGUMENT
    assert call(Dv=600, wsn=need) == m.ERR_INVALID_ARGUMENT
    assert call(Dqk=512, wsn=need) == m.ERR_UNSUPPORTED
    assert call(H=100, wsn=need) == m.ERR_UNSUPPORTED
    assert call(H=256, wsn=need) == m.ERR_UNSUPPORTED
    assert call(S=1 << 22, wsn=need) == m.ERR_UNSUPPORTED
    assert call(q=MIS, wsn=need) == m.ERR_INVALID_ARGUMENT
    assert call(out=None, wsn=need) == m.ERR_INVALID_ARGUMENT
    assert call(scale=float("inf"), wsn=need) == m.ERR_INVALID_ARGUMENT
    assert call(wsn=need - 1) == m.ERR_WORKSPACE_TOO_SMALL
    assert m.mla_decode_workspace_size(2, 100, 4096) == 0


def test_mla_workspace_covers_the_partials(m):
    # at least one fp32 partial row (Dv values + m, l) per head per 4096 rows
    for B, H, S in ((1, 16, 1), (4, 128, 131072), (3, 64, 1000), (16, 128, 4096)):
        need = m.mla_decode_workspace_size(B, H, S)
        assert need >= B * H * 514 * 4
        assert need % 256 == 0


def test_rope_validation(m):
    lib = m.lib()
    r = _rope(m, scaling=m.ROPE_PLAIN, base=1e4)
    assert lib.rope_apply(P, P, P, -1, 2, 128, 256, 128, r, None) == m.ERR_INVALID_ARGUMENT
    assert lib.rope_apply(P, P, P, 4, 2, 12, 24, 12, r, None) == m.ERR_UNSUPPORTED
    assert lib.rope_apply(P, P, P, 4, 2, 128, 250, 128, r, None) == m.ERR_INVALID_ARGUMENT
    assert lib.rope_apply(MIS, P, P, 4, 2, 128, 256, 128, r, None) == m.ERR_INVALID_ARGUMENT
    assert lib.rope_apply(P, P, None, 4, 2, 128, 256, 128, r, None) == m.ERR_INVALID_ARGUMENT
    assert lib.rope_apply(P, P, P, 0, 2, 128, 256, 128, r, None) == m.OK   # empty: no-op
    bad = _rope(m, scaling=m.ROPE_PLAIN, base=0.5)
    assert lib.rope_apply(P, P, P, 4, 2, 128, 256, 128, bad, None) == m.ERR_INVALID_ARGUMENT


def test_dynamic_ntk_validation(m):
    """Dynamic NTK needs L_train > 0 and factor 1; rope_apply needs the call's
    current length, the other entry points take it from their own sizes."""
    lib = m.lib()
    dyn = dict(scaling=m.ROPE_DYNAMIC_NTK, base=1e4, original_max_position=4096)
    ok = _rope(m, current_len=8192, **dyn)
    assert lib.rope_apply(P, P, P, 0, 2, 128, 256, 128, ok, None) == m.OK
    assert lib.rope_apply(P, P, P, 4, 2, 128, 256, 128, _rope(m, **dyn), None) == m.ERR_INVALID_ARGUMENT
    assert lib.rope_apply(P, P, P, 4, 2, 128, 256, 128,
                          _rope(m, current_len=-3, **dyn), None) == m.ERR_INVALID_ARGUMENT
    no_train = dict(dyn, original_max_position=0)
    assert lib.rope_apply(P, P, P, 4, 2, 128, 256, 128,
                          _rope(m, current_len=10, **no_train), None) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, rope=_rope(m, **no_train)) == m.ERR_INVALID_ARGUMENT
    assert _decode(m, rope=_rope(m, factor=2.0, **dyn)) == m.ERR_INVALID_ARGUMENT
    # decode and prefill accept it without current_len
    assert m.gqa_prefill_workspace_size(1, 8, 64, 128, dyn) > 0
    assert m.gqa_prefill_workspace_size(1, 8, 64, 128, no_train) == 0
