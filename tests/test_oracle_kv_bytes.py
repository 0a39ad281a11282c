"""Exact-integer pins of the KV-bytes closed forms against printed values."""
from conftest import golden_rows
from oracle import kv_bytes


def test_llama2_70b_table():
    for _, layers, kv, hd, bpe, kib, gib in golden_rows("kv_bytes_llama2_70b.txt"):
        b = kv_bytes.kv_bytes_per_token(int(layers), int(kv), int(hd), int(bpe))
        assert b == int(kib) * 1024
        assert b * 32768 * 16 == int(float(gib)) * 2 ** 30


def test_mla_v3():
    for L, h, hd, dc, dr, bpe, mha_kib, mla_kib, ratio, mla_b in golden_rows("kv_bytes_mla_v3.txt"):
        mha = kv_bytes.kv_bytes_per_token(int(L), int(h), int(hd), int(bpe))
        mla = kv_bytes.mla_kv_bytes_per_token(int(L), int(dc), int(dr), int(bpe))
        assert mha == int(mha_kib) * 1024
        assert mla == int(mla_b)
        assert f"{mla / 1024:.1f}" == mla_kib
        assert f"{mha / mla:.1f}" == ratio


def test_llama2_7b():
    for layers, kv, hd, bpe, tokens, total in golden_rows("kv_bytes_llama2_7b.txt"):
        b = kv_bytes.kv_bytes_per_token(int(layers), int(kv), int(hd), int(bpe))
        assert b * int(tokens) == int(total)
