"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention, RoPE or selection arithmetic.  It only

* describes the five workloads (sizes, seeds, RoPE parameters as plain data),
* draws seeded N(0, 1) data (numpy PCG64 on the host, or torch's seeded
  generator on the device for the multi-GiB caches), and
* converts fp32 <-> bf16 bit patterns (round-to-nearest-even), so that both
  sides consume exactly the same bf16 values.

bf16 tensors travel as ``numpy.uint16`` bit patterns on the host; the oracle
widens them to float64 with :func:`bf16_bits_to_f64`, the GPU side views them as
``torch.bfloat16``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# bf16 bit conversions (input preparation, not part of the method)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def bf16_bits_to_f64(b) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def randn_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) samples drawn as float32, rounded to bf16 bits."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


# ---------------------------------------------------------------------------
# RoPE settings as plain data (each side builds its own struct from this)
# ---------------------------------------------------------------------------

ROPE_NONE, ROPE_PLAIN, ROPE_PI, ROPE_NTK, ROPE_YARN, ROPE_DYNAMIC_NTK = 0, 1, 2, 3, 4, 5


def rope_settings(scaling: int, base: float = 10000.0, factor: float = 1.0,
                  rotary_dim: int = 0, original_max_position: int = 0,
                  yarn_alpha: float = 1.0, yarn_beta: float = 32.0,
                  yarn_mscale: int = 1, current_len: int = 0) -> dict:
    return dict(scaling=scaling, rotary_dim=rotary_dim, base=base, factor=factor,
                original_max_position=original_max_position, yarn_alpha=yarn_alpha,
                yarn_beta=yarn_beta, yarn_mscale=yarn_mscale, current_len=current_len)


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class TinyConfig:
    """Tiny causal attention: B=2, T=10, C=64, 8 heads of dim 8, RoPE base 1e4."""
    B: int = 2
    T: int = 10
    C: int = 64
    n_head: int = 8
    n_kv_options: tuple = (8, 2, 1)
    seed: int = 0

    @property
    def head_dim(self) -> int:
        return self.C // self.n_head

    def rope(self) -> dict:
        return rope_settings(ROPE_PLAIN, base=10000.0)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    B: int
    Hq: int
    Hkv: int
    D: int
    S_max: int
    seed: int
    rope_kind: str            # "plain", "yarn" or "dynamic_ntk" (L_train = yarn_L_train)
    base: float
    ragged_lo: Optional[int] = None   # seq_lens ~ U{lo..S_max} when set
    yarn_factor: float = 4.0
    yarn_L_train: int = 8192

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    def rope(self) -> dict:
        if self.rope_kind == "yarn":
            return rope_settings(ROPE_YARN, base=self.base, factor=self.yarn_factor,
                                 original_max_position=self.yarn_L_train,
                                 yarn_alpha=1.0, yarn_beta=32.0, yarn_mscale=1)
        if self.rope_kind == "dynamic_ntk":
            return rope_settings(ROPE_DYNAMIC_NTK, base=self.base,
                                 original_max_position=self.yarn_L_train)
        return rope_settings(ROPE_PLAIN, base=self.base)

    def seq_lens(self) -> np.ndarray:
        if self.ragged_lo is None:
            return np.full(self.B, self.S_max, dtype=np.int32)
        rng = np.random.Generator(np.random.PCG64(self.seed + 1000))
        return rng.integers(self.ragged_lo, self.S_max, size=self.B,
                            endpoint=True).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    seed: int
    base: float
    ntk_factor: float

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def rope(self) -> dict:
        return rope_settings(ROPE_NTK, base=self.base, factor=self.ntk_factor)


@dataclasses.dataclass(frozen=True)
class SparseConfig:
    B: int
    H: int
    S_max: int
    Dqk: int
    Dv: int
    D_idx: int
    top_k: int
    seed: int
    d_nope: int = 128       # per-head content dim used for the score scale
    d_rope: int = 64        # decoupled RoPE dim

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    def seq_lens(self) -> np.ndarray:
        return np.full(self.B, self.S_max, dtype=np.int32)


@dataclasses.dataclass(frozen=True)
class QsaConfig:
    """QSA decode: GQA attention over the tokens of the top 512 micro-blocks."""
    B: int
    Hq: int
    Hkv: int
    D: int
    S_max: int
    H_I: int
    D_idx: int
    seed: int
    base: float = 1.0e4
    rotary_dim: int = 64      # block-key RoPE on the first 64 indexer dims

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def block_rope(self) -> dict:
        return rope_settings(ROPE_PLAIN, base=self.base, rotary_dim=self.rotary_dim)

    def seq_lens(self) -> np.ndarray:
        return np.full(self.B, self.S_max, dtype=np.int32)


TINY = TinyConfig()
DECODE_4K = DecodeConfig(B=16, Hq=64, Hkv=8, D=128, S_max=4096, seed=1,
                         rope_kind="plain", base=500000.0)
DECODE_32K_YARN = DecodeConfig(B=16, Hq=64, Hkv=8, D=128, S_max=32768, seed=2,
                               rope_kind="yarn", base=500000.0, ragged_lo=16384)
PREFILL_8K = PrefillConfig(B=1, T=8192, Hq=32, Hkv=8, D=128, seed=3, base=1.0e6,
                           ntk_factor=4.0)
SPARSE_128K = SparseConfig(B=4, H=128, S_max=131072, Dqk=576, Dv=512, D_idx=128,
                           top_k=2048, seed=4)
QSA_128K = QsaConfig(B=4, Hq=32, Hkv=4, D=128, S_max=131072, H_I=64, D_idx=128, seed=5)


# ---------------------------------------------------------------------------
# Host generators (numpy PCG64): exact and identical on every machine
# ---------------------------------------------------------------------------


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tiny_inputs(n_kv: int, cfg: TinyConfig = TINY) -> dict:
    """x ~ N(0,1) [B,T,C]; Wq ~ N(0,1)/sqrt(C) [C,C]; Wk, Wv [C, hd*n_kv].

    Returns the fp32 draws and the projected, head-split Q/K/V rounded to bf16
    (projection in float64, then fp32 -> bf16).  Projection is input
    preparation: the library receives already-projected Q/K/V.
    """
    rng = _rng(cfg.seed)
    C, H, hd = cfg.C, cfg.n_head, cfg.head_dim
    x = rng.standard_normal((cfg.B, cfg.T, C), dtype=np.float32)
    wq = (rng.standard_normal((C, C), dtype=np.float32) / np.float32(math.sqrt(C))).astype(np.float32)
    wk = (rng.standard_normal((C, hd * n_kv), dtype=np.float32) / np.float32(math.sqrt(C))).astype(np.float32)
    wv = (rng.standard_normal((C, hd * n_kv), dtype=np.float32) / np.float32(math.sqrt(C))).astype(np.float32)
    x64 = x.astype(np.float64)

    def split(y, n):
        return y.reshape(cfg.B, cfg.T, n, hd).transpose(0, 2, 1, 3)

    q = split(x64 @ wq.astype(np.float64), H)
    k = split(x64 @ wk.astype(np.float64), n_kv)
    v = split(x64 @ wv.astype(np.float64), n_kv)
    return dict(x=x, wq=wq, wk=wk, wv=wv,
                q=f32_to_bf16_bits(np.ascontiguousarray(q.astype(np.float32))),
                k=f32_to_bf16_bits(np.ascontiguousarray(k.astype(np.float32))),
                v=f32_to_bf16_bits(np.ascontiguousarray(v.astype(np.float32))))


def decode_inputs_host(B, Hq, Hkv, D, S_max, seed, seq_lens=None) -> dict:
    """Host-drawn decode inputs: q [B,Hq,D], K/V cache [B,Hkv,S_max,D] (bf16 bits)."""
    rng = _rng(seed)
    q = randn_bf16(rng, (B, Hq, D))
    k = randn_bf16(rng, (B, Hkv, S_max, D))
    v = randn_bf16(rng, (B, Hkv, S_max, D))
    if seq_lens is None:
        seq_lens = np.full(B, S_max, dtype=np.int32)
    return dict(q=q, k=k, v=v, seq_lens=np.asarray(seq_lens, dtype=np.int32))


def prefill_inputs_host(B, T, Hq, Hkv, D, seed) -> dict:
    rng = _rng(seed)
    return dict(q=randn_bf16(rng, (B, Hq, T, D)),
                k=randn_bf16(rng, (B, Hkv, T, D)),
                v=randn_bf16(rng, (B, Hkv, T, D)))


def sparse_inputs_host(B, H, S_max, Dqk, D_idx, seed, seq_lens=None) -> dict:
    rng = _rng(seed)
    q = randn_bf16(rng, (B, H, Dqk))
    latent = randn_bf16(rng, (B, S_max, Dqk))
    q_idx = randn_bf16(rng, (B, D_idx))
    k_idx = randn_bf16(rng, (B, S_max, D_idx))
    if seq_lens is None:
        seq_lens = np.full(B, S_max, dtype=np.int32)
    return dict(q=q, latent=latent, q_index=q_idx, k_index=k_idx,
                seq_lens=np.asarray(seq_lens, dtype=np.int32))


# ---------------------------------------------------------------------------
# Device generators (torch, seeded) for the full-size caches
# ---------------------------------------------------------------------------


def device_randn_bf16(shape, seed: int, device="cuda"):
    """Seeded N(0,1) drawn on the device in fp32 and rounded to bf16 (RNE)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=gen, device=device,
                                    dtype=torch.float32).to(torch.bfloat16)
    return out


def bf16_tensor_to_f64(t) -> np.ndarray:
    """Copy a (device) bf16 tensor to host float64, exactly."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f64(bits)
