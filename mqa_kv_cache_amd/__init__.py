"""Thin Python binding of libgqa_attn.so (grouped-query attention over a bf16
KV cache on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gqa_attn.h``.  PyTorch is used
for device memory and the current stream.  There is no fallback: importing
this package fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MQA_KV_CACHE_AMD_LIB names another build of the same library (e.g. one
# with a sanitized host layer); the default is the in-tree build.
LIB_PATH = os.environ.get("MQA_KV_CACHE_AMD_LIB") or os.path.join(_HERE, "libgqa_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -m mqa_kv_cache_amd.build, or "
        "__graft_entry__.build()); there is no non-HIP fallback")

_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_DEVICE = 0, 1, 2, 3, 4
ROPE_NONE, ROPE_PLAIN, ROPE_PI, ROPE_NTK, ROPE_YARN, ROPE_DYNAMIC_NTK = 0, 1, 2, 3, 4, 5

EXPORTED = [
    "rope_apply", "gqa_decode", "gqa_decode_parts", "gqa_decode_append", "gqa_decode_window",
    "gqa_decode_sink_window", "gqa_decode_noalloc", "gqa_decode_workspace_size",
    "gqa_decode_workspace_size_parts", "gqa_decode_partial", "gqa_decode_combine",
    "gqa_prefill_causal", "gqa_prefill_window", "gqa_prefill_sink_window", "gqa_prefill_fp16",
    "gqa_prefill_workspace_size",
    "topk_sparse_decode", "topk_sparse_decode_workspace_size", "topk_sparse_decode_weighted",
    "qsa_sparse_decode", "qsa_sparse_decode_workspace_size",
    "mla_decode",
    "mla_decode_workspace_size", "kv_bytes_per_token",
    "mla_kv_bytes_per_token", "gqa_status_string",
]


class RopeParams(ctypes.Structure):
    _fields_ = [
        ("scaling", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("base", ctypes.c_double),
        ("factor", ctypes.c_double),
        ("original_max_position", ctypes.c_int32),
        ("yarn_mscale", ctypes.c_int32),
        ("yarn_alpha", ctypes.c_double),
        ("yarn_beta", ctypes.c_double),
        ("current_len", ctypes.c_int32),
    ]


class GqaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.gqa_status_string(status).decode()} (status {status})")


_c_void_p, _c_int32, _c_int64, _c_size_t = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_rope_p = ctypes.POINTER(RopeParams)

_lib.gqa_status_string.restype = ctypes.c_char_p
_lib.gqa_status_string.argtypes = [_c_int32]
_lib.kv_bytes_per_token.restype = _c_int64
_lib.kv_bytes_per_token.argtypes = [_c_int32] * 4
_lib.mla_kv_bytes_per_token.restype = _c_int64
_lib.mla_kv_bytes_per_token.argtypes = [_c_int32] * 4
_lib.rope_apply.restype = _c_int32
_lib.rope_apply.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_int64, _c_int32, _c_int32,
                            _c_int64, _c_int64, _rope_p, _c_void_p]
_lib.gqa_decode_workspace_size.restype = _c_size_t
_lib.gqa_decode_workspace_size.argtypes = [_c_int32] * 5
_lib.gqa_decode_workspace_size_parts.restype = _c_size_t
_lib.gqa_decode_workspace_size_parts.argtypes = [_c_int32] * 6
_lib.gqa_decode.restype = _c_int32
_lib.gqa_decode.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int32, _c_int32,
                            _c_int32, _c_int32, _c_int32, ctypes.c_float, _rope_p, _c_void_p,
                            _c_void_p, _c_size_t, _c_void_p]
_lib.gqa_decode_append.restype = _c_int32
_lib.gqa_decode_append.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, ctypes.c_float,
                                   _rope_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]
_lib.gqa_decode_window.restype = _c_int32
_lib.gqa_decode_window.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                   _c_int32, ctypes.c_float, _rope_p, _c_void_p, _c_void_p,
                                   _c_size_t, _c_void_p]
_lib.gqa_decode_sink_window.restype = _c_int32
_lib.gqa_decode_sink_window.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _c_int32, _c_int32, _c_int32, _c_int32,
                                        _c_int32, _c_int32, _c_int32, _c_int32, ctypes.c_float,
                                        _rope_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]
_lib.gqa_decode_noalloc.restype = _c_int32
_lib.gqa_decode_noalloc.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int32, _c_int32,
                                    _c_int32, _c_int32, _c_int32, ctypes.c_float, _rope_p,
                                    _c_void_p, _c_void_p]
_lib.gqa_decode_parts.restype = _c_int32
_lib.gqa_decode_parts.argtypes = _lib.gqa_decode.argtypes[:-1] + [_c_int32, _c_void_p]
_lib.gqa_decode_partial.restype = _c_int32
_lib.gqa_decode_partial.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int32, _c_int32,
                                    _c_int32, _c_int32, _c_int32, ctypes.c_float, _rope_p,
                                    _c_void_p, _c_size_t, _c_int32, _c_void_p]
_lib.gqa_decode_combine.restype = _c_int32
_lib.gqa_decode_combine.argtypes = [_c_void_p, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                    _c_void_p, _c_size_t, _c_int32, _c_void_p, _c_void_p]
_lib.gqa_prefill_workspace_size.restype = _c_size_t
_lib.gqa_prefill_workspace_size.argtypes = [_c_int32] * 4 + [_rope_p]
_lib.gqa_prefill_causal.restype = _c_int32
_lib.gqa_prefill_causal.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_int32, _c_int32, _c_int32,
                                    _c_int32, _c_int32, ctypes.c_float, _rope_p, _c_void_p,
                                    _c_void_p, _c_size_t, _c_void_p]
_lib.gqa_prefill_window.restype = _c_int32
_lib.gqa_prefill_window.argtypes = (_lib.gqa_prefill_causal.argtypes[:8] + [_c_int32]
                                    + _lib.gqa_prefill_causal.argtypes[8:])
_lib.gqa_prefill_sink_window.restype = _c_int32
_lib.gqa_prefill_sink_window.argtypes = (_lib.gqa_prefill_causal.argtypes[:8] + [_c_int32, _c_int32]
                                         + _lib.gqa_prefill_causal.argtypes[8:])
_lib.gqa_prefill_fp16.restype = _c_int32
_lib.gqa_prefill_fp16.argtypes = _lib.gqa_prefill_sink_window.argtypes
_lib.topk_sparse_decode_workspace_size.restype = _c_size_t
_lib.topk_sparse_decode_workspace_size.argtypes = [_c_int32] * 4
_lib.topk_sparse_decode.restype = _c_int32
_lib.topk_sparse_decode.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                    _c_int32, ctypes.c_float, _c_void_p, _c_void_p, _c_void_p,
                                    _c_size_t, _c_void_p]
_lib.topk_sparse_decode_weighted.restype = _c_int32
_lib.topk_sparse_decode_weighted.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                             _c_void_p, _c_int32, _c_int32, _c_int32, _c_int32,
                                             _c_int32, _c_int32, _c_int32, _c_int32, ctypes.c_float,
                                             _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]
_lib.qsa_sparse_decode_workspace_size.restype = _c_size_t
_lib.qsa_sparse_decode_workspace_size.argtypes = [_c_int32] * 3
_lib.qsa_sparse_decode.restype = _c_int32
_lib.qsa_sparse_decode.argtypes = ([_c_void_p] * 6 + [_c_int32] * 7
                                   + [ctypes.c_float, _rope_p, _c_void_p, _c_void_p, _c_void_p,
                                      _c_size_t, _c_void_p])
_lib.mla_decode_workspace_size.restype = _c_size_t
_lib.mla_decode_workspace_size.argtypes = [_c_int32] * 3
_lib.mla_decode.restype = _c_int32
_lib.mla_decode.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_int32, _c_int32, _c_int32, _c_int32,
                            _c_int32, ctypes.c_float, _c_void_p, _c_void_p, _c_size_t, _c_void_p]


def lib() -> ctypes.CDLL:
    return _lib


def rope_params(settings) -> "ctypes.pointer | None":
    """dict(scaling, rotary_dim, base, factor, original_max_position, yarn_alpha,
    yarn_beta, yarn_mscale, current_len) -> pointer to the C struct (None stays None)."""
    if settings is None:
        return None
    if isinstance(settings, RopeParams):
        return ctypes.pointer(settings)
    p = RopeParams(int(settings.get("scaling", ROPE_NONE)), int(settings.get("rotary_dim", 0)),
                   float(settings.get("base", 10000.0)), float(settings.get("factor", 1.0)),
                   int(settings.get("original_max_position", 0)),
                   int(settings.get("yarn_mscale", 1)), float(settings.get("yarn_alpha", 1.0)),
                   float(settings.get("yarn_beta", 32.0)), int(settings.get("current_len", 0)))
    return ctypes.pointer(p)


def _check(status: int, where: str):
    if status != OK:
        raise GqaError(status, where)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=torch.bfloat16, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t, want, name):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def kv_bytes_per_token(layers: int, n_kv_heads: int, head_dim: int, bytes_per_elem: int = 2) -> int:
    return int(_lib.kv_bytes_per_token(layers, n_kv_heads, head_dim, bytes_per_elem))


def mla_kv_bytes_per_token(layers: int, d_latent: int, d_rope: int, bytes_per_elem: int = 2) -> int:
    return int(_lib.mla_kv_bytes_per_token(layers, d_latent, d_rope, bytes_per_elem))


def rope_apply(x: torch.Tensor, positions: torch.Tensor, rope, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """x: bf16 [n_tok, n_heads, head_dim] (last dim contiguous, any token/head
    strides); positions: int32 [n_tok].  Returns out (same strides as x);
    out=x rotates in place."""
    if x.dim() != 3:
        raise ValueError("x must be [n_tok, n_heads, head_dim]")
    n_tok, n_heads, head_dim = x.shape
    _dev(x, "x", contiguous=False)
    if x.stride(2) != 1:
        raise ValueError("x must be contiguous in its last dim")
    if out is None:
        out = torch.empty_strided(x.size(), x.stride(), dtype=x.dtype, device=x.device)
    _dev(out, "out", contiguous=False)
    if out.stride() != x.stride() or out.shape != x.shape:
        raise ValueError("out must have the shape and strides of x")
    _dev(positions, "positions", dtype=torch.int32)
    _shape(positions, (n_tok,), "positions")
    st = _lib.rope_apply(x.data_ptr(), out.data_ptr(), positions.data_ptr(), n_tok, n_heads,
                         head_dim, x.stride(0), x.stride(1), rope_params(rope), _stream(stream))
    _check(st, "rope_apply")
    return out


def gqa_decode_workspace_size(B, Hq, Hkv, D, S_max, n_parts=None) -> int:
    if n_parts is None:
        return int(_lib.gqa_decode_workspace_size(B, Hq, Hkv, D, S_max))
    return int(_lib.gqa_decode_workspace_size_parts(B, Hq, Hkv, D, S_max, n_parts))


def gqa_decode(q, k_cache, v_cache, seq_lens, scale: float, q_rope=None, out=None,
               workspace=None, n_parts: int | None = None, stream=None) -> torch.Tensor:
    """q [B,Hq,D], k_cache/v_cache [B,Hkv,S_max,D] (bf16, keys post-RoPE),
    seq_lens int32 [B] on the device.  Returns out [B,Hq,D] bf16."""
    B, Hq, D = q.shape
    Bk, Hkv, S_max, Dk = k_cache.shape
    _shape(k_cache, (B, Hkv, S_max, D), "k_cache")
    _shape(v_cache, (B, Hkv, S_max, D), "v_cache")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _shape(out, (B, Hq, D), "out")
    _dev(out, "out")
    need = gqa_decode_workspace_size(B, Hq, Hkv, D, S_max, n_parts)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv,
            D, S_max, float(scale), rope_params(q_rope), out.data_ptr(), workspace.data_ptr(),
            workspace.numel())
    if n_parts is None:
        st = _lib.gqa_decode(*args, _stream(stream))
    else:
        st = _lib.gqa_decode_parts(*args, int(n_parts), _stream(stream))
    _check(st, "gqa_decode")
    return out


def gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, scale: float, q_rope=None, out=None,
                       stream=None) -> torch.Tensor:
    """gqa_decode without a workspace (the library's static per-device scratch;
    calls overlapping on one device race).  Pass `out` to allocate nothing."""
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    _shape(k_cache, (B, Hkv, S_max, D), "k_cache")
    _shape(v_cache, (B, Hkv, S_max, D), "v_cache")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _shape(out, (B, Hq, D), "out")
    _dev(out, "out")
    st = _lib.gqa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 seq_lens.data_ptr(), B, Hq, Hkv, D, S_max, float(scale),
                                 rope_params(q_rope), out.data_ptr(), _stream(stream))
    _check(st, "gqa_decode_noalloc")
    return out


def gqa_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float, q_rope=None,
                      out=None, workspace=None, stream=None) -> torch.Tensor:
    """A decode step with its cache write: k_new/v_new [B,Hkv,D] bf16 (k_new
    not rotated) go into row seq_lens[b]-1 of k_cache/v_cache (k_new rotated
    there with q_rope), then q [B,Hq,D] attends.  Returns out [B,Hq,D] bf16;
    k_cache and v_cache are updated in place."""
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    _shape(k_cache, (B, Hkv, S_max, D), "k_cache")
    _shape(v_cache, (B, Hkv, S_max, D), "v_cache")
    _shape(k_new, (B, Hkv, D), "k_new")
    _shape(v_new, (B, Hkv, D), "v_new")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _dev(t, nm)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _shape(out, (B, Hq, D), "out")
    _dev(out, "out")
    need = gqa_decode_workspace_size(B, Hq, Hkv, D, S_max)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = _lib.gqa_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, S_max,
                                float(scale), rope_params(q_rope), out.data_ptr(),
                                workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "gqa_decode_append")
    return out


def gqa_decode_window(q, k_cache, v_cache, seq_lens, scale: float, window: int = 0,
                      rolling: bool = False, k_new=None, v_new=None, q_rope=None, out=None,
                      workspace=None, stream=None, sinks: int = 0) -> torch.Tensor:
    """gqa_decode over the last `window` positions of a linear cache, or of a
    rolling buffer (rolling=True: position t in slot t mod S_max; window 0
    attends to every filled slot, 0 < window <= S_max - sinks to the last
    `window` positions, whose slots may wrap), optionally writing the new
    token's k_new/v_new [B,Hkv,D] first.  sinks > 0 (gqa_decode_sink_window)
    also keeps the first `sinks` positions visible (linear cache) or in the
    buffer's first slots (rolling).  Returns out [B,Hq,D] bf16."""
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    _shape(k_cache, (B, Hkv, S_max, D), "k_cache")
    _shape(v_cache, (B, Hkv, S_max, D), "v_cache")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _shape(k_new, (B, Hkv, D), "k_new")
        _shape(v_new, (B, Hkv, D), "v_new")
        _dev(k_new, "k_new")
        _dev(v_new, "v_new")
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _shape(out, (B, Hq, D), "out")
    _dev(out, "out")
    need = gqa_decode_workspace_size(B, Hq, Hkv, D, S_max)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    kn = k_new.data_ptr() if k_new is not None else None
    vn = v_new.data_ptr() if v_new is not None else None
    if sinks:
        st = _lib.gqa_decode_sink_window(q.data_ptr(), kn, vn, k_cache.data_ptr(),
                                         v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D,
                                         S_max, int(sinks), int(window), int(bool(rolling)),
                                         float(scale), rope_params(q_rope), out.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), _stream(stream))
        _check(st, "gqa_decode_sink_window")
        return out
    st = _lib.gqa_decode_window(q.data_ptr(), kn, vn, k_cache.data_ptr(),
                                v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, S_max,
                                int(window), int(bool(rolling)), float(scale), rope_params(q_rope),
                                out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream(stream))
    _check(st, "gqa_decode_window")
    return out


def gqa_decode_partial(q, k_cache, v_cache, seq_lens, scale: float, workspace, q_rope=None,
                       n_parts: int = 0, stream=None) -> None:
    """Phase 1 of gqa_decode: per-split softmax states into `workspace`."""
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    _shape(k_cache, (B, Hkv, S_max, D), "k_cache")
    _shape(v_cache, (B, Hkv, S_max, D), "v_cache")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = _lib.gqa_decode_partial(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 seq_lens.data_ptr(), B, Hq, Hkv, D, S_max, float(scale),
                                 rope_params(q_rope), workspace.data_ptr(), workspace.numel(),
                                 int(n_parts), _stream(stream))
    _check(st, "gqa_decode_partial")


def gqa_decode_combine(seq_lens, B, Hq, Hkv, D, S_max, workspace, out, n_parts: int = 0,
                       stream=None) -> torch.Tensor:
    """Phase 2 of gqa_decode: merge the per-split states into out [B,Hq,D] bf16."""
    _shape(seq_lens, (B,), "seq_lens")
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    _dev(workspace, "workspace", dtype=torch.uint8)
    _shape(out, (B, Hq, D), "out")
    _dev(out, "out")
    st = _lib.gqa_decode_combine(seq_lens.data_ptr(), B, Hq, Hkv, D, S_max, workspace.data_ptr(),
                                 workspace.numel(), int(n_parts), out.data_ptr(), _stream(stream))
    _check(st, "gqa_decode_combine")
    return out


def gqa_prefill_workspace_size(B, Hkv, T, D, rope=None) -> int:
    return int(_lib.gqa_prefill_workspace_size(B, Hkv, T, D, rope_params(rope)))


def gqa_prefill_causal(q, k, v, scale: float, rope=None, out=None, workspace=None,
                       stream=None, window: int = 0, sinks: int = 0,
                       fp16_scores: bool = False) -> torch.Tensor:
    """q [B,Hq,T,D], k/v [B,Hkv,T,D] bf16 (pre-RoPE).  Returns out [B,Hq,T,D].
    window > 0: sliding window (row i sees keys i-window+1 .. i); sinks > 0
    keeps keys 0 .. sinks-1 visible beside it (gqa_prefill_sink_window);
    fp16_scores: one-product fp16 scores (gqa_prefill_fp16)."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    _shape(k, (B, Hkv, T, D), "k")
    _shape(v, (B, Hkv, T, D), "v")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm)
    if out is None:
        out = torch.empty_like(q)
    _shape(out, q.shape, "out")
    _dev(out, "out")
    need = gqa_prefill_workspace_size(B, Hkv, T, D, rope)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    if fp16_scores or sinks:
        fn = _lib.gqa_prefill_fp16 if fp16_scores else _lib.gqa_prefill_sink_window
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, Hq, Hkv, D, int(sinks),
                int(window), float(scale), rope_params(rope), out.data_ptr(),
                workspace.data_ptr(), workspace.numel(), _stream(stream))
        _check(st, "gqa_prefill_fp16" if fp16_scores else "gqa_prefill_sink_window")
        return out
    if window:
        st = _lib.gqa_prefill_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, Hq, Hkv, D,
                                     int(window), float(scale), rope_params(rope), out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream(stream))
        _check(st, "gqa_prefill_window")
        return out
    st = _lib.gqa_prefill_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, Hq, Hkv, D,
                                 float(scale), rope_params(rope), out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "gqa_prefill_causal")
    return out


def topk_sparse_decode_workspace_size(B, H, S_max, top_k) -> int:
    return int(_lib.topk_sparse_decode_workspace_size(B, H, S_max, top_k))


def topk_sparse_decode(q, latent, q_index, k_index, seq_lens, top_k: int, scale: float, Dv: int = 512,
                       topk_idx=None, out=None, workspace=None, stream=None):
    """q [B,H,Dqk], latent [B,S_max,Dqk], q_index [B,D_idx], k_index [B,S_max,D_idx] (bf16),
    seq_lens int32 [B].  Returns (topk_idx int32 [B,top_k], out bf16 [B,H,Dv])."""
    B, H, Dqk = q.shape
    S_max = latent.shape[1]
    D_idx = q_index.shape[1]
    _shape(latent, (B, S_max, Dqk), "latent")
    _shape(q_index, (B, D_idx), "q_index")
    _shape(k_index, (B, S_max, D_idx), "k_index")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (latent, "latent"), (q_index, "q_index"), (k_index, "k_index")):
        _dev(t, nm)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if topk_idx is None:
        topk_idx = torch.empty((B, top_k), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=q.device)
    _shape(topk_idx, (B, top_k), "topk_idx")
    _shape(out, (B, H, Dv), "out")
    _dev(topk_idx, "topk_idx", dtype=torch.int32)
    _dev(out, "out")
    need = topk_sparse_decode_workspace_size(B, H, S_max, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = _lib.topk_sparse_decode(q.data_ptr(), latent.data_ptr(), q_index.data_ptr(),
                                 k_index.data_ptr(), seq_lens.data_ptr(), B, H, Dqk, Dv, D_idx,
                                 S_max, int(top_k), float(scale), topk_idx.data_ptr(),
                                 out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                 _stream(stream))
    _check(st, "topk_sparse_decode")
    return topk_idx, out


def topk_sparse_decode_weighted(q, latent, q_index, w_index, k_index, seq_lens, top_k: int,
                                scale: float, Dv: int = 512, topk_idx=None, out=None,
                                workspace=None, stream=None):
    """topk_sparse_decode with the multi-head weighted indexer: q_index
    [B,H_I,D_idx] bf16, w_index [B,H_I] float32.  Returns (topk_idx, out)."""
    B, H, Dqk = q.shape
    S_max = latent.shape[1]
    H_I, D_idx = q_index.shape[1], q_index.shape[2]
    _shape(latent, (B, S_max, Dqk), "latent")
    _shape(q_index, (B, H_I, D_idx), "q_index")
    _shape(w_index, (B, H_I), "w_index")
    _shape(k_index, (B, S_max, D_idx), "k_index")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (latent, "latent"), (q_index, "q_index"), (k_index, "k_index")):
        _dev(t, nm)
    _dev(w_index, "w_index", dtype=torch.float32)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if topk_idx is None:
        topk_idx = torch.empty((B, top_k), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=q.device)
    _shape(topk_idx, (B, top_k), "topk_idx")
    _shape(out, (B, H, Dv), "out")
    _dev(topk_idx, "topk_idx", dtype=torch.int32)
    _dev(out, "out")
    need = topk_sparse_decode_workspace_size(B, H, S_max, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = _lib.topk_sparse_decode_weighted(q.data_ptr(), latent.data_ptr(), q_index.data_ptr(),
                                          w_index.data_ptr(), k_index.data_ptr(),
                                          seq_lens.data_ptr(), B, H, H_I, Dqk, Dv, D_idx, S_max,
                                          int(top_k), float(scale), topk_idx.data_ptr(),
                                          out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                          _stream(stream))
    _check(st, "topk_sparse_decode_weighted")
    return topk_idx, out


QSA_TOKENS = 4 * 512 + 3


def qsa_sparse_decode_workspace_size(B, Hq, S_max) -> int:
    return int(_lib.qsa_sparse_decode_workspace_size(B, Hq, S_max))


def qsa_sparse_decode(q, k_cache, v_cache, q_index, k_index, seq_lens, scale: float,
                      block_rope=None, token_idx=None, out=None, workspace=None, stream=None):
    """q [B,Hq,D] (rotated), k/v caches [B,Hkv,S_max,D], q_index [B,H_I,D_idx]
    (rotated), k_index [B,S_max,D_idx] (pre-RoPE), all bf16; seq_lens int32
    [B].  Returns (token_idx int32 [B,2051], out bf16 [B,Hq,D])."""
    B, Hq, D = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    H_I, D_idx = q_index.shape[1], q_index.shape[2]
    _shape(k_cache, (B, Hkv, S_max, D), "k_cache")
    _shape(v_cache, (B, Hkv, S_max, D), "v_cache")
    _shape(q_index, (B, H_I, D_idx), "q_index")
    _shape(k_index, (B, S_max, D_idx), "k_index")
    _shape(seq_lens, (B,), "seq_lens")
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (q_index, "q_index"),
                  (k_index, "k_index")):
        _dev(t, nm)
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if token_idx is None:
        token_idx = torch.empty((B, QSA_TOKENS), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _shape(token_idx, (B, QSA_TOKENS), "token_idx")
    _shape(out, (B, Hq, D), "out")
    _dev(token_idx, "token_idx", dtype=torch.int32)
    _dev(out, "out")
    need = qsa_sparse_decode_workspace_size(B, Hq, S_max)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = _lib.qsa_sparse_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                q_index.data_ptr(), k_index.data_ptr(), seq_lens.data_ptr(), B, Hq,
                                Hkv, D, H_I, D_idx, S_max, float(scale), rope_params(block_rope),
                                token_idx.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _stream(stream))
    _check(st, "qsa_sparse_decode")
    return token_idx, out


def mla_decode_workspace_size(B, H, S_max) -> int:
    return int(_lib.mla_decode_workspace_size(B, H, S_max))


def mla_decode(q, latent, seq_lens, scale: float, Dv: int = 512, out=None, workspace=None,
               stream=None):
    """q [B,H,Dqk], latent [B,S_max,Dqk] (bf16), seq_lens int32 [B].
    Returns out bf16 [B,H,Dv]: every head attends to all latent rows < seq_lens[b]."""
    B, H, Dqk = q.shape
    S_max = latent.shape[1]
    _shape(latent, (B, S_max, Dqk), "latent")
    _shape(seq_lens, (B,), "seq_lens")
    _dev(q, "q")
    _dev(latent, "latent")
    _dev(seq_lens, "seq_lens", dtype=torch.int32)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=q.device)
    _shape(out, (B, H, Dv), "out")
    _dev(out, "out")
    need = mla_decode_workspace_size(B, H, S_max)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", dtype=torch.uint8)
    st = _lib.mla_decode(q.data_ptr(), latent.data_ptr(), seq_lens.data_ptr(), B, H, Dqk, Dv, S_max,
                         float(scale), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                         _stream(stream))
    _check(st, "mla_decode")
    return out
