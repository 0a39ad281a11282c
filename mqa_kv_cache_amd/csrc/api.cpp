// C ABI of libgqa_attn: argument validation on the host, then launches on
// the caller's stream.  Nothing here touches the device before validation
// has passed, so every error path is testable without a GPU.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "host_common.h"

namespace gqa {

static bool finite(double x) { return std::isfinite(x); }

gqa_status rope_prepare(const gqa_rope_params* p, int32_t head_dim, RopeDev* out, int64_t cur_len) {
    std::memset(out, 0, sizeof(*out));
    out->pos_scale = 1.0;
    out->amp = 1.0f;
    if (p == nullptr || p->scaling == GQA_ROPE_NONE) return GQA_OK;
    if (p->scaling < GQA_ROPE_PLAIN || p->scaling > GQA_ROPE_DYNAMIC_NTK) return GQA_ERR_INVALID_ARGUMENT;
    const int32_t rd = p->rotary_dim == 0 ? head_dim : p->rotary_dim;
    if (rd < 2 || (rd & 1) || rd > head_dim) return GQA_ERR_INVALID_ARGUMENT;
    if ((rd % 8) != 0 || rd / 2 > kMaxRotaryHalf) return GQA_ERR_UNSUPPORTED;
    if (!finite(p->base) || !(p->base > 1.0)) return GQA_ERR_INVALID_ARGUMENT;
    if (!finite(p->factor)) return GQA_ERR_INVALID_ARGUMENT;
    if (p->scaling == GQA_ROPE_PLAIN || p->scaling == GQA_ROPE_DYNAMIC_NTK) {
        if (p->factor != 1.0) return GQA_ERR_INVALID_ARGUMENT;
    } else if (!(p->factor >= 1.0)) {
        return GQA_ERR_INVALID_ARGUMENT;
    }
    const int half = rd / 2;
    double s = p->factor;
    if (p->scaling == GQA_ROPE_DYNAMIC_NTK) {
        // s = max(1, L_cur / L_train) ([transformer架构] §1.2 ④), then NTK
        if (p->original_max_position <= 0 || rd <= 2 || cur_len < 0) return GQA_ERR_INVALID_ARGUMENT;
        if (cur_len == 0) {
            out->dyn_train = p->original_max_position;
            out->dyn_exp = -2.0 / (double)(rd - 2);
        } else {
            s = std::max(1.0, (double)cur_len / (double)p->original_max_position);
        }
    }
    double base = p->base;
    if (p->scaling == GQA_ROPE_NTK || (p->scaling == GQA_ROPE_DYNAMIC_NTK && cur_len > 0)) {
        if (rd <= 2) return GQA_ERR_INVALID_ARGUMENT;
        base = p->base * std::pow(s, (double)rd / (double)(rd - 2));  // b' = b s^(d/(d-2))
    }
    if (p->scaling == GQA_ROPE_YARN) {
        if (p->original_max_position <= 0 || !finite(p->yarn_alpha) || !finite(p->yarn_beta) ||
            !(p->yarn_beta > p->yarn_alpha))
            return GQA_ERR_INVALID_ARGUMENT;
    }
    for (int i = 0; i < half; ++i) {
        const double th = std::pow(base, -2.0 * i / (double)rd);
        double eff = th;
        if (p->scaling == GQA_ROPE_YARN) {
            // r = turns of this pair within L_train; ramp 0 below alpha, 1 above beta
            const double r = (double)p->original_max_position * th / (2.0 * M_PI);
            double gamma;
            if (r > p->yarn_beta) gamma = 1.0;
            else if (r <= p->yarn_alpha) gamma = 0.0;
            else gamma = (r - p->yarn_alpha) / (p->yarn_beta - p->yarn_alpha);
            eff = (1.0 - gamma) * th / s + gamma * th;
        }
        out->theta[i] = eff;
    }
    if (p->scaling == GQA_ROPE_PI) out->pos_scale = 1.0 / s;
    if (p->scaling == GQA_ROPE_YARN && p->yarn_mscale) out->amp = (float)(0.1 * std::log(s) + 1.0);
    out->half = half;
    return GQA_OK;
}

static gqa_status from_hip(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_DEVICE; }

}  // namespace gqa

using namespace gqa;

extern "C" {

const char* gqa_status_string(int32_t status) {
    switch (status) {
        case GQA_OK: return "ok";
        case GQA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
        case GQA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case GQA_ERR_DEVICE: return "device error";
        default: return "unknown status";
    }
}

int64_t kv_bytes_per_token(int32_t layers, int32_t n_kv_heads, int32_t head_dim, int32_t bytes_per_elem) {
    if (layers < 0 || n_kv_heads < 0 || head_dim < 0 || bytes_per_elem < 0) return -1;
    __int128 v = (__int128)2 * layers * n_kv_heads * head_dim * bytes_per_elem;
    if (v > (__int128)INT64_MAX) return -1;
    return (int64_t)v;
}

int64_t mla_kv_bytes_per_token(int32_t layers, int32_t d_latent, int32_t d_rope, int32_t bytes_per_elem) {
    if (layers < 0 || d_latent < 0 || d_rope < 0 || bytes_per_elem < 0) return -1;
    __int128 v = (__int128)layers * ((__int128)d_latent + d_rope) * bytes_per_elem;
    if (v > (__int128)INT64_MAX) return -1;
    return (int64_t)v;
}

gqa_status rope_apply(const void* in, void* out, const int32_t* positions, int64_t n_tok,
                      int32_t n_heads, int32_t head_dim, int64_t stride_tok, int64_t stride_head,
                      const gqa_rope_params* rope, void* stream) {
    if (n_tok < 0 || n_heads < 1 || head_dim < 1 || stride_tok < 0 || stride_head < 0)
        return GQA_ERR_INVALID_ARGUMENT;
    if ((head_dim % 8) != 0 || head_dim > 1024) return GQA_ERR_UNSUPPORTED;
    if ((stride_tok % 8) != 0 || (stride_head % 8) != 0) return GQA_ERR_INVALID_ARGUMENT;
    RopeDev rd;
    if (rope && rope->scaling == GQA_ROPE_DYNAMIC_NTK && rope->current_len < 1)
        return GQA_ERR_INVALID_ARGUMENT;
    gqa_status st = rope_prepare(rope, head_dim, &rd, rope ? rope->current_len : 0);
    if (st != GQA_OK) return st;
    if (n_tok == 0) return GQA_OK;
    if (!in || !out || !aligned16(in) || !aligned16(out)) return GQA_ERR_INVALID_ARGUMENT;
    if (rd.half > 0 && !positions) return GQA_ERR_INVALID_ARGUMENT;
    return from_hip(launch_rope_apply(in, out, positions, n_tok, n_heads, head_dim, stride_tok,
                                      stride_head, rd, (hipStream_t)stream));
}

static gqa_status check_decode_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max) {
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || S_max < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv) return GQA_ERR_INVALID_ARGUMENT;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (Hq / Hkv > 64) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)S_max * D * 2 >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv > 65535 * 65535LL) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

static int32_t pick_parts(int32_t n_parts) { return n_parts == 0 ? kDecodeDefaultParts : n_parts; }

static bool parts_ok(int32_t n_parts) { return n_parts >= 1 && n_parts <= (1 << 20); }

size_t gqa_decode_workspace_size_parts(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max,
                                       int32_t n_parts) {
    if (check_decode_shape(B, Hq, Hkv, D, S_max) != GQA_OK) return 0;
    n_parts = pick_parts(n_parts);
    if (!parts_ok(n_parts)) return 0;
    return decode_layout(B, Hq, Hkv, D, n_parts).total;
}

size_t gqa_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max) {
    return gqa_decode_workspace_size_parts(B, Hq, Hkv, D, S_max, 0);
}

gqa_status gqa_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t S_max, float scale, const gqa_rope_params* q_rope,
                              void* workspace, size_t workspace_bytes, int32_t n_parts,
                              void* stream) {
    gqa_status st = check_decode_shape(B, Hq, Hkv, D, S_max);
    if (st != GQA_OK) return st;
    n_parts = pick_parts(n_parts);
    if (!parts_ok(n_parts)) return GQA_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !k_cache || !v_cache || !seq_lens || !workspace) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    RopeDev rd;
    st = rope_prepare(q_rope, D, &rd, 0);
    if (st != GQA_OK) return st;
    const DecodeLayout lay = decode_layout(B, Hq, Hkv, D, n_parts);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(launch_gqa_decode_partial(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max,
                                              scale, rd, workspace, lay, (hipStream_t)stream));
}

gqa_status gqa_decode_combine(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t S_max, const void* workspace, size_t workspace_bytes,
                              int32_t n_parts, void* out, void* stream) {
    gqa_status st = check_decode_shape(B, Hq, Hkv, D, S_max);
    if (st != GQA_OK) return st;
    n_parts = pick_parts(n_parts);
    if (!parts_ok(n_parts)) return GQA_ERR_INVALID_ARGUMENT;
    if (!seq_lens || !workspace || !out) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    const DecodeLayout lay = decode_layout(B, Hq, Hkv, D, n_parts);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(launch_gqa_decode_combine(seq_lens, B, Hq, Hkv, D, S_max, workspace, lay, out,
                                              (hipStream_t)stream));
}

gqa_status gqa_decode_parts(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t S_max, float scale, const gqa_rope_params* q_rope, void* out,
                            void* workspace, size_t workspace_bytes, int32_t n_parts,
                            void* stream) {
    if (!out) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(out)) return GQA_ERR_INVALID_ARGUMENT;
    gqa_status st = gqa_decode_partial(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max, scale,
                                       q_rope, workspace, workspace_bytes, n_parts, stream);
    if (st != GQA_OK) return st;
    return gqa_decode_combine(seq_lens, B, Hq, Hkv, D, S_max, workspace, workspace_bytes, n_parts,
                              out, stream);
}

gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                      int32_t S_max, float scale, const gqa_rope_params* q_rope, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return gqa_decode_parts(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max, scale, q_rope, out,
                            workspace, workspace_bytes, 0, stream);
}

gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t S_max, float scale, const gqa_rope_params* q_rope,
                              void* out, void* stream) {
    // the same validation as gqa_decode, then the size check against the
    // static scratch; nothing is allocated
    gqa_status st = check_decode_shape(B, Hq, Hkv, D, S_max);
    if (st != GQA_OK) return st;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return GQA_ERR_INVALID_ARGUMENT;
    RopeDev rd;
    st = rope_prepare(q_rope, D, &rd, 0);
    if (st != GQA_OK) return st;
    const DecodeLayout lay = decode_layout(B, Hq, Hkv, D, kDecodeDefaultParts);
    if (lay.total > kNoAllocScratchBytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    st = from_hip(noalloc_scratch(&ws));
    if (st != GQA_OK) return st;
    st = from_hip(launch_gqa_decode_partial(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max,
                                            scale, rd, ws, lay, (hipStream_t)stream));
    if (st != GQA_OK) return st;
    return from_hip(launch_gqa_decode_combine(seq_lens, B, Hq, Hkv, D, S_max, ws, lay, out,
                                              (hipStream_t)stream));
}

gqa_status gqa_decode_sink_window(const void* q, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, const int32_t* seq_lens, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t S_max, int32_t sinks,
                                  int32_t window, int32_t rolling, float scale,
                                  const gqa_rope_params* q_rope, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    gqa_status st = check_decode_shape(B, Hq, Hkv, D, S_max);
    if (st != GQA_OK) return st;
    if (!std::isfinite(scale) || window < 0 || sinks < 0 || (rolling != 0 && rolling != 1))
        return GQA_ERR_INVALID_ARGUMENT;
    if (rolling && (sinks >= S_max || window > S_max - sinks)) return GQA_ERR_INVALID_ARGUMENT;
    if ((k_new == nullptr) != (v_new == nullptr)) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !k_cache || !v_cache || !seq_lens || !workspace || !out)
        return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || (k_new && (!aligned16(k_new) || !aligned16(v_new))) ||
        !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    RopeDev rd;
    st = rope_prepare(q_rope, D, &rd, 0);
    if (st != GQA_OK) return st;
    const DecodeLayout lay = decode_layout(B, Hq, Hkv, D, kDecodeDefaultParts);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    if (!rolling && window == 0) sinks = 0;   // no band: every row is attended already
    st = from_hip(launch_gqa_decode_partial(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max,
                                            scale, rd, workspace, lay, (hipStream_t)stream, k_new,
                                            v_new, window, rolling, sinks));
    if (st != GQA_OK) return st;
    return from_hip(launch_gqa_decode_combine(seq_lens, B, Hq, Hkv, D, S_max, workspace, lay, out,
                                              (hipStream_t)stream, window, rolling, sinks));
}

gqa_status gqa_decode_window(const void* q, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const int32_t* seq_lens, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t S_max, int32_t window, int32_t rolling,
                             float scale, const gqa_rope_params* q_rope, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return gqa_decode_sink_window(q, k_new, v_new, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max,
                                  0, window, rolling, scale, q_rope, out, workspace,
                                  workspace_bytes, stream);
}

gqa_status gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const int32_t* seq_lens, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t S_max, float scale,
                             const gqa_rope_params* q_rope, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (!k_new || !v_new) return GQA_ERR_INVALID_ARGUMENT;
    return gqa_decode_window(q, k_new, v_new, k_cache, v_cache, seq_lens, B, Hq, Hkv, D, S_max, 0,
                             0, scale, q_rope, out, workspace, workspace_bytes, stream);
}

static gqa_status check_prefill_shape(int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv) return GQA_ERR_INVALID_ARGUMENT;
    if (D != 8 && D != 16 && D != 32 && D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)T * D * 2 >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq > 65535) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

size_t gqa_prefill_workspace_size(int32_t B, int32_t Hkv, int32_t T, int32_t D,
                                  const gqa_rope_params* rope) {
    if (B < 1 || Hkv < 1 || T < 1 || D < 1) return 0;
    RopeDev rd;
    if (rope_prepare(rope, D, &rd, T) != GQA_OK) return 0;
    return 3 * prefill_prep_bytes(B, Hkv, T, D);
}

// Every prefill entry point: validation, then the pre-pass and main kernel.
static gqa_status prefill_common(const void* q, const void* k, const void* v, int32_t B, int32_t T,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t sinks, int32_t window,
                                 float scale, const gqa_rope_params* rope, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 int32_t fp16_scores) {
    gqa_status st = check_prefill_shape(B, T, Hq, Hkv, D);
    if (st != GQA_OK) return st;
    if (!std::isfinite(scale) || window < 0 || sinks < 0) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return GQA_ERR_INVALID_ARGUMENT;
    RopeDev rd;
    st = rope_prepare(rope, D, &rd, T);
    if (st != GQA_OK) return st;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GQA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < 3 * prefill_prep_bytes(B, Hkv, T, D)) return GQA_ERR_WORKSPACE_TOO_SMALL;
    // a window of T or more keys (or none) is the causal mask, and sinks only
    // matter beside a band that leaves keys out
    if (window >= T) window = 0;
    if (window == 0 || sinks >= T) {
        window = 0;
        sinks = 0;
    }
    return from_hip(launch_gqa_prefill(q, k, v, B, T, Hq, Hkv, D, scale, rd, out, workspace,
                                       (hipStream_t)stream, window, sinks, fp16_scores));
}

gqa_status gqa_prefill_window(const void* q, const void* k, const void* v, int32_t B, int32_t T,
                              int32_t Hq, int32_t Hkv, int32_t D, int32_t window, float scale,
                              const gqa_rope_params* rope, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return prefill_common(q, k, v, B, T, Hq, Hkv, D, 0, window, scale, rope, out, workspace,
                          workspace_bytes, stream, 0);
}

gqa_status gqa_prefill_causal(const void* q, const void* k, const void* v, int32_t B, int32_t T,
                              int32_t Hq, int32_t Hkv, int32_t D, float scale,
                              const gqa_rope_params* rope, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return prefill_common(q, k, v, B, T, Hq, Hkv, D, 0, 0, scale, rope, out, workspace,
                          workspace_bytes, stream, 0);
}

gqa_status gqa_prefill_sink_window(const void* q, const void* k, const void* v, int32_t B,
                                   int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t sinks,
                                   int32_t window, float scale, const gqa_rope_params* rope,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    return prefill_common(q, k, v, B, T, Hq, Hkv, D, sinks, window, scale, rope, out, workspace,
                          workspace_bytes, stream, 0);
}

gqa_status gqa_prefill_fp16(const void* q, const void* k, const void* v, int32_t B, int32_t T,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t sinks, int32_t window,
                            float scale, const gqa_rope_params* rope, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return prefill_common(q, k, v, B, T, Hq, Hkv, D, sinks, window, scale, rope, out, workspace,
                          workspace_bytes, stream, 1);
}

static gqa_status check_sparse_shape(int32_t B, int32_t H, int32_t Dqk, int32_t Dv, int32_t D_idx,
                                     int32_t S_max, int32_t top_k) {
    if (B < 1 || H < 1 || Dqk < 1 || Dv < 1 || D_idx < 1 || S_max < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (top_k < 1 || top_k > S_max || Dv > Dqk) return GQA_ERR_INVALID_ARGUMENT;
    if (Dqk != 576 || Dv != 512 || D_idx != 128) return GQA_ERR_UNSUPPORTED;
    if ((H % 16) || H > 128) return GQA_ERR_UNSUPPORTED;
    if (top_k > 4096) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)S_max * Dqk * 2 >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

size_t topk_sparse_decode_workspace_size(int32_t B, int32_t H, int32_t S_max, int32_t top_k) {
    if (check_sparse_shape(B, H, 576, 512, 128, S_max, top_k) != GQA_OK) return 0;
    return sparse_layout(B, H, S_max, top_k).total;
}

gqa_status topk_sparse_decode(const void* q, const void* latent, const void* q_index,
                              const void* k_index, const int32_t* seq_lens, int32_t B, int32_t H,
                              int32_t Dqk, int32_t Dv, int32_t D_idx, int32_t S_max, int32_t top_k,
                              float scale, int32_t* topk_idx, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
    gqa_status st = check_sparse_shape(B, H, Dqk, Dv, D_idx, S_max, top_k);
    if (st != GQA_OK) return st;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !latent || !q_index || !k_index || !seq_lens || !topk_idx || !out || !workspace)
        return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(latent) || !aligned16(q_index) || !aligned16(k_index) ||
        !aligned16(topk_idx) || !aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    const SparseLayout lay = sparse_layout(B, H, S_max, top_k);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(launch_topk_sparse_decode(q, latent, q_index, k_index, seq_lens, B, H, S_max,
                                              top_k, scale, topk_idx, out, workspace, lay,
                                              (hipStream_t)stream));
}

gqa_status topk_sparse_decode_weighted(const void* q, const void* latent, const void* q_index,
                                       const float* w_index, const void* k_index,
                                       const int32_t* seq_lens, int32_t B, int32_t H, int32_t H_I,
                                       int32_t Dqk, int32_t Dv, int32_t D_idx, int32_t S_max,
                                       int32_t top_k, float scale, int32_t* topk_idx, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    gqa_status st = check_sparse_shape(B, H, Dqk, Dv, D_idx, S_max, top_k);
    if (st != GQA_OK) return st;
    if (H_I < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (H_I != 16 && H_I != 32 && H_I != 48 && H_I != 64) return GQA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !latent || !q_index || !w_index || !k_index || !seq_lens || !topk_idx || !out ||
        !workspace)
        return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(latent) || !aligned16(q_index) || !aligned16(k_index) ||
        !aligned16(topk_idx) || !aligned16(out) || (reinterpret_cast<uintptr_t>(w_index) & 3u) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    const SparseLayout lay = sparse_layout(B, H, S_max, top_k);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(launch_topk_sparse_decode(q, latent, q_index, k_index, seq_lens, B, H, S_max,
                                              top_k, scale, topk_idx, out, workspace, lay,
                                              (hipStream_t)stream, w_index, H_I));
}

size_t qsa_sparse_decode_workspace_size(int32_t B, int32_t Hq, int32_t S_max) {
    if (B < 1 || Hq < 1 || S_max < 1) return 0;
    return qsa_layout(B, Hq, S_max).total;
}

gqa_status qsa_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                             const void* q_index, const void* k_index, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t H_I,
                             int32_t D_idx, int32_t S_max, float scale,
                             const gqa_rope_params* block_rope, int32_t* token_idx, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || H_I < 1 || D_idx < 1 || S_max < 1)
        return GQA_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv) return GQA_ERR_INVALID_ARGUMENT;
    if (D != 128 || D_idx != 128 || Hq / Hkv > 16) return GQA_ERR_UNSUPPORTED;
    if (H_I != 16 && H_I != 32 && H_I != 48 && H_I != 64) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)S_max * D * 2 >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (block_rope && block_rope->scaling == GQA_ROPE_DYNAMIC_NTK) return GQA_ERR_UNSUPPORTED;
    RopeDev rd;
    gqa_status st = rope_prepare(block_rope, D_idx, &rd, 1);
    if (st != GQA_OK) return st;
    if (!q || !k_cache || !v_cache || !q_index || !k_index || !seq_lens || !token_idx || !out ||
        !workspace)
        return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q_index) ||
        !aligned16(k_index) || !aligned16(token_idx) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    const QsaLayout lay = qsa_layout(B, Hq, S_max);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(launch_qsa_sparse_decode(q, k_cache, v_cache, q_index, k_index, seq_lens, B, Hq,
                                             Hkv, H_I, S_max, scale, rd, token_idx, out, workspace,
                                             lay, (hipStream_t)stream));
}

static gqa_status check_mla_shape(int32_t B, int32_t H, int32_t Dqk, int32_t Dv, int32_t S_max) {
    if (B < 1 || H < 1 || Dqk < 1 || Dv < 1 || S_max < 1 || Dv > Dqk) return GQA_ERR_INVALID_ARGUMENT;
    if (Dqk != 576 || Dv != 512) return GQA_ERR_UNSUPPORTED;
    if ((H % 16) || H > 128) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)S_max * Dqk * 2 >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

size_t mla_decode_workspace_size(int32_t B, int32_t H, int32_t S_max) {
    if (check_mla_shape(B, H, 576, 512, S_max) != GQA_OK) return 0;
    return mla_layout(B, H, S_max).total;
}

gqa_status mla_decode(const void* q, const void* latent, const int32_t* seq_lens, int32_t B,
                      int32_t H, int32_t Dqk, int32_t Dv, int32_t S_max, float scale, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
    gqa_status st = check_mla_shape(B, H, Dqk, Dv, S_max);
    if (st != GQA_OK) return st;
    if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (!q || !latent || !seq_lens || !out || !workspace) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(latent) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return GQA_ERR_INVALID_ARGUMENT;
    const MlaLayout lay = mla_layout(B, H, S_max);
    if (workspace_bytes < lay.total) return GQA_ERR_WORKSPACE_TOO_SMALL;
    return from_hip(launch_mla_decode(q, latent, seq_lens, B, H, S_max, scale, out, workspace, lay,
                                      (hipStream_t)stream));
}

}  // extern "C"
