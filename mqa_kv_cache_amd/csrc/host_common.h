// Internal declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/gqa_attn.h"

namespace gqa {

constexpr int kMaxRotaryHalf = 128;   // rotary_dim <= 256

// RoPE frequencies prepared on the host (fp64) and passed by value to kernels.
struct RopeDev {
    double theta[kMaxRotaryHalf];  // effective theta_i after the scaling
    double pos_scale;              // multiplies the position (PI: 1/s)
    float amp;                     // multiplies cos and sin (YaRN temperature)
    int32_t half;                  // rotary_dim / 2; 0 = no rotation
    int32_t dyn_train;             // > 0: Dynamic NTK per sequence with this L_train; theta
                                   // holds the unscaled base^(-2i/d) and the kernel multiplies
                                   // theta_i by s^(dyn_exp * i), s = max(1, L / L_train)
    double dyn_exp;                // -2 / (d - 2)
};

// Validates `p` against head_dim and fills `out`.  p == NULL or NONE gives
// half = 0.  cur_len is the call's sequence length for Dynamic NTK: > 0 folds
// s into the table; 0 leaves s to the kernel, per sequence (decode).
gqa_status rope_prepare(const gqa_rope_params* p, int32_t head_dim, RopeDev* out, int64_t cur_len);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ----- launchers (defined next to their kernels) ---------------------------
hipError_t launch_rope_apply(const void* in, void* out, const int32_t* positions, int64_t n_tok,
                             int32_t n_heads, int32_t head_dim, int64_t stride_tok,
                             int64_t stride_head, const RopeDev& rope, hipStream_t s);

struct DecodeLayout {
    int32_t n_parts;       // equal row ranges of the global row space (one wave each)
    int64_t slots;         // 4 (ceil(n_parts / 4) + B*Hkv) partial-state slots
    size_t o_bytes;        // partial outputs  fp32 [slots][g][D]
    size_t ml_bytes;       // partial (m, l)   fp32 [slots][g][2]
    size_t total;
};
constexpr int32_t kDecodeDefaultParts = 1024;
// The no-allocation decode keeps its states in a static device array of this
// size (one per device); noalloc_scratch returns the current device's copy.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);
DecodeLayout decode_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t n_parts);

hipError_t launch_gqa_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t D, int32_t S_max, float scale, const RopeDev& rope,
                                     void* workspace, const DecodeLayout& lay, hipStream_t s,
                                     const void* k_new = nullptr, const void* v_new = nullptr,
                                     int32_t window = 0, int32_t rolling = 0, int32_t sinks = 0);
hipError_t launch_gqa_decode_combine(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t D, int32_t S_max, const void* workspace,
                                     const DecodeLayout& lay, void* out, hipStream_t s,
                                     int32_t window = 0, int32_t rolling = 0, int32_t sinks = 0);

// Bytes of one prepared tensor (K hi rows, K lo rows or fp16 V^T tiles) for
// prefill; the workspace holds three of them.
size_t prefill_prep_bytes(int32_t B, int32_t Hkv, int32_t T, int32_t D);

// window 0 = causal; sinks > 0 keeps keys < sinks visible beside the band;
// fp16_scores != 0 selects the one-product fp16 score path.
hipError_t launch_gqa_prefill(const void* q, const void* k, const void* v, int32_t B, int32_t T,
                              int32_t Hq, int32_t Hkv, int32_t D, float scale,
                              const RopeDev& rope, void* out, void* workspace, hipStream_t s,
                              int32_t window, int32_t sinks, int32_t fp16_scores);

struct SparseLayout {
    size_t scores_bytes;   // fp32 [B][S_max rounded up to 4]
    size_t hist_bytes;     // u32 [B][4096] first-digit histogram
    size_t cand_bytes;     // u32 [B][key chunks][4096] keys in bins >= the threshold bin per
                           // chunk, u32 [B][key chunks][4096] their indices, u32 [B][key chunks]
                           // their counts
    size_t info_bytes;     // per-batch threshold bin and the count above it
    size_t refine_bytes;   // multi-head indexers' band re-scoring: u32 [B][8] state, u32 [B][256]
                           // band, f64 [B][256] exact scores, u32 [B][4096] keys certainly in
    size_t o_bytes;        // fp32 attention partials
    size_t ml_bytes;
    size_t total;
    int32_t n_chunks;      // attention splits over the selected rows
    int32_t n_key_chunks;  // 4096-key chunks of the scores
};
SparseLayout sparse_layout(int32_t B, int32_t H, int32_t S_max, int32_t top_k);

struct QsaLayout {
    SparseLayout sel;         // radix select over the block scores (no attention part)
    int32_t n_blk_max;        // S_max / 4 (at least 1)
    int32_t n_chunks;         // 128-token attention chunks of the 2051-token budget
    size_t cnt_bytes;         // int32 [B] complete blocks per row
    size_t blk_bytes;         // int32 [B][512] selected blocks
    size_t o_bytes;           // fp32 [B][Hq][n_chunks][128] partial outputs
    size_t ml_bytes;          // fp32 [B][Hq][n_chunks][2]
    size_t total;
};
QsaLayout qsa_layout(int32_t B, int32_t Hq, int32_t S_max);
hipError_t launch_qsa_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const void* q_index, const void* k_index,
                                    const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t H_I, int32_t S_max, float scale, const RopeDev& rope,
                                    int32_t* tok, void* out, void* workspace, const QsaLayout& lay,
                                    hipStream_t s);

struct MlaLayout {
    int32_t rows_per_split;   // latent rows per workgroup (a multiple of 32)
    int32_t n_split;          // row ranges per batch row
    size_t o_bytes;           // fp32 partial outputs [B][H][n_split][512]
    size_t ml_bytes;          // fp32 (m, l) [B][H][n_split][2]
    size_t total;
};
MlaLayout mla_layout(int32_t B, int32_t H, int32_t S_max);
hipError_t launch_mla_decode(const void* q, const void* latent, const int32_t* seq_lens, int32_t B,
                             int32_t H, int32_t S_max, float scale, void* out, void* workspace,
                             const MlaLayout& lay, hipStream_t s);

hipError_t launch_topk_sparse_decode(const void* q, const void* latent, const void* q_index,
                                     const void* k_index, const int32_t* seq_lens, int32_t B,
                                     int32_t H, int32_t S_max, int32_t top_k, float scale,
                                     int32_t* topk_idx, void* out, void* workspace,
                                     const SparseLayout& lay, hipStream_t s, const float* w_index = nullptr,
                                     int32_t H_I = 0);

}  // namespace gqa
