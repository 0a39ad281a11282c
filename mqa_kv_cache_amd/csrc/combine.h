// Merge of split-K partial softmax states (shared by dense and sparse decode).
#pragma once

#include "device_common.h"

namespace gqa {
namespace {

// One wave per (batch, head).  Partials of split s hold m_s (running max of
// the base-2 scores), l_s (sum of 2^(score - m_s)) and o_s (the matching
// unnormalised weighted sum of V rows).  The softmax over the union is
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// an exact rewriting of the single-pass softmax.  The number of splits of
// batch b is ceil(min(seq_lens[b], cap) / rows_per_split).
template <int D>
__global__ __launch_bounds__(256) void combine_partials_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, int H, int S_max, int cap, int rows_per_split,
    int n_split_max, int BH, uint16_t* __restrict__ out) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (idx >= BH) return;
    const int b = idx / H;
    const int L = min(min(max(seq_lens[b], 1), S_max), cap);
    const int ns = (L + rows_per_split - 1) / rows_per_split;
    const float* ml = part_ml + (size_t)idx * n_split_max * 2;
    const float* po = part_o + (size_t)idx * n_split_max * D;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    float den = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = fast_exp2(ml[2 * s] - M);
        den += w * ml[2 * s + 1];
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += w * po[(size_t)s * D + lane * PER + j];
    }
    const float inv = 1.0f / den;
    uint16_t* o = out + (size_t)idx * D + lane * PER;
    if constexpr (PER == 1) {
        o[0] = (uint16_t)f32_to_bf16_bits(acc[0] * inv);
    } else {
#pragma unroll
        for (int j = 0; j < PER; j += 2)
            *reinterpret_cast<uint32_t*>(o + j) = pack_bf16x2(acc[j] * inv, acc[j + 1] * inv);
    }
}

}  // namespace
}  // namespace gqa
