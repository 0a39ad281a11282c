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
template <int D>   // D a multiple of 256 (each lane holds D/64 >= 4 contiguous values)
__global__ __launch_bounds__(256) void combine_partials_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, int H, int S_max, int cap, int rows_per_split,
    int n_split_max, int BH, uint16_t* __restrict__ out) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int idx = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (idx >= BH) return;
    const int b = idx / H;
    const float* ml = part_ml + (size_t)idx * n_split_max * 2;
    const float* po = part_o + (size_t)idx * n_split_max * D + lane * PER;
    // The states of the first 64 splits are requested with seq_lens, in one
    // round trip: their slots do not depend on the split count, which only
    // says how many of them hold this call's values.  Slots past it hold
    // stale bytes (possibly not finite): they are masked by selects and
    // branches, never multiplied by a zero weight.  Lane s holds the (m, l)
    // of split s; the o rows of the first 16 splits are loaded up front
    // (they do not depend on the weights), further splits four at a time.
    constexpr int kFirst = 16;
    f32x4 v0[kFirst][PER / 4];
#pragma unroll
    for (int jj = 0; jj < kFirst; ++jj) {
        const f32x4* src = reinterpret_cast<const f32x4*>(po + (size_t)min(jj, n_split_max - 1) * D);
#pragma unroll
        for (int e = 0; e < PER / 4; ++e) v0[jj][e] = src[e];
    }
    float m0 = -INFINITY, l0 = 0.f;
    if (lane < n_split_max) {
        m0 = ml[2 * lane];
        l0 = ml[2 * lane + 1];
    }
    const int L = min(min(max(seq_lens[b], 1), S_max), cap);
    const int ns = (L + rows_per_split - 1) / rows_per_split;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    float den = 0.f, M_run = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const int cn = min(64, ns - s0);
        float m, l;
        if (s0 == 0) {
            m = m0;
            l = l0;
        } else {
            m = lane < cn ? ml[2 * (s0 + lane)] : -INFINITY;
            l = lane < cn ? ml[2 * (s0 + lane) + 1] : 0.f;
        }
        if (lane >= cn) {
            m = -INFINITY;
            l = 0.f;
        }
        const float M = wave_max(m);
        const float M_new = fmaxf(M_run, M);   // finite: every split holds a row
        const float rescale = fast_exp2(M_run - M_new);
        den *= rescale;
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] *= rescale;
        const float wl = lane < cn ? fast_exp2(m - M_new) : 0.f;
        den += wave_sum(wl * l);
        int j0 = 0;
        if (s0 == 0) {
#pragma unroll
            for (int jj = 0; jj < kFirst; ++jj) {
                if (jj < cn) {                          // wave-uniform
                    const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                __builtin_bit_cast(int, wl), jj));
#pragma unroll
                    for (int e = 0; e < PER / 4; ++e)
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[4 * e + c] += wgt * v0[jj][e][c];
                }
            }
            j0 = kFirst;
        }
        for (; j0 < cn; j0 += 4) {
            f32x4 v[4][PER / 4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int sj = s0 + min(j0 + jj, cn - 1);   // past the end: a valid split, weight 0
                const f32x4* src = reinterpret_cast<const f32x4*>(po + (size_t)sj * D);
#pragma unroll
                for (int e = 0; e < PER / 4; ++e) v[jj][e] = src[e];
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float wgt = j0 + jj < cn ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, wl), min(j0 + jj, 63)))
                                               : 0.f;
#pragma unroll
                for (int e = 0; e < PER / 4; ++e)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[4 * e + c] += wgt * v[jj][e][c];
            }
        }
        M_run = M_new;
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
