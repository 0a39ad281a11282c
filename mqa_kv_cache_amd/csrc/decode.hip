// Single-token GQA decode over a bf16 KV cache: split-K flash-decode on
// gfx950 MFMA.
//
// The decode step of [注意力变体与MoE] "生成时的瓶颈" reads every cached K/V row
// once per new token; with GQA the g query heads of a group read the same
// rows ([注意力变体与MoE] "MQA 与 GQA": a real kernel lets the heads of a
// group share the bytes instead of copying K/V, raising arithmetic intensity
// g-fold).  Here the sharing happens inside the matrix core: one wave holds
// the group's g <= 16 rotated queries as the B operand of a 16x16x32 bf16
// MFMA, so every K/V byte loaded from HBM feeds all g heads at once.
//
// Per wave, one split of the context (split_rows rows of one (batch, kv
// head)), in tiles of 32 rows:
//   S^T[32 rows][16 heads] = K_tile . Q^T          (K as A operand, 8 MFMAs x2 for q hi/lo)
//   online softmax per head in fp32 (base-2; scale*log2(e) is folded into q)
//   O^T[128 d][16 heads] += V_tile^T . P^T          (8 MFMAs)
// The S^T accumulator layout is exactly the P^T operand layout the second
// MFMA needs, so probabilities never leave their lane.  V^T operands come
// from 16-byte row loads transposed 8x8 in registers.  Every K and V load is
// a 16-byte buffer load; a group of 16 lanes covers 64 contiguous bytes of a
// K row or a whole 256-byte V row.  Loads past seq_len return zero through
// the buffer descriptor's bound, so ragged tails need no branches.
//
// The combine kernel merges the per-split (m, l, o) with the usual
// log-sum-exp rescaling; the result equals the softmax over the whole row.
#include "device_common.h"
#include "combine.h"

namespace gqa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int NB>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ seq_lens, int Hq, int Hkv,
    int S_max, float qscale, RopeDev rope, float* __restrict__ part_o,
    float* __restrict__ part_ml, int split_rows, int n_split_max) {
    constexpr int KU = D / 32;  // MFMA k-steps over the head dim
    constexpr int VN = D / 8;   // lanes of a 16-lane group that carry V columns
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int G = lane >> 4, n = lane & 15;
    const int b = blockIdx.z, kv = blockIdx.y;
    const int split = blockIdx.x * 4 + wave;
    const int g = Hq / Hkv;

    const int L = min(max(seq_lens[b], 1), S_max);
    const int r0 = split * split_rows;
    if (r0 >= L) return;
    const int r1 = min(r0 + split_rows, L);

    // ---- queries of the group: RoPE at position L-1, times scale*log2(e), as hi+lo bf16
    u32x4 qhi[NB][KU], qlo[NB][KU];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int hl = nb * 16 + n;
        const bool valid = hl < g;
        const uint16_t* qrow = q + ((size_t)b * Hq + (size_t)kv * g + (valid ? hl : 0)) * D;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int d0 = 32 * u + 8 * G;
            u32x4 raw = valid ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = bf16_lo(raw[j]);
                x[2 * j + 1] = bf16_hi(raw[j]);
            }
            if (rope.half) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int i = d0 / 2 + p;
                    if (i < rope.half) {
                        float c, s;
                        rope_cos_sin(rope, (double)(L - 1), i, c, s);
                        const float xe = x[2 * p], xo = x[2 * p + 1];
                        x[2 * p] = xe * c - xo * s;
                        x[2 * p + 1] = xe * s + xo * c;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = x[2 * j] * qscale, c2 = x[2 * j + 1] * qscale;
                const uint32_t ha = f32_to_bf16_bits(a), hc = f32_to_bf16_bits(c2);
                qhi[nb][u][j] = ha | (hc << 16);
                qlo[nb][u][j] = pack_bf16x2(a - __uint_as_float(ha << 16), c2 - __uint_as_float(hc << 16));
            }
        }
    }

    const size_t slice = ((size_t)b * Hkv + kv) * (size_t)S_max * D;
    const uint32_t nbytes = (uint32_t)L * D * 2u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_cache + slice, nbytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_cache + slice, nbytes);

    f32x4 o[NB][8];
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int t = 0; t < 8; ++t) o[nb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.f;
    }

    for (int t0 = r0; t0 < r1; t0 += 32) {
        u32x4 kreg[2][KU], vreg[8];
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int u = 0; u < KU; ++u)
                kreg[th][u] = buf_load16(kr, (uint32_t)(((t0 + 16 * th + n) * D + 32 * u + 8 * G) * 2));
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t off = (n < VN) ? (uint32_t)(((t0 + slot_row(G, r)) * D + 8 * n) * 2)
                                          : 0x80000000u;  // out of range -> zeros
            vreg[r] = buf_load16(vr, off);
        }

        u32x4 vt[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) vt[t] = column_of(vreg, t);

        const bool tail = (t0 + 32 > r1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            f32x4 sc[2];
#pragma unroll
            for (int th = 0; th < 2; ++th) {
                sc[th] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    sc[th] = mfma16(kreg[th][u], qhi[nb][u], sc[th]);
                    sc[th] = mfma16(kreg[th][u], qlo[nb][u], sc[th]);
                }
            }
            if (tail) {
#pragma unroll
                for (int th = 0; th < 2; ++th)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (t0 + 16 * th + 4 * G + i >= r1) sc[th][i] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                             fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
            mx = fmaxf(mx, wave_shfl_xor(mx, 16));
            mx = fmaxf(mx, wave_shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[nb], mx);
            const float alpha = fast_exp2(m_run[nb] - m_new);
            float p[2][4];
            float ls = 0.f;
#pragma unroll
            for (int th = 0; th < 2; ++th)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[th][i] = fast_exp2(sc[th][i] - m_new);
                    ls += p[th][i];
                }
            ls += wave_shfl_xor(ls, 16);
            ls += wave_shfl_xor(ls, 32);
            l_run[nb] = l_run[nb] * alpha + ls;
            m_run[nb] = m_new;
            u32x4 pb;
            pb[0] = pack_bf16x2(p[0][0], p[0][1]);
            pb[1] = pack_bf16x2(p[0][2], p[0][3]);
            pb[2] = pack_bf16x2(p[1][0], p[1][1]);
            pb[3] = pack_bf16x2(p[1][2], p[1][3]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                o[nb][t] *= alpha;
                o[nb][t] = mfma16(vt[t], pb, o[nb][t]);
            }
        }
    }

    // ---- partial (m, l, o) of this split
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int hl = nb * 16 + n;
        if (hl >= g) continue;
        const size_t idx = ((size_t)b * Hq + (size_t)kv * g + hl) * n_split_max + split;
        float* po = part_o + idx * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 8 * (4 * G + i);  // this lane holds d = d0 + t, t = 0..7
            if (d0 < D) {
                *reinterpret_cast<f32x4*>(po + d0) =
                    f32x4{o[nb][0][i], o[nb][1][i], o[nb][2][i], o[nb][3][i]};
                *reinterpret_cast<f32x4*>(po + d0 + 4) =
                    f32x4{o[nb][4][i], o[nb][5][i], o[nb][6][i], o[nb][7][i]};
            }
        }
        if (G == 0) {
            part_ml[idx * 2] = m_run[nb];
            part_ml[idx * 2 + 1] = l_run[nb];
        }
    }
}

template <int D, int NB>
void launch_split(dim3 grid, hipStream_t s, const void* q, const void* k, const void* v,
                  const int32_t* sl, int Hq, int Hkv, int S_max, float qscale, const RopeDev& rope,
                  float* po, float* pml, int split_rows, int nsm) {
    hipLaunchKernelGGL((decode_split_kernel<D, NB>), grid, dim3(256), 0, s,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sl, Hq, Hkv,
                       S_max, qscale, rope, po, pml, split_rows, nsm);
}

}  // namespace

DecodeLayout decode_layout(int32_t B, int32_t Hq, int32_t D, int32_t S_max, int32_t split_rows) {
    DecodeLayout l;
    l.split_rows = split_rows;
    l.n_split_max = (S_max + split_rows - 1) / split_rows;
    const size_t units = (size_t)B * Hq * l.n_split_max;
    l.o_bytes = (units * D * sizeof(float) + 255) & ~(size_t)255;
    l.ml_bytes = (units * 2 * sizeof(float) + 255) & ~(size_t)255;
    l.total = l.o_bytes + l.ml_bytes;
    return l;
}

int32_t decode_default_split(int32_t B, int32_t Hkv, int32_t S_max) {
    // Aim for about 4096 waves over the whole cache (16 per CU on 256 CUs).
    const int64_t rows = (int64_t)B * Hkv * S_max;
    int64_t p = rows / 4096;
    int32_t split = 128;
    while (split < p && split < 1024) split *= 2;
    return split;
}

hipError_t launch_gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t S_max, float scale, const RopeDev& rope, void* out,
                             void* workspace, const DecodeLayout& lay, hipStream_t s) {
    float* po = reinterpret_cast<float*>(workspace);
    float* pml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + lay.o_bytes);
    const int g = Hq / Hkv;
    const int NB = (g + 15) / 16;
    const float qscale = scale * kLog2e;
    dim3 grid((lay.n_split_max + 3) / 4, Hkv, B);
    if (D == 128) {
        if (NB == 1) launch_split<128, 1>(grid, s, q, k_cache, v_cache, seq_lens, Hq, Hkv, S_max, qscale, rope, po, pml, lay.split_rows, lay.n_split_max);
        else if (NB == 2) launch_split<128, 2>(grid, s, q, k_cache, v_cache, seq_lens, Hq, Hkv, S_max, qscale, rope, po, pml, lay.split_rows, lay.n_split_max);
        else launch_split<128, 4>(grid, s, q, k_cache, v_cache, seq_lens, Hq, Hkv, S_max, qscale, rope, po, pml, lay.split_rows, lay.n_split_max);
    } else {
        if (NB == 1) launch_split<64, 1>(grid, s, q, k_cache, v_cache, seq_lens, Hq, Hkv, S_max, qscale, rope, po, pml, lay.split_rows, lay.n_split_max);
        else if (NB == 2) launch_split<64, 2>(grid, s, q, k_cache, v_cache, seq_lens, Hq, Hkv, S_max, qscale, rope, po, pml, lay.split_rows, lay.n_split_max);
        else launch_split<64, 4>(grid, s, q, k_cache, v_cache, seq_lens, Hq, Hkv, S_max, qscale, rope, po, pml, lay.split_rows, lay.n_split_max);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int BH = B * Hq;
    dim3 cgrid((BH + 3) / 4);
    if (D == 128)
        hipLaunchKernelGGL((combine_partials_kernel<128>), cgrid, dim3(256), 0, s, po, pml, seq_lens,
                           Hq, S_max, S_max, lay.split_rows, lay.n_split_max, BH, (uint16_t*)out);
    else
        hipLaunchKernelGGL((combine_partials_kernel<64>), cgrid, dim3(256), 0, s, po, pml, seq_lens,
                           Hq, S_max, S_max, lay.split_rows, lay.n_split_max, BH, (uint16_t*)out);
    return hipGetLastError();
}

}  // namespace gqa
