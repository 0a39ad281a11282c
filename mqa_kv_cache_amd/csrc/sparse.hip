// DSA-style top-k sparse decode over an MLA latent cache on gfx950:
//   o = Attn(q, KV[TopK(ReLU(K_I . q_I))])
// ([稀疏注意力] "改进一：DSA", the selection chain; [transformer架构] §2.2 (1)-(2);
// [attention] DSA ①-③).
//
// 1. indexer_kernel: one HBM pass over the indexer keys.  Four lanes share a
//    128-dim row (64 contiguous bytes per lane per load); products of bf16
//    values are exact in fp64 and are summed in fp64, then rounded once to
//    fp32 and passed through ReLU.
//    The pass also builds the first radix-select histogram (top 12 bits of
//    the non-negative fp32 score) in LDS and flushes it with atomics.
// 2. top-k selection by radix select over the fp32 score bits: the first
//    12-bit digit comes from the indexer's histogram; per 2048-key chunk a
//    workgroup writes the keys at or above the bin holding the k-th score
//    (every selected key is one of them) in index order; one workgroup per
//    batch row then finds the exact k-th key T from those entries (or by
//    extra passes over the scores when that bin is huge) and writes, in
//    ascending index order, every key above T plus the first equal-to-T
//    keys until k are taken.
// 3. sparse_attn_kernel: MQA attention of the H heads over the gathered
//    latent rows (the indexed rows are read straight from the cache; no copy
//    of the selection is made).  Same MFMA structure as the dense decode:
//    S^T = C . Q^T over 576 dims, softmax, O^T += C[:, :512]^T . P^T; a
//    workgroup covers 32 heads and 128 selected rows staged through LDS;
//    eight waves each score 16 heads over 32 rows, exchange maxima, P and
//    row sums through LDS, and each writes 128 of the 512 output dims of
//    its 16 heads over all 128 rows: one partial (m, l, o) per head goes to
//    combine_partials_kernel.
// 4. mla_dense_kernel: the same attention over every row of the context
//    (dense absorbed-MLA decode), 64 heads per workgroup, the rows streamed
//    through a ring of LDS buffers.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "combine.h"

namespace gqa {
namespace {

constexpr int kDqk = 576, kDv = 512, kDidx = 128;
constexpr int kHistBins = 4096;      // first digit: score bits 31..20
constexpr int kRowsPerChunk = 128;   // selected rows per attention wave
constexpr int kEntCap = 12288;       // LDS entries (keys in bins >= the threshold bin) per row
constexpr float kLog2e = 1.4426950408889634f;

// Sum over each group of four lanes, every lane receiving it (DPP quad
// permutations xor 1 and xor 2, no LDS round trip).  The terms here are sums
// of exact bf16 x bf16 products, so the fp64 result does not depend on the
// order.
template <int CTRL>
__device__ __forceinline__ double dpp_add(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return v + __hiloint2double(hi, lo);
}
__device__ __forceinline__ double quad_sum(double v) {
    // quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), [2,3,0,1] = 0x4E (lane ^ 2)
    return dpp_add<0x4E>(dpp_add<0xB1>(v));
}

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// 1. indexer
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void indexer_kernel(
    const uint16_t* __restrict__ q_index, const uint16_t* __restrict__ k_index,
    const int32_t* __restrict__ seq_lens, int S_max, int S_stride, int rows_per_block,
    float* __restrict__ scores, uint32_t* __restrict__ hist) {
    __shared__ uint32_t lh[kHistBins];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // four lanes per key row, 32 dims each: lane -> row lr, quarter qq
    const int lr = lane >> 2, qq = lane & 3;
    const int b = blockIdx.y;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int r_begin = blockIdx.x * rows_per_block;
    const int r_end = min(r_begin + rows_per_block, L);
    for (int i = tid; i < kHistBins; i += 256) lh[i] = 0u;
    __syncthreads();
    if (r_begin < r_end) {
        // lane quarter qq holds dims 32 c + 8 qq + (0..7), c = 0..3, so each
        // load instruction covers 64 contiguous bytes of each of 16 rows
        double qv[32];
        const uint16_t* qrow = q_index + (size_t)b * kDidx + 8 * qq;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 qraw = *reinterpret_cast<const u32x4*>(qrow + 32 * c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qv[8 * c + 2 * j] = (double)bf16_lo(qraw[j]);
                qv[8 * c + 2 * j + 1] = (double)bf16_hi(qraw[j]);
            }
        }
        // the descriptor covers exactly this block's rows: loads past them
        // return zeros without memory traffic, so every load is unconditional
        // and the compiler's wait counts stay exact across the loop
        const int nrows = r_end - r_begin;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(
            k_index + ((size_t)b * S_max + r_begin) * kDidx, (uint32_t)nrows * kDidx * 2u);
        const __amdgpu_buffer_rsrc_t sr =
            make_rsrc(scores + (size_t)b * S_stride + r_begin, (uint32_t)nrows * 4u);
        constexpr int RA = 2;   // 16-row groups per wave step: 32 rows, 8 KB per register set
        // two register sets: the next step's rows are requested before this
        // step's rows are reduced
        auto load = [&](u32x4 (&raw)[RA][4], int r) {
#pragma unroll
            for (int a = 0; a < RA; ++a)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    raw[a][c] = buf_load16_nt(kr, (uint32_t)(((r + 16 * a + lr) * kDidx + 32 * c + 8 * qq) * 2));
        };
        auto reduce = [&](const u32x4 (&raw)[RA][4], int r) {
#pragma unroll
            for (int a = 0; a < RA; ++a) {
                double acc = 0.0;
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc = fma(qv[8 * c + 2 * j], (double)bf16_lo(raw[a][c][j]), acc);
                        acc = fma(qv[8 * c + 2 * j + 1], (double)bf16_hi(raw[a][c][j]), acc);
                    }
                acc = quad_sum(acc);
                const int row = r + 16 * a + lr;   // local to the block
                const float sc = acc > 0.0 ? (float)acc : 0.0f;   // ReLU, +0 for ties
                // every lane stores (lanes of a row's other quarters and rows
                // past the block fall outside the descriptor and are dropped),
                // so no branch around a memory access blurs the wait counts
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), sr,
                                                      qq == 0 ? (uint32_t)row * 4u : 0x80000000u, 0, 0);
                const uint32_t bin = __float_as_uint(sc) >> 20;
                if (qq == 0 && row < nrows && bin) atomicAdd(&lh[bin], 1u);
            }
        };
        constexpr int kWaveRows = 16 * RA;
        constexpr int kStep = kWaveRows * 4;   // rows per workgroup step (4 waves)
        u32x4 ra[RA][4], rb[RA][4];
        const int n_steps = (nrows + kStep - 1) / kStep;   // uniform over the workgroup
        int r = kWaveRows * wave;
        load(ra, r);
        for (int st = 0; st + 1 < n_steps; st += 2) {   // no early exit: one loop state
            load(rb, r + kStep);
            reduce(ra, r);
            load(ra, r + 2 * kStep);
            reduce(rb, r + kStep);
            r += 2 * kStep;
        }
        if (n_steps & 1) reduce(ra, r);
    }
    __syncthreads();
    for (int i = tid; i < kHistBins; i += 256)
        if (lh[i]) atomicAdd(&hist[(size_t)b * kHistBins + i], lh[i]);
}

// ---------------------------------------------------------------------------
// 1b. multi-head weighted indexer ([稀疏注意力] DSA ①):
//     I_s = sum_j w_j ReLU(q_j . k_s) over H_I = 16 NHB heads.
// S^T = K . Q^T on MFMA (16 keys x 16 heads per product, four 32-dim
// k-steps), so the key rows stream from HBM once for all heads.  ReLU and
// the weights are applied in fp32 per (key, head); the heads are summed in
// the lane (over the NHB head blocks) and across the 16 lanes of the head
// index (DPP).  The sums are fp32 (MFMA accumulation), not the exact dots of
// the single-head indexer.  Scores are stored as order-preserving keys (sign
// bit flipped for non-negative values, all bits for negative ones) because
// the weights may be negative; the radix select below works on those keys
// unchanged, and zero is always +0 so that equal scores stay equal keys.
__device__ __forceinline__ float dpp_fadd(float v, int ctrl_id) {
    int x;
    switch (ctrl_id) {   // (a switch keeps the DPP control a constant)
        case 0: x = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false); break;   // lane ^ 1
        case 1: x = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false); break;   // lane ^ 2
        case 2: x = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false); break;  // 7 - lane in 8
        default: x = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false); break; // 15 - lane in 16
    }
    return v + __int_as_float(x);
}
// Sum over the 16 lanes of a row; every lane receives the same value.
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_fadd(v, 0);
    v = dpp_fadd(v, 1);
    v = dpp_fadd(v, 2);
    return dpp_fadd(v, 3);
}
__device__ __forceinline__ uint32_t order_key(float v) {
    v = (v == 0.0f) ? 0.0f : v;   // -0 -> +0
    const uint32_t u = __float_as_uint(v);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}

template <int NHB>
__global__ __launch_bounds__(256) void indexer_weighted_kernel(
    const uint16_t* __restrict__ q_index, const float* __restrict__ w_index,
    const uint16_t* __restrict__ k_index, const int32_t* __restrict__ seq_lens, int S_max,
    int S_stride, int rows_per_block, uint32_t* __restrict__ keys, uint32_t* __restrict__ hist) {
    constexpr int HI = 16 * NHB;
    __shared__ uint32_t lh[kHistBins];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4, n = lane & 15;
    const int b = blockIdx.y;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int r_begin = blockIdx.x * rows_per_block;
    const int r_end = min(r_begin + rows_per_block, L);
    for (int i = tid; i < kHistBins; i += 256) lh[i] = 0u;
    __syncthreads();
    if (r_begin < r_end) {
        // B operand: lane (G, n) holds head 16 hb + n, dims 32 u + 8 G .. +7
        u32x4 qf[NHB][4];
        float w[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const uint16_t* qrow = q_index + ((size_t)b * HI + 16 * hb + n) * kDidx + 8 * G;
#pragma unroll
            for (int u = 0; u < 4; ++u) qf[hb][u] = *reinterpret_cast<const u32x4*>(qrow + 32 * u);
            w[hb] = w_index[(size_t)b * HI + 16 * hb + n];
        }
        // descriptors cover exactly this block's rows: loads past them read
        // zeros and stores past them are dropped, so the loop has no branch
        // around a memory access
        const int nrows = r_end - r_begin;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(
            k_index + ((size_t)b * S_max + r_begin) * kDidx, (uint32_t)nrows * kDidx * 2u);
        const __amdgpu_buffer_rsrc_t sr =
            make_rsrc(keys + (size_t)b * S_stride + r_begin, (uint32_t)nrows * 4u);
        // the largest squared key norm seen (rows past the block read as zero)
        float kmax = 0.f;
        // A operand of 16-key group g: lane (G, n) holds key 16 g + n, dims
        // 32 u + 8 G .. +7 (each load covers 64 contiguous bytes of 16 rows)
        auto load = [&](u32x4 (&kk)[4], int g) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kk[u] = buf_load16_nt(kr, (uint32_t)(((16 * g + n) * kDidx + 32 * u + 8 * G) * 2));
        };
        auto score = [&](const u32x4 (&kk)[4], int g) {
            // |k|^2 of key 16 g + n: this lane's 32 dims, then its four lane groups
            float n2 = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = bf16_lo(kk[u][j]), c = bf16_hi(kk[u][j]);
                    n2 = fmaf(a, a, fmaf(c, c, n2));
                }
            kmax = fmaxf(kmax, rows4_sum(n2));
            float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = mfma16(kk[u], qf[hb][u], acc);
                // lane (G, n): keys 16 g + 4 G + i of head 16 hb + n
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = fmaf(w[hb], fmaxf(acc[i], 0.0f), t[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = row16_sum(t[i]);
            // lane n < 4 of each row stores key 16 g + 4 G + n
            const float v = n == 0 ? t[0] : n == 1 ? t[1] : n == 2 ? t[2] : t[3];
            const uint32_t key = order_key(v);
            const int row = 16 * g + 4 * G + n;
            __builtin_amdgcn_raw_buffer_store_b32(key, sr, n < 4 ? (uint32_t)row * 4u : 0x80000000u, 0, 0);
            const uint32_t bin = key >> 20;
            if (n < 4 && row < nrows && bin) atomicAdd(&lh[bin], 1u);
        };
        // groups g = wave, wave + 4, ...: the four waves read adjacent 4 KB
        // blocks; two register sets, the next group requested first
        const int n_groups = (nrows + 15) / 16;
        const int n_steps = (n_groups + 3) / 4;   // uniform over the workgroup
        u32x4 ka[4], kb[4];
        int g = wave;
        load(ka, g);
        for (int st = 0; st + 1 < n_steps; st += 2) {   // no early exit: one loop state
            load(kb, g + 4);
            score(ka, g);
            load(ka, g + 8);
            score(kb, g + 4);
            g += 8;
        }
        if (n_steps & 1) score(ka, g);
        // bin 0 of the first-digit histogram is implied by the row length, so
        // its slot carries the row's largest squared key norm (fp32 bits of a
        // non-negative value order like the value) for the exact re-scoring
        kmax = wave_max(kmax);
        if (lane == 0) atomicMax(&hist[(size_t)b * kHistBins], __float_as_uint(kmax));
    }
    __syncthreads();
    for (int i = tid; i < kHistBins; i += 256)
        if (i && lh[i]) atomicAdd(&hist[(size_t)b * kHistBins + i], lh[i]);
}

// ---------------------------------------------------------------------------
// 2. top-k selection (an exact radix select on 12 + 12 + 8 key bits):
//    topk_compact_kernel  per (2048-key chunk, batch row): first digit B1
//                         from the histogram; the keys in bins >= B1 as
//                         ordered (key, index) entries to the chunk's slice
//    topk_finish_kernel   per batch row: exact k-th key T from the entries
//                         (two more digits), ties to take, and the selected
//                         indices in ascending order
// Keys are order-preserving bit patterns of the fp32 scores, so unsigned
// order is score order.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
// threads per chunk workgroup: its first-digit scan over the 4096 bins is
// the latency the chunk kernel waits on; 512 threads (8 bins, 4 keys each)
// gave the top-k call 66.3 us against 70.3 with 256 and 75.1 with 128, 66.5
// with 1024
constexpr int kChunkThreads = 512;
// keys per chunk workgroup: 2048 gave the top-k call 69.8 us against 70.7
// with 4096 and 72.4 with 8192 (more chunk workgroups fill more CUs); the
// finish kernel gives each chunk a thread, so a row may span at most
// kSelThreads chunks (2^21 keys), which the entry points' limits keep
constexpr int kChunkKeys = 2048;

struct SelInfo {
    uint32_t B1;       // first-digit bin of the k-th largest key
    uint32_t above;    // keys in first-digit bins above B1
};

// Inclusive prefix sum of one value per thread across a block of NT threads.
template <int NT>
__device__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    if (wave == 0) {
        uint32_t w = lane < NT / 64 ? wsum[lane] : 0u;
#pragma unroll
        for (int o = 1; o < NT / 64; o <<= 1) {
            const uint32_t t = __shfl_up(w, o, 64);
            if (lane >= o) w += t;
        }
        if (lane < NT / 64) wsum[lane] = w;   // inclusive wave totals
    }
    __syncthreads();
    const uint32_t add = wave ? wsum[wave - 1] : 0u;
    __syncthreads();
    return v + add;
}

// Over a histogram h[0..nbins) in LDS, find the largest bin B with
// (count in bins >= B) >= need.  Writes B and the count in bins > B to
// out[0], out[1].  Every thread of the NT-thread block must call it.
template <int NT>
__device__ void find_crossing(const uint32_t* h, int nbins, uint32_t need, uint32_t* wsum,
                              uint32_t* out) {
    const int per = (nbins + NT - 1) / NT;
    const int t = threadIdx.x;             // thread t owns bins [hi - per, hi), from the top
    const int hi = nbins - t * per;
    const int lo = max(hi - per, 0);
    uint32_t c = 0;
    for (int i = lo; i < hi; ++i) c += h[i];
    const uint32_t incl = block_inclusive_scan<NT>(c, wsum);   // count in bins >= lo
    const uint32_t excl = incl - c;                             // count in bins >= hi
    if (excl < need && incl >= need) {
        uint32_t acc = excl;
        for (int i = hi - 1; i >= lo; --i) {
            if (acc + h[i] >= need) {
                out[0] = (uint32_t)i;
                out[1] = acc;
                break;
            }
            acc += h[i];
        }
    }
    __syncthreads();
}

// Loads the first-digit histogram of batch b (bin 0 implied by L) and finds
// the bin holding the k-th largest key: out = {B1, count above B1}.
template <int NT>
__device__ void first_digit(const uint32_t* hist_g, int b, int L, int k, uint32_t* h,
                            uint32_t* wsum, uint32_t* out) {
    uint32_t nz = 0;
    for (int i = threadIdx.x; i < kHistBins; i += NT) {
        const uint32_t v = i ? hist_g[(size_t)b * kHistBins + i] : 0u;
        h[i] = v;
        nz += v;
    }
    const uint32_t tot = block_inclusive_scan<NT>(nz, wsum);
    if (threadIdx.x == NT - 1) h[0] = (uint32_t)L - tot;
    __syncthreads();
    find_crossing<NT>(h, kHistBins, (uint32_t)k, wsum, out);
}

// Per 2048-key chunk: the keys of the threshold bin and of the bins above it
// (every selected key is one of them), and with lower_bins = 1 those of the
// bin below as well (where the re-scored band of the multi-head indexers can
// reach), as (key, index) entries in index order, to the chunk's own slice (its index range of the entry arrays);
// their number to ent_cnt[b][c]: no cross-workgroup atomics.  Wave w owns a
// contiguous quarter of the chunk, its keys requested before the histogram
// work so both latencies overlap; the order within a wave comes from
// ballot/mbcnt.  With k = L every index is selected: the chunk writes its
// indices straight to the output, and chunk 0 writes the -1 padding.
constexpr int kKeysPerLane = kChunkKeys / kChunkThreads;     // 4

__global__ __launch_bounds__(kChunkThreads) void topk_compact_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ hist_g,
    const int32_t* __restrict__ seq_lens, int S_max, int S_stride, int top_k,
    uint32_t* __restrict__ ent_key, uint32_t* __restrict__ ent_idx, uint32_t* __restrict__ ent_cnt,
    int n_chunks, SelInfo* __restrict__ info, int32_t* __restrict__ topk_idx, int lower_bins) {
    constexpr int NW = kChunkThreads / 64;
    constexpr int span = kChunkKeys / NW;
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t wsum[NW];
    __shared__ uint32_t res[2];
    __shared__ uint32_t wcnt[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y, c = blockIdx.x;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int k = min(top_k, L);
    int32_t* outp = topk_idx + (size_t)b * top_k;
    if (c == 0)
        for (int i = k + tid; i < top_k; i += kChunkThreads) outp[i] = -1;
    const int c0 = c * kChunkKeys;
    if (c0 >= L) return;
    const int c1 = min(c0 + kChunkKeys, L);
    if (k == L) {   // everything is selected
        for (int j = c0 + tid; j < c1; j += kChunkThreads) outp[j] = j;
        return;
    }
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(scores + (size_t)b * S_stride);
    const int j0 = min(c0 + wave * span, c1), j1 = min(j0 + span, c1);
    uint32_t kv[kKeysPerLane];
#pragma unroll
    for (int it = 0; it < kKeysPerLane; ++it) {
        const int j = j0 + 64 * it + lane;
        kv[it] = j < j1 ? keys[j] : 0u;
    }
    first_digit<kChunkThreads>(hist_g, b, L, k, h, wsum, res);
    const uint32_t B1 = res[0];
    if (c == 0 && tid == 0) info[b] = SelInfo{B1, res[1]};
    const uint32_t B0 = B1 > (uint32_t)lower_bins ? B1 - (uint32_t)lower_bins : 0u;   // lowest bin kept
    uint32_t n_w = 0;
#pragma unroll
    for (int it = 0; it < kKeysPerLane; ++it)
        n_w += (uint32_t)__popcll(__ballot(j0 + 64 * it + lane < j1 && (kv[it] >> 20) >= B0));
    if (lane == 0) wcnt[wave] = n_w;
    __syncthreads();
    uint32_t pos = 0;
    for (int w2 = 0; w2 < wave; ++w2) pos += wcnt[w2];
    const size_t slice = ((size_t)b * n_chunks + c) * kChunkKeys;
#pragma unroll
    for (int it = 0; it < kKeysPerLane; ++it) {
        const int j = j0 + 64 * it + lane;
        const bool keep = j < j1 && (kv[it] >> 20) >= B0;
        const uint64_t mask = __ballot(keep);
        const uint32_t p = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (keep) {
            ent_key[slice + p] = kv[it];
            ent_idx[slice + p] = (uint32_t)j;
        }
        pos += (uint32_t)__popcll(mask);
    }
    if (tid == 0) {
        uint32_t n = 0;
        for (int w2 = 0; w2 < NW; ++w2) n += wcnt[w2];
        ent_cnt[(size_t)b * n_chunks + c] = n;
    }
}

// Radix passes 2 and 3 (12 and 8 bits) over the keys of the threshold bin B1
// that `next(i)` yields for i in [0, n): the k-th largest key T and the
// number of keys equal to T to take (need on entry: what is still to be
// taken at bin B1).  Every thread of the block calls it.
template <typename KeyAt>
__device__ void lower_digits(uint32_t B1, uint32_t need, uint32_t n, KeyAt key_at, uint32_t* h,
                             uint32_t* wsum, uint32_t* res, uint32_t& T, uint32_t& ties) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kHistBins; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += kSelThreads) {
        const uint32_t key = key_at(i);
        if ((key >> 20) == B1) atomicAdd(&h[(key >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    find_crossing<kSelThreads>(h, kHistBins, need, wsum, res);
    const uint32_t pre = (B1 << 12) | res[0];
    need -= res[1];
    __syncthreads();
    for (int i = tid; i < 256; i += kSelThreads) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += kSelThreads) {
        const uint32_t key = key_at(i);
        if ((key >> 8) == pre) atomicAdd(&h[key & 0xFFu], 1u);
    }
    __syncthreads();
    find_crossing<kSelThreads>(h, 256, need, wsum, res);
    T = (pre << 8) | res[0];
    ties = need - res[1];
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Exact selection for the multi-head indexers.  Their scores are fp32 sums
// from the matrix cores, within eps of the exact value.  Let T be the k-th
// largest fp32 score: a key whose fp32 score exceeds T + 2 eps is in the
// exact top k (every key whose exact score is at least its exact score has
// an fp32 score above T, and fewer than k do), and a key below T - 2 eps is
// out.  So only the band [T - 2 eps, T + 2 eps] is re-scored, in fp64
// (products of bf16 values are exact; the sums of 128 of them are exact in
// fp64 for any realistic spread of exponents), and the band's places go to
// its best keys by exact score, ties to the lower index.
//   weighted (DSA ①):  e_s = sum_h w_h ReLU(q_h . k_s).  An fp32 sum of n
//     terms errs by at most gamma_n = n 2^-24 (to first order) times the sum
//     of their magnitudes: 130 for each head's dot (bounded by |q_h| |k_s|,
//     Cauchy-Schwarz) and about 72 for the weighted sum over the heads
//     (whose terms are again at most |w_h| |q_h| |k_s|), so
//     |e - E| <= 202 2^-24 W |k_s| < 2^-16.3 W |k_s|, W = sum_h |w_h| |q_h|;
//     eps = 2^-15 W max_s |k_s| (twice that), the row's largest key norm
//     coming from the indexer pass;
//   QSA blocks (①-②):  e_j = sum_h ReLU(q_h . bk_j), |bk_j| = 1: the dots err
//     by gamma_130 |q_h| plus the fp32 block key's own error (a few units of
//     2^-22 relative) and the hi + lo split's 2^-17, the head sum by
//     gamma_72; eps = 2^-14 sum_h |q_h| + 2^-20 |T| (about twice that); the
//     block key is recomputed in fp64 (mean of the four keys, L2 norm, RoPE
//     at 4 j) for the exact score.
// Three steps: the finish kernel finds T and the band and writes the band
// and the keys certainly in (sorted by index) to the workspace; the band
// kernel scores the band on up to 16 CUs per row (an fp64 contraction on the
// matrix cores); the merge kernel ranks the band by exact score and merges.
// For the weighted indexer (whose band is the wider) the entries include the
// bin below the threshold bin as well, so the band is found among them
// unless it reaches two bins down; otherwise the band's keys below the
// threshold bin come from a scan of the row.  A band of more
// than kBandCap keys (long runs of near-equal scores), or one from a row whose
// entries overflowed LDS, keeps the fp32 selection, which is then exact up
// to those near-ties only.
constexpr int kBandCap = 256;
constexpr int kSureCap = 4096;   // keys certainly in: fewer than k <= 4096

struct RefineArgs {
    int mode;                  // 0: none (exact one-head scores), 1: weighted, 2: QSA blocks
    int H_I;                   // indexer heads (<= 64)
    const uint16_t* q_index;   // [B][H_I][128] bf16
    const float* w_index;      // [B][H_I] (weighted)
    const uint16_t* k_index;   // [B][S_tok][128] bf16 indexer keys
    int S_tok;                 // rows of k_index per batch row
    const uint32_t* knorm;     // weighted: fp32 bits of the row's largest |k_s|^2, row stride kHistBins
    RopeDev rope;              // QSA block-key RoPE (half 0: none)
    int lower_bins;            // the entries hold bins >= B1 - lower_bins (0 or 1)
    // per-row band state in the workspace
    uint32_t* state;           // [B][8]: active, band size nb, keys certainly in c_in, need
    uint32_t* band_idx;        // [B][kBandCap]
    double* band_score;        // [B][kBandCap]
    uint32_t* sure_in;         // [B][kSureCap] ascending
};

// fp32 score of an order-preserving key
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key >> 31) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// The band for one batch row, after the fp32 radix select found the k-th
// key T (lk/li: the E entries of keys in bins >= B1 in index order;
// keys_row: the row's n_keys fp32 keys).  Writes the band, the keys
// certainly in (ascending) and the row's state (active = 1) to the
// workspace and returns true, or returns false when the band does not
// qualify (nothing written; the caller finishes the row in fp32).  Every
// thread of the block calls it.
__device__ bool band_setup(const RefineArgs& ra, int b, int n_keys, int k, uint32_t T, uint32_t B1,
                           const uint32_t* lk, const uint32_t* li, uint32_t E,
                           const uint32_t* keys_row, uint32_t* wsum, uint32_t* res, double* qn_h,
                           float* fshared) {
    static_assert(kSelThreads == 16 * 64, "16 threads per indexer head");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t* qrow0 = ra.q_index + (size_t)b * ra.H_I * kDidx;
    // ---- eps: |q_h| (times |w_h|) by 16 threads per head, 8 dims each
    {
        const int hh = tid >> 4, part = tid & 15;
        double sq = 0.0;
        if (hh < ra.H_I) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow0 + (size_t)hh * kDidx + 8 * part);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double a = bf16_lo(v[i]), c = bf16_hi(v[i]);
                sq = fma(a, a, fma(c, c, sq));
            }
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
        if (part == 0) {
            double qn = sqrt(sq);
            if (hh < ra.H_I && ra.mode == 1) qn *= fabs((double)ra.w_index[(size_t)b * ra.H_I + hh]);
            qn_h[hh] = hh < ra.H_I ? qn : 0.0;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const double qn = wave_sum_f64(qn_h[lane]);
        if (lane == 0) {
            const double fT = key_value(T);
            double eps;
            if (ra.mode == 1)
                eps = 0x1p-15 * qn * sqrt((double)__uint_as_float(ra.knorm[(size_t)b * kHistBins]));
            else
                eps = 0x1p-14 * qn + 0x1p-20 * fabs(fT);
            eps = 2.0 * eps + 0x1p-20 * fabs(fT) + 1e-30;   // the band's half width, rounding slack
            fshared[0] = (float)(fT - eps);
            fshared[1] = (float)(fT + eps);
            res[0] = 0u;                                    // band members found
        }
    }
    __syncthreads();
    const float lo_v = fshared[0], hi_v = fshared[1];
    // keys of lo_v (rounded down) and hi_v (rounded up) in key order
    auto okey = [](float v) {
        v = (v == 0.0f) ? 0.0f : v;
        const uint32_t u = __float_as_uint(v);
        return (u >> 31) ? ~u : (u | 0x80000000u);
    };
    const uint32_t K_lo = okey(lo_v) - 1u, K_hi = okey(hi_v) + 1u;
    uint32_t* band = ra.band_idx + (size_t)b * kBandCap;
    uint32_t* sure = ra.sure_in + (size_t)b * kSureCap;
    // ---- sure-in entries (key > K_hi) in index order, band entries appended
    const uint32_t per = (E + kSelThreads - 1) / kSelThreads;
    const uint32_t e0 = min((uint32_t)tid * per, E), e1 = min(e0 + per, E);
    uint32_t nin = 0;
    for (uint32_t e = e0; e < e1; ++e) {
        const uint32_t key = lk[e];
        nin += key > K_hi;
        if (key >= K_lo && key <= K_hi) {
            const uint32_t at = atomicAdd(&res[0], 1u);
            if (at < (uint32_t)kBandCap) band[at] = li[e];
        }
    }
    uint32_t pos = block_inclusive_scan<kSelThreads>(nin, wsum) - nin;
    for (uint32_t e = e0; e < e1; ++e)
        if (lk[e] > K_hi && pos < (uint32_t)kSureCap) sure[pos++] = li[e];
    if (tid == kSelThreads - 1) res[1] = pos;      // keys certainly selected
    // the band may reach below the lowest first-digit bin of the entries
    // (the threshold bin, or the one below it): those keys are found in the
    // row itself (four keys per request, several in flight)
    const uint32_t B0 = B1 > (uint32_t)ra.lower_bins ? B1 - (uint32_t)ra.lower_bins : 0u;   // entries: bins >= B0
    if (K_lo < (B0 << 20)) {
        const int n4 = n_keys >> 2;
        const u32x4* k4 = reinterpret_cast<const u32x4*>(keys_row);
        auto test = [&](uint32_t key, int i) {
            if (key >= K_lo && key < (B0 << 20)) {
                const uint32_t at = atomicAdd(&res[0], 1u);
                if (at < (uint32_t)kBandCap) band[at] = (uint32_t)i;
            }
        };
        constexpr int kU = 4;
        for (int i0 = tid; i0 < n4; i0 += kU * kSelThreads) {
            u32x4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int i = i0 + u * kSelThreads;
                v[u] = i < n4 ? k4[i] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int i = i0 + u * kSelThreads;
                if (i < n4)
#pragma unroll
                    for (int c = 0; c < 4; ++c) test(v[u][c], 4 * i + c);
            }
        }
        for (int i = 4 * n4 + tid; i < n_keys; i += kSelThreads) test(keys_row[i], i);
    }
    __syncthreads();
    const uint32_t nb = res[0], c_in = res[1];
    const int need = k - (int)c_in;
    if (nb > (uint32_t)kBandCap || need < 0 || need > (int)nb) return false;   // uniform
    if (tid == 0) {
        uint32_t* st = ra.state + (size_t)b * 8;
        st[1] = nb;
        st[2] = c_in;
        st[3] = (uint32_t)need;
        st[0] = 1u;
    }
    return true;
}

// One workgroup per batch row does the whole selection.  The first digit
// (the bin B1 holding the k-th largest key, and the count above it) comes
// from the indexer's histogram; the entries (keys in bins >= B1, and for the
// weighted indexer the bin below too: every selected key and every band
// member is one of them) are gathered from the row into LDS in index order:
// each thread takes 16 consecutive keys per pass (one pass is 16384 keys,
// the next pass's keys requested before this pass's are sorted out),
// counts its entries, one block scan places them.  Their number is known
// from the histogram before the row is read; when it exceeds the LDS
// capacity the digit passes and the ordered pass run over the row's keys in
// global memory instead (slow, and only for rows with huge runs of
// near-equal scores).  Then the two lower digit passes give the exact k-th
// key T, and the selected indices (keys > T, and the first `ties` keys == T
// by index) are written in ascending order from two block scans.
constexpr int kSelKeysPerThread = 16;
constexpr int kSelPass = kSelThreads * kSelKeysPerThread;   // keys per pass
// Rows of at most this many keys take the one-kernel select; longer rows
// the two-kernel one (the chunk workgroups read a row in parallel, where one
// workgroup's reads of it run at ~20 GB/s: 32 us for 131072 keys against
// 18 us for the two kernels; at 32768 keys the one kernel was faster, 16
// against 18.7 us, until the chunk kernel's 512 threads: since then the QSA
// call over 32768-block rows takes 74.1-74.3 us with the two kernels against
// 76.0-76.4 with one).
constexpr int kSelOneKernelMax = 16384;

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ hist_g,
    const int32_t* __restrict__ seq_lens, int S_max, int S_stride, int top_k,
    int32_t* __restrict__ topk_idx, RefineArgs ra) {
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t lk[kEntCap], li[kEntCap];
    __shared__ uint32_t wsum[kSelThreads / 64];
    __shared__ uint32_t res[2];
    __shared__ double qn_h[64];
    __shared__ float fshared[2];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    if (ra.mode != 0 && tid == 0) ra.state[(size_t)b * 8] = 0u;   // band kernels: nothing to do
    const int L = min(max(seq_lens[b], 1), S_max);
    const int k = min(top_k, L);
    int32_t* outp = topk_idx + (size_t)b * top_k;
    for (int i = k + tid; i < top_k; i += kSelThreads) outp[i] = -1;
    if (k == L) {                                  // everything is selected
        for (int j = tid; j < L; j += kSelThreads) outp[j] = j;
        return;
    }
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(scores + (size_t)b * S_stride);
    // the first pass's keys are requested before the histogram work
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    u32x4v kv[kSelKeysPerThread / 4], kn[kSelKeysPerThread / 4];
    auto load_pass = [&](int r0, u32x4v (&v)[kSelKeysPerThread / 4]) {
        const int j0 = r0 + tid * kSelKeysPerThread;
#pragma unroll
        for (int u = 0; u < kSelKeysPerThread / 4; ++u) {
            const int j = j0 + 4 * u;   // a multiple of 4; the row is padded to 4 keys
            v[u] = j < L ? *reinterpret_cast<const u32x4v*>(keys + j) : u32x4v{0u, 0u, 0u, 0u};
        }
    };
    load_pass(0, kv);
    first_digit<kSelThreads>(hist_g, b, L, k, h, wsum, res);
    const uint32_t B1 = res[0], above = res[1];
    const uint32_t need = (uint32_t)k - above;
    const uint32_t B0 = B1 > (uint32_t)ra.lower_bins ? B1 - (uint32_t)ra.lower_bins : 0u;
    uint32_t E = above + h[B1] + (B0 < B1 ? h[B0] : 0u);   // entries: keys in bins >= B0
    uint32_t T, ties;
    if (E <= (uint32_t)kEntCap) {                  // uniform
        uint32_t base = 0;
        for (int r0 = 0; r0 < L; r0 += kSelPass) {   // uniform trip count
            const bool more = r0 + kSelPass < L;
            if (more) load_pass(r0 + kSelPass, kn);
            const int j0 = r0 + tid * kSelKeysPerThread;
            uint32_t c = 0;
#pragma unroll
            for (int u = 0; u < kSelKeysPerThread / 4; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) c += j0 + 4 * u + q < L && (kv[u][q] >> 20) >= B0;
            uint32_t p = base + block_inclusive_scan<kSelThreads>(c, wsum) - c;
            if (c)
#pragma unroll
                for (int u = 0; u < kSelKeysPerThread / 4; ++u)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int j = j0 + 4 * u + q;
                        if (j < L && (kv[u][q] >> 20) >= B0 && p < (uint32_t)kEntCap) {
                            lk[p] = kv[u][q];
                            li[p] = (uint32_t)j;
                            ++p;
                        }
                    }
            if (tid == kSelThreads - 1) res[0] = p;
            __syncthreads();
            base = res[0];
            __syncthreads();
            if (more)
#pragma unroll
                for (int u = 0; u < kSelKeysPerThread / 4; ++u) kv[u] = kn[u];
        }
        E = base;                                  // equal to the histogram's count
        lower_digits(B1, need, E, [&](uint32_t i) { return lk[i]; }, h, wsum, res, T, ties);
        if (ra.mode != 0 &&
            band_setup(ra, b, L, k, T, B1, lk, li, E, keys, wsum, res, qn_h, fshared))
            return;                                // the band kernels finish the row
        // thread t takes entries [t per, (t + 1) per): ranks of ties and
        // output slots from two block scans
        const uint32_t per = (E + kSelThreads - 1) / kSelThreads;
        const uint32_t e0 = min((uint32_t)tid * per, E), e1 = min(e0 + per, E);
        uint32_t eq = 0;
        for (uint32_t e = e0; e < e1; ++e) eq += lk[e] == T;
        uint32_t eq_seen = block_inclusive_scan<kSelThreads>(eq, wsum) - eq;
        uint32_t take = 0;
        for (uint32_t e = e0, r = eq_seen; e < e1; ++e) {
            const uint32_t key = lk[e];
            take += key > T || (key == T && r++ < ties);
        }
        uint32_t p = block_inclusive_scan<kSelThreads>(take, wsum) - take;
        for (uint32_t e = e0; e < e1; ++e) {
            const uint32_t key = lk[e];
            bool tk = key > T;
            if (key == T) tk = eq_seen++ < ties;
            if (tk && p < (uint32_t)k) outp[p++] = (int32_t)li[e];   // p < k always holds
        }
        return;
    }
    // too many entries for LDS: digit passes over the row's keys, then the
    // ordered pass in 1024-key tiles of the row
    lower_digits(B1, need, (uint32_t)L, [&](uint32_t i) { return keys[i]; }, h, wsum, res, T, ties);
    uint32_t eq_base = 0, sel_base = 0;
    for (uint32_t t0 = 0; t0 < (uint32_t)L; t0 += kSelThreads) {
        const uint32_t e = t0 + tid;
        const uint32_t key = e < (uint32_t)L ? keys[e] : 0u;
        const uint32_t eqf = e < (uint32_t)L && key == T;
        const uint32_t eq_incl = block_inclusive_scan<kSelThreads>(eqf, wsum);
        const uint32_t tk = e < (uint32_t)L && (key > T || (eqf && eq_base + eq_incl - eqf < ties));
        const uint32_t t_incl = block_inclusive_scan<kSelThreads>(tk, wsum);
        if (tk && sel_base + t_incl - tk < (uint32_t)k) outp[sel_base + t_incl - tk] = (int32_t)e;
        if (tid == kSelThreads - 1) {
            res[0] = eq_incl;
            res[1] = t_incl;
        }
        __syncthreads();
        eq_base += res[0];
        sel_base += res[1];
        __syncthreads();
    }
}

// One workgroup per batch row: the exact k-th key T from the entries, then
// the selected indices in ascending order (keys > T, and the first `ties`
// keys == T by index).  The entries (at most k - 1 above the threshold bin
// plus the bin itself) normally fit in LDS: there the two digit passes and
// an ordered pass with two block scans finish the row.  A threshold bin too
// large for LDS takes the digit passes over the row's keys and the ordered
// pass in 1024-entry tiles over the entries in global memory (slow, and only
// for rows with huge runs of near-equal scores).
__global__ __launch_bounds__(kSelThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int S_max, int S_stride,
    int top_k, const uint32_t* __restrict__ ent_key, const uint32_t* __restrict__ ent_idx,
    const uint32_t* __restrict__ ent_cnt, int n_chunks, const SelInfo* __restrict__ info,
    int32_t* __restrict__ topk_idx, RefineArgs ra) {
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t lk[kEntCap], li[kEntCap];
    __shared__ uint16_t emap[kEntCap];
    __shared__ uint32_t wsum[kSelThreads / 64];
    __shared__ uint32_t res[2];
    __shared__ double qn_h[64];
    __shared__ float fshared[2];
    __shared__ uint32_t cstart[kSelThreads];   // entry offset of each chunk
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    if (ra.mode != 0 && tid == 0) ra.state[(size_t)b * 8] = 0u;   // band kernels: nothing to do
    const int L = min(max(seq_lens[b], 1), S_max);
    const int k = min(top_k, L);
    if (k == L) return;                        // written by the compact kernel
    const SelInfo fd = info[b];
    const uint32_t B1 = fd.B1;
    const uint32_t need = (uint32_t)k - fd.above;
    const int nkc = min(n_chunks, (L + kChunkKeys - 1) / kChunkKeys);
    const uint32_t cnt = tid < nkc ? ent_cnt[(size_t)b * n_chunks + tid] : 0u;
    const uint32_t incl = block_inclusive_scan<kSelThreads>(cnt, wsum);
    if (tid < nkc) cstart[tid] = incl - cnt;
    if (tid == kSelThreads - 1) res[0] = incl;
    __syncthreads();
    const uint32_t E = res[0];
    __syncthreads();
    const size_t row = (size_t)b * n_chunks * kChunkKeys;
    int32_t* outp = topk_idx + (size_t)b * top_k;
    uint32_t T, ties;
    if (E <= (uint32_t)kEntCap) {
        // the chunk of every entry (an LDS map: wave w fills chunks w, w + 16,
        // ...), then every thread requests all its entries at once
        for (int c = wave; c < nkc; c += kSelThreads / 64) {
            const uint32_t n_c = (c + 1 < nkc ? cstart[c + 1] : E) - cstart[c];
            for (uint32_t i = lane; i < n_c; i += 64) emap[cstart[c] + i] = (uint16_t)c;
        }
        __syncthreads();
        static_assert(kEntCap % kSelThreads == 0, "whole entries per thread");
        constexpr int kPerThread = kEntCap / kSelThreads;   // 12
        uint32_t ek[kPerThread], ei[kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const uint32_t e = u * kSelThreads + tid;
            ek[u] = ei[u] = 0u;
            if (e < E) {
                const int c = emap[e];
                const size_t at = row + (size_t)c * kChunkKeys + (e - cstart[c]);
                ek[u] = ent_key[at];
                ei[u] = ent_idx[at];
            }
        }
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const uint32_t e = u * kSelThreads + tid;
            if (e < E) {
                lk[e] = ek[u];
                li[e] = ei[u];
            }
        }
        __syncthreads();
        lower_digits(B1, need, E, [&](uint32_t i) { return lk[i]; }, h, wsum, res, T, ties);
        if (ra.mode != 0 &&
            band_setup(ra, b, L, k, T, B1, lk, li, E,
                       reinterpret_cast<const uint32_t*>(scores + (size_t)b * S_stride), wsum, res,
                       qn_h, fshared))
            return;                            // the band kernels finish the row
        // thread t takes entries [t per, (t + 1) per): ranks of ties and
        // output slots from two block scans
        const uint32_t per = (E + kSelThreads - 1) / kSelThreads;
        const uint32_t e0 = min((uint32_t)tid * per, E), e1 = min(e0 + per, E);
        uint32_t eq = 0;
        for (uint32_t e = e0; e < e1; ++e) eq += lk[e] == T;
        uint32_t eq_seen = block_inclusive_scan<kSelThreads>(eq, wsum) - eq;
        uint32_t take = 0;
        for (uint32_t e = e0, r = eq_seen; e < e1; ++e) {
            const uint32_t key = lk[e];
            take += key > T || (key == T && r++ < ties);
        }
        uint32_t p = block_inclusive_scan<kSelThreads>(take, wsum) - take;
        for (uint32_t e = e0; e < e1; ++e) {
            const uint32_t key = lk[e];
            bool tk = key > T;
            if (key == T) tk = eq_seen++ < ties;
            if (tk && p < (uint32_t)k) outp[p++] = (int32_t)li[e];   // p < k always holds
        }
        return;
    }
    // the threshold bin overflowed LDS: digit passes over the row's keys
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(scores + (size_t)b * S_stride);
    lower_digits(B1, need, (uint32_t)L, [&](uint32_t i) { return keys[i]; }, h, wsum, res, T, ties);
    uint32_t eq_base = 0, sel_base = 0;
    for (uint32_t t0 = 0; t0 < E; t0 += kSelThreads) {
        const uint32_t e = t0 + tid;
        uint32_t key = 0u, idx = 0u;
        if (e < E) {
            int lo = 0, hi = nkc;                // the chunk holding entry e
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (cstart[mid] <= e) lo = mid;
                else hi = mid;
            }
            const size_t at = row + (size_t)lo * kChunkKeys + (e - cstart[lo]);
            key = ent_key[at];
            idx = ent_idx[at];
        }
        const uint32_t eqf = e < E && key == T;
        const uint32_t eq_incl = block_inclusive_scan<kSelThreads>(eqf, wsum);
        const uint32_t tk = e < E && (key > T || (eqf && eq_base + eq_incl - eqf < ties));
        const uint32_t t_incl = block_inclusive_scan<kSelThreads>(tk, wsum);
        if (tk && sel_base + t_incl - tk < (uint32_t)k) outp[sel_base + t_incl - tk] = (int32_t)idx;
        if (tid == kSelThreads - 1) {
            res[0] = eq_incl;
            res[1] = t_incl;
        }
        __syncthreads();
        eq_base += res[0];
        sel_base += res[1];
        __syncthreads();
    }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Raw indexer-key words of band member m for lane `lane` (pair `lane` of
// its key row, or of the four rows of its block); zero past the band.
__device__ __forceinline__ void band_rows(const RefineArgs& ra, const uint32_t* krows, const uint32_t* band,
                                          uint32_t m, uint32_t nb, int lane, uint32_t (&r)[4]) {
    r[0] = r[1] = r[2] = r[3] = 0u;
    if (m >= nb) return;
    const size_t j = band[m];
    if (ra.mode == 1) {
        r[0] = krows[j * (kDidx / 2) + lane];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = krows[(4 * j + i) * (kDidx / 2) + lane];
    }
}

// Band member m's 128-dim vector x in fp64 from its raw key words (lane l:
// dims 2l, 2l+1): the key itself, or the block key (mean of the four keys,
// L2 norm, RoPE at position 4 j).  A member past the band gives zeros.
__device__ __forceinline__ void band_vector(const RefineArgs& ra, const uint32_t* band, uint32_t m,
                                            uint32_t nb, const uint32_t (&r)[4], int lane, double& x0,
                                            double& x1) {
    if (ra.mode == 1) {
        x0 = (double)bf16_lo(r[0]);
        x1 = (double)bf16_hi(r[0]);
        return;
    }
    x0 = x1 = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x0 += (double)bf16_lo(r[i]);
        x1 += (double)bf16_hi(r[i]);
    }
    x0 *= 0.25;
    x1 *= 0.25;
    const double nrm = sqrt(wave_sum_f64(x0 * x0 + x1 * x1));
    if (nrm > 0.0) {
        x0 /= nrm;
        x1 /= nrm;
    } else {
        x0 = x1 = 0.0;
    }
    if (m < nb && lane < ra.rope.half) {
        const double a = (double)(4 * (int)band[m]) * ra.rope.pos_scale * ra.rope.theta[lane];
        double sn, c;
        sincos(a, &sn, &c);
        c *= (double)ra.rope.amp;
        sn *= (double)ra.rope.amp;
        const double y0 = x0 * c - x1 * sn, y1 = x0 * sn + x1 * c;
        x0 = y0;
        x1 = y1;
    }
}

// The band's best `need` keys (exact score, then lower index) merged with
// the keys certainly in, ascending, into the row's output: one workgroup per
// batch row.  Each lane holds band entries lane + 64 i; a wave counts for
// one member at a time how many entries rank ahead of it (ballots), then how
// many chosen entries have a lower index: its place among the chosen.  The
// lists are requested whole, with the row's state, before it is known how
// much of them the row uses (the workspace slices are always in bounds).
__global__ __launch_bounds__(kSelThreads) void band_merge_kernel(RefineArgs ra, int top_k,
                                                                 int32_t* __restrict__ topk_idx) {
    static_assert(kBandCap == 4 * 64 && kSelThreads == 1024 && kSureCap == 4 * kSelThreads,
                  "four band entries per lane, four sure entries per thread");
    __shared__ uint32_t sure[kSureCap];
    __shared__ uint32_t bidx[kBandCap], bsorted[kBandCap], bflag[kBandCap];
    __shared__ double bscore[kBandCap];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const uint32_t* st = ra.state + (size_t)b * 8;
    const uint32_t active = st[0], nb = st[1], c_in = st[2], need = st[3];
    const u32x4 sv = reinterpret_cast<const u32x4*>(ra.sure_in + (size_t)b * kSureCap)[tid];
    uint32_t bi = 0u;
    double bs = 0.0;
    if (tid < kBandCap) {
        bi = ra.band_idx[(size_t)b * kBandCap + tid];
        bs = ra.band_score[(size_t)b * kBandCap + tid];
    }
    if (active == 0u) return;            // uniform
    reinterpret_cast<u32x4*>(sure)[tid] = sv;
    if (tid < kBandCap) {
        bidx[tid] = bi;
        bscore[tid] = bs;
    }
    __syncthreads();
    double su[4];
    uint32_t iu[4];
    bool vu[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = lane + 64 * i;
        vu[i] = u < nb;
        su[i] = vu[i] ? bscore[u] : 0.0;
        iu[i] = vu[i] ? bidx[u] : 0u;
    }
    for (uint32_t m = wave; m < nb; m += kSelThreads / 64) {
        const double sm = bscore[m];
        const uint32_t my = bidx[m];
        uint32_t ahead = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ahead += __popcll(__ballot(vu[i] && (su[i] > sm || (su[i] == sm && iu[i] < my))));
        if (lane == 0) bflag[m] = ahead < need;
    }
    __syncthreads();
    bool cu[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cu[i] = vu[i] && bflag[lane + 64 * i];
    for (uint32_t m = wave; m < nb; m += kSelThreads / 64) {
        if (!bflag[m]) continue;         // uniform over the wave
        const uint32_t my = bidx[m];
        uint32_t below = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) below += __popcll(__ballot(cu[i] && iu[i] < my));
        if (lane == 0) bsorted[below] = my;
    }
    __syncthreads();
    auto lower = [](const uint32_t* a, uint32_t n, uint32_t x) {   // # of a[0..n) below x
        uint32_t lo = 0, hi = n;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (a[mid] < x) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    int32_t* outp = topk_idx + (size_t)b * top_k;
    for (uint32_t i = tid; i < c_in; i += kSelThreads) {
        const uint32_t x = sure[i];
        outp[i + lower(bsorted, need, x)] = (int32_t)x;
    }
    for (uint32_t i = tid; i < need; i += kSelThreads) {
        const uint32_t x = bsorted[i];
        outp[i + lower(sure, c_in, x)] = (int32_t)x;
    }
}

// Exact fp64 scores of 16 band members (m0 = 16 blockIdx.x) of batch row
// blockIdx.y: the products of the H_I query heads with the members' vectors
// as an fp64 contraction on the matrix cores (16 x 16 x 4 tiles).  Wave w
// builds member m0 + w's vector into the B operand tile xb (column w), then
// multiplies head tile w % 4 with the tile over dim quarter w / 4 (8 steps
// of four dims); the quarters' partial dots are summed in order, then ReLU,
// weight, and the heads summed (four per wave, then the 16 waves in order).
// Operand layouts of the 16 x 16 x 4 fp64 instruction: lane l gives
// A[l % 16][l / 16] (head 16 ht + l % 16, dim 4 s + l / 16, from qs) and
// B[l / 16][l % 16] (dim 4 s + l / 16 of column l % 16), and holds
// D[l / 16 + 4 r][l % 16] in register r.  B element (s, l) sits at
// s * 64 + (l ^ (s & 31)) in xb, which spreads the builders' stores (two
// dims of one column per lane) over the banks.  The band entry and its key rows are requested before the row's state is
// known, with the row index clamped into the key array, so those loads stay
// in bounds whatever the workspace holds.
__global__ __launch_bounds__(kSelThreads) void band_score_kernel(RefineArgs ra) {
    __shared__ u32x4 qs[16 * 64];        // dims 8 p4 .. 8 p4 + 7 of head h at [p4][h]
    __shared__ double xb[32 * 64];
    __shared__ double pd[4][64][16];     // [dim quarter][head][member] partial dots
    __shared__ double ws[16][16];        // [wave][member] sums of four heads
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y;
    const uint32_t m0 = 16u * blockIdx.x;
    const uint32_t* st = ra.state + (size_t)b * 8;
    const uint32_t active = st[0], nb = st[1];
    const uint32_t* band = ra.band_idx + (size_t)b * kBandCap;
    const uint32_t* krows = reinterpret_cast<const uint32_t*>(ra.k_index + (size_t)b * ra.S_tok * kDidx);
    // requests first: this wave's member rows, the query slice, the weight
    const uint32_t n_rows = ra.mode == 1 ? (uint32_t)ra.S_tok : (uint32_t)ra.S_tok / 4;   // keys or blocks
    uint32_t r[4] = {0u, 0u, 0u, 0u};
    if (n_rows > 0) {
        const uint32_t j = min(band[m0 + wave], n_rows - 1);
        if (ra.mode == 1) {
            r[0] = krows[(size_t)j * (kDidx / 2) + lane];
            r[1] = r[2] = r[3] = 0u;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = krows[(4 * (size_t)j + i) * (kDidx / 2) + lane];
        }
    }
    const int hh = tid >> 4, p4 = tid & 15;
    const u32x4 qv = hh < ra.H_I
        ? *reinterpret_cast<const u32x4*>(ra.q_index + ((size_t)b * ra.H_I + hh) * kDidx + 8 * p4)
        : u32x4{0u, 0u, 0u, 0u};
    const double wh = hh >= ra.H_I ? 0.0 : ra.mode == 1 ? (double)ra.w_index[(size_t)b * ra.H_I + hh] : 1.0;
    if (active == 0u || m0 >= nb) return;   // the row was finished in fp32, or no members here (uniform)
    if (m0 + wave >= nb) r[0] = r[1] = r[2] = r[3] = 0u;
    qs[p4 * 64 + hh] = qv;
    {
        double x0, x1;
        band_vector(ra, band, m0 + wave, nb, r, lane, x0, x1);
        const int s0 = lane >> 1, l0 = wave + 32 * (lane & 1);   // B lanes c + 16 q, q = 2 (lane % 2), + 1
        xb[s0 * 64 + (l0 ^ (s0 & 31))] = x0;
        xb[s0 * 64 + ((l0 + 16) ^ (s0 & 31))] = x1;
    }
    __syncthreads();
    {
        const int ht = wave & 3, kq = wave >> 2, col = lane & 15, qd = lane >> 4;
        const uint16_t* qh = reinterpret_cast<const uint16_t*>(qs);
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s = 8 * kq; s < 8 * kq + 8; ++s) {
            const int d = 4 * s + qd;
            const uint32_t q16 = qh[((d >> 3) * 64 + 16 * ht + col) * 8 + (d & 7)];
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(q16 << 16),
                                                       xb[s * 64 + (lane ^ (s & 31))], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) pd[kq][16 * ht + qd + 4 * i][col] = acc[i];
    }
    __syncthreads();
    {
        // thread (head hh, member p4): the full dot, ReLU, weight; four heads
        // per wave summed across lanes (xor 16, 32), then the waves in order
        const double dot = ((pd[0][hh][p4] + pd[1][hh][p4]) + pd[2][hh][p4]) + pd[3][hh][p4];
        double v = wh * fmax(dot, 0.0);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (lane < 16) ws[wave][lane] = v;
    }
    __syncthreads();
    if (tid < 16 && m0 + tid < nb) {
        double sc = 0.0;
#pragma unroll
        for (int w = 0; w < 16; ++w) sc += ws[w][tid];
        ra.band_score[(size_t)b * kBandCap + m0 + tid] = sc;
    }
}


// ---------------------------------------------------------------------------
// 3. attention over the selected latent rows
// ---------------------------------------------------------------------------
// One workgroup per (128 selected rows, 32 heads, batch row), eight waves:
// two head groups of 16 heads times four 32-row sub-chunks.  The gathered
// latent rows are copied straight from global memory into LDS by buffer
// loads (all four sub-chunks requested at once, so the gather latency is
// paid once), each row fetched once per 32 heads.  Wave (group, sub-chunk)
// computes the scores of its sub-chunk,
//   S^T[32 rows][16 heads] = C . Q^T   (18 k-steps of 16x16x32 bf16 MFMA),
// the four waves of a head group exchange their row maxima through LDS, so
// each forms P = exp2(S - M) with the chunk's exact maximum M (no running
// rescale), and hand P (hi + lo bf16, in the layout of the PV operand) and
// its row sums to each other through LDS.  Then wave (group, sc) computes
// output dims 128 sc .. +127 over all 128 rows,
//   O^T[128 dims][16 heads] = C[:, dims]^T . P^T,
// and writes them: no softmax states are merged inside the workgroup, and
// the partial write is spread over all eight waves.  P is kept in the LDS
// bytes of latent dims 512..575 (the rope part, read only by the scores),
// which are free once every wave has its scores.  One partial per (chunk,
// head) goes to combine_partials_kernel.
// (Two waves walking the four sub-chunks one after the other: 1.5 us slower
// per call; 64 or 128 heads per workgroup, fewer re-reads of each row but
// fewer workgroups: 1.5 and 10 us slower.  Merging the four waves' softmax
// states through LDS instead of splitting the output dims took two more
// barrier rounds and left the partial write to two waves.)
constexpr int kSubRows = 32;                         // rows per LDS sub-chunk
constexpr int kRowBytes = kDqk * 2;                  // 1152
constexpr int kRowStride = kRowBytes + 32;           // padded to 296 dwords (8 mod 16): see below
constexpr int kSubCopies = (kSubRows * kRowStride + 1023) / 1024;   // 1 KB copies per sub-chunk
constexpr int kSubBytes = kSubCopies * 1024;         // the last copy spills into slack nothing reads
constexpr int kAttnWaves = 8;
constexpr int kAttnGroups = 2;                       // 16 heads each
constexpr int kPBytes = 2 * kDv;                     // byte offset of the P slot in a row (dim 512)
static_assert(kDqk - kDv == 64 && kSubRows == 2 * 16, "P of a wave: 16 rows x 128 B of rope dims");

__global__ __launch_bounds__(64 * kAttnWaves) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ seq_lens, int H, int S_max,
    int top_k, float qscale, float* __restrict__ part_o, float* __restrict__ part_ml,
    int n_chunks) {
    constexpr int KU = kDqk / 32;
    __shared__ __attribute__((aligned(16))) uint8_t rows0[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rows1[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rows2[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rows3[kSubBytes];
    __shared__ int32_t sel_s[kRowsPerChunk];
    __shared__ float mx_s[kAttnGroups][4][16];
    __shared__ float l_s[kAttnGroups][4][16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hgw = wave & 1, sc = wave >> 1;
    const int G = lane >> 4, n = lane & 15;
    const int chunk = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int k = min(top_k, L);
    const int c0 = chunk * kRowsPerChunk;
    if (c0 >= k) return;                        // whole workgroup
    const int c1 = min(c0 + kRowsPerChunk, k);
    const int h = hg * (16 * kAttnGroups) + 16 * hgw + n;
    const bool heads = hg * (16 * kAttnGroups) + 16 * hgw < H;   // wave-uniform (H % 16 == 0)

    // the selected indices, then q (its latency overlaps the copies)
    int32_t sel = -1;
    if (tid < kRowsPerChunk && c0 + tid < c1) sel = topk_idx[(size_t)b * top_k + c0 + tid];
    u32x4 qf[KU];
    const uint16_t* qrow = q + ((size_t)b * H + (heads ? h : 0)) * kDqk;
#pragma unroll
    for (int u = 0; u < KU; ++u) qf[u] = *reinterpret_cast<const u32x4*>(qrow + 32 * u + 8 * G);
    if (tid < kRowsPerChunk) sel_s[tid] = sel;
    __syncthreads();

    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(latent + (size_t)b * S_max * kDqk, (uint32_t)S_max * kDqk * 2u);
    // copy j of sub-chunk s fills LDS bytes [1024 j, +1024) of its buffer,
    // lane l the 16 bytes at 1024 j + 16 l (row x / kRowStride, column
    // x mod kRowStride); wave w takes copies j = 8 i + w of every sub-chunk.
    // Rows past the selection read zeros (no traffic), so P = 0 meets V = 0.
    constexpr int kCopiesPerWave = (kSubCopies + kAttnWaves - 1) / kAttnWaves;
    int rr[kCopiesPerWave], cc[kCopiesPerWave];
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) {
        const int x = 1024 * (kAttnWaves * i + wave) + 16 * lane;
        rr[i] = x / kRowStride;
        cc[i] = x - rr[i] * kRowStride;
    }
    auto copy_sub = [&](int s2, uint8_t* dst) {
        int idx[kCopiesPerWave];
#pragma unroll
        for (int i = 0; i < kCopiesPerWave; ++i) idx[i] = sel_s[kSubRows * s2 + min(rr[i], kSubRows - 1)];
        int wv = wave;
        asm volatile("" : "+s"(wv));
#pragma unroll
        for (int i = 0; i < kCopiesPerWave; ++i) {
            const int j = kAttnWaves * i + wv;
            if (j < kSubCopies) {
                const bool ok = rr[i] < kSubRows && cc[i] < kRowBytes && idx[i] >= 0;
                const uint32_t voff = ok ? (uint32_t)idx[i] * kRowBytes + (uint32_t)cc[i] : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, dst + 1024 * j, 16, voff, 0, 0, 0);
            }
        }
    };
    copy_sub(0, rows0);
    copy_sub(1, rows1);
    copy_sub(2, rows2);
    copy_sub(3, rows3);
    // every wave's copies and q are complete, then the barrier makes all
    // copies visible (the asm memory clobber keeps the LDS reads below it)
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");

    uint8_t* const mine = sc == 0 ? rows0 : sc == 1 ? rows1 : sc == 2 ? rows2 : rows3;
    const int p0 = c0 + kSubRows * sc;
    // scores of the sub-chunk: sc2[th][i] is row 16 th + 4G + i, head n
    f32x4 sc2[2];
    float mx = -INFINITY;
    if (heads && p0 < c1) {
        const uint8_t* kb = mine + n * kRowStride + 16 * G;
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            sc2[th] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < KU; ++u)
                sc2[th] = mfma16(*reinterpret_cast<const u32x4*>(kb + 16 * th * kRowStride + 64 * u), qf[u], sc2[th]);
        }
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc2[th][i] *= qscale;
                if (p0 + 16 * th + 4 * G + i >= c1) sc2[th][i] = -INFINITY;
            }
        mx = fmaxf(fmaxf(fmaxf(sc2[0][0], sc2[0][1]), fmaxf(sc2[0][2], sc2[0][3])),
                   fmaxf(fmaxf(sc2[1][0], sc2[1][1]), fmaxf(sc2[1][2], sc2[1][3])));
        mx = rows4_max(mx);
    } else {
        sc2[0] = sc2[1] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    if (G == 0) mx_s[hgw][sc][n] = mx;
    // maxima visible; every wave is past its score reads, so the rope dims
    // of the row buffers are free for P
    __syncthreads();

    // the chunk's maximum (finite for a head wave: row c0 < c1 is in
    // sub-chunk 0), P and its row sums
    const float M = fmaxf(fmaxf(mx_s[hgw][0][n], mx_s[hgw][1][n]), fmaxf(mx_s[hgw][2][n], mx_s[hgw][3][n]));
    float pr[2][4];
    float ls = 0.f;
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[th][i] = heads ? fast_exp2(sc2[th][i] - M) : 0.f;
            ls += pr[th][i];
        }
    ls = rows4_sum(ls);
    u32x4 ph, pl;
    pack_p_hilo(pr, ph, pl);
    // the wave's P: rows 16 hgw + lane / 4 of its buffer, bytes
    // kPBytes + 32 (lane % 4) (hi) and + 16 (lo)
    auto pslot = [&](uint8_t* buf) { return buf + (16 * hgw + (lane >> 2)) * kRowStride + kPBytes + 32 * (lane & 3); };
    *reinterpret_cast<u32x4*>(pslot(mine)) = ph;
    *reinterpret_cast<u32x4*>(pslot(mine) + 16) = pl;
    if (G == 0) l_s[hgw][sc][n] = ls;
    __syncthreads();                            // P and the row sums visible
    if (!heads) return;

    // O^T for dims 128 sc .. +127 over the chunk's sub-chunks:
    // o[t][i] is dim 128 sc + 8 (4G + i) + t of head n
    f32x4 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        if (c0 + kSubRows * s2 >= c1) break;    // wave-uniform: the rest has P = 0
        uint8_t* const buf = s2 == 0 ? rows0 : s2 == 1 ? rows1 : s2 == 2 ? rows2 : rows3;
        const u32x4 qh = *reinterpret_cast<const u32x4*>(pslot(buf));
        const u32x4 ql = *reinterpret_cast<const u32x4*>(pslot(buf) + 16);
        u32x4 vr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            vr[r] = *reinterpret_cast<const u32x4*>(buf + slot_row(G, r) * kRowStride + (128 * sc + 8 * n) * 2);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const u32x4 vc = column_of(vr, t);
            o[t] = mfma16(vc, qh, o[t]);
            o[t] = mfma16(vc, ql, o[t]);
        }
    }

    const size_t idx = ((size_t)b * H + h) * n_chunks + chunk;
    float* po = part_o + idx * kDv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d0 = 128 * sc + 8 * (4 * G + i);
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]};
        *reinterpret_cast<f32x4*>(po + d0 + 4) = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]};
    }
    if (sc == 0 && G == 0) {
        part_ml[idx * 2] = M;
        part_ml[idx * 2 + 1] = l_s[hgw][0][n] + l_s[hgw][1][n] + l_s[hgw][2][n] + l_s[hgw][3][n];
    }
}

// ---------------------------------------------------------------------------
// 4. dense absorbed-MLA decode (no selection: every row of the context).
// The same MQA attention as sparse_attn_kernel over contiguous rows.  One
// workgroup per (row range, 16*NW heads, batch row), one wave per SIMD (the
// 16-head output tile and the 576-dim query need more than half the register
// file).  The head groups of one row range are consecutive on one XCD, so the
// second group reads the range from that XCD's L2.  The range is streamed
// through a ring of four LDS sub-chunk buffers: once every wave is past
// sub-chunk s-1, sub-chunk s+3 is requested into its buffer, so three
// sub-chunks are always in flight.  Requests past the range read zeros
// without traffic, so every step issues the same copies and the explicit
// wait counts hold to the end.
//
// Softmax reference.  The running maximum of the online softmax is fixed at
// the first sub-chunk's maximum m0 (per head); later rows take
// p = 2^(s - m0) directly: floating point keeps its relative precision at
// any scale, and s - m0 below kMlaHeadroom keeps p <= 2^32 (sums far inside
// fp32 range for any latent value below 2^70 in magnitude).  The main loop then has no
// branch, which keeps the 128-register output tile in place in the
// accumulation registers (a rescale branch makes the compiler copy the tile
// through ordinary registers every step and starves the score product of
// registers for its LDS reads).  A workgroup in which some score rises
// further above m0 recomputes its range with the rescaling online softmax.
constexpr float kMlaHeadroom = 32.f;

// QK^T of one 32-row sub-chunk for the wave's 16 heads: sc[th][i] is the
// scaled base-2 score of row p0 + 16 th + 4 G + i (-inf past c1).  Key
// reads are issued in batches of six per row half ahead of their MFMAs.
__device__ __forceinline__ void dense_scores(const uint8_t* rows, const u32x4 (&qf)[kDqk / 32],
                                             f32x4 (&sc)[2], int p0, int c1, float qscale, int G,
                                             int n) {
    constexpr int KU = kDqk / 32;
    // batches of two k-slices for both row halves (four reads, four MFMAs),
    // two batches in flight ahead of the MFMAs that use them
    constexpr int NBT = KU / 2;
    const uint8_t* kb = rows + n * kRowStride + 16 * G;
    u32x4 kr[NBT][4];
    auto load = [&](int g) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            kr[g][2 * j] = *reinterpret_cast<const u32x4*>(kb + 64 * (2 * g + j));
            kr[g][2 * j + 1] = *reinterpret_cast<const u32x4*>(kb + 16 * kRowStride + 64 * (2 * g + j));
        }
    };
    sc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    sc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);
    load(0);
    load(1);
#pragma unroll
    for (int g = 0; g < NBT; ++g) {
        if (g + 2 < NBT) load(g + 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            sc[0] = mfma16(kr[g][2 * j], qf[2 * g + j], sc[0]);
            sc[1] = mfma16(kr[g][2 * j + 1], qf[2 * g + j], sc[1]);
        }
    }
    // the order above, held against the scheduler's short LDS latency model
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int g = 0; g < NBT; ++g) {
        if (g + 2 < NBT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[th][i] *= qscale;
            if (p0 + 16 * th + 4 * G + i >= c1) sc[th][i] = -INFINITY;
        }
}

__device__ __forceinline__ float dense_rowmax(const f32x4 (&sc)[2]) {
    const float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                           fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    return rows4_max(mx);   // the head's max over the 32 rows
}

// p = 2^(s - m), l += sum p, o += V^T p for the sub-chunk.  p enters the
// MFMA as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi), sharing each V
// operand: p is then carried to 2^-17 relative instead of bf16's 2^-9, so no
// row's weight, the largest included, is rounded to bf16 precision.
//
// V^T operands come from gfx950's transposing LDS read: within each 16-lane
// group, lane 4a + c of a ds_read_b64_tr_b16 receives element c of the
// 8-byte chunks addressed by lanes a, a+4, a+8 and a+12.  Lane r of group G
// addresses row (4G + r/4) [second read: 16 + 4G + r/4] at dims
// tb + 4 (r mod 4)..+3, so lane n receives dim tb + n of the four rows: the
// tile's A operand, with k = the rows slot_row(G, 0..7) that the P operand
// uses, and the output tile o[dq][t] (tb = 128 dq + 16 t) holds dims
// tb + 4G + i.
// Banks (measured with the LDS bank-conflict counter on gfx950): a
// transposing 8-byte read serves 32 lanes at a time from 64 banks, a 16-byte
// read 16 lanes (lanes 0-7 with 16-23, and so on).  With the row stride at
// 8 mod 16 dwords, the eight rows of a transposing read start 8 dwords apart
// mod 64 and each reads 8 consecutive dwords: all 64 banks once; the score
// reads (row n, 16-byte column G) and the top-k path's row reads also cover
// the banks once.
__device__ __forceinline__ void dense_pv(const uint8_t* rows, const f32x4 (&sc)[2], float m,
                                         f32x4 (&o)[4][8], float& l_run, int G, int n) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    float pr[2][4];
    float ls = 0.f;
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[th][i] = fast_exp2(sc[th][i] - m);
            ls += pr[th][i];
        }
    l_run += rows4_sum(ls);
    u32x4 ph, pl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = pr[k >> 1][2 * (k & 1)], c = pr[k >> 1][2 * (k & 1) + 1];
        const u32x2 hl = split_bf16x2(a, c);
        ph[k] = hl[0];
        pl[k] = hl[1];
    }
    const uint8_t* v0 = rows + (4 * G + (n >> 2)) * kRowStride + 8 * (n & 3);
    const uint8_t* v1 = v0 + 16 * kRowStride;
    // per 128-dim quarter: 16 reads, then the hi products of its eight tiles,
    // then the lo products (no MFMA waits on the one just before it)
#pragma unroll
    for (int dq = 0; dq < 4; ++dq) {
        u32x4 col[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int off = (128 * dq + 16 * t) * 2;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + off));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v1 + off));
            col[t] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) o[dq][t] = mfma16(col[t], ph, o[dq][t]);
#pragma unroll
        for (int t = 0; t < 8; ++t) o[dq][t] = mfma16(col[t], pl, o[dq][t]);
    }
}

// The rescaling online softmax for one sub-chunk (the recompute path): the
// running max follows the scores, o and l are rescaled when it moves.
__device__ __forceinline__ void dense_pv_rescale(const uint8_t* rows, const f32x4 (&sc)[2],
                                                 float& m_run, f32x4 (&o)[4][8], float& l_run,
                                                 int G, int n) {
    const float m_new = fmaxf(m_run, dense_rowmax(sc));
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
        const float alpha = fast_exp2(m_run - m_new);   // 0 on the first sub-chunk
        l_run *= alpha;
#pragma unroll
        for (int dq = 0; dq < 4; ++dq)
#pragma unroll
            for (int t = 0; t < 8; ++t) o[dq][t] *= alpha;
        m_run = m_new;
    }
    dense_pv(rows, sc, m_run, o, l_run, G, n);
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void mla_dense_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
    const int32_t* __restrict__ seq_lens, int H, int S_max, int rows_per_split, float qscale,
    float* __restrict__ part_o, float* __restrict__ part_ml, int n_split, int n_hg, int n_units) {
    constexpr int KU = kDqk / 32;
    __shared__ __attribute__((aligned(16))) uint8_t rows0[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rows1[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rows2[kSubBytes];
    __shared__ __attribute__((aligned(16))) uint8_t rows3[kSubBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4, n = lane & 15;
    // workgroups go round-robin over the 8 XCDs: id and id + 8 share an XCD,
    // so the n_hg head groups of a unit (batch row, row range) are 8 apart
    const int id = blockIdx.x;
    const int hg = (id >> 3) % n_hg;
    const int unit = (id & 7) + 8 * ((id >> 3) / n_hg);
    if (unit >= n_units) return;                // whole workgroup
    const int b = unit / n_split, split = unit - b * n_split;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int c0 = split * rows_per_split;
    if (c0 >= L) return;                        // whole workgroup
    const int c1 = min(c0 + rows_per_split, L);
    const int nsub = (c1 - c0 + kSubRows - 1) / kSubRows;
    const int h = hg * (16 * NW) + 16 * wave + n;
    const bool heads = hg * (16 * NW) + 16 * wave < H;   // wave-uniform (H % 16 == 0)

    u32x4 qf[KU];
    const uint16_t* qrow = q + ((size_t)b * H + (heads ? h : 0)) * kDqk;
#pragma unroll
    for (int u = 0; u < KU; ++u) qf[u] = *reinterpret_cast<const u32x4*>(qrow + 32 * u + 8 * G);

    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(latent + (size_t)b * S_max * kDqk, (uint32_t)S_max * kDqk * 2u);
    // copy j = NW * i + wave of a sub-chunk fills LDS bytes [1024 j, +1024),
    // lane l the 16 bytes at x = 1024 j + 16 l: row x / kRowStride, column
    // x mod kRowStride (the padding after a row's kRowBytes is not read)
    // rel: the copy's byte offset within the sub-chunk's rows, or ~0u for the
    // padding bytes; it lies in the sub-chunk's first lim rows exactly when
    // rel < lim * kRowBytes
    constexpr int kCopiesPerWave = (kSubCopies + NW - 1) / NW;
    uint32_t rel[kCopiesPerWave];
#pragma unroll
    for (int i = 0; i < kCopiesPerWave; ++i) {
        const int x = 1024 * (NW * i + wave) + 16 * lane;
        const int rr = x / kRowStride, cc = x - rr * kRowStride;
        rel[i] = rr < kSubRows && cc < kRowBytes ? (uint32_t)(rr * kRowBytes + cc) : ~0u;
    }
    auto copy_sub = [&](int sub, uint8_t* dst) {
        const int r0 = c0 + kSubRows * sub;
        const int lim = max(min(c1 - r0, kSubRows), 0);   // rows of this sub-chunk
        const uint32_t lim_bytes = (uint32_t)lim * kRowBytes;
        const uint32_t base = (uint32_t)r0 * kRowBytes;
        int wv = wave;
        asm volatile("" : "+s"(wv));
#pragma unroll
        for (int i = 0; i < kCopiesPerWave; ++i) {
            // only the last copy index can pass kSubCopies for some waves
            if (i + 1 < kCopiesPerWave || NW * i + wv < kSubCopies) {
                const uint32_t voff = rel[i] < lim_bytes ? base + rel[i] : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, dst + 1024 * (NW * i + wv), 16, voff, 0, 0, 0);
            }
        }
    };
    // q is complete before the copies are issued (the compiler's wait counts
    // do not include loads into LDS)
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
    copy_sub(0, rows0);
    copy_sub(1, rows1);
    copy_sub(2, rows2);

    f32x4 o[4][8];
#pragma unroll
    for (int dq = 0; dq < 4; ++dq)
#pragma unroll
        for (int t = 0; t < 8; ++t) o[dq][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float l_run = 0.f;

    // step s: this wave's copies of s are done once at most those of s+1 and
    // s+2 are outstanding (every wave issues at least kCopiesMin per
    // sub-chunk); after the barrier every wave is past s-1, whose buffer
    // takes s+3.  (lgkmcnt(0) too: this wave's LDS reads of s-1 are complete
    // before the barrier that lets the copy of s+3 overwrite them.)
    constexpr int kCopiesMin = kSubCopies / NW;
    constexpr int kAhead = 2 * kCopiesMin;
    static_assert(kAhead < 64, "vmcnt range");
    auto enter = [&](int sub, uint8_t* next3) {
        __builtin_amdgcn_s_waitcnt(0x0070 | (kAhead & 15) | ((kAhead >> 4) << 14));
        asm volatile("s_barrier" ::: "memory");
        copy_sub(sub + 3, next3);
    };
    f32x4 sc[2];
    enter(0, rows3);
    dense_scores(rows0, qf, sc, c0, c1, qscale, G, n);
    const float m0 = dense_rowmax(sc);          // finite: row c0 < c1 is visible
    if (heads) dense_pv(rows0, sc, m0, o, l_run, G, n);
    bool high = false;                          // a score above m0 + kMlaHeadroom
    auto step = [&](int sub, const uint8_t* cur, uint8_t* next3) {
        enter(sub, next3);
        if (heads) {
            dense_scores(cur, qf, sc, c0 + kSubRows * sub, c1, qscale, G, n);
            high |= dense_rowmax(sc) > m0 + kMlaHeadroom;
            dense_pv(cur, sc, m0, o, l_run, G, n);
        }
    };
    // unrolled by eight: the compiler's own wait for copies into LDS cannot
    // tell the ring's buffers apart across the loop's back edge and waits for
    // every earlier copy in the first two steps after it
    for (int sub = 1; sub < nsub; sub += 8) {
        step(sub, rows1, rows0);
        if (sub + 1 >= nsub) break;
        step(sub + 1, rows2, rows1);
        if (sub + 2 >= nsub) break;
        step(sub + 2, rows3, rows2);
        if (sub + 3 >= nsub) break;
        step(sub + 3, rows0, rows3);
        if (sub + 4 >= nsub) break;
        step(sub + 4, rows1, rows0);
        if (sub + 5 >= nsub) break;
        step(sub + 5, rows2, rows1);
        if (sub + 6 >= nsub) break;
        step(sub + 6, rows3, rows2);
        if (sub + 7 >= nsub) break;
        step(sub + 7, rows0, rows3);
    }
    __builtin_amdgcn_s_waitcnt(0);              // the copies past the range
    float m_run = m0;
    if (__syncthreads_or(high)) {
        // recompute the range with the rescaling online softmax, one
        // sub-chunk at a time through rows0
#pragma unroll
        for (int dq = 0; dq < 4; ++dq)
#pragma unroll
            for (int t = 0; t < 8; ++t) o[dq][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        for (int sub = 0; sub < nsub; ++sub) {
            copy_sub(sub, rows0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (heads) {
                dense_scores(rows0, qf, sc, c0 + kSubRows * sub, c1, qscale, G, n);
                dense_pv_rescale(rows0, sc, m_run, o, l_run, G, n);
            }
            __syncthreads();
        }
    }
    if (!heads) return;

    const size_t idx = ((size_t)b * H + h) * n_split + split;
    float* po = part_o + idx * kDv + 4 * G;
#pragma unroll
    for (int dq = 0; dq < 4; ++dq)
#pragma unroll
        for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(po + 128 * dq + 16 * t) = o[dq][t];
    if (G == 0) {
        part_ml[idx * 2] = m_run;
        part_ml[idx * 2 + 1] = l_run;
    }
}

constexpr int kMlaWaves = 4;   // 64 heads per workgroup, one wave per SIMD
constexpr int kMlaTargetWgs = 256;
constexpr int kMlaMinRows = 256;

// ---------------------------------------------------------------------------
// 5. QSA ([attention] Qwen Sparse Attention ①-④): micro-block selection, then
//    standard sparse GQA over the selected tokens.
//    qsa_block_kernel   one HBM pass over the indexer keys: per complete
//                       4-token block the mean key, L2-normalised, rotated at
//                       the block's first position (fp32, fp64 angles), fed
//                       to the MFMA as hi + lo bf16 terms against the H_I
//                       query heads; ReLU per head, summed; order keys and
//                       the first-digit histogram as for the token indexer
//    (the radix select of section 2 then takes the top 512 blocks)
//    gqa_gather_attn_kernel  per (128 selected tokens, kv head, batch row):
//                       the tokens expanded from the selected blocks (their
//                       4 tokens each, then the 0-3 tail tokens; the kv head
//                       0 workgroups write the list out), the tokens' K and
//                       V rows gathered into LDS, the
//                       decode MFMA scheme over D = 128 for the group's
//                       g <= 16 query heads, a partial (m, l, o) per head
//    qsa_combine_kernel the partials merged per (batch, head)
// ---------------------------------------------------------------------------
constexpr int kQsaBlock = 4;
constexpr int kQsaTopBlocks = 512;
constexpr int kQsaTokens = kQsaBlock * kQsaTopBlocks + kQsaBlock - 1;   // 2051
constexpr int kGD = 128;                      // head dim of the GQA attention
constexpr int kGRowStride = kGD * 2 + 16;     // 272 B: 8 consecutive rows on distinct banks
constexpr int kGChunk = 128;                  // selected tokens per attention workgroup
constexpr int kGSub = 32;                     // rows per sub-chunk
constexpr int kGSubBytes = kGSub * kGRowStride;                  // 8704
constexpr int kGSubCopies = (kGSubBytes + 1023) / 1024;          // 9 copies of 1 KB
constexpr int kGBufBytes = kGSubCopies * 1024;

constexpr int kQsaBlocksPerWg = 256;          // 16 groups of 16 blocks (1024 keys)

template <int NHB>
__global__ __launch_bounds__(256) void qsa_block_kernel(
    const uint16_t* __restrict__ q_index, const uint16_t* __restrict__ k_index,
    const int32_t* __restrict__ seq_lens, int S_max, int KS, RopeDev rope,
    uint32_t* __restrict__ keys, uint32_t* __restrict__ hist) {
    constexpr int HI = 16 * NHB;
    __shared__ uint32_t lh[kHistBins];
    // The rotation of block 16 g + n of the workgroup (position
    // 4 k_begin + 64 g + 4 n) is the product of two table entries:
    // ta[g][i] at 4 k_begin + 64 g (amplitude included) and tb[n][i] at 4 n,
    // each from an fp64-reduced angle (the product adds ~2 fp32 roundings).
    __shared__ f32x2 ta[16][kDidx / 2], tb[16][kDidx / 2];
    __shared__ u32x4 qs[4 * NHB][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4, n = lane & 15;
    const int b = blockIdx.y;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int nb = L / kQsaBlock;                            // complete blocks
    const int k_begin = blockIdx.x * kQsaBlocksPerWg;
    const int k_end = min(k_begin + kQsaBlocksPerWg, nb);
    if (k_begin >= k_end) return;                            // whole workgroup
    // requests first (theta, the query heads, this wave's first group of
    // keys), then the tables while they are in flight
    static_assert(kDidx / 2 == 64, "one rotary pair per lane");
    const double th_lane = rope.theta[lane];                 // rope.half <= kDidx / 2
    // the query heads' B-operand fragments, shared by the four waves through
    // LDS: qs[4 hb + u][lane (G, n)] = head 16 hb + n, dims 32 u + 8 G .. +7
    u32x4 qv[NHB];
#pragma unroll
    for (int i = 0; i < NHB; ++i) {
        const int e = tid + 256 * i, f = e >> 6, l = e & 63;
        qv[i] = *reinterpret_cast<const u32x4*>(
            q_index + ((size_t)b * HI + 16 * (f >> 2) + (l & 15)) * kDidx + 32 * (f & 3) + 8 * (l >> 4));
    }
    const int nbl = k_end - k_begin;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(
        k_index + ((size_t)b * S_max + (size_t)kQsaBlock * k_begin) * kDidx,
        (uint32_t)nbl * kQsaBlock * kDidx * 2u);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(keys + (size_t)b * KS + k_begin, (uint32_t)nbl * 4u);
    // lane (G, n): block 16 g + n, dims 32 u + 8 G .. +7 of its 4 keys.
    // Wave w takes groups w, w + 4, w + 8, w + 12 (all 16 of the workgroup),
    // keys requested two groups ahead in three register sets; groups past
    // the range read zeros through the resource bound, and their stores fall
    // outside the score descriptor (their histogram updates are skipped).
    u32x4 b0[kQsaBlock][4], b1[kQsaBlock][4], b2[kQsaBlock][4];
    auto load_group = [&](int g, u32x4 (&dst)[kQsaBlock][4]) {
#pragma unroll
        for (int r = 0; r < kQsaBlock; ++r)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                dst[r][u] = buf_load16_nt(
                    kr, (uint32_t)((((16 * g + n) * kQsaBlock + r) * kDidx + 32 * u + 8 * G) * 2));
    };
    load_group(wave, b0);
    load_group(wave + 4, b1);
#pragma unroll
    for (int i = 0; i < NHB; ++i) qs[(tid + 256 * i) >> 6][(tid + 256 * i) & 63] = qv[i];
    for (int i = tid; i < kHistBins; i += 256) lh[i] = 0u;
    if (lane < rope.half) {
        // thread (wave, lane): pair i = lane, table rows wave + 4 t
        const double th = th_lane * rope.pos_scale;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int r = wave + 4 * t;
            float c, sn;
            if (r < 16) {
                cos_sin_fp64_angle(th * (4.0 * k_begin + 64.0 * r), c, sn);
                ta[r][lane] = f32x2{c * rope.amp, sn * rope.amp};
            } else {
                cos_sin_fp64_angle(th * (4.0 * (r - 16)), c, sn);
                tb[r - 16][lane] = f32x2{c, sn};
            }
        }
    }
    __syncthreads();
    auto step = [&](int st, const u32x4 (&raw)[kQsaBlock][4]) {
        const int g = 4 * st + wave;                     // 16-block group of this wave
        float mk[4][8];
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float e0 = 0.f, e1 = 0.f;
#pragma unroll
                for (int r = 0; r < kQsaBlock; ++r) {
                    e0 += bf16_lo(raw[r][u][j]);
                    e1 += bf16_hi(raw[r][u][j]);
                }
                mk[u][2 * j] = 0.25f * e0;
                mk[u][2 * j + 1] = 0.25f * e1;
                ss = fmaf(mk[u][2 * j], mk[u][2 * j], ss);
                ss = fmaf(mk[u][2 * j + 1], mk[u][2 * j + 1], ss);
            }
        ss = rows4_sum(ss);                              // the block's 128 dims
        const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
        u32x4 ahi[4], alo[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float xe = mk[u][2 * p] * inv, xo = mk[u][2 * p + 1] * inv;
                const int i = 16 * u + 4 * G + p;        // pair (2i, 2i+1)
                if (i < rope.half) {
                    const f32x2 a = ta[g][i], bt = tb[n][i];
                    const float c = a.x * bt.x - a.y * bt.y, sn = a.x * bt.y + a.y * bt.x;
                    const float ye = xe * c - xo * sn, yo = xe * sn + xo * c;
                    xe = ye;
                    xo = yo;
                }
                const u32x2 hl = split_bf16x2(xe, xo);
                ahi[u][p] = hl[0];
                alo[u][p] = hl[1];
            }
        float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 qb = qs[4 * hb + u][lane];
                acc = mfma16(ahi[u], qb, acc);
                acc = mfma16(alo[u], qb, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] += fmaxf(acc[i], 0.0f);   // blocks 4 G + i, head 16 hb + n
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = row16_sum(t[i]);
        const float v = n == 0 ? t[0] : n == 1 ? t[1] : n == 2 ? t[2] : t[3];
        const uint32_t key = order_key(v);
        const int row = 16 * g + 4 * G + n;
        __builtin_amdgcn_raw_buffer_store_b32(key, sr, n < 4 ? (uint32_t)row * 4u : 0x80000000u, 0, 0);
        const uint32_t bin = key >> 20;
        if (n < 4 && row < nbl && bin) atomicAdd(&lh[bin], 1u);
    };
    static_assert(kQsaBlocksPerWg == 4 * 4 * 16, "four steps of four waves of 16 blocks");
    load_group(wave + 8, b2);
    step(0, b0);
    load_group(wave + 12, b0);
    step(1, b1);
    step(2, b2);
    step(3, b0);
    __syncthreads();
    for (int i = tid; i < kHistBins; i += 256)
        if (lh[i]) atomicAdd(&hist[(size_t)b * kHistBins + i], lh[i]);
}

// the block histogram cleared (nz words) and the complete blocks per batch
// row written (the radix select's "lengths"), in one launch
__global__ void qsa_prep_kernel(uint32_t* __restrict__ hist, int nz, const int32_t* __restrict__ seq_lens,
                                int S_max, int B, int32_t* __restrict__ cnt) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < nz) hist[i] = 0u;
    if (i < B) cnt[i] = min(max(seq_lens[i], 1), S_max) / kQsaBlock;
}

// Token i of a batch row's list: the tokens of the selected blocks
// (ascending, as the blocks are), then the tail; -1 after.  With no complete
// block only the tail is taken.
__device__ __forceinline__ int32_t qsa_token(const int32_t* __restrict__ blk_row, int L, int i) {
    const int nb = L / kQsaBlock;
    const int c = min(kQsaTopBlocks, nb);
    if (i < kQsaBlock * c) return kQsaBlock * blk_row[i / kQsaBlock] + (i & 3);
    if (i < L - kQsaBlock * nb + kQsaBlock * c) return kQsaBlock * nb + (i - kQsaBlock * c);
    return -1;
}

__device__ __forceinline__ int qsa_n_tokens(int L) {
    const int nb = L / kQsaBlock;
    return kQsaBlock * min(kQsaTopBlocks, nb) + (L - kQsaBlock * nb);
}

// One sub-chunk of 32 gathered rows (K in kb, V in vb, rows at kGRowStride):
// S^T = K.Q^T over 128 dims, lazy online softmax (probabilities < 2^8),
// O^T += V^T.P^T.  Rows p0 + 16 th + 4 G + i >= c1 are masked.
__device__ __forceinline__ void gqa_gather_step(const uint8_t* kb, const uint8_t* vb,
                                                const u32x4 (&qf)[4], f32x4 (&o)[8], float& m_run,
                                                float& l_run, int p0, int c1, float qscale, int G,
                                                int n) {
    f32x4 sc[2];
#pragma unroll
    for (int th = 0; th < 2; ++th) {
        sc[th] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint8_t* kr = kb + (16 * th + n) * kGRowStride + 16 * G;
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[th] = mfma16(*reinterpret_cast<const u32x4*>(kr + 64 * u), qf[u], sc[th]);
    }
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[th][i] *= qscale;
            if (p0 + 16 * th + 4 * G + i >= c1) sc[th][i] = -INFINITY;
        }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = rows4_max(mx);                    // finite: row p0 < c1 is visible
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] *= alpha;
        m_run = m_new;
    }
    float pr[2][4];
    float ls = 0.f;
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[th][i] = fast_exp2(sc[th][i] - m_run);
            ls += pr[th][i];
        }
    l_run += rows4_sum(ls);
    u32x4 ph, pl;
    pack_p_hilo(pr, ph, pl);
    u32x4 vr[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        vr[r] = *reinterpret_cast<const u32x4*>(vb + slot_row(G, r) * kGRowStride + 16 * n);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const u32x4 vc = column_of(vr, t);
        o[t] = mfma16(vc, ph, o[t]);
        o[t] = mfma16(vc, pl, o[t]);
    }
}

// grid (chunks of 128 selected tokens, Hkv, B), one wave: the kv head's g
// query heads (g <= 16).  The chunk's tokens are expanded from the selected
// blocks (and written to tok by the kv head 0 workgroups, -1 padding
// included); all four sub-chunks' K and V rows are requested at once (one
// gather latency per workgroup).
__global__ __launch_bounds__(64) void gqa_gather_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ seq_lens, int Hq, int Hkv, int S_max, float qscale,
    int32_t* __restrict__ tok, float* __restrict__ part_o, float* __restrict__ part_ml, int n_chunks) {
    __shared__ __attribute__((aligned(16))) uint8_t k0[kGBufBytes], k1[kGBufBytes], k2[kGBufBytes], k3[kGBufBytes];
    __shared__ __attribute__((aligned(16))) uint8_t v0[kGBufBytes], v1[kGBufBytes], v2[kGBufBytes], v3[kGBufBytes];
    __shared__ int32_t sel_s[kGChunk];
    const int lane = threadIdx.x;
    const int G = lane >> 4, n = lane & 15;
    const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
    const int g = Hq / Hkv;
    const int L = min(max(seq_lens[b], 1), S_max);
    const int n_tok = qsa_n_tokens(L);
    const int c0 = chunk * kGChunk;
    const int32_t* blk_row = blk + (size_t)b * kQsaTopBlocks;
    if (kv == 0)
        for (int i = c0 + lane; i < min(c0 + kGChunk, kQsaTokens); i += 64)
            tok[(size_t)b * kQsaTokens + i] = qsa_token(blk_row, L, i);
    if (c0 >= n_tok) return;                       // whole workgroup
    const int c1 = min(c0 + kGChunk, n_tok);
    const int nsub = (c1 - c0 + kGSub - 1) / kGSub;

    u32x4 qf[4];
    const bool head = n < g;
    const uint16_t* qrow = q + ((size_t)b * Hq + (size_t)kv * g + (head ? n : 0)) * kGD + 8 * G;
#pragma unroll
    for (int u = 0; u < 4; ++u) qf[u] = *reinterpret_cast<const u32x4*>(qrow + 32 * u);
    for (int i = lane; i < kGChunk; i += 64) sel_s[i] = c0 + i < c1 ? qsa_token(blk_row, L, c0 + i) : -1;
    __syncthreads();

    const size_t slice = ((size_t)b * Hkv + kv) * S_max * kGD;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_cache + slice, (uint32_t)S_max * kGD * 2u);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_cache + slice, (uint32_t)S_max * kGD * 2u);
    // copy j of a sub-chunk fills LDS bytes [1024 j, +1024): lane l the 16
    // bytes at x = 1024 j + 16 l, row x / kGRowStride, column x mod it
    auto copy_sub = [&](int s, uint8_t* kd, uint8_t* vd) {
#pragma unroll
        for (int j = 0; j < kGSubCopies; ++j) {
            const int x = 1024 * j + 16 * lane;
            const int rr = x / kGRowStride, cc = x - rr * kGRowStride;
            const int row = sel_s[kGSub * s + min(rr, kGSub - 1)];
            const bool ok = rr < kGSub && cc < kGD * 2 && row >= 0;
            const uint32_t voff = ok ? (uint32_t)row * (kGD * 2) + (uint32_t)cc : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kd + 1024 * j, 16, voff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vd + 1024 * j, 16, voff, 0, 0, 0);
        }
    };
    // q is complete before the copies are issued (the compiler's wait counts
    // do not include loads into LDS)
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
    copy_sub(0, k0, v0);
    copy_sub(1, k1, v1);
    copy_sub(2, k2, v2);
    copy_sub(3, k3, v3);

    f32x4 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // sub-chunk s is complete once at most the copies of the later ones are
    // outstanding (2 kGSubCopies per sub-chunk, in issue order)
    constexpr int kPer = 2 * kGSubCopies;
    static_assert(3 * kPer < 64, "vmcnt range");
    auto wait_sub = [&](auto later) {
        constexpr int v = decltype(later)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70 | (v & 15) | ((v >> 4) << 14));
        asm volatile("s_barrier" ::: "memory");
    };
    wait_sub(std::integral_constant<int, 3 * kPer>{});
    gqa_gather_step(k0, v0, qf, o, m_run, l_run, c0, c1, qscale, G, n);
    if (nsub > 1) {
        wait_sub(std::integral_constant<int, 2 * kPer>{});
        gqa_gather_step(k1, v1, qf, o, m_run, l_run, c0 + kGSub, c1, qscale, G, n);
    }
    if (nsub > 2) {
        wait_sub(std::integral_constant<int, kPer>{});
        gqa_gather_step(k2, v2, qf, o, m_run, l_run, c0 + 2 * kGSub, c1, qscale, G, n);
    }
    if (nsub > 3) {
        wait_sub(std::integral_constant<int, 0>{});
        gqa_gather_step(k3, v3, qf, o, m_run, l_run, c0 + 3 * kGSub, c1, qscale, G, n);
    }
    __builtin_amdgcn_s_waitcnt(0);                 // copies of unused sub-chunks
    if (!head) return;
    const size_t idx = ((size_t)b * Hq + (size_t)kv * g + n) * n_chunks + chunk;
    float* po = part_o + idx * kGD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d0 = 8 * (4 * G + i);            // this lane holds d = d0 + t for head n
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]};
        *reinterpret_cast<f32x4*>(po + d0 + 4) = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]};
    }
    if (G == 0) {
        part_ml[idx * 2] = m_run;
        part_ml[idx * 2 + 1] = l_run;
    }
}

constexpr int kGChunks = (kQsaTokens + kGChunk - 1) / kGChunk;   // 17

// one wave per (batch, head): the chunks' partials merged (log-sum-exp).
// Lane c < nc holds chunk c's (m, l); for the output lane l holds dims 2 l
// and 2 l + 1, and every chunk's pair is requested at once (a chunk past nc
// re-reads the last one, with weight 0).
__global__ __launch_bounds__(256) void qsa_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int32_t* __restrict__ seq_lens, int Hq,
                                                          int S_max, int BH, uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int idx = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (idx >= BH) return;
    const int b = idx / Hq;
    const float* ml = part_ml + (size_t)idx * kGChunks * 2;
    const float* po = part_o + (size_t)idx * kGChunks * kGD + 2 * lane;
    // every chunk's state is requested together with seq_lens (one round
    // trip); the chunks past this row's count hold stale bytes, masked below
    // by selects and branches, never multiplied by a zero weight
    float2 p[kGChunks];
#pragma unroll
    for (int c = 0; c < kGChunks; ++c) p[c] = *reinterpret_cast<const float2*>(po + (size_t)c * kGD);
    float mc = -INFINITY, lc = 0.f;
    if (lane < kGChunks) {
        mc = ml[2 * lane];
        lc = ml[2 * lane + 1];
    }
    const int L = min(max(seq_lens[b], 1), S_max);
    const int nc = (qsa_n_tokens(L) + kGChunk - 1) / kGChunk;   // 1 .. kGChunks
    if (lane >= nc) {
        mc = -INFINITY;
        lc = 0.f;
    }
    float M = mc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
    const float w = lane < nc ? fast_exp2(mc - M) : 0.f;
    float den = w * lc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) den += __shfl_xor(den, d, 64);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int c = 0; c < kGChunks; ++c) {
        if (c < nc) {                              // wave-uniform
            const float wc = __shfl(w, c, 64);
            a0 += wc * p[c].x;
            a1 += wc * p[c].y;
        }
    }
    const float inv = 1.0f / den;
    *reinterpret_cast<uint32_t*>(out + (size_t)idx * kGD + 2 * lane) = pack_bf16x2(a0 * inv, a1 * inv);
}

}  // namespace

// The band re-scoring's buffers in the workspace region of refine_bytes.
static void refine_buffers(char* w, int32_t B, RefineArgs& ra) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    ra.state = reinterpret_cast<uint32_t*>(w);
    w += al((size_t)B * 8 * sizeof(uint32_t));
    ra.band_idx = reinterpret_cast<uint32_t*>(w);
    w += al((size_t)B * kBandCap * sizeof(uint32_t));
    ra.band_score = reinterpret_cast<double*>(w);
    w += al((size_t)B * kBandCap * sizeof(double));
    ra.sure_in = reinterpret_cast<uint32_t*>(w);
}

SparseLayout sparse_layout(int32_t B, int32_t H, int32_t S_max, int32_t top_k) {
    SparseLayout l{};
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    l.n_chunks = (top_k + kRowsPerChunk - 1) / kRowsPerChunk;
    l.n_key_chunks = (S_max + kChunkKeys - 1) / kChunkKeys;
    l.scores_bytes = al((size_t)B * ((S_max + 3) & ~3) * sizeof(float));
    l.hist_bytes = al((size_t)B * kHistBins * sizeof(uint32_t));
    // entries in per-chunk slices: keys [B][key chunks][4096], indices
    // [B][key chunks][4096], then their counts [B][key chunks]
    l.cand_bytes = al((size_t)B * l.n_key_chunks * (2 * kChunkKeys + 1) * sizeof(uint32_t));
    l.info_bytes = al((size_t)B * sizeof(SelInfo));
    l.refine_bytes = al((size_t)B * 8 * sizeof(uint32_t)) + al((size_t)B * kBandCap * sizeof(uint32_t)) +
                     al((size_t)B * kBandCap * sizeof(double)) + al((size_t)B * kSureCap * sizeof(uint32_t));
    l.o_bytes = al((size_t)B * H * l.n_chunks * kDv * sizeof(float));
    l.ml_bytes = al((size_t)B * H * l.n_chunks * 2 * sizeof(float));
    l.total = l.scores_bytes + l.hist_bytes + l.cand_bytes + l.info_bytes + l.refine_bytes +
              l.o_bytes + l.ml_bytes;
    return l;
}

QsaLayout qsa_layout(int32_t B, int32_t Hq, int32_t S_max) {
    QsaLayout l{};
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    l.n_blk_max = std::max(S_max / kQsaBlock, 1);
    l.sel = sparse_layout(B, 0, l.n_blk_max, kQsaTopBlocks);
    l.cnt_bytes = al((size_t)B * sizeof(int32_t));
    l.blk_bytes = al((size_t)B * kQsaTopBlocks * sizeof(int32_t));
    l.n_chunks = kGChunks;
    l.o_bytes = al((size_t)B * Hq * l.n_chunks * kGD * sizeof(float));
    l.ml_bytes = al((size_t)B * Hq * l.n_chunks * 2 * sizeof(float));
    l.total = l.sel.total + l.cnt_bytes + l.blk_bytes + l.o_bytes + l.ml_bytes;
    return l;
}

hipError_t launch_qsa_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const void* q_index, const void* k_index,
                                    const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t H_I, int32_t S_max, float scale, const RopeDev& rope,
                                    int32_t* tok, void* out, void* workspace, const QsaLayout& lay,
                                    hipStream_t s) {
    char* w = reinterpret_cast<char*>(workspace);
    const SparseLayout& sl = lay.sel;
    uint32_t* keys = reinterpret_cast<uint32_t*>(w);
    float* scores = reinterpret_cast<float*>(w);
    w += sl.scores_bytes;
    uint32_t* hist = reinterpret_cast<uint32_t*>(w);
    w += sl.hist_bytes;
    uint32_t* cand = reinterpret_cast<uint32_t*>(w);
    uint32_t* cand_idx = cand + (size_t)B * sl.n_key_chunks * kChunkKeys;
    uint32_t* cand_cnt = cand_idx + (size_t)B * sl.n_key_chunks * kChunkKeys;
    w += sl.cand_bytes;
    SelInfo* info = reinterpret_cast<SelInfo*>(w);
    w += sl.info_bytes;
    char* refine = w;
    w += sl.refine_bytes;
    w += sl.o_bytes + sl.ml_bytes;   // (empty)
    int32_t* cnt = reinterpret_cast<int32_t*>(w);
    w += lay.cnt_bytes;
    int32_t* blk = reinterpret_cast<int32_t*>(w);
    w += lay.blk_bytes;
    float* po = reinterpret_cast<float*>(w);
    w += lay.o_bytes;
    float* pml = reinterpret_cast<float*>(w);
    const int NB = lay.n_blk_max;
    const int KS = (NB + 3) & ~3;
    const int nkc = sl.n_key_chunks;
    if (nkc > kSelThreads) return hipErrorInvalidValue;   // one finish thread per chunk

    const int nz = B * kHistBins;
    hipLaunchKernelGGL(qsa_prep_kernel, dim3((std::max(nz, (int)B) + 255) / 256), dim3(256), 0, s, hist, nz,
                       seq_lens, S_max, B, cnt);
    const dim3 igrid((NB + kQsaBlocksPerWg - 1) / kQsaBlocksPerWg, B);
    const uint16_t* qi = (const uint16_t*)q_index;
    const uint16_t* ki = (const uint16_t*)k_index;
    switch (H_I) {
        case 16:
            hipLaunchKernelGGL((qsa_block_kernel<1>), igrid, dim3(256), 0, s, qi, ki, seq_lens, S_max, KS,
                               rope, keys, hist);
            break;
        case 32:
            hipLaunchKernelGGL((qsa_block_kernel<2>), igrid, dim3(256), 0, s, qi, ki, seq_lens, S_max, KS,
                               rope, keys, hist);
            break;
        case 48:
            hipLaunchKernelGGL((qsa_block_kernel<3>), igrid, dim3(256), 0, s, qi, ki, seq_lens, S_max, KS,
                               rope, keys, hist);
            break;
        case 64:
            hipLaunchKernelGGL((qsa_block_kernel<4>), igrid, dim3(256), 0, s, qi, ki, seq_lens, S_max, KS,
                               rope, keys, hist);
            break;
        default:
            return hipErrorInvalidValue;
    }

    RefineArgs ra{};   // the block scores are fp32: re-score the band at the 512th
    ra.mode = 2;
    ra.H_I = H_I;
    ra.q_index = qi;
    ra.k_index = ki;
    ra.S_tok = S_max;
    ra.rope = rope;
    refine_buffers(refine, B, ra);
    if (NB <= kSelOneKernelMax) {
        hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(kSelThreads), 0, s, scores, hist, cnt, NB,
                           KS, kQsaTopBlocks, blk, ra);
    } else {
        hipLaunchKernelGGL(topk_compact_kernel, dim3(nkc, B), dim3(kChunkThreads), 0, s, scores, hist,
                           cnt, NB, KS, kQsaTopBlocks, cand, cand_idx, cand_cnt, nkc, info, blk,
                           ra.lower_bins);
        hipLaunchKernelGGL(topk_finish_kernel, dim3(B), dim3(kSelThreads), 0, s, scores, cnt, NB, KS,
                           kQsaTopBlocks, cand, cand_idx, cand_cnt, nkc, info, blk, ra);
    }
    hipLaunchKernelGGL(band_score_kernel, dim3(kBandCap / 16, B), dim3(kSelThreads), 0, s, ra);
    hipLaunchKernelGGL(band_merge_kernel, dim3(B), dim3(kSelThreads), 0, s, ra, kQsaTopBlocks, blk);
    hipLaunchKernelGGL(gqa_gather_attn_kernel, dim3(kGChunks, Hkv, B), dim3(64), 0, s,
                       (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, blk,
                       seq_lens, Hq, Hkv, S_max, scale * kLog2e, tok, po, pml, kGChunks);
    const int BH = B * Hq;
    hipLaunchKernelGGL(qsa_combine_kernel, dim3((BH + 3) / 4), dim3(256), 0, s, po, pml, seq_lens, Hq,
                       S_max, BH, (uint16_t*)out);
    return hipGetLastError();
}

MlaLayout mla_layout(int32_t B, int32_t H, int32_t S_max) {
    MlaLayout l{};
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    // One workgroup per CU (256): every range writes H partial rows of 2 KiB
    // that the merge reads back, so ranges are made as long as filling the
    // machine allows (whole sub-chunks, at least kMlaMinRows rows).
    const int n_hg = (H + 16 * kMlaWaves - 1) / (16 * kMlaWaves);
    const int want = std::max(1, (kMlaTargetWgs + B * n_hg - 1) / (B * n_hg));
    const int per = (S_max + want - 1) / want;
    l.rows_per_split = std::max(kMlaMinRows, (per + kSubRows - 1) / kSubRows * kSubRows);
    l.n_split = (S_max + l.rows_per_split - 1) / l.rows_per_split;
    l.o_bytes = al((size_t)B * H * l.n_split * kDv * sizeof(float));
    l.ml_bytes = al((size_t)B * H * l.n_split * 2 * sizeof(float));
    l.total = l.o_bytes + l.ml_bytes;
    return l;
}

hipError_t launch_mla_decode(const void* q, const void* latent, const int32_t* seq_lens, int32_t B,
                             int32_t H, int32_t S_max, float scale, void* out, void* workspace,
                             const MlaLayout& lay, hipStream_t s) {
    float* po = reinterpret_cast<float*>(workspace);
    float* pml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + lay.o_bytes);
    const int n_hg = (H + 16 * kMlaWaves - 1) / (16 * kMlaWaves);
    const int n_units = B * lay.n_split;
    const int grid = 8 * n_hg * ((n_units + 7) / 8);
    hipLaunchKernelGGL((mla_dense_kernel<kMlaWaves>), dim3(grid), dim3(64 * kMlaWaves), 0, s,
                       (const uint16_t*)q, (const uint16_t*)latent, seq_lens, H, S_max,
                       lay.rows_per_split, scale * kLog2e, po, pml, lay.n_split, n_hg, n_units);
    const int BH = B * H;
    hipLaunchKernelGGL((combine_partials_kernel<kDv>), dim3((BH + 3) / 4), dim3(256), 0, s, po, pml,
                       seq_lens, H, S_max, S_max, lay.rows_per_split, lay.n_split, BH, (uint16_t*)out);
    return hipGetLastError();
}

hipError_t launch_topk_sparse_decode(const void* q, const void* latent, const void* q_index,
                                     const void* k_index, const int32_t* seq_lens, int32_t B,
                                     int32_t H, int32_t S_max, int32_t top_k, float scale,
                                     int32_t* topk_idx, void* out, void* workspace,
                                     const SparseLayout& lay, hipStream_t s, const float* w_index,
                                     int32_t H_I) {
    char* w = reinterpret_cast<char*>(workspace);
    float* scores = reinterpret_cast<float*>(w);
    w += lay.scores_bytes;
    uint32_t* hist = reinterpret_cast<uint32_t*>(w);
    w += lay.hist_bytes;
    uint32_t* cand = reinterpret_cast<uint32_t*>(w);
    uint32_t* cand_idx = cand + (size_t)B * lay.n_key_chunks * kChunkKeys;
    uint32_t* cand_cnt = cand_idx + (size_t)B * lay.n_key_chunks * kChunkKeys;
    w += lay.cand_bytes;
    SelInfo* info = reinterpret_cast<SelInfo*>(w);
    w += lay.info_bytes;
    char* refine = w;
    w += lay.refine_bytes;
    float* po = reinterpret_cast<float*>(w);
    w += lay.o_bytes;
    float* pml = reinterpret_cast<float*>(w);
    const int S_stride = (S_max + 3) & ~3;
    const int nkc = lay.n_key_chunks;
    if (nkc > kSelThreads) return hipErrorInvalidValue;   // one finish thread per chunk

    const int nz = B * kHistBins;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((nz + 255) / 256), dim3(256), 0, s, hist, nz);
    const int rows_per_block = 1024;
    const dim3 igrid((S_max + rows_per_block - 1) / rows_per_block, B);
    uint32_t* keys = reinterpret_cast<uint32_t*>(scores);
    const uint16_t* qi = (const uint16_t*)q_index;
    const uint16_t* ki = (const uint16_t*)k_index;
    switch (H_I) {
        case 0:
            hipLaunchKernelGGL(indexer_kernel, igrid, dim3(256), 0, s, qi, ki, seq_lens, S_max,
                               S_stride, rows_per_block, scores, hist);
            break;
        case 16:
            hipLaunchKernelGGL((indexer_weighted_kernel<1>), igrid, dim3(256), 0, s, qi, w_index, ki,
                               seq_lens, S_max, S_stride, rows_per_block, keys, hist);
            break;
        case 32:
            hipLaunchKernelGGL((indexer_weighted_kernel<2>), igrid, dim3(256), 0, s, qi, w_index, ki,
                               seq_lens, S_max, S_stride, rows_per_block, keys, hist);
            break;
        case 48:
            hipLaunchKernelGGL((indexer_weighted_kernel<3>), igrid, dim3(256), 0, s, qi, w_index, ki,
                               seq_lens, S_max, S_stride, rows_per_block, keys, hist);
            break;
        case 64:
            hipLaunchKernelGGL((indexer_weighted_kernel<4>), igrid, dim3(256), 0, s, qi, w_index, ki,
                               seq_lens, S_max, S_stride, rows_per_block, keys, hist);
            break;
        default:
            return hipErrorInvalidValue;
    }

    RefineArgs ra{};
    if (H_I > 0) {   // the weighted indexer's fp32 scores: re-score the band at the k-th
        ra.mode = 1;
        ra.H_I = H_I;
        ra.q_index = qi;
        ra.w_index = w_index;
        ra.k_index = ki;
        ra.S_tok = S_max;
        ra.knorm = hist;
        ra.lower_bins = 1;
        refine_buffers(refine, B, ra);
    }
    if (S_max <= kSelOneKernelMax) {
        hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(kSelThreads), 0, s, scores, hist, seq_lens,
                           S_max, S_stride, top_k, topk_idx, ra);
    } else {
        hipLaunchKernelGGL(topk_compact_kernel, dim3(nkc, B), dim3(kChunkThreads), 0, s, scores, hist,
                           seq_lens, S_max, S_stride, top_k, cand, cand_idx, cand_cnt, nkc, info,
                           topk_idx, ra.lower_bins);
        hipLaunchKernelGGL(topk_finish_kernel, dim3(B), dim3(kSelThreads), 0, s, scores, seq_lens, S_max,
                           S_stride, top_k, cand, cand_idx, cand_cnt, nkc, info, topk_idx, ra);
    }
    if (ra.mode != 0) {
        hipLaunchKernelGGL(band_score_kernel, dim3(kBandCap / 16, B), dim3(kSelThreads), 0, s, ra);
        hipLaunchKernelGGL(band_merge_kernel, dim3(B), dim3(kSelThreads), 0, s, ra, top_k, topk_idx);
    }
    hipLaunchKernelGGL(sparse_attn_kernel,
                       dim3(lay.n_chunks, (H + 16 * kAttnGroups - 1) / (16 * kAttnGroups), B),
                       dim3(64 * kAttnWaves), 0, s,
                       (const uint16_t*)q, (const uint16_t*)latent, topk_idx, seq_lens, H, S_max,
                       top_k, scale * kLog2e, po, pml, lay.n_chunks);
    const int BH = B * H;
    hipLaunchKernelGGL((combine_partials_kernel<kDv>), dim3((BH + 3) / 4), dim3(256), 0, s, po, pml,
                       seq_lens, H, S_max, top_k, kRowsPerChunk, lay.n_chunks, BH, (uint16_t*)out);
    return hipGetLastError();
}

}  // namespace gqa
