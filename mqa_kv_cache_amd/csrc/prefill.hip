// Causal GQA prefill on gfx950 MFMA (32x32x16; scores from hi + lo bf16 operands by
// default or fp16; P.V in fp16; fp32 accumulation).
//
// Prefill is a dense contraction: K/V are reused by every later query
// ([注意力变体与MoE] "生成时的瓶颈", last paragraph), so it runs on the matrix
// cores.  The operation is the pages' causal attention ([注意力变体与MoE]
// "MQA 与 GQA", attention(): q k^T / sqrt(hd), strict upper triangle masked,
// softmax, weighted sum of V) with RoPE on Q and K ([transformer架构] §1.1).
//
// Score precision.  RoPE is fused into the load, so the rotated Q and K are
// not bf16 inputs any more and must be rounded to reach the matrix cores.
// Rounding both to one 16-bit term perturbs every logit by up to
// 2^-11 |q~||k~| (fp16): with a sharp softmax (scores spread over several
// units) that alone moves outputs past 2e-3 + 1e-2 |ref|.  The default
// (SPLIT) path therefore carries rotated Q and K as hi + lo bf16 terms
// (hi = bf16(x), lo = bf16(x - hi): ~2^-17 relative) and forms each score
// from three products, Kh.Qh + Kh.Ql + Kl.Qh (the dropped Kl.Ql is ~2^-18
// of the score); the fast path rounds both to fp16 and needs one product.
// P is fp16 in both (2^-11 on weights that l sums exactly as rounded), V
// converts from bf16 to fp16 exactly inside the fp16 range, and fp16 and
// bf16 MFMA run at the same rate.
//
// Pre-pass (one read of K and V): K is rotated at its position and stored as
// bf16 hi and lo rows (SPLIT) or fp16 rows; V is stored as fp16 and
// transposed per 64-key tile, key columns permuted to match the P^T operand.
// Every later query tile re-reads these tiles, so neither the rotation nor
// the transpose is repeated.
//
// Masks: causal (key j <= query i); with a window w, the band
// i - w + 1 <= j <= i ([transformer架构] §2.5.1); with s sink tokens
// (StreamingLLM, [attention] "Slide Window Attention (SWA)", 修复方案 1) keys
// j < s stay visible as well: the band plus the first s columns
// ([transformer架构] §2.5.4).  A workgroup's key tiles are the sink tiles
// (those holding keys < s) followed by the tiles of its band; the two runs
// merge when the band reaches down to the sinks.
//
// Main kernel: one workgroup (4 waves) per (batch, q head, 128-query tile);
// wave w owns 32 queries.  Query tiles are issued heaviest (latest) first so
// the causal triangle balances across the machine.  Per 64-key tile:
//   * the workgroup stages K (rows padded by 16 B) and V^T in LDS;
//   * S^T[64 keys][32 queries] = K . Q^T   (K from LDS as A, Q^T in registers as B)
//   * online softmax per query in base 2 (scale*log2(e) is folded into Q)
//   * O^T[D][32 queries] += V^T . P^T       (P^T straight from the S^T accumulators)
// The S^T accumulator layout is the P^T operand layout, so probabilities
// never cross lanes; the only cross-lane step is one xor-32 shuffle for each
// max and sum.  Q is rotated while it is loaded (fp64 angle, fp32 sincos).
#include "device_common.h"

namespace gqa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int BM = 128;   // queries per workgroup (4 waves x 32)

// Minimum resident waves per SIMD requested from the register allocator.
#ifndef GQA_PREFILL_MIN_WAVES
#define GQA_PREFILL_MIN_WAVES 2
#endif
constexpr int BN = 64;    // keys per tile
#ifndef GQA_PREFILL_XCDS
#define GQA_PREFILL_XCDS 8
#endif
constexpr int kXcds = GQA_PREFILL_XCDS;   // XCDs that share the dispatch round-robin

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32h(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32b(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// One score product step: fp16 operands (fast path) or the three products
// of the hi + lo bf16 operands (SPLIT).
template <bool SPLIT>
__device__ __forceinline__ f32x16 score_mfma(u32x4 kh, u32x4 kl, u32x4 qh, u32x4 ql, f32x16 c) {
    if constexpr (SPLIT) {
        c = mfma32b(kh, qh, c);
        c = mfma32b(kh, ql, c);
        return mfma32b(kl, qh, c);
    } else {
        return mfma32h(kh, qh, c);
    }
}

// fp32 -> fp16 x2, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

// Column of 4-key chunk a (0..3) inside its 16-key group in the V^T tile:
// chunks are stored in the order 0, 2, 1, 3 so lane group h reads its
// keys {4h..4h+3, 8+4h..8+4h+3} as one 16-byte run.
__device__ __forceinline__ int chunk_col(int a) { return (a == 0) ? 0 : (a == 1) ? 8 : (a == 2) ? 4 : 12; }

template <int D>
struct Geo {
    static constexpr int DP = D < 16 ? 16 : D;            // head dim padded to one MFMA k-step
    static constexpr int KSTEPS = DP / 16;                // MFMA k-steps for S^T
    static constexpr int MT = D < 32 ? 1 : D / 32;        // O^T m-tiles of 32 d rows (D < 32 is zero-padded)
    // LDS rows are padded by 16 bytes so the 32 rows that one MFMA operand
    // read touches (same column) fall on distinct banks.
    static constexpr int KSTR = D + 8;                    // K tile row stride (fp16 elements)
    static constexpr int VSTR = BN + 8;                   // V^T tile row stride (fp16 elements)
    // Copies of a tile (see RowCopy) cover RPI padded rows each and always
    // write a whole 1 KB, so each buffer has room for the last copy's spill.
    static constexpr int K_RPI = 1024 / (2 * KSTR), K_N = (BN + K_RPI - 1) / K_RPI;
    static constexpr int V_RPI = 1024 / (2 * VSTR), V_N = (D + V_RPI - 1) / V_RPI;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int K_ELEMS = cmax(BN * KSTR, (K_N - 1) * K_RPI * KSTR + 512);
    static constexpr int V_ELEMS = cmax((D < 32 ? 32 : D) * VSTR, (V_N - 1) * V_RPI * VSTR + 512);
};

// Copies the rows of one tile (prepared fp16 K rows or V^T rows) from global
// memory straight into padded LDS rows, with no register staging.  A
// wave-wide 16-byte buffer load fills 1 KB of LDS starting where its M0 base
// points, lane l writing bytes [16 l, 16 l + 16).  Each copy starts at a row
// boundary and covers RPI whole padded rows; the lanes past them write the
// start of the next row, the same bytes the next copy writes, so overlapping
// copies agree, and the last copy spills into slack after the tile that
// nothing reads (its source rows are the next tile's, or past the buffer).
// Lanes on row padding read past the buffer end, which fetches nothing and
// stores zeros.  With this shape one per-lane offset serves every copy of
// every tile, and no copy needs a lane mask.
template <int ROWS, int ROW_BYTES, int STRIDE>
struct RowCopy {
    static constexpr int RPI = 1024 / STRIDE;                 // whole rows per copy
    static constexpr int N = (ROWS + RPI - 1) / RPI;          // copies per tile
    uint32_t voff;                                            // this lane's source offset within a copy
    __device__ __forceinline__ explicit RowCopy(int lane) {
        const int x = 16 * lane;
        const int rr = x / STRIDE;
        const int col = x - rr * STRIDE;
        voff = col < ROW_BYTES ? (uint32_t)(rr * ROW_BYTES + col) : 0x80000000u;
    }
    __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t src, uint32_t tile_off, uint16_t* dst,
                                        int wave) const {
#pragma unroll
        for (int i = 0; i < (N + 3) / 4; ++i) {
            const int j = 4 * i + wave;                       // wave-uniform
            if (j < N)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst + j * RPI * (STRIDE / 2), 16, voff,
                                                         tile_off + (uint32_t)(j * RPI * ROW_BYTES), 0, 0);
        }
    }
};

// K operand (A of S^T = K . Q^T): key row r, dims 8c .. 8c+7 (zero past D).
template <int D>
__device__ __forceinline__ u32x4 k_frag(const uint16_t* k_s, int r, int c) {
    if (D < 16 && 8 * c >= D) return u32x4{0, 0, 0, 0};
    return *reinterpret_cast<const u32x4*>(&k_s[r * Geo<D>::KSTR + 8 * c]);
}
// V^T operand (A of O^T += V^T . P^T): d row, key columns 8c .. 8c+7 (zero past D).
template <int D>
__device__ __forceinline__ u32x4 v_frag(const uint16_t* vt_s, int d, int c) {
    if (D < 32 && d >= D) return u32x4{0, 0, 0, 0};
    return *reinterpret_cast<const u32x4*>(&vt_s[d * Geo<D>::VSTR + 8 * c]);
}

// Rescaling of the running output is lazy: the reference maximum m_run is
// only raised when some query's tile maximum exceeds it by more than
// kLazy (in base-2 units), so the probabilities stay below 2^kLazy (well
// inside fp16) and most tiles skip the rescale.  O and l always share the
// same reference, so O / l is unchanged.
constexpr float kLazy = 8.0f;

// S^T[64 keys][32 queries] = K . Q^T for one tile (two 32-key halves).
template <int D, bool SPLIT>
__device__ __forceinline__ void qk_tile(const uint16_t* k_s, const uint16_t* kl_s,
                                        const u32x4 (&qf)[Geo<D>::KSTEPS],
                                        const u32x4 (&qfl)[Geo<D>::KSTEPS], f32x16 (&s)[2], int n,
                                        int h) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[st][e] = 0.f;
#pragma unroll
        for (int u = 0; u < Geo<D>::KSTEPS; ++u)
            s[st] = score_mfma<SPLIT>(k_frag<D>(k_s, 32 * st + n, 2 * u + h),
                                      SPLIT ? k_frag<D>(kl_s, 32 * st + n, 2 * u + h) : u32x4{},
                                      qf[u], qfl[u], s[st]);
    }
}

// Causal mask: keys past the lane's query qi (only the diagonal tile has any).
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int ks, int qi, int h) {
    // key = ks + 32 st + 8 j + 4 h + i is masked when 32 st + 8 j + i > lim;
    // lim is opaque so the 32 compares happen here rather than being hoisted
    // into (spilled) scalar masks
    int lim = qi - ks - 4 * h;
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (32 * st + 8 * j + i > lim) s[st][4 * j + i] = -INFINITY;
}

// Sliding window (band mask): keys below the lane's query qi minus
// (window - 1) are masked, except the sink keys (key < sinks); only the
// sink tiles and the first band tiles of a wave hold any.
__device__ __forceinline__ void mask_low(f32x16 (&s)[2], int ks, int qi, int h, int window,
                                         int sinks) {
    // key = ks + 32 st + 8 j + 4 h + i is masked when slim <= 32 st + 8 j + i < lim
    int lim = qi - window + 1 - ks - 4 * h;
    int slim = sinks - ks - 4 * h;
    asm volatile("" : "+v"(lim), "+v"(slim));
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 32 * st + 8 * j + i;
                if (kk < lim && kk >= slim) s[st][4 * j + i] = -INFINITY;
            }
}

// The reference maximum while a query has seen no visible key yet (only with
// a window, on a wave's first tiles): exp2(-inf - 0) = 0 instead of NaN.
__device__ __forceinline__ float ref_max(float m_run) { return m_run == -INFINITY ? 0.f : m_run; }

// Folds the tile's row maxima into m_run (lazily, see kLazy).  Without a
// window every tile a wave processes holds a visible key for each query; with
// one, a query's first tiles may hold none (m_run then stays -inf, and the
// rescale and ref_max keep that from producing NaN).
template <int D>
__device__ __forceinline__ void tile_max(const f32x16 (&s)[2], f32x16 (&o)[Geo<D>::MT],
                                         float& m_run, float& l_run) {
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[st][e]);
    mx = halves_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy)) {
        asm volatile("" ::: "memory");   // keep the rescale behind the (rarely taken) branch
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);   // no key seen yet: nothing to scale
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < Geo<D>::MT; ++mt) o[mt] *= alpha;
        m_run = m_new;
    }
}

// acc + lo + hi of a packed fp16 pair (one dot2 instruction).
__device__ __forceinline__ float sum_f16x2(uint32_t pk, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), one, acc, false);
}

// P = exp2(S - m) as fp16 pairs in the P^T operand layout (step 2 st + c
// holds keys 32 st + 16 c .. +15); returns the lane's part of the row sum.
__device__ __forceinline__ float probs(const f32x16 (&s)[2], float m, u32x4 (&pb)[4]) {
    float ls = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float p0 = fast_exp2(s[st][8 * c + 2 * w] - m);
                const float p1 = fast_exp2(s[st][8 * c + 2 * w + 1] - m);
                const uint32_t pk = pack_f16x2(p0, p1);
                pb[2 * st + c][w] = pk;
                ls = sum_f16x2(pk, ls);
            }
    return ls;
}

// O^T[D][32 queries] += V^T . P^T over the tile's four 16-key steps.
template <int D>
__device__ __forceinline__ void pv_tile(const uint16_t* vt_s, const u32x4 (&pb)[4],
                                        f32x16 (&o)[Geo<D>::MT], int n, int h) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int mt = 0; mt < Geo<D>::MT; ++mt)
            o[mt] = mfma32h(v_frag<D>(vt_s, 32 * mt + n, 2 * k4 + h), pb[k4], o[mt]);
}

// One pipelined step, written as explicit groups that the scheduler may not
// mix (sched_barrier): phase A issues the S^T MFMAs of the next tile, each
// with one K fragment read two MFMAs ahead and a slice of the softmax of the
// current tile; phase B issues the P.V MFMAs of the current tile, each with
// one V fragment read two ahead and a slice of the next tile's maximum.  The
// VALU work then runs under the matrix pipe instead of between its bursts,
// and phase A's last two groups already read phase B's first V fragments.
template <int D, bool SPLIT>
__device__ __forceinline__ void pipelined_step(const uint16_t* k_nx, const uint16_t* kl_nx,
                                               const uint16_t* v_cu,
                                               const u32x4 (&qf)[Geo<D>::KSTEPS],
                                               const u32x4 (&qfl)[Geo<D>::KSTEPS],
                                               const f32x16 (&s_c)[2], f32x16 (&s_n)[2],
                                               f32x16 (&o)[Geo<D>::MT], float& m_run, float& l_run,
                                               bool diag_next, bool low_next, int window, int sinks,
                                               int ks_next, int qi, int n, int h) {
    constexpr int KS = Geo<D>::KSTEPS, MT = Geo<D>::MT;
    constexpr int NQK = 2 * KS;          // S^T MFMA steps of a tile (three MFMAs each when SPLIT)
    constexpr int NPV = 4 * MT;          // P.V MFMAs of a tile
    constexpr int PAIRS = 16 / NQK;      // probability pairs per phase-A group
    constexpr int MAXV = 32 / NPV;       // scores per phase-B group
    const float m = ref_max(m_run);

    // ---- phase A: S^T(next) || P(current)
    u32x4 kf[NQK], kfl[NQK];
    u32x4 vf[NPV];
    u32x4 pb[4];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 2 && i < NQK; ++i) {
        kf[i] = k_frag<D>(k_nx, 32 * (i / KS) + n, 2 * (i % KS) + h);
        if constexpr (SPLIT) kfl[i] = k_frag<D>(kl_nx, 32 * (i / KS) + n, 2 * (i % KS) + h);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_n[st][e] = 0.f;
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
        if (i + 2 < NQK) {
            kf[i + 2] = k_frag<D>(k_nx, 32 * ((i + 2) / KS) + n, 2 * ((i + 2) % KS) + h);
            if constexpr (SPLIT) kfl[i + 2] = k_frag<D>(kl_nx, 32 * ((i + 2) / KS) + n, 2 * ((i + 2) % KS) + h);
        } else if (i + 2 - NQK < NPV) {   // the first V fragments of phase B, read under phase A
            vf[i + 2 - NQK] = v_frag<D>(v_cu, 32 * ((i + 2 - NQK) % MT) + n, 2 * ((i + 2 - NQK) / MT) + h);
        }
        s_n[i / KS] = score_mfma<SPLIT>(kf[i], kfl[i], qf[i % KS], qfl[i % KS], s_n[i / KS]);
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int p = i * PAIRS + q;             // pair: st = p / 8, c = (p / 4) % 2, w = p % 4
            const int st = p >> 3, c = (p >> 2) & 1, w = p & 3;
            const float p0 = fast_exp2(s_c[st][8 * c + 2 * w] - m);
            const float p1 = fast_exp2(s_c[st][8 * c + 2 * w + 1] - m);
            const uint32_t pk = pack_f16x2(p0, p1);
            pb[2 * st + c][w] = pk;
            ls = sum_f16x2(pk, ls);     // the row sum sees the same rounded P as the MFMA
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    l_run += halves_sum(ls);
    if (diag_next) mask_tile(s_n, ks_next, qi, h);
    if (low_next) mask_low(s_n, ks_next, qi, h, window, sinks);

    // ---- phase B: O += V.P(current) || max S^T(next)
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < NPV; ++g) {
        if (g + 2 < NPV) vf[g + 2] = v_frag<D>(v_cu, 32 * ((g + 2) % MT) + n, 2 * ((g + 2) / MT) + h);
        o[g % MT] = mfma32h(vf[g], pb[g / MT], o[g % MT]);
#pragma unroll
        for (int q = 0; q < MAXV; ++q) {
            const int e = g * MAXV + q;
            mx = fmaxf(mx, s_n[e >> 4][e & 15]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    mx = halves_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy)) {
        asm volatile("" ::: "memory");   // keep the rescale behind the (rarely taken) branch
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);   // no key seen yet: nothing to scale
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
        m_run = m_new;
    }
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(256, SPLIT ? 1 : GQA_PREFILL_MIN_WAVES) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kh, const uint16_t* __restrict__ kl,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ out, int T, int T_pad, int Hq, int Hkv,
    float qscale, RopeDev rope, int window, int sinks) {
    using Gm = Geo<D>;
    // Two buffers per operand, as separate LDS objects: the compiler then
    // tells the tile being read from the one being copied into, and does not
    // make the reads wait for the copy in flight.  (The lo K buffers hold
    // nothing on the fast path.)
    constexpr int KL_ELEMS = SPLIT ? Gm::K_ELEMS : 8;
    __shared__ __attribute__((aligned(16))) uint16_t k_s0[Gm::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t k_s1[Gm::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t kl_s0[KL_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t kl_s1[KL_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vt_s0[Gm::V_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vt_s1[Gm::V_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;
    const int n_qt = (T + BM - 1) / BM;
    const int g = Hq / Hkv;
    int qt, hq, b, kvh;
    {
        // Work order: heaviest (latest) query tiles first.  Workgroups are
        // handed to the 8 XCDs round-robin by linear id; when the (batch, kv
        // head) groups divide evenly over them, each XCD takes whole groups so
        // the K/V tiles that its query tiles share stay in its own L2.
        const int L = blockIdx.x;
        const int G = (int)gridDim.x / (n_qt * g);   // B * Hkv
        if (G % kXcds == 0) {
            const int x = L % kXcds, k = L / kXcds;
            const int per_qt = (G / kXcds) * g;
            const int r = k / per_qt, rem = k - r * per_qt;
            const int jg = rem / g, hl = rem - jg * g;
            const int grp = x + kXcds * jg;
            b = grp / Hkv;
            kvh = grp - b * Hkv;
            hq = kvh * g + hl;
            qt = n_qt - 1 - r;
        } else {
            const int per_qt = G * g;       // B * Hq
            const int r = L / per_qt, rem = L - r * per_qt;
            b = rem / Hq;
            hq = rem - b * Hq;
            kvh = hq / g;
            qt = n_qt - 1 - r;
        }
    }
    const int q0 = qt * BM + 32 * wave;      // first query of this wave
    const int qi = q0 + n;                    // this lane's query

    const size_t qbase = ((size_t)b * Hq + hq) * (size_t)T * D;
    const size_t kvbase = ((size_t)b * Hkv + kvh) * (size_t)T_pad * D;
    const int q_last_wg = min(qt * BM + BM - 1, T - 1);
    // Key tiles of this workgroup.  With a window (band mask) the band starts
    // at the tile holding the first key its first query sees (kt0); with s
    // sink tokens the ns = ceil(s / 64) sink tiles come first when they lie
    // below kt0 (ns_sep of them), otherwise the band already covers them.
    // Logical tile t is physical tile t (t < ns_sep) or kt0 + t - ns_sep.
    int kt0 = window > 0 ? max(0, qt * BM - window + 1) / BN : 0;
    const int ns = (window > 0 && sinks > 0) ? (sinks + BN - 1) / BN : 0;
    int ns_sep = ns;
    if (kt0 <= ns) {
        kt0 = 0;
        ns_sep = 0;
    }
    const int n_kt = q_last_wg / BN + 1 - kt0 + ns_sep;
    auto phys = [&](int t) { return t < ns_sep ? t : kt0 + t - ns_sep; };

    const uint32_t kv_bytes = (uint32_t)T_pad * D * 2u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kh + kvbase, kv_bytes);
    const __amdgpu_buffer_rsrc_t klr = make_rsrc(SPLIT ? kl + kvbase : kh + kvbase, kv_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vt + kvbase, kv_bytes);   // V^T tiles: [T_pad/64][D][64]
    auto tile_off = [&](int t) { return (uint32_t)phys(t) * BN * D * 2u; };
    const RowCopy<BN, 2 * D, 2 * Gm::KSTR> kcopy(lane);
    const RowCopy<D, 2 * BN, 2 * Gm::VSTR> vcopy(lane);
    auto copy_k = [&](int t, uint16_t* dst, uint16_t* dst_lo, int wv) {
        kcopy.run(kr, tile_off(t), dst, wv);
        if constexpr (SPLIT) kcopy.run(klr, tile_off(t), dst_lo, wv);
    };
    // the first tile's copy overlaps the Q load and rotation
    copy_k(0, k_s0, kl_s0, wave);
    vcopy.run(vr, tile_off(0), vt_s0, wave);

    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + qbase, (uint32_t)T * D * 2u);
    // ---- Q^T operands: lane holds query qi, dims 16u + 8h .. +7, rotated and
    // scaled: hi + lo bf16 (SPLIT) or fp16
    u32x4 qf[Gm::KSTEPS], qfl[Gm::KSTEPS];
#pragma unroll
    for (int u = 0; u < Gm::KSTEPS; ++u) {
        const int d0 = 16 * u + 8 * h;
        u32x4 raw = (d0 < D && qi < T) ? buf_load16(qr, (uint32_t)((qi * D + d0) * 2)) : u32x4{0, 0, 0, 0};
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16_lo(raw[j]);
            x[2 * j + 1] = bf16_hi(raw[j]);
        }
        if (rope.half && d0 < D) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int i = d0 / 2 + p;
                if (i < rope.half) {
                    float c, s;
                    rope_cos_sin(rope, (double)qi, i, c, s);
                    const float xe = x[2 * p], xo = x[2 * p + 1];
                    x[2 * p] = xe * c - xo * s;
                    x[2 * p + 1] = xe * s + xo * c;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (SPLIT) {
                const u32x2 hl = split_bf16x2(x[2 * j] * qscale, x[2 * j + 1] * qscale);
                qf[u][j] = hl[0];
                qfl[u][j] = hl[1];
            } else {
                qf[u][j] = pack_f16x2(x[2 * j] * qscale, x[2 * j + 1] * qscale);
                qfl[u][j] = 0u;
            }
        }
    }

    f32x16 o[Gm::MT];
#pragma unroll
    for (int mt = 0; mt < Gm::MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mt][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Software pipeline over 64-key tiles.  K runs one tile ahead of V:
    // step t computes S^T of tile t+1 (MFMA) while it turns the scores of
    // tile t into probabilities (VALU), then accumulates P.V of tile t while
    // it takes the maximum of tile t+1.  Tile t of K lives in k_s[t & 1] and
    // of V in vt_s[t & 1] (separate LDS objects, named statically through an
    // unroll by two, so reads never wait for an unrelated copy in flight).
    // At the top of step t every wave waits for its own copies and meets the
    // barrier; all waves are then done with K(t) and V(t-1), so the copies
    // of K(t+2) and V(t+1) go into those buffers.  This wave's queries see
    // tiles 0 .. n_w-1 and only the last of them holds keys past its first
    // query (q0 is a multiple of 32, tiles are 64 wide); a wave done early
    // keeps copying its share and meeting the barriers of the others.
    const int n_w = min((q0 + 31) / BN + 1 - kt0 + ns_sep, n_kt);
    // tile t holds keys below some query's band (other than sinks) when its
    // first key is below the wave's last query's lower bound
    auto low = [&](int t) { return window > 0 && phys(t) * BN < q0 + 32 - window; };
    if (n_kt > 1) copy_k(1, k_s1, kl_s1, wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s_cur[2];
    qk_tile<D, SPLIT>(k_s0, kl_s0, qf, qfl, s_cur, n, h);
    if (n_w == 1) mask_tile(s_cur, phys(0) * BN, qi, h);
    if (low(0)) mask_low(s_cur, phys(0) * BN, qi, h, window, sinks);
    tile_max<D>(s_cur, o, m_run, l_run);

    auto top = [&](int t, uint16_t* k_dst, uint16_t* kl_dst, uint16_t* v_dst) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // the wave index is made opaque here so the copy addresses are formed
        // per step with a few scalar ops instead of being hoisted (and spilled)
        int wv = wave;
        asm volatile("" : "+s"(wv));
        if (t + 2 < n_kt) copy_k(t + 2, k_dst, kl_dst, wv);
        if (t + 1 < n_kt) vcopy.run(vr, tile_off(t + 1), v_dst, wv);
    };
    // a step with a next tile: scores s_cur -> P.V, S^T of tile t+1 -> s_nxt
    auto full = [&](int t, f32x16 (&s_c)[2], f32x16 (&s_n)[2], const uint16_t* k_next,
                    const uint16_t* kl_next, const uint16_t* v_cur, uint16_t* k_dst,
                    uint16_t* kl_dst, uint16_t* v_dst) {
        top(t, k_dst, kl_dst, v_dst);
        pipelined_step<D, SPLIT>(k_next, kl_next, v_cur, qf, qfl, s_c, s_n, o, m_run, l_run,
                                 t + 1 == n_w - 1, low(t + 1), window, sinks, phys(t + 1) * BN, qi,
                                 n, h);
    };
    // this wave's last step
    auto last = [&](int t, const f32x16 (&s_c)[2], const uint16_t* v_cur, uint16_t* k_dst,
                    uint16_t* kl_dst, uint16_t* v_dst) {
        top(t, k_dst, kl_dst, v_dst);
        u32x4 pb[4];
        l_run += halves_sum(probs(s_c, ref_max(m_run), pb));
        pv_tile<D>(v_cur, pb, o, n, h);
    };
    f32x16 s_alt[2];
    int t = 0;
    for (; t + 2 < n_w; t += 2) {
        full(t, s_cur, s_alt, k_s1, kl_s1, vt_s0, k_s0, kl_s0, vt_s1);
        full(t + 1, s_alt, s_cur, k_s0, kl_s0, vt_s1, k_s1, kl_s1, vt_s0);
    }
    if (t + 1 < n_w) {
        full(t, s_cur, s_alt, k_s1, kl_s1, vt_s0, k_s0, kl_s0, vt_s1);
        last(t + 1, s_alt, vt_s1, k_s1, kl_s1, vt_s0);
        t += 2;
    } else {
        last(t, s_cur, vt_s0, k_s0, kl_s0, vt_s1);
        t += 1;
    }
    for (; t < n_kt; ++t) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t & 1) {
            if (t + 2 < n_kt) copy_k(t + 2, k_s1, kl_s1, wave);
            if (t + 1 < n_kt) vcopy.run(vr, tile_off(t + 1), vt_s0, wave);
        } else {
            if (t + 2 < n_kt) copy_k(t + 2, k_s0, kl_s0, wave);
            if (t + 1 < n_kt) vcopy.run(vr, tile_off(t + 1), vt_s1, wave);
        }
    }

    // ---- normalise and write: lane holds query qi, d = 32 mt + 8 j + 4 h + i
    if (qi < T) {
        const float inv = 1.0f / l_run;
        uint16_t* orow = out + qbase + (size_t)qi * D;
#pragma unroll
        for (int mt = 0; mt < Gm::MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * mt + 8 * j + 4 * h;
                if (d0 < D) {
                    u32x2 w;
                    w[0] = pack_bf16x2(o[mt][4 * j + 0] * inv, o[mt][4 * j + 1] * inv);
                    w[1] = pack_bf16x2(o[mt][4 * j + 2] * inv, o[mt][4 * j + 3] * inv);
                    *reinterpret_cast<u32x2*>(orow + d0) = w;
                }
            }
    }
}

// Pre-pass, one block per (64-key tile, kv head, batch):
//   K  -> RoPE at its position (fp64 angle, fp32 sincos) -> bf16 hi and lo
//         rows (SPLIT) or fp16 rows                                     [B][Hkv][T_pad][D]
//   V  -> fp16 (exact for bf16 values in fp16 range), transposed per tile into
//         [B][Hkv][T_pad/64][D][64] with key columns permuted for the P^T operand.
// Rows at or past T are written as zeros.
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) void prefill_prep_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ kh,
    uint16_t* __restrict__ kl, uint16_t* __restrict__ vt, int T, int T_pad, int Hkv, RopeDev rope) {
    __shared__ float cs_c[BN * kMaxRotaryHalf / 2];
    __shared__ float cs_s[BN * kMaxRotaryHalf / 2];
    constexpr int CPR = D / 8;
    const int tid = threadIdx.x;
    const int kt = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int ks = kt * BN;
    const int half = rope.half;   // <= D/2 <= 64
    const size_t in_base = ((size_t)b * Hkv + kvh) * (size_t)T * D;
    const size_t out_base = ((size_t)b * Hkv + kvh) * (size_t)T_pad * D;
    // the tile's K and V chunks are requested first; the cos/sin table is
    // formed while they are in flight
    constexpr int NK = (BN * CPR + 255) / 256;          // K chunks per thread
    constexpr int NV = ((BN / 4) * CPR + 255) / 256;    // V 4-row groups per thread
    u32x4 kraw[NK], vraw[NV][4];
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int c = tid + 256 * j;
        const int key = c / CPR, dc = c - key * CPR;
        const int t = ks + key;
        kraw[j] = (c < BN * CPR && t < T)
                      ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + in_base + (size_t)t * D + 8 * dc))
                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = tid + 256 * j;
        const int kg = c / CPR, dc = c - kg * CPR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = ks + 4 * kg + r;
            vraw[j][r] = (c < (BN / 4) * CPR && t < T)
                             ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + in_base + (size_t)t * D + 8 * dc))
                             : u32x4{0, 0, 0, 0};
        }
    }
    for (int e = tid; e < BN * half; e += 256) {
        const int tl = e / half, i = e - tl * half;
        float c, sn;
        rope_cos_sin(rope, (double)(ks + tl), i, c, sn);
        cs_c[e] = c;
        cs_s[e] = sn;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int c = tid + 256 * j;
        if (c >= BN * CPR) break;
        const int key = c / CPR, dc = c - key * CPR;
        const int t = ks + key;
        u32x4 val, lo;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float xe = bf16_lo(kraw[j][p]), xo = bf16_hi(kraw[j][p]);
            const int i = 4 * dc + p;
            if (i < half) {
                const float cc = cs_c[key * half + i], ss = cs_s[key * half + i];
                const float ye = xe * cc - xo * ss, yo = xe * ss + xo * cc;
                xe = ye;
                xo = yo;
            }
            if constexpr (SPLIT) {
                const u32x2 hl = split_bf16x2(xe, xo);
                val[p] = hl[0];
                lo[p] = hl[1];
            } else {
                val[p] = pack_f16x2(xe, xo);
            }
        }
        *reinterpret_cast<u32x4*>(kh + out_base + (size_t)t * D + 8 * dc) = val;   // zeros past T
        if constexpr (SPLIT) *reinterpret_cast<u32x4*>(kl + out_base + (size_t)t * D + 8 * dc) = lo;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = tid + 256 * j;
        if (c >= (BN / 4) * CPR) break;
        const int kg = c / CPR, dc = c - kg * CPR;
        u32x4 r4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int w = 0; w < 4; ++w) r4[r][w] = pack_f16x2(bf16_lo(vraw[j][r][w]), bf16_hi(vraw[j][r][w]));
        const int col = 16 * (kg >> 2) + chunk_col(kg & 3);
        uint16_t* tile = vt + out_base + (size_t)kt * D * BN;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int w = t >> 1;
            u32x2 pr;
            if (t & 1) {
                pr[0] = (r4[0][w] >> 16) | (r4[1][w] & 0xFFFF0000u);
                pr[1] = (r4[2][w] >> 16) | (r4[3][w] & 0xFFFF0000u);
            } else {
                pr[0] = (r4[0][w] & 0xFFFFu) | (r4[1][w] << 16);
                pr[1] = (r4[2][w] & 0xFFFFu) | (r4[3][w] << 16);
            }
            *reinterpret_cast<u32x2*>(tile + (size_t)(8 * dc + t) * BN + col) = pr;
        }
    }
}

template <int D, bool SPLIT>
void launch_d(const void* q, const void* k, const void* v, void* out, void* kh, void* kl, void* vt,
              int B, int T, int Hq, int Hkv, float qscale, const RopeDev& rope, int window,
              int sinks, hipStream_t s) {
    const int T_pad = (T + BN - 1) / BN * BN;
    hipLaunchKernelGGL((prefill_prep_kernel<D, SPLIT>), dim3(T_pad / BN, Hkv, B), dim3(256), 0, s,
                       (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)kh, (uint16_t*)kl,
                       (uint16_t*)vt, T, T_pad, Hkv, rope);
    dim3 grid((T + BM - 1) / BM * Hq * B);   // one workgroup per (query tile, q head, batch)
    hipLaunchKernelGGL((prefill_kernel<D, SPLIT>), grid, dim3(256), 0, s, (const uint16_t*)q,
                       (const uint16_t*)kh, (const uint16_t*)kl, (const uint16_t*)vt,
                       (uint16_t*)out, T, T_pad, Hq, Hkv, qscale, rope, window, sinks);
}

template <bool SPLIT>
void launch_p(const void* q, const void* k, const void* v, void* out, void* kh, void* kl, void* vt,
              int B, int T, int Hq, int Hkv, int D, float qscale, const RopeDev& rope, int window,
              int sinks, hipStream_t s) {
    switch (D) {
        case 8: launch_d<8, SPLIT>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, qscale, rope, window, sinks, s); break;
        case 16: launch_d<16, SPLIT>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, qscale, rope, window, sinks, s); break;
        case 32: launch_d<32, SPLIT>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, qscale, rope, window, sinks, s); break;
        case 64: launch_d<64, SPLIT>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, qscale, rope, window, sinks, s); break;
        default: launch_d<128, SPLIT>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, qscale, rope, window, sinks, s); break;
    }
}

}  // namespace

size_t prefill_prep_bytes(int32_t B, int32_t Hkv, int32_t T, int32_t D) {
    const size_t T_pad = ((size_t)T + BN - 1) / BN * BN;
    return (((size_t)B * Hkv * T_pad * D * 2) + 255) & ~(size_t)255;
}

hipError_t launch_gqa_prefill(const void* q, const void* k, const void* v, int32_t B, int32_t T,
                              int32_t Hq, int32_t Hkv, int32_t D, float scale, const RopeDev& rope,
                              void* out, void* workspace, hipStream_t s, int32_t window,
                              int32_t sinks, int32_t fp16_scores) {
    const float qscale = scale * kLog2e;
    const size_t pb = prefill_prep_bytes(B, Hkv, T, D);
    void* kh = workspace;
    void* kl = reinterpret_cast<char*>(workspace) + pb;
    void* vt = reinterpret_cast<char*>(workspace) + 2 * pb;
    if (fp16_scores)
        launch_p<false>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, D, qscale, rope, window, sinks, s);
    else
        launch_p<true>(q, k, v, out, kh, kl, vt, B, T, Hq, Hkv, D, qscale, rope, window, sinks, s);
    return hipGetLastError();
}

}  // namespace gqa
