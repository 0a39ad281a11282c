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
// Work split: the rows of every (batch, kv head) context are concatenated
// into one global row space (batch-major, kv head, row) of
// total = Hkv * sum_b seq_lens[b] rows, cut into n_parts equal ranges of
// R = ceil(total / n_parts) rows.  Wave w streams range w, which may span
// several contexts; it emits one partial softmax state per (context, range)
// piece.  Every wave therefore moves the same number of bytes whatever the
// length mix, and a wave starts up (q load, RoPE) once per piece rather
// than once per short split.  Piece p of context i (starting at global row
// x) is stored at slot floor(x / R) + i, so slots are unique and the states
// of one context are contiguous.  Per piece, in tiles of 32 rows:
//   S^T[32 rows][16 heads] = K_tile . Q^T     (K as A operand; q as hi+lo bf16, 2x8 MFMAs)
//   online softmax per head in fp32 (base 2; scale*log2(e) is folded into q)
//   O^T[D][16 heads]      += V_tile^T . P^T   (8 MFMAs for D = 128)
// The S^T accumulator layout is exactly the P^T operand layout the second
// MFMA needs, so probabilities never leave their lane.  V^T operands come
// from 16-byte row loads transposed 8x8 in registers.  The next tile's loads
// are issued before the current tile's math (two register sets), so each
// wave keeps a whole tile (16 KB) in flight.  All K/V loads are 16-byte
// buffer loads bounded at the split's end: rows past it read as zero with
// no memory traffic, so ragged tails and the prefetch past the end cost
// nothing.
//
// combine_partials_kernel merges the per-split (m, l, o) with log-sum-exp
// rescaling; the result equals the softmax over the whole row.
#include "device_common.h"

namespace gqa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;
constexpr int kWaves = 4;   // waves per workgroup (each an independent work item)


template <int D>
struct DecodeTile {
    static constexpr int KU = D / 32;  // MFMA k-steps over the head dim
    u32x4 k[2][KU];
    u32x4 v[8];
};

template <int D>
__device__ __forceinline__ void load_tile(DecodeTile<D>& t, __amdgpu_buffer_rsrc_t kr,
                                          __amdgpu_buffer_rsrc_t vr, int t0, int G, int n) {
    constexpr int VN = D / 8;   // lanes of a 16-lane group that carry V columns
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int u = 0; u < DecodeTile<D>::KU; ++u)
            t.k[th][u] = buf_load16_nt(kr, (uint32_t)(((t0 + 16 * th + n) * D + 32 * u + 8 * G) * 2));
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint32_t off = (n < VN) ? (uint32_t)(((t0 + slot_row(G, r)) * D + 8 * n) * 2)
                                      : 0x80000000u;  // out of range -> zeros
        t.v[r] = buf_load16_nt(vr, off);
    }
}

template <int D, int NB>
__device__ __forceinline__ void tile_math(const DecodeTile<D>& t, int t0, int r1, int G,
                                          const u32x4 (&qhi)[NB][D / 32],
                                          const u32x4 (&qlo)[NB][D / 32], f32x4 (&o)[NB][8],
                                          float (&m_run)[NB], float (&l_run)[NB]) {
    constexpr int KU = D / 32;
    const bool tail = (t0 + 32 > r1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        f32x4 sc[2];
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            sc[th] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                sc[th] = mfma16(t.k[th][u], qhi[nb][u], sc[th]);
                sc[th] = mfma16(t.k[th][u], qlo[nb][u], sc[th]);
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
        mx = rows4_max(mx);   // over the 4 lane groups: the head's max over the 32 rows
        // Lazy rescale: the reference maximum only moves when some head's tile
        // maximum exceeds it by more than kLazy (base 2), so probabilities stay
        // below 2^kLazy and most tiles skip the O rescale.  O and l share the
        // reference, so O / l is unchanged.  Finite: row t0 < r1 is visible.
        if (__builtin_amdgcn_ballot_w64(mx > m_run[nb] + kLazy)) {
            asm volatile("" ::: "memory");   // keep the rescale behind the (rarely taken) branch
            const float m_new = fmaxf(m_run[nb], mx);
            const float alpha = fast_exp2(m_run[nb] - m_new);
            l_run[nb] *= alpha;
#pragma unroll
            for (int c = 0; c < 8; ++c) o[nb][c] *= alpha;
            m_run[nb] = m_new;
        }
        float p[2][4];
        float ls = 0.f;
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[th][i] = fast_exp2(sc[th][i] - m_run[nb]);
                ls += p[th][i];
            }
        l_run[nb] += rows4_sum(ls);
        u32x4 pb;
        pb[0] = pack_bf16x2(p[0][0], p[0][1]);
        pb[1] = pack_bf16x2(p[0][2], p[0][3]);
        pb[2] = pack_bf16x2(p[1][0], p[1][1]);
        pb[3] = pack_bf16x2(p[1][2], p[1][3]);
#pragma unroll
        for (int c = 0; c < 8; ++c) o[nb][c] = mfma16(column_of(t.v, c), pb, o[nb][c]);
    }
}

// The row space shared by the decode kernel and the combine: per batch b the
// contexts of its Hkv heads, each seq_lens[b] rows (clamped to [1, S_max]).
// The lengths are read by the wave's lanes in chunks of 64 and prefix-summed
// across the lanes, so the wave pays one load round trip per 64 batches
// instead of one per batch.
struct RowSpace {
    int64_t total;
    int64_t R;
};
// Which cache rows a context's new token attends to ([transformer架构]
// §2.5.1 sliding window: query i sees keys i-w+1 .. i; §2.5.2 rolling
// buffer: position t lives in slot t mod S_max).  Linear cache: positions
// max(0, L-window) .. L-1 are rows of the same index (window 0: all L);
// rolling buffer: every filled slot, min(L, S_max) of them from row 0.  The
// query's position is L-1 in both (keys are cached after RoPE).
struct CacheView {
    int window;    // 0 = no window
    int rolling;   // 1 = rolling buffer of S_max slots (window 0)
};
struct CtxGeom {
    int lo;        // first cache row
    int n;         // rows attended
    int qpos;      // the new token's position
    int newrow;    // the cache row of that position
};
__device__ __forceinline__ CtxGeom ctx_geom(const int32_t* seq_lens, int b, int S_max,
                                           const CacheView& cv) {
    const int raw = max(seq_lens[b], 1);
    if (cv.rolling) {
        const int n = min(raw, S_max);
        return CtxGeom{0, n, raw - 1, (int)((unsigned)(raw - 1) % (unsigned)S_max)};
    }
    const int L = min(raw, S_max);
    const int lo = cv.window > 0 ? max(0, L - cv.window) : 0;
    return CtxGeom{lo, L - lo, L - 1, L - 1};
}
__device__ __forceinline__ int ctx_len(const int32_t* seq_lens, int b, int S_max,
                                       const CacheView& cv) {
    return ctx_geom(seq_lens, b, S_max, cv).n;
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int64_t wave_scan_incl(int64_t x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}
__device__ __forceinline__ RowSpace row_space(const int32_t* seq_lens, int B, int Hkv, int S_max,
                                              int n_parts, int lane, const CacheView& cv) {
    int64_t total = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        int64_t rows = bb < B ? (int64_t)Hkv * ctx_len(seq_lens, bb, S_max, cv) : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) rows += __shfl_xor(rows, o, 64);
        total += rows;
    }
    return RowSpace{total, (total + n_parts - 1) / n_parts};
}
// The context holding global row x < total: batch b, the global row `base` of
// its (kv 0, row 0), and its number of attended rows L.
__device__ __forceinline__ void locate(const int32_t* seq_lens, int B, int Hkv, int S_max,
                                       int64_t x, int lane, const CacheView& cv, int& b,
                                       int64_t& base, int& L) {
    int64_t run = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        const int Lb = bb < B ? ctx_len(seq_lens, bb, S_max, cv) : 0;
        const int64_t incl = wave_scan_incl((int64_t)Hkv * Lb, lane);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(bb < B && x < run + incl);
        if (hit) {
            const int f = __builtin_ctzll(hit);
            b = c0 + f;
            L = __shfl(Lb, f, 64);
            base = run + __shfl(incl, f, 64) - (int64_t)Hkv * L;
            return;
        }
        run += __shfl(incl, 63, 64);
    }
    b = B;   // not reached for x < total
    base = run;
    L = 1;
}

// Per-lane RoPE frequencies of the q dims this lane holds (dims 32u + 8G ..
// +7, pairs i = 16u + 4G + p), read once per wave: the table sits in the
// kernel arguments and a lane-dependent index would otherwise cost a memory
// round trip per pair.
template <int D>
struct QFreq {
    double th[D / 32][4];
};
template <int D>
__device__ __forceinline__ void load_freq(const RopeDev& rope, int G, QFreq<D>& f) {
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int i = 16 * u + 4 * G + p;
            f.th[u][p] = i < rope.half ? rope.theta[i] : 0.0;
        }
}
// cos/sin of angle pos * pos_scale * theta, reduced to [-pi, pi] in fp64,
// then fp32 sincos, both scaled by amp (the same steps as rope_cos_sin).
__device__ __forceinline__ void cos_sin_theta(double theta, double pos, const RopeDev& r, float& c,
                                              float& s) {
    const double two_pi_hi = 6.283185307179586232;
    const double two_pi_lo = 2.4492935982947064e-16;
    const double a = pos * r.pos_scale * theta;
    const double k = rint(a * 0.15915494309189535);
    double red = fma(-k, two_pi_hi, a);
    red = fma(-k, two_pi_lo, red);
    float sv, cv;
    sincosf((float)red, &sv, &cv);
    c = cv * r.amp;
    s = sv * r.amp;
}

// Dynamic NTK ([transformer架构] §1.2 ④) for a sequence of current length L:
// theta_i * s^(-2i/(d-2)), s = max(1, L / L_train), i.e. the frequency of the
// NTK base b s^(d/(d-2)); log2 s is 0 (no change) when the setting is not
// dynamic or L <= L_train.
__device__ __forceinline__ double dyn_log2s(const RopeDev& r, int L) {
    return (r.dyn_train > 0 && L > r.dyn_train) ? log2((double)L / (double)r.dyn_train) : 0.0;
}
__device__ __forceinline__ double dyn_theta(double th, int i, double l2s, const RopeDev& r) {
    return l2s > 0.0 ? th * exp2(r.dyn_exp * (double)i * l2s) : th;
}

// Raw q rows of the group's heads (issued before the first tile loads, so
// waiting for them does not wait for the tiles).
template <int D, int NB>
__device__ __forceinline__ void load_q_raw(const uint16_t* q, int b, int kv, int Hq, int g, int G,
                                           int n, u32x4 (&raw)[NB][D / 32]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int hl = nb * 16 + n;
        const bool valid = hl < g;
        const uint16_t* qrow = q + ((size_t)b * Hq + (size_t)kv * g + (valid ? hl : 0)) * D;
#pragma unroll
        for (int u = 0; u < D / 32; ++u)
            raw[nb][u] = valid ? *reinterpret_cast<const u32x4*>(qrow + 32 * u + 8 * G) : u32x4{0, 0, 0, 0};
    }
}
// Rotates q at position L-1, folds in scale*log2(e) and splits it into the
// hi + lo bf16 pair the two MFMA passes use.
template <int D, int NB>
__device__ __forceinline__ void prep_q(const u32x4 (&raw)[NB][D / 32], const QFreq<D>& fq, int L,
                                       float qscale, const RopeDev& rope, int G,
                                       u32x4 (&qhi)[NB][D / 32], u32x4 (&qlo)[NB][D / 32]) {
    constexpr int KU = D / 32;
    float cs[KU][4], sn[KU][4];
    if (rope.half) {
        const double l2s = dyn_log2s(rope, L);
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int p = 0; p < 4; ++p)
                cos_sin_theta(dyn_theta(fq.th[u][p], 16 * u + 4 * G + p, l2s, rope), (double)(L - 1),
                              rope, cs[u][p], sn[u][p]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int d0 = 32 * u + 8 * G;
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = bf16_lo(raw[nb][u][j]);
                x[2 * j + 1] = bf16_hi(raw[nb][u][j]);
            }
            if (rope.half) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (d0 / 2 + p < rope.half) {
                        const float xe = x[2 * p], xo = x[2 * p + 1];
                        x[2 * p] = xe * cs[u][p] - xo * sn[u][p];
                        x[2 * p + 1] = xe * sn[u][p] + xo * cs[u][p];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = x[2 * j] * qscale, c2 = x[2 * j + 1] * qscale;
                const u32x2 hl = split_bf16x2(a, c2);
                qhi[nb][u][j] = hl[0];
                qlo[nb][u][j] = hl[1];
            }
        }
}

// The decode step's cache write, fused: the new token's row (position L-1,
// the last row of its context) is taken from k_new / v_new instead of the
// cache.  The key is rotated at L-1 with the frequencies this lane already
// holds for q (the K pairs a lane holds are its q pairs), amplitude included,
// and rounded to bf16; the value is used as given.  Both are also written to
// row L-1 of the caches.  The new rows are read with q (so no wait of their
// own) and kept in registers; the tile loop only swaps registers (no memory
// access inside it, so its load pipelining and wait counts are those of the
// plain kernel), and the stores follow the loop.
struct AppendArgs {
    const uint16_t* k_new;   // [B][Hkv][D] bf16, not rotated
    const uint16_t* v_new;   // [B][Hkv][D] bf16
    uint16_t* k_cache;       // the caches the kernel reads, written at row L-1
    uint16_t* v_cache;
};

template <int D>
struct NewRow {
    u32x4 k[D / 32];   // lane (G, n): dims 32 u + 8 G .. +7 (rotated in place by rotate_new_key)
    u32x4 v;           // lane (G, n), n < D/8: dims 8 n .. +7
};

template <int D>
__device__ __forceinline__ void load_new_row(NewRow<D>& nr, const AppendArgs& app, size_t nrow,
                                             int G, int n) {
#pragma unroll
    for (int u = 0; u < D / 32; ++u) nr.k[u] = *reinterpret_cast<const u32x4*>(app.k_new + nrow + 32 * u + 8 * G);
    nr.v = n < D / 8 ? *reinterpret_cast<const u32x4*>(app.v_new + nrow + 8 * n) : u32x4{0, 0, 0, 0};
}

template <int D>
__device__ __forceinline__ void rotate_new_key(NewRow<D>& nr, int L, const QFreq<D>& fq,
                                               const RopeDev& rope, int G) {
    const double l2s = dyn_log2s(rope, L);
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
        u32x4 w;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float xe = bf16_lo(nr.k[u][p]), xo = bf16_hi(nr.k[u][p]);
            if (16 * u + 4 * G + p < rope.half) {
                float c, sn;
                cos_sin_theta(dyn_theta(fq.th[u][p], 16 * u + 4 * G + p, l2s, rope), (double)(L - 1),
                              rope, c, sn);
                const float ye = xe * c - xo * sn, yo = xe * sn + xo * c;
                xe = ye;
                xo = yo;
            }
            w[p] = pack_bf16x2(xe, xo);
        }
        nr.k[u] = w;
    }
}

// Swap the new row into the tile that holds it (rr = its row in the tile,
// wave-uniform): K row rr is lane n = rr & 15 of half rr >> 4; V row rr is
// register rs of lane group Gs (see slot_row).
template <int D>
__device__ __forceinline__ void swap_new_row(DecodeTile<D>& t, const NewRow<D>& nr, int rr, int G,
                                             int n) {
    const int th = rr >> 4, nn = rr & 15;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            if (h2 == th && n == nn) t.k[h2][u] = nr.k[u];
    const int Gs = rr < 16 ? rr >> 2 : (rr - 16) >> 2;
    const int rs = rr < 16 ? (rr & 3) : 4 + ((rr - 16) & 3);
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2)
        if (r2 == rs && G == Gs && n < D / 8) t.v[r2] = nr.v;
}

template <int D>
__device__ __forceinline__ void store_new_row(const NewRow<D>& nr, uint16_t* krow, uint16_t* vrow,
                                              int rr, int G, int n) {
    if (n == (rr & 15))
#pragma unroll
        for (int u = 0; u < D / 32; ++u) *reinterpret_cast<u32x4*>(krow + 32 * u + 8 * G) = nr.k[u];
    const int Gs = rr < 16 ? rr >> 2 : (rr - 16) >> 2;
    if (G == Gs && n < D / 8) *reinterpret_cast<u32x4*>(vrow + 8 * n) = nr.v;
}

template <int D, int NB, bool APPEND>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ seq_lens, int B, int Hq,
    int Hkv, int S_max, float qscale, RopeDev rope, float* __restrict__ part_o,
    float* __restrict__ part_ml, int n_parts, AppendArgs app, CacheView cv) {
    constexpr int KU = D / 32;
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, n = lane & 15;
    const int g = Hq / Hkv;
    // wave-uniform by construction; readfirstlane lets the compiler keep every
    // derived address and buffer descriptor in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (w >= n_parts) return;
    const RowSpace rs = row_space(seq_lens, B, Hkv, S_max, n_parts, lane, cv);
    int64_t gs = (int64_t)w * rs.R;
    const int64_t ge = min(gs + rs.R, rs.total);
    if (gs >= ge) return;

    // locate the context holding global row gs
    int b, L;
    int64_t base;   // global row of (b, kv 0, row 0)
    locate(seq_lens, B, Hkv, S_max, gs, lane, cv, b, base, L);
    b = __builtin_amdgcn_readfirstlane(b);
    L = __builtin_amdgcn_readfirstlane(L);
    CtxGeom geo = ctx_geom(seq_lens, b, S_max, cv);   // geo.n == L
    int kv = (int)((gs - base) / L);
    QFreq<D> fq;
    load_freq<D>(rope, G, fq);

    while (gs < ge) {
        const int64_t ctx0 = base + (int64_t)kv * L;        // global row of this context's row 0
        const int r0 = (int)(gs - ctx0);
        const int r1 = (int)min((int64_t)L, ge - ctx0);

        // rows r of the piece are cache rows geo.lo + r; buffers end at this
        // piece's last row: the prefetch past it reads zeros for free
        const size_t slice = ((size_t)b * Hkv + kv) * (size_t)S_max * D;
        const size_t first = slice + (size_t)geo.lo * D;
        const uint32_t nbytes = (uint32_t)r1 * D * 2u;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_cache + first, nbytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_cache + first, nbytes);

        // q is requested first, then the first tiles; q is prepared while the
        // tiles are in flight
        u32x4 qraw[NB][KU];
        load_q_raw<D, NB>(q, b, kv, Hq, g, G, n, qraw);
        [[maybe_unused]] NewRow<D> nr;
        if constexpr (APPEND) load_new_row<D>(nr, app, ((size_t)b * Hkv + kv) * D, G, n);
        DecodeTile<D> ta, tb;
        load_tile<D>(ta, kr, vr, r0, G, n);

        u32x4 qhi[NB][KU], qlo[NB][KU];
        prep_q<D, NB>(qraw, fq, geo.qpos + 1, qscale, rope, G, qhi, qlo);
        // the new token's row, as a row of this context's attended range
        const int r_new = geo.newrow - geo.lo;
        const bool ends = APPEND && r0 <= r_new && r_new < r1;   // this piece holds it
        const int rr_new = (r_new - r0) & 31;                     // its row in its tile
        if constexpr (APPEND)
            if (ends) rotate_new_key<D>(nr, geo.qpos + 1, fq, rope, G);

        f32x4 o[NB][8];
        float m_run[NB], l_run[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int c = 0; c < 8; ++c) o[nb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run[nb] = -INFINITY;
            l_run[nb] = 0.f;
        }

        auto fix = [&](DecodeTile<D>& t, int t0) {
            if constexpr (APPEND)
                if (ends && t0 <= r_new && r_new < t0 + 32) swap_new_row<D>(t, nr, rr_new, G, n);
        };
        for (int t0 = r0;;) {
            load_tile<D>(tb, kr, vr, t0 + 32, G, n);
            fix(ta, t0);
            tile_math<D, NB>(ta, t0, r1, G, qhi, qlo, o, m_run, l_run);
            t0 += 32;
            if (t0 >= r1) break;
            load_tile<D>(ta, kr, vr, t0 + 32, G, n);
            fix(tb, t0);
            tile_math<D, NB>(tb, t0, r1, G, qhi, qlo, o, m_run, l_run);
            t0 += 32;
            if (t0 >= r1) break;
        }

        if constexpr (APPEND)
            if (ends) {
                const size_t row = slice + (size_t)geo.newrow * D;
                store_new_row<D>(nr, app.k_cache + row, app.v_cache + row, rr_new, G, n);
            }

        // ---- partial (m, l, o) of this piece
        const int64_t slot = gs / rs.R + ((int64_t)b * Hkv + kv);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int hl = nb * 16 + n;
            if (hl >= g) continue;
            const size_t idx = (size_t)slot * g + hl;
            float* po = part_o + idx * D;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 8 * (4 * G + i);  // this lane holds d = d0 + c, c = 0..7
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

        // ---- next context
        gs = ctx0 + r1;
        if (++kv == Hkv) {
            kv = 0;
            base += (int64_t)Hkv * L;
            if (++b >= B) break;
            geo = ctx_geom(seq_lens, b, S_max, cv);
            L = geo.n;
        }
    }
}

// One wave per (batch, q head): merges the states of the pieces of its
// context, slots floor(x/R) + i for the global rows x of context i.  Lane j
// reads the (m, l) of piece j, so the maximum and the weights take one
// round trip, and the o rows of the first 16 pieces (lane: D/64 values) are
// requested in the same round trip; further pieces are read eight at a time.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, int B, int Hq, int Hkv, int S_max, int n_parts,
    uint16_t* __restrict__ out, CacheView cv) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int idx = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (idx >= B * Hq) return;
    const int b = idx / Hq, h = idx - b * Hq;
    const int g = Hq / Hkv, kv = h / g, hl = h - kv * g;
    // one pass over seq_lens gives both the row space total and the global
    // row of (b, kv 0, row 0) (the prefix over the batches before b)
    int64_t total = 0, base = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int bb = c0 + lane;
        int64_t rows = bb < B ? (int64_t)Hkv * ctx_len(seq_lens, bb, S_max, cv) : 0;
        int64_t before = bb < b ? rows : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            rows += __shfl_xor(rows, o, 64);
            before += __shfl_xor(before, o, 64);
        }
        total += rows;
        base += before;
    }
    const int64_t R = (total + n_parts - 1) / n_parts;
    const int L = ctx_len(seq_lens, b, S_max, cv);
    const int64_t x0 = base + (int64_t)kv * L;
    const int64_t ctx = (int64_t)b * Hkv + kv;
    const int64_t s0 = x0 / R + ctx;
    const int np = (int)((x0 + L - 1) / R + ctx - s0 + 1);
    const size_t pstride = (size_t)g * D;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    float den = 0.f, M_run = -INFINITY;
    for (int c0 = 0; c0 < np; c0 += 64) {          // one chunk unless > 64 pieces
        const int cn = min(64, np - c0);
        const float* pbase = part_o + ((size_t)(s0 + c0) * g + hl) * D + lane * PER;
        // the o rows of the first 16 pieces are requested with the (m, l)
        // pair: they do not depend on the weights
        constexpr int kFirst = 16;
        float v0[kFirst][PER];
#pragma unroll
        for (int jj = 0; jj < kFirst; ++jj)
#pragma unroll
            for (int e = 0; e < PER; ++e) v0[jj][e] = jj < cn ? pbase[jj * pstride + e] : 0.f;
        float m = -INFINITY, l = 0.f;
        if (lane < cn) {
            const size_t i2 = (size_t)(s0 + c0 + lane) * g + hl;
            m = part_ml[i2 * 2];
            l = part_ml[i2 * 2 + 1];
        }
        float M = m;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, wave_shfl_xor(M, o));
        const float M_new = fmaxf(M_run, M);       // finite: every piece has a row
        const float rescale = fast_exp2(M_run - M_new);
        den *= rescale;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] *= rescale;
        const float wl = lane < cn ? fast_exp2(m - M_new) : 0.f;
        float dsum = wl * l;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dsum += wave_shfl_xor(dsum, o);
        den += dsum;
#pragma unroll
        for (int jj = 0; jj < kFirst; ++jj) {
            const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), jj));
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wgt * v0[jj][e];
        }
        for (int j0 = kFirst; j0 < cn; j0 += 8) {
            float v[8][PER];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                for (int e = 0; e < PER; ++e) v[jj][e] = j0 + jj < cn ? pbase[(j0 + jj) * pstride + e] : 0.f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float wgt = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), min(j0 + jj, 63)));
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += wgt * v[jj][e];
            }
        }
        M_run = M_new;
    }
    const float inv = 1.0f / den;
    uint16_t* o = out + (size_t)idx * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
        o[0] = (uint16_t)f32_to_bf16_bits(acc[0] * inv);
    }
}

template <int D, int NB>
void launch_split(hipStream_t s, const void* q, const void* k, const void* v, const int32_t* sl,
                  int B, int Hq, int Hkv, int S_max, float qscale, const RopeDev& rope, float* po,
                  float* pml, int n_parts, const AppendArgs& app, const CacheView& cv) {
    const dim3 grid((n_parts + kWaves - 1) / kWaves);
    if (app.k_new)
        hipLaunchKernelGGL((decode_split_kernel<D, NB, true>), grid, dim3(64 * kWaves), 0, s,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sl, B, Hq,
                           Hkv, S_max, qscale, rope, po, pml, n_parts, app, cv);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, NB, false>), grid, dim3(64 * kWaves), 0, s,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sl, B, Hq,
                           Hkv, S_max, qscale, rope, po, pml, n_parts, app, cv);
}

}  // namespace

DecodeLayout decode_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t n_parts) {
    DecodeLayout l;
    l.n_parts = n_parts;
    l.slots = (int64_t)n_parts + (int64_t)B * Hkv;
    const size_t units = (size_t)l.slots * (Hq / Hkv);
    l.o_bytes = (units * D * sizeof(float) + 255) & ~(size_t)255;
    l.ml_bytes = (units * 2 * sizeof(float) + 255) & ~(size_t)255;
    l.total = l.o_bytes + l.ml_bytes;
    return l;
}

hipError_t launch_gqa_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t D, int32_t S_max, float scale, const RopeDev& rope,
                                     void* workspace, const DecodeLayout& lay, hipStream_t s,
                                     const void* k_new, const void* v_new, int32_t window,
                                     int32_t rolling) {
    const CacheView cv{window, rolling};
    const AppendArgs app{(const uint16_t*)k_new, (const uint16_t*)v_new,
                         k_new ? (uint16_t*)const_cast<void*>(k_cache) : nullptr,
                         k_new ? (uint16_t*)const_cast<void*>(v_cache) : nullptr};
    float* po = reinterpret_cast<float*>(workspace);
    float* pml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + lay.o_bytes);
    const int g = Hq / Hkv;
    const int NB = (g + 15) / 16;
    const float qscale = scale * kLog2e;
    const int np = lay.n_parts;
    if (D == 128) {
        if (NB == 1) launch_split<128, 1>(s, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, S_max, qscale, rope, po, pml, np, app, cv);
        else if (NB == 2) launch_split<128, 2>(s, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, S_max, qscale, rope, po, pml, np, app, cv);
        else launch_split<128, 4>(s, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, S_max, qscale, rope, po, pml, np, app, cv);
    } else {
        if (NB == 1) launch_split<64, 1>(s, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, S_max, qscale, rope, po, pml, np, app, cv);
        else if (NB == 2) launch_split<64, 2>(s, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, S_max, qscale, rope, po, pml, np, app, cv);
        else launch_split<64, 4>(s, q, k_cache, v_cache, seq_lens, B, Hq, Hkv, S_max, qscale, rope, po, pml, np, app, cv);
    }
    return hipGetLastError();
}

hipError_t launch_gqa_decode_combine(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t D, int32_t S_max, const void* workspace,
                                     const DecodeLayout& lay, void* out, hipStream_t s,
                                     int32_t window, int32_t rolling) {
    const CacheView cv{window, rolling};
    const float* po = reinterpret_cast<const float*>(workspace);
    const float* pml = reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) + lay.o_bytes);
    dim3 cgrid((B * Hq + 3) / 4);
    if (D == 128)
        hipLaunchKernelGGL((decode_combine_kernel<128>), cgrid, dim3(256), 0, s, po, pml, seq_lens,
                           B, Hq, Hkv, S_max, lay.n_parts, (uint16_t*)out, cv);
    else
        hipLaunchKernelGGL((decode_combine_kernel<64>), cgrid, dim3(256), 0, s, po, pml, seq_lens,
                           B, Hq, Hkv, S_max, lay.n_parts, (uint16_t*)out, cv);
    return hipGetLastError();
}

}  // namespace gqa
