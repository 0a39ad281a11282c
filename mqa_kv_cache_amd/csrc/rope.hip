// Standalone RoPE ([transformer架构] §1.1 rotation, §1.2 PI / NTK / YaRN).
//
// One block covers a group of tokens.  Each thread first requests up to
// eight 16-byte chunks (4 adjacent pairs each) of the block's (token, head)
// rows, then, while they are in flight, the block forms cos/sin of each
// (token, frequency) once in LDS (fp64 angle, reduced, fp32 sincos, times
// the YaRN amplitude), so the transcendental work is shared by all heads of
// a token and hidden behind the loads.  The kernel is HBM-bound: each
// element is read once and written once.  The stores take the nontemporal
// policy and the loads the default one: on the 8K prefill's Q rows (67 MB
// each way) that ran in 21.7 us against 27.9 us with both nontemporal and
// 28.5 us with both default (16 chunks per thread instead of 8: slower).
#include "device_common.h"

namespace gqa {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeChunks = 8;        // 16-byte chunks per thread per pass
constexpr int kRopeLdsFloats = 4096;  // per table (cos and sin): TB * half <= 4096

__global__ __launch_bounds__(kRopeThreads) void rope_apply_kernel(
    const uint16_t* __restrict__ in, uint16_t* __restrict__ out, const int32_t* __restrict__ positions,
    int64_t n_tok, int n_heads, int head_dim, int64_t stride_tok, int64_t stride_head, RopeDev rope,
    int tok_per_block) {
    __shared__ float cs_c[kRopeLdsFloats];
    __shared__ float cs_s[kRopeLdsFloats];
    const int half = rope.half;
    const int64_t tok0 = (int64_t)blockIdx.x * tok_per_block;
    const int chunks = head_dim / 8;
    const int items = n_heads * chunks;
    const int rot_chunks = (2 * half) / 8;
    const int total = tok_per_block * items;
    const int tid = threadIdx.x;
    for (int base = 0; base < total; base += kRopeThreads * kRopeChunks) {
        u32x4 v[kRopeChunks];
        int64_t off[kRopeChunks];
        int tl[kRopeChunks], cc[kRopeChunks];
#pragma unroll
        for (int k = 0; k < kRopeChunks; ++k) {
            const int it = base + tid + kRopeThreads * k;
            tl[k] = it / items;
            const int rem = it - tl[k] * items;
            const int h = rem / chunks;
            cc[k] = rem - h * chunks;
            const bool ok = it < total && tok0 + tl[k] < n_tok;
            off[k] = ok ? (tok0 + tl[k]) * stride_tok + (int64_t)h * stride_head + 8 * cc[k] : -1;
            if (ok) v[k] = *reinterpret_cast<const u32x4*>(in + off[k]);
        }
        if (base == 0) {
            for (int e = tid; e < tok_per_block * half; e += kRopeThreads) {
                const int t = e / half, i = e - t * half;
                const int64_t tok = tok0 + t;
                if (tok < n_tok) {
                    float c, sn;
                    rope_cos_sin(rope, positions ? (double)positions[tok] : (double)tok, i, c, sn);
                    cs_c[e] = c;
                    cs_s[e] = sn;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int k = 0; k < kRopeChunks; ++k) {
            if (off[k] < 0) continue;
            if (cc[k] < rot_chunks) {
                const float* cp = cs_c + tl[k] * half + 4 * cc[k];
                const float* sp = cs_s + tl[k] * half + 4 * cc[k];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float xe = bf16_lo(v[k][p]), xo = bf16_hi(v[k][p]);
                    v[k][p] = pack_bf16x2(xe * cp[p] - xo * sp[p], xe * sp[p] + xo * cp[p]);
                }
                __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(out + off[k]));
            } else if (out != in) {
                __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(out + off[k]));
            }
        }
    }
}

}  // namespace

// positions == nullptr: the position of token t is t (used to rotate K for prefill).
hipError_t launch_rope_apply(const void* in, void* out, const int32_t* positions, int64_t n_tok,
                             int32_t n_heads, int32_t head_dim, int64_t stride_tok,
                             int64_t stride_head, const RopeDev& rope, hipStream_t s) {
    if (n_tok == 0) return hipSuccess;
    const int items = n_heads * (head_dim / 8);
    int tb = kRopeThreads * kRopeChunks / items;
    if (tb < 1) tb = 1;
    if (tb > 64) tb = 64;
    if (rope.half > 0) {
        while (tb > 1 && tb * rope.half > kRopeLdsFloats) tb /= 2;
    }
    const int64_t blocks = (n_tok + tb - 1) / tb;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rope_apply_kernel, dim3((unsigned)blocks), dim3(kRopeThreads), 0, s,
                       (const uint16_t*)in, (uint16_t*)out, positions, n_tok, n_heads, head_dim,
                       stride_tok, stride_head, rope, tb);
    return hipGetLastError();
}

}  // namespace gqa
