// Standalone RoPE ([transformer架构] §1.1 rotation, §1.2 PI / NTK / YaRN).
//
// One block covers a group of tokens.  The block first forms cos/sin of each
// (token, frequency) once in LDS (fp64 angle, reduced, fp32 sincos, times the
// YaRN amplitude), then every thread rotates 16-byte chunks (4 adjacent
// pairs) of the (token, head) rows, so the transcendental work is shared by
// all heads of a token.  The kernel is HBM-bound: each element is read once
// and written once.
#include "device_common.h"

namespace gqa {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeLdsFloats = 4096;  // per table (cos and sin): TB * half <= 4096

__global__ __launch_bounds__(kRopeThreads) void rope_apply_kernel(
    const uint16_t* __restrict__ in, uint16_t* __restrict__ out, const int32_t* __restrict__ positions,
    int64_t n_tok, int n_heads, int head_dim, int64_t stride_tok, int64_t stride_head, RopeDev rope,
    int tok_per_block) {
    __shared__ float cs_c[kRopeLdsFloats];
    __shared__ float cs_s[kRopeLdsFloats];
    const int half = rope.half;
    const int64_t tok0 = (int64_t)blockIdx.x * tok_per_block;
    for (int e = threadIdx.x; e < tok_per_block * half; e += kRopeThreads) {
        const int tl = e / half, i = e - tl * half;
        const int64_t tok = tok0 + tl;
        if (tok < n_tok) {
            float c, s;
            rope_cos_sin(rope, positions ? (double)positions[tok] : (double)tok, i, c, s);
            cs_c[e] = c;
            cs_s[e] = s;
        }
    }
    __syncthreads();
    const int chunks = head_dim / 8;
    const int items = n_heads * chunks;
    const int rot_chunks = (2 * half) / 8;
    for (int it = threadIdx.x; it < tok_per_block * items; it += kRopeThreads) {
        const int tl = it / items;
        const int rem = it - tl * items;
        const int h = rem / chunks, c = rem - h * chunks;
        const int64_t tok = tok0 + tl;
        if (tok >= n_tok) continue;
        const int64_t off = tok * stride_tok + (int64_t)h * stride_head + 8 * c;
        u32x4 v = *reinterpret_cast<const u32x4*>(in + off);
        if (c < rot_chunks) {
            const float* cc = cs_c + tl * half + 4 * c;
            const float* ss = cs_s + tl * half + 4 * c;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float xe = bf16_lo(v[p]), xo = bf16_hi(v[p]);
                v[p] = pack_bf16x2(xe * cc[p] - xo * ss[p], xe * ss[p] + xo * cc[p]);
            }
            *reinterpret_cast<u32x4*>(out + off) = v;
        } else if (out != in) {
            *reinterpret_cast<u32x4*>(out + off) = v;
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
    int tb = kRopeThreads / items;
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

hipError_t launch_rope_rows(const void* in, void* out, int64_t n_tok, int32_t n_heads,
                            int32_t head_dim, int64_t stride_tok, int64_t stride_head,
                            const RopeDev& rope, hipStream_t s) {
    return launch_rope_apply(in, out, nullptr, n_tok, n_heads, head_dim, stride_tok, stride_head,
                             rope, s);
}

}  // namespace gqa
