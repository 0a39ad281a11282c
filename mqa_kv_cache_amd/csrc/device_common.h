// Device-side helpers shared by the gfx950 kernels of libgqa_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.h"

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): the conversion
// is gfx950's v_cvt_pk_bf16_f32, one instruction per pair of values.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// a and b each as hi + lo bf16 terms: hi = bf16(x), lo = bf16(x - hi)
// (x to about 2^-17 relative), packed in pairs: {hi pair, lo pair}.
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
    const uint32_t hi = pack_bf16x2(a, b);
    return u32x2{hi, pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u))};
}

// The probabilities of a 32-row tile as the P^T operand of the PV product,
// in two bf16 terms (hi = bf16(p), lo = bf16(p - hi)): p reaches the matrix
// core to about 2^-17 relative instead of bf16's 2^-9, which a sharp softmax
// with cancelling values needs (a dominant row's single-term rounding error
// alone can exceed the output tolerance).  p[th][i] is row 16 th + 4 G + i.
__device__ __forceinline__ void pack_p_hilo(const float (&p)[2][4], u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x2 hl = split_bf16x2(p[th][2 * j], p[th][2 * j + 1]);
            hi[2 * th + j] = hl[0];
            lo[2 * th + j] = hl[1];
        }
}

// ---------------------------------------------------------------------------
// Buffer resources: loads outside [0, num_bytes) return zero, so tails and
// ragged lengths need no branches and can never fault.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    // dword 3 = 0x00020000: raw (untyped) 32-bit data format on gfx9-family parts.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// Streaming variant: the nontemporal (nt) cache policy, for data read once.
// On this part it lets a whole-chip read stream run ~12% faster than with
// the default policy (measured with a plain read kernel, 6.8 vs 6.0 TB/s).
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}

// ---------------------------------------------------------------------------
// MFMA 16x16x32 bf16 -> fp32 (gfx950).  Lane l = 16*G + n:
//   A operand: A[m = n][k = 8G .. 8G+7]
//   B operand: B[k = 8G .. 8G+7][n]
//   C/D:       C[m = 4G + i][n], i = 0..3
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// RoPE cos/sin of pair i at position pos: angle formed in fp64, reduced to
// [-pi, pi] in fp64, then an fp32 sincos; both scaled by the amplitude.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void cos_sin_fp64_angle(double a, float& c, float& s) {
    const double two_pi_hi = 6.283185307179586232;
    const double two_pi_lo = 2.4492935982947064e-16;
    double k = rint(a * 0.15915494309189535);
    double red = fma(-k, two_pi_hi, a);
    red = fma(-k, two_pi_lo, red);
    sincosf((float)red, &s, &c);
}
__device__ __forceinline__ void rope_cos_sin_theta(const RopeDev& r, double pos, double theta, float& c,
                                                   float& s) {
    float sv, cv;
    cos_sin_fp64_angle(pos * r.pos_scale * theta, cv, sv);
    c = cv * r.amp;
    s = sv * r.amp;
}

__device__ __forceinline__ void rope_cos_sin(const RopeDev& r, double pos, int i, float& c, float& s) {
    rope_cos_sin_theta(r, pos, r.theta[i], c, s);
}

// Row (within a 32-row tile) that k-slot r of lane group G stands for.  It is
// the row the S^T accumulator of that lane group holds in register r:
// rows 4G..4G+3 of the first 16-row half, 16+4G..16+4G+3 of the second.
__device__ __forceinline__ int slot_row(int G, int r) {
    return (r < 4) ? (4 * G + r) : (16 + 4 * G + (r - 4));
}

// Column t (0..7) of an 8x8 bf16 block held as 8 rows of 16 bytes, packed as
// one MFMA operand whose k-slots are the rows.
__device__ __forceinline__ u32x4 column_of(const u32x4 (&rows)[8], int t) {
    u32x4 r;
    const int w = t >> 1;
    if (t & 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (rows[2 * j][w] >> 16) | (rows[2 * j + 1][w] & 0xFFFF0000u);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (rows[2 * j][w] & 0xFFFFu) | (rows[2 * j + 1][w] << 16);
    }
    return r;
}

// max and sum over the 64 lanes (every lane active), wave-uniform result:
// DPP swaps within quads, half rows and rows reduce each 16-lane row, and
// the four row results are combined from lanes 0, 16, 32, 48.
template <int Ctrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float rowlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp_f<0x140>(x));   // row_mirror
    return fmaxf(fmaxf(rowlane_f(x, 0), rowlane_f(x, 16)), fmaxf(rowlane_f(x, 32), rowlane_f(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    return (rowlane_f(x, 0) + rowlane_f(x, 16)) + (rowlane_f(x, 32) + rowlane_f(x, 48));
}

// Both halves of the wave's values of v, through the gfx950 lane-half swap
// (a VALU op, no LDS round trip): every lane gets lane (l mod 32)'s value as
// the first element and lane 32 + (l mod 32)'s as the second, so a max or sum
// of the pair is bit-identical in both halves.  The instruction is written
// out: this toolchain's optimizer replaces the second result of the builtin
// with the first.  The nops cover the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void halves(float v, float& lo, float& hi) {
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    lo = a;
    hi = b;
}
// Max / sum over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48), through the gfx950 row swaps: the 16-lane swap pairs rows (0,1) and
// (2,3), the half swap then pairs the two results.  Bit-identical in every
// lane.
__device__ __forceinline__ void rows16(float v, float& lo, float& hi) {
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    lo = a;
    hi = b;
}
__device__ __forceinline__ float rows4_max(float v) {
    float lo, hi, a, b;
    rows16(v, lo, hi);
    halves(fmaxf(lo, hi), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float rows4_sum(float v) {
    float lo, hi, a, b;
    rows16(v, lo, hi);
    halves(lo + hi, a, b);
    return a + b;
}
__device__ __forceinline__ float halves_max(float v) {
    float lo, hi;
    halves(v, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float halves_sum(float v) {
    float lo, hi;
    halves(v, lo, hi);
    return lo + hi;
}

}  // namespace gqa
