// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

constexpr float kLn2 = 0.693147180559945309f;

// Exact fp32 value of a bf16 stored as its 16 bits.
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 bits (a in the low half), round to nearest even:
// one gfx950 v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// An empty volatile asm statement: code in a branch that holds it cannot be
// speculated, so cheap-looking vector work (64 multiplies, 32 selects) stays
// behind its wave-uniform branch.
__device__ __forceinline__ void keep_branch() { __asm__ volatile(""); }

// One RoPE pair in fp64, products and sums rounded separately (no contraction),
// then fp64 -> fp32 (nearest even).  Caller rounds on to bf16 if needed.
__device__ __forceinline__ void rope_pair_f64(float x0, float x1, double c, double s,
                                              float& r0, float& r1) {
#pragma clang fp contract(off)
    double a = (double)x0, b = (double)x1;
    double p0 = a * c;
    double p1 = b * s;
    double p2 = a * s;
    double p3 = b * c;
    r0 = (float)(p0 - p1);
    r1 = (float)(p2 + p3);
}

// Rotate 8 consecutive bf16 elements (4 pairs) at head-dim offset d0 of a row at
// position pos; tab is [npos][d/2] of (cos, sin).
__device__ __forceinline__ uint4 rope8_bf16(uint4 x, const double2* __restrict__ tab_row, int d0) {
    const double2* t = tab_row + (d0 >> 1);
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        double2 cs = t[j];
        float r0, r1;
        rope_pair_f64(bf16_lo(w[j]), bf16_hi(w[j]), cs.x, cs.y, r0, r1);
        w[j] = pack_bf16x2(r0, r1);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One pair rotated by the negative angle (the transpose of rope_pair_f64).
__device__ __forceinline__ void rope_pair_t_f64(float x0, float x1, double c, double s,
                                                float& r0, float& r1) {
#pragma clang fp contract(off)
    double a = (double)x0, b = (double)x1;
    double p0 = a * c;
    double p1 = b * s;
    double p2 = a * s;
    double p3 = b * c;
    r0 = (float)(p0 + p1);
    r1 = (float)(p3 - p2);
}

// Rotate 4 consecutive fp32 elements (2 pairs).
__device__ __forceinline__ float4 rope4_f32(float4 x, const double2* __restrict__ tab_row, int d0) {
    const double2* t = tab_row + (d0 >> 1);
    double2 c0 = t[0], c1 = t[1];
    float4 r;
    rope_pair_f64(x.x, x.y, c0.x, c0.y, r.x, r.y);
    rope_pair_f64(x.z, x.w, c1.x, c1.y, r.z, r.w);
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace attn
