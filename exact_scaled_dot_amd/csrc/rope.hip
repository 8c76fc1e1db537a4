// RoPE: the one-pass rotation kernels.
//
// Adjacent pairs (x_2j, x_2j+1) of a row at position p rotate by p * theta_j,
// theta_j = base^(-2j/d) ("Transformer Architecture Breakdown", section 3.1;
// "coding-interview attention from scratch", section 三.5).  The rotation is
// evaluated in fp64 from the (cos, sin) table of rope_table.cpp, and the result
// is rounded fp64 -> fp32 (-> bf16), nearest even.

#include "device_common.h"
#include "launch.h"

namespace attn {

// Grid: x covers the N rows of one (batch, head) slice, 256 vectors per
// workgroup; y walks the slices, kSPT at a time, so each thread has kSPT
// loads in flight.  Within a slice the vector index is below
// N * d / 8 <= 2^28 (N <= 2^22, d <= 512), so the row and the position come
// from 32-bit arithmetic (a shift when d is 64 or 128, VPR != 0); only the
// slice offset is 64-bit.
constexpr int kMaxGridY = 65535;
constexpr int kSPT = 4;  // slices per thread and step

// One thread rotates 8 bf16 (4 pairs) of a row.
template <int VPR>
__global__ void __launch_bounds__(256)
rope_bf16_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ out, long long slices,
                 int N, int d, int pos_offset, const double2* __restrict__ tab) {
    const int vpr = VPR ? VPR : d >> 3;  // 16-byte vectors per row
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= N * vpr) return;
    const int n = i / vpr;
    const int d0 = (i - n * vpr) << 3;
    const double2* trow = tab + (size_t)(pos_offset + n) * (d >> 1);
    // kSPT slices per step, their loads issued before any rotation
    for (long long s0 = (long long)blockIdx.y * kSPT; s0 < slices; s0 += (long long)gridDim.y * kSPT) {
        uint4 v[kSPT];
#pragma unroll
        for (int j = 0; j < kSPT; ++j)
            if (s0 + j < slices)
                v[j] = *reinterpret_cast<const uint4*>(x + ((size_t)(s0 + j) * N + n) * d + d0);
#pragma unroll
        for (int j = 0; j < kSPT; ++j)
            if (s0 + j < slices)
                *reinterpret_cast<uint4*>(out + ((size_t)(s0 + j) * N + n) * d + d0) =
                    rope8_bf16(v[j], trow, d0);
    }
}

// One thread rotates 4 fp32 (2 pairs) of a row.
template <int VPR>
__global__ void __launch_bounds__(256)
rope_f32_kernel(const float* __restrict__ x, float* __restrict__ out, long long slices, int N,
                int d, int pos_offset, const double2* __restrict__ tab) {
    const int vpr = VPR ? VPR : d >> 2;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= N * vpr) return;
    const int n = i / vpr;
    const int d0 = (i - n * vpr) << 2;
    const double2* trow = tab + (size_t)(pos_offset + n) * (d >> 1);
    for (long long s0 = (long long)blockIdx.y * kSPT; s0 < slices; s0 += (long long)gridDim.y * kSPT) {
        float4 v[kSPT];
#pragma unroll
        for (int j = 0; j < kSPT; ++j)
            if (s0 + j < slices)
                v[j] = *reinterpret_cast<const float4*>(x + ((size_t)(s0 + j) * N + n) * d + d0);
#pragma unroll
        for (int j = 0; j < kSPT; ++j)
            if (s0 + j < slices)
                *reinterpret_cast<float4*>(out + ((size_t)(s0 + j) * N + n) * d + d0) =
                    rope4_f32(v[j], trow, d0);
    }
}

static dim3 grid_for(long long slices, int N, int vpr) {
    const long long gx = ((long long)N * vpr + 255) / 256;
    const long long steps = (slices + kSPT - 1) / kSPT;
    const long long gy = steps < kMaxGridY ? steps : kMaxGridY;
    return dim3((unsigned)gx, (unsigned)gy);
}

hipError_t launch_rope_bf16(const uint16_t* x, uint16_t* out, long long rows, int N, int d,
                            int pos_offset, const double2* tab, hipStream_t stream) {
    if (rows == 0 || N == 0) return hipSuccess;
    const long long slices = rows / N;
    const dim3 g = grid_for(slices, N, d / 8);
    if (d == 128)
        rope_bf16_kernel<16><<<g, 256, 0, stream>>>(x, out, slices, N, d, pos_offset, tab);
    else if (d == 64)
        rope_bf16_kernel<8><<<g, 256, 0, stream>>>(x, out, slices, N, d, pos_offset, tab);
    else
        rope_bf16_kernel<0><<<g, 256, 0, stream>>>(x, out, slices, N, d, pos_offset, tab);
    return hipGetLastError();
}

hipError_t launch_rope_f32(const float* x, float* out, long long rows, int N, int d,
                           int pos_offset, const double2* tab, hipStream_t stream) {
    if (rows == 0 || N == 0) return hipSuccess;
    const long long slices = rows / N;
    const dim3 g = grid_for(slices, N, d / 4);
    if (d == 128)
        rope_f32_kernel<32><<<g, 256, 0, stream>>>(x, out, slices, N, d, pos_offset, tab);
    else if (d == 64)
        rope_f32_kernel<16><<<g, 256, 0, stream>>>(x, out, slices, N, d, pos_offset, tab);
    else
        rope_f32_kernel<0><<<g, 256, 0, stream>>>(x, out, slices, N, d, pos_offset, tab);
    return hipGetLastError();
}

}  // namespace attn
