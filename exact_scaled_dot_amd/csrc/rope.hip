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

// One thread rotates 8 bf16 (4 pairs) of a row.
__global__ void __launch_bounds__(256)
rope_bf16_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ out,
                 long long nvec, int N, int d, int pos_offset,
                 const double2* __restrict__ tab) {
    const int vec_per_row = d >> 3;
    const int half = d >> 1;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < nvec;
         i += (long long)gridDim.x * blockDim.x) {
        const long long row = i / vec_per_row;
        const int d0 = (int)(i - row * vec_per_row) << 3;
        const int pos = pos_offset + (int)(row % N);
        uint4 v = *reinterpret_cast<const uint4*>(x + row * d + d0);
        *reinterpret_cast<uint4*>(out + row * d + d0) = rope8_bf16(v, tab + (size_t)pos * half, d0);
    }
}

// One thread rotates 4 fp32 (2 pairs) of a row.
__global__ void __launch_bounds__(256)
rope_f32_kernel(const float* __restrict__ x, float* __restrict__ out, long long nvec, int N,
                int d, int pos_offset, const double2* __restrict__ tab) {
    const int vec_per_row = d >> 2;
    const int half = d >> 1;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < nvec;
         i += (long long)gridDim.x * blockDim.x) {
        const long long row = i / vec_per_row;
        const int d0 = (int)(i - row * vec_per_row) << 2;
        const int pos = pos_offset + (int)(row % N);
        float4 v = *reinterpret_cast<const float4*>(x + row * d + d0);
        *reinterpret_cast<float4*>(out + row * d + d0) = rope4_f32(v, tab + (size_t)pos * half, d0);
    }
}

static int grid_for(long long nvec) {
    long long g = (nvec + 255) / 256;
    if (g > 256 * 64) g = 256 * 64;  // grid-stride beyond 64 workgroups per CU
    return (int)(g < 1 ? 1 : g);
}

hipError_t launch_rope_bf16(const uint16_t* x, uint16_t* out, long long rows, int N, int d,
                            int pos_offset, const double2* tab, hipStream_t stream) {
    const long long nvec = rows * (d / 8);
    if (nvec == 0) return hipSuccess;
    rope_bf16_kernel<<<grid_for(nvec), 256, 0, stream>>>(x, out, nvec, N, d, pos_offset, tab);
    return hipGetLastError();
}

hipError_t launch_rope_f32(const float* x, float* out, long long rows, int N, int d,
                           int pos_offset, const double2* tab, hipStream_t stream) {
    const long long nvec = rows * (d / 4);
    if (nvec == 0) return hipSuccess;
    rope_f32_kernel<<<grid_for(nvec), 256, 0, stream>>>(x, out, nvec, N, d, pos_offset, tab);
    return hipGetLastError();
}

}  // namespace attn
