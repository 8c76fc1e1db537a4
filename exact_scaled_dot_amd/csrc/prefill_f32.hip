// Tiled exact attention forward for fp32 inputs (vector ALU, fp32 arithmetic).
//
// Same method as the bf16 kernel (online softmax over K/V tiles staged in LDS,
// "coding-interview attention from scratch", section 三.7), but one thread owns
// one query row and every product is an fp32 FMA, so fp32 inputs keep fp32
// precision end to end.  K/V tiles of 32 keys are shared by the 128 rows of a
// workgroup through LDS; reads of a K or V row are LDS broadcasts.  With a
// sliding window w (causal), the key loop starts at the first tile the
// workgroup's first row can see and keys at or below position p-w are masked.

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kRowsF = 128;  // query rows (threads) per workgroup
constexpr int kBcF = 32;     // keys per tile

template <int D, bool CAUSAL, bool ROPE, bool WINDOW>
__global__ void __launch_bounds__(kRowsF)
prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                   const float* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, float scale_log2,
                   const double2* __restrict__ tab, int nrb, int win, int o_bf16) {
    static_assert(!WINDOW || CAUSAL, "the sliding window is built for causal attention");
    __shared__ __attribute__((aligned(16))) float Ks[kBcF * D];
    __shared__ __attribute__((aligned(16))) float Vs[kBcF * D];

    const int tid = threadIdx.x;
    const int units = B * Hq;
    int rb = blockIdx.x / units;
    const int unit = blockIdx.x - rb * units;
    if (CAUSAL) rb = nrb - 1 - rb;
    const int hq = unit % Hq;
    const int b = unit / Hq;
    const int g = hq / (Hq / Hkv);

    const int qi = rb * kRowsF + tid;
    const int off = Nk - Nq;
    const int qpos = off + qi;
    const bool ok = qi < Nq;

    float qv[D];
    {
        const float* qrow = q + (((size_t)b * Hq + hq) * Nq + (ok ? qi : 0)) * D;
        const double2* trow = ROPE ? tab + (size_t)(ok ? qpos : 0) * (D / 2) : nullptr;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += 4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (ok) {
                x = *reinterpret_cast<const float4*>(qrow + d0);
                if (ROPE) x = rope4_f32(x, trow, d0);
            }
            qv[d0] = x.x; qv[d0 + 1] = x.y; qv[d0 + 2] = x.z; qv[d0 + 3] = x.w;
        }
    }
    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    int kend = Nk;
    if (CAUSAL) kend = min(Nk, off + min(Nq, (rb + 1) * kRowsF));
    const float* kbase = k + ((size_t)b * Hkv + g) * (size_t)Nk * D;
    const float* vbase = v + ((size_t)b * Hkv + g) * (size_t)Nk * D;

    const int kbeg = WINDOW ? max(0, off + rb * kRowsF - win + 1) / kBcF * kBcF : 0;
    for (int key0 = kbeg; key0 < kend; key0 += kBcF) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < (kBcF * D / 4) / kRowsF; ++i) {
            const int c = tid + kRowsF * i;
            const int r = c / (D / 4);
            const int col = (c - r * (D / 4)) * 4;
            float4 xk = make_float4(0.f, 0.f, 0.f, 0.f), xv = xk;
            if (key0 + r < Nk) {
                xk = *reinterpret_cast<const float4*>(kbase + (size_t)(key0 + r) * D + col);
                xv = *reinterpret_cast<const float4*>(vbase + (size_t)(key0 + r) * D + col);
            }
            *reinterpret_cast<float4*>(&Ks[r * D + col]) = xk;
            *reinterpret_cast<float4*>(&Vs[r * D + col]) = xv;
        }
        __syncthreads();

        float s[kBcF];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBcF; ++j) {
            float a = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) a = fmaf(qv[d], Ks[j * D + d], a);
            const int key = key0 + j;
            const bool vis = key < Nk && (!CAUSAL || key <= qpos) && (!WINDOW || key > qpos - win);
            s[j] = vis ? a * scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < kBcF; ++j) {
            s[j] = fast_exp2(s[j] - m_use);
            psum += s[j];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float a = acc[d] * alpha;
#pragma unroll
            for (int j = 0; j < kBcF; ++j) a = fmaf(s[j], Vs[j * D + d], a);
            acc[d] = a;
        }
    }
    if (!ok) return;
    const float inv = 1.f / l_run;
    const size_t orow = (((size_t)b * Hq + hq) * Nq + qi) * D;
#pragma unroll
    for (int d0 = 0; d0 < D; d0 += 4) {
        const float4 r = make_float4(acc[d0] * inv, acc[d0 + 1] * inv, acc[d0 + 2] * inv,
                                     acc[d0 + 3] * inv);
        if (o_bf16)  // the fp32 value rounded to the nearest bf16 (even on ties)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + orow + d0) =
                make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
        else
            *reinterpret_cast<float4*>(static_cast<float*>(o) + orow + d0) = r;
    }
    if (lse != nullptr) lse[((size_t)b * Hq + hq) * Nq + qi] = (m_run + fast_log2(l_run)) * kLn2;
}

template <int D, bool CAUSAL, bool ROPE, bool WINDOW>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const int nrb = (a.Nq + kRowsF - 1) / kRowsF;
    const long long nwg = (long long)nrb * a.B * a.Hq;
    if (nwg == 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    prefill_f32_kernel<D, CAUSAL, ROPE, WINDOW><<<(unsigned)nwg, kRowsF, 0, stream>>>(
        static_cast<const float*>(a.q), static_cast<const float*>(a.k),
        static_cast<const float*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, scale_log2,
        a.rope_tab, nrb, WINDOW ? a.window : 0, a.o_bf16);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const bool rope = a.rope_tab != nullptr;
    if (a.window > 0)
        return rope ? launch_t<D, true, true, true>(a, stream) : launch_t<D, true, false, true>(a, stream);
    if (a.causal)
        return rope ? launch_t<D, true, true, false>(a, stream) : launch_t<D, true, false, false>(a, stream);
    return rope ? launch_t<D, false, true, false>(a, stream) : launch_t<D, false, false, false>(a, stream);
}

}  // namespace

hipError_t launch_prefill_f32(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
