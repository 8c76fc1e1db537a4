// Tiled exact attention forward for bf16 inputs on gfx950 MFMA.
//
// The method ("Transformer Architecture Breakdown", sections 4.2-4.3;
// "Attention mechanisms: from alignment to efficient long context", section 19):
// a block of query rows stays on chip, K/V tiles stream past it, and each row
// keeps a running max m, running sum l and an output accumulator that is
// rescaled by exp(m_old - m_new) whenever the max grows
// ("coding-interview attention from scratch", section 三.7).  The score tile
// lives only in registers.  The loop runs over query blocks in the outer
// (grid) dimension, the sequence-parallel order the FlashAttention-2 row of the
// comparison table in "Transformer Architecture Breakdown", section 4.3 names.
//
// gfx950 mapping
//   * workgroup = 4 waves; each wave owns 32 query rows of one query head.
//     Waves of one workgroup cover the query heads of one KV head (GQA group),
//     so each K/V tile is read from memory once per group of heads.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator a lane
//     holds one query (column) and 16 keys, so the row max and sum need one
//     exchange between the two 32-lane halves.
//   * O^T += V^T P^T on the same MFMA; P goes from the S accumulator into the B
//     operand without leaving registers (the k-slot order is permuted the same
//     way in both operands).  V is stored transposed in LDS for the A operand.
//   * softmax in the exp2 domain: x = s * scale * log2(e) in fp32.
//   * causal: tiles wholly above a wave's diagonal are skipped, the element mask
//     is applied from the scores' key and query positions; heavy row blocks are
//     launched first.

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32;   // query rows per wave
constexpr int kBc = 64;     // keys per tile
constexpr int kKPad = 8;    // bf16 elements of padding per K row in LDS
constexpr int kVPad = 4;    // bf16 elements of padding per V^T row in LDS

template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(256, 2)
prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, float* __restrict__ o,
                    float* __restrict__ lse, int B, int Hq, int Hkv, int Nq, int Nk,
                    float scale_log2, const double2* __restrict__ tab, int hpw, int wph,
                    int nchunks, int nrb) {
    constexpr int KS = D + kKPad;       // K row stride in LDS (elements)
    constexpr int VS = kBc + kVPad;     // V^T row stride in LDS (elements)
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kBc * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int G = Hq / Hkv;

    // ---- which tile of work this workgroup owns
    const int units = B * Hkv * nchunks;
    int rb = blockIdx.x / units;
    const int unit = blockIdx.x - rb * units;
    if (CAUSAL) rb = nrb - 1 - rb;  // heaviest row blocks first
    const int chunk = unit % nchunks;
    const int bg = unit / nchunks;
    const int g = bg % Hkv;
    const int b = bg / Hkv;

    const int hc = wave / wph;
    const int sub = wave - hc * wph;
    const int hg = chunk * hpw + hc;
    const bool active = (hc < hpw) && (hg < G);
    const int hq = g * G + (active ? hg : 0);

    const int row0 = rb * wph * kRows;                 // first query row of the workgroup
    const int wrow0 = row0 + sub * kRows;              // first query row of this wave
    const int qi = wrow0 + l32;                        // this lane's query row
    const int off = Nk - Nq;                           // position of query i is off + i
    const int qpos = off + qi;

    int kend = Nk;
    if (CAUSAL) kend = min(Nk, off + min(Nq, row0 + wph * kRows));
    const int ntiles = (kend + kBc - 1) / kBc;
    const int wave_last = off + min(Nq - 1, wrow0 + kRows - 1);  // last key this wave may see

    // ---- Q fragment (B operand of S^T = K Q^T): query l32, d = 16s + 8*half .. +7
    bf16x8 qf[D / 16];
    {
        const bool ok = active && qi < Nq;
        const uint16_t* qrow = q + (((size_t)b * Hq + hq) * Nq + (ok ? qi : 0)) * D;
        const double2* trow = ROPE ? tab + (size_t)(ok ? qpos : 0) * (D / 2) : nullptr;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const int d0 = 16 * s + 8 * half;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (ok) {
                x = *reinterpret_cast<const uint4*>(qrow + d0);
                if (ROPE) x = rope8_bf16(x, trow, d0);
            }
            qf[s] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const uint16_t* kbase = k + ((size_t)b * Hkv + g) * (size_t)Nk * D;
    const uint16_t* vbase = v + ((size_t)b * Hkv + g) * (size_t)Nk * D;

    for (int t = 0; t < ntiles; ++t) {
        const int key0 = t * kBc;
        __syncthreads();  // previous tile fully consumed
        // ---- K tile -> LDS, row-major with padding
#pragma unroll
        for (int i = 0; i < (kBc * D / 8) / 256; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (D / 8);
            const int col = (c - r * (D / 8)) * 8;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (key0 + r < Nk) x = *reinterpret_cast<const uint4*>(kbase + (size_t)(key0 + r) * D + col);
            *reinterpret_cast<uint4*>(&Ks[r * KS + col]) = x;
        }
        // ---- V tile -> LDS transposed: thread takes 4 keys x 8 dims
        if (tid < (kBc / 4) * (D / 8)) {
            const int dc = tid % (D / 8);
            const int kg = tid / (D / 8);
            uint32_t w[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 4 * kg + r;
                uint4 x = make_uint4(0, 0, 0, 0);
                if (key < Nk) x = *reinterpret_cast<const uint4*>(vbase + (size_t)key * D + dc * 8);
                w[r][0] = x.x; w[r][1] = x.y; w[r][2] = x.z; w[r][3] = x.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = (e & 1) ? 16 : 0;
                const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xffff;
                const uint32_t a1 = (w[1][e >> 1] >> sh) & 0xffff;
                const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xffff;
                const uint32_t a3 = (w[3][e >> 1] >> sh) & 0xffff;
                uint2 pk = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
                *reinterpret_cast<uint2*>(&Vt[(dc * 8 + e) * VS + 4 * kg]) = pk;
            }
        }
        __syncthreads();

        if (!active) continue;
        if (CAUSAL && key0 > wave_last) continue;  // whole tile above this wave's diagonal

        // ---- S^T = K Q^T : two 32-key blocks
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + l32) * KS + 16 * s + 8 * half]);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
            }
        }

        // ---- scale, mask, online softmax (exp2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                float x = sacc[kb][i] * scale_log2;
                const bool vis = (key < Nk) && (!CAUSAL || key <= qpos);
                x = vis ? x : -INFINITY;
                sacc[kb][i] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(sacc[kb][i] - m_use);
                sacc[kb][i] = p;
                psum += p;
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                uint4 pw;
                pw.x = pack_bf16x2(sacc[kb][8 * ss + 0], sacc[kb][8 * ss + 1]);
                pw.y = pack_bf16x2(sacc[kb][8 * ss + 2], sacc[kb][8 * ss + 3]);
                pw.z = pack_bf16x2(sacc[kb][8 * ss + 4], sacc[kb][8 * ss + 5]);
                pw.w = pack_bf16x2(sacc[kb][8 * ss + 6], sacc[kb][8 * ss + 7]);
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
                const int kk = kb * 32 + 16 * ss + 4 * half;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const uint16_t* vrow = &Vt[(32 * db + l32) * VS];
                    const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kk);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vrow + kk + 8);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
                }
            }
        }
    }

    if (!active || qi >= Nq) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    float* orow = o + (((size_t)b * Hq + hq) * Nq + qi) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = 32 * db + 8 * i4 + 4 * half;
            float4 r = make_float4(oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv,
                                   oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
            *reinterpret_cast<float4*>(orow + d) = r;
        }
    }
    if (lse != nullptr && half == 0)
        lse[((size_t)b * Hq + hq) * Nq + qi] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool ROPE>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    const int hpw = G < kWaves ? G : kWaves;          // query heads per workgroup
    const int wph = kWaves / hpw;                      // waves per head
    const int nchunks = (G + hpw - 1) / hpw;
    const int rows_per_wg = wph * kRows;
    const int nrb = (a.Nq + rows_per_wg - 1) / rows_per_wg;
    const long long nwg = (long long)nrb * a.B * a.Hkv * nchunks;
    if (nwg == 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    prefill_bf16_kernel<D, CAUSAL, ROPE><<<(unsigned)nwg, 256, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
        static_cast<const uint16_t*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, scale_log2,
        a.rope_tab, hpw, wph, nchunks, nrb);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const bool rope = a.rope_tab != nullptr;
    if (a.causal) return rope ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
    return rope ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
