// Decode: one query token per sequence against a contiguous KV cache.
//
// Each new query attends to every cached key with no mask ("coding-interview
// attention from scratch", section 三.6).  Decode reads every cached K/V row
// once per step, so it is bound by memory bandwidth ("Transformer Architecture
// Breakdown", Key Topic 3).  To spread one sequence over many compute units the
// cache is split along its length: a split workgroup turns one chunk of keys
// into a partial state (max and sum in the exp2 domain folded into
// lse2 = m + log2 l, and the chunk-normalised O), and a merge kernel combines
// the partials of a row exactly with the two-part rule of "Transformer
// Architecture Breakdown", section 4.2 (and "Transformer Architecture
// Deconstructed", online softmax), generalised to any number of parts:
//   M = max_c lse2_c,  w_c = 2^(lse2_c - M),  O = sum_c w_c O_c / sum_c w_c,
//   lse = (M + log2 sum_c w_c) * ln 2.
//
// gfx950 mapping of the split kernel (256 keys, one KV head, GP query heads):
//   * S = K q^T on v_mfma_f32_16x16x32_bf16: A = 16 cached keys, B = the query
//     heads of the group (columns), so every K row is read from memory once and
//     serves all heads that share it.  For MFMA step s the four lanes that hold
//     one key read its d range [32s, 32s + 32) (64 contiguous bytes); the same
//     d-slot order is used for q, so the dot products are unchanged.
//   * P V on the vector ALU: V rows stream in 16-byte pieces, weights come from
//     LDS as broadcasts; partial sums are reduced across lanes, then waves.

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kCh = kDecodeChunk;  // keys per workgroup
constexpr int kKeysPerWave = kCh / 4;

template <int D, int GP>
__global__ void __launch_bounds__(256)
decode_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ lens,
                    float* __restrict__ ws_o, float* __restrict__ ws_lse, int B, int Hq,
                    int Hkv, int max_len, float scale_log2, int nchunks, int nhch) {
    static_assert(D == 64 || D == 128, "head dim");
    constexpr int NS = D / 32;          // MFMA k-steps over d
    constexpr int NDC = D / 8;          // 16-byte pieces per row
    constexpr int NKS = 64 / NDC;       // key slots per wave in the PV loop
    __shared__ float Pl[kCh][GP];
    __shared__ float redm[4][16];
    __shared__ float reds[4][16];
    __shared__ float accs[4][GP][D];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int quarter = lane >> 4;

    int idx = blockIdx.x;
    const int c = idx % nchunks;
    idx /= nchunks;
    const int hch = idx % nhch;
    idx /= nhch;
    const int g = idx % Hkv;
    const int b = idx / Hkv;
    const int G = Hq / Hkv;
    const int h0 = g * G + hch * GP;             // first query head of this workgroup
    const int nh = min(GP, G - hch * GP);        // heads handled here

    int len = lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int k0 = c * kCh;
    if (k0 >= len) return;

    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)max_len * D;
    const uint16_t* kb = k + kvoff;
    const uint16_t* vb = v + kvoff;
    const int wk0 = k0 + wave * kKeysPerWave;    // first key of this wave

    // ---- issue all K and V loads of this wave's keys
    uint4 kf[4][NS];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        const int key = wk0 + 16 * grp + r16;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (key < len) x = *reinterpret_cast<const uint4*>(kb + (size_t)key * D + 32 * s + 8 * quarter);
            kf[grp][s] = x;
        }
    }
    const int dc = lane % NDC;
    const int ks = lane / NDC;
    uint4 vf[kKeysPerWave / NKS];
#pragma unroll
    for (int it = 0; it < kKeysPerWave / NKS; ++it) {
        const int key = wk0 + ks + NKS * it;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (key < len) x = *reinterpret_cast<const uint4*>(vb + (size_t)key * D + 8 * dc);
        vf[it] = x;
    }

    // ---- q operand: column r16 = head, k-slots 8*quarter.. = d 32s + 8*quarter ..
    bf16x8 qf[NS];
    {
        const bool ok = r16 < nh;
        const uint16_t* qrow = q + ((size_t)b * Hq + h0 + (ok ? r16 : 0)) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (ok) x = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * quarter);
            qf[s] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- scores: lane holds head r16, keys 16*grp + 4*quarter + i
    float sc[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        f32x4 acc = f32x4{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[grp][s]), qf[s], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = wk0 + 16 * grp + 4 * quarter + i;
            const float x = key < len ? acc[i] * scale_log2 : -INFINITY;
            sc[grp][i] = x;
            mx = fmaxf(mx, x);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lane < 16) redm[wave][lane] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(redm[0][r16], redm[1][r16]), fmaxf(redm[2][r16], redm[3][r16]));
    // M is finite: key k0 < len is visible in every workgroup that runs
    float ls = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(sc[grp][i] - M);
            ls += p;
            if (r16 < GP) Pl[wave * kKeysPerWave + 16 * grp + 4 * quarter + i][r16] = p;
        }
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (lane < 16) reds[wave][lane] = ls;
    __syncthreads();  // Pl and reds complete

    // ---- P V on the vector ALU: lane takes 8 dims (dc) of keys ks, ks+NKS, ...
    float acc[GP][8];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int it = 0; it < kKeysPerWave / NKS; ++it) {
        const int kl = wave * kKeysPerWave + ks + NKS * it;
        float pw[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) pw[h] = Pl[kl][h];
        const uint32_t w[4] = {vf[it].x, vf[it].y, vf[it].z, vf[it].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const float x0 = bf16_lo(w[e2]);
            const float x1 = bf16_hi(w[e2]);
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                acc[h][2 * e2] = fmaf(pw[h], x0, acc[h][2 * e2]);
                acc[h][2 * e2 + 1] = fmaf(pw[h], x1, acc[h][2 * e2 + 1]);
            }
        }
    }
    // reduce over the key slots of a wave (lanes sharing dc)
#pragma unroll
    for (int sh = NDC; sh < 64; sh <<= 1) {
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], sh);
    }
    if (ks == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) accs[wave][h][8 * dc + e] = acc[h][e];
    }
    __syncthreads();
    // ---- combine the 4 waves and write the chunk's partial state
    for (int i = tid; i < nh * D; i += 256) {
        const int h = i / D;
        const int d = i - h * D;
        const float lsum = reds[0][h] + reds[1][h] + reds[2][h] + reds[3][h];
        const float ov = (accs[0][h][d] + accs[1][h][d] + accs[2][h][d] + accs[3][h][d]) / lsum;
        const size_t row = ((size_t)b * Hq + h0 + h) * nchunks + c;
        ws_o[row * D + d] = ov;
        if (d == 0) {
            const float Mh = fmaxf(fmaxf(redm[0][h], redm[1][h]), fmaxf(redm[2][h], redm[3][h]));
            ws_lse[row] = Mh + fast_log2(lsum);
        }
    }
}

// One workgroup (256 threads) per (sequence, query head).  The chunk weights
// w_c = 2^(lse2_c - M) are formed in parallel over chunks; then thread t sums
// dim t % D over every (256 / D)-th chunk and the partial sums meet in LDS.
template <int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    const int32_t* __restrict__ lens, float* __restrict__ o,
                    float* __restrict__ lse, int Hq, int max_len, int nchunks) {
    constexpr int NSPLIT = 256 / D;
    __shared__ float wts[1024];
    __shared__ float red[8];
    __shared__ float part[NSPLIT][D];
    const int bh = blockIdx.x;
    const int b = bh / Hq;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int len = lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int nc = (len + kCh - 1) / kCh;
    if (nc == 0) {  // no visible key: empty sum
        if (tid < D) o[(size_t)bh * D + tid] = 0.f;
        if (lse != nullptr && tid == 0) lse[bh] = -INFINITY;
        return;
    }
    const float* lrow = ws_lse + (size_t)bh * nchunks;
    const float* orow = ws_o + (size_t)bh * nchunks * D;
    // max over chunks
    float M = -INFINITY;
    for (int c = tid; c < nc; c += 256) M = fmaxf(M, lrow[c]);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    // weights and their sum (chunks beyond the LDS buffer are re-read below)
    float ws = 0.f;
    for (int c = tid; c < nc; c += 256) {
        const float w = fast_exp2(lrow[c] - M);
        if (c < 1024) wts[c] = w;
        ws += w;
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) ws += __shfl_xor(ws, sh);
    if (lane == 0) red[4 + wave] = ws;
    __syncthreads();
    const float wsum = red[4] + red[5] + red[6] + red[7];
    const int d = tid % D;
    const int j = tid / D;
    float acc = 0.f;
    for (int c = j; c < nc; c += NSPLIT) {
        const float w = c < 1024 ? wts[c] : fast_exp2(lrow[c] - M);
        acc = fmaf(w, orow[(size_t)c * D + d], acc);
    }
    part[j][d] = acc;
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < NSPLIT; ++i) t += part[i][tid];
        o[(size_t)bh * D + tid] = t / wsum;
        if (lse != nullptr && tid == 0) lse[bh] = (M + fast_log2(wsum)) * kLn2;
    }
}

template <int D, int GP>
hipError_t launch_split(const DecodeArgs& a, float scale_log2, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    const int nhch = (G + GP - 1) / GP;
    const long long nwg = (long long)a.nchunks * nhch * a.Hkv * a.B;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    decode_split_kernel<D, GP><<<(unsigned)nwg, 256, 0, stream>>>(
        a.q, a.k, a.v, a.lens, a.ws_o, a.ws_lse, a.B, a.Hq, a.Hkv, a.max_len, scale_log2,
        a.nchunks, nhch);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const int G = a.Hq / a.Hkv;
    hipError_t e;
    if (G == 1) e = launch_split<D, 1>(a, scale_log2, stream);
    else if (G == 2) e = launch_split<D, 2>(a, scale_log2, stream);
    else if (G <= 4) e = launch_split<D, 4>(a, scale_log2, stream);
    else if (G <= 8) e = launch_split<D, 8>(a, scale_log2, stream);
    else e = launch_split<D, 16>(a, scale_log2, stream);
    if (e != hipSuccess) return e;
    decode_merge_kernel<D><<<(unsigned)(a.B * a.Hq), 256, 0, stream>>>(
        a.ws_o, a.ws_lse, a.lens, a.o, a.lse, a.Hq, a.max_len, a.nchunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.Hq == 0) return hipSuccess;
    if (a.d == 64) return launch_decode_d<64>(a, stream);
    if (a.d == 128) return launch_decode_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
