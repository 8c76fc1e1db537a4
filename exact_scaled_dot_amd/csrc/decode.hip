// Decode: T new query tokens per sequence against a contiguous KV cache.
//
// With T = 1 the new query attends to every cached key with no mask
// ("coding-interview attention from scratch", section 三.6).  With T > 1 (the
// same page, section 八 question 5: verifying several drafted tokens at once)
// the cache already holds the new tokens' K/V and new token t, at position
// len - T + t, sees cache rows 0 .. len - T + t: the whole history plus a lower
// triangle over the new rows.  Decode reads every cached K/V row
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
// gfx950 mapping of the split kernel (one KV head, up to 16 query columns,
// 2048 keys, 1024 for a paged cache: 256 or 128 per wave, 8 waves).  A column is one (query head, new token)
// pair; the G*T columns of a KV head are G*T consecutive rows of q, so they
// are numbered in that order and each keeps its own last visible key:
//   * each wave streams its K rows and then its V rows in 32-key batches
//     through a ring of four register slots (three batches always in flight,
//     V loads start while the last K batches are in use); every load reads
//     whole 256-byte rows and is unconditional, so the compiler keeps the
//     batches in flight.
//   * S = K q^T on v_mfma_f32_16x16x32_bf16 with the cached keys as rows and
//     the KV head's query columns as columns, so each K row is read once for
//     all queries that share it.  K rows go through a wave-private LDS slice;
//     for MFMA step s the four lanes holding one key read its d range
//     [32s, 32s + 32) there, and q uses the same d-slot order.  All scores of a
//     wave stay in registers, so the per-column max is exact and nothing is
//     rescaled.
//   * V goes through a wave-private LDS slice and O = P V runs on the same
//     MFMA: P (bf16) comes straight from the score registers as the A operand,
//     the V operand is read with the transposing LDS load ds_read_b64_tr_b16.  O is normalised by the sum of the rounded
//     weights (v_dot2c_f32_bf16), the log-sum by the fp32 sum.
//   * the eight waves' partial states are merged in LDS with the same rule the
//     merge kernel uses, giving one partial state per chunk.  (At 1024 keys
//     per chunk the fp32 partial states of a 4-token decode cost 5% of the
//     cache bytes; at 2048 half that, and one-token decode is unchanged.  The
//     paged kernel keeps 1024: at 2048 its per-block load resources spill.)
//   * paged cache ("Attention mechanisms: from alignment to efficient long
//     context", section 20; "Transformer Architecture Breakdown", Paged
//     Attention): the pools are [num_blocks, Hkv, block_size, d] and token p of
//     sequence b lives in block table[b][p / block_size] at row p % block_size.
//     One load instruction covers 4 (d = 128) or 8 (d = 64) consecutive keys,
//     which never straddle a block of 16 or more rows, so each instruction gets
//     a scalar buffer resource whose base is its block and whose size is the
//     block's rows below the sequence length: rows past the end read as zeros,
//     as in the contiguous case, and the loads stay unconditional.  A wave
//     fetches its (at most eight) table entries once, one per lane, and picks
//     each instruction's entry with v_readlane.

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kSplitWaves = 8;          // waves per split workgroup
// Cache policy of the K/V loads: non-temporal (the nt bit of the buffer load).
// Every cache row is read exactly once per call, so keeping it out of L2 and
// the Infinity Cache costs nothing, and the stream then runs at 6.2 instead of
// 5.5 TB/s (same bytes, same results).
constexpr int kStream = 2;
constexpr int kBatch = 32;              // keys per streamed batch

__device__ __forceinline__ float sum_bf16x2(uint32_t two, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, two), one, acc, false);
}

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Order this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int GP, bool PAGED>
__global__ void __launch_bounds__(kSplitWaves * 64)
decode_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ lens,
                    float* __restrict__ ws_o, float* __restrict__ ws_lse, int B, int Hq,
                    int Hkv, int T, int max_len, float scale_log2, int nchunks, int nhch,
                    const double2* __restrict__ tab, const int32_t* __restrict__ table,
                    int max_blocks, int lbs, int num_blocks) {
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(GP >= 1 && GP <= 16, "columns per workgroup");
    constexpr int kCh = decode_chunk(PAGED);          // keys per workgroup
    constexpr int kWaveKeys = kCh / kSplitWaves;      // keys per wave
    constexpr int kNB = kWaveKeys / kBatch;           // batches per wave
    static_assert(kWaveKeys <= 64 * 16, "a wave's table entries fit its lanes (blocks >= 16)");
    constexpr int NS = D / 32;          // QK MFMA k-steps over d
    constexpr int NDB = D / 16;         // PV output blocks of 16 dims
    constexpr int VSD = D + 16;         // V row stride in LDS: 8 banks mod 64
    constexpr int KSD = D + 8;          // K row stride in LDS: 4 banks mod 64
    constexpr int NW = kSplitWaves;
    __shared__ __attribute__((aligned(16))) uint16_t Vl[NW][kBatch * VSD];
    __shared__ float cm[NW][16], cl[NW][16], cr[NW][16], cw[NW][16];
    __shared__ float co[NW][GP][D];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int quarter = lane >> 4;

    // Chunk-major order: all first chunks of every (sequence, KV head) come first,
    // so the workgroups past a sequence's end (which exit at once) are not
    // interleaved with the heavy ones.
    const int per_c = B * Hkv * nhch;
    const int c = blockIdx.x / per_c;
    int idx = blockIdx.x - c * per_c;
    const int hch = idx % nhch;
    idx /= nhch;
    const int g = idx % Hkv;
    const int b = idx / Hkv;
    const int G = Hq / Hkv;
    const int NC = G * T;                        // columns of this KV head
    const int f0 = hch * GP;                     // first column of this workgroup
    const size_t row0 = ((size_t)b * Hq + (size_t)g * G) * T + f0;  // its q / output row
    const int nh = min(GP, NC - f0);             // columns handled here

    int len = lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int k0 = c * kCh;
    if (k0 >= len) return;
    // last key visible to this lane's column (r16): its own position
    const int lim = len - T + (f0 + min(r16, nh - 1)) % T;

    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)max_len * D;
    const uint16_t* kb = k + kvoff;
    const uint16_t* vb = v + kvoff;
    const int wk0 = k0 + wave * kWaveKeys;                   // first key of this wave
    const int wn = max(0, min(kWaveKeys, lim + 1 - wk0));    // keys this column sees here

    // paged: lane i holds the physical block of this wave's i-th block of keys
    // (indices past the sequence's last block repeat that block; entries are
    // clamped into the pool)
    int ent = 0;
    if constexpr (PAGED) {
        const int nblk = (len + (1 << lbs) - 1) >> lbs;  // >= 1: len > k0 >= 0
        ent = table[(size_t)b * max_blocks + min((wk0 >> lbs) + lane, nblk - 1)];
        ent = min(max(ent, 0), num_blocks - 1);
    }

    // ---- one stream per wave: K batches 0..kNB-1, then V batches 0..kNB-1, each
    //      32 keys x D bf16 = VPL 16-byte pieces per lane, through a ring of
    //      NSLOT register slots, so NSLOT-1 batches are in flight (V loads start
    //      while the last K batches are still being used).
    constexpr int VPL = kBatch * (D / 8) / 64;
    static_assert(VPL == 2 * NS, "a K batch and a V batch fill the same slot");
    constexpr int NSLOT = 4;
    u32x4 ring[NSLOT][VPL];
    // Piece j of batch bi (K or V): key 32*bi + (lane + 64j) / (D/8),
    // d 8*((lane + 64j) % (D/8)): every load instruction reads whole rows.
    // Buffer loads: the base sits in a scalar resource whose size is the
    // sequence's valid rows, a lane only holds a 32-bit offset, and rows past
    // the end come back as zeros (finite data; their scores are masked to
    // -inf, so their weights are exactly 0).  The loads are unconditional, so
    // the compiler can count them in flight.
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kb), (short)0, len * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vb), (short)0, len * D * 2, 0x00020000);
    const int lane_off = (lane / (D / 8)) * D * 2 + (lane % (D / 8)) * 16;  // bytes
    constexpr int KPJ = 64 / (D / 8);                                         // keys per j
    constexpr int JSTEP = KPJ * D * 2;                                        // bytes per j
    auto sload = [&](int e, int slot) {
        const int bi = e < kNB ? e : e - kNB;
        if constexpr (PAGED) {
            const uint16_t* pool = e < kNB ? k : v;
            // one resource per 16 keys (the smallest block), shared by the
            // JPG load instructions that cover them
            constexpr int JPG = 16 / KPJ;
#pragma unroll
            for (int gi = 0; gi < VPL / JPG; ++gi) {
                const int key = wk0 + kBatch * bi + 16 * gi;  // first key of the group
                const int ks = key & -(1 << lbs);             // first key of its block
                const int phys = __builtin_amdgcn_readlane(ent, (key >> lbs) - (wk0 >> lbs));
                const int nvalid = min(max(len - ks, 0), 1 << lbs);
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t*>(pool + ((size_t)phys * Hkv + g) * ((size_t)D << lbs)),
                    (short)0, nvalid * D * 2, 0x00020000);
#pragma unroll
                for (int jj = 0; jj < JPG; ++jj)
                    ring[slot][gi * JPG + jj] = __builtin_amdgcn_raw_buffer_load_b128(
                        r, (key - ks) * D * 2 + JSTEP * jj + lane_off, 0, kStream);
            }
        } else {
            const int boff = (wk0 + kBatch * bi) * D * 2 + lane_off;
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                ring[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(e < kNB ? rk : rv, boff + JSTEP * j, 0, kStream);
        }
    };
#pragma unroll
    for (int e = 0; e < NSLOT - 1; ++e) sload(e, e);

    // ---- q operand (B of S = K q^T): column r16, d-slots 32s + 8*quarter ..
    //      (columns past the last one read a valid row and are zeroed).  With
    //      RoPE the query is rotated at its own position (cached keys are stored
    //      rotated); a column without keys (lim < 0) uses position 0, unread.
    bf16x8 qf[NS];
    {
        const bool ok = r16 < nh;
        const uint16_t* qrow = q + (row0 + min(r16, nh - 1)) * D;
        const double2* trow = tab + (size_t)max(lim, 0) * (D / 2);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 x = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * quarter);
            if (tab != nullptr) x = rope8_bf16(x, trow, 32 * s + 8 * quarter);
            if (!ok) x = make_uint4(0, 0, 0, 0);
            qf[s] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- pass over K: scores.  Lane holds head r16, keys 32*bi + 16*grp + 4*quarter + i.
    //      K rows go through the wave's LDS slice (row stride D + 8: 4 banks apart,
    //      so the 16-byte operand reads of 16 rows hit distinct banks).
    uint16_t* vl = Vl[wave];
    float sc[kNB][8];
#pragma unroll
    for (int bi = 0; bi < kNB; ++bi) {
        __builtin_amdgcn_sched_barrier(0);  // keep each batch's loads where the ring puts them
        sload(bi + NSLOT - 1, (bi + NSLOT - 1) % NSLOT);
        wave_lds_sync();  // the previous batch's operand reads are done
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int cc = lane + 64 * j;
            const int kr = cc / (D / 8);
            *reinterpret_cast<u32x4*>(vl + kr * KSD + (cc - kr * (D / 8)) * 8) = ring[bi % NSLOT][j];
        }
        wave_lds_sync();
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 kx = *reinterpret_cast<const u32x4*>(vl + (16 * grp + r16) * KSD + 32 * s + 8 * quarter);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx), qf[s], acc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kBatch * bi + 16 * grp + 4 * quarter + i;
                sc[bi][4 * grp + i] = key < wn ? acc[i] : -INFINITY;
            }
        }
    }

    // ---- exact per-head max of this wave, weights, sums
    float mx = -INFINITY;
#pragma unroll
    for (int bi = 0; bi < kNB; ++bi)
#pragma unroll
        for (int j = 0; j < 8; j += 2) mx = fmaxf(mx, fmaxf(sc[bi][j], sc[bi][j + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m2 = mx * scale_log2;                  // -inf when the wave has no key
    const float neg = (m2 == -INFINITY) ? 0.f : -m2;
    float lsum = 0.f, rsum = 0.f;
    uint4 pa[kNB];
#pragma unroll
    for (int bi = 0; bi < kNB; ++bi) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(fmaf(sc[bi][j], scale_log2, neg));
            lsum += p[j];
        }
        pa[bi].x = pack_bf16x2(p[0], p[1]);
        pa[bi].y = pack_bf16x2(p[2], p[3]);
        pa[bi].z = pack_bf16x2(p[4], p[5]);
        pa[bi].w = pack_bf16x2(p[6], p[7]);
        rsum = sum_bf16x2(pa[bi].x, rsum);
        rsum = sum_bf16x2(pa[bi].y, rsum);
        rsum = sum_bf16x2(pa[bi].z, rsum);
        rsum = sum_bf16x2(pa[bi].w, rsum);
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);

    // ---- pass over V: O = P V.  Lane output: head 4*quarter + i, dim 16*db + r16.
    f32x4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};
    const int w16 = lane & 15;
    const int trow = 4 * quarter + (w16 >> 2);  // key row this lane addresses
    const int tcol = 4 * (w16 & 3);
#pragma unroll
    for (int bi = 0; bi < kNB; ++bi) {
        const int e = kNB + bi;
        __builtin_amdgcn_sched_barrier(0);
        if (e + NSLOT - 1 < 2 * kNB) sload(e + NSLOT - 1, (e + NSLOT - 1) % NSLOT);
        wave_lds_sync();  // previous batch's reads are done before it is overwritten
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int cc = lane + 64 * j;
            const int kr = cc / (D / 8);
            const int col = (cc - kr * (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(vl + kr * VSD + col) = ring[e % NSLOT][j];
        }
        wave_lds_sync();
        const bf16x8 a = __builtin_bit_cast(bf16x8, pa[bi]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const uint16_t* vp = vl + trow * VSD + 16 * db + tcol;
            const s16x4 lo = lds_read_tr(vp);
            const s16x4 hi = lds_read_tr(vp + 16 * VSD);
            const bf16x8 bv = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, oacc[db], 0, 0, 0);
        }
    }

    // ---- merge the eight waves' states in LDS
    if (quarter == 0) {
        cm[wave][r16] = m2;
        cl[wave][r16] = lsum;
        cr[wave][r16] = rsum;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * quarter + i;
        if (h < GP) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) co[wave][h][16 * db + r16] = oacc[db][i];
        }
    }
    __syncthreads();
    // per column: the common max, each wave's weight divided by the merged
    // denominator, and the chunk's lse (one thread per column)
    if (tid < nh) {
        const int h = tid;
        float M = cm[0][h];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, cm[w][h]);
        float f[NW];
        float rs = 0.f, ls = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            // 0 for a wave without keys for this column
            f[w] = cm[w][h] == -INFINITY ? 0.f : fast_exp2(cm[w][h] - M);
            rs = fmaf(f[w], cr[w][h], rs);
            ls = fmaf(f[w], cl[w][h], ls);
        }
        // a column with no key in this chunk (a new token before it) gets the
        // empty state (weights 0, lse -inf); the merge kernel never reads it
        const bool empty = M == -INFINITY;
        const float inv = empty ? 0.f : 1.f / rs;
#pragma unroll
        for (int w = 0; w < NW; ++w) cw[w][h] = f[w] * inv;
        ws_lse[(row0 + h) * nchunks + c] = empty ? -INFINITY : M + fast_log2(ls);
    }
    __syncthreads();
    // The partial outputs go out with the non-temporal hint: while the cache
    // stream saturates HBM, a workgroup's plain stores keep it alive for
    // microseconds after its last load (measured: 16 columns per KV head
    // 459 -> 440 us for the decode batch, bit-identical).
    for (int i = tid; i < nh * D; i += NW * 64) {
        const int h = i / D;
        const int d = i - h * D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc = fmaf(cw[w][h], co[w][h][d], acc);
        __builtin_nontemporal_store(acc, &ws_o[((row0 + h) * nchunks + c) * D + d]);
    }
}

// One workgroup (256 threads) per output row (sequence, query head, new
// token).  Only the chunks holding keys the row can see are merged.  The chunk
// weights w_c = 2^(lse2_c - M) are formed in parallel over chunks; then thread
// t sums dim t % D over every (256 / D)-th chunk and the partial sums meet in
// LDS.
template <int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    const int32_t* __restrict__ lens, void* __restrict__ o,
                    float* __restrict__ lse, int Hq, int T, int max_len, int nchunks,
                    int kCh, int o_bf16) {
    constexpr int NSPLIT = 256 / D;
    __shared__ float wts[1024];
    __shared__ float red[8];
    __shared__ float part[NSPLIT][D];
    const int bh = blockIdx.x;  // output row
    const int b = bh / (Hq * T);
    const int t = bh % T;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int len = lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int nvis = max(0, len - T + t + 1);  // keys 0 .. len-T+t
    const int nc = (nvis + kCh - 1) / kCh;
    // O as fp32, or rounded to the nearest bf16 (even on ties)
    auto store_o = [&](int dd, float x) {
        if (o_bf16) {
            static_cast<uint16_t*>(o)[(size_t)bh * D + dd] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
        } else {
            static_cast<float*>(o)[(size_t)bh * D + dd] = x;
        }
    };
    if (nc == 0) {  // no visible key: empty sum
        if (tid < D) store_o(tid, 0.f);
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
    int c = j;
    for (; c + 7 * NSPLIT < nc; c += 8 * NSPLIT) {  // eight loads in flight
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = orow[(size_t)(c + u * NSPLIT) * D + d];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int cu = c + u * NSPLIT;
            acc = fmaf(cu < 1024 ? wts[cu] : fast_exp2(lrow[cu] - M), x[u], acc);
        }
    }
    for (; c < nc; c += NSPLIT) {
        const float w = c < 1024 ? wts[c] : fast_exp2(lrow[c] - M);
        acc = fmaf(w, orow[(size_t)c * D + d], acc);
    }
    part[j][d] = acc;
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < NSPLIT; ++i) t += part[i][tid];
        store_o(tid, t / wsum);
        if (lse != nullptr && tid == 0) lse[bh] = (M + fast_log2(wsum)) * kLn2;
    }
}

template <int D, int GP, bool PAGED>
hipError_t launch_split(const DecodeArgs& a, float scale_log2, hipStream_t stream) {
    const long long NC = (long long)(a.Hq / a.Hkv) * a.T;
    const long long nhch = (NC + GP - 1) / GP;
    const long long nwg = (long long)a.nchunks * nhch * a.Hkv * a.B;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    decode_split_kernel<D, GP, PAGED><<<(unsigned)nwg, kSplitWaves * 64, 0, stream>>>(
        a.q, a.k, a.v, a.lens, a.ws_o, a.ws_lse, a.B, a.Hq, a.Hkv, a.T, a.max_len, scale_log2,
        a.nchunks, (int)nhch, a.rope_tab, a.table, a.max_blocks, a.block_log2, a.num_blocks);
    return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_split_gp(const DecodeArgs& a, float scale_log2, hipStream_t stream) {
    const long long NC = (long long)(a.Hq / a.Hkv) * a.T;  // columns per KV head
    if (NC == 1) return launch_split<D, 1, PAGED>(a, scale_log2, stream);
    if (NC == 2) return launch_split<D, 2, PAGED>(a, scale_log2, stream);
    if (NC <= 4) return launch_split<D, 4, PAGED>(a, scale_log2, stream);
    if (NC <= 8) return launch_split<D, 8, PAGED>(a, scale_log2, stream);
    return launch_split<D, 16, PAGED>(a, scale_log2, stream);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const hipError_t e = a.table ? launch_split_gp<D, true>(a, scale_log2, stream)
                                 : launch_split_gp<D, false>(a, scale_log2, stream);
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.Hq * a.T;
    if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    decode_merge_kernel<D><<<(unsigned)rows, 256, 0, stream>>>(
        a.ws_o, a.ws_lse, a.lens, a.o, a.lse, a.Hq, a.T, a.max_len, a.nchunks, a.chunk, a.o_bf16);
    return hipGetLastError();
}

}  // namespace

// ---- the allocation-free decode entry point's partial states
//
// One fixed array per device holds the split kernel's partial states for
// attn_decode_noalloc, so that call needs no allocation.  Host code never
// passes the array's name to a kernel (on the host it only stands in for the
// symbol); it uses the device address that hipGetSymbolAddress returns, once
// per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    try {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_ptr[dev] == nullptr) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev] = p;
        }
        *ptr = g_scratch_ptr[dev];
    } catch (...) {
        return hipErrorUnknown;
    }
    return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.Hq == 0) return hipSuccess;
    if (a.d == 64) return launch_decode_d<64>(a, stream);
    if (a.d == 128) return launch_decode_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
