// Attention backward for bf16 inputs on gfx950 MFMA.
//
// The forward keeps only the per-row log-sum-exp; the backward recomputes each
// score tile from Q, K and that statistic instead of storing P ("Transformer
// Architecture Deconstructed", recomputation strategy in the backward pass;
// "Attention mechanisms: from alignment to efficient long context", section
// 19).  With P = exp(scale * Q K^T - lse) (masked entries 0) and the upstream
// gradient dO, the gradient of O = P V is
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// the last two using rowsum(P * dP) = dO . O for the softmax Jacobian.
//
// Three kernels:
//   * prep: per query row, dO rounded to bf16 for the matrix cores, D = dO . O
//     (fp32) from that rounded dO, lse converted to the log2 domain.
//   * dK/dV: a workgroup owns 256 keys of one KV head (8 waves x 32 keys; K of
//     a wave held in registers and V in the wave's slice of LDS as MFMA
//     operands, which keeps the wave within 256 registers) and streams
//     64-query tiles of Q and dO of every query head that reads this KV head
//     through LDS (all heads of a tile in a row, tiles in an order that keeps
//     the workgroups of one KV head on the same tile), so the GQA sum over
//     heads happens in the accumulators.  Each tile
//     takes two updates of 32 queries between barriers, so the two waves of a
//     SIMD drift out of phase within a tile; a wave skips an update whose rows
//     see none of its keys (causal).  Per update and wave: S = Q K^T and
//     dP = dO V^T (row-read A operands), then
//     dV += P^T dO and dK += dS^T Q with P and dS straight from the score
//     registers as A operands and dO, Q read with the transposing LDS load.
//   * dQ: 8 waves, 32 query rows each, GQA heads sharing K/V tiles of 64
//     keys: S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T with K read
//     transposed; a wave skips the 32-key halves past its last row (causal).
// In both, the element mask runs only where an update crosses a diagonal or
// the end of K (a wave-uniform branch, applied to the scores in place), and
// the dP accumulator starts from -D, so the products leave dP - D and dS is
// one multiply.
// Both stream their tiles through two LDS buffers with one barrier per tile:
// the next tile is loaded while the current one is computed (dK/dV straight
// into LDS, dQ through registers).
// A tile is read both by rows (16 bytes per lane; 16 lanes per LDS cycle take
// 16 consecutive rows, conflict-free when the row stride is 4 banks mod 64) and
// transposed (a 16-lane group takes 32 bytes of each of four rows, the rows of
// one k-slot group).  The pairing of score rows with tile rows is free as long
// as both operands of a product use the same one, so within each 16-row block
// score row 4a + e is taken from tile row 4e + a (perm16): the four rows of a
// k-slot group are then 4 rows apart, 16 banks apart at that stride, and both
// kinds of read are conflict-free on one copy of the tile.

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kRP = 8;       // row pad (elements) of tiles read by rows: stride = 4 banks mod 64
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Tile row of score row s: within each 16-row block, 4a + e -> 4e + a.
__device__ __forceinline__ int perm16(int s) {
    return (s & ~15) | ((s & 3) << 2) | ((s >> 2) & 3);
}

// Transposed 32x16 operand fragment from a row-major LDS tile whose rows are
// paired with score rows by perm16: lane l gets column c0 + l % 32 of the
// score rows r0 + 4h + {0..3}, r0 + 8 + 4h + {0..3} (h = l / 32), the k-slot
// order in which score accumulators hand over rows, i.e. of the tile rows
// r0 + h + {0, 4, 8, 12} and r0 + 2 + h + {0, 4, 8, 12}.
__device__ __forceinline__ bf16x8 tr_fragment(const uint16_t* tile, int stride, int r0, int c0,
                                              int lane) {
    const int grp = lane >> 4;
    const int w16 = lane & 15;
    const int row = r0 + 4 * (w16 >> 2) + (grp >> 1);
    const int col = c0 + 16 * (grp & 1) + 4 * (w16 & 3);
    const s16x4 lo = lds_read_tr(tile + row * stride + col);
    const s16x4 hi = lds_read_tr(tile + (row + 2) * stride + col);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------------------ prep
template <int D>
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const float* __restrict__ o, const float* __restrict__ dout,
                const float* __restrict__ lse, uint16_t* __restrict__ do16,
                float* __restrict__ dvec, float* __restrict__ lse2, long long rows) {
    constexpr int LPR = D / 8;  // lanes per row, 8 elements each
    const long long gt = blockIdx.x * 256LL + threadIdx.x;
    const long long row = gt / LPR;
    const int c = (int)(gt % LPR) * 8;
    float acc = 0.f;
    if (row < rows) {
        const float4* op = reinterpret_cast<const float4*>(o + row * D + c);
        const float4* dp = reinterpret_cast<const float4*>(dout + row * D + c);
        const float4 o0 = op[0], o1 = op[1], d0 = dp[0], d1 = dp[1];
        u32x4 pk = {pack_bf16x2(d0.x, d0.y), pack_bf16x2(d0.z, d0.w),
                    pack_bf16x2(d1.x, d1.y), pack_bf16x2(d1.z, d1.w)};
        *reinterpret_cast<u32x4*>(do16 + row * D + c) = pk;
        // D from the rounded dO that the products use, so that dP - D is
        // formed from one and the same dO
        const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc += bf16_lo(pk[j]) * ov[2 * j] + bf16_hi(pk[j]) * ov[2 * j + 1];
    }
#pragma unroll
    for (int sh = LPR / 2; sh >= 1; sh >>= 1) acc += __shfl_xor(acc, sh);
    if (row < rows && c == 0) {
        dvec[row] = acc;
        lse2[row] = lse[row] * kLog2e;
    }
}

// ------------------------------------------------------------------ dK, dV
constexpr int kKW = 8;        // waves per dK/dV workgroup (two per SIMD)
constexpr int kKeysW = 32;    // keys per wave
constexpr int kQT = 64;       // queries per tile (two 32-query updates per barrier)
constexpr int kQS = 32;       // queries per update

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kKW * 64, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const uint16_t* __restrict__ do16,
                const float* __restrict__ lse2, const float* __restrict__ dvec,
                float* __restrict__ dk, float* __restrict__ dv, int B, int Hq, int Hkv, int Nq,
                int Nk, float scale_log2, float scale, const double2* __restrict__ tab) {
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    constexpr int RS = D + kRP;  // tile row stride: 4 banks mod 64
    // Tiles go from memory straight into LDS (buffer_load ... lds, 1 KB per
    // instruction), so each tile is a separate object sized to whole
    // instructions: the compiler then knows the loads into one buffer do not
    // alias the reads from the other.
    constexpr int RSZ = (kQT * RS + 511) / 512 * 512;
    __shared__ __attribute__((aligned(16))) uint16_t Qr0[RSZ], Qr1[RSZ], Or0[RSZ], Or1[RSZ];
    auto Qr = [&](int P) -> uint16_t* { return P ? Qr1 : Qr0; };
    auto Or = [&](int P) -> uint16_t* { return P ? Or1 : Or0; };
    __shared__ __attribute__((aligned(16))) float Ls[2][kQT];
    __shared__ __attribute__((aligned(16))) float Dsh[2][kQT];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int G = Hq / Hkv;
    const int off = Nk - Nq;  // query i sits at position off + i

    const int units = B * Hkv;
    const int kb = blockIdx.x / units;  // key block: low blocks see the most queries, go first
    const int unit = blockIdx.x - kb * units;
    const int g = unit % Hkv;
    const int b = unit / Hkv;
    const int k0 = kb * kKW * kKeysW;
    const int kw0 = k0 + wave * kKeysW;

    // K and V of this wave's keys as B operands: key kw0 + l32, d 16s + 8*half .. +7
    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)Nk * D;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k + kvoff), (short)0, Nk * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(v + kvoff), (short)0, Nk * D * 2, 0x00020000);
    // K of this wave's keys in registers; V in this wave's slice of LDS (row
    // stride 4 banks mod 64), read as the B operand of dP = dO V^T
    bf16x8 kf[D / 16];
    __shared__ __attribute__((aligned(16))) uint16_t Vw[kKW][kKeysW * RS];
    uint16_t* vw = Vw[wave];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const int boff = ((kw0 + l32) * D + 16 * s + 8 * half) * 2;
        kf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, boff, 0, 0));
        *reinterpret_cast<u32x4*>(vw + l32 * RS + 16 * s + 8 * half) =
            __builtin_amdgcn_raw_buffer_load_b128(rv, boff, 0, 0);
    }
    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) { dka[i] = f32x16{}; dva[i] = f32x16{}; }

    // The loop runs over (query head of the group, query tile) pairs, the
    // tiles from the first holding a position >= k0 (causal) to the last.
    // Pair it+1 is loaded into the other LDS buffer while pair it is computed
    // (per 32-query update: S and dP, then P and dS, then dV and dK); the
    // buffer parity is a constant in the loop unrolled by two, so every LDS
    // address is a per-lane base plus an immediate; one barrier per pair.  Two waves share each SIMD, so one's
    // vector and LDS work overlaps the other's matrix products.
    const int qstart = CAUSAL ? max(0, k0 - off) / kQT * kQT : 0;
    const int ntq = (Nq - qstart + kQT - 1) / kQT;
    const int niter = G * ntq;
    const int key = kw0 + l32;  // this lane's key (column of the score tile)
    // the first query row that sees this key (past the end of K: none)
    const int qmin = key < Nk ? (CAUSAL ? key - off : 0) : 0x7fffffff;
    struct Pair {
        float l, d;  // this thread's slot of the tile's statistics: lse (log2) and -D
    };
    // One copy of a 32-row tile into LDS: instruction j writes 16-byte slots
    // 64 j .. 64 j + 63, slot s holding row s / SPR, chunk s % SPR of the
    // padded layout (pad slots and the slack past the last row get harmless
    // copies); a wave past the last instruction repeats it.
    auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, uint16_t* dst, int stride, int q0) {
        const int spr = stride / 8;
        const int ninst = (kQT * spr + 63) / 64;
#pragma unroll
        for (int i = 0; i < (kQT * RS / 8 / 64 + kKW) / kKW; ++i) {
            const int j = min(wave + kKW * i, ninst - 1);  // wave-uniform
            const int slot = 64 * j + lane;
            const int rr = slot / spr;
            const int ch = slot - rr * spr;
            const int col = (ch < CPR ? ch : 0) * 8;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(dst + 512 * j), 16,
                ((q0 + rr) * D + col) * 2, 0, 0, 0);
        }
    };
    // Pair it is query head it % G of tile it / G counted from one end: the
    // heads of a tile follow each other, and the tiles are taken so that the
    // workgroups of one KV head read the same tile at about the same time.
    // The first half of the key blocks (one dispatch wave of workgroups at
    // these sizes) all start together, so they run from the last tile down,
    // each stopping at its own first tile.  The second half start one by one
    // as those finish, the last to finish first (it has the fewest tiles), so
    // they run up from their own first tile: a workgroup that starts later
    // starts at a later tile, by as many tiles as its start was delayed.
    // Workgroups go to the eight XCDs in turn, so when B * Hkv is a multiple
    // of 8 those of one KV head share an XCD and its L2, which then serves
    // most of their tile reads: 85% L2 hits against 25% when every workgroup
    // ran up from its own first tile, with 0.8 instead of 3.7 GB fetched from
    // behind the L2 on the causal GQA N = 8192 backward (2.9% less time).
    const int nkb = (Nk + kKW * kKeysW - 1) / (kKW * kKeysW);
    const bool up = kb >= (nkb + 1) / 2;
    auto tile_of = [&](int tq) { return up ? tq : ntq - 1 - tq; };
    auto tile_q0 = [&](int it) { return qstart + tile_of(it / G) * kQT; };
    auto gload = [&](int it, int P, Pair& r) {  // pairs past the last repeat it (never used)
        it = min(it, niter - 1);
        const int tq = it / G;
        const int hh = it - tq * G;
        const int q0 = qstart + tile_of(tq) * kQT;
        const size_t qoff = ((size_t)b * Hq + g * G + hh) * (size_t)Nq;
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(q + qoff * D), (short)0, Nq * D * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(do16 + qoff * D), (short)0, Nq * D * 2, 0x00020000);
        dma(rq, Qr(P), RS, q0);
        dma(ro, Or(P), RS, q0);
        // every thread fetches the statistics of score row tid % 64, i.e. of
        // tile row perm16(tid % 64) (the same value for the same slot, so the
        // stores need no branch).  Buffer loads bounded to this head's rows:
        // rows past Nq read 0, and their lse becomes +inf (P = 2^-inf = 0) by
        // an add, not a select of a load
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(lse2 + qoff), (short)0, Nq * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(dvec + qoff), (short)0, Nq * 4, 0x00020000);
        const int qr = q0 + perm16(lane);
        r.l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, qr * 4, 0, 0)) +
              (qr < Nq ? 0.f : INFINITY);
        r.d = -__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, qr * 4, 0, 0));
    };
    auto store_stats = [&](int buf, const Pair& r) {
        Ls[buf][lane] = r.l;
        Dsh[buf][lane] = r.d;
    };
    // S = Q K^T and dP = dO V^T of one tile: lane holds key column l32 and
    // score rows 8*(i/4) + 4*half + i%4, i.e. the queries of tile rows perm16
    // of those
    const int prow = perm16(l32);  // tile row of this lane's A operand
    auto scores = [&](int buf, int sub, f32x16& sa, f32x16& pa) {
        sa = f32x16{};
        // dP accumulates onto -D, so the products leave dP - D
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dsh[buf][kQS * sub + 8 * j + 4 * half]);
#pragma unroll
            for (int e = 0; e < 4; ++e) pa[4 * j + e] = d4[e];
        }
        const uint16_t* Qb = Qr(buf) + kQS * RS * sub;
        const uint16_t* Ob = Or(buf) + kQS * RS * sub;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&Qb[prow * RS + 16 * s + 8 * half]);
            sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[s], sa, 0, 0, 0);
            const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&Ob[prow * RS + 16 * s + 8 * half]);
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&vw[l32 * RS + 16 * s + 8 * half]);
            pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bv, pa, 0, 0, 0);
        }
    };
    // P and dS of one tile, then dV += P^T dO and dK += dS^T Q over its 32
    // queries (two k-steps)
    auto accumulate = [&](int buf, int sub, int q0, f32x16& sa, const f32x16& pa) {
        // the element mask, only where the update's queries cross this wave's
        // diagonal or its keys run past the end of K (a uniform branch): a
        // hidden pair's score becomes -inf, so its P = 2^-inf = 0
        if (kw0 + kKeysW > Nk || (CAUSAL && q0 + off < kw0 + kKeysW - 1)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qi = q0 + perm16(8 * (i >> 2) + 4 * half + (i & 3));
                sa[i] = qi >= qmin ? sa[i] : -INFINITY;
            }
        }
        uint32_t pw[2][4], dw[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][kQS * sub + 8 * j + 4 * half]);
            float p[4], ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * j + e;
                p[e] = fast_exp2(fmaf(sa[i], scale_log2, -l4[e]));
                ds[e] = p[e] * pa[i];
            }
            pw[j >> 1][2 * (j & 1)] = pack_bf16x2(p[0], p[1]);
            pw[j >> 1][2 * (j & 1) + 1] = pack_bf16x2(p[2], p[3]);
            dw[j >> 1][2 * (j & 1)] = pack_bf16x2(ds[0], ds[1]);
            dw[j >> 1][2 * (j & 1) + 1] = pack_bf16x2(ds[2], ds[3]);
        }
        const uint16_t* Qb = Qr(buf);
        const uint16_t* Ob = Or(buf);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 p4 = {pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]};
            const u32x4 d4 = {dw[ks][0], dw[ks][1], dw[ks][2], dw[ks][3]};
            const bf16x8 pA = __builtin_bit_cast(bf16x8, p4);
            const bf16x8 dA = __builtin_bit_cast(bf16x8, d4);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x8 bo = tr_fragment(Ob, RS, kQS * sub + 16 * ks, 32 * db, lane);
                dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pA, bo, dva[db], 0, 0, 0);
                const bf16x8 bq = tr_fragment(Qb, RS, kQS * sub + 16 * ks, 32 * db, lane);
                dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dA, bq, dka[db], 0, 0, 0);
            }
        }
    };

    // prologue: pair 0 in buffer 0
    auto dma_wait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
    Pair X;
    gload(0, 0, X);
    store_stats(0, X);
    dma_wait();
    __syncthreads();
    auto step = [&](int it, int P) {
        // buffer P^1 held pair it-1, last read before the previous barrier
        gload(it + 1, P ^ 1, X);
        // keep the loads here, a whole pair ahead of their use
        __builtin_amdgcn_sched_barrier(0);
        const int q0 = tile_q0(it);
#pragma unroll
        for (int u = 0; u < kQT / kQS; ++u) {
            // one update at a time: overlapped by the scheduler, two updates
            // no longer fit the registers
            __builtin_amdgcn_sched_barrier(0);
            // skip an update none of whose rows sees a key of this wave
            if (!CAUSAL || q0 + kQS * u + kQS - 1 >= kw0 - off) {
                f32x16 sc, pc;
                scores(P, u, sc, pc);
                accumulate(P, u, q0 + kQS * u, sc, pc);
            }
        }
        store_stats(P ^ 1, X);
        dma_wait();
        __syncthreads();
    };
    int it = 0;
    for (; it + 1 < niter; it += 2) {
        step(it, 0);
        step(it + 1, 1);
    }
    if (it < niter) step(it, 0);

    // lane holds d column 32*db + l32 of key rows kw0 + 8*(i/4) + 4*half + i%4.
    // With RoPE, dK is rotated back here: the pair (2j, 2j+1) of a row sits in
    // lanes l and l ^ 1, which swap values; each computes its own element of
    // the transposed rotation at the key's position.
    float* dkb = dk + kvoff;
    float* dvb = dv + kvoff;
    const bool odd = l32 & 1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kr = kw0 + 8 * (i >> 2) + 4 * half + (i & 3);
            float g = dka[db][i] * scale;
            if (tab != nullptr) {  // uniform
                const float other = __shfl_xor(g, 1);
                const double2 cs = tab[(size_t)min(kr, Nk - 1) * (D / 2) + ((32 * db + l32) >> 1)];
                float r0, r1;
                rope_pair_t_f64(odd ? other : g, odd ? g : other, cs.x, cs.y, r0, r1);
                g = odd ? r1 : r0;
            }
            if (kr < Nk) {
                dkb[(size_t)kr * D + 32 * db + l32] = g;
                dvb[(size_t)kr * D + 32 * db + l32] = dva[db][i];
            }
        }
    }
}

// ------------------------------------------------------------------ dQ
constexpr int kQW = 8;       // waves per dQ workgroup
constexpr int kRows = 32;    // query rows per wave
constexpr int kBc = 64;      // keys per tile
constexpr int kVS = 8;       // V tile row pad (row reads only)

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kQW * 64, 1)
bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ v, const uint16_t* __restrict__ do16,
              const float* __restrict__ lse2, const float* __restrict__ dvec,
              float* __restrict__ dq, int B, int Hq, int Hkv, int Nq, int Nk, float scale_log2,
              float scale, int hpw, int wph, int nchunks, int nrb, const double2* __restrict__ tab) {
    constexpr int NT = kQW * 64;
    constexpr int VS = D + kVS;
    constexpr int CPR = D / 8;
    constexpr int LPT = kBc * CPR / NT;
    static_assert(LPT >= 1 && (kBc * CPR) % NT == 0, "tile/thread mismatch");
    constexpr int RS = D + kRP;
    __shared__ __attribute__((aligned(16))) uint16_t Kr[2][kBc * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBc * VS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int G = Hq / Hkv;

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

    const int row0 = rb * wph * kRows;
    const int qi = row0 + sub * kRows + l32;
    const int off = Nk - Nq;
    const int qpos = off + qi;
    const int klast = CAUSAL ? min(Nk - 1, qpos) : Nk - 1;  // last key this row sees
    // last key any row of this wave sees (causal): later 32-key halves are skipped
    const int wave_klast = off + min(Nq - 1, row0 + sub * kRows + kRows - 1);
    // last key every row of this wave sees (causal): keys up to it need no mask
    const int wave_kfirst = off + row0 + sub * kRows;
    int kend = Nk;
    if (CAUSAL) kend = min(Nk, off + min(Nq, row0 + wph * kRows));
    const int ntiles = (kend + kBc - 1) / kBc;

    // Q and dO of this lane's row as B operands (d 16s + 8*half .. +7), the
    // row's lse (log2) and D
    const bool ok = active && qi < Nq;
    const size_t qrow = ((size_t)b * Hq + hq) * Nq + (ok ? qi : 0);
    bf16x8 qf[D / 16], of[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        uint4 x = *reinterpret_cast<const uint4*>(q + qrow * D + 16 * s + 8 * half);
        uint4 y = *reinterpret_cast<const uint4*>(do16 + qrow * D + 16 * s + 8 * half);
        if (!ok) { x = make_uint4(0, 0, 0, 0); y = x; }
        qf[s] = __builtin_bit_cast(bf16x8, x);
        of[s] = __builtin_bit_cast(bf16x8, y);
    }
    const float lrow = ok ? lse2[qrow] : INFINITY;
    const float drow = ok ? dvec[qrow] : 0.f;
    // dP^T accumulates onto -D (this lane's row), so the products leave dP - D
    f32x16 negd;
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = -drow;

    const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)Nk * D;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k + kvoff), (short)0, Nk * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(v + kvoff), (short)0, Nk * D * 2, 0x00020000);

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

    // tile t+1 is loaded into registers while tile t is computed, then stored
    // into the other LDS buffer; one barrier per tile
    u32x4 pk[LPT], pv[LPT];
    auto gload = [&](int key0) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = tid + NT * i;
            const int r = c / CPR;
            const int col = (c - r * CPR) * 8;
            pk[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((key0 + r) * D + col) * 2, 0, 0);
            pv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((key0 + r) * D + col) * 2, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = tid + NT * i;
            const int r = c / CPR;
            const int col = (c - r * CPR) * 8;
            *reinterpret_cast<u32x4*>(&Kr[buf][r * RS + col]) = pk[i];
            *reinterpret_cast<u32x4*>(&Vs[buf][r * VS + col]) = pv[i];
        }
    };
    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int key0 = t * kBc;
        const int buf = t & 1;
        if (t + 1 < ntiles) gload(key0 + kBc);
        const uint16_t* Krb = Kr[buf];
        const uint16_t* Vt = Vs[buf];
        const int prow = perm16(l32);  // tile row (key) of this lane's A operands
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (CAUSAL && key0 + 32 * kb > wave_klast) break;  // wave-uniform
            // S^T = K Q^T and dP^T = V dO^T for 32 keys: lane holds query l32,
            // score rows 8*(i/4) + 4*half + i%4, i.e. the keys of tile rows
            // key0 + 32kb + perm16 of those
            f32x16 sacc = f32x16{}, pacc = negd;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&Krb[(kb * 32 + prow) * RS + 16 * s + 8 * half]);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[s], sacc, 0, 0, 0);
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Vt[(kb * 32 + prow) * VS + 16 * s + 8 * half]);
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[s], pacc, 0, 0, 0);
            }
            // the element mask, only where these keys cross the diagonal of the
            // wave's first row or run past the end of K (a uniform branch)
            if (key0 + 32 * kb + 31 >= Nk || (CAUSAL && key0 + 32 * kb + 31 > wave_kfirst)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = key0 + kb * 32 + perm16(8 * (i >> 2) + 4 * half + (i & 3));
                    sacc[i] = kk <= klast ? sacc[i] : -INFINITY;
                }
            }
            uint32_t da[2][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float ds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * j + e;
                    const float p = fast_exp2(fmaf(sacc[i], scale_log2, -lrow));
                    ds[e] = p * pacc[i];
                }
                da[j >> 1][2 * (j & 1)] = pack_bf16x2(ds[0], ds[1]);
                da[j >> 1][2 * (j & 1) + 1] = pack_bf16x2(ds[2], ds[3]);
            }
            // dQ^T += K^T dS^T over these 32 keys (two k-steps)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 d4 = {da[ks][0], da[ks][1], da[ks][2], da[ks][3]};
                const bf16x8 dB = __builtin_bit_cast(bf16x8, d4);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 ak = tr_fragment(Krb, RS, kb * 32 + 16 * ks, 32 * db, lane);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, dB, acc[db], 0, 0, 0);
                }
            }
        }
        // the other buffer was last read before the previous barrier
        if (t + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    if (!ok) return;
    // lane holds row qi, d = 32db + 8*i4 + 4*half + 0..3: two whole pairs, which
    // with RoPE are rotated back at the query's position
    float* drow_out = dq + qrow * D;
    const double2* trow = tab != nullptr ? tab + (size_t)qpos * (D / 2) : nullptr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = 32 * db + 8 * i4 + 4 * half;
            float4 r = make_float4(acc[db][4 * i4] * scale, acc[db][4 * i4 + 1] * scale,
                                   acc[db][4 * i4 + 2] * scale, acc[db][4 * i4 + 3] * scale);
            if (trow != nullptr) {  // uniform
                const double2 t0 = trow[d >> 1], t1 = trow[(d >> 1) + 1];
                rope_pair_t_f64(r.x, r.y, t0.x, t0.y, r.x, r.y);
                rope_pair_t_f64(r.z, r.w, t1.x, t1.y, r.z, r.w);
            }
            *reinterpret_cast<float4*>(drow_out + d) = r;
        }
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
    const long long rows = (long long)a.B * a.Hq * a.Nq;
    const long long nprep = (rows * (D / 8) + 255) / 256;
    if (nprep > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    bwd_prep_kernel<D><<<(unsigned)nprep, 256, 0, stream>>>(a.o, a.dout, a.lse, a.do16, a.dvec,
                                                           a.lse2, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);

    const long long nkb = (a.Nk + kKW * kKeysW - 1) / (kKW * kKeysW);
    const long long nwg1 = nkb * a.B * a.Hkv;
    if (nwg1 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.causal)
        bwd_dkdv_kernel<D, true><<<(unsigned)nwg1, kKW * 64, 0, stream>>>(
            a.q, a.k, a.v, a.do16, a.lse2, a.dvec, a.dk, a.dv, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
            scale_log2, a.scale, a.rope_t);
    else
        bwd_dkdv_kernel<D, false><<<(unsigned)nwg1, kKW * 64, 0, stream>>>(
            a.q, a.k, a.v, a.do16, a.lse2, a.dvec, a.dk, a.dv, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
            scale_log2, a.scale, a.rope_t);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int G = a.Hq / a.Hkv;
    const int hpw = G < kQW ? G : kQW;
    const int wph = kQW / hpw;
    const int nchunks = (G + hpw - 1) / hpw;
    const int nrb = (a.Nq + wph * kRows - 1) / (wph * kRows);
    const long long nwg2 = (long long)nrb * a.B * a.Hkv * nchunks;
    if (nwg2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.causal)
        bwd_dq_kernel<D, true><<<(unsigned)nwg2, kQW * 64, 0, stream>>>(
            a.q, a.k, a.v, a.do16, a.lse2, a.dvec, a.dq, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
            scale_log2, a.scale, hpw, wph, nchunks, nrb, a.rope_t);
    else
        bwd_dq_kernel<D, false><<<(unsigned)nwg2, kQW * 64, 0, stream>>>(
            a.q, a.k, a.v, a.do16, a.lse2, a.dvec, a.dq, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
            scale_log2, a.scale, hpw, wph, nchunks, nrb, a.rope_t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.Hq == 0 || a.Nq == 0) return hipSuccess;
    if (a.d == 64) return launch_bwd_d<64>(a, stream);
    if (a.d == 128) return launch_bwd_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
