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
//   * workgroup = 8 waves, two per SIMD; at d = 128 each wave owns 64 query
//     rows of one query head as two 32-row blocks (at d = 64, one block of 32).
//     Every K and V operand a wave reads from LDS feeds the products of both
//     blocks, and the 512 query rows of a workgroup share each K/V tile: half
//     the LDS operand reads and three quarters of the tile loads per product of
//     one 32-row block per wave with three waves per SIMD.  The waves of a
//     workgroup cover query heads of one KV head (GQA group), so a tile is read
//     from memory once per group of heads.  The O accumulators of both blocks
//     and the Q operands of the first stay in registers; the second block's Q
//     rows sit in the wave's slice of LDS (256 registers per wave would not
//     hold both).  Each wave runs a plain sequence per 32 keys (scores, mask,
//     max, rescale, weights, P V for both blocks); the two blocks' independent
//     chains and the other wave of the SIMD give the overlap of matrix and
//     vector work.
//   * K/V tiles of 64 keys are double-buffered in LDS.  The tiles arrive
//     straight from memory (buffer_load ... lds) while the previous tile is
//     used, with one barrier per tile; each tile takes two online-softmax
//     updates of 32 keys.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator a lane
//     holds one query (column) and 16 keys, so a row lives in two lanes, one in
//     each 32-lane half.  The halves exchange their maxima only when one of
//     them may move the row's reference (below), and their sums at the end.
//   * O^T += V^T P^T on the same MFMA; P goes from the S accumulator into the B
//     operand without leaving registers (the k-slot order is permuted the same
//     way in both operands).  V stays row-major in LDS and the A operand is
//     read with the gfx950 transposing LDS load (ds_read_b64_tr_b16).
//   * softmax in the exp2 domain: p = 2^(s * scale * log2(e) - m) with one FMA
//     and one v_exp_f32 per score.  The reference max m of a row moves only when
//     the row max exceeds it by more than 8 (a factor 2^8), so most updates skip
//     the rescale of O and l; O and l always share one reference, so the result
//     is the same exact recurrence.  A lane tests its own 16 scores against the
//     threshold, and only when some lane of the wave passes it is the row max
//     formed across the halves and the reference moved.  O is divided by the sum of the bf16-rounded
//     weights that entered the P V product (a true convex combination of V
//     rows); the logsumexp uses the fp32 sum.
//   * causal: a workgroup stops at the last tile its rows can see, a wave skips
//     32-key blocks past its last row, the element mask is applied only on
//     blocks that cross a wave's diagonal or the end of K, and heavy row blocks
//     are launched first.
//   * sliding window w ("Attention mechanisms: from alignment to efficient long
//     context", section 11; causal only): a query at position p sees keys
//     p-w+1 .. p, so a workgroup also starts at the first tile its first row
//     can see, and blocks that cross a wave's lower window edge are masked too.
//     Work per row is then O(w) instead of O(N).

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// waves per workgroup: two per SIMD (256 registers each at d = 128)
template <int D>
constexpr int waves_for() { return 8; }
// 32-row query blocks per wave: two at d = 128, so each K and V operand read
// from LDS feeds two products; one at d = 64, so that a workgroup of one query
// head covers 256 rows and short sequences still give many workgroups
template <int D>
constexpr int blocks_for() { return D == 128 ? 2 : 1; }
constexpr int kRows = 32;   // query rows per wave
constexpr int kBc = 64;     // keys per tile
constexpr int kKPad = 8;    // K rows: stride = 4 banks mod 64, conflict-free 16-byte operand reads
constexpr int kVPad = 32;   // V rows: stride = 16 banks mod 64, conflict-free transposed reads
constexpr float kLazy = 8.f;  // keep the reference max until a row max exceeds it by 2^8

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t two, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, two), one, acc, false);
}

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
}

template <int D, bool CAUSAL, bool ROPE, bool WINDOW>
__global__ void __launch_bounds__(waves_for<D>() * 64, 1)
prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, void* __restrict__ o,
                    float* __restrict__ lse, int B, int Hq, int Hkv, int Nq, int Nk,
                    float scale_log2, const double2* __restrict__ tab, int hpw, int wph,
                    int nchunks, int nrb, int win, int o_bf16) {
    static_assert(!WINDOW || CAUSAL, "the sliding window is built for causal attention");
    constexpr int kWaves = waves_for<D>();
    constexpr int NB = blocks_for<D>();
    constexpr int WR = kRows * NB;      // query rows per wave
    constexpr int KS = D + kKPad;       // K row stride in LDS (elements)
    constexpr int VS = D + kVPad;       // V row stride in LDS (elements)
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    // one object per buffer, so the compiler knows that the tile loads into
    // one buffer do not alias the reads from the other
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[kBc * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[kBc * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[kBc * VS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs1[kBc * VS];
    auto kbuf = [&](int P) -> uint16_t* { return P ? Ks1 : Ks0; };
    auto vbuf = [&](int P) -> uint16_t* { return P ? Vs1 : Vs0; };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    const int row0 = rb * wph * WR;                    // first query row of the workgroup
    const int wrow0 = row0 + sub * WR;                 // first query row of this wave
    const int off = Nk - Nq;                           // position of query i is off + i
    int qi[NB], qpos[NB], blk_first[NB], blk_lo[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        qi[nb] = wrow0 + 32 * nb + l32;                // this lane's query row in block nb
        qpos[nb] = off + qi[nb];
        blk_first[nb] = off + wrow0 + 32 * nb;
        blk_lo[nb] = off + min(Nq - 1, wrow0 + 32 * nb + 31) - win + 1;
    }

    int kend = Nk;
    if (CAUSAL) kend = min(Nk, off + min(Nq, row0 + wph * WR));
    // window: the first key any row of the workgroup sees, rounded down to a tile
    const int kbeg = WINDOW ? max(0, off + row0 - win + 1) / kBc * kBc : 0;
    const int ntiles = (kend - kbeg + kBc - 1) / kBc;
    const int wave_last = off + min(Nq - 1, wrow0 + WR - 1);  // last key this wave may see

    const uint16_t* kbase = k + ((size_t)b * Hkv + g) * (size_t)Nk * D;
    const uint16_t* vbase = v + ((size_t)b * Hkv + g) * (size_t)Nk * D;

    // ---- tile loads: memory straight into LDS (buffer_load ... lds).  One
    //      instruction writes lane L's 16 bytes at its LDS base + 16 L, so a
    //      padded tile is filled in 16-byte slots, slot s holding row s / SPR,
    //      chunk s % SPR; the pad slot of a row receives a copy of its first
    //      chunk.  The scalar resource spans this head's Nk rows, so rows past
    //      the end read as zeros and no load needs a branch.
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kbase), (short)0, Nk * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vbase), (short)0, Nk * D * 2, 0x00020000);
    auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, uint16_t* dstbuf, int stride, int key0) __attribute__((always_inline)) {
        static_assert(kBc == 64, "one load instruction per 64 slots = per slot column");
        const int spr = stride / 8;  // 16-byte slots per padded row
        const int ninst = spr;       // kBc rows x spr slots / 64 lanes
        // no branch: a wave past the last instruction repeats it, writing the
        // same bytes to the same slots
#pragma unroll
        for (int i = 0; i < (ninst + kWaves - 1) / kWaves; ++i) {
            const int j = min(wave + kWaves * i, ninst - 1);  // wave-uniform
            const int slot = 64 * j + lane;
            const int r = slot / spr;
            const int ch = slot - r * spr;
            const int col = (ch < CPR ? ch : 0) * 8;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(dstbuf + 512 * j), 16,
                ((key0 + r) * D + col) * 2, 0, 0, 0);
        }
    };
    auto dma_wait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

    // ---- Q fragment (B operand of S^T = K Q^T): query l32, d = 16s + 8*half .. +7
    // Q of block 0 in registers; of block 1 (if any) in this wave's LDS slice
    // (row stride 4 banks mod 64: conflict-free 16-byte reads), written once
    // here and read by this wave only (before any read the prologue barrier
    // has passed)
    constexpr int QS = D + kKPad;
    __shared__ __attribute__((aligned(16))) uint16_t Qw[NB > 1 ? kWaves * 32 * QS : 8];
    uint16_t* qw = Qw + (NB > 1 ? wave * 32 * QS : 0);
    bf16x8 qf[D / 16];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const bool ok = active && qi[nb] < Nq;
        const uint16_t* qrow = q + (((size_t)b * Hq + hq) * Nq + (ok ? qi[nb] : 0)) * D;
        const double2* trow = ROPE ? tab + (size_t)(ok ? qpos[nb] : 0) * (D / 2) : nullptr;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const int d0 = 16 * s + 8 * half;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (ok) {
                x = *reinterpret_cast<const uint4*>(qrow + d0);
                if (ROPE) x = rope8_bf16(x, trow, d0);
            }
            if (nb == 0)
                qf[s] = __builtin_bit_cast(bf16x8, x);
            else
                *reinterpret_cast<uint4*>(qw + l32 * QS + d0) = x;
        }
    }

    f32x16 oacc[NB][D / 32];
    float m_run[NB], l_run[NB], r_run[NB], neg_m[NB], grow_at[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[nb][i] = f32x16{};
        m_run[nb] = -INFINITY;   // reference max (log2 domain) of this lane's row
        l_run[nb] = 0.f;         // this lane's share of the row sum (fp32 weights): for lse
        r_run[nb] = 0.f;         // same sum of the bf16-rounded weights the MFMA used: for O
        neg_m[nb] = 0.f;         // -m (0 while m is -inf)
        grow_at[nb] = -INFINITY; // raw row max above which the reference moves
    }

    // transposed-read addressing for the V operand (A of O^T += V^T P^T)
    const int grp = lane >> 4;          // 16-lane group
    const int w16 = lane & 15;
    const int vrow_in = w16 >> 2;       // which of 4 keys this lane addresses
    const int vcol_in = 16 * (grp & 1) + 4 * (w16 & 3);
    const int vkey_h = 4 * (grp >> 1);  // = 4 * half

    // ---- the pieces of an online-softmax update over 32 keys (forced inline:
    //      left as calls, the blocks' accumulators would live in memory)
    // the element mask of block x for the 32 keys from key0 (a uniform branch:
    // only blocks that cross the diagonal, the window edge or the end of K)
    auto mask = [&](int x, f32x16& s, int key0) __attribute__((always_inline)) {
        const bool need_mask = (key0 + 32 > Nk) || (CAUSAL && key0 + 31 > blk_first[x]) ||
                               (WINDOW && key0 < blk_lo[x]);
        if (need_mask) {
            keep_branch();
            // element i holds key kl + c_i with c_i = 8 (i / 4) + i % 4
            const int kl = key0 + 4 * half;
            const int hi = (CAUSAL ? min(qpos[x], Nk - 1) : Nk - 1) - kl;
            const int lo = WINDOW ? qpos[x] - win + 1 - kl : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int ci = 8 * (i >> 2) + (i & 3);
                const bool vis = ci <= hi && (!WINDOW || ci >= lo);
                s[i] = vis ? s[i] : -INFINITY;
            }
        }
    };
    // max of the 16 scores a lane holds: a tree of three-input maxima (depth 3)
    auto lanemax = [&](const f32x16& s) __attribute__((always_inline)) {
        const float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
        const float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
        const float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
        const float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
        const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
        return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
    };
    // the row max from the two halves' maxima: v_permlane32_swap gives lanes
    // 0-31 (r[0]) and lanes 32-63 (r[1]) in both halves, with no LDS round trip
    auto rowmax = [&](float mx) __attribute__((always_inline)) {
        const unsigned u = __builtin_bit_cast(unsigned, mx);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        // opaque to the optimiser: left visible, the max of the two results
        // is folded into the first one alone
        unsigned lo = r[0], hi = r[1];
        asm volatile("" : "+v"(lo), "+v"(hi));
        return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
    };
    // weights p = 2^(s scale log2(e) - m), their fp32 sum (pairwise), their
    // bf16 packing and the sum of the packed values (two chains)
    auto expo = [&](int x, const f32x16& sc, uint4 (&pw)[2]) __attribute__((always_inline)) {
        float lsum[2], rsum[2];
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(sc[8 * ss + e], scale_log2, neg_m[x]));
            lsum[ss] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            pw[ss].x = pack_bf16x2(p[0], p[1]);
            pw[ss].y = pack_bf16x2(p[2], p[3]);
            pw[ss].z = pack_bf16x2(p[4], p[5]);
            pw[ss].w = pack_bf16x2(p[6], p[7]);
            rsum[ss] = sum_bf16x2(pw[ss].w, sum_bf16x2(pw[ss].z, sum_bf16x2(pw[ss].y, sum_bf16x2(pw[ss].x, 0.f))));
        }
        l_run[x] += lsum[0] + lsum[1];
        r_run[x] += rsum[0] + rsum[1];
    };
    f32x16 sc[NB];
    uint4 pw[NB][2];
    // S_x^T = K Q_x^T for every block x; each K operand feeds all of them
    auto qk_all = [&](const uint16_t* Kt) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sc[nb] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kt[l32 * KS + 16 * s + 8 * half]);
            sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[0], 0, 0, 0);
            if constexpr (NB > 1) {
                const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&qw[l32 * QS + 16 * s + 8 * half]);
                sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, sc[1], 0, 0, 0);
            }
        }
    };
    // O_x^T += V^T P_x^T for every block x; each V operand feeds all of them
    auto pv_all = [&](const uint16_t* Vt) __attribute__((always_inline)) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int kbase_l = 16 * ss + vkey_h + vrow_in;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const uint16_t* vp = Vt + kbase_l * VS + 32 * db + vcol_in;
                const s16x4 lo = lds_read_tr(vp);
                const s16x4 hi = lds_read_tr(vp + 8 * VS);
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    oacc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        a, __builtin_bit_cast(bf16x8, pw[nb][ss]), oacc[nb][db], 0, 0, 0);
            }
        }
    };
    // the weights of every block for the 32 keys from key0: masks, then the
    // row maxima of all blocks, one rescale decision for all of them (a block
    // whose reference does not move takes alpha = 1), then all weights, so
    // the independent chains of the blocks interleave
    auto sm_all = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mask(nb, sc[nb], key0);
        // a lane's own half of a row decides whether the wave takes the rescale
        // path; only there is the row max formed across the halves, so that
        // both halves of a row move their reference together
        float mx[NB];
        bool any = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            mx[nb] = lanemax(sc[nb]);
            any = any || mx[nb] > grow_at[nb];
        }
        if (__ballot(any)) {
            keep_branch();
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                mx[nb] = rowmax(mx[nb]);
                const bool grow = mx[nb] > grow_at[nb];
                const float m_new = grow ? mx[nb] * scale_log2 : m_run[nb];
                const float alpha = grow ? fast_exp2(m_run[nb] - m_new) : 1.f;
                l_run[nb] *= alpha;
                r_run[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[nb][db] *= alpha;
                m_run[nb] = m_new;
                neg_m[nb] = (m_new == -INFINITY) ? 0.f : -m_new;
                grow_at[nb] = (m_new + kLazy) / scale_log2;
            }
        }
        // the weights are the one long stretch of pure vector work: the wave
        // raises its issue priority for it, so the other wave of the SIMD gets
        // the matrix cores around it
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) expo(nb, sc[nb], pw[nb]);
        __builtin_amdgcn_s_setprio(0);
    };
    // One online-softmax update over 32 keys held in LDS (rows Kt, Vt) for
    // the wave's row blocks; tile t (64 keys in buffer P = t & 1, a constant
    // at every call) takes two of them while K/V(t+1) arrive in the other
    // buffer.
    auto step = [&](int t, int P) __attribute__((always_inline)) {
        const int key0 = kbeg + t * kBc;
        // K/V(t+1) replace K/V(t-1), last read before the previous barrier
        dma(rk, kbuf(P ^ 1), KS, key0 + kBc);
        dma(rv, vbuf(P ^ 1), VS, key0 + kBc);
        qk_all(kbuf(P));
        sm_all(key0);
        pv_all(vbuf(P));
        // the second half is skipped when no key of it is visible to any row of
        // the wave (causal tail, end of K)
        if (key0 + 32 < Nk && (!CAUSAL || key0 + 32 <= wave_last)) {
            qk_all(kbuf(P) + 32 * KS);
            sm_all(key0 + 32);
            pv_all(vbuf(P) + 32 * VS);
        }
        dma_wait();
        __syncthreads();
    };
    dma(rk, Ks0, KS, kbeg);
    dma(rv, Vs0, VS, kbeg);
    dma_wait();
    __syncthreads();
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(t, 0);
        step(t + 1, 1);
    }
    if (t < ntiles) step(t, 0);

    if (!active) return;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if (qi[nb] >= Nq) continue;
        // O is the convex combination with the weights the MFMA actually used
        // (their bf16 roundings), so it is normalised by their sum; lse uses the
        // fp32 sum.
        const float l_tot = l_run[nb] + __shfl_xor(l_run[nb], 32);
        const float r_tot = r_run[nb] + __shfl_xor(r_run[nb], 32);
        const float inv = 1.f / r_tot;
        const size_t orow = (((size_t)b * Hq + hq) * Nq + qi[nb]) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d = 32 * db + 8 * i4 + 4 * half;
                float4 r = make_float4(oacc[nb][db][4 * i4 + 0] * inv, oacc[nb][db][4 * i4 + 1] * inv,
                                       oacc[nb][db][4 * i4 + 2] * inv, oacc[nb][db][4 * i4 + 3] * inv);
                if (o_bf16)
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + orow + d) =
                        make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
                else
                    *reinterpret_cast<float4*>(static_cast<float*>(o) + orow + d) = r;
            }
        }
        if (lse != nullptr && half == 0)
            lse[((size_t)b * Hq + hq) * Nq + qi[nb]] = (m_run[nb] + fast_log2(l_tot)) * kLn2;
    }
}

template <int D, bool CAUSAL, bool ROPE, bool WINDOW>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    // query heads per workgroup: the largest common divisor of the group size
    // and the wave count, so every wave of a workgroup has rows to work on
    int hpw = 1;
    constexpr int kWaves = waves_for<D>();
    for (int c = 1; c <= kWaves; ++c)
        if (kWaves % c == 0 && G % c == 0) hpw = c;
    const int wph = kWaves / hpw;                      // waves per head
    const int nchunks = (G + hpw - 1) / hpw;
    const int rows_per_wg = wph * kRows * blocks_for<D>();
    const int nrb = (a.Nq + rows_per_wg - 1) / rows_per_wg;
    const long long nwg = (long long)nrb * a.B * a.Hkv * nchunks;
    if (nwg == 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    prefill_bf16_kernel<D, CAUSAL, ROPE, WINDOW><<<(unsigned)nwg, kWaves * 64, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
        static_cast<const uint16_t*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, scale_log2,
        a.rope_tab, hpw, wph, nchunks, nrb, WINDOW ? a.window : 0, a.o_bf16);
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

hipError_t launch_prefill_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, stream);
    if (a.d == 128) return launch_d<128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
