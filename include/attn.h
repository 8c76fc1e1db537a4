/*
 * attn.h - exact scaled-dot-product attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so.  Every entry point takes plain device pointers, sizes
 * and a HIP stream, returns an attn_status and never throws.  Work is queued
 * asynchronously on `stream`; no entry point synchronises the device.
 *
 * What is computed (page titles, sections):
 *   O = softmax(scale * Q K^T + M) V with M = 0 (no mask) or the causal mask
 *   (minus infinity above the diagonal), per query head, as in
 *   "Transformer Architecture Breakdown", section 1.2 and Key Topic 5, and
 *   "Attention mechanisms: from alignment to efficient long context", Notation.
 *   The score matrix is processed in tiles with the online-softmax recurrence
 *   (running max, running sum, rescaled accumulator: "Transformer Architecture
 *   Breakdown", section 4.2; "coding-interview attention from scratch", 三.7),
 *   so it never reaches device memory.
 *
 * Layouts (all contiguous, head dimension fastest, 64-bit offsets inside):
 *   q   [B, Hq,  Nq, d]      k, v [B, Hkv, Nk, d]     (dtype of the call)
 *   o   [B, Hq,  Nq, d] fp32 lse  [B, Hq, Nq] fp32 natural-log logsumexp
 *   (the chunked-prefill and multi-token decode calls can store O as bf16)
 *   Query head h reads KV head h / (Hq / Hkv): MHA (Hkv = Hq), GQA, MQA
 *   (Hkv = 1) ("coding-interview attention from scratch", 三.4).
 *
 * Causal alignment: query i sits at position Nk - Nq + i, key j at j; key j is
 * visible to query i iff j <= Nk - Nq + i (the bottom-right alignment the
 * from-scratch page gives for t new tokens over a cache, section 八 question 5).
 * Causal calls need Nq <= Nk, so no row is fully masked.
 *
 * RoPE (rope_base > 0): adjacent pairs (x_2j, x_2j+1) of Q and K rotate by
 * position * theta_j, theta_j = rope_base^(-2j/d) ("Transformer Architecture
 * Breakdown", section 3.1; "coding-interview attention from scratch", 三.5);
 * V is not rotated.  The rotation is evaluated in fp64 (cos/sin from the C
 * library) and rounded to the input dtype (fp64 -> fp32 -> bf16, nearest-even)
 * before the product, so the result is the attention of the rounded rotated
 * operands.
 *
 * RoPE positions must be below 2^22 (4,194,304; larger ones return
 * ATTN_ERR_UNSUPPORTED): every K row range attn_fwd accepts at d = 128.
 *
 * Ownership: the caller owns every buffer, including workspaces.  The library
 * keeps one device table of fp64 cos/sin per (device, rope_base, d) covering
 * positions 0 .. P - 1, P the largest position count asked for so far rounded
 * up to a power of two (at least 1024; P * d / 2 * 16 bytes, at most 4 GiB at
 * d = 128).  It is built on the first RoPE call that needs it, or a longer
 * one: the host evaluates it with the C library in pieces of at most 16 MB and
 * uploads them with blocking copies (hipMalloc, hipMemcpy).  Such a call made
 * while its stream is being captured into a graph returns ATTN_ERR_HIP before
 * any allocation, so code that captures makes one RoPE call of the longest
 * length beforehand.  Older tables stay allocated until exit (kernels queued
 * earlier may still read them).
 * Entry points are thread-safe; calls that share a workspace must be ordered by
 * the caller (same stream or events).
 *
 * The *_workspace_bytes queries return 0 when the call needs no workspace or
 * an argument they read is out of range (a size below 1, a dtype the call does
 * not take), and SIZE_MAX where the size does not fit in size_t; no workspace
 * matches that, so such a call fails (ATTN_ERR_WORKSPACE, unless an argument
 * check before the workspace check fails first).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_BF16 = 0, /* bfloat16 inputs (bits in uint16 storage) */
    ATTN_F32 = 1   /* float32 inputs */
} attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,     /* bad argument: null pointer, negative size, Hq % Hkv,
                                 causal, windowed or RoPE call with Nq > Nk,
                                 non-finite scale, misaligned pointer (16 bytes
                                 needed), scale <= 0, window < 1 ... */
    ATTN_ERR_UNSUPPORTED = 2, /* valid but not built: d not in {64, 128}, f32 decode,
                                 a decode cache row range of 2 GiB or more */
    ATTN_ERR_HIP = 3,         /* a HIP call or kernel launch failed */
    ATTN_ERR_WORKSPACE = 4    /* workspace missing or smaller than required */
} attn_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_str(int status);

/* Bytes of workspace attn_fwd needs: B*Hkv*Nk*d elements of the input dtype
 * for the rotated K when rope_base > 0, else 0. */
size_t attn_fwd_workspace_bytes(int B, int Hkv, int Nk, int d, float rope_base,
                                attn_dtype dtype);

/*
 * Prefill / full attention forward.
 *   q, k, v     device pointers, layouts above, element type `dtype`.
 *   o           device fp32 [B,Hq,Nq,d], written.
 *   lse         device fp32 [B,Hq,Nq] or NULL; natural-log logsumexp of each
 *               row's visible scaled scores.
 *   B, Hq, Hkv, Nq, Nk, d   sizes; B = 0, Hq = 0 or Nq = 0 is a no-op.
 *               Hkv >= 1, Hq % Hkv == 0, Nk >= 1, d in {64, 128}.
 *   causal      0 or 1.
 *   scale       finite multiplier of Q K^T, > 0 (1/sqrt(d) for standard attention).
 *   rope_base   0 = no RoPE, else a finite base > 0; RoPE needs Nq <= Nk
 *               (query positions Nk - Nq + i are then >= 0).
 *   workspace   device buffer of attn_fwd_workspace_bytes(...) bytes (may be
 *               NULL when that is 0); holds the rotated K during the call.
 * All validation happens on the host before any HIP call.
 */
int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
             float scale, float rope_base, attn_dtype dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Causal sliding-window attention forward ("Attention mechanisms: from
 * alignment to efficient long context", section 11): a query at position p
 * sees the keys at positions p - window + 1 .. p (and never one past p), so
 * each row costs O(window) instead of O(Nk).  Positions follow the causal
 * bottom-right alignment above (query i at Nk - Nq + i).  Every row sees at
 * least its own position, so no row is empty.
 *   window      >= 1; a window of Nk or more keys equals attn_fwd(causal = 1).
 *   Other arguments, layouts, workspace and errors as attn_fwd with causal = 1
 *   (Nq <= Nk required).
 */
int attn_fwd_window(const void* q, const void* k, const void* v, float* o, float* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, int window,
                    float scale, float rope_base, attn_dtype dtype,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked prefill against a KV cache ("coding-interview attention from
 * scratch", section 八 question 5: Nq new tokens over a cache whose last Nq rows
 * are their own K/V; the score block is all visible over the earlier rows and
 * lower-triangular over the new ones).  Query i sits at position Nk - Nq + i
 * and sees keys 0 .. Nk - Nq + i (attn_fwd's causal bottom-right rule).  The
 * cached keys are used as given: with RoPE they are stored already rotated
 * (as attn_decode_multi assumes), and only the queries are rotated, each at its
 * own position, exactly as attn_fwd rotates Q.  So attn_prefill_cached on keys
 * from attn_rope_apply(k, rope_base, 0) equals attn_fwd(causal = 1) on k, bit
 * for bit (it runs the same attention kernel, without the rotation pass of K).
 *   q          device [B, Hq, Nq, d], dtype.
 *   k_cache, v_cache  device [B, Hkv, Nk, d], dtype; Nq <= Nk.
 *   o          device [B, Hq, Nq, d]: fp32 when o_dtype = ATTN_F32, bf16 when
 *              ATTN_BF16 (each element the fp32 result rounded to the nearest
 *              bf16, ties to even).
 *   lse        device fp32 [B, Hq, Nq] or NULL.
 *   scale, rope_base, dtype: as attn_fwd.  No workspace is needed.
 * Errors as attn_fwd with causal = 1; an unknown o_dtype is ATTN_ERR_INVALID.
 */
int attn_prefill_cached(const void* q, const void* k_cache, const void* v_cache, void* o,
                        float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        float rope_base, attn_dtype dtype, attn_dtype o_dtype, hipStream_t stream);

/* Bytes of workspace attn_bwd needs: dO in bf16 and two fp32 values per query
 * row, plus the rotated Q and K (bf16) when rope_base > 0; 0 for fp32. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, float rope_base,
                                attn_dtype dtype);

/*
 * Backward pass of attn_fwd: the gradients of L = sum(dout * O) with respect
 * to q, k and v.  The score tiles are recomputed from q, k and the forward's
 * lse instead of being stored ("Transformer Architecture Deconstructed",
 * recomputation strategy in the backward pass; "Attention mechanisms: from
 * alignment to efficient long context", section 19).  With P the attention
 * weights (masked entries 0):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),
 *   dQ = scale * dS K,  dK = scale * dS^T Q,
 * summed over the query heads that share a KV head.  With RoPE the gradients
 * are taken with respect to the rows before rotation (the rounding of the
 * rotated rows counts as the identity).
 *   q, k, v    device bf16, as given to attn_fwd (dtype must be ATTN_BF16).
 *   o, lse     device fp32 [B,Hq,Nq,d], [B,Hq,Nq]: attn_fwd's outputs for the
 *              same arguments.
 *   dout       device fp32 [B,Hq,Nq,d] upstream gradient; rounded to bf16 for
 *              the matrix products.
 *   dq         device fp32 [B,Hq,Nq,d];  dk, dv  device fp32 [B,Hkv,Nk,d]
 *              (written, not accumulated).
 *   causal, scale, rope_base  as attn_fwd.
 *   workspace  device buffer of attn_bwd_workspace_bytes(...) bytes, 256-byte
 *              aligned.
 * Errors as attn_fwd; ATTN_F32 returns ATTN_ERR_UNSUPPORTED.
 */
int attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const float* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, int causal, float scale, float rope_base, attn_dtype dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace attn_decode needs for partial (max/sum, O) states. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int d);

/*
 * Decode: one query per sequence against a contiguous KV cache, no mask, no
 * RoPE (cached keys are stored already rotated), as in "coding-interview
 * attention from scratch", 三.6.  The cache is split along its length; every
 * chunk yields a partial (max, sum, O) state and a second kernel merges them
 * exactly ("Transformer Architecture Breakdown", section 4.2 merge rule).
 *   q          device [B, Hq, d] bf16.
 *   k_cache, v_cache  device [B, Hkv, max_len, d] bf16; sequence b uses rows
 *              0 .. seq_lens[b]-1; rows past that are never read.
 *   seq_lens   device int32 [B]; values are clamped to [0, max_len].  A length
 *              of 0 yields O = 0 and lse = -inf.
 *   o          device fp32 [B, Hq, d];  lse  device fp32 [B, Hq] or NULL.
 *   workspace  device buffer of attn_decode_workspace_bytes(...) bytes.
 * dtype must be ATTN_BF16 (ATTN_F32 returns ATTN_ERR_UNSUPPORTED); one
 * sequence's K (or V) rows, max_len * d * 2 bytes, must stay under 2 GiB.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seq_lens, float* o, float* lse,
                int B, int Hq, int Hkv, int max_len, int d, float scale,
                attn_dtype dtype, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* Capacity of the static per-device array behind attn_decode_noalloc. */
#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)

/*
 * attn_decode without a workspace argument, for callers that cannot allocate
 * device memory at call time: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments (minus the
 * workspace), arithmetic, results (bit for bit) and errors as attn_decode.
 * The partial states live in one static array of ATTN_DECODE_NOALLOC_MAX_BYTES
 * per device, part of the library's code object and held until the process
 * ends; the call allocates nothing.
 *   Limit: attn_decode_workspace_bytes(B, Hq, Hkv, max_len, d) must be at most
 *   ATTN_DECODE_NOALLOC_MAX_BYTES (e.g. B = 32, Hq = 32, max_len = 32768,
 *   d = 128 needs 8.5 MB); larger sizes return ATTN_ERR_WORKSPACE before any
 *   HIP call.
 *   Sharing: every call on one device uses the same array and leaves its
 *   contents behind (nothing in it needs to start at zero: the merge reads
 *   only partial states the same call wrote).  Calls whose work overlaps on
 *   one device (other streams, other threads, overlapping graph replays)
 *   race on the array and give wrong results; order them.
 * The first call on a device looks up the array's device address once
 * (hipGetSymbolAddress); later calls make no HIP call besides the launches.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, float* o, float* lse,
                        int B, int Hq, int Hkv, int max_len, int d, float scale,
                        attn_dtype dtype, hipStream_t stream);

/* Bytes of workspace attn_decode_multi needs: B*Hq*T*ceil(max_len/2048)
 * partial states of d + 1 floats (256-byte aligned split). */
size_t attn_decode_multi_workspace_bytes(int B, int Hq, int Hkv, int T, int max_len, int d);

/*
 * Multi-token decode: T new query tokens per sequence against a contiguous KV
 * cache that already holds their K/V, as when several drafted tokens are
 * verified at once ("coding-interview attention from scratch", section 八
 * question 5: the t x (len + t) score block is all visible over the history and
 * lower-triangular over the new tokens).  With n = seq_lens[b] (clamped to
 * [0, max_len]) new token t sits at position n - T + t and sees cache rows
 * 0 .. n - T + t; a token whose position is negative (n < T) sees no key and
 * gets O = 0, lse = -inf.  T = 1 with rope_base = 0 is attn_decode.
 *   q          device [B, Hq, T, d] bf16.
 *   k_cache, v_cache  device [B, Hkv, max_len, d] bf16, keys stored already
 *              rotated when RoPE is used; rows past seq_lens[b] are never read.
 *   seq_lens   device int32 [B].
 *   o          device [B, Hq, T, d]: fp32 when o_dtype = ATTN_F32, bf16 when
 *              ATTN_BF16 (the fp32 result rounded to the nearest bf16, ties to
 *              even; tokens without keys get 0).
 *   lse        device fp32 [B, Hq, T] or NULL.
 *   rope_base  0 = queries used as given, else each query is rotated at its
 *              own position (fp64, rounded to bf16) as attn_fwd rotates Q.
 *   workspace  device buffer of attn_decode_multi_workspace_bytes(...) bytes,
 *              256-byte aligned.
 * Every KV head's G*T queries (G = Hq / Hkv) share one read of the cache when
 * G*T <= 16; larger G*T re-read it once per 16 queries (from cache memory when
 * the rereads run together), so long chunks of new tokens belong to attn_fwd.
 * dtype must be ATTN_BF16; limits and errors as attn_decode, and B*Hq*T must
 * fit in 31 bits.
 */
int attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int max_len, int d, float scale,
                      float rope_base, attn_dtype dtype, attn_dtype o_dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace attn_decode_paged needs: B*Hq*T*ceil(max_len/1024)
 * partial states of d + 1 floats with max_len = max_blocks * block_size (the
 * paged kernel splits the cache into chunks of 1024 keys); 0 when that
 * product overflows. */
size_t attn_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int T, int max_blocks,
                                         int block_size, int d);

/*
 * Multi-token decode over a paged KV cache ("Attention mechanisms: from
 * alignment to efficient long context", section 20; "Transformer Architecture
 * Breakdown", Paged Attention).  The arithmetic is that of attn_decode_multi;
 * only where the K/V rows live changes: token position p of sequence b is row
 * p % block_size of physical block block_table[b * max_blocks + p / block_size].
 *   q          device [B, Hq, T, d] bf16.
 *   k_pool, v_pool  device [num_blocks, Hkv, block_size, d] bf16 (a block holds
 *              block_size consecutive tokens of every KV head).
 *   block_table  device int32 [B, max_blocks]; the entries for the blocks that
 *              hold rows 0 .. seq_lens[b]-1 must name physical blocks (values
 *              are clamped into [0, num_blocks) before use); later entries are
 *              never used to read memory.
 *   seq_lens   device int32 [B], clamped to [0, max_blocks * block_size].  Rows
 *              at or past seq_lens[b] inside its last block are never read.
 *   block_size power of two in [16, 4096] (16 is the usual choice).
 *   o, lse, T, scale, rope_base, dtype, o_dtype, workspace: as
 *              attn_decode_multi, with attn_decode_paged_workspace_bytes(...)
 *              bytes of workspace.
 * Errors: num_blocks or max_blocks < 1, or a null table -> ATTN_ERR_INVALID;
 * another block_size, or max_blocks * block_size * d * 2 >= 2^31 ->
 * ATTN_ERR_UNSUPPORTED; otherwise as attn_decode_multi.
 */
int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int num_blocks, int block_size,
                      int max_blocks, int d, float scale, float rope_base, attn_dtype dtype,
                      attn_dtype o_dtype, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * RoPE on its own: out[b,h,n,:] = rotate(x[b,h,n,:], position pos_offset + n),
 * rounded to `dtype` exactly as attn_fwd rounds the rotated operands.
 * x, out  device [B, H, N, d] of `dtype` (may alias).  d a multiple of 8
 *         (bf16) or 4 (fp32), at most 512.  pos_offset + N <= 2^22, else
 *         ATTN_ERR_UNSUPPORTED.
 */
int attn_rope_apply(const void* x, void* out, int B, int H, int N, int d,
                    int pos_offset, float rope_base, attn_dtype dtype,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
