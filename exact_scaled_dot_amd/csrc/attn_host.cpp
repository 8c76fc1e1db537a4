// C ABI of libattn: argument validation, workspace sizing and dispatch.
//
// Every argument is checked on the host before the first HIP call, so invalid
// input never reaches a kernel.  Status codes are returned; nothing throws.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "attn.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 64 || d == 128; }

size_t elem_size(attn_dtype t) { return t == ATTN_F32 ? 4 : 2; }

bool known_dtype(int t) { return t == ATTN_BF16 || t == ATTN_F32; }

bool log_enabled() {
    // read once; the initialisation of a local static is thread-safe
    static const bool on = [] {
        const char* s = std::getenv("ATTN_LOG");
        return s != nullptr && s[0] == '1';
    }();
    return on;
}

// Workspace sizes saturate: a product or sum that does not fit in size_t
// becomes SIZE_MAX, which no workspace can match, so the call that checks it
// fails with ATTN_ERR_WORKSPACE instead of accepting a wrapped-around size.
size_t mul_sat(size_t a, size_t b) {
    size_t r;
    return __builtin_mul_overflow(a, b, &r) ? SIZE_MAX : r;
}

size_t add_sat(size_t a, size_t b) {
    size_t r;
    return __builtin_add_overflow(a, b, &r) ? SIZE_MAX : r;
}

size_t align256(size_t x) { return x > SIZE_MAX - 255 ? SIZE_MAX : (x + 255) & ~(size_t)255; }

int fail(int code, const char* what) {
    if (log_enabled()) fprintf(stderr, "[attn] %s: %s\n", attn_status_str(code), what);
    return code;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
        default: return "ATTN_ERR_UNKNOWN";
    }
}

size_t attn_fwd_workspace_bytes(int B, int Hkv, int Nk, int d, float rope_base, attn_dtype dtype) {
    if (!(rope_base > 0.f) || B <= 0 || Hkv <= 0 || Nk <= 0 || d <= 0 || !known_dtype(dtype))
        return 0;
    return mul_sat(mul_sat(mul_sat(mul_sat((size_t)B, (size_t)Hkv), (size_t)Nk), (size_t)d),
                   elem_size(dtype));
}

}  // extern "C"

namespace {

// Shared body of attn_fwd (window = 0) and attn_fwd_window (window >= 1, causal).
// rotate_k: with RoPE, K is rotated into the workspace first (attn_fwd);
// otherwise K is used as given (keys stored already rotated, attn_prefill_cached).
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int window,
             float scale, float rope_base, attn_dtype dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream,
             bool rotate_k = true, attn_dtype o_dtype = ATTN_F32) {
    if (B < 0 || Hq < 0 || Nq < 0) return fail(ATTN_ERR_INVALID, "negative size");
    if (Hkv < 1 || Nk < 1 || d < 1) return fail(ATTN_ERR_INVALID, "Hkv, Nk and d must be >= 1");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq must be a multiple of Hkv");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1");
    if (causal && Nq > Nk) return fail(ATTN_ERR_INVALID, "causal needs Nq <= Nk");
    if (window < 0 || (window > 0 && !causal)) return fail(ATTN_ERR_INVALID, "window must be >= 1 and causal");
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_INVALID, "scale must be finite and > 0");
    if (rope_base != 0.f && !(std::isfinite(rope_base) && rope_base > 0.f))
        return fail(ATTN_ERR_INVALID, "rope_base must be 0 or a finite positive base");
    if (rope_base != 0.f && Nq > Nk)
        return fail(ATTN_ERR_INVALID, "RoPE needs Nq <= Nk (query positions Nk-Nq+i must be >= 0)");
    if (rope_base != 0.f && Nk > attn::kMaxRopePositions)
        return fail(ATTN_ERR_UNSUPPORTED, "RoPE positions must be below 2^22");
    if (!known_dtype(dtype)) return fail(ATTN_ERR_INVALID, "unknown dtype");
    if (!known_dtype(o_dtype)) return fail(ATTN_ERR_INVALID, "unknown output dtype");
    if (!supported_d(d)) return fail(ATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
    if ((long long)Nk * d * 4 >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "one head's K (or V) must be under 2 GiB (32-bit buffer offsets)");
    if (B == 0 || Hq == 0 || Nq == 0) return ATTN_OK;
    if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(ATTN_ERR_INVALID, "q, k, v, o must be 16-byte aligned");
    const bool rope = rope_base > 0.f;
    const size_t need = rotate_k ? attn_fwd_workspace_bytes(B, Hkv, Nk, d, rope_base, dtype) : 0;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or too small for the rotated K");
    if (need > 0 && !aligned16(workspace)) return fail(ATTN_ERR_INVALID, "workspace must be 16-byte aligned");

    attn::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
    a.causal = causal; a.scale = scale; a.rope_tab = nullptr;
    a.window = window < Nk ? window : 0;  // a window covering every key is plain causal
    a.o_bf16 = o_dtype == ATTN_BF16 ? 1 : 0;

    if (rope) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice");
        const double2* tab = nullptr;
        const int rc = attn::rope_table(dev, rope_base, d, Nk, stream, &tab);
        if (rc != ATTN_OK) return fail(rc, "RoPE table (not built while a stream is captured)");
        if (rotate_k) {
            // K rotated once into the workspace; Q is rotated as it is loaded.
            const long long rows = (long long)B * Hkv * Nk;
            if (dtype == ATTN_BF16)
                e = attn::launch_rope_bf16(static_cast<const uint16_t*>(k), static_cast<uint16_t*>(workspace),
                                           rows, Nk, d, 0, tab, stream);
            else
                e = attn::launch_rope_f32(static_cast<const float*>(k), static_cast<float*>(workspace),
                                          rows, Nk, d, 0, tab, stream);
            if (e != hipSuccess) return fail(ATTN_ERR_HIP, "rope launch");
            a.k = workspace;
        }
        a.rope_tab = tab;
    }
    hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, stream)
                                      : attn::launch_prefill_f32(a, stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, hipGetErrorString(e));
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
             float scale, float rope_base, attn_dtype dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, 0, scale, rope_base, dtype,
                    workspace, workspace_bytes, stream);
}

int attn_fwd_window(const void* q, const void* k, const void* v, float* o, float* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, int window,
                    float scale, float rope_base, attn_dtype dtype,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (window < 1) return fail(ATTN_ERR_INVALID, "window must be >= 1");
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, 1, window, scale, rope_base, dtype,
                    workspace, workspace_bytes, stream);
}

int attn_prefill_cached(const void* q, const void* k_cache, const void* v_cache, void* o,
                        float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        float rope_base, attn_dtype dtype, attn_dtype o_dtype, hipStream_t stream) {
    return fwd_impl(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nq, Nk, d, 1, 0, scale, rope_base,
                    dtype, nullptr, 0, stream, /*rotate_k=*/false, o_dtype);
}

// Partial states of the split decode: one per (row, chunk of `chunk` keys),
// d floats of O then one float of lse, the two arrays 256-byte aligned.
static size_t decode_ws_bytes(int B, int Hq, int Hkv, int T, int max_len, int d, int chunk) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || max_len <= 0 || d <= 0) return 0;
    const size_t nch = ((size_t)max_len + (size_t)chunk - 1) / (size_t)chunk;
    const size_t rows = mul_sat(mul_sat(mul_sat((size_t)B, (size_t)Hq), (size_t)T), nch);
    const size_t o_bytes = align256(mul_sat(mul_sat(rows, (size_t)d), sizeof(float)));
    return add_sat(o_bytes, mul_sat(rows, sizeof(float)));
}

size_t attn_decode_multi_workspace_bytes(int B, int Hq, int Hkv, int T, int max_len, int d) {
    return decode_ws_bytes(B, Hq, Hkv, T, max_len, d, attn::decode_chunk(false));
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int d) {
    return attn_decode_multi_workspace_bytes(B, Hq, Hkv, 1, max_len, d);
}

size_t attn_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int T, int max_blocks,
                                         int block_size, int d) {
    if (max_blocks <= 0 || block_size <= 0) return 0;
    const long long max_len = (long long)max_blocks * block_size;
    if (max_len > 0x7fffffffLL) return 0;
    return decode_ws_bytes(B, Hq, Hkv, T, (int)max_len, d, attn::decode_chunk(true));
}

}  // extern "C"

namespace {

// Shared body of the three decode entry points.  table == nullptr: contiguous
// caches [B, Hkv, max_len, d]; otherwise pools [num_blocks, Hkv, block_size, d]
// addressed through table [B, max_blocks] (max_len = max_blocks * block_size).
int decode_impl(const void* q, const void* k, const void* v, const int32_t* table,
                const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int T,
                int max_len, int num_blocks, int block_size, int max_blocks, int d, float scale,
                float rope_base, attn_dtype dtype, attn_dtype o_dtype, void* workspace,
                size_t workspace_bytes, hipStream_t stream, bool use_scratch = false) {
    if (B < 0 || Hq < 0) return fail(ATTN_ERR_INVALID, "negative size");
    if (Hkv < 1 || T < 1 || max_len < 1 || d < 1)
        return fail(ATTN_ERR_INVALID, "Hkv, T, max_len and d must be >= 1");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq must be a multiple of Hkv");
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_INVALID, "scale must be finite and > 0");
    if (rope_base != 0.f && !(std::isfinite(rope_base) && rope_base > 0.f))
        return fail(ATTN_ERR_INVALID, "rope_base must be 0 or a finite positive base");
    if (!known_dtype(dtype)) return fail(ATTN_ERR_INVALID, "unknown dtype");
    if (!known_dtype(o_dtype)) return fail(ATTN_ERR_INVALID, "unknown output dtype");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode is built for bf16");
    if (!supported_d(d)) return fail(ATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
    if ((long long)max_len * d * 2 >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "one sequence's cache must be under 2 GiB (32-bit buffer offsets)");
    if ((long long)B * Hq * T > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "B * Hq * T must fit in 31 bits");
    if (rope_base > 0.f && max_len > attn::kMaxRopePositions)
        return fail(ATTN_ERR_UNSUPPORTED, "RoPE positions must be below 2^22");
    if (B == 0 || Hq == 0) return ATTN_OK;
    if (!q || !k || !v || !seq_lens || !o) return fail(ATTN_ERR_INVALID, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(ATTN_ERR_INVALID, "q, caches and o must be 16-byte aligned");
    const int chunk = attn::decode_chunk(table != nullptr);
    const size_t need = decode_ws_bytes(B, Hq, Hkv, T, max_len, d, chunk);
    if (use_scratch) {
        // the partial states go to the library's static per-device array
        if (need > attn::kNoAllocScratchBytes)
            return fail(ATTN_ERR_WORKSPACE,
                        "partial states exceed the static scratch (ATTN_DECODE_NOALLOC_MAX_BYTES)");
        const hipError_t e = attn::noalloc_scratch(&workspace);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "static scratch address");
        workspace_bytes = attn::kNoAllocScratchBytes;
    }
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "decode workspace missing or too small");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(ATTN_ERR_INVALID, "decode workspace must be 256-byte aligned");

    attn::DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.lens = seq_lens;
    a.o = o; a.lse = lse;
    a.o_bf16 = o_dtype == ATTN_BF16 ? 1 : 0;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.T = T; a.max_len = max_len; a.d = d; a.scale = scale;
    a.rope_tab = nullptr;
    a.table = table;
    a.max_blocks = max_blocks;
    a.num_blocks = num_blocks;
    a.block_log2 = 0;
    while ((1 << a.block_log2) < block_size) ++a.block_log2;
    if (rope_base > 0.f) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice");
        const int rc = attn::rope_table(dev, rope_base, d, max_len, stream, &a.rope_tab);
        if (rc != ATTN_OK) return fail(rc, "RoPE table (not built while a stream is captured)");
    }
    a.chunk = chunk;
    a.nchunks = (max_len + chunk - 1) / chunk;
    const size_t rows = (size_t)B * Hq * T * a.nchunks;
    size_t o_bytes = (rows * d * sizeof(float) + 255) & ~(size_t)255;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
    hipError_t e = attn::launch_decode_bf16(a, stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, hipGetErrorString(e));
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int max_len, int d, float scale,
                      float rope_base, attn_dtype dtype, attn_dtype o_dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    return decode_impl(q, k_cache, v_cache, nullptr, seq_lens, o, lse, B, Hq, Hkv, T, max_len,
                       0, 1, 0, d, scale, rope_base, dtype, o_dtype, workspace, workspace_bytes,
                       stream);
}

int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      int B, int Hq, int Hkv, int T, int num_blocks, int block_size,
                      int max_blocks, int d, float scale, float rope_base, attn_dtype dtype,
                      attn_dtype o_dtype, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    if (num_blocks < 1 || max_blocks < 1)
        return fail(ATTN_ERR_INVALID, "num_blocks and max_blocks must be >= 1");
    if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "block_size must be a power of two in [16, 4096]");
    if ((long long)max_blocks * block_size > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "max_blocks * block_size must fit in 31 bits");
    if (B > 0 && Hq > 0 && block_table == nullptr) return fail(ATTN_ERR_INVALID, "null block table");
    return decode_impl(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, T,
                       max_blocks * block_size, num_blocks, block_size, max_blocks, d, scale,
                       rope_base, dtype, o_dtype, workspace, workspace_bytes, stream);
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seq_lens, float* o, float* lse,
                int B, int Hq, int Hkv, int max_len, int d, float scale,
                attn_dtype dtype, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
    return attn_decode_multi(q, k_cache, v_cache, seq_lens, o, lse, B, Hq, Hkv, 1, max_len, d,
                             scale, 0.f, dtype, ATTN_F32, workspace, workspace_bytes, stream);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, float* o, float* lse,
                        int B, int Hq, int Hkv, int max_len, int d, float scale,
                        attn_dtype dtype, hipStream_t stream) {
    return decode_impl(q, k_cache, v_cache, nullptr, seq_lens, o, lse, B, Hq, Hkv, 1, max_len,
                       0, 1, 0, d, scale, 0.f, dtype, ATTN_F32, nullptr, 0, stream,
                       /*use_scratch=*/true);
}

// Workspace of attn_bwd, in order (each section 256-byte aligned): dO in bf16
// [B,Hq,Nq,d], D [B,Hq,Nq] fp32, lse2 [B,Hq,Nq] fp32, then with RoPE the
// rotated Q [B,Hq,Nq,d] and K [B,Hkv,Nk,d] in bf16.
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, float rope_base,
                                attn_dtype dtype) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || dtype != ATTN_BF16)
        return 0;
    const size_t rows = mul_sat(mul_sat((size_t)B, (size_t)Hq), (size_t)Nq);
    const size_t rows_d2 = align256(mul_sat(mul_sat(rows, (size_t)d), 2));
    size_t n = add_sat(rows_d2, mul_sat(2, align256(mul_sat(rows, 4))));
    if (rope_base > 0.f) {
        const size_t k_d2 = mul_sat(mul_sat(mul_sat(mul_sat((size_t)B, (size_t)Hkv), (size_t)Nk),
                                            (size_t)d), 2);
        n = add_sat(add_sat(n, rows_d2), align256(k_d2));
    }
    return n;
}

int attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const float* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, int causal, float scale, float rope_base, attn_dtype dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || Hq < 0 || Nq < 0) return fail(ATTN_ERR_INVALID, "negative size");
    if (Hkv < 1 || Nk < 1 || d < 1) return fail(ATTN_ERR_INVALID, "Hkv, Nk and d must be >= 1");
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq must be a multiple of Hkv");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1");
    if (causal && Nq > Nk) return fail(ATTN_ERR_INVALID, "causal needs Nq <= Nk");
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_INVALID, "scale must be finite and > 0");
    if (rope_base != 0.f && !(std::isfinite(rope_base) && rope_base > 0.f))
        return fail(ATTN_ERR_INVALID, "rope_base must be 0 or a finite positive base");
    if (rope_base != 0.f && Nq > Nk)
        return fail(ATTN_ERR_INVALID, "RoPE needs Nq <= Nk (query positions Nk-Nq+i must be >= 0)");
    if (!known_dtype(dtype)) return fail(ATTN_ERR_INVALID, "unknown dtype");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the backward pass is built for bf16");
    if (!supported_d(d)) return fail(ATTN_ERR_UNSUPPORTED, "head dim must be 64 or 128");
    if ((long long)Nk * d * 4 >= (1LL << 31) || (long long)Nq * d * 4 >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "one head's Q, K or V must be under 2 GiB (32-bit buffer offsets)");
    if (rope_base != 0.f && Nk > attn::kMaxRopePositions)
        return fail(ATTN_ERR_UNSUPPORTED, "RoPE positions must be below 2^22");
    if (B == 0 || Hq == 0 || Nq == 0) return ATTN_OK;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
        return fail(ATTN_ERR_INVALID, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return fail(ATTN_ERR_INVALID, "q, k, v, o, dout, dq, dk, dv must be 16-byte aligned");
    const size_t need = attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, rope_base, dtype);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "backward workspace missing or too small");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(ATTN_ERR_INVALID, "backward workspace must be 256-byte aligned");

    const size_t rows = (size_t)B * Hq * Nq;
    char* w = static_cast<char*>(workspace);
    attn::BwdArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = o; a.lse = lse; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
    a.causal = causal; a.scale = scale;
    a.do16 = reinterpret_cast<uint16_t*>(w);
    w += align256(rows * d * 2);
    a.dvec = reinterpret_cast<float*>(w);
    w += align256(rows * 4);
    a.lse2 = reinterpret_cast<float*>(w);
    w += align256(rows * 4);
    const double2* tab = nullptr;
    hipError_t e = hipSuccess;
    if (rope_base > 0.f) {
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice");
        const int rc = attn::rope_table(dev, rope_base, d, Nk, stream, &tab);
        if (rc != ATTN_OK) return fail(rc, "RoPE table (not built while a stream is captured)");
        uint16_t* qr = reinterpret_cast<uint16_t*>(w);
        w += align256(rows * d * 2);
        uint16_t* kr = reinterpret_cast<uint16_t*>(w);
        // the rotated operands exactly as the forward pass forms them
        e = attn::launch_rope_bf16(a.q, qr, (long long)rows, Nq, d, Nk - Nq, tab, stream);
        if (e == hipSuccess)
            e = attn::launch_rope_bf16(a.k, kr, (long long)B * Hkv * Nk, Nk, d, 0, tab, stream);
        if (e != hipSuccess) return fail(ATTN_ERR_HIP, "rope launch");
        a.q = qr;
        a.k = kr;
    }
    // the kernels take the gradients with respect to the rotated rows back to
    // the rows before rotation as they store them
    a.rope_t = tab;
    e = attn::launch_bwd_bf16(a, stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, hipGetErrorString(e));
    return ATTN_OK;
}

int attn_rope_apply(const void* x, void* out, int B, int H, int N, int d,
                    int pos_offset, float rope_base, attn_dtype dtype,
                    hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0 || pos_offset < 0) return fail(ATTN_ERR_INVALID, "negative size");
    if (d < 2 || d % 2) return fail(ATTN_ERR_INVALID, "RoPE needs an even head dim");
    if (!(std::isfinite(rope_base) && rope_base > 0.f)) return fail(ATTN_ERR_INVALID, "rope_base must be finite and > 0");
    if (!known_dtype(dtype)) return fail(ATTN_ERR_INVALID, "unknown dtype");
    if (d % (dtype == ATTN_BF16 ? 8 : 4) != 0 || d > 512)
        return fail(ATTN_ERR_UNSUPPORTED, "head dim must be a multiple of 8 (bf16) / 4 (f32), <= 512");
    if ((long long)pos_offset + N > attn::kMaxRopePositions)
        return fail(ATTN_ERR_UNSUPPORTED, "RoPE positions must be below 2^22");
    if (B == 0 || H == 0 || N == 0) return ATTN_OK;
    if (!x || !out) return fail(ATTN_ERR_INVALID, "null pointer");
    if (!aligned16(x) || !aligned16(out)) return fail(ATTN_ERR_INVALID, "x and out must be 16-byte aligned");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice");
    const double2* tab = nullptr;
    const int rc = attn::rope_table(dev, rope_base, d, pos_offset + N, stream, &tab);
    if (rc != ATTN_OK) return fail(rc, "RoPE table (not built while a stream is captured)");
    const long long rows = (long long)B * H * N;
    if (dtype == ATTN_BF16)
        e = attn::launch_rope_bf16(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(out), rows, N, d,
                                   pos_offset, tab, stream);
    else
        e = attn::launch_rope_f32(static_cast<const float*>(x), static_cast<float*>(out), rows, N, d,
                                  pos_offset, tab, stream);
    return e == hipSuccess ? ATTN_OK : fail(ATTN_ERR_HIP, hipGetErrorString(e));
}

}  // extern "C"
