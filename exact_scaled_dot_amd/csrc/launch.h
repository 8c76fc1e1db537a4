// Internal launchers behind the C ABI (host side).  Arguments are validated by
// the entry points in attn_host.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

struct FwdArgs {
    const void* q;
    const void* k;  // rotated K when RoPE is on
    const void* v;
    void* o;        // fp32, or bf16 when o_bf16
    float* lse;
    int B, Hq, Hkv, Nq, Nk, d;
    int causal;
    int window;  // > 0: causal sliding window of this many keys; 0: none
    float scale;
    const double2* rope_tab;  // null: no RoPE on Q
    int o_bf16;               // 1: O stored as bf16 (nearest even from the fp32 value)
};

hipError_t launch_prefill_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const FwdArgs& a, hipStream_t stream);

// out[bh, n, :] = rotate(x[bh, n, :], pos_offset + n)
hipError_t launch_rope_bf16(const uint16_t* x, uint16_t* out, long long rows, int N, int d,
                            int pos_offset, const double2* tab, hipStream_t stream);
hipError_t launch_rope_f32(const float* x, float* out, long long rows, int N, int d,
                           int pos_offset, const double2* tab, hipStream_t stream);

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* lens;
    void* o;        // fp32, or bf16 when o_bf16
    float* lse;
    int B, Hq, Hkv, T, max_len, d;  // T new query tokens per sequence
    float scale;
    const double2* rope_tab;  // null: no RoPE on the queries
    // paged cache (table != null): k, v are pools [num_blocks, Hkv, 2^block_log2, d],
    // table [B, max_blocks]; max_len = max_blocks << block_log2
    const int32_t* table;
    int max_blocks, block_log2, num_blocks;
    float* ws_o;    // [B, Hq, T, nchunks, d]
    float* ws_lse;  // [B, Hq, T, nchunks] (log2 domain)
    int nchunks;
    int chunk;      // keys per split workgroup (decode_chunk(paged))
    int o_bf16;     // 1: O stored as bf16 (nearest even from the fp32 value)
};

// Keys per split workgroup: 2048 for a contiguous cache (half the partial
// states of 1024, which matters once several new tokens share a chunk); 1024
// for a paged cache, whose per-block load resources need the registers.
constexpr int kDecodeChunk = 2048;
constexpr int kDecodeChunkPaged = 1024;
constexpr int decode_chunk(bool paged) { return paged ? kDecodeChunkPaged : kDecodeChunk; }

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// Size of the per-device static array that holds attn_decode_noalloc's
// partial states (ATTN_DECODE_NOALLOC_MAX_BYTES in attn.h).
constexpr size_t kNoAllocScratchBytes = ATTN_DECODE_NOALLOC_MAX_BYTES;

// Device address of the current device's copy of that array, looked up with
// hipGetSymbolAddress on the first call per device.
hipError_t noalloc_scratch(void** ptr);

struct BwdArgs {
    const uint16_t* q;   // rotated Q when RoPE is on
    const uint16_t* k;   // rotated K when RoPE is on
    const uint16_t* v;
    const float* o;
    const float* lse;
    const float* dout;
    float* dq;
    float* dk;
    float* dv;
    int B, Hq, Hkv, Nq, Nk, d;
    int causal;
    float scale;
    uint16_t* do16;  // workspace: dO in bf16 [B, Hq, Nq, d]
    float* dvec;     // workspace: rowsum(dO * O) [B, Hq, Nq]
    float* lse2;     // workspace: lse * log2(e) [B, Hq, Nq]
    // RoPE table (null: no RoPE).  The kernels store dQ and dK rotated back
    // (the transpose of the rotation, fp64, rounded to fp32) at their rows'
    // positions: queries at Nk - Nq + i, keys at j.
    const double2* rope_t;
};

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// Largest number of RoPE positions (0 .. kMaxRopePositions - 1) any call may
// use: every K row range the forward accepts at d = 128 (Nk * d * 4 < 2^31).
constexpr int kMaxRopePositions = 1 << 22;

// Device table of (cos, sin) in fp64, [npos][d/2], covering positions
// 0 .. npos - 1 (or more); created or grown on demand (rope_table.cpp).
// Returns an attn_status; *tab is set on ATTN_OK.  Building refuses to run
// while `stream` is being captured (ATTN_ERR_HIP).
int rope_table(int device, float base, int d, int npos, hipStream_t stream, const double2** tab);

}  // namespace attn
