// Stand-ins for the HIP runtime calls and the kernel launchers that the
// library's host code (attn_host.cpp, rope_table.cpp) makes, so that code can
// be built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// run on a machine without a GPU.  Test infrastructure only: never linked
// into libattn.so.
//
// "Device" memory is host memory (hipMalloc = malloc, hipMemcpy = memcpy), the
// launchers record their arguments and succeed, and a flag makes every stream
// report that it is being captured.  The stub_* functions let the tests read
// what was recorded.

#include <cstdlib>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "attn.h"
#include "launch.h"

namespace {

int g_capturing = 0;
int g_calls[8] = {};
attn::FwdArgs g_fwd{};
attn::DecodeArgs g_dec{};
attn::BwdArgs g_bwd{};
const void* g_rope_in[2] = {};
const void* g_rope_out[2] = {};
int g_rope_n = 0;
alignas(256) unsigned char g_scratch[attn::kNoAllocScratchBytes];

enum { kPrefillBf16, kPrefillF32, kRopeBf16, kRopeF32, kDecode, kBwd, kScratch };

}  // namespace

extern "C" {

hipError_t hipGetDevice(int* device) {
    *device = 0;
    return hipSuccess;
}

const char* hipGetErrorString(hipError_t) { return "stub"; }

hipError_t hipMalloc(void** ptr, size_t size) {
    *ptr = std::malloc(size ? size : 1);
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipFree(void* ptr) {
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t size, hipMemcpyKind) {
    std::memcpy(dst, src, size);
    return hipSuccess;
}

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
    *status = g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}

// ---- inspection hooks for the tests
void stub_reset() {
    std::memset(g_calls, 0, sizeof g_calls);
    g_fwd = attn::FwdArgs{};
    g_dec = attn::DecodeArgs{};
    g_bwd = attn::BwdArgs{};
    g_rope_n = 0;
}
void stub_set_capturing(int on) { g_capturing = on; }
int stub_calls(int which) { return which >= 0 && which < 8 ? g_calls[which] : -1; }
const void* stub_fwd_k() { return g_fwd.k; }
const void* stub_fwd_rope_tab() { return g_fwd.rope_tab; }
int stub_fwd_o_bf16() { return g_fwd.o_bf16; }
int stub_fwd_window() { return g_fwd.window; }
const void* stub_dec_ws_o() { return g_dec.ws_o; }
const void* stub_dec_ws_lse() { return g_dec.ws_lse; }
int stub_dec_nchunks() { return g_dec.nchunks; }
int stub_dec_o_bf16() { return g_dec.o_bf16; }
const void* stub_dec_rope_tab() { return g_dec.rope_tab; }
const void* stub_bwd_q() { return g_bwd.q; }
const void* stub_bwd_k() { return g_bwd.k; }
const void* stub_rope_out(int i) { return i >= 0 && i < 2 ? g_rope_out[i] : nullptr; }
const void* stub_scratch() { return g_scratch; }

}  // extern "C"

namespace attn {

hipError_t launch_prefill_bf16(const FwdArgs& a, hipStream_t) {
    ++g_calls[kPrefillBf16];
    g_fwd = a;
    return hipSuccess;
}

hipError_t launch_prefill_f32(const FwdArgs& a, hipStream_t) {
    ++g_calls[kPrefillF32];
    g_fwd = a;
    return hipSuccess;
}

static void record_rope(const void* x, void* out) {
    if (g_rope_n < 2) {
        g_rope_in[g_rope_n] = x;
        g_rope_out[g_rope_n] = out;
    }
    ++g_rope_n;
}

hipError_t launch_rope_bf16(const uint16_t* x, uint16_t* out, long long, int, int, int,
                            const double2*, hipStream_t) {
    ++g_calls[kRopeBf16];
    record_rope(x, out);
    return hipSuccess;
}

hipError_t launch_rope_f32(const float* x, float* out, long long, int, int, int, const double2*,
                           hipStream_t) {
    ++g_calls[kRopeF32];
    record_rope(x, out);
    return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t) {
    ++g_calls[kDecode];
    g_dec = a;
    return hipSuccess;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t) {
    ++g_calls[kBwd];
    g_bwd = a;
    return hipSuccess;
}

hipError_t noalloc_scratch(void** ptr) {
    ++g_calls[kScratch];
    *ptr = g_scratch;
    return hipSuccess;
}

}  // namespace attn
