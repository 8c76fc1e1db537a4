// Thread-safe stand-ins for the HIP runtime calls and kernel launchers that
// the library's host code (attn_host.cpp, rope_table.cpp) makes, for the
// ThreadSanitizer build driven by tsan_driver.cpp.  "Device" memory is host
// memory; the launchers count calls atomically and succeed.  Test
// infrastructure only: never linked into libattn.so.

#include <atomic>
#include <cstdlib>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "attn.h"
#include "launch.h"

namespace {
std::atomic<long> g_launches{0};
alignas(256) unsigned char g_scratch[attn::kNoAllocScratchBytes];
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
    *status = hipStreamCaptureStatusNone;
    return hipSuccess;
}

long stub_launches() { return g_launches.load(); }

}  // extern "C"

namespace attn {

hipError_t launch_prefill_bf16(const FwdArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_f32(const FwdArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_rope_bf16(const uint16_t*, uint16_t*, long long, int, int, int, const double2*,
                            hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_rope_f32(const float*, float*, long long, int, int, int, const double2*,
                           hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_decode_bf16(const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_bf16(const BwdArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t noalloc_scratch(void** ptr) {
    *ptr = g_scratch;
    return hipSuccess;
}

}  // namespace attn
