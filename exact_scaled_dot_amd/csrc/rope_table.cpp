// RoPE (cos, sin) tables: fp64, built on the host with the C library, kept on
// the device.
//
// Pair j of a row at position p turns by the angle p * theta_j with
// theta_j = base^(-2j/d) ("Transformer Architecture Breakdown", section 3.1;
// "coding-interview attention from scratch", section 三.5).  Entry [p][j] holds
// cos and sin of the fp64 product p * theta_j, with theta_j from pow, both from
// the C library, so the kernels rotate with exactly the values a host
// evaluation in fp64 uses.
//
// Host code only, and nothing here throws: every failure becomes a status.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "attn.h"
#include "launch.h"

namespace attn {

namespace {

struct Table {
    double2* ptr = nullptr;
    int npos = 0;
};

std::mutex g_tab_mu;
std::map<std::tuple<int, uint32_t, int>, Table> g_tabs;

// host staging per upload: at most 16 MB of table at a time
constexpr size_t kStageBytes = size_t(16) << 20;

int build(double2* dev, float base, int d, int npos) {
    const int half = d / 2;
    std::vector<double> theta(half);
    for (int j = 0; j < half; ++j) theta[j] = std::pow((double)base, -2.0 * j / d);
    const int step = (int)std::max<size_t>(1, kStageBytes / (sizeof(double2) * half));
    std::vector<double2> host((size_t)std::min(step, npos) * half);
    for (int p0 = 0; p0 < npos; p0 += step) {
        const int n = std::min(step, npos - p0);
        for (int p = 0; p < n; ++p)
            for (int j = 0; j < half; ++j) {
                const double ang = (double)(p0 + p) * theta[j];
                host[(size_t)p * half + j] = make_double2(std::cos(ang), std::sin(ang));
            }
        const hipError_t e = hipMemcpy(dev + (size_t)p0 * half, host.data(),
                                       (size_t)n * half * sizeof(double2), hipMemcpyHostToDevice);
        if (e != hipSuccess) return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

}  // namespace

int rope_table(int device, float base, int d, int npos, hipStream_t stream, const double2** tab) {
    *tab = nullptr;
    if (npos < 1 || npos > kMaxRopePositions || d < 2 || d % 2) return ATTN_ERR_UNSUPPORTED;
    try {
        uint32_t bits;
        std::memcpy(&bits, &base, sizeof bits);
        std::lock_guard<std::mutex> lock(g_tab_mu);
        Table& t = g_tabs[std::make_tuple(device, bits, d)];
        if (t.ptr && t.npos >= npos) {
            *tab = t.ptr;
            return ATTN_OK;
        }
        // Building uploads with blocking copies, which a stream being captured
        // into a graph must not see (the null stream is never captured).
        if (stream != nullptr) {
            hipStreamCaptureStatus cap_status = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(stream, &cap_status) != hipSuccess ||
                cap_status != hipStreamCaptureStatusNone)
                return ATTN_ERR_HIP;
        }
        // Grow to a power of two of at least 1024 positions (a few growing
        // calls do not each rebuild), at most kMaxRopePositions.  An older,
        // smaller table stays allocated: kernels queued on some stream may
        // still read it.
        int cap = 1024;
        while (cap < npos) cap *= 2;
        if (cap > kMaxRopePositions) cap = kMaxRopePositions;
        double2* dev = nullptr;
        if (hipMalloc(&dev, (size_t)cap * (d / 2) * sizeof(double2)) != hipSuccess) return ATTN_ERR_HIP;
        const int rc = build(dev, base, d, cap);
        if (rc != ATTN_OK) {
            (void)hipFree(dev);
            return rc;
        }
        t.ptr = dev;
        t.npos = cap;
        *tab = dev;
        return ATTN_OK;
    } catch (...) {  // allocation failure (host staging, map node) or a lock error
        return ATTN_ERR_HIP;
    }
}

}  // namespace attn
