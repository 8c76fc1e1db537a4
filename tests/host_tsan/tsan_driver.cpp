// Many host threads calling the C ABI at once, against the stand-in runtime of
// stubs_tsan.cpp, built with -fsanitize=thread: the entry points' claim to be
// thread-safe, including the first calls that build and grow the RoPE tables
// concurrently.  Device pointers are fake addresses the stubs never touch.
// Exit status 0 when every call returned the expected status; any data race
// is reported by ThreadSanitizer.  Test infrastructure only.

#include <cstdint>
#include <cstdio>
#include <thread>
#include <vector>

#include "attn.h"

extern "C" long stub_launches();

namespace {

void* P(uintptr_t k) { return reinterpret_cast<void*>(k << 24); }  // 16-byte aligned fakes

int worker(int t) {
    int bad = 0;
    const float bases[3] = {10000.f, 500000.f, 20000.f};
    static unsigned char ws_pool[16][1 << 12] __attribute__((aligned(256)));
    for (int it = 0; it < 40; ++it) {
        const float base = bases[(t + it) % 3];
        const int Nk = 64 << ((t * 7 + it) % 8);  // 64 .. 8192 keys: tables grow while others read
        const int Nq = Nk / 2;
        hipStream_t s = reinterpret_cast<hipStream_t>(0x1000 + t);
        bad += attn_fwd(P(1), P(2), P(3), static_cast<float*>(P(4)), static_cast<float*>(P(5)),
                        1, 8, 2, Nq, Nk, 128, 1, 0.088f, base, ATTN_BF16, P(6), size_t(1) << 40,
                        s) != ATTN_OK;
        bad += attn_fwd_window(P(1), P(2), P(3), static_cast<float*>(P(4)), nullptr, 1, 4, 4, Nq,
                               Nk, 64, 128, 0.125f, base, ATTN_BF16, P(6), size_t(1) << 40,
                               s) != ATTN_OK;
        bad += attn_rope_apply(P(1), P(2), 2, 3, Nk, 128, it, base, ATTN_F32, s) != ATTN_OK;
        bad += attn_bwd(P(1), P(2), P(3), static_cast<float*>(P(4)), static_cast<float*>(P(5)),
                        static_cast<float*>(P(7)), static_cast<float*>(P(8)),
                        static_cast<float*>(P(9)), static_cast<float*>(P(10)), 1, 8, 2, Nq, Nk, 128,
                        1, 0.088f, base, ATTN_BF16, P(6), size_t(1) << 40, s) != ATTN_OK;
        bad += attn_decode_multi(P(1), P(2), P(3), static_cast<const int32_t*>(P(11)), P(4),
                                 static_cast<float*>(P(5)), 4, 8, 2, 4, Nk, 128, 0.088f, base,
                                 ATTN_BF16, ATTN_BF16, P(6), size_t(1) << 40, s) != ATTN_OK;
        bad += attn_decode_noalloc(P(1), P(2), P(3), static_cast<const int32_t*>(P(11)),
                                   static_cast<float*>(P(4)), static_cast<float*>(P(5)), 2, 8, 2, Nk,
                                   128, 0.088f, ATTN_BF16, s) != ATTN_OK;
        // rejected calls and queries
        bad += attn_fwd(P(1), P(2), P(3), static_cast<float*>(P(4)), nullptr, 1, 8, 3, 1, 1, 128, 1,
                        0.1f, 0.f, ATTN_BF16, nullptr, 0, s) != ATTN_ERR_INVALID;
        bad += attn_decode(P(1), P(2), P(3), static_cast<const int32_t*>(P(11)),
                           static_cast<float*>(P(4)), nullptr, 1, 8, 2, 100, 128, 0.1f, ATTN_BF16,
                           ws_pool[t % 16], 16, s) != ATTN_ERR_WORKSPACE;
        bad += attn_fwd_workspace_bytes(2, 8, Nk, 128, base, ATTN_BF16) != size_t(2) * 8 * Nk * 128 * 2;
        bad += attn_status_str(it % 6)[0] != 'A';
    }
    return bad;
}

}  // namespace

int main() {
    const int n = 16;
    std::vector<int> bad(n, 0);
    std::vector<std::thread> th;
    for (int t = 0; t < n; ++t) th.emplace_back([t, &bad] { bad[t] = worker(t); });
    for (auto& x : th) x.join();
    int total = 0;
    for (int b : bad) total += b;
    std::printf("threads %d, unexpected statuses %d, launches %ld\n", n, total, stub_launches());
    return total == 0 ? 0 : 1;
}
