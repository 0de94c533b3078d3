// host_sanitize_driver.cpp -- drives the host side of libep (configuration
// checks, buffer sizes, layout geometry and the argument checks of every call)
// over millions of configurations mixing ordinary and extreme values (0, 1,
// powers of two, each limit and one past it, INT32_MAX), so that a build of
// the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
// reports any out-of-bounds access or undefined arithmetic (signed overflow
// above all).  No HIP call is made: every entry point is called with missing
// buffers, which it must reject before enqueuing anything.
//
// Test infrastructure: built and run by tests/test_host_sanitized.py.
// Usage: host_sanitize_driver [configurations] [seed]
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ep.h"

static uint64_t state;

// xorshift64 (Marsaglia, "Xorshift RNGs", 2003).
static uint64_t next_u64() {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}

template <int N>
static int32_t pick(const int32_t (&v)[N]) {
    return v[next_u64() % N];
}

int main(int argc, char **argv) {
    const long n = argc > 1 ? atol(argv[1]) : 1000000;
    state = argc > 2 ? strtoull(argv[2], nullptr, 10) : 88172645463325252ull;
    if (state == 0) state = 1;
    const int32_t Ss[] = {1, 2, 3, 16, 255, 65535, 65536};
    const int32_t Ts[] = {0, 1, 7, 4096, 1 << 20, 1 << 29, (1 << 30) - 1, 1 << 30, (1 << 30) + 1, INT32_MAX, -1};
    const int32_t Ks[] = {1, 2, 8, 31, 32, 33, 0};
    const int32_t Rs[] = {1, 2, 16, 63, 64, 65};
    const int32_t Els[] = {1, 3, 16, 1024};
    const int32_t Hs[] = {8, 128, 7168, 262144, 262152, 12};
    const int32_t As[] = {1, 2, 128, 1 << 20, INT32_MAX, 0};
    const int32_t Cs[] = {0, 1, 255, 4096, INT32_MAX, -1};
    const int32_t Extra[] = {0, 1, 3, 1 << 20, INT32_MAX, -1};
    long accepted = 0, large = 0;
    for (long it = 0; it < n; ++it) {
        ep_config_t c;
        c.num_src_ranks = pick(Ss);
        c.num_tokens = pick(Ts);
        c.num_topk = pick(Ks);
        c.num_ranks = pick(Rs);
        c.num_experts = c.num_ranks * pick(Els);
        c.hidden = pick(Hs);
        const int64_t nmax = (int64_t)c.num_tokens + pick(Extra);
        c.num_max_tokens_per_rank = nmax > INT32_MAX ? INT32_MAX : (nmax < INT32_MIN ? INT32_MIN : (int32_t)nmax);
        c.x_dtype = (int32_t)(next_u64() % 3);
        c.expand = (int32_t)(next_u64() % 3);
        c.expert_alignment = pick(As);
        c.num_layout_cus = pick(Cs);
        c.flags = (int32_t)(next_u64() % 5);  // Direct Recv X, one-launch layout, both, and an unknown bit
        c.num_scaleout_ranks = (int32_t)(next_u64() % 4);
        ep_sizes_t s;
        if (ep_query_sizes(&c, &s) != EP_OK) continue;
        ++accepted;
        if (s.recv_x > (1ull << 34)) ++large;
        if (s.recv_rows > (uint64_t)INT32_MAX || s.layout_scratch == 0) {
            printf("configuration %ld: receive rows %llu or layout scratch %llu out of range\n", it,
                   (unsigned long long)s.recv_rows, (unsigned long long)s.layout_scratch);
            return 1;
        }
        if (ep_layout(&c, nullptr, nullptr, nullptr) == EP_OK ||
            ep_layout_no_alloc(&c, nullptr, nullptr, nullptr) == EP_OK ||
            ep_dispatch(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, EP_PHASE_ALL, nullptr) == EP_OK ||
            ep_layout_dispatch(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == EP_OK ||
            ep_combine(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == EP_OK) {
            printf("configuration %ld: a call accepted missing buffers\n", it);
            return 1;
        }
    }
    printf("%ld configurations, %ld accepted, %ld with receive rows over 16 GiB: ok\n", n, accepted, large);
    return 0;
}
