// Drives the C entry points of abi.cpp on the host (launchers stubbed by
// abi_stubs.cpp) with random valid and invalid requests, under the address and
// undefined-behaviour sanitizers.  Pointers are fake aligned addresses: no
// request reaches a device.  Exit status 0 when every return code is one the
// request allows and every launch plan passed the stubs' checks.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "gdn.h"

namespace sanitize {
extern int launches;
extern int failures;
extern const int32_t* expected_parent;
}  // namespace sanitize

static int bad = 0;
#define EXPECT(cond)                                                                   \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            std::fprintf(stderr, "expectation failed: %s (line %d)\n", #cond, __LINE__); \
            ++bad;                                                                     \
        }                                                                              \
    } while (0)

static void* const F = reinterpret_cast<void*>(0x10000);  // 16-byte aligned, never dereferenced
static float* const FF = reinterpret_cast<float*>(0x10000);

static gdn_shape shape(int B, int N, int hqk, int hv, int dk, int dv, int qkv = GDN_BF16, int out = GDN_F32,
                       int pers = GDN_F16) {
    gdn_shape s;
    s.batch = B; s.n_nodes = N; s.h_qk = hqk; s.h_v = hv; s.d_k = dk; s.d_v = dv; s.n_slots = B > 0 ? B : 1;
    s.qkv_dtype = qkv; s.out_dtype = out; s.persist_dtype = pers; s.scale = 1.0f;
    return s;
}

static std::vector<int32_t> random_tree(std::mt19937& rng, int n, int max_depth) {
    std::vector<int32_t> p(n), d(n);
    p[0] = -1; d[0] = 1;
    for (int i = 1; i < n; ++i) {
        std::vector<int> ok;
        for (int j = 0; j < i; ++j)
            if (d[j] < max_depth) ok.push_back(j);
        p[i] = ok[rng() % ok.size()];
        d[i] = d[p[i]] + 1;
    }
    return p;
}

int main() {
    std::mt19937 rng(12345);
    const int dks[3] = {32, 64, 128};
    // trees: every walk visits each node from its parent's state (checked by the stub)
    for (int it = 0; it < 3000; ++it) {
        const int n = 1 + rng() % GDN_MAX_NODES;
        const int B = 1 + rng() % 40;
        const bool per_seq = rng() % 2;
        std::vector<int32_t> par;
        for (int b = 0; b < (per_seq ? B : 1); ++b) {
            auto t = random_tree(rng, n, 2 + rng() % (GDN_MAX_TREE_DEPTH - 1));
            par.insert(par.end(), t.begin(), t.end());
        }
        uint16_t walk[GDN_MAX_NODES];
        int32_t slots = -1;
        EXPECT(gdn_tree_walk(par.data(), n, walk, &slots) == GDN_OK);
        EXPECT(slots >= 0 && slots < GDN_MAX_TREE_DEPTH);
        const int dk = dks[rng() % 3];
        const int hqk = 1 + rng() % 4, hv = hqk * (1 + rng() % 6), dv = 16 * (1 + rng() % 16);
        gdn_shape s = shape(B, n, hqk, hv, dk, dv);
        sanitize::expected_parent = par.data();
        const int rc = gdn_verify_tree(&s, par.data(), per_seq ? B : 1, F, F, F, FF, FF, FF, nullptr, F, F,
                                       nullptr, nullptr);
        EXPECT(rc == GDN_OK || rc == GDN_ERR_UNSUPPORTED);
        const int32_t* acc = reinterpret_cast<const int32_t*>(F);
        // the fused commit + tree verify plans the same walks
        const int rcf = gdn_commit_verify_tree(&s, acc, F, par.data(), per_seq ? B : 1, F, F, F, FF, FF, FF,
                                               nullptr, F, F, nullptr, nullptr);
        EXPECT(rcf == rc);
        sanitize::expected_parent = nullptr;
        EXPECT(gdn_commit_replay(&s, par.data(), per_seq ? B : 1, acc, F, F, F, FF, FF, FF, nullptr, nullptr,
                                 nullptr) == GDN_OK);
        gdn_conv_shape cs = {B, n, 8 * (1 + (int)(rng() % 64)), 2 + (int)(rng() % 7), B, GDN_BF16};
        EXPECT(gdn_conv_commit(&cs, par.data(), per_seq ? B : 1, acc, F, F, nullptr, nullptr, nullptr) == GDN_OK);
        // broken trees are refused
        if (n >= 2) {
            std::vector<int32_t> broken(par.begin(), par.begin() + n);
            broken[1 + rng() % (n - 1)] = n;  // a parent that is not earlier
            EXPECT(gdn_tree_walk(broken.data(), n, walk, &slots) == GDN_ERR_PARENT);
            EXPECT(gdn_verify_tree(&s, broken.data(), 1, F, F, F, FF, FF, FF, nullptr, F, F, nullptr, nullptr) ==
                   GDN_ERR_PARENT);
        }
    }
    // chains, fused commits, replays, commits: random shapes, valid and invalid
    for (int it = 0; it < 20000; ++it) {
        const int B = (int)(rng() % 600) - 2, N = (int)(rng() % 36) - 1;
        const int hqk = 1 + rng() % 17, hv = hqk * (1 + rng() % 8) + ((rng() % 9) == 0 ? 1 : 0);
        const int dk = (rng() % 7) == 0 ? 96 : dks[rng() % 3];
        const int dv = (rng() % 9) == 0 ? 24 : 16 * (1 + rng() % 16);
        const int qkv = rng() % 3, out = rng() % 4, pers = rng() % 3;
        gdn_shape s = shape(B, N, hqk, hv, dk, dv, qkv, out, pers);
        const int32_t* acc = reinterpret_cast<const int32_t*>(F);
        int rc = gdn_verify_chain(&s, F, F, F, FF, FF, FF, nullptr, F, F, FF, nullptr, nullptr);
        EXPECT(rc <= 0 && rc >= GDN_ERR_SLOT);
        rc = gdn_commit_verify_chain(&s, acc, F, FF, F, F, F, FF, FF, FF, nullptr, F, F, FF + 4096, nullptr,
                                     nullptr);
        EXPECT(rc <= 0 && rc >= GDN_ERR_SLOT);
        const int32_t chain_par[GDN_MAX_NODES + 1] = {-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15,
                                                      16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31};
        rc = gdn_commit_verify_tree(&s, acc, F, chain_par, 1, F, F, F, FF, FF, FF, nullptr, F, F, nullptr, nullptr);
        EXPECT(rc <= 0 && rc >= GDN_ERR_SLOT);
        rc = gdn_replay_verify_chain(&s, acc, F, F, F, FF, FF, F, F, F, FF, FF, FF, nullptr, F, nullptr, nullptr,
                                     nullptr, nullptr);
        EXPECT(rc <= 0 && rc >= GDN_ERR_SLOT);
        rc = gdn_commit(&s, acc, F, FF, FF, nullptr, nullptr, nullptr);
        EXPECT(rc <= 0 && rc >= GDN_ERR_SLOT);
        rc = gdn_commit_index(acc, reinterpret_cast<int32_t*>(F), B, N, rng() % 4, B * (N > 0 ? N : 1) + 1,
                              nullptr, nullptr);
        EXPECT(rc <= 0 && rc >= GDN_ERR_SLOT);
        const bool valid = B >= 0 && N >= 1 && N <= GDN_MAX_NODES && hv % hqk == 0 && dk != 96 && dv != 24 &&
                           qkv != GDN_F16 && out != 3 && !(pers == GDN_BF16);
        if (valid && B > 0) EXPECT(gdn_verify_chain(&s, F, F, F, FF, FF, FF, nullptr, F, F, FF, nullptr, nullptr) ==
                                   GDN_OK);
    }
    // prefill: equal lengths and packed sequences
    for (int it = 0; it < 5000; ++it) {
        const int B = (int)(rng() % 80), T = (int)(rng() % 3000);
        const int hqk = 1 + rng() % 8, hv = hqk * (1 + rng() % 6), dk = dks[rng() % 3], dv = 32 * (1 + rng() % 8);
        gdn_shape s = shape(B, T, hqk, hv, dk, dv, rng() % 2, rng() % 3);
        const size_t need = gdn_prefill_workspace_bytes(&s);
        int rc = gdn_prefill_chunked(&s, F, F, F, FF, FF, FF, nullptr, F, F, need, nullptr, nullptr);
        EXPECT(rc == GDN_OK);
        if (need > 16)
            EXPECT(gdn_prefill_chunked(&s, F, F, F, FF, FF, FF, nullptr, F, F, need - 16, nullptr, nullptr) ==
                   GDN_ERR_WORKSPACE);
        std::vector<int32_t> cu(B + 1, 0);
        for (int b = 0; b < B; ++b) cu[b + 1] = cu[b] + (int)(rng() % 700);
        s.n_nodes = cu[B];
        const size_t vneed = gdn_prefill_varlen_workspace_bytes(&s, cu.data());
        const int interval = 1 + rng() % 5;
        rc = gdn_prefill_varlen(&s, cu.data(), F, F, F, FF, FF, FF, nullptr, F, FF, interval, F, vneed, nullptr,
                                nullptr);
        EXPECT(rc == GDN_OK);
        EXPECT(gdn_prefill_boundary_states(cu.data(), B, interval) >= 0);
        if (B > 1) {
            std::swap(cu[1], cu[2]);
            if (cu[1] > cu[2])
                EXPECT(gdn_prefill_varlen(&s, cu.data(), F, F, F, FF, FF, FF, nullptr, F, FF, interval, F, vneed,
                                          nullptr, nullptr) == GDN_ERR_SHAPE);
        }
    }
    for (int c = -12; c <= 1; ++c) EXPECT(gdn_status_string(c) != nullptr);
    std::printf("launches %d, launch-check failures %d, expectation failures %d\n", sanitize::launches,
                sanitize::failures, bad);
    return (bad == 0 && sanitize::failures == 0 && sanitize::launches > 0) ? 0 : 1;
}
