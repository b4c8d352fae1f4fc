// Host-side stand-ins for the kernel launchers of the HIP library, linked with
// abi.cpp into a CPU program built with the address and undefined-behaviour
// sanitizers.  Each one records the launch and checks the configuration the
// host code computed against what the kernels assume (grid, lanes, LDS, tree
// walk), so the validation and planning paths of abi.cpp run under the
// sanitizers without a GPU.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gdn_internal.h"

namespace sanitize {
int launches = 0;
int failures = 0;
const int32_t* expected_parent = nullptr;  // the tree the next tree launch must walk (one per launch)
int expected_nodes = 0;
}  // namespace sanitize

#define CHECK(cond)                                                                           \
    do {                                                                                      \
        if (!(cond)) {                                                                        \
            std::fprintf(stderr, "launch check failed: %s (%s:%d)\n", #cond, __FILE__, __LINE__); \
            ++sanitize::failures;                                                             \
        }                                                                                     \
    } while (0)

namespace gdn {

// The depth-first walk must visit every node once, each from its parent's state:
// the previous step's state (no restore) or the fork slot saved after the parent.
static void check_walk(const uint16_t* step, int n, const int32_t* parent, int fork_slots) {
    int slot_node[kMaxForkSlots];
    for (int i = 0; i < kMaxForkSlots; ++i) slot_node[i] = -2;
    int seen[kMaxNodes] = {0};
    int cur = -1;  // the node whose state the registers hold (-1: the cached state)
    int prev_save = -1;  // the slot the previous step saved (the kernel reads a slot one step early)
    for (int i = 0; i < n; ++i) {
        const uint16_t c = step[i];
        const int node = sched_node(c);
        CHECK(node >= 0 && node < n);
        if (node < 0 || node >= n) return;
        int from = cur;
        if (c & kSchedRestore) {
            const int sl = sched_restore_slot(c);
            CHECK(sl < fork_slots);
            CHECK(sl != prev_save);
            from = slot_node[sl];
        }
        CHECK(from == parent[node]);
        CHECK(seen[node] == 0);
        seen[node] = 1;
        cur = node;
        prev_save = -1;
        if (c & kSchedSave) {
            const int sl = sched_save_slot(c);
            CHECK(sl < fork_slots);
            slot_node[sl] = node;
            prev_save = sl;
        }
    }
    for (int i = 0; i < n; ++i) CHECK(seen[i] == 1);
}

hipError_t launch_verify(const VerifyArgs& a, const TreeSched* t, int d_k, int m_groups, int epl, int pm,
                         int waves, size_t lds, int grid, hipStream_t) {
    ++sanitize::launches;
    CHECK(d_k == 32 || d_k == 64 || d_k == 128);
    CHECK(epl == 8 && (m_groups == 1 || m_groups == 2));
    CHECK(waves >= 1 && waves <= 4);
    const int rows_per_wave = m_groups * (64 / (d_k / epl));
    CHECK(a.rows_per_wg == waves * rows_per_wave);
    CHECK(a.rows_per_wg * a.slices == a.d_v);
    CHECK(grid == a.n_seq * a.h_v * a.slices);
    CHECK(lds <= (size_t)kMaxLdsBytes);
    CHECK(pm >= 0 && pm <= 2);
    CHECK(a.group * a.h_qk == a.h_v);
    if (a.accepted_prev != nullptr) {
        // a fused commit reads the previous step's node and writes the state cache
        CHECK(a.persist_prev != nullptr && a.state_w != nullptr);
        if (t != nullptr) CHECK(a.final_prev == nullptr);
    }
    if (t != nullptr) {
        // every step reads a fork slot (slot 0 when it restores nothing)
        const int slots = a.fork_slots < 1 ? 1 : a.fork_slots;
        CHECK(lds >= (size_t)slots * a.rows_per_wg * d_k * 4);
    }
    if (t != nullptr && sanitize::expected_parent != nullptr) {
        const int trees = a.per_seq_tree ? a.n_seq : 1;
        for (int i = 0; i < trees; ++i)
            check_walk(t->step[i], a.n_nodes, sanitize::expected_parent + (size_t)(a.seq0 + i) * a.n_nodes *
                                                                          (a.per_seq_tree ? 1 : 0),
                       a.fork_slots);
    }
    return hipSuccess;
}

hipError_t launch_replay(const VerifyArgs& a, const TreeParents* p, int kind, int d_k, int m_groups, int epl, int,
                         int waves, size_t lds, int grid, hipStream_t) {
    ++sanitize::launches;
    CHECK(kind == kReplayChain || kind == kReplayTree || kind == kReplayVerifyChain);
    CHECK(a.rows_per_wg == waves * m_groups * (64 / (d_k / epl)));
    CHECK(grid == a.n_seq * a.h_v * a.slices);
    CHECK(lds <= (size_t)kMaxLdsBytes);
    if (kind == kReplayTree) {
        CHECK(p != nullptr);
        const int trees = a.per_seq_tree ? a.n_seq : 1;
        for (int i = 0; p != nullptr && i < trees; ++i)
            for (int n = 0; n < a.n_nodes; ++n) CHECK(p->p[i][n] < n);
    }
    return hipSuccess;
}

hipError_t launch_commit(const CommitArgs& a, bool, int grid, int block, hipStream_t) {
    ++sanitize::launches;
    CHECK(block == 256);
    CHECK((long long)a.tiles_per_head * block * 8 >= a.head_elems);
    CHECK(grid == a.batch * a.h_v * a.tiles_per_head);
    return hipSuccess;
}

hipError_t launch_commit_index(const IndexCommitArgs& a, hipStream_t) {
    ++sanitize::launches;
    CHECK((long long)a.draft_row0 + (long long)a.batch * a.n_nodes <= a.n_slots);
    return hipSuccess;
}

hipError_t launch_conv_commit(const ConvArgs& a, const TreeParents* p, int grid, hipStream_t) {
    ++sanitize::launches;
    CHECK(a.keep >= 1 && a.keep <= kMaxConvKeep);
    CHECK(grid % a.wg_per_seq == 0);
    CHECK((long long)a.wg_per_seq * 256 >= a.pieces);
    if (!a.chain) CHECK(p != nullptr);
    return hipSuccess;
}

// the workspace of `units` 64-token chunk units: per value head T' and P (f16 C x C) and
// three gate rows (fp32 C), per q/k head K and Q (f16 C x d_k)
size_t prefill_workspace_bytes(long long units, int h_qk, int h_v, int d_k) {
    const long long C = GDN_PREFILL_CHUNK;
    return (size_t)(units * (h_v * (2 * C * C * 2 + 3 * C * 4) + h_qk * (2 * C * (long long)d_k * 2)));
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillSeqs& s, int d_k, int out_dtype, hipStream_t) {
    ++sanitize::launches;
    CHECK(d_k == 32 || d_k == 64 || d_k == 128);
    CHECK(out_dtype == GDN_F32 || out_dtype == GDN_F16 || out_dtype == GDN_BF16);
    CHECK(a.batch >= 1 && a.units >= 1);
    if (a.varlen) {
        CHECK(a.batch <= kMaxPrefillSeqs);  // the per-sequence tables
        CHECK(s.unit0[0] == 0 && s.unit0[a.batch] == a.units);
        for (int b = 0; b < a.batch; ++b) {
            const int nch = s.unit0[b + 1] - s.unit0[b];
            CHECK(nch == (s.len[b] + GDN_PREFILL_CHUNK - 1) / GDN_PREFILL_CHUNK);
            CHECK(s.len[b] >= 0 && s.tok0[b] >= 0);
        }
    } else {
        CHECK(a.units == a.batch * ((a.T + GDN_PREFILL_CHUNK - 1) / GDN_PREFILL_CHUNK));
    }
    return hipSuccess;
}

}  // namespace gdn
