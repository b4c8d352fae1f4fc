// abi.cpp -- the C entry points declared in gdn.h: host-side validation,
// tree walk planning and launch configuration.  Every check runs before any
// HIP call, so a rejected request enqueues nothing and touches no buffer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "gdn.h"
#include "gdn_internal.h"

using namespace gdn;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dtype(int32_t d) { return d == GDN_F32 || d == GDN_BF16 || d == GDN_F16; }

// Checks shared by verify (chain and tree): sizes, dtypes, pointers.
int check_verify(const gdn_shape* sh, const void* q, const void* k, const void* v, const float* alpha,
                 const float* beta, const float* state, const int32_t* state_slot, const void* out,
                 const void* persist, const float* final_state) {
    if (sh == nullptr) return GDN_ERR_NULL;
    if (sh->batch < 0 || sh->n_nodes < 1 || sh->n_nodes > GDN_MAX_NODES) return GDN_ERR_SHAPE;
    if (sh->h_qk < 1 || sh->h_v < 1 || sh->h_v % sh->h_qk != 0) return GDN_ERR_SHAPE;
    if (sh->d_k != 32 && sh->d_k != 64 && sh->d_k != 128) return GDN_ERR_SHAPE;
    if (sh->d_v < 16 || sh->d_v > 256 || sh->d_v % 16 != 0) return GDN_ERR_SHAPE;
    if (state_slot != nullptr && sh->n_slots < 1) return GDN_ERR_SHAPE;
    // per-node offsets of persisted states are 32-bit in the kernels
    if ((long long)sh->h_v * sh->d_v * sh->d_k * GDN_MAX_NODES >= (1LL << 32)) return GDN_ERR_SHAPE;
    if (!valid_dtype(sh->qkv_dtype) || !valid_dtype(sh->out_dtype) || !valid_dtype(sh->persist_dtype))
        return GDN_ERR_DTYPE;
    if (sh->qkv_dtype == GDN_F16) return GDN_ERR_DTYPE;
    if (persist != nullptr && sh->persist_dtype == GDN_BF16) return GDN_ERR_DTYPE;
    if (!std::isfinite(sh->scale)) return GDN_ERR_SHAPE;
    if (sh->batch == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !state) return GDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16)) return GDN_ERR_ALIGN;
    if (!aligned(alpha, 4) || !aligned(beta, 4) || !aligned(state_slot, 4)) return GDN_ERR_ALIGN;
    if (!aligned(out, 4) || !aligned(persist, 16) || !aligned(final_state, 16)) return GDN_ERR_ALIGN;
    return GDN_OK;
}

struct VerifyPlan {
    int m_groups, epl, waves, rows_per_wg, slices;
    size_t lds;
};

// LDS staging of one workgroup: k and q rows (fp32), per-node coefficients
// (4 floats), beta * v for the workgroup's rows, and the tree walk.
size_t stage_bytes(int n, int d_k, int rows) {
    const int floats = (2 * n * d_k + 4 * n + n * rows + n + 3) & ~3;
    return (size_t)floats * 4;
}

// Lane layout: 8 state elements per lane and M row groups per wave, so a
// wave holds R = M * 512 / d_k rows.  Large launches at d_k = 128 take two row
// groups (bandwidth-bound; halves the per-node LDS traffic of k and q per
// row); small ones take one (more waves in flight for a batch-1 step).  Waves
// per workgroup: the most (<= 4) whose rows divide d_v and whose LDS fits.
// (A 16-element layout -- one wave per SIMD at batch 1 -- measured slower:
// verify 11.3 us against 10.0 us, the tree 19.8 us against 15.0 us.  Eight
// waves per workgroup at batch 1 -- half the workgroups, half the staging --
// measured the same: fused step 10.7-11.8 us against 10.7 us.)
// A tree walk reads a fork slot every step (slot 0 when the step restores
// nothing), so a tree launch reserves at least one slot.
int plan_verify(const gdn_shape* sh, int fork_slots, VerifyPlan* p, int blocks = 1, bool tree = false) {
    const int rpg = 512 / sh->d_k;
    int m = 1;
    const long long waves_m1 = (long long)sh->batch * sh->h_v * (sh->d_v / rpg);
    if (sh->d_k == 128 && fork_slots == 0 && waves_m1 >= 16384 && sh->d_v % (2 * rpg) == 0) m = 2;
    const int R = m * rpg;
    if (sh->d_v % R != 0) return GDN_ERR_UNSUPPORTED;
    for (int w = 4; w >= 1; w /= 2) {
        if (sh->d_v % (w * R) != 0) continue;
        const int rows = w * R;
        const size_t lds = (size_t)blocks * stage_bytes(sh->n_nodes, sh->d_k, rows) +
                           (size_t)(tree && fork_slots < 1 ? 1 : fork_slots) * rows * sh->d_k * 4;
        if (lds > (size_t)kMaxLdsBytes) continue;
        p->m_groups = m;
        p->epl = 8;
        p->waves = w;
        p->rows_per_wg = rows;
        p->slices = sh->d_v / rows;
        p->lds = lds;
        return GDN_OK;
    }
    return GDN_ERR_UNSUPPORTED;
}

VerifyArgs make_args(const gdn_shape* sh, const VerifyPlan& p, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* state, const int32_t* state_slot,
                     void* out, void* persist, float* final_state, int32_t* status) {
    VerifyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.state_slot = state_slot;
    a.out = out; a.persist = persist; a.final_state = final_state; a.status = status;
    a.seq0 = 0; a.n_seq = sh->batch; a.batch = sh->batch; a.n_nodes = sh->n_nodes; a.h_qk = sh->h_qk; a.h_v = sh->h_v;
    a.d_v = sh->d_v; a.n_slots = sh->n_slots; a.group = sh->h_v / sh->h_qk;
    a.rows_per_wg = p.rows_per_wg; a.slices = p.slices;
    a.qkv_bf16 = sh->qkv_dtype == GDN_BF16; a.out_dtype = sh->out_dtype;
    a.fork_slots = 0; a.per_seq_tree = 0; a.scale = sh->scale;
    // Write-once outputs go out with non-temporal stores in small launches (measured
    // faster at batch 1: the end-of-kernel drain is shorter) and with plain stores in
    // large ones (measured faster at 384 units); the switch is at 256 MB of states written.
    const size_t pbytes = persist == nullptr ? 0 : (sh->persist_dtype == GDN_F16 ? 2 : 4);
    const double written = (double)sh->batch * sh->n_nodes * sh->h_v * sh->d_v * sh->d_k * pbytes;
    a.nt_stores = written < 256.0 * (1 << 20);
    return a;
}

int persist_mode(const gdn_shape* sh, const void* persist) {
    if (persist == nullptr) return 0;
    return sh->persist_dtype == GDN_F16 ? 1 : 2;
}

// Validate one parent array and write its depth-first walk.  Children are
// visited in index order; a node with two or more children is saved to the
// next free fork slot after it is computed and released when its last child
// starts, so live slots form a stack along the current root path (at most
// depth - 1 of them).  A restored slot is live from its save to the restore,
// so no step in between writes it; in particular a step never restores the
// slot the step before it saved (the kernel reads a step's slot one step early).
int plan_tree(const int32_t* par, int n, uint16_t* walk, int* max_slots) {
    int depth[GDN_MAX_NODES], nchild[GDN_MAX_NODES], started[GDN_MAX_NODES], slot_of[GDN_MAX_NODES];
    int first_child[GDN_MAX_NODES], next_sib[GDN_MAX_NODES], last_child[GDN_MAX_NODES];
    if (par[0] != -1) return GDN_ERR_PARENT;
    for (int i = 0; i < n; ++i) {
        nchild[i] = 0; started[i] = 0; slot_of[i] = -1; first_child[i] = -1; next_sib[i] = -1; last_child[i] = -1;
    }
    depth[0] = 1;
    for (int i = 1; i < n; ++i) {
        const int p = par[i];
        if (p < 0 || p >= i) return GDN_ERR_PARENT;
        depth[i] = depth[p] + 1;
        if (depth[i] > GDN_MAX_TREE_DEPTH) return GDN_ERR_PARENT;
        ++nchild[p];
        if (first_child[p] < 0) first_child[p] = i; else next_sib[last_child[p]] = i;
        last_child[p] = i;
    }
    int stack[GDN_MAX_NODES], sp = 0, top = 0, prev = -1, steps = 0, prev_save = -1;
    stack[sp++] = 0;
    while (sp > 0) {
        const int x = stack[--sp];
        uint16_t code = (uint16_t)x;
        if (x != 0) {
            const int p = par[x];
            if (p != prev) {
                if (slot_of[p] < 0 || slot_of[p] != top - 1 || slot_of[p] == prev_save)
                    return GDN_ERR_PARENT;  // cannot happen
                code |= kSchedRestore | (uint16_t)(slot_of[p] << 6);
            }
            if (++started[p] == nchild[p] && nchild[p] >= 2) { --top; slot_of[p] = -1; }
        }
        prev_save = -1;
        if (nchild[x] >= 2) {
            if (top >= kMaxForkSlots) return GDN_ERR_PARENT;
            prev_save = top;
            slot_of[x] = top++;
            code |= kSchedSave | (uint16_t)(slot_of[x] << 11);
            if (top > *max_slots) *max_slots = top;
        }
        walk[steps++] = code;
        prev = x;
        // push children so the lowest index is visited first
        int kids[GDN_MAX_NODES], nk = 0;
        for (int c = first_child[x]; c >= 0; c = next_sib[c]) kids[nk++] = c;
        for (int i = nk - 1; i >= 0; --i) stack[sp++] = kids[i];
    }
    return steps == n ? GDN_OK : GDN_ERR_PARENT;
}

}  // namespace

extern "C" {

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "a size is out of range or inconsistent";
        case GDN_ERR_DTYPE: return "dtype not allowed here";
        case GDN_ERR_ALIGN: return "pointer not aligned as required";
        case GDN_ERR_PARENT: return "parent array is not a valid tree";
        case GDN_ERR_NODE: return "accepted node out of range";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_UNSUPPORTED: return "request not supported by this library";
        case GDN_ERR_HIP: return "HIP launch failed";
        case GDN_ERR_SLOT: return "state slot out of range";
        case GDN_ERR_RANGE: return "a prefill value is outside the f16 range";
        case GDN_ERR_INTERNAL: return "an index check of the debug build failed";
        default: return "unknown status";
    }
}

int gdn_tree_walk(const int32_t* parent, int32_t n_nodes, uint16_t* walk, int32_t* fork_slots) {
    if (parent == nullptr || walk == nullptr || fork_slots == nullptr) return GDN_ERR_NULL;
    if (n_nodes < 1 || n_nodes > GDN_MAX_NODES) return GDN_ERR_SHAPE;
    int slots = 0;
    const int rc = plan_tree(parent, n_nodes, walk, &slots);
    *fork_slots = rc == GDN_OK ? slots : 0;
    return rc;
}

int gdn_verify_chain(const gdn_shape* shape, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* state,
                     const int32_t* state_slot, void* out, void* persist, float* final_state,
                     int32_t* status, void* stream) {
    int rc = check_verify(shape, q, k, v, alpha, beta, state, state_slot, out, persist, final_state);
    if (rc != GDN_OK || shape->batch == 0) return rc;
    if (final_state == state && state_slot != nullptr) return GDN_ERR_SHAPE;  // in-place needs slot = b
    VerifyPlan p;
    if ((rc = plan_verify(shape, 0, &p)) != GDN_OK) return rc;
    VerifyArgs a = make_args(shape, p, q, k, v, alpha, beta, state, state_slot, out, persist, final_state, status);
    const long long grid = (long long)shape->batch * shape->h_v * p.slices;
    if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
    hipError_t e = launch_verify(a, nullptr, shape->d_k, p.m_groups, p.epl, persist_mode(shape, persist), p.waves,
                                 p.lds, (int)grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_commit_verify_chain(const gdn_shape* shape, const int32_t* accepted_prev, const void* persist_prev,
                            const float* final_prev, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                            void* out, void* persist, float* final_state, int32_t* status, void* stream) {
    int rc = check_verify(shape, q, k, v, alpha, beta, state, state_slot, out, persist, final_state);
    if (rc != GDN_OK || shape->batch == 0) return rc;
    if (accepted_prev == nullptr || persist_prev == nullptr) return GDN_ERR_NULL;
    if (shape->persist_dtype != GDN_F16 && shape->persist_dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (!aligned(accepted_prev, 4) || !aligned(persist_prev, 16) || !aligned(final_prev, 16)) return GDN_ERR_ALIGN;
    if (final_state != nullptr && final_state == state) return GDN_ERR_SHAPE;
    VerifyPlan p;
    if ((rc = plan_verify(shape, 0, &p)) != GDN_OK) return rc;
    VerifyArgs a = make_args(shape, p, q, k, v, alpha, beta, state, state_slot, out, persist, final_state, status);
    a.accepted_prev = accepted_prev;
    a.persist_prev = persist_prev;
    a.final_prev = final_prev;
    a.state_w = state;
    a.persist_prev_f16 = shape->persist_dtype == GDN_F16;
    const long long grid = (long long)shape->batch * shape->h_v * p.slices;
    if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
    hipError_t e = launch_verify(a, nullptr, shape->d_k, p.m_groups, p.epl, persist_mode(shape, persist), p.waves,
                                 p.lds, (int)grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

namespace {

// The previous step's accepted node, committed inside a tree verify's state load.
struct TreeCommit {
    const int32_t* accepted_prev;
    const void* persist_prev;
    float* state;
};

// Walk planning and launches of a tree verify (fused with the commit of the
// previous step when `commit` is set).  Every tree is validated before anything
// is launched; one tree per sequence goes kTreesPerLaunch sequences per launch.
int tree_verify(const gdn_shape* shape, const int32_t* parent, int32_t n_trees, const void* q, const void* k,
                const void* v, const float* alpha, const float* beta, const float* state,
                const int32_t* state_slot, void* out, void* persist, int32_t* status, const TreeCommit* commit,
                void* stream) {
    if (parent == nullptr) return GDN_ERR_NULL;
    const int B = shape->batch, N = shape->n_nodes;
    if (!(n_trees == 1 || (n_trees == B && B > 0))) return GDN_ERR_SHAPE;
    int rc, max_slots = 0;
    uint16_t walk[GDN_MAX_NODES];
    for (int t = 0; t < n_trees; ++t)
        if ((rc = plan_tree(parent + (size_t)t * N, N, walk, &max_slots)) != GDN_OK) return rc;
    if (B == 0) return GDN_OK;
    VerifyPlan p;
    if ((rc = plan_verify(shape, max_slots, &p, 1, true)) != GDN_OK) return rc;
    VerifyArgs a = make_args(shape, p, q, k, v, alpha, beta, state, state_slot, out, persist, nullptr, status);
    a.fork_slots = max_slots;
    if (commit != nullptr) {
        a.accepted_prev = commit->accepted_prev;
        a.persist_prev = commit->persist_prev;
        a.state_w = commit->state;
        a.persist_prev_f16 = shape->persist_dtype == GDN_F16;
    }
    const int pm = persist_mode(shape, persist);
    TreeSched ts;
    std::memset(&ts, 0, sizeof(ts));
    if (n_trees == 1) {
        plan_tree(parent, N, ts.step[0], &max_slots);
        a.per_seq_tree = 0;
        const long long grid = (long long)B * shape->h_v * p.slices;
        if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
        hipError_t e = launch_verify(a, &ts, shape->d_k, p.m_groups, p.epl, pm, p.waves, p.lds, (int)grid,
                                     static_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    a.per_seq_tree = 1;
    for (int s0 = 0; s0 < B; s0 += kTreesPerLaunch) {
        const int ns = (B - s0 < kTreesPerLaunch) ? (B - s0) : kTreesPerLaunch;
        for (int t = 0; t < ns; ++t) plan_tree(parent + (size_t)(s0 + t) * N, N, ts.step[t], &max_slots);
        a.seq0 = s0;
        a.n_seq = ns;
        const int grid = ns * shape->h_v * p.slices;
        hipError_t e = launch_verify(a, &ts, shape->d_k, p.m_groups, p.epl, pm, p.waves, p.lds, grid,
                                     static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

}  // namespace

int gdn_verify_tree(const gdn_shape* shape, const int32_t* parent, int32_t n_trees, const void* q,
                    const void* k, const void* v, const float* alpha, const float* beta,
                    const float* state, const int32_t* state_slot, void* out, void* persist,
                    int32_t* status, void* stream) {
    const int rc = check_verify(shape, q, k, v, alpha, beta, state, state_slot, out, persist, nullptr);
    if (rc != GDN_OK) return rc;
    return tree_verify(shape, parent, n_trees, q, k, v, alpha, beta, state, state_slot, out, persist, status,
                       nullptr, stream);
}

int gdn_commit_verify_tree(const gdn_shape* shape, const int32_t* accepted_prev, const void* persist_prev,
                           const int32_t* parent, int32_t n_trees, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                           void* out, void* persist, int32_t* status, void* stream) {
    const int rc = check_verify(shape, q, k, v, alpha, beta, state, state_slot, out, persist, nullptr);
    if (rc != GDN_OK) return rc;
    if (shape->batch > 0 && (accepted_prev == nullptr || persist_prev == nullptr)) return GDN_ERR_NULL;
    if (shape->persist_dtype != GDN_F16 && shape->persist_dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (!aligned(accepted_prev, 4) || !aligned(persist_prev, 16)) return GDN_ERR_ALIGN;
    const TreeCommit c{accepted_prev, persist_prev, state};
    return tree_verify(shape, parent, n_trees, q, k, v, alpha, beta, state, state_slot, out, persist, status, &c,
                       stream);
}

int gdn_commit_replay(const gdn_shape* shape, const int32_t* parent, int32_t n_trees,
                      const int32_t* accepted_node, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                      int32_t* status, void* stream) {
    int rc = check_verify(shape, q, k, v, alpha, beta, state, state_slot, nullptr, nullptr, nullptr);
    if (rc != GDN_OK) return rc;
    const int B = shape->batch, N = shape->n_nodes;
    if (parent != nullptr) {
        if (!(n_trees == 1 || (n_trees == B && B > 0))) return GDN_ERR_SHAPE;
        int slots = 0;
        uint16_t walk[GDN_MAX_NODES];
        for (int t = 0; t < n_trees; ++t)
            if ((rc = plan_tree(parent + (size_t)t * N, N, walk, &slots)) != GDN_OK) return rc;
    }
    if (B == 0) return GDN_OK;
    if (accepted_node == nullptr) return GDN_ERR_NULL;
    if (!aligned(accepted_node, 4)) return GDN_ERR_ALIGN;
    VerifyPlan p;
    if ((rc = plan_verify(shape, 0, &p)) != GDN_OK) return rc;
    VerifyArgs a = make_args(shape, p, q, k, v, alpha, beta, state, state_slot, nullptr, nullptr, nullptr, status);
    a.accepted_prev = accepted_node;
    a.state_w = state;
    a.nt_stores = (double)B * shape->h_v * shape->d_v * shape->d_k * 4 < 256.0 * (1 << 20);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (parent == nullptr) {
        const long long grid = (long long)B * shape->h_v * p.slices;
        if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
        hipError_t e = launch_replay(a, nullptr, kReplayChain, shape->d_k, p.m_groups, p.epl, 0, p.waves, p.lds, (int)grid, st);
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    TreeParents tp;
    std::memset(&tp, 0, sizeof(tp));
    const int per_seq = n_trees > 1;
    a.per_seq_tree = per_seq;
    const int span = per_seq ? kTreesPerLaunch : B;
    for (int s0 = 0; s0 < B; s0 += span) {
        const int ns = (B - s0 < span) ? (B - s0) : span;
        for (int t = 0; t < (per_seq ? ns : 1); ++t)
            for (int n = 0; n < N; ++n) tp.p[t][n] = (int8_t)parent[(size_t)(per_seq ? s0 + t : 0) * N + n];
        a.seq0 = s0;
        a.n_seq = ns;
        const long long grid = (long long)ns * shape->h_v * p.slices;
        if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
        hipError_t e = launch_replay(a, &tp, kReplayTree, shape->d_k, p.m_groups, p.epl, 0, p.waves, p.lds, (int)grid, st);
        if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

int gdn_replay_verify_chain(const gdn_shape* shape, const int32_t* accepted_prev, const void* q_prev,
                            const void* k_prev, const void* v_prev, const float* alpha_prev,
                            const float* beta_prev, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                            void* out, void* persist, float* final_state, int32_t* status, void* stream) {
    int rc = check_verify(shape, q, k, v, alpha, beta, state, state_slot, out, persist, final_state);
    if (rc != GDN_OK || shape->batch == 0) return rc;
    if (!accepted_prev || !q_prev || !k_prev || !v_prev || !alpha_prev || !beta_prev) return GDN_ERR_NULL;
    if (!aligned(accepted_prev, 4) || !aligned(alpha_prev, 4) || !aligned(beta_prev, 4)) return GDN_ERR_ALIGN;
    if (!aligned(q_prev, 16) || !aligned(k_prev, 16) || !aligned(v_prev, 16)) return GDN_ERR_ALIGN;
    if (final_state != nullptr && final_state == state) return GDN_ERR_SHAPE;
    VerifyPlan p;
    if ((rc = plan_verify(shape, 0, &p, 2)) != GDN_OK) return rc;
    VerifyArgs a = make_args(shape, p, q, k, v, alpha, beta, state, state_slot, out, persist, final_state, status);
    a.accepted_prev = accepted_prev;
    a.state_w = state;
    a.rq = q_prev; a.rk = k_prev; a.rv = v_prev; a.ralpha = alpha_prev; a.rbeta = beta_prev;
    {
        const double head = (double)shape->batch * shape->h_v * shape->d_v * shape->d_k;
        const size_t pb = persist == nullptr ? 0 : (shape->persist_dtype == GDN_F16 ? 2 : 4);
        const double written = head * (4 + (final_state ? 4 : 0) + (double)shape->n_nodes * pb);
        a.nt_stores = written < 256.0 * (1 << 20);
    }
    const long long grid = (long long)shape->batch * shape->h_v * p.slices;
    if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
    hipError_t e = launch_replay(a, nullptr, kReplayVerifyChain, shape->d_k, p.m_groups, p.epl, persist_mode(shape, persist),
                                 p.waves, p.lds, (int)grid, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_commit(const gdn_shape* shape, const int32_t* accepted_node, const void* persist,
               const float* final_state, float* state, const int32_t* state_slot, int32_t* status,
               void* stream) {
    if (shape == nullptr) return GDN_ERR_NULL;
    const gdn_shape* sh = shape;
    if (sh->batch < 0 || sh->n_nodes < 1 || sh->n_nodes > GDN_MAX_NODES || sh->h_v < 1) return GDN_ERR_SHAPE;
    if (sh->d_k != 32 && sh->d_k != 64 && sh->d_k != 128) return GDN_ERR_SHAPE;
    if (sh->d_v < 16 || sh->d_v > 256 || sh->d_v % 16 != 0) return GDN_ERR_SHAPE;
    if (state_slot != nullptr && sh->n_slots < 1) return GDN_ERR_SHAPE;
    if (sh->persist_dtype != GDN_F16 && sh->persist_dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (sh->batch == 0) return GDN_OK;
    if (!accepted_node || !persist || !state) return GDN_ERR_NULL;
    if (!aligned(persist, 16) || !aligned(state, 16) || !aligned(final_state, 16)) return GDN_ERR_ALIGN;
    if (!aligned(accepted_node, 4) || !aligned(state_slot, 4)) return GDN_ERR_ALIGN;
    CommitArgs a;
    std::memset(&a, 0, sizeof(a));
    a.accepted = accepted_node; a.persist = persist; a.final_state = final_state; a.state = state;
    a.state_slot = state_slot; a.status = status; a.batch = sh->batch; a.n_nodes = sh->n_nodes;
    a.h_v = sh->h_v; a.head_elems = sh->d_v * sh->d_k; a.n_slots = sh->n_slots;
    const int block = 256;
    a.tiles_per_head = (a.head_elems / 8 + block - 1) / block;
    const long long grid = (long long)sh->batch * sh->h_v * a.tiles_per_head;
    if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
    hipError_t e = launch_commit(a, sh->persist_dtype == GDN_F16, (int)grid, block, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_commit_index(const int32_t* accepted_node, int32_t* state_slot, int32_t batch, int32_t n_nodes,
                     int32_t draft_row0, int32_t n_slots, int32_t* status, void* stream) {
    if (batch < 0 || n_nodes < 1 || n_nodes > GDN_MAX_NODES || draft_row0 < 0 || n_slots < 1) return GDN_ERR_SHAPE;
    if ((long long)draft_row0 + (long long)batch * n_nodes > n_slots) return GDN_ERR_SHAPE;
    if (batch == 0) return GDN_OK;
    if (accepted_node == nullptr || state_slot == nullptr) return GDN_ERR_NULL;
    if (!aligned(accepted_node, 4) || !aligned(state_slot, 4) || !aligned(status, 4)) return GDN_ERR_ALIGN;
    IndexCommitArgs a;
    a.accepted = accepted_node; a.state_slot = state_slot; a.status = status; a.batch = batch;
    a.n_nodes = n_nodes; a.draft_row0 = draft_row0; a.n_slots = n_slots;
    return launch_commit_index(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_conv_commit(const gdn_conv_shape* shape, const int32_t* parent, int32_t n_trees,
                    const int32_t* accepted_node, const void* x, void* conv_state,
                    const int32_t* state_slot, int32_t* status, void* stream) {
    if (shape == nullptr) return GDN_ERR_NULL;
    const gdn_conv_shape* sh = shape;
    if (sh->batch < 0 || sh->n_nodes < 1 || sh->n_nodes > GDN_MAX_NODES) return GDN_ERR_SHAPE;
    if (sh->width < 2 || sh->width > GDN_MAX_CONV_WIDTH || sh->channels < 1) return GDN_ERR_SHAPE;
    if (state_slot != nullptr && sh->n_slots < 1) return GDN_ERR_SHAPE;
    if (!valid_dtype(sh->dtype)) return GDN_ERR_DTYPE;
    const long long row = (long long)sh->channels * (sh->dtype == GDN_F32 ? 4 : 2);
    if (row % 16 != 0 || row / 16 > 0x7fffffffLL) return GDN_ERR_SHAPE;
    const int B = sh->batch, N = sh->n_nodes;
    int rc;
    if (parent != nullptr) {
        if (!(n_trees == 1 || (n_trees == B && B > 0))) return GDN_ERR_SHAPE;
        int slots = 0;
        uint16_t walk[GDN_MAX_NODES];
        for (int t = 0; t < n_trees; ++t)
            if ((rc = plan_tree(parent + (size_t)t * N, N, walk, &slots)) != GDN_OK) return rc;
    }
    if (B == 0) return GDN_OK;
    if (!accepted_node || !x || !conv_state) return GDN_ERR_NULL;
    if (!aligned(x, 16) || !aligned(conv_state, 16)) return GDN_ERR_ALIGN;
    if (!aligned(accepted_node, 4) || !aligned(state_slot, 4)) return GDN_ERR_ALIGN;
    ConvArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = static_cast<const unsigned char*>(x);
    a.hist = static_cast<unsigned char*>(conv_state);
    a.accepted = accepted_node; a.state_slot = state_slot; a.status = status;
    a.n_nodes = N; a.keep = sh->width - 1; a.pieces = (int32_t)(row / 16); a.n_slots = sh->n_slots;
    a.batch = B;
    a.wg_per_seq = (a.pieces + 255) / 256;
    a.chain = parent == nullptr;
    a.per_seq_tree = n_trees > 1;
    TreeParents tp;
    std::memset(&tp, 0, sizeof(tp));
    const int span = a.per_seq_tree ? kTreesPerLaunch : B;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int s0 = 0; s0 < B; s0 += span) {
        const int ns = (B - s0 < span) ? (B - s0) : span;
        if (parent != nullptr)
            for (int t = 0; t < (a.per_seq_tree ? ns : 1); ++t)
                for (int n = 0; n < N; ++n)
                    tp.p[t][n] = (int8_t)parent[(size_t)(a.per_seq_tree ? s0 + t : 0) * N + n];
        a.seq0 = s0;
        const long long grid = (long long)ns * a.wg_per_seq;
        if (grid > 0x7fffffffLL) return GDN_ERR_SHAPE;
        if (launch_conv_commit(a, &tp, (int)grid, st) != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

namespace {
int check_prefill(const gdn_shape* sh) {
    if (sh == nullptr) return GDN_ERR_NULL;
    if (sh->batch < 0 || sh->n_nodes < 0) return GDN_ERR_SHAPE;
    if (sh->h_qk < 1 || sh->h_v < 1 || sh->h_v % sh->h_qk != 0) return GDN_ERR_SHAPE;
    if (sh->d_k != 32 && sh->d_k != 64 && sh->d_k != 128) return GDN_ERR_SHAPE;
    if (sh->d_v < 32 || sh->d_v > 256 || sh->d_v % 32 != 0) return GDN_ERR_SHAPE;
    if (sh->h_v / sh->h_qk > 128) return GDN_ERR_UNSUPPORTED;  // the prepare kernel keeps every group's gates in LDS
    if (sh->qkv_dtype != GDN_F32 && sh->qkv_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (!valid_dtype(sh->out_dtype)) return GDN_ERR_DTYPE;
    if (!std::isfinite(sh->scale)) return GDN_ERR_SHAPE;
    return GDN_OK;
}
}  // namespace

}  // extern "C"

namespace gdn {
int check_prefill_call(const gdn_shape* sh, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const float* state, const int32_t* state_slot, const void* out,
                       bool* empty) {
    *empty = false;
    const int rc = check_prefill(sh);
    if (rc != GDN_OK) return rc;
    if (state_slot != nullptr && sh->n_slots < 1) return GDN_ERR_SHAPE;
    if (sh->batch == 0 || sh->n_nodes == 0) {
        *empty = true;
        return GDN_OK;
    }
    if ((long long)sh->batch * sh->n_nodes > 0x7fffffffLL) return GDN_ERR_SHAPE;
    if (!q || !k || !v || !alpha || !beta || !state || !out) return GDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return GDN_ERR_ALIGN;
    if (!aligned(alpha, 4) || !aligned(beta, 4) || !aligned(state, 4) || !aligned(state_slot, 4))
        return GDN_ERR_ALIGN;
    return GDN_OK;
}
}  // namespace gdn

extern "C" {

size_t gdn_prefill_workspace_bytes(const gdn_shape* shape) {
    if (check_prefill(shape) != GDN_OK || shape->batch == 0 || shape->n_nodes == 0) return 0;
    const long long units = (long long)shape->batch * ((shape->n_nodes + GDN_PREFILL_CHUNK - 1) / GDN_PREFILL_CHUNK);
    return prefill_workspace_bytes(units, shape->h_qk, shape->h_v, shape->d_k);
}

int gdn_prefill_chunked(const gdn_shape* shape, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, float* state, const int32_t* state_slot,
                        void* out, void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
    bool empty = false;
    const int rc = gdn::check_prefill_call(shape, q, k, v, alpha, beta, state, state_slot, out, &empty);
    if (rc != GDN_OK || empty) return rc;
    const gdn_shape* sh = shape;
    const size_t need = gdn_prefill_workspace_bytes(sh);
    if (workspace == nullptr || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GDN_ERR_ALIGN;
    PrefillArgs a;
    std::memset(&a, 0, sizeof(a));
    a.workspace = workspace;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.state_slot = state_slot;
    a.out = out; a.status = status; a.batch = sh->batch; a.T = sh->n_nodes; a.h_qk = sh->h_qk; a.h_v = sh->h_v;
    a.d_v = sh->d_v; a.group = sh->h_v / sh->h_qk; a.slices = sh->d_v / 32; a.n_slots = sh->n_slots;
    a.qkv_bf16 = sh->qkv_dtype == GDN_BF16; a.scale = sh->scale;
    a.varlen = 0;
    a.units = sh->batch * ((sh->n_nodes + GDN_PREFILL_CHUNK - 1) / GDN_PREFILL_CHUNK);
    a.batch_total = sh->batch;
    a.tokens_total = (int64_t)sh->batch * sh->n_nodes;
    PrefillSeqs seqs;
    std::memset(&seqs, 0, sizeof(seqs));
    hipError_t e = launch_prefill(a, seqs, sh->d_k, sh->out_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

namespace {
// cu_seqlens: batch + 1 nondecreasing offsets from 0 to the total token count.
int check_cu_seqlens(const int32_t* cu, int batch, int total) {
    if (cu == nullptr) return GDN_ERR_NULL;
    if (cu[0] != 0 || cu[batch] != total) return GDN_ERR_SHAPE;
    for (int b = 0; b < batch; ++b)
        if (cu[b + 1] < cu[b]) return GDN_ERR_SHAPE;
    return GDN_OK;
}
long long chunks_of(int T) { return (T + GDN_PREFILL_CHUNK - 1) / GDN_PREFILL_CHUNK; }
}  // namespace

int64_t gdn_prefill_boundary_states(const int32_t* cu_seqlens, int32_t batch, int32_t state_interval) {
    if (cu_seqlens == nullptr || batch < 0 || state_interval < 1) return -1;
    if (check_cu_seqlens(cu_seqlens, batch, cu_seqlens[batch]) != GDN_OK) return -1;
    int64_t n = 0;
    for (int b = 0; b < batch; ++b)
        n += (cu_seqlens[b + 1] - cu_seqlens[b]) / ((int64_t)GDN_PREFILL_CHUNK * state_interval);
    return n;
}

size_t gdn_prefill_varlen_workspace_bytes(const gdn_shape* shape, const int32_t* cu_seqlens) {
    if (check_prefill(shape) != GDN_OK || shape->batch == 0) return 0;
    if (check_cu_seqlens(cu_seqlens, shape->batch, shape->n_nodes) != GDN_OK) return 0;
    // launches take up to kMaxPrefillSeqs sequences each and reuse the workspace in turn
    long long most = 0;
    for (int s0 = 0; s0 < shape->batch; s0 += kMaxPrefillSeqs) {
        long long units = 0;
        for (int b = s0; b < shape->batch && b < s0 + kMaxPrefillSeqs; ++b)
            units += chunks_of(cu_seqlens[b + 1] - cu_seqlens[b]);
        if (units > most) most = units;
    }
    return most == 0 ? 0 : prefill_workspace_bytes(most, shape->h_qk, shape->h_v, shape->d_k);
}

int gdn_prefill_varlen(const gdn_shape* shape, const int32_t* cu_seqlens, const void* q, const void* k,
                       const void* v, const float* alpha, const float* beta, float* state,
                       const int32_t* state_slot, void* out, float* chunk_states, int32_t state_interval,
                       void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
    int rc = check_prefill(shape);
    if (rc != GDN_OK) return rc;
    const gdn_shape* sh = shape;
    if (state_slot != nullptr && sh->n_slots < 1) return GDN_ERR_SHAPE;
    if (sh->batch == 0) return GDN_OK;
    if ((rc = check_cu_seqlens(cu_seqlens, sh->batch, sh->n_nodes)) != GDN_OK) return rc;
    if (chunk_states != nullptr && state_interval < 1) return GDN_ERR_SHAPE;
    if (sh->n_nodes == 0) return GDN_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !out) return GDN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return GDN_ERR_ALIGN;
    if (!aligned(alpha, 4) || !aligned(beta, 4) || !aligned(state, 4) || !aligned(state_slot, 4) ||
        !aligned(chunk_states, 4))
        return GDN_ERR_ALIGN;
    const size_t need = gdn_prefill_varlen_workspace_bytes(sh, cu_seqlens);
    if (workspace == nullptr || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GDN_ERR_ALIGN;
    PrefillArgs a;
    std::memset(&a, 0, sizeof(a));
    a.workspace = workspace;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.state_slot = state_slot;
    a.out = out; a.status = status; a.T = 0; a.h_qk = sh->h_qk; a.h_v = sh->h_v;
    a.d_v = sh->d_v; a.group = sh->h_v / sh->h_qk; a.slices = sh->d_v / 32; a.n_slots = sh->n_slots;
    a.qkv_bf16 = sh->qkv_dtype == GDN_BF16; a.scale = sh->scale;
    a.varlen = 1;
    a.chunk_states = chunk_states;
    a.state_interval = chunk_states != nullptr ? state_interval : 1;
    a.batch_total = sh->batch;
    a.tokens_total = sh->n_nodes;
    a.n_chunk_states = chunk_states != nullptr ? gdn_prefill_boundary_states(cu_seqlens, sh->batch, state_interval) : 0;
    const long long span = (long long)GDN_PREFILL_CHUNK * a.state_interval;
    long long cst = 0;
    for (int s0 = 0; s0 < sh->batch; s0 += kMaxPrefillSeqs) {
        const int ns = sh->batch - s0 < kMaxPrefillSeqs ? sh->batch - s0 : kMaxPrefillSeqs;
        PrefillSeqs seqs;
        std::memset(&seqs, 0, sizeof(seqs));
        long long units = 0;
        for (int i = 0; i <= ns; ++i) {
            seqs.unit0[i] = (int32_t)units;
            seqs.cst0[i] = (int32_t)cst;
            if (i < ns) {
                const int T = cu_seqlens[s0 + i + 1] - cu_seqlens[s0 + i];
                seqs.tok0[i] = cu_seqlens[s0 + i];
                seqs.len[i] = T;
                units += chunks_of(T);
                cst += T / span;
            }
        }
        if (units == 0) continue;
        if (cst > 0x7fffffffLL) return GDN_ERR_SHAPE;
        a.batch = ns;
        a.seq0 = s0;
        a.units = (int32_t)units;
        hipError_t e = launch_prefill(a, seqs, sh->d_k, sh->out_dtype, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

}  // extern "C"
