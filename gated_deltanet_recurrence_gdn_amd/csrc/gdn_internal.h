// gdn_internal.h -- kernel argument blocks and launch entry points shared by
// the host dispatch (abi.cpp) and the gfx950 kernels (*.hip).  Internal to
// the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"

namespace gdn {

constexpr int kMaxNodes = GDN_MAX_NODES;
constexpr int kTreesPerLaunch = 16;  // tree schedules carried in one kernarg block
constexpr int kMaxForkSlots = GDN_MAX_TREE_DEPTH - 1;
constexpr int kMaxLdsBytes = 160 * 1024;  // LDS of one gfx950 compute unit, all of it usable by one workgroup
constexpr int kDefaultLdsBytes = 64 * 1024;  // dynamic LDS a launch may use without the attribute below
constexpr int kMaxDevices = 64;

// Allows launches of kernel K (a __global__ function) to take up to
// kMaxLdsBytes of dynamic LDS on the current device.  The attribute is set once
// per kernel and device; concurrent first calls may both set it (the call is
// idempotent), and the flag is an atomic, so calls from several host threads
// are safe.
template <auto K>
inline hipError_t allow_max_lds() {
    static std::atomic<uint64_t> done{0};  // bit d: set on device d
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < kMaxDevices ? uint64_t{1} << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(K), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLdsBytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// Compute units of the current device, queried once per device (an atomic cache).
int device_cus();

// One step of a tree walk (depth-first order), packed in 16 bits:
//   bits 0-4   node index
//   bit  5     restore the working state from fork slot (bits 6-9) first
//   bit  10    after the node, save the working state to fork slot (bits 11-14)
// Node 0 (the root) always comes first and starts from the cached state; a
// step without the restore bit continues from the previous step's state.
constexpr uint16_t kSchedRestore = 1u << 5;
constexpr uint16_t kSchedSave = 1u << 10;
__host__ __device__ constexpr int sched_node(uint16_t c) { return c & 31; }
__host__ __device__ constexpr int sched_restore_slot(uint16_t c) { return (c >> 6) & 15; }
__host__ __device__ constexpr int sched_save_slot(uint16_t c) { return (c >> 11) & 15; }

// Index checks of the debug build (-DGDN_DEBUG, the same source): an access
// of `span` elements at index i of an array of n elements that would pass its
// end is reported through the launch's status word (GDN_ERR_INTERNAL) and
// clamped into the array, so it still touches valid memory.  The release
// build compiles the checks away (GDN_AT(i, ...) is i).
#ifdef GDN_DEBUG
__device__ __forceinline__ size_t gdn_checked(size_t i, size_t span, size_t n, int32_t* status) {
    if (i + span <= n) return i;
    if (status != nullptr) status[0] = GDN_ERR_INTERNAL;
    return n >= span ? n - span : 0;
}
#define GDN_AT(i, span, n, status) ::gdn::gdn_checked((size_t)(i), (size_t)(span), (size_t)(n), (status))
#else
#define GDN_AT(i, span, n, status) (i)
#endif

struct VerifyArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* state;
    const int32_t* state_slot;
    void* out;
    void* persist;
    float* final_state;
    int32_t* status;
    int32_t seq0;        // first sequence handled by this launch
    int32_t n_seq;       // sequences handled by this launch
    int32_t batch;       // sequences of the call (the arrays' leading dimension)
    int32_t n_nodes;
    int32_t h_qk;
    int32_t h_v;
    int32_t d_v;
    int32_t n_slots;     // valid slot range when state_slot != nullptr
    int32_t group;       // h_v / h_qk
    int32_t rows_per_wg; // value rows of one head handled by one workgroup
    int32_t slices;      // d_v / rows_per_wg
    int32_t qkv_bf16;    // 1: q, k, v are bf16; 0: fp32
    int32_t out_dtype;   // gdn_dtype
    int32_t fork_slots;  // fork slots reserved in LDS (tree walks)
    int32_t per_seq_tree;// 0: tree 0 for every sequence; 1: tree b - seq0
    float scale;
    // fused commit of the previous step (accepted_prev == nullptr: off; final_prev: chains only)
    const int32_t* accepted_prev;
    const void* persist_prev;
    const float* final_prev;
    float* state_w;      // the state cache written by the fused commit (same buffer as `state`)
    int32_t persist_prev_f16;
    int32_t nt_stores;   // 1: write-once outputs with non-temporal stores
    // commit by replay (replay launches only): the replayed block's inputs; for the
    // replay-only launch they are q, k, v, alpha, beta above and these stay null
    const void* rq;
    const void* rk;
    const void* rv;
    const float* ralpha;
    const float* rbeta;
};

// Parent arrays of up to kTreesPerLaunch trees, for a replay along the root
// path of a node chosen on the device (tree replay launches only).
struct TreeParents {
    int8_t p[kTreesPerLaunch][kMaxNodes];
};

// What a verify-family launch does.
enum VerifyKind : int {
    kVerifyChain = 0,        // chain verify
    kCommitVerifyChain = 5,  // the persisted-copy commit of the previous block fused into a chain verify
    kVerifyTree = 1,         // tree verify, host-planned depth-first walk
    kReplayChain = 2,        // commit by replay of nodes 0 .. accepted
    kReplayTree = 3,         // commit by replay of the accepted node's root path
    kReplayVerifyChain = 4,  // replay commit of the previous chain block, then verify the next
    kCommitVerifyTree = 6,   // the persisted-copy commit of the previous block fused into a tree verify
};

// Depth-first walk of up to kTreesPerLaunch trees (tree launches only).
struct TreeSched {
    uint16_t step[kTreesPerLaunch][kMaxNodes];
};

struct CommitArgs {
    const int32_t* accepted;
    const void* persist;
    const float* final_state;
    float* state;
    const int32_t* state_slot;
    int32_t* status;
    int32_t batch;
    int32_t n_nodes;
    int32_t h_v;
    int32_t head_elems;     // d_v * d_k
    int32_t tiles_per_head; // workgroups per (sequence, head)
    int32_t n_slots;
};

struct IndexCommitArgs {
    const int32_t* accepted;
    int32_t* state_slot;
    int32_t* status;
    int32_t batch;
    int32_t n_nodes;
    int32_t draft_row0;
    int32_t n_slots;
};
hipError_t launch_commit_index(const IndexCommitArgs& a, hipStream_t stream);

// Commit of the causal-convolution history (conv_commit.hip).
constexpr int kMaxConvKeep = GDN_MAX_CONV_WIDTH - 1;
struct ConvArgs {
    const unsigned char* x;      // [B][N][C] block inputs
    unsigned char* hist;         // [slots][keep][C] history, updated in place
    const int32_t* accepted;
    const int32_t* state_slot;
    int32_t* status;
    int32_t n_nodes;
    int32_t keep;         // W - 1 history rows
    int32_t pieces;       // 16-byte pieces per row (C * element size / 16)
    int32_t wg_per_seq;   // workgroups per sequence
    int32_t n_slots;
    int32_t seq0;         // first sequence of this launch
    int32_t batch;        // sequences of the call (the arrays' leading dimension)
    int32_t chain;        // 1: parents are n - 1
    int32_t per_seq_tree; // 0: tree 0 for every sequence; 1: tree b - seq0
};

// Per-sequence tables of a varlen prefill launch (up to kMaxPrefillSeqs
// sequences): first token in the packed token dimension and token count (the
// launch covers tokens tok0 .. tok0 + len - 1 of each sequence; a launch may
// cover a chunk-aligned middle part of a longer sequence), first chunk unit
// (workspace block) and first emitted boundary state, the last two with one
// past-the-end entry.
constexpr int kMaxPrefillSeqs = 64;
struct PrefillSeqs {
    int32_t tok0[kMaxPrefillSeqs];
    int32_t len[kMaxPrefillSeqs];
    int32_t unit0[kMaxPrefillSeqs + 1];
    int32_t cst0[kMaxPrefillSeqs + 1];
};

struct PrefillArgs {
    void* workspace; // see prefill_workspace_bytes
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    float* state;
    const int32_t* state_slot;
    void* out;
    int32_t* status;
    int32_t batch;
    int32_t T;       // tokens per sequence
    int32_t h_qk;
    int32_t h_v;
    int32_t d_v;
    int32_t group;   // h_v / h_qk
    int32_t slices;  // scan workgroups per head (set by the launcher from d_v)
    int32_t n_slots;
    int32_t qkv_bf16;
    float scale;
    int32_t varlen;         // 0: batch sequences of T tokens; 1: per-sequence tables (PrefillSeqs)
    int32_t units;          // chunk units (workspace blocks) of this launch
    float* chunk_states;    // nullable: states at chunk-interval boundaries
    int32_t state_interval; // chunks between emitted states (>= 1 when chunk_states is set)
    int32_t seq_states;     // boundary states emitted per sequence (equal-length launches)
    int32_t seq0;           // first sequence of this launch (index of state_slot and of state rows)
    // array extents, for the debug build's index checks
    int32_t batch_total;    // sequences of the call (state rows without slots)
    int64_t tokens_total;   // tokens of the q, k, v, alpha, beta and out arrays
    int64_t n_chunk_states; // boundary states chunk_states holds
};

// Verify kernel launch.  d_k selects the instantiation; m_groups is the number
// of row groups each wave keeps and epl the state elements per lane (8; see
// verify.hip); persist_mode 0 = none,
// 1 = f16, 2 = fp32; tree == nullptr launches the chain kernel.  A set
// a.accepted_prev launches the fused commit + verify of the same shape.
hipError_t launch_verify(const VerifyArgs& a, const TreeSched* tree, int d_k, int m_groups, int epl,
                         int persist_mode, int waves_per_wg, size_t lds_bytes, int grid,
                         hipStream_t stream);
// The fused commit + tree verify instances (their own translation unit);
// launch_verify forwards to it.
hipError_t launch_commit_verify_tree(const VerifyArgs& a, const TreeSched& tree, int d_k, int m_groups, int epl,
                                     int persist_mode, int waves_per_wg, size_t lds_bytes, int grid,
                                     hipStream_t stream);

// Replay launches (kind kReplayChain, kReplayTree or kReplayVerifyChain); parents is
// used by kReplayTree only.
hipError_t launch_replay(const VerifyArgs& a, const TreeParents* parents, int kind, int d_k, int m_groups,
                         int epl, int persist_mode, int waves_per_wg, size_t lds_bytes, int grid,
                         hipStream_t stream);

// Chunked prefill: a parallel prepare kernel per (chunk unit, q/k head) writes
// the state-independent chunk operands to the workspace; a scan kernel per
// (sequence, value head, 32 value columns) then walks the chunks.  `units` is
// the number of 64-token chunk units of the launch (one workspace block each).
size_t prefill_workspace_bytes(long long units, int h_qk, int h_v, int d_k);
// The host checks of a chunked prefill call (shape, pointers, alignment); *empty
// is set for a call with no tokens or no sequences (nothing to launch).
int check_prefill_call(const gdn_shape* sh, const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const float* state, const int32_t* state_slot, const void* out,
                       bool* empty);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillSeqs& seqs, int d_k, int out_dtype, hipStream_t stream);

hipError_t launch_commit(const CommitArgs& a, bool persist_f16, int grid, int block,
                         hipStream_t stream);

hipError_t launch_conv_commit(const ConvArgs& a, const TreeParents* parents, int grid, hipStream_t stream);

}  // namespace gdn
