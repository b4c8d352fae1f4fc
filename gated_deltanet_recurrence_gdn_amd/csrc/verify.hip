// verify.hip -- the verify-family kernels of gfx950: chain and tree verify, the
// fused commit + chain verify and the commits by replay, instantiated over the
// lane layouts, persist modes and output types, with their host launchers.  The
// body they share (mapping, staging, node loop) is in verify_body.h.
#include "verify_body.h"

namespace gdn {
namespace {

// Kernel template arguments: <d_k, row groups per wave M, elements per lane
// EPL, persist mode (0 none, 1 f16, 2 fp32), output dtype (0 fp32, 1 bf16,
// 2 f16), non-temporal stores>.
template <int DK, int M, int EPL, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void verify_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, EPL, kVerifyChain, PMODE, OUT, NT>(a, nullptr, nullptr);
}

// The fused commit + verify launch: the same body with the commit in its state
// load (a compile-time kind, so the plain verify waits on no commit store).
template <int DK, int M, int EPL, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void commit_verify_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, EPL, kCommitVerifyChain, PMODE, OUT, NT>(a, nullptr, nullptr);
}

template <int DK, int M, int EPL, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void verify_tree_kernel(const VerifyArgs a, const TreeSched t) {
    const int bl = xcd_logical_block(blockIdx.x, gridDim.x) / (a.slices * a.h_v);
    verify_body<DK, M, EPL, kVerifyTree, PMODE, OUT, NT>(a, t.step[a.per_seq_tree ? bl : 0], nullptr);
}

template <int DK, int M, int EPL, bool NT>
__global__ __launch_bounds__(256) void replay_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, EPL, kReplayChain, 0, 0, NT>(a, nullptr, nullptr);
}

template <int DK, int M, int EPL, bool NT>
__global__ __launch_bounds__(256) void replay_tree_kernel(const VerifyArgs a, const TreeParents t) {
    const int bl = xcd_logical_block(blockIdx.x, gridDim.x) / (a.slices * a.h_v);
    verify_body<DK, M, EPL, kReplayTree, 0, 0, NT>(a, nullptr, t.p[a.per_seq_tree ? bl : 0]);
}

template <int DK, int M, int EPL, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void replay_verify_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, EPL, kReplayVerifyChain, PMODE, OUT, NT>(a, nullptr, nullptr);
}

template <int DK, int M, int EPL, int PMODE, int OUT>
hipError_t launch_one(const VerifyArgs& a, const TreeSched* t, int waves, size_t lds, int grid, hipStream_t st) {
    if (t != nullptr && a.nt_stores)
        return go<&verify_tree_kernel<DK, M, EPL, PMODE, OUT, true>>(grid, waves, lds, st, a, *t);
    if (t != nullptr)
        return go<&verify_tree_kernel<DK, M, EPL, PMODE, OUT, false>>(grid, waves, lds, st, a, *t);
    if (a.accepted_prev != nullptr && a.nt_stores)
        return go<&commit_verify_chain_kernel<DK, M, EPL, PMODE, OUT, true>>(grid, waves, lds, st, a);
    if (a.accepted_prev != nullptr)
        return go<&commit_verify_chain_kernel<DK, M, EPL, PMODE, OUT, false>>(grid, waves, lds, st, a);
    if (a.nt_stores) return go<&verify_chain_kernel<DK, M, EPL, PMODE, OUT, true>>(grid, waves, lds, st, a);
    return go<&verify_chain_kernel<DK, M, EPL, PMODE, OUT, false>>(grid, waves, lds, st, a);
}

template <int DK, int M, int EPL, int PMODE>
hipError_t launch_dkmp(const VerifyArgs& a, const TreeSched* t, int waves, size_t lds, int grid, hipStream_t st) {
    switch (a.out_dtype) {
        case GDN_F32: return launch_one<DK, M, EPL, PMODE, 0>(a, t, waves, lds, grid, st);
        case GDN_BF16: return launch_one<DK, M, EPL, PMODE, 1>(a, t, waves, lds, grid, st);
        case GDN_F16: return launch_one<DK, M, EPL, PMODE, 2>(a, t, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int M, int EPL>
hipError_t launch_dkm(const VerifyArgs& a, const TreeSched* t, int pmode, int waves, size_t lds, int grid,
                      hipStream_t st) {
    switch (pmode) {
        case 0: return launch_dkmp<DK, M, EPL, 0>(a, t, waves, lds, grid, st);
        case 1: return launch_dkmp<DK, M, EPL, 1>(a, t, waves, lds, grid, st);
        case 2: return launch_dkmp<DK, M, EPL, 2>(a, t, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int M, int EPL, int PM, int OT>
hipError_t launch_rv(const VerifyArgs& a, int waves, size_t lds, int grid, hipStream_t st) {
    if (a.nt_stores) return go<&replay_verify_chain_kernel<DK, M, EPL, PM, OT, true>>(grid, waves, lds, st, a);
    return go<&replay_verify_chain_kernel<DK, M, EPL, PM, OT, false>>(grid, waves, lds, st, a);
}

template <int DK, int M, int EPL, int PM>
hipError_t launch_rv_out(const VerifyArgs& a, int waves, size_t lds, int grid, hipStream_t st) {
    switch (a.out_dtype) {
        case GDN_F32: return launch_rv<DK, M, EPL, PM, 0>(a, waves, lds, grid, st);
        case GDN_BF16: return launch_rv<DK, M, EPL, PM, 1>(a, waves, lds, grid, st);
        case GDN_F16: return launch_rv<DK, M, EPL, PM, 2>(a, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int M, int EPL>
hipError_t launch_replay_dkm(const VerifyArgs& a, const TreeParents* tp, int kind, int pmode, int waves, size_t lds,
                             int grid, hipStream_t st) {
    if (kind == kReplayChain) {
        if (a.nt_stores) return go<&replay_chain_kernel<DK, M, EPL, true>>(grid, waves, lds, st, a);
        return go<&replay_chain_kernel<DK, M, EPL, false>>(grid, waves, lds, st, a);
    }
    if (kind == kReplayTree) {
        if (a.nt_stores) return go<&replay_tree_kernel<DK, M, EPL, true>>(grid, waves, lds, st, a, *tp);
        return go<&replay_tree_kernel<DK, M, EPL, false>>(grid, waves, lds, st, a, *tp);
    }
    if (kind != kReplayVerifyChain) return hipErrorInvalidValue;
    // outputs in fp32, f16 or bf16; node states persisted or not (the replay design persists none)
    switch (pmode) {
        case 0: return launch_rv_out<DK, M, EPL, 0>(a, waves, lds, grid, st);
        case 1: return launch_rv_out<DK, M, EPL, 1>(a, waves, lds, grid, st);
        case 2: return launch_rv_out<DK, M, EPL, 2>(a, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The lane layouts built: 8 elements per lane; d_k 128 with one or two row
// groups, d_k 64 and 32 with one.
hipError_t launch_replay(const VerifyArgs& a, const TreeParents* parents, int kind, int d_k, int m_groups, int epl,
                         int persist_mode, int waves, size_t lds, int grid, hipStream_t st) {
    if (d_k == 128 && m_groups == 1 && epl == 8) return launch_replay_dkm<128, 1, 8>(a, parents, kind, persist_mode, waves, lds, grid, st);
    if (d_k == 128 && m_groups == 2 && epl == 8) return launch_replay_dkm<128, 2, 8>(a, parents, kind, persist_mode, waves, lds, grid, st);
    if (d_k == 64 && m_groups == 1 && epl == 8) return launch_replay_dkm<64, 1, 8>(a, parents, kind, persist_mode, waves, lds, grid, st);
    if (d_k == 32 && m_groups == 1 && epl == 8) return launch_replay_dkm<32, 1, 8>(a, parents, kind, persist_mode, waves, lds, grid, st);
    return hipErrorInvalidValue;
}

hipError_t launch_verify(const VerifyArgs& a, const TreeSched* tree, int d_k, int m_groups, int epl, int persist_mode,
                         int waves, size_t lds, int grid, hipStream_t st) {
    if (tree != nullptr && a.accepted_prev != nullptr)
        return launch_commit_verify_tree(a, *tree, d_k, m_groups, epl, persist_mode, waves, lds, grid, st);
    if (d_k == 128 && m_groups == 1 && epl == 8) return launch_dkm<128, 1, 8>(a, tree, persist_mode, waves, lds, grid, st);
    if (d_k == 128 && m_groups == 2 && epl == 8) return launch_dkm<128, 2, 8>(a, tree, persist_mode, waves, lds, grid, st);
    if (d_k == 64 && m_groups == 1 && epl == 8) return launch_dkm<64, 1, 8>(a, tree, persist_mode, waves, lds, grid, st);
    if (d_k == 32 && m_groups == 1 && epl == 8) return launch_dkm<32, 1, 8>(a, tree, persist_mode, waves, lds, grid, st);
    return hipErrorInvalidValue;
}

}  // namespace gdn
