// commit_verify_tree.hip -- the fused commit + tree verify of gfx950: one launch
// per tree decode step.  The previous step's accepted node (its persisted copy,
// widened to fp32) is the starting state of the next tree's walk and is written
// back to the state cache on the way, as in the fused chain step; the body is
// the verify body of verify_body.h.  Page "400 tok/s with Qwen3.5", section
// "Handling recurrent state" (the state is set to the accepted boundary before
// the next verification) and page "Qwen3.6 27B: From 20 t/s to 184 t/s",
// section "Diffusion applied to text" (a tree verified in one pass).
#include "verify_body.h"

namespace gdn {
namespace {

template <int DK, int M, int EPL, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void commit_verify_tree_kernel(const VerifyArgs a, const TreeSched t) {
    const int bl = xcd_logical_block(blockIdx.x, gridDim.x) / (a.slices * a.h_v);
    verify_body<DK, M, EPL, kCommitVerifyTree, PMODE, OUT, NT>(a, t.step[a.per_seq_tree ? bl : 0], nullptr);
}

template <int DK, int M, int EPL, int PMODE, int OUT>
hipError_t launch_one(const VerifyArgs& a, const TreeSched& t, int waves, size_t lds, int grid, hipStream_t st) {
    if (a.nt_stores) return go<&commit_verify_tree_kernel<DK, M, EPL, PMODE, OUT, true>>(grid, waves, lds, st, a, t);
    return go<&commit_verify_tree_kernel<DK, M, EPL, PMODE, OUT, false>>(grid, waves, lds, st, a, t);
}

template <int DK, int M, int EPL, int PMODE>
hipError_t launch_out(const VerifyArgs& a, const TreeSched& t, int waves, size_t lds, int grid, hipStream_t st) {
    switch (a.out_dtype) {
        case GDN_F32: return launch_one<DK, M, EPL, PMODE, 0>(a, t, waves, lds, grid, st);
        case GDN_BF16: return launch_one<DK, M, EPL, PMODE, 1>(a, t, waves, lds, grid, st);
        case GDN_F16: return launch_one<DK, M, EPL, PMODE, 2>(a, t, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DK, int M, int EPL>
hipError_t launch_pm(const VerifyArgs& a, const TreeSched& t, int pmode, int waves, size_t lds, int grid,
                     hipStream_t st) {
    switch (pmode) {
        case 0: return launch_out<DK, M, EPL, 0>(a, t, waves, lds, grid, st);
        case 1: return launch_out<DK, M, EPL, 1>(a, t, waves, lds, grid, st);
        case 2: return launch_out<DK, M, EPL, 2>(a, t, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_commit_verify_tree(const VerifyArgs& a, const TreeSched& t, int d_k, int m_groups, int epl,
                                     int persist_mode, int waves, size_t lds, int grid, hipStream_t st) {
    if (d_k == 128 && m_groups == 1 && epl == 8) return launch_pm<128, 1, 8>(a, t, persist_mode, waves, lds, grid, st);
    if (d_k == 128 && m_groups == 2 && epl == 8) return launch_pm<128, 2, 8>(a, t, persist_mode, waves, lds, grid, st);
    if (d_k == 64 && m_groups == 1 && epl == 8) return launch_pm<64, 1, 8>(a, t, persist_mode, waves, lds, grid, st);
    if (d_k == 32 && m_groups == 1 && epl == 8) return launch_pm<32, 1, 8>(a, t, persist_mode, waves, lds, grid, st);
    return hipErrorInvalidValue;
}

}  // namespace gdn
