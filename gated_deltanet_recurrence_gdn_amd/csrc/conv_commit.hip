// conv_commit.hip -- commit of the causal-convolution input history (gfx950).
//
// Page "400 tok/s with Qwen3.5", section "Handling recurrent state": the
// convolution history is committed to the same boundary as the recurrent
// state.  A causal convolution of width W reads the current input row and the
// W - 1 rows before it, so a sequence keeps its last W - 1 input rows, oldest
// first, as history[slot][W-1][C].  After a draft block is verified, the
// accepted stream is the history followed by the inputs of the accepted
// node's root path (nodes 0 .. a of a chain; the ancestors of a, root first,
// of a tree), and the new history is that stream's last W - 1 rows:
//     row i  <-  x[b][ancestor of a at distance W-2-i]   if that ancestor exists
//                history[slot][i + depth(a)]              otherwise
// Bytes are moved verbatim (any element type).  One thread moves one 16-byte
// piece of a row for every history row: it reads all its sources before it
// writes, so the in-place shift of history rows is safe.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__global__ __launch_bounds__(256) void conv_commit_kernel(const ConvArgs a, const TreeParents t) {
    const int bl = blockIdx.x / a.wg_per_seq;
    const int b = a.seq0 + bl;
    const int piece = (blockIdx.x % a.wg_per_seq) * blockDim.x + threadIdx.x;
    const bool lead = threadIdx.x == 0 && blockIdx.x % a.wg_per_seq == 0;

    const int acc = a.accepted[b];
    if (acc < 0 || acc >= a.n_nodes) {
        if (lead && a.status != nullptr) a.status[0] = GDN_ERR_NODE;
        return;
    }
    int s = b;
    if (a.state_slot != nullptr) {
        s = a.state_slot[b];
        if (s < 0 || s >= a.n_slots) {
            if (lead && a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
            return;
        }
    }
    if (piece >= a.pieces) return;

    // depth of the accepted node (nodes on its root path; uniform)
    const int8_t* par = a.chain ? nullptr : t.p[a.per_seq_tree ? bl : 0];
    int depth = acc + 1;
    if (!a.chain) {
        depth = 0;
        for (int n = acc; n >= 0; n = par[n]) ++depth;
    }
    const size_t row = (size_t)a.pieces * 16;
    unsigned char* hist = a.hist + (size_t)s * a.keep * row + (size_t)piece * 16;
    const unsigned char* xb = a.x + (size_t)b * a.n_nodes * row + (size_t)piece * 16;
    // (debug build: every row read or written stays inside its array)
    [[maybe_unused]] const size_t hist_end = (size_t)(a.state_slot != nullptr ? a.n_slots : a.batch) * a.keep * row;
    [[maybe_unused]] const size_t x_end = (size_t)a.batch * a.n_nodes * row;
    // history row keep-1-k takes the ancestor at distance k when the path is that
    // long, else the old history row keep-1-k+depth; all sources are read first
    u32x4 v[kMaxConvKeep];
    int n = acc;  // the ancestor at distance k
#pragma unroll
    for (int k = 0; k < kMaxConvKeep; ++k) {
        if (k < a.keep) {
            const unsigned char* src =
                k < depth ? a.x + GDN_AT(xb - a.x + (size_t)n * row, 16, x_end, a.status)
                          : a.hist + GDN_AT(hist - a.hist + (size_t)(a.keep - 1 - k + depth) * row, 16, hist_end, a.status);
            v[k] = *reinterpret_cast<const u32x4*>(src);
            if (k < depth) n = a.chain ? n - 1 : par[n];
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxConvKeep; ++k)
        if (k < a.keep)
            *reinterpret_cast<u32x4*>(a.hist + GDN_AT(hist - a.hist + (size_t)(a.keep - 1 - k) * row, 16, hist_end,
                                                      a.status)) = v[k];
}

}  // namespace

hipError_t launch_conv_commit(const ConvArgs& a, const TreeParents* t, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(conv_commit_kernel, dim3(grid), dim3(256), 0, stream, a, *t);
    return hipGetLastError();
}

}  // namespace gdn
