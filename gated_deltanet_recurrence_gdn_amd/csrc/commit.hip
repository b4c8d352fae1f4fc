// commit.hip -- copy the accepted node's state into the state cache (gfx950).
//
// Page "400 tok/s with Qwen3.5", section "Handling recurrent state": after
// verification the recurrent state is set to the accepted boundary, and a
// fully accepted block uses the verified state directly.  Here the boundary
// state is the node's persisted copy (f16 widened exactly to fp32, or fp32),
// or the exact fp32 final state when the whole chain was accepted.
//
// One workgroup covers 256 x 8 consecutive elements of one (sequence, head);
// each lane moves one 16-byte f16 (or 32-byte fp32) vector and writes 32
// bytes.  The accepted index and the slot are read per workgroup from device
// memory, so no host synchronisation is needed between verify and commit.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <bool F16, bool NT>
__global__ __launch_bounds__(256) void commit_kernel(const CommitArgs a) {
    int blk = blockIdx.x;
    const int tile = blk % a.tiles_per_head;
    blk /= a.tiles_per_head;
    const int h = blk % a.h_v;
    const int b = blk / a.h_v;

    const int acc = a.accepted[b];
    if (acc < 0 || acc >= a.n_nodes) {
        if (tile == 0 && h == 0 && threadIdx.x == 0 && a.status != nullptr) a.status[0] = GDN_ERR_NODE;
        return;
    }
    int s = b;
    if (a.state_slot != nullptr) {
        s = a.state_slot[b];
        if (s < 0 || s >= a.n_slots) {
            if (tile == 0 && h == 0 && threadIdx.x == 0 && a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
            return;
        }
    }
    const size_t e = ((size_t)tile * blockDim.x + threadIdx.x) * 8;
    if (e >= (size_t)a.head_elems) return;
    [[maybe_unused]] const size_t heads = (size_t)a.batch * a.h_v;
    float* dst = a.state + GDN_AT(((size_t)s * a.h_v + h) * a.head_elems + e, 8,
                                  (size_t)(a.state_slot != nullptr ? a.n_slots : a.batch) * a.h_v * a.head_elems,
                                  a.status);
    f32x4 x0, x1;
    if (a.final_state != nullptr && acc == a.n_nodes - 1) {
        const float* src = a.final_state + GDN_AT(((size_t)b * a.h_v + h) * a.head_elems + e, 8,
                                                  heads * a.head_elems, a.status);
        x0 = *reinterpret_cast<const f32x4*>(src);
        x1 = *reinterpret_cast<const f32x4*>(src + 4);
    } else {
        const size_t off = GDN_AT((((size_t)b * a.n_nodes + acc) * a.h_v + h) * a.head_elems + e, 8,
                                  heads * a.n_nodes * a.head_elems, a.status);
        if constexpr (F16) {
            const f16x8 hv = *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(a.persist) + off);
            x0 = f32x4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
            x1 = f32x4{(float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]};
        } else {
            const float* src = static_cast<const float*>(a.persist) + off;
            x0 = *reinterpret_cast<const f32x4*>(src);
            x1 = *reinterpret_cast<const f32x4*>(src + 4);
        }
    }
    store_stream<NT>(x0, reinterpret_cast<f32x4*>(dst));
    store_stream<NT>(x1, reinterpret_cast<f32x4*>(dst + 4));
}

// Index-table commit: one thread per sequence writes the row of its accepted
// node into the index table (page "LightSeek's TokenSpeed Hits 580 Tokens per
// Second on Qwen3.5's 400B Model", section "How they actually got there":
// move pointers, not data).
__global__ __launch_bounds__(256) void commit_index_kernel(const IndexCommitArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.batch) return;
    const int acc = a.accepted[b];
    const long long row = (long long)a.draft_row0 + (long long)b * a.n_nodes + acc;
    if (acc < 0 || acc >= a.n_nodes) {
        if (a.status != nullptr) a.status[0] = GDN_ERR_NODE;
        return;
    }
    if (row >= a.n_slots) {
        if (a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
        return;
    }
    a.state_slot[b] = (int32_t)row;
}

}  // namespace

hipError_t launch_commit_index(const IndexCommitArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(commit_index_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, bool persist_f16, int grid, int block, hipStream_t stream) {
    // non-temporal stores for small commits (shorter drain), plain ones for large (faster streaming)
    const bool nt = (double)a.batch * a.h_v * a.head_elems * 4 < 256.0 * (1 << 20);
    if (persist_f16) {
        if (nt) hipLaunchKernelGGL((commit_kernel<true, true>), dim3(grid), dim3(block), 0, stream, a);
        else hipLaunchKernelGGL((commit_kernel<true, false>), dim3(grid), dim3(block), 0, stream, a);
    } else {
        if (nt) hipLaunchKernelGGL((commit_kernel<false, true>), dim3(grid), dim3(block), 0, stream, a);
        else hipLaunchKernelGGL((commit_kernel<false, false>), dim3(grid), dim3(block), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace gdn
