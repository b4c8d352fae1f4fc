// verify.hip -- state-resident verify of a draft chain or tree (gfx950).
//
// Per (sequence b, value head h) the d_v x d_k fp32 state S evolves over the
// draft nodes by the gated delta rule, written in rank-1 form:
//     kh = S k,  qh = S q                     (both from the parent state)
//     u  = beta (v - alpha kh)
//     S' = alpha S + u k^T                    (= alpha S (I - beta k k^T) + beta v k^T)
//     o  = scale (alpha qh + (q.k) u)         (= scale S' q, the updated state read)
// Page "400 tok/s with Qwen3.5", section "Handling recurrent state": the
// working state stays on chip across the whole verification block.  Page
// "We got 207 tok/s with Qwen3.5-27B on an RTX 3090", section "Key wins": the
// recurrence kernel itself writes every node's state in f16.
//
// Mapping.  Every value row S[j][:] evolves independently given k and q, so
// a head is split over workgroups by rows.  A row of d_k fp32 is spread over
// LPR = d_k / 8 lanes, 8 consecutive elements each, so one wave holds
// RPG = 64 / LPR rows per row group and M row groups (R = M * RPG rows).
// The two row reductions (S k and S q) are DPP sums over the LPR lanes of a
// row; the persisted f16 row is written with one 16-byte store per lane, a
// full 256-byte row per 16 lanes.  The state never leaves VGPRs between
// nodes; only the persisted copies, the outputs and the final state are
// written.  All per-node inputs (k, q rows as fp32, this slice of v, the
// gates and q.k) are staged once into LDS, so the node loop issues no global
// loads and never waits on the vector-memory counter.
//
// Trees are walked depth first (the host computes the walk): a node whose
// parent is the previous node continues in registers; otherwise the parent's
// exact fp32 state is restored from an LDS fork slot saved when the parent
// (a branch point) was computed.  A chain is the walk 0, 1, ..., N-1.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int M, bool TREE, int PMODE>
__device__ __forceinline__ void verify_body(const VerifyArgs& a, const uint16_t* walk) {
    constexpr int LPR = DK / 8;   // lanes per state row
    constexpr int RPG = 64 / LPR; // rows per row group
    constexpr int R = M * RPG;    // rows per wave
    extern __shared__ __align__(16) float lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nthr = blockDim.x, nwaves = nthr >> 6;

    int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int slice = blk % a.slices;
    blk /= a.slices;
    const int h = blk % a.h_v;
    const int bl = blk / a.h_v;
    const int b = a.seq0 + bl;
    const int g = h / a.group;
    const int N = a.n_nodes;
    const int DV = a.d_v;
    const int rows = a.rows_per_wg;
    const int row0 = slice * rows;

    int s = b;
    if (a.state_slot != nullptr) {
        s = a.state_slot[b];
        if (s < 0 || s >= a.n_slots) {
            if (tid == 0 && a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
            return;
        }
    }

    // LDS: k[N][DK], q[N][DK], v[N][rows], alpha[N], beta[N], qk[N], fork slots.
    float* kL = lds;
    float* qL = kL + N * DK;
    float* vL = qL + N * DK;
    float* aL = vL + N * rows;
    float* bL = aL + N;
    float* qkL = bL + N;
    const int stage_floats = (2 * N * DK + N * rows + 3 * N + 3) & ~3;
    float* forkL = lds + stage_floats;

    // 1. this wave's state rows -> VGPRs (issued first; its latency overlaps staging)
    const int c = lane % LPR, r = lane / LPR;
    const int wrow = wave * R;  // first row of this wave inside the slice
    const size_t head_elems = (size_t)DV * DK;
    float S[M][8];
    {
        const float* src = a.state + ((size_t)s * a.h_v + h) * head_elems + (size_t)(row0 + wrow + r) * DK + 8 * c;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + (size_t)m * RPG * DK);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + (size_t)m * RPG * DK + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[m][e] = x0[e];
                S[m][4 + e] = x1[e];
            }
        }
    }

    // 2. stage k, q (as fp32) and q.k for every node
    const bool bf16 = a.qkv_bf16 != 0;
    const int chunks = N * LPR;  // 8-element chunks per tensor
    for (int base = wave * 64; base < chunks; base += nthr) {
        const int e = base + lane;
        float part = 0.f;
        if (e < chunks) {
            const int n = e / LPR, cc = e % LPR;
            const size_t src = (((size_t)b * N + n) * a.h_qk + g) * DK + 8 * cc;
            float kf[8], qf[8];
            load8_as_f32(a.k, src, bf16, kf);
            load8_as_f32(a.q, src, bf16, qf);
            float* kd = kL + n * DK + 8 * cc;
            float* qd = qL + n * DK + 8 * cc;
            *reinterpret_cast<f32x4*>(kd) = f32x4{kf[0], kf[1], kf[2], kf[3]};
            *reinterpret_cast<f32x4*>(kd + 4) = f32x4{kf[4], kf[5], kf[6], kf[7]};
            *reinterpret_cast<f32x4*>(qd) = f32x4{qf[0], qf[1], qf[2], qf[3]};
            *reinterpret_cast<f32x4*>(qd + 4) = f32x4{qf[4], qf[5], qf[6], qf[7]};
#pragma unroll
            for (int i = 0; i < 8; ++i) part = fmaf(kf[i], qf[i], part);
        }
        part = group_sum<LPR>(part);
        if (e < chunks && (e % LPR) == 0) qkL[e / LPR] = part;
    }
    // this slice of v, and the gates
    for (int e = tid; e < N * rows; e += nthr) {
        const int n = e / rows, j = e % rows;
        vL[e] = load1_as_f32(a.v, (((size_t)b * N + n) * a.h_v + h) * DV + row0 + j, bf16);
    }
    for (int n = tid; n < N; n += nthr) {
        aL[n] = a.alpha[((size_t)b * N + n) * a.h_v + h];
        bL[n] = a.beta[((size_t)b * N + n) * a.h_v + h];
    }
    __syncthreads();

    // 3. node loop: reductions, update, persist, output
    const size_t node_elems = (size_t)a.h_v * head_elems;  // persist elements per node
    const size_t prow = (size_t)h * head_elems + (size_t)(row0 + wrow + r) * DK + 8 * c;
    const int fork_stride = nwaves * R * DK;
    float* myfork = forkL + wrow * DK;
    for (int st = 0; st < N; ++st) {
        int node = st;
        uint16_t code = 0;
        if constexpr (TREE) {
            code = walk[st];
            node = sched_node(code);
            if (code & kSchedRestore) {
                const float* src = myfork + sched_restore_slot(code) * fork_stride;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + (m * 64 + lane) * 8);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + (m * 64 + lane) * 8 + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        S[m][e] = x0[e];
                        S[m][4 + e] = x1[e];
                    }
                }
            }
        }
        float kf[8], qf[8];
        {
            const f32x4 k0 = *reinterpret_cast<const f32x4*>(kL + node * DK + 8 * c);
            const f32x4 k1 = *reinterpret_cast<const f32x4*>(kL + node * DK + 8 * c + 4);
            const f32x4 q0 = *reinterpret_cast<const f32x4*>(qL + node * DK + 8 * c);
            const f32x4 q1 = *reinterpret_cast<const f32x4*>(qL + node * DK + 8 * c + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[e] = k0[e];
                kf[4 + e] = k1[e];
                qf[e] = q0[e];
                qf[4 + e] = q1[e];
            }
        }
        const float al = aL[node], be = bL[node], qk = qkL[node];
        const size_t nbase = ((size_t)b * N + node);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float pk = 0.f, pq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pk = fmaf(S[m][e], kf[e], pk);
                pq = fmaf(S[m][e], qf[e], pq);
            }
            pk = group_sum<LPR>(pk);
            pq = group_sum<LPR>(pq);
            const int vr = wrow + m * RPG + r;  // row inside the slice
            const float vj = vL[node * rows + vr];
            const float u = be * (vj - al * pk);
            const float o = a.scale * (al * pq + qk * u);
#pragma unroll
            for (int e = 0; e < 8; ++e) S[m][e] = fmaf(al, S[m][e], u * kf[e]);
            if constexpr (PMODE == 1) {
                f16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = (_Float16)S[m][e];
                *reinterpret_cast<f16x8*>(static_cast<_Float16*>(a.persist) + nbase * node_elems + prow +
                                          (size_t)m * RPG * DK) = hv;
            } else if constexpr (PMODE == 2) {
                float* dst = static_cast<float*>(a.persist) + nbase * node_elems + prow + (size_t)m * RPG * DK;
                *reinterpret_cast<f32x4*>(dst) = f32x4{S[m][0], S[m][1], S[m][2], S[m][3]};
                *reinterpret_cast<f32x4*>(dst + 4) = f32x4{S[m][4], S[m][5], S[m][6], S[m][7]};
            }
            if (a.out != nullptr && c == 0)
                store_out(a.out, (nbase * a.h_v + h) * DV + row0 + vr, o, a.out_dtype);
        }
        if constexpr (TREE) {
            if (code & kSchedSave) {
                float* dst = myfork + sched_save_slot(code) * fork_stride;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    *reinterpret_cast<f32x4*>(dst + (m * 64 + lane) * 8) = f32x4{S[m][0], S[m][1], S[m][2], S[m][3]};
                    *reinterpret_cast<f32x4*>(dst + (m * 64 + lane) * 8 + 4) = f32x4{S[m][4], S[m][5], S[m][6], S[m][7]};
                }
            }
        }
    }

    // 4. final state (chains): the exact fp32 state after node N-1
    if constexpr (!TREE) {
        if (a.final_state != nullptr) {
            float* dst = a.final_state + ((size_t)b * a.h_v + h) * head_elems + (size_t)(row0 + wrow + r) * DK + 8 * c;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float* d = dst + (size_t)m * RPG * DK;
                *reinterpret_cast<f32x4*>(d) = f32x4{S[m][0], S[m][1], S[m][2], S[m][3]};
                *reinterpret_cast<f32x4*>(d + 4) = f32x4{S[m][4], S[m][5], S[m][6], S[m][7]};
            }
        }
    }
}

template <int DK, int M, int PMODE>
__global__ __launch_bounds__(256) void verify_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, false, PMODE>(a, nullptr);
}

template <int DK, int M, int PMODE>
__global__ __launch_bounds__(256) void verify_tree_kernel(const VerifyArgs a, const TreeSched t) {
    const int bl = xcd_logical_block(blockIdx.x, gridDim.x) / (a.slices * a.h_v);
    verify_body<DK, M, true, PMODE>(a, t.step[a.per_seq_tree ? bl : 0]);
}

template <int DK, int M, int PMODE>
hipError_t launch_dkmp(const VerifyArgs& a, const TreeSched* t, int waves, size_t lds, int grid,
                       hipStream_t st) {
    if (t != nullptr)
        hipLaunchKernelGGL((verify_tree_kernel<DK, M, PMODE>), dim3(grid), dim3(64 * waves), lds, st, a, *t);
    else
        hipLaunchKernelGGL((verify_chain_kernel<DK, M, PMODE>), dim3(grid), dim3(64 * waves), lds, st, a);
    return hipGetLastError();
}

template <int DK, int M>
hipError_t launch_dkm(const VerifyArgs& a, const TreeSched* t, int pmode, int waves, size_t lds,
                      int grid, hipStream_t st) {
    switch (pmode) {
        case 0: return launch_dkmp<DK, M, 0>(a, t, waves, lds, grid, st);
        case 1: return launch_dkmp<DK, M, 1>(a, t, waves, lds, grid, st);
        case 2: return launch_dkmp<DK, M, 2>(a, t, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, const TreeSched* tree, int d_k, int m_groups,
                         int persist_mode, int waves_per_wg, size_t lds_bytes, int grid,
                         hipStream_t stream) {
    if (d_k == 128 && m_groups == 1) return launch_dkm<128, 1>(a, tree, persist_mode, waves_per_wg, lds_bytes, grid, stream);
    if (d_k == 128 && m_groups == 2) return launch_dkm<128, 2>(a, tree, persist_mode, waves_per_wg, lds_bytes, grid, stream);
    if (d_k == 64 && m_groups == 1) return launch_dkm<64, 1>(a, tree, persist_mode, waves_per_wg, lds_bytes, grid, stream);
    if (d_k == 32 && m_groups == 1) return launch_dkm<32, 1>(a, tree, persist_mode, waves_per_wg, lds_bytes, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
