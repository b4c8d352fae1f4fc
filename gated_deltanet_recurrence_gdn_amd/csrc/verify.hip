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

// Output element store in the output dtype (OUT: 0 fp32, 1 bf16, 2 f16).
template <int OUT>
__device__ __forceinline__ void put_out(void* out, size_t idx, float o) {
    if constexpr (OUT == 0) static_cast<float*>(out)[idx] = o;
    else if constexpr (OUT == 2) static_cast<_Float16*>(out)[idx] = (_Float16)o;
    else static_cast<uint16_t*>(out)[idx] = f32_to_bf16(o);
}

// Per-node operands a lane needs, read from LDS one node ahead of use.
template <int M>
struct NodeOps {
    float k[8], q[8];
    f32x4 coef;  // alpha, beta, q.k, unused
    float vb[M]; // beta * v for this lane's rows
};

template <int DK, int M>
__device__ __forceinline__ void read_node(NodeOps<M>& x, const float* kL, const float* qL, const f32x4* cL,
                                          const float* vbL, int node, int c, int vr0, int rows) {
    constexpr int RPG = 64 / (DK / 8);
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(kL + node * DK + 8 * c);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(kL + node * DK + 8 * c + 4);
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(qL + node * DK + 8 * c);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(qL + node * DK + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x.k[e] = k0[e];
        x.k[4 + e] = k1[e];
        x.q[e] = q0[e];
        x.q[4 + e] = q1[e];
    }
    x.coef = cL[node];
#pragma unroll
    for (int m = 0; m < M; ++m) x.vb[m] = vbL[node * rows + vr0 + m * RPG];
}

template <int DK, int M, bool TREE, int PMODE, int OUT, bool NT>
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
    // fused commit of the previous step: its accepted node must be in range
    int acc = 0;
    if (a.accepted_prev != nullptr) {
        acc = a.accepted_prev[b];
        if (acc < 0 || acc >= N) {
            if (tid == 0 && a.status != nullptr) a.status[0] = GDN_ERR_NODE;
            return;
        }
    }

    // LDS: k[N][DK], q[N][DK] (fp32), coef[N] (alpha, beta, q.k), beta*v[N][rows],
    // walk[N] (trees), then the fork slots.
    float* kL = lds;
    float* qL = kL + N * DK;
    f32x4* cL = reinterpret_cast<f32x4*>(qL + N * DK);
    float* vbL = reinterpret_cast<float*>(cL + N);
    int* walkL = reinterpret_cast<int*>(vbL + N * rows);
    const int stage_floats = (2 * N * DK + 4 * N + N * rows + N + 3) & ~3;
    float* forkL = lds + stage_floats;

    // 1. this wave's state rows -> VGPRs (issued first; the loads overlap staging)
    const int c = lane % LPR, r = lane / LPR;
    const int wrow = wave * R;  // first row of this wave inside the slice
    const size_t head_elems = (size_t)DV * DK;
    float S[M][8];
    const size_t my_rows = (size_t)(row0 + wrow + r) * DK + 8 * c;  // this lane's first element in a head
    if (a.accepted_prev == nullptr) {
        const float* src = a.state + ((size_t)s * a.h_v + h) * head_elems + my_rows;
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
    } else {
        // Commit while loading: the initial state is the previous step's accepted node
        // (its exact fp32 final state when the whole block was accepted, else its persisted
        // copy widened to fp32); it is also written back to the state cache.
        if (a.final_prev != nullptr && acc == N - 1) {
            const float* src = a.final_prev + ((size_t)b * a.h_v + h) * head_elems + my_rows;
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
        } else if (a.persist_prev_f16) {
            const _Float16* src = static_cast<const _Float16*>(a.persist_prev) +
                                  (((size_t)b * N + acc) * a.h_v + h) * head_elems + my_rows;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const f16x8 hv = *reinterpret_cast<const f16x8*>(src + (size_t)m * RPG * DK);
#pragma unroll
                for (int e = 0; e < 8; ++e) S[m][e] = (float)hv[e];
            }
        } else {
            const float* src = static_cast<const float*>(a.persist_prev) +
                               (((size_t)b * N + acc) * a.h_v + h) * head_elems + my_rows;
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
        float* dst = a.state_w + ((size_t)s * a.h_v + h) * head_elems + my_rows;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            store_stream<NT>(f32x4{S[m][0], S[m][1], S[m][2], S[m][3]}, reinterpret_cast<f32x4*>(dst + (size_t)m * RPG * DK));
            store_stream<NT>(f32x4{S[m][4], S[m][5], S[m][6], S[m][7]},
                         reinterpret_cast<f32x4*>(dst + (size_t)m * RPG * DK + 4));
        }
    }

    // 2. stage every node's inputs.  One pass issues all of a thread's global
    //    loads (k and q chunks, beta * v, the gates) before any LDS store, so
    //    the common case (N * d_k / 8 <= threads) costs one memory round trip.
    const bool bf16 = a.qkv_bf16 != 0;
    const int chunks = N * LPR;  // 8-element chunks of k (and of q)
    const int nvb = N * rows;
    const int items = chunks > nvb ? chunks : nvb;
    for (int base = wave * 64; base < items; base += nthr) {
        const int e = base + lane;
        float kf[8], qf[8], vv = 0.f, vbeta = 0.f, ga = 0.f, gb = 0.f;
        const bool has_kq = e < chunks, has_v = e < nvb, has_g = e < N;
        if (has_kq) {
            const size_t src = (((size_t)b * N + e / LPR) * a.h_qk + g) * DK + 8 * (e % LPR);
            load8_as_f32(a.k, src, bf16, kf);
            load8_as_f32(a.q, src, bf16, qf);
        }
        if (has_v) {
            const int n = e / rows, j = e % rows;
            vv = load1_as_f32(a.v, (((size_t)b * N + n) * a.h_v + h) * DV + row0 + j, bf16);
            vbeta = a.beta[((size_t)b * N + n) * a.h_v + h];
        }
        if (has_g) {
            ga = a.alpha[((size_t)b * N + e) * a.h_v + h];
            gb = a.beta[((size_t)b * N + e) * a.h_v + h];
        }
        float part = 0.f;
        if (has_kq) {
            float* kd = kL + (e / LPR) * DK + 8 * (e % LPR);
            float* qd = qL + (e / LPR) * DK + 8 * (e % LPR);
            *reinterpret_cast<f32x4*>(kd) = f32x4{kf[0], kf[1], kf[2], kf[3]};
            *reinterpret_cast<f32x4*>(kd + 4) = f32x4{kf[4], kf[5], kf[6], kf[7]};
            *reinterpret_cast<f32x4*>(qd) = f32x4{qf[0], qf[1], qf[2], qf[3]};
            *reinterpret_cast<f32x4*>(qd + 4) = f32x4{qf[4], qf[5], qf[6], qf[7]};
#pragma unroll
            for (int i = 0; i < 8; ++i) part = fmaf(kf[i], qf[i], part);
        }
        part = group_sum<LPR>(part);
        if (has_kq && (e % LPR) == 0) reinterpret_cast<float*>(cL + e / LPR)[2] = part;
        if (has_v) vbL[e] = vbeta * vv;
        if (has_g) {
            reinterpret_cast<float*>(cL + e)[0] = ga;
            reinterpret_cast<float*>(cL + e)[1] = gb;
            if constexpr (TREE) walkL[e] = walk[e];
        }
    }
    __syncthreads();

    // 3. node loop: reductions, update, persist, output; next node's operands
    //    are read from LDS while the current node computes.
    const size_t node_elems = (size_t)a.h_v * head_elems;  // persist elements per node
    const size_t prow = (size_t)h * head_elems + (size_t)(row0 + wrow + r) * DK + 8 * c;
    const int fork_stride = nwaves * R * DK;
    float* myfork = forkL + wrow * DK;
    const float scale = a.scale;
    const int vr0 = wrow + r;  // this lane's first row inside the slice

    // One node: optional fork restore, the two row reductions, the update,
    // the persisted copy, the output, optional fork save.
    auto step = [&](const NodeOps<M>& x, int code) {
        const int node = sched_node((uint16_t)code);
        if constexpr (TREE) {
            if (code & kSchedRestore) {
                const float* src = myfork + sched_restore_slot((uint16_t)code) * fork_stride;
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
        const float al = x.coef[0];
        const float bal = x.coef[1] * al;     // beta * alpha
        const float sal = scale * al;         // scale * alpha
        const float sqk = scale * x.coef[2];  // scale * (q . k)
        const size_t nbase = ((size_t)b * N + node);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            // two accumulators per product halve the dependent FMA chain
            float pk0 = S[m][0] * x.k[0], pk1 = S[m][1] * x.k[1];
            float pq0 = S[m][0] * x.q[0], pq1 = S[m][1] * x.q[1];
#pragma unroll
            for (int e = 2; e < 8; e += 2) {
                pk0 = fmaf(S[m][e], x.k[e], pk0);
                pk1 = fmaf(S[m][e + 1], x.k[e + 1], pk1);
                pq0 = fmaf(S[m][e], x.q[e], pq0);
                pq1 = fmaf(S[m][e + 1], x.q[e + 1], pq1);
            }
            const float pk = group_sum<LPR>(pk0 + pk1);
            const float pq = group_sum<LPR>(pq0 + pq1);
            const float u = fmaf(-bal, pk, x.vb[m]);  // beta (v - alpha S k)
            const float o = fmaf(sal, pq, sqk * u);   // scale (alpha S q + (q.k) u)
#pragma unroll
            for (int e = 0; e < 8; ++e) S[m][e] = fmaf(al, S[m][e], u * x.k[e]);
            // persisted states are written once and read later by commit, never by this kernel
            if constexpr (PMODE == 1) {
                f16x8 hv;
#pragma unroll
                for (int e = 0; e < 8; ++e) hv[e] = (_Float16)S[m][e];
                store_stream<NT>(hv, reinterpret_cast<f16x8*>(static_cast<_Float16*>(a.persist) + nbase * node_elems +
                                                          prow + (size_t)m * RPG * DK));
            } else if constexpr (PMODE == 2) {
                float* dst = static_cast<float*>(a.persist) + nbase * node_elems + prow + (size_t)m * RPG * DK;
                store_stream<NT>(f32x4{S[m][0], S[m][1], S[m][2], S[m][3]}, reinterpret_cast<f32x4*>(dst));
                store_stream<NT>(f32x4{S[m][4], S[m][5], S[m][6], S[m][7]}, reinterpret_cast<f32x4*>(dst + 4));
            }
            if (a.out != nullptr && c == 0)
                put_out<OUT>(a.out, (nbase * a.h_v + h) * DV + row0 + vr0 + m * RPG, o);
        }
        if constexpr (TREE) {
            if (code & kSchedSave) {
                float* dst = myfork + sched_save_slot((uint16_t)code) * fork_stride;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    *reinterpret_cast<f32x4*>(dst + (m * 64 + lane) * 8) = f32x4{S[m][0], S[m][1], S[m][2], S[m][3]};
                    *reinterpret_cast<f32x4*>(dst + (m * 64 + lane) * 8 + 4) = f32x4{S[m][4], S[m][5], S[m][6], S[m][7]};
                }
            }
        }
    };
    auto code_at = [&](int st) { return TREE ? walkL[st < N ? st : N - 1] : (st < N ? st : N - 1); };

    // Two operand buffers in ping-pong: while one node computes, the next
    // node's operands are already on their way from LDS.
    NodeOps<M> opA, opB;
    int codeA = code_at(0), codeB;
    read_node<DK, M>(opA, kL, qL, cL, vbL, sched_node((uint16_t)codeA), c, vr0, rows);
    for (int st = 0; st < N; st += 2) {
        codeB = code_at(st + 1);
        read_node<DK, M>(opB, kL, qL, cL, vbL, sched_node((uint16_t)codeB), c, vr0, rows);
        step(opA, codeA);
        if (st + 1 >= N) break;
        codeA = code_at(st + 2);
        read_node<DK, M>(opA, kL, qL, cL, vbL, sched_node((uint16_t)codeA), c, vr0, rows);
        step(opB, codeB);
    }

    // 4. final state (chains): the exact fp32 state after node N-1
    if constexpr (!TREE) {
        if (a.final_state != nullptr) {
            float* dst = a.final_state + ((size_t)b * a.h_v + h) * head_elems + (size_t)(row0 + wrow + r) * DK + 8 * c;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float* d = dst + (size_t)m * RPG * DK;
                store_stream<NT>(f32x4{S[m][0], S[m][1], S[m][2], S[m][3]}, reinterpret_cast<f32x4*>(d));
                store_stream<NT>(f32x4{S[m][4], S[m][5], S[m][6], S[m][7]}, reinterpret_cast<f32x4*>(d + 4));
            }
        }
    }
}

template <int DK, int M, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void verify_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, false, PMODE, OUT, NT>(a, nullptr);
}

// The fused commit + verify launch: the same body, under its own symbol so kernel
// traces and counters tell it apart from a plain verify.
template <int DK, int M, int PMODE, int OUT, bool NT>
__global__ __launch_bounds__(256) void commit_verify_chain_kernel(const VerifyArgs a) {
    verify_body<DK, M, false, PMODE, OUT, NT>(a, nullptr);
}

template <int DK, int M, int PMODE, int OUT>
__global__ __launch_bounds__(256) void verify_tree_kernel(const VerifyArgs a, const TreeSched t) {
    const int bl = xcd_logical_block(blockIdx.x, gridDim.x) / (a.slices * a.h_v);
    verify_body<DK, M, true, PMODE, OUT, true>(a, t.step[a.per_seq_tree ? bl : 0]);
}

template <int DK, int M, int PMODE, int OUT>
hipError_t launch_one(const VerifyArgs& a, const TreeSched* t, int waves, size_t lds, int grid, hipStream_t st) {
    if (t != nullptr)
        hipLaunchKernelGGL((verify_tree_kernel<DK, M, PMODE, OUT>), dim3(grid), dim3(64 * waves), lds, st, a, *t);
    else if (a.accepted_prev != nullptr && a.nt_stores)
        hipLaunchKernelGGL((commit_verify_chain_kernel<DK, M, PMODE, OUT, true>), dim3(grid), dim3(64 * waves), lds,
                           st, a);
    else if (a.accepted_prev != nullptr)
        hipLaunchKernelGGL((commit_verify_chain_kernel<DK, M, PMODE, OUT, false>), dim3(grid), dim3(64 * waves), lds,
                           st, a);
    else if (a.nt_stores)
        hipLaunchKernelGGL((verify_chain_kernel<DK, M, PMODE, OUT, true>), dim3(grid), dim3(64 * waves), lds, st, a);
    else
        hipLaunchKernelGGL((verify_chain_kernel<DK, M, PMODE, OUT, false>), dim3(grid), dim3(64 * waves), lds, st, a);
    return hipGetLastError();
}

template <int DK, int M, int PMODE>
hipError_t launch_dkmp(const VerifyArgs& a, const TreeSched* t, int waves, size_t lds, int grid, hipStream_t st) {
    switch (a.out_dtype) {
        case GDN_F32: return launch_one<DK, M, PMODE, 0>(a, t, waves, lds, grid, st);
        case GDN_BF16: return launch_one<DK, M, PMODE, 1>(a, t, waves, lds, grid, st);
        case GDN_F16: return launch_one<DK, M, PMODE, 2>(a, t, waves, lds, grid, st);
        default: return hipErrorInvalidValue;
    }
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
