// verify_body.h -- the state-resident verify body shared by the verify family of
// launches (gfx950); included by the sources that instantiate its kernels.
//
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
// LPR = d_k / EPL lanes, EPL elements each (the launches use EPL = 8; the body
// also takes 16, computing every node bit-identically), so one wave holds RPG = 64 / LPR rows per row group and M row groups
// (R = M * RPG rows).  Lane c of a row holds the 8-element chunks c, c + LPR,
// ... of it.  The two row reductions (S k and S q) are DPP sums over the LPR
// lanes of a row; each persisted f16 chunk is one 16-byte store, and the
// chunks of one store instruction cover LPR * 16 contiguous bytes of a row.
// The state never leaves VGPRs between nodes; only the persisted copies, the
// outputs and the final state are written.  All per-node inputs (k, q rows as
// fp32, this slice of v, the gates and q.k) are staged once into LDS, so the
// node loop issues no global loads and never waits on the vector-memory
// counter.
//
// Trees are walked depth first (the host computes the walk): a node whose
// parent is the previous node continues in registers; otherwise the parent's
// exact fp32 state is restored from an LDS fork slot saved when the parent
// (a branch point) was computed.  A chain is the walk 0, 1, ..., N-1.
#include "gdn_device.h"
#pragma once

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
template <int M, int EPL>
struct NodeOps {
    float k[EPL], q[EPL];
    f32x4 coef;  // alpha, beta alpha, scale alpha, scale (q.k)
    float vb[M]; // beta * v for this lane's rows
};

template <int DK, int M, int EPL>
__device__ __forceinline__ void read_node(NodeOps<M, EPL>& x, const float* kL, const float* qL, const f32x4* cL,
                                          const float* vbL, int node, int c, int vr0, int rows) {
    constexpr int LPR = DK / EPL, RPG = 64 / LPR;
#pragma unroll
    for (int j = 0; j < EPL / 8; ++j) {
        const int off = node * DK + 8 * (c + LPR * j);
        const f32x4 k0 = *reinterpret_cast<const f32x4*>(kL + off);
        const f32x4 k1 = *reinterpret_cast<const f32x4*>(kL + off + 4);
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(qL + off);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(qL + off + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x.k[8 * j + e] = k0[e];
            x.k[8 * j + 4 + e] = k1[e];
            x.q[8 * j + e] = q0[e];
            x.q[8 * j + 4 + e] = q1[e];
        }
    }
    x.coef = cL[node];
#pragma unroll
    for (int m = 0; m < M; ++m) x.vb[m] = vbL[node * rows + vr0 + m * RPG];
}

// Inputs of one block of draft nodes.
struct BlockIn {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
};

// One block's staging area in LDS: k[N][DK] and q[N][DK] as fp32, the node
// coefficients (alpha, beta alpha, scale alpha, scale (q.k)) as f32x4 [N] --
// the products formed once here, in fp32 as the node step would form them --
// beta * v [N][rows] for the workgroup's rows, and walk[N] (tree walk codes or
// a replay path).
template <int DK>
struct StageArea {
    float* kL;
    float* qL;
    f32x4* cL;
    float* vbL;
    int* walkL;
    __device__ static int floats(int N, int rows) { return (2 * N * DK + 4 * N + N * rows + N + 3) & ~3; }
    __device__ StageArea(float* base, int N, int rows) {
        kL = base;
        qL = kL + N * DK;
        cL = reinterpret_cast<f32x4*>(qL + N * DK);
        vbL = reinterpret_cast<float*>(cL + N);
        walkL = reinterpret_cast<int*>(vbL + N * rows);
    }
};

// Staging of every node's inputs of NB blocks into LDS, one item per lane: an
// 8-element chunk of k and of q, one beta * v entry and one node's gates (of
// every block).  A lane's global loads are unconditional (indices clamped into
// range, the dtype entering only through addresses) and converted only when
// stored, so they all issue back to back and cost one memory round trip; the
// first item of every lane is loaded before the state rows (which may wait on
// the slot and accepted-node lookups) and stored after them, so that round
// trip overlaps the state's.  An item past the last one loads clamped
// duplicates and stores nothing.  `walk` (tree verify only) goes to block 0's walk
// area.
template <int NB>
struct StageRegs {
    u32x4 k[NB][2], q[NB][2];  // bf16: the 8 elements in [0] ([1] repeats it); fp32: 4 in each
    uint32_t v[NB];            // the 32-bit word holding v (bf16: one of its halves)
    float vbeta[NB], ga[NB], gb[NB];
    bool v_hi;                 // bf16 v in the upper half of its word
};

template <int DK>
struct StageItem {
    int e, chunks, nvb, N;
    __device__ bool kq() const { return e < chunks; }
    __device__ bool v() const { return e < nvb; }
    __device__ bool g() const { return e < N; }
};

template <int DK, int NB>
__device__ __forceinline__ void stage_load(StageRegs<NB>& r, const StageItem<DK>& it, const BlockIn (&in)[2],
                                           const VerifyArgs& a, int b, int h, int g, int row0) {
    constexpr int LPR = DK / 8;
    const int N = a.n_nodes, rows = a.rows_per_wg, DV = a.d_v;
    const bool bf16 = a.qkv_bf16 != 0;
    const size_t esz = bf16 ? 2 : 4;
    const int ekq = it.e < it.chunks ? it.e : it.chunks - 1;
    const int ev = it.e < it.nvb ? it.e : it.nvb - 1;
    const int eg = it.e < it.N ? it.e : it.N - 1;
    const size_t kqi = GDN_AT((((size_t)b * N + ekq / LPR) * a.h_qk + g) * DK + 8 * (ekq % LPR), 8,
                              (size_t)a.batch * N * a.h_qk * DK, a.status);
    const int n = ev / rows;
    const size_t vi = GDN_AT((((size_t)b * N + n) * a.h_v + h) * DV + row0 + ev % rows, 1,
                             (size_t)a.batch * N * a.h_v * DV, a.status);
    [[maybe_unused]] const size_t ng = (size_t)a.batch * N * a.h_v;  // gate entries
    const size_t vb = bf16 ? (vi * 2) & ~(size_t)3 : vi * 4;
    r.v_hi = bf16 && (vi & 1);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const unsigned char* kp = static_cast<const unsigned char*>(in[i].k) + kqi * esz;
        const unsigned char* qp = static_cast<const unsigned char*>(in[i].q) + kqi * esz;
        r.k[i][0] = *reinterpret_cast<const u32x4*>(kp);
        r.k[i][1] = *reinterpret_cast<const u32x4*>(kp + (bf16 ? 0 : 16));
        r.q[i][0] = *reinterpret_cast<const u32x4*>(qp);
        r.q[i][1] = *reinterpret_cast<const u32x4*>(qp + (bf16 ? 0 : 16));
        r.v[i] = *reinterpret_cast<const uint32_t*>(static_cast<const unsigned char*>(in[i].v) + vb);
        r.vbeta[i] = in[i].beta[GDN_AT(((size_t)b * N + n) * a.h_v + h, 1, ng, a.status)];
        r.ga[i] = in[i].alpha[GDN_AT(((size_t)b * N + eg) * a.h_v + h, 1, ng, a.status)];
        r.gb[i] = in[i].beta[GDN_AT(((size_t)b * N + eg) * a.h_v + h, 1, ng, a.status)];
    }
}

__device__ __forceinline__ void raw8_to_f32(const u32x4 (&w)[2], bool bf16, float (&x)[8]) {
    if (bf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[0][i]);
            x[2 * i + 1] = bf16_hi(w[0][i]);
        }
    } else {
        const f32x4 lo = __builtin_bit_cast(f32x4, w[0]), hi = __builtin_bit_cast(f32x4, w[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = lo[i];
            x[4 + i] = hi[i];
        }
    }
}

template <int DK, int NB>
__device__ __forceinline__ void stage_store(const StageRegs<NB>& r, const StageItem<DK>& it, bool bf16,
                                            float scale, const StageArea<DK> (&sa)[2], const uint16_t* walk) {
    constexpr int LPR = DK / 8;
    const int e = it.e;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        float kf[8], qf[8];
        raw8_to_f32(r.k[i], bf16, kf);
        raw8_to_f32(r.q[i], bf16, qf);
        float part = 0.f;
        if (it.kq()) {
            float* kd = sa[i].kL + (e / LPR) * DK + 8 * (e % LPR);
            float* qd = sa[i].qL + (e / LPR) * DK + 8 * (e % LPR);
            *reinterpret_cast<f32x4*>(kd) = f32x4{kf[0], kf[1], kf[2], kf[3]};
            *reinterpret_cast<f32x4*>(kd + 4) = f32x4{kf[4], kf[5], kf[6], kf[7]};
            *reinterpret_cast<f32x4*>(qd) = f32x4{qf[0], qf[1], qf[2], qf[3]};
            *reinterpret_cast<f32x4*>(qd + 4) = f32x4{qf[4], qf[5], qf[6], qf[7]};
#pragma unroll
            for (int j = 0; j < 8; ++j) part = fmaf(kf[j], qf[j], part);
        }
        part = group_sum<LPR>(part);
        if (it.kq() && (e % LPR) == 0) reinterpret_cast<float*>(sa[i].cL + e / LPR)[3] = scale * part;
        if (it.v()) {
            const float vv = !bf16 ? __builtin_bit_cast(float, r.v[i]) : r.v_hi ? bf16_hi(r.v[i]) : bf16_lo(r.v[i]);
            sa[i].vbL[e] = r.vbeta[i] * vv;
        }
        if (it.g()) {
            reinterpret_cast<float*>(sa[i].cL + e)[0] = r.ga[i];
            reinterpret_cast<float*>(sa[i].cL + e)[1] = r.gb[i] * r.ga[i];
            reinterpret_cast<float*>(sa[i].cL + e)[2] = scale * r.ga[i];
            if (i == 0 && walk != nullptr) sa[0].walkL[e] = walk[e];
        }
    }
}

// Where a lane's rows sit: the lane holds chunks c, c + LPR, ... of rows
// wrow + r + m RPG, m < M, of the workgroup's slice.
struct LaneRows {
    int b, h, row0, wrow, r, c;
};

// This lane's part of rows wrow + r + m RPG of a d_v x DK fp32 head.
template <int DK, int M, int EPL>
__device__ __forceinline__ void load_rows(float (&S)[M][EPL], const float* head_base, const LaneRows& L) {
    constexpr int LPR = DK / EPL, RPG = 64 / LPR;
    const float* src = head_base + (size_t)(L.row0 + L.wrow + L.r) * DK + 8 * L.c;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < EPL / 8; ++j) {
            const float* p = src + (size_t)m * RPG * DK + 8 * LPR * j;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[m][8 * j + e] = x0[e];
                S[m][8 * j + 4 + e] = x1[e];
            }
        }
}

template <int DK, int M, int EPL, bool NT>
__device__ __forceinline__ void store_state_rows(float* head_base, const LaneRows& L, const float (&S)[M][EPL]) {
    constexpr int LPR = DK / EPL, RPG = 64 / LPR;
    float* dst = head_base + (size_t)(L.row0 + L.wrow + L.r) * DK + 8 * L.c;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < EPL / 8; ++j) {
            float* d = dst + (size_t)m * RPG * DK + 8 * LPR * j;
            store_stream<NT>(f32x4{S[m][8 * j], S[m][8 * j + 1], S[m][8 * j + 2], S[m][8 * j + 3]},
                             reinterpret_cast<f32x4*>(d));
            store_stream<NT>(f32x4{S[m][8 * j + 4], S[m][8 * j + 5], S[m][8 * j + 6], S[m][8 * j + 7]},
                             reinterpret_cast<f32x4*>(d + 4));
        }
}

// The state rows a lane holds, loaded raw (16-byte words, unconditionally, the
// element type entering only through addresses) and widened to fp32 later, so
// the loads are in flight while the wave does other work.  F16: the eight
// elements of a chunk in w[..][0] (w[..][1] repeats it); fp32: four in each.
template <int M, int EPL>
struct RowsRaw {
    u32x4 w[M][EPL / 8][2];
};

template <int DK, int M, int EPL>
__device__ __forceinline__ void load_rows_raw(RowsRaw<M, EPL>& r, const void* head_base, bool f16,
                                              const LaneRows& L) {
    constexpr int LPR = DK / EPL, RPG = 64 / LPR;
    const size_t esz = f16 ? 2 : 4;
    const unsigned char* src = static_cast<const unsigned char*>(head_base) +
                               ((size_t)(L.row0 + L.wrow + L.r) * DK + 8 * L.c) * esz;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < EPL / 8; ++j) {
            const unsigned char* p = src + ((size_t)m * RPG * DK + 8 * LPR * j) * esz;
            r.w[m][j][0] = *reinterpret_cast<const u32x4*>(p);
            r.w[m][j][1] = *reinterpret_cast<const u32x4*>(p + (f16 ? 0 : 16));
        }
}

template <int M, int EPL>
__device__ __forceinline__ void widen_rows(float (&S)[M][EPL], const RowsRaw<M, EPL>& r, bool f16) {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < EPL / 8; ++j) {
            if (f16) {
                const f16x8 hv = __builtin_bit_cast(f16x8, r.w[m][j][0]);
#pragma unroll
                for (int e = 0; e < 8; ++e) S[m][8 * j + e] = (float)hv[e];
            } else {
                const f32x4 lo = __builtin_bit_cast(f32x4, r.w[m][j][0]), hi = __builtin_bit_cast(f32x4, r.w[m][j][1]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[m][8 * j + e] = lo[e];
                    S[m][8 * j + 4 + e] = hi[e];
                }
            }
        }
}

// The node loop over n_steps steps of one staged block: per step the optional
// fork restore, the two row reductions, the update, the persisted copy, the
// output, the optional fork save.  CODES: step st runs node walk[st] (a tree
// walk, or a replay path); otherwise step st runs node st.  FORKS (tree walks):
// the codes carry fork bits.  The walk codes sit in one register (lane i holds
// code i, read with a lane-select), so no step waits on LDS for its code; the
// next step's operands -- and, FORKS, its fork slot, read whether or not it
// restores -- are read from LDS while the current step computes.  Reading the
// slot one step early is safe because a slot being restored is live: no save
// between the parent's and the child's steps writes it (the walk's fork slots
// form a stack).
// OUTS = false (a replay): no outputs, so neither S q nor o is formed.
template <int DK, int M, int EPL, bool CODES, bool FORKS, int PMODE, int OUT, bool NT, bool OUTS = true>
__device__ __forceinline__ void node_loop(float (&S)[M][EPL], const StageArea<DK>& sa, int n_steps,
                                          const VerifyArgs& a, void* out, const LaneRows& L, float* myfork,
                                          int fork_stride) {
    static_assert(!FORKS || CODES, "fork bits come with walk codes");
    static_assert(kMaxNodes <= 64, "one walk code per lane");
    constexpr int LPR = DK / EPL, RPG = 64 / LPR, NJ = EPL / 8;
    const int lane = threadIdx.x & 63, c = L.c, b = L.b, h = L.h;
    const int N = a.n_nodes, DV = a.d_v, rows = a.rows_per_wg;
    const size_t head_elems = (size_t)DV * DK;
    // per-node strides fit 32 bits (the host bounds h_v d_v d_k * 32 below 2^32):
    // a lane's persist and output addresses are a base plus node * stride
    const uint32_t pstride = (uint32_t)(a.h_v * head_elems);  // persist elements per node
    const uint32_t ostride = (uint32_t)(a.h_v * DV);          // output elements per node
    const int vr0 = L.wrow + L.r;  // this lane's first row inside the slice
    const size_t seq0 = (size_t)b * N;
    const size_t pbase = seq0 * pstride + (size_t)h * head_elems + (size_t)(L.row0 + vr0) * DK + 8 * c;
    const size_t obase = seq0 * ostride + (size_t)h * DV + L.row0 + vr0;
    using Slot = float[M][EPL];

    auto step = [&](const NodeOps<M, EPL>& x, const Slot& fork_in, int code) {
        const int node = sched_node((uint16_t)code);
        if constexpr (FORKS) {
            if (code & kSchedRestore) {
                // a branch on the wave-uniform code, not eight selects on every step
                // (an empty volatile asm keeps the compiler from flattening it)
                asm volatile("");
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) S[m][e] = fork_in[m][e];
            }
        }
        const float al = x.coef[0];
        const float bal = x.coef[1];  // beta * alpha
        const float sal = x.coef[2];  // scale * alpha
        const float sqk = x.coef[3];  // scale * (q . k)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            // Row sums in one fixed order for every layout: each 8-element chunk
            // is summed with two accumulators (even and odd elements), and the
            // chunk sums of a row meet in the binary tree of the DPP steps over
            // LPR lanes.  With two chunks per lane (LPR = 8 at d_k = 128), lane c
            // holds chunks c and c + 8: each chunk's sum runs the 8-lane tree on
            // its own, leaving the sums of chunks 0-7 and 8-15, which are then
            // added -- the same tree the 16-lane layout forms, so a node's state
            // is bit-identical whichever layout a launch takes.
            float pk = 0.f, pq = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int e0 = 8 * j;
                float pk0 = S[m][e0] * x.k[e0], pk1 = S[m][e0 + 1] * x.k[e0 + 1];
                float pq0 = S[m][e0] * x.q[e0], pq1 = S[m][e0 + 1] * x.q[e0 + 1];
#pragma unroll
                for (int e = e0 + 2; e < e0 + 8; e += 2) {
                    pk0 = fmaf(S[m][e], x.k[e], pk0);
                    pk1 = fmaf(S[m][e + 1], x.k[e + 1], pk1);
                    if constexpr (OUTS) {
                        pq0 = fmaf(S[m][e], x.q[e], pq0);
                        pq1 = fmaf(S[m][e + 1], x.q[e + 1], pq1);
                    }
                }
                float sk = pk0 + pk1, sq = 0.f;
                if constexpr (OUTS) {
                    sq = pq0 + pq1;
                    group_sum2<LPR>(sk, sq);
                } else {
                    sk = group_sum<LPR>(sk);
                }
                if (j == 0) {
                    pk = sk;
                    pq = sq;
                } else {
                    pk += sk;
                    pq += sq;
                }
            }
            const float u = fmaf(-bal, pk, x.vb[m]);  // beta (v - alpha S k)
            const float o = fmaf(sal, pq, sqk * u);   // scale (alpha S q + (q.k) u)
#pragma unroll
            for (int e = 0; e < EPL; ++e) S[m][e] = fmaf(al, S[m][e], u * x.k[e]);
            if constexpr (PMODE == 1) opaque_f32x8(S[m]);  // the persisted f16 is this fp32 state rounded
            // persisted states are written once and read later by commit, never by this kernel
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const size_t at = GDN_AT(pbase + (uint32_t)node * pstride + (uint32_t)(m * RPG * DK + 8 * LPR * j), 8,
                                         (size_t)a.batch * N * pstride, a.status);
                if constexpr (PMODE == 1) {
                    const float* x = &S[m][8 * j];
                    const f16x8 hv = to_f16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
                    store_stream<NT>(hv, reinterpret_cast<f16x8*>(static_cast<_Float16*>(a.persist) + at));
                } else if constexpr (PMODE == 2) {
                    // fp32 node states: plain stores (two 16-byte halves of each lane's 32 bytes;
                    // written non-temporally, the half-line pieces measured 18% slower)
                    float* dst = static_cast<float*>(a.persist) + at;
                    store_stream<false>(f32x4{S[m][8 * j], S[m][8 * j + 1], S[m][8 * j + 2], S[m][8 * j + 3]},
                                     reinterpret_cast<f32x4*>(dst));
                    store_stream<false>(f32x4{S[m][8 * j + 4], S[m][8 * j + 5], S[m][8 * j + 6], S[m][8 * j + 7]},
                                     reinterpret_cast<f32x4*>(dst + 4));
                }
            }
            if (OUTS && out != nullptr && c == 0)
                put_out<OUT>(out, GDN_AT(obase + (uint32_t)node * ostride + (uint32_t)(m * RPG), 1,
                                         (size_t)a.batch * N * ostride, a.status), o);
        }
        if constexpr (FORKS) {
            if (code & kSchedSave) {
                float* dst = myfork + sched_save_slot((uint16_t)code) * fork_stride;
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int j = 0; j < 2 * NJ; ++j)
                        *reinterpret_cast<f32x4*>(dst + (m * 64 + lane) * EPL + 4 * j) =
                            f32x4{S[m][4 * j], S[m][4 * j + 1], S[m][4 * j + 2], S[m][4 * j + 3]};
            }
        }
    };
    // this lane's fork-slot entry of a step's restore slot (slot 0 without the bit)
    auto read_fork = [&](Slot& r, int code) {
        if constexpr (FORKS) {
            const float* src = myfork + sched_restore_slot((uint16_t)code) * fork_stride;
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int j = 0; j < 2 * NJ; ++j) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + (m * 64 + lane) * EPL + 4 * j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[m][4 * j + e] = x0[e];
                }
        }
    };
    const int wcode = CODES && lane < n_steps ? sa.walkL[lane] : 0;
    auto code_at = [&](int st) {
        const int x = st < n_steps ? st : n_steps - 1;
        return CODES ? __builtin_amdgcn_readlane(wcode, x) : x;
    };

    // Two operand buffers in ping-pong: while one node computes, the next
    // node's operands are already on their way from LDS.
    NodeOps<M, EPL> opA, opB;
    Slot fkA, fkB;
    int codeA = code_at(0), codeB;
    read_node<DK, M, EPL>(opA, sa.kL, sa.qL, sa.cL, sa.vbL, sched_node((uint16_t)codeA), c, vr0, rows);
    read_fork(fkA, codeA);
    for (int st = 0; st < n_steps; st += 2) {
        codeB = code_at(st + 1);
        read_node<DK, M, EPL>(opB, sa.kL, sa.qL, sa.cL, sa.vbL, sched_node((uint16_t)codeB), c, vr0, rows);
        read_fork(fkB, codeB);
        step(opA, fkA, codeA);
        if (st + 1 >= n_steps) break;
        codeA = code_at(st + 2);
        read_node<DK, M, EPL>(opA, sa.kL, sa.qL, sa.cL, sa.vbL, sched_node((uint16_t)codeA), c, vr0, rows);
        read_fork(fkA, codeA);
        step(opB, fkB, codeB);
    }
}

// One launch of the verify family (see VerifyKind).  The per-node arithmetic
// is the same in every kind, so a node's state does not depend on whether it
// was reached by a chain, a tree walk or a replay.
template <int DK, int M, int EPL, int KIND, int PMODE, int OUT, bool NT>
__device__ __forceinline__ void verify_body(const VerifyArgs& a, const uint16_t* walk, const int8_t* par) {
    constexpr int LPR = DK / EPL; // lanes per state row
    constexpr int RPG = 64 / LPR; // rows per row group
    constexpr int R = M * RPG;    // rows per wave
    constexpr bool TREE = KIND == kVerifyTree || KIND == kCommitVerifyTree;  // a host-planned walk with forks
    constexpr bool REPLAY = KIND == kReplayChain || KIND == kReplayTree || KIND == kReplayVerifyChain;
    constexpr int NB = KIND == kReplayVerifyChain ? 2 : 1;  // staged blocks
    constexpr bool FUSED = KIND == kCommitVerifyChain || KIND == kCommitVerifyTree;  // the commit is part of the state load
    constexpr bool HAS_ACC = FUSED || REPLAY;                // an accepted node is read per sequence
    extern __shared__ __align__(16) float lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = a.rows_per_wg / R;  // the launch's block is 64 nwaves threads

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

    // 2a. the first staging item of this lane: global loads issued before the state's
    // (and before the slot and accepted-node lookups the state load waits on)
    const BlockIn in[2] = {{KIND == kReplayVerifyChain ? a.rq : a.q, KIND == kReplayVerifyChain ? a.rk : a.k,
                            KIND == kReplayVerifyChain ? a.rv : a.v, KIND == kReplayVerifyChain ? a.ralpha : a.alpha,
                            KIND == kReplayVerifyChain ? a.rbeta : a.beta},
                           {a.q, a.k, a.v, a.alpha, a.beta}};
    // A tree (up to 32 nodes) has more staging items than threads; its first two
    // items per lane are loaded up front, so their loads share one round trip.
    constexpr int NI = TREE ? 2 : 1;
    const uint16_t* stage_walk = TREE ? walk : nullptr;
    StageItem<DK> item[NI];
    StageRegs<NB> sr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        item[i].chunks = N * (DK / 8);
        item[i].nvb = N * rows;
        item[i].N = N;
        item[i].e = wave * 64 + lane + i * 64 * nwaves;
        stage_load<DK, NB>(sr[i], item[i], in, a, b, h, g, row0);
    }
    const int items = item[0].chunks > item[0].nvb ? item[0].chunks : item[0].nvb;


    // The slot and the accepted node of the committed block (fused commit or replay)
    // are both read before anything is stored, so they are scalar loads, whose wait
    // does not also wait for the staging loads in flight.
    int s = b;
    if (a.state_slot != nullptr) s = a.state_slot[b];
    int acc = 0;
    if constexpr (HAS_ACC) acc = a.accepted_prev[b];
    if (a.state_slot != nullptr && (s < 0 || s >= a.n_slots)) {
        if (tid == 0 && a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
        return;
    }
    // the accepted node must be in range
    if (HAS_ACC && (acc < 0 || acc >= N)) {
        if (tid == 0 && a.status != nullptr) a.status[0] = GDN_ERR_NODE;
        return;
    }

    const int stage_floats = StageArea<DK>::floats(N, rows);
    // (the second area is used by a replay + verify only)
    const StageArea<DK> sa[2] = {StageArea<DK>(lds, N, rows), StageArea<DK>(lds + stage_floats, N, rows)};
    float* forkL = lds + NB * stage_floats;

    // 1. this wave's state rows -> VGPRs
    LaneRows L;
    L.b = b;
    L.h = h;
    L.row0 = row0;
    L.c = lane % LPR;
    L.r = lane / LPR;
    L.wrow = wave * R;  // first row of this wave inside the slice
#ifdef GDN_DEBUG
    // the lane's last row inside the head
    L.wrow = (int)GDN_AT(L.row0 + L.wrow + L.r + (M - 1) * RPG, 1, DV, a.status) - (L.row0 + L.r + (M - 1) * RPG);
#endif
    const size_t head_elems = (size_t)DV * DK;
    // extents of the state array and of the per-sequence head arrays (debug build's checks)
    [[maybe_unused]] const size_t state_end =
        (size_t)(a.state_slot != nullptr ? a.n_slots : a.batch) * a.h_v * head_elems;
    [[maybe_unused]] const size_t heads_end = (size_t)a.batch * a.h_v * head_elems;
    float* cache_head = (a.state_w != nullptr ? a.state_w : const_cast<float*>(a.state)) +
                        GDN_AT(((size_t)s * a.h_v + h) * head_elems, head_elems, state_end, a.status);
    // The starting state: the cached state, or (fused commit) the previous step's accepted
    // node -- its exact fp32 final state when the whole chain was accepted, else (and
    // always after a tree) its persisted copy, widened to fp32 -- which is also written
    // back to the state cache.
    // Its loads are issued first; the staging's LDS work runs while they are in flight.
    const void* src_head = a.state + GDN_AT(((size_t)s * a.h_v + h) * head_elems, head_elems, state_end, a.status);
    bool src_f16 = false;
    if constexpr (FUSED) {
        if (!TREE && a.final_prev != nullptr && acc == N - 1) {
            src_head = a.final_prev + GDN_AT(((size_t)b * a.h_v + h) * head_elems, head_elems, heads_end, a.status);
        } else {
            src_f16 = a.persist_prev_f16 != 0;
            const size_t off = GDN_AT((((size_t)b * N + acc) * a.h_v + h) * head_elems, head_elems,
                                      heads_end * N, a.status);
            src_head = src_f16 ? static_cast<const void*>(static_cast<const _Float16*>(a.persist_prev) + off)
                               : static_cast<const void*>(static_cast<const float*>(a.persist_prev) + off);
        }
    }
    RowsRaw<M, EPL> raw;
    load_rows_raw<DK, M, EPL>(raw, src_head, src_f16, L);

    // 2b. stage every node's inputs (both blocks of a replay + verify): the items
    // loaded above, then any further ones (when N * d_k / 8 exceeds them)
#pragma unroll
    for (int i = 0; i < NI; ++i) stage_store<DK, NB>(sr[i], item[i], a.qkv_bf16 != 0, a.scale, sa, stage_walk);
    for (int base = wave * 64 + NI * 64 * nwaves; base < items; base += 64 * nwaves) {  // wave-uniform bound
        StageItem<DK> it = item[0];
        it.e = base + lane;
        stage_load<DK, NB>(sr[0], it, in, a, b, h, g, row0);
        stage_store<DK, NB>(sr[0], it, a.qkv_bf16 != 0, a.scale, sa, stage_walk);
    }

    // 1b. the state rows in fp32 (and, fused, the commit)
    float S[M][EPL];
    widen_rows<M, EPL>(S, raw, src_f16);
    if constexpr (FUSED) store_state_rows<DK, M, EPL, NT>(cache_head, L, S);

    // a tree replay runs the accepted node's root path, root first
    int n_steps = N;
    if constexpr (KIND == kReplayChain || KIND == kReplayVerifyChain) n_steps = acc + 1;
    if constexpr (KIND == kReplayTree) {
        int d = 0;
        for (int x = acc; x >= 0 && d < kMaxNodes; x = par[x]) ++d;
        n_steps = d;
        if (tid == 0) {
            int x = acc;
            for (int i = d - 1; i >= 0; --i) {
                sa[0].walkL[i] = x;
                x = par[x];
            }
        }
    }
    __syncthreads();

    // 3. the node loops
    const int fork_stride = nwaves * R * DK;
    float* myfork = forkL + L.wrow * DK;
    if constexpr (REPLAY) {
        // replay of the committed block: no outputs, no persisted copies; the result
        // is the committed state
        node_loop<DK, M, EPL, KIND == kReplayTree, false, 0, OUT, NT, false>(S, sa[0], n_steps, a, nullptr, L, myfork,
                                                                      fork_stride);
        store_state_rows<DK, M, EPL, NT>(cache_head, L, S);
    }
    if constexpr (KIND == kReplayVerifyChain || !REPLAY) {
        node_loop<DK, M, EPL, TREE, TREE, PMODE, OUT, NT>(S, sa[NB - 1], N, a, a.out, L, myfork, fork_stride);
        // 4. final state (chains): the exact fp32 state after node N-1
        if constexpr (!TREE) {
            if (a.final_state != nullptr)
                store_state_rows<DK, M, EPL, NT>(
                    a.final_state + GDN_AT(((size_t)b * a.h_v + h) * head_elems, head_elems, heads_end, a.status), L,
                    S);
        }
    }
}

// Launch of kernel K; a launch over 64 KB of LDS first allows K all of it.
template <auto K, typename... Args>
hipError_t go(int grid, int waves, size_t lds, hipStream_t st, Args... args) {
    if (lds > (size_t)kDefaultLdsBytes) {
        const hipError_t e = allow_max_lds<K>();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(K, dim3(grid), dim3(64 * waves), lds, st, args...);
    return hipGetLastError();
}

}  // namespace
}  // namespace gdn
