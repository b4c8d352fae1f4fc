// prefill.hip -- chunked (WY / UT) prefill of the gated delta rule on gfx950.
//
// The pages name chunked linear-attention prefill as an engine feature (page
// "We got 207 tok/s with Qwen3.5-27B on an RTX 3090", section "Prefill"); the
// chunk algebra here is derived from the rule.  With H = S^T (d_k x d_v) and
// a chunk of C = 64 tokens starting from H_0:
//   l_t = sum_{s<=t} log alpha_s,  gamma_t = e^{l_t},  Gamma_{t,i} = e^{l_t - l_i}
//   A   = strict_lower(beta_t Gamma_{t,i} k_t.k_i),  T = (I + A)^{-1},  T' = T diag(beta)
//   R   = V - diag(gamma) K H_0,                   U = T' R
//   O   = scale [diag(gamma) Q H_0 + (Gamma o tril(Q K^T)) U]
//   H_C = gamma_C H_0 + K^T diag(Gamma_{C,.}) U
// (U = T' R is the usual W / U' form, T diag(beta) V - T diag(beta gamma) K H_0,
// with the product by T applied once to the combined right-hand side.)
//
// Two kernels.
//  * prepare (one workgroup per (sequence, chunk, q/k head), all in
//    parallel): everything that does not depend on the state -- K K^T and
//    Q K^T on the matrix cores once per q/k head, then per value head on one
//    wave the gates, the masked matrices, and the UT transform
//    T = (I + A)^{-1} in fp32 (16 x 16 diagonal blocks by forward
//    substitution, off-diagonal blocks by v_mfma_f32_16x16x4_f32).  It writes
//    T' and P = Gamma o tril(Q K^T) in f16, the per-token gate factors, and
//    K, Q in f16 (once per q/k head) to the workspace, every matrix in the
//    scan's operand-fragment order.
//  * scan (one workgroup per (sequence, value head, 64 or 32 value columns),
//    sequential over chunks): per 16 columns a chain wave keeps the state in
//    accumulators for the whole prompt and forms K H, R, U = T' R and the
//    state update, and an output wave forms Q H and O = gamma Q H + P U, all
//    with v_mfma_f32_16x16x32_f16 from operands that buffer-to-LDS loads
//    brought in during the previous chunk.
// All matrix-core operands are f16 with fp32 accumulation: the bf16 inputs are
// exact in f16 within the f16 range, and the derived operands (T', R, P, U, H)
// keep f16's 11-bit significand, enough for the parity bar where bf16 is not.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kC = GDN_PREFILL_CHUNK;  // tokens per chunk
constexpr float kLogFloor = -80.f;     // log alpha is clamped here (a zero gate -> e^-80)
constexpr float kLog2e = 1.44269504088896340736f;

// Gate arithmetic runs in base 2 on the hardware's v_log_f32 / v_exp_f32
// (about 1 ulp each): l2_t = sum log2 alpha_s, clamped per token at
// kLogFloor / ln 2, and every factor is 2^(difference of l2).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16(const h8& a, const h8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// MFMA operand fragment of a row-major f16 matrix X (leading dimension ld):
// rows row0 + lane % 16, contraction columns k0 + 8 * (lane / 16) .. + 8.
__device__ __forceinline__ h8 frag(const _Float16* X, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const h8*>(X + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ h8 to_h8(const float (&x)[8]) {
    // a whole-vector conversion: one packed convert per pair
    typedef float f8 __attribute__((ext_vector_type(8)));
    const f8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    return __builtin_convertvector(v, h8);
}

// Two accumulator tiles (rows 4 g + r of each) as one f16 operand fragment:
// whole-vector conversions (one packed convert per pair, round to nearest even).
__device__ __forceinline__ h8 pack_h8(const f32x4& lo, const f32x4& hi) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 a = __builtin_convertvector(lo, h4), b = __builtin_convertvector(hi, h4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Raw 16-byte loads of 8 elements (bf16 or fp32 source, BF16 fixed at compile
// time) kept in registers until they are converted into LDS; fp32 needs two.
// Loads are unconditional (callers clamp the index), so no load waits on a
// branch merge.
struct Raw8 {
    u32x4 w0, w1;
};
template <bool BF16>
__device__ __forceinline__ void raw_load(Raw8& r, const void* base, size_t idx) {
    if constexpr (BF16) {
        r.w0 = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
    } else {
        r.w0 = *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + idx);
        r.w1 = *reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + idx + 4);
    }
}
// `bad` is set when an element is outside the f16 range (|x| > 65504, or not a
// number): the matrix-core operands would not hold it.
template <bool BF16>
__device__ __forceinline__ h8 raw_to_h8(const Raw8& r, bool valid, bool& bad) {
    float x[8];
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(r.w0[i]);
            x[2 * i + 1] = bf16_hi(r.w0[i]);
        }
    } else {
        // whole-vector bit casts: a bit cast of one ext_vector element was
        // lowered to element 0 for every index by this compiler
        const f32x4 lo = __builtin_bit_cast(f32x4, r.w0), hi = __builtin_bit_cast(f32x4, r.w1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = lo[i];
            x[4 + i] = hi[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[i] = valid ? x[i] : 0.f;
        bad |= !(__builtin_fabsf(x[i]) <= 65504.f);
    }
    return to_h8(x);
}

// Row order of the scan's 16-row tiles (see the scan kernel): row c of tile
// `tile` when tiles (2u, 2u+1) form one 32-wide contraction block.
__device__ __forceinline__ int pair_row(int tile, int c) {
    return 32 * (tile >> 1) + 8 * (c >> 2) + 4 * (tile & 1) + (c & 3);
}

// Workspace layout (bytes), per chunk unit u (a sequence's chunk ck is unit
// unit0 + ck; units of one launch are numbered sequence after sequence):
//   T', P  [units][h_v][C x C]     f16, T' = T diag(beta)
//   gates  [units][h_v][3][C]      fp32: gamma_t, beta_t, Gamma_{C,t}
//   K, Q   [units][h_qk][C x d_k]  f16
// The matrices are stored in the scan's operand-fragment order: fragment f
// (1 KB) holds, for lane l = 16 g + c, the 8 contraction-consecutive values of
// row pair_row(tile, c) starting at column 32 (block) + 8 g, at f * 1 KB + 16 l.
// K and Q: f = tile * (d_k / 32) + block over the C x d_k matrix; T' and P: the six
// lower-triangular (tile, block) pairs in the order (0,0) (1,0) (2,0) (2,1)
// (3,0) (3,1).  So every load of the scan is one contiguous kilobyte.
struct WsLayout {
    size_t T, P, G, K, Q, total;
};
__host__ __device__ inline WsLayout ws_layout(size_t units, int h_qk, int h_v, int d_k) {
    WsLayout w;
    w.T = 0;
    w.P = w.T + units * h_v * kC * kC * 2;
    w.G = w.P + units * h_v * kC * kC * 2;
    w.K = w.G + units * h_v * 3 * kC * 4;
    w.Q = w.K + units * h_qk * (size_t)d_k * kC * 2;
    w.total = w.Q + units * h_qk * (size_t)d_k * kC * 2;
    return w;
}

// Where sequence b of a launch lives: its first token in the packed token
// dimension, its tokens, its first chunk unit and chunk count, and the index
// of its first emitted boundary state.  Equal-length launches compute these;
// varlen launches read them from the host-built tables.
struct SeqInfo {
    int tok0, T, unit0, nch, cst0;
};
__device__ __forceinline__ SeqInfo seq_info(const PrefillArgs& a, const PrefillSeqs& t, int b) {
    SeqInfo q;
    if (a.varlen) {
        q.tok0 = t.tok0[b];
        q.T = t.len[b];
        q.unit0 = t.unit0[b];
        q.nch = t.unit0[b + 1] - q.unit0;
        q.cst0 = t.cst0[b];
    } else {
        q.T = a.T;
        q.nch = (a.T + kC - 1) / kC;
        q.tok0 = b * a.T;
        q.unit0 = b * q.nch;
        q.cst0 = b * a.seq_states;
    }
    return q;
}

// ---------------------------------------------------------------------------
// prepare: one (sequence, chunk, q/k head) per workgroup
// ---------------------------------------------------------------------------
// K and Q are loaded and, once per q/k head on the matrix cores, the 10 lower
// 16 x 16 tiles of K K^T (four on wave 0, two on each other wave) and, on
// waves 1-3, the 12 tiles of (Q K^T)^T that P's six fragments need, kept in
// the registers of the wave that formed them.  The (Q K^T)^T tiles take keys
// in rows pair_row(pi, .) and queries in columns pair_row(pt, .), so tiles
// (2v, p) and (2v + 1, p) are P's fragment (p, v) as they stand: P's
// fragments go from those registers to the workspace, never through LDS.
// Every value head's gates are formed up front, one head per wave.  Then the
// value heads, one after another: the K K^T tiles become the tiles of
// A = strict_lower(beta_t Gamma_{t,i} k_t.k_i) in LDS; one wave forms the
// diagonal 16 x 16 blocks of T = (I + A)^-1 by forward substitution while the
// others write P = Gamma o tril(Q K^T); the off-diagonal blocks follow one
// column per wave (three, two and one blocks, v_mfma_f32_16x16x4_f32); then
// all four write T' = T diag(beta) and, in the same phase, form the next value
// head's A in the other of two A buffers (three barriers per value head).
// Lower tiles are kept tile-major: tile (it, jt), jt <= it, is tile number
// it (it + 1) / 2 + jt, element (r, c) at r * kTS + c: rows padded to 20 floats
// (16-byte aligned), so the column reads of the matrix-core operands and the
// row reads of the output fragments fall on different banks.  The working set
// reuses the LDS of the K, Q chunk; four workgroups fit a CU.
__device__ __forceinline__ constexpr int tix(int it, int jt) { return it * (it + 1) / 2 + jt; }
constexpr int kTS = 20;           // row stride of a 16 x 16 fp32 tile in LDS (floats)
constexpr int kTile = 16 * kTS;   // floats per tile
__device__ __forceinline__ constexpr int tile_row(int tx) { return tx < 1 ? 0 : tx < 3 ? 1 : tx < 6 ? 2 : 3; }

// The working set: A of two value heads (buffer j % 2 for head j, so the
// next head's A is formed while this head's T' goes out) and the T of one.
// The diagonal tiles of T replace those of its head's A (each is read in full
// before it is overwritten); the off-diagonal tiles of T have their own slots.
struct PrepHead {
    float A[2][10][kTile];  // strict lower beta Gamma K K^T; diagonal tiles then hold T
    float To[6][kTile];     // off-diagonal tiles of T = (I + A)^-1
    __device__ float* T(int b, int it, int jt) { return it == jt ? A[b][tix(it, it)] : To[tix(it, jt) - it]; }
};

// LDS: the gates of the q/k head's `group` value heads ([group][2][64] fp32:
// l2_t, beta_t), then the K, Q chunk [token][d_k + 8] (f16), whose bytes the
// value-head working set takes over once the Gram tiles are formed.
template <int DK>
struct PrepLds {
    static constexpr int kLdK = DK + 8;
    static constexpr size_t kIn = 2 * (size_t)kC * kLdK * 2;
    static constexpr size_t kUnion = kIn > sizeof(PrepHead) ? kIn : sizeof(PrepHead);
    static size_t bytes(int group) { return (size_t)group * 2 * kC * 4 + kUnion; }
};

// Orders this wave's LDS accesses for the compiler where lanes exchange data
// through LDS (the hardware keeps one wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// A workgroup barrier for data exchanged through plain LDS stores: waits for
// this wave's LDS operations only, so its loads (the next chunk's operands)
// and its global stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The gates of token t0 + lane of value head hv (alpha = 1, beta = 0 past the
// sequence's end: no-op tokens).
struct Gate {
    float al, bt;
};
__device__ __forceinline__ Gate load_gate(const PrefillArgs& a, const SeqInfo& sq, int t0, int hv) {
    const int lane = threadIdx.x & 63;
    const bool in = t0 + lane < sq.T;
    const size_t gi = GDN_AT(((size_t)sq.tok0 + (in ? t0 + lane : sq.T - 1)) * a.h_v + hv, 1,
                             (size_t)a.tokens_total * a.h_v, a.status);
    Gate gt;
    gt.al = a.alpha[gi];
    gt.bt = a.beta[gi];
    if (!in) {
        gt.al = 1.f;
        gt.bt = 0.f;
    }
    return gt;
}

// One value head's gates on one wave (lane = token): l2_t by a prefix sum of
// the clamped log2 alpha; l2_t and beta_t to LDS, gamma_t, beta_t and
// Gamma_{C,t} to the workspace.
__device__ __forceinline__ void head_gates(const Gate gt, float* gl, float* gw) {
    const int lane = threadIdx.x & 63;
    float x = fmaxf(log2_fast(gt.al), kLogFloor * kLog2e);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    const float lC = __shfl(x, 63, 64);
    gl[lane] = x;
    gl[kC + lane] = gt.bt;
    gw[lane] = exp2_fast(x);
    gw[kC + lane] = gt.bt;
    gw[2 * kC + lane] = exp2_fast(lC - x);
}

// The (tile, block) pair of fragment f (0 .. 5) of a lower-triangular C x C
// operand, in the scan's order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
__device__ __forceinline__ constexpr int frag_tile(int f) { return f < 2 ? f : 2 + (f - 2) / 2; }
__device__ __forceinline__ constexpr int frag_blk(int f) { return f < 2 ? 0 : (f - 2) % 2; }

// Fragment f of T' = T diag(beta) (T of buffer b), f16, to the workspace.
// Lane (c, lg) writes row pair_row(tile, c), columns 32 blk + 8 lg .. + 8.
__device__ __forceinline__ void write_tprime(PrepHead& W, int b, const float* gl, _Float16* dst, int f) {
    const int lane = threadIdx.x & 63, c = lane & 15, lg = lane >> 4;
    const int tile = frag_tile(f), blk = frag_blk(f);
    const int t = pair_row(tile, c), i0 = 32 * blk + 8 * lg;
    const int it = t >> 4, jt = i0 >> 4;
    h8 v;
    if (jt <= it) {
        const float* row = W.T(b, it, jt) + (t & 15) * kTS + (i0 & 15);
        const f32x4 xa = *reinterpret_cast<const f32x4*>(row), xb = *reinterpret_cast<const f32x4*>(row + 4);
        float x[8];
        const f32x4 ba = *reinterpret_cast<const f32x4*>(gl + kC + i0);
        const f32x4 bb = *reinterpret_cast<const f32x4*>(gl + kC + i0 + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = i0 + e <= t ? (e < 4 ? xa[e] * ba[e] : xb[e - 4] * bb[e - 4]) : 0.f;
        v = to_h8(x);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)0.f;
    }
    *reinterpret_cast<h8*>(dst + (f * 64 + lane) * 8) = v;
}

// Column JB of T below the diagonal on one wave, top to bottom:
// T_ij = -T_ii Y_i with Y_i = A_iJ T_JJ + sum_{J<k<i} A_ik T_kJ.  The column's
// blocks stay in this wave's registers (accumulator layout: lane (c, lg) holds
// rows 4 lg + r, column c), so each one feeds the next as the products' B
// operand by contracting over k = 4 lg + s (lane (c, lg) supplies its own
// register s); the terms with T_JJ contract over k = 4 s + lg from LDS.  The
// columns need only the diagonal blocks, so they run side by side on three
// waves (v_mfma_f32_16x16x4_f32).
template <int JB>
__device__ __forceinline__ void offdiag_column(PrepHead& W, int b) {
    const int lane = threadIdx.x & 63, c = lane & 15, lg = lane >> 4;
    constexpr int N = 3 - JB;  // blocks below the diagonal
    const float* Tjj = W.T(b, JB, JB);
    f32x4 tcol[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const int ib = JB + 1 + n;
        const float* Aij = W.A[b][tix(ib, JB)];
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(Aij[c * kTS + 4 * s + lg], Tjj[(4 * s + lg) * kTS + c], y, 0, 0, 0);
#pragma unroll
        for (int m = 0; m < n; ++m) {
            const float* Aik = W.A[b][tix(ib, JB + 1 + m)];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(Aik[c * kTS + 4 * lg + s], tcol[m][s], y, 0, 0, 0);
        }
        const float* Ti = W.T(b, ib, ib);
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(Ti[c * kTS + 4 * lg + s], y[s], x, 0, 0, 0);
        tcol[n] = -x;
    }
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) W.T(b, JB + 1 + n, JB)[(4 * lg + r) * kTS + c] = tcol[n][r];
}

// Forward substitution of (I + A) x = e_jc for a strictly lower 16 x 16 block A,
// in column order: once x[m] is final, A[t][m] x[m] leaves every later x[t].
// Lane (bb, jc) holds column jc of its block's A (a[t] = A[t][jc]), so A[t][m] is
// lane m's a[t], broadcast to the 16 lanes of the block's DPP row (row_newbcast:m):
// one instruction per product, no LDS reads.
// x += bcast_M(a) n in one fused multiply-add (one rounding, as fmaf): the
// two-operand v_fmac_f32 takes a DPP source, the three-operand v_fma_f32 the
// compiler otherwise selects does not on gfx950 (it emitted a separate DPP move
// per product).  a is never written by a vector instruction here (LDS loads
// only), so the DPP read needs no wait states after its producer.
template <int M>
__device__ __forceinline__ float fmac_row_bcast(float x, float a, float n) {
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                 : "+v"(x)
                 : "v"(a), "v"(n), "n"(M));
    return x;
}
template <int M>
__device__ __forceinline__ void fwd_column(const float (&a)[16], float (&x)[16]) {
    if constexpr (M < 15) {
        const float nx = -x[M];
#pragma unroll
        for (int t = M + 1; t < 16; ++t) x[t] = fmac_row_bcast<M>(x[t], a[t], nx);
        fwd_column<M + 1>(a, x);
    }
}

template <int DK, bool BF16>
__global__ __launch_bounds__(256) void prefill_prepare_kernel(const PrefillArgs a, const PrefillSeqs seqs) {
    constexpr int kLdK = DK + 8;
    constexpr int KSD = DK / 32;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int g = blk % a.h_qk;
    const int u = blk / a.h_qk;  // chunk unit
    int b;
    if (a.varlen) {
        b = 0;
        while (seqs.unit0[b + 1] <= u) ++b;  // the sequence holding unit u (empty ones are skipped)
    } else {
        b = u / ((a.T + kC - 1) / kC);
    }
    const SeqInfo sq = seq_info(a, seqs, b);
    const int ck = u - sq.unit0;
    const int t0 = ck * kC;
    const WsLayout ws = ws_layout(a.units, a.h_qk, a.h_v, DK);
    unsigned char* wsb = static_cast<unsigned char*>(a.workspace);
    const size_t unit_q = (size_t)u * a.h_qk + g;
    const size_t unit_v0 = (size_t)u * a.h_v + (size_t)g * a.group;  // the first value head's unit block
    float* gates = reinterpret_cast<float*>(lds_raw);  // [group][2][64]
    unsigned char* un = lds_raw + (size_t)a.group * 2 * kC * 4;
    _Float16* Kf = reinterpret_cast<_Float16*>(un);
    _Float16* Qf = Kf + kC * kLdK;
    PrepHead& W = *reinterpret_cast<PrepHead*>(un);

    // the gates of this wave's first value head, loaded with K and Q
    const Gate gate0 = wave < a.group ? load_gate(a, sq, t0, g * a.group + wave) : Gate{1.f, 0.f};

    // 1. K, Q chunk -> LDS (f16).  All loads are issued first (token index
    //    clamped into the sequence), then converted and stored; rows past T are zero.
    {
        constexpr int NK = kC * DK / 8 / 256;  // 8-element chunks per thread
        Raw8 rk[NK], rq[NK];
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            const int e = tid + 256 * n;
            const int t = e / (DK / 8), d = 8 * (e % (DK / 8));
            const int tc = t0 + t < sq.T ? t0 + t : sq.T - 1;
            const size_t src = GDN_AT((((size_t)sq.tok0 + tc) * a.h_qk + g) * DK + d, 8,
                                      (size_t)a.tokens_total * a.h_qk * DK, a.status);
            raw_load<BF16>(rk[n], a.k, src);
            raw_load<BF16>(rq[n], a.q, src);
        }
        bool bad = false;
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            const int e = tid + 256 * n;
            const int t = e / (DK / 8), d = 8 * (e % (DK / 8));
            const bool valid = t0 + t < sq.T;
            *reinterpret_cast<h8*>(&Kf[t * kLdK + d]) = raw_to_h8<BF16>(rk[n], valid, bad);
            *reinterpret_cast<h8*>(&Qf[t * kLdK + d]) = raw_to_h8<BF16>(rq[n], valid, bad);
        }
        if (bad && a.status != nullptr) a.status[0] = GDN_ERR_RANGE;
    }
    // every value head's gates, one head per wave at a time
    for (int j = wave; j < a.group; j += 4) {
        float* gw = reinterpret_cast<float*>(wsb + ws.G) +
                    GDN_AT((unit_v0 + j) * 3 * kC, 3 * kC, (size_t)a.units * a.h_v * 3 * kC, a.status);
        head_gates(j == wave ? gate0 : load_gate(a, sq, t0, g * a.group + j), gates + j * 2 * kC, gw);
    }
    __syncthreads();

    // 2. On the matrix cores (registers of the wave that forms them): K K^T's lower tiles
    //    (wave 0 tiles 0-3, wave w > 0 tiles 2 + 2 w and 3 + 2 w) and, on waves 1-3, the
    //    (Q K^T)^T tiles of P's fragments 2 (w - 1) and 2 (w - 1) + 1: tiles (2 v, p) and
    //    (2 v + 1, p) of fragment (p, v), keys in rows pair_row(2 v + h, .), queries in
    //    columns pair_row(p, .).  K and Q -> workspace in fragment order.
    const int nkk = wave == 0 ? 4 : 2;          // K K^T tiles of this wave (uniform)
    const int kk0 = wave == 0 ? 0 : 2 + 2 * wave;
    f32x4 kk[4], pq[2][2];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        if (jj < nkk) {
            const int tx = kk0 + jj;
            const int it = tile_row(tx), jt = tx - it * (it + 1) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks)
                acc = mfma16(frag(Kf, kLdK, 16 * it, 32 * ks, lane), frag(Kf, kLdK, 16 * jt, 32 * ks, lane), acc);
            kk[jj] = acc;
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int sf = 0; sf < 2; ++sf) {
            const int f = 2 * (wave - 1) + sf, p = frag_tile(f), v = frag_blk(f);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const _Float16* kr = Kf + pair_row(2 * v + h, c) * kLdK + 8 * lg;
                const _Float16* qr = Qf + pair_row(p, c) * kLdK + 8 * lg;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    acc = mfma16(*reinterpret_cast<const h8*>(kr + 32 * ks), *reinterpret_cast<const h8*>(qr + 32 * ks),
                                 acc);
                pq[sf][h] = acc;
            }
        }
    }
    {
        _Float16* kw = reinterpret_cast<_Float16*>(wsb + ws.K) + unit_q * kC * DK;
        _Float16* qw = reinterpret_cast<_Float16*>(wsb + ws.Q) + unit_q * kC * DK;
        constexpr int PIECES = DK * kC / 8;
        for (int e = tid; e < 2 * PIECES; e += 256) {
            const int m = e / PIECES, i = e % PIECES;
            const int f = i / 64, l = i % 64, cc = l & 15, gg = l >> 4;
            const int row = pair_row(f / KSD, cc), col = 32 * (f % KSD) + 8 * gg;
            const h8 v = *reinterpret_cast<const h8*>(&(m == 0 ? Kf : Qf)[row * kLdK + col]);
            *reinterpret_cast<h8*>((m == 0 ? kw : qw) + 8 * i) = v;
        }
    }
    __syncthreads();  // K, Q are dead: the working set takes their bytes

    // This wave's K K^T tiles -> the A tiles of value head j in buffer b: strictly lower (i < t),
    // carrying beta_t.  Selects, not branches: i and t vary over the wave.
    auto form_a = [&](int j, int b) {
        const float* gl = gates + j * 2 * kC;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (jj < nkk) {
                const int tx = kk0 + jj;
                const int it = tile_row(tx), jt = tx - it * (it + 1) / 2;
                const f32x4 lt = *reinterpret_cast<const f32x4*>(gl + 16 * it + 4 * lg);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(gl + kC + 16 * it + 4 * lg);
                const float li = gl[16 * jt + c];
                const int i = 16 * jt + c;
                float* dst = W.A[b][tx];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * it + 4 * lg + r;
                    const float e2 = exp2_fast(lt[r] - li);
                    dst[(4 * lg + r) * kTS + c] = i < t ? bt[r] * e2 * kk[jj][r] : 0.f;
                }
            }
        }
    };
    // Waves 1-3: P's fragments 2 (w - 1) and 2 (w - 1) + 1 of value head j, straight from the
    // (Q K^T)^T registers: lane (c, lg) holds queries t = pair_row(p, c) and keys
    // i = pair_row(2 v + h, 4 lg + r) = 32 v + 8 lg + 4 h + r.
    auto write_p = [&](int j, _Float16* Pw) {
        const float* gl = gates + j * 2 * kC;
#pragma unroll
        for (int sf = 0; sf < 2; ++sf) {
            const int f = 2 * (wave - 1) + sf, p = frag_tile(f), v = frag_blk(f);
            const int t = pair_row(p, c);
            const float lt = gl[t];
            f32x4 x[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i0 = 32 * v + 8 * lg + 4 * h;
                const f32x4 li = *reinterpret_cast<const f32x4*>(gl + i0);
#pragma unroll
                for (int r = 0; r < 4; ++r) x[h][r] = i0 + r <= t ? exp2_fast(lt - li[r]) * pq[sf][h][r] : 0.f;
            }
            *reinterpret_cast<h8*>(Pw + (f * 64 + lane) * 8) = pack_h8(x[0], x[1]);
        }
    };

    // 3. the value heads one after another, all four waves on each; head j's A in buffer j % 2
    form_a(0, 0);
    __syncthreads();
    for (int j = 0; j < a.group; ++j) {
        const int b = j & 1;
        const float* gl = gates + j * 2 * kC;  // l2_t [64], beta_t [64]
        const size_t unit_v = unit_v0 + j;
        if (wave == 0) {
            // diagonal 16 x 16 blocks of T by forward substitution, one column of one block
            // per lane: lane (bb, jc) reads column jc of A_bb once, then solves for column jc
            // of T_bb (see fwd_column)
            const int bb = lane >> 4, jc = lane & 15;
            const float* Ab = W.A[b][tix(bb, bb)];
            float av[16], x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                av[t] = Ab[t * kTS + jc];
                x[t] = t == jc ? 1.f : 0.f;
            }
            fwd_column<0>(av, x);
#pragma unroll
            for (int t = 0; t < 16; ++t) W.T(b, bb, bb)[t * kTS + jc] = x[t];  // after all reads of A_bb
        } else {
            // meanwhile P's fragments (two per wave)
            write_p(j, reinterpret_cast<_Float16*>(wsb + ws.P) + unit_v * kC * kC);
        }
        __syncthreads();
        // the off-diagonal blocks, one column per wave
        if (wave == 0) offdiag_column<0>(W, b);
        else if (wave == 1) offdiag_column<1>(W, b);
        else if (wave == 2) offdiag_column<2>(W, b);
        __syncthreads();
        // T' = T diag(beta) fragments, and the next value head's A in the other buffer
        _Float16* Tw = reinterpret_cast<_Float16*>(wsb + ws.T) + unit_v * kC * kC;
        write_tprime(W, b, gl, Tw, wave);
        if (wave < 2) write_tprime(W, b, gl, Tw, wave + 4);
        if (j + 1 < a.group) form_a(j + 1, b ^ 1);
        __syncthreads();  // the next value head overwrites T's tiles
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, value head, 16 NSL value columns)
// ---------------------------------------------------------------------------
// Value columns never mix in the recurrence (R, U, O and the state update act
// on each column of H separately), so a pair of waves owns 16 columns of one
// head for the whole prompt.  The state slice H[:, j0 .. j0+16) stays in
// accumulators, and every product's result feeds the next product from the
// lane that produced it, because 16-row tiles are paired into 32-wide
// contraction blocks with a matching row order:
//   the accumulator of a 16 x 16 x 32 product gives lane (c, g) = (lane % 16,
//   lane / 16) rows 4g .. 4g+3; the B operand wants rows 8g .. 8g+7 of a
//   32-row block.  Tile pair (2u, 2u+1) therefore covers rows
//   32u + 8g + 4h + r of the block (h = tile & 1, r = 0..3), and the A operand
//   of the producing product reads its row c from pair_row(tile, c).
// So K H and Q H take the state as B straight from the accumulators, U = T' R
// takes R = V - gamma K H, and O and the state update take U, all without
// moving data between lanes.
//
// All slices of a workgroup read the same A operands of their head.  The
// chain waves' (K, T', with V and the gates) come into LDS once per workgroup:
// buffer loads that write LDS directly (no registers), split between the
// output waves, two chunks ahead into one of three LDS blocks.  The LDS copy
// is in fragment order -- fragment f, lane l at f * 1 KB + 16 l -- so an
// operand read is one conflict-free 16-byte LDS read (K^T: two transposing
// reads of the K fragments).  The output waves' Q and P go straight into
// their registers one chunk ahead.  Two barriers per chunk: at the top, after
// each output wave's wait for its loads of the chunk (publishing the chunk,
// and telling every wave that the block of the chunk before is free), and in
// the middle, where the chain waves hand U to the output waves.

// Buffer resources: a uniform base per matrix and chunk, bounded by its size,
// so a load past it returns zero and a store past it is dropped (the rows of a
// ragged last chunk past T).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// One chunk's block in LDS, the chain waves' operands.  Fragments (1 KB each):
// K [p][u], then T' over the six lower-triangular (p, v <= p / 2) pairs
// (rounded up to a multiple of NSL fragments); then V rows [64][the
// workgroup's 16 NSL columns] in the input dtype, then gamma_t and
// Gamma_{C,t}.  K^T is not stored: the chain wave reads it from the K
// fragments with transposing LDS reads.  Q and P, which only the output
// waves read, go to their registers instead (OutOps).
template <int DK, bool BF16, int NSL>
struct ChunkBlock {
    static constexpr int NT = DK / 16, KB = DK / 32, NP = kC / 16, VB = kC / 32;
    static constexpr int NTRI = (6 + NSL - 1) / NSL * NSL;
    static constexpr int K0 = 0, T0 = K0 + NP * KB;
    static constexpr int NFRAG = T0 + NTRI;
    static constexpr int COLS = 16 * NSL;              // value columns of the workgroup
    static constexpr int VROW = COLS * (BF16 ? 2 : 4);  // bytes of one V row
    static constexpr int NVI = kC * VROW / 1024;       // V loads
    static constexpr int V0 = NFRAG * 1024;
    static constexpr int G0 = V0 + kC * VROW;          // gamma [64], Gamma_C [64] (fp32)
    static constexpr int BYTES = G0 + 2 * kC * 4;
    // load instructions per chunk, NSL per slot (one per output wave): every
    // boundary between matrices falls on a slot boundary
    static constexpr int NLOAD = NFRAG + NVI + NSL;
    static_assert(T0 % NSL == 0 && NFRAG % NSL == 0 && NVI % NSL == 0, "slot boundaries");
};
__device__ __forceinline__ constexpr int tri(int p, int v) { return p < 2 ? p : 2 * p - 2 + v; }

template <int DK>
struct ScanCtx {
    const PrefillArgs* a;
    const unsigned char* wsb;
    WsLayout ws;
    int b, h, g, nch, col0, cols;  // the workgroup's first value column and column count
    int tok0, T, unit0;            // the sequence's first token, tokens and first chunk unit
    __device__ int clamp_ck(int ck) const { return ck < nch ? ck : nch - 1; }
    // the chunk's block of a per-value-head array (per_unit bytes per head and chunk)
    __device__ rsrc_t ws_v(size_t arr, uint32_t per_unit, int ck) const {
        return make_rsrc(wsb + arr + ((size_t)unit0 * a->h_v + h) * per_unit +
                             (size_t)(uint32_t)clamp_ck(ck) * (uint32_t)(a->h_v * per_unit),
                         per_unit);
    }
    __device__ rsrc_t ws_q(size_t arr, uint32_t per_unit, int ck) const {
        return make_rsrc(wsb + arr + ((size_t)unit0 * a->h_qk + g) * per_unit +
                             (size_t)(uint32_t)clamp_ck(ck) * (uint32_t)(a->h_qk * per_unit),
                         per_unit);
    }
    // the workgroup's columns of the rows of chunk ck of a [B][T][h_v][d_v]
    // tensor, bounded at the sequence's last token
    __device__ rsrc_t rows(const void* base, int esz, int ck) const {
        const int t0 = clamp_ck(ck) * kC;
        const int n = T - t0 < kC ? T - t0 : kC;
        const size_t row = (size_t)a->h_v * a->d_v;
        return make_rsrc(static_cast<const unsigned char*>(base) +
                             (((size_t)tok0 + t0) * row + (size_t)h * a->d_v + col0) * esz,
                         (uint32_t)(((size_t)(n - 1) * row + cols) * esz));
    }
};

// Loads of one chunk into an LDS block.  ChunkBlock's load instructions are
// split between the NSL output waves: output wave sl issues instruction
// i = NSL k + sl for slot k.  Every matrix boundary is a slot boundary, so all
// instructions of a slot read the same matrix and the slot's code is the same
// for every wave; the wave enters only through per-lane offsets and a uniform
// LDS base.
struct DmaCtx {
    rsrc_t kw, tw, gw, vw;
    uint32_t vf, vv, vg;  // per-lane source offsets of fragment, V and gate loads (this wave's)
    uint32_t vstep;       // source bytes between this wave's consecutive V loads
    unsigned char* dst;   // LDS block + 1 KB sl
    unsigned char* gdst;  // LDS gate area: gamma (even sl) or Gamma_C (odd sl)
};

template <int DK, bool BF16, int NSL>
__device__ __forceinline__ DmaCtx dma_ctx(const ScanCtx<DK>& X, int ck, unsigned char* blk, int sl) {
    using CB = ChunkBlock<DK, BF16, NSL>;
    const PrefillArgs& a = *X.a;
    constexpr int VSZ = BF16 ? 2 : 4;
    constexpr int RPL = 1024 / CB::VROW;  // V rows per load
    const int lane = threadIdx.x & 63;
    const uint32_t rowb = (uint32_t)(a.h_v * a.d_v * VSZ);
    DmaCtx d;
    d.kw = X.ws_q(X.ws.K, kC * DK * 2, ck);
    d.tw = X.ws_v(X.ws.T, kC * kC * 2, ck);
    d.gw = X.ws_v(X.ws.G, 3 * kC * 4, ck);
    d.vw = X.rows(a.v, VSZ, ck);
    // fragments are stored in load order: lane l of fragment f at f KB + 16 l
    d.vf = 16 * lane + 1024 * sl;
    // V load n, lane l: row n RPL + 16 l / VROW, byte (16 l) % VROW of the workgroup's columns
    d.vv = (uint32_t)((16 * lane / CB::VROW + RPL * sl) * rowb + (16 * lane) % CB::VROW);
    d.vstep = NSL * RPL * rowb;
    // gamma (even sl) and Gamma_C (odd sl), 64 fp32 each (with four waves, twice over)
    d.vg = 4 * lane + 2 * kC * 4 * (sl & 1);
    d.dst = blk + 1024 * sl;
    d.gdst = blk + CB::G0 + kC * 4 * (sl & 1);
    return d;
}

template <int DK, bool BF16, int NSL, int K>
__device__ __forceinline__ void dma_slot(const DmaCtx& d) {
    using CB = ChunkBlock<DK, BF16, NSL>;
    constexpr int i0 = NSL * K;  // this slot's first instruction
    if constexpr (i0 < CB::NFRAG) {
        constexpr int base = i0 < CB::T0 ? CB::K0 : CB::T0;
        const rsrc_t r = i0 < CB::T0 ? d.kw : d.tw;
        if constexpr (NSL * 1024 < 4096) {
            // slots pair up inside a matrix and share one LDS base: the instruction offset
            // (the second of a pair) moves the source and the LDS address alike
            constexpr int pb = base + 2 * NSL * ((i0 - base) / (2 * NSL));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(d.dst + 1024 * pb), 16, d.vf,
                                                     1024 * (pb - base), 1024 * (i0 - pb), 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(d.dst + 1024 * i0), 16, d.vf, 1024 * (i0 - base),
                                                     0, 0);
        }
    } else if constexpr (i0 < CB::NFRAG + CB::NVI) {
        constexpr int n0 = (i0 - CB::NFRAG) / NSL;  // this wave's V load index
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.vw, (lds_void*)(d.dst + 1024 * i0), 16, d.vv, n0 * d.vstep, 0, 0);
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.gw, (lds_void*)d.gdst, 4, d.vg, 0, 0, 0);
    }
}

template <int DK, bool BF16, int NSL, int K, int KEND>
__device__ __forceinline__ void dma_slots(const DmaCtx& d) {
    if constexpr (K < KEND) {
        dma_slot<DK, BF16, NSL, K>(d);
        dma_slots<DK, BF16, NSL, K + 1, KEND>(d);
    }
}

__device__ __forceinline__ h8 frag_at(const unsigned char* blk, int f) {
    return *reinterpret_cast<const h8*>(blk + f * 1024 + 16 * (threadIdx.x & 63));
}

// The state update's A operand K^T (tile t over d_k, block v over tokens),
// read from the K fragments with two transposing reads.  ds_read_b64_tr_b16
// gives lane c of a 16-lane group element e = value c % 4 of the 8 bytes that
// lane 4 e + c / 4 of the group addressed.  Lane 4 e + q of group g therefore
// addresses K[token 32 v + 8 g + 4 h + e][d_k 32 (t / 2) + 8 q + 4 (t % 2) ..+4]
// for half h, and lane (c, g) receives K^T[pair_row(t, c)][32 v + 8 g + 4 h + e].
template <int DK>
__device__ __forceinline__ h8 kt_frag(const unsigned char* blk, int t, int v) {
    typedef short s4v __attribute__((ext_vector_type(4)));
    typedef _Float16 h4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4v lds_s4;
    constexpr int KB = DK / 32;
    const int lane = threadIdx.x & 63, g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    h8 r;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const unsigned char* p =
            blk + ((2 * v + hh) * KB + (t >> 1)) * 1024 + (16 * q + 4 * g + e) * 16 + 8 * (t & 1);
        const h4v x = __builtin_bit_cast(h4v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p));
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * hh + j] = x[j];
    }
    return r;
}

// Output rows staged in LDS per slice (both output waves stage their halves):
// row t at t * RB + (t / 8) * 32 (the skew keeps the four rows one store
// instruction touches on different banks).
template <int OUT>
struct OStage {
    static constexpr int ESZ = OUT == 0 ? 4 : 2;
    static constexpr int RB = 16 * ESZ;
    static constexpr int BYTES = kC * RB + (kC / 8) * 32;
    __device__ static int at(int t) { return t * RB + (t >> 3) * 32; }
};

// The staged outputs of chunk ck -> HBM, 16-byte stores of whole row pieces.
template <int DK, int OUT>
__device__ __forceinline__ void write_out(const ScanCtx<DK>& X, const unsigned char* ost, int ck, int sl) {
    using OS = OStage<OUT>;
    const PrefillArgs& a = *X.a;
    const int lane = threadIdx.x & 63;
    const rsrc_t ow = X.rows(a.out, OS::ESZ, ck);
    const uint32_t rstride = (uint32_t)(a.h_v * a.d_v * OS::ESZ);
    constexpr int PER_ROW = OS::RB / 16;  // 16-byte pieces per row
#pragma unroll
    for (int n = 0; n < PER_ROW; ++n) {
        const int t = lane;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ost + OS::at(t) + 16 * n);
        __builtin_amdgcn_raw_buffer_store_b128(v, ow, t * rstride + (16 * sl) * OS::ESZ + 16 * n, 0, 0);
    }
}

template <int OUT>
__device__ __forceinline__ void stage_o(unsigned char* ost, int t, int c, float o) {
    unsigned char* p = ost + OStage<OUT>::at(t) + c * OStage<OUT>::ESZ;
    if constexpr (OUT == 0) *reinterpret_cast<float*>(p) = o;
    else if constexpr (OUT == 2) *reinterpret_cast<_Float16*>(p) = (_Float16)o;
    else *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(o);
}

// The products of one chunk, split so that each wave runs on its own SIMD:
//   chain wave (one per 16-column slice):
//                K H (u-major) | R = V - gamma K H | U = T' R | U -> LDS |
//                barrier | state update (v-major) | next state -> LDS
//   output wave (one per 32-row half of the chunk, both slices):
//                Q H (the states from LDS) | barrier | U <- LDS | O += P U |
//                outputs staged; it also issues the loads of the chunk after next.
// Each wave's steps are one static sequence (the chain wave's A operands read
// from LDS D steps ahead, the output wave's from its registers); the order is
// pinned with scheduling barriers.
template <int DK>
struct Plan {
    static constexpr int NT = DK / 16, KB = DK / 32, NP = kC / 16, VB = kC / 32;
    static constexpr int NKH = NP * KB, NU = 6, NST = NT * VB, NQ = NP * KB, NPU = 6;
    // chain wave
    static constexpr int A_U = NKH, A_ST = A_U + NU, A_END = A_ST + NST;
    // output wave
    static constexpr int B_PU = NQ, B_END = B_PU + NPU;
    static constexpr int D = 6;        // operand reads in flight ahead of the MFMAs
    static constexpr int NEXTRA = 25;  // chain wave: V (16), gamma (4), Gamma_C (4), gamma_C (1)
};
// the (tile, block) pairs of U = T' R and O += P U, block-major
__device__ __forceinline__ constexpr int tri_p(int k) { return k < 4 ? k : k - 2; }
__device__ __forceinline__ constexpr int tri_v(int k) { return k < 4 ? 0 : 1; }

// chain wave: the A operand of step s
template <int DK, int S>
__device__ __forceinline__ h8 chain_operand(const unsigned char* blk) {
    using PL = Plan<DK>;
    using CB = ChunkBlock<DK, true, 2>;  // fragment indices depend on neither the V dtype nor NSL
    if constexpr (S < PL::A_U) return frag_at(blk, CB::K0 + (S % PL::NP) * PL::KB + S / PL::NP);
    else if constexpr (S < PL::A_ST) return frag_at(blk, CB::T0 + tri(tri_p(S - PL::A_U), tri_v(S - PL::A_U)));
    else return kt_frag<DK>(blk, (S - PL::A_ST) % PL::NT, (S - PL::A_ST) / PL::NT);
}
// The output wave's A operands of one chunk -- Q's fragments in product order,
// then P's six -- in registers.  Only the output wave reads them, so they come
// from the workspace straight into its registers, one chunk ahead, instead of
// through LDS: each register takes the next chunk's fragment right after the
// product that reads it has been issued.
// The two output waves of a workgroup split the chunk by rows: wave H owns
// output rows 32 H .. 32 H + 31 (row tiles 2 H and 2 H + 1) of both slices, so
// each Q and P fragment is loaded by one wave only and serves both slices'
// products.  Steps j < NQ: Q H with tile 2 H + j % 2 and state block j / 2;
// then P U over the (tile, U block) pairs of the half's tiles.
template <int DK, int H>
struct OutPlan {
    static constexpr int KB = DK / 32;
    static constexpr int NQ = 2 * KB, NPU = H == 0 ? 2 : 4;
    static constexpr int B_PU = NQ, B_END = NQ + NPU;
    static constexpr int NUB = H == 0 ? 1 : 2;  // U blocks the half's products read
    __device__ static constexpr int pu_p(int k) { return H == 0 ? k : 2 + k % 2; }
    __device__ static constexpr int pu_v(int k) { return H == 0 ? 0 : k / 2; }
};
template <int DK, int H>
struct OutOps {
    h8 f[OutPlan<DK, H>::B_END];
};
struct OutSrc {
    rsrc_t q, p;  // the chunk's Q (per q/k head) and P (per value head) in the workspace
};
template <int DK>
__device__ __forceinline__ OutSrc out_src(const ScanCtx<DK>& X, int ck) {
    return {X.ws_q(X.ws.Q, kC * DK * 2, ck), X.ws_v(X.ws.P, kC * kC * 2, ck)};
}
template <int DK, int H, int S>
__device__ __forceinline__ h8 load_out_op(const OutSrc& r) {
    using OP = OutPlan<DK, H>;
    const int lo = 16 * (threadIdx.x & 63);
    u32x4 w;
    if constexpr (S < OP::B_PU)
        w = __builtin_amdgcn_raw_buffer_load_b128(r.q, lo + 1024 * ((2 * H + S % 2) * OP::KB + S / 2), 0, 0);
    else
        w = __builtin_amdgcn_raw_buffer_load_b128(r.p, lo + 1024 * tri(OP::pu_p(S - OP::B_PU), OP::pu_v(S - OP::B_PU)),
                                                  0, 0);
    return __builtin_bit_cast(h8, w);
}
template <int DK, int H, int S>
__device__ __forceinline__ void load_out_ops(OutOps<DK, H>& ops, const OutSrc& r) {
    if constexpr (S < OutPlan<DK, H>::B_END) {
        ops.f[S] = load_out_op<DK, H, S>(r);
        load_out_ops<DK, H, S + 1>(ops, r);
    }
}

// The state (f16, as the products' B operand) and U (f16) handed from the
// chain wave to the output waves of a slice, in operand order: 16 bytes per
// lane per operand.  LAG (output waves one chunk behind the chain): three
// copies of the state (the copy a chunk starts from is written at the end of
// the chunk before and read during the chunk after) and two of U (written
// during its chunk, read during the next), so no copy is written while it may
// be read; without LAG one of each, ordered by the middle barrier.
template <int DK, bool LAG>
struct Xchg {
    static constexpr int KB = DK / 32, VB = kC / 32;
    static constexpr int NSB = LAG ? 3 : 1, NUB = LAG ? 2 : 1;
    static constexpr int SBB = KB * 1024, UBB = VB * 1024;  // bytes of one copy
    static constexpr int UB0 = NSB * SBB, BYTES = UB0 + NUB * UBB;
    __device__ static int sb(int ck) { return (LAG ? ck % 3 : 0) * SBB; }  // the state chunk ck starts from
    __device__ static int ub(int ck) { return UB0 + (LAG ? ck % 2 : 0) * UBB; }  // chunk ck's U
};
__device__ __forceinline__ void put_h8(unsigned char* base, int i, const h8& v) {
    *reinterpret_cast<h8*>(base + i * 1024 + 16 * (threadIdx.x & 63)) = v;
}
__device__ __forceinline__ h8 get_h8(const unsigned char* base, int i) {
    return *reinterpret_cast<const h8*>(base + i * 1024 + 16 * (threadIdx.x & 63));
}

template <int DK>
struct ChainRegs {
    using PL = Plan<DK>;
    h8 (&sb)[PL::KB];  // the chunk's starting state (f16), replaced by the next chunk's at the end
    f32x4 kh[PL::NP], uu[PL::NP];
    h8 rb[PL::VB], ug[PL::VB];
    h8 fa[PL::A_END];
    float vx[PL::NP][4];  // V at this lane's rows (fp32 V)
    u32x2 vr[PL::NP];     // the same, two bf16 per word (bf16 V)
    f32x4 gp[PL::NP], gq[PL::NP];
    float gC;
};

// The chain wave's reads besides its A operands, in issue order: gamma_C first
// (the state decays during K H), then V, gamma and Gamma_C at this lane's rows.
template <int DK, bool BF16, int NSL, int EI>
__device__ __forceinline__ void extra_read(ChainRegs<DK>& x, const unsigned char* blk, int sl) {
    using CB = ChunkBlock<DK, BF16, NSL>;
    constexpr int E = EI == 0 ? 24 : EI - 1;
    const int lane = threadIdx.x & 63, c = lane & 15, lg = lane >> 4;
    const float* gam = reinterpret_cast<const float*>(blk + CB::G0);
    if constexpr (E < 16) {
        constexpr int p = E / 4, r = E % 4;
        if constexpr (BF16) {
            // one transposing read per row block: lane 4 e + q of the group addresses row
            // pair_row(p, 4 lg) + e, columns 4 q .. 4 q + 3 of the slice, so lane c receives
            // its column c of the block's four rows
            if constexpr (r == 0) {
                typedef short s4v __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) s4v lds_s4;
                const int e = (lane >> 2) & 3, q = lane & 3;
                const unsigned char* vp = blk + CB::V0 + (pair_row(p, 4 * lg) + e) * CB::VROW + (16 * sl + 4 * q) * 2;
                // kept raw: widened where R is formed, so no wait for the read here
                x.vr[p] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)vp));
            }
        } else {
            const unsigned char* vp = blk + CB::V0 + (pair_row(p, 4 * lg) + r) * CB::VROW + (16 * sl + c) * 4;
            x.vx[p][r] = *reinterpret_cast<const float*>(vp);
        }
    } else if constexpr (E < 20) {
        x.gp[E - 16] = *reinterpret_cast<const f32x4*>(gam + pair_row(E - 16, 4 * lg));
    } else if constexpr (E < 24) {
        x.gq[E - 20] = *reinterpret_cast<const f32x4*>(gam + kC + pair_row(E - 20, 4 * lg));
    } else {
        x.gC = gam[kC - 1];
    }
}
template <int DK, bool BF16, int NSL, int E, int EEND>
__device__ __forceinline__ void extra_reads(ChainRegs<DK>& x, const unsigned char* blk, int sl) {
    if constexpr (E < EEND) {
        extra_read<DK, BF16, NSL, E>(x, blk, sl);
        extra_reads<DK, BF16, NSL, E + 1, EEND>(x, blk, sl);
    }
}

template <int DK, bool BF16, int NSL, bool LAG, int S>
__device__ __forceinline__ void chain_step(ChainRegs<DK>& x, f32x4 (&st)[DK / 16], const unsigned char* blk,
                                           unsigned char* xu, unsigned char* xs, int sl) {
    using PL = Plan<DK>;
    constexpr int NP = PL::NP, NT = PL::NT, VB = PL::VB, KB = PL::KB;
    if constexpr (S < PL::A_END) {
        if constexpr (S + PL::D < PL::A_END) x.fa[S + PL::D] = chain_operand<DK, S + PL::D>(blk);
        if constexpr (S < PL::NKH)
            extra_reads<DK, BF16, NSL, S * PL::NEXTRA / PL::NKH, (S + 1) * PL::NEXTRA / PL::NKH>(x, blk, sl);
        // the state decays by gamma_C, one tile per step while K H runs (its products read
        // the f16 copy), so the multiplies issue under the products instead of before the update
        static_assert(2 + NT <= PL::A_ST, "decay steps end before the update");
        if constexpr (S >= 2 && S - 2 < NT) st[S - 2] = x.gC * st[S - 2];
        if constexpr (BF16 && S == PL::NKH - 1) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                x.vx[p][0] = bf16_lo(x.vr[p][0]);
                x.vx[p][1] = bf16_hi(x.vr[p][0]);
                x.vx[p][2] = bf16_lo(x.vr[p][1]);
                x.vx[p][3] = bf16_hi(x.vr[p][1]);
            }
        }
        if constexpr (S == PL::A_U) {
            // R = V - gamma K H at this lane's rows pair_row(p, 4 lg) + r
#pragma unroll
            for (int v = 0; v < VB; ++v)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int p = 2 * v + hh;
                        x.rb[v][4 * hh + r] = (_Float16)fmaf(-x.gp[p][r], x.kh[p][r], x.vx[p][r]);
                    }
        }
        if constexpr (S == PL::A_ST) {
            // U in f16 to the output waves; U scaled by Gamma_{C,t} here
#pragma unroll
            for (int v = 0; v < VB; ++v) {
                put_h8(xu, v, pack_h8(x.uu[2 * v], x.uu[2 * v + 1]));
                x.ug[v] = pack_h8(x.gq[2 * v] * x.uu[2 * v], x.gq[2 * v + 1] * x.uu[2 * v + 1]);
            }
            // U published (the output waves wait here for it); LAG: they read it a chunk later
            if constexpr (!LAG) lds_barrier();
        }
        if constexpr (S < PL::A_U) {
            constexpr int p = S % NP, u = S / NP;
            x.kh[p] = mfma16(x.fa[S], x.sb[u], x.kh[p]);
        } else if constexpr (S < PL::A_ST) {
            constexpr int p = tri_p(S - PL::A_U), v = tri_v(S - PL::A_U);
            x.uu[p] = mfma16(x.fa[S], x.rb[v], x.uu[p]);
        } else {
            constexpr int t = (S - PL::A_ST) % NT, v = (S - PL::A_ST) / NT;
            st[t] = mfma16(x.fa[S], x.ug[v], st[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
        chain_step<DK, BF16, NSL, LAG, S + 1>(x, st, blk, xu, xs, sl);
    } else {
        if constexpr (LAG) {
            // U of this chunk has landed before the state copy goes out: the output waves read U
            // after the next barrier, which this wave passes without waiting for its LDS writes
            // (with few update products no operand read of this chunk follows the U writes)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            asm volatile("" ::: "memory");
        }
        // the next chunk's starting state as the products' B operand, kept for this wave's
        // next K H and handed to the output waves
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            x.sb[u] = pack_h8(st[2 * u], st[2 * u + 1]);
            put_h8(xs, u, x.sb[u]);
        }
    }
}

template <int DK, int NSL>
struct OutRegs {
    h8 sb[NSL][DK / 32], ub[NSL][kC / 32];
    f32x4 o[NSL][2];
    f32x4 gp[2];
};

// The output wave's view of the chunk it computes: slice s's starting state at
// sb + s * XC, its U at ub + s * XC and its output staging at ost + s * OST.
struct OutPlaces {
    const unsigned char* sb;
    const unsigned char* ub;
    unsigned char* ost;
};

template <int DK, int OUT, bool BF16, int NSL, int NB>
struct ScanLayout;

template <int DK, int OUT, bool BF16, int NSL, int NB, int H, int S>
__device__ __forceinline__ void out_step(OutRegs<DK, NSL>& x, OutOps<DK, H>& ops, const OutSrc& nsrc,
                                         const unsigned char* blk, const OutPlaces& pl, float scale, const DmaCtx& d) {
    using OP = OutPlan<DK, H>;
    using CB = ChunkBlock<DK, BF16, NSL>;
    using L = ScanLayout<DK, OUT, BF16, NSL, NB>;
    constexpr int NSLOT = CB::NLOAD / NSL;
    if constexpr (S < OP::B_END) {
        if constexpr (S == OP::B_PU) {
            const int lg = (threadIdx.x & 63) >> 4;
            const float* gam = reinterpret_cast<const float*>(blk + CB::G0);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                // LAG: the gate rows came with the chunk, a chunk ago (x.gp)
                if constexpr (!L::LAG) x.gp[i] = *reinterpret_cast<const f32x4*>(gam + pair_row(2 * H + i, 4 * lg));
#pragma unroll
                for (int q = 0; q < NSL; ++q) x.o[q][i] = x.gp[i] * x.o[q][i];  // gamma Q H
            }
            // U from the chain waves (the next chunk's loads stay in flight); LAG: published
            // by the chunk's barrier
            if constexpr (!L::LAG) lds_barrier();
#pragma unroll
            for (int q = 0; q < NSL; ++q)
#pragma unroll
                for (int v = 0; v < OP::NUB; ++v) x.ub[q][v] = get_h8(pl.ub + q * L::XC, v);
        }
        // one operand, the products of every slice
        if constexpr (S < OP::B_PU) {
            constexpr int i = S % 2, u = S / 2;
#pragma unroll
            for (int q = 0; q < NSL; ++q) x.o[q][i] = mfma16(ops.f[S], x.sb[q][u], x.o[q][i]);
        } else {
            constexpr int i = OP::pu_p(S - OP::B_PU) - 2 * H, v = OP::pu_v(S - OP::B_PU);
#pragma unroll
            for (int q = 0; q < NSL; ++q) x.o[q][i] = mfma16(ops.f[S], x.ub[q][v], x.o[q][i]);
        }
        ops.f[S] = load_out_op<DK, H, S>(nsrc);  // the next chunk's operand
        __builtin_amdgcn_sched_barrier(0);
        out_step<DK, OUT, BF16, NSL, NB, H, S + 1>(x, ops, nsrc, blk, pl, scale, d);
    } else {
        // O -> staging (written out at the start of the next pass)
        const int lane = threadIdx.x & 63, c = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int q = 0; q < NSL; ++q)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    stage_o<OUT>(pl.ost + q * L::OST, pair_row(2 * H + i, 4 * lg) + r, c, scale * x.o[q][i][r]);
        // with three blocks, the loads of the chunk after next into LDS, after this chunk's
        // register loads, so that the next chunk's in-order wait for those leaves these in flight
        if constexpr (NB == 3) dma_slots<DK, BF16, NSL, 0, NSLOT>(d);
    }
}

// One chunk of a chain wave: U goes to xu, the next chunk's starting state to xs.
template <int DK, bool BF16, int NSL, bool LAG>
__device__ __forceinline__ void chain_chunk(f32x4 (&st)[DK / 16], h8 (&sb)[DK / 32], const unsigned char* blk,
                                            unsigned char* xu, unsigned char* xs, int sl) {
    using PL = Plan<DK>;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    ChainRegs<DK> x{sb};
#pragma unroll
    for (int p = 0; p < PL::NP; ++p) x.kh[p] = x.uu[p] = z;
    x.fa[0] = chain_operand<DK, 0>(blk);
    x.fa[1] = chain_operand<DK, 1>(blk);
    x.fa[2] = chain_operand<DK, 2>(blk);
    x.fa[3] = chain_operand<DK, 3>(blk);
    x.fa[4] = chain_operand<DK, 4>(blk);
    x.fa[5] = chain_operand<DK, 5>(blk);
    static_assert(Plan<DK>::D == 6, "prologue reads D operands");
    chain_step<DK, BF16, NSL, LAG, 0>(x, st, blk, xu, xs, sl);
}

// The start of an output wave's chunk: the state it starts from (every slice's),
// zero outputs, and the gate rows (LAG; otherwise read from the block later).
template <int DK, int OUT, bool BF16, int NSL, int NB>
__device__ __forceinline__ void out_begin(OutRegs<DK, NSL>& x, const OutPlaces& pl, const f32x4 (&gp)[2]) {
    using L = ScanLayout<DK, OUT, BF16, NSL, NB>;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    x.gp[0] = gp[0];
    x.gp[1] = gp[1];
#pragma unroll
    for (int q = 0; q < NSL; ++q) {
#pragma unroll
        for (int u = 0; u < DK / 32; ++u) x.sb[q][u] = get_h8(pl.sb + q * L::XC, u);
        x.o[q][0] = x.o[q][1] = z;
    }
}

// One chunk of an output wave (after out_begin): blk is the chunk's LDS block
// (its gate rows, unless LAG).
template <int DK, int OUT, bool BF16, int NSL, int NB, int H>
__device__ __forceinline__ void out_chunk(OutRegs<DK, NSL>& x, OutOps<DK, H>& ops, const OutSrc& nsrc,
                                          const unsigned char* blk, const OutPlaces& pl, float scale,
                                          const DmaCtx& d) {
    out_step<DK, OUT, BF16, NSL, NB, H, 0>(x, ops, nsrc, blk, pl, scale, d);
}

// NB LDS blocks for the chain waves' operands: with three, chunk c is in use,
// c + 1 landed or landing and c + 2 being loaded (one workgroup per CU); with
// two (two workgroups per CU, for launches of more workgroups than CUs), c + 1
// is loaded during c.
// LAG (three blocks): the output waves compute each chunk during the next one,
// from double-buffered hand-offs and staging, so the chunk has one barrier.
template <int DK, int OUT, bool BF16, int NSL, int NB>
struct ScanLayout {
    static constexpr int NBUF = NB;
    static constexpr bool LAG = NB == 3;
    using XG = Xchg<DK, LAG>;
    static constexpr int BLK = ChunkBlock<DK, BF16, NSL>::BYTES;
    static constexpr int XC = XG::BYTES;
    static constexpr int OST = OStage<OUT>::BYTES;
    static constexpr int NOST = LAG ? 2 : 1;  // staging copies (slice s of copy j at j NSL OST + s OST)
    static constexpr int BYTES = NBUF * BLK + NSL * (XC + NOST * OST);
    __device__ static int ost(int ck) { return (LAG ? ck % 2 : 0) * NSL * OST; }
};

// Output wave H (rows 32 H .. 32 H + 31 of both slices; it writes out slice H's
// staged outputs, which both output waves stage).  Every pass starts with its
// wait for its loads (loads into LDS and registers count as vector-memory
// operations, which the barrier alone does not wait for) and the barrier that
// publishes the chunk with the chain waves' starting state.  Without LAG, pass
// ck computes chunk ck alongside the chain waves (U handed over at the middle
// barrier); with LAG, pass ck computes chunk ck - 1 from what the chain waves
// published during it (one more pass at the end), and keeps chunk ck's gate
// rows in registers for the next pass, so no wave reads a block after the
// loads of a later chunk into it may have been issued.
template <int DK, int OUT, bool BF16, int NSL, int NB, int H>
__device__ __forceinline__ void out_wave(const ScanCtx<DK>& X, unsigned char* lds_raw, float scale) {
    using L = ScanLayout<DK, OUT, BF16, NSL, NB>;
    using XG = typename L::XG;
    using CB = ChunkBlock<DK, BF16, NSL>;
    static_assert(NSL == 2 && kC == 64, "two output waves, one per 32-row half of a chunk");
    constexpr int NDMA = CB::NLOAD / NSL;  // LDS loads per chunk and output wave
    static_assert(NDMA < 64, "vmcnt field of the top wait");
    const unsigned char* xcb = lds_raw + L::NBUF * L::BLK;
    unsigned char* ostb = lds_raw + L::NBUF * L::BLK + NSL * L::XC;
    const int lg = (threadIdx.x & 63) >> 4;
    OutOps<DK, H> ops;
    load_out_ops<DK, H, 0>(ops, out_src(X, 0));
#pragma unroll
    for (int c0 = 0; c0 < NB - 1; ++c0)
        dma_slots<DK, BF16, NSL, 0, NDMA>(dma_ctx<DK, BF16, NSL>(X, c0, lds_raw + c0 * L::BLK, H));
    // the top wait: with three blocks everything but the last NDMA loads (those of chunk
    // ck + 1, issued last) has landed; with two, everything
    constexpr int VMC = NB == 3 ? NDMA : 0;
    if constexpr (!L::LAG) {
        // pass ck computes chunk ck (the gate rows come from its block at the middle barrier)
        const OutPlaces pl = {xcb + XG::sb(0), xcb + XG::ub(0), ostb};
        const f32x4 gz[2] = {};
        for (int ck = 0; ck < X.nch; ++ck) {
            // this chunk's LDS block and registers, and the previous chunk's stores, have landed
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt((VMC & 15) | (VMC >> 4) << 14 | 0x0070);  // vmcnt(VMC) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            // the chunk's starting states first: the products wait on them, the stores below do not
            OutRegs<DK, NSL> x;
            out_begin<DK, OUT, BF16, NSL, NB>(x, pl, gz);
            __builtin_amdgcn_sched_barrier(0);
            if (ck > 0) write_out<DK, OUT>(X, ostb + H * L::OST, ck - 1, H);
            // chunk ck + NB - 1 (the last chunks load themselves again into an idle block: harmless);
            // with two blocks its loads go out here, a whole chunk ahead of their use
            const DmaCtx d = dma_ctx<DK, BF16, NSL>(X, ck + NB - 1, lds_raw + ((ck + NB - 1) % NB) * L::BLK, H);
            if constexpr (NB == 2) dma_slots<DK, BF16, NSL, 0, NDMA>(d);
            out_chunk<DK, OUT, BF16, NSL, NB, H>(x, ops, out_src(X, ck + 1), lds_raw + (ck % L::NBUF) * L::BLK, pl,
                                                 scale, d);
        }
    } else {
        f32x4 gp[2] = {};  // gate rows (gamma at this wave's rows) of the chunk computed next
        for (int ck = 0; ck <= X.nch; ++ck) {
            // this chunk's LDS block and registers, and the stores of two passes ago, have landed
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt((VMC & 15) | (VMC >> 4) << 14 | 0x0070);  // vmcnt(VMC) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const int cw = ck - 2;  // the chunk staged in the previous pass
            const int cc = ck - 1;  // the chunk this pass computes
            // this pass's LDS offsets as opaque scalars (otherwise loop strength reduction keeps one
            // address register per access, rebuilt every pass)
            int ow = L::ost(cw), od = ((ck + NB - 1) % NB) * L::BLK, og = (ck % L::NBUF) * L::BLK + CB::G0;
            int ob = (cc % L::NBUF) * L::BLK, os = XG::sb(cc), ou = XG::ub(cc), oo = L::ost(cc);
            asm volatile("" : "+s"(ow), "+s"(od), "+s"(og), "+s"(ob), "+s"(os), "+s"(ou), "+s"(oo));
            if (cw >= 0) write_out<DK, OUT>(X, ostb + ow + H * L::OST, cw, H);
            // chunk ck + 2 (the last chunks load themselves again into an idle block: harmless)
            const DmaCtx d = dma_ctx<DK, BF16, NSL>(X, ck + NB - 1, lds_raw + od, H);
            f32x4 gn[2] = {gp[0], gp[1]};
            if (ck < X.nch) {
                const float* gam = reinterpret_cast<const float*>(lds_raw + og);
#pragma unroll
                for (int i = 0; i < 2; ++i) gn[i] = *reinterpret_cast<const f32x4*>(gam + pair_row(2 * H + i, 4 * lg));
            }
            if (cc >= 0) {
                const OutPlaces pl = {xcb + os, xcb + ou, ostb + oo};
                OutRegs<DK, NSL> x;
                out_begin<DK, OUT, BF16, NSL, NB>(x, pl, gp);
                out_chunk<DK, OUT, BF16, NSL, NB, H>(x, ops, out_src(X, cc + 1), lds_raw + ob, pl, scale, d);
            } else {
                dma_slots<DK, BF16, NSL, 0, NDMA>(d);  // the first pass computes nothing; its loads still go out
            }
            gp[0] = gn[0];
            gp[1] = gn[1];
        }
    }
    // both output waves' staging of the last chunk is in place
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    write_out<DK, OUT>(X, ostb + L::ost(X.nch - 1) + H * L::OST, X.nch - 1, H);
    // the last chunks' repeated loads into LDS land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
}

// One workgroup of 2 NSL waves per (sequence, value head, 16 NSL value
// columns): waves 0 .. NSL-1 are the chain waves of the NSL 16-column slices,
// waves NSL .. 2 NSL - 1 the output waves (each one half of every slice's
// output rows).
template <int DK, int OUT, bool BF16, int NSL, int NB>
__global__ __launch_bounds__(128 * NSL) void prefill_scan_kernel(const PrefillArgs a, const PrefillSeqs seqs) {
    using L = ScanLayout<DK, OUT, BF16, NSL, NB>;
    constexpr int NT = DK / 16;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const bool chain = w < NSL;
    const int sl = chain ? w : w - NSL;  // chain wave: slice (value columns col0 + 16 sl ..); output wave: half
    const int c = lane & 15, lg = lane >> 4;
    int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int grp = blk % a.slices;
    blk /= a.slices;
    ScanCtx<DK> X;
    X.a = &a;
    X.wsb = static_cast<const unsigned char*>(a.workspace);
    X.h = blk % a.h_v;
    X.b = blk / a.h_v;
    X.g = X.h / a.group;
    const SeqInfo sq = seq_info(a, seqs, X.b);
    if (sq.nch == 0) return;  // an empty sequence: its state stays as it is (uniform over the workgroup)
    X.nch = sq.nch;
    X.tok0 = sq.tok0;
    X.T = sq.T;
    X.unit0 = sq.unit0;
    X.ws = ws_layout(a.units, a.h_qk, a.h_v, DK);
    X.cols = 16 * NSL;
    X.col0 = X.cols * grp;

    int s = a.seq0 + X.b;
    if (a.state_slot != nullptr) {
        s = a.state_slot[a.seq0 + X.b];
        if (s < 0 || s >= a.n_slots) {
            if (threadIdx.x == 0 && a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
            return;  // uniform over the workgroup: every wave leaves before any barrier
        }
    }
    using XG = typename L::XG;
    unsigned char* xc = lds_raw + L::NBUF * L::BLK + sl * L::XC;
    float* stp = a.state + GDN_AT((((size_t)s * a.h_v + X.h) * a.d_v + X.col0 + 16 * sl + c) * DK, DK,
                                  (size_t)(a.state_slot != nullptr ? a.n_slots : a.batch_total) * a.h_v * a.d_v * DK,
                                  a.status);
    // Each role runs its own loop (the same barriers per chunk), so the registers of one role's
    // loop-carried values are not held by the other.  Every chunk starts with the output waves'
    // wait for their loads of the chunk (loads into LDS and registers count as vector-memory
    // operations, which the barrier alone does not wait for) and a barrier that publishes the
    // chunk with the chain waves' starting state; every wave is then done with the LDS block of
    // the chunk before, which the chunk after next is loaded into.
    if (chain) {
        // lane (c, g) holds H[d_k][j] = S[j][d_k] for d_k = pair_row(t, 4g + r)
        f32x4 st[NT];
        h8 sb[DK / 32];  // st in f16, the B operand of K H and Q H
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[t][r] = stp[pair_row(t, 4 * lg) + r];
#pragma unroll
        for (int u = 0; u < DK / 32; ++u) {
            sb[u] = pack_h8(st[2 * u], st[2 * u + 1]);
            put_h8(xc + XG::sb(0), u, sb[u]);
        }
        for (int ck = 0; ck < X.nch; ++ck) {
            if constexpr (L::LAG) {
                // No wait for this wave's LDS writes: U of the chunk before, which the output waves
                // read after this barrier, landed before that chunk's state copy went out (chain_step);
                // the state copy is read a pass later and lands before this wave's first operand wait
                // of this chunk (LDS operations complete in order).
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            } else {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            // LAG: the chunk's LDS offsets as opaque scalars; otherwise loop strength reduction keeps
            // one address register per operand read, rebuilt every chunk with a vector add
            int ob = (ck % L::NBUF) * L::BLK, ou = XG::ub(ck), os = XG::sb(ck + 1);
            if constexpr (L::LAG) asm volatile("" : "+s"(ob), "+s"(ou), "+s"(os));
            chain_chunk<DK, BF16, NSL, L::LAG>(st, sb, lds_raw + ob, xc + ou, xc + os, sl);
            // the state after every state_interval-th full chunk, for prefix caching
            if (a.chunk_states != nullptr && (ck + 1) % a.state_interval == 0 && (ck + 1) * kC <= X.T) {
                const size_t m = (size_t)sq.cst0 + (ck + 1) / a.state_interval - 1;
                float* csp = a.chunk_states + GDN_AT(((m * a.h_v + X.h) * a.d_v + X.col0 + 16 * sl + c) * DK, DK,
                                                     (size_t)a.n_chunk_states * a.h_v * a.d_v * DK, a.status);
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) csp[pair_row(t, 4 * lg) + r] = st[t][r];
            }
        }
        // the output waves' remaining barriers: LAG, the pass that computes the last chunk (after
        // this wave's hand-offs of it have landed); then the one after their last staging
        if constexpr (L::LAG) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        __syncthreads();
        // A value outside the f16 range on the way (an input V, a right-hand side R or the
        // state's f16 copy) makes the state non-finite, and it stays so: report it.
        bool finite = true;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                finite &= __builtin_isfinite(st[t][r]);
                stp[pair_row(t, 4 * lg) + r] = st[t][r];
            }
        if (!finite && a.status != nullptr) a.status[0] = GDN_ERR_RANGE;
    } else {
        if (sl == 0) out_wave<DK, OUT, BF16, NSL, NB, 0>(X, lds_raw, a.scale);
        else out_wave<DK, OUT, BF16, NSL, NB, 1>(X, lds_raw, a.scale);
    }
}
template <int DK, int OUT, bool BF16, int NSL, int NB>
hipError_t launch_scan_nb(const PrefillArgs& s, const PrefillSeqs& seqs, long long grid, hipStream_t st) {
    constexpr size_t lds = ScanLayout<DK, OUT, BF16, NSL, NB>::BYTES;
    static_assert(lds <= kMaxLdsBytes, "scan LDS");
    hipError_t e = allow_max_lds<&prefill_scan_kernel<DK, OUT, BF16, NSL, NB>>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_scan_kernel<DK, OUT, BF16, NSL, NB>), dim3((int)grid), dim3(128 * NSL), lds, st, s,
                       seqs);
    return hipGetLastError();
}

// Three LDS blocks when the workgroups fit the CUs one each; two (two
// workgroups per CU, each hiding the other's waits) when there are more
// workgroups than CUs.
template <int DK, int OUT, bool BF16, int NSL>
hipError_t launch_scan_nsl(const PrefillArgs& a, const PrefillSeqs& seqs, hipStream_t st) {
    PrefillArgs s = a;
    s.slices = a.d_v / (16 * NSL);
    const long long grid = (long long)a.batch * a.h_v * s.slices;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    // two blocks pay only where two workgroups then fit a CU's 160 KB of LDS
    constexpr bool TWO_FIT = 2 * ScanLayout<DK, OUT, BF16, NSL, 2>::BYTES <= 160 * 1024;
    if constexpr (TWO_FIT) {
        if (grid > device_cus()) return launch_scan_nb<DK, OUT, BF16, NSL, 2>(s, seqs, grid, st);
    }
    return launch_scan_nb<DK, OUT, BF16, NSL, 3>(s, seqs, grid, st);
}

// Two 16-column slices per workgroup: with four (one fetch of each chunk's
// operands for 64 columns, two waves per SIMD) the chain waves shared their
// SIMDs and the scan measured 25% slower.
template <int DK, int OUT, bool BF16>
hipError_t launch_scan(const PrefillArgs& a, const PrefillSeqs& seqs, hipStream_t st) {
    return launch_scan_nsl<DK, OUT, BF16, 2>(a, seqs, st);
}

template <int DK, bool BF16>
hipError_t launch_dk(const PrefillArgs& a, const PrefillSeqs& seqs, int out_dtype, int prep_grid, hipStream_t st) {
    const size_t lds = PrepLds<DK>::bytes(a.group);
    if (lds > (size_t)kMaxLdsBytes) return hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    if (lds > (size_t)kDefaultLdsBytes && (e = allow_max_lds<&prefill_prepare_kernel<DK, BF16>>()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((prefill_prepare_kernel<DK, BF16>), dim3(prep_grid), dim3(256), lds, st, a, seqs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    switch (out_dtype) {
        case GDN_F32: return launch_scan<DK, 0, BF16>(a, seqs, st);
        case GDN_BF16: return launch_scan<DK, 1, BF16>(a, seqs, st);
        case GDN_F16: return launch_scan<DK, 2, BF16>(a, seqs, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DK>
hipError_t launch_dk_any(const PrefillArgs& a, const PrefillSeqs& seqs, int out_dtype, int prep_grid, hipStream_t st) {
    return a.qkv_bf16 ? launch_dk<DK, true>(a, seqs, out_dtype, prep_grid, st)
                      : launch_dk<DK, false>(a, seqs, out_dtype, prep_grid, st);
}

}  // namespace

int device_cus() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    const bool cache = dev >= 0 && dev < kMaxDevices;
    if (cache && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    if (cache) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

size_t prefill_workspace_bytes(long long units, int h_qk, int h_v, int d_k) {
    return ws_layout((size_t)units, h_qk, h_v, d_k).total;
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillSeqs& seqs, int d_k, int out_dtype, hipStream_t stream) {
    const long long prep = (long long)a.units * a.h_qk;
    if (prep > 0x7fffffffLL) return hipErrorInvalidValue;
    if (prep == 0) return hipSuccess;
    switch (d_k) {
        case 32: return launch_dk_any<32>(a, seqs, out_dtype, (int)prep, stream);
        case 64: return launch_dk_any<64>(a, seqs, out_dtype, (int)prep, stream);
        case 128: return launch_dk_any<128>(a, seqs, out_dtype, (int)prep, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
