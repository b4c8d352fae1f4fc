// prefill.hip -- chunked (WY / UT) prefill of the gated delta rule on gfx950.
//
// The pages name chunked linear-attention prefill as an engine feature (page
// "We got 207 tok/s with Qwen3.5-27B on an RTX 3090", section "Prefill"); the
// chunk algebra here is derived from the rule.  With H = S^T (d_k x d_v) and
// a chunk of C = 64 tokens starting from H_0:
//   l_t = sum_{s<=t} log alpha_s,  gamma_t = e^{l_t},  Gamma_{t,i} = e^{l_t - l_i}
//   A   = strict_lower(beta_t Gamma_{t,i} k_t.k_i),  T = (I + A)^{-1}
//   R   = diag(beta) V - diag(beta gamma) K H_0,     U = T R
//   O   = scale [diag(gamma) Q H_0 + (Gamma o tril(Q K^T)) U]
//   H_C = gamma_C H_0 + K^T diag(Gamma_{C,.}) U
// (U = T R is the usual W / U' form, T diag(beta) V - T diag(beta gamma) K H_0,
// with the product by T applied once to the combined right-hand side.)
//
// Two kernels.
//  * prepare (one workgroup per (sequence, chunk, value head), all in
//    parallel): everything that does not depend on the state -- the gates,
//    K K^T and Q K^T on the matrix cores, the masked matrices, and the UT
//    transform T = (I + A)^{-1} in fp32 (16 x 16 diagonal blocks by forward
//    substitution, off-diagonal blocks by v_mfma_f32_16x16x4_f32).  It writes
//    T and P = Gamma o tril(Q K^T) in f16, the per-token gate factors, and
//    K^T in f16 (once per q/k head) to the workspace.
//  * scan (one workgroup per (sequence, value head, 32 value columns),
//    sequential over chunks): the state slice stays in MFMA accumulators for
//    the whole prompt; per chunk it forms K H, Q H, R, U = T R, O and the
//    state update with v_mfma_f32_16x16x32_f16, while the next chunk's
//    operands are already being loaded into registers.
// All matrix-core operands are f16 with fp32 accumulation: the bf16 inputs are
// exact in f16 within the f16 range, and the derived operands (T, R, P, U, H)
// keep f16's 11-bit significand, enough for the parity bar where bf16 is not.
// Every matrix in LDS keeps its contraction index contiguous, so an operand
// fragment is one 16-byte LDS read per lane.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kC = GDN_PREFILL_CHUNK;  // tokens per chunk
constexpr int kDVS = 32;               // value columns per scan workgroup
constexpr int kLdT = kC + 8;           // row length (halves) of token-contiguous matrices
constexpr int kLdF = kC + 4;           // row length (floats) of the fp32 A and T matrices
constexpr float kLogFloor = -80.f;     // log alpha is clamped here (a zero gate -> e^-80)

__device__ __forceinline__ f32x4 mfma16(const h8& a, const h8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// MFMA operand fragment of a row-major f16 matrix X (leading dimension ld):
// rows row0 + lane % 16, contraction columns k0 + 8 * (lane / 16) .. + 8.
__device__ __forceinline__ h8 frag(const _Float16* X, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const h8*>(X + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ h8 to_h8(const float (&x)[8]) {
    h8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)x[i];
    return r;
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
template <bool BF16>
__device__ __forceinline__ h8 raw_to_h8(const Raw8& r, bool valid) {
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
    for (int i = 0; i < 8; ++i) x[i] = valid ? x[i] : 0.f;
    return to_h8(x);
}

// Workspace layout (bytes), per sequence b and chunk c:
//   T, P   [B][nch][h_v][C][C]     f16
//   gates  [B][nch][h_v][3][C]     fp32: gamma_t, beta_t, Gamma_{C,t}
//   KT     [B][nch][h_qk][d_k][C]  f16   (K transposed)
//   K, Q   [B][nch][h_qk][C][d_k]  f16   (converted once, read by every slice)
struct WsLayout {
    size_t T, P, G, KT, K, Q, total;
};
__host__ __device__ inline WsLayout ws_layout(int B, int nch, int h_qk, int h_v, int d_k) {
    WsLayout w;
    const size_t units = (size_t)B * nch;
    w.T = 0;
    w.P = w.T + units * h_v * kC * kC * 2;
    w.G = w.P + units * h_v * kC * kC * 2;
    w.KT = w.G + units * h_v * 3 * kC * 4;
    w.K = w.KT + units * h_qk * (size_t)d_k * kC * 2;
    w.Q = w.K + units * h_qk * (size_t)d_k * kC * 2;
    w.total = w.Q + units * h_qk * (size_t)d_k * kC * 2;
    return w;
}

// ---------------------------------------------------------------------------
// prepare: one (sequence, chunk, value head) per workgroup
// ---------------------------------------------------------------------------
template <int DK>
struct PrepLds {
    static constexpr int kLdK = DK + 8;
    union {
        struct {
            _Float16 Kf[kC * kLdK];  // K chunk [token][d_k]
            _Float16 Qf[kC * kLdK];  // Q chunk [token][d_k]
        } in;
        struct {
            float A[kC * kLdF];   // strict lower beta Gamma K K^T
            float Tm[kC * kLdF];  // (I + A)^-1
        } ut;
    } u;
    _Float16 P[kC * kLdT];  // Gamma o tril(Q K^T)
    float Y[4][16 * 16];    // per-wave scratch block
    float ell[kC], al[kC], be[kC];
};

template <int DK, bool BF16>
__global__ __launch_bounds__(256) void prefill_prepare_kernel(const PrefillArgs a) {
    constexpr int kLdK = DK + 8;
    constexpr int KSD = DK / 32;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    PrepLds<DK>& L = *reinterpret_cast<PrepLds<DK>*>(lds_raw);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = (a.T + kC - 1) / kC;
    int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int h = blk % a.h_v;
    blk /= a.h_v;
    const int ck = blk % nch;
    const int b = blk / nch;
    const int g = h / a.group;
    const int t0 = ck * kC;
    const WsLayout ws = ws_layout(a.batch, nch, a.h_qk, a.h_v, DK);
    unsigned char* wsb = static_cast<unsigned char*>(a.workspace);
    const size_t unit_v = ((size_t)b * nch + ck) * a.h_v + h;
    const size_t unit_q = ((size_t)b * nch + ck) * a.h_qk + g;

    // 1. K, Q chunk -> LDS (f16); gates -> LDS.  All loads are issued first
    //    (token index clamped into the sequence), then converted and stored.
    {
        constexpr int NK = kC * DK / 8 / 256;  // 8-element chunks per thread
        Raw8 rk[NK], rq[NK];
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            const int e = tid + 256 * n;
            const int t = e / (DK / 8), d = 8 * (e % (DK / 8));
            const int tc = t0 + t < a.T ? t0 + t : a.T - 1;
            const size_t src = (((size_t)b * a.T + tc) * a.h_qk + g) * DK + d;
            raw_load<BF16>(rk[n], a.k, src);
            raw_load<BF16>(rq[n], a.q, src);
        }
        const int tg = t0 + (tid & 63) < a.T ? t0 + (tid & 63) : a.T - 1;
        const float al = a.alpha[((size_t)b * a.T + tg) * a.h_v + h];
        const float be = a.beta[((size_t)b * a.T + tg) * a.h_v + h];
#pragma unroll
        for (int n = 0; n < NK; ++n) {
            const int e = tid + 256 * n;
            const int t = e / (DK / 8), d = 8 * (e % (DK / 8));
            const bool valid = t0 + t < a.T;
            *reinterpret_cast<h8*>(&L.u.in.Kf[t * kLdK + d]) = raw_to_h8<BF16>(rk[n], valid);
            *reinterpret_cast<h8*>(&L.u.in.Qf[t * kLdK + d]) = raw_to_h8<BF16>(rq[n], valid);
        }
        if (tid < kC) {
            const bool in = t0 + tid < a.T;
            L.al[tid] = in ? al : 1.f;
            L.be[tid] = in ? be : 0.f;
        }
    }
    __syncthreads();

    // 2. gates (wave 0): l_t by a wave prefix sum; gamma_t, Gamma_{C,t} -> workspace.
    //    K^T -> workspace (waves 1-3, once per q/k head).
    if (wave == 0) {
        float x = fmaxf(logf(L.al[lane]), kLogFloor);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        L.ell[lane] = x;
        const float lC = __shfl(x, 63, 64);
        float* gw = reinterpret_cast<float*>(wsb + ws.G) + unit_v * 3 * kC;
        gw[lane] = expf(x);
        gw[kC + lane] = L.be[lane];
        gw[2 * kC + lane] = expf(lC - x);
    } else if (h % a.group == 0) {
        _Float16* kt = reinterpret_cast<_Float16*>(wsb + ws.KT) + unit_q * DK * kC;
        _Float16* kw = reinterpret_cast<_Float16*>(wsb + ws.K) + unit_q * kC * DK;
        _Float16* qw = reinterpret_cast<_Float16*>(wsb + ws.Q) + unit_q * kC * DK;
        for (int e = tid - 64; e < DK * (kC / 8); e += 192) {
            const int d = e / (kC / 8), tt = 8 * (e % (kC / 8));
            h8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = L.u.in.Kf[(tt + i) * kLdK + d];
            *reinterpret_cast<h8*>(kt + d * kC + tt) = v;
            const int t = e / (DK / 8), dd = 8 * (e % (DK / 8));
            *reinterpret_cast<h8*>(kw + t * DK + dd) = *reinterpret_cast<const h8*>(&L.u.in.Kf[t * kLdK + dd]);
            *reinterpret_cast<h8*>(qw + t * DK + dd) = *reinterpret_cast<const h8*>(&L.u.in.Qf[t * kLdK + dd]);
        }
    }
    __syncthreads();

    // 3. Gram products on the lower 16 x 16 tiles (job = matrix x tile), kept in registers
    f32x4 gram[5];
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
        const int job = wave + 4 * jj;
        const int mat = job / 10, tix = job % 10;
        const int it = tix < 1 ? 0 : tix < 3 ? 1 : tix < 6 ? 2 : 3;
        const int jt = tix - it * (it + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
            acc = mfma16(frag(mat ? L.u.in.Qf : L.u.in.Kf, kLdK, 16 * it, 32 * ks, lane),
                         frag(L.u.in.Kf, kLdK, 16 * jt, 32 * ks, lane), acc);
        gram[jj] = acc;
    }
    __syncthreads();  // K, Q are dead: A and T overwrite them
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
        const int job = wave + 4 * jj;
        const int mat = job / 10, tix = job % 10;
        const int it = tix < 1 ? 0 : tix < 3 ? 1 : tix < 6 ? 2 : 3;
        const int jt = tix - it * (it + 1) / 2;
        const int i = 16 * jt + (lane & 15);
        const float li = L.ell[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * it + 4 * (lane >> 4) + r;
            const float gm = expf(L.ell[t] - li);
            if (mat == 0) L.u.ut.A[t * kLdF + i] = (t > i) ? L.be[t] * gm * gram[jj][r] : 0.f;
            else L.P[t * kLdT + i] = (_Float16)((t >= i) ? gm * gram[jj][r] : 0.f);
        }
    }
    // the upper tiles of P are zero
    for (int e = tid; e < 6 * 256; e += 256) {
        const int ut = e / 256, w = e % 256;
        const int it = ut < 3 ? 0 : ut < 5 ? 1 : 2;
        const int jt = ut < 3 ? 1 + ut : ut < 5 ? ut - 1 : 3;
        L.P[(16 * it + w / 16) * kLdT + 16 * jt + w % 16] = (_Float16)0.f;
    }
    __syncthreads();

    // 4. T = (I + A)^-1: diagonal 16 x 16 blocks, column j per lane (wave = block)
    {
        const int bb = wave, j = lane & 15;
        const float* Ab = L.u.ut.A + 16 * bb * kLdF + 16 * bb;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float arow[16];
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(Ab + t * kLdF + 4 * m4);
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * m4 + e] = v[e];
            }
            float sum = (t == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < t; ++m) sum = fmaf(-arow[m], x[m], sum);
            x[t] = sum;
        }
        if (lane < 16) {
#pragma unroll
            for (int t = 0; t < 16; ++t) L.u.ut.Tm[(16 * bb + t) * kLdF + 16 * bb + j] = x[t];
        }
    }
    __syncthreads();
    // off-diagonal blocks, by distance: X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
        const int j = wave, i = wave + dist;
        const bool active = i < 4;
        if (active) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = j; kk < i; ++kk) {
                const float* Lb = L.u.ut.A + 16 * i * kLdF + 16 * kk;
                const float* Rb = L.u.ut.Tm + 16 * kk * kLdF + 16 * j;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Lb[(lane & 15) * kLdF + 4 * s + (lane >> 4)],
                                                               Rb[(4 * s + (lane >> 4)) * kLdF + (lane & 15)], acc,
                                                               0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) L.Y[wave][(4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[r];
        }
        __syncthreads();
        if (active) {
            const float* Xi = L.u.ut.Tm + 16 * i * kLdF + 16 * i;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Xi[(lane & 15) * kLdF + 4 * s + (lane >> 4)],
                                                           L.Y[wave][(4 * s + (lane >> 4)) * 16 + (lane & 15)], acc,
                                                           0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                L.u.ut.Tm[(16 * i + 4 * (lane >> 4) + r) * kLdF + 16 * j + (lane & 15)] = -acc[r];
        }
        __syncthreads();
    }

    // 5. T (f16, zero above the diagonal) and P -> workspace, 16-byte stores
    _Float16* Tw = reinterpret_cast<_Float16*>(wsb + ws.T) + unit_v * kC * kC;
    _Float16* Pw = reinterpret_cast<_Float16*>(wsb + ws.P) + unit_v * kC * kC;
    for (int e = tid; e < kC * kC / 8; e += 256) {
        const int t = e / (kC / 8), i0 = 8 * (e % (kC / 8));
        h8 tv;
#pragma unroll
        for (int i = 0; i < 8; ++i) tv[i] = (_Float16)((i0 + i <= t) ? L.u.ut.Tm[t * kLdF + i0 + i] : 0.f);
        *reinterpret_cast<h8*>(Tw + t * kC + i0) = tv;
        *reinterpret_cast<h8*>(Pw + t * kC + i0) = *reinterpret_cast<const h8*>(&L.P[t * kLdT + i0]);
    }
}

// ---------------------------------------------------------------------------
// scan: one (sequence, value head, 32 value columns) per workgroup
// ---------------------------------------------------------------------------
template <int DK>
struct ScanLds {
    static constexpr int kLdK = DK + 8;
    _Float16 Kf[kC * kLdK];    // K chunk [token][d_k]
    _Float16 Qf[kC * kLdK];    // Q chunk [token][d_k]
    _Float16 KT[DK * kLdT];    // K^T [d_k][token]
    _Float16 Tt[kC * kLdT];    // T [token][token]
    _Float16 P[kC * kLdT];     // Gamma o tril(Q K^T)
    _Float16 Vs[kC * (kDVS + 8)];  // V slice [token][value col]
    _Float16 RT[kDVS * kLdT];  // R^T [value col][token]
    _Float16 UT[kDVS * kLdT];  // U^T
    _Float16 UG[kDVS * kLdT];  // (Gamma_{C,t} U)^T
    _Float16 Sf[kDVS * kLdK];  // state slice (f16) [value col][d_k]
    float Os[kC * (kDVS + 4)]; // this chunk's outputs (fp32) [token][value col]
    float gam[kC], bet[kC], gC[kC];
};

template <int DK>
struct ScanRegs {
    static constexpr int NK = kC * DK / 8 / 256;  // 16-byte chunks per thread of K (and Q, K^T)
    u32x4 k[NK], q[NK], kt[NK], tt[2], pp[2];
    Raw8 v;
    float g0, g1, g2;
};

// Issue every global load of chunk ck (token indices clamped into the
// sequence; the invalid rows are zeroed when stored).
template <int DK, bool BF16>
__device__ __forceinline__ void scan_load(ScanRegs<DK>& R, const PrefillArgs& a, const unsigned char* wsb,
                                          const WsLayout& ws, int b, int h, int g, int ck, int nch, int col0,
                                          int tid) {
    constexpr int NK = ScanRegs<DK>::NK;
    const int t0 = ck * kC;
    const int tmax = a.T - 1;
    const size_t unit_v = ((size_t)b * nch + ck) * a.h_v + h;
    const size_t unit_q = ((size_t)b * nch + ck) * a.h_qk + g;
    const uint16_t* ktw = reinterpret_cast<const uint16_t*>(wsb + ws.KT) + unit_q * DK * kC;
    const uint16_t* kw = reinterpret_cast<const uint16_t*>(wsb + ws.K) + unit_q * kC * DK;
    const uint16_t* qw = reinterpret_cast<const uint16_t*>(wsb + ws.Q) + unit_q * kC * DK;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
        R.k[n] = *reinterpret_cast<const u32x4*>(kw + 8 * (tid + 256 * n));
        R.q[n] = *reinterpret_cast<const u32x4*>(qw + 8 * (tid + 256 * n));
        R.kt[n] = *reinterpret_cast<const u32x4*>(ktw + 8 * (tid + 256 * n));
    }
    const uint16_t* tw = reinterpret_cast<const uint16_t*>(wsb + ws.T) + unit_v * kC * kC;
    const uint16_t* pw = reinterpret_cast<const uint16_t*>(wsb + ws.P) + unit_v * kC * kC;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        R.tt[n] = *reinterpret_cast<const u32x4*>(tw + 8 * (tid + 256 * n));
        R.pp[n] = *reinterpret_cast<const u32x4*>(pw + 8 * (tid + 256 * n));
    }
    {
        const int t = tid / (kDVS / 8), j = 8 * (tid % (kDVS / 8));
        const int tc = t0 + t < tmax ? t0 + t : tmax;
        raw_load<BF16>(R.v, a.v, (((size_t)b * a.T + tc) * a.h_v + h) * a.d_v + col0 + j);
    }
    const float* gw = reinterpret_cast<const float*>(wsb + ws.G) + unit_v * 3 * kC;
    R.g0 = gw[tid & 63];
    R.g1 = gw[kC + (tid & 63)];
    R.g2 = gw[2 * kC + (tid & 63)];
}

template <int DK, bool BF16>
__device__ __forceinline__ void scan_store(const ScanRegs<DK>& R, ScanLds<DK>& L, int tid, int t0, int T) {
    constexpr int NK = ScanRegs<DK>::NK;
    constexpr int kLdK = DK + 8;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
        const int e = tid + 256 * n;
        const int t = e / (DK / 8), d = 8 * (e % (DK / 8));
        *reinterpret_cast<u32x4*>(&L.Kf[t * kLdK + d]) = R.k[n];  // zero rows past T come from prepare
        *reinterpret_cast<u32x4*>(&L.Qf[t * kLdK + d]) = R.q[n];
        const int dd = e / (kC / 8), tt = 8 * (e % (kC / 8));
        *reinterpret_cast<u32x4*>(&L.KT[dd * kLdT + tt]) = R.kt[n];
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e = tid + 256 * n;
        const int t = e / (kC / 8), i0 = 8 * (e % (kC / 8));
        *reinterpret_cast<u32x4*>(&L.Tt[t * kLdT + i0]) = R.tt[n];
        *reinterpret_cast<u32x4*>(&L.P[t * kLdT + i0]) = R.pp[n];
    }
    {
        const int t = tid / (kDVS / 8), j = 8 * (tid % (kDVS / 8));
        *reinterpret_cast<h8*>(&L.Vs[t * (kDVS + 8) + j]) = raw_to_h8<BF16>(R.v, t0 + t < T);
    }
    if (tid < kC) {
        L.gam[tid] = R.g0;
        L.bet[tid] = R.g1;
        L.gC[tid] = R.g2;
    }
}

// One chunk's outputs, staged in LDS as fp32 [token][value col] and written
// out as 16-byte rows of the output dtype.
template <int OUT>
__device__ __forceinline__ void write_out(const float* Os, const PrefillArgs& a, int b, int h, int col0, int t0,
                                          int tid) {
    constexpr int EPT = OUT == 0 ? 4 : 8;  // elements per 16-byte store
    constexpr int PER_ROW = kDVS / EPT;
    for (int e = tid; e < kC * PER_ROW; e += 256) {
        const int t = e / PER_ROW, j = EPT * (e % PER_ROW);
        if (t0 + t >= a.T) continue;
        const float* src = Os + t * (kDVS + 4) + j;
        const size_t idx = (((size_t)b * a.T + t0 + t) * a.h_v + h) * a.d_v + col0 + j;
        if constexpr (OUT == 0) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + idx) = *reinterpret_cast<const f32x4*>(src);
        } else if constexpr (OUT == 2) {
            h8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (_Float16)src[i];
            *reinterpret_cast<h8*>(static_cast<_Float16*>(a.out) + idx) = v;
        } else {
            u32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = (uint32_t)f32_to_bf16(src[2 * i]) | ((uint32_t)f32_to_bf16(src[2 * i + 1]) << 16);
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + idx) = v;
        }
    }
}

template <int DK, int OUT, bool BF16>
__global__ __launch_bounds__(256) void prefill_scan_kernel(const PrefillArgs a) {
    constexpr int kLdK = DK + 8;
    constexpr int NT = DK / 16;      // d_k tiles
    constexpr int KSD = DK / 32;     // contraction steps over d_k
    constexpr int STW = 2 * NT / 4;  // state tiles per wave
    extern __shared__ __align__(16) unsigned char lds_raw[];
    ScanLds<DK>& L = *reinterpret_cast<ScanLds<DK>*>(lds_raw);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    const int slice = blk % a.slices;
    blk /= a.slices;
    const int h = blk % a.h_v;
    const int b = blk / a.h_v;
    const int g = h / a.group;
    const int col0 = slice * kDVS;
    const int nch = (a.T + kC - 1) / kC;
    const WsLayout ws = ws_layout(a.batch, nch, a.h_qk, a.h_v, DK);
    const unsigned char* wsb = static_cast<const unsigned char*>(a.workspace);

    int s = b;
    if (a.state_slot != nullptr) {
        s = a.state_slot[b];
        if (s < 0 || s >= a.n_slots) {
            if (tid == 0 && a.status != nullptr) a.status[0] = GDN_ERR_SLOT;
            return;
        }
    }
    float* stp = a.state + ((size_t)s * a.h_v + h) * (size_t)a.d_v * DK;

    // state tiles: x = wave * STW + y -> value tile x / NT, d_k tile x % NT;
    // lane holds S[col0 + 16 vt + 4 (lane / 16) + r][16 dt + lane % 16]
    f32x4 st[STW];
#pragma unroll
    for (int y = 0; y < STW; ++y) {
        const int x = wave * STW + y, vt = x / NT, dt = x % NT;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st[y][r] = stp[(size_t)(col0 + 16 * vt + 4 * (lane >> 4) + r) * DK + 16 * dt + (lane & 15)];
    }
#pragma unroll
    for (int y = 0; y < STW; ++y) {
        const int x = wave * STW + y, vt = x / NT, dt = x % NT;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            L.Sf[(16 * vt + 4 * (lane >> 4) + r) * kLdK + 16 * dt + (lane & 15)] = (_Float16)st[y][r];
    }

    ScanRegs<DK> R;
    scan_load<DK, BF16>(R, a, wsb, ws, b, h, g, 0, nch, col0, tid);
    const int it = wave;            // row block of the per-token products
    const int ksmax = it / 2;       // T and P are lower triangular
    const int tb = 16 * it + 4 * (lane >> 4);  // first token row held by this lane
    for (int ck = 0; ck < nch; ++ck) {
        const int t0 = ck * kC;
        scan_store<DK, BF16>(R, L, tid, t0, a.T);
        if (ck + 1 < nch) scan_load<DK, BF16>(R, a, wsb, ws, b, h, g, ck + 1, nch, col0, tid);
        // the previous chunk's outputs leave after this chunk's loads are issued, so the wait
        // for this chunk's prefetched operands never waits on output stores
        if (ck > 0) write_out<OUT>(L.Os, a, b, h, col0, t0 - kC, tid);
        __syncthreads();

        // K H and Q H for rows 16 it, both value tiles; R = beta V - beta gamma K H
        f32x4 oacc[2], kh[2];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) kh[vt] = oacc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const h8 ak = frag(L.Kf, kLdK, 16 * it, 32 * ks, lane);
            const h8 aq = frag(L.Qf, kLdK, 16 * it, 32 * ks, lane);
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                const h8 sb = frag(L.Sf, kLdK, 16 * vt, 32 * ks, lane);
                kh[vt] = mfma16(ak, sb, kh[vt]);
                oacc[vt] = mfma16(aq, sb, oacc[vt]);
            }
        }
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
            const int col = 16 * vt + (lane & 15);
            h4 r4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float bt = L.bet[tb + r], gt = L.gam[tb + r];
                const float vv = (float)L.Vs[(tb + r) * (kDVS + 8) + col];
                r4[r] = (_Float16)(bt * (vv - gt * kh[vt][r]));
                oacc[vt][r] *= gt;
            }
            *reinterpret_cast<h4*>(&L.RT[col * kLdT + tb]) = r4;
        }
        __syncthreads();

        // U = T R
        f32x4 uacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        for (int ks = 0; ks <= ksmax; ++ks) {
            const h8 at = frag(L.Tt, kLdT, 16 * it, 32 * ks, lane);
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) uacc[vt] = mfma16(at, frag(L.RT, kLdT, 16 * vt, 32 * ks, lane), uacc[vt]);
        }
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
            const f32x4 u = uacc[vt];
            const int col = 16 * vt + (lane & 15);
            h4 u4, g4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u4[r] = (_Float16)u[r];
                g4[r] = (_Float16)(L.gC[tb + r] * u[r]);
            }
            *reinterpret_cast<h4*>(&L.UT[col * kLdT + tb]) = u4;
            *reinterpret_cast<h4*>(&L.UG[col * kLdT + tb]) = g4;
        }
        __syncthreads();

        // O = scale (gamma Q H + P U) -> LDS (written out with the next chunk's staging)
        for (int ks = 0; ks <= ksmax; ++ks) {
            const h8 ap = frag(L.P, kLdT, 16 * it, 32 * ks, lane);
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) oacc[vt] = mfma16(ap, frag(L.UT, kLdT, 16 * vt, 32 * ks, lane), oacc[vt]);
        }
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
            const int col = 16 * vt + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) L.Os[(tb + r) * (kDVS + 4) + col] = a.scale * oacc[vt][r];
        }
        // state: H_C = gamma_C H_0 + K^T diag(Gamma_C) U  (as S = H^T on the accumulators)
        // a wave's state tiles share one value tile (STW <= NT), so one U fragment serves them all
        const float gc = L.gam[kC - 1];
        const int vtw = (wave * STW) / NT;
#pragma unroll
        for (int y = 0; y < STW; ++y)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[y][r] *= gc;
#pragma unroll
        for (int ks = 0; ks < kC / 32; ++ks) {
            const h8 au = frag(L.UG, kLdT, 16 * vtw, 32 * ks, lane);
#pragma unroll
            for (int y = 0; y < STW; ++y) {
                const int dt = (wave * STW + y) % NT;
                st[y] = mfma16(au, frag(L.KT, kLdT, 16 * dt, 32 * ks, lane), st[y]);
            }
        }
        __syncthreads();  // every read of this chunk's LDS data is done
#pragma unroll
        for (int y = 0; y < STW; ++y) {
            const int x = wave * STW + y, vt = x / NT, dt = x % NT;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                L.Sf[(16 * vt + 4 * (lane >> 4) + r) * kLdK + 16 * dt + (lane & 15)] = (_Float16)st[y][r];
        }
    }

    write_out<OUT>(L.Os, a, b, h, col0, (nch - 1) * kC, tid);  // last chunk's outputs
    // final state, in place
#pragma unroll
    for (int y = 0; y < STW; ++y) {
        const int x = wave * STW + y, vt = x / NT, dt = x % NT;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            stp[(size_t)(col0 + 16 * vt + 4 * (lane >> 4) + r) * DK + 16 * dt + (lane & 15)] = st[y][r];
    }
}

template <typename K>
hipError_t set_lds(K kernel, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds);
}

template <int DK, int OUT, bool BF16>
hipError_t launch_scan(const PrefillArgs& a, int grid, hipStream_t st) {
    const size_t lds = sizeof(ScanLds<DK>);
    hipError_t e = set_lds(&prefill_scan_kernel<DK, OUT, BF16>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_scan_kernel<DK, OUT, BF16>), dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int DK, bool BF16>
hipError_t launch_dk(const PrefillArgs& a, int out_dtype, int prep_grid, int scan_grid, hipStream_t st) {
    const size_t lds = sizeof(PrepLds<DK>);
    hipError_t e = set_lds(&prefill_prepare_kernel<DK, BF16>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_prepare_kernel<DK, BF16>), dim3(prep_grid), dim3(256), lds, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    switch (out_dtype) {
        case GDN_F32: return launch_scan<DK, 0, BF16>(a, scan_grid, st);
        case GDN_BF16: return launch_scan<DK, 1, BF16>(a, scan_grid, st);
        case GDN_F16: return launch_scan<DK, 2, BF16>(a, scan_grid, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DK>
hipError_t launch_dk_any(const PrefillArgs& a, int out_dtype, int prep_grid, int scan_grid, hipStream_t st) {
    return a.qkv_bf16 ? launch_dk<DK, true>(a, out_dtype, prep_grid, scan_grid, st)
                      : launch_dk<DK, false>(a, out_dtype, prep_grid, scan_grid, st);
}

}  // namespace

size_t prefill_workspace_bytes(int batch, int T, int h_qk, int h_v, int d_k) {
    const int nch = (T + kC - 1) / kC;
    return ws_layout(batch, nch, h_qk, h_v, d_k).total;
}

hipError_t launch_prefill(const PrefillArgs& a, int d_k, int out_dtype, hipStream_t stream) {
    const int nch = (a.T + kC - 1) / kC;
    const long long prep = (long long)a.batch * nch * a.h_v;
    const long long scan = (long long)a.batch * a.h_v * a.slices;
    if (prep > 0x7fffffffLL || scan > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (d_k) {
        case 32: return launch_dk_any<32>(a, out_dtype, (int)prep, (int)scan, stream);
        case 64: return launch_dk_any<64>(a, out_dtype, (int)prep, (int)scan, stream);
        case 128: return launch_dk_any<128>(a, out_dtype, (int)prep, (int)scan, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
