// Backward pass of the chunkwise delta rule, every form: the gate-aware backward
// the Gated DeltaNet-2 abstract pairs with its chunkwise WY forward.  The split-
// gate form (bwd2_*) has its own factor and gradient kernels (below); the two
// state chains are shared, switched by SPLIT.
//
// Per chunk of C = 64 rows with incoming state S [dv, dk] and cumulative
// log-decay G [C, dk] (channel-wise; a scalar decay is broadcast):
//   E[r, j]  = exp(G_r - G_j) per channel, j <= r          (pairwise, never overflows)
//   Abar     = StrictTril(sum_c k_r k_j E),  T = (I + diag(beta) Abar)^-1
//   Khat = k e^G, Qhat = q e^G, Kbar = k e^{G_C - G}, gamma = e^{G_C}
//   W = T diag(beta) Khat,  U = T diag(beta) v,  Mq = Tril0(sum_c q_r k_j E)
//   Vt = U - W S^T,  O = Qhat S^T + Mq Vt,  S_next = S Diag(gamma) + Vt^T Kbar
// The backward is four launches:
//   1. bwd_prep    (one workgroup per chunk) the state-independent factors;
//   2. bwd_fchain  (per head and 32 value rows) the states entering each chunk
//                  and Vt, one chunk after another;
//   3. bwd_rchain  (same split) dS carried backwards: dVt = Mq^T dO + Kbar dS'^T,
//                  dS = dS' Diag(gamma) + dO^T Qhat - dVt^T W;
//   4. bwd_grads   (one workgroup per chunk) every input gradient from the
//                  saved factors, states and dVt.
// Everything is fp32; intermediates live in a workspace with one fixed-size
// record per (batch, head, chunk).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kBC = 64;     // chunk length
constexpr int kBVT = 32;    // value rows per chain workgroup
constexpr int kCW = 8;      // waves per chain workgroup (two per SIMD: one hides the
                            // other's LDS and matrix-core latency)
constexpr int kCT = 64 * kCW;
constexpr int kGT = 512;    // threads of the gradient workgroup
constexpr int kGW = kGT / 64;
constexpr int kRT = kGT / 64;   // its threads per row for row sums

// One 16 x 16 output tile of an fp32 product on the matrix cores:
// acc += A[i0, i0 + 16) x [k0, k1)  *  B[k0, k1) x [j0, j0 + 16), k1 - k0 a multiple
// of 4; A(i, k) and B(k, j) read the operands in whatever layout they have.
// v_mfma_f32_16x16x4f32: lane l supplies A(i0 + l % 16, k + l / 16) and
// B(k + l / 16, j0 + l % 16); element q of the result is row i0 + 4 (l / 16) + q,
// column j0 + l % 16.
template <class FA, class FB>
__device__ __forceinline__ f32x4 mm_tile(f32x4 acc, int i0, int j0, int k0, int k1, const FA& A,
                                         const FB& B) {
    const int l = threadIdx.x & 63;
    const int ai = i0 + (l & 15), bj = j0 + (l & 15), kk = l >> 4;
#pragma unroll 16
    for (int k = k0; k < k1; k += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(ai, k + kk), B(k + kk, bj), acc, 0, 0, 0);
    return acc;
}

// mm_tile with the k range split into two interleaved accumulation chains
// (k1 - k0 a multiple of 8), which the matrix core runs back to back.
template <class FA, class FB>
__device__ __forceinline__ f32x4 mm_tile_k2(f32x4 acc, int i0, int j0, int k0, int k1, const FA& A,
                                            const FB& B) {
    const int l = threadIdx.x & 63;
    const int ai = i0 + (l & 15), bj = j0 + (l & 15), kk = l >> 4;
    f32x4 other = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = k0; k < k1; k += 8) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(ai, k + kk), B(k + kk, bj), acc, 0, 0, 0);
        other = __builtin_amdgcn_mfma_f32_16x16x4f32(A(ai, k + 4 + kk), B(k + 4 + kk, bj), other, 0, 0, 0);
    }
    return acc + other;
}

// Two tiles with the same rows i0 and columns j0, j1: one A read feeds both
// accumulation chains.
template <class FA, class FB>
__device__ __forceinline__ void mm_tile2(f32x4& acc0, f32x4& acc1, int i0, int j0, int j1, int k0, int k1,
                                         const FA& A, const FB& B) {
    const int l = threadIdx.x & 63;
    const int ai = i0 + (l & 15), b0 = j0 + (l & 15), b1 = j1 + (l & 15), kk = l >> 4;
#pragma unroll 16
    for (int k = k0; k < k1; k += 4) {
        const float a = A(ai, k + kk);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, B(k + kk, b0), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, B(k + kk, b1), acc1, 0, 0, 0);
    }
}

// Pairwise sums with a per-channel factor, as products: for the 16 x 16 tile at
// rows r0, channels c0,
//   ROW:  sum_{j <= r} M(r, j) X(j, c) e^{G(r, c) - G(j, c)}
//   !ROW: sum_{j >= r} M(j, r) X(j, c) e^{G(j, c) - G(r, c)}
// (M is zero outside those ranges).  Each 16-row block J of j contributes one
// product over its rows, with e^{...} split at a reference row of J: the last
// row for ROW and the first for !ROW, so that the factor inside the product is
// at most 1 and the one applied afterwards exceeds 1 only within block J (at most
// e^{85} under the decay bound).
template <bool ROW, class FM, class FX, class FG>
__device__ __forceinline__ f32x4 pair_tile(int r0, int c0, const FM& M, const FX& X, const FG& G) {
    const int l = threadIdx.x & 63;
    const int I = r0 / 16;
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    for (int J = ROW ? 0 : I; ROW ? (J <= I) : (J < kBC / 16); ++J) {
        const int ref = ROW ? 16 * J + 15 : 16 * J;
        const f32x4 acc = mm_tile(
            f32x4{0.f, 0.f, 0.f, 0.f}, r0, c0, 16 * J, 16 * J + 16,
            [&](int r, int j) { return ROW ? M(r, j) : M(j, r); },
            [&](int j, int c) { return X(j, c) * __expf(ROW ? G(ref, c) - G(j, c) : G(j, c) - G(ref, c)); });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 4 * (l >> 4) + q, c = c0 + (l & 15);
            out[q] = fmaf(acc[q], __expf(ROW ? G(r, c) - G(ref, c) : G(ref, c) - G(r, c)), out[q]);
        }
    }
    return out;
}

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global loads (the chains keep next-chunk loads in flight across it).
__device__ __forceinline__ void lds_only_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// T = (I + diag(rs) A)^-1 for a strictly lower C x C matrix A (row stride lda;
// rs = nullptr means no row scale).  Called by the 64 lanes of one wave, lane col
// computing column col by forward substitution with the column held in registers
// (fully unrolled), each row's sum split over four independent accumulators.
__device__ __forceinline__ void unit_lower_inverse(const float* A, int lda, const float* rs, float* T,
                                                   int ldt, int col) {
    float t[kBC];
#pragma unroll
    for (int r = 0; r < kBC; ++r) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < r; ++j) acc[j & 3] = fmaf(A[r * lda + j], t[j], acc[j & 3]);
        float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        if (rs) sum *= rs[r];
        t[r] = (r == col ? 1.f : 0.f) - sum;
    }
#pragma unroll
    for (int r = 0; r < kBC; ++r) T[r * ldt + col] = t[r];
}

// Workspace record of one (batch, head, chunk), in floats.
template <int DK, int DV>
struct BwdWs {
    static constexpr int64_t C = kBC;
    static constexpr int64_t oG = 0;                // G            [C][DK]
    static constexpr int64_t oT = oG + C * DK;      // T            [C][C]
    static constexpr int64_t oAb = oT + C * C;      // Abar         [C][C]
    static constexpr int64_t oMq = oAb + C * C;     // Mq           [C][C]
    static constexpr int64_t oW = oMq + C * C;      // W            [C][DK]
    static constexpr int64_t oQh = oW + C * DK;     // Qhat         [C][DK]
    static constexpr int64_t oKb = oQh + C * DK;    // Kbar         [C][DK]
    static constexpr int64_t oKh = oKb + C * DK;    // Khat         [C][DK]
    static constexpr int64_t oU = oKh + C * DK;     // U            [C][DV]
    static constexpr int64_t oGam = oU + C * DV;    // gamma        [DK]
    static constexpr int64_t oS = oGam + DK;        // S entering   [DV][DK]
    static constexpr int64_t odS = oS + DV * DK;    // dS leaving   [DV][DK]
    static constexpr int64_t oVt = odS + DV * DK;   // Vt           [C][DV]
    static constexpr int64_t odVt = oVt + C * DV;   // dVt          [C][DV]
    static constexpr int64_t odW = odVt + C * DV;   // dW           [C][DK]
    static constexpr int64_t odX = odW + C * DK;    // dX           [C][DK]
    static constexpr int64_t odQh = odX + C * DK;   // dQhat, then dG [C][DK]
    static constexpr int64_t odKb = odQh + C * DK;  // dKbar        [C][DK]
    static constexpr int64_t size = odKb + C * DK;
    static constexpr int64_t oEb = oKb;             // (the split-gate chains' Ebar; unused here)
};

// Workspace record of the split-gate form (Gated DeltaNet-2).  The names the
// state chains share with the single-step-size record carry the split-gate
// factors: oU holds Ut, oVt holds Y, odVt holds dY and oMq holds Me.
template <int DK, int DV>
struct BwdWs2 {
    static constexpr int64_t C = kBC;
    static constexpr int64_t oG = 0;                // G        [C][DK]
    static constexpr int64_t oT = oG + C * DK;      // T        [C][C]
    static constexpr int64_t oAk = oT + C * C;      // Ak       [C][C]
    static constexpr int64_t oMq = oAk + C * C;     // Me       [C][C]
    static constexpr int64_t oMk = oMq + C * C;     // Mk       [C][C]
    static constexpr int64_t oW = oMk + C * C;      // W        [C][DK]
    static constexpr int64_t oQh = oW + C * DK;     // Qhat
    static constexpr int64_t oKb = oQh + C * DK;    // Kbar
    static constexpr int64_t oEb = oKb + C * DK;    // Ebar
    static constexpr int64_t oKh = oEb + C * DK;    // Khat
    static constexpr int64_t oZ = oKh + C * DK;     // Z = Ak X [C][DV]
    static constexpr int64_t oU = oZ + C * DV;      // Ut = T Z [C][DV]
    static constexpr int64_t oGam = oU + C * DV;    // gamma    [DK]
    static constexpr int64_t oS = oGam + DK;        // S entering [DV][DK]
    static constexpr int64_t odS = oS + DV * DK;    // dS leaving [DV][DK]
    static constexpr int64_t oVt = odS + DV * DK;   // Y        [C][DV]
    static constexpr int64_t odVt = oVt + C * DV;   // dY       [C][DV]
    static constexpr int64_t odMe = odVt + C * DV;  // scratch: dMe, dMk, dAe, dAk [C][C]
    static constexpr int64_t odMk = odMe + C * C;
    static constexpr int64_t odAe = odMk + C * C;
    static constexpr int64_t odAk = odAe + C * C;
    static constexpr int64_t odW = odAk + C * C;    // dW, dKhat, dQhat (then dG), dKbar, dEbar [C][DK]
    static constexpr int64_t odKh = odW + C * DK;
    static constexpr int64_t odQh = odKh + C * DK;
    static constexpr int64_t odKb = odQh + C * DK;
    static constexpr int64_t odEb = odKb + C * DK;
    static constexpr int64_t odZ = odEb + C * DK;   // dZ       [C][DV]
    static constexpr int64_t size = odZ + C * DV;
};

__device__ __forceinline__ int64_t tok_index(const BwdArgs& p, int b, int t, int h) {
    return (static_cast<int64_t>(b) * p.T + t) * p.H + h;
}
// the query/key row of value head h (groups of H / Hk consecutive value heads)
__device__ __forceinline__ int64_t qk_index(const BwdArgs& p, int b, int t, int h) {
    return (static_cast<int64_t>(b) * p.T + t) * p.Hk + h / (p.H / p.Hk);
}
// dq or dk of value head h at token index vi ([B, T, H] order): straight to the
// output, or to the fp32 per-value-head buffer that is summed over groups later
template <typename E>
__device__ __forceinline__ void store_qk_grad(void* out, float* out32, int64_t vi, int DK, int c, float x) {
    if (out32) out32[vi * DK + c] = x;
    else store_elem<E>(out, vi * DK + c, x);
}

// ---------------------------------------------------------------- 1. factors
template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kGT) void bwd_prep_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs<DK, DV> L;
    constexpr int LD = (DK > DV ? DK : DV) + 4;   // padded row stride (4 mod 64 words)
    __shared__ float sK[kBC * (DK + 4)];
    __shared__ float sX[kBC * LD];                // q, then beta Khat, then beta v
    __shared__ float sG[kBC * (DK + 4)];
    __shared__ float sA[kBC * (kBC + 4)];
    __shared__ float sT[kBC * (kBC + 4)];
    __shared__ float sBeta[kBC];
    const int u = blockIdx.x, tid = threadIdx.x;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;

    for (int e = tid; e < kBC * DK; e += kGT) {
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        const int64_t ti = tok_index(p, b, t0 + min(r, Cn - 1), h);
        const int64_t qi = qk_index(p, b, t0 + min(r, Cn - 1), h);
        sK[r * (DK + 4) + c] = ok ? load_elem<E>(p.k, qi * DK + c) : 0.f;
        sX[r * LD + c] = ok ? load_elem<E>(p.q, qi * DK + c) : 0.f;
        float gv = 0.f;
        if constexpr (VAR == 1) gv = ok ? load_elem<E>(p.g, ti) : 0.f;
        if constexpr (VAR >= 2) gv = ok ? load_elem<E>(p.g, ti * DK + c) : 0.f;
        sG[r * (DK + 4) + c] = gv;
    }
    // FG^2-GDN (VAR 4): the step sizes sit on the key side (E = beta ⊙ k in the
    // columns of Abar and Mq and in Kbar); the rows take 1
    if (tid < kBC) sBeta[tid] = tid < Cn ? (VAR == 4 ? 1.f : load_elem<E>(p.beta, tok_index(p, b, t0 + tid, h))) : 0.f;
    __syncthreads();
    if (tid < DK) {   // in-chunk cumulative log-decay per channel
        float acc = 0.f;
        for (int r = 0; r < kBC; ++r) {
            acc += sG[r * (DK + 4) + tid];
            sG[r * (DK + 4) + tid] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kGT) R[L::oG + e] = sG[(e / DK) * (DK + 4) + e % DK];
    if (tid < DK) R[L::oGam + tid] = __expf(sG[(kBC - 1) * (DK + 4) + tid]);
    // Abar (strictly lower) and Mq (lower, diagonal included)
    const int w = tid >> 6, l = tid & 63;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (VAR >= 2) {
        // a factor per channel: e^{G_r - G_j} = e^{G_r - G_ref} e^{G_ref - G_j} with the
        // reference at the last row of j's 16-row block, folded into the operands of
        // each tile product (at most e^{85} inside one block under the decay bound)
        for (int t = w; t < 16; t += kGW) {
            const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            f32x4 ab = z4, mq = z4;
            if (j0 <= r0) {
                const float* gref = sG + (j0 + 15) * (DK + 4);
                auto Bk = [&](int c, int j) {
                    float x = sK[j * (DK + 4) + c] * __expf(gref[c] - sG[j * (DK + 4) + c]);
                    if constexpr (VAR == 4) x *= load_elem<E>(p.beta, tok_index(p, b, t0 + min(j, Cn - 1), h) * DK + c);
                    return x;
                };
                ab = mm_tile(z4, r0, j0, 0, DK,
                             [&](int r, int c) { return sK[r * (DK + 4) + c] * __expf(sG[r * (DK + 4) + c] - gref[c]); }, Bk);
                mq = mm_tile(z4, r0, j0, 0, DK,
                             [&](int r, int c) { return sX[r * LD + c] * __expf(sG[r * (DK + 4) + c] - gref[c]); }, Bk);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + 4 * (l >> 4) + q, j = j0 + (l & 15);
                const float a_ = j < r ? ab[q] : 0.f;
                sA[r * (kBC + 4) + j] = a_;
                R[L::oAb + r * kBC + j] = a_;
                R[L::oMq + r * kBC + j] = j <= r ? mq[q] : 0.f;
            }
        }
    } else {                    // K K^T and Q K^T on the matrix cores, then e^{G_r - G_j}
        for (int t = w; t < 16; t += kGW) {
            const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            const f32x4 ab = mm_tile(z4, r0, j0, 0, DK, [&](int r, int c) { return sK[r * (DK + 4) + c]; },
                                     [&](int c, int j) { return sK[j * (DK + 4) + c]; });
            const f32x4 mq = mm_tile(z4, r0, j0, 0, DK, [&](int r, int c) { return sX[r * LD + c]; },
                                     [&](int c, int j) { return sK[j * (DK + 4) + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + 4 * (l >> 4) + q, j = j0 + (l & 15);
                const float ex = (VAR == 1 && j <= r) ? __expf(sG[r * (DK + 4)] - sG[j * (DK + 4)]) : 1.f;
                const float a_ = j < r ? ab[q] * ex : 0.f;
                sA[r * (kBC + 4) + j] = a_;
                R[L::oAb + r * kBC + j] = a_;
                R[L::oMq + r * kBC + j] = j <= r ? mq[q] * ex : 0.f;
            }
        }
    }
    __syncthreads();
    // T = (I + diag(beta) Abar)^-1 by forward substitution, one column per thread
    if (tid < kBC) unit_lower_inverse(sA, kBC + 4, sBeta, sT, kBC + 4, tid);
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kGT) R[L::oT + e] = sT[(e / kBC) * (kBC + 4) + e % kBC];
    // key and query factors; sX becomes X = beta Khat
    for (int e = tid; e < kBC * DK; e += kGT) {
        const int r = e / DK, c = e % DK;
        const float G = sG[r * (DK + 4) + c];
        const float eg = __expf(G);
        const float kk = sK[r * (DK + 4) + c];
        R[L::oKh + e] = kk * eg;
        R[L::oQh + e] = sX[r * LD + c] * eg;
        float kb = kk * __expf(sG[(kBC - 1) * (DK + 4) + c] - G);
        if constexpr (VAR == 4) kb *= load_elem<E>(p.beta, tok_index(p, b, t0 + min(r, Cn - 1), h) * DK + c);
        R[L::oKb + e] = kb;
        sX[r * LD + c] = sBeta[r] * kk * eg;
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DK / 16); t += kGW) {   // W = T X
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * (kBC + 4) + j]; },
                                  [&](int j, int c) { return sX[j * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oW + (r0 + 4 * (l >> 4) + q) * DK + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kGT) {   // Y = beta v
        const int r = e / DV, i = e % DV;
        sX[r * LD + i] = r < Cn ? sBeta[r] * load_elem<E>(p.v, tok_index(p, b, t0 + r, h) * DV + i) : 0.f;
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DV / 16); t += kGW) {   // U = T Y
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * (kBC + 4) + j]; },
                                  [&](int j, int i) { return sX[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oU + (r0 + 4 * (l >> 4) + q) * DV + c0 + (l & 15)] = acc[q];
    }
}

// Workgroup -> (head, value tile) of the two chain kernels.  Workgroups are
// dispatched round-robin over the 8 XCDs; the NVT value tiles of one head get
// ids 8 apart, so they run on the same XCD and share its L2 for the chunk
// records they all read (with tiles of one head on different XCDs every tile
// fetched the records from HBM).  The grid is chain_grid(); ids past the last
// head return at once.
__device__ __forceinline__ bool chain_block(const BwdArgs& p, int NVT, int& bh, int& i0) {
    const int x = blockIdx.x, groups = (p.B * p.H + 7) / 8;
    bh = (x % 8) * groups + x / (8 * NVT);
    i0 = ((x / 8) % NVT) * kBVT;
    return bh < p.B * p.H;
}
inline unsigned chain_grid(const BwdArgs& a, int DV) {
    return static_cast<unsigned>((a.B * a.H + 7) / 8) * 8u * static_cast<unsigned>(DV / kBVT);
}

// ------------------------------------------------------ 2. forward state chain
// Single step size:  Vt = U - W S^T,   S = S Diag(gamma) + Vt^T Kbar.
// Split gates:       Y = Ut + W S^T,   S = S Diag(gamma) - Y^T Ebar + X^T Kbar.
template <class L, typename E, int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(kCT) void bwd_fchain_kernel(BwdArgs p, float* ws, int N) {
    constexpr int NVT = DV / kBVT;
    // Row strides against LDS bank conflicts in the matrix-core operand reads:
    // an operand read along its rows by the 16 lanes of a group (sS, sW) takes a
    // stride of 4 mod 64 words; one read down its columns (sKb, sEb, sVt, sXt)
    // takes 16 mod 64, so the four k-rows of one read fall in different banks.
    constexpr int SS = DK + 4, SW = DK + 4, SK = DK + 16, SV = kBVT + 16;
    __shared__ __attribute__((aligned(16))) float sS[kBVT * SS];
    __shared__ __attribute__((aligned(16))) float sVt[kBC * SV];
    __shared__ __attribute__((aligned(16))) float sW[kBC * SW];
    __shared__ __attribute__((aligned(16))) float sKb[kBC * SK];
    __shared__ __attribute__((aligned(16))) float sEb[SPLIT ? kBC * SK : 4];
    __shared__ __attribute__((aligned(16))) float sXt[SPLIT ? kBC * SV : 4];
    __shared__ float sGam[DK];
    const int tid = threadIdx.x;
    int bh, i0;
    if (!chain_block(p, NVT, bh, i0)) return;
    const int b = bh / p.H, h = bh % p.H;
    for (int e = tid; e < kBVT * DK; e += kCT) {
        const int i = e / DK, c = e % DK;
        sS[i * SS + c] = p.S0 ? p.S0[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c] : 0.f;
    }
    // the next chunk's operands are fetched into registers while this chunk's
    // products run, and written to LDS at the top of the next step
    const int w = tid >> 6, l = tid & 63;
    constexpr int NP = kBC * DK / 4 / kCT;          // 16-byte pieces per thread per operand
    constexpr int MT = (kBC / 16) * (kBVT / 16) / kCW;  // Vt tiles per wave
    float4 pW[NP], pK[NP], pE[SPLIT ? NP : 1];
    float pU[MT][4];
    float pG = 0.f;
    auto fetch = [&](int n) {
        const float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            pW[j] = *reinterpret_cast<const float4*>(R + L::oW + idx);
            pK[j] = *reinterpret_cast<const float4*>(R + L::oKb + idx);
            if constexpr (SPLIT) pE[j] = *reinterpret_cast<const float4*>(R + L::oEb + idx);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = w + kCW * m, r0 = 16 * (t / (kBVT / 16)), c0 = 16 * (t % (kBVT / 16));
#pragma unroll
            for (int q = 0; q < 4; ++q) pU[m][q] = R[L::oU + (r0 + 4 * (l >> 4) + q) * DV + i0 + c0 + (l & 15)];
        }
        pG = tid < DK ? R[L::oGam + tid] : 0.f;
    };
    auto put4 = [&](float* dst, int ld, int idx, float4 v) {
        *reinterpret_cast<float4*>(dst + (idx / DK) * ld + idx % DK) = v;
    };
    fetch(0);
    for (int n = 0; n < N; ++n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            put4(sW, SW, idx, pW[j]);
            put4(sKb, SK, idx, pK[j]);
            if constexpr (SPLIT) put4(sEb, SK, idx, pE[j]);
        }
        float uu[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) uu[m][q] = pU[m][q];
        if (tid < DK) sGam[tid] = pG;
        if constexpr (SPLIT) {   // X = w v for this tile's value columns
            const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
            for (int e = tid; e < kBC * kBVT; e += kCT) {
                const int r = e / kBVT, i = e % kBVT;
                float x = 0.f;
                if (r < Cn) {
                    const int64_t vi = tok_index(p, b, t0 + r, h) * DV + i0 + i;
                    x = load_elem<E>(p.wgate, vi) * load_elem<E>(p.v, vi);
                }
                sXt[r * SV + i] = x;
            }
        }
        lds_only_barrier();
        if (n + 1 < N) fetch(n + 1);
        for (int e = tid; e < kBVT * DK; e += kCT) {
            const int i = e / DK, c = e % DK;
            R[L::oS + (i0 + i) * DK + c] = sS[i * SS + c];
        }
        constexpr float sgn = SPLIT ? 1.f : -1.f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {   // Vt = U - W S^T  /  Y = Ut + W S^T
            const int t = w + kCW * m, r0 = 16 * (t / (kBVT / 16)), c0 = 16 * (t % (kBVT / 16));
            const f32x4 acc = mm_tile_k2(f32x4{0.f, 0.f, 0.f, 0.f}, r0, c0, 0, DK,
                                         [&](int r, int c) { return sW[r * SW + c]; },
                                         [&](int c, int i) { return sS[i * SS + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + 4 * (l >> 4) + q, i = c0 + (l & 15);
                const float val = uu[m][q] + sgn * acc[q];
                sVt[r * SV + i] = val;
                R[L::oVt + r * DV + i0 + i] = val;
            }
        }
        lds_only_barrier();
        // S = S Diag(gamma) + Vt^T Kbar  /  - Y^T Ebar + X^T Kbar.  Tile t covers state
        // rows 16 (t % 2), channels 16 (t / 2); with two tiles per wave, t and t + kCW
        // share their rows and run as one pair of chains.
        constexpr int NTS = (kBVT / 16) * (DK / 16);
        static_assert(NTS == kCW || NTS == 2 * kCW, "state tiles per wave");
        {
            const int t = w, ii0 = 16 * (t % (kBVT / 16)), cc0 = 16 * (t / (kBVT / 16));
            const int cc1 = cc0 + 16 * (kCW / (kBVT / 16));
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
            auto vt = [&](int i, int r) { return sVt[r * SV + i]; };
            auto nvt = [&](int i, int r) { return -sVt[r * SV + i]; };
            auto xt = [&](int i, int r) { return sXt[r * SV + i]; };
            auto kb = [&](int r, int c) { return sKb[r * SK + c]; };
            auto eb = [&](int r, int c) { return sEb[r * SK + c]; };
            if constexpr (NTS == 2 * kCW) {
                if constexpr (SPLIT) {
                    mm_tile2(acc0, acc1, ii0, cc0, cc1, 0, kBC, nvt, eb);
                    mm_tile2(acc0, acc1, ii0, cc0, cc1, 0, kBC, xt, kb);
                } else {
                    mm_tile2(acc0, acc1, ii0, cc0, cc1, 0, kBC, vt, kb);
                }
            } else {
                if constexpr (SPLIT) {
                    acc0 = mm_tile_k2(acc0, ii0, cc0, 0, kBC, nvt, eb);
                    acc0 = mm_tile_k2(acc0, ii0, cc0, 0, kBC, xt, kb);
                } else {
                    acc0 = mm_tile_k2(acc0, ii0, cc0, 0, kBC, vt, kb);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ii0 + 4 * (l >> 4) + q, c = cc0 + (l & 15);
                sS[i * SS + c] = fmaf(sS[i * SS + c], sGam[c], acc0[q]);
                if constexpr (NTS == 2 * kCW) {
                    const int c1 = cc1 + (l & 15);
                    sS[i * SS + c1] = fmaf(sS[i * SS + c1], sGam[c1], acc1[q]);
                }
            }
        }
        lds_only_barrier();
    }
}

// ------------------------------------------------------ 3. reverse state chain
// Single step size:  dVt = Mq^T dO + Kbar dS'^T,     dS = dS' Diag(gamma) + dO^T Qhat - dVt^T W.
// Split gates:       dY = -(Me^T dO + Ebar dS'^T),   dS = dS' Diag(gamma) + dO^T Qhat + dY^T W.
template <class L, typename E, int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(kCT) void bwd_rchain_kernel(BwdArgs p, float* ws, int N) {
    constexpr int NVT = DV / kBVT;
    // row strides against bank conflicts (see the forward chain), within the LDS:
    // 4 mod 64 words for operands read along rows (sdS, sA1); 16 mod 64 for dO and
    // dVt, read down columns in both products (conflict-free); 8 mod 64 for the
    // other column-read operands (at most two-way: 16 would not fit in 160 KB)
    constexpr int SD = DK + 4, SA = DK + 4, SB = DK + 8, SO = kBVT + 16, SMQ = kBC + 8;
    __shared__ __attribute__((aligned(16))) float sdS[kBVT * SD];
    __shared__ __attribute__((aligned(16))) float sdVt[kBC * SO];
    __shared__ __attribute__((aligned(16))) float sdO[kBC * SO];
    __shared__ __attribute__((aligned(16))) float sM[kBC * SMQ];
    __shared__ __attribute__((aligned(16))) float sA1[kBC * SA];
    __shared__ __attribute__((aligned(16))) float sA2[kBC * SB];
    __shared__ __attribute__((aligned(16))) float sQh[kBC * SB];
    __shared__ float sGam[DK];
    const int tid = threadIdx.x;
    int bh, i0;
    if (!chain_block(p, NVT, bh, i0)) return;
    const int b = bh / p.H, h = bh % p.H;
    for (int e = tid; e < kBVT * DK; e += kCT) {
        const int i = e / DK, c = e % DK;
        sdS[i * SD + c] = p.dST ? p.dST[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c] : 0.f;
    }
    // the previous chunk's operands are fetched into registers during this step
    constexpr int NP = kBC * DK / 4 / kCT;
    constexpr int NM = kBC * kBC / 4 / kCT;
    constexpr int NO = kBC * kBVT / kCT;
    float4 pM[NM], pA[NP], pQ[NP], pW[NP];
    float pO[NO];
    float pG = 0.f;
    auto fetch = [&](int n) {
        const float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
#pragma unroll
        for (int j = 0; j < NM; ++j) pM[j] = *reinterpret_cast<const float4*>(R + L::oMq + 4 * (tid + kCT * j));
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            pA[j] = *reinterpret_cast<const float4*>(R + (SPLIT ? L::oEb : L::oKb) + idx);
            pQ[j] = *reinterpret_cast<const float4*>(R + L::oQh + idx);
            pW[j] = *reinterpret_cast<const float4*>(R + L::oW + idx);
        }
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int e = tid + kCT * j, r = e / kBVT, i = e % kBVT;
            pO[j] = r < Cn ? load_elem<E>(p.dO, tok_index(p, b, t0 + r, h) * DV + i0 + i) : 0.f;
        }
        pG = tid < DK ? R[L::oGam + tid] : 0.f;
    };
    auto put4 = [&](float* dst, int idx, int ld, int row, float4 v) {
        *reinterpret_cast<float4*>(dst + (idx / row) * ld + idx % row) = v;
    };
    fetch(N - 1);
    for (int n = N - 1; n >= 0; --n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
#pragma unroll
        for (int j = 0; j < NM; ++j) put4(sM, 4 * (tid + kCT * j), SMQ, kBC, pM[j]);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            put4(sA1, idx, SA, DK, pA[j]);
            put4(sQh, idx, SB, DK, pQ[j]);
            put4(sA2, idx, SB, DK, pW[j]);
        }
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int e = tid + kCT * j;
            sdO[(e / kBVT) * SO + e % kBVT] = pO[j];
        }
        if (tid < DK) sGam[tid] = pG;
        lds_only_barrier();
        if (n > 0) fetch(n - 1);
        for (int e = tid; e < kBVT * DK; e += kCT) {
            const int i = e / DK, c = e % DK;
            R[L::odS + (i0 + i) * DK + c] = sdS[i * SD + c];
        }
        const int w = tid >> 6, l = tid & 63;
        for (int t = w; t < (kBC / 16) * (kBVT / 16); t += kCW) {   // dVt = Mq^T dO + Kbar dS^T
            const int r0 = 16 * (t / (kBVT / 16)), c0 = 16 * (t % (kBVT / 16));
            f32x4 acc = mm_tile_k2(f32x4{0.f, 0.f, 0.f, 0.f}, r0, c0, 0, kBC,
                                   [&](int r, int m) { return sM[m * SMQ + r]; },
                                   [&](int m, int i) { return sdO[m * SO + i]; });
            acc = mm_tile_k2(acc, r0, c0, 0, DK, [&](int r, int c) { return sA1[r * SA + c]; },
                             [&](int c, int i) { return sdS[i * SD + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + 4 * (l >> 4) + q, i = c0 + (l & 15);
                const float val = SPLIT ? -acc[q] : acc[q];
                sdVt[r * SO + i] = val;
                R[L::odVt + r * DV + i0 + i] = val;
            }
        }
        lds_only_barrier();
        // dS = dS Diag(gamma) + dO^T Qhat -/+ dVt^T W, tiles paired as in the forward chain
        constexpr int NTS = (kBVT / 16) * (DK / 16);
        static_assert(NTS == kCW || NTS == 2 * kCW, "state tiles per wave");
        {
            const int t = w, ii0 = 16 * (t % (kBVT / 16)), cc0 = 16 * (t / (kBVT / 16));
            const int cc1 = cc0 + 16 * (kCW / (kBVT / 16));
            auto dot = [&](int i, int r) { return sdO[r * SO + i]; };
            auto qh = [&](int r, int c) { return sQh[r * SB + c]; };
            auto dvt = [&](int i, int r) { return (SPLIT ? 1.f : -1.f) * sdVt[r * SO + i]; };
            auto wm = [&](int r, int c) { return sA2[r * SB + c]; };
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
            if constexpr (NTS == 2 * kCW) {
                mm_tile2(acc0, acc1, ii0, cc0, cc1, 0, kBC, dot, qh);
                mm_tile2(acc0, acc1, ii0, cc0, cc1, 0, kBC, dvt, wm);
            } else {
                acc0 = mm_tile_k2(acc0, ii0, cc0, 0, kBC, dot, qh);
                acc0 = mm_tile_k2(acc0, ii0, cc0, 0, kBC, dvt, wm);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ii0 + 4 * (l >> 4) + q, c = cc0 + (l & 15);
                sdS[i * SD + c] = fmaf(sdS[i * SD + c], sGam[c], acc0[q]);
                if constexpr (NTS == 2 * kCW) {
                    const int c1 = cc1 + (l & 15);
                    sdS[i * SD + c1] = fmaf(sdS[i * SD + c1], sGam[c1], acc1[q]);
                }
            }
        }
        lds_only_barrier();
    }
    if (p.gS0) {
        for (int e = tid; e < kBVT * DK; e += kCT) {
            const int i = e / DK, c = e % DK;
            p.gS0[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c] = sdS[i * SD + c];
        }
    }
}

// ------------------------------------------------------------ 4. gradients
// Products run on the matrix cores as 16 x 16 tiles spread over the eight waves;
// the per-element pairwise sums of the channel-wise decay stay on the VALU.
template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kGT) void bwd_grads_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs<DK, DV> L;
    constexpr int CP = kBC + 4;
    constexpr int LD = (DK > DV ? DK : DV) + 4;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;   // region size
    constexpr int QR = 32;            // rows of S (or dS') staged at a time
    static_assert(QR * (DK + 4) <= kBC * CP, "S quarter must fit the second C x C buffer");
    __shared__ float sM1[kBC * CP];   // dMq (then dMq E)
    __shared__ float sM2[kBC * CP];   // S quarters; dT; dA; dAbar (then dAbar E)
    __shared__ float sR[3 * RS];      // three staging regions
    __shared__ float sBeta[kBC];
    __shared__ float sCol[2 * DK];    // column terms of the last row of dG
    __shared__ float sPart[kGT];      // per-thread partial column sums
    float* R0 = sR;
    float* R1 = sR + RS;
    float* R2 = sR + 2 * RS;
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // element q of a tile at (i0, j0) in this lane
    auto ti = [&](int i0, int q) { return i0 + 4 * (l >> 4) + q; };
    auto tj = [&](int j0) { return j0 + (l & 15); };
    constexpr int TCD = (kBC / 16) * (DK / 16);   // C x DK tiles
    constexpr int TCV = (kBC / 16) * (DV / 16);   // C x DV tiles
    constexpr int TCC = (kBC / 16) * (kBC / 16);  // C x C tiles

    if (tid < kBC) sBeta[tid] = tid < Cn ? (VAR == 4 ? 1.f : load_elem<E>(p.beta, tix(tid))) : 0.f;
    for (int e = tid; e < kBC * DV; e += kGT) {   // dO -> R0, Vt -> R1, dVt -> R2
        const int r = e / DV, i = e % DV;
        R0[r * LD + i] = r < Cn ? load_elem<E>(p.dO, tix(r) * DV + i) : 0.f;
        R1[r * LD + i] = R[L::oVt + e];
        R2[r * LD + i] = R[L::odVt + e];
    }
    constexpr int TPC = kGT / DK;   // threads per column for column sums
    {   // sum_i S dS' per column, TPC partial sums combined in a fixed order
        const int c = tid % DK, part = tid / DK;
        float acc = 0.f;
#pragma unroll 16
        for (int i = part * (DV / TPC); i < (part + 1) * (DV / TPC); ++i)
            acc = fmaf(R[L::oS + i * DK + c], R[L::odS + i * DK + c], acc);
        sPart[tid] = acc;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int part = 0; part < TPC; ++part) acc += sPart[part * DK + tid];
        sCol[tid] = R[L::oGam + tid] * acc;
    }
    for (int t = w; t < TCC; t += kGW) {            // dMq = Tril0(dO Vt^T)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 acc = mm_tile(z4, r0, j0, 0, DV, [&](int r, int i) { return R0[r * LD + i]; },
                                  [&](int i, int j) { return R1[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), j = tj(j0);
            sM1[r * CP + j] = j <= r ? acc[q] : 0.f;
        }
    }
    {   // dQhat = dO S, dW = -dVt S, then dKbar = Vt dS', with S and dS' staged by rows
        constexpr int MT = TCD / kGW;   // tiles per wave
        f32x4 aq[MT], aw[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) aq[m] = aw[m] = z4;
        // row blocks of S, then of dS', double-buffered through registers: the next
        // block's loads are in flight while the current block's products run
        constexpr int NPF = QR * DK / kGT;
        float pf[NPF];
        auto fetch_rows = [&](int64_t src, int i0) {
#pragma unroll
            for (int j = 0; j < NPF; ++j) pf[j] = R[src + i0 * DK + tid + kGT * j];
        };
        fetch_rows(L::oS, 0);
        for (int pass = 0; pass < 2; ++pass) {
            for (int i0 = 0; i0 < DV; i0 += QR) {
                __syncthreads();
#pragma unroll
                for (int j = 0; j < NPF; ++j) {
                    const int e = tid + kGT * j;
                    sM2[(e / DK) * (DK + 4) + e % DK] = pf[j];
                }
                __syncthreads();
                if (i0 + QR < DV) fetch_rows(pass == 0 ? L::oS : L::odS, i0 + QR);
                else if (pass == 0) fetch_rows(L::odS, 0);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                    auto Bs = [&](int i, int c) { return sM2[(i - i0) * (DK + 4) + c]; };
                    if (pass == 0) {
                        aq[m] = mm_tile(aq[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R0[r * LD + i]; }, Bs);
                        aw[m] = mm_tile(aw[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return -R2[r * LD + i]; }, Bs);
                    } else {
                        aq[m] = mm_tile(aq[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R1[r * LD + i]; }, Bs);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = ti(r0, q), c = tj(c0);
                    if (pass == 0) {
                        R[L::odQh + r * DK + c] = aq[m][q];
                        R[L::odW + r * DK + c] = aw[m][q];
                    } else {
                        R[L::odKb + r * DK + c] = aq[m][q];
                    }
                }
                aq[m] = z4;
            }
        }
    }
    __syncthreads();
    {   // sum_r dKbar Kbar per column
        const int c = tid % DK, part = tid / DK;
        float acc = 0.f;
#pragma unroll 16
        for (int r = part * (kBC / TPC); r < (part + 1) * (kBC / TPC); ++r)
            acc = fmaf(R[L::odKb + r * DK + c], R[L::oKb + r * DK + c], acc);
        sPart[tid] = acc;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int part = 0; part < TPC; ++part) acc += sPart[part * DK + tid];
        sCol[DK + tid] = acc;
    }
    // dT = dW X^T + dVt Y^T with X = beta Khat, Y = beta v
    for (int e = tid; e < kBC * DK; e += kGT) {   // dW -> R0, X -> R1
        const int r = e / DK, c = e % DK;
        R0[r * LD + c] = R[L::odW + e];
        R1[r * LD + c] = sBeta[r] * R[L::oKh + e];
    }
    __syncthreads();
    f32x4 adt[TCC / kGW];
#pragma unroll
    for (int m = 0; m < TCC / kGW; ++m) {
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        adt[m] = mm_tile(z4, r0, j0, 0, DK, [&](int r, int c) { return R0[r * LD + c]; },
                         [&](int c, int j) { return R1[j * LD + c]; });
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kGT) {   // Y -> R1
        const int r = e / DV, i = e % DV;
        R1[r * LD + i] = r < Cn ? sBeta[r] * load_elem<E>(p.v, tix(r) * DV + i) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < TCC / kGW; ++m) {
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        adt[m] = mm_tile(adt[m], r0, j0, 0, DV, [&](int r, int i) { return R2[r * LD + i]; },
                         [&](int i, int j) { return R1[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) sM2[ti(r0, q) * CP + tj(j0)] = adt[m][q];
    }
    __syncthreads();
    // dA = -T^T dT T^T (strictly lower); T -> R1[0 .. C*CP), tmp -> R1[C*CP ..)
    float* sT = R1;
    float* sTmp = R1 + kBC * CP;
    for (int e = tid; e < kBC * kBC; e += kGT) sT[(e / kBC) * CP + e % kBC] = R[L::oT + e];
    __syncthreads();
    for (int t = w; t < TCC; t += kGW) {            // tmp = dT T^T
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 acc = mm_tile(z4, r0, j0, 0, kBC, [&](int r, int m) { return sM2[r * CP + m]; },
                                  [&](int m, int j) { return sT[j * CP + m]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) sTmp[ti(r0, q) * CP + tj(j0)] = acc[q];
    }
    __syncthreads();
    for (int t = w; t < TCC; t += kGW) {            // dA = -T^T tmp, masked
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 acc = mm_tile(z4, r0, j0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                  [&](int m, int j) { return sTmp[m * CP + j]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), j = tj(j0);
            sM2[r * CP + j] = j < r ? -acc[q] : 0.f;
        }
    }
    for (int t = w; t < TCD; t += kGW) {            // dX = T^T dW (dKhat = beta dX)
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                  [&](int m, int c) { return R0[m * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::odX + ti(r0, q) * DK + tj(c0)] = acc[q];
    }
    __syncthreads();
    for (int t = w; t < TCV; t += kGW) {            // dY = T^T dVt -> dv = beta dY; dY -> R0
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                  [&](int m, int i) { return R2[m * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), i = tj(c0);
            R0[r * LD + i] = acc[q];
            if (r < Cn) store_elem<E>(p.gv, tix(r) * DV + i, sBeta[r] * acc[q]);
        }
    }
    __syncthreads();
    if constexpr (VAR != 4) {   // dbeta: kRT threads per row, fixed-order sums
        const int r = tid / kRT, qt = tid % kRT;
        float db = 0.f;
        for (int c = qt * (DK / kRT); c < (qt + 1) * (DK / kRT); ++c)
            db = fmaf(R[L::odX + r * DK + c], R[L::oKh + r * DK + c], db);
        if (r < Cn)
            for (int i = qt * (DV / kRT); i < (qt + 1) * (DV / kRT); ++i)
                db = fmaf(R0[r * LD + i], load_elem<E>(p.v, tix(r) * DV + i), db);
        for (int j = qt * (kBC / kRT); j < (qt + 1) * (kBC / kRT); ++j)
            db = fmaf(sM2[r * CP + j], R[L::oAb + r * kBC + j], db);
#pragma unroll
        for (int m = 1; m < kRT; m <<= 1) db += __shfl_xor(db, m);
        if (qt == 0 && r < Cn) store_elem<E>(p.gbeta, tix(r), db);
    }
    __syncthreads();
    // q, k, G -> R0, R1, R2; dAbar = beta dA
    for (int e = tid; e < kBC * kBC; e += kGT) sM2[(e / kBC) * CP + e % kBC] *= sBeta[e / kBC];
    for (int e = tid; e < kBC * DK; e += kGT) {
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        R0[r * LD + c] = ok ? load_elem<E>(p.q, qk_index(p, b, t0 + r, h) * DK + c) : 0.f;
        R1[r * LD + c] = ok ? load_elem<E>(p.k, qk_index(p, b, t0 + r, h) * DK + c) : 0.f;
        R2[r * LD + c] = R[L::oG + e];
    }
    __syncthreads();
    // a1 = sum_{j<=r} dMq[r,j] k_j E,  a2 = sum_{j>=r} dMq[j,r] q_j E,
    // a3 = sum_{j<r} dAbar[r,j] k_j E,  a4 = sum_{j>r} dAbar[j,r] k_j E,  E = e^{G_r - G_j} (row r >= j)
    // the workspace terms of a tile's four elements are loaded before its products
    struct Pre {
        float dQh[4], dX[4], dKb[4];
    };
    auto preload = [&](int r0, int c0) {
        Pre pr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = ti(r0, q) * DK + tj(c0);
            pr.dQh[q] = R[L::odQh + e];
            pr.dX[q] = R[L::odX + e];
            pr.dKb[q] = R[L::odKb + e];
        }
        return pr;
    };
    auto finish = [&](int r, int c, float a1, float a2, float a3, float a4, float dQh, float dX_,
                      float dKb) {
        const float Gr = R2[r * LD + c];
        const float qr = R0[r * LD + c], kr = R1[r * LD + c];
        const float eg = (VAR == 0) ? 1.f : __expf(Gr);
        const float ebar = (VAR == 0) ? 1.f : __expf(R2[(kBC - 1) * LD + c] - Gr);
        const int e = r * DK + c;
        const float dKh = sBeta[r] * dX_;
        if (r < Cn) {
            store_qk_grad<E>(p.gq, p.gq32, tix(r), DK, c, fmaf(dQh, eg, a1));
            store_qk_grad<E>(p.gk, p.gk32, tix(r), DK, c, a2 + a3 + a4 + dKh * eg + dKb * ebar);
        }
        R[L::odQh + e] = qr * a1 - kr * a2 + kr * a3 - kr * a4 + dKh * kr * eg + dQh * qr * eg
                         - dKb * kr * ebar;
    };
    if constexpr (VAR == 4) {
        // FG^2-GDN: the key is k on the row side (Khat, the rows of Abar) and
        // e = beta ⊙ k on the column side (the columns of Abar and Mq, Kbar).
        // a2 and a4 (sums over the column index) are gradients of e; a1 and a3
        // take e as their operand.  Pass 1 forms a2 + a4 with q and k in R0, R1;
        // R1 then becomes e for pass 2.
        auto Gf = [&](int r, int c) { return R2[r * LD + c]; };
        auto M1 = [&](int r, int j) { return sM1[r * CP + j]; };
        auto M2 = [&](int r, int j) { return sM2[r * CP + j]; };
        auto Qf = [&](int j, int c) { return R0[j * LD + c]; };
        auto Kf = [&](int j, int c) { return R1[j * LD + c]; };
        constexpr int MTG = TCD / kGW;
        static_assert(TCD % kGW == 0, "tiles per wave");
        f32x4 colg[MTG];
#pragma unroll
        for (int m = 0; m < MTG; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            colg[m] = pair_tile<false>(r0, c0, M1, Qf, Gf) + pair_tile<false>(r0, c0, M2, Kf, Gf);
        }
        __syncthreads();
        for (int e = tid; e < kBC * DK; e += kGT) {
            const int r = e / DK, c = e % DK;
            R1[r * LD + c] *= r < Cn ? load_elem<E>(p.beta, tix(r) * DK + c) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MTG; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            const Pre pr = preload(r0, c0);
            const f32x4 a1 = pair_tile<true>(r0, c0, M1, Kf, Gf);
            const f32x4 a3 = pair_tile<true>(r0, c0, M2, Kf, Gf);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ti(r0, q), c = tj(c0);
                const float Gr = R2[r * LD + c];
                const float qr = R0[r * LD + c], er = R1[r * LD + c];
                const bool ok = r < Cn;
                const float kr = ok ? load_elem<E>(p.k, qk_index(p, b, t0 + r, h) * DK + c) : 0.f;
                const float br = ok ? load_elem<E>(p.beta, tix(r) * DK + c) : 0.f;
                const float eg = __expf(Gr), ebar = __expf(R2[(kBC - 1) * LD + c] - Gr);
                const float dKh = pr.dX[q];                     // rows carry beta = 1
                const float dE = colg[m][q] + pr.dKb[q] * ebar;  // gradient of e_r
                if (ok) {
                    store_qk_grad<E>(p.gq, p.gq32, tix(r), DK, c, fmaf(pr.dQh[q], eg, a1[q]));
                    store_qk_grad<E>(p.gk, p.gk32, tix(r), DK, c, a3[q] + dKh * eg + br * dE);
                    store_elem<E>(p.gbeta, tix(r) * DK + c, kr * dE);
                }
                R[L::odQh + r * DK + c] = qr * a1[q] - er * colg[m][q] + kr * a3[q] + dKh * kr * eg +
                                          pr.dQh[q] * qr * eg - pr.dKb[q] * er * ebar;
            }
        }
    } else if constexpr (VAR == 2) {
        auto Gf = [&](int r, int c) { return R2[r * LD + c]; };
        auto M1 = [&](int r, int j) { return sM1[r * CP + j]; };
        auto M2 = [&](int r, int j) { return sM2[r * CP + j]; };
        auto Qf = [&](int j, int c) { return R0[j * LD + c]; };
        auto Kf = [&](int j, int c) { return R1[j * LD + c]; };
        for (int t = w; t < TCD; t += kGW) {
            const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            const Pre pr = preload(r0, c0);
            const f32x4 a1 = pair_tile<true>(r0, c0, M1, Kf, Gf);
            const f32x4 a2 = pair_tile<false>(r0, c0, M1, Qf, Gf);
            const f32x4 a3 = pair_tile<true>(r0, c0, M2, Kf, Gf);
            const f32x4 a4 = pair_tile<false>(r0, c0, M2, Kf, Gf);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                finish(ti(r0, q), tj(c0), a1[q], a2[q], a3[q], a4[q], pr.dQh[q], pr.dX[q], pr.dKb[q]);
        }
    } else {
        // the decay factor is one number per (r, j): fold it into dMq and dAbar and
        // take the four sums as products
        if constexpr (VAR == 1) {
            for (int e = tid; e < kBC * kBC; e += kGT) {
                const int r = e / kBC, j = e % kBC;
                if (j <= r) {
                    const float ex = __expf(R2[r * LD] - R2[j * LD]);
                    sM1[r * CP + j] *= ex;
                    sM2[r * CP + j] *= ex;
                }
            }
            __syncthreads();
        }
        for (int t = w; t < TCD; t += kGW) {
            const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            const Pre pr = preload(r0, c0);
            const f32x4 a1 = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM1[r * CP + j]; },
                                     [&](int j, int c) { return R1[j * LD + c]; });
            const f32x4 a2 = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM1[j * CP + r]; },
                                     [&](int j, int c) { return R0[j * LD + c]; });
            const f32x4 a3 = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM2[r * CP + j]; },
                                     [&](int j, int c) { return R1[j * LD + c]; });
            const f32x4 a4 = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM2[j * CP + r]; },
                                     [&](int j, int c) { return R1[j * LD + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q)
                finish(ti(r0, q), tj(c0), a1[q], a2[q], a3[q], a4[q], pr.dQh[q], pr.dX[q], pr.dKb[q]);
        }
    }
    if constexpr (VAR != 0) {
        __syncthreads();
        if (tid < DK) {   // reverse cumulative sum over rows; G_C's terms enter at the last row
            const int c = tid;
            float dgv[kBC];
#pragma unroll
            for (int r = 0; r < kBC; ++r) dgv[r] = R[L::odQh + r * DK + c];
            float acc = sCol[c] + sCol[DK + c];
#pragma unroll
            for (int r = kBC - 1; r >= 0; --r) {
                acc += dgv[r];
                if constexpr (VAR >= 2) {
                    if (r < Cn) store_elem<E>(p.gg, tix(r) * DK + c, acc);
                } else {
                    R[L::odQh + r * DK + c] = acc;
                }
            }
        }
        if constexpr (VAR == 1) {   // scalar decay: sum over channels, 4 threads per row
            __syncthreads();
            const int r = tid / kRT, qt = tid % kRT;
            float s = 0.f;
            for (int c = qt * (DK / kRT); c < (qt + 1) * (DK / kRT); ++c) s += R[L::odQh + r * DK + c];
#pragma unroll
            for (int m = 1; m < kRT; m <<= 1) s += __shfl_xor(s, m);
            if (qt == 0 && r < Cn) store_elem<E>(p.gg, tix(r), s);
        }
    }
}

// --------------------------------------------- split gates: 1. factors
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kGT) void bwd2_prep_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs2<DK, DV> L;
    constexpr int LD = (DK > DV ? DK : DV) + 4;
    constexpr int CP = kBC + 4;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;
    __shared__ float sK[kBC * (DK + 4)];
    __shared__ float sG[kBC * (DK + 4)];
    __shared__ float sR1[RS];
    __shared__ float sR2[RS];
    __shared__ float sM[kBC * CP];
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };

    for (int e = tid; e < kBC * DK; e += kGT) {   // k, b k, g
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        const float kk = ok ? load_elem<E>(p.k, qk_index(p, b, t0 + r, h) * DK + c) : 0.f;
        sK[r * (DK + 4) + c] = kk;
        sR1[r * LD + c] = ok ? load_elem<E>(p.beta, tix(r) * DK + c) * kk : 0.f;
        sG[r * (DK + 4) + c] = ok ? load_elem<E>(p.g, tix(r) * DK + c) : 0.f;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < kBC; ++r) {
            acc += sG[r * (DK + 4) + tid];
            sG[r * (DK + 4) + tid] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kGT) R[L::oG + e] = sG[(e / DK) * (DK + 4) + e % DK];
    if (tid < DK) R[L::oGam + tid] = __expf(sG[(kBC - 1) * (DK + 4) + tid]);
    // pairwise factors with the reference at the last row of j's 16-row block
    auto aexp = [&](int r, int c, const float* gref) { return __expf(sG[r * (DK + 4) + c] - gref[c]); };
    auto bexp = [&](int j, int c, const float* gref) { return __expf(gref[c] - sG[j * (DK + 4) + c]); };
    for (int t = w; t < 16; t += kGW) {           // Ae -> sM, Ak -> workspace (strictly lower)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        f32x4 ae = z4, ak = z4;
        if (j0 <= r0) {
            const float* gref = sG + (j0 + 15) * (DK + 4);
            auto Ak_ = [&](int r, int c) { return sK[r * (DK + 4) + c] * aexp(r, c, gref); };
            ae = mm_tile(z4, r0, j0, 0, DK, Ak_, [&](int c, int j) { return sR1[j * LD + c] * bexp(j, c, gref); });
            ak = mm_tile(z4, r0, j0, 0, DK, Ak_, [&](int c, int j) { return sK[j * (DK + 4) + c] * bexp(j, c, gref); });
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 4 * (l >> 4) + q, j = j0 + (l & 15);
            sM[r * CP + j] = j < r ? ae[q] : 0.f;
            R[L::oAk + r * kBC + j] = j < r ? ak[q] : 0.f;
        }
    }
    __syncthreads();
    float* sT = sR2;
    if (tid < kBC) unit_lower_inverse(sM, CP, nullptr, sT, CP, tid);   // T = (I + Ae)^-1
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kGT) R[L::oT + e] = sT[(e / kBC) * CP + e % kBC];
    for (int e = tid; e < kBC * DK; e += kGT) {   // Ebar, Kbar, Khat; Khat -> sR1
        const int r = e / DK, c = e % DK;
        const float G = sG[r * (DK + 4) + c];
        const float eg = __expf(G), eb = __expf(sG[(kBC - 1) * (DK + 4) + c] - G);
        const float kk = sK[r * (DK + 4) + c];
        R[L::oEb + e] = sR1[r * LD + c] * eb;
        R[L::oKb + e] = kk * eb;
        R[L::oKh + e] = kk * eg;
        sR1[r * LD + c] = kk * eg;
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DK / 16); t += kGW) {   // W = T Khat
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * CP + j]; },
                                  [&](int j, int c) { return sR1[j * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oW + (r0 + 4 * (l >> 4) + q) * DK + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kGT) {   // X = w v -> sR1
        const int r = e / DV, i = e % DV;
        float x = 0.f;
        if (r < Cn) x = load_elem<E>(p.wgate, tix(r) * DV + i) * load_elem<E>(p.v, tix(r) * DV + i);
        sR1[r * LD + i] = x;
    }
    for (int e = tid; e < kBC * kBC; e += kGT) sM[(e / kBC) * CP + e % kBC] = R[L::oAk + e];
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DV / 16); t += kGW) {   // Z = Ak X
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM[r * CP + j]; },
                                  [&](int j, int i) { return sR1[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oZ + (r0 + 4 * (l >> 4) + q) * DV + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DV / 16); t += kGW) {   // Ut = T Z
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * CP + j]; },
                                  [&](int j, int i) { return R[L::oZ + j * DV + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oU + (r0 + 4 * (l >> 4) + q) * DV + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kGT) {   // q -> sR1, b k -> sR2, Qhat
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        const float qq = ok ? load_elem<E>(p.q, qk_index(p, b, t0 + r, h) * DK + c) : 0.f;
        sR1[r * LD + c] = qq;
        sR2[r * LD + c] = ok ? load_elem<E>(p.beta, tix(r) * DK + c) * sK[r * (DK + 4) + c] : 0.f;
        R[L::oQh + e] = qq * __expf(sG[r * (DK + 4) + c]);
    }
    __syncthreads();
    for (int t = w; t < 16; t += kGW) {           // Me, Mk (lower, diagonal included)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        f32x4 me = z4, mk = z4;
        if (j0 <= r0) {
            const float* gref = sG + (j0 + 15) * (DK + 4);
            auto Aq = [&](int r, int c) { return sR1[r * LD + c] * aexp(r, c, gref); };
            me = mm_tile(z4, r0, j0, 0, DK, Aq, [&](int c, int j) { return sR2[j * LD + c] * bexp(j, c, gref); });
            mk = mm_tile(z4, r0, j0, 0, DK, Aq, [&](int c, int j) { return sK[j * (DK + 4) + c] * bexp(j, c, gref); });
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 4 * (l >> 4) + q, j = j0 + (l & 15);
            R[L::oMq + r * kBC + j] = j <= r ? me[q] : 0.f;
            R[L::oMk + r * kBC + j] = j <= r ? mk[q] : 0.f;
        }
    }
}

// ------------------------------------------ split gates: 4. gradients
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kGT) void bwd2_grads_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs2<DK, DV> L;
    constexpr int CP = kBC + 4;
    constexpr int LD = (DK > DV ? DK : DV) + 4;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;
    constexpr int QR = 32;
    constexpr int TPC = kGT / DK;
    constexpr int TCD = (kBC / 16) * (DK / 16);
    constexpr int TCV = (kBC / 16) * (DV / 16);
    constexpr int TCC = (kBC / 16) * (kBC / 16);
    constexpr int MT = TCD / kGW;
    __shared__ float sM1[kBC * CP];
    __shared__ float sM2[kBC * CP];
    __shared__ float sR[3 * RS];
    __shared__ float sCol[2 * DK];
    __shared__ float sPart[kGT];
    float* R0 = sR;
    float* R1 = sR + RS;
    float* R2 = sR + 2 * RS;
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    auto ti = [&](int i0, int q) { return i0 + 4 * (l >> 4) + q; };
    auto tj = [&](int j0) { return j0 + (l & 15); };
    auto xval = [&](int r, int i) {   // X = w v (zero past the sequence)
        if (r >= Cn) return 0.f;
        const int64_t vi = tix(r) * DV + i;
        return load_elem<E>(p.wgate, vi) * load_elem<E>(p.v, vi);
    };
    // stage rows [i0, i0 + QR) of a [DV][DK] workspace matrix into sM2
    // row blocks of a [DV][DK] workspace matrix, double-buffered through registers:
    // fetch_rows issues the loads, put_rows writes them to sM2 (after a barrier)
    constexpr int NPF = QR * DK / kGT;
    float pf[NPF];
    auto fetch_rows = [&](int64_t src, int i0) {
#pragma unroll
        for (int j = 0; j < NPF; ++j) pf[j] = R[src + i0 * DK + tid + kGT * j];
    };
    auto put_rows = [&]() {
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int e = tid + kGT * j;
            sM2[(e / DK) * (DK + 4) + e % DK] = pf[j];
        }
    };

    for (int e = tid; e < kBC * DV; e += kGT) {   // dO -> R0, Y -> R1, X -> R2
        const int r = e / DV, i = e % DV;
        R0[r * LD + i] = r < Cn ? load_elem<E>(p.dO, tix(r) * DV + i) : 0.f;
        R1[r * LD + i] = R[L::oVt + e];
        R2[r * LD + i] = xval(r, i);
    }
    {   // sum_i S dS' per column
        const int c = tid % DK, part = tid / DK;
        float acc = 0.f;
#pragma unroll 16
        for (int i = part * (DV / TPC); i < (part + 1) * (DV / TPC); ++i)
            acc = fmaf(R[L::oS + i * DK + c], R[L::odS + i * DK + c], acc);
        sPart[tid] = acc;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int part = 0; part < TPC; ++part) acc += sPart[part * DK + tid];
        sCol[tid] = R[L::oGam + tid] * acc;
    }
    for (int t = w; t < TCC; t += kGW) {          // dMe = -Tril0(dO Y^T), dMk = Tril0(dO X^T)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 me = mm_tile(z4, r0, j0, 0, DV, [&](int r, int i) { return R0[r * LD + i]; },
                                 [&](int i, int j) { return R1[j * LD + i]; });
        const f32x4 mk = mm_tile(z4, r0, j0, 0, DV, [&](int r, int i) { return R0[r * LD + i]; },
                                 [&](int i, int j) { return R2[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), j = tj(j0);
            R[L::odMe + r * kBC + j] = j <= r ? -me[q] : 0.f;
            R[L::odMk + r * kBC + j] = j <= r ? mk[q] : 0.f;
        }
    }
    {   // dQhat = dO S; then dEbar = -Y dS', dKbar = X dS'
        f32x4 a1[MT], a2[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) a1[m] = a2[m] = z4;
        fetch_rows(L::oS, 0);
        for (int i0 = 0; i0 < DV; i0 += QR) {
            __syncthreads();
            put_rows();
            __syncthreads();
            fetch_rows(i0 + QR < DV ? L::oS : L::odS, i0 + QR < DV ? i0 + QR : 0);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                a1[m] = mm_tile(a1[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R0[r * LD + i]; },
                                [&](int i, int c) { return sM2[(i - i0) * (DK + 4) + c]; });
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
            for (int q = 0; q < 4; ++q) R[L::odQh + ti(r0, q) * DK + tj(c0)] = a1[m][q];
            a1[m] = z4;
        }
        for (int i0 = 0; i0 < DV; i0 += QR) {
            __syncthreads();
            put_rows();
            __syncthreads();
            if (i0 + QR < DV) fetch_rows(L::odS, i0 + QR);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                auto Bs = [&](int i, int c) { return sM2[(i - i0) * (DK + 4) + c]; };
                a1[m] = mm_tile(a1[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return -R1[r * LD + i]; }, Bs);
                a2[m] = mm_tile(a2[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R2[r * LD + i]; }, Bs);
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                R[L::odEb + ti(r0, q) * DK + tj(c0)] = a1[m][q];
                R[L::odKb + ti(r0, q) * DK + tj(c0)] = a2[m][q];
            }
        }
    }
    __syncthreads();
    {   // sum_r (dKbar Kbar + dEbar Ebar) per column
        const int c = tid % DK, part = tid / DK;
        float acc = 0.f;
        for (int r = part * (kBC / TPC); r < (part + 1) * (kBC / TPC); ++r) {
            acc = fmaf(R[L::odKb + r * DK + c], R[L::oKb + r * DK + c], acc);
            acc = fmaf(R[L::odEb + r * DK + c], R[L::oEb + r * DK + c], acc);
        }
        sPart[tid] = acc;
    }
    for (int e = tid; e < kBC * DV; e += kGT) R0[(e / DV) * LD + e % DV] = R[L::odVt + e];   // dY -> R0
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int part = 0; part < TPC; ++part) acc += sPart[part * DK + tid];
        sCol[DK + tid] = acc;
    }
    {   // dW = dY S
        f32x4 a1[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) a1[m] = z4;
        fetch_rows(L::oS, 0);
        for (int i0 = 0; i0 < DV; i0 += QR) {
            __syncthreads();
            put_rows();
            __syncthreads();
            if (i0 + QR < DV) fetch_rows(L::oS, i0 + QR);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                a1[m] = mm_tile(a1[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R0[r * LD + i]; },
                                [&](int i, int c) { return sM2[(i - i0) * (DK + 4) + c]; });
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
            for (int q = 0; q < 4; ++q) R[L::odW + ti(r0, q) * DK + tj(c0)] = a1[m][q];
        }
    }
    float* sT = R1;   // Y is no longer needed
    float* sTmp = R1 + kBC * CP;
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kGT) sT[(e / kBC) * CP + e % kBC] = R[L::oT + e];
    __syncthreads();
    for (int t = w; t < TCV; t += kGW) {          // dZ = T^T dY
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                  [&](int m, int i) { return R0[m * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::odZ + ti(r0, q) * DV + tj(c0)] = acc[q];
    }
    for (int t = w; t < TCD; t += kGW) {          // dKhat = T^T dW
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                  [&](int m, int c) { return R[L::odW + m * DK + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::odKh + ti(r0, q) * DK + tj(c0)] = acc[q];
    }
    for (int t = w; t < TCC; t += kGW) {          // dT = dW Khat^T + dY Z^T
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        f32x4 acc = mm_tile(z4, r0, j0, 0, DK, [&](int r, int c) { return R[L::odW + r * DK + c]; },
                            [&](int c, int j) { return R[L::oKh + j * DK + c]; });
        acc = mm_tile(acc, r0, j0, 0, DV, [&](int r, int i) { return R0[r * LD + i]; },
                      [&](int i, int j) { return R[L::oZ + j * DV + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) sM1[ti(r0, q) * CP + tj(j0)] = acc[q];
    }
    __syncthreads();
    for (int t = w; t < TCC; t += kGW) {          // tmp = dT T^T
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 acc = mm_tile(z4, r0, j0, 0, kBC, [&](int r, int m) { return sM1[r * CP + m]; },
                                  [&](int m, int j) { return sT[j * CP + m]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) sTmp[ti(r0, q) * CP + tj(j0)] = acc[q];
    }
    __syncthreads();
    for (int t = w; t < TCC; t += kGW) {          // dAe = -T^T tmp, dAk = StrictTril(dZ X^T)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 ae = mm_tile(z4, r0, j0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                 [&](int m, int j) { return sTmp[m * CP + j]; });
        const f32x4 ak = mm_tile(z4, r0, j0, 0, DV, [&](int r, int i) { return R[L::odZ + r * DV + i]; },
                                 [&](int i, int j) { return R2[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), j = tj(j0);
            R[L::odAe + r * kBC + j] = j < r ? -ae[q] : 0.f;
            R[L::odAk + r * kBC + j] = j < r ? ak[q] : 0.f;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kGT)
        R0[(e / DV) * LD + e % DV] = (e / DV) < Cn ? load_elem<E>(p.dO, tix(e / DV) * DV + e % DV) : 0.f;
    __syncthreads();
    for (int t = w; t < TCV; t += kGW) {          // dX = Mk^T dO + Kbar dS'^T + Ak^T dZ -> dv, dw
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        f32x4 acc = mm_tile(z4, r0, c0, 0, kBC, [&](int r, int m) { return R[L::oMk + m * kBC + r]; },
                            [&](int m, int i) { return R0[m * LD + i]; });
        acc = mm_tile(acc, r0, c0, 0, DK, [&](int r, int c) { return R[L::oKb + r * DK + c]; },
                      [&](int c, int i) { return R[L::odS + i * DK + c]; });
        acc = mm_tile(acc, r0, c0, 0, kBC, [&](int r, int m) { return R[L::oAk + m * kBC + r]; },
                      [&](int m, int i) { return R[L::odZ + m * DV + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), i = tj(c0);
            if (r < Cn) {
                const int64_t vi = tix(r) * DV + i;
                store_elem<E>(p.gv, vi, load_elem<E>(p.wgate, vi) * acc[q]);
                store_elem<E>(p.gw, vi, load_elem<E>(p.v, vi) * acc[q]);
            }
        }
    }
    __syncthreads();
    // pairwise passes on 16 x 16 tiles of (r, c); accumulators per tile element
    f32x4 aq[MT], ak[MT], abk[MT], ag[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) aq[m] = ak[m] = abk[m] = ag[m] = z4;
    auto stage = [&](float* dst, int what) {   // 0 q, 1 k, 2 b k, 3 G
        for (int e = tid; e < kBC * DK; e += kGT) {
            const int r = e / DK, c = e % DK;
            float x;
            if (what == 3) {
                x = R[L::oG + e];
            } else if (r >= Cn) {
                x = 0.f;
            } else if (what == 0) {
                x = load_elem<E>(p.q, qk_index(p, b, t0 + r, h) * DK + c);
            } else {
                x = load_elem<E>(p.k, qk_index(p, b, t0 + r, h) * DK + c);
                if (what == 2) x *= load_elem<E>(p.beta, tix(r) * DK + c);
            }
            dst[r * LD + c] = x;
        }
    };
    auto Gf = [&](int r, int c) { return R2[r * LD + c]; };
    auto M1 = [&](int r, int j) { return sM1[r * CP + j]; };
    auto M2 = [&](int r, int j) { return sM2[r * CP + j]; };
    auto X0 = [&](int j, int c) { return R0[j * LD + c]; };
    auto X1 = [&](int j, int c) { return R1[j * LD + c]; };
    auto tile_of = [&](int m, int& r0, int& c0) {
        const int t = w + kGW * m;
        r0 = 16 * (t / (DK / 16));
        c0 = 16 * (t % (DK / 16));
    };
    // pass 1: Me (q, b k) and Mk (q, k) with G; q -> R0, b k -> R1, G -> R2
    for (int e = tid; e < kBC * kBC; e += kGT) {
        sM1[(e / kBC) * CP + e % kBC] = R[L::odMe + e];
        sM2[(e / kBC) * CP + e % kBC] = R[L::odMk + e];
    }
    stage(R0, 0);
    stage(R2, 3);
    stage(R1, 2);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {   // Me terms
        int r0, c0;
        tile_of(m, r0, c0);
        const f32x4 row = pair_tile<true>(r0, c0, M1, X1, Gf);
        const f32x4 col = pair_tile<false>(r0, c0, M1, X0, Gf);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), c = tj(c0);
            aq[m][q] += row[q];
            abk[m][q] += col[q];
            ag[m][q] += R0[r * LD + c] * row[q] - R1[r * LD + c] * col[q];
        }
    }
    __syncthreads();
    stage(R1, 1);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {   // Mk terms; k -> R1
        int r0, c0;
        tile_of(m, r0, c0);
        const f32x4 row = pair_tile<true>(r0, c0, M2, X1, Gf);
        const f32x4 col = pair_tile<false>(r0, c0, M2, X0, Gf);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), c = tj(c0);
            aq[m][q] += row[q];
            ak[m][q] += col[q];
            ag[m][q] += R0[r * LD + c] * row[q] - R1[r * LD + c] * col[q];
        }
    }
    __syncthreads();
    // pass 2: Ae (k, b k) and Ak (k, k); b k -> R0
    for (int e = tid; e < kBC * kBC; e += kGT) {
        sM1[(e / kBC) * CP + e % kBC] = R[L::odAe + e];
        sM2[(e / kBC) * CP + e % kBC] = R[L::odAk + e];
    }
    stage(R0, 2);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int r0, c0;
        tile_of(m, r0, c0);
        const f32x4 rowe = pair_tile<true>(r0, c0, M1, X0, Gf);
        const f32x4 cole = pair_tile<false>(r0, c0, M1, X1, Gf);
        const f32x4 rowk = pair_tile<true>(r0, c0, M2, X1, Gf);
        const f32x4 colk = pair_tile<false>(r0, c0, M2, X1, Gf);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), c = tj(c0);
            const float kr = R1[r * LD + c], bkr = R0[r * LD + c];
            ak[m][q] += rowe[q] + rowk[q] + colk[q];
            abk[m][q] += cole[q];
            ag[m][q] += kr * rowe[q] - bkr * cole[q] + kr * rowk[q] - kr * colk[q];
        }
    }
    // row factors, outputs, dG
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int r0, c0;
        tile_of(m, r0, c0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), c = tj(c0), e = r * DK + c;
            const float Gr = R2[r * LD + c];
            const float eg = __expf(Gr), eb = __expf(R2[(kBC - 1) * LD + c] - Gr);
            const float kr = R1[r * LD + c], bkr = R0[r * LD + c];
            const float dQh = R[L::odQh + e], dKh = R[L::odKh + e];
            const float dKb = R[L::odKb + e], dEb = R[L::odEb + e];
            const float q_ = aq[m][q] + dQh * eg;
            const float kpart = ak[m][q] + dKh * eg + dKb * eb;
            const float dbk = abk[m][q] + dEb * eb;
            const float qr = r < Cn ? load_elem<E>(p.q, qk_index(p, b, t0 + r, h) * DK + c) : 0.f;
            const float dg = ag[m][q] + dKh * kr * eg + dQh * qr * eg - dKb * kr * eb - dEb * bkr * eb;
            if (r < Cn) {
                const float br = load_elem<E>(p.beta, tix(r) * DK + c);
                store_qk_grad<E>(p.gq, p.gq32, tix(r), DK, c, q_);
                store_qk_grad<E>(p.gk, p.gk32, tix(r), DK, c, kpart + dbk * br);
                store_elem<E>(p.gbeta, tix(r) * DK + c, dbk * kr);
            }
            R[L::odQh + e] = dg;
        }
    }
    __syncthreads();
    if (tid < DK) {
        const int c = tid;
        float dgv[kBC];
#pragma unroll
        for (int r = 0; r < kBC; ++r) dgv[r] = R[L::odQh + r * DK + c];
        float acc = sCol[c] + sCol[DK + c];
#pragma unroll
        for (int r = kBC - 1; r >= 0; --r) {
            acc += dgv[r];
            if (r < Cn) store_elem<E>(p.gg, tix(r) * DK + c, acc);
        }
    }
}

template <typename E, int DK, int DV>
hipError_t launch_bwd2_dims(const BwdArgs& a, hipStream_t s) {
    typedef BwdWs2<DK, DV> L;
    const int N = (a.T + kBC - 1) / kBC;
    const int64_t units = static_cast<int64_t>(a.B) * a.H * N;
    if (units > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    hipMemPool_t pool;
    hipError_t e = workspace_pool(&pool);
    if (e != hipSuccess) return e;
    float* ws = nullptr;
    e = hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(units * L::size * 4), pool, s);
    if (e != hipSuccess) return e;
    const dim3 blk(kCT);
    const unsigned chains = chain_grid(a, DV);
    hipLaunchKernelGGL((bwd2_prep_kernel<E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
    e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd_fchain_kernel<L, E, DK, DV, true>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd_rchain_kernel<L, E, DK, DV, true>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd2_grads_kernel<E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(ws, s);
    return e == hipSuccess ? f : e;
}

template <typename E>
hipError_t launch_bwd2_dtype(const BwdArgs& a, hipStream_t s) {
    if (a.dk == 128 && a.dv == 128) return launch_bwd2_dims<E, 128, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_bwd2_dims<E, 128, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_bwd2_dims<E, 64, 128>(a, s);
    return launch_bwd2_dims<E, 64, 64>(a, s);
}

// dq, dk of grouped query/key heads: the sum over each group of value heads
template <typename E>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(BwdArgs p, int64_t n) {
    const int G = p.H / p.Hk;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * 256) {
        const int c = static_cast<int>(e % p.dk);
        const int64_t row = e / p.dk;                 // (b * T + t) * Hk + hk
        const int64_t tok = row / p.Hk, hk = row % p.Hk;
        float sq = 0.f, sk = 0.f;
        for (int g2 = 0; g2 < G; ++g2) {
            const int64_t vi = (tok * p.H + hk * G + g2) * p.dk + c;
            sq += p.gq32[vi];
            sk += p.gk32[vi];
        }
        store_elem<E>(p.gq, e, sq);
        store_elem<E>(p.gk, e, sk);
    }
}

// With grouped query/key heads the kernels write per-value-head dq, dk to fp32
// buffers from the pool, summed into the outputs by one more launch.
template <typename E>
hipError_t bwd_with_groups(BwdArgs a, hipStream_t s, hipError_t (*run)(const BwdArgs&, hipStream_t)) {
    if (a.Hk == a.H) {
        a.gq32 = a.gk32 = nullptr;
        return run(a, s);
    }
    hipMemPool_t pool;
    hipError_t e = workspace_pool(&pool);
    if (e != hipSuccess) return e;
    const int64_t per = static_cast<int64_t>(a.B) * a.T * a.H * a.dk;
    float* buf = nullptr;
    e = hipMallocFromPoolAsync(reinterpret_cast<void**>(&buf), static_cast<size_t>(2 * per * 4), pool, s);
    if (e != hipSuccess) return e;
    a.gq32 = buf;
    a.gk32 = buf + per;
    e = run(a, s);
    if (e == hipSuccess) {
        const int64_t n = static_cast<int64_t>(a.B) * a.T * a.Hk * a.dk;
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, int64_t(1) << 16);
        hipLaunchKernelGGL((bwd_group_sum_kernel<E>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a, n);
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(buf, s);
    return e == hipSuccess ? f : e;
}

template <int VAR, typename E, int DK, int DV>
hipError_t launch_bwd_dims(const BwdArgs& a, hipStream_t s) {
    typedef BwdWs<DK, DV> L;
    const int N = (a.T + kBC - 1) / kBC;
    const int64_t units = static_cast<int64_t>(a.B) * a.H * N;
    if (units > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    hipMemPool_t pool;
    hipError_t e = workspace_pool(&pool);
    if (e != hipSuccess) return e;
    float* ws = nullptr;
    e = hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(units * L::size * 4), pool, s);
    if (e != hipSuccess) return e;
    const dim3 blk(kCT);
    const unsigned chains = chain_grid(a, DV);
    hipLaunchKernelGGL((bwd_prep_kernel<VAR, E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
    e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd_fchain_kernel<L, E, DK, DV, false>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd_rchain_kernel<L, E, DK, DV, false>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd_grads_kernel<VAR, E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(ws, s);
    return e == hipSuccess ? f : e;
}

template <int VAR, typename E>
hipError_t launch_bwd_var(const BwdArgs& a, hipStream_t s) {
    if (a.dk == 128 && a.dv == 128) return launch_bwd_dims<VAR, E, 128, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_bwd_dims<VAR, E, 128, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_bwd_dims<VAR, E, 64, 128>(a, s);
    return launch_bwd_dims<VAR, E, 64, 64>(a, s);
}

template <int VAR>
hipError_t launch_bwd_dtype(int dtype, const BwdArgs& a, hipStream_t s) {
    return dtype == 0 ? bwd_with_groups<F32>(a, s, launch_bwd_var<VAR, F32>)
                      : bwd_with_groups<BF16>(a, s, launch_bwd_var<VAR, BF16>);
}

}  // namespace

hipError_t launch_bwd(int variant, int dtype, const BwdArgs& a, hipStream_t s) {
    switch (variant) {
        case 0: return launch_bwd_dtype<0>(dtype, a, s);
        case 1: return launch_bwd_dtype<1>(dtype, a, s);
        case 2: return launch_bwd_dtype<2>(dtype, a, s);
        case 4: return launch_bwd_dtype<4>(dtype, a, s);
        default: return dtype == 0 ? bwd_with_groups<F32>(a, s, launch_bwd2_dtype<F32>)
                                   : bwd_with_groups<BF16>(a, s, launch_bwd2_dtype<BF16>);
    }
}

}  // namespace dr
