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
constexpr int kBT = 256;    // threads per workgroup
constexpr int kBVT = 32;    // value rows per chain workgroup

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

// ---------------------------------------------------------------- 1. factors
template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kBT) void bwd_prep_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs<DK, DV> L;
    constexpr int LD = (DK > DV ? DK : DV) + 1;   // padded row stride
    __shared__ float sK[kBC * (DK + 1)];
    __shared__ float sX[kBC * LD];                // q, then beta Khat, then beta v
    __shared__ float sG[kBC * (DK + 1)];
    __shared__ float sA[kBC * (kBC + 1)];
    __shared__ float sT[kBC * (kBC + 1)];
    __shared__ float sBeta[kBC];
    const int u = blockIdx.x, tid = threadIdx.x;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;

    for (int e = tid; e < kBC * DK; e += kBT) {
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        const int64_t ti = tok_index(p, b, t0 + min(r, Cn - 1), h);
        sK[r * (DK + 1) + c] = ok ? load_elem<E>(p.k, ti * DK + c) : 0.f;
        sX[r * LD + c] = ok ? load_elem<E>(p.q, ti * DK + c) : 0.f;
        float gv = 0.f;
        if constexpr (VAR == 1) gv = ok ? load_elem<E>(p.g, ti) : 0.f;
        if constexpr (VAR == 2) gv = ok ? load_elem<E>(p.g, ti * DK + c) : 0.f;
        sG[r * (DK + 1) + c] = gv;
    }
    if (tid < kBC) sBeta[tid] = tid < Cn ? load_elem<E>(p.beta, tok_index(p, b, t0 + tid, h)) : 0.f;
    __syncthreads();
    if (tid < DK) {   // in-chunk cumulative log-decay per channel
        float acc = 0.f;
        for (int r = 0; r < kBC; ++r) {
            acc += sG[r * (DK + 1) + tid];
            sG[r * (DK + 1) + tid] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kBT) R[L::oG + e] = sG[(e / DK) * (DK + 1) + e % DK];
    if (tid < DK) R[L::oGam + tid] = __expf(sG[(kBC - 1) * (DK + 1) + tid]);
    // Abar (strictly lower) and Mq (lower, diagonal included)
    for (int e = tid; e < kBC * kBC; e += kBT) {
        const int r = e / kBC, j = e % kBC;
        float ab = 0.f, mq = 0.f;
        if (j <= r) {
            const float* kr = sK + r * (DK + 1);
            const float* kj = sK + j * (DK + 1);
            const float* qr = sX + r * LD;
            if constexpr (VAR == 2) {
                const float* gr = sG + r * (DK + 1);
                const float* gj = sG + j * (DK + 1);
                for (int c = 0; c < DK; ++c) {
                    const float w = kj[c] * __expf(gr[c] - gj[c]);
                    ab = fmaf(kr[c], w, ab);
                    mq = fmaf(qr[c], w, mq);
                }
            } else {
                for (int c = 0; c < DK; ++c) {
                    ab = fmaf(kr[c], kj[c], ab);
                    mq = fmaf(qr[c], kj[c], mq);
                }
                if constexpr (VAR == 1) {
                    const float ex = __expf(sG[r * (DK + 1)] - sG[j * (DK + 1)]);
                    ab *= ex;
                    mq *= ex;
                }
            }
            if (j == r) ab = 0.f;
        }
        sA[r * (kBC + 1) + j] = ab;
        R[L::oAb + e] = ab;
        R[L::oMq + e] = mq;
    }
    __syncthreads();
    // T = (I + diag(beta) Abar)^-1 by forward substitution, one column per thread
    if (tid < kBC) {
        const int col = tid;
        for (int r = 0; r < kBC; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
            const float br = sBeta[r];
            for (int j = col; j < r; ++j) acc = fmaf(-br * sA[r * (kBC + 1) + j], sT[j * (kBC + 1) + col], acc);
            sT[r * (kBC + 1) + col] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) R[L::oT + e] = sT[(e / kBC) * (kBC + 1) + e % kBC];
    // key and query factors; sX becomes X = beta Khat
    for (int e = tid; e < kBC * DK; e += kBT) {
        const int r = e / DK, c = e % DK;
        const float G = sG[r * (DK + 1) + c];
        const float eg = __expf(G);
        const float kk = sK[r * (DK + 1) + c];
        R[L::oKh + e] = kk * eg;
        R[L::oQh + e] = sX[r * LD + c] * eg;
        R[L::oKb + e] = kk * __expf(sG[(kBC - 1) * (DK + 1) + c] - G);
        sX[r * LD + c] = sBeta[r] * kk * eg;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kBT) {   // W = T X
        const int r = e / DK, c = e % DK;
        float acc = 0.f;
        for (int j = 0; j <= r; ++j) acc = fmaf(sT[r * (kBC + 1) + j], sX[j * LD + c], acc);
        R[L::oW + e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // Y = beta v
        const int r = e / DV, i = e % DV;
        sX[r * LD + i] = r < Cn ? sBeta[r] * load_elem<E>(p.v, tok_index(p, b, t0 + r, h) * DV + i) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // U = T Y
        const int r = e / DV, i = e % DV;
        float acc = 0.f;
        for (int j = 0; j <= r; ++j) acc = fmaf(sT[r * (kBC + 1) + j], sX[j * LD + i], acc);
        R[L::oU + e] = acc;
    }
}

// ------------------------------------------------------ 2. forward state chain
// Single step size:  Vt = U - W S^T,   S = S Diag(gamma) + Vt^T Kbar.
// Split gates:       Y = Ut + W S^T,   S = S Diag(gamma) - Y^T Ebar + X^T Kbar.
template <class L, typename E, int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(kBT) void bwd_fchain_kernel(BwdArgs p, float* ws, int N) {
    constexpr int NVT = DV / kBVT;
    __shared__ float sS[kBVT * (DK + 1)];
    __shared__ float sVt[kBC * (kBVT + 1)];
    __shared__ float sW[kBC * (DK + 1)];
    __shared__ float sKb[kBC * (DK + 1)];
    __shared__ float sEb[SPLIT ? kBC * (DK + 1) : 1];
    __shared__ float sXt[SPLIT ? kBC * (kBVT + 1) : 1];
    __shared__ float sGam[DK];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / NVT, i0 = (blockIdx.x % NVT) * kBVT;
    const int b = bh / p.H, h = bh % p.H;
    for (int e = tid; e < kBVT * DK; e += kBT) {
        const int i = e / DK, c = e % DK;
        sS[i * (DK + 1) + c] = p.S0 ? p.S0[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c] : 0.f;
    }
    for (int n = 0; n < N; ++n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        for (int e = tid; e < kBC * DK; e += kBT) {
            const int r = e / DK, c = e % DK;
            sW[r * (DK + 1) + c] = R[L::oW + e];
            sKb[r * (DK + 1) + c] = R[L::oKb + e];
            if constexpr (SPLIT) sEb[r * (DK + 1) + c] = R[L::oEb + e];
        }
        if constexpr (SPLIT) {   // X = w v for this tile's value columns
            const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
            for (int e = tid; e < kBC * kBVT; e += kBT) {
                const int r = e / kBVT, i = e % kBVT;
                float x = 0.f;
                if (r < Cn) {
                    const int64_t vi = tok_index(p, b, t0 + r, h) * DV + i0 + i;
                    x = load_elem<E>(p.wgate, vi) * load_elem<E>(p.v, vi);
                }
                sXt[r * (kBVT + 1) + i] = x;
            }
        }
        if (tid < DK) sGam[tid] = R[L::oGam + tid];
        __syncthreads();
        for (int e = tid; e < kBVT * DK; e += kBT) {
            const int i = e / DK, c = e % DK;
            R[L::oS + (i0 + i) * DK + c] = sS[i * (DK + 1) + c];
        }
        constexpr float sgn = SPLIT ? 1.f : -1.f;
        for (int e = tid; e < kBC * kBVT; e += kBT) {   // Vt = U - W S^T  /  Y = Ut + W S^T
            const int r = e / kBVT, i = e % kBVT;
            float acc = R[L::oU + r * DV + i0 + i];
            for (int c = 0; c < DK; ++c) acc = fmaf(sgn * sW[r * (DK + 1) + c], sS[i * (DK + 1) + c], acc);
            sVt[r * (kBVT + 1) + i] = acc;
            R[L::oVt + r * DV + i0 + i] = acc;
        }
        __syncthreads();
        for (int e = tid; e < kBVT * DK; e += kBT) {
            const int i = e / DK, c = e % DK;
            float acc = sS[i * (DK + 1) + c] * sGam[c];
            if constexpr (SPLIT) {
                for (int r = 0; r < kBC; ++r) {
                    acc = fmaf(-sVt[r * (kBVT + 1) + i], sEb[r * (DK + 1) + c], acc);
                    acc = fmaf(sXt[r * (kBVT + 1) + i], sKb[r * (DK + 1) + c], acc);
                }
            } else {
                for (int r = 0; r < kBC; ++r) acc = fmaf(sVt[r * (kBVT + 1) + i], sKb[r * (DK + 1) + c], acc);
            }
            sS[i * (DK + 1) + c] = acc;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------ 3. reverse state chain
// Single step size:  dVt = Mq^T dO + Kbar dS'^T,     dS = dS' Diag(gamma) + dO^T Qhat - dVt^T W.
// Split gates:       dY = -(Me^T dO + Ebar dS'^T),   dS = dS' Diag(gamma) + dO^T Qhat + dY^T W.
template <class L, typename E, int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(kBT) void bwd_rchain_kernel(BwdArgs p, float* ws, int N) {
    constexpr int NVT = DV / kBVT;
    __shared__ float sdS[kBVT * (DK + 1)];
    __shared__ float sdVt[kBC * (kBVT + 1)];
    __shared__ float sdO[kBC * (kBVT + 1)];
    __shared__ float sM[kBC * (kBC + 1)];
    __shared__ float sA1[kBC * (DK + 1)];
    __shared__ float sA2[kBC * (DK + 1)];
    __shared__ float sGam[DK];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / NVT, i0 = (blockIdx.x % NVT) * kBVT;
    const int b = bh / p.H, h = bh % p.H;
    for (int e = tid; e < kBVT * DK; e += kBT) {
        const int i = e / DK, c = e % DK;
        sdS[i * (DK + 1) + c] = p.dST ? p.dST[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c] : 0.f;
    }
    for (int n = N - 1; n >= 0; --n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
        for (int e = tid; e < kBC * kBC; e += kBT) sM[(e / kBC) * (kBC + 1) + e % kBC] = R[L::oMq + e];
        for (int e = tid; e < kBC * DK; e += kBT)
            sA1[(e / DK) * (DK + 1) + e % DK] = R[(SPLIT ? L::oEb : L::oKb) + e];
        for (int e = tid; e < kBC * kBVT; e += kBT) {
            const int r = e / kBVT, i = e % kBVT;
            sdO[r * (kBVT + 1) + i] = r < Cn ? load_elem<E>(p.dO, tok_index(p, b, t0 + r, h) * DV + i0 + i) : 0.f;
        }
        if (tid < DK) sGam[tid] = R[L::oGam + tid];
        __syncthreads();
        for (int e = tid; e < kBVT * DK; e += kBT) {
            const int i = e / DK, c = e % DK;
            R[L::odS + (i0 + i) * DK + c] = sdS[i * (DK + 1) + c];
        }
        for (int e = tid; e < kBC * kBVT; e += kBT) {   // dVt = Mq^T dO + Kbar dS^T
            const int r = e / kBVT, i = e % kBVT;
            float acc = 0.f;
            for (int m = r; m < kBC; ++m) acc = fmaf(sM[m * (kBC + 1) + r], sdO[m * (kBVT + 1) + i], acc);
            for (int c = 0; c < DK; ++c) acc = fmaf(sA1[r * (DK + 1) + c], sdS[i * (DK + 1) + c], acc);
            if constexpr (SPLIT) acc = -acc;
            sdVt[r * (kBVT + 1) + i] = acc;
            R[L::odVt + r * DV + i0 + i] = acc;
        }
        __syncthreads();
        for (int e = tid; e < kBC * DK; e += kBT) {
            const int r = e / DK, c = e % DK;
            sA1[r * (DK + 1) + c] = R[L::oQh + e];
            sA2[r * (DK + 1) + c] = R[L::oW + e];
        }
        __syncthreads();
        for (int e = tid; e < kBVT * DK; e += kBT) {    // dS = dS Diag(gamma) + dO^T Qhat - dVt^T W
            const int i = e / DK, c = e % DK;
            float acc = sdS[i * (DK + 1) + c] * sGam[c];
            for (int r = 0; r < kBC; ++r) {
                acc = fmaf(sdO[r * (kBVT + 1) + i], sA1[r * (DK + 1) + c], acc);
                acc = fmaf((SPLIT ? 1.f : -1.f) * sdVt[r * (kBVT + 1) + i], sA2[r * (DK + 1) + c], acc);
            }
            sdS[i * (DK + 1) + c] = acc;
        }
        __syncthreads();
    }
    if (p.gS0) {
        for (int e = tid; e < kBVT * DK; e += kBT) {
            const int i = e / DK, c = e % DK;
            p.gS0[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c] = sdS[i * (DK + 1) + c];
        }
    }
}

// ------------------------------------------------------------ 4. gradients
template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kBT) void bwd_grads_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs<DK, DV> L;
    constexpr int CP = kBC + 1;
    constexpr int LD = (DK > DV ? DK : DV) + 1;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;   // region size
    __shared__ float sM1[kBC * CP];   // dMq
    __shared__ float sM2[kBC * CP];   // dT, then dA, then dAbar
    __shared__ float sR[3 * RS];      // three staging regions
    __shared__ float sBeta[kBC];
    __shared__ float sCol[5 * DK];    // column terms of the last row of dG
    float* R0 = sR;
    float* R1 = sR + RS;
    float* R2 = sR + 2 * RS;
    const int u = blockIdx.x, tid = threadIdx.x;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };

    if (tid < kBC) sBeta[tid] = tid < Cn ? load_elem<E>(p.beta, tix(tid)) : 0.f;
    for (int e = tid; e < kBC * DV; e += kBT) {   // dO -> R0, Vt -> R1, dVt -> R2
        const int r = e / DV, i = e % DV;
        R0[r * LD + i] = r < Cn ? load_elem<E>(p.dO, tix(r) * DV + i) : 0.f;
        R1[r * LD + i] = R[L::oVt + e];
        R2[r * LD + i] = R[L::odVt + e];
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // dMq = Tril0(dO Vt^T)
        const int r = e / kBC, j = e % kBC;
        float acc = 0.f;
        if (j <= r)
            for (int i = 0; i < DV; ++i) acc = fmaf(R0[r * LD + i], R1[j * LD + i], acc);
        sM1[r * CP + j] = acc;
    }
    // dQhat = dO S, dW = -dVt S, dKbar = Vt dS': thread owns column c, rows rr
    {
        constexpr int TPC = kBT / DK;             // threads per column
        constexpr int NR = kBC / TPC;             // rows per thread
        const int c = tid % DK, rq = tid / DK;
        float aq[NR], aw[NR], ak[NR];
#pragma unroll
        for (int m = 0; m < NR; ++m) aq[m] = aw[m] = ak[m] = 0.f;
        float sds = 0.f;
        for (int i = 0; i < DV; ++i) {
            const float s = R[L::oS + i * DK + c];
            const float ds = R[L::odS + i * DK + c];
            sds = fmaf(s, ds, sds);
#pragma unroll
            for (int m = 0; m < NR; ++m) {
                const int r = rq + TPC * m;
                aq[m] = fmaf(R0[r * LD + i], s, aq[m]);
                aw[m] = fmaf(-R2[r * LD + i], s, aw[m]);
                ak[m] = fmaf(R1[r * LD + i], ds, ak[m]);
            }
        }
        float kbsum = 0.f;
#pragma unroll
        for (int m = 0; m < NR; ++m) {
            const int r = rq + TPC * m;
            R[L::odQh + r * DK + c] = aq[m];
            R[L::odW + r * DK + c] = aw[m];
            R[L::odKb + r * DK + c] = ak[m];
            kbsum = fmaf(ak[m], R[L::oKb + r * DK + c], kbsum);
        }
        // the last row's column terms: gamma * sum_i S dS' (same in every thread of
        // the column) and this thread's part of sum_r dKbar Kbar
        if (rq == 0) sCol[c] = R[L::oGam + c] * sds;
        sCol[DK * (1 + rq) + c] = kbsum;
    }
    __syncthreads();
    // dT = dW X^T + dVt Y^T with X = beta Khat, Y = beta v
    for (int e = tid; e < kBC * DK; e += kBT) {   // dW -> R0, X -> R1
        const int r = e / DK, c = e % DK;
        R0[r * LD + c] = R[L::odW + e];
        R1[r * LD + c] = sBeta[r] * R[L::oKh + e];
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {
        const int r = e / kBC, j = e % kBC;
        float acc = 0.f;
        for (int c = 0; c < DK; ++c) acc = fmaf(R0[r * LD + c], R1[j * LD + c], acc);
        sM2[r * CP + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // Y -> R1
        const int r = e / DV, i = e % DV;
        R1[r * LD + i] = r < Cn ? sBeta[r] * load_elem<E>(p.v, tix(r) * DV + i) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {
        const int r = e / kBC, j = e % kBC;
        float acc = sM2[r * CP + j];
        for (int i = 0; i < DV; ++i) acc = fmaf(R2[r * LD + i], R1[j * LD + i], acc);
        sM2[r * CP + j] = acc;
    }
    __syncthreads();
    // dA = -T^T dT T^T (strictly lower); T -> R1[0 .. C*CP), tmp -> R1[C*CP ..)
    float* sT = R1;
    float* sTmp = R1 + kBC * CP;
    for (int e = tid; e < kBC * kBC; e += kBT) sT[(e / kBC) * CP + e % kBC] = R[L::oT + e];
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // tmp = dT T^T
        const int r = e / kBC, j = e % kBC;
        float acc = 0.f;
        for (int m = 0; m <= j; ++m) acc = fmaf(sM2[r * CP + m], sT[j * CP + m], acc);
        sTmp[r * CP + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // dA = -T^T tmp, masked
        const int r = e / kBC, j = e % kBC;
        float acc = 0.f;
        if (j < r)
            for (int m = r; m < kBC; ++m) acc = fmaf(-sT[m * CP + r], sTmp[m * CP + j], acc);
        sM2[r * CP + j] = acc;
    }
    __syncthreads();
    // dX = T^T dW (kept for dKhat), dY = T^T dVt -> dv, and dbeta; 4 threads per row
    {
        const int r = tid / 4, qt = tid % 4;
        float db = 0.f;
        for (int c = qt * (DK / 4); c < (qt + 1) * (DK / 4); ++c) {
            float acc = 0.f;
            for (int m = r; m < kBC; ++m) acc = fmaf(sT[m * CP + r], R0[m * LD + c], acc);
            R[L::odX + r * DK + c] = acc;
            db = fmaf(acc, R[L::oKh + r * DK + c], db);
        }
        for (int i = qt * (DV / 4); i < (qt + 1) * (DV / 4); ++i) {
            float acc = 0.f;
            for (int m = r; m < kBC; ++m) acc = fmaf(sT[m * CP + r], R2[m * LD + i], acc);
            if (r < Cn) {
                const float vv = load_elem<E>(p.v, tix(r) * DV + i);
                db = fmaf(acc, vv, db);
                store_elem<E>(p.gv, tix(r) * DV + i, sBeta[r] * acc);
            }
        }
        for (int j = qt * (kBC / 4); j < (qt + 1) * (kBC / 4); ++j)
            db = fmaf(sM2[r * CP + j], R[L::oAb + r * kBC + j], db);
        db += __shfl_xor(db, 1);
        db += __shfl_xor(db, 2);
        if (qt == 0 && r < Cn) store_elem<E>(p.gbeta, tix(r), db);
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) sM2[(e / kBC) * CP + e % kBC] *= sBeta[e / kBC];   // dAbar
    // q, k, G -> R0, R1, R2
    for (int e = tid; e < kBC * DK; e += kBT) {
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        R0[r * LD + c] = ok ? load_elem<E>(p.q, tix(r) * DK + c) : 0.f;
        R1[r * LD + c] = ok ? load_elem<E>(p.k, tix(r) * DK + c) : 0.f;
        R2[r * LD + c] = R[L::oG + e];
    }
    __syncthreads();
    // per element (r, c): pairwise sums with E = exp(G_r - G_j)
    for (int e = tid; e < kBC * DK; e += kBT) {
        const int r = e / DK, c = e % DK;
        const float Gr = R2[r * LD + c];
        const float qr = R0[r * LD + c], kr = R1[r * LD + c];
        float a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f;
        for (int j = 0; j < kBC; ++j) {
            const float Gj = R2[j * LD + c];
            if (j <= r) {
                const float ex = (VAR == 0) ? 1.f : __expf(Gr - Gj);
                const float kj = R1[j * LD + c] * ex;
                a1 = fmaf(sM1[r * CP + j], kj, a1);
                a3 = fmaf(sM2[r * CP + j], kj, a3);   // dAbar is zero on the diagonal
            }
            if (j >= r) {
                const float ex = (VAR == 0) ? 1.f : __expf(Gj - Gr);
                a2 = fmaf(sM1[j * CP + r], R0[j * LD + c] * ex, a2);
                a4 = fmaf(sM2[j * CP + r], R1[j * LD + c] * ex, a4);
            }
        }
        const float eg = (VAR == 0) ? 1.f : __expf(Gr);
        const float ebar = (VAR == 0) ? 1.f : __expf(R2[(kBC - 1) * LD + c] - Gr);
        const float dQh = R[L::odQh + e];
        const float dKh = sBeta[r] * R[L::odX + e];
        const float dKb = R[L::odKb + e];
        if (r < Cn) {
            store_elem<E>(p.gq, tix(r) * DK + c, fmaf(dQh, eg, a1));
            store_elem<E>(p.gk, tix(r) * DK + c, a2 + a3 + a4 + dKh * eg + dKb * ebar);
        }
        // dG: pairwise terms plus the row factors (Khat, Qhat, Kbar); overwrites dQhat
        const float dG = qr * a1 - kr * a2 + kr * a3 - kr * a4 + dKh * kr * eg + dQh * qr * eg
                         - dKb * kr * ebar;
        R[L::odQh + e] = dG;
    }
    if constexpr (VAR != 0) {
        __syncthreads();
        if (tid < DK) {   // reverse cumulative sum over rows; G_C's terms enter at the last row
            const int c = tid;
            float acc = sCol[c];
            for (int q2 = 0; q2 < kBT / DK; ++q2) acc += sCol[DK * (1 + q2) + c];
            for (int r = kBC - 1; r >= 0; --r) {
                acc += R[L::odQh + r * DK + c];
                if constexpr (VAR == 2) {
                    if (r < Cn) store_elem<E>(p.gg, tix(r) * DK + c, acc);
                } else {
                    R[L::odQh + r * DK + c] = acc;
                }
            }
        }
        if constexpr (VAR == 1) {   // scalar decay: sum over channels, 4 threads per row
            __syncthreads();
            const int r = tid / 4, qt = tid % 4;
            float s = 0.f;
            for (int c = qt * (DK / 4); c < (qt + 1) * (DK / 4); ++c) s += R[L::odQh + r * DK + c];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            if (qt == 0 && r < Cn) store_elem<E>(p.gg, tix(r), s);
        }
    }
}

// --------------------------------------------- split gates: 1. factors
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kBT) void bwd2_prep_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs2<DK, DV> L;
    constexpr int LD = (DK > DV ? DK : DV) + 1;
    constexpr int CP = kBC + 1;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;
    __shared__ float sK[kBC * (DK + 1)];
    __shared__ float sG[kBC * (DK + 1)];
    __shared__ float sR1[RS];
    __shared__ float sR2[RS];
    __shared__ float sM[kBC * CP];
    const int u = blockIdx.x, tid = threadIdx.x;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };

    for (int e = tid; e < kBC * DK; e += kBT) {   // k, b k, g
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        const float kk = ok ? load_elem<E>(p.k, tix(r) * DK + c) : 0.f;
        sK[r * (DK + 1) + c] = kk;
        sR1[r * LD + c] = ok ? load_elem<E>(p.beta, tix(r) * DK + c) * kk : 0.f;
        sG[r * (DK + 1) + c] = ok ? load_elem<E>(p.g, tix(r) * DK + c) : 0.f;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < kBC; ++r) {
            acc += sG[r * (DK + 1) + tid];
            sG[r * (DK + 1) + tid] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kBT) R[L::oG + e] = sG[(e / DK) * (DK + 1) + e % DK];
    if (tid < DK) R[L::oGam + tid] = __expf(sG[(kBC - 1) * (DK + 1) + tid]);
    for (int e = tid; e < kBC * kBC; e += kBT) {  // Ae -> sM, Ak -> workspace (strictly lower)
        const int r = e / kBC, j = e % kBC;
        float ae = 0.f, ak = 0.f;
        if (j < r) {
            for (int c = 0; c < DK; ++c) {
                const float ex = __expf(sG[r * (DK + 1) + c] - sG[j * (DK + 1) + c]);
                const float kr = sK[r * (DK + 1) + c] * ex;
                ae = fmaf(kr, sR1[j * LD + c], ae);
                ak = fmaf(kr, sK[j * (DK + 1) + c], ak);
            }
        }
        sM[r * CP + j] = ae;
        R[L::oAk + e] = ak;
    }
    __syncthreads();
    float* sT = sR2;
    if (tid < kBC) {   // T = (I + Ae)^-1
        const int col = tid;
        for (int r = 0; r < kBC; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
            for (int j = col; j < r; ++j) acc = fmaf(-sM[r * CP + j], sT[j * CP + col], acc);
            sT[r * CP + col] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) R[L::oT + e] = sT[(e / kBC) * CP + e % kBC];
    for (int e = tid; e < kBC * DK; e += kBT) {   // Ebar, Kbar, Khat; Khat -> sR1
        const int r = e / DK, c = e % DK;
        const float G = sG[r * (DK + 1) + c];
        const float eg = __expf(G), eb = __expf(sG[(kBC - 1) * (DK + 1) + c] - G);
        const float kk = sK[r * (DK + 1) + c];
        R[L::oEb + e] = sR1[r * LD + c] * eb;
        R[L::oKb + e] = kk * eb;
        R[L::oKh + e] = kk * eg;
        sR1[r * LD + c] = kk * eg;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kBT) {   // W = T Khat
        const int r = e / DK, c = e % DK;
        float acc = 0.f;
        for (int j = 0; j <= r; ++j) acc = fmaf(sT[r * CP + j], sR1[j * LD + c], acc);
        R[L::oW + e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // X = w v -> sR1
        const int r = e / DV, i = e % DV;
        float x = 0.f;
        if (r < Cn) x = load_elem<E>(p.wgate, tix(r) * DV + i) * load_elem<E>(p.v, tix(r) * DV + i);
        sR1[r * LD + i] = x;
    }
    for (int e = tid; e < kBC * kBC; e += kBT) sM[(e / kBC) * CP + e % kBC] = R[L::oAk + e];
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // Z = Ak X
        const int r = e / DV, i = e % DV;
        float acc = 0.f;
        for (int j = 0; j < r; ++j) acc = fmaf(sM[r * CP + j], sR1[j * LD + i], acc);
        R[L::oZ + e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // Ut = T Z
        const int r = e / DV, i = e % DV;
        float acc = 0.f;
        for (int j = 0; j <= r; ++j) acc = fmaf(sT[r * CP + j], R[L::oZ + j * DV + i], acc);
        R[L::oU + e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DK; e += kBT) {   // q -> sR1, b k -> sR2, Qhat
        const int r = e / DK, c = e % DK;
        const bool ok = r < Cn;
        const float qq = ok ? load_elem<E>(p.q, tix(r) * DK + c) : 0.f;
        sR1[r * LD + c] = qq;
        sR2[r * LD + c] = ok ? load_elem<E>(p.beta, tix(r) * DK + c) * sK[r * (DK + 1) + c] : 0.f;
        R[L::oQh + e] = qq * __expf(sG[r * (DK + 1) + c]);
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // Me, Mk (lower, diagonal included)
        const int r = e / kBC, j = e % kBC;
        float me = 0.f, mk = 0.f;
        if (j <= r) {
            for (int c = 0; c < DK; ++c) {
                const float qe = sR1[r * LD + c] * __expf(sG[r * (DK + 1) + c] - sG[j * (DK + 1) + c]);
                me = fmaf(qe, sR2[j * LD + c], me);
                mk = fmaf(qe, sK[j * (DK + 1) + c], mk);
            }
        }
        R[L::oMq + e] = me;
        R[L::oMk + e] = mk;
    }
}

// ------------------------------------------ split gates: 4. gradients
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kBT) void bwd2_grads_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs2<DK, DV> L;
    constexpr int CP = kBC + 1;
    constexpr int LD = (DK > DV ? DK : DV) + 1;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;
    constexpr int NE = kBC * DK / kBT;   // (r, c) entries per thread
    __shared__ float sM1[kBC * CP];
    __shared__ float sM2[kBC * CP];
    __shared__ float sR[3 * RS];
    __shared__ float sCol[5 * DK];
    float* R0 = sR;
    float* R1 = sR + RS;
    float* R2 = sR + 2 * RS;
    const int u = blockIdx.x, tid = threadIdx.x;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };
    auto xval = [&](int r, int i) {   // X = w v (zero past the sequence)
        if (r >= Cn) return 0.f;
        const int64_t vi = tix(r) * DV + i;
        return load_elem<E>(p.wgate, vi) * load_elem<E>(p.v, vi);
    };

    for (int e = tid; e < kBC * DV; e += kBT) {   // dO -> R0, Y -> R1, X -> R2
        const int r = e / DV, i = e % DV;
        R0[r * LD + i] = r < Cn ? load_elem<E>(p.dO, tix(r) * DV + i) : 0.f;
        R1[r * LD + i] = R[L::oVt + e];
        R2[r * LD + i] = xval(r, i);
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // dMe = -Tril0(dO Y^T), dMk = Tril0(dO X^T)
        const int r = e / kBC, j = e % kBC;
        float me = 0.f, mk = 0.f;
        if (j <= r) {
            for (int i = 0; i < DV; ++i) {
                me = fmaf(-R0[r * LD + i], R1[j * LD + i], me);
                mk = fmaf(R0[r * LD + i], R2[j * LD + i], mk);
            }
        }
        R[L::odMe + e] = me;
        R[L::odMk + e] = mk;
    }
    constexpr int TPC = kBT / DK;
    constexpr int NR = kBC / TPC;
    const int cc = tid % DK, rq = tid / DK;
    {   // dQhat = dO S, dEbar = -Y dS', dKbar = X dS'; column terms of the last row
        float aq[NR], ae[NR], ak[NR];
#pragma unroll
        for (int m = 0; m < NR; ++m) aq[m] = ae[m] = ak[m] = 0.f;
        float sds = 0.f;
        for (int i = 0; i < DV; ++i) {
            const float s_ = R[L::oS + i * DK + cc];
            const float ds = R[L::odS + i * DK + cc];
            sds = fmaf(s_, ds, sds);
#pragma unroll
            for (int m = 0; m < NR; ++m) {
                const int r = rq + TPC * m;
                aq[m] = fmaf(R0[r * LD + i], s_, aq[m]);
                ae[m] = fmaf(-R1[r * LD + i], ds, ae[m]);
                ak[m] = fmaf(R2[r * LD + i], ds, ak[m]);
            }
        }
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < NR; ++m) {
            const int r = rq + TPC * m;
            R[L::odQh + r * DK + cc] = aq[m];
            R[L::odEb + r * DK + cc] = ae[m];
            R[L::odKb + r * DK + cc] = ak[m];
            part = fmaf(ak[m], R[L::oKb + r * DK + cc], part);
            part = fmaf(ae[m], R[L::oEb + r * DK + cc], part);
        }
        if (rq == 0) sCol[cc] = R[L::oGam + cc] * sds;
        sCol[DK * (1 + rq) + cc] = part;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) R0[(e / DV) * LD + e % DV] = R[L::odVt + e];   // dY -> R0
    __syncthreads();
    {   // dW = dY S
        float aw[NR];
#pragma unroll
        for (int m = 0; m < NR; ++m) aw[m] = 0.f;
        for (int i = 0; i < DV; ++i) {
            const float s_ = R[L::oS + i * DK + cc];
#pragma unroll
            for (int m = 0; m < NR; ++m) aw[m] = fmaf(R0[(rq + TPC * m) * LD + i], s_, aw[m]);
        }
#pragma unroll
        for (int m = 0; m < NR; ++m) R[L::odW + (rq + TPC * m) * DK + cc] = aw[m];
    }
    float* sT = R1;   // Y is no longer needed
    for (int e = tid; e < kBC * kBC; e += kBT) sT[(e / kBC) * CP + e % kBC] = R[L::oT + e];
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // dZ = T^T dY
        const int r = e / DV, i = e % DV;
        float acc = 0.f;
        for (int m = r; m < kBC; ++m) acc = fmaf(sT[m * CP + r], R0[m * LD + i], acc);
        R[L::odZ + e] = acc;
    }
    for (int e = tid; e < kBC * DK; e += kBT) {   // dKhat = T^T dW
        const int r = e / DK, c = e % DK;
        float acc = 0.f;
        for (int m = r; m < kBC; ++m) acc = fmaf(sT[m * CP + r], R[L::odW + m * DK + c], acc);
        R[L::odKh + e] = acc;
    }
    for (int e = tid; e < kBC * kBC; e += kBT) {  // dT = dW Khat^T + dY Z^T
        const int r = e / kBC, j = e % kBC;
        float acc = 0.f;
        for (int c = 0; c < DK; ++c) acc = fmaf(R[L::odW + r * DK + c], R[L::oKh + j * DK + c], acc);
        for (int i = 0; i < DV; ++i) acc = fmaf(R0[r * LD + i], R[L::oZ + j * DV + i], acc);
        sM1[r * CP + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // tmp = dT T^T
        const int r = e / kBC, j = e % kBC;
        float acc = 0.f;
        for (int m = 0; m <= j; ++m) acc = fmaf(sM1[r * CP + m], sT[j * CP + m], acc);
        sM2[r * CP + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < kBC * kBC; e += kBT) {  // dAe = -T^T tmp; dAk = StrictTril(dZ X^T)
        const int r = e / kBC, j = e % kBC;
        float dae = 0.f, dak = 0.f;
        if (j < r) {
            for (int m = r; m < kBC; ++m) dae = fmaf(-sT[m * CP + r], sM2[m * CP + j], dae);
            for (int i = 0; i < DV; ++i) dak = fmaf(R[L::odZ + r * DV + i], R2[j * LD + i], dak);
        }
        R[L::odAe + e] = dae;
        R[L::odAk + e] = dak;
    }
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) R0[(e / DV) * LD + e % DV] = (e / DV) < Cn ? load_elem<E>(p.dO, tix(e / DV) * DV + e % DV) : 0.f;
    __syncthreads();
    for (int e = tid; e < kBC * DV; e += kBT) {   // dX = Mk^T dO + Kbar dS'^T + Ak^T dZ -> dv, dw
        const int r = e / DV, i = e % DV;
        float acc = 0.f;
        for (int m = r; m < kBC; ++m) acc = fmaf(R[L::oMk + m * kBC + r], R0[m * LD + i], acc);
        for (int c = 0; c < DK; ++c) acc = fmaf(R[L::oKb + r * DK + c], R[L::odS + i * DK + c], acc);
        for (int m = r + 1; m < kBC; ++m) acc = fmaf(R[L::oAk + m * kBC + r], R[L::odZ + m * DV + i], acc);
        if (r < Cn) {
            const int64_t vi = tix(r) * DV + i;
            store_elem<E>(p.gv, vi, load_elem<E>(p.wgate, vi) * acc);
            store_elem<E>(p.gw, vi, load_elem<E>(p.v, vi) * acc);
        }
    }
    __syncthreads();
    // pairwise passes; thread entries e = tid + kBT m: (r, c) = (e / DK, e % DK)
    float aq[NE], ak[NE], abk[NE], ag[NE];
#pragma unroll
    for (int m = 0; m < NE; ++m) aq[m] = ak[m] = abk[m] = ag[m] = 0.f;
    auto stage = [&](float* dst, int what) {   // 0 q, 1 k, 2 b k, 3 G
        for (int e = tid; e < kBC * DK; e += kBT) {
            const int r = e / DK, c = e % DK;
            float x;
            if (what == 3) {
                x = R[L::oG + e];
            } else if (r >= Cn) {
                x = 0.f;
            } else if (what == 0) {
                x = load_elem<E>(p.q, tix(r) * DK + c);
            } else {
                x = load_elem<E>(p.k, tix(r) * DK + c);
                if (what == 2) x *= load_elem<E>(p.beta, tix(r) * DK + c);
            }
            dst[r * LD + c] = x;
        }
    };
    // pass 1: Me (q, b k) and Mk (q, k) with G
    for (int e = tid; e < kBC * kBC; e += kBT) {
        sM1[(e / kBC) * CP + e % kBC] = R[L::odMe + e];
        sM2[(e / kBC) * CP + e % kBC] = R[L::odMk + e];
    }
    stage(R0, 0);
    stage(R2, 3);
    stage(R1, 2);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE; ++m) {   // Me terms
        const int e = tid + kBT * m, r = e / DK, c = e % DK;
        const float Gr = R2[r * LD + c];
        float row = 0.f, col = 0.f;
        for (int j = 0; j < kBC; ++j) {
            const float ex = __expf(j <= r ? Gr - R2[j * LD + c] : R2[j * LD + c] - Gr);
            if (j <= r) row = fmaf(sM1[r * CP + j], R1[j * LD + c] * ex, row);
            if (j >= r) col = fmaf(sM1[j * CP + r], R0[j * LD + c] * ex, col);
        }
        aq[m] += row;
        abk[m] += col;
        ag[m] += R0[r * LD + c] * row - R1[r * LD + c] * col;
    }
    __syncthreads();
    stage(R1, 1);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE; ++m) {   // Mk terms
        const int e = tid + kBT * m, r = e / DK, c = e % DK;
        const float Gr = R2[r * LD + c];
        float row = 0.f, col = 0.f;
        for (int j = 0; j < kBC; ++j) {
            const float ex = __expf(j <= r ? Gr - R2[j * LD + c] : R2[j * LD + c] - Gr);
            if (j <= r) row = fmaf(sM2[r * CP + j], R1[j * LD + c] * ex, row);
            if (j >= r) col = fmaf(sM2[j * CP + r], R0[j * LD + c] * ex, col);
        }
        aq[m] += row;
        ak[m] += col;
        ag[m] += R0[r * LD + c] * row - R1[r * LD + c] * col;
    }
    __syncthreads();
    // pass 2: Ae (k, b k) and Ak (k, k); b k -> R0
    for (int e = tid; e < kBC * kBC; e += kBT) {
        sM1[(e / kBC) * CP + e % kBC] = R[L::odAe + e];
        sM2[(e / kBC) * CP + e % kBC] = R[L::odAk + e];
    }
    stage(R0, 2);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + kBT * m, r = e / DK, c = e % DK;
        const float Gr = R2[r * LD + c];
        float rowe = 0.f, cole = 0.f, rowk = 0.f, colk = 0.f;
        for (int j = 0; j < kBC; ++j) {
            if (j == r) continue;
            const float ex = __expf(j < r ? Gr - R2[j * LD + c] : R2[j * LD + c] - Gr);
            if (j < r) {
                rowe = fmaf(sM1[r * CP + j], R0[j * LD + c] * ex, rowe);
                rowk = fmaf(sM2[r * CP + j], R1[j * LD + c] * ex, rowk);
            } else {
                cole = fmaf(sM1[j * CP + r], R1[j * LD + c] * ex, cole);
                colk = fmaf(sM2[j * CP + r], R1[j * LD + c] * ex, colk);
            }
        }
        const float kr = R1[r * LD + c], bkr = R0[r * LD + c];
        ak[m] += rowe + rowk + colk;
        abk[m] += cole;
        ag[m] += kr * rowe - bkr * cole + kr * rowk - kr * colk;
    }
    // row factors, outputs, dG
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + kBT * m, r = e / DK, c = e % DK;
        const float Gr = R2[r * LD + c];
        const float eg = __expf(Gr), eb = __expf(R2[(kBC - 1) * LD + c] - Gr);
        const float kr = R1[r * LD + c], bkr = R0[r * LD + c];
        const float dQh = R[L::odQh + e], dKh = R[L::odKh + e];
        const float dKb = R[L::odKb + e], dEb = R[L::odEb + e];
        const float q_ = aq[m] + dQh * eg;
        const float kpart = ak[m] + dKh * eg + dKb * eb;
        const float dbk = abk[m] + dEb * eb;
        const float qr = r < Cn ? load_elem<E>(p.q, tix(r) * DK + c) : 0.f;
        ag[m] += dKh * kr * eg + dQh * qr * eg - dKb * kr * eb - dEb * bkr * eb;
        if (r < Cn) {
            const float br = load_elem<E>(p.beta, tix(r) * DK + c);
            store_elem<E>(p.gq, tix(r) * DK + c, q_);
            store_elem<E>(p.gk, tix(r) * DK + c, kpart + dbk * br);
            store_elem<E>(p.gbeta, tix(r) * DK + c, dbk * kr);
        }
        R[L::odQh + e] = ag[m];
    }
    __syncthreads();
    if (tid < DK) {
        const int c = tid;
        float acc = sCol[c];
        for (int q2 = 0; q2 < TPC; ++q2) acc += sCol[DK * (1 + q2) + c];
        for (int r = kBC - 1; r >= 0; --r) {
            acc += R[L::odQh + r * DK + c];
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
    const dim3 blk(kBT);
    const unsigned chains = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * (DV / kBVT);
    hipLaunchKernelGGL((bwd2_prep_kernel<E, DK, DV>), dim3(static_cast<unsigned>(units)), blk, 0, s, a, ws, N);
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
        hipLaunchKernelGGL((bwd2_grads_kernel<E, DK, DV>), dim3(static_cast<unsigned>(units)), blk, 0, s, a, ws, N);
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
    const dim3 blk(kBT);
    const unsigned chains = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * (DV / kBVT);
    hipLaunchKernelGGL((bwd_prep_kernel<VAR, E, DK, DV>), dim3(static_cast<unsigned>(units)), blk, 0, s, a, ws, N);
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
        hipLaunchKernelGGL((bwd_grads_kernel<VAR, E, DK, DV>), dim3(static_cast<unsigned>(units)), blk, 0, s, a, ws, N);
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
    return dtype == 0 ? launch_bwd_var<VAR, F32>(a, s) : launch_bwd_var<VAR, BF16>(a, s);
}

}  // namespace

hipError_t launch_bwd(int variant, int dtype, const BwdArgs& a, hipStream_t s) {
    switch (variant) {
        case 0: return launch_bwd_dtype<0>(dtype, a, s);
        case 1: return launch_bwd_dtype<1>(dtype, a, s);
        case 2: return launch_bwd_dtype<2>(dtype, a, s);
        default: return dtype == 0 ? launch_bwd2_dtype<F32>(a, s) : launch_bwd2_dtype<BF16>(a, s);
    }
}

}  // namespace dr
