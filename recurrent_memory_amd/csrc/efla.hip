// Exact-flow step sizes (EFLA): beta_eff = (1 - exp(-beta |k|^2)) / |k|^2.
//
// The delta-rule write S' + beta (v - S' k) k^T is one Euler step of length
// beta of dS/dtau = (v - S k) k^T.  k k^T has the single non-zero eigenvalue
// |k|^2, so exp(-tau k k^T) = I - (1 - exp(-tau |k|^2)) / |k|^2 k k^T, and the
// flow over the same length lands on a delta-rule write with the step size
// above ("Delta-Rule Linear Attention" topic page, EFLA card: the rank-one
// dynamics collapse the matrix exponential and the input integral).
//
// One pass over k: LPR lanes share a query/key row, each loading 16 bytes, and
// the group of value heads that reads that row gets its step sizes from the
// same norm.  Pure HBM streaming; no LDS.
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kEflaThreads = 256;
constexpr int kEflaRows = 4;   // rows per lane group per iteration

template <typename E, int DK>
__global__ __launch_bounds__(kEflaThreads) void efla_beta_kernel(EflaArgs p, int64_t rows) {
    typedef typename E::T Raw;
    constexpr int EPL = 16 / E::bytes;   // elements per 16-byte load
    constexpr int LPR = DK / EPL;        // lanes per row: 8, 16 or 32
    constexpr int RPB = kEflaThreads / LPR;
    static_assert(LPR >= 8 && LPR <= 32, "row split");
    const int sub = threadIdx.x % LPR;
    const int G = p.H / p.Hk;            // value heads per query/key head
    // each group of LPR lanes takes kEflaRows rows, all loads issued before any use
    const int64_t stride = static_cast<int64_t>(gridDim.x) * RPB * kEflaRows;
    for (int64_t r0 = (static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR) * kEflaRows;
         r0 < rows; r0 += stride) {
        uint4 piece[kEflaRows];
        float b0[kEflaRows];   // beta of the first value head this lane serves, per row
#pragma unroll
        for (int u = 0; u < kEflaRows; ++u) {
            const int64_t r = r0 + u < rows ? r0 + u : rows - 1;
            piece[u] = *reinterpret_cast<const uint4*>(static_cast<const Raw*>(p.k) + r * DK + sub * EPL);
            const int64_t idx = (r / p.Hk) * p.H + (r % p.Hk) * G + sub;
            b0[u] = sub < G ? load_elem<E>(p.beta, idx) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kEflaRows; ++u) {
            float ss = 0.f;
            if constexpr (E::bytes == 4) {
                const float x[4] = {__uint_as_float(piece[u].x), __uint_as_float(piece[u].y),
                                    __uint_as_float(piece[u].z), __uint_as_float(piece[u].w)};
#pragma unroll
                for (int e = 0; e < 4; ++e) ss = fmaf(x[e], x[e], ss);
            } else {
                const uint32_t w[4] = {piece[u].x, piece[u].y, piece[u].z, piece[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(w[e] << 16);
                    const float hi = __uint_as_float(w[e] & 0xffff0000u);
                    ss = fmaf(lo, lo, ss);
                    ss = fmaf(hi, hi, ss);
                }
            }
            // rows occupy aligned groups of LPR lanes, so the xor butterfly stays inside one row
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
            const int64_t r = r0 + u;
            if (r >= rows) break;
            const int64_t tok = r / p.Hk;    // b * T + t
            const int hk = static_cast<int>(r % p.Hk);
            for (int i = sub; i < G; i += LPR) {
                const int64_t idx = tok * p.H + static_cast<int64_t>(hk) * G + i;
                const float beta = i == sub ? b0[u] : load_elem<E>(p.beta, idx);
                const float be = ss > 0.f ? -expm1f(-beta * ss) / ss : beta;
                store_elem<E>(p.beta_eff, idx, be);
            }
        }
    }
}

template <typename E>
hipError_t launch_dtype(const EflaArgs& a, hipStream_t s) {
    const int64_t rows = static_cast<int64_t>(a.B) * a.T * a.Hk;
    const int lpr = a.dk / (16 / E::bytes);
    const int64_t rpb = kEflaThreads / lpr * kEflaRows;
    const int64_t blocks = (rows + rpb - 1) / rpb;
    const dim3 grid(static_cast<unsigned>(blocks < (int64_t(1) << 20) ? blocks : (int64_t(1) << 20)));
    if (a.dk == 128) hipLaunchKernelGGL((efla_beta_kernel<E, 128>), grid, dim3(kEflaThreads), 0, s, a, rows);
    else hipLaunchKernelGGL((efla_beta_kernel<E, 64>), grid, dim3(kEflaThreads), 0, s, a, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_efla_beta(int dtype, const EflaArgs& a, hipStream_t s) {
    return dtype == 0 ? launch_dtype<F32>(a, s) : launch_dtype<BF16>(a, s);
}

}  // namespace dr
