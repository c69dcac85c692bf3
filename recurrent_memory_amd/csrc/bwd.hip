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
// Intermediates are fp32 and live in a workspace with one fixed-size record per
// (batch, head, chunk).  With fp32 inputs the products run on the fp32 matrix
// instruction; with bf16 inputs each fp32 operand is split into bf16 hi + lo and
// a product is hi*hi + hi*lo + lo*hi on the bf16 matrix cores (the chains use
// their own kernels for this, bwd_fchain_split / bwd_rchain_split).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "chunk_ops.h"
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
// Element q of the result in lane l is row i0 + 4 (l / 16) + q, column j0 + l % 16.
//
// SM (bf16 inputs): each fp32 operand is split into two bf16 values, x = hi + lo + e
// with hi and lo rounded to nearest even in turn, so |e| <= 2^-18 |x|, and the
// product is taken as hi*hi + hi*lo + lo*hi on the bf16 matrix cores with fp32
// accumulation.  The dropped lo*lo term and the split errors leave a relative
// error of about 2^-17 per product term; a 32-deep k step takes 3 instructions of
// the bf16 kind instead of 8 fp32 ones, each doing a quarter of the work per cycle.
// Otherwise (fp32 inputs) the products run on the fp32 matrix instruction.
// Operand layouts (g = l / 16, c = l % 16):
//   v_mfma_f32_16x16x32_bf16: lane l supplies A(i0 + c, k + 8 g + e) and
//     B(k + 8 g + e, j0 + c), e = 0..7;
//   v_mfma_f32_16x16x16_bf16: the same with 4 g + e, e = 0..3;
//   v_mfma_f32_16x16x4f32: A(i0 + c, k + g) and B(k + g, j0 + c).
template <typename E>
constexpr bool kSplitMM = std::is_same<E, BF16>::value;

__device__ __forceinline__ void split_bf16(float x, bf16_t& hi, bf16_t& lo) {
    hi = static_cast<bf16_t>(x);
    lo = static_cast<bf16_t>(x - static_cast<float>(hi));
}
// (AX, BX: the operand is exact in bf16, its lo part zero and its term skipped)
template <bool AX = false, bool BX = false>
__device__ __forceinline__ f32x4 mfma_split8(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                             const bf16x8& bl, f32x4 acc) {
    if constexpr (!AX) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    if constexpr (!BX) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <bool AX = false, bool BX = false>
__device__ __forceinline__ f32x4 mfma_split4(const bf16x4& ah, const bf16x4& al, const bf16x4& bh,
                                             const bf16x4& bl, f32x4 acc) {
    auto s = [](const bf16x4& v) { return __builtin_bit_cast(s16x4, v); };
    if constexpr (!AX) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(s(al), s(bh), acc, 0, 0, 0);
    if constexpr (!BX) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(s(ah), s(bl), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(s(ah), s(bh), acc, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// LDS transpose load of 16-bit elements: within each group of 16 lanes, lane p
// supplies the address of 4 consecutive elements and lane i receives element
// i % 4 of the piece addressed by lane 4 j + i / 4, j = 0..3.  Lane p of group g
// points at row r0 + 4 g + p / 4, columns c0 + 4 (p % 4) of a row-major array;
// lane c then holds rows r0 + 4 g + j of column c0 + c.
__device__ __forceinline__ bf16x4 tr_load_b16(const uint16_t* base, int ld, int r0, int c0, int g, int c) {
    const uint16_t* q = base + (r0 + 4 * g + (c >> 2)) * ld + c0 + 4 * (c & 3);
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(q)));
}
// An operand accessor whose values are exact in bf16 (bf16 inputs as loaded, or
// zero): its lo part is zero, so it is only rounded, and the products with its
// lo part are skipped.
template <class F>
struct Exact {
    F f;
    __device__ __forceinline__ float operator()(int a, int b) const { return f(a, b); }
};
template <class F>
__device__ __forceinline__ Exact<F> exact(const F& f) { return Exact<F>{f}; }
template <class F>
struct IsExact : std::false_type {};
template <class F>
struct IsExact<Exact<F>> : std::true_type {};

template <class F>
__device__ __forceinline__ void split_one(const F& A, int i, int j, bf16_t& h, bf16_t& lo) {
    if constexpr (IsExact<F>::value) {
        h = static_cast<bf16_t>(A(i, j));
        lo = static_cast<bf16_t>(0.f);
    } else {
        split_bf16(A(i, j), h, lo);
    }
}
// operand pieces of lane (g, c) for a k step of 8 N: A(ai, k + N g + e) and B(k + N g + e, bj)
template <int N, class V, class FA, class FB>
__device__ __forceinline__ void split_operands(V& ah, V& al, V& bh, V& bl, int ai, int bj, int k, int g,
                                               const FA& A, const FB& B) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
        bf16_t h, lo;
        split_one(A, ai, k + N * g + e, h, lo);
        ah[e] = h;
        al[e] = lo;
        split_one(B, k + N * g + e, bj, h, lo);
        bh[e] = h;
        bl[e] = lo;
    }
}

template <bool SM, class FA, class FB>
__device__ __forceinline__ f32x4 mm_tile(f32x4 acc, int i0, int j0, int k0, int k1, const FA& A,
                                         const FB& B) {
    const int l = threadIdx.x & 63;
    const int ai = i0 + (l & 15), bj = j0 + (l & 15), g = l >> 4;
    int k = k0;
    if constexpr (SM) {
#pragma unroll 4
        for (; k + 32 <= k1; k += 32) {
            bf16x8 ah, al, bh, bl;
            split_operands<8>(ah, al, bh, bl, ai, bj, k, g, A, B);
            acc = mfma_split8<IsExact<FA>::value, IsExact<FB>::value>(ah, al, bh, bl, acc);
        }
        if (k + 16 <= k1) {
            bf16x4 ah, al, bh, bl;
            split_operands<4>(ah, al, bh, bl, ai, bj, k, g, A, B);
            acc = mfma_split4<IsExact<FA>::value, IsExact<FB>::value>(ah, al, bh, bl, acc);
            k += 16;
        }
    }
#pragma unroll 16
    for (; k < k1; k += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(ai, k + g), B(k + g, bj), acc, 0, 0, 0);
    return acc;
}

// The state chains with fp32 inputs (bwd_fchain_kernel, bwd_rchain_kernel; bf16
// inputs take the split-operand chains below) use two more fp32 forms:
// mm_tile with the k range split into two interleaved accumulation chains
// (k1 - k0 a multiple of 8), which the matrix core runs back to back,
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

// and two tiles with the same rows i0 and columns j0, j1, one A read feeding
// both accumulation chains.
template <class FA, class FB>
__device__ __forceinline__ void mm_tile2(f32x4& acc0, f32x4& acc1, int i0, int j0, int j1, int k0, int k1,
                                         const FA& A, const FB& B) {
    const int l = threadIdx.x & 63;
    const int ai = i0 + (l & 15), b0 = j0 + (l & 15), b1 = j1 + (l & 15), g = l >> 4;
#pragma unroll 16
    for (int k = k0; k < k1; k += 4) {
        const float a = A(ai, k + g);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, B(k + g, b0), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, B(k + g, b1), acc1, 0, 0, 0);
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
template <bool ROW, bool SM, class FM, class FX, class FG>
__device__ __forceinline__ f32x4 pair_tile(int r0, int c0, const FM& M, const FX& X, const FG& G) {
    const int l = threadIdx.x & 63;
    const int I = r0 / 16;
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    for (int J = ROW ? 0 : I; ROW ? (J <= I) : (J < kBC / 16); ++J) {
        const int ref = ROW ? 16 * J + 15 : 16 * J;
        const f32x4 acc = mm_tile<SM>(
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

// Loop over the elements e = tid, tid + STRIDE, ... < N of a tile with the trip
// count fixed at compile time and the body unrolled by 8, so that the global
// loads of 8 iterations are issued before the first of them is waited for (with
// a run-time trip count each iteration waited for its own loads; unrolling
// completely made the gradient kernel spill registers).  Loads in the body read
// a valid address on every lane (rows past the end of the sequence are clamped
// to its last row and the value is selected away afterwards): a load under a
// branch is waited for inside the branch.
#define DR_TILE_FOR(e, N, STRIDE)                         \
    static_assert((N) % (STRIDE) == 0, "tile split");     \
    _Pragma("unroll 8") for (int e##_it = 0, e = tid; e##_it < (N) / (STRIDE); ++e##_it, e += (STRIDE))

// T = (I + diag(rs) A)^-1 for the strictly lower kBC x kBC matrix A (rs == nullptr:
// no row scaling), called by every thread of the workgroup, in 16-row blocks:
//   1. the four diagonal blocks T_ii = L_ii^-1 (L = I + diag(rs) A) by substitution
//      in registers, one lane of wave 0 per column of one block;
//   2. the blocks below the diagonal, T_ij = -T_ii sum_{j <= k < i} L_ik T_kj, for
//      block column j on wave j, block rows i = j + 1, ... in turn, each as two
//      matrix-core products with the partial sum passed through Z (16 x 20 floats
//      per wave, 3 waves).
// (Substituting whole 64-row columns, one lane per column, kept seven of the
// eight waves idle for the length of the substitution.)
template <bool SM>
__device__ __forceinline__ void unit_lower_inverse_blocked(const float* A, int lda, const float* rs, float* T,
                                                           int ldt, float* Z) {
    static_assert(kBC == 64, "four 16-row blocks");
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    if (w == 0) {
        const int o = 16 * (l >> 4), col = l & 15;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < r; ++j) acc[j & 3] = fmaf(A[(o + r) * lda + o + j], t[j], acc[j & 3]);
            float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            if (rs) sum *= rs[o + r];
            t[r] = (r == col ? 1.f : 0.f) - sum;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) T[(o + r) * ldt + o + col] = t[r];
    }
    for (int e = tid; e < kBC * kBC; e += blockDim.x) {   // the blocks above the diagonal
        const int r = e / kBC, c = e % kBC;
        if (c / 16 > r / 16) T[r * ldt + c] = 0.f;
    }
    __syncthreads();
    if (w < 3) {
        const int j0 = 16 * w;
        float* z = Z + w * (16 * 20);
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        for (int i0 = j0 + 16; i0 < kBC; i0 += 16) {
            // Z = sum_{j <= k < i} L_ik T_kj: rows of L left of the diagonal block are rs A
            const f32x4 zz = mm_tile<SM>(z4, i0, j0, j0, i0,
                                     [&](int r, int k) { return rs ? rs[r] * A[r * lda + k] : A[r * lda + k]; },
                                     [&](int k, int c) { return T[k * ldt + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) z[(4 * (l >> 4) + q) * 20 + (l & 15)] = zz[q];
            // T_ij = -T_ii Z (the wave's own LDS writes are seen by its later reads)
            const f32x4 tt = mm_tile<SM>(z4, 0, 0, 0, 16, [&](int r, int k) { return T[(i0 + r) * ldt + i0 + k]; },
                                     [&](int k, int c) { return z[k * 20 + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) T[(i0 + 4 * (l >> 4) + q) * ldt + j0 + (l & 15)] = -tt[q];
        }
    }
    __syncthreads();
}

// Workspace record of one (batch, head, chunk), in floats.  The forward chain
// writes Vt over U (each lane reads its U elements before it writes the same Vt
// elements; nothing else reads U).  The gradient kernel, the record's last
// reader, keeps three [C][DK] intermediates (dQhat, dX, dKbar) in it; they
// occupy the field it never reads (W) and those it has read before writing them
// (Vt, dVt), so the record grows only where 3 DK exceeds DK + 2 DV.  (dW goes
// from its accumulators to LDS.)
template <int DK, int DV>
struct BwdWs {
    static constexpr bool kRowGate = false;
    static constexpr int64_t C = kBC;
    static constexpr int64_t oG = 0;                // G            [C][DK]
    static constexpr int64_t oT = oG + C * DK;      // T            [C][C]
    static constexpr int64_t oAb = oT + C * C;      // Abar         [C][C]
    static constexpr int64_t oMq = oAb + C * C;     // Mq           [C][C]
    static constexpr int64_t oQh = oMq + C * C;     // Qhat         [C][DK]
    static constexpr int64_t oKb = oQh + C * DK;    // Kbar         [C][DK]
    static constexpr int64_t oKh = oKb + C * DK;    // Khat         [C][DK]
    static constexpr int64_t oGam = oKh + C * DK;   // gamma        [DK]
    static constexpr int64_t oS = oGam + DK;        // S entering   [DV][DK]
    static constexpr int64_t odS = oS + DV * DK;    // dS leaving   [DV][DK]
    static constexpr int64_t oW = odS + DV * DK;    // W            [C][DK]
    static constexpr int64_t oU = oW + C * DK;      // U, then Vt   [C][DV]
    static constexpr int64_t oVt = oU;              // Vt           [C][DV]
    static constexpr int64_t odVt = oVt + C * DV;   // dVt          [C][DV]
    // the gradient kernel's intermediates, over W, Vt, dVt
    static constexpr int64_t odQh = oW;             // dQhat, then dG [C][DK]
    static constexpr int64_t odX = odQh + C * DK;   // dX           [C][DK]
    static constexpr int64_t odKb = odX + C * DK;   // dKbar        [C][DK]
    static constexpr int64_t size = (odVt + C * DV > odKb + C * DK) ? odVt + C * DV : odKb + C * DK;
    static constexpr int64_t oEb = oKb;             // (the split-gate chains' Ebar; unused here)
};

// Workspace record of the ungated and scalar-decay forms.  Their decay is one
// number per row, so G is kept per row and the decay-scaled copies of q and k
// (Qhat = q e^G, Khat = k e^G, Kbar = k e^{G_C - G}) are rebuilt from the inputs
// where they are read, with the same factors: less workspace, and that much less
// written by the factor kernel and read by the others.  The gradient kernel's
// intermediates overlay W, Vt and dVt as in BwdWs.
template <int DK, int DV>
struct BwdWsS {
    static constexpr bool kRowGate = true;
    static constexpr int64_t C = kBC;
    static constexpr int64_t oG = 0;                // G            [C] (one value per row)
    static constexpr int64_t oT = oG + C;           // T            [C][C]
    static constexpr int64_t oAb = oT + C * C;      // Abar         [C][C]
    static constexpr int64_t oMq = oAb + C * C;     // Mq           [C][C]
    static constexpr int64_t oGam = oMq + C * C;    // gamma        [DK]
    static constexpr int64_t oS = oGam + DK;        // S entering   [DV][DK]
    static constexpr int64_t odS = oS + DV * DK;    // dS leaving   [DV][DK]
    static constexpr int64_t oW = odS + DV * DK;    // W            [C][DK]
    static constexpr int64_t oU = oW + C * DK;      // U, then Vt   [C][DV]
    static constexpr int64_t oVt = oU;              // Vt           [C][DV]
    static constexpr int64_t odVt = oVt + C * DV;   // dVt          [C][DV]
    static constexpr int64_t odQh = oW;             // dQhat, then dG [C][DK]
    static constexpr int64_t odX = odQh + C * DK;   // dX           [C][DK]
    static constexpr int64_t odKb = odX + C * DK;   // dKbar        [C][DK]
    static constexpr int64_t size = (odVt + C * DV > odKb + C * DK) ? odVt + C * DV : odKb + C * DK;
};
// record layout of a one-step-size form
template <int VAR, int DK, int DV>
using BwdWs1 = typename std::conditional<(VAR <= 1), BwdWsS<DK, DV>, BwdWs<DK, DV>>::type;

// Workspace record of the split-gate form (Gated DeltaNet-2).  The names the
// state chains share with the single-step-size record carry the split-gate
// factors: oU holds Ut, oVt holds Y, odVt holds dY and oMq holds Me.
template <int DK, int DV>
struct BwdWs2 {
    static constexpr bool kRowGate = false;
    static constexpr int64_t C = kBC;
    static constexpr int64_t oG = 0;                // G        [C][DK]
    static constexpr int64_t oT = oG + C * DK;      // T        [C][C]
    static constexpr int64_t oAk = oT + C * C;      // Ak       [C][C]
    static constexpr int64_t oMk = oAk + C * C;     // Mk       [C][C]
    static constexpr int64_t oKb = oMk + C * C;     // Kbar     [C][DK]
    static constexpr int64_t oEb = oKb + C * DK;    // Ebar
    static constexpr int64_t oKh = oEb + C * DK;    // Khat
    static constexpr int64_t oZ = oKh + C * DK;     // Z = Ak X [C][DV]
    static constexpr int64_t oGam = oZ + C * DV;    // gamma    [DK]
    static constexpr int64_t oS = oGam + DK;        // S entering [DV][DK]
    static constexpr int64_t odS = oS + DV * DK;    // dS leaving [DV][DK]
    // fields the gradient kernel never reads (Me, W, Qhat, Ut) or reads first (Y,
    // then dY): its intermediates overlay them, in the order they are first
    // written.  Those written before dY is read (dMe, dMk, dQhat, dEbar, dKbar)
    // must end before dY, hence the padding when C + DK > 2 DV.
    static constexpr int64_t kPre = 2 * C * C + 3 * C * DK;
    static constexpr int64_t kAvail = C * C + 2 * C * DK + 2 * C * DV;
    static constexpr int64_t oMq = odS + DV * DK;   // Me       [C][C]
    static constexpr int64_t oW = oMq + C * C;      // W        [C][DK]
    static constexpr int64_t oQh = oW + C * DK;     // Qhat     [C][DK]
    static constexpr int64_t oU = oQh + C * DK;     // Ut = T Z [C][DV]
    static constexpr int64_t oVt = oU + C * DV;     // Y        [C][DV]
    static constexpr int64_t odVt = oVt + C * DV + (kPre > kAvail ? kPre - kAvail : 0);   // dY [C][DV]
    static constexpr int64_t odMe = oMq;            // dMe, dMk [C][C]
    static constexpr int64_t odMk = odMe + C * C;
    static constexpr int64_t odQh = odMk + C * C;   // dQhat (then dG), dEbar, dKbar [C][DK]
    static constexpr int64_t odEb = odQh + C * DK;
    static constexpr int64_t odKb = odEb + C * DK;
    static constexpr int64_t odZ = odKb + C * DK;   // dZ       [C][DV]
    static constexpr int64_t odKh = odZ + C * DV;   // dKhat    [C][DK]
    static constexpr int64_t odAe = odKh + C * DK;  // dAe, dAk [C][C]
    static constexpr int64_t odAk = odAe + C * C;
    static constexpr int64_t size = (odVt + C * DV > odAk + C * C) ? odVt + C * DV : odAk + C * C;
    static_assert(odKb + C * DK <= odVt, "intermediates written before dY is read end before it");
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
    typedef BwdWs1<VAR, DK, DV> L;
    constexpr int LD = (DK > DV ? DK : DV) + 4;   // padded row stride (4 mod 64 words)
    __shared__ __attribute__((aligned(16))) float sK[kBC * (DK + 4)];
    __shared__ __attribute__((aligned(16))) float sX[kBC * LD];   // q, then beta Khat, then beta v
    __shared__ __attribute__((aligned(16))) float sG[kBC * (DK + 4)];
    __shared__ float sA[kBC * (kBC + 4)];
    __shared__ float sT[kBC * (kBC + 4)];
    __shared__ float sBeta[kBC + 1];              // (+ a spare slot, never read)
    __shared__ float sZ[3 * 16 * 20];             // scratch of the blocked inverse
    const int u = blockIdx.x, tid = threadIdx.x;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;

    const float4 z4v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto put = [](float* dst, float4 x) { *reinterpret_cast<float4*>(dst) = x; };
    // beta first, so that its wait is covered by the tile loads (every thread
    // loads from a valid row: no load sits in a branch)
    const float bt = VAR == 4 ? 1.f : load_elem<E>(p.beta, tok_index(p, b, t0 + min(tid % kBC, Cn - 1), h));
    DR_TILE_FOR(e, kBC * DK / 4, kGT) {   // four consecutive channels per thread
        const int r = 4 * e / DK, c = 4 * e % DK;
        const bool ok = r < Cn;
        const int64_t ti = tok_index(p, b, t0 + min(r, Cn - 1), h);
        const int64_t qi = qk_index(p, b, t0 + min(r, Cn - 1), h);
        const float4 kv = load4<E>(p.k, qi * DK + c), qv = load4<E>(p.q, qi * DK + c);
        float4 gv = z4v;
        if constexpr (VAR == 1) {
            const float g1 = load_elem<E>(p.g, ti);
            gv = make_float4(g1, g1, g1, g1);
        }
        if constexpr (VAR >= 2) {
            gv = load4<E>(p.g, ti * DK + c);
            gv = make_float4(fmaxf(gv.x, kLogDecayFloor), fmaxf(gv.y, kLogDecayFloor),
                             fmaxf(gv.z, kLogDecayFloor), fmaxf(gv.w, kLogDecayFloor));
        }
        put(sK + r * (DK + 4) + c, ok ? kv : z4v);
        put(sX + r * LD + c, ok ? qv : z4v);
        put(sG + r * (DK + 4) + c, ok ? gv : z4v);
    }
    // FG^2-GDN (VAR 4): the step sizes sit on the key side (E = beta ⊙ k in the
    // columns of Abar and Mq and in Kbar); the rows take 1
    // (threads past the chunk write a spare slot: a store under a branch would
    // pull the load of bt into the branch and wait for it there)
    sBeta[min(tid, kBC)] = tid < Cn ? bt : 0.f;
    // v, loaded now and used after W: its loads overlap the factor products
    constexpr int NV4 = kBC * DV / 4 / kGT;
    float4 pv[NV4];
#pragma unroll
    for (int j = 0; j < NV4; ++j) {
        const int e = tid + kGT * j, r = 4 * e / DV, i = 4 * e % DV;
        pv[j] = load4<E>(p.v, tok_index(p, b, t0 + min(r, Cn - 1), h) * DV + i);
    }
    __syncthreads();
    if (tid < DK) {   // in-chunk cumulative log-decay per channel
        float acc = 0.f;
        for (int r = 0; r < kBC; ++r) {
            acc += sG[r * (DK + 4) + tid];
            sG[r * (DK + 4) + tid] = acc;
        }
    }
    __syncthreads();
    if constexpr (L::kRowGate) {
        if (tid < kBC) R[L::oG + tid] = sG[tid * (DK + 4)];
    } else {
        DR_TILE_FOR(e, kBC * DK / 4, kGT) {
            const int r = 4 * e / DK, c = 4 * e % DK;
            put(R + L::oG + 4 * e, *reinterpret_cast<const float4*>(sG + r * (DK + 4) + c));
        }
    }
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
                ab = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK,
                             [&](int r, int c) { return sK[r * (DK + 4) + c] * __expf(sG[r * (DK + 4) + c] - gref[c]); }, Bk);
                mq = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK,
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
            // (q and k as loaded: exact in bf16 with bf16 inputs)
            const f32x4 ab = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, exact([&](int r, int c) { return sK[r * (DK + 4) + c]; }),
                                     exact([&](int c, int j) { return sK[j * (DK + 4) + c]; }));
            const f32x4 mq = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, exact([&](int r, int c) { return sX[r * LD + c]; }),
                                     exact([&](int c, int j) { return sK[j * (DK + 4) + c]; }));
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
    unit_lower_inverse_blocked<kSplitMM<E>>(sA, kBC + 4, sBeta, sT, kBC + 4, sZ);
    for (int e = tid; e < kBC * kBC; e += kGT) R[L::oT + e] = sT[(e / kBC) * (kBC + 4) + e % kBC];
    // key and query factors; sX becomes X = beta Khat
    DR_TILE_FOR(e, kBC * DK / 4, kGT) {
        const int r = 4 * e / DK, c = 4 * e % DK;
        const float4 G = *reinterpret_cast<const float4*>(sG + r * (DK + 4) + c);
        const float4 GC = *reinterpret_cast<const float4*>(sG + (kBC - 1) * (DK + 4) + c);
        const float4 kk = *reinterpret_cast<const float4*>(sK + r * (DK + 4) + c);
        const float4 qq = *reinterpret_cast<const float4*>(sX + r * LD + c);
        const float4 eg = make_float4(__expf(G.x), __expf(G.y), __expf(G.z), __expf(G.w));
        float4 kb = make_float4(kk.x * __expf(GC.x - G.x), kk.y * __expf(GC.y - G.y), kk.z * __expf(GC.z - G.z),
                                kk.w * __expf(GC.w - G.w));
        if constexpr (VAR == 4) {
            const float4 bv = load4<E>(p.beta, tok_index(p, b, t0 + min(r, Cn - 1), h) * DK + c);
            kb = make_float4(kb.x * bv.x, kb.y * bv.y, kb.z * bv.z, kb.w * bv.w);
        }
        const float4 kh = make_float4(kk.x * eg.x, kk.y * eg.y, kk.z * eg.z, kk.w * eg.w);
        if constexpr (!L::kRowGate) {
            put(R + L::oKh + 4 * e, kh);
            put(R + L::oQh + 4 * e, make_float4(qq.x * eg.x, qq.y * eg.y, qq.z * eg.z, qq.w * eg.w));
            put(R + L::oKb + 4 * e, kb);
        }
        const float br = sBeta[r];
        put(sX + r * LD + c, make_float4(br * kh.x, br * kh.y, br * kh.z, br * kh.w));
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DK / 16); t += kGW) {   // W = T X
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * (kBC + 4) + j]; },
                                  [&](int j, int c) { return sX[j * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oW + (r0 + 4 * (l >> 4) + q) * DK + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NV4; ++j) {   // Y = beta v
        const int e = tid + kGT * j, r = 4 * e / DV, i = 4 * e % DV;
        const float br = sBeta[r];
        put(sX + r * LD + i, r < Cn ? make_float4(br * pv[j].x, br * pv[j].y, br * pv[j].z, br * pv[j].w) : z4v);
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DV / 16); t += kGW) {   // U = T Y
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * (kBC + 4) + j]; },
                                  [&](int j, int i) { return sX[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oU + (r0 + 4 * (l >> 4) + q) * DV + c0 + (l & 15)] = acc[q];
    }
}

// The factor kernel of the ungated and scalar-decay forms with bf16 inputs.  q,
// k and v are exact in bf16, so they are staged as bf16 (half the LDS of fp32
// copies, v over q once Mq is formed: two workgroups fit on a CU and each covers
// the other's loads) and the products that take them need no split: Abar = K K^T
// and Mq = Q K^T are single bf16 products, and W = T diag(beta e^G) K, U = T
// diag(beta) V take the per-row factors into T's columns, split T and use K and
// V as loaded.  G is summed in row order, as bwd_prep_kernel does.
template <int VAR, int DK, int DV>
__global__ __launch_bounds__(kGT, 2) void bwd_prep_bf16_kernel(BwdArgs p, float* ws, int N) {
    static_assert(VAR <= 1, "one decay value per row");
    typedef BwdWsS<DK, DV> L;
    typedef BF16 E;
    constexpr int LB = DK + 8;                    // bf16 q, k rows
    constexpr int LV = DV + 8;                    // bf16 v rows
    constexpr int LQV = LB > LV ? LB : LV;
    constexpr int LF = kBC + 4;                   // fp32 C x C rows
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBC * LB];
    __shared__ __attribute__((aligned(16))) uint16_t sQV[kBC * LQV];   // q, then v
    __shared__ __attribute__((aligned(16))) float sA[kBC * LF];
    __shared__ __attribute__((aligned(16))) float sT[kBC * LF];
    __shared__ float sBeta[kBC + 1];              // (+ a spare slot, never read)
    __shared__ float sG[kBC];                     // raw gates, then G
    __shared__ float sF[kBC];                     // beta_j e^{G_j}
    __shared__ float sZ[3 * 16 * 20];             // scratch of the blocked inverse
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, cl = l & 15;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // beta and the raw gate of each row (rows past the end: 0)
    const float bt = load_elem<E>(p.beta, tok_index(p, b, t0 + min(tid % kBC, Cn - 1), h));
    float gr = 0.f;
    if constexpr (VAR == 1) gr = load_elem<E>(p.g, tok_index(p, b, t0 + min(tid % kBC, Cn - 1), h));
    // q, k and v rows, 16 bytes a piece (rows past the end zeroed)
    constexpr int PK = DK / 8, PV = DV / 8;
    static_assert(kBC * PK % kGT == 0 && kBC * PV % kGT == 0, "piece split");
    uint4 pq[kBC * PK / kGT], pk[kBC * PK / kGT], pv[kBC * PV / kGT];
#pragma unroll
    for (int j = 0; j < kBC * PK / kGT; ++j) {
        const int e = tid + kGT * j, r = e / PK, c = 8 * (e % PK);
        const int64_t qi = qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + c;
        pq[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qi);
        pk[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + qi);
    }
#pragma unroll
    for (int j = 0; j < kBC * PV / kGT; ++j) {
        const int e = tid + kGT * j, r = e / PV, c = 8 * (e % PV);
        pv[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) +
                                                tok_index(p, b, t0 + min(r, Cn - 1), h) * DV + c);
    }
    auto sel = [](bool ok, uint4 x) { return ok ? x : make_uint4(0, 0, 0, 0); };
    sBeta[min(tid, kBC)] = tid < Cn ? bt : 0.f;
    if (tid < kBC) sG[tid] = tid < Cn ? gr : 0.f;
#pragma unroll
    for (int j = 0; j < kBC * PK / kGT; ++j) {
        const int e = tid + kGT * j, r = e / PK, c = 8 * (e % PK);
        *reinterpret_cast<uint4*>(sQV + r * LQV + c) = sel(r < Cn, pq[j]);
        *reinterpret_cast<uint4*>(sK + r * LB + c) = sel(r < Cn, pk[j]);
    }
    __syncthreads();
    // G_r = sum_{j <= r} g_j in row order, lane r of wave 0
    float G = 0.f;
    if (w == 0) {
#pragma unroll 8
        for (int j = 0; j < kBC; ++j) G += j <= l ? sG[j] : 0.f;
    }
    __syncthreads();
    if (w == 0) {
        sG[l] = G;
        sF[l] = sBeta[l] * __expf(G);
        R[L::oG + l] = G;
    }
    __syncthreads();
    if (tid < DK) R[L::oGam + tid] = __expf(sG[kBC - 1]);
    // Abar (strictly lower) and Mq (lower, diagonal included): K K^T and Q K^T,
    // then e^{G_r - G_j}
    for (int t = w; t < 16; t += kGW) {
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const uint16_t* krow = sK + (j0 + cl) * LB;
        const f32x4 ab = Ops<BF16>::template nat<DK>(z4, sK + (r0 + cl) * LB, krow, g);
        const f32x4 mq = Ops<BF16>::template nat<DK>(z4, sQV + (r0 + cl) * LQV, krow, g);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 4 * g + q, j = j0 + cl;
            const float ex = (VAR == 1 && j <= r) ? __expf(sG[r] - sG[j]) : 1.f;
            const float a_ = j < r ? ab[q] * ex : 0.f;
            sA[r * LF + j] = a_;
            R[L::oAb + r * kBC + j] = a_;
            R[L::oMq + r * kBC + j] = j <= r ? mq[q] * ex : 0.f;
        }
    }
    __syncthreads();
    // v over q (Mq is formed)
#pragma unroll
    for (int j = 0; j < kBC * PV / kGT; ++j) {
        const int e = tid + kGT * j, r = e / PV, c = 8 * (e % PV);
        *reinterpret_cast<uint4*>(sQV + r * LQV + c) = sel(r < Cn, pv[j]);
    }
    // T = (I + diag(beta) Abar)^-1
    unit_lower_inverse_blocked<true>(sA, LF, sBeta, sT, LF, sZ);
    for (int e = tid; e < kBC * kBC; e += kGT) R[L::oT + e] = sT[(e / kBC) * LF + e % kBC];
    __syncthreads();
    // W = (T diag(beta e^G)) K and U = (T diag(beta)) V: A = T with its column
    // factors, split; B as loaded (exact), read by the LDS transpose load.  Lane
    // (g, c) holds k = k0 + 4 g + e and k0 + 16 + 4 g + e for both operands.
    auto tfrag = [&](int r0, int k0, bool withG, bf16x8& ah, bf16x8& al) {
        const float* trow = sT + (r0 + cl) * LF + k0 + 4 * g;
        const float4 a0 = *reinterpret_cast<const float4*>(trow), a1 = *reinterpret_cast<const float4*>(trow + 16);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = k0 + 4 * g + (e < 4 ? e : 12 + e);
            bf16_t hh, ll;
            split_bf16(av[e] * (withG ? sF[j] : sBeta[j]), hh, ll);
            ah[e] = hh;
            al[e] = ll;
        }
    };
    const bf16x8 zb = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int t = w; t < (kBC / 16) * (DK / 16); t += kGW) {
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        f32x4 acc = z4;
#pragma unroll
        for (int k0 = 0; k0 < kBC; k0 += 32) {
            bf16x8 ah, al;
            tfrag(r0, k0, true, ah, al);
            const bf16x8 bh = cat8(tr_load_b16(sK, LB, k0, c0, g, cl), tr_load_b16(sK, LB, k0 + 16, c0, g, cl));
            acc = mfma_split8<false, true>(ah, al, bh, zb, acc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oW + (r0 + 4 * g + q) * DK + c0 + cl] = acc[q];
    }
    for (int t = w; t < (kBC / 16) * (DV / 16); t += kGW) {
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        f32x4 acc = z4;
#pragma unroll
        for (int k0 = 0; k0 < kBC; k0 += 32) {
            bf16x8 ah, al;
            tfrag(r0, k0, false, ah, al);
            const bf16x8 bh = cat8(tr_load_b16(sQV, LQV, k0, c0, g, cl), tr_load_b16(sQV, LQV, k0 + 16, c0, g, cl));
            acc = mfma_split8<false, true>(ah, al, bh, zb, acc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oU + (r0 + 4 * g + q) * DV + c0 + cl] = acc[q];
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
    static_assert(!kSplitMM<E>, "fp32 inputs; bf16 inputs take the split-operand chain");
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
    if (p.S0) {   // (the branch outside the loop: inside, each load was waited for in turn)
        DR_TILE_FOR(e, kBVT * DK, kCT) {
            const int i = e / DK, c = e % DK;
            sS[i * SS + c] = p.S0[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c];
        }
    } else {
        DR_TILE_FOR(e, kBVT * DK, kCT) sS[(e / DK) * SS + e % DK] = 0.f;
    }
    // the next chunk's operands are fetched into registers while this chunk's
    // products run, and written to LDS at the top of the next step
    const int w = tid >> 6, l = tid & 63;
    constexpr int NP = kBC * DK / 4 / kCT;          // 16-byte pieces per thread per operand
    constexpr int MT = (kBC / 16) * (kBVT / 16) / kCW;  // Vt tiles per wave
    float4 pW[NP], pK[NP], pE[SPLIT ? NP : 1];
    float pU[MT][4];
    float pG = 0.f;
    // per-row decay (row-gate record): Kbar = k e^{G_C - G_r}, k fetched raw
    float pGr[L::kRowGate ? NP : 1], pGC = 0.f;
    float4 pXw = make_float4(0.f, 0.f, 0.f, 0.f), pXv = pXw;   // split gates: w and v of X = w v
    static_assert(kBC * kBVT == 4 * kCT, "X: four columns per thread");
    auto fetch = [&](int n) {
        const float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        if constexpr (SPLIT) {   // this tile's value columns, rows past the end from the last row
            const int t0 = n * kBC, Cn = min(kBC, p.T - t0), r = 4 * tid / kBVT, i = 4 * tid % kBVT;
            const int64_t vi = tok_index(p, b, t0 + min(r, Cn - 1), h) * DV + i0 + i;
            pXw = load4<E>(p.wgate, vi);
            pXv = load4<E>(p.v, vi);
        }
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            pW[j] = *reinterpret_cast<const float4*>(R + L::oW + idx);
            if constexpr (L::kRowGate) {   // rows past the end from the last row, zeroed when stored
                const int r = idx / DK, c = idx % DK, Cn = min(kBC, p.T - n * kBC);
                pK[j] = load4<E>(p.k, qk_index(p, b, n * kBC + min(r, Cn - 1), h) * DK + c);
                pGr[j] = R[L::oG + r];
            } else {
                pK[j] = *reinterpret_cast<const float4*>(R + L::oKb + idx);
            }
            if constexpr (SPLIT) pE[j] = *reinterpret_cast<const float4*>(R + L::oEb + idx);
        }
        if constexpr (L::kRowGate) pGC = R[L::oG + kBC - 1];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = w + kCW * m, r0 = 16 * (t / (kBVT / 16)), c0 = 16 * (t % (kBVT / 16));
#pragma unroll
            for (int q = 0; q < 4; ++q) pU[m][q] = R[L::oU + (r0 + 4 * (l >> 4) + q) * DV + i0 + c0 + (l & 15)];
        }
        pG = R[L::oGam + min(tid, DK - 1)];   // every lane loads: no branch, no wait in it
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
            if constexpr (L::kRowGate) {
                const bool ok = idx / DK < min(kBC, p.T - n * kBC);
                const float f = __expf(pGC - pGr[j]);
                const float4 kv = pK[j];
                put4(sKb, SK, idx, ok ? make_float4(kv.x * f, kv.y * f, kv.z * f, kv.w * f) : make_float4(0.f, 0.f, 0.f, 0.f));
            } else {
                put4(sKb, SK, idx, pK[j]);
            }
            if constexpr (SPLIT) put4(sEb, SK, idx, pE[j]);
        }
        float uu[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) uu[m][q] = pU[m][q];
        sGam[min(tid, DK - 1)] = pG;   // lanes past DK rewrite the last entry with its own value
        if constexpr (SPLIT) {   // X = w v for this tile's value columns (fetched a step ahead)
            const int Cn = min(kBC, p.T - n * kBC), r = 4 * tid / kBVT, i = 4 * tid % kBVT;
            *reinterpret_cast<float4*>(sXt + r * SV + i) =
                r < Cn ? make_float4(pXw.x * pXv.x, pXw.y * pXv.y, pXw.z * pXv.z, pXw.w * pXv.w)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
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
    static_assert(!kSplitMM<E>, "fp32 inputs; bf16 inputs take the split-operand chain");
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
    if (p.dST) {
        DR_TILE_FOR(e, kBVT * DK, kCT) {
            const int i = e / DK, c = e % DK;
            sdS[i * SD + c] = p.dST[(static_cast<int64_t>(bh) * DV + i0 + i) * DK + c];
        }
    } else {
        DR_TILE_FOR(e, kBVT * DK, kCT) sdS[(e / DK) * SD + e % DK] = 0.f;
    }
    // the previous chunk's operands are fetched into registers during this step
    constexpr int NP = kBC * DK / 4 / kCT;
    constexpr int NM = kBC * kBC / 4 / kCT;
    constexpr int NO = kBC * kBVT / kCT;
    float4 pM[NM], pA[NP], pQ[NP], pW[NP];
    float pO[NO];
    float pG = 0.f;
    // per-row decay (row-gate record): Kbar = k e^{G_C - G_r}, Qhat = q e^{G_r}, q and k fetched raw
    float pGr[L::kRowGate ? NP : 1], pGC = 0.f;
    auto fetch = [&](int n) {
        const float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
#pragma unroll
        for (int j = 0; j < NM; ++j) pM[j] = *reinterpret_cast<const float4*>(R + L::oMq + 4 * (tid + kCT * j));
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            if constexpr (L::kRowGate) {   // rows past the end from the last row, zeroed when stored
                const int r = idx / DK, c = idx % DK;
                const int64_t qi = qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + c;
                pA[j] = load4<E>(p.k, qi);
                pQ[j] = load4<E>(p.q, qi);
                pGr[j] = R[L::oG + r];
            } else {
                pA[j] = *reinterpret_cast<const float4*>(R + (SPLIT ? L::oEb : L::oKb) + idx);
                pQ[j] = *reinterpret_cast<const float4*>(R + L::oQh + idx);
            }
            pW[j] = *reinterpret_cast<const float4*>(R + L::oW + idx);
        }
        if constexpr (L::kRowGate) pGC = R[L::oG + kBC - 1];
#pragma unroll
        for (int j = 0; j < NO; ++j) {   // rows past the end: the last row, zeroed when stored
            const int e = tid + kCT * j, r = e / kBVT, i = e % kBVT;
            pO[j] = load_elem<E>(p.dO, tok_index(p, b, t0 + min(r, Cn - 1), h) * DV + i0 + i);
        }
        pG = R[L::oGam + min(tid, DK - 1)];   // every lane loads: no branch, no wait in it
    };
    auto put4 = [&](float* dst, int idx, int ld, int row, float4 v) {
        *reinterpret_cast<float4*>(dst + (idx / row) * ld + idx % row) = v;
    };
    fetch(N - 1);
    for (int n = N - 1; n >= 0; --n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
#pragma unroll
        for (int j = 0; j < NM; ++j) put4(sM, 4 * (tid + kCT * j), SMQ, kBC, pM[j]);
        const int Cn = min(kBC, p.T - n * kBC);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            if constexpr (L::kRowGate) {
                const bool ok = idx / DK < Cn;
                const float fb = __expf(pGC - pGr[j]), fq = __expf(pGr[j]);
                const float4 kv = pA[j], qv = pQ[j], z = make_float4(0.f, 0.f, 0.f, 0.f);
                put4(sA1, idx, SA, DK, ok ? make_float4(kv.x * fb, kv.y * fb, kv.z * fb, kv.w * fb) : z);
                put4(sQh, idx, SB, DK, ok ? make_float4(qv.x * fq, qv.y * fq, qv.z * fq, qv.w * fq) : z);
            } else {
                put4(sA1, idx, SA, DK, pA[j]);
                put4(sQh, idx, SB, DK, pQ[j]);
            }
            put4(sA2, idx, SB, DK, pW[j]);
        }
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int e = tid + kCT * j;
            sdO[(e / kBVT) * SO + e % kBVT] = e / kBVT < Cn ? pO[j] : 0.f;
        }
        sGam[min(tid, DK - 1)] = pG;   // lanes past DK rewrite the last entry with its own value
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

// The reverse chain with bf16 inputs: the operands are split into bf16 hi and lo
// once, when they are staged in LDS (natural row-major layouts, 16-byte padded
// rows), rather than by every lane at every read, and each product's k step of
// 32 is three v_mfma_f32_16x16x32_bf16 on fragments read 8 bytes at a time.  A
// contraction over the columns of a stored matrix reads its rows with plain
// 8-byte loads; one over the rows uses the LDS transpose load.  Within a k step
// of 32, lane (g, c) holds k = k0 + 4 g + e in slots e = 0..3 and
// k0 + 16 + 4 g + (e - 4) in slots 4..7, the same order for both operands.  dS is
// carried in fp32 accumulators by the waves that update it; LDS holds its split
// copy for the products of the next step.
struct Frag {
    bf16x8 h, l;
};
__device__ __forceinline__ bf16x4 ld4(const uint16_t* q) { return *reinterpret_cast<const bf16x4*>(q); }
// k along the columns of a row-major array: row `row`, k block k0
__device__ __forceinline__ Frag frag_row(const uint16_t* hi, const uint16_t* lo, int ld, int row, int k0, int g) {
    const int o = row * ld + k0 + 4 * g;
    return Frag{cat8(ld4(hi + o), ld4(hi + o + 16)), cat8(ld4(lo + o), ld4(lo + o + 16))};
}
// k along the rows of a row-major array: rows k0 + 4 g .., column n0 + c
__device__ __forceinline__ Frag frag_tr(const uint16_t* hi, const uint16_t* lo, int ld, int k0, int n0, int g, int c) {
    return Frag{cat8(tr_load_b16(hi, ld, k0, n0, g, c), tr_load_b16(hi, ld, k0 + 16, n0, g, c)),
                cat8(tr_load_b16(lo, ld, k0, n0, g, c), tr_load_b16(lo, ld, k0 + 16, n0, g, c))};
}
__device__ __forceinline__ f32x4 mma3(const Frag& a, const Frag& b, f32x4 acc) {
    return mfma_split8(a.h, a.l, b.h, b.l, acc);
}
__device__ __forceinline__ uint32_t split_pair(float x, float y, uint32_t& lo) {
    bf16_t xh, xl, yh, yl;
    split_bf16(x, xh, xl);
    split_bf16(y, yh, yl);
    lo = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, xl)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, yl)) << 16);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, xh)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, yh)) << 16);
}
// four consecutive elements, split, to hi and lo (8 bytes each)
__device__ __forceinline__ void put_split4(uint16_t* hi, uint16_t* lo, int o, float4 v) {
    uint32_t l0, l1;
    const uint32_t h0 = split_pair(v.x, v.y, l0), h1 = split_pair(v.z, v.w, l1);
    *reinterpret_cast<uint2*>(hi + o) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(lo + o) = make_uint2(l0, l1);
}
__device__ __forceinline__ void put_split1(uint16_t* hi, uint16_t* lo, int o, float x) {
    bf16_t h, l;
    split_bf16(x, h, l);
    hi[o] = __builtin_bit_cast(uint16_t, h);
    lo[o] = __builtin_bit_cast(uint16_t, l);
}

template <class L, typename E, int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(kCT) void bwd_rchain_split_kernel(BwdArgs p, float* ws, int N) {
    constexpr int NVT = DV / kBVT;
    constexpr int LM = kBC + 8, LO = kBVT + 8, LK = DK + 8, LT = kBC + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sMh[kBC * LM], sMl[kBC * LM];      // Mq (Me)   [m][r]
    __shared__ __attribute__((aligned(16))) uint16_t sOh[kBC * LO], sOl[kBC * LO];      // dO        [m][i]
    __shared__ __attribute__((aligned(16))) uint16_t sAh[kBC * LK], sAl[kBC * LK];      // Kbar (Ebar) [r][c]
    __shared__ __attribute__((aligned(16))) uint16_t sSh[kBVT * LK], sSl[kBVT * LK];    // dS'       [i][c]
    __shared__ __attribute__((aligned(16))) uint16_t sVh[kBVT * LT], sVl[kBVT * LT];    // -dVt (split gates: dY) [i][m]
    __shared__ __attribute__((aligned(16))) uint16_t sQh[kBC * LK], sQl[kBC * LK];      // Qhat      [m][c]
    __shared__ __attribute__((aligned(16))) uint16_t sWh[kBC * LK], sWl[kBC * LK];      // W         [m][c]
    __shared__ float sGam[DK];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, cl = l & 15;
    int bh, i0;
    if (!chain_block(p, NVT, bh, i0)) return;
    const int b = bh / p.H, h = bh % p.H;
    // dS tiles of this wave (accumulator layout): rows ii0 + 4 g + q, column cc + cl
    constexpr int NTS = (kBVT / 16) * (DK / 16);
    static_assert(NTS == kCW || NTS == 2 * kCW, "state tiles per wave");
    constexpr int TW = NTS / kCW;
    const int ii0 = 16 * (w % (kBVT / 16));
    int cc[TW];
    cc[0] = 16 * (w / (kBVT / 16));
    if constexpr (TW == 2) cc[1] = cc[0] + 16 * (kCW / (kBVT / 16));
    f32x4 dS[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dS[u][q] = p.dST ? p.dST[(static_cast<int64_t>(bh) * DV + i0 + ii0 + 4 * g + q) * DK + cc[u] + cl] : 0.f;
    }
    constexpr int NP = kBC * DK / 4 / kCT;
    constexpr int NM = kBC * kBC / 4 / kCT;
    constexpr int NO = kBC * kBVT / kCT;
    float4 pM[NM], pA[NP], pQ[NP], pW[NP];
    float pO[NO];
    float pG = 0.f;
    float pGr[L::kRowGate ? NP : 1], pGC = 0.f;
    auto fetch = [&](int n) {
        const float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
#pragma unroll
        for (int j = 0; j < NM; ++j) pM[j] = *reinterpret_cast<const float4*>(R + L::oMq + 4 * (tid + kCT * j));
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            if constexpr (L::kRowGate) {   // rows past the end from the last row, zeroed when stored
                const int r = idx / DK, c = idx % DK;
                const int64_t qi = qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + c;
                pA[j] = load4<E>(p.k, qi);
                pQ[j] = load4<E>(p.q, qi);
                pGr[j] = R[L::oG + r];
            } else {
                pA[j] = *reinterpret_cast<const float4*>(R + (SPLIT ? L::oEb : L::oKb) + idx);
                pQ[j] = *reinterpret_cast<const float4*>(R + L::oQh + idx);
            }
            pW[j] = *reinterpret_cast<const float4*>(R + L::oW + idx);
        }
        if constexpr (L::kRowGate) pGC = R[L::oG + kBC - 1];
#pragma unroll
        for (int j = 0; j < NO; ++j) {   // rows past the end: the last row, zeroed when stored
            const int e = tid + kCT * j, r = e / kBVT, i = e % kBVT;
            pO[j] = load_elem<E>(p.dO, tok_index(p, b, t0 + min(r, Cn - 1), h) * DV + i0 + i);
        }
        pG = R[L::oGam + min(tid, DK - 1)];   // every lane loads: no branch, no wait in it
    };
    fetch(N - 1);
    for (int n = N - 1; n >= 0; --n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int Cn = min(kBC, p.T - n * kBC);
        // ---- stage this chunk's operands, split
#pragma unroll
        for (int j = 0; j < NM; ++j) {
            const int idx = 4 * (tid + kCT * j);
            put_split4(sMh, sMl, (idx / kBC) * LM + idx % kBC, pM[j]);
        }
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j), o = (idx / DK) * LK + idx % DK;
            float4 av = pA[j], qv = pQ[j];
            if constexpr (L::kRowGate) {
                const bool ok = idx / DK < Cn;
                const float fb = __expf(pGC - pGr[j]), fq = __expf(pGr[j]);
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                av = ok ? make_float4(av.x * fb, av.y * fb, av.z * fb, av.w * fb) : z;
                qv = ok ? make_float4(qv.x * fq, qv.y * fq, qv.z * fq, qv.w * fq) : z;
            }
            put_split4(sAh, sAl, o, av);
            put_split4(sQh, sQl, o, qv);
            put_split4(sWh, sWl, o, pW[j]);
        }
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int e = tid + kCT * j;
            put_split1(sOh, sOl, (e / kBVT) * LO + e % kBVT, e / kBVT < Cn ? pO[j] : 0.f);
        }
        sGam[min(tid, DK - 1)] = pG;   // lanes past DK rewrite the last entry with its own value
        // dS' (leaving this chunk): to the record and, split, to LDS
#pragma unroll
        for (int u = 0; u < TW; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ii0 + 4 * g + q, c = cc[u] + cl;
                R[L::odS + (i0 + i) * DK + c] = dS[u][q];
                put_split1(sSh, sSl, i * LK + c, dS[u][q]);
            }
        }
        lds_only_barrier();
        if (n > 0) fetch(n - 1);
        // ---- dVt = Mq^T dO + Kbar dS'^T (split gates: dY = -(Me^T dO + Ebar dS'^T)), one tile per wave
        for (int t = w; t < (kBC / 16) * (kBVT / 16); t += kCW) {
            const int r0 = 16 * (t / (kBVT / 16)), c0 = 16 * (t % (kBVT / 16));
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32)
                acc = mma3(frag_tr(sMh, sMl, LM, k0, r0, g, cl), frag_tr(sOh, sOl, LO, k0, c0, g, cl), acc);
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32)
                acc = mma3(frag_row(sAh, sAl, LK, r0 + cl, k0, g), frag_row(sSh, sSl, LK, c0 + cl, k0, g), acc);
            // record: dVt (dY); LDS: -acc for the dS products in both forms, as [i][m]
            float4 nv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = r0 + 4 * g + q, i = c0 + cl;
                R[L::odVt + r * DV + i0 + i] = SPLIT ? -acc[q] : acc[q];
            }
            nv = make_float4(-acc[0], -acc[1], -acc[2], -acc[3]);
            put_split4(sVh, sVl, (c0 + cl) * LT + r0 + 4 * g, nv);
        }
        lds_only_barrier();
        // ---- dS = dS' Diag(gamma) + dO^T Qhat - dVt^T W  (split gates: + dY^T W)
        {
            f32x4 acc[TW];
#pragma unroll
            for (int u = 0; u < TW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32) {
                const Frag ao = frag_tr(sOh, sOl, LO, k0, ii0, g, cl);
                const Frag av = frag_row(sVh, sVl, LT, ii0 + cl, k0, g);
#pragma unroll
                for (int u = 0; u < TW; ++u) {
                    acc[u] = mma3(ao, frag_tr(sQh, sQl, LK, k0, cc[u], g, cl), acc[u]);
                    acc[u] = mma3(av, frag_tr(sWh, sWl, LK, k0, cc[u], g, cl), acc[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                const float gm = sGam[cc[u] + cl];
#pragma unroll
                for (int q = 0; q < 4; ++q) dS[u][q] = fmaf(dS[u][q], gm, acc[u][q]);
            }
        }
        lds_only_barrier();
    }
    if (p.gS0) {
#pragma unroll
        for (int u = 0; u < TW; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                p.gS0[(static_cast<int64_t>(bh) * DV + i0 + ii0 + 4 * g + q) * DK + cc[u] + cl] = dS[u][q];
        }
    }
}

// The forward chain with bf16 inputs, built like bwd_rchain_split_kernel: operands
// split once at staging, S carried in fp32 accumulators by the waves that update
// it, its split copy in LDS for the next step's W S^T.
template <class L, typename E, int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(kCT) void bwd_fchain_split_kernel(BwdArgs p, float* ws, int N) {
    constexpr int NVT = DV / kBVT;
    constexpr int LK = DK + 8, LT = kBC + 8, LX = kBVT + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sWh[kBC * LK], sWl[kBC * LK];      // W         [r][c]
    __shared__ __attribute__((aligned(16))) uint16_t sKh[kBC * LK], sKl[kBC * LK];      // Kbar      [r][c]
    __shared__ __attribute__((aligned(16))) uint16_t sEh[SPLIT ? kBC * LK : 8], sEl[SPLIT ? kBC * LK : 8];   // Ebar
    __shared__ __attribute__((aligned(16))) uint16_t sXh[SPLIT ? kBC * LX : 8], sXl[SPLIT ? kBC * LX : 8];   // X = w v [r][i]
    __shared__ __attribute__((aligned(16))) uint16_t sSh[kBVT * LK], sSl[kBVT * LK];    // S entering [i][c]
    __shared__ __attribute__((aligned(16))) uint16_t sVh[kBVT * LT], sVl[kBVT * LT];    // Vt (split gates: -Y) [i][r]
    __shared__ float sGam[DK];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, cl = l & 15;
    int bh, i0;
    if (!chain_block(p, NVT, bh, i0)) return;
    const int b = bh / p.H, h = bh % p.H;
    constexpr int NTS = (kBVT / 16) * (DK / 16);
    static_assert(NTS == kCW || NTS == 2 * kCW, "state tiles per wave");
    constexpr int TW = NTS / kCW;
    const int ii0 = 16 * (w % (kBVT / 16));
    int cc[TW];
    cc[0] = 16 * (w / (kBVT / 16));
    if constexpr (TW == 2) cc[1] = cc[0] + 16 * (kCW / (kBVT / 16));
    f32x4 S[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            S[u][q] = p.S0 ? p.S0[(static_cast<int64_t>(bh) * DV + i0 + ii0 + 4 * g + q) * DK + cc[u] + cl] : 0.f;
    }
    constexpr int NP = kBC * DK / 4 / kCT;
    static_assert((kBC / 16) * (kBVT / 16) == kCW, "one Vt tile per wave");
    float4 pW[NP], pK[NP], pE[SPLIT ? NP : 1];
    float pU[4];
    float pG = 0.f;
    float pGr[L::kRowGate ? NP : 1], pGC = 0.f;
    float4 pXw = make_float4(0.f, 0.f, 0.f, 0.f), pXv = pXw;
    static_assert(kBC * kBVT == 4 * kCT, "X: four columns per thread");
    const int vr0 = 16 * (w / (kBVT / 16)), vc0 = 16 * (w % (kBVT / 16));   // this wave's Vt tile
    auto fetch = [&](int n) {
        const float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
        if constexpr (SPLIT) {   // this tile's value columns, rows past the end from the last row
            const int r = 4 * tid / kBVT, i = 4 * tid % kBVT;
            const int64_t vi = tok_index(p, b, t0 + min(r, Cn - 1), h) * DV + i0 + i;
            pXw = load4<E>(p.wgate, vi);
            pXv = load4<E>(p.v, vi);
        }
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j);
            pW[j] = *reinterpret_cast<const float4*>(R + L::oW + idx);
            if constexpr (L::kRowGate) {
                const int r = idx / DK, c = idx % DK;
                pK[j] = load4<E>(p.k, qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + c);
                pGr[j] = R[L::oG + r];
            } else {
                pK[j] = *reinterpret_cast<const float4*>(R + L::oKb + idx);
            }
            if constexpr (SPLIT) pE[j] = *reinterpret_cast<const float4*>(R + L::oEb + idx);
        }
        if constexpr (L::kRowGate) pGC = R[L::oG + kBC - 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) pU[q] = R[L::oU + (vr0 + 4 * g + q) * DV + i0 + vc0 + cl];
        pG = R[L::oGam + min(tid, DK - 1)];
    };
    fetch(0);
    for (int n = 0; n < N; ++n) {
        float* R = ws + (static_cast<int64_t>(bh) * N + n) * L::size;
        const int Cn = min(kBC, p.T - n * kBC);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int idx = 4 * (tid + kCT * j), o = (idx / DK) * LK + idx % DK;
            put_split4(sWh, sWl, o, pW[j]);
            float4 kv = pK[j];
            if constexpr (L::kRowGate) {
                const float f = __expf(pGC - pGr[j]);
                kv = idx / DK < Cn ? make_float4(kv.x * f, kv.y * f, kv.z * f, kv.w * f) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            put_split4(sKh, sKl, o, kv);
            if constexpr (SPLIT) put_split4(sEh, sEl, o, pE[j]);
        }
        if constexpr (SPLIT) {   // X = w v for this tile's value columns (fetched a step ahead)
            const int r = 4 * tid / kBVT, i = 4 * tid % kBVT;
            put_split4(sXh, sXl, r * LX + i,
                       r < Cn ? make_float4(pXw.x * pXv.x, pXw.y * pXv.y, pXw.z * pXv.z, pXw.w * pXv.w)
                              : make_float4(0.f, 0.f, 0.f, 0.f));
        }
        float uu[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) uu[q] = pU[q];
        sGam[min(tid, DK - 1)] = pG;   // lanes past DK rewrite the last entry with its own value
        // S entering this chunk: to the record and, split, to LDS
#pragma unroll
        for (int u = 0; u < TW; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = ii0 + 4 * g + q, c = cc[u] + cl;
                R[L::oS + (i0 + i) * DK + c] = S[u][q];
                put_split1(sSh, sSl, i * LK + c, S[u][q]);
            }
        }
        lds_only_barrier();
        if (n + 1 < N) fetch(n + 1);
        // ---- Vt = U - W S^T  /  Y = Ut + W S^T, one tile per wave
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32)
                acc = mma3(frag_row(sWh, sWl, LK, vr0 + cl, k0, g), frag_row(sSh, sSl, LK, vc0 + cl, k0, g), acc);
            float4 vv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = vr0 + 4 * g + q, i = vc0 + cl;
                const float val = SPLIT ? uu[q] + acc[q] : uu[q] - acc[q];
                R[L::oVt + r * DV + i0 + i] = val;
                vv[q] = SPLIT ? -val : val;   // the operand of the state update
            }
            put_split4(sVh, sVl, (vc0 + cl) * LT + vr0 + 4 * g, make_float4(vv[0], vv[1], vv[2], vv[3]));
        }
        lds_only_barrier();
        // ---- S = S Diag(gamma) + Vt^T Kbar  /  - Y^T Ebar + X^T Kbar
        {
            f32x4 acc[TW];
#pragma unroll
            for (int u = 0; u < TW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32) {
                const Frag av = frag_row(sVh, sVl, LT, ii0 + cl, k0, g);
                if constexpr (SPLIT) {
                    const Frag ax = frag_tr(sXh, sXl, LX, k0, ii0, g, cl);
#pragma unroll
                    for (int u = 0; u < TW; ++u) {
                        acc[u] = mma3(av, frag_tr(sEh, sEl, LK, k0, cc[u], g, cl), acc[u]);
                        acc[u] = mma3(ax, frag_tr(sKh, sKl, LK, k0, cc[u], g, cl), acc[u]);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < TW; ++u) acc[u] = mma3(av, frag_tr(sKh, sKl, LK, k0, cc[u], g, cl), acc[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                const float gm = sGam[cc[u] + cl];
#pragma unroll
                for (int q = 0; q < 4; ++q) S[u][q] = fmaf(S[u][q], gm, acc[u][q]);
            }
        }
        lds_only_barrier();
    }
}

// ------------------------------------------------------------ 4. gradients
// Products run on the matrix cores as 16 x 16 tiles spread over the eight waves;
// the per-element pairwise sums of the channel-wise decay stay on the VALU.
template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kGT) void bwd_grads_kernel(BwdArgs p, float* ws, int N) {
    typedef BwdWs1<VAR, DK, DV> L;
    constexpr int CP = kBC + 4;
    constexpr int LD = (DK > DV ? DK : DV) + 4;
    constexpr int RS = (kBC * LD > 2 * kBC * CP) ? kBC * LD : 2 * kBC * CP;   // region size
    constexpr int QR = 32;            // rows of S (or dS') staged at a time
    static_assert(QR * (DK + 4) <= kBC * CP, "S quarter must fit the second C x C buffer");
    __shared__ __attribute__((aligned(16))) float sM1[kBC * CP];   // dMq (then dMq E)
    __shared__ __attribute__((aligned(16))) float sM2[kBC * CP];   // S quarters; dT; dA; dAbar (then dAbar E)
    __shared__ __attribute__((aligned(16))) float sR[3 * RS];      // three staging regions
    __shared__ float sBeta[kBC + 1];  // (+ a spare slot, never read)
    __shared__ float sCol[2 * DK];    // column terms of the last row of dG
    __shared__ float4 sPart[kGT];     // per-thread partial sums of four columns
    __shared__ float sGrow[kBC];      // G per row (row-gate record)
    __shared__ float sRed[kGW * 16];  // per-wave column sums of dKbar Kbar
    // ungated and scalar-decay forms with bf16 inputs: G per row in sGrow, and
    // the four sums of dG as products on split copies of dMq and dAbar
    constexpr bool kRS = L::kRowGate && kSplitMM<E>;
    float* R0 = sR;
    float* R1 = sR + RS;
    float* R2 = sR + 2 * RS;
    // bf16 inputs: a region may hold a matrix split into bf16 hi and lo planes
    // (rows of LR), read as 8-byte fragments
    constexpr int LR = (DK > DV ? DK : DV) + 8;
    static_assert(2 * kBC * LR * 2 <= RS * 4, "a split region fits a staging region");
    uint16_t* R0h = reinterpret_cast<uint16_t*>(R0);
    uint16_t* R0l = R0h + kBC * LR;
    uint16_t* R1h = reinterpret_cast<uint16_t*>(R1);
    uint16_t* R1l = R1h + kBC * LR;
    uint16_t* R2h = reinterpret_cast<uint16_t*>(R2);
    uint16_t* R2l = R2h + kBC * LR;
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };
    // the gate of (row r < Cn, channel c) is at or above the log-decay floor (a
    // gate clamped to the floor has no gradient)
    auto gate_kept = [&](int r, int c) { return load_elem<E>(p.g, tix(r) * DK + c) >= kLogDecayFloor; };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // element q of a tile at (i0, j0) in this lane
    auto ti = [&](int i0, int q) { return i0 + 4 * (l >> 4) + q; };
    auto tj = [&](int j0) { return j0 + (l & 15); };
    constexpr int TCD = (kBC / 16) * (DK / 16);   // C x DK tiles
    constexpr int TCV = (kBC / 16) * (DV / 16);   // C x DV tiles
    constexpr int TCC = (kBC / 16) * (kBC / 16);  // C x C tiles

    const float4 z4v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto put = [](float* dst, float4 x) { *reinterpret_cast<float4*>(dst) = x; };
    auto get = [](const float* src) { return *reinterpret_cast<const float4*>(src); };
    auto fma4 = [](float4 a, float4 b, float4 c) {
        return make_float4(fmaf(a.x, b.x, c.x), fmaf(a.y, b.y, c.y), fmaf(a.z, b.z, c.z), fmaf(a.w, b.w, c.w));
    };
    // beta (every thread loads from a valid row and stores, threads past the
    // chunk to a spare slot: no load sits in a branch)
    {
        const float bt = VAR == 4 ? 1.f : load_elem<E>(p.beta, tix(min(tid % kBC, Cn - 1)));
        sBeta[min(tid, kBC)] = tid < Cn ? bt : 0.f;
    }
    if constexpr (L::kRowGate) {
        if (tid < kBC) sGrow[tid] = R[L::oG + tid];
    }
    DR_TILE_FOR(e, kBC * DV / 4, kGT) {   // dO -> R0, Vt -> R1, dVt -> R2 (four columns per thread)
        const int r = 4 * e / DV, i = 4 * e % DV;
        const float4 d = load4<E>(p.dO, tix(min(r, Cn - 1)) * DV + i);
        if constexpr (kSplitMM<E>) {   // split planes (dO: exact, its lo plane zero)
            put_split4(R0h, R0l, r * LR + i, r < Cn ? d : z4v);
            put_split4(R1h, R1l, r * LR + i, get(R + L::oVt + 4 * e));
            put_split4(R2h, R2l, r * LR + i, get(R + L::odVt + 4 * e));
        } else {
            put(R0 + r * LD + i, r < Cn ? d : z4v);
            put(R1 + r * LD + i, get(R + L::oVt + 4 * e));
            put(R2 + r * LD + i, get(R + L::odVt + 4 * e));
        }
    }
    // column sums: thread (part, four columns); the parts combined in a fixed order
    constexpr int CG = DK / 4, NPART = kGT / CG;
    auto col_total = [&](int c) {
        float acc = 0.f;
        for (int part = 0; part < NPART; ++part) {
            const float4 v = sPart[part * CG + c / 4];
            acc += (c & 3) == 0 ? v.x : (c & 3) == 1 ? v.y : (c & 3) == 2 ? v.z : v.w;
        }
        return acc;
    };
    __syncthreads();   // dO, Vt and dVt staged
    for (int t = w; t < TCC; t += kGW) {            // dMq = Tril0(dO Vt^T)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        f32x4 acc = z4;
        if constexpr (kSplitMM<E>) {
#pragma unroll
            for (int k0 = 0; k0 < DV; k0 += 32) {
                const Frag ao = frag_row(R0h, R0l, LR, r0 + (l & 15), k0, l >> 4);
                const Frag av = frag_row(R1h, R1l, LR, j0 + (l & 15), k0, l >> 4);
                acc = mfma_split8<true, false>(ao.h, ao.l, av.h, av.l, acc);   // dO exact
            }
        } else {
            acc = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DV, exact([&](int r, int i) { return R0[r * LD + i]; }),
                                      [&](int i, int j) { return R1[j * LD + i]; });
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), j = tj(j0);
            sM1[r * CP + j] = j <= r ? acc[q] : 0.f;
        }
    }
    // sum_i S dS' per column, from the staged row blocks: a thread's elements of
    // a block sit in the same four columns in every block, and it keeps those of
    // S until the matching block of dS' arrives
    float4 sds = z4v;
    float kbs = 0.f;   // this lane's part of sum_r dKbar Kbar in its column
    {   // dQhat = dO S, dW = -dVt S, then dKbar = Vt dS', with S and dS' staged by rows
        constexpr int MT = TCD / kGW;   // tiles per wave
        f32x4 aq[MT], aw[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) aq[m] = aw[m] = z4;
        // row blocks of S, then of dS', double-buffered through registers: the next
        // block's loads are in flight while the current block's products run
        constexpr int NPF = QR * DK / 4 / kGT;
        float4 pf[NPF];
        float4 keepS[DV / QR][NPF];
        static_assert(kGT % (DK / 4) == 0, "the same columns in every block");
        auto fetch_rows = [&](int64_t src, int i0) {
#pragma unroll
            for (int j = 0; j < NPF; ++j) pf[j] = get(R + src + i0 * DK + 4 * (tid + kGT * j));
        };
        fetch_rows(L::oS, 0);
        // Kbar at this lane's dKbar elements, for the per-column sum of dKbar Kbar:
        // row-gate record, k (rows past the end from the last row; Kbar = k e^{G_C - G_r}
        // is formed where it is used); otherwise Kbar from the record.  Loaded here
        // so that the passes cover the loads.  A wave's tiles all sit in the 16
        // columns 16 (w mod DK / 16) + [0, 16).
        float kraw[MT][4];
        static_assert(kGW % (DK / 16) == 0, "a wave's tiles share their columns");
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (L::kRowGate)
                    kraw[m][q] = load_elem<E>(p.k, qk_index(p, b, t0 + min(ti(r0, q), Cn - 1), h) * DK + tj(c0));
                else
                    kraw[m][q] = R[L::oKb + ti(r0, q) * DK + tj(c0)];
            }
        }
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int i0 = 0; i0 < DV; i0 += QR) {
                __syncthreads();
                if (pass == 1 && i0 == 0) {   // dW over dO, which pass 1 does not read
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = ti(r0, q), c = tj(c0);
                            if constexpr (kSplitMM<E>) put_split1(R0h, R0l, r * LR + c, -aw[m][q]);
                            else R0[r * LD + c] = aw[m][q];
                        }
                    }
                }
                // bf16 inputs: the rows are staged split (bf16 hi and lo, rows of
                // DK + 8) and read by the LDS transpose load; the A rows are read
                // 16 bytes at a time and split in registers
                constexpr int LS = DK + 8;
                uint16_t* sSh = reinterpret_cast<uint16_t*>(sM2);
                uint16_t* sSl = sSh + QR * LS;
                static_assert(2 * QR * LS * 2 <= kBC * CP * 4, "split rows fit the second C x C buffer");
#pragma unroll
                for (int j = 0; j < NPF; ++j) {
                    const int e = 4 * (tid + kGT * j);
                    if constexpr (kSplitMM<E>) put_split4(sSh, sSl, (e / DK) * LS + e % DK, pf[j]);
                    else put(sM2 + (e / DK) * (DK + 4) + e % DK, pf[j]);
                    if (pass == 0) keepS[i0 / QR][j] = pf[j];
                    else sds = fma4(keepS[i0 / QR][j], pf[j], sds);
                }
                __syncthreads();
                if (i0 + QR < DV) fetch_rows(pass == 0 ? L::oS : L::odS, i0 + QR);
                else if (pass == 0) fetch_rows(L::odS, 0);
                if constexpr (kSplitMM<E>) {
                    static_assert(QR == 32, "one k step per row block");
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                        const Frag bs = frag_tr(sSh, sSl, LS, 0, c0, l >> 4, l & 15);
                        // A: rows r0 + c of dO, dVt (pass 0) or Vt (pass 1), split planes;
                        // dW accumulates +dVt S and is negated when written
                        if (pass == 0) {
                            const Frag ao = frag_row(R0h, R0l, LR, r0 + (l & 15), i0, l >> 4);   // dO exact
                            aq[m] = mfma_split8<true, false>(ao.h, ao.l, bs.h, bs.l, aq[m]);
                            const Frag av = frag_row(R2h, R2l, LR, r0 + (l & 15), i0, l >> 4);
                            aw[m] = mfma_split8(av.h, av.l, bs.h, bs.l, aw[m]);
                        } else {
                            const Frag av = frag_row(R1h, R1l, LR, r0 + (l & 15), i0, l >> 4);
                            aq[m] = mfma_split8(av.h, av.l, bs.h, bs.l, aq[m]);
                        }
                    }
                    continue;
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                    auto Bs = [&](int i, int c) { return sM2[(i - i0) * (DK + 4) + c]; };
                    if (pass == 0) {
                        aq[m] = mm_tile<kSplitMM<E>>(aq[m], r0, c0, i0, i0 + QR, exact([&](int r, int i) { return R0[r * LD + i]; }), Bs);
                        aw[m] = mm_tile<kSplitMM<E>>(aw[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return -R2[r * LD + i]; }, Bs);
                    } else {
                        aq[m] = mm_tile<kSplitMM<E>>(aq[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R1[r * LD + i]; }, Bs);
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
                    } else {
                        R[L::odKb + r * DK + c] = aq[m][q];
                        if constexpr (L::kRowGate)
                            kbs = fmaf(aq[m][q], r < Cn ? kraw[m][q] * __expf(sGrow[kBC - 1] - sGrow[r]) : 0.f, kbs);
                        else
                            kbs = fmaf(aq[m][q], kraw[m][q], kbs);
                    }
                }
                aq[m] = z4;
            }
        }
    }
    // sum_r dKbar Kbar: over the four lanes of a column, then the waves that share it
    kbs += __shfl_xor(kbs, 16, 64);
    kbs += __shfl_xor(kbs, 32, 64);
    if (l < 16) sRed[w * 16 + l] = kbs;
    sPart[tid] = sds;   // part tid / (DK / 4), columns 4 (tid % (DK / 4)) + [0, 4)
    __syncthreads();
    if (tid < DK) {
        sCol[tid] = R[L::oGam + tid] * col_total(tid);
        float a = 0.f;
        for (int v = tid / 16; v < kGW; v += DK / 16) a += sRed[v * 16 + tid % 16];
        sCol[DK + tid] = a;
    }
    // bf16 inputs: operands staged split (bf16 hi and lo planes) or split as read,
    // lane (g, c) holding k = k0 + 4 g + e and k0 + 16 + 4 g + e in slot e
    const int g = l >> 4, cl = l & 15;
    auto split8 = [](const float (&v)[8]) {
        Frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16_t hh, ll;
            split_bf16(v[e], hh, ll);
            f.h[e] = hh;
            f.l[e] = ll;
        }
        return f;
    };
    auto arow = [&](const float* X, int ld, int row, int k0) {   // X[row][k]
        const float4 a0 = get(X + row * ld + k0 + 4 * g), a1 = get(X + row * ld + k0 + 16 + 4 * g);
        const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        return split8(v);
    };
    auto bcol = [&](const float* X, int ld, int k0, int col) {   // X[k][col]
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = X[(k0 + 4 * g + (e < 4 ? e : 12 + e)) * ld + col];
        return split8(v);
    };
    // dT = dW X^T + dVt Y^T with X = beta Khat, Y = beta v
    DR_TILE_FOR(e, kBC * DK / 4, kGT) {   // X -> R1 (dW is in R0)
        const int r = 4 * e / DK, c = 4 * e % DK;
        float4 kh;
        if constexpr (L::kRowGate) {   // Khat = k e^{G_r}, zero past the end
            const float4 kv = load4<E>(p.k, qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + c);
            const float f = __expf(R[L::oG + r]);
            kh = r < Cn ? make_float4(kv.x * f, kv.y * f, kv.z * f, kv.w * f) : z4v;
        } else {
            kh = get(R + L::oKh + 4 * e);
        }
        const float br = sBeta[r];
        const float4 x = make_float4(br * kh.x, br * kh.y, br * kh.z, br * kh.w);
        if constexpr (kSplitMM<E>) put_split4(R1h, R1l, r * LR + c, x);
        else put(R1 + r * LD + c, x);
    }
    __syncthreads();
    f32x4 adt[TCC / kGW];
#pragma unroll
    for (int m = 0; m < TCC / kGW; ++m) {
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        if constexpr (kSplitMM<E>) {
            adt[m] = z4;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32)
                adt[m] = mma3(frag_row(R0h, R0l, LR, r0 + cl, k0, g), frag_row(R1h, R1l, LR, j0 + cl, k0, g), adt[m]);
        } else {
            adt[m] = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, [&](int r, int c) { return R0[r * LD + c]; },
                             [&](int c, int j) { return R1[j * LD + c]; });
        }
    }
    __syncthreads();
    DR_TILE_FOR(e, kBC * DV / 4, kGT) {   // Y -> R1
        const int r = 4 * e / DV, i = 4 * e % DV;
        const float4 vv = load4<E>(p.v, tix(min(r, Cn - 1)) * DV + i);
        const float br = sBeta[r];
        const float4 y = r < Cn ? make_float4(br * vv.x, br * vv.y, br * vv.z, br * vv.w) : z4v;
        if constexpr (kSplitMM<E>) put_split4(R1h, R1l, r * LR + i, y);
        else put(R1 + r * LD + i, y);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < TCC / kGW; ++m) {
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        if constexpr (kSplitMM<E>) {
#pragma unroll
            for (int k0 = 0; k0 < DV; k0 += 32)
                adt[m] = mma3(frag_row(R2h, R2l, LR, r0 + cl, k0, g), frag_row(R1h, R1l, LR, j0 + cl, k0, g), adt[m]);
        } else {
            adt[m] = mm_tile<kSplitMM<E>>(adt[m], r0, j0, 0, DV, [&](int r, int i) { return R2[r * LD + i]; },
                             [&](int i, int j) { return R1[j * LD + i]; });
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) sM2[ti(r0, q) * CP + tj(j0)] = adt[m][q];
    }
    __syncthreads();
    // dA = -T^T dT T^T (strictly lower); T -> R1[0 .. C*CP), tmp -> R1[C*CP ..)
    float* sTmp = R1 + kBC * CP;
    if constexpr (kSplitMM<E>) {
        // bf16 inputs: T staged split (bf16 hi and lo, rows of C + 4) where the
        // fp32 T would be, and read as 8-byte fragments (k = k0 + 4 g + e and
        // k0 + 16 + 4 g + e); the other operand of each product split as read
        constexpr int LT2 = kBC + 4;
        static_assert(2 * kBC * LT2 * 2 <= kBC * CP * 4, "split T fits where T was");
        uint16_t* Th = reinterpret_cast<uint16_t*>(R1);
        uint16_t* Tl = Th + kBC * LT2;
        DR_TILE_FOR(e, kBC * kBC / 4, kGT) put_split4(Th, Tl, (4 * e / kBC) * LT2 + 4 * e % kBC, get(R + L::oT + 4 * e));
        __syncthreads();
        for (int t = w; t < TCC; t += kGW) {            // tmp = dT T^T
            const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            f32x4 acc = z4;
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32)
                acc = mma3(arow(sM2, CP, r0 + cl, k0), frag_row(Th, Tl, LT2, j0 + cl, k0, g), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q) sTmp[ti(r0, q) * CP + tj(j0)] = acc[q];
        }
        __syncthreads();
        for (int t = w; t < TCC; t += kGW) {            // dA = -T^T tmp, masked
            const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            f32x4 acc = z4;
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32)
                acc = mma3(frag_tr(Th, Tl, LT2, k0, r0, g, cl), bcol(sTmp, CP, k0, j0 + cl), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ti(r0, q), j = tj(j0);
                sM2[r * CP + j] = j < r ? -acc[q] : 0.f;
            }
        }
        for (int t = w; t < TCD; t += kGW) {            // dX = T^T dW (dKhat = beta dX)
            const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            f32x4 acc = z4;
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32)
                acc = mma3(frag_tr(Th, Tl, LT2, k0, r0, g, cl), frag_tr(R0h, R0l, LR, k0, c0, g, cl), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q) R[L::odX + ti(r0, q) * DK + tj(c0)] = acc[q];
        }
        __syncthreads();
        for (int t = w; t < TCV; t += kGW) {            // dY = T^T dVt -> dv = beta dY; dY -> R0
            const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
            f32x4 acc = z4;
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32)
                acc = mma3(frag_tr(Th, Tl, LT2, k0, r0, g, cl), frag_tr(R2h, R2l, LR, k0, c0, g, cl), acc);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ti(r0, q), i = tj(c0);
                R0[r * LD + i] = acc[q];
                if (r < Cn) store_elem<E>(p.gv, tix(r) * DV + i, sBeta[r] * acc[q]);
            }
        }
        __syncthreads();
    } else {
        float* sT = R1;
        DR_TILE_FOR(e, kBC * kBC / 4, kGT) put(sT + (4 * e / kBC) * CP + 4 * e % kBC, get(R + L::oT + 4 * e));
        __syncthreads();
        for (int t = w; t < TCC; t += kGW) {            // tmp = dT T^T
            const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, kBC, [&](int r, int m) { return sM2[r * CP + m]; },
                                      [&](int m, int j) { return sT[j * CP + m]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) sTmp[ti(r0, q) * CP + tj(j0)] = acc[q];
        }
        __syncthreads();
        for (int t = w; t < TCC; t += kGW) {            // dA = -T^T tmp, masked
            const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                      [&](int m, int j) { return sTmp[m * CP + j]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ti(r0, q), j = tj(j0);
                sM2[r * CP + j] = j < r ? -acc[q] : 0.f;
            }
        }
        for (int t = w; t < TCD; t += kGW) {            // dX = T^T dW (dKhat = beta dX)
            const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                      [&](int m, int c) { return R0[m * LD + c]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) R[L::odX + ti(r0, q) * DK + tj(c0)] = acc[q];
        }
        __syncthreads();
        for (int t = w; t < TCV; t += kGW) {            // dY = T^T dVt -> dv = beta dY; dY -> R0
            const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
            const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                      [&](int m, int i) { return R2[m * LD + i]; });
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ti(r0, q), i = tj(c0);
                R0[r * LD + i] = acc[q];
                if (r < Cn) store_elem<E>(p.gv, tix(r) * DV + i, sBeta[r] * acc[q]);
            }
        }
        __syncthreads();
    }
    if constexpr (VAR != 4) {   // dbeta: kRT threads per row, fixed-order sums
        const int r = tid / kRT, qt = tid % kRT;
        float db = 0.f;
        if constexpr (L::kRowGate) {   // Khat = k e^{G_r} rebuilt, four channels per load
            const int64_t krow = qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + qt * (DK / kRT);
            float4 kv[DK / kRT / 4];
#pragma unroll
            for (int m = 0; m < DK / kRT / 4; ++m) kv[m] = load4<E>(p.k, krow + 4 * m);
            const float khf = r < Cn ? __expf(R[L::oG + r]) : 0.f;
#pragma unroll
            for (int m = 0; m < DK / kRT / 4; ++m) {
                const float4 dx = get(R + L::odX + r * DK + qt * (DK / kRT) + 4 * m);
                db = fmaf(dx.x, kv[m].x * khf, db);
                db = fmaf(dx.y, kv[m].y * khf, db);
                db = fmaf(dx.z, kv[m].z * khf, db);
                db = fmaf(dx.w, kv[m].w * khf, db);
            }
        } else {
#pragma unroll
            for (int k = 0; k < DK / kRT; ++k) {
                const int c = qt * (DK / kRT) + k;
                db = fmaf(R[L::odX + r * DK + c], R[L::oKh + r * DK + c], db);
            }
        }
        const int64_t vrow = tix(min(r, Cn - 1)) * DV;
        float dv_ = 0.f;
#pragma unroll
        for (int k = 0; k < DV / kRT; ++k) {
            const int i = qt * (DV / kRT) + k;
            dv_ = fmaf(R0[r * LD + i], load_elem<E>(p.v, vrow + i), dv_);
        }
        db += r < Cn ? dv_ : 0.f;
#pragma unroll
        for (int k = 0; k < kBC / kRT; ++k) {
            const int j = qt * (kBC / kRT) + k;
            db = fmaf(sM2[r * CP + j], R[L::oAb + r * kBC + j], db);
        }
#pragma unroll
        for (int m = 1; m < kRT; m <<= 1) db += __shfl_xor(db, m);
        if (qt == 0 && r < Cn) store_elem<E>(p.gbeta, tix(r), db);
    }
    __syncthreads();
    // q, k, G -> R0, R1, R2; dAbar = beta dA
    for (int e = tid; e < kBC * kBC; e += kGT) sM2[(e / kBC) * CP + e % kBC] *= sBeta[e / kBC];
    DR_TILE_FOR(e, kBC * DK / 4, kGT) {
        const int r = 4 * e / DK, c = 4 * e % DK;
        const bool ok = r < Cn;
        const int64_t qi = qk_index(p, b, t0 + min(r, Cn - 1), h) * DK + c;
        const float4 qv = load4<E>(p.q, qi), kv = load4<E>(p.k, qi);
        put(R0 + r * LD + c, ok ? qv : z4v);
        put(R1 + r * LD + c, ok ? kv : z4v);
        if constexpr (kRS) {
        } else if constexpr (L::kRowGate) {
            const float gr = R[L::oG + r];
            put(R2 + r * LD + c, make_float4(gr, gr, gr, gr));
        } else {
            put(R2 + r * LD + c, get(R + L::oG + 4 * e));
        }
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
        const float Gr = kRS ? sGrow[r] : R2[r * LD + c];
        const float GC = kRS ? sGrow[kBC - 1] : R2[(kBC - 1) * LD + c];
        const float qr = R0[r * LD + c], kr = R1[r * LD + c];
        const float eg = (VAR == 0) ? 1.f : __expf(Gr);
        const float ebar = (VAR == 0) ? 1.f : __expf(GC - Gr);
        const int e = r * DK + c;
        const float dKh = sBeta[r] * dX_;
        if (r < Cn) {
            store_qk_grad<E>(p.gq, p.gq32, tix(r), DK, c, fmaf(dQh, eg, a1));
            store_qk_grad<E>(p.gk, p.gk32, tix(r), DK, c, a2 + a3 + a4 + dKh * eg + dKb * ebar);
        }
        float dG = qr * a1 - kr * a2 + kr * a3 - kr * a4 + dKh * kr * eg + dQh * qr * eg - dKb * kr * ebar;
        if constexpr (VAR != 1) R[L::odQh + e] = dG;
        // scalar decay: the G_C terms of channel c join its last row before the
        // sum over channels (they largely cancel against it)
        if constexpr (VAR == 1) dG += r == Cn - 1 ? sCol[c] + sCol[DK + c] : 0.f;
        return dG;
    };
    // scalar decay: the gate's gradient needs only the channel sums of dG per
    // row; per 16-column tile they are reduced over its 16 lanes and kept in
    // sRow[column tile][row] (sPart is free by now)
    float* sRow = reinterpret_cast<float*>(sPart);
    static_assert((DK / 16) * kBC <= 4 * kGT, "row sums fit sPart");
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
            colg[m] = pair_tile<false, kSplitMM<E>>(r0, c0, M1, Qf, Gf) + pair_tile<false, kSplitMM<E>>(r0, c0, M2, Kf, Gf);
        }
        __syncthreads();
        DR_TILE_FOR(e, kBC * DK, kGT) {
            const int r = e / DK, c = e % DK;
            const float bv = load_elem<E>(p.beta, tix(min(r, Cn - 1)) * DK + c);
            R1[r * LD + c] *= r < Cn ? bv : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MTG; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            const Pre pr = preload(r0, c0);
            const f32x4 a1 = pair_tile<true, kSplitMM<E>>(r0, c0, M1, Kf, Gf);
            const f32x4 a3 = pair_tile<true, kSplitMM<E>>(r0, c0, M2, Kf, Gf);
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
            const f32x4 a1 = pair_tile<true, kSplitMM<E>>(r0, c0, M1, Kf, Gf);
            const f32x4 a2 = pair_tile<false, kSplitMM<E>>(r0, c0, M1, Qf, Gf);
            const f32x4 a3 = pair_tile<true, kSplitMM<E>>(r0, c0, M2, Kf, Gf);
            const f32x4 a4 = pair_tile<false, kSplitMM<E>>(r0, c0, M2, Kf, Gf);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                finish(ti(r0, q), tj(c0), a1[q], a2[q], a3[q], a4[q], pr.dQh[q], pr.dX[q], pr.dKb[q]);
        }
    } else if constexpr (kRS) {
        // the decay factor is one number per (r, j): fold it into dMq and dAbar,
        // split them into R2 (free for the row-gate record), and take the four
        // sums as products with q and k as loaded (exact in bf16)
        constexpr int LM = kBC + 4;
        static_assert(4 * kBC * LM * 2 <= RS * 4, "split C x C copies fit a staging region");
        uint16_t* M1h = reinterpret_cast<uint16_t*>(R2);
        uint16_t* M1l = M1h + kBC * LM;
        uint16_t* M2h = M1l + kBC * LM;
        uint16_t* M2l = M2h + kBC * LM;
        for (int e = tid; e < kBC * kBC; e += kGT) {
            const int r = e / kBC, j = e % kBC;
            const float ex = (VAR == 1 && j <= r) ? __expf(sGrow[r] - sGrow[j]) : 1.f;
            put_split1(M1h, M1l, r * LM + j, sM1[r * CP + j] * ex);
            put_split1(M2h, M2l, r * LM + j, sM2[r * CP + j] * ex);
        }
        __syncthreads();
        const bf16x8 zb = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int t = w; t < TCD; t += kGW) {
            const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
            const Pre pr = preload(r0, c0);
            f32x4 a1 = z4, a2 = z4, a3 = z4, a4 = z4;
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 32) {
                // k and q down the rows j = k0 + 4 g + e and k0 + 16 + 4 g + e, column c0 + c
                bf16x8 kb, qb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = k0 + 4 * (l >> 4) + (e < 4 ? e : 12 + e);
                    kb[e] = static_cast<bf16_t>(R1[j * LD + c0 + (l & 15)]);
                    qb[e] = static_cast<bf16_t>(R0[j * LD + c0 + (l & 15)]);
                }
                const Frag m1r = frag_row(M1h, M1l, LM, r0 + (l & 15), k0, l >> 4);
                const Frag m1t = frag_tr(M1h, M1l, LM, k0, r0, l >> 4, l & 15);
                const Frag m2r = frag_row(M2h, M2l, LM, r0 + (l & 15), k0, l >> 4);
                const Frag m2t = frag_tr(M2h, M2l, LM, k0, r0, l >> 4, l & 15);
                a1 = mfma_split8<false, true>(m1r.h, m1r.l, kb, zb, a1);
                a2 = mfma_split8<false, true>(m1t.h, m1t.l, qb, zb, a2);
                a3 = mfma_split8<false, true>(m2r.h, m2r.l, kb, zb, a3);
                a4 = mfma_split8<false, true>(m2t.h, m2t.l, kb, zb, a4);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float x = finish(ti(r0, q), tj(c0), a1[q], a2[q], a3[q], a4[q], pr.dQh[q], pr.dX[q], pr.dKb[q]);
                if constexpr (VAR == 1) {
#pragma unroll
                    for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m);
                    if ((l & 15) == 0) sRow[(c0 / 16) * kBC + ti(r0, q)] = x;
                }
            }
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
            // (q and k as loaded: exact in bf16 with bf16 inputs)
            const f32x4 a1 = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM1[r * CP + j]; },
                                     exact([&](int j, int c) { return R1[j * LD + c]; }));
            const f32x4 a2 = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM1[j * CP + r]; },
                                     exact([&](int j, int c) { return R0[j * LD + c]; }));
            const f32x4 a3 = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM2[r * CP + j]; },
                                     exact([&](int j, int c) { return R1[j * LD + c]; }));
            const f32x4 a4 = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM2[j * CP + r]; },
                                     exact([&](int j, int c) { return R1[j * LD + c]; }));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float x = finish(ti(r0, q), tj(c0), a1[q], a2[q], a3[q], a4[q], pr.dQh[q], pr.dX[q], pr.dKb[q]);
                if constexpr (VAR == 1) {
#pragma unroll
                    for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m);
                    if ((l & 15) == 0) sRow[(c0 / 16) * kBC + ti(r0, q)] = x;
                }
            }
        }
    }
    if constexpr (VAR == 1) {
        // dg_r = sum_{r' >= r} sum_c dG[r', c] (the G_C terms are in the last row):
        // the channel sums of the rows, then a reverse scan over the rows on wave 0
        __syncthreads();
        if (w == 0) {
            float rs = 0.f;
#pragma unroll
            for (int cb = 0; cb < DK / 16; ++cb) rs += sRow[cb * kBC + l];
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float t = __shfl_down(rs, m);
                if (l + m < 64) rs += t;
            }
            if (l < Cn) store_elem<E>(p.gg, tix(l), rs);
        }
    }
    if constexpr (VAR >= 2) {
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
                // a gate clamped at the floor has no gradient
                if (r < Cn) store_elem<E>(p.gg, tix(r) * DK + c, gate_kept(r, c) ? acc : 0.f);
            }
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
    __shared__ __attribute__((aligned(16))) float sK[kBC * (DK + 4)];
    __shared__ __attribute__((aligned(16))) float sG[kBC * (DK + 4)];
    __shared__ __attribute__((aligned(16))) float sR1[RS];
    __shared__ __attribute__((aligned(16))) float sR2[RS];
    __shared__ __attribute__((aligned(16))) float sM[kBC * CP];
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };
    const float4 z4v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto put = [](float* dst, float4 x) { *reinterpret_cast<float4*>(dst) = x; };
    auto get = [](const float* src) { return *reinterpret_cast<const float4*>(src); };
    auto mul4 = [](float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); };

    DR_TILE_FOR(e, kBC * DK / 4, kGT) {   // k, b k, g (four channels per thread)
        const int r = 4 * e / DK, c = 4 * e % DK;
        const bool ok = r < Cn;
        const int rc = min(r, Cn - 1);
        const float4 kv = load4<E>(p.k, qk_index(p, b, t0 + rc, h) * DK + c);
        const float4 bv = load4<E>(p.beta, tix(rc) * DK + c);
        const float4 g4 = load4<E>(p.g, tix(rc) * DK + c);
        const float4 gv = make_float4(fmaxf(g4.x, kLogDecayFloor), fmaxf(g4.y, kLogDecayFloor),
                                      fmaxf(g4.z, kLogDecayFloor), fmaxf(g4.w, kLogDecayFloor));
        put(sK + r * (DK + 4) + c, ok ? kv : z4v);
        put(sR1 + r * LD + c, ok ? mul4(bv, kv) : z4v);
        put(sG + r * (DK + 4) + c, ok ? gv : z4v);
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
    DR_TILE_FOR(e, kBC * DK / 4, kGT) put(R + L::oG + 4 * e, get(sG + (4 * e / DK) * (DK + 4) + 4 * e % DK));
    if (tid < DK) R[L::oGam + tid] = __expf(sG[(kBC - 1) * (DK + 4) + tid]);
    // pairwise factors with the reference at the last row of j's 16-row block
    auto aexp = [&](int r, int c, const float* gref) { return __expf(sG[r * (DK + 4) + c] - gref[c]); };
    auto bexp = [&](int j, int c, const float* gref) { return __expf(gref[c] - sG[j * (DK + 4) + c]); };
    static_assert(16 % kGW == 0, "C x C tiles per wave");
    f32x4 akr[16 / kGW];                          // Ak, kept for Z = Ak X
#pragma unroll
    for (int m = 0; m < 16 / kGW; ++m) {          // Ae -> sM, Ak -> workspace (strictly lower)
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        f32x4 ae = z4, ak = z4;
        if (j0 <= r0) {
            const float* gref = sG + (j0 + 15) * (DK + 4);
            auto Ak_ = [&](int r, int c) { return sK[r * (DK + 4) + c] * aexp(r, c, gref); };
            ae = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, Ak_, [&](int c, int j) { return sR1[j * LD + c] * bexp(j, c, gref); });
            ak = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, Ak_, [&](int c, int j) { return sK[j * (DK + 4) + c] * bexp(j, c, gref); });
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 4 * (l >> 4) + q, j = j0 + (l & 15);
            sM[r * CP + j] = j < r ? ae[q] : 0.f;
            ak[q] = j < r ? ak[q] : 0.f;
            R[L::oAk + r * kBC + j] = ak[q];
        }
        akr[m] = ak;
    }
    __syncthreads();
    float* sT = sR2;
    unit_lower_inverse_blocked<kSplitMM<E>>(sM, CP, nullptr, sT, CP, sR2 + kBC * CP);   // T = (I + Ae)^-1
    for (int e = tid; e < kBC * kBC; e += kGT) R[L::oT + e] = sT[(e / kBC) * CP + e % kBC];
    DR_TILE_FOR(e, kBC * DK / 4, kGT) {   // Ebar, Kbar, Khat; Khat -> sR1
        const int r = 4 * e / DK, c = 4 * e % DK;
        const float4 G = get(sG + r * (DK + 4) + c), GC = get(sG + (kBC - 1) * (DK + 4) + c);
        const float4 eg = make_float4(__expf(G.x), __expf(G.y), __expf(G.z), __expf(G.w));
        const float4 eb = make_float4(__expf(GC.x - G.x), __expf(GC.y - G.y), __expf(GC.z - G.z), __expf(GC.w - G.w));
        const float4 kk = get(sK + r * (DK + 4) + c);
        const float4 kh = mul4(kk, eg);
        put(R + L::oEb + 4 * e, mul4(get(sR1 + r * LD + c), eb));
        put(R + L::oKb + 4 * e, mul4(kk, eb));
        put(R + L::oKh + 4 * e, kh);
        put(sR1 + r * LD + c, kh);
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DK / 16); t += kGW) {   // W = T Khat
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * CP + j]; },
                                  [&](int j, int c) { return sR1[j * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oW + (r0 + 4 * (l >> 4) + q) * DK + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
    DR_TILE_FOR(e, kBC * DV / 4, kGT) {   // X = w v -> sR1
        const int r = 4 * e / DV, i = 4 * e % DV;
        const int64_t vi = tix(min(r, Cn - 1)) * DV + i;
        const float4 x = mul4(load4<E>(p.wgate, vi), load4<E>(p.v, vi));
        put(sR1 + r * LD + i, r < Cn ? x : z4v);
    }
#pragma unroll
    for (int m = 0; m < 16 / kGW; ++m) {   // Ak from registers -> sM (Ae is no longer needed)
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) sM[(r0 + 4 * (l >> 4) + q) * CP + j0 + (l & 15)] = akr[m][q];
    }
    __syncthreads();
    constexpr int TZ = (kBC / 16) * (DV / 16) / kGW;   // Z tiles per wave
    static_assert((kBC / 16) * (DV / 16) % kGW == 0, "Z tiles per wave");
    f32x4 zr[TZ];
#pragma unroll
    for (int m = 0; m < TZ; ++m) {   // Z = Ak X
        const int t = w + kGW * m, r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        zr[m] = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sM[r * CP + j]; },
                        [&](int j, int i) { return sR1[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oZ + (r0 + 4 * (l >> 4) + q) * DV + c0 + (l & 15)] = zr[m][q];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < TZ; ++m) {   // Z -> sR1 (X is no longer needed)
        const int t = w + kGW * m, r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
#pragma unroll
        for (int q = 0; q < 4; ++q) sR1[(r0 + 4 * (l >> 4) + q) * LD + c0 + (l & 15)] = zr[m][q];
    }
    __syncthreads();
    for (int t = w; t < (kBC / 16) * (DV / 16); t += kGW) {   // Ut = T Z
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int j) { return sT[r * CP + j]; },
                                  [&](int j, int i) { return sR1[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::oU + (r0 + 4 * (l >> 4) + q) * DV + c0 + (l & 15)] = acc[q];
    }
    __syncthreads();
    DR_TILE_FOR(e, kBC * DK / 4, kGT) {   // q -> sR1, b k -> sR2, Qhat
        const int r = 4 * e / DK, c = 4 * e % DK;
        const bool ok = r < Cn;
        const int rc = min(r, Cn - 1);
        const float4 qv = load4<E>(p.q, qk_index(p, b, t0 + rc, h) * DK + c);
        const float4 bv = load4<E>(p.beta, tix(rc) * DK + c);
        const float4 qq = ok ? qv : z4v;
        const float4 G = get(sG + r * (DK + 4) + c);
        put(sR1 + r * LD + c, qq);
        put(sR2 + r * LD + c, ok ? mul4(bv, get(sK + r * (DK + 4) + c)) : z4v);
        put(R + L::oQh + 4 * e, mul4(qq, make_float4(__expf(G.x), __expf(G.y), __expf(G.z), __expf(G.w))));
    }
    __syncthreads();
    for (int t = w; t < 16; t += kGW) {           // Me, Mk (lower, diagonal included)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        f32x4 me = z4, mk = z4;
        if (j0 <= r0) {
            const float* gref = sG + (j0 + 15) * (DK + 4);
            auto Aq = [&](int r, int c) { return sR1[r * LD + c] * aexp(r, c, gref); };
            me = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, Aq, [&](int c, int j) { return sR2[j * LD + c] * bexp(j, c, gref); });
            mk = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DK, Aq, [&](int c, int j) { return sK[j * (DK + 4) + c] * bexp(j, c, gref); });
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
    constexpr int TCD = (kBC / 16) * (DK / 16);
    constexpr int TCV = (kBC / 16) * (DV / 16);
    constexpr int TCC = (kBC / 16) * (kBC / 16);
    constexpr int MT = TCD / kGW;
    __shared__ __attribute__((aligned(16))) float sM1[kBC * CP];
    __shared__ __attribute__((aligned(16))) float sM2[kBC * CP];
    __shared__ __attribute__((aligned(16))) float sR[3 * RS];
    __shared__ float sCol[2 * DK];
    __shared__ float4 sPart[kGT];     // per-thread partial sums of four columns
    float* R0 = sR;
    float* R1 = sR + RS;
    float* R2 = sR + 2 * RS;
    const int u = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int bh = u / N, n = u % N, b = bh / p.H, h = bh % p.H;
    const int t0 = n * kBC, Cn = min(kBC, p.T - t0);
    float* R = ws + static_cast<int64_t>(u) * L::size;
    auto tix = [&](int r) { return tok_index(p, b, t0 + r, h); };
    // the gate of (row r < Cn, channel c) is at or above the log-decay floor (a
    // gate clamped to the floor has no gradient)
    auto gate_kept = [&](int r, int c) { return load_elem<E>(p.g, tix(r) * DK + c) >= kLogDecayFloor; };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const float4 z4v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto put = [](float* dst, float4 x) { *reinterpret_cast<float4*>(dst) = x; };
    auto get = [](const float* src) { return *reinterpret_cast<const float4*>(src); };
    auto ti = [&](int i0, int q) { return i0 + 4 * (l >> 4) + q; };
    auto tj = [&](int j0) { return j0 + (l & 15); };
    // stage rows [i0, i0 + QR) of a [DV][DK] workspace matrix into sM2
    // row blocks of a [DV][DK] workspace matrix, double-buffered through registers:
    // fetch_rows issues the loads, put_rows writes them to sM2 (after a barrier)
    constexpr int NPF = QR * DK / 4 / kGT;
    float4 pf[NPF];
    auto fetch_rows = [&](int64_t src, int i0) {
#pragma unroll
        for (int j = 0; j < NPF; ++j) pf[j] = get(R + src + i0 * DK + 4 * (tid + kGT * j));
    };
    auto put_rows = [&]() {
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int e = 4 * (tid + kGT * j);
            put(sM2 + (e / DK) * (DK + 4) + e % DK, pf[j]);
        }
    };
    // column sums: thread (part, four columns); the parts combined in a fixed order
    auto fma4 = [](float4 x, float4 y, float4 c) {
        return make_float4(fmaf(x.x, y.x, c.x), fmaf(x.y, y.y, c.y), fmaf(x.z, y.z, c.z), fmaf(x.w, y.w, c.w));
    };
    constexpr int CG = DK / 4, NPART = kGT / CG;
    auto col_total = [&](int c) {
        float acc = 0.f;
        for (int part = 0; part < NPART; ++part) {
            const float4 v = sPart[part * CG + c / 4];
            acc += (c & 3) == 0 ? v.x : (c & 3) == 1 ? v.y : (c & 3) == 2 ? v.z : v.w;
        }
        return acc;
    };

    DR_TILE_FOR(e, kBC * DV / 4, kGT) {   // dO -> R0, Y -> R1, X -> R2 (four columns per thread)
        const int r = 4 * e / DV, i = 4 * e % DV;
        const int64_t vi = tix(min(r, Cn - 1)) * DV + i;
        const float4 d = load4<E>(p.dO, vi), wv = load4<E>(p.wgate, vi), vv = load4<E>(p.v, vi);
        put(R0 + r * LD + i, r < Cn ? d : z4v);
        put(R1 + r * LD + i, get(R + L::oVt + 4 * e));
        put(R2 + r * LD + i, r < Cn ? make_float4(wv.x * vv.x, wv.y * vv.y, wv.z * vv.z, wv.w * vv.w) : z4v);
    }
    {   // sum_i S dS' per column
        const int c = 4 * (tid % CG), part = tid / CG, rp = DV / NPART;
        float4 acc = z4v;
#pragma unroll
        for (int k = 0; k < rp; ++k) {
            const int i = part * rp + k;
            acc = fma4(get(R + L::oS + i * DK + c), get(R + L::odS + i * DK + c), acc);
        }
        sPart[tid] = acc;
    }
    __syncthreads();
    if (tid < DK) sCol[tid] = R[L::oGam + tid] * col_total(tid);
    for (int t = w; t < TCC; t += kGW) {          // dMe = -Tril0(dO Y^T), dMk = Tril0(dO X^T)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        // (dO as loaded: exact in bf16 with bf16 inputs)
        const f32x4 me = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DV, exact([&](int r, int i) { return R0[r * LD + i]; }),
                                 [&](int i, int j) { return R1[j * LD + i]; });
        const f32x4 mk = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DV, exact([&](int r, int i) { return R0[r * LD + i]; }),
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
                a1[m] = mm_tile<kSplitMM<E>>(a1[m], r0, c0, i0, i0 + QR, exact([&](int r, int i) { return R0[r * LD + i]; }),
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
                a1[m] = mm_tile<kSplitMM<E>>(a1[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return -R1[r * LD + i]; }, Bs);
                a2[m] = mm_tile<kSplitMM<E>>(a2[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R2[r * LD + i]; }, Bs);
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
        const int c = 4 * (tid % CG), part = tid / CG, rp = kBC / NPART;
        float4 acc = z4v;
#pragma unroll
        for (int k = 0; k < rp; ++k) {
            const int r = part * rp + k;
            acc = fma4(get(R + L::odKb + r * DK + c), get(R + L::oKb + r * DK + c), acc);
            acc = fma4(get(R + L::odEb + r * DK + c), get(R + L::oEb + r * DK + c), acc);
        }
        sPart[tid] = acc;
    }
    DR_TILE_FOR(e, kBC * DV / 4, kGT) put(R0 + (4 * e / DV) * LD + 4 * e % DV, get(R + L::odVt + 4 * e));   // dY -> R0
    __syncthreads();
    if (tid < DK) sCol[DK + tid] = col_total(tid);
    // dW = dY S, kept in registers (the workspace copy is not needed)
    f32x4 dWr[MT];
    {
#pragma unroll
        for (int m = 0; m < MT; ++m) dWr[m] = z4;
        fetch_rows(L::oS, 0);
        for (int i0 = 0; i0 < DV; i0 += QR) {
            __syncthreads();
            put_rows();
            __syncthreads();
            if (i0 + QR < DV) fetch_rows(L::oS, i0 + QR);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
                dWr[m] = mm_tile<kSplitMM<E>>(dWr[m], r0, c0, i0, i0 + QR, [&](int r, int i) { return R0[r * LD + i]; },
                                 [&](int i, int c) { return sM2[(i - i0) * (DK + 4) + c]; });
            }
        }
    }
    // Every operand of the products below is staged in LDS (read from the
    // workspace inside the product loops they cost half the kernel's time):
    // T and tmp in R1, dW in R2 in place of X (X = w v is staged again from
    // the inputs for dAk), second operands of dT 64 columns at a time in sM2.
    float* sT = R1;   // Y is no longer needed
    float* sTmp = R1 + kBC * CP;
    __syncthreads();
    DR_TILE_FOR(e, kBC * kBC / 4, kGT) put(sT + (4 * e / kBC) * CP + 4 * e % kBC, get(R + L::oT + 4 * e));
#pragma unroll
    for (int m = 0; m < MT; ++m) {   // dW -> R2
        const int t = w + kGW * m, r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
#pragma unroll
        for (int q = 0; q < 4; ++q) R2[ti(r0, q) * LD + tj(c0)] = dWr[m][q];
    }
    __syncthreads();
    constexpr int MV = TCV / kGW;   // C x DV tiles per wave
    static_assert(TCV % kGW == 0 && TCC % kGW == 0, "tiles per wave");
    for (int t = w; t < TCV; t += kGW) {          // dZ = T^T dY (to the workspace until R0 is free)
        const int r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int k) { return sT[k * CP + r]; },
                                  [&](int k, int i) { return R0[k * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::odZ + ti(r0, q) * DV + tj(c0)] = acc[q];
    }
    for (int t = w; t < TCD; t += kGW) {          // dKhat = T^T dW
        const int r0 = 16 * (t / (DK / 16)), c0 = 16 * (t % (DK / 16));
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int k) { return sT[k * CP + r]; },
                                  [&](int k, int c) { return R2[k * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) R[L::odKh + ti(r0, q) * DK + tj(c0)] = acc[q];
    }
    // dT = dW Khat^T + dY Z^T
    f32x4 dTr[TCC / kGW];
#pragma unroll
    for (int m = 0; m < TCC / kGW; ++m) dTr[m] = z4;
    for (int h0 = 0; h0 < DK; h0 += 64) {   // Khat[:, h0, h0 + 64) -> sM2
        DR_TILE_FOR(e, kBC * 64 / 4, kGT) {
            const int r = 4 * e / 64, c = 4 * e % 64;
            put(sM2 + r * CP + c, get(R + L::oKh + r * DK + h0 + c));
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TCC / kGW; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            dTr[m] = mm_tile<kSplitMM<E>>(dTr[m], r0, j0, h0, h0 + 64, [&](int r, int c) { return R2[r * LD + c]; },
                             [&](int c, int j) { return sM2[j * CP + c - h0]; });
        }
        __syncthreads();
    }
    for (int h0 = 0; h0 < DV; h0 += 64) {   // Z[:, h0, h0 + 64) -> sM2
        DR_TILE_FOR(e, kBC * 64 / 4, kGT) {
            const int r = 4 * e / 64, i = 4 * e % 64;
            put(sM2 + r * CP + i, get(R + L::oZ + r * DV + h0 + i));
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TCC / kGW; ++m) {
            const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
            dTr[m] = mm_tile<kSplitMM<E>>(dTr[m], r0, j0, h0, h0 + 64, [&](int r, int i) { return R0[r * LD + i]; },
                             [&](int i, int j) { return sM2[j * CP + i - h0]; });
        }
        __syncthreads();
    }
#pragma unroll
    for (int m = 0; m < TCC / kGW; ++m) {   // dT -> sM1; dZ -> R0 (dY is no longer needed)
        const int t = w + kGW * m, r0 = 16 * (t / 4), j0 = 16 * (t % 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) sM1[ti(r0, q) * CP + tj(j0)] = dTr[m][q];
    }
    DR_TILE_FOR(e, kBC * DV / 4, kGT) put(R0 + (4 * e / DV) * LD + 4 * e % DV, get(R + L::odZ + 4 * e));
    DR_TILE_FOR(e, kBC * DV / 4, kGT) {   // X = w v -> R2 (nor is dW)
        const int r = 4 * e / DV, i = 4 * e % DV;
        const int64_t vi = tix(min(r, Cn - 1)) * DV + i;
        const float4 wv = load4<E>(p.wgate, vi), vv = load4<E>(p.v, vi);
        put(R2 + r * LD + i, r < Cn ? make_float4(wv.x * vv.x, wv.y * vv.y, wv.z * vv.z, wv.w * vv.w) : z4v);
    }
    __syncthreads();
    for (int t = w; t < TCC; t += kGW) {          // tmp = dT T^T
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 acc = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, kBC, [&](int r, int m) { return sM1[r * CP + m]; },
                                  [&](int m, int j) { return sT[j * CP + m]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) sTmp[ti(r0, q) * CP + tj(j0)] = acc[q];
    }
    __syncthreads();
    for (int t = w; t < TCC; t += kGW) {          // dAe = -T^T tmp, dAk = StrictTril(dZ X^T)
        const int r0 = 16 * (t / 4), j0 = 16 * (t % 4);
        const f32x4 ae = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, kBC, [&](int r, int m) { return sT[m * CP + r]; },
                                 [&](int m, int j) { return sTmp[m * CP + j]; });
        const f32x4 ak = mm_tile<kSplitMM<E>>(z4, r0, j0, 0, DV, [&](int r, int i) { return R0[r * LD + i]; },
                                 [&](int i, int j) { return R2[j * LD + i]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), j = tj(j0);
            R[L::odAe + r * kBC + j] = j < r ? -ae[q] : 0.f;
            R[L::odAk + r * kBC + j] = j < r ? ak[q] : 0.f;
        }
    }
    __syncthreads();
    // dX = Mk^T dO + Ak^T dZ + Kbar dS'^T -> dv, dw: Mk -> sM1, Ak -> sM2, dO -> R2
    // (X is no longer needed), Kbar -> R1 (nor are T and tmp); then dS' -> R0, R2
    DR_TILE_FOR(e, kBC * kBC / 4, kGT) {
        const int r = 4 * e / kBC, j = 4 * e % kBC;
        put(sM1 + r * CP + j, get(R + L::oMk + 4 * e));
        put(sM2 + r * CP + j, get(R + L::oAk + 4 * e));
    }
    DR_TILE_FOR(e, kBC * DV / 4, kGT) {
        const int r = 4 * e / DV, i = 4 * e % DV;
        const float4 d = load4<E>(p.dO, tix(min(r, Cn - 1)) * DV + i);
        put(R2 + r * LD + i, r < Cn ? d : z4v);
    }
    DR_TILE_FOR(e, kBC * DK / 4, kGT) put(R1 + (4 * e / DK) * LD + 4 * e % DK, get(R + L::oKb + 4 * e));
    __syncthreads();
    f32x4 dXr[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) {
        const int t = w + kGW * m, r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        dXr[m] = mm_tile<kSplitMM<E>>(z4, r0, c0, 0, kBC, [&](int r, int k) { return sM1[k * CP + r]; },
                         exact([&](int k, int i) { return R2[k * LD + i]; }));   // dO as loaded
        dXr[m] = mm_tile<kSplitMM<E>>(dXr[m], r0, c0, 0, kBC, [&](int r, int k) { return sM2[k * CP + r]; },
                         [&](int k, int i) { return R0[k * LD + i]; });
    }
    __syncthreads();
    static_assert(DV <= 128 && kBC * LD <= RS, "dS' rows in R0 and R2");
    DR_TILE_FOR(e, DV * DK / 4, kGT) {   // dS' rows [0, 64) -> R0, [64, DV) -> R2
        const int i = 4 * e / DK, c = 4 * e % DK;
        put((i < 64 ? R0 + i * LD : R2 + (i - 64) * LD) + c, get(R + L::odS + 4 * e));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MV; ++m) {
        const int t = w + kGW * m, r0 = 16 * (t / (DV / 16)), c0 = 16 * (t % (DV / 16));
        const float* dsb = c0 < 64 ? R0 : R2 - 64 * LD;   // row i of dS' at dsb + i LD
        dXr[m] = mm_tile<kSplitMM<E>>(dXr[m], r0, c0, 0, DK, [&](int r, int c) { return R1[r * LD + c]; },
                         [&](int c, int i) { return dsb[i * LD + c]; });
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = ti(r0, q), i = tj(c0);
            if (r < Cn) {
                const int64_t vi = tix(r) * DV + i;
                store_elem<E>(p.gv, vi, load_elem<E>(p.wgate, vi) * dXr[m][q]);
                store_elem<E>(p.gw, vi, load_elem<E>(p.v, vi) * dXr[m][q]);
            }
        }
    }
    __syncthreads();
    // pairwise passes on 16 x 16 tiles of (r, c); accumulators per tile element
    f32x4 aq[MT], ak[MT], abk[MT], ag[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) aq[m] = ak[m] = abk[m] = ag[m] = z4;
    auto stage = [&](float* dst, int what) {   // 0 q, 1 k, 2 b k, 3 G
        if (what == 3) {
            DR_TILE_FOR(e, kBC * DK / 4, kGT) put(dst + (4 * e / DK) * LD + 4 * e % DK, get(R + L::oG + 4 * e));
        } else {
            const void* src = what == 0 ? p.q : p.k;
            DR_TILE_FOR(e, kBC * DK / 4, kGT) {
                const int r = 4 * e / DK, c = 4 * e % DK;
                const int rc = min(r, Cn - 1);
                float4 x = load4<E>(src, qk_index(p, b, t0 + rc, h) * DK + c);
                if (what == 2) {
                    const float4 bv = load4<E>(p.beta, tix(rc) * DK + c);
                    x = make_float4(x.x * bv.x, x.y * bv.y, x.z * bv.z, x.w * bv.w);
                }
                put(dst + r * LD + c, r < Cn ? x : z4v);
            }
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
    DR_TILE_FOR(e, kBC * kBC / 4, kGT) {
        put(sM1 + (4 * e / kBC) * CP + 4 * e % kBC, get(R + L::odMe + 4 * e));
        put(sM2 + (4 * e / kBC) * CP + 4 * e % kBC, get(R + L::odMk + 4 * e));
    }
    stage(R0, 0);
    stage(R2, 3);
    stage(R1, 2);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {   // Me terms
        int r0, c0;
        tile_of(m, r0, c0);
        const f32x4 row = pair_tile<true, kSplitMM<E>>(r0, c0, M1, X1, Gf);
        const f32x4 col = pair_tile<false, kSplitMM<E>>(r0, c0, M1, X0, Gf);
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
        const f32x4 row = pair_tile<true, kSplitMM<E>>(r0, c0, M2, X1, Gf);
        const f32x4 col = pair_tile<false, kSplitMM<E>>(r0, c0, M2, X0, Gf);
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
    DR_TILE_FOR(e, kBC * kBC / 4, kGT) {
        put(sM1 + (4 * e / kBC) * CP + 4 * e % kBC, get(R + L::odAe + 4 * e));
        put(sM2 + (4 * e / kBC) * CP + 4 * e % kBC, get(R + L::odAk + 4 * e));
    }
    stage(R0, 2);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int r0, c0;
        tile_of(m, r0, c0);
        const f32x4 rowe = pair_tile<true, kSplitMM<E>>(r0, c0, M1, X0, Gf);
        const f32x4 cole = pair_tile<false, kSplitMM<E>>(r0, c0, M1, X1, Gf);
        const f32x4 rowk = pair_tile<true, kSplitMM<E>>(r0, c0, M2, X1, Gf);
        const f32x4 colk = pair_tile<false, kSplitMM<E>>(r0, c0, M2, X1, Gf);
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
            if (r < Cn) store_elem<E>(p.gg, tix(r) * DK + c, gate_kept(r, c) ? acc : 0.f);
        }
    }
}

template <typename E, int DK, int DV>
hipError_t launch_bwd2_dims(const BwdArgs& a, hipStream_t s) {
    const int N = (a.T + kBC - 1) / kBC;
    const int64_t units = static_cast<int64_t>(a.B) * a.H * N;
    if (units > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    float* ws = static_cast<float*>(a.ws);   // one record per unit (bwd_workspace_bytes)
    const dim3 blk(kCT);
    const unsigned chains = chain_grid(a, DV);
    hipLaunchKernelGGL((bwd2_prep_kernel<E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        if constexpr (kSplitMM<E>)
            hipLaunchKernelGGL((bwd_fchain_split_kernel<BwdWs2<DK, DV>, E, DK, DV, true>), dim3(chains), blk, 0, s, a, ws, N);
        else
            hipLaunchKernelGGL((bwd_fchain_kernel<BwdWs2<DK, DV>, E, DK, DV, true>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        if constexpr (kSplitMM<E>)
            hipLaunchKernelGGL((bwd_rchain_split_kernel<BwdWs2<DK, DV>, E, DK, DV, true>), dim3(chains), blk, 0, s, a, ws, N);
        else
            hipLaunchKernelGGL((bwd_rchain_kernel<BwdWs2<DK, DV>, E, DK, DV, true>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd2_grads_kernel<E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
        e = hipGetLastError();
    }
    return e;
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

// With grouped query/key heads the kernels write per-value-head dq, dk to two
// fp32 buffers at the end of the workspace, summed into the outputs by one more
// launch.
template <typename E>
hipError_t bwd_with_groups(int variant, BwdArgs a, hipStream_t s, hipError_t (*run)(const BwdArgs&, hipStream_t)) {
    if (a.Hk == a.H) {
        a.gq32 = a.gk32 = nullptr;
        return run(a, s);
    }
    const size_t per = round_up_256(static_cast<size_t>(a.B) * a.T * a.H * a.dk * 4);
    unsigned char* buf = static_cast<unsigned char*>(a.ws) + bwd_workspace_bytes(variant, a.B, a.T, a.H, a.H, a.dk, a.dv);
    a.gq32 = reinterpret_cast<float*>(buf);
    a.gk32 = reinterpret_cast<float*>(buf + per);
    hipError_t e = run(a, s);
    if (e == hipSuccess) {
        const int64_t n = static_cast<int64_t>(a.B) * a.T * a.Hk * a.dk;
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, int64_t(1) << 16);
        hipLaunchKernelGGL((bwd_group_sum_kernel<E>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a, n);
        e = hipGetLastError();
    }
    return e;
}

template <int VAR, typename E, int DK, int DV>
hipError_t launch_bwd_dims(const BwdArgs& a, hipStream_t s) {
    const int N = (a.T + kBC - 1) / kBC;
    const int64_t units = static_cast<int64_t>(a.B) * a.H * N;
    if (units > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    float* ws = static_cast<float*>(a.ws);   // one record per unit (bwd_workspace_bytes)
    const dim3 blk(kCT);
    const unsigned chains = chain_grid(a, DV);
    if constexpr (VAR <= 1 && kSplitMM<E>)
        hipLaunchKernelGGL((bwd_prep_bf16_kernel<VAR, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<VAR, E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        if constexpr (kSplitMM<E>)
            hipLaunchKernelGGL((bwd_fchain_split_kernel<BwdWs1<VAR, DK, DV>, E, DK, DV, false>), dim3(chains), blk, 0, s, a, ws, N);
        else
            hipLaunchKernelGGL((bwd_fchain_kernel<BwdWs1<VAR, DK, DV>, E, DK, DV, false>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        if constexpr (kSplitMM<E>)
            hipLaunchKernelGGL((bwd_rchain_split_kernel<BwdWs1<VAR, DK, DV>, E, DK, DV, false>), dim3(chains), blk, 0, s, a, ws, N);
        else
            hipLaunchKernelGGL((bwd_rchain_kernel<BwdWs1<VAR, DK, DV>, E, DK, DV, false>), dim3(chains), blk, 0, s, a, ws, N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL((bwd_grads_kernel<VAR, E, DK, DV>), dim3(static_cast<unsigned>(units)), dim3(kGT), 0, s, a, ws, N);
        e = hipGetLastError();
    }
    return e;
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
    return dtype == 0 ? bwd_with_groups<F32>(VAR, a, s, launch_bwd_var<VAR, F32>)
                      : bwd_with_groups<BF16>(VAR, a, s, launch_bwd_var<VAR, BF16>);
}

}  // namespace

template <int DK, int DV>
size_t bwd_records_bytes(int variant, int64_t units) {
    const int64_t rec = variant == 3 ? BwdWs2<DK, DV>::size : variant <= 1 ? BwdWsS<DK, DV>::size : BwdWs<DK, DV>::size;
    return round_up_256(static_cast<size_t>(units * rec * 4));
}

size_t bwd_workspace_bytes(int variant, int B, int T, int H, int Hk, int dk, int dv) {
    const int64_t units = static_cast<int64_t>(B) * H * ((T + kBC - 1) / kBC);
    size_t n;
    if (dk == 128) n = dv == 128 ? bwd_records_bytes<128, 128>(variant, units) : bwd_records_bytes<128, 64>(variant, units);
    else n = dv == 128 ? bwd_records_bytes<64, 128>(variant, units) : bwd_records_bytes<64, 64>(variant, units);
    if (Hk != H) n += 2 * round_up_256(static_cast<size_t>(B) * T * H * dk * 4);   // per-value-head dq, dk
    return n;
}

hipError_t launch_bwd(int variant, int dtype, const BwdArgs& a, hipStream_t s) {
    switch (variant) {
        case 0: return launch_bwd_dtype<0>(dtype, a, s);
        case 1: return launch_bwd_dtype<1>(dtype, a, s);
        case 2: return launch_bwd_dtype<2>(dtype, a, s);
        case 4: return launch_bwd_dtype<4>(dtype, a, s);
        default: return dtype == 0 ? bwd_with_groups<F32>(3, a, s, launch_bwd2_dtype<F32>)
                                   : bwd_with_groups<BF16>(3, a, s, launch_bwd2_dtype<BF16>);
    }
}

}  // namespace dr
