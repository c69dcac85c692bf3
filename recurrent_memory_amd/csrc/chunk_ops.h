// MFMA and LDS building blocks shared by the chunkwise kernels (gfx950).
//
// Layout conventions (16x16 tiles, 64-lane wave, g = lane / 16, c = lane % 16):
//  - an fp32 accumulator tile holds rows 4 g + i (i = 0..3) of column c;
//  - a contraction over the rows of such a tile uses it directly as an MFMA
//    operand ("register tile"), once the other operand is read from LDS with
//    the same row order (the k index of MFMA slot (g, i) is the same for the
//    A and the B operand, whatever order the hardware sums them in);
//  - LDS matrices are row-major with a padded leading dimension.
#pragma once

#include "common.h"

namespace dr {
namespace {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroup barrier that waits only for this wave's LDS traffic.  A plain
// __syncthreads() also drains outstanding global loads (vmcnt(0)), which would
// pull the next chunk's prefetch onto the critical path at every barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS transpose load (16-bit elements).  Within each group of 16 lanes, lane
// p supplies the address of 4 consecutive elements; lane i receives element
// i % 4 of the piece addressed by lane 4 j + i / 4, for j = 0..3.  Lane p of
// group g therefore points at row r0 + 4 g + p / 4, columns c0 + 4 (p % 4) of
// a row-major tile, and lane c receives rows r0 + 4 g + j of column c0 + c.
__device__ __forceinline__ bf16x4 tr_load(const uint16_t* base, int ld, int r0, int c0, int g, int c) {
    const uint16_t* p = base + (r0 + 4 * g + (c >> 2)) * ld + c0 + 4 * (c & 3);
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Operand handling per input dtype.  S = LDS storage element, R = a 16x16
// register tile converted to operand form (4 values per lane).
template <typename E>
struct Ops;

template <>
struct Ops<BF16> {
    typedef uint16_t S;
    typedef bf16x4 R;
    static constexpr int kPad = 8;  // LDS row padding in elements (16 bytes)
    __device__ static __forceinline__ S enc(float x) { return f32_to_bf16_bits(x); }
    __device__ static __forceinline__ R to_reg(f32x4 x) {
        R r;
        r[0] = static_cast<bf16_t>(x[0]);
        r[1] = static_cast<bf16_t>(x[1]);
        r[2] = static_cast<bf16_t>(x[2]);
        r[3] = static_cast<bf16_t>(x[3]);
        return r;
    }
    // acc += A[16 x K] · B[16 x K]^T, both row-major in LDS; arow/brow point
    // at this lane's row (tile row lane % 16).  Fragments are read first.
    template <int K>
    __device__ static __forceinline__ f32x4 nat(f32x4 acc, const S* arow, const S* brow, int g) {
        bf16x8 a[K / 32], b[K / 32];
#pragma unroll
        for (int k = 0; k < K / 32; ++k) {
            a[k] = *reinterpret_cast<const bf16x8*>(arow + 32 * k + 8 * g);
            b[k] = *reinterpret_cast<const bf16x8*>(brow + 32 * k + 8 * g);
        }
#pragma unroll
        for (int k = 0; k < K / 32; ++k) acc = mfma32(a[k], b[k], acc);
        return acc;
    }
    // acc += A[16 x 16 (T1 - T0)] · [X[T0]; ...; X[T1 - 1]]: contraction over
    // the rows of register tiles.  arow points at this lane's row of A in LDS;
    // A's column 16 t + 4 g + i pairs with row 4 g + i of tile t.  An odd tile
    // count ends with a zero-padded 16x16x32 step: the 16x16x16 instruction is
    // not mixed in, because hipcc (ROCm 7.2) can issue it without the wait
    // states required after a 16x16x32 MFMA that produced its accumulator.
    template <int T0, int T1, int N>
    __device__ static __forceinline__ f32x4 reg(f32x4 acc, const S* arow, const R (&X)[N], int g) {
        constexpr int NP = (T1 - T0 + 1) / 2;
        bf16x8 a[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int t = T0 + 2 * q;
            const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(arow + 16 * t + 4 * g);
            bf16x4 a1 = {0, 0, 0, 0};
            if (t + 1 < T1) a1 = *reinterpret_cast<const bf16x4*>(arow + 16 * (t + 1) + 4 * g);
            a[q] = cat(a0, a1);
        }
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int t = T0 + 2 * q;
            const bf16x4 z = {0, 0, 0, 0};
            const bf16x8 b = cat(X[t], t + 1 < T1 ? X[t + 1] : z);
            acc = mfma32(a[q], b, acc);
        }
        return acc;
    }
    // acc += M^T[rows c0 .. c0 + 15] · [X[0]; ...; X[NT - 1]] where M is a
    // row-major (chunk row, column) tile in LDS with leading dimension ld:
    // the A operand is M transposed, read with the transpose load.
    template <int NT, int N>
    __device__ static __forceinline__ f32x4 regT(f32x4 acc, const S* M, int ld, int c0, const R (&X)[N],
                                               int g, int c) {
        constexpr int NP = (NT + 1) / 2;
        const bf16x4 z = {0, 0, 0, 0};
        bf16x8 a[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q)
            a[q] = cat(tr_load(M, ld, 32 * q, c0, g, c), 2 * q + 1 < NT ? tr_load(M, ld, 32 * q + 16, c0, g, c) : z);
#pragma unroll
        for (int q = 0; q < NP; ++q) acc = mfma32(a[q], cat(X[2 * q], 2 * q + 1 < NT ? X[2 * q + 1] : z), acc);
        return acc;
    }
    // A 16 x 16 tile of a row-major LDS matrix in accumulator layout:
    // element i of lane (g, c) is M[r0 + 4 g + i][c0 + c].
    __device__ static __forceinline__ f32x4 acc_tile(const S* M, int ld, int r0, int c0, int g, int c) {
        const bf16x4 v = tr_load(M, ld, r0, c0, g, c);
        return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                     static_cast<float>(v[3])};
    }
};

template <>
struct Ops<F32> {
    typedef float S;
    typedef f32x4 R;
    static constexpr int kPad = 4;
    __device__ static __forceinline__ S enc(float x) { return x; }
    __device__ static __forceinline__ R to_reg(f32x4 x) { return x; }
    template <int K>
    __device__ static __forceinline__ f32x4 nat(f32x4 acc, const S* arow, const S* brow, int g) {
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 4) acc = mfma4(arow[k0 + g], brow[k0 + g], acc);
        return acc;
    }
    template <int T0, int T1, int N>
    __device__ static __forceinline__ f32x4 reg(f32x4 acc, const S* arow, const R (&X)[N], int g) {
#pragma unroll
        for (int t = T0; t < T1; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma4(arow[16 * t + 4 * g + i], X[t][i], acc);
        }
        return acc;
    }
    template <int NT, int N>
    __device__ static __forceinline__ f32x4 regT(f32x4 acc, const S* M, int ld, int c0, const R (&X)[N],
                                               int g, int c) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma4(M[(16 * t + 4 * g + i) * ld + c0 + c], X[t][i], acc);
        }
        return acc;
    }
    __device__ static __forceinline__ f32x4 acc_tile(const S* M, int ld, int r0, int c0, int g, int c) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = M[(r0 + 4 * g + i) * ld + c0 + c];
        return v;
    }
};

// fp32 operands in LDS and registers; each product is hi*hi + hi*lo + lo*hi of
// the bf16 split x = hi + lo + e (|e| <= 2^-18 |x|, both parts rounded to nearest
// even), fp32 accumulation: a relative error of about 2^-17 per product term.
struct SplitTile {
    bf16x4 h, l;
};
template <>
struct Ops<F32S> {
    typedef float S;
    typedef SplitTile R;
    static constexpr int kPad = 4;
    __device__ static __forceinline__ S enc(float x) { return x; }
    __device__ static __forceinline__ void split(float x, bf16_t& h, bf16_t& l) {
        h = static_cast<bf16_t>(x);
        l = static_cast<bf16_t>(x - static_cast<float>(h));
    }
    __device__ static __forceinline__ R to_reg(f32x4 x) {
        R r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16_t h, l;
            split(x[i], h, l);
            r.h[i] = h;
            r.l[i] = l;
        }
        return r;
    }
    __device__ static __forceinline__ R split4(float4 v) { return to_reg(f32x4{v.x, v.y, v.z, v.w}); }
    __device__ static __forceinline__ f32x4 mma(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                                const bf16x8& bl, f32x4 acc) {
        acc = mfma32(al, bh, acc);
        acc = mfma32(ah, bl, acc);
        return mfma32(ah, bh, acc);
    }
    // acc += A[16 x K] · B[16 x K]^T, both row-major in LDS (lane slot e of group
    // g holds k = 32 k0 + 8 g + e for both operands)
    template <int K>
    __device__ static __forceinline__ f32x4 nat(f32x4 acc, const S* arow, const S* brow, int g) {
#pragma unroll
        for (int k = 0; k < K; k += 32) {
            const R a0 = split4(*reinterpret_cast<const float4*>(arow + k + 8 * g));
            const R a1 = split4(*reinterpret_cast<const float4*>(arow + k + 8 * g + 4));
            const R b0 = split4(*reinterpret_cast<const float4*>(brow + k + 8 * g));
            const R b1 = split4(*reinterpret_cast<const float4*>(brow + k + 8 * g + 4));
            acc = mma(cat(a0.h, a1.h), cat(a0.l, a1.l), cat(b0.h, b1.h), cat(b0.l, b1.l), acc);
        }
        return acc;
    }
    // contraction over the rows of register tiles, as Ops<BF16>::reg (two tiles
    // per 16x16x32 step, an odd count padded with zeros)
    template <int T0, int T1, int N>
    __device__ static __forceinline__ f32x4 reg(f32x4 acc, const S* arow, const R (&X)[N], int g) {
        const bf16x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int t = T0; t < T1; t += 2) {
            const R a0 = split4(*reinterpret_cast<const float4*>(arow + 16 * t + 4 * g));
            R a1 = {z, z};
            if (t + 1 < T1) a1 = split4(*reinterpret_cast<const float4*>(arow + 16 * (t + 1) + 4 * g));
            const bf16x4 x1h = t + 1 < T1 ? X[t + 1].h : z, x1l = t + 1 < T1 ? X[t + 1].l : z;
            acc = mma(cat(a0.h, a1.h), cat(a0.l, a1.l), cat(X[t].h, x1h), cat(X[t].l, x1l), acc);
        }
        return acc;
    }
    // acc += M^T[rows c0 .. c0 + 15] · [X[0]; ...; X[NT - 1]], M row-major in LDS
    template <int NT, int N>
    __device__ static __forceinline__ f32x4 regT(f32x4 acc, const S* M, int ld, int c0, const R (&X)[N],
                                               int g, int c) {
        const bf16x4 z = {0, 0, 0, 0};
        auto col = [&](int t) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = M[(16 * t + 4 * g + i) * ld + c0 + c];
            return to_reg(v);
        };
#pragma unroll
        for (int t = 0; t < NT; t += 2) {
            const R a0 = col(t);
            R a1 = {z, z};
            if (t + 1 < NT) a1 = col(t + 1);
            const bf16x4 x1h = t + 1 < NT ? X[t + 1].h : z, x1l = t + 1 < NT ? X[t + 1].l : z;
            acc = mma(cat(a0.h, a1.h), cat(a0.l, a1.l), cat(X[t].h, x1h), cat(X[t].l, x1l), acc);
        }
        return acc;
    }
    __device__ static __forceinline__ f32x4 acc_tile(const S* M, int ld, int r0, int c0, int g, int c) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = M[(r0 + 4 * g + i) * ld + c0 + c];
        return v;
    }
};

}  // namespace
}  // namespace dr
