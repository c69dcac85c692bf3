// DeltaTTT-pre: a two-layer memory whose layers each learn by delta-rule steps
// (DeltaTTT summary, paperlayer.ai, §4.1 "Layerwise memory optimization" and
// the Pre schedule; Appendix A, chunkwise scan of DeltaTTT).
//
// The first layer A [dv, dk] learns keys -> values.  In the Pre schedule the
// second layer's write key for token t comes from the first layer's state
// before token t's write, so the second layer is an ordinary delta-rule scan
// whose keys and queries are known once the first scan is done:
//   r_t = A'_t k_t            (A'_t = A_{t-1} Diag(a1_t), the first layer's prediction)
//   h_t = unit(silu(r_t)),    z_t = unit(silu(A_t q_t))
//   B_t = B'_t + beta2_t (v_t - B'_t h_t) h_t^T,   o_t = B_t z_t
// The pre-write reads r_t come from a second first-layer scan with shifted
// queries: its readout after token s is A_s (a1_{s+1} ⊙ k_{s+1}) = r_{s+1}, and
// r_0 = A'_0 k_0 is one matrix-vector product per head.  So the whole layer is
// five launches: r_0, the shifted queries, the two first-layer scans and the
// key/query transform, then the second-layer scan, each scan being delta_fwd's
// chunkwise kernel.
//
// bf16 operands are first widened to fp32 and the whole layer runs on the fp32
// path; only the output is rounded back to bf16.  The intermediate reads, keys
// and queries then carry no bf16 rounding: with bf16 keys and queries the
// second layer's readout B_t z_t picks up a rounding error of the size of what
// B_t stores, which is large next to |o_t| when z_t is nearly orthogonal to it.
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kTttThreads = 256;

// 16 bytes of dtype elements <-> fp32
template <typename E>
struct Vec16 {
    static constexpr int N = 16 / E::bytes;
    __device__ static void unpack(const uint4& u, float (&x)[N]) {
        if constexpr (E::bytes == 4) {
            x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
            x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
        } else {
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
                x[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(w[i] >> 16));
            }
        }
    }
    __device__ static uint4 pack(const float (&x)[N]) {
        if constexpr (E::bytes == 4) {
            return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
        } else {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i])) |
                       (static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i + 1])) << 16);
            return make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
};

// q_s[b, s, h, :] = a1(b, s + 1, h) k[b, s + 1, h, :] for s < T - 1; zero at s = T - 1.
// 16 bytes per thread (d_k is a multiple of 64, so a piece never straddles rows).
template <typename E, int VAR>
__global__ __launch_bounds__(kTttThreads) void ttt_shift_kernel(TttArgs p, int64_t npieces) {
    typedef Vec16<E> V;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kTttThreads;
    for (int64_t iv = static_cast<int64_t>(blockIdx.x) * kTttThreads + threadIdx.x; iv < npieces; iv += stride) {
        const int64_t e = iv * V::N;
        const int64_t row = e / p.dk;              // (b, s, h)
        const int s = static_cast<int>((row / p.H) % p.T);
        uint4 out = make_uint4(0u, 0u, 0u, 0u);
        if (s + 1 < p.T) {
            const int64_t next = row + p.H;        // (b, s + 1, h)
            out = *reinterpret_cast<const uint4*>(static_cast<const typename E::T*>(p.k) + next * p.dk + e % p.dk);
            if constexpr (VAR == 1) {
                const float a = __expf(load_elem<E>(p.g1, next));
                float x[V::N];
                V::unpack(out, x);
#pragma unroll
                for (int i = 0; i < V::N; ++i) x[i] *= a;
                out = V::pack(x);
            }
        }
        *reinterpret_cast<uint4*>(static_cast<typename E::T*>(p.qs) + e) = out;
    }
}

// r0[b, h, i] = a1(b, 0, h) sum_c A0[b, h, i, c] k[b, 0, h, c]; zero without A0.
// One workgroup per (b, h), one value row per thread.
template <typename E, int VAR>
__global__ __launch_bounds__(kTttThreads) void ttt_r0_kernel(TttArgs p) {
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh % p.H;
    const int64_t krow = static_cast<int64_t>(b) * p.T * p.H + h;   // token 0 of sequence b
    float a = 1.f;
    if constexpr (VAR == 1) a = __expf(load_elem<E>(p.g1, krow));
    for (int i = threadIdx.x; i < p.dv; i += kTttThreads) {
        float acc = 0.f;
        if (p.A0) {
            const float* row = p.A0 + (static_cast<int64_t>(bh) * p.dv + i) * p.dk;
            for (int c = 0; c < p.dk; ++c) acc = fmaf(row[c], load_elem<E>(p.k, krow * p.dk + c), acc);
        }
        store_elem<E>(p.r0, static_cast<int64_t>(bh) * p.dv + i, a * acc);
    }
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

// Per row (b, t, h): r = r_t (r0 at t = 0, else the shifted scan's readout of
// token t - 1), h = unit(silu(r)), z = unit(silu(o1)); a zero vector stays
// zero.  LPR lanes per row, 16 bytes each; the row sums are xor butterflies
// within the LPR lanes.
template <typename E, int DV>
__global__ __launch_bounds__(kTttThreads) void ttt_glue_kernel(TttArgs p, int64_t rows) {
    typedef Vec16<E> V;
    typedef typename E::T Raw;
    constexpr int LPR = DV / V::N;                 // 8, 16 or 32
    constexpr int RPB = kTttThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * RPB;
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR; row < rows; row += stride) {
        const int h = static_cast<int>(row % p.H);
        const int64_t bt = row / p.H;
        const int t = static_cast<int>(bt % p.T);
        const int64_t b = bt / p.T;
        const Raw* rsrc = t == 0 ? static_cast<const Raw*>(p.r0) + (b * p.H + h) * DV
                                 : static_cast<const Raw*>(p.rd) + (row - p.H) * DV;
        float r[V::N], z[V::N];
        V::unpack(*reinterpret_cast<const uint4*>(rsrc + sub * V::N), r);
        V::unpack(*reinterpret_cast<const uint4*>(static_cast<const Raw*>(p.o1) + row * DV + sub * V::N), z);
        float sr = 0.f, sz = 0.f;
#pragma unroll
        for (int i = 0; i < V::N; ++i) {
            r[i] = silu(r[i]);
            z[i] = silu(z[i]);
            sr += r[i] * r[i];
            sz += z[i] * z[i];
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {
            sr += __shfl_xor(sr, m, LPR);
            sz += __shfl_xor(sz, m, LPR);
        }
        const float ir = sr > 0.f ? rsqrtf(sr) : 0.f, iz = sz > 0.f ? rsqrtf(sz) : 0.f;
#pragma unroll
        for (int i = 0; i < V::N; ++i) {
            r[i] *= ir;
            z[i] *= iz;
        }
        *reinterpret_cast<uint4*>(static_cast<Raw*>(p.hk) + row * DV + sub * V::N) = V::pack(r);
        *reinterpret_cast<uint4*>(static_cast<Raw*>(p.zq) + row * DV + sub * V::N) = V::pack(z);
    }
}

// dst[i] = src[i] between bf16 and fp32 (either direction), 8 elements per
// thread and step; the last n % 8 elements one by one.
template <typename From, typename To>
__global__ __launch_bounds__(kTttThreads) void ttt_convert_kernel(const void* src, void* dst, int64_t n) {
    const int64_t n8 = n / 8, stride = static_cast<int64_t>(gridDim.x) * kTttThreads;
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kTttThreads + threadIdx.x;
    for (int64_t i = i0; i < n8; i += stride) {
        float x[8];
        if constexpr (From::bytes == 2) {
            Vec16<BF16>::unpack(reinterpret_cast<const uint4*>(src)[i], x);
        } else {
            float y[4];
            Vec16<F32>::unpack(reinterpret_cast<const uint4*>(src)[2 * i], y);
            for (int j = 0; j < 4; ++j) x[j] = y[j];
            Vec16<F32>::unpack(reinterpret_cast<const uint4*>(src)[2 * i + 1], y);
            for (int j = 0; j < 4; ++j) x[4 + j] = y[j];
        }
        if constexpr (To::bytes == 2) {
            reinterpret_cast<uint4*>(dst)[i] = Vec16<BF16>::pack(x);
        } else {
            const float lo[4] = {x[0], x[1], x[2], x[3]}, hi[4] = {x[4], x[5], x[6], x[7]};
            reinterpret_cast<uint4*>(dst)[2 * i] = Vec16<F32>::pack(lo);
            reinterpret_cast<uint4*>(dst)[2 * i + 1] = Vec16<F32>::pack(hi);
        }
    }
    for (int64_t i = 8 * n8 + i0; i < n; i += stride) store_elem<To>(dst, i, load_elem<From>(src, i));
}

unsigned grid_for(int64_t work, int per_block) {
    const int64_t blocks = (work + per_block - 1) / per_block;
    return static_cast<unsigned>(blocks < 16384 ? (blocks > 0 ? blocks : 1) : 16384);
}

// Pieces of the workspace: shifted queries, their readouts, the first-layer
// readouts, the second layer's keys and queries, the token-0 reads.
struct TttPieces {
    int64_t qs, rd, o1, hk, zq, r0, total;
};
TttPieces ttt_pieces(int64_t eb, int B, int T, int H, int dk, int dv) {
    const int64_t tok = static_cast<int64_t>(B) * T * H;
    auto up = [](int64_t bytes) { return static_cast<int64_t>(round_up_256(static_cast<size_t>(bytes))); };
    TttPieces p;
    p.qs = 0;
    p.rd = p.qs + up(tok * dk * eb);
    p.o1 = p.rd + up(tok * dv * eb);
    p.hk = p.o1 + up(tok * dv * eb);
    p.zq = p.hk + up(tok * dv * eb);
    p.r0 = p.zq + up(tok * dv * eb);
    p.total = p.r0 + up(static_cast<int64_t>(B) * H * dv * eb);
    return p;
}

// split: the scans' products as three bf16 terms of the split fp32 operands (the
// bf16-input path, whose tolerance is that of bf16 data)
template <typename E, int VAR>
hipError_t launch_ttt_typed(TttArgs a, hipStream_t s, bool split = false) {
    const int64_t tok = static_cast<int64_t>(a.B) * a.T * a.H;
    const int64_t nq = tok * a.dk;
    const TttPieces pc = ttt_pieces(E::bytes, a.B, a.T, a.H, a.dk, a.dv);
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    a.qs = ws + pc.qs;
    a.rd = ws + pc.rd;
    a.o1 = ws + pc.o1;
    a.hk = ws + pc.hk;
    a.zq = ws + pc.zq;
    a.r0 = ws + pc.r0;
    hipError_t e;
    // the two reads of A0 come before the first-layer scan that may overwrite it
    hipLaunchKernelGGL((ttt_r0_kernel<E, VAR>), dim3(static_cast<unsigned>(a.B * a.H)), dim3(kTttThreads), 0, s, a);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int64_t pieces = nq / Vec16<E>::N;
        hipLaunchKernelGGL((ttt_shift_kernel<E, VAR>), dim3(grid_for(pieces, kTttThreads)), dim3(kTttThreads), 0, s, a, pieces);
        e = hipGetLastError();
    }
    const int dt = E::bytes == 4 ? 0 : 1;
    if (e == hipSuccess) {   // pre-write reads: readouts of the shifted queries
        FwdArgs f{a.B, a.T, a.H, a.dk, a.dv, a.qs, a.k, a.v, a.beta1, nullptr, a.g1, a.A0, a.rd, nullptr, a.H};
        e = split ? launch_fwd_split(VAR, f, s) : launch_fwd(VAR, dt, f, s);
    }
    if (e == hipSuccess) {   // first layer: readout after the write, final state
        FwdArgs f{a.B, a.T, a.H, a.dk, a.dv, a.q, a.k, a.v, a.beta1, nullptr, a.g1, a.A0, a.o1, a.AT, a.H};
        e = split ? launch_fwd_split(VAR, f, s) : launch_fwd(VAR, dt, f, s);
    }
    if (e == hipSuccess) {
        constexpr int N = Vec16<E>::N;
        if (a.dv == 128)
            hipLaunchKernelGGL((ttt_glue_kernel<E, 128>), dim3(grid_for(tok, kTttThreads / (128 / N))), dim3(kTttThreads), 0, s, a, tok);
        else
            hipLaunchKernelGGL((ttt_glue_kernel<E, 64>), dim3(grid_for(tok, kTttThreads / (64 / N))), dim3(kTttThreads), 0, s, a, tok);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {   // second layer: keys h, queries z, the same values
        FwdArgs f{a.B, a.T, a.H, a.dv, a.dv, a.zq, a.hk, a.v, a.beta2, nullptr, a.g2, a.B0, a.o, a.BT, a.H};
        e = split ? launch_fwd_split(VAR, f, s) : launch_fwd(VAR, dt, f, s);
    }
    return e;
}

// bf16 operands: fp32 copies of q, k, v, beta1, g1, beta2, g2 and of the output
// come first in the workspace, then the fp32 path's own pieces.
struct TttWide {
    int64_t q, k, v, b1, g1, b2, g2, o, rest, total;
};
TttWide ttt_wide(int B, int T, int H, int dk, int dv) {
    const int64_t tok = static_cast<int64_t>(B) * T * H;
    auto up = [](int64_t bytes) { return static_cast<int64_t>(round_up_256(static_cast<size_t>(bytes))); };
    TttWide w;
    w.q = 0;
    w.k = w.q + up(tok * dk * 4);
    w.v = w.k + up(tok * dk * 4);
    w.b1 = w.v + up(tok * dv * 4);
    w.g1 = w.b1 + up(tok * 4);
    w.b2 = w.g1 + up(tok * 4);
    w.g2 = w.b2 + up(tok * 4);
    w.o = w.g2 + up(tok * 4);
    w.rest = w.o + up(tok * dv * 4);
    w.total = w.rest + ttt_pieces(4, B, T, H, dk, dv).total;
    return w;
}

hipError_t ttt_convert(bool to_f32, const void* src, void* dst, int64_t n, hipStream_t s) {
    const unsigned grid = grid_for((n + 7) / 8, kTttThreads);
    if (to_f32) hipLaunchKernelGGL((ttt_convert_kernel<BF16, F32>), dim3(grid), dim3(kTttThreads), 0, s, src, dst, n);
    else hipLaunchKernelGGL((ttt_convert_kernel<F32, BF16>), dim3(grid), dim3(kTttThreads), 0, s, src, dst, n);
    return hipGetLastError();
}

template <int VAR>
hipError_t launch_ttt_wide(const TttArgs& a, hipStream_t s) {
    const int64_t tok = static_cast<int64_t>(a.B) * a.T * a.H;
    const TttWide w = ttt_wide(a.B, a.T, a.H, a.dk, a.dv);
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    TttArgs f = a;
    f.q = ws + w.q;
    f.k = ws + w.k;
    f.v = ws + w.v;
    f.beta1 = ws + w.b1;
    f.beta2 = ws + w.b2;
    f.g1 = VAR == 1 ? ws + w.g1 : nullptr;
    f.g2 = VAR == 1 ? ws + w.g2 : nullptr;
    f.o = ws + w.o;
    f.ws = ws + w.rest;
    const void* from[] = {a.q, a.k, a.v, a.beta1, a.beta2, a.g1, a.g2};
    const void* to[] = {f.q, f.k, f.v, f.beta1, f.beta2, f.g1, f.g2};
    const int64_t n[] = {tok * a.dk, tok * a.dk, tok * a.dv, tok, tok, tok, tok};
    hipError_t e = hipSuccess;
    for (int i = 0; i < (VAR == 1 ? 7 : 5) && e == hipSuccess; ++i)
        e = ttt_convert(true, from[i], const_cast<void*>(to[i]), n[i], s);
    if (e == hipSuccess) e = launch_ttt_typed<F32, VAR>(f, s, true);
    if (e == hipSuccess) e = ttt_convert(false, f.o, a.o, tok * a.dv, s);
    return e;
}

}  // namespace

size_t ttt_workspace_bytes(int dtype, int B, int T, int H, int dk, int dv) {
    if (dtype == 0) return static_cast<size_t>(ttt_pieces(4, B, T, H, dk, dv).total);
    return static_cast<size_t>(ttt_wide(B, T, H, dk, dv).total);
}

hipError_t launch_ttt_pre(int variant, int dtype, const TttArgs& a, hipStream_t s) {
    if (dtype == 0) return variant == 0 ? launch_ttt_typed<F32, 0>(a, s) : launch_ttt_typed<F32, 1>(a, s);
    return variant == 0 ? launch_ttt_wide<0>(a, s) : launch_ttt_wide<1>(a, s);
}

}  // namespace dr
