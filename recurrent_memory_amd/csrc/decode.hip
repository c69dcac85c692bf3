// Single-token decode update of the gated delta rule, state updated in place.
//
// Decode moves the whole fp32 state through HBM once in each direction per
// token and does < 1 flop per byte ("Delta-Rule Linear Attention" topic page,
// GDN FPGA decode card), so the kernel is organised around streaming the
// state: one workgroup per (batch, head) state matrix, 256 threads in eight
// 32-lane groups, each group owning every eighth value row.  A lane holds
// d_k/32 consecutive key columns of each of its rows, so every row is one
// coalesced 512-byte (d_k = 128) read and write.  The small per-token
// operands are requested first, then every state row; the rows are finished
// in four batches, so the writes of a batch overlap the reads still arriving
// for the next ones.
//
// Per row i (value channel) with a = exp(g) and S' = S·Diag(a):
//   r_i  = S'_i · k          (read)        s_i = S'_i · q
//   single step size:  u_i = beta (v_i - r_i);  S_i = S'_i + u_i k
//                      o_i = s_i + u_i (k·q)
//   split gates:       x_i = w_i v_i;  S_i = S'_i - r_i (b ⊙ k) + x_i k
//                      o_i = s_i - r_i ((b ⊙ k)·q) + x_i (k·q)
//   step size per key channel (FG^2-GDN):
//                      u_i = v_i - r_i;  S_i = S'_i + u_i (beta ⊙ k)
//                      o_i = s_i + u_i ((beta ⊙ k)·q)
// which is o = S q read after the write, without a second pass over S.
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kDecodeThreads = 256;

template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeArgs p) {
    constexpr int CPL = DK / 32;       // key columns per lane
    constexpr int RPG = DV / 8;        // rows per 32-lane group
    static_assert(RPG == 8 || RPG == 16, "row layout");
    const int bh = blockIdx.x;         // b * H + h
    const int grp = threadIdx.x >> 5;  // 0..7
    const int li = threadIdx.x & 31;
    const int64_t tok = bh;            // token index in [B, H] layouts
    // its query/key row in [B, Hk]: value heads share a query/key head in groups
    const int64_t qtok = static_cast<int64_t>(bh / p.H) * p.Hk + (bh % p.H) / (p.H / p.Hk);
    const int c0 = li * CPL;

    float* S = p.S + static_cast<int64_t>(bh) * DV * DK;

    // The small per-token operands first, then every state row: the rows
    // arrive in issue order, so the first batch below waits only for its own.
    float kk[CPL], qq[CPL], aa[CPL], bk[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        kk[c] = load_elem<E>(p.k, qtok * DK + c0 + c);
        qq[c] = load_elem<E>(p.q, qtok * DK + c0 + c);
        if constexpr (VAR == 0) {
            aa[c] = 0.0f;
        } else if constexpr (VAR == 1) {
            aa[c] = load_elem<E>(p.g, tok);
        } else {
            aa[c] = fmaxf(load_elem<E>(p.g, tok * DK + c0 + c), kLogDecayFloor);
        }
        if constexpr (VAR >= 3) bk[c] = load_elem<E>(p.beta, tok * DK + c0 + c);
        else bk[c] = 0.0f;
    }
    float beta_s = 0.f;
    if constexpr (VAR < 3) beta_s = load_elem<E>(p.beta, tok);
    float st[RPG][CPL];
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
        const float* row = S + static_cast<int64_t>(grp + 8 * j) * DK + c0;
        if constexpr (CPL == 4) {
            float4 x = *reinterpret_cast<const float4*>(row);
            st[j][0] = x.x; st[j][1] = x.y; st[j][2] = x.z; st[j][3] = x.w;
        } else {
            float2 x = *reinterpret_cast<const float2*>(row);
            st[j][0] = x.x; st[j][1] = x.y;
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        aa[c] = VAR == 0 ? 1.0f : __expf(aa[c]);
        if constexpr (VAR >= 3) bk[c] *= kk[c];
    }
    float kq = 0.f, bkq = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        kq += kk[c] * qq[c];
        bkq += bk[c] * qq[c];
    }
    kq = half_wave_sum(kq);
    if constexpr (VAR >= 3) bkq = half_wave_sum(bkq);

    // Rows in four batches: a batch is reduced, updated and written back while
    // the loads of the later batches are still arriving.
    constexpr int NBATCH = RPG >= 4 ? 4 : RPG;
    constexpr int RB = RPG / NBATCH;   // rows per batch
    constexpr int NV = 2 * RB;         // partial dot products per lane and batch
#pragma unroll
    for (int bt = 0; bt < NBATCH; ++bt) {
        float val[NV];
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
            const int j = bt * RB + jj;
            float r = 0.f, s = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                st[j][c] *= aa[c];
                r += st[j][c] * kk[c];
                s += st[j][c] * qq[c];
            }
            val[jj] = r;
            val[RB + jj] = s;
        }
        // Transpose-reduce across the 32 lanes: each step halves the number of
        // values a lane carries; at the end lane li holds the full sum of value
        // index (li >> (5 - log2 NV)).
        int n = NV;
#pragma unroll
        for (int sh = 16; sh >= 1; sh >>= 1) {
            if (n > 1) {
                const bool upper = (li & sh) != 0;
#pragma unroll
                for (int i = 0; i < n / 2; ++i) {
                    float keep = upper ? val[n / 2 + i] : val[i];
                    float send = upper ? val[i] : val[n / 2 + i];
                    val[i] = keep + __shfl_xor(send, sh, 32);
                }
                n >>= 1;
            } else {
                val[0] += __shfl_xor(val[0], sh, 32);
            }
        }
        constexpr int kShift = NV == 32 ? 0 : NV == 16 ? 1 : NV == 8 ? 2 : NV == 4 ? 3 : 4;  // log2(32 / NV)
        const int idx = li >> kShift;               // value index this lane holds
        // r of row idx sits at value idx, s of row idx at value RB + idx.
        const float other = __shfl_xor(val[0], RB << kShift, 32);
        const bool owner = idx < RB && (li & ((1 << kShift) - 1)) == 0;
        const int orow = grp + 8 * (bt * RB + idx);  // value row this lane finishes
        float coef_u = 0.f, coef_x = 0.f;
        if (idx < RB) {
            const float r = val[0], s = other;
            const float vi = load_elem<E>(p.v, tok * DV + orow);
            float o;
            if constexpr (VAR == 3) {
                const float x = load_elem<E>(p.wgate, tok * DV + orow) * vi;
                coef_u = r;
                coef_x = x;
                o = s - r * bkq + x * kq;
            } else if constexpr (VAR == 4) {
                const float u = vi - r;
                coef_u = u;
                o = s + u * bkq;
            } else {
                const float u = beta_s * (vi - r);
                coef_u = u;
                o = s + u * kq;
            }
            if (owner) store_elem<E>(p.o, tok * DV + orow, o);
        }
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
            const int j = bt * RB + jj;
            const int src = jj << kShift;
            const float u = __shfl(coef_u, src, 32);
            float x = 0.f;
            if constexpr (VAR == 3) x = __shfl(coef_x, src, 32);
            float* row = S + static_cast<int64_t>(grp + 8 * j) * DK + c0;
            float out[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if constexpr (VAR == 3) out[c] = st[j][c] - u * bk[c] + x * kk[c];
                else if constexpr (VAR == 4) out[c] = st[j][c] + u * bk[c];
                else out[c] = st[j][c] + u * kk[c];
            }
            if constexpr (CPL == 4) {
                *reinterpret_cast<float4*>(row) = make_float4(out[0], out[1], out[2], out[3]);
            } else {
                *reinterpret_cast<float2*>(row) = make_float2(out[0], out[1]);
            }
        }
    }
}

template <int VAR, typename E>
hipError_t launch_decode_dims(const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H));
    const dim3 block(kDecodeThreads);
    if (a.dk == 128 && a.dv == 128) hipLaunchKernelGGL((decode_kernel<VAR, E, 128, 128>), grid, block, 0, s, a);
    else if (a.dk == 128 && a.dv == 64) hipLaunchKernelGGL((decode_kernel<VAR, E, 128, 64>), grid, block, 0, s, a);
    else if (a.dk == 64 && a.dv == 128) hipLaunchKernelGGL((decode_kernel<VAR, E, 64, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<VAR, E, 64, 64>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int VAR>
hipError_t launch_decode_dtype(int dtype, const DecodeArgs& a, hipStream_t s) {
    return dtype == 0 ? launch_decode_dims<VAR, F32>(a, s) : launch_decode_dims<VAR, BF16>(a, s);
}

}  // namespace

hipError_t launch_decode(int variant, int dtype, const DecodeArgs& a, hipStream_t s) {
    switch (variant) {
        case 0: return launch_decode_dtype<0>(dtype, a, s);
        case 1: return launch_decode_dtype<1>(dtype, a, s);
        case 2: return launch_decode_dtype<2>(dtype, a, s);
        case 3: return launch_decode_dtype<3>(dtype, a, s);
        default: return launch_decode_dtype<4>(dtype, a, s);
    }
}

}  // namespace dr
