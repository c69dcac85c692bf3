// Chunkwise-parallel forward of the gated delta rule on gfx950.
//
// The recurrence is affine in the previous memory (DeltaTTT summary,
// paperlayer.ai, §2 Background), so a chunk of C = 64 tokens acts on its
// incoming state S in closed form; the decay is absorbed into the keys and
// the chunk's erase steps are collected in a unit lower-triangular (WY/UT)
// factor (Gated DeltaNet-2 abstract, thelatestinai.com/papers/2607.07953:
// chunkwise WY algorithm with decay absorbed into the erase factors).
//
// Per chunk, with G_r the in-chunk cumulative log-decay, Q^ = Q ⊙ e^G,
// K^ = K ⊙ e^G, K- = K ⊙ e^(G_C - G) and (rows r, columns j)
//   A[r,j] = beta_r Σ_c k_rc k_jc e^(G_rc - G_jc)   (j < r)
//   P[r,j] =        Σ_c q_rc k_jc e^(G_rc - G_jc)   (j <= r)
//   T  = (I + A)^-1                                  unit lower triangular
//   V~ = T (beta ⊙ (V - K^ S^T))                     row j = beta_j (v_j - S'_j k_j)
//   O  = Q^ S^T + P V~                               readout after each write
//   S^T <- Diag(e^G_C) S^T + K-^T V~
//
// Work decomposition.  One workgroup of four 64-lane waves owns one
// (batch, head, 64-column value tile); each wave owns 16 value columns and
// keeps its 128 x 16 slice of S^T in fp32 MFMA accumulators for the whole
// sequence, so the state never leaves the chip between chunks.  The outputs
// of one MFMA feed the next one directly from registers: an accumulator tile
// holds rows 4*(lane/16)+i of column lane%16, which is exactly the operand
// layout of a contraction over those rows, once the other operand is read
// from LDS with the same row order.  Where that other operand is needed
// transposed (K^T for the state update, the value tile in accumulator
// layout) it is read with the gfx950 LDS transpose load, so no transposed
// copy is kept.  The key-side work of a chunk (K K^T, Q K^T, the triangular
// inverse) is shared by the four waves through LDS.  Value columns are
// independent (row i of S only ever mixes with v_i), so the value tiles of one
// head need no communication.
//
// The next chunk's q, k, v, beta and g are loaded into registers while the
// current chunk is computed; barriers wait for LDS traffic only.
//
// Numerics: MFMA operands are in the input dtype (bf16 x bf16 or fp32 x fp32
// products, fp32 accumulation); the state, the cumulative gates and the
// triangular inverse are fp32.
#include "chunk_ops.h"
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kC = 64;            // chunk length
constexpr int kWaves = 4;         // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kVT = 16 * kWaves;  // value columns per workgroup

// Lower-triangular 16x16 tiles (R, J), J <= R, of a 64x64 chunk matrix.
__device__ __forceinline__ void tri_tile(int idx, int& R, int& J) {
    // idx: 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3)
    R = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
    J = idx - (R * (R + 1)) / 2;
}

template <typename E, int DK>
struct Layout {
    typedef typename Ops<E>::S S;
    static constexpr int P = Ops<E>::kPad;
    static constexpr int LDQ = DK + P;   // q, k rows (chunk row major)
    static constexpr int LDV = kVT + P;  // value tile, output staging
    static constexpr int LDP = kC + P;   // P, T in operand dtype
    static constexpr int LDF = kC + 4;   // fp32 A and T
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + kC * LDQ * sizeof(S);
    static constexpr int oV = oK + kC * LDQ * sizeof(S);
    static constexpr int oP = oV + kC * LDV * sizeof(S);
    static constexpr int oTe = oP + kC * LDP * sizeof(S);
    static constexpr int oT = oTe + (sizeof(S) == 4 ? 0 : kC * LDP * sizeof(S));
    static constexpr int oA = oT + kC * LDF * 4;  // also the output staging buffer
    static constexpr int oVec = oA + kC * LDF * 4;
    // fp32 per-row vectors: beta, G, e^G, e^(G_C - G), and gamma = e^G_C
    static constexpr int bytes = oVec + (4 * kC + 4) * 4;
    static_assert(kC * LDV * sizeof(S) <= kC * LDF * 4, "output staging fits in A");
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int VAR, typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void prefill_kernel(FwdArgs p) {
    static_assert(VAR == 0 || VAR == 1, "channel-wise gates use their own kernel");
    typedef Ops<E> O_;
    typedef typename O_::S S;
    typedef typename O_::R R;
    typedef Layout<E, DK> L;
    constexpr bool kBF = sizeof(S) == 2;
    constexpr int NVT = DV / kVT;        // value tiles per head
    constexpr int NKT = DK / 16;         // key-channel tiles
    constexpr int EPC = 16 / sizeof(S);  // elements per 16-byte piece

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
    S* sQ = reinterpret_cast<S*>(smem + L::oQ);
    S* sK = reinterpret_cast<S*>(smem + L::oK);
    S* sV = reinterpret_cast<S*>(smem + L::oV);
    S* sP = reinterpret_cast<S*>(smem + L::oP);
    S* sTe = reinterpret_cast<S*>(smem + L::oTe);
    float* sT = reinterpret_cast<float*>(smem + L::oT);
    float* sA = reinterpret_cast<float*>(smem + L::oA);
    S* sO = reinterpret_cast<S*>(smem + L::oA);
    float* sBeta = reinterpret_cast<float*>(smem + L::oVec);
    float* sG = sBeta + kC;
    float* sEG = sG + kC;
    float* sEGC = sEG + kC;
    float* sGam = sEGC + kC;

    // Workgroup -> (head, value tile).  Workgroups are dispatched round-robin
    // over the 8 XCDs; the NVT tiles of one head get ids that are 8 apart, so
    // they run on the same XCD and share its L2 for q and k.
    const int x = blockIdx.x;
    const int vt = (x / 8) % NVT;
    const int bh = (x % 8) + 8 * (x / (8 * NVT));
    if (bh >= p.B * p.H) return;
    const int b = bh / p.H, h = bh % p.H;
    const int Hk = p.Hk, hk = h / (p.H / p.Hk);   // this value head's query/key head
    const int T = p.T, H = p.H;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int vc0 = vt * kVT + 16 * w;   // first value column of this wave

    // S^T slice: ST[t][i] = S[vc0 + c][16 t + 4 g + i].
    f32x4 ST[NKT];
    {
        const float* s0 = p.S0 ? p.S0 + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK : nullptr;
        // (the test outside the loop: a load under a branch inside it was waited
        // for before the next one was issued)
        if (s0) {
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                const float4 v4 = *reinterpret_cast<const float4*>(s0 + 16 * t + 4 * g);
                ST[t] = f32x4{v4.x, v4.y, v4.z, v4.w};
            }
        } else {
#pragma unroll
            for (int t = 0; t < NKT; ++t) ST[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // Global -> register prefetch of one chunk in coalesced 16-byte pieces
    // (piece p = tid + 256 j: row p / pieces-per-row).  Loads are unconditional
    // (rows past the end of the sequence re-read its last row) so no branch
    // forces an early wait; padding rows are zeroed when the registers are
    // committed to LDS at the top of the next chunk.
    constexpr int CPR = DK / EPC;                 // q/k pieces per row
    constexpr int VPR = kVT / EPC;                // value pieces per row
    constexpr int NPF = kC * CPR / kThreads;      // q/k pieces per thread
    constexpr int NPV = kC * VPR / kThreads;      // value pieces per thread
    static_assert(NPF * kThreads == kC * CPR && NPV * kThreads == kC * VPR, "piece split");
    typedef typename E::T Raw;
    uint4 pq[NPF], pk[NPF], pv[NPV];
    Raw pbeta = Raw(0), pg = Raw(0);
    const int nchunks = (T + kC - 1) / kC;
    auto prefetch = [&](int n) {
        const int t0 = n * kC;
        const int last = min(kC, T - t0) - 1;
        const int64_t tokb = static_cast<int64_t>(b) * T + t0;
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int pidx = tid + kThreads * j;
            const int64_t off = ((tokb + min(pidx / CPR, last)) * Hk + hk) * DK + (pidx % CPR) * EPC;
            pq[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.q) + off);
            pk[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.k) + off);
        }
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int pidx = tid + kThreads * j;
            const int64_t off = ((tokb + min(pidx / VPR, last)) * H + h) * DV + vt * kVT + (pidx % VPR) * EPC;
            pv[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.v) + off);
        }
        if (w == 0) {
            const int64_t tok = (tokb + min(lane, last)) * H + h;
            pbeta = static_cast<const Raw*>(p.beta)[tok];
            if constexpr (VAR == 1) pg = static_cast<const Raw*>(p.g)[tok];
        }
    };
    auto raw_to_f32 = [](Raw r) -> float {
        if constexpr (sizeof(Raw) == 4) return __builtin_bit_cast(float, r);
        else return bf16_bits_to_f32(r);
    };

    prefetch(0);
    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * kC;
        const int Cn = min(kC, T - t0);
        const int64_t tok0 = (static_cast<int64_t>(b) * T + t0) * H + h;  // token (b, t0, h)

        // ---- commit the prefetched chunk to LDS (rows past the end are zeroed)
        {
            const bool rowok = lane < Cn;
            auto sel = [](bool ok, uint4 v) {
                return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
            };
#pragma unroll
            for (int j = 0; j < NPF; ++j) {
                const int pidx = tid + kThreads * j;
                const int row = pidx / CPR, cc = pidx % CPR;
                *reinterpret_cast<uint4*>(sQ + row * L::LDQ + cc * EPC) = sel(row < Cn, pq[j]);
                *reinterpret_cast<uint4*>(sK + row * L::LDQ + cc * EPC) = sel(row < Cn, pk[j]);
            }
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                const int pidx = tid + kThreads * j;
                const int row = pidx / VPR, cc = pidx % VPR;
                *reinterpret_cast<uint4*>(sV + row * L::LDV + cc * EPC) = sel(row < Cn, pv[j]);
            }
            if (w == 0) {
                sBeta[lane] = rowok ? raw_to_f32(pbeta) : 0.f;
                float G = 0.f;
                if constexpr (VAR == 1) {
                    G = rowok ? raw_to_f32(pg) : 0.f;
#pragma unroll
                    for (int s = 1; s < 64; s <<= 1) {
                        const float y = __shfl_up(G, s, 64);
                        if (lane >= s) G += y;
                    }
                }
                const float GC = __shfl(G, 63, 64);
                sG[lane] = G;
                sEG[lane] = VAR == 0 ? 1.f : __expf(G);
                sEGC[lane] = VAR == 0 ? 1.f : __expf(GC - G);
                if (lane == 0) sGam[0] = VAR == 0 ? 1.f : __expf(GC);
            }
        }
        lds_barrier();
        if (n + 1 < nchunks) prefetch(n + 1);

        // ---- A = beta ⊙ (K K^T ⊙ Gamma), strictly lower, fp32
        for (int idx = w; idx < 10; idx += kWaves) {
            int R, J;
            tri_tile(idx, R, J);
            const int col = 16 * J + c;
            float brow[4], grow[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                brow[i] = sBeta[16 * R + 4 * g + i];
                grow[i] = sG[16 * R + 4 * g + i];
            }
            const float gcol = sG[col];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = O_::template nat<DK>(acc, sK + (16 * R + c) * L::LDQ, sK + (16 * J + c) * L::LDQ, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * R + 4 * g + i;
                float val = acc[i] * brow[i];
                if constexpr (VAR == 1) val *= __expf(grow[i] - gcol);
                sA[row * L::LDF + col] = row > col ? val : 0.f;
            }
        }
        lds_barrier();

        // ---- wave 0: diagonal 16x16 blocks of T; waves 1..3: P = Q K^T ⊙ Gamma
        if (w == 0) {
            // Lane (block rb, column j) solves (I + A_bb) x = e_j by columns:
            // once x[m] is final, every later row i subtracts A[i][m] x[m].
            const int rb = 16 * (lane >> 4);
            const int j = lane & 15;
            float a[16][16];
#pragma unroll
            for (int i = 1; i < 16; ++i) {
#pragma unroll
                for (int m4 = 0; m4 < i; m4 += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(sA + (rb + i) * L::LDF + rb + m4);
                    a[i][m4] = v.x;
                    a[i][m4 + 1] = v.y;
                    a[i][m4 + 2] = v.z;
                    a[i][m4 + 3] = v.w;
                }
            }
            float xs[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) xs[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
#pragma unroll
                for (int i = m + 1; i < 16; ++i) xs[i] -= a[i][m] * xs[m];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sT[(rb + i) * L::LDF + rb + j] = xs[i];
                if constexpr (kBF) sTe[(rb + i) * L::LDP + rb + j] = O_::enc(xs[i]);
            }
        } else {
            for (int idx = w - 1; idx < 10; idx += kWaves - 1) {
                int R, J;
                tri_tile(idx, R, J);
                const int col = 16 * J + c;
                float grow[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) grow[i] = sG[16 * R + 4 * g + i];
                const float gcol = sG[col];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = O_::template nat<DK>(acc, sQ + (16 * R + c) * L::LDQ, sK + (16 * J + c) * L::LDQ, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * R + 4 * g + i;
                    float val = acc[i];
                    if constexpr (VAR == 1) val *= __expf(grow[i] - gcol);
                    sP[row * L::LDP + col] = O_::enc(row >= col ? val : 0.f);
                }
            }
        }
        lds_barrier();

        // ---- off-diagonal blocks of T: T_RJ = -T_RR · Σ_{M=J}^{R-1} A_RM T_MJ,
        //      by distance R - J = 1, 2, 3 (fp32 MFMA)
#pragma unroll
        for (int dist = 1; dist <= 3; ++dist) {
            if (w < 4 - dist) {
                const int J = w, R = w + dist;
                float av[3][4], tv[3][4], dv[4];
#pragma unroll
                for (int mm = 0; mm < dist; ++mm) {
                    const int M = J + mm;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        av[mm][ks] = sA[(16 * R + c) * L::LDF + 16 * M + 4 * ks + g];
                        tv[mm][ks] = sT[(16 * M + 4 * ks + g) * L::LDF + 16 * J + c];
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) dv[i] = sT[(16 * R + c) * L::LDF + 16 * R + 4 * g + i];
                f32x4 inner = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mm = 0; mm < dist; ++mm) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) inner = mfma4(av[mm][ks], tv[mm][ks], inner);
                }
                f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) out = mfma4(dv[i], inner[i], out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * R + 4 * g + i, col = 16 * J + c;
                    sT[row * L::LDF + col] = -out[i];
                    if constexpr (kBF) sTe[row * L::LDP + col] = O_::enc(-out[i]);
                }
            }
            lds_barrier();
        }

        // ---- the state-dependent chain, per wave (16 value columns)
        {
            const S* Te = kBF ? sTe : reinterpret_cast<const S*>(sT);
            constexpr int LDTe = kBF ? L::LDP : L::LDF;
            float eg[4][4], egc[4][4], bt[4][4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * m + 4 * g + i;
                    eg[m][i] = sEG[row];
                    egc[m][i] = sEGC[row];
                    bt[m][i] = sBeta[row];
                }
            }
            const float gam = sGam[0];
            R STr[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) STr[t] = O_::to_reg(ST[t]);
            f32x4 X[4], Y[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                X[m] = O_::template reg<0, NKT>(f32x4{0.f, 0.f, 0.f, 0.f}, sK + (16 * m + c) * L::LDQ, STr, g);
                Y[m] = O_::template reg<0, NKT>(f32x4{0.f, 0.f, 0.f, 0.f}, sQ + (16 * m + c) * L::LDQ, STr, g);
            }
            // R = beta ⊙ (V - e^G ⊙ K S^T)
            R Rr[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 v = O_::acc_tile(sV, L::LDV, 16 * m, 16 * w, g, c);
                f32x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = bt[m][i] * (v[i] - eg[m][i] * X[m][i]);
                Rr[m] = O_::to_reg(r);
            }
            // V~ = T R  (T lower triangular: tile m needs tiles 0..m)
            f32x4 Vt[4];
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            Vt[0] = O_::template reg<0, 1>(zero, Te + (0 + c) * LDTe, Rr, g);
            Vt[1] = O_::template reg<0, 2>(zero, Te + (16 + c) * LDTe, Rr, g);
            Vt[2] = O_::template reg<0, 3>(zero, Te + (32 + c) * LDTe, Rr, g);
            Vt[3] = O_::template reg<0, 4>(zero, Te + (48 + c) * LDTe, Rr, g);
            R Vtr[4], Vgr[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                Vtr[m] = O_::to_reg(Vt[m]);
                f32x4 vg;
#pragma unroll
                for (int i = 0; i < 4; ++i) vg[i] = egc[m][i] * Vt[m][i];
                Vgr[m] = O_::to_reg(vg);
            }
            // S^T <- e^G_C S^T + K^T (e^(G_C - G) ⊙ V~)
#pragma unroll
            for (int t = 0; t < NKT; ++t)
                ST[t] = O_::template regT<4>(ST[t] * gam, sK, L::LDQ, 16 * t, Vgr, g, c);
            // O = e^G ⊙ Q S^T + P V~
            f32x4 Ot[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i) Ot[m][i] = eg[m][i] * Y[m][i];
            }
            Ot[0] = O_::template reg<0, 1>(Ot[0], sP + (0 + c) * L::LDP, Vtr, g);
            Ot[1] = O_::template reg<0, 2>(Ot[1], sP + (16 + c) * L::LDP, Vtr, g);
            Ot[2] = O_::template reg<0, 3>(Ot[2], sP + (32 + c) * L::LDP, Vtr, g);
            Ot[3] = O_::template reg<0, 4>(Ot[3], sP + (48 + c) * L::LDP, Vtr, g);
            // sO aliases sA: the last reads of sA were before the final level barrier.
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sO[(16 * m + 4 * g + i) * L::LDV + 16 * w + c] = O_::enc(Ot[m][i]);
            }
        }
        lds_barrier();
        // ---- coalesced store of the chunk's outputs (this tile's kVT columns)
        {
            for (int idx = tid; idx < kC * VPR; idx += kThreads) {
                const int row = idx / VPR, cc = idx % VPR;
                if (row < Cn) {
                    const int64_t off = (tok0 + static_cast<int64_t>(row) * H) * DV + vt * kVT + cc * EPC;
                    *reinterpret_cast<uint4*>(static_cast<S*>(p.o) + off) =
                        *reinterpret_cast<const uint4*>(sO + row * L::LDV + cc * EPC);
                }
            }
        }
        // No barrier needed here: the next chunk writes the sA/sO region only
        // after its commit barrier, and everything else the chain read was
        // consumed before the barrier above.
    }

    if (p.ST) {
        float* st = p.ST + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            *reinterpret_cast<float4*>(st + 16 * t + 4 * g) = make_float4(ST[t][0], ST[t][1], ST[t][2], ST[t][3]);
    }
}

template <int VAR, typename E, int DK, int DV>
hipError_t launch_one(const FwdArgs& a, hipStream_t s) {
    constexpr int NVT = DV / kVT;
    const int bh = a.B * a.H;
    const int groups = (bh + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups) * 8u * NVT);
    hipLaunchKernelGGL((prefill_kernel<VAR, E, DK, DV>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int VAR, typename E>
hipError_t launch_dims(const FwdArgs& a, hipStream_t s) {
    if (a.dk == 128 && a.dv == 128) return launch_one<VAR, E, 128, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_one<VAR, E, 128, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_one<VAR, E, 64, 128>(a, s);
    return launch_one<VAR, E, 64, 64>(a, s);
}

}  // namespace

hipError_t launch_fwd_split(int variant, const FwdArgs& a, hipStream_t s) {
    return variant == 0 ? launch_dims<0, F32S>(a, s) : launch_dims<1, F32S>(a, s);
}

hipError_t launch_fwd(int variant, int dtype, const FwdArgs& a, hipStream_t s) {
    if (variant >= 2) return launch_fwd_channel(variant, dtype, a, s);
    if (dtype == 1) return launch_fwd_pipelined(variant, a, s);   // bf16: pipelined kernel
    return variant == 0 ? launch_dims<0, F32>(a, s) : launch_dims<1, F32>(a, s);   // fp32
}

}  // namespace dr
