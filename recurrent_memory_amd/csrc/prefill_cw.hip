// Chunkwise forward of the delta rule with channel-wise decay on gfx950:
// Kimi Delta Attention (one step size beta_t) and Gated DeltaNet-2 (a
// channel-wise erase gate b_t on the key side and a channel-wise write gate
// w_t on the value side, reducing to KDA when both equal beta_t; Gated
// DeltaNet-2 abstract, thelatestinai.com/papers/2607.07953, whose chunkwise WY
// algorithm absorbs the channel-wise decay into asymmetric erase factors).
//
// Decay per key channel cannot be pulled out of the C x C products as a
// row/column scale, so the keys carry it, split into two factors.  Every
// factor here has the form e^(G_later - G_earlier) <= 1, taken relative to the
// boundaries of 16-token blocks, so no factor over- or underflows unless the
// true quantity is itself negligible:
//   G_r     cumulative log-decay inside the sub-chunk (per channel)
//   b(R)    last row before block R (G = 0 before the sub-chunk)
//   Kh_r  = k_r ⊙ e^(G_r - G_b(R))       queries likewise (Qh)
//   Ki_j  = k_j ⊙ e^(G_b(R) - G_j)       (diagonal blocks only; >= 1, bounded
//                                         by the decay inside one block)
//   Ke_j  = k_j ⊙ e^(G_end(J) - G_j)     (end of j's own block)
//   Kb_j  = k_j ⊙ e^(G_C - G_j)          (state update)
// so that k_r · e^(G_r - G_j) k_j = Kh_r · Ki_j inside a block and Kh_r · Ke_j
// across adjacent blocks (the two references coincide).  The state enters
// each block decayed to the block start, S ⊙ e^(G_b(R)), so the read K^ S^T
// never multiplies a small key by a large factor.
//
// One step size (KDA), per sub-chunk of C tokens:
//   A = StrictTril(diag(beta) Kh Kx^T), T = (I + A)^-1, P = Tril(Qh Kx^T)
//   V~ = T (beta ⊙ (V - X)),  X_R = Kh_R (S ⊙ e^G_b(R))^T
//   O  = Y + P V~,            Y_R = Qh_R (S ⊙ e^G_b(R))^T
//   S^T <- Diag(e^G_C) S^T + Kb^T V~
// Split gates (Gated DeltaNet-2), E = b ⊙ K, W = w ⊙ V:
//   A_e = StrictTril(Kh Ex^T), A_k = StrictTril(Kh Kx^T), T = (I + A_e)^-1
//   Z = X + A_k W,  Y~ = T Z           (row j = S'_j k_j, the erase read)
//   O = Y + M_k W - M_e Y~,  M_k = Tril(Qh Kx^T), M_e = Tril(Qh Ex^T)
//   S^T <- Diag(e^G_C) S^T + Kb^T W - Eb^T Y~
// (Kx, Ex: Ki/Ei on diagonal blocks, Ke/Ee below them.)
// A step size per key channel (FG^2-GDN: the residual is written along
// E = beta ⊙ K, "Delta-Rule Linear Attention" topic page, FG^2-GDN card) is the
// split form with the write along E and no write gate: W = V, and A_k, M_k
// and Kb are replaced by A_e, M_e and Eb (FwdArgs::keywrite).
//
// With bf16 operands the decay-scaled queries are kept as a hi + lo pair of
// bf16 values (two MFMAs per query-side product): a single rounding of
// q ⊙ e^(G - G_b) would make nearly orthogonal q·k products lose most of
// their relative precision.
//
// The sub-chunk is 32 tokens for bf16 inputs (two 16-token blocks) and 16
// for fp32 inputs; the result does not depend on the sub-chunk length in exact
// arithmetic.  Work decomposition, operand layouts and the register-tile
// contractions are those of the scalar-decay kernels: one workgroup of four
// waves per (batch, head, 16 value columns); the four waves share the
// key-side work and wave 0 keeps the 128 x 16 slice of the fp32 state in MFMA
// accumulators for the whole sequence.
#include "chunk_ops.h"
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kWavesCW = 4;
constexpr int kThreadsCW = 64 * kWavesCW;
// Value columns per workgroup: one 16-column tile, whose state wave 0 carries.
// The four waves share the key-side work of every sub-chunk; a narrow value
// tile gives B * H * d_v / 16 workgroups, enough to fill the chip for the
// head counts of the channel-wise workloads.
constexpr int kVTCW = 16;

template <typename E, int DK, int NB, bool SPLIT>
struct LayoutCW {
    typedef typename Ops<E>::S S;
    static constexpr int C = 16 * NB;
    static constexpr int P = Ops<E>::kPad;
    static constexpr int LDK = DK + P;     // [C][DK] operand matrices
    static constexpr int LDV = kVTCW + P;  // value (or w ⊙ v) tile, output staging
    static constexpr int LDM = C + P;      // C x C in operand dtype
    static constexpr int LDF = C + 4;      // C x C fp32
    static constexpr int KM = C * LDK * sizeof(S);
    static constexpr int KE = (NB - 1) * 16 * LDK * sizeof(S);
    static constexpr int MM = C * LDM * sizeof(S);
    static constexpr int MF = C * LDF * 4;
    static constexpr int oKh = 0;
    static constexpr int oQh = oKh + KM;
    static constexpr int oQl = oQh + KM;                  // low half of Qh (bf16 operands)
    static constexpr int oKi = oQl + (sizeof(S) == 2 ? KM : 0);
    static constexpr int oKb = oKi + KM;
    static constexpr int oKe = oKb + KM;
    static constexpr int oEi = oKe + KE;
    static constexpr int oEb = oEi + (SPLIT ? KM : 0);
    static constexpr int oEe = oEb + (SPLIT ? KM : 0);
    static constexpr int oRawG = oEe + (SPLIT ? KE : 0);  // raw g; later the output staging
    static constexpr int oRawB = oRawG + KM;              // raw erase gate (split gates)
    static constexpr int oV = oRawB + (SPLIT ? KM : 0);
    static constexpr int oA = oV + C * LDV * sizeof(S);   // A or A_e (fp32)
    static constexpr int oT = oA + MF;                    // T (fp32)
    static constexpr int oTe = oT + MF;                   // T (operand dtype)
    static constexpr int oP = oTe + MM;                   // P or M_k
    static constexpr int oAk = oP + MM;                   // A_k (split gates)
    static constexpr int oMe = oAk + (SPLIT ? MM : 0);    // M_e (split gates)
    static constexpr int oVec = oMe + (SPLIT ? MM : 0);
    // fp32 vectors: beta[C], e^G_b(R)[NB][DK], e^G_C[DK]
    static constexpr int bytes = oVec + (C + (NB + 1) * DK) * 4;
    static_assert(C * LDV * sizeof(S) <= KM, "output staging fits in the raw-gate buffer");
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int VAR, typename E, int DK, int DV, int NB>
__global__ __launch_bounds__(kThreadsCW) void prefill_cw_kernel(FwdArgs p) {
    constexpr bool SPLIT = VAR == 3;
    static_assert(VAR == 2 || VAR == 3, "channel-wise decay forms");
    typedef Ops<E> O_;
    typedef typename O_::S S;
    typedef typename O_::R R;
    typedef LayoutCW<E, DK, NB, SPLIT> L;
    constexpr bool kBF = sizeof(S) == 2;
    constexpr int C = L::C;
    constexpr int NVT = DV / kVTCW;
    constexpr int NKT = DK / 16;
    constexpr int EPC = 16 / sizeof(S);

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
    S* sKh = reinterpret_cast<S*>(smem + L::oKh);
    S* sQh = reinterpret_cast<S*>(smem + L::oQh);
    S* sQl = reinterpret_cast<S*>(smem + L::oQl);
    S* sKi = reinterpret_cast<S*>(smem + L::oKi);
    S* sKb = reinterpret_cast<S*>(smem + L::oKb);
    S* sKe = reinterpret_cast<S*>(smem + L::oKe);
    S* sEi = reinterpret_cast<S*>(smem + L::oEi);
    S* sEb = reinterpret_cast<S*>(smem + L::oEb);
    S* sEe = reinterpret_cast<S*>(smem + L::oEe);
    S* sRawG = reinterpret_cast<S*>(smem + L::oRawG);
    S* sRawB = reinterpret_cast<S*>(smem + L::oRawB);
    S* sO = reinterpret_cast<S*>(smem + L::oRawG);
    S* sV = reinterpret_cast<S*>(smem + L::oV);
    float* sA = reinterpret_cast<float*>(smem + L::oA);
    float* sT = reinterpret_cast<float*>(smem + L::oT);
    S* sTe = reinterpret_cast<S*>(smem + L::oTe);
    S* sP = reinterpret_cast<S*>(smem + L::oP);
    S* sAk = reinterpret_cast<S*>(smem + L::oAk);
    S* sMe = reinterpret_cast<S*>(smem + L::oMe);
    float* sBeta = reinterpret_cast<float*>(smem + L::oVec);
    float* sEgb = sBeta + C;          // [NB][DK]
    float* sGam = sEgb + NB * DK;     // [DK]

    const int x = blockIdx.x;
    const int vt = (x / 8) % NVT;
    const int bh = (x % 8) + 8 * (x / (8 * NVT));
    if (bh >= p.B * p.H) return;
    const int b = bh / p.H, h = bh % p.H;
    const int T = p.T, H = p.H;
    const int Hk = p.Hk, hk = h / (p.H / p.Hk);   // this value head's query/key head
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int vc0 = vt * kVTCW;
    const bool chain = (w == 0);   // the wave that carries the state

    f32x4 ST[NKT];
    {
        const float* s0 = (p.S0 && chain) ? p.S0 + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK : nullptr;
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

    // Register prefetch of one sub-chunk (coalesced 16-byte pieces; rows past
    // the end re-read the last row and are zeroed at commit).
    constexpr int CPR = DK / EPC;                        // pieces per q/k/g/b row
    constexpr int NPK = (C * CPR + kThreadsCW - 1) / kThreadsCW;
    constexpr int VPR = kVTCW / EPC;                     // pieces per value row
    constexpr int NPV = (C * VPR + kThreadsCW - 1) / kThreadsCW;
    typedef typename E::T Raw;
    uint4 pq[NPK], pk[NPK], pg[NPK], pb[NPK], pv[NPV], pw[NPV];
    Raw pbeta = Raw(0);
    const int nchunks = (T + C - 1) / C;
    // per-thread element offsets relative to the first token of a sub-chunk
    // (32-bit, computed once); only the last, partial sub-chunk clamps rows
    uint32_t koff[NPK], qkoff[NPK], voff[NPV];
#pragma unroll
    for (int j = 0; j < NPK; ++j) {
        const int pidx = tid + kThreadsCW * j;
        const int row = min(pidx / CPR, C - 1), cc = pidx % CPR;
        koff[j] = static_cast<uint32_t>(row * H * DK + cc * EPC);
        qkoff[j] = static_cast<uint32_t>(row * Hk * DK + cc * EPC);
    }
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
        const int pidx = tid + kThreadsCW * j;
        const int row = min(pidx / VPR, C - 1), cc = pidx % VPR;
        voff[j] = static_cast<uint32_t>(row * H * DV + cc * EPC);
    }
    auto prefetch = [&](int n) {
        const int t0 = n * C;
        const int last = min(C, T - t0) - 1;
        const int64_t tokb = static_cast<int64_t>(b) * T + t0;
        if (last == C - 1) {   // whole sub-chunk: uniform base + thread offset
            const int64_t kb = (tokb * H + h) * DK, vb = (tokb * H + h) * DV + vt * kVTCW;
            const int64_t qb = (tokb * Hk + hk) * DK;
#pragma unroll
            for (int j = 0; j < NPK; ++j) {
                pq[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.q) + qb + qkoff[j]);
                pk[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.k) + qb + qkoff[j]);
                pg[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.g) + kb + koff[j]);
                if constexpr (SPLIT) pb[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.beta) + kb + koff[j]);
            }
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                pv[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.v) + vb + voff[j]);
                if (SPLIT && !p.keywrite) pw[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.wgate) + vb + voff[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NPK; ++j) {
                const int pidx = tid + kThreadsCW * j;
                const int row = min(min(pidx / CPR, C - 1), last), cc = pidx % CPR;
                const int64_t off = ((tokb + row) * H + h) * DK + cc * EPC;
                const int64_t qoff = ((tokb + row) * Hk + hk) * DK + cc * EPC;
                pq[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.q) + qoff);
                pk[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.k) + qoff);
                pg[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.g) + off);
                if constexpr (SPLIT) pb[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.beta) + off);
            }
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                const int pidx = tid + kThreadsCW * j;
                const int row = min(min(pidx / VPR, C - 1), last), cc = pidx % VPR;
                const int64_t off = ((tokb + row) * H + h) * DV + vt * kVTCW + cc * EPC;
                pv[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.v) + off);
                if (SPLIT && !p.keywrite) pw[j] = *reinterpret_cast<const uint4*>(static_cast<const S*>(p.wgate) + off);
            }
        }
        if constexpr (!SPLIT) {
            if (tid < C) pbeta = static_cast<const Raw*>(p.beta)[(tokb + min(tid, last)) * H + h];
        }
    };
    auto raw_to_f32 = [](Raw r) -> float {
        if constexpr (sizeof(Raw) == 4) return __builtin_bit_cast(float, r);
        else return bf16_bits_to_f32(r);
    };

    prefetch(0);
    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int Cn = min(C, T - t0);
        const int64_t tokb = static_cast<int64_t>(b) * T + t0;

        // ---- commit: raw q -> sQh, raw k -> sKh, raw g (and b), value tile
        {
            auto sel = [](bool ok, uint4 v) {
                return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
            };
#pragma unroll
            for (int j = 0; j < NPK; ++j) {
                const int pidx = tid + kThreadsCW * j;
                if (pidx < C * CPR) {
                    const int row = pidx / CPR, cc = pidx % CPR;
                    const bool ok = row < Cn;
                    *reinterpret_cast<uint4*>(sQh + row * L::LDK + cc * EPC) = sel(ok, pq[j]);
                    *reinterpret_cast<uint4*>(sKh + row * L::LDK + cc * EPC) = sel(ok, pk[j]);
                    *reinterpret_cast<uint4*>(sRawG + row * L::LDK + cc * EPC) = sel(ok, pg[j]);
                    if constexpr (SPLIT)
                        *reinterpret_cast<uint4*>(sRawB + row * L::LDK + cc * EPC) = sel(ok, pb[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                const int pidx = tid + kThreadsCW * j;
                if (pidx < C * VPR) {
                    const int row = pidx / VPR, cc = pidx % VPR;
                    uint4 v = sel(row < Cn, pv[j]);
                    if (SPLIT && !p.keywrite) {
                        // W = w ⊙ v, rounded once to the operand dtype
                        const S* ve = reinterpret_cast<const S*>(&v);
                        const uint4 wv = pw[j];
                        const S* we = reinterpret_cast<const S*>(&wv);
                        S prod[EPC];
#pragma unroll
                        for (int e = 0; e < EPC; ++e) {
                            float a, bb;
                            if constexpr (kBF) {
                                a = bf16_bits_to_f32(ve[e]);
                                bb = bf16_bits_to_f32(we[e]);
                            } else {
                                a = ve[e];
                                bb = we[e];
                            }
                            prod[e] = O_::enc(a * bb);
                        }
                        v = *reinterpret_cast<const uint4*>(prod);
                    }
                    *reinterpret_cast<uint4*>(sV + row * L::LDV + cc * EPC) = v;
                }
            }
            if constexpr (!SPLIT) {
                if (tid < C) sBeta[tid] = tid < Cn ? raw_to_f32(pbeta) : 0.f;
            }
        }
        lds_barrier();
        if (n + 1 < nchunks) prefetch(n + 1);

        // ---- per channel: cumulative decay and the decay-carrying key copies.
        // Thread (channel pair cp, row group rq): channels 2 cp, 2 cp + 1 and
        // RPT consecutive rows; the NRQ row groups of a channel pair are
        // adjacent lanes, which exchange their partial decay sums by shuffles.
        {
            constexpr int NRQ = 2 * kThreadsCW / DK;   // row groups per channel pair
            constexpr int RPT = C / NRQ;               // rows per thread
            static_assert(RPT >= 1 && C % NRQ == 0 && 16 % RPT == 0, "row split");
            const int rq = tid % NRQ, cp = tid / NRQ;
            const int ch = 2 * cp, r0 = rq * RPT;
            auto ld2 = [&](const S* m, int r) -> float2 {
                const S* q = m + r * L::LDK + ch;
                if constexpr (kBF) {
                    const uint32_t u = *reinterpret_cast<const uint32_t*>(q);
                    return make_float2(bf16_bits_to_f32(static_cast<uint16_t>(u & 0xffffu)),
                                       bf16_bits_to_f32(static_cast<uint16_t>(u >> 16)));
                } else {
                    return *reinterpret_cast<const float2*>(q);
                }
            };
            auto st2 = [&](S* m, int r, float x0, float x1) {
                S* q = m + r * L::LDK + ch;
                if constexpr (kBF) {
                    *reinterpret_cast<uint32_t*>(q) = static_cast<uint32_t>(O_::enc(x0)) |
                                                      (static_cast<uint32_t>(O_::enc(x1)) << 16);
                } else {
                    *reinterpret_cast<float2*>(q) = make_float2(x0, x1);
                }
            };
            // raw log-decays of this thread's rows and their sum
            float g0[RPT], g1[RPT];
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const float2 v = ld2(sRawG, r0 + j);
                g0[j] = fmaxf(v.x, kLogDecayFloor);
                g1[j] = fmaxf(v.y, kLogDecayFloor);
                p0 += g0[j];
                p1 += g1[j];
            }
            // exclusive prefix over the row groups, and the block-start and
            // chunk-end values (G is the running sum of the raw log-decays)
            float e0 = 0.f, e1 = 0.f, tot0 = 0.f, tot1 = 0.f, bs0 = 0.f, bs1 = 0.f;
            const int my_block = r0 / 16;
#pragma unroll
            for (int q = 0; q < NRQ; ++q) {
                const float s0 = __shfl(p0, (lane & ~(NRQ - 1)) + q, 64);
                const float s1 = __shfl(p1, (lane & ~(NRQ - 1)) + q, 64);
                if (q < rq) { e0 += s0; e1 += s1; }
                if (q * RPT < 16 * my_block) { bs0 += s0; bs1 += s1; }
                tot0 += s0;
                tot1 += s1;
            }
            const float GC0 = tot0, GC1 = tot1;
            // end of block 0 (the only block that has a next block when NB = 2)
            float end0 = 0.f, end1 = 0.f;
            if constexpr (NB > 1) {
#pragma unroll
                for (int q = 0; q < NRQ; ++q) {
                    const float s0 = __shfl(p0, (lane & ~(NRQ - 1)) + q, 64);
                    const float s1 = __shfl(p1, (lane & ~(NRQ - 1)) + q, 64);
                    if (q * RPT < 16) { end0 += s0; end1 += s1; }
                }
            }
            // e^(G_end(R) - G_b(R)) for this thread's block (rows of block 0 only)
            const float eb0 = NB > 1 ? __expf(end0 - bs0) : 0.f, eb1 = NB > 1 ? __expf(end1 - bs1) : 0.f;
            float G0 = e0, G1 = e1;
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int r = r0 + j;
                G0 += g0[j];
                G1 += g1[j];
                const float2 kv = ld2(sKh, r), qv = ld2(sQh, r);
                const float fh0 = __expf(G0 - bs0), fh1 = __expf(G1 - bs1);
                const float fi0 = __expf(bs0 - G0), fi1 = __expf(bs1 - G1);
                const float fc0 = __expf(GC0 - G0), fc1 = __expf(GC1 - G1);
                st2(sKh, r, kv.x * fh0, kv.y * fh1);
                const float qh0 = qv.x * fh0, qh1 = qv.y * fh1;
                st2(sQh, r, qh0, qh1);
                if constexpr (kBF)
                    st2(sQl, r, qh0 - bf16_bits_to_f32(O_::enc(qh0)), qh1 - bf16_bits_to_f32(O_::enc(qh1)));
                st2(sKi, r, kv.x * fi0, kv.y * fi1);
                st2(sKb, r, kv.x * fc0, kv.y * fc1);
                // e^(G_end - G_r) = e^(G_b - G_r) e^(G_end - G_b), both within one block
                const float fe0 = fi0 * eb0, fe1 = fi1 * eb1;
                if (my_block < NB - 1) st2(sKe, r, kv.x * fe0, kv.y * fe1);
                if constexpr (SPLIT) {
                    const float2 bv = ld2(sRawB, r);
                    const float ev0 = bv.x * kv.x, ev1 = bv.y * kv.y;
                    st2(sEi, r, ev0 * fi0, ev1 * fi1);
                    st2(sEb, r, ev0 * fc0, ev1 * fc1);
                    if (my_block < NB - 1) st2(sEe, r, ev0 * fe0, ev1 * fe1);
                    if (p.keywrite) st2(sKb, r, ev0 * fc0, ev1 * fc1);   // Kb = Eb
                }
            }
            if (rq == 0) {
                sEgb[ch] = 1.f;
                sEgb[ch + 1] = 1.f;
                if constexpr (NB > 1) {
                    sEgb[DK + ch] = __expf(end0);
                    sEgb[DK + ch + 1] = __expf(end1);
                }
                sGam[ch] = __expf(GC0);
                sGam[ch + 1] = __expf(GC1);
            }
        }
        lds_barrier();

        // ---- C x C products over 16x16 tiles (R, J), J <= R.  Tasks (matrix,
        // tile) go round-robin over the waves; a wave requests the operand
        // fragments of all its tasks before its first MFMA.
        {
            constexpr int NTILE = NB * (NB + 1) / 2;
            constexpr int NMAT = SPLIT ? 4 : 2;
            constexpr int NTASK = NTILE * NMAT;
            constexpr int MAXT = (NTASK + kWavesCW - 1) / kWavesCW;
            // mat 0: A (or A_e)   1: P (or M_k)   2: A_k   3: M_e
            auto task_rj = [](int tix, int& Rr, int& Jr) {
                Rr = tix == 0 ? 0 : 1;
                Jr = tix == 2 ? 1 : 0;
            };
            f32x4 acc[MAXT];
#pragma unroll
            for (int k = 0; k < MAXT; ++k) {
                const int task = w + kWavesCW * k;
                acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (task < NTASK) {
                    const int mat = task / NTILE, tix = task % NTILE;
                    int Rr, Jr;
                    task_rj(tix, Rr, Jr);
                    const bool useQ = mat == 1 || mat == 3;
                    const bool useE = SPLIT && (mat == 0 || mat == 3 || p.keywrite);
                    const S* arow = (useQ ? sQh : sKh) + (16 * Rr + c) * L::LDK;
                    const S* bsrc = Jr == Rr ? (useE ? sEi : sKi) : (useE ? sEe : sKe);
                    const S* brow = bsrc + (16 * Jr + c) * L::LDK;
                    acc[k] = O_::template nat<DK>(acc[k], arow, brow, g);
                    if (kBF && useQ) acc[k] = O_::template nat<DK>(acc[k], sQl + (16 * Rr + c) * L::LDK, brow, g);
                }
            }
#pragma unroll
            for (int k = 0; k < MAXT; ++k) {
                const int task = w + kWavesCW * k;
                if (task < NTASK) {
                    const int mat = task / NTILE, tix = task % NTILE;
                    int Rr, Jr;
                    task_rj(tix, Rr, Jr);
                    const bool strict = mat == 0 || mat == 2;
                    const int col = 16 * Jr + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * Rr + 4 * g + i;
                        float val = acc[k][i];
                        if (!SPLIT && mat == 0) val *= sBeta[row];
                        val = (strict ? row > col : row >= col) ? val : 0.f;
                        if (mat == 0) sA[row * L::LDF + col] = val;
                        else if (mat == 1) sP[row * L::LDM + col] = O_::enc(val);
                        else if (mat == 2) sAk[row * L::LDM + col] = O_::enc(val);
                        else sMe[row * L::LDM + col] = O_::enc(val);
                    }
                }
            }
        }
        lds_barrier();

        // ---- T = (I + A)^-1: diagonal 16x16 blocks by column substitution,
        //      then (two blocks) T_10 = -T_11 A_10 T_00
        if (w == 0 && lane < 16 * NB) {
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
                if constexpr (kBF) sTe[(rb + i) * L::LDM + rb + j] = O_::enc(xs[i]);
            }
        }
        lds_barrier();
        if constexpr (NB == 2) {
            if (w == 0) {
                float av[4], tv[4], dv[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    av[ks] = sA[(16 + c) * L::LDF + 4 * ks + g];
                    tv[ks] = sT[(4 * ks + g) * L::LDF + c];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) dv[i] = sT[(16 + c) * L::LDF + 16 + 4 * g + i];
                f32x4 inner = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) inner = mfma4(av[ks], tv[ks], inner);
                f32x4 out = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) out = mfma4(dv[i], inner[i], out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 + 4 * g + i;
                    sT[row * L::LDF + c] = -out[i];
                    if constexpr (kBF) sTe[row * L::LDM + c] = O_::enc(-out[i]);
                }
            }
            lds_barrier();
        }

        // ---- state-dependent chain (wave 0, 16 value columns)
        if (chain) {
            const S* Te = kBF ? sTe : reinterpret_cast<const S*>(sT);
            constexpr int LDTe = kBF ? L::LDM : L::LDF;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            f32x4 X[NB], Y[NB];
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                // the state decayed to the start of block m, per key channel
                R STr[NKT];
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    f32x4 s = ST[t];
                    if (m > 0) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[i] *= sEgb[m * DK + 16 * t + 4 * g + i];
                    }
                    STr[t] = O_::to_reg(s);
                }
                X[m] = O_::template reg<0, NKT>(zero, sKh + (16 * m + c) * L::LDK, STr, g);
                Y[m] = O_::template reg<0, NKT>(zero, sQh + (16 * m + c) * L::LDK, STr, g);
                if constexpr (kBF) Y[m] = O_::template reg<0, NKT>(Y[m], sQl + (16 * m + c) * L::LDK, STr, g);
            }
            f32x4 Vr[NB];
#pragma unroll
            for (int m = 0; m < NB; ++m) Vr[m] = O_::acc_tile(sV, L::LDV, 16 * m, 0, g, c);
            f32x4 Ot[NB];
            R Ur[NB];   // V~ (one step size) or W (split gates), operand form
            R Wn[NB];   // split gates: -Y~, operand form
            if constexpr (!SPLIT) {
                R Rr[NB];
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    f32x4 r;
#pragma unroll
                    for (int i = 0; i < 4; ++i) r[i] = sBeta[16 * m + 4 * g + i] * (Vr[m][i] - X[m][i]);
                    Rr[m] = O_::to_reg(r);
                }
                f32x4 Vt[NB];
                Vt[0] = O_::template reg<0, 1>(zero, Te + c * LDTe, Rr, g);
                if constexpr (NB == 2) Vt[1] = O_::template reg<0, 2>(zero, Te + (16 + c) * LDTe, Rr, g);
#pragma unroll
                for (int m = 0; m < NB; ++m) Ur[m] = O_::to_reg(Vt[m]);
                Ot[0] = O_::template reg<0, 1>(Y[0], sP + c * L::LDM, Ur, g);
                if constexpr (NB == 2) Ot[1] = O_::template reg<0, 2>(Y[1], sP + (16 + c) * L::LDM, Ur, g);
            } else {
#pragma unroll
                for (int m = 0; m < NB; ++m) Ur[m] = O_::to_reg(Vr[m]);
                // Z = X + A_k W, Y~ = T Z
                R Zr[NB];
                Zr[0] = O_::to_reg(O_::template reg<0, 1>(X[0], sAk + c * L::LDM, Ur, g));
                if constexpr (NB == 2) Zr[1] = O_::to_reg(O_::template reg<0, 2>(X[1], sAk + (16 + c) * L::LDM, Ur, g));
                f32x4 Yt[NB];
                Yt[0] = O_::template reg<0, 1>(zero, Te + c * LDTe, Zr, g);
                if constexpr (NB == 2) Yt[1] = O_::template reg<0, 2>(zero, Te + (16 + c) * LDTe, Zr, g);
#pragma unroll
                for (int m = 0; m < NB; ++m) Wn[m] = O_::to_reg(-Yt[m]);
                // O = Y + M_k W - M_e Y~
                Ot[0] = O_::template reg<0, 1>(O_::template reg<0, 1>(Y[0], sP + c * L::LDM, Ur, g),
                                               sMe + c * L::LDM, Wn, g);
                if constexpr (NB == 2)
                    Ot[1] = O_::template reg<0, 2>(O_::template reg<0, 2>(Y[1], sP + (16 + c) * L::LDM, Ur, g),
                                                   sMe + (16 + c) * L::LDM, Wn, g);
            }
            // S^T <- Diag(e^G_C) S^T + Kb^T U  (- Eb^T Y~ for split gates)
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                f32x4 s = ST[t];
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] *= sGam[16 * t + 4 * g + i];
                s = O_::template regT<NB>(s, sKb, L::LDK, 16 * t, Ur, g, c);
                if constexpr (SPLIT) s = O_::template regT<NB>(s, sEb, L::LDK, 16 * t, Wn, g, c);
                ST[t] = s;
            }
            // sO aliases the raw-gate buffer, last read in the per-channel pass.
#pragma unroll
            for (int m = 0; m < NB; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sO[(16 * m + 4 * g + i) * L::LDV + c] = O_::enc(Ot[m][i]);
            }
        }
        lds_barrier();
        {
            constexpr int OPR = kVTCW / EPC;
            for (int idx = tid; idx < C * OPR; idx += kThreadsCW) {
                const int row = idx / OPR, cc = idx % OPR;
                if (row < Cn) {
                    const int64_t off = ((tokb + row) * H + h) * DV + vt * kVTCW + cc * EPC;
                    *reinterpret_cast<uint4*>(static_cast<S*>(p.o) + off) =
                        *reinterpret_cast<const uint4*>(sO + row * L::LDV + cc * EPC);
                }
            }
        }
        // The next sub-chunk's commit writes sQh/sKh/sRawG (= sO) and sV: the
        // output store above reads sO, so wait for it.
        lds_barrier();
    }

    if (p.ST && chain) {
        float* st = p.ST + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            *reinterpret_cast<float4*>(st + 16 * t + 4 * g) = make_float4(ST[t][0], ST[t][1], ST[t][2], ST[t][3]);
    }
}

template <int VAR, typename E, int DK, int DV>
hipError_t launch_cw_one(const FwdArgs& a, hipStream_t s) {
    constexpr int NVT = DV / kVTCW;
    constexpr int NB = sizeof(typename Ops<E>::S) == 2 ? 2 : 1;
    const int groups = (a.B * a.H + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups) * 8u * NVT);
    hipLaunchKernelGGL((prefill_cw_kernel<VAR, E, DK, DV, NB>), grid, dim3(kThreadsCW), 0, s, a);
    return hipGetLastError();
}

template <int VAR, typename E>
hipError_t launch_cw_dims(const FwdArgs& a, hipStream_t s) {
    if (a.dk == 128 && a.dv == 128) return launch_cw_one<VAR, E, 128, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_cw_one<VAR, E, 128, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_cw_one<VAR, E, 64, 128>(a, s);
    return launch_cw_one<VAR, E, 64, 64>(a, s);
}

}  // namespace

// variant 2: one step size (KDA); 3: split gates (Gated DeltaNet-2); 4: a step
// size per key channel (FG^2-GDN), run as the split form with keywrite set
hipError_t launch_fwd_channel(int variant, int dtype, const FwdArgs& a, hipStream_t s) {
    if (dtype == 1) return launch_fwd_channel_two_pass(variant, a, s);   // bf16: two passes
    if (variant == 2) return launch_cw_dims<2, F32>(a, s);
    FwdArgs b = a;
    b.keywrite = variant == 4 ? 1 : 0;
    return launch_cw_dims<3, F32>(b, s);
}

}  // namespace dr
