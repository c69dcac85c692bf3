// Two-pass chunkwise forward for the channel-wise decay forms with bf16
// operands on gfx950: Kimi Delta Attention (one step size beta_t) and Gated
// DeltaNet-2 (channel-wise erase gate b_t on the key side, write gate w_t on
// the value side; Gated DeltaNet-2 abstract, thelatestinai.com/papers/
// 2607.07953, whose chunkwise WY algorithm absorbs the channel-wise decay into
// asymmetric erase factors).  The algebra per sub-chunk of C = 32 tokens (two
// 16-token blocks) is that of the single-pass kernel in prefill_cw.hip:
//   Kh_r = k_r ⊙ e^(G_r - G_b(R)), Qh likewise (kept as a bf16 hi + lo pair),
//   Kb_j = k_j ⊙ e^(G_C - G_j), and for the C x C products the diagonal-block
//   copies Ki_j = k_j ⊙ e^(G_b(R) - G_j) and the below-diagonal copies
//   Ke_j = k_j ⊙ e^(G_end(J) - G_j);
// one step size:
//   A = StrictTril(diag(beta) Kh Kx^T), T = (I + A)^-1, P = Tril(Qh Kx^T)
//   V~ = T (beta ⊙ (V - X)), X_R = Kh_R (S ⊙ e^G_b(R))^T
//   O = Y + P V~, Y_R = Qh_R (S ⊙ e^G_b(R))^T, S^T <- Diag(e^G_C) S^T + Kb^T V~
// split gates (E = b ⊙ K, W = w ⊙ V):
//   A_e = StrictTril(Kh Ex^T), A_k = StrictTril(Kh Kx^T), T = (I + A_e)^-1
//   Z = X + A_k W, Y~ = T Z, O = Y + M_k W - M_e Y~
//   S^T <- Diag(e^G_C) S^T + Kb^T W - Eb^T Y~
// A step size per key channel (FG^2-GDN, FwdArgs::keywrite) writes along
// E = beta ⊙ K with no write gate.  As the split form it has W = V, A_k = A_e,
// M_k = M_e and Kb = Eb, so Y~ = T (X + A_e V) and V - Y~ = T (V - X): it is the
// one-step-size form with beta = 1 on the rows and E in place of K on the key
// side of A, P and the state update, which is how it runs here.
//
// Everything above except X, Y and the state lines is the same for every
// value tile of a head, and it is most of the work.  Pass 1 computes it once
// per (batch, head, sub-chunk), all sub-chunks in parallel, and writes it to a
// workspace as the exact LDS image that pass 2 reads (a "blob": MFMA operand
// fragments of 16 bytes per lane, 1 KB per fragment, lane-linear, plus the
// per-channel decay vectors).  Pass 2 runs the recurrence per (batch, head, 32
// value columns): two waves each carry a 128 x 16 slice of S^T in fp32
// accumulators and run sub-chunk n, while a third wave copies the blob of
// sub-chunk n + 2 into LDS with global_load_lds: one linear stream, no
// address arithmetic, and no copy instructions in the waves that carry the
// state (issuing them there stalled those waves by about 2K cycles a step).
//
// The state's key channels are held in a permuted order (tile t, lane (g, c),
// element i <-> channel 32 (t / 2) + 8 g + 4 (t % 2) + i), so that two state
// tiles paired as one B operand cover 8 consecutive channels and a key/query
// fragment is one contiguous 16-byte piece of a row.
#include <algorithm>
#include <atomic>

#include "chunk_ops.h"
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kC2 = 32;          // sub-chunk length (two 16-token blocks)
constexpr int kPrepThreads = 256;
constexpr int kChainWaves = 2;   // 16 value columns each
constexpr int kVT2 = 16 * kChainWaves;

// key channel held by element i of lane group g in state tile t
__device__ __forceinline__ int perm_chan(int t, int g, int i) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i; }

// Byte offsets of one sub-chunk's blob.  Fragments: 64 lanes x 16 bytes.
template <int DK, bool SPLIT>
struct Blob {
    static constexpr int NKP = DK / 32;   // 32-channel k steps
    static constexpr int NKT = DK / 16;   // 16-channel state tiles
    static constexpr int F = 1024;
    static constexpr int oKh = 0;                    // [block m][k step q]: Kh[16 m + c][32 q + 8 g ..]
    static constexpr int oQh = oKh + 2 * NKP * F;    // Qh hi
    static constexpr int oQl = oQh + 2 * NKP * F;    // Qh lo
    static constexpr int oKb = oQl + 2 * NKP * F;    // [tile t]: Kb^T, row = channel of state row c
    static constexpr int oEb = oKb + NKT * F;        // split gates: Eb^T
    static constexpr int oT = oEb + (SPLIT ? NKT * F : 0);   // [block m]: row 16 m + c of T
    static constexpr int oP = oT + 2 * F;            // P (or M_k)
    static constexpr int oAk = oP + 2 * F;           // split gates: A_k
    static constexpr int oMe = oAk + (SPLIT ? 2 * F : 0);    // split gates: M_e
    static constexpr int oVec = oMe + (SPLIT ? 2 * F : 0);
    // fp32 vectors: e^(G_end(0)) [DK] and e^(G_C) [DK], both in state order,
    // then beta [C]
    static constexpr int vE1 = 0, vGam = DK, vBeta = 2 * DK;
    static constexpr int bytes = ((oVec + (2 * DK + kC2) * 4 + F - 1) / F) * F;
};

// ----------------------------------------------------------------- pass 1
template <int DK, bool SPLIT>
struct PrepLds {
    static constexpr int C = kC2;
    static constexpr int LDK = DK + 8;     // bf16 [C][DK] operand copies
    static constexpr int LDM = C + 8;      // bf16 C x C
    static constexpr int LDF = C + 4;      // fp32 C x C
    static constexpr int KM = C * LDK * 2;
    static constexpr int KE = 16 * LDK * 2;
    static constexpr int MM = C * LDM * 2;
    static constexpr int MF = C * LDF * 4;
    // live for the whole unit: the copies that go into the blob
    static constexpr int oKh = 0;
    static constexpr int oQh = oKh + KM;
    static constexpr int oQl = oQh + KM;
    static constexpr int oKb = oQl + KM;
    static constexpr int oEb = oKb + KM;
    // one region used three times, separated by barriers: the raw gates,
    // then the copies that only the C x C products read, then their results
    static constexpr int oR = oEb + (SPLIT ? KM : 0);
    static constexpr int oRawG = oR;
    static constexpr int oRawB = oRawG + KM;
    static constexpr int oKi = oR;
    static constexpr int oKe = oKi + KM;
    static constexpr int oEi = oKe + KE;
    static constexpr int oEe = oEi + (SPLIT ? KM : 0);
    static constexpr int oA = oR;                         // A or A_e (fp32)
    static constexpr int oT = oA + MF;                    // T (fp32)
    static constexpr int oTe = oT + MF;                   // T (bf16)
    static constexpr int oP = oTe + MM;                   // P or M_k
    static constexpr int oAk = oP + MM;
    static constexpr int oMe = oAk + (SPLIT ? MM : 0);
    static constexpr int R1 = 2 * KM;   // raw g and raw b (split gates, or FG^2-GDN's step sizes)
    static constexpr int R2 = (SPLIT ? 2 : 1) * (KM + KE);
    static constexpr int R3 = 2 * MF + (SPLIT ? 4 : 2) * MM;
    static constexpr int RB = R1 > R2 ? (R1 > R3 ? R1 : R3) : (R2 > R3 ? R2 : R3);
    static constexpr int oVec = oR + RB;                  // beta[C], e^G_b [2][DK], e^G_C [DK]
    static constexpr int bytes = oVec + (C + 3 * DK) * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Persistent: workgroup i handles units i, i + gridDim.x, ... (unit = head *
// NC + sub-chunk) and loads the raw inputs of its next unit into registers
// while it works on the current one.
template <int DK, bool SPLIT>
__global__ __launch_bounds__(kPrepThreads, 2) void cw_prep_kernel(FwdArgs p, unsigned char* ws, int NC, int total) {
    typedef PrepLds<DK, SPLIT> L;
    typedef Blob<DK, SPLIT> BL;
    constexpr int C = kC2;
    constexpr int NB = 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
    uint16_t* sKh = reinterpret_cast<uint16_t*>(smem + L::oKh);
    uint16_t* sQh = reinterpret_cast<uint16_t*>(smem + L::oQh);
    uint16_t* sQl = reinterpret_cast<uint16_t*>(smem + L::oQl);
    uint16_t* sKi = reinterpret_cast<uint16_t*>(smem + L::oKi);
    uint16_t* sKb = reinterpret_cast<uint16_t*>(smem + L::oKb);
    uint16_t* sKe = reinterpret_cast<uint16_t*>(smem + L::oKe);
    uint16_t* sEi = reinterpret_cast<uint16_t*>(smem + L::oEi);
    uint16_t* sEb = reinterpret_cast<uint16_t*>(smem + L::oEb);
    uint16_t* sEe = reinterpret_cast<uint16_t*>(smem + L::oEe);
    uint16_t* sRawG = reinterpret_cast<uint16_t*>(smem + L::oRawG);
    uint16_t* sRawB = reinterpret_cast<uint16_t*>(smem + L::oRawB);
    float* sA = reinterpret_cast<float*>(smem + L::oA);
    float* sT = reinterpret_cast<float*>(smem + L::oT);
    uint16_t* sTe = reinterpret_cast<uint16_t*>(smem + L::oTe);
    uint16_t* sP = reinterpret_cast<uint16_t*>(smem + L::oP);
    uint16_t* sAk = reinterpret_cast<uint16_t*>(smem + L::oAk);
    uint16_t* sMe = reinterpret_cast<uint16_t*>(smem + L::oMe);
    float* sBeta = reinterpret_cast<float*>(smem + L::oVec);
    float* sEgb = sBeta + C;          // [NB][DK]
    float* sGam = sEgb + NB * DK;     // [DK]

    const int T = p.T, H = p.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    // raw q, k, g (and the erase gate) of a unit: 16-byte pieces; rows past
    // the end of the sequence are zero (zero decay, no key, no query)
    constexpr int PPR = DK / 8;                       // pieces per row
    constexpr int NPC = C * PPR / kPrepThreads;       // pieces per thread
    static_assert(C * PPR % kPrepThreads == 0, "piece split");
    uint4 rq[NPC], rk[NPC], rg[NPC], rb[NPC];
    uint16_t rbeta = 0;
    auto fetch = [&](int unit) {
        const int ubh = unit / NC, un = unit % NC;
        const int ub = ubh / H, uh = ubh % H;
        const int uhk = uh / (H / p.Hk);   // the value head's query/key head
        const int ucn = min(C, T - un * C);
        const int64_t utok = static_cast<int64_t>(ub) * T + un * C;
#pragma unroll
        for (int j = 0; j < NPC; ++j) {
            const int idx = tid + kPrepThreads * j;
            const int row = idx / PPR, cc = idx % PPR;
            rq[j] = make_uint4(0, 0, 0, 0);
            rk[j] = rq[j];
            rg[j] = rq[j];
            rb[j] = rq[j];
            if (row < ucn) {
                const int64_t off = ((utok + row) * H + uh) * DK + 8 * cc;
                const int64_t qoff = ((utok + row) * p.Hk + uhk) * DK + 8 * cc;
                rq[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qoff);
                rk[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + qoff);
                rg[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.g) + off);
                if (SPLIT || p.keywrite) rb[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.beta) + off);
            }
        }
        if constexpr (!SPLIT) {
            rbeta = 0;
            if (tid < ucn)   // FG^2-GDN: the step sizes sit on the key side, rows take 1
                rbeta = p.keywrite ? uint16_t(0x3F80) : static_cast<const uint16_t*>(p.beta)[(utok + tid) * H + uh];
        }
    };
    if (static_cast<int>(blockIdx.x) < total) fetch(blockIdx.x);
    for (int unit = blockIdx.x; unit < total; unit += gridDim.x) {
    const int bh = unit / NC, n = unit % NC;
    // ---- commit the raw inputs, then start fetching the next unit's
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
        const int idx = tid + kPrepThreads * j;
        const int row = idx / PPR, cc = idx % PPR;
        *reinterpret_cast<uint4*>(sQh + row * L::LDK + 8 * cc) = rq[j];
        *reinterpret_cast<uint4*>(sKh + row * L::LDK + 8 * cc) = rk[j];
        *reinterpret_cast<uint4*>(sRawG + row * L::LDK + 8 * cc) = rg[j];
        if (SPLIT || p.keywrite) *reinterpret_cast<uint4*>(sRawB + row * L::LDK + 8 * cc) = rb[j];
    }
    if constexpr (!SPLIT) {
        if (tid < C) sBeta[tid] = bf16_bits_to_f32(rbeta);
    }
    __syncthreads();
    if (unit + static_cast<int>(gridDim.x) < total) fetch(unit + gridDim.x);

    // ---- per channel: cumulative decay and the decay-carrying copies.
    // Thread (channel pair cp, row group rq): channels 2 cp, 2 cp + 1 and RPT
    // consecutive rows.  A wave holds CPW channel pairs, and the row groups of a
    // pair are lanes CPW apart, which exchange their partial decay sums by
    // shuffles: the lanes of one half-wave then read and write CPW consecutive
    // words of each of two row groups, rows 16 * 32 / DK apart, in different LDS
    // banks (with the row groups of a pair in adjacent lanes, groups 0 and 2
    // shared their banks).
    {
        constexpr int NRQ = 2 * kPrepThreads / DK;
        constexpr int RPT = C / NRQ;
        constexpr int CPW = 64 / NRQ;
        static_assert(RPT >= 1 && C % NRQ == 0 && 16 % RPT == 0, "row split");
        const int rq = lane / CPW, cp = w * CPW + lane % CPW;
        const int ch = 2 * cp, r0 = rq * RPT;
        auto ld2 = [&](const uint16_t* m, int r) -> float2 {
            const uint32_t u = *reinterpret_cast<const uint32_t*>(m + r * L::LDK + ch);
            return make_float2(bf16_bits_to_f32(static_cast<uint16_t>(u & 0xffffu)),
                               bf16_bits_to_f32(static_cast<uint16_t>(u >> 16)));
        };
        auto st2 = [&](uint16_t* m, int r, float x0, float x1) {
            *reinterpret_cast<uint32_t*>(m + r * L::LDK + ch) =
                static_cast<uint32_t>(f32_to_bf16_bits(x0)) | (static_cast<uint32_t>(f32_to_bf16_bits(x1)) << 16);
        };
        float g0[RPT], g1[RPT], b0[RPT], b1[RPT];
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const float2 v = ld2(sRawG, r0 + j);
            g0[j] = fmaxf(v.x, kLogDecayFloor);
            g1[j] = fmaxf(v.y, kLogDecayFloor);
            p0 += g0[j];
            p1 += g1[j];
            if (SPLIT || p.keywrite) {
                const float2 bv = ld2(sRawB, r0 + j);
                b0[j] = bv.x;
                b1[j] = bv.y;
            }
        }
        // the copies below overwrite the raw gates
        __syncthreads();
        float e0 = 0.f, e1 = 0.f, tot0 = 0.f, tot1 = 0.f, bs0 = 0.f, bs1 = 0.f, end0 = 0.f, end1 = 0.f;
        const int my_block = r0 / 16;
#pragma unroll
        for (int q = 0; q < NRQ; ++q) {
            const float s0 = __shfl(p0, q * CPW + lane % CPW, 64);
            const float s1 = __shfl(p1, q * CPW + lane % CPW, 64);
            if (q < rq) { e0 += s0; e1 += s1; }
            if (q * RPT < 16 * my_block) { bs0 += s0; bs1 += s1; }
            if (q * RPT < 16) { end0 += s0; end1 += s1; }
            tot0 += s0;
            tot1 += s1;
        }
        const float GC0 = tot0, GC1 = tot1;
        // e^(G_end(0) - G_b(R)) for rows of block 0
        const float eb0 = __expf(end0 - bs0), eb1 = __expf(end1 - bs1);
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
            st2(sQl, r, qh0 - bf16_bits_to_f32(f32_to_bf16_bits(qh0)), qh1 - bf16_bits_to_f32(f32_to_bf16_bits(qh1)));
            // FG^2-GDN in the one-step-size form: the key-side copies (the columns of
            // A and P, and the state update) carry the step sizes, E = beta ⊙ k
            const bool kw = !SPLIT && p.keywrite;
            const float kc0 = kw ? b0[j] * kv.x : kv.x, kc1 = kw ? b1[j] * kv.y : kv.y;
            st2(sKi, r, kc0 * fi0, kc1 * fi1);
            st2(sKb, r, kc0 * fc0, kc1 * fc1);
            // e^(G_end - G_r) = e^(G_b - G_r) e^(G_end - G_b), both within one block
            const float fe0 = fi0 * eb0, fe1 = fi1 * eb1;
            if (my_block == 0) st2(sKe, r, kc0 * fe0, kc1 * fe1);
            if constexpr (SPLIT) {
                const float ev0 = b0[j] * kv.x, ev1 = b1[j] * kv.y;
                st2(sEi, r, ev0 * fi0, ev1 * fi1);
                st2(sEb, r, ev0 * fc0, ev1 * fc1);
                if (my_block == 0) st2(sEe, r, ev0 * fe0, ev1 * fe1);
            }
        }
        if (rq == 0) {
            sEgb[ch] = 1.f;
            sEgb[ch + 1] = 1.f;
            sEgb[DK + ch] = __expf(end0);
            sEgb[DK + ch + 1] = __expf(end1);
            sGam[ch] = __expf(GC0);
            sGam[ch + 1] = __expf(GC1);
        }
    }
    __syncthreads();

    // ---- C x C products over 16x16 tiles (R, J), J <= R; tasks (matrix,
    // tile) go round-robin over the waves.
    {
        constexpr int NTILE = 3;
        constexpr int NMAT = SPLIT ? 4 : 2;
        constexpr int NTASK = NTILE * NMAT;
        constexpr int NW = kPrepThreads / 64;
        constexpr int MAXT = (NTASK + NW - 1) / NW;
        // mat 0: A (or A_e)   1: P (or M_k)   2: A_k   3: M_e
        auto task_rj = [](int tix, int& Rr, int& Jr) {
            Rr = tix == 0 ? 0 : 1;
            Jr = tix == 2 ? 1 : 0;
        };
        f32x4 acc[MAXT];
#pragma unroll
        for (int k = 0; k < MAXT; ++k) {
            const int task = w + NW * k;
            acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (task < NTASK) {
                const int mat = task / NTILE, tix = task % NTILE;
                int Rr, Jr;
                task_rj(tix, Rr, Jr);
                const bool useQ = mat == 1 || mat == 3;
                const bool useE = SPLIT && (mat == 0 || mat == 3);
                const uint16_t* arow = (useQ ? sQh : sKh) + (16 * Rr + c) * L::LDK;
                const uint16_t* bsrc = Jr == Rr ? (useE ? sEi : sKi) : (useE ? sEe : sKe);
                const uint16_t* brow = bsrc + (16 * Jr + c) * L::LDK;
                acc[k] = Ops<BF16>::template nat<DK>(acc[k], arow, brow, g);
                if (useQ) acc[k] = Ops<BF16>::template nat<DK>(acc[k], sQl + (16 * Rr + c) * L::LDK, brow, g);
            }
        }
        // the results below overwrite the copies read above
        __syncthreads();
#pragma unroll
        for (int k = 0; k < MAXT; ++k) {
            const int task = w + NW * k;
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
                    else if (mat == 1) sP[row * L::LDM + col] = f32_to_bf16_bits(val);
                    else if (mat == 2) sAk[row * L::LDM + col] = f32_to_bf16_bits(val);
                    else sMe[row * L::LDM + col] = f32_to_bf16_bits(val);
                }
            }
        }
    }
    __syncthreads();

    // ---- T = (I + A)^-1: diagonal 16x16 blocks by column substitution (fp32),
    // then T_10 = -T_11 A_10 T_00 (fp32 MFMA)
    if (w == 0 && lane < 32) {
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
            sTe[(rb + i) * L::LDM + rb + j] = f32_to_bf16_bits(xs[i]);
        }
    }
    __syncthreads();
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
        for (int i = 0; i < 4; ++i) sTe[(16 + 4 * g + i) * L::LDM + c] = f32_to_bf16_bits(-out[i]);
    }
    __syncthreads();

    // ---- the blob: fragments in the chain's lane order
    unsigned char* blob = ws + (static_cast<int64_t>(bh) * NC + n) * BL::bytes;
    // row fragments of Kh, Qh, Ql: lane (g, c) of fragment (m, q) holds
    // row 16 m + c, columns 32 q + 8 g .. + 7
    for (int idx = tid; idx < 3 * 2 * BL::NKP * 64; idx += kPrepThreads) {
        const int mat = idx / (2 * BL::NKP * 64), f = (idx / 64) % (2 * BL::NKP), l = idx % 64;
        const int m = f / BL::NKP, q = f % BL::NKP;
        const uint16_t* src = (mat == 0 ? sKh : mat == 1 ? sQh : sQl) + (16 * m + (l & 15)) * L::LDK + 32 * q + 8 * (l >> 4);
        const int off = (mat == 0 ? BL::oKh : mat == 1 ? BL::oQh : BL::oQl) + f * 1024 + l * 16;
        *reinterpret_cast<uint4*>(blob + off) = *reinterpret_cast<const uint4*>(src);
    }
    // transposed key copies for the state update: lane (g, c) of fragment t
    // holds rows 4 g .. + 3 and 16 + 4 g .. + 3 of the channel that row c of
    // state tile t holds
    for (int idx = tid; idx < (SPLIT ? 2 : 1) * BL::NKT * 64; idx += kPrepThreads) {
        const int mat = idx / (BL::NKT * 64), t = (idx / 64) % BL::NKT, l = idx % 64;
        const int lg = l >> 4, lc = l & 15;
        const int ch = perm_chan(t, lc >> 2, lc & 3);
        const uint16_t* src = (mat == 0 ? sKb : sEb) + ch;
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            wv[i / 2] = static_cast<uint32_t>(src[(4 * lg + i) * L::LDK]) |
                        (static_cast<uint32_t>(src[(4 * lg + i + 1) * L::LDK]) << 16);
            wv[2 + i / 2] = static_cast<uint32_t>(src[(16 + 4 * lg + i) * L::LDK]) |
                            (static_cast<uint32_t>(src[(16 + 4 * lg + i + 1) * L::LDK]) << 16);
        }
        *reinterpret_cast<uint4*>(blob + (mat == 0 ? BL::oKb : BL::oEb) + t * 1024 + l * 16) =
            make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    // C x C row fragments: lane (g, c) of fragment m holds row 16 m + c,
    // columns 4 g .. + 3 (block 0) and 16 + 4 g .. + 3 (block 1; zero for m = 0)
    for (int idx = tid; idx < (SPLIT ? 4 : 2) * 2 * 64; idx += kPrepThreads) {
        const int mat = idx / 128, m = (idx / 64) % 2, l = idx % 64;
        const int lg = l >> 4, lc = l & 15;
        const uint16_t* M = mat == 0 ? sTe : mat == 1 ? sP : mat == 2 ? sAk : sMe;
        const uint16_t* row = M + (16 * m + lc) * L::LDM;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * lg);
        const uint2 hi = m == 0 ? make_uint2(0, 0) : *reinterpret_cast<const uint2*>(row + 16 + 4 * lg);
        const int base = mat == 0 ? BL::oT : mat == 1 ? BL::oP : mat == 2 ? BL::oAk : BL::oMe;
        *reinterpret_cast<uint4*>(blob + base + m * 1024 + l * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    // per-channel vectors in state order, and beta
    float* vec = reinterpret_cast<float*>(blob + BL::oVec);
    for (int k = tid; k < DK; k += kPrepThreads) {
        const int t = k / 16, lg = (k / 4) % 4, i = k % 4;
        const int ch = perm_chan(t, lg, i);
        vec[BL::vE1 + k] = sEgb[DK + ch];
        vec[BL::vGam + k] = sGam[ch];
    }
    if (tid < C) vec[BL::vBeta + tid] = SPLIT ? 0.f : sBeta[tid];
    // the next unit's commit overwrites the LDS read above
    __syncthreads();
    }
}

// ----------------------------------------------------------------- pass 2
typedef __attribute__((address_space(3))) void lds_void2;

__device__ __forceinline__ void blob_to_lds(const unsigned char* src, unsigned char* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_void2*)(lds), 16, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf4(f32x4 x) {
    bf16x4 r;
    r[0] = static_cast<bf16_t>(x[0]);
    r[1] = static_cast<bf16_t>(x[1]);
    r[2] = static_cast<bf16_t>(x[2]);
    r[3] = static_cast<bf16_t>(x[3]);
    return r;
}

template <int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(64 * (kChainWaves + 1)) __attribute__((amdgpu_waves_per_eu(1, 1)))
void cw_chain_kernel(FwdArgs p, const unsigned char* ws, int NC) {
    typedef Blob<DK, SPLIT> BL;
    constexpr int NKP = BL::NKP, NKT = BL::NKT;
    constexpr int NVT = DV / kVT2;
    constexpr int LDV = 16 + 8;                 // value staging rows (bf16)
    constexpr int SLOTS = 3;
    constexpr int NBL = BL::bytes / 1024;       // 1 KB copy instructions per blob
    constexpr int STAGE = kChainWaves * 2 * kC2 * LDV * 2;   // value staging
    __shared__ __attribute__((aligned(16))) unsigned char smem[SLOTS * BL::bytes + STAGE + 256];   // + touch sink
    const int x = blockIdx.x;
    const int groups = (p.B * p.H + 7) / 8;
    const int vt = (x / 8) % NVT;
    const int bh = (x % 8) * groups + x / (8 * NVT);
    if (bh >= p.B * p.H) return;
    const int b = bh / p.H, h = bh % p.H;
    const int T = p.T, H = p.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    auto slot = [&](int n) { return smem + (n % SLOTS) * BL::bytes; };
    if (w == kChainWaves) {
        // ---- loader: the blob of sub-chunk n + 2 during step n; instruction
        // j copies bytes 1024 j .. + 1023 (lane l: 16 l .. + 15).  One barrier
        // per step, matching the chain waves'.
        const unsigned char* wsh = ws + static_cast<int64_t>(bh) * NC * BL::bytes + 16 * lane;
        // blob min(n, NC - 1) into slot(n): past the end the copy repeats the
        // last blob into a slot that no wave reads any more (it held blob
        // n - 3), so every step issues the same loads
        auto copy_blob = [&](int n) {
            const unsigned char* src = wsh + static_cast<int64_t>(min(n, NC - 1)) * BL::bytes;
            unsigned char* dst = slot(n);
#pragma unroll
            for (int j = 0; j < NBL; ++j) blob_to_lds(src + 1024 * j, dst + 1024 * j);
        };
        // Blobs come from HBM cold, and a stream of such copies held a step to
        // about 30 bytes per ns per CU (misses in flight per CU over memory
        // latency), while copies that hit L2 cost little.  So during step n
        // each of the head's NVT value-tile workgroups (all on one XCD, sharing
        // its L2) touches its share of blob n + 4, pieces j = vt (mod NVT), one
        // 4-byte load per lane and piece (every 128-byte line of the piece).
        // The blob is then in L2 when it is copied two steps later, and the
        // cold reads are spread over NVT CUs.  The touches are global-to-LDS
        // loads into a 256-byte area that nothing reads: with no register
        // result, nothing ever waits for them except the counter below.
        // Every touch is issued (piece and blob indices clamped), so each step
        // issues the same loads.
        constexpr int kTouch = (NBL + NVT - 1) / NVT;   // touch loads per step
        static_assert(kTouch >= 1 && kTouch <= 63, "touch count");
        constexpr int kWaitCopy = (kTouch & 15) | ((kTouch >> 4) << 14) | 0x0F70;   // vmcnt(kTouch)
        const unsigned char* wsu = ws + static_cast<int64_t>(bh) * NC * BL::bytes;   // this head's blobs
        uint32_t toff[kTouch];   // lane offset of each touch within a blob
#pragma unroll
        for (int i = 0; i < kTouch; ++i) toff[i] = 16 * lane + 1024 * min(vt + NVT * i, NBL - 1);
        unsigned char* sink = smem + SLOTS * BL::bytes + STAGE;
        auto step = [&](int n) {
            copy_blob(n + 2);
            const unsigned char* src = wsu + static_cast<int64_t>(min(n + 4, NC - 1)) * BL::bytes;
#pragma unroll
            for (int i = 0; i < kTouch; ++i) __builtin_amdgcn_global_load_lds(src + toff[i], (lds_void2*)(sink), 4, 0, 0);
            // the copy (and the touches of step n - 1) have landed; this
            // step's touches may not have
            __builtin_amdgcn_s_waitcnt(kWaitCopy);
            lds_barrier();
        };
        // The copy of blob n + 2 issued in step n must have landed by the end
        // of step n: the chain waves read blob n + 2 into registers during
        // step n + 1, one step ahead of its use.
        if (NC > 0) copy_blob(0);
        if (NC > 1) copy_blob(1);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
        for (int n = 0; n < NC; ++n) step(n);
        return;
    }
    const int vc0 = vt * kVT2 + 16 * w;
    uint16_t* sV = reinterpret_cast<uint16_t*>(smem + SLOTS * BL::bytes) + w * 2 * kC2 * LDV;   // v, then w

    f32x4 ST[NKT];
    {
        const float* s0 = p.S0 ? p.S0 + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK : nullptr;
        // (the test outside the loop: a load under a branch inside it was waited
        // for before the next one was issued)
        if (s0) {
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                const float4 v4 = *reinterpret_cast<const float4*>(s0 + perm_chan(t, g, 0));
                ST[t] = f32x4{v4.x, v4.y, v4.z, v4.w};
            }
        } else {
#pragma unroll
            for (int t = 0; t < NKT; ++t) ST[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the state has landed before the loop
    }
    // value (and write-gate) rows: lane = 2 row + half, 8 columns per lane
    uint4 pv = make_uint4(0, 0, 0, 0), pw = pv;
    auto vload = [&](int n) {
        const int row = lane >> 1;
        const int t = min(n * kC2 + row, T - 1);
        const int64_t off = ((static_cast<int64_t>(b) * T + t) * H + h) * DV + vc0 + 8 * (lane & 1);
        pv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + off);
        if constexpr (SPLIT) pw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.wgate) + off);
    };
    const int vvo = (4 * g + (c >> 2)) * LDV + 4 * (c & 3);   // transpose reads of the staged rows
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // Operands of sub-chunk n that open its step (the key/query fragments
    // and decay vector of X and Y, and the staged value rows) are read during
    // step n - 1, right after their registers are last used: blob n is
    // complete from the start of step n - 1, and the value rows are the
    // wave's own.
    bf16x8 kh[2 * NKP], qh[2 * NKP], ql[2 * NKP];
    f32x4 e1v[NKT];
    bf16x4 vv[2], wr[2];
    // the rest of sub-chunk n's operands, read during step n - 1 after the
    // state update, when their registers are free
    bf16x8 tf[2], pf[2], af[2], mf[2], kbt[NKT], ebt[NKT];
    f32x4 gmv[NKT], btv[2];
    auto read_rest = [&](int n) {
        const unsigned char* bl = slot(n) + 16 * lane;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            tf[m] = *reinterpret_cast<const bf16x8*>(bl + BL::oT + m * 1024);
            pf[m] = *reinterpret_cast<const bf16x8*>(bl + BL::oP + m * 1024);
            if constexpr (SPLIT) {
                af[m] = *reinterpret_cast<const bf16x8*>(bl + BL::oAk + m * 1024);
                mf[m] = *reinterpret_cast<const bf16x8*>(bl + BL::oMe + m * 1024);
            }
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            kbt[t] = *reinterpret_cast<const bf16x8*>(bl + BL::oKb + t * 1024);
            if constexpr (SPLIT) ebt[t] = *reinterpret_cast<const bf16x8*>(bl + BL::oEb + t * 1024);
        }
        const float* vec = reinterpret_cast<const float*>(slot(n) + BL::oVec);
#pragma unroll
        for (int t = 0; t < NKT; ++t) gmv[t] = *reinterpret_cast<const f32x4*>(vec + BL::vGam + 16 * t + 4 * g);
#pragma unroll
        for (int m = 0; m < 2; ++m) btv[m] = *reinterpret_cast<const f32x4*>(vec + BL::vBeta + 16 * m + 4 * g);
    };
    auto read_xy = [&](int n) {
        const unsigned char* bl = slot(n) + 16 * lane;
#pragma unroll
        for (int f = 0; f < 2 * NKP; ++f) {
            kh[f] = *reinterpret_cast<const bf16x8*>(bl + BL::oKh + f * 1024);
            qh[f] = *reinterpret_cast<const bf16x8*>(bl + BL::oQh + f * 1024);
            ql[f] = *reinterpret_cast<const bf16x8*>(bl + BL::oQl + f * 1024);
        }
        const float* vec = reinterpret_cast<const float*>(slot(n) + BL::oVec);
#pragma unroll
        for (int t = 0; t < NKT; ++t) e1v[t] = *reinterpret_cast<const f32x4*>(vec + BL::vE1 + 16 * t + 4 * g);
    };
    // stage the value rows of sub-chunk n (rows past the end are zero;
    // component-wise selects, since a whole-vector select sends the registers
    // through scratch memory) and read them back in accumulator layout
    auto stage_v = [&](int n) {
        const bool ok = (lane >> 1) < min(kC2, T - n * kC2);
        auto sel = [ok](uint4 v) { return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u); };
        *reinterpret_cast<uint4*>(sV + (lane >> 1) * LDV + 8 * (lane & 1)) = sel(pv);
        if constexpr (SPLIT) *reinterpret_cast<uint4*>(sV + kC2 * LDV + (lane >> 1) * LDV + 8 * (lane & 1)) = sel(pw);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            vv[m] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(sV + 16 * m * LDV + vvo)));
            if constexpr (SPLIT)
                wr[m] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(sV + kC2 * LDV + 16 * m * LDV + vvo)));
        }
    };
    if (NC > 0) vload(0);
    __syncthreads();
    if (NC > 0) {
        read_xy(0);
        read_rest(0);
        stage_v(0);
        if (NC > 1) vload(1);
    }
    bf16x4 od[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};   // output rows being stored
    uint16_t* oad[2] = {nullptr, nullptr};          // and their addresses
    for (int n = 0; n < NC; ++n) {
        const int Cn = min(kC2, T - n * kC2);
        // the state, and the state decayed to the start of block 1, as B operands
        bf16x8 SP0[NKP], SP1[NKP];
#pragma unroll
        for (int q = 0; q < NKP; ++q) {
            SP0[q] = cat(to_bf4(ST[2 * q]), to_bf4(ST[2 * q + 1]));
            SP1[q] = cat(to_bf4(ST[2 * q] * e1v[2 * q]), to_bf4(ST[2 * q + 1] * e1v[2 * q + 1]));
        }
        // X_m = Kh_m S_m^T (accumulator layout), Y_m = (Qh + Ql)_m S_m^T
        // transposed (lane (g, c): row 16 m + c, value columns 4 g .. + 3)
        f32x4 X[2] = {zero, zero}, Yt[2] = {zero, zero};
#pragma unroll
        for (int q = 0; q < NKP; ++q) {
            X[0] = mfma32(kh[q], SP0[q], X[0]);
            Yt[0] = mfma32(SP0[q], qh[q], Yt[0]);
            Yt[0] = mfma32(SP0[q], ql[q], Yt[0]);
            X[1] = mfma32(kh[NKP + q], SP1[q], X[1]);
            Yt[1] = mfma32(SP1[q], qh[NKP + q], Yt[1]);
            Yt[1] = mfma32(SP1[q], ql[NKP + q], Yt[1]);
        }
        // (the last step reads a slot that nothing writes any more)
        read_xy(n + 1 < NC ? n + 1 : n);
        bf16x8 U01, Wn01;   // the value-side operand of the state update (and -Y~)
        f32x4 Ot[2];
        if constexpr (!SPLIT) {
            bf16x4 Rb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                f32x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = btv[m][i] * (static_cast<float>(vv[m][i]) - X[m][i]);
                Rb[m] = to_bf4(r);
            }
            const bf16x8 R01 = cat(Rb[0], Rb[1]);
            const f32x4 Vt0 = mfma32(tf[0], R01, zero);
            const f32x4 Vt1 = mfma32(tf[1], R01, zero);
            U01 = cat(to_bf4(Vt0), to_bf4(Vt1));
#pragma unroll
            for (int m = 0; m < 2; ++m) Ot[m] = mfma32(U01, pf[m], Yt[m]);
        } else {
            bf16x4 Wb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                f32x4 wv;
#pragma unroll
                for (int i = 0; i < 4; ++i) wv[i] = static_cast<float>(vv[m][i]) * static_cast<float>(wr[m][i]);
                Wb[m] = to_bf4(wv);
            }
            U01 = cat(Wb[0], Wb[1]);
            // Z = X + A_k W, Y~ = T Z
            const f32x4 Z0 = mfma32(af[0], U01, X[0]);
            const f32x4 Z1 = mfma32(af[1], U01, X[1]);
            const bf16x8 Z01 = cat(to_bf4(Z0), to_bf4(Z1));
            const f32x4 Y0 = mfma32(tf[0], Z01, zero);
            const f32x4 Y1 = mfma32(tf[1], Z01, zero);
            Wn01 = cat(to_bf4(-Y0), to_bf4(-Y1));
            // O = Y + M_k W - M_e Y~
#pragma unroll
            for (int m = 0; m < 2; ++m) Ot[m] = mfma32(Wn01, mf[m], mfma32(U01, pf[m], Yt[m]));
        }
        // S^T <- Diag(e^G_C) S^T + Kb^T U (- Eb^T Y~)
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            f32x4 s = mfma32(kbt[t], U01, ST[t] * gmv[t]);
            if constexpr (SPLIT) s = mfma32(ebt[t], Wn01, s);
            ST[t] = s;
        }
        read_rest(n + 1 < NC ? n + 1 : n);
        // The next value rows are staged before this step's outputs are
        // stored: staging waits for the value load, and with the (masked,
        // so uncounted) stores issued after it that wait becomes a wait for
        // every store in flight.  Placed here it covers the stores of the
        // previous step, which have had a whole step to drain.
        if (n + 1 < NC) {
            stage_v(n + 1);
            if (n + 2 < NC) vload(n + 2);
        }
        // outputs: row 16 m + c, value columns vc0 + 4 g .. + 3.  The store
        // registers (data and address) stay reserved until the next step
        // refills them, so no instruction waits for the stores to drain.
        asm volatile("" ::"v"(od[0]), "v"(od[1]), "v"(oad[0]), "v"(oad[1]));
        uint16_t* orow = static_cast<uint16_t*>(p.o) + ((static_cast<int64_t>(b) * T + n * kC2 + c) * H + h) * DV + vc0 + 4 * g;
        const int64_t mstride = static_cast<int64_t>(16) * H * DV;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            od[m] = to_bf4(Ot[m]);
            oad[m] = orow + m * mstride;
            if (16 * m + c < Cn) *reinterpret_cast<bf16x4*>(oad[m]) = od[m];
        }
        // this wave's reads of the slot are done (the loader refills it in
        // the next step); the blob of sub-chunk n + 1 has landed
        lds_barrier();
    }
    if (p.ST) {
        float* st = p.ST + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            *reinterpret_cast<float4*>(st + perm_chan(t, g, 0)) = make_float4(ST[t][0], ST[t][1], ST[t][2], ST[t][3]);
    }
}


// Workgroups of pass 1 resident on the device at once (it is persistent).
template <int DK, bool SPLIT>
hipError_t prep_resident(int* out) {
    static std::atomic<int> cached{0};   // per template instance; one device model
    int r = cached.load(std::memory_order_relaxed);
    if (r == 0) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cw_prep_kernel<DK, SPLIT>, kPrepThreads, 0);
        if (e != hipSuccess) return e;
        r = std::max(1, cus * per_cu);
        cached.store(r, std::memory_order_relaxed);
    }
    *out = r;
    return hipSuccess;
}

template <int DK, int DV, bool SPLIT>
hipError_t launch_two_pass(const FwdArgs& a, hipStream_t s) {
    // the blobs live in the caller's workspace (fwd_workspace_bytes)
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    const int NC = (a.T + kC2 - 1) / kC2;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    const int64_t total = heads * NC;   // pass-1 units
    if (total > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
    if (NC > 0) {
        int resident = 0;
        hipError_t e = prep_resident<DK, SPLIT>(&resident);
        if (e != hipSuccess) return e;
        const unsigned grid = static_cast<unsigned>(std::min<int64_t>(total, resident));
        hipLaunchKernelGGL((cw_prep_kernel<DK, SPLIT>), dim3(grid), dim3(kPrepThreads), 0, s, a, ws, NC, static_cast<int>(total));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NVT = DV / kVT2;
    const int groups = static_cast<int>((heads + 7) / 8);
    hipLaunchKernelGGL((cw_chain_kernel<DK, DV, SPLIT>), dim3(static_cast<unsigned>(groups) * 8u * NVT), dim3(64 * (kChainWaves + 1)), 0, s, a,
                       ws, NC);
    return hipGetLastError();
}

template <bool SPLIT>
hipError_t launch_two_pass_dims(const FwdArgs& a, hipStream_t s) {
    if (a.dk == 128 && a.dv == 128) return launch_two_pass<128, 128, SPLIT>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_two_pass<128, 64, SPLIT>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_two_pass<64, 128, SPLIT>(a, s);
    return launch_two_pass<64, 64, SPLIT>(a, s);
}

}  // namespace

template <int DK, bool SPLIT>
size_t blob_workspace(int B, int T, int H) {
    const int64_t NC = (T + kC2 - 1) / kC2;
    return round_up_256(static_cast<size_t>(static_cast<int64_t>(B) * H * NC) * Blob<DK, SPLIT>::bytes);
}

size_t fwd_workspace_bytes(int variant, int dtype, int B, int T, int H, int dk, int dv) {
    (void)dv;
    if (variant < 2 || dtype != 1) return 0;   // only the two-pass channel-wise forward has one
    const bool split = variant == 3;
    if (dk == 128) return split ? blob_workspace<128, true>(B, T, H) : blob_workspace<128, false>(B, T, H);
    return split ? blob_workspace<64, true>(B, T, H) : blob_workspace<64, false>(B, T, H);
}

hipError_t launch_fwd_channel_two_pass(int variant, const FwdArgs& a, hipStream_t s) {
    FwdArgs b = a;
    b.keywrite = variant == 4 ? 1 : 0;
    if (variant == 3) return launch_two_pass_dims<true>(b, s);
    return launch_two_pass_dims<false>(b, s);   // KDA, and FG^2-GDN in the one-step-size form
}

}  // namespace dr
