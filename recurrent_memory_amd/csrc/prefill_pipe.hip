// Software-pipelined chunkwise forward for the ungated and scalar-decay forms
// (DeltaNet, Gated DeltaNet) with bf16 operands on gfx950.
//
// The algebra is that of the chunkwise WY evaluation (Gated DeltaNet-2
// abstract, thelatestinai.com/papers/2607.07953; the update is affine in the
// previous memory, DeltaTTT summary, paperlayer.ai, §2):
//   A  = diag(beta) StrictTril(K K^T ⊙ Gamma),  T = (I + A)^-1
//   P  = Tril(Q K^T ⊙ Gamma),                   Gamma[r,j] = e^(G_r - G_j)
//   V~ = T (beta ⊙ (V - e^G ⊙ K S^T))
//   O  = e^G ⊙ Q S^T + P V~
//   S^T <- e^G_C S^T + K^T (e^(G_C - G) ⊙ V~)
// Only the last three lines depend on the state, so the blocks of A and T
// and P of chunk n + 1 can be built while chunk n runs through the state.
// T is applied by block forward substitution over the four 16-row blocks,
//   V~_J = T_JJ (R_J - Σ_{M<J} A_JM V~_M),   R = beta ⊙ (V - e^G ⊙ K S^T),
// which needs only the diagonal blocks T_JJ = (I + A_JJ)^-1 and the
// off-diagonal blocks of A.  One workgroup of four waves per (batch, head,
// 32 value columns):
//   waves 0, 1 ("chain")  chunk n: the state-dependent lines above, 16 value
//                         columns each, S^T in fp32 accumulators throughout;
//   wave 2 ("T builder")  chunk n + 1: the diagonal blocks of A from K K^T,
//                         T_JJ by substitution (fp32), and the off-diagonal
//                         blocks A_JM by MFMA;
//   wave 3                issues the HBM -> LDS loads of q and k of chunk
//                         n + 2, builds P of chunk n + 1 and the per-row decay
//                         vectors of chunk n + 2.
// Each step ends in one barrier.  LDS holds q/k in three slots (n, n + 1,
// n + 2), the T/A blocks and P in two.
#include "chunk_ops.h"
#include "common.h"
#include "kernels.h"

namespace dr {
namespace {

constexpr int kCP = 64;          // chunk length
constexpr int kVTP = 32;         // value columns per workgroup
constexpr int kThreadsP = 256;   // 4 waves
// One 16x16 fp32 diagonal block in LDS: rows of 20 floats (16-byte aligned);
// blocks 16 bytes further apart than 16 rows so that the four blocks read at
// once fall in different banks.
constexpr int kDS = 16 * 20 + 4;

// q/k tiles in LDS: unpadded rows of DK bf16; the 16-byte piece p of row r
// sits in slot p ^ swz(r).  The swizzle keeps both read patterns free of bank
// conflicts within 16 lanes: 16 B from one piece column of 16 consecutive
// rows, and the transpose read (4 consecutive rows x 4 consecutive pieces, 8 B
// from each).  The first needs swz to be one-to-one on r mod 16, the second
// needs rows 4 a .. 4 a + 3 to differ in the bits of swz above the low two.
// For DK = 128 a row spans all 64 banks; for DK = 64 two rows do, so there
// only rows of equal parity can collide.
template <int DK>
__device__ __forceinline__ int swz(int r) {
    if constexpr (DK == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
// element offset of (row r, column col) in a q/k tile; col % 8 + width <= 8
template <int DK>
__device__ __forceinline__ int qk_off(int r, int col) {
    return r * DK + ((((col >> 3) ^ swz<DK>(r))) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// 8-byte LDS transpose read at a per-lane address (see tr_load)
__device__ __forceinline__ bf16x4 tr_read(const uint16_t* p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p)));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves only (no
// LDS-pipe instructions, so nothing here is ordered behind loads into LDS):
// shifts within each 16-lane row, then the last lane of a row is broadcast to
// the rows after it.  DPP controls: row_shr:n = 0x110 + n, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143; lanes without a source read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_move<0x111, 0xf>(x);
    x += dpp_move<0x112, 0xf>(x);
    x += dpp_move<0x114, 0xf>(x);
    x += dpp_move<0x118, 0xf>(x);
    x += dpp_move<0x142, 0xa>(x);
    x += dpp_move<0x143, 0xc>(x);
    return x;
}
// value of x in lane l (wave-uniform result)
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// 16 bytes per lane from global memory straight into LDS: lane l writes bytes
// 16 l .. 16 l + 15 after the wave-uniform address lds.  Completion is counted
// by vmcnt, like any global load.
__device__ __forceinline__ void load_to_lds16(const uint16_t* src, uint16_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds), 16, 0, 0);
}

// Barrier for waves that issued global-to-LDS loads: their data must have
// landed (vmcnt) before other waves may read it.
__device__ __forceinline__ void dma_lds_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


// Empty use that keeps four 8-byte register values (and their registers) live.
__device__ __forceinline__ void keep_alive(const bf16x4 (&v)[4]) {
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
}
__device__ __forceinline__ void keep_alive(uint16_t* const (&v)[4]) {
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
}

template <int DK>
struct LayoutP {
    static constexpr int LDP = kCP + 8;  // bf16 T, P rows
    static constexpr int LDV = 16 + 8;   // bf16 per-wave value / output staging
    static constexpr int QK = kCP * DK * 2;
    static constexpr int MP = kCP * LDP * 2;
    static constexpr int VEC = (9 * kCP + 4) * 4;    // per-row vectors of one chunk
    static constexpr int oQ = 0;                     // [3] slots
    static constexpr int oK = oQ + 3 * QK;           // [3]
    static constexpr int oTe = oK + 3 * QK;          // [2]
    static constexpr int oP = oTe + 2 * MP;          // [2]
    static constexpr int oVec = oP + 2 * MP;         // [3]
    static constexpr int oAd = oVec + 3 * VEC;       // T builder: diagonal A blocks, fp32 [4][kDS]
    static constexpr int oVw = oAd + 4 * kDS * 4;      // chain waves: [2][64][LDV] bf16
    static constexpr int bytes = oVw + 2 * kCP * LDV * 2;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Component-wise select (a whole-vector select of register arrays makes the
// compiler address them through scratch memory).
__device__ __forceinline__ uint4 sel_rows(bool ok, uint4 v) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    bf16x4 r;
    r[0] = static_cast<bf16_t>(x[0]);
    r[1] = static_cast<bf16_t>(x[1]);
    r[2] = static_cast<bf16_t>(x[2]);
    r[3] = static_cast<bf16_t>(x[3]);
    return r;
}

template <int VAR, int DK, int DV>
__global__ __launch_bounds__(kThreadsP) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_pipe_kernel(FwdArgs p) {
    static_assert(VAR == 0 || VAR == 1, "scalar or no decay");
    typedef LayoutP<DK> L;
    constexpr int NVT = DV / kVTP;
    constexpr int NKT = DK / 16;   // 16-wide key-channel tiles
    constexpr int NKK = DK / 32;   // 32-wide k steps

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
    uint16_t* sQs = reinterpret_cast<uint16_t*>(smem + L::oQ);
    uint16_t* sKs = reinterpret_cast<uint16_t*>(smem + L::oK);
    uint16_t* sTes = reinterpret_cast<uint16_t*>(smem + L::oTe);
    uint16_t* sPs = reinterpret_cast<uint16_t*>(smem + L::oP);
    float* sVecs = reinterpret_cast<float*>(smem + L::oVec);
    float* sAd = reinterpret_cast<float*>(smem + L::oAd);
    uint16_t* sVw = reinterpret_cast<uint16_t*>(smem + L::oVw);
    auto qslot = [&](int n) { return sQs + (n % 3) * (L::QK / 2); };
    auto kslot = [&](int n) { return sKs + (n % 3) * (L::QK / 2); };
    auto teslot = [&](int n) { return sTes + (n & 1) * (L::MP / 2); };
    auto pslot = [&](int n) { return sPs + (n & 1) * (L::MP / 2); };
    auto vslot = [&](int n) { return sVecs + (n % 3) * (L::VEC / 4); };
    // vector slot layout: [0,64) beta, [64,128) G (cumulative log-decay),
    // [128,192) e^G, [192,256) e^(G_C - G), [256] gamma = e^G_C,
    // [260,324) u_r = e^(G_r - G_16floor(r/16)), [324 + 64 (R - 1) + j] =
    // w_R[j] = e^(G_16R - G_j) for R = 1..3 (used for j < 16 R), [516,580)
    // beta_r u_r.  For r in block R > J, e^(G_r - G_j) = u_r w_R[j] with both
    // factors in (0, 1].

    // Workgroup -> (head, value tile).  Workgroups are dispatched round-robin
    // over the 8 XCDs.  The NVT tiles of one head get ids 8 apart, so they run
    // on the same XCD and share its L2 for q and k, and each XCD takes a run
    // of consecutive heads: in the [B, T, H, d] layout a head is one fixed
    // d-element column of every token row, and heads that are congruent
    // modulo 8 on one XCD made all of its traffic use the same address bits
    // (those workgroups ran 17% longer).
    const int x = blockIdx.x;
    const int groups = (p.B * p.H + 7) / 8;
    const int vt = (x / 8) % NVT;
    const int bh = (x % 8) * groups + x / (8 * NVT);
    if (bh >= p.B * p.H) return;
    const int b = bh / p.H, h = bh % p.H;
    const int T = p.T, H = p.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int N = (T + kCP - 1) / kCP;
    const int64_t tokb = static_cast<int64_t>(b) * T;
    auto token = [&](int n, int row) -> int64_t {   // clamped to the sequence
        const int t = min(n * kCP + row, T - 1);
        return (tokb + t) * H + h;
    };
    auto rows_in = [&](int n) { return min(kCP, T - n * kCP); };

    // ------------------------------------------------------------------ chain
    if (w < 2) {
        const int vc0 = vt * kVTP + 16 * w;
        uint16_t* sV = sVw + w * kCP * L::LDV;
        // S^T register tiles: tile t, lane (g, c), element i holds value
        // column vc0 + c at key channel 32 (t / 2) + 8 g + 4 (t % 2) + i.  Two
        // tiles paired as one B operand then hold channels 32 q + 8 g .. + 7 at
        // lane (g, c): eight consecutive channels, one 16-byte piece of a key
        // row, so the A operands of X and Y are single 16-byte LDS reads.
        auto chan = [&](int t) { return 32 * (t >> 1) + 8 * g + 4 * (t & 1); };
        f32x4 ST[NKT];
        {
            const float* s0 = p.S0 ? p.S0 + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK : nullptr;
            // (the test outside the loop: a load under a branch inside it was waited
            // for before the next one was issued)
            if (s0) {
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    const float4 v4 = *reinterpret_cast<const float4*>(s0 + chan(t));
                    ST[t] = f32x4{v4.x, v4.y, v4.z, v4.w};
                }
            } else {
#pragma unroll
                for (int t = 0; t < NKT; ++t) ST[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // the initial state has landed before the loop starts: otherwise
            // the wait for it is placed at the top of the loop body, where it
            // also waits for every store and load of the previous step
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        }
        // value prefetch: lane = chunk row, two 16-byte pieces (16 columns)
        uint4 pv0 = make_uint4(0, 0, 0, 0), pv1 = make_uint4(0, 0, 0, 0);
        auto vload = [&](int n) {
            const uint16_t* src = static_cast<const uint16_t*>(p.v) + token(n, lane) * DV + vc0;
            pv0 = *reinterpret_cast<const uint4*>(src);
            pv1 = *reinterpret_cast<const uint4*>(src + 8);
        };
        // A-operand fragments of K and Q for X = K S^T and Y = Q S^T: fragment
        // (m, q) of lane (g, c) holds row 16 m + c, columns 32 q + 8 g .. + 7,
        // the channel order of the S^T tiles paired two by two.
        constexpr int NKP = NKT / 2;
        // lane parts of every LDS address the chain uses (loop invariant)
        int xo[NKP], kto[NKT];
#pragma unroll
        for (int q = 0; q < NKP; ++q) xo[q] = qk_off<DK>(c, 32 * q + 8 * g);
        // transpose reads of K: within a 16-lane group, lane i receives element
        // i % 4 of the 8-byte piece addressed by lane 4 j + i / 4, j = 0..3.
        // Lane (g, c) points at row r0 + 4 g + c / 4, columns
        // 32 (t / 2) + 8 (c % 4) + 4 (t % 2) .. + 3, so lane c receives rows
        // r0 + 4 g .. + 3 of the channel that row c of S^T tile t holds (r0 a
        // multiple of 16 leaves the swizzle unchanged).
#pragma unroll
        for (int t = 0; t < NKT; ++t) kto[t] = qk_off<DK>(4 * g + (c >> 2), 32 * (t >> 1) + 8 * (c & 3) + 4 * (t & 1));
        const int tpo = c * L::LDP + 4 * g;                       // T, P rows
        const int vvo = (4 * g + (c >> 2)) * L::LDV + 4 * (c & 3);  // value tile, transposed
        // Operands of chunk n that are complete one step before chunk n is
        // processed (q, k, the per-row vectors and the wave's own value tile)
        // are read during the step before it, each group right after the
        // last use of the registers it refills, so the reads overlap that
        // step's products.  T and P of chunk n are built during that step
        // and are read at the start of step n.
        bf16x8 kx[4][NKP], qx[4][NKP];   // A operands of X = K S^T, Y = Q S^T
        bf16x8 kt[NKT][2];               // K^T fragments for the state update
        f32x4 bt[4], eg[4], egc[4];
        float egr[4];                    // e^G of row 16 m + c (outputs are kept transposed)
        float gam = 1.f;
        bf16x4 vv[4];                    // value tile in accumulator layout (rows 4 g + i, column c)
        auto read_xy = [&](int n) {
            const uint16_t* sK = kslot(n);
            const uint16_t* sQ = qslot(n);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int q = 0; q < NKP; ++q) {
                    const int rb = 16 * m * DK;
                    kx[m][q] = *reinterpret_cast<const bf16x8*>(sK + rb + xo[q]);
                    qx[m][q] = *reinterpret_cast<const bf16x8*>(sQ + rb + xo[q]);
                }
            }
        };
        // value tile and the vectors of the R epilogue
        auto read_rv = [&](int n) {
            const bool ok = lane < rows_in(n);
            // commit the value tile of chunk n to the wave's staging area
            *reinterpret_cast<uint4*>(sV + lane * L::LDV) = sel_rows(ok, pv0);
            *reinterpret_cast<uint4*>(sV + lane * L::LDV + 8) = sel_rows(ok, pv1);
            if (n + 1 < N) vload(n + 1);
            const float* vec = vslot(n);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bt[m] = *reinterpret_cast<const f32x4*>(vec + 16 * m + 4 * g);
                eg[m] = *reinterpret_cast<const f32x4*>(vec + 128 + 16 * m + 4 * g);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) vv[m] = tr_read(sV + 16 * m * L::LDV + vvo);
        };
        auto read_kt = [&](int n) {
            const uint16_t* sK = kslot(n);
            const float* vec = vslot(n);
#pragma unroll
            for (int m = 0; m < 4; ++m) egc[m] = *reinterpret_cast<const f32x4*>(vec + 192 + 16 * m + 4 * g);
            gam = vec[256];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    kt[t][q] = cat(tr_read(sK + 32 * q * DK + kto[t]), tr_read(sK + (32 * q + 16) * DK + kto[t]));
            }
        };
        auto read_egr = [&](int n) {
            const float* vec = vslot(n);
#pragma unroll
            for (int m = 0; m < 4; ++m) egr[m] = vec[128 + 16 * m + c];
        };
        const bf16x4 z4 = {0, 0, 0, 0};
        bf16x4 od[4] = {z4, z4, z4, z4};   // output rows being stored
        uint16_t* oad[4] = {nullptr, nullptr, nullptr, nullptr};   // and their addresses
        for (int s = -2; s < N; ++s) {
            if (s >= 0) {
                const int Cn = rows_in(s);
                const uint16_t* Te = teslot(s);
                const uint16_t* Pm = pslot(s);
                // diagonal blocks T_mm and off-diagonal blocks A_mJ (lane
                // (g, c): row 16 m + c, columns 16 J + 4 g .. + 3) and the
                // lower-triangular rows of P, as A operands: row 16 m + c,
                // column tiles paired (0, 1) and (2, 3); an unpaired tile is
                // padded with zeros
                bf16x4 td[4], Ab[4][3];
                bf16x8 pf[4][2];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    td[m] = *reinterpret_cast<const bf16x4*>(Te + 16 * m * L::LDP + 16 * m + tpo);
#pragma unroll
                    for (int J = 0; J < m; ++J) Ab[m][J] = *reinterpret_cast<const bf16x4*>(Te + 16 * m * L::LDP + 16 * J + tpo);
#pragma unroll
                    for (int q = 0; q <= m / 2; ++q) {
                        const int off = 16 * m * L::LDP + 32 * q + tpo;
                        const bool two = 2 * q + 1 <= m;
                        const bf16x4 p0 = *reinterpret_cast<const bf16x4*>(Pm + off);
                        pf[m][q] = cat(p0, two ? *reinterpret_cast<const bf16x4*>(Pm + off + 16) : z4);
                    }
                }
                // ---- X = K S^T (accumulator layout), Y = Q S^T (transposed:
                // swapping the operands makes lane (g, c) hold row 16 m + c,
                // value columns 4 g .. + 3)
                bf16x8 STp[NKP];
#pragma unroll
                for (int q = 0; q < NKP; ++q) STp[q] = cat(to_bf16x4(ST[2 * q]), to_bf16x4(ST[2 * q + 1]));
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                f32x4 X[4], Yt[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    X[m] = zero;
                    Yt[m] = zero;
                }
#pragma unroll
                for (int q = 0; q < NKP; ++q) {
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        X[m] = mfma32(kx[m][q], STp[q], X[m]);
                        Yt[m] = mfma32(STp[q], qx[m][q], Yt[m]);
                    }
                }
                // (at the last step these read slots that nothing writes any more)
                read_xy(s + 1);
                // ---- R = beta (V - e^G X);  V~ = (I + A)^-1 R by block forward
                // substitution: V~_J = T_JJ (R_J - sum_{M<J} A_JM V~_M)
                f32x4 Rf[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) Rf[m][i] = bt[m][i] * (static_cast<float>(vv[m][i]) - eg[m][i] * X[m][i]);
                }
                read_rv(s + 1);
                f32x4 Vt[4];
                bf16x4 Vtr[4], Vgr[4];
                Vt[0] = mfma32(cat(td[0], z4), cat(to_bf16x4(Rf[0]), z4), zero);
                Vtr[0] = to_bf16x4(Vt[0]);
                const f32x4 y1 = mfma32(cat(Ab[1][0], z4), cat(Vtr[0], z4), zero);
                Vt[1] = mfma32(cat(td[1], z4), cat(to_bf16x4(Rf[1] - y1), z4), zero);
                Vtr[1] = to_bf16x4(Vt[1]);
                const bf16x8 V01 = cat(Vtr[0], Vtr[1]);
                const f32x4 y2 = mfma32(cat(Ab[2][0], Ab[2][1]), V01, zero);
                f32x4 y3 = mfma32(cat(Ab[3][0], Ab[3][1]), V01, zero);
                Vt[2] = mfma32(cat(td[2], z4), cat(to_bf16x4(Rf[2] - y2), z4), zero);
                Vtr[2] = to_bf16x4(Vt[2]);
                y3 = mfma32(cat(Ab[3][2], z4), cat(Vtr[2], z4), y3);
                Vt[3] = mfma32(cat(td[3], z4), cat(to_bf16x4(Rf[3] - y3), z4), zero);
                Vtr[3] = to_bf16x4(Vt[3]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    f32x4 vg;
#pragma unroll
                    for (int i = 0; i < 4; ++i) vg[i] = egc[m][i] * Vt[m][i];
                    Vgr[m] = to_bf16x4(vg);
                }
                // ---- S^T <- gamma S^T + K^T (e^(G_C - G) V~)
                const bf16x8 Vg01 = cat(Vgr[0], Vgr[1]), Vg23 = cat(Vgr[2], Vgr[3]);
#pragma unroll
                for (int t = 0; t < NKT; ++t) ST[t] = mfma32(kt[t][1], Vg23, mfma32(kt[t][0], Vg01, ST[t] * gam));
                read_kt(s + 1);
                // ---- O = e^G Y + P V~, transposed like Y
                const bf16x8 V2z = cat(Vtr[2], z4), V23 = cat(Vtr[2], Vtr[3]), V0z = cat(Vtr[0], z4);
                f32x4 Ot[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) Ot[m] = Yt[m] * egr[m];
                read_egr(s + 1);
                Ot[0] = mfma32(V0z, pf[0][0], Ot[0]);
                Ot[1] = mfma32(V01, pf[1][0], Ot[1]);
                Ot[2] = mfma32(V2z, pf[2][1], mfma32(V01, pf[2][0], Ot[2]));
                Ot[3] = mfma32(V23, pf[3][1], mfma32(V01, pf[3][0], Ot[3]));
                // The registers that feed the global stores (data and address)
                // stay reserved until the next step refills them (empty asm
                // use): overwriting a store's source register earlier makes the
                // compiler wait for the store to complete.
                keep_alive(od);
                keep_alive(oad);
                uint16_t* orow = static_cast<uint16_t*>(p.o) + token(s, c) * DV + vc0 + 4 * g;
                const int64_t mstride = static_cast<int64_t>(16) * H * DV;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    od[m] = to_bf16x4(Ot[m]);
                    oad[m] = orow + m * mstride;
                    if (16 * m + c < Cn) *reinterpret_cast<bf16x4*>(oad[m]) = od[m];
                }
            }
            if (s == -1) {
                vload(0);
                read_xy(0);
                read_rv(0);
                read_kt(0);
                read_egr(0);
            }
            lds_barrier();
        }
        if (p.ST) {
            float* st = p.ST + (static_cast<int64_t>(bh) * DV + vc0 + c) * DK;
#pragma unroll
            for (int t = 0; t < NKT; ++t)
                *reinterpret_cast<float4*>(st + chan(t)) =
                    make_float4(ST[t][0], ST[t][1], ST[t][2], ST[t][3]);
        }
        return;
    }

    // ------------------------------------------------- key side (waves 2, 3)
    // Wave 3 stages q, k, beta and g of chunk n + 2 at the start of a step (so
    // the loads get the whole step to land) and builds P of chunk n + 1; wave
    // 2 builds A and T of chunk n + 1.  q and k go straight from HBM into LDS
    // (global_load_lds: lane l of instruction j fills bytes 1024 j + 16 l of
    // the slot, so each lane fetches the piece that the swizzle puts there);
    // no registers are held and no LDS write instructions are spent on them.
    // Rows past the end of the sequence hold copies of its last token: their
    // beta is zero, which removes them from every product that reaches an
    // output or the state.
    const bool lw = (w == 3);   // loader and P builder; wave 2 builds T
    // (A prefetch of chunk n + 3 into L2 by 4-byte loads, one per 128-byte
    // line, made every workgroup of heads h = 1 mod 4 about 18% slower with
    // cold inputs, and the whole kernel with it; the loads are not issued.)
    uint16_t pbeta = 0, pg = 0;
    // Per-lane element offsets of the pieces this lane fetches, relative to
    // the first token of a chunk (32-bit; computed once).
    constexpr int RPI = 512 / DK;   // rows per 1 KB instruction
    constexpr int PPR = DK / 8;     // 16-byte pieces per row
    constexpr int NJ = kCP / RPI;   // instructions per tile
    // q and k rows: value heads share a query/key head in groups of H / Hk
    const int Hk = p.Hk, hk = h / (H / Hk);
    uint32_t qk_lane_off[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = j * RPI + lane / PPR;
        qk_lane_off[j] = static_cast<uint32_t>(r * Hk * DK + 8 * ((lane % PPR) ^ swz<DK>(r)));
    }
    auto load_tile = [&](const uint16_t* src, uint16_t* dst, int n) {
        if (n * kCP + kCP <= T) {   // whole chunk: wave-uniform base + lane offset
            const uint16_t* base = src + ((tokb + n * kCP) * Hk + hk) * DK;
#pragma unroll
            for (int j = 0; j < NJ; ++j) load_to_lds16(base + qk_lane_off[j], dst + 512 * j);
        } else {                    // last, partial chunk: rows clamped to the sequence
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int r = j * RPI + lane / PPR;
                const int piece = (lane % PPR) ^ swz<DK>(r);
                const int64_t tq = (tokb + min(n * kCP + r, T - 1)) * Hk + hk;
                load_to_lds16(src + tq * DK + 8 * piece, dst + 512 * j);
            }
        }
    };
    auto load_vec = [&](int n) {
        pbeta = static_cast<const uint16_t*>(p.beta)[token(n, lane)];
        if constexpr (VAR == 1) pg = static_cast<const uint16_t*>(p.g)[token(n, lane)];
    };
    auto commit_vec = [&](int n) {   // per-row vectors of chunk n
        const int Cn = rows_in(n);
        float* vec = vslot(n);
        const bool ok = lane < Cn;
        const float beta = ok ? bf16_bits_to_f32(pbeta) : 0.f;
        float G = 0.f;
        if constexpr (VAR == 1) G = wave_prefix_sum(ok ? bf16_bits_to_f32(pg) : 0.f);
        // G at lanes 0, 16, 32, 48 (block starts) and 63 (chunk end)
        const float G0 = lane_value(G, 0), G16 = lane_value(G, 16), G32 = lane_value(G, 32),
                    G48 = lane_value(G, 48), GC = lane_value(G, 63);
        const float Gb = lane < 16 ? G0 : lane < 32 ? G16 : lane < 48 ? G32 : G48;
        vec[lane] = beta;
        vec[64 + lane] = G;
        vec[128 + lane] = VAR == 0 ? 1.f : __expf(G);
        vec[192 + lane] = VAR == 0 ? 1.f : __expf(GC - G);
        if (lane == 0) vec[256] = VAR == 0 ? 1.f : __expf(GC);
        vec[260 + lane] = VAR == 0 ? 1.f : __expf(G - Gb);
        vec[324 + lane] = VAR == 0 ? 1.f : __expf(G16 - G);
        vec[388 + lane] = VAR == 0 ? 1.f : __expf(G32 - G);
        vec[452 + lane] = VAR == 0 ? 1.f : __expf(G48 - G);
        vec[516 + lane] = VAR == 0 ? beta : beta * __expf(G - Gb);
    };
    // A-operand fragment: lane (g, c) holds row 16 R + c, columns 32 kk + 8 g .. + 7
    auto frag = [&](const uint16_t* tile, int Rt, int kk) {
        const int r = 16 * Rt + c;
        return *reinterpret_cast<const bf16x8*>(tile + qk_off<DK>(r, 32 * kk + 8 * g));
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    for (int s = -2; s < N; ++s) {
        const int nl = s + 2;   // chunk staged during this step
        const int nb = s + 1;   // chunk whose T (wave 2) or P (wave 3) is built now
        if (lw && nl < N) {     // stage chunk nl: the loads get the whole step to land
            load_vec(nl);
            load_tile(static_cast<const uint16_t*>(p.k), kslot(nl), nl);
            load_tile(static_cast<const uint16_t*>(p.q), qslot(nl), nl);
        }
        if (nb >= 0 && nb < N) {
            const float* vec = vslot(nb);
            bf16x8 kf[4][NKK];
#pragma unroll
            for (int Rt = 0; Rt < 4; ++Rt) {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) kf[Rt][kk] = frag(kslot(nb), Rt, kk);
            }
            // per-row vectors of chunk nb: rows 16 R + c and rows 16 R + 4 g .. + 3
            float gc[4];
            f32x4 gr[4], wv[4][3];   // wv[R][J] = w_R[16 J + 4 g .. + 3]
#pragma unroll
            for (int Rt = 0; Rt < 4; ++Rt) {
                gc[Rt] = vec[64 + 16 * Rt + c];
                gr[Rt] = *reinterpret_cast<const f32x4*>(vec + 64 + 16 * Rt + 4 * g);
#pragma unroll
                for (int Jt = 0; Jt < Rt; ++Jt)
                    wv[Rt][Jt] = *reinterpret_cast<const f32x4*>(vec + 324 + 64 * (Rt - 1) + 16 * Jt + 4 * g);
            }
            if (!lw) {
                // ---- diagonal blocks of A: K_R K_R^T in accumulator layout
                // (rows 4 g + i, column c), scaled and masked to A_RR, stored
                // column-major (sAd[R][col][row]: one 16-byte piece per lane)
#pragma unroll
                for (int Rt = 0; Rt < 4; ++Rt) {
                    const f32x4 br = *reinterpret_cast<const f32x4*>(vec + 16 * Rt + 4 * g);
                    f32x4 acc = zero;
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) acc = mfma32(kf[Rt][kk], kf[Rt][kk], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float val = acc[i] * br[i];
                        if constexpr (VAR == 1) val *= __expf(gr[Rt][i] - gc[Rt]);
                        acc[i] = (4 * g + i > c) ? val : 0.f;
                    }
                    *reinterpret_cast<f32x4*>(sAd + Rt * kDS + c * 20 + 4 * g) = acc;
                }
                // ---- diagonal blocks of T by backward substitution on the
                // transposed system: lane (block rb, j) solves (I + A_bb)^T y = e_j,
                // which gives row j of T_bb = (I + A_bb)^-1:
                //   y_i = [i == j] - Σ_{m > i} A[m][i] y_m,  i = 15 .. 0
                const int rb = lane >> 4, j = lane & 15;
                const float* Ab = sAd + rb * kDS;
                f32x4 col[16][4];
#pragma unroll
                for (int i = 0; i < 15; ++i) {
#pragma unroll
                    for (int q = (i + 1) / 4; q < 4; ++q) col[i][q] = *reinterpret_cast<const f32x4*>(Ab + i * 20 + 4 * q);
                }
                // ---- off-diagonal blocks of A, computed while the columns are
                // in flight.  Swapping the two operands of K_J K_R^T leaves lane
                // (g, c) with A[16 R + c][16 J + 4 g + i], the A-operand layout
                // of the chain's block substitution; they are stored below the
                // diagonal blocks of T in the same slot (one 8-byte write each).
                uint16_t* Tm = teslot(nb);
#pragma unroll
                for (int Rt = 1; Rt < 4; ++Rt) {
                    const float fr = vec[516 + 16 * Rt + c];   // beta_r u_r
#pragma unroll
                    for (int Jt = 0; Jt < Rt; ++Jt) {
                        f32x4 acc = zero;
#pragma unroll
                        for (int kk = 0; kk < NKK; ++kk) acc = mfma32(kf[Jt][kk], kf[Rt][kk], acc);
                        // beta_r e^(G_r - G_j) = (beta_r u_r) w_R[j]
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= fr * wv[Rt][Jt][i];
                        *reinterpret_cast<bf16x4*>(Tm + (16 * Rt + c) * L::LDP + 16 * Jt + 4 * g) = to_bf16x4(acc);
                    }
                }
                // column-oriented: once y_m is final it is subtracted from every
                // y_i, i < m, so each level is 15 - m independent FMAs rather
                // than one chain of 120 dependent ones
                float y[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) y[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 15; m >= 1; --m) {
#pragma unroll
                    for (int i = 0; i < m; ++i) y[i] -= col[i][m / 4][m % 4] * y[m];
                }
                // bf16 diagonal block of T: row j of block rb, 16 columns
                uint16_t* Te = teslot(nb) + (16 * rb + j) * L::LDP + 16 * rb;
                uint32_t hw[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    hw[2 * q] = static_cast<uint32_t>(f32_to_bf16_bits(y[4 * q])) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(y[4 * q + 1])) << 16);
                    hw[2 * q + 1] = static_cast<uint32_t>(f32_to_bf16_bits(y[4 * q + 2])) |
                                    (static_cast<uint32_t>(f32_to_bf16_bits(y[4 * q + 3])) << 16);
                }
                // written through a float vector type: type-based alias analysis
                // then separates these stores from the global-to-LDS loads in
                // flight (they target q/k slots), so no wait for them is inserted
                *reinterpret_cast<f32x4*>(Te) = __builtin_bit_cast(f32x4, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                *reinterpret_cast<f32x4*>(Te + 8) = __builtin_bit_cast(f32x4, make_uint4(hw[4], hw[5], hw[6], hw[7]));
            } else {
                // ---- P = Tril(Q K^T ⊙ Gamma), transposed products: lane (g, c)
                // holds P[16 R + c][16 J + 4 g + i] and writes it as one 8-byte piece
                bf16x8 qf[4][NKK];
#pragma unroll
                for (int Rt = 0; Rt < 4; ++Rt) {
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) qf[Rt][kk] = frag(qslot(nb), Rt, kk);
                }
                float uc[4];
#pragma unroll
                for (int Rt = 0; Rt < 4; ++Rt) uc[Rt] = vec[260 + 16 * Rt + c];
                uint16_t* Pm = pslot(nb);
#pragma unroll
                for (int Rt = 0; Rt < 4; ++Rt) {
#pragma unroll
                    for (int Jt = 0; Jt <= Rt; ++Jt) {
                        f32x4 acc = zero;
#pragma unroll
                        for (int kk = 0; kk < NKK; ++kk) acc = mfma32(kf[Jt][kk], qf[Rt][kk], acc);
                        if (Jt < Rt) {   // e^(G_r - G_j) = u_r w_R[j]
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[i] *= uc[Rt] * wv[Rt][Jt][i];
                        } else {         // diagonal block: masked, exact exponent
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float val = acc[i];
                                if constexpr (VAR == 1) val *= __expf(gc[Rt] - gr[Jt][i]);
                                acc[i] = (c >= 4 * g + i) ? val : 0.f;
                            }
                        }
                        *reinterpret_cast<bf16x4*>(Pm + (16 * Rt + c) * L::LDP + 16 * Jt + 4 * g) = to_bf16x4(acc);
                    }
                }
            }
        }
        if (lw && nl < N) commit_vec(nl);
        dma_lds_barrier();
    }
}

template <int VAR, int DK, int DV>
hipError_t launch_pipe_one(const FwdArgs& a, hipStream_t s) {
    constexpr int NVT = DV / kVTP;
    const int groups = (a.B * a.H + 7) / 8;
    const dim3 grid(static_cast<unsigned>(groups) * 8u * NVT);
    hipLaunchKernelGGL((prefill_pipe_kernel<VAR, DK, DV>), grid, dim3(kThreadsP), 0, s, a);
    return hipGetLastError();
}

template <int VAR>
hipError_t launch_pipe_dims(const FwdArgs& a, hipStream_t s) {
    if (a.dk == 128 && a.dv == 128) return launch_pipe_one<VAR, 128, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch_pipe_one<VAR, 128, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch_pipe_one<VAR, 64, 128>(a, s);
    return launch_pipe_one<VAR, 64, 64>(a, s);
}

}  // namespace

hipError_t launch_fwd_pipelined(int variant, const FwdArgs& a, hipStream_t s) {
    return variant == 0 ? launch_pipe_dims<0>(a, s) : launch_pipe_dims<1>(a, s);
}

}  // namespace dr
