// Internal launcher interface between the C ABI (abi.hip) and the kernels.
// Arguments have been validated by the caller; launchers only pick a template
// instance, size the grid and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

struct FwdArgs {
    int B, T, H, dk, dv;
    const void* q;
    const void* k;
    const void* v;
    const void* beta;   // beta [B,T,H], or [B,T,H,dk]: the erase gate (split gates)
                        // or the step size per key channel (keywrite)
    const void* wgate;  // write gate [B,T,H,dv] (split gates) or nullptr
    const void* g;      // log-decay: nullptr, [B,T,H] or [B,T,H,dk]
    const float* S0;    // [B,H,dv,dk] or nullptr (zero state)
    void* o;            // [B,T,H,dv]
    float* ST;          // [B,H,dv,dk] or nullptr
    int Hk;             // query/key heads (divides H): q, k are [B,T,Hk,dk] and
                        // value head h reads query/key head h / (H / Hk)
    int keywrite = 0;   // channel-decay kernels: 1 = FG^2-GDN, the residual is
                        // written along E = beta ⊙ k and there is no write gate
                        // (the split form with W = V, A_k = A_e, M_k = M_e, Kb = Eb,
                        // or the one-step-size form with E on the key side)
    void* ws = nullptr; // device workspace of fwd_workspace_bytes() bytes (256-byte
                        // aligned) when that is not zero
};

struct DecodeArgs {
    int B, H, dk, dv;
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const void* wgate;
    const void* g;
    float* S;  // [B,H,dv,dk], in place
    void* o;   // [B,H,dv]
    int Hk;    // query/key heads (divides H): q, k are [B,Hk,dk]
};

struct EflaArgs {
    int B, T, H, Hk, dk;
    const void* k;     // [B,T,Hk,dk]
    const void* beta;  // [B,T,H]
    void* beta_eff;    // [B,T,H]; may equal beta
};

struct BwdArgs {
    int B, T, H, dk, dv;
    const void* q;       // [B,T,H,dk]
    const void* k;
    const void* v;       // [B,T,H,dv]
    const void* beta;    // [B,T,H]
    const void* g;       // nullptr, [B,T,H] or [B,T,H,dk]
    const float* S0;     // [B,H,dv,dk] or nullptr
    const void* dO;      // [B,T,H,dv]
    const float* dST;    // [B,H,dv,dk] or nullptr
    void* gq;            // gradients, same layouts as the inputs
    void* gk;
    void* gv;
    void* gbeta;
    void* gg;            // nullptr for the ungated form
    float* gS0;          // [B,H,dv,dk] or nullptr
    const void* wgate;   // split gates: write gate [B,T,H,dv] (beta is then the
    void* gw;            // erase gate [B,T,H,dk]) and its gradient; else nullptr
    int Hk;              // query/key heads (divides H); q, k, dq, dk are [B,T,Hk,dk]
    float* gq32;         // grouped heads only: per-value-head dq, dk [B,T,H,dk] fp32,
    float* gk32;         // summed over each group into gq, gk afterwards; else nullptr
    void* ws = nullptr;  // device workspace of bwd_workspace_bytes() bytes (256-byte aligned)
};

// variant: 0 ungated, 1 scalar decay, 2 channel decay, 3 split gates,
// 4 a step size per key channel (FG^2-GDN).  dtype: 0 fp32, 1 bf16.
//
// Device workspace of each entry point in bytes (0 when it needs none).  The
// caller allocates it; the launchers carve it into 256-byte aligned pieces.
size_t fwd_workspace_bytes(int variant, int dtype, int B, int T, int H, int dk, int dv);
size_t bwd_workspace_bytes(int variant, int B, int T, int H, int Hk, int dk, int dv);
size_t ttt_workspace_bytes(int dtype, int B, int T, int H, int dk, int dv);
inline size_t round_up_256(size_t n) { return (n + 255) / 256 * 256; }

hipError_t launch_fwd(int variant, int dtype, const FwdArgs& a, hipStream_t stream);
// software-pipelined bf16 kernel for variants 0 and 1, called by launch_fwd
hipError_t launch_fwd_pipelined(int variant, const FwdArgs& a, hipStream_t stream);
// fp32 operands, products as three bf16 terms of split operands (variants 0, 1)
hipError_t launch_fwd_split(int variant, const FwdArgs& a, hipStream_t stream);
// channel-wise decay forms (variant 2 or 3), called by launch_fwd
hipError_t launch_fwd_channel(int variant, int dtype, const FwdArgs& a, hipStream_t stream);
// channel-wise decay forms with bf16 operands, two passes (state-independent
// operands of every sub-chunk first, then the recurrence), called by
// launch_fwd_channel
hipError_t launch_fwd_channel_two_pass(int variant, const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode(int variant, int dtype, const DecodeArgs& a, hipStream_t stream);
// exact-flow step sizes (dtype 0 fp32, 1 bf16)
hipError_t launch_efla_beta(int dtype, const EflaArgs& a, hipStream_t stream);
// backward of every form (variant 0 .. 3)
hipError_t launch_bwd(int variant, int dtype, const BwdArgs& a, hipStream_t stream);

// DeltaTTT-pre: two chained delta-rule memory layers (variant 0 or 1 for both)
struct TttArgs {
    int B, T, H, dk, dv;
    const void* q;       // [B,T,H,dk]
    const void* k;
    const void* v;       // [B,T,H,dv]
    const void* beta1;   // [B,T,H] first layer
    const void* g1;      // [B,T,H] or nullptr
    const void* beta2;   // [B,T,H] second layer
    const void* g2;      // [B,T,H] or nullptr
    const float* A0;     // [B,H,dv,dk] or nullptr
    const float* B0;     // [B,H,dv,dv] or nullptr
    void* o;             // [B,T,H,dv]
    float* AT;           // [B,H,dv,dk] or nullptr (may equal A0)
    float* BT;           // [B,H,dv,dv] or nullptr (may equal B0)
    void* ws = nullptr;  // device workspace of ttt_workspace_bytes() bytes
    // pieces of the workspace (set by the launcher)
    void* qs = nullptr;  // [B,T,H,dk] shifted queries a1 ⊙ k of the next token
    void* rd = nullptr;  // [B,T,H,dv] their readouts: pre-write reads of tokens 1..T
    void* r0 = nullptr;  // [B,H,dv] pre-write read of token 0
    void* o1 = nullptr;  // [B,T,H,dv] first-layer readout after the write
    void* hk = nullptr;  // [B,T,H,dv] second-layer write keys
    void* zq = nullptr;  // [B,T,H,dv] second-layer queries
};
hipError_t launch_ttt_pre(int variant, int dtype, const TttArgs& a, hipStream_t stream);

}  // namespace dr
