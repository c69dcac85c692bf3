/*
 * deltarule.h — C ABI of the MI355X (gfx950) gated delta-rule library.
 *
 * The library evaluates the delta-rule recurrence of a linear matrix memory
 * S (d_v rows, d_k columns, fp32) over a sequence of tokens.  For token t with
 * query q_t, key k_t (d_k), value v_t (d_v) and decay a_t = exp(g_t):
 *
 *   S' = S · Diag(a_t)                         decay the key columns
 *   r  = S' k_t                                read the memory at the key
 *   S  = S' + beta_t (v_t - r) k_t^T           DR_DELTANET, DR_GDN, DR_KDA
 *   S  = S' - r (b_t ⊙ k_t)^T + (w_t ⊙ v_t) k_t^T      DR_GDN2
 *   S  = S' + (v_t - r) (beta_t ⊙ k_t)^T                 DR_FG2 (beta_t per key channel)
 *   o_t = S q_t                                readout after the write
 *
 * Sources (web pages):
 *  - delta rule = one serial gradient step of a linear memory on
 *    1/2 ||S k - v||^2, read before write: "DeltaTTT: Layerwise Optimization
 *    for Nonlinear Recurrent Memory" summary (paperlayer.ai), §2 Background,
 *    §4.1; "Gated DeltaNet-2" abstract (thelatestinai.com/papers/2607.07953);
 *  - scalar head-wise decay (Gated DeltaNet) and channel-wise decay (Kimi
 *    Delta Attention): "Delta-Rule Linear Attention" topic page, FG^2-GDN card;
 *  - split channel-wise erase gate b_t and write gate w_t, reducing to KDA when
 *    both are the same scalar: Gated DeltaNet-2 abstract.  The placement of b on
 *    the key side of the erase term is this library's reading of that abstract;
 *  - a channel-wise step size (FG^2-GDN): "Delta-Rule Linear Attention" topic
 *    page, FG^2-GDN card, which likens it to per-coordinate optimizers.  Taking
 *    the key channels as the coordinates of the gradient step on
 *    1/2 ||S' k - v||^2 gives the DR_FG2 line above, which equals DR_KDA when
 *    beta_t is a constant vector; that choice of axis is this library's reading.
 *    The card's FG^2-GDN+ (separate key-side erase and value-side write scales)
 *    is DR_GDN2;
 *  - the update is affine in the previous memory, so chunks of tokens can be
 *    evaluated in parallel (DeltaTTT summary, §2), by a chunkwise WY algorithm
 *    with channel-wise decay absorbed into the erase factors (Gated DeltaNet-2
 *    abstract): that is how delta_fwd evaluates it;
 *  - decode is one read and one write pass over each state matrix per token
 *    ("Delta-Rule Linear Attention" topic page, GDN FPGA decode card).
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers on the current HIP device, dense
 *    and row-major with the shapes given below (no strides).  Every pointer
 *    must be 16-byte aligned.  The caller owns every buffer, and no per-call
 *    state is kept.  The library allocates no device memory.
 *  - Workspace.  delta_fwd (channel-wise decay forms with DR_BF16 operands),
 *    delta_bwd and delta_ttt_pre need temporary device memory, which the caller
 *    passes as (workspace, workspace_bytes).  The matching *_workspace_bytes
 *    query returns the size for a descriptor (0 when none is needed; then
 *    workspace may be NULL).  A needed workspace must be 256-byte aligned, at
 *    least that large (DR_E_WORKSPACE otherwise) and disjoint from every tensor
 *    argument (DR_E_ALIAS).  Its contents on entry do not matter and are
 *    undefined on return; calls that share one workspace must be ordered (one
 *    stream, or events), otherwise they race.
 *  - dtype (dr_desc.dtype) is the element type of q, k, v, beta, wgate, g and
 *    o.  The state (S0, S_T, S) is always fp32.
 *  - The stream argument is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous: they enqueue kernels and return without synchronising.
 *  - Every argument is validated on the host before any HIP call.  Errors are
 *    returned as a dr_status and never abort; C++ exceptions never cross the
 *    ABI.  On an error nothing has been enqueued and no output was touched.
 *  - Results are deterministic: no atomics, fixed reduction order.
 *  - Supported sizes: d_k, d_v in {64, 128}; chunk = 64; any T >= 1 (the
 *    last chunk is masked when T is not a multiple of 64).  Limits (DR_E_SHAPE
 *    beyond them): B * T * H <= 2^34, B * H <= 2^20, B * H * ceil(T / 64)
 *    <= 2^22 and H <= 2^18 - 1, which keep every grid and every 32-bit offset
 *    inside a chunk within range.
 */
#ifndef DELTARULE_H
#define DELTARULE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DR_ABI_VERSION 5

typedef enum {
    DR_DELTANET = 0, /* a = 1: no decay, g must be NULL                          */
    DR_GDN = 1,      /* scalar decay per (token, head): g is [B,T,H]             */
    DR_KDA = 2,      /* channel-wise decay: g is [B,T,H,d_k]                     */
    DR_GDN2 = 3,     /* channel-wise decay + erase gate b + write gate w         */
    DR_FG2 = 4       /* channel-wise decay + step size per key channel (FG^2-GDN) */
} dr_variant;

typedef enum { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;

typedef enum {
    DR_OK = 0,
    DR_E_NULLPTR = 1,     /* a required pointer (or the descriptor) is NULL       */
    DR_E_SHAPE = 2,       /* a size is out of range (B, T, H < 1, decode T != 1,
                             H_k < 0, H_k > H or H_k not dividing H, or beyond
                             the limits stated above)                           */
    DR_E_UNSUPPORTED = 3, /* unknown variant/dtype, unsupported d_k/d_v/chunk, or
                             a pointer given that the variant does not take     */
    DR_E_ALIGN = 4,       /* a pointer is not 16-byte aligned (the workspace: not
                             256-byte aligned)                                  */
    DR_E_DEVICE = 5,      /* no HIP device, or the current device is not gfx950   */
    DR_E_LAUNCH = 6,      /* the kernel launch failed (hipGetLastError)           */
    DR_E_ALIAS = 7,       /* an output overlaps an input it may not alias, or the
                             workspace overlaps a tensor argument                */
    DR_E_WORKSPACE = 8    /* workspace NULL or smaller than the size query says  */
} dr_status;

typedef struct {
    int32_t B;       /* batch                                                  */
    int32_t T;       /* tokens per sequence (1 for delta_decode)               */
    int32_t H;       /* heads                                                  */
    int32_t d_k;     /* key/query width                                        */
    int32_t d_v;     /* value width                                            */
    int32_t chunk;   /* chunk length of the chunkwise evaluation; must be 64   */
    int32_t variant; /* dr_variant                                             */
    int32_t dtype;   /* dr_dtype                                               */
    int32_t H_k;     /* query/key heads; 0 means H.  Otherwise H_k must divide
                        H: q and k are [.., H_k, d_k] and value head h reads
                        query/key head h / (H / H_k), so each group of H / H_k
                        consecutive value heads shares one query/key head
                        (Grouped Value Attention: "Delta-Rule Linear Attention"
                        topic page, GDN FPGA decode card).  beta, wgate, g, o
                        and the state stay per value head (H).                 */
} dr_desc;

/*
 * delta_fwd — chunkwise-parallel forward pass over whole sequences.
 *
 *   q, k   [B, T, H_k, d_k] dtype (H_k = H unless desc->H_k says otherwise)
 *   v      [B, T, H, d_v]   dtype
 *   beta   DR_DELTANET/GDN/KDA: step size beta [B, T, H];
 *          DR_GDN2: erase gate b [B, T, H, d_k];
 *          DR_FG2: step size per key channel [B, T, H, d_k]              dtype
 *   wgate  DR_GDN2: write gate w [B, T, H, d_v]; otherwise must be NULL  dtype
 *   g      log-decay log(a) <= 0: DR_DELTANET must be NULL; DR_GDN
 *          [B, T, H]; DR_KDA/DR_GDN2/DR_FG2 [B, T, H, d_k]                dtype
 *   S0     initial state [B, H, d_v, d_k] fp32; NULL means zero
 *   o      output [B, T, H, d_v] dtype (written); must not overlap any input
 *   S_T    final state [B, H, d_v, d_k] fp32 (written); NULL if not wanted;
 *          may be the same pointer as S0 (in-place update) but must not
 *          otherwise overlap an input
 *
 *   workspace, workspace_bytes
 *          device workspace of at least delta_fwd_workspace_bytes(desc) bytes
 *          (see the conventions above); NULL and 0 when that is 0.  Only the
 *          channel-wise forms with DR_BF16 operands use one: B * H * ceil(T / 32)
 *          blocks of 38 KiB (DR_GDN2: 50 KiB) for d_k = 128, 21 KiB (29 KiB) for
 *          d_k = 64, rounded up to 256 bytes
 *
 * Channel-wise decays (DR_KDA, DR_GDN2, DR_FG2) are evaluated with exponents taken
 * relative to the boundaries of 16-token blocks, which keeps every factor inside
 * the fp32 range as long as one channel's log-decay summed over 16 tokens stays
 * above about -85.  To guarantee that, every per-token channel log-decay is
 * clamped to -85/16 = -5.3125 (a decay factor of about 0.0049 per token) when it
 * is loaded, by delta_fwd, delta_decode and delta_bwd alike: a gate below the
 * floor acts as the floor, and delta_bwd returns a zero dg for it.  Gates at or
 * above the floor are used as given.  The scalar decay of DR_GDN needs no floor.
 */
dr_status delta_fwd_workspace_bytes(const dr_desc* desc, size_t* bytes);
dr_status delta_fwd(const dr_desc* desc, const void* q, const void* k, const void* v,
                    const void* beta, const void* wgate, const void* g, const float* S0,
                    void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream);

/*
 * delta_fwd_noalloc — delta_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments and results are those of delta_fwd without the
 * workspace: where delta_fwd needs one (channel-wise decay forms with DR_BF16
 * operands), this entry point uses a scratch array of 64 MiB compiled into the
 * library, one per GPU, held until the process ends; no call allocates or frees
 * anything.  Descriptors whose delta_fwd_workspace_bytes exceed 64 MiB return
 * DR_E_WORKSPACE (for d_k = 128: B * H * ceil(T / 32) <= 1724 blocks for
 * DR_KDA and DR_FG2, 1310 for DR_GDN2).  Every call on one GPU shares that
 * GPU's scratch: calls that may overlap in time on one GPU (different streams,
 * several host threads) race and must be ordered by the caller.  The scratch
 * needs no clearing: each call writes every byte it reads.
 */
dr_status delta_fwd_noalloc(const dr_desc* desc, const void* q, const void* k, const void* v,
                            const void* beta, const void* wgate, const void* g, const float* S0,
                            void* o, float* S_T, void* stream);

/*
 * delta_decode — one token per sequence, state updated in place.
 *
 *   desc->T must be 1; shapes as delta_fwd with the T axis removed:
 *   q, k [B, H_k, d_k]; v [B, H, d_v]; beta [B, H] (DR_GDN2: b, DR_FG2: the
 *   step sizes, [B, H, d_k]);
 *   wgate [B, H, d_v] (DR_GDN2 only); g NULL / [B, H] / [B, H, d_k];
 *   S      state [B, H, d_v, d_k] fp32, read and overwritten in place
 *   o      output [B, H, d_v] dtype; must not overlap any input or S
 *
 * Each state matrix is read once and written once.
 */
dr_status delta_decode(const dr_desc* desc, const void* q, const void* k, const void* v,
                       const void* beta, const void* wgate, const void* g, float* S, void* o,
                       void* stream);

/*
 * delta_efla_beta — step sizes of the exact-flow form of the delta rule (EFLA:
 * "Delta-Rule Linear Attention" topic page, EFLA card).  The delta-rule write
 * is one explicit Euler step of length beta of the flow dS/dtau = (v - S k) k^T;
 * because k k^T has rank one, the flow over that length has the closed form of
 * a delta-rule write with the step size
 *
 *   beta_eff = (1 - exp(-beta ||k||^2)) / ||k||^2      (beta_eff = beta if k = 0)
 *
 * so an EFLA layer is delta_fwd / delta_decode called with beta_eff in place of
 * beta.  Decay, where the variant has one, is applied before the write as usual.
 *
 *   desc     variant DR_DELTANET, DR_GDN or DR_KDA (a single step size per
 *            token; DR_GDN2 and DR_FG2 return DR_E_UNSUPPORTED); T = 1 serves
 *            decode
 *   k        [B, T, H_k, d_k] dtype
 *   beta     [B, T, H] dtype, beta >= 0
 *   beta_eff [B, T, H] dtype (written, rounded to nearest even for bf16);
 *            may be the same pointer as beta (in place), must not overlap k
 *
 * ||k||^2 is summed in fp32 over the dtype values of k; exp(-x) - 1 is
 * evaluated without cancellation for small beta ||k||^2.
 */
dr_status delta_efla_beta(const dr_desc* desc, const void* k, const void* beta, void* beta_eff,
                          void* stream);

/*
 * delta_bwd — gradients of delta_fwd with respect to every input: the
 * gate-aware backward pass of the chunkwise form ("Gated DeltaNet-2" abstract:
 * a backward that keeps training chunkwise-parallel).  The forward states are
 * recomputed from the inputs; nothing from a delta_fwd call is needed.
 *
 *   desc, q, k, v, beta, wgate, g, S0   exactly as given to delta_fwd
 *   dO     [B, T, H, d_v] dtype: gradient arriving at o
 *   dS_T   [B, H, d_v, d_k] fp32: gradient arriving at the final state; NULL = 0
 *   dq, dk [B, T, H_k, d_k], dv [B, T, H, d_v]                     dtype (written)
 *   dbeta  [B, T, H]; DR_GDN2: gradient of the erase gate, DR_FG2: of the step
 *          sizes, [B, T, H, d_k]                                          dtype (written)
 *   dwgate DR_GDN2: gradient of the write gate [B, T, H, d_v]; otherwise must be NULL
 *   dg     DR_DELTANET: must be NULL; DR_GDN [B, T, H]; DR_KDA/DR_GDN2/DR_FG2 [B, T, H, d_k]
 *          dtype (written): gradient of the log-decay g
 *   dS0    [B, H, d_v, d_k] fp32 (written), gradient of S0; NULL if not wanted
 *
 * Channel-wise decays (DR_KDA, DR_GDN2, DR_FG2) are clamped to the same floor
 * as in delta_fwd, -85/16 per token (pairwise factors are split at a reference
 * row of each 16-token block); dg is zero for a gate below the floor.
 *
 * Grouped query/key heads (H_k < H): q, k, dq and dk are [B, T, H_k, d_k]; dq and
 * dk are summed over each group of value heads, through two fp32 buffers of
 * [B, T, H, d_k] at the end of the workspace.  Outputs must not overlap any input
 * or one another.  Intermediates are fp32; with fp32 inputs the products run in
 * fp32, with DR_BF16 inputs each fp32 operand of a product is split into two
 * bf16 values (hi + lo) and the product taken as hi*hi + hi*lo + lo*hi with fp32
 * accumulation (about 2^-17 relative error per product term).
 *
 *   workspace, workspace_bytes
 *          at least delta_bwd_workspace_bytes(desc) bytes: B * H * ceil(T / 64)
 *          records, rounded up to 256 bytes, plus the two grouped-head buffers
 *          when H_k < H.  A record is, for d_k/d_v = 128/128 (128/64, 64/128,
 *          64/64): DR_DELTANET and DR_GDN 272.75 KiB (208.75, 192.5, 128.5);
 *          DR_KDA and DR_FG2 400.5 KiB (336.5, 256.25, 192.25); DR_GDN2
 *          560.5 KiB (464.5, 368.25, 304.25)
 */
dr_status delta_bwd_workspace_bytes(const dr_desc* desc, size_t* bytes);
dr_status delta_bwd(const dr_desc* desc, const void* q, const void* k, const void* v,
                    const void* beta, const void* wgate, const void* g, const float* S0,
                    const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                    void* dbeta, void* dwgate, void* dg, float* dS0, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * delta_ttt_pre — DeltaTTT-pre: a two-layer memory whose layers each learn by
 * delta-rule steps ("DeltaTTT: Layerwise Optimization for Nonlinear Recurrent
 * Memory" summary, paperlayer.ai, §4.1 layerwise memory optimization and the
 * Pre schedule; Appendix A, chunkwise scan).  The first layer A [d_v, d_k]
 * learns keys -> values; the second layer B [d_v, d_v] learns the intermediate
 * representation -> value.  In the Pre schedule the intermediate representation
 * of token t comes from the first layer's state before token t's write.  Per
 * token, with silu(x) = x / (1 + e^-x) and unit(x) = x / ||x|| (0 stays 0):
 *
 *   A' = A Diag(a1_t); r = A' k_t; A = A' + beta1_t (v_t - r) k_t^T
 *   h  = unit(silu(r));            z = unit(silu(A q_t))
 *   B' = B a2_t;       s = B' h;   B = B' + beta2_t (v_t - s) h^T
 *   o_t = B z
 *
 * The summary prints none of these formulas: SiLU, the unit-normalised second-
 * layer key and query, and the readout after the write are this library's
 * readings (SiLU is the nonlinearity of its two-layer memories).  Evaluated as
 * two chunkwise first-layer scans (one of them on shifted queries, whose
 * readouts are the pre-write reads r), a key/query transform and one chunkwise
 * second-layer scan; every scan is delta_fwd's kernel.
 *
 *   desc   variant DR_DELTANET or DR_GDN (both layers); H_k must be 0 or H;
 *          d_k the key width of the first layer, d_v the value width (and both
 *          widths of the second layer)
 *   q, k   [B, T, H, d_k] dtype;  v [B, T, H, d_v] dtype
 *   beta1, beta2  step sizes of the two layers [B, T, H] dtype
 *   g1, g2 log-decays of the two layers [B, T, H] dtype (DR_GDN), NULL (DR_DELTANET)
 *   A0     [B, H, d_v, d_k] fp32 or NULL (zero);  B0 [B, H, d_v, d_v] fp32 or NULL
 *   o      [B, T, H, d_v] dtype (written); must not overlap any input
 *   A_T, B_T  final states, fp32 (written) or NULL; A_T may be A0 and B_T may be
 *          B0 (in place), otherwise no output may overlap an input or another output
 *
 *   workspace, workspace_bytes
 *          at least delta_ttt_pre_workspace_bytes(desc) bytes: the intermediate
 *          tensors (shifted queries, reads, first-layer readouts, keys and
 *          queries of the second layer), each rounded up to 256 bytes.
 *
 * No backward.
 */
dr_status delta_ttt_pre_workspace_bytes(const dr_desc* desc, size_t* bytes);
dr_status delta_ttt_pre(const dr_desc* desc, const void* q, const void* k, const void* v,
                        const void* beta1, const void* g1, const void* beta2, const void* g2,
                        const float* A0, const float* B0, void* o, float* A_T, float* B_T,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* dr_status_str(int status);

/* DR_ABI_VERSION of the loaded library. */
int dr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTARULE_H */
