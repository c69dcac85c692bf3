// C ABI of the gated delta-rule library: host-side validation, device check and
// dispatch to the kernel launchers.  See include/deltarule.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/deltarule.h"
#include "kernels.h"

namespace {

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Span span_of(const void* p, int64_t elems, int64_t elem_bytes) {
    Span s;
    if (p != nullptr) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + static_cast<uintptr_t>(elems * elem_bytes);
    }
    return s;
}

bool overlap(const Span& a, const Span& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Elements of each operand for a descriptor (T tokens per sequence), and the
// number of query/key heads.
struct Sizes {
    int64_t qk, v, beta, wgate, g, state;
    int Hk;
};

dr_status check_desc(const dr_desc* d, bool decode, Sizes* sz) {
    if (d == nullptr) return DR_E_NULLPTR;
    if (d->variant < DR_DELTANET || d->variant > DR_FG2) return DR_E_UNSUPPORTED;
    if (d->dtype != DR_F32 && d->dtype != DR_BF16) return DR_E_UNSUPPORTED;
    if (d->B < 1 || d->H < 1 || d->T < 1) return DR_E_SHAPE;
    if (decode && d->T != 1) return DR_E_SHAPE;
    if ((d->d_k != 64 && d->d_k != 128) || (d->d_v != 64 && d->d_v != 128)) return DR_E_UNSUPPORTED;
    if (d->chunk != 64) return DR_E_UNSUPPORTED;
    if (d->H_k < 0 || d->H_k > d->H || (d->H_k > 0 && d->H % d->H_k != 0)) return DR_E_SHAPE;
    sz->Hk = d->H_k == 0 ? d->H : d->H_k;
    const int64_t tok = static_cast<int64_t>(d->B) * d->T * d->H;
    // Keep every element index inside int64, every grid below 2^31 threads
    // (the widest grids: 8 value tiles of 256 threads per head, and one
    // 512-thread workgroup per 64-token chunk of every head in the backward)
    // and the kernels' 32-bit offsets within a chunk (64 rows of H_k heads of
    // d_k elements) below 2^31.
    if (tok > (int64_t(1) << 34)) return DR_E_SHAPE;
    const int64_t heads = static_cast<int64_t>(d->B) * d->H;
    if (heads > (int64_t(1) << 20)) return DR_E_SHAPE;
    if (heads * ((d->T + 63) / 64) > (int64_t(1) << 22)) return DR_E_SHAPE;
    if (static_cast<int64_t>(d->H) * 64 * 128 > (int64_t(1) << 31) - 1) return DR_E_SHAPE;
    sz->qk = static_cast<int64_t>(d->B) * d->T * sz->Hk * d->d_k;
    sz->v = tok * d->d_v;
    sz->beta = (d->variant == DR_GDN2 || d->variant == DR_FG2) ? tok * d->d_k : tok;
    sz->wgate = d->variant == DR_GDN2 ? tok * d->d_v : 0;
    sz->g = d->variant == DR_DELTANET ? 0 : (d->variant == DR_GDN ? tok : tok * d->d_k);
    sz->state = static_cast<int64_t>(d->B) * d->H * d->d_v * d->d_k;
    return DR_OK;
}

dr_status check_gate_ptrs(const dr_desc* d, const void* beta, const void* wgate, const void* g) {
    if (beta == nullptr) return DR_E_NULLPTR;
    if (d->variant == DR_GDN2) {
        if (wgate == nullptr) return DR_E_NULLPTR;
    } else if (wgate != nullptr) {
        return DR_E_UNSUPPORTED;
    }
    if (d->variant == DR_DELTANET) {
        if (g != nullptr) return DR_E_UNSUPPORTED;
    } else if (g == nullptr) {
        return DR_E_NULLPTR;
    }
    return DR_OK;
}

// The caller's workspace: present and large enough when one is needed,
// 256-byte aligned, and disjoint from every tensor argument.
dr_status check_workspace(size_t need, const void* ws, size_t ws_bytes, const Span* spans, int n) {
    if (need == 0) return DR_OK;
    if (ws == nullptr || ws_bytes < need) return DR_E_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return DR_E_ALIGN;
    Span w;
    w.lo = reinterpret_cast<uintptr_t>(ws);
    w.hi = w.lo + need;
    for (int i = 0; i < n; ++i)
        if (overlap(w, spans[i])) return DR_E_ALIAS;
    return DR_OK;
}

// Every check of delta_fwd's tensor arguments (sizes, pointers, alignment,
// aliasing); spans receives the byte ranges of the 9 tensors.
constexpr int kFwdSpans = 9;
dr_status check_fwd_args(const dr_desc* desc, const void* q, const void* k, const void* v,
                         const void* beta, const void* wgate, const void* g, const float* S0,
                         const void* o, const float* S_T, Sizes* szp, Span* spans) {
    Sizes& sz = *szp;
    dr_status st = check_desc(desc, false, &sz);
    if (st != DR_OK) return st;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return DR_E_NULLPTR;
    st = check_gate_ptrs(desc, beta, wgate, g);
    if (st != DR_OK) return st;
    const void* ptrs[] = {q, k, v, beta, wgate, g, S0, o, S_T};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return DR_E_ALIGN;
    const int64_t eb = desc->dtype == DR_F32 ? 4 : 2;
    const Span in[] = {span_of(q, sz.qk, eb),       span_of(k, sz.qk, eb),
                       span_of(v, sz.v, eb),        span_of(beta, sz.beta, eb),
                       span_of(wgate, sz.wgate, eb), span_of(g, sz.g, eb),
                       span_of(S0, sz.state, 4)};
    const Span so = span_of(o, sz.v, eb);
    const Span sst = span_of(S_T, sz.state, 4);
    for (const Span& s : in) {
        if (overlap(so, s)) return DR_E_ALIAS;
    }
    for (int i = 0; i < 6; ++i)
        if (overlap(sst, in[i])) return DR_E_ALIAS;
    if (overlap(sst, in[6]) && static_cast<const void*>(S_T) != static_cast<const void*>(S0))
        return DR_E_ALIAS;
    if (overlap(sst, so)) return DR_E_ALIAS;
    for (int i = 0; i < 7; ++i) spans[i] = in[i];
    spans[7] = so;
    spans[8] = sst;
    return DR_OK;
}

dr_status launch_forward(const dr_desc* desc, const Sizes& sz, const void* q, const void* k,
                         const void* v, const void* beta, const void* wgate, const void* g,
                         const float* S0, void* o, float* S_T, void* ws, void* stream) {
    dr::FwdArgs a{desc->B, desc->T, desc->H, desc->d_k, desc->d_v, q, k, v, beta, wgate, g,
                  S0, o, S_T, sz.Hk};
    a.ws = ws;
    const hipError_t e = dr::launch_fwd(desc->variant, desc->dtype, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DR_OK : DR_E_LAUNCH;
}

std::atomic<int> g_arch_state[64];  // per device: 0 unknown, 1 gfx950, 2 other

dr_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return DR_E_DEVICE;
    }
    if (dev < 64) {
        const int st = g_arch_state[dev].load(std::memory_order_acquire);
        if (st == 1) return DR_OK;
        if (st == 2) return DR_E_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return DR_E_DEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
    return ok ? DR_OK : DR_E_DEVICE;
}

// Device scratch of delta_fwd_noalloc: one array per GPU, part of the code
// object, held until the process ends.  Host code never uses the name itself
// (in host code it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// The scratch address of the current device (NULL if it cannot be resolved).
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

dr_status delta_fwd_workspace_bytes(const dr_desc* desc, size_t* bytes) {
    try {
        if (bytes == nullptr) return DR_E_NULLPTR;
        Sizes sz;
        const dr_status st = check_desc(desc, false, &sz);
        if (st != DR_OK) return st;
        *bytes = dr::fwd_workspace_bytes(desc->variant, desc->dtype, desc->B, desc->T, desc->H,
                                         desc->d_k, desc->d_v);
        return DR_OK;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_fwd(const dr_desc* desc, const void* q, const void* k, const void* v,
                    const void* beta, const void* wgate, const void* g, const float* S0,
                    void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        Sizes sz;
        Span spans[kFwdSpans];
        dr_status st = check_fwd_args(desc, q, k, v, beta, wgate, g, S0, o, S_T, &sz, spans);
        if (st != DR_OK) return st;
        const size_t need = dr::fwd_workspace_bytes(desc->variant, desc->dtype, desc->B, desc->T,
                                                    desc->H, desc->d_k, desc->d_v);
        st = check_workspace(need, workspace, workspace_bytes, spans, kFwdSpans);
        if (st != DR_OK) return st;
        st = check_device();
        if (st != DR_OK) return st;
        return launch_forward(desc, sz, q, k, v, beta, wgate, g, S0, o, S_T, need ? workspace : nullptr, stream);
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_fwd_noalloc(const dr_desc* desc, const void* q, const void* k, const void* v,
                            const void* beta, const void* wgate, const void* g, const float* S0,
                            void* o, float* S_T, void* stream) {
    try {
        Sizes sz;
        Span spans[kFwdSpans];
        dr_status st = check_fwd_args(desc, q, k, v, beta, wgate, g, S0, o, S_T, &sz, spans);
        if (st != DR_OK) return st;
        const size_t need = dr::fwd_workspace_bytes(desc->variant, desc->dtype, desc->B, desc->T,
                                                    desc->H, desc->d_k, desc->d_v);
        if (need > kScratchBytes) return DR_E_WORKSPACE;
        st = check_device();
        if (st != DR_OK) return st;
        void* ws = nullptr;
        if (need > 0) {
            ws = scratch_address();
            if (ws == nullptr) return DR_E_DEVICE;
        }
        return launch_forward(desc, sz, q, k, v, beta, wgate, g, S0, o, S_T, ws, stream);
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_decode(const dr_desc* desc, const void* q, const void* k, const void* v,
                       const void* beta, const void* wgate, const void* g, float* S, void* o,
                       void* stream) {
    try {
        Sizes sz;
        dr_status st = check_desc(desc, true, &sz);
        if (st != DR_OK) return st;
        if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || S == nullptr)
            return DR_E_NULLPTR;
        st = check_gate_ptrs(desc, beta, wgate, g);
        if (st != DR_OK) return st;
        const void* ptrs[] = {q, k, v, beta, wgate, g, S, o};
        for (const void* p : ptrs)
            if (p != nullptr && !aligned16(p)) return DR_E_ALIGN;
        const int64_t eb = desc->dtype == DR_F32 ? 4 : 2;
        const Span in[] = {span_of(q, sz.qk, eb),       span_of(k, sz.qk, eb),
                           span_of(v, sz.v, eb),        span_of(beta, sz.beta, eb),
                           span_of(wgate, sz.wgate, eb), span_of(g, sz.g, eb),
                           span_of(S, sz.state, 4)};
        const Span so = span_of(o, sz.v, eb);
        for (const Span& s : in)
            if (overlap(so, s)) return DR_E_ALIAS;
        for (int i = 0; i < 6; ++i)
            if (overlap(in[6], in[i])) return DR_E_ALIAS;

        st = check_device();
        if (st != DR_OK) return st;
        dr::DecodeArgs a{desc->B, desc->H, desc->d_k, desc->d_v, q, k, v, beta, wgate, g, S, o,
                         sz.Hk};
        const hipError_t e = dr::launch_decode(desc->variant, desc->dtype, a,
                                               static_cast<hipStream_t>(stream));
        return e == hipSuccess ? DR_OK : DR_E_LAUNCH;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

// DeltaTTT-pre's extra shape rules (both layers DeltaNet or GDN, no grouped heads)
dr_status check_ttt_desc(const dr_desc* desc, Sizes* sz) {
    const dr_status st = check_desc(desc, false, sz);
    if (st != DR_OK) return st;
    if (desc->variant != DR_DELTANET && desc->variant != DR_GDN) return DR_E_UNSUPPORTED;
    if (sz->Hk != desc->H) return DR_E_UNSUPPORTED;
    return DR_OK;
}

dr_status delta_ttt_pre_workspace_bytes(const dr_desc* desc, size_t* bytes) {
    try {
        if (bytes == nullptr) return DR_E_NULLPTR;
        Sizes sz;
        const dr_status st = check_ttt_desc(desc, &sz);
        if (st != DR_OK) return st;
        *bytes = dr::ttt_workspace_bytes(desc->dtype, desc->B, desc->T, desc->H, desc->d_k, desc->d_v);
        return DR_OK;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_ttt_pre(const dr_desc* desc, const void* q, const void* k, const void* v,
                        const void* beta1, const void* g1, const void* beta2, const void* g2,
                        const float* A0, const float* B0, void* o, float* A_T, float* B_T,
                        void* workspace, size_t workspace_bytes, void* stream) {
    try {
        Sizes sz;
        dr_status st = check_ttt_desc(desc, &sz);
        if (st != DR_OK) return st;
        if (q == nullptr || k == nullptr || v == nullptr || beta1 == nullptr || beta2 == nullptr ||
            o == nullptr)
            return DR_E_NULLPTR;
        if (desc->variant == DR_GDN) {
            if (g1 == nullptr || g2 == nullptr) return DR_E_NULLPTR;
        } else if (g1 != nullptr || g2 != nullptr) {
            return DR_E_UNSUPPORTED;
        }
        const void* ptrs[] = {q, k, v, beta1, g1, beta2, g2, A0, B0, o, A_T, B_T};
        for (const void* p : ptrs)
            if (p != nullptr && !aligned16(p)) return DR_E_ALIGN;
        const int64_t eb = desc->dtype == DR_F32 ? 4 : 2;
        const int64_t bstate = static_cast<int64_t>(desc->B) * desc->H * desc->d_v * desc->d_v;
        const Span in[] = {span_of(q, sz.qk, eb),      span_of(k, sz.qk, eb),
                           span_of(v, sz.v, eb),       span_of(beta1, sz.beta, eb),
                           span_of(g1, sz.g, eb),      span_of(beta2, sz.beta, eb),
                           span_of(g2, sz.g, eb),      span_of(A0, sz.state, 4),
                           span_of(B0, bstate, 4)};
        const Span so = span_of(o, sz.v, eb), sa = span_of(A_T, sz.state, 4), sb = span_of(B_T, bstate, 4);
        for (const Span& s : in)
            if (overlap(so, s)) return DR_E_ALIAS;
        for (int i = 0; i < 9; ++i) {
            if (overlap(sa, in[i]) && !(i == 7 && static_cast<const void*>(A_T) == static_cast<const void*>(A0)))
                return DR_E_ALIAS;
            if (overlap(sb, in[i]) && !(i == 8 && static_cast<const void*>(B_T) == static_cast<const void*>(B0)))
                return DR_E_ALIAS;
        }
        if (overlap(sa, so) || overlap(sb, so) || overlap(sa, sb)) return DR_E_ALIAS;
        const size_t need = dr::ttt_workspace_bytes(desc->dtype, desc->B, desc->T, desc->H, desc->d_k,
                                                    desc->d_v);
        const Span all[] = {in[0], in[1], in[2], in[3], in[4], in[5], in[6], in[7], in[8], so, sa, sb};
        st = check_workspace(need, workspace, workspace_bytes, all, 12);
        if (st != DR_OK) return st;

        st = check_device();
        if (st != DR_OK) return st;
        dr::TttArgs a{desc->B, desc->T, desc->H, desc->d_k, desc->d_v, q, k, v, beta1, g1, beta2, g2,
                      A0, B0, o, A_T, B_T};
        a.ws = workspace;
        const hipError_t e = dr::launch_ttt_pre(desc->variant, desc->dtype, a, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? DR_OK : DR_E_LAUNCH;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_efla_beta(const dr_desc* desc, const void* k, const void* beta, void* beta_eff,
                          void* stream) {
    try {
        Sizes sz;
        dr_status st = check_desc(desc, false, &sz);
        if (st != DR_OK) return st;
        if (desc->variant == DR_GDN2 || desc->variant == DR_FG2) return DR_E_UNSUPPORTED;
        if (k == nullptr || beta == nullptr || beta_eff == nullptr) return DR_E_NULLPTR;
        if (!aligned16(k) || !aligned16(beta) || !aligned16(beta_eff)) return DR_E_ALIGN;
        const int64_t eb = desc->dtype == DR_F32 ? 4 : 2;
        const Span sk = span_of(k, sz.qk, eb), sb = span_of(beta, sz.beta, eb);
        const Span so = span_of(beta_eff, sz.beta, eb);
        if (overlap(so, sk)) return DR_E_ALIAS;
        if (overlap(so, sb) && beta_eff != beta) return DR_E_ALIAS;

        st = check_device();
        if (st != DR_OK) return st;
        dr::EflaArgs a{desc->B, desc->T, desc->H, sz.Hk, desc->d_k, k, beta, beta_eff};
        const hipError_t e = dr::launch_efla_beta(desc->dtype, a, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? DR_OK : DR_E_LAUNCH;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_bwd_workspace_bytes(const dr_desc* desc, size_t* bytes) {
    try {
        if (bytes == nullptr) return DR_E_NULLPTR;
        Sizes sz;
        const dr_status st = check_desc(desc, false, &sz);
        if (st != DR_OK) return st;
        *bytes = dr::bwd_workspace_bytes(desc->variant, desc->B, desc->T, desc->H, sz.Hk, desc->d_k,
                                         desc->d_v);
        return DR_OK;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

dr_status delta_bwd(const dr_desc* desc, const void* q, const void* k, const void* v,
                    const void* beta, const void* wgate, const void* g, const float* S0,
                    const void* dO, const float* dS_T, void* dq, void* dk, void* dv,
                    void* dbeta, void* dwgate, void* dg, float* dS0, void* workspace,
                    size_t workspace_bytes, void* stream) {
    try {
        Sizes sz;
        dr_status st = check_desc(desc, false, &sz);
        if (st != DR_OK) return st;
        if (q == nullptr || k == nullptr || v == nullptr || dO == nullptr || dq == nullptr ||
            dk == nullptr || dv == nullptr || dbeta == nullptr)
            return DR_E_NULLPTR;
        st = check_gate_ptrs(desc, beta, wgate, g);
        if (st != DR_OK) return st;
        if ((desc->variant == DR_DELTANET) != (dg == nullptr))
            return desc->variant == DR_DELTANET ? DR_E_UNSUPPORTED : DR_E_NULLPTR;
        if ((desc->variant == DR_GDN2) != (dwgate != nullptr))
            return desc->variant == DR_GDN2 ? DR_E_NULLPTR : DR_E_UNSUPPORTED;
        const void* ptrs[] = {q, k, v, beta, wgate, g, S0, dO, dS_T, dq, dk, dv, dbeta, dwgate, dg, dS0};
        for (const void* p : ptrs)
            if (p != nullptr && !aligned16(p)) return DR_E_ALIGN;
        const int64_t eb = desc->dtype == DR_F32 ? 4 : 2;
        const Span in[] = {span_of(q, sz.qk, eb),   span_of(k, sz.qk, eb),  span_of(v, sz.v, eb),
                           span_of(beta, sz.beta, eb), span_of(wgate, sz.wgate, eb),
                           span_of(g, sz.g, eb),    span_of(S0, sz.state, 4),
                           span_of(dO, sz.v, eb),   span_of(dS_T, sz.state, 4)};
        const Span out[] = {span_of(dq, sz.qk, eb), span_of(dk, sz.qk, eb), span_of(dv, sz.v, eb),
                            span_of(dbeta, sz.beta, eb), span_of(dwgate, sz.wgate, eb),
                            span_of(dg, sz.g, eb),   span_of(dS0, sz.state, 4)};
        for (int i = 0; i < 7; ++i) {
            for (const Span& s : in)
                if (overlap(out[i], s)) return DR_E_ALIAS;
            for (int j = 0; j < i; ++j)
                if (overlap(out[i], out[j])) return DR_E_ALIAS;
        }
        const size_t need = dr::bwd_workspace_bytes(desc->variant, desc->B, desc->T, desc->H, sz.Hk,
                                                    desc->d_k, desc->d_v);
        const Span all[] = {in[0], in[1], in[2], in[3], in[4], in[5], in[6], in[7], in[8],
                            out[0], out[1], out[2], out[3], out[4], out[5], out[6]};
        st = check_workspace(need, workspace, workspace_bytes, all, 16);
        if (st != DR_OK) return st;

        st = check_device();
        if (st != DR_OK) return st;
        dr::BwdArgs a{desc->B, desc->T, desc->H, desc->d_k, desc->d_v, q, k, v, beta, g, S0, dO,
                      dS_T, dq, dk, dv, dbeta, dg, dS0, wgate, dwgate, sz.Hk, nullptr, nullptr};
        a.ws = workspace;
        const hipError_t e = dr::launch_bwd(desc->variant, desc->dtype, a,
                                            static_cast<hipStream_t>(stream));
        return e == hipSuccess ? DR_OK : DR_E_LAUNCH;
    } catch (...) {
        return DR_E_LAUNCH;
    }
}

const char* dr_status_str(int s) {
    switch (s) {
        case DR_OK: return "ok";
        case DR_E_NULLPTR: return "null pointer";
        case DR_E_SHAPE: return "bad shape";
        case DR_E_UNSUPPORTED: return "unsupported variant, dtype, size or argument";
        case DR_E_ALIGN: return "pointer not 16-byte aligned";
        case DR_E_DEVICE: return "no gfx950 HIP device";
        case DR_E_LAUNCH: return "kernel launch failed";
        case DR_E_ALIAS: return "output overlaps an input";
        case DR_E_WORKSPACE: return "workspace missing or smaller than the size query reports";
        default: return "unknown status";
    }
}

int dr_abi_version(void) { return DR_ABI_VERSION; }

}  // extern "C"
