// C ABI of libttt_la.so: validation, kernel plan, workspace, launches.
// The operation and every argument are documented in include/ttt_la.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "device_common.h"
#include "internal.h"
#include "ttt_la.h"

struct ttt_la_s {
    ttt_la_desc desc;
    ttt::Shape shape;
    bool fast;
    ttt::FastPlan fp;
    void* workspace;
    size_t workspace_bytes;
    int device;
    unsigned epoch;      // completed launches of the fused path (its counter targets)
    // measurement hook
    std::vector<hipEvent_t> ev_begin, ev_end;
    int calls;           // timed calls so far
    int every;           // time one call in `every`
    int seen;            // calls since the timing was set
    // the backward's two time-reversed forwards run beside the first one on their
    // own streams (created on first use; default priority)
    hipStream_t aux[2];
    hipEvent_t fork, join[2];
    bool aux_ready;
};

namespace {

using ttt::Shape;

constexpr uint32_t kModeMask = TTT_LA_BIDIRECTIONAL | TTT_LA_ETA_PER_TOKEN | TTT_LA_ETA_SOFTPLUS;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(int dtype) { return dtype == TTT_LA_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

int check_desc(const ttt_la_desc* d) {
    if (!d) return TTT_LA_ERR_INVALID_ARG;
    if (d->B < 1 || d->H < 1 || d->T < 1) return TTT_LA_ERR_INVALID_ARG;
    if (d->d_k < 1 || d->d_v < 1 || d->d_phi < 1) return TTT_LA_ERR_INVALID_ARG;
    if (d->dtype != TTT_LA_F32 && d->dtype != TTT_LA_BF16) return TTT_LA_ERR_INVALID_ARG;
    if (d->phi != TTT_LA_PHI_IDENTITY && d->phi != TTT_LA_PHI_SWIGLU) return TTT_LA_ERR_INVALID_ARG;
    if (d->chunk < 0 || d->segments < 0) return TTT_LA_ERR_INVALID_ARG;
    if (d->value_split < 0 || d->value_split > 2) return TTT_LA_ERR_INVALID_ARG;
    if (d->launch < TTT_LA_LAUNCH_AUTO || d->launch > TTT_LA_LAUNCH_PREFIX) return TTT_LA_ERR_INVALID_ARG;
    if (d->phi == TTT_LA_PHI_SWIGLU) {
        if (!d->w1 || !d->w3) return TTT_LA_ERR_INVALID_ARG;
        if (!aligned(d->w1, 16) || !aligned(d->w3, 16)) return TTT_LA_ERR_INVALID_ARG;
    } else {
        if (d->w1 || d->w3) return TTT_LA_ERR_INVALID_ARG;
        if (d->d_phi != d->d_k) return TTT_LA_ERR_INVALID_ARG;
    }
    // supported shapes
    if (d->d_k != 64 && d->d_k != 128) return TTT_LA_ERR_UNSUPPORTED;
    if (d->d_v != 64 && d->d_v != 128) return TTT_LA_ERR_UNSUPPORTED;
    if (d->phi == TTT_LA_PHI_SWIGLU && (d->d_phi % 128 != 0 || d->d_phi > 512)) return TTT_LA_ERR_UNSUPPORTED;
    if (d->chunk != 0 && d->chunk != 64 && d->chunk != 128) return TTT_LA_ERR_UNSUPPORTED;
    const long long widest = std::max(d->d_k, std::max(d->d_v, d->d_phi));
    if ((long long)d->B * d->H * d->T * widest >= (1LL << 31)) return TTT_LA_ERR_UNSUPPORTED;
    return TTT_LA_OK;
}

int check_forward(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
                  float eta_scalar, float beta, uint32_t mode, const void* o) {
    if (!q || !k || !v || !o) return TTT_LA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return TTT_LA_ERR_INVALID_ARG;
    if (mode & ~kModeMask) return TTT_LA_ERR_INVALID_ARG;
    const bool per_tok = (mode & TTT_LA_ETA_PER_TOKEN) != 0;
    const bool softp = (mode & TTT_LA_ETA_SOFTPLUS) != 0;
    if (per_tok && softp) return TTT_LA_ERR_INVALID_ARG;
    if (per_tok || softp) {
        if (!eta || !aligned(eta, 4)) return TTT_LA_ERR_INVALID_ARG;
    } else {
        if (eta) return TTT_LA_ERR_INVALID_ARG;
        if (!std::isfinite(eta_scalar)) return TTT_LA_ERR_INVALID_ARG;
    }
    if (!(beta >= 0.0f && beta < 1.0f)) return TTT_LA_ERR_INVALID_ARG;  // also rejects NaN
    const size_t eb = elem_bytes(d->dtype);
    const size_t nt = (size_t)d->B * d->H * d->T;
    const size_t qk_bytes = nt * d->d_k * eb, v_bytes = nt * d->d_v * eb;
    const size_t eta_bytes = (per_tok || softp) ? nt * sizeof(float) : 0;
    if (overlaps(o, v_bytes, q, qk_bytes) || overlaps(o, v_bytes, k, qk_bytes) ||
        overlaps(o, v_bytes, v, v_bytes) || overlaps(o, v_bytes, eta, eta_bytes))
        return TTT_LA_ERR_INVALID_ARG;
    if (d->phi == TTT_LA_PHI_SWIGLU) {
        const size_t w_bytes = (size_t)d->H * d->d_phi * d->d_k * eb;
        if (overlaps(o, v_bytes, d->w1, w_bytes) || overlaps(o, v_bytes, d->w3, w_bytes))
            return TTT_LA_ERR_INVALID_ARG;
    }
    return TTT_LA_OK;
}

bool state_ok(const void* p) { return !p || aligned(p, 16); }

// ttt_la_forward_state: forward checks, causal only, state pointers aligned, outputs
// disjoint from everything except (in place) their own input
int check_forward_state(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
                        float eta_scalar, float beta, uint32_t mode, const float* S0, const float* M0, const void* o,
                        const float* S_T, const float* M_T) {
    int st = check_forward(d, q, k, v, eta, eta_scalar, beta, mode, o);
    if (st != TTT_LA_OK) return st;
    if (mode & TTT_LA_BIDIRECTIONAL) return TTT_LA_ERR_INVALID_ARG;
    if (!state_ok(S0) || !state_ok(M0) || !state_ok(S_T) || !state_ok(M_T)) return TTT_LA_ERR_INVALID_ARG;
    const size_t eb = elem_bytes(d->dtype);
    const size_t nt = (size_t)d->B * d->H * d->T;
    const size_t sb = (size_t)d->B * d->H * d->d_v * d->d_phi * sizeof(float);
    const size_t qk_bytes = nt * d->d_k * eb, v_bytes = nt * d->d_v * eb;
    const size_t eta_bytes = eta ? nt * sizeof(float) : 0;
    const size_t w_bytes = d->phi == TTT_LA_PHI_SWIGLU ? (size_t)d->H * d->d_phi * d->d_k * eb : 0;
    const void* states[4] = {S0, M0, S_T, M_T};
    for (const void* x : states) {
        if (overlaps(x, sb, q, qk_bytes) || overlaps(x, sb, k, qk_bytes) || overlaps(x, sb, v, v_bytes) ||
            overlaps(x, sb, eta, eta_bytes) || overlaps(x, sb, o, v_bytes) || overlaps(x, sb, d->w1, w_bytes) ||
            overlaps(x, sb, d->w3, w_bytes))
            return TTT_LA_ERR_INVALID_ARG;
    }
    if (overlaps(S_T, sb, M_T, sb)) return TTT_LA_ERR_INVALID_ARG;
    if (S_T != S0 && overlaps(S_T, sb, S0, sb)) return TTT_LA_ERR_INVALID_ARG;
    if (M_T != M0 && overlaps(M_T, sb, M0, sb)) return TTT_LA_ERR_INVALID_ARG;
    if (overlaps(S_T, sb, M0, sb) || overlaps(M_T, sb, S0, sb)) return TTT_LA_ERR_INVALID_ARG;
    return TTT_LA_OK;
}

// ttt_la_step: one token per (b, h); S, M required, disjoint from each other and
// from every other argument
int check_step(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
               float eta_scalar, float beta, uint32_t mode, const float* S, const float* M, const void* o) {
    if (!q || !k || !v || !o || !S || !M) return TTT_LA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return TTT_LA_ERR_INVALID_ARG;
    if (!aligned(S, 16) || !aligned(M, 16)) return TTT_LA_ERR_INVALID_ARG;
    if (mode & ~kModeMask) return TTT_LA_ERR_INVALID_ARG;
    if (mode & TTT_LA_BIDIRECTIONAL) return TTT_LA_ERR_INVALID_ARG;
    const bool per_tok = (mode & TTT_LA_ETA_PER_TOKEN) != 0;
    const bool softp = (mode & TTT_LA_ETA_SOFTPLUS) != 0;
    if (per_tok && softp) return TTT_LA_ERR_INVALID_ARG;
    if (per_tok || softp) {
        if (!eta || !aligned(eta, 4)) return TTT_LA_ERR_INVALID_ARG;
    } else {
        if (eta) return TTT_LA_ERR_INVALID_ARG;
        if (!std::isfinite(eta_scalar)) return TTT_LA_ERR_INVALID_ARG;
    }
    if (!(beta >= 0.0f && beta < 1.0f)) return TTT_LA_ERR_INVALID_ARG;
    const size_t eb = elem_bytes(d->dtype);
    const size_t n = (size_t)d->B * d->H;
    const size_t qk_bytes = n * d->d_k * eb, v_bytes = n * d->d_v * eb;
    const size_t eta_bytes = eta ? n * sizeof(float) : 0;
    const size_t sb = n * d->d_v * d->d_phi * sizeof(float);
    const size_t w_bytes = d->phi == TTT_LA_PHI_SWIGLU ? (size_t)d->H * d->d_phi * d->d_k * eb : 0;
    if (overlaps(o, v_bytes, q, qk_bytes) || overlaps(o, v_bytes, k, qk_bytes) || overlaps(o, v_bytes, v, v_bytes) ||
        overlaps(o, v_bytes, eta, eta_bytes) || overlaps(o, v_bytes, d->w1, w_bytes) ||
        overlaps(o, v_bytes, d->w3, w_bytes))
        return TTT_LA_ERR_INVALID_ARG;
    if (overlaps(S, sb, M, sb)) return TTT_LA_ERR_INVALID_ARG;
    const void* states[2] = {S, M};
    for (const void* x : states) {
        if (overlaps(x, sb, q, qk_bytes) || overlaps(x, sb, k, qk_bytes) || overlaps(x, sb, v, v_bytes) ||
            overlaps(x, sb, eta, eta_bytes) || overlaps(x, sb, o, v_bytes) || overlaps(x, sb, d->w1, w_bytes) ||
            overlaps(x, sb, d->w3, w_bytes))
            return TTT_LA_ERR_INVALID_ARG;
    }
    return TTT_LA_OK;
}

Shape shape_of(const ttt_la_desc& d) {
    Shape s;
    s.B = d.B;
    s.H = d.H;
    s.T = d.T;
    s.d_k = d.d_k;
    s.d_v = d.d_v;
    s.d_phi = d.d_phi;
    s.bf16 = d.dtype == TTT_LA_BF16;
    s.swiglu = d.phi == TTT_LA_PHI_SWIGLU;
    s.w1 = d.w1;
    s.w3 = d.w3;
    return s;
}

int eta_kind_of(uint32_t mode) {
    if (mode & TTT_LA_ETA_PER_TOKEN) return ttt::ETA_PER_TOKEN;
    if (mode & TTT_LA_ETA_SOFTPLUS) return ttt::ETA_SOFTPLUS;
    return ttt::ETA_SCALAR;
}

void release_events(ttt_la_s* h) {
    for (hipEvent_t e : h->ev_begin) (void)hipEventDestroy(e);
    for (hipEvent_t e : h->ev_end) (void)hipEventDestroy(e);
    h->ev_begin.clear();
    h->ev_end.clear();
    h->calls = 0;
    h->seen = 0;
}

}  // namespace

extern "C" {

const char* ttt_la_status_string(int status) {
    switch (status) {
        case TTT_LA_OK: return "ok";
        case TTT_LA_ERR_INVALID_ARG: return "invalid argument";
        case TTT_LA_ERR_UNSUPPORTED: return "unsupported shape or setting";
        case TTT_LA_ERR_HIP: return "HIP runtime error";
        case TTT_LA_ERR_OOM: return "out of device memory";
        default: return "unknown status";
    }
}

int ttt_la_check(const ttt_la_desc* desc, const void* q, const void* k, const void* v, const float* eta,
                 float eta_scalar, float beta, uint32_t mode, const void* o) {
    int st = check_desc(desc);
    if (st != TTT_LA_OK || q == nullptr) return st;
    return check_forward(desc, q, k, v, eta, eta_scalar, beta, mode, o);
}

int ttt_la_check_state(const ttt_la_desc* desc, int32_t call, const void* q, const void* k, const void* v,
                       const float* eta, float eta_scalar, float beta, uint32_t mode, const float* s_in,
                       const float* m_in, const void* o, const float* s_out, const float* m_out) {
    int st = check_desc(desc);
    if (st != TTT_LA_OK) return st;
    if (call == 0)
        return check_forward_state(desc, q, k, v, eta, eta_scalar, beta, mode, s_in, m_in, o, s_out, m_out);
    if (call == 1) {
        if (s_in != s_out || m_in != m_out) return TTT_LA_ERR_INVALID_ARG;
        return check_step(desc, q, k, v, eta, eta_scalar, beta, mode, s_in, m_in, o);
    }
    return TTT_LA_ERR_INVALID_ARG;
}

int ttt_la_create(const ttt_la_desc* desc, ttt_la_t* out) {
    if (!out) return TTT_LA_ERR_INVALID_ARG;
    *out = nullptr;
    int st = check_desc(desc);
    if (st != TTT_LA_OK) return st;

    ttt_la_s* h = new (std::nothrow) ttt_la_s();
    if (!h) return TTT_LA_ERR_OOM;
    h->desc = *desc;
    h->shape = shape_of(*desc);
    h->workspace = nullptr;
    h->workspace_bytes = 0;
    h->calls = 0;
    h->every = 1;
    h->seen = 0;
    h->epoch = 0;
    h->fast = desc->dtype == TTT_LA_BF16 && ttt::fast_supported(h->shape, desc->chunk);
    if (h->fast) {
        h->fp = ttt::fast_plan(h->shape, desc->chunk, desc->segments, desc->value_split, desc->launch);
        h->workspace_bytes = h->fp.summary_bytes + h->fp.partial_bytes + h->fp.zero_bytes;
    }
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return TTT_LA_ERR_HIP;
    }
    if (!h->fast && ttt::generic_smem_bytes(h->shape) > 160 * 1024) {
        delete h;
        return TTT_LA_ERR_UNSUPPORTED;
    }
    if (h->workspace_bytes) {
        hipError_t e = hipMalloc(&h->workspace, h->workspace_bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            delete h;
            return e == hipErrorOutOfMemory ? TTT_LA_ERR_OOM : TTT_LA_ERR_HIP;
        }
        if (h->fast && h->fp.zero_bytes) {
            // counters of the single-launch path: they start at zero and only grow
            char* zp = static_cast<char*>(h->workspace) + h->fp.summary_bytes + h->fp.partial_bytes;
            if (hipMemset(zp, 0, h->fp.zero_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
                (void)hipGetLastError();
                (void)hipFree(h->workspace);
                delete h;
                return TTT_LA_ERR_HIP;
            }
        }
    }
    *out = h;
    return TTT_LA_OK;
}

}  // extern "C"

namespace {

// the timing events of the next launch (null when the hook is off)
void next_events(ttt_la_s* h, hipEvent_t* eb, hipEvent_t* ee) {
    *eb = *ee = nullptr;
    if (!h->ev_begin.empty() && h->seen++ % h->every == 0) {
        const size_t slot = (size_t)h->calls % h->ev_begin.size();
        *eb = h->ev_begin[slot];
        *ee = h->ev_end[slot];
        h->calls++;
    }
}

int enqueue_forward(ttt_la_s* h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                    float beta, uint32_t mode, const float* S0, const float* M0, void* o, float* S_T, float* M_T,
                    void* hip_stream, bool timed = true, bool reverse = false, void* workspace = nullptr) {
    if (!workspace) workspace = h->workspace;
    ttt::FwdArgs a{};
    a.reverse = reverse;
    a.q = q;
    a.k = k;
    a.v = v;
    a.eta = eta;
    a.eta_scalar = eta_scalar;
    a.beta = beta;
    a.eta_kind = eta_kind_of(mode);
    a.bidirectional = (mode & TTT_LA_BIDIRECTIONAL) != 0;
    a.o = o;
    a.stream = static_cast<hipStream_t>(hip_stream);
    a.S0 = S0;
    a.M0 = M0;
    a.S_T = S_T;
    a.M_T = M_T;
    const bool state_io = S0 || M0 || S_T || M_T;

    hipEvent_t eb = nullptr, ee = nullptr;
    if (timed) next_events(h, &eb, &ee);
    hipError_t e;
    if (h->fast && (h->fp.wide || !state_io)) {
        a.epoch = h->epoch + 1;
        e = ttt::launch_fast(h->shape, h->fp, workspace, a, eb, ee, nullptr);
        const bool fused_ran = h->fp.fused && !a.bidirectional && !state_io;
        if (e == hipErrorCooperativeLaunchTooLarge && fused_ran) {
            // the fused grid cannot be resident right now: same result in three launches
            ttt::FastPlan p3 = h->fp;
            p3.fused = false;
            e = ttt::launch_fast(h->shape, p3, workspace, a, eb, ee, nullptr);
        } else if (e == hipSuccess && fused_ran) {
            h->epoch++;
        }
    } else {
        // fp32 inputs, and the carried-state calls of the 16x16-tile shapes
        if (reverse) return TTT_LA_ERR_INVALID_ARG;
        e = ttt::launch_generic(h->shape, a, eb, ee);
    }
    return e == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

bool backward_supported(const ttt_la_desc& d) { return d.phi == TTT_LA_PHI_IDENTITY && d.d_k == d.d_v; }

// one [B, H, T, d] tensor in the handle's dtype
size_t tensor_bytes(const ttt_la_desc& d) { return (size_t)d.B * d.H * d.T * d.d_v * elem_bytes(d.dtype); }

// The 32x32-tile plans of three launches (decided from the descriptor alone: a
// single or prefix launch was not asked for) read the time-reversed operands in
// reverse order themselves.
bool reversed_in_kernel(const ttt_la_desc& d) {
    const Shape s = shape_of(d);
    return d.dtype == TTT_LA_BF16 && ttt::fast_supported(s, d.chunk) && ttt::wide_supported(s) && d.value_split != 2 &&
           d.launch != TTT_LA_LAUNCH_SINGLE && d.launch != TTT_LA_LAUNCH_PREFIX;
}

// Workspace of the backward.  Bidirectional: the two forward outputs.  Causal,
// reversed in the kernels: the two forward outputs, then a segment-summary area
// for each of the two reversed forwards (they run beside the first one, which uses
// the handle's).  Causal otherwise: q, k, v, dO reversed in time, then the outputs.
size_t backward_ws_bytes(const ttt_la_desc& d, uint32_t mode) {
    if (mode & TTT_LA_BIDIRECTIONAL) return 2 * tensor_bytes(d);
    if (reversed_in_kernel(d)) {
        const ttt::FastPlan p = ttt::fast_plan(shape_of(d), d.chunk, d.segments, d.value_split, d.launch);
        return 2 * tensor_bytes(d) + 2 * p.summary_bytes;
    }
    return 6 * tensor_bytes(d);
}

// streams and events of the concurrent reversed forwards; false if any is missing
// (the failure is cleared from the HIP error state, so that it cannot be reported
// by a later launch check)
bool ensure_aux(ttt_la_s* h) {
    if (h->aux_ready) return true;
    bool ok = true;
    for (int i = 0; i < 2 && ok; ++i)
        if (!h->aux[i] && hipStreamCreateWithFlags(&h->aux[i], hipStreamNonBlocking) != hipSuccess) ok = false;
    if (ok && !h->fork && hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) != hipSuccess) ok = false;
    for (int i = 0; i < 2 && ok; ++i)
        if (!h->join[i] && hipEventCreateWithFlags(&h->join[i], hipEventDisableTiming) != hipSuccess) ok = false;
    if (!ok) {
        (void)hipGetLastError();
        return false;
    }
    h->aux_ready = true;
    return true;
}

int check_backward(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
                   float eta_scalar, float beta, uint32_t mode, const void* dO, const void* dQ, const void* dK,
                   const void* dV, const float* dEta, const void* ws, size_t ws_bytes) {
    int st = check_forward(d, q, k, v, eta, eta_scalar, beta, mode, dQ);
    if (st != TTT_LA_OK) return st;
    if (!backward_supported(*d)) return TTT_LA_ERR_UNSUPPORTED;
    if (!dO || !dK || !dV) return TTT_LA_ERR_INVALID_ARG;
    if (!aligned(dO, 16) || !aligned(dK, 16) || !aligned(dV, 16)) return TTT_LA_ERR_INVALID_ARG;
    if (dEta && !aligned(dEta, 4)) return TTT_LA_ERR_INVALID_ARG;
    const size_t need = backward_ws_bytes(*d, mode);
    if (need && (!ws || !aligned(ws, 16) || ws_bytes < need)) return TTT_LA_ERR_INVALID_ARG;
    const size_t tb = tensor_bytes(*d);
    const size_t nt = (size_t)d->B * d->H * d->T;
    const size_t eta_bytes = eta ? nt * sizeof(float) : 0;
    const void* outs[4] = {dQ, dK, dV, dEta};
    const size_t out_bytes[4] = {tb, tb, tb, nt * sizeof(float)};
    const void* ins[5] = {q, k, v, dO, eta};
    const size_t in_bytes[5] = {tb, tb, tb, tb, eta_bytes};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return TTT_LA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return TTT_LA_ERR_INVALID_ARG;
        if (overlaps(outs[i], out_bytes[i], ws, need)) return TTT_LA_ERR_INVALID_ARG;
    }
    for (int j = 0; j < 5; ++j)
        if (overlaps(ws, need, ins[j], in_bytes[j])) return TTT_LA_ERR_INVALID_ARG;
    return TTT_LA_OK;
}

}  // namespace

extern "C" {

int ttt_la_check_backward(const ttt_la_desc* desc, const void* q, const void* k, const void* v, const float* eta,
                          float eta_scalar, float beta, uint32_t mode, const void* dO, const void* dQ,
                          const void* dK, const void* dV, const float* dEta, const void* workspace,
                          size_t workspace_bytes) {
    int st = check_desc(desc);
    if (st != TTT_LA_OK) return st;
    return check_backward(desc, q, k, v, eta, eta_scalar, beta, mode, dO, dQ, dK, dV, dEta, workspace,
                          workspace_bytes);
}

int ttt_la_backward_workspace(ttt_la_t h, uint32_t mode, size_t* bytes) {
    if (!h || !bytes) return TTT_LA_ERR_INVALID_ARG;
    *bytes = 0;
    if (mode & ~kModeMask) return TTT_LA_ERR_INVALID_ARG;
    if (!backward_supported(h->desc)) return TTT_LA_ERR_UNSUPPORTED;
    *bytes = backward_ws_bytes(h->desc, mode);
    return TTT_LA_OK;
}

int ttt_la_backward(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                    float beta, uint32_t mode, const void* dO, void* dQ, void* dK, void* dV, float* dEta,
                    void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_backward(&h->desc, q, k, v, eta, eta_scalar, beta, mode, dO, dQ, dK, dV, dEta, workspace,
                            workspace_bytes);
    if (st != TTT_LA_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const bool bidir = (mode & TTT_LA_BIDIRECTIONAL) != 0;
    const size_t tb = tensor_bytes(h->desc);
    char* ws = static_cast<char*>(workspace);
    // the 32x32-tile kernels of three launches read and write in reverse time order
    // themselves; the other plans get reversed copies
    const bool rev_in_kernel = !bidir && reversed_in_kernel(h->desc);
    // With in-kernel reversal, u and w (each with its own summary area) run on two
    // more streams beside dq: they start after everything enqueued so far on
    // hip_stream, and hip_stream waits for them before the finalize pass (all on
    // hip_stream if the streams cannot be made).
    const bool conc = rev_in_kernel && ensure_aux(h);
    if (conc) {
        if (hipEventRecord(h->fork, stream) != hipSuccess) return TTT_LA_ERR_HIP;
        for (int i = 0; i < 2; ++i)
            if (hipStreamWaitEvent(h->aux[i], h->fork, 0) != hipSuccess) return TTT_LA_ERR_HIP;
    }
    // dq: the forward with (q, k, v) -> (dO, v, k) and the caller's rates
    st = enqueue_forward(h, dO, v, k, eta, eta_scalar, beta, mode, nullptr, nullptr, dQ, nullptr, nullptr,
                         hip_stream, false);
    if (st != TTT_LA_OK) return st;
    void *U, *W;
    if (rev_in_kernel) {
        U = ws;
        W = ws + tb;
        char* ws_u = ws + 2 * tb;
        char* ws_w = ws_u + h->fp.summary_bytes;
        void* su = conc ? static_cast<void*>(h->aux[0]) : hip_stream;
        void* sw = conc ? static_cast<void*>(h->aux[1]) : hip_stream;
        st = enqueue_forward(h, k, q, dO, nullptr, 1.0f, beta, TTT_LA_CAUSAL, nullptr, nullptr, U, nullptr, nullptr,
                             su, false, true, ws_u);
        if (st != TTT_LA_OK) return st;
        st = enqueue_forward(h, v, dO, q, nullptr, 1.0f, beta, TTT_LA_CAUSAL, nullptr, nullptr, W, nullptr, nullptr,
                             sw, false, true, ws_w);
        if (st != TTT_LA_OK) return st;
        if (conc) {
            for (int i = 0; i < 2; ++i) {
                if (hipEventRecord(h->join[i], h->aux[i]) != hipSuccess) return TTT_LA_ERR_HIP;
                if (hipStreamWaitEvent(stream, h->join[i], 0) != hipSuccess) return TTT_LA_ERR_HIP;
            }
        }
    } else if (!bidir) {
        // rate-1 forwards over the reversed sequence: u from (k, q, dO), w from (v, dO, q)
        char *Rq = ws, *Rk = ws + tb, *Rv = ws + 2 * tb, *RdO = ws + 3 * tb;
        U = ws + 4 * tb;
        W = ws + 5 * tb;
        const void* src[4] = {q, k, v, dO};
        void* dst[4] = {Rq, Rk, Rv, RdO};
        if (ttt::launch_reverse(src, dst, 4, (size_t)h->desc.B * h->desc.H, h->desc.T,
                                h->desc.d_v * elem_bytes(h->desc.dtype), stream) != hipSuccess)
            return TTT_LA_ERR_HIP;
        st = enqueue_forward(h, Rk, Rq, RdO, nullptr, 1.0f, beta, TTT_LA_CAUSAL, nullptr, nullptr, U, nullptr,
                             nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
        st = enqueue_forward(h, Rv, RdO, Rq, nullptr, 1.0f, beta, TTT_LA_CAUSAL, nullptr, nullptr, W, nullptr,
                             nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
    } else {
        // every query reads the final state: rate-1, momentum-free bidirectional forwards
        U = ws;
        W = ws + tb;
        st = enqueue_forward(h, k, q, dO, nullptr, 1.0f, 0.0f, TTT_LA_BIDIRECTIONAL, nullptr, nullptr, U, nullptr,
                             nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
        st = enqueue_forward(h, v, dO, q, nullptr, 1.0f, 0.0f, TTT_LA_BIDIRECTIONAL, nullptr, nullptr, W, nullptr,
                             nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
    }
    ttt::BackArgs b{};
    b.u = U;
    b.w = W;
    b.v = v;
    b.eta = eta;
    b.dk = dK;
    b.dv = dV;
    b.deta = dEta;
    b.eta_scalar = eta_scalar;
    b.beta = beta;
    b.eta_kind = eta_kind_of(mode);
    b.causal = !bidir;
    b.uw_reversed = !bidir && !rev_in_kernel;
    b.stream = stream;
    return ttt::launch_finalize_grads(h->shape, b) == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

int ttt_la_forward(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                   float beta, uint32_t mode, void* o, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_forward(&h->desc, q, k, v, eta, eta_scalar, beta, mode, o);
    if (st != TTT_LA_OK) return st;
    return enqueue_forward(h, q, k, v, eta, eta_scalar, beta, mode, nullptr, nullptr, o, nullptr, nullptr,
                           hip_stream);
}

int ttt_la_forward_state(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta,
                         float eta_scalar, float beta, uint32_t mode, const float* S0, const float* M0, void* o,
                         float* S_T, float* M_T, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_forward_state(&h->desc, q, k, v, eta, eta_scalar, beta, mode, S0, M0, o, S_T, M_T);
    if (st != TTT_LA_OK) return st;
    // the prefix plan of the 32x32-tile kernels has no workspace for the entry state
    if (h->fast && h->fp.wide && h->fp.prefix) return TTT_LA_ERR_UNSUPPORTED;
    return enqueue_forward(h, q, k, v, eta, eta_scalar, beta, mode, S0, M0, o, S_T, M_T, hip_stream);
}

int ttt_la_step(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                float beta, uint32_t mode, float* S, float* M, void* o, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_step(&h->desc, q, k, v, eta, eta_scalar, beta, mode, S, M, o);
    if (st != TTT_LA_OK) return st;
    ttt::StepArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.eta = eta;
    a.eta_scalar = eta_scalar;
    a.beta = beta;
    a.eta_kind = eta_kind_of(mode);
    a.S = S;
    a.M = M;
    a.o = o;
    a.stream = static_cast<hipStream_t>(hip_stream);
    hipEvent_t eb, ee;
    next_events(h, &eb, &ee);
    const hipError_t e = ttt::launch_step(h->shape, a, eb, ee);
    return e == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

void ttt_la_destroy(ttt_la_t h) {
    if (!h) return;
    release_events(h);
    for (int i = 0; i < 2; ++i) {
        if (h->aux[i]) (void)hipStreamDestroy(h->aux[i]);
        if (h->join[i]) (void)hipEventDestroy(h->join[i]);
    }
    if (h->fork) (void)hipEventDestroy(h->fork);
    if (h->workspace) (void)hipFree(h->workspace);
    delete h;
}

int ttt_la_get_plan(ttt_la_t h, ttt_la_plan* plan) {
    if (!h || !plan) return TTT_LA_ERR_INVALID_ARG;
    std::memset(plan, 0, sizeof(*plan));
    const Shape& s = h->shape;
    plan->workspace_bytes = h->workspace_bytes;
    if (h->fast) {
        plan->path = h->fp.wide ? 2 : 1;
        plan->chunk = h->fp.chunk;
        plan->segments = h->fp.segments;
        plan->seg_len = h->fp.seg_len;
        plan->dv_split = h->fp.dv_split;
        plan->phi_split = h->fp.phi_split;
        plan->grid_main = s.n_seq() * h->fp.dv_split * h->fp.phi_split * h->fp.segments;
        plan->n_kernels = (h->fp.fused || h->fp.prefix) ? 1
                                      : 1 + (h->fp.segments > 1 ? 1 : 0) +
                                            (h->fp.segments > 2 || h->fp.sum_split == 2 ? 1 : 0) +
                                            (h->fp.phi_split > 1 ? 1 : 0);
    } else {
        plan->path = 0;
        plan->chunk = 16;
        plan->segments = 1;
        plan->seg_len = s.T;
        plan->dv_split = s.d_v / 16;
        plan->phi_split = 1;
        plan->grid_main = s.n_seq() * (s.d_v / 16);
        plan->n_kernels = 1;
    }
    return TTT_LA_OK;
}

int ttt_la_wait_status(ttt_la_t h, int32_t* failed) {
    if (!h || !failed) return TTT_LA_ERR_INVALID_ARG;
    *failed = 0;
    if (!(h->fast && h->fp.wide && h->fp.fused)) return TTT_LA_OK;
    unsigned flag = 0;
    const char* src = static_cast<const char*>(h->workspace) + ttt::wide_flag_offset(h->shape, h->fp);
    if (hipMemcpy(&flag, src, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) {
        (void)hipGetLastError();
        return TTT_LA_ERR_HIP;
    }
    *failed = flag != 0;
    return TTT_LA_OK;
}

int ttt_la_enable_kernel_timing(ttt_la_t h, int32_t n_slots) { return ttt_la_enable_kernel_timing_every(h, n_slots, 1); }

int ttt_la_enable_kernel_timing_every(ttt_la_t h, int32_t n_slots, int32_t every) {
    if (!h || n_slots < 0 || every < 1) return TTT_LA_ERR_INVALID_ARG;
    release_events(h);
    h->every = every;
    for (int32_t i = 0; i < n_slots; ++i) {
        // timestamps only: no system-scope fence (an L2 write-back) around the kernel
        hipEvent_t a = nullptr, b = nullptr;
        if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess ||
            hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            release_events(h);
            return TTT_LA_ERR_HIP;
        }
        h->ev_begin.push_back(a);
        h->ev_end.push_back(b);
    }
    return TTT_LA_OK;
}

int ttt_la_kernel_times(ttt_la_t h, float* ms, int32_t capacity, int32_t* count) {
    if (!h || !count || (capacity > 0 && !ms)) return TTT_LA_ERR_INVALID_ARG;
    *count = 0;
    const int slots = (int)h->ev_begin.size();
    if (slots == 0) return TTT_LA_OK;
    const int n = std::min(h->calls, slots);
    const int first = h->calls - n;  // oldest call still held
    for (int i = 0; i < n && *count < capacity; ++i) {
        const int slot = (first + i) % slots;
        if (hipEventSynchronize(h->ev_end[slot]) != hipSuccess) return TTT_LA_ERR_HIP;
        float t = 0.0f;
        if (hipEventElapsedTime(&t, h->ev_begin[slot], h->ev_end[slot]) != hipSuccess) return TTT_LA_ERR_HIP;
        ms[(*count)++] = t;
    }
    return TTT_LA_OK;
}

}  // extern "C"
