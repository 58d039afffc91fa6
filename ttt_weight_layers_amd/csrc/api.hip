// C ABI of libttt_la.so: validation, kernel plan, workspace, launches.
// The operation and every argument are documented in include/ttt_la.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "device_common.h"
#include "internal.h"
#include "ttt_la.h"

struct ttt_la_s {
    ttt_la_desc desc;
    ttt_la_hints hints;
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

constexpr uint32_t kModeMask =
    TTT_LA_BIDIRECTIONAL | TTT_LA_ETA_PER_TOKEN | TTT_LA_ETA_SOFTPLUS | TTT_LA_LOSS_MSE | TTT_LA_WEIGHT_NORM;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(int dtype) { return dtype == TTT_LA_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

Shape shape_of(const ttt_la_desc& d);

// a tensor of B*H*T*max(d_k, d_v, d_phi) elements reaches 2^31: such shapes run the
// plain and carried-state forwards on the 32x32-tile plan only
bool big_shape(const ttt_la_desc& d) {
    const long long widest = std::max(d.d_k, std::max(d.d_v, d.d_phi));
    return (long long)d.B * d.H * d.T * widest >= (1LL << 31);
}

int check_desc(const ttt_la_desc* d) {
    if (!d) return TTT_LA_ERR_INVALID_ARG;
    if (d->B < 1 || d->H < 1 || d->T < 1) return TTT_LA_ERR_INVALID_ARG;
    if (d->d_k < 1 || d->d_v < 1 || d->d_phi < 1) return TTT_LA_ERR_INVALID_ARG;
    if (d->dtype != TTT_LA_F32 && d->dtype != TTT_LA_BF16) return TTT_LA_ERR_INVALID_ARG;
    if (d->phi != TTT_LA_PHI_IDENTITY && d->phi != TTT_LA_PHI_SWIGLU) return TTT_LA_ERR_INVALID_ARG;
    if (d->chunk < 0) return TTT_LA_ERR_INVALID_ARG;
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
    // past 2^31 elements a tensor: only the 32x32-tile plan, whose kernels offset rows
    // in 64 bits (the token count itself stays below 2^31)
    if (big_shape(*d)) {
        if ((long long)d->B * d->H * d->T >= (1LL << 31)) return TTT_LA_ERR_UNSUPPORTED;
        if (!ttt::fast_supported(shape_of(*d), d->chunk) || !ttt::wide_supported(shape_of(*d)))
            return TTT_LA_ERR_UNSUPPORTED;
    }
    return TTT_LA_OK;
}

// plan hints; null = all automatic
int check_hints(const ttt_la_hints* h) {
    if (!h) return TTT_LA_OK;
    if (h->segments < 0) return TTT_LA_ERR_INVALID_ARG;
    if (h->value_split < 0 || h->value_split > 2) return TTT_LA_ERR_INVALID_ARG;
    if (h->launch < TTT_LA_LAUNCH_AUTO || h->launch > TTT_LA_LAUNCH_PREFIX) return TTT_LA_ERR_INVALID_ARG;
    return TTT_LA_OK;
}

ttt_la_hints hints_or_auto(const ttt_la_hints* h) {
    ttt_la_hints r{};
    if (h) r = *h;
    return r;
}

Shape shape_of(const ttt_la_desc& d);

int check_forward(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
                  float eta_scalar, float beta, uint32_t mode, const void* o, bool state_call = false) {
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
    // beyond 2^31 elements a tensor: the dot-product loss without weight normalisation
    if (big_shape(*d) && (mode & (TTT_LA_LOSS_MSE | TTT_LA_WEIGHT_NORM))) return TTT_LA_ERR_UNSUPPORTED;
    // the delta rule runs for one configuration (no momentum, causal, bf16 identity map,
    // square state of width 64 or 128)
    if ((mode & TTT_LA_LOSS_MSE) &&
        (beta != 0.0f || (mode & TTT_LA_BIDIRECTIONAL) || !ttt::delta_supported(shape_of(*d))))
        return TTT_LA_ERR_UNSUPPORTED;
    // weight normalisation: causal, dot-product loss (and an entry state: forward_state only)
    if (mode & TTT_LA_WEIGHT_NORM) {
        if (!state_call || (mode & (TTT_LA_BIDIRECTIONAL | TTT_LA_LOSS_MSE))) return TTT_LA_ERR_INVALID_ARG;
        if (!ttt::wn_supported(shape_of(*d))) return TTT_LA_ERR_UNSUPPORTED;
    }
    return TTT_LA_OK;
}

bool state_ok(const void* p) { return !p || aligned(p, 16); }

// ttt_la_forward_state: forward checks, causal only, state pointers aligned, outputs
// disjoint from everything except (in place) their own input
int check_forward_state(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
                        float eta_scalar, float beta, uint32_t mode, const float* S0, const float* M0, const void* o,
                        const float* S_T, const float* M_T) {
    int st = check_forward(d, q, k, v, eta, eta_scalar, beta, mode, o, true);
    if (st != TTT_LA_OK) return st;
    if (mode & TTT_LA_BIDIRECTIONAL) return TTT_LA_ERR_INVALID_ARG;
    // the delta rule carries S alone (it runs without momentum)
    if ((mode & TTT_LA_LOSS_MSE) && (M0 || M_T)) return TTT_LA_ERR_INVALID_ARG;
    if ((mode & TTT_LA_WEIGHT_NORM) && !S0) return TTT_LA_ERR_INVALID_ARG;   // the target row norms
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
    if ((mode & TTT_LA_LOSS_MSE) && (mode & TTT_LA_WEIGHT_NORM)) return TTT_LA_ERR_INVALID_ARG;
    // the delta-rule step holds a whole row of S in registers
    if ((mode & TTT_LA_LOSS_MSE) && !ttt::step_row_in_registers(shape_of(*d))) return TTT_LA_ERR_UNSUPPORTED;
    if ((mode & TTT_LA_WEIGHT_NORM) && !ttt::wn_supported(shape_of(*d))) return TTT_LA_ERR_UNSUPPORTED;
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
        case TTT_LA_ERR_TOO_LARGE: return "needs more scratch memory than the static maximum";
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

int ttt_la_check_hints(const ttt_la_hints* hints) { return check_hints(hints); }

int ttt_la_create(const ttt_la_desc* desc, ttt_la_t* out) { return ttt_la_create_hinted(desc, nullptr, out); }

int ttt_la_create_hinted(const ttt_la_desc* desc, const ttt_la_hints* hints, ttt_la_t* out) {
    if (!out) return TTT_LA_ERR_INVALID_ARG;
    *out = nullptr;
    int st = check_desc(desc);
    if (st != TTT_LA_OK) return st;
    if ((st = check_hints(hints)) != TTT_LA_OK) return st;

    ttt_la_s* h = new (std::nothrow) ttt_la_s();
    if (!h) return TTT_LA_ERR_OOM;
    h->desc = *desc;
    h->hints = hints_or_auto(hints);
    h->shape = shape_of(*desc);
    h->workspace = nullptr;
    h->workspace_bytes = 0;
    h->calls = 0;
    h->every = 1;
    h->seen = 0;
    h->epoch = 0;
    h->fast = desc->dtype == TTT_LA_BF16 && ttt::fast_supported(h->shape, desc->chunk);
    if (h->fast) {
        h->fp = ttt::fast_plan(h->shape, desc->chunk, h->hints.segments, h->hints.value_split, h->hints.launch);
        h->workspace_bytes = h->fp.summary_bytes + h->fp.partial_bytes + h->fp.zero_bytes;
    }
    // the weight-normalised recurrence puts the SwiGLU features of q and k at the start of
    // the workspace (the plan's areas are not in use during that call)
    if (ttt::wn_supported(h->shape))
        h->workspace_bytes = std::max(h->workspace_bytes, ttt::wn_workspace_bytes(h->shape));
    // so does the delta rule its chunk inverses (not past 2^31 elements, where the
    // delta rule is not run)
    if (!big_shape(*desc)) h->workspace_bytes = std::max(h->workspace_bytes, ttt::delta_workspace_bytes(h->shape));
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return TTT_LA_ERR_HIP;
    }
    if (!h->fast && ttt::generic_smem_bytes(h->shape) > 160 * 1024) {
        delete h;
        return TTT_LA_ERR_UNSUPPORTED;
    }
    // past 2^31 elements only the 32x32-tile plan (a value-split hint picks another)
    if (big_shape(*desc) && !(h->fast && h->fp.wide)) {
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
    if (mode & TTT_LA_WEIGHT_NORM) {
        // validated by check_forward_state: the recurrent kernel (the SwiGLU features go
        // to the handle's workspace first)
        if (ttt::wn_workspace_bytes(h->shape) > h->workspace_bytes || reverse) return TTT_LA_ERR_UNSUPPORTED;
        e = ttt::launch_wn(h->shape, h->workspace, a, eb, ee);
    } else if (mode & TTT_LA_LOSS_MSE) {
        // validated by check_forward: the chunk inverses go to the handle's workspace
        e = ttt::launch_delta(h->shape, a, h->workspace, h->workspace_bytes, eb, ee);
    } else if (h->fast && (h->fp.wide || !state_io)) {
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
        if (!state_io && ttt::short_supported(h->shape)) e = ttt::launch_short(h->shape, a, eb, ee);
        else e = ttt::launch_generic(h->shape, a, eb, ee);
    }
    return e == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

bool backward_supported(const ttt_la_desc& d) { return d.phi == TTT_LA_PHI_IDENTITY; }

// one [B, H, T, d_v] tensor in the handle's dtype (v, dO, dv); key_bytes: [B, H, T, d_k]
size_t tensor_bytes(const ttt_la_desc& d) { return (size_t)d.B * d.H * d.T * d.d_v * elem_bytes(d.dtype); }
size_t key_bytes(const ttt_la_desc& d) { return (size_t)d.B * d.H * d.T * d.d_k * elem_bytes(d.dtype); }

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// The forwards of the backward that produce dq and dk run with queries and keys of width
// d_v and values of width d_k: for d_k != d_v that is another shape, with its own plan
// and segment-summary area in the workspace.
Shape swapped_shape(const ttt_la_desc& d) {
    Shape s = shape_of(d);
    s.d_k = d.d_v;
    s.d_v = d.d_k;
    s.d_phi = d.d_v;
    return s;
}

size_t swapped_area(const ttt_la_desc& d, const ttt_la_hints& hn) {
    if (d.d_k == d.d_v) return 0;
    const Shape ss = swapped_shape(d);
    if (d.dtype != TTT_LA_BF16 || !ttt::fast_supported(ss, d.chunk)) return 0;
    const ttt::FastPlan p = ttt::fast_plan(ss, d.chunk, hn.segments, hn.value_split, hn.launch);
    return align256(p.summary_bytes + p.partial_bytes + p.zero_bytes);
}

// one forward of the swapped shape (no carried state, not reversed in the kernel)
hipError_t swapped_forward(const ttt_la_desc& d, const ttt_la_hints& hn, void* area, const void* q, const void* k,
                           const void* v, const float* eta, float eta_scalar, float beta, uint32_t mode, void* o,
                           hipStream_t st) {
    const Shape ss = swapped_shape(d);
    ttt::FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.eta = eta;
    a.eta_scalar = eta_scalar;
    a.beta = beta;
    a.eta_kind = eta_kind_of(mode);
    a.bidirectional = (mode & TTT_LA_BIDIRECTIONAL) != 0;
    a.o = o;
    a.stream = st;
    if (d.dtype == TTT_LA_BF16 && ttt::fast_supported(ss, d.chunk)) {
        ttt::FastPlan p = ttt::fast_plan(ss, d.chunk, hn.segments, hn.value_split, hn.launch);
        p.fused = false;   // its counters would need a zeroed area of their own
        return ttt::launch_fast(ss, p, area, a, nullptr, nullptr, nullptr);
    }
    if (ttt::short_supported(ss)) return ttt::launch_short(ss, a, nullptr, nullptr);
    return ttt::launch_generic(ss, a, nullptr, nullptr);
}

// The 32x32-tile plans of three launches (decided from the descriptor alone: a
// single or prefix launch was not asked for) read the time-reversed operands in
// reverse order themselves.
bool reversed_in_kernel(const ttt_la_desc& d, const ttt_la_hints& hn) {
    const Shape s = shape_of(d);
    return d.dtype == TTT_LA_BF16 && ttt::fast_supported(s, d.chunk) && ttt::wide_supported(s) &&
           hn.value_split != 2 && hn.launch != TTT_LA_LAUNCH_SINGLE && hn.launch != TTT_LA_LAUNCH_PREFIX;
}

// Workspace of the backward.  Bidirectional: the two forward outputs.  Causal,
// reversed in the kernels: the two forward outputs, then a segment-summary area
// for each of the two reversed forwards (they run beside the first one, which uses
// the handle's).  Causal otherwise: q, k, v, dO reversed in time, then the outputs.
size_t backward_ws_bytes(const ttt_la_desc& d, const ttt_la_hints& hn, uint32_t mode) {
    const size_t vb = align256(tensor_bytes(d)), kb = align256(key_bytes(d));
    if (mode & TTT_LA_BIDIRECTIONAL) return vb + kb + swapped_area(d, hn);
    if (reversed_in_kernel(d, hn)) {
        const ttt::FastPlan p = ttt::fast_plan(shape_of(d), d.chunk, hn.segments, hn.value_split, hn.launch);
        return 2 * tensor_bytes(d) + 2 * p.summary_bytes;
    }
    // reversed q, k, v, dO, then U (d_v wide) and W (d_k wide), then the swapped plan's area
    return 3 * (kb + vb) + swapped_area(d, hn);
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

int check_backward(const ttt_la_desc* d, const ttt_la_hints& hn, const void* q, const void* k, const void* v, const float* eta,
                   float eta_scalar, float beta, uint32_t mode, const void* dO, const void* dQ, const void* dK,
                   const void* dV, const float* dEta, const void* ws, size_t ws_bytes) {
    int st = check_forward(d, q, k, v, eta, eta_scalar, beta, mode, dQ);
    if (st == TTT_LA_OK && (mode & TTT_LA_LOSS_MSE)) return TTT_LA_ERR_UNSUPPORTED;   // no delta-rule backward
    if (st != TTT_LA_OK) return st;
    if (big_shape(*d)) return TTT_LA_ERR_UNSUPPORTED;
    if (!backward_supported(*d)) return TTT_LA_ERR_UNSUPPORTED;
    if (!dO || !dK || !dV) return TTT_LA_ERR_INVALID_ARG;
    if (!aligned(dO, 16) || !aligned(dK, 16) || !aligned(dV, 16)) return TTT_LA_ERR_INVALID_ARG;
    if (dEta && !aligned(dEta, 4)) return TTT_LA_ERR_INVALID_ARG;
    const size_t need = backward_ws_bytes(*d, hn, mode);
    if (need && (!ws || !aligned(ws, 16) || ws_bytes < need)) return TTT_LA_ERR_INVALID_ARG;
    const size_t tb = tensor_bytes(*d), kb = key_bytes(*d);
    const size_t nt = (size_t)d->B * d->H * d->T;
    const size_t eta_bytes = eta ? nt * sizeof(float) : 0;
    const void* outs[4] = {dQ, dK, dV, dEta};
    const size_t out_bytes[4] = {kb, kb, tb, nt * sizeof(float)};
    const void* ins[5] = {q, k, v, dO, eta};
    const size_t in_bytes[5] = {kb, kb, tb, tb, eta_bytes};
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

// ---- backward through the SwiGLU feature map ----

// Workspace of ttt_la_backward_swiglu (offsets in bytes, each 256-aligned), rows = B H T,
// P = d_phi / 128 feature slices:
//   phi_q, phi_k   P x rows x 128 bf16: the features, slice-major
//   dphi_q         P x rows x 128: dL/dphi(q), slice by slice
//   w              P x rows x 128: dL/dphi(k) / (eta c), slice by slice
//   u              rows x 128: the rate-1 forward giving dv and the rate gradient
//   rq, rk, rdo    rows x 128 each (causal only): q, k, dO reversed in time
//   sum            segment summaries of the feature-space forwards (d = 128 plan)
//   part           per-slice partial outputs of the SwiGLU forward
//   dwpart         fp32 partial sums of dW1, dW3
struct SwBwdLayout {
    size_t phi_q, phi_k, dphi_q, w, u, rq, rk, rdo, sum, part, dwpart, total;
};

Shape feature_shape(const Shape& s) {
    Shape f = s;
    f.swiglu = false;
    f.d_k = f.d_v = f.d_phi = 128;
    f.w1 = f.w3 = nullptr;
    return f;
}

SwBwdLayout swiglu_bwd_layout(const ttt_la_desc& d, uint32_t mode) {
    const Shape s = shape_of(d);
    const size_t rows = (size_t)s.n_seq() * s.T, P = s.d_phi / 128, E = 2;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    SwBwdLayout L{};
    L.phi_q = take(P * rows * 128 * E);
    L.phi_k = take(P * rows * 128 * E);
    L.dphi_q = take(P * rows * 128 * E);
    L.w = take(P * rows * 128 * E);
    L.u = take(rows * 128 * E);
    if (!(mode & TTT_LA_BIDIRECTIONAL)) {
        L.rq = take(rows * 128 * E);
        L.rk = take(rows * 128 * E);
        L.rdo = take(rows * 128 * E);
    }
    L.sum = take(ttt::fast_plan(feature_shape(s), 0, 0, 0, 0).summary_bytes);
    L.part = take(ttt::fast_plan(s, d.chunk, 0, 0, 0).partial_bytes);
    L.dwpart = take(ttt::swiglu_chain_dw_partial_bytes(s));
    L.total = off;
    return L;
}

bool swiglu_backward_ok(const ttt_la_desc& d) {
    return d.phi == TTT_LA_PHI_SWIGLU && ttt::swiglu_backward_supported(shape_of(d));
}

int check_backward_swiglu(const ttt_la_desc* d, const void* q, const void* k, const void* v, const float* eta,
                          float eta_scalar, float beta, uint32_t mode, const void* dO, const void* dQ, const void* dK,
                          const void* dV, const float* dEta, const float* dW1, const float* dW3, const void* ws,
                          size_t ws_bytes) {
    int st = check_forward(d, q, k, v, eta, eta_scalar, beta, mode, dQ);
    if (st != TTT_LA_OK) return st;
    if (big_shape(*d)) return TTT_LA_ERR_UNSUPPORTED;
    if (mode & TTT_LA_LOSS_MSE) return TTT_LA_ERR_UNSUPPORTED;
    if (!swiglu_backward_ok(*d)) return TTT_LA_ERR_UNSUPPORTED;
    if (!dO || !dQ || !dK || !dV || !dW1 || !dW3) return TTT_LA_ERR_INVALID_ARG;
    if (!aligned(dO, 16) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(dW1, 16) ||
        !aligned(dW3, 16))
        return TTT_LA_ERR_INVALID_ARG;
    if (dEta && !aligned(dEta, 4)) return TTT_LA_ERR_INVALID_ARG;
    const size_t need = swiglu_bwd_layout(*d, mode).total;
    if (!ws || !aligned(ws, 256) || ws_bytes < need) return TTT_LA_ERR_INVALID_ARG;
    const size_t tb = tensor_bytes(*d);
    const size_t nt = (size_t)d->B * d->H * d->T;
    const size_t wb = (size_t)d->H * d->d_phi * d->d_k * sizeof(float);
    const size_t w_in = (size_t)d->H * d->d_phi * d->d_k * 2;
    const void* outs[6] = {dQ, dK, dV, dEta, dW1, dW3};
    const size_t out_bytes[6] = {tb, tb, tb, nt * sizeof(float), wb, wb};
    const void* ins[7] = {q, k, v, dO, eta, d->w1, d->w3};
    const size_t in_bytes[7] = {tb, tb, tb, tb, eta ? nt * sizeof(float) : 0, w_in, w_in};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return TTT_LA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return TTT_LA_ERR_INVALID_ARG;
        if (overlaps(outs[i], out_bytes[i], ws, need)) return TTT_LA_ERR_INVALID_ARG;
    }
    for (int j = 0; j < 7; ++j)
        if (overlaps(ws, need, ins[j], in_bytes[j])) return TTT_LA_ERR_INVALID_ARG;
    return TTT_LA_OK;
}

// one forward of the d = 128 identity plan on feature slices (no handle state touched)
hipError_t feature_forward(const Shape& sf, const ttt::FastPlan& pf, void* ws_sum, const void* q, const void* k,
                           const void* v, const float* eta, float eta_scalar, float beta, int eta_kind, bool bidir,
                           bool reverse, void* o, hipStream_t st) {
    ttt::FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.eta = eta;
    a.eta_scalar = eta_scalar;
    a.beta = beta;
    a.eta_kind = eta_kind;
    a.bidirectional = bidir;
    a.reverse = reverse;
    a.o = o;
    a.stream = st;
    return ttt::launch_fast(sf, pf, ws_sum, a, nullptr, nullptr, nullptr);
}

}  // namespace

extern "C" {

int ttt_la_check_backward(const ttt_la_desc* desc, const ttt_la_hints* hints, const void* q, const void* k,
                          const void* v, const float* eta, float eta_scalar, float beta, uint32_t mode,
                          const void* dO, const void* dQ, const void* dK, const void* dV, const float* dEta,
                          const void* workspace, size_t workspace_bytes) {
    int st = check_desc(desc);
    if (st != TTT_LA_OK) return st;
    if ((st = check_hints(hints)) != TTT_LA_OK) return st;
    return check_backward(desc, hints_or_auto(hints), q, k, v, eta, eta_scalar, beta, mode, dO, dQ, dK, dV, dEta, workspace,
                          workspace_bytes);
}

int ttt_la_backward_workspace(ttt_la_t h, uint32_t mode, size_t* bytes) {
    if (!h || !bytes) return TTT_LA_ERR_INVALID_ARG;
    *bytes = 0;
    if (mode & ~kModeMask) return TTT_LA_ERR_INVALID_ARG;
    if (swiglu_backward_ok(h->desc)) {
        *bytes = swiglu_bwd_layout(h->desc, mode).total;
        return TTT_LA_OK;
    }
    if (!backward_supported(h->desc)) return TTT_LA_ERR_UNSUPPORTED;
    *bytes = backward_ws_bytes(h->desc, h->hints, mode);
    return TTT_LA_OK;
}

int ttt_la_backward_swiglu(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta,
                           float eta_scalar, float beta, uint32_t mode, const void* dO, void* dQ, void* dK, void* dV,
                           float* dEta, float* dW1, float* dW3, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_backward_swiglu(&h->desc, q, k, v, eta, eta_scalar, beta, mode, dO, dQ, dK, dV, dEta, dW1, dW3,
                                   workspace, workspace_bytes);
    if (st != TTT_LA_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const bool bidir = (mode & TTT_LA_BIDIRECTIONAL) != 0;
    const int kind = eta_kind_of(mode);
    const Shape& s = h->shape;
    const Shape sf = feature_shape(s);
    const ttt::FastPlan pf = ttt::fast_plan(sf, 0, 0, 0, 0);
    const SwBwdLayout L = swiglu_bwd_layout(h->desc, mode);
    char* ws = static_cast<char*>(workspace);
    const size_t rows = (size_t)s.n_seq() * s.T, slice = rows * 128 * 2;
    const int P = s.d_phi / 128;
    auto ok = [](hipError_t e) { return e == hipSuccess; };
#define TTT_TRY(x)                     \
    do {                               \
        if (!ok(x)) {                  \
            (void)hipGetLastError();   \
            return TTT_LA_ERR_HIP;     \
        }                              \
    } while (0)
    TTT_TRY(ttt::launch_swiglu_features(s, q, ws + L.phi_q, stream));
    TTT_TRY(ttt::launch_swiglu_features(s, k, ws + L.phi_k, stream));
    for (int p = 0; p < P; ++p) {
        // dL/dphi(q): the forward with (q, k, v) -> (dO, v, phi(k)) and the caller's rates
        TTT_TRY(feature_forward(sf, pf, ws + L.sum, dO, v, ws + L.phi_k + p * slice, eta, eta_scalar, beta, kind,
                                bidir, false, ws + L.dphi_q + p * slice, stream));
        // w: rate-1 forward of (v, dO, phi(q)), over the reversed sequence when causal (the
        // d = 128 kernels read and write the rows in reverse order themselves)
        TTT_TRY(feature_forward(sf, pf, ws + L.sum, v, dO, ws + L.phi_q + p * slice, nullptr, 1.0f,
                                bidir ? 0.0f : beta, 0, bidir, !bidir, ws + L.w + p * slice, stream));
    }
    // u: rate-1 SwiGLU forward of (k, q, dO), over reversed copies when causal
    {
        ttt::FwdArgs a{};
        a.eta = nullptr;
        a.eta_scalar = 1.0f;
        a.eta_kind = 0;
        a.bidirectional = bidir;
        a.beta = bidir ? 0.0f : beta;
        a.o = ws + L.u;
        a.stream = stream;
        if (bidir) {
            a.q = k;
            a.k = q;
            a.v = dO;
        } else {
            const void* src[3] = {q, k, dO};
            void* dst[3] = {ws + L.rq, ws + L.rk, ws + L.rdo};
            TTT_TRY(ttt::launch_reverse(src, dst, 3, (size_t)s.n_seq(), s.T, 128 * 2, stream));
            a.q = ws + L.rk;
            a.k = ws + L.rq;
            a.v = ws + L.rdo;
        }
        TTT_TRY(ttt::launch_fast(s, h->fp, ws + L.part, a, nullptr, nullptr, nullptr));
    }
    // dv and the rate gradient from u
    {
        ttt::BackArgs b{};
        b.u = ws + L.u;
        b.w = ws + L.u;
        b.v = v;
        b.eta = eta;
        b.dk = nullptr;
        b.dv = dV;
        b.deta = dEta;
        b.eta_scalar = eta_scalar;
        b.beta = beta;
        b.eta_kind = kind;
        b.causal = !bidir;
        b.uw_reversed = !bidir;
        b.stream = stream;
        TTT_TRY(ttt::launch_finalize_grads(s, b));
    }
    // through phi: dq from q and dphi(q), dk from k and w scaled by eta c, then dW1, dW3 from both
    TTT_TRY(ttt::launch_swiglu_chain_dx(s, q, ws + L.dphi_q, dQ, eta, eta_scalar, beta, kind, false, bidir, stream));
    TTT_TRY(ttt::launch_swiglu_chain_dx(s, k, ws + L.w, dK, eta, eta_scalar, beta, kind, true, bidir, stream));
    TTT_TRY(ttt::launch_swiglu_chain_dw(s, q, k, ws + L.dphi_q, ws + L.w, eta, eta_scalar, beta, kind, bidir,
                                        reinterpret_cast<float*>(ws + L.dwpart), dW1, dW3, stream));
#undef TTT_TRY
    return TTT_LA_OK;
}

int ttt_la_backward(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                    float beta, uint32_t mode, const void* dO, void* dQ, void* dK, void* dV, float* dEta,
                    void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_backward(&h->desc, h->hints, q, k, v, eta, eta_scalar, beta, mode, dO, dQ, dK, dV, dEta, workspace,
                            workspace_bytes);
    if (st != TTT_LA_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const bool bidir = (mode & TTT_LA_BIDIRECTIONAL) != 0;
    const size_t tb = tensor_bytes(h->desc);
    char* ws = static_cast<char*>(workspace);
    // the 32x32-tile kernels of three launches read and write in reverse time order
    // themselves; the other plans get reversed copies
    const bool rev_in_kernel = !bidir && reversed_in_kernel(h->desc, h->hints);
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
    const ttt_la_desc& dd = h->desc;
    const bool swapped = dd.d_k != dd.d_v;
    const size_t vb = align256(tb), kb = align256(key_bytes(dd));
    // the swapped shape's summary area sits at the end of the workspace
    void* sw_area = swapped ? ws + backward_ws_bytes(dd, h->hints, mode) - swapped_area(dd, h->hints) : nullptr;
    auto fwd_swapped = [&](const void* q_, const void* k_, const void* v_, const float* e_, float es_, float b_,
                           uint32_t m_, void* o_) {
        return swapped_forward(dd, h->hints, sw_area, q_, k_, v_, e_, es_, b_, m_, o_, stream) == hipSuccess
                   ? TTT_LA_OK
                   : TTT_LA_ERR_HIP;
    };
    // dq: the forward with (q, k, v) -> (dO, v, k) and the caller's rates (queries and
    // keys of width d_v, values of width d_k)
    st = swapped ? fwd_swapped(dO, v, k, eta, eta_scalar, beta, mode, dQ)
                 : enqueue_forward(h, dO, v, k, eta, eta_scalar, beta, mode, nullptr, nullptr, dQ, nullptr, nullptr,
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
        char *Rq = ws, *Rk = ws + kb, *Rv = ws + 2 * kb, *RdO = ws + 2 * kb + vb;
        U = ws + 2 * kb + 2 * vb;
        W = ws + 2 * kb + 3 * vb;
        const void* src_k[2] = {q, k};
        void* dst_k[2] = {Rq, Rk};
        const void* src_v[2] = {v, dO};
        void* dst_v[2] = {Rv, RdO};
        const size_t eb = elem_bytes(dd.dtype);
        if (ttt::launch_reverse(src_k, dst_k, 2, (size_t)dd.B * dd.H, dd.T, dd.d_k * eb, stream) != hipSuccess ||
            ttt::launch_reverse(src_v, dst_v, 2, (size_t)dd.B * dd.H, dd.T, dd.d_v * eb, stream) != hipSuccess)
            return TTT_LA_ERR_HIP;
        st = enqueue_forward(h, Rk, Rq, RdO, nullptr, 1.0f, beta, TTT_LA_CAUSAL, nullptr, nullptr, U, nullptr,
                             nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
        st = swapped ? fwd_swapped(Rv, RdO, Rq, nullptr, 1.0f, beta, TTT_LA_CAUSAL, W)
                     : enqueue_forward(h, Rv, RdO, Rq, nullptr, 1.0f, beta, TTT_LA_CAUSAL, nullptr, nullptr, W,
                                       nullptr, nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
    } else {
        // every query reads the final state: rate-1, momentum-free bidirectional forwards
        U = ws;
        W = ws + vb;
        st = enqueue_forward(h, k, q, dO, nullptr, 1.0f, 0.0f, TTT_LA_BIDIRECTIONAL, nullptr, nullptr, U, nullptr,
                             nullptr, hip_stream, false);
        if (st != TTT_LA_OK) return st;
        st = swapped ? fwd_swapped(v, dO, q, nullptr, 1.0f, 0.0f, TTT_LA_BIDIRECTIONAL, W)
                     : enqueue_forward(h, v, dO, q, nullptr, 1.0f, 0.0f, TTT_LA_BIDIRECTIONAL, nullptr, nullptr, W,
                                       nullptr, nullptr, hip_stream, false);
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
    if (!swapped) return ttt::launch_finalize_grads(h->shape, b) == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
    // widths differ: dv and the rate gradient from u (d_v wide), then dk from w (d_k wide)
    b.dk = nullptr;
    if (ttt::launch_finalize_grads(h->shape, b) != hipSuccess) return TTT_LA_ERR_HIP;
    ttt::BackArgs bk = b;
    bk.u = W;
    bk.w = W;
    bk.v = W;           // read for the rate term only, which this pass does not write
    bk.dv = dK;
    bk.deta = nullptr;
    Shape sk = h->shape;
    sk.d_v = dd.d_k;
    return ttt::launch_finalize_grads(sk, bk) == hipSuccess ? TTT_LA_OK : TTT_LA_ERR_HIP;
}

int ttt_la_forward(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                   float beta, uint32_t mode, void* o, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_forward(&h->desc, q, k, v, eta, eta_scalar, beta, mode, o);
    if (st != TTT_LA_OK) return st;
    return enqueue_forward(h, q, k, v, eta, eta_scalar, beta, mode, nullptr, nullptr, o, nullptr, nullptr,
                           hip_stream);
}

}  // extern "C"

// ---- forward without allocation: scratch in a static device array ----

namespace {

// One copy per device, allocated by the runtime with the code object and held until
// the process ends.  In host code `scratch` names a host-side stand-in: only the
// address hipGetSymbolAddress returns for the current device may reach a kernel.
static __device__ __align__(256) unsigned char scratch[TTT_LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// this device's copy of the array, resolved on the first call on the device
int device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return TTT_LA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return TTT_LA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return TTT_LA_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TTT_LA_OK;
}

}  // namespace

extern "C" {

int ttt_la_forward_noalloc(const ttt_la_desc* desc, const ttt_la_hints* hints, const void* q, const void* k,
                           const void* v, const float* eta, float eta_scalar, float beta, uint32_t mode, void* o,
                           void* hip_stream) {
    int st = check_desc(desc);
    if (st != TTT_LA_OK) return st;
    if ((st = check_hints(hints)) != TTT_LA_OK) return st;
    if ((st = check_forward(desc, q, k, v, eta, eta_scalar, beta, mode, o)) != TTT_LA_OK) return st;
    const Shape s = shape_of(*desc);
    const ttt_la_hints hn = hints_or_auto(hints);
    ttt::FwdArgs a{};
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
    hipError_t e;
    if (mode & TTT_LA_LOSS_MSE) {
        // the chunk inverses in the scratch array when they fit, else the one-pass walk
        const size_t need = ttt::delta_workspace_bytes(s);
        void* ws = nullptr;
        if (need && need <= TTT_LA_NOALLOC_SCRATCH_BYTES && (st = device_scratch(&ws)) != TTT_LA_OK) return st;
        e = ttt::launch_delta(s, a, ws, ws ? (size_t)TTT_LA_NOALLOC_SCRATCH_BYTES : 0, nullptr, nullptr);
    } else if (desc->dtype == TTT_LA_BF16 && ttt::fast_supported(s, desc->chunk)) {
        ttt::FastPlan p = ttt::fast_plan(s, desc->chunk, hn.segments, hn.value_split, hn.launch);
        if (big_shape(*desc) && !p.wide) return TTT_LA_ERR_UNSUPPORTED;
        // the single-launch form keeps counters that must persist from call to call
        // of one handle: three launches instead, which compute the same
        p.fused = false;
        const size_t need = p.summary_bytes + p.partial_bytes;
        if (need > TTT_LA_NOALLOC_SCRATCH_BYTES) return TTT_LA_ERR_TOO_LARGE;
        void* ws = nullptr;
        if (need && (st = device_scratch(&ws)) != TTT_LA_OK) return st;
        e = ttt::launch_fast(s, p, ws, a, nullptr, nullptr, nullptr);
    } else {
        if (ttt::short_supported(s)) {
            e = ttt::launch_short(s, a, nullptr, nullptr);
        } else {
            if (ttt::generic_smem_bytes(s) > 160 * 1024) return TTT_LA_ERR_UNSUPPORTED;
            e = ttt::launch_generic(s, a, nullptr, nullptr);
        }
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return TTT_LA_ERR_HIP;
    }
    return TTT_LA_OK;
}

int ttt_la_forward_state(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta,
                         float eta_scalar, float beta, uint32_t mode, const float* S0, const float* M0, void* o,
                         float* S_T, float* M_T, void* hip_stream) {
    if (!h) return TTT_LA_ERR_INVALID_ARG;
    int st = check_forward_state(&h->desc, q, k, v, eta, eta_scalar, beta, mode, S0, M0, o, S_T, M_T);
    if (st != TTT_LA_OK) return st;
    // the prefix plan of the 32x32-tile kernels has no workspace for the entry state
    // (the delta rule has kernels of its own, outside the plan)
    if (!(mode & TTT_LA_LOSS_MSE) && h->fast && h->fp.wide && h->fp.prefix) return TTT_LA_ERR_UNSUPPORTED;
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
    a.weight_norm = (mode & TTT_LA_WEIGHT_NORM) != 0;
    a.mse = (mode & TTT_LA_LOSS_MSE) != 0;
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
        plan->path = h->fp.wide ? 2 : (h->fp.swiglu32 ? 3 : 1);
        plan->chunk = h->fp.chunk;
        plan->segments = h->fp.segments;
        plan->seg_len = h->fp.seg_len;
        plan->dv_split = h->fp.dv_split;
        plan->phi_split = h->fp.phi_split;
        plan->grid_main = s.n_seq() * h->fp.dv_split * h->fp.phi_split * h->fp.segments;
        plan->n_kernels = h->fp.swiglu32 ? 2
                          : (h->fp.fused || h->fp.prefix) ? 1
                                      : 1 + (h->fp.segments > 1 ? 1 : 0) +
                                            (h->fp.segments > 2 || h->fp.sum_split == 2 ? 1 : 0) +
                                            (h->fp.phi_split > 1 ? 1 : 0);
    } else if (ttt::short_supported(s)) {
        // forwards without carried state; the carried-state calls take path 0
        plan->path = 4;
        plan->chunk = 64;
        plan->segments = 1;
        plan->seg_len = s.T;
        plan->dv_split = s.d_v / 64;
        plan->phi_split = 1;
        plan->grid_main = ttt::short_grid(s);
        plan->n_kernels = 1;
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
    if (flag != 0) {
        // reported once: the flag covers the forwards since the previous read
        if (hipMemset(const_cast<char*>(src), 0, sizeof(flag)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            return TTT_LA_ERR_HIP;
        }
    }
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
