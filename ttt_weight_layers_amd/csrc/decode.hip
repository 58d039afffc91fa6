// One recurrent step of the TTT layer (decode): for every sequence (b, h) a
// single new token updates the carried fast weight and is read out,
//
//   M <- beta M + eta v phi(k)^T,   S <- S + M,   o = S phi(q),
//
// the token-by-token form that Table 2 of the thelatestinai.com page lists as
// the recurrent implementation of each variant (per-token lr and momentum in
// SGD; the SwiGLU feature map of Variant 2), one gradient step per entry on a
// fixed-size matrix (wpnews.pro commentary).
//
// The step reads and writes the whole fp32 state once and does under half a
// flop per byte of it: it is bound by HBM bandwidth.  One workgroup of four waves owns 16
// value rows of one sequence's S and M; each wave walks four rows, its 64 lanes
// covering consecutive features (8 bytes a lane, 512 bytes a wave access), and
// reduces the readout of each row across the wave.  The features
// phi(q), phi(k) of the token are formed once per workgroup in LDS (the SwiGLU
// map as two fp32 dot products per feature against the frozen W1, W3 rows).

#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace ttt {
namespace {

constexpr int SR = 16;          // value rows per workgroup
constexpr int STHREADS = 256;   // four waves, four rows each

struct StepParams {
    const void* q;
    const void* k;
    const void* v;
    const float* eta;
    const void* w1;
    const void* w3;
    void* o;
    float* S;
    float* M;
    float eta_scalar;
    float beta;
    int eta_kind;
    int H, d_k, d_v, d_phi;
    int n_rblk;                 // row blocks per sequence (d_v / SR)
};

template <typename TI, bool SWIGLU>
__global__ void __launch_bounds__(STHREADS) step_kernel(StepParams p) {
    extern __shared__ float smem[];
    const int d_k = p.d_k, d_phi = p.d_phi;
    float* sPq = smem;                 // phi(q) [d_phi]
    float* sPk = sPq + d_phi;          // phi(k) [d_phi]
    float* sXq = sPk + d_phi;          // SwiGLU: raw q, k [d_k] each
    float* sXk = sXq + d_k;

    const int tid = threadIdx.x;
    const int seq = blockIdx.x / p.n_rblk;
    const int r0 = (blockIdx.x % p.n_rblk) * SR;
    const TI* q = static_cast<const TI*>(p.q) + (size_t)seq * d_k;
    const TI* k = static_cast<const TI*>(p.k) + (size_t)seq * d_k;
    const TI* v = static_cast<const TI*>(p.v) + (size_t)seq * p.d_v;
    TI* o = static_cast<TI*>(p.o) + (size_t)seq * p.d_v;

    if constexpr (!SWIGLU) {
        for (int f = tid; f < d_phi; f += STHREADS) {
            sPq[f] = load_as_f32(q, f);
            sPk[f] = load_as_f32(k, f);
        }
    } else {
        const int h = seq % p.H;
        const TI* w1 = static_cast<const TI*>(p.w1) + (size_t)h * d_phi * d_k;
        const TI* w3 = static_cast<const TI*>(p.w3) + (size_t)h * d_phi * d_k;
        for (int d = tid; d < d_k; d += STHREADS) {
            sXq[d] = load_as_f32(q, d);
            sXk[d] = load_as_f32(k, d);
        }
        __syncthreads();
        // phi(x)_f = silu(W1_f . x) (W3_f . x)
        for (int f = tid; f < d_phi; f += STHREADS) {
            float uq = 0.f, gq = 0.f, uk = 0.f, gk = 0.f;
            for (int d = 0; d < d_k; ++d) {
                const float a = load_as_f32(w1, (size_t)f * d_k + d);
                const float b = load_as_f32(w3, (size_t)f * d_k + d);
                uq = fmaf(a, sXq[d], uq);
                gq = fmaf(b, sXq[d], gq);
                uk = fmaf(a, sXk[d], uk);
                gk = fmaf(b, sXk[d], gk);
            }
            sPq[f] = silu_f32(uq) * gq;
            sPk[f] = silu_f32(uk) * gk;
        }
    }
    __syncthreads();

    const float et = eta_at(p.eta_kind, p.eta, p.eta_scalar, (size_t)seq);
    const float beta = p.beta;
    const int lane = tid & 63, wave = tid >> 6;
    for (int rr = 0; rr < SR / 4; ++rr) {
        const int row = r0 + 4 * wave + rr;
        const float ev = et * load_as_f32(v, row);
        float* Sr = p.S + ((size_t)seq * p.d_v + row) * d_phi;
        float* Mr = p.M + ((size_t)seq * p.d_v + row) * d_phi;
        float acc = 0.0f;
        // two consecutive features a lane, 512 bytes a wave access (d_phi is a
        // multiple of 64: every pair is whole)
        for (int c = 2 * lane; c < d_phi; c += 128) {
            f32x2 m = *reinterpret_cast<const f32x2*>(Mr + c);
            f32x2 s = *reinterpret_cast<const f32x2*>(Sr + c);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                m[e] = fmaf(beta, m[e], ev * sPk[c + e]);
                s[e] += m[e];
                acc = fmaf(s[e], sPq[c + e], acc);
            }
            *reinterpret_cast<f32x2*>(Mr + c) = m;
            *reinterpret_cast<f32x2*>(Sr + c) = s;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (lane == 0) store_from_f32(o, row, acc);
    }
}

}  // namespace

size_t step_smem_bytes(const Shape& s) {
    return (size_t)(2 * s.d_phi + (s.swiglu ? 2 * s.d_k : 0)) * sizeof(float);
}

hipError_t launch_step(const Shape& s, const StepArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end) {
    StepParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.eta = a.eta;
    p.w1 = s.w1;
    p.w3 = s.w3;
    p.o = a.o;
    p.S = a.S;
    p.M = a.M;
    p.eta_scalar = a.eta_scalar;
    p.beta = a.beta;
    p.eta_kind = a.eta_kind;
    p.H = s.H;
    p.d_k = s.d_k;
    p.d_v = s.d_v;
    p.d_phi = s.d_phi;
    p.n_rblk = s.d_v / SR;
    const size_t smem = step_smem_bytes(s);
    const dim3 grid((unsigned)(s.n_seq() * p.n_rblk)), block(STHREADS);
    void* args[] = {&p};
    const void* fn = s.bf16 ? (s.swiglu ? (const void*)step_kernel<uint16_t, true> : (const void*)step_kernel<uint16_t, false>)
                            : (s.swiglu ? (const void*)step_kernel<float, true> : (const void*)step_kernel<float, false>);
    return hipExtLaunchKernel(fn, grid, block, args, smem, a.stream, ev_begin, ev_end, 0);
}

}  // namespace ttt
