// Gradients of the TTT-layer forward (identity feature map, d_k = d_v): the
// parallel form is trained end to end (Figure 4 of the thelatestinai.com page
// reports its training speed), so the chunked path needs its backward.
//
// With L = sum(o * dO), c_r = sum_{u<=r} beta^u and eta_s the rate of token s,
// the gradients of the causal layer are forwards of the same layer on permuted
// operands, two of them over the time-reversed sequence (R reverses t):
//   dq = forward(q <- dO, k <- v, v <- k; rates eta)
//   u  = R forward(R k, R q, R dO; rate 1),   w = R forward(R v, R dO, R q; rate 1)
//   dv_s = eta_s u_s,   dk_s = eta_s w_s,   deta_s = v_s . u_s
// (u_s = sum_{t>=s} c_{t-s} (q_t . k_s) dO_t).  Bidirectionally every query
// reads the final state, and with rate-1, beta = 0 bidirectional forwards
// u = forward(k, q, dO), w = forward(v, dO, q):
//   dv_s = eta_s c_{T-1-s} u_s,  dk_s = eta_s c_{T-1-s} w_s,  deta_s = c_{T-1-s} v_s . u_s.
// The forwards run on the library's own kernels; this file holds the two
// memory-bound helpers: reversal of sequences along t, and the final scaling
// (with the rate gradient, chained through softplus when the rates are logits).

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace ttt {
namespace {

// dst[seq, t, :] = src[seq, T-1-t, :] for up to four tensors (blockIdx.y), one
// thread per 16 bytes
struct ReverseParams {
    const uint8_t* src[4];
    uint8_t* dst[4];
    int T;
    int row_units;        // 16-byte units per row
    size_t n_units;       // per tensor
};

__global__ void __launch_bounds__(256) reverse_rows(ReverseParams p) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.n_units) return;
    const int y = blockIdx.y;
    const size_t row = i / p.row_units, u = i % p.row_units;
    const size_t seq = row / p.T;
    const int t = (int)(row % p.T);
    const size_t src_row = seq * p.T + (p.T - 1 - t);
    const u32x4 x = *reinterpret_cast<const u32x4*>(p.src[y] + (src_row * p.row_units + u) * 16);
    *reinterpret_cast<u32x4*>(p.dst[y] + i * 16) = x;
}

struct FinalizeParams {
    const void* u;        // [n_seq, T, d] forward outputs (reversed in time when causal)
    const void* w;
    const void* v;
    const float* eta;
    void* dk;
    void* dv;
    float* deta;          // may be null
    float eta_scalar;
    float beta;
    int eta_kind;
    int causal;
    int uw_reversed;
    int T, d;
    size_t n_rows;
};

// 16 bytes a lane: a row (b, h, s) of d values is d / VE consecutive lanes, a
// wave 64 VE / d rows (d = 64 or 128)
template <typename TI>
__device__ __forceinline__ void load_vec(const TI* p, float* out);
template <>
__device__ __forceinline__ void load_vec<uint16_t>(const uint16_t* p, float* out) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(u[i] << 16);
        out[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load_vec<float>(const float* p, float* out) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = u[i];
}
template <typename TI>
__device__ __forceinline__ void store_vec(TI* p, const float* x);
template <>
__device__ __forceinline__ void store_vec<uint16_t>(uint16_t* p, const float* x) {
    *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                                         pack_bf16x2(x[6], x[7])};
}
template <>
__device__ __forceinline__ void store_vec<float>(float* p, const float* x) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}

template <typename TI>
__global__ void __launch_bounds__(256) finalize_grads(FinalizeParams p) {
    constexpr int VE = 16 / sizeof(TI);
    const int lpr = p.d / VE;                                  // lanes per row: 4 .. 32
    const int lane = threadIdx.x & 63;
    const size_t row = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / lpr) + lane / lpr;
    const bool live = row < p.n_rows;
    const size_t r = live ? row : 0;
    const int j0 = (lane % lpr) * VE;
    const size_t seq = r / p.T;
    const int s = (int)(r % p.T);
    // the forward outputs of token s (at T-1-s when they are stored reversed)
    const size_t src = p.uw_reversed ? seq * p.T + (p.T - 1 - s) : r;
    float c = 1.0f;
    if (!p.causal && p.beta != 0.0f) {
        // c_{T-1-s} = sum_{r=0}^{T-1-s} beta^r = (1 - beta^{T-s}) / (1 - beta)
        c = (1.0f - powf(p.beta, (float)(p.T - s))) / (1.0f - p.beta);
    }
    const float e = eta_at(p.eta_kind, p.eta, p.eta_scalar, r);
    float u[VE], w[VE], v[VE];
    load_vec(static_cast<const TI*>(p.u) + src * p.d + j0, u);
    if (p.dk) load_vec(static_cast<const TI*>(p.w) + src * p.d + j0, w);
    load_vec(static_cast<const TI*>(p.v) + r * p.d + j0, v);
    float dv[VE], dk[VE], dot = 0.0f;
#pragma unroll
    for (int i = 0; i < VE; ++i) {
        dv[i] = e * c * u[i];
        dk[i] = p.dk ? e * c * w[i] : 0.0f;
        dot = fmaf(v[i], u[i], dot);
    }
    if (live) {
        store_vec(static_cast<TI*>(p.dv) + r * p.d + j0, dv);
        // no dk when the key gradient is formed elsewhere (through the SwiGLU feature map)
        if (p.dk) store_vec(static_cast<TI*>(p.dk) + r * p.d + j0, dk);
    }
    // the row's lanes are consecutive and lpr is a power of two
    for (int off = lpr / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (live && lane % lpr == 0 && p.deta) {
        float g = c * dot;                               // dL/deta_s
        if (p.eta_kind == ETA_SOFTPLUS) {
            const float a = p.eta[r];
            g *= 1.0f / (1.0f + __expf(-a));             // d softplus(a) / da = sigmoid(a)
        }
        p.deta[r] = g;
    }
}

}  // namespace

hipError_t launch_reverse(const void* const* src, void* const* dst, int count, size_t n_seq, int T, size_t row_bytes,
                          hipStream_t st) {
    ReverseParams p{};
    for (int i = 0; i < count; ++i) {
        p.src[i] = static_cast<const uint8_t*>(src[i]);
        p.dst[i] = static_cast<uint8_t*>(dst[i]);
    }
    p.T = T;
    p.row_units = (int)(row_bytes / 16);
    p.n_units = n_seq * (size_t)T * p.row_units;
    const dim3 grid((unsigned)((p.n_units + 255) / 256), (unsigned)count);
    hipLaunchKernelGGL(reverse_rows, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_finalize_grads(const Shape& s, const BackArgs& a) {
    FinalizeParams p{};
    p.u = a.u;
    p.w = a.w;
    p.v = a.v;
    p.eta = a.eta;
    p.dk = a.dk;
    p.dv = a.dv;
    p.deta = a.deta;
    p.eta_scalar = a.eta_scalar;
    p.beta = a.beta;
    p.eta_kind = a.eta_kind;
    p.causal = a.causal ? 1 : 0;
    p.uw_reversed = a.uw_reversed ? 1 : 0;
    p.T = s.T;
    p.d = s.d_v;
    p.n_rows = (size_t)s.n_seq() * s.T;
    // rows per workgroup: four waves of 64 VE / d rows (VE = 16 / element bytes)
    const size_t rows_per_wg = 4 * (size_t)(64 * (16 / (s.bf16 ? 2 : 4)) / s.d_v);
    const dim3 grid((unsigned)((p.n_rows + rows_per_wg - 1) / rows_per_wg));
    if (s.bf16)
        hipLaunchKernelGGL(finalize_grads<uint16_t>, grid, dim3(256), 0, a.stream, p);
    else
        hipLaunchKernelGGL(finalize_grads<float>, grid, dim3(256), 0, a.stream, p);
    return hipGetLastError();
}

}  // namespace ttt
