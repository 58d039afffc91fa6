// Weight-normalised recurrent forward: Variant 1 of Table 2 on the
// thelatestinai.com page (Variant 2 with the weight normalisation kept; the table
// gives it a recurrent implementation only).  The pages do not define the
// normalisation; the reading implemented here: after each token's update every
// row of the fast weight S (one output unit: its weights over the d_phi features)
// is rescaled to the Euclidean norm that row has in the entry state S0, and the
// momentum buffer is left as it is.  Per token t:
//   M <- beta M + eta_t v_t phi(k_t)^T,   S~ = S + M,
//   S <- S~ with row i scaled by ||S0[i,:]|| / ||S~[i,:]||,   o_t = S phi(q_t).
//
// Rows are independent (row i meets only v_t[i] and o_t[i]), so a workgroup owns
// 16 rows of one sequence and walks its tokens in order: 16 lanes a row, d_phi / 16
// features a lane, the row in registers.  S is kept as c U with a per-row scalar c
// (U starts as S0 with c = 1): the token adds M / c to U, and the normalisation is
// the new scalar c = ||S0 row|| / ||U row||; likewise M is kept as rho Ms with
// rho = beta^t.  One pass over the lane's features gives the updates, ||U||^2 and
// U . phi(q) together; the two sums are reduced over the row's 16 lanes at once and
// o_t = c (U . phi(q)).  Per feature and token that is four fused multiply-adds on
// the vector ALUs.
//
// The features of q and k (the SwiGLU feature map's, formed beforehand into the
// workspace, or q and k themselves), v of the workgroup's rows and the rates of
// 16 tokens at a time are staged in LDS as fp32; the next 16 tokens' are loaded
// into registers while the current ones are used.

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ttt {
namespace {

constexpr int NR = 16;      // rows per workgroup
constexpr int NTH = 256;    // threads: 16 lanes a row
constexpr int NTC = 16;     // tokens per staged chunk

struct WnParams {
    const void* q;          // [seq][T][d_k] in TI (identity map: the features)
    const void* k;
    const void* v;          // [seq][T][d_v] in TI
    const uint16_t* phq;    // SwiGLU map: features [P][seq * T][128] bf16 (null otherwise)
    const uint16_t* phk;
    const float* eta;
    float eta_scalar, beta;
    int eta_kind;
    const float* S0;        // [seq][d_v][d_phi] fp32
    const float* M0;        // may be null (zero)
    float* S_T;             // may be null
    float* M_T;             // may be null
    void* o;                // [seq][T][d_v] in TI
    int T, d_v, n_rb, n_units;
    size_t n_rows;          // seq * T: the slice stride of phq, phk
};

// sum over the 16 lanes of a row (every lane gets it): swaps within pairs and quads,
// then of the quads of each half (row_half_mirror) and of the halves (row_mirror), on
// DPP moves instead of LDS permutes
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void row16_sum2(float& a, float& b) {
    a = dpp_add<0xB1>(a);    // quad_perm [1, 0, 3, 2]
    b = dpp_add<0xB1>(b);
    a = dpp_add<0x4E>(a);    // quad_perm [2, 3, 0, 1]
    b = dpp_add<0x4E>(b);
    a = dpp_add<0x141>(a);   // row_half_mirror
    b = dpp_add<0x141>(b);
    a = dpp_add<0x140>(a);   // row_mirror
    b = dpp_add<0x140>(b);
}

template <typename TI> __device__ __forceinline__ float ld1(const TI* p, size_t i);
template <> __device__ __forceinline__ float ld1<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
template <typename TI> __device__ __forceinline__ void st1(TI* p, size_t i, float x);
template <> __device__ __forceinline__ void st1<float>(float* p, size_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void st1<uint16_t>(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }

// FPT features a lane (d_phi = 16 FPT): lane pp of a row owns the contiguous features
// pp FPT .. pp FPT + FPT - 1, staged with a pitch of PITCH floats between lanes so that
// the 16 lanes' 16-byte reads fall on distinct banks
template <int FPT, typename TI, bool MOM>
__global__ void __launch_bounds__(NTH) wn_forward(WnParams p) {
    constexpr int DPHI = 16 * FPT;
    constexpr int PITCH = FPT == 4 ? 4 : FPT + 4;     // floats between two lanes' features
    constexpr int TOKF = 16 * PITCH;                  // floats per staged token
    __shared__ __attribute__((aligned(16))) float sK[NTC * TOKF];
    __shared__ __attribute__((aligned(16))) float sQ[NTC * TOKF];
    __shared__ float sV[NTC * NR];
    __shared__ float sE[NTC];
    __shared__ float sO[NTC * NR];

    const int tid = threadIdx.x;
    const int r = tid >> 4, pp = tid & 15;
    // XCD-aware: the row blocks of one sequence, which stage the same features, are
    // consecutive units and share an XCD's L2
    const int unit = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (unit >= p.n_units) return;
    const int rb = unit % p.n_rb;
    const size_t seq = unit / p.n_rb;
    const int row = rb * NR + r;                      // value row of S
    const size_t srow = seq * p.T;
    const int T = p.T, d_v = p.d_v;
    const float beta = p.beta;

    // ---- the row: U = S0, c = 1; M = M0 ----
    float u[FPT], m[FPT];
    {
        const size_t base = (seq * d_v + row) * (size_t)DPHI + (size_t)pp * FPT;
#pragma unroll
        for (int j = 0; j < FPT; j += 4) {
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(p.S0 + base + j);
            const f32x4 m4 = p.M0 ? *reinterpret_cast<const f32x4*>(p.M0 + base + j) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u[j + e] = s4[e];
                m[j + e] = m4[e];
            }
        }
    }
    float n0sq = 0.0f;
#pragma unroll
    for (int j = 0; j < FPT; ++j) n0sq = fmaf(u[j], u[j], n0sq);
    {
        float unused = 0.0f;
        row16_sum2(n0sq, unused);
    }
    const float n0 = sqrtf(n0sq);
    const float inv_n0 = n0 > 0.0f ? 1.0f / n0 : 0.0f;
    // S = c U.  A zero row stays zero (c = 0, and U does not move).
    float c = n0 > 0.0f ? 1.0f : 0.0f, ic = c;
    constexpr float RHO_MIN = 0x1p-60f;
    float rho = 1.0f;

    // ---- staging: 16-byte groups of VE consecutive features; group i of a chunk is
    // token i / (DPHI / VE), features VE (i % (DPHI / VE)) ..; thread tid loads groups
    // tid + NTH e and writes them to [token][lane chunk][index] as fp32 ----
    constexpr bool BF = !std::is_same<TI, float>::value;
    constexpr int VE = BF ? 8 : 4;                    // features a group (SwiGLU features are bf16)
    constexpr int GPT = DPHI / VE;                    // groups a token
    constexpr int GR = (NTC * GPT + NTH - 1) / NTH;   // groups a thread stages per array
    u32x4 rk[GR], rq[GR];
    float rv = 0.0f, re = 0.0f;
    auto group_at = [&](const void* x, const uint16_t* ph, int t, int f) -> u32x4 {
        const size_t rowi = srow + t;
        if (ph) return *reinterpret_cast<const u32x4*>(ph + ((size_t)(f >> 7) * p.n_rows + rowi) * 128 + (f & 127));
        return *reinterpret_cast<const u32x4*>(static_cast<const TI*>(x) + rowi * DPHI + f);
    };
    auto fetch = [&](int t0) {
#pragma unroll
        for (int e = 0; e < GR; ++e) {
            const int i = tid + NTH * e;
            const int tt = i / GPT, f = VE * (i % GPT);
            const int t = t0 + tt;
            const bool ok = i < NTC * GPT && t < T;
            rk[e] = ok ? group_at(p.k, p.phk, t, f) : u32x4{0u, 0u, 0u, 0u};
            rq[e] = ok ? group_at(p.q, p.phq, t, f) : u32x4{0u, 0u, 0u, 0u};
        }
        {
            const int tt = tid / NR, rr = tid % NR;   // NTC x NR = 256 values
            const int t = t0 + tt;
            rv = t < T ? ld1<TI>(static_cast<const TI*>(p.v), (srow + t) * d_v + rb * NR + rr) : 0.0f;
        }
        if (tid < NTC) {
            const int t = t0 + tid;
            re = t < T ? eta_at(p.eta_kind, p.eta, p.eta_scalar, srow + t) : 0.0f;
        }
    };
    // a group's features as fp32, four at a time (a run of four never crosses a lane chunk)
    auto put_group = [&](float* dst, const u32x4& g, int tt, int f) {
#pragma unroll
        for (int h = 0; h < VE / 4; ++h) {
            f32x4 x4;
            if constexpr (BF) {
                const uint32_t w0 = g[2 * h], w1 = g[2 * h + 1];
                x4 = f32x4{__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xffff0000u), __uint_as_float(w1 << 16),
                           __uint_as_float(w1 & 0xffff0000u)};
            } else {
                x4 = f32x4{__uint_as_float(g[0]), __uint_as_float(g[1]), __uint_as_float(g[2]), __uint_as_float(g[3])};
            }
            const int ff = f + 4 * h;
            *reinterpret_cast<f32x4*>(dst + tt * TOKF + (ff / FPT) * PITCH + (ff % FPT)) = x4;
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int e = 0; e < GR; ++e) {
            const int i = tid + NTH * e;
            if (i < NTC * GPT) {
                const int tt = i / GPT, f = VE * (i % GPT);
                put_group(sK, rk[e], tt, f);
                put_group(sQ, rq[e], tt, f);
            }
        }
        sV[tid] = rv;
        if (tid < NTC) sE[tid] = re;
    };

    fetch(0);
    for (int t0 = 0; t0 < T; t0 += NTC) {
        __syncthreads();   // the previous chunk's staging and outputs are used up
        put();
        __syncthreads();
        if (t0 + NTC < T) fetch(t0 + NTC);
        const int n = min(NTC, T - t0);
        for (int tt = 0; tt < n; ++tt) {
            const float* kf = sK + tt * TOKF + pp * PITCH;
            const float* qf = sQ + tt * TOKF + pp * PITCH;
            const float cv = sE[tt] * sV[tt * NR + r];
            // M = rho Ms with the workgroup-uniform scale rho = beta^t: the decay goes to
            // rho, and the token adds (eta v / rho) phi(k) to Ms (one multiply-add); Ms
            // absorbs rho when it would fall below RHO_MIN.  Without momentum M is the
            // token's own term.
            float cm, cu;
            if constexpr (MOM) {
                rho *= beta;
                if (rho < RHO_MIN) {
#pragma unroll
                    for (int j = 0; j < FPT; ++j) m[j] *= rho;
                    rho = 1.0f;
                }
                cm = cv * __builtin_amdgcn_rcpf(rho);
                cu = ic * rho;
            } else {
                cm = cv;
                cu = ic;
            }
            // four partial sums each, so that the accumulations are not one serial chain
            float ss4[4] = {0.f, 0.f, 0.f, 0.f}, dd4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < FPT; j += 4) {
                const f32x4 k4 = *reinterpret_cast<const f32x4*>(kf + j);
                const f32x4 q4 = *reinterpret_cast<const f32x4*>(qf + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    m[j + e] = MOM ? fmaf(cm, k4[e], m[j + e]) : cm * k4[e];
                    u[j + e] = fmaf(cu, m[j + e], u[j + e]);
                    ss4[e] = fmaf(u[j + e], u[j + e], ss4[e]);
                    dd4[e] = fmaf(u[j + e], q4[e], dd4[e]);
                }
            }
            float ss = (ss4[0] + ss4[1]) + (ss4[2] + ss4[3]);
            float dd = (dd4[0] + dd4[1]) + (dd4[2] + dd4[3]);
            row16_sum2(ss, dd);
            if (n0 > 0.0f) {
                if (ss > 0.0f) {
                    c = n0 * __builtin_amdgcn_rsqf(ss);
                    ic = sqrtf(ss) * inv_n0;
                } else {          // S~ row is zero: so is S; restart the scale
                    c = 1.0f;
                    ic = 1.0f;
                }
            }
            if (pp == 0) sO[tt * NR + r] = c * dd;
        }
        __syncthreads();
        {
            const int tt = tid / NR, rr = tid % NR;
            if (tt < n) st1<TI>(static_cast<TI*>(p.o), (srow + t0 + tt) * d_v + rb * NR + rr, sO[tt * NR + rr]);
        }
    }
    // ---- final state: S = c U, M ----
    const size_t base = (seq * d_v + row) * (size_t)DPHI + (size_t)pp * FPT;
#pragma unroll
    for (int j = 0; j < FPT; j += 4) {
        if (p.S_T)
            *reinterpret_cast<f32x4*>(p.S_T + base + j) = f32x4{c * u[j], c * u[j + 1], c * u[j + 2], c * u[j + 3]};
        if (p.M_T)
            *reinterpret_cast<f32x4*>(p.M_T + base + j) = f32x4{rho * m[j], rho * m[j + 1], rho * m[j + 2], rho * m[j + 3]};
    }
}

template <int FPT, typename TI, bool MOM>
hipError_t launch_wn_mom(const WnParams& p, int n_seq, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
    const dim3 grid((unsigned)((n_seq * p.n_rb + 7) / 8 * 8)), block(NTH);
    if (eb || ee) {
        WnParams a = p;
        void* args[] = {&a};
        return hipExtLaunchKernel(reinterpret_cast<const void*>(wn_forward<FPT, TI, MOM>), grid, block, args, 0, st, eb,
                                  ee, 0);
    }
    hipLaunchKernelGGL((wn_forward<FPT, TI, MOM>), grid, block, 0, st, p);
    return hipGetLastError();
}

template <int FPT, typename TI>
hipError_t launch_wn_one(const WnParams& p, int n_seq, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
    return p.beta != 0.0f ? launch_wn_mom<FPT, TI, true>(p, n_seq, st, eb, ee)
                          : launch_wn_mom<FPT, TI, false>(p, n_seq, st, eb, ee);
}

template <typename TI>
hipError_t launch_wn_ti(const WnParams& p, int d_phi, int n_seq, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
    switch (d_phi) {
        case 64: return launch_wn_one<4, TI>(p, n_seq, st, eb, ee);
        case 128: return launch_wn_one<8, TI>(p, n_seq, st, eb, ee);
        case 256: return launch_wn_one<16, TI>(p, n_seq, st, eb, ee);
        case 512: return launch_wn_one<32, TI>(p, n_seq, st, eb, ee);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool wn_supported(const Shape& s) {
    const bool widths = s.d_v % NR == 0 && (s.d_phi == 64 || s.d_phi == 128 || s.d_phi == 256 || s.d_phi == 512);
    if (s.swiglu) return widths && s.bf16 && s.d_k == 128 && s.d_phi % 128 == 0;
    return widths && s.d_k == s.d_phi;
}

size_t wn_workspace_bytes(const Shape& s) {
    // the SwiGLU features of q and k, slice-major bf16
    return s.swiglu ? 2 * (size_t)s.n_seq() * s.T * s.d_phi * 2 : 0;
}

hipError_t launch_wn(const Shape& s, void* workspace, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (!wn_supported(s) || a.bidirectional || a.reverse || !a.S0) return hipErrorInvalidValue;
    WnParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.eta = a.eta;
    p.eta_scalar = a.eta_scalar;
    p.beta = a.beta;
    p.eta_kind = a.eta_kind;
    p.S0 = a.S0;
    p.M0 = a.M0;
    p.S_T = a.S_T;
    p.M_T = a.M_T;
    p.o = a.o;
    p.T = s.T;
    p.d_v = s.d_v;
    p.n_rb = s.d_v / NR;
    p.n_units = s.n_seq() * p.n_rb;
    p.n_rows = (size_t)s.n_seq() * s.T;
    if (s.swiglu) {
        uint16_t* phq = static_cast<uint16_t*>(workspace);
        uint16_t* phk = phq + p.n_rows * s.d_phi;
        hipError_t e = launch_swiglu_features(s, a.q, phq, a.stream);
        if (e == hipSuccess) e = launch_swiglu_features(s, a.k, phk, a.stream);
        if (e != hipSuccess) return e;
        p.phq = phq;
        p.phk = phk;
    }
    return s.bf16 ? launch_wn_ti<uint16_t>(p, s.d_phi, s.n_seq(), a.stream, ev_begin, ev_end)
                  : launch_wn_ti<float>(p, s.d_phi, s.n_seq(), a.stream, ev_begin, ev_end);
}

}  // namespace ttt
