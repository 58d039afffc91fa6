// One recurrent step of the TTT layer (decode): for every sequence (b, h) a
// single new token updates the carried fast weight and is read out,
//
//   M <- beta M + eta v phi(k)^T,   S <- S + M,   o = S phi(q),
//
// the token-by-token form that Table 2 of the thelatestinai.com page lists as
// the recurrent implementation of each variant (per-token lr and momentum in
// SGD; the SwiGLU feature map of Variant 2), one gradient step per entry on a
// fixed-size matrix (wpnews.pro commentary).  With the mean-squared binding
// loss (the MSE inner-loop loss of the Modular TTT abstract, mlsanity.com page)
// the value factor of the step is the residual at the given state:
//
//   M <- beta M + eta (v - S phi(k)) phi(k)^T,   S <- S + M,   o = S phi(q).
//
// The step reads and writes the whole fp32 state once and does under half a
// flop per byte of it: it is bound by HBM bandwidth.  One workgroup of four waves owns 16
// value rows (32 with the SwiGLU map) of one sequence's S and M; each wave takes
// its rows at once, its 64
// lanes covering consecutive features (8 bytes a lane, 512 bytes a wave access),
// and reduces the readout of each row across the wave.  The features
// phi(q), phi(k) of the token are formed once per workgroup in LDS (the SwiGLU
// map against the frozen W1, W3 rows: on the matrix cores for bf16, as fp32 dot
// products otherwise).  The first rows of S and M are requested before the
// features are formed.

#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace ttt {
namespace {

constexpr int STHREADS = 256;   // four waves
// value rows per workgroup: 16 (four a wave); 32 with the SwiGLU map, so that
// fewer workgroups form the same features of a token
constexpr int SR_PLAIN = 16, SR_SWIGLU = 32;

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
    int n_rblk;                 // row blocks per sequence (d_v / rows per workgroup)
};

// 16 bytes of a row (8 bf16 or 4 fp32) as fp32
__device__ __forceinline__ void load16_as_f32(const uint16_t* p, float* out) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(u[i] << 16);
        out[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load16_as_f32(const float* p, float* out) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = u[i];
}

// what a step does with each row: the plain step, the weight-normalised one
// (Variant 1), the mean-squared loss (the last two hold the whole row in registers)
enum RowRule { ROW_PLAIN = 0, ROW_WN = 1, ROW_MSE = 2 };

template <typename TI, bool SWIGLU, int SR, int RULE>
__global__ void __launch_bounds__(STHREADS) step_kernel(StepParams p) {
    constexpr bool WN = RULE == ROW_WN;
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

    // this wave's rows: the token's value entries, the rate and the first 512-byte
    // slice of each row of S and M are requested before the features are formed,
    // so that their latency overlaps that of the token's loads
    const float et = eta_at(p.eta_kind, p.eta, p.eta_scalar, (size_t)seq);
    const float beta = p.beta;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int RW = SR / 4;      // rows of this wave
    const int row0 = r0 + RW * wave;
    float* __restrict__ S = p.S + ((size_t)seq * p.d_v + row0) * d_phi;
    float* __restrict__ M = p.M + ((size_t)seq * p.d_v + row0) * d_phi;
    float ev[RW], acc[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        ev[rr] = load_as_f32(v, row0 + rr);
        acc[rr] = 0.0f;
    }
    // the first NPRE slices of 128 features of every row (the whole row when
    // d_phi <= 128 NPRE), loaded at once
    constexpr int NPRE = SWIGLU ? 4 : 1;
    const int c0 = 2 * lane;
    f32x2 m0[NPRE][RW], s0[NPRE][RW];
#pragma unroll
    for (int it = 0; it < NPRE; ++it) {
        const int c = c0 + 128 * it;
        if (c < d_phi) {
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                m0[it][rr] = *reinterpret_cast<const f32x2*>(M + (size_t)rr * d_phi + c);
                s0[it][rr] = *reinterpret_cast<const f32x2*>(S + (size_t)rr * d_phi + c);
            }
        }
    }

    if constexpr (!SWIGLU) {
        for (int f = tid; f < d_phi; f += STHREADS) {
            sPq[f] = load_as_f32(q, f);
            sPk[f] = load_as_f32(k, f);
        }
    } else if constexpr (sizeof(TI) == 2) {
        // bf16: W1 x and W3 x on the matrix cores, 32 features a product with q in
        // column 0 and k in column 1 of the B operand (the other 30 columns zero):
        // lane l supplies W[f0 + l % 32][k0 + 8 (l / 32) ..] and, for l % 32 < 2, the
        // same eight entries of q or k; D[i][j] lands in lane j + 32 ((i / 4) % 2),
        // register 4 (i / 8) + i % 4
        const int h = seq % p.H;
        const uint16_t* w1 = static_cast<const uint16_t*>(p.w1) + (size_t)h * d_phi * d_k;
        const uint16_t* w3 = static_cast<const uint16_t*>(p.w3) + (size_t)h * d_phi * d_k;
        const int j = lane & 31, kh = lane >> 5;
        const uint16_t* xrow = j == 0 ? q : k;
        // k-steps of 16 (d_k is 64 or 128).  The operands of every step are requested
        // before the first product, with no branch around a load (a branch made the
        // compiler wait for each load in turn): steps past d_k re-read the last
        // step, and their B column is zeroed
        constexpr int KS = 8;
        const int ks = d_k / 16;
        for (int f0 = 32 * wave; f0 < d_phi; f0 += 4 * 32) {
            u32x4 a1[KS], a3[KS], b[KS];
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const int k0 = 16 * min(st, ks - 1) + 8 * kh;
                a1[st] = *reinterpret_cast<const u32x4*>(w1 + (size_t)(f0 + j) * d_k + k0);
                a3[st] = *reinterpret_cast<const u32x4*>(w3 + (size_t)(f0 + j) * d_k + k0);
                b[st] = *reinterpret_cast<const u32x4*>(xrow + k0);
            }
            f32x16 u1 = {}, u3 = {};
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const u32x4 bs = (j < 2 && st < ks) ? b[st] : u32x4{0u, 0u, 0u, 0u};
                u1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1[st]),
                                                             __builtin_bit_cast(bf16x8, bs), u1, 0, 0, 0);
                u3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a3[st]),
                                                             __builtin_bit_cast(bf16x8, bs), u3, 0, 0, 0);
            }
            if (j < 2) {
                float* dst = j == 0 ? sPq : sPk;
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[f0 + 8 * (r >> 2) + 4 * kh + (r & 3)] = silu_f32(u1[r]) * u3[r];
            }
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
        // phi(x)_f = silu(W1_f . x) (W3_f . x): one thread per feature, its rows of
        // W1 and W3 read 16 bytes at a time
        for (int f = tid; f < d_phi; f += STHREADS) {
            float uq = 0.f, gq = 0.f, uk = 0.f, gk = 0.f;
            const TI* a = w1 + (size_t)f * d_k;
            const TI* b = w3 + (size_t)f * d_k;
            constexpr int VE = 16 / sizeof(TI);     // elements per 16-byte load
            for (int d0 = 0; d0 < d_k; d0 += VE) {
                float av[VE], bv[VE];
                load16_as_f32(a + d0, av);
                load16_as_f32(b + d0, bv);
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    uq = fmaf(av[e], sXq[d0 + e], uq);
                    gq = fmaf(bv[e], sXq[d0 + e], gq);
                    uk = fmaf(av[e], sXk[d0 + e], uk);
                    gk = fmaf(bv[e], sXk[d0 + e], gk);
                }
            }
            sPq[f] = silu_f32(uq) * gq;
            sPk[f] = silu_f32(uk) * gk;
        }
    }
    __syncthreads();

#pragma unroll
    for (int rr = 0; rr < RW; ++rr) ev[rr] *= et;
    // two consecutive features a lane, 512 bytes a wave access (d_phi is a
    // multiple of 64: every pair is whole); the rows' loads are issued together
    auto row_step = [&](int c, f32x2* m, f32x2* sv) {
        const float pk0 = sPk[c], pk1 = sPk[c + 1], pq0 = sPq[c], pq1 = sPq[c + 1];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            m[rr][0] = fmaf(beta, m[rr][0], ev[rr] * pk0);
            m[rr][1] = fmaf(beta, m[rr][1], ev[rr] * pk1);
            sv[rr][0] += m[rr][0];
            sv[rr][1] += m[rr][1];
            acc[rr] = fmaf(sv[rr][0], pq0, fmaf(sv[rr][1], pq1, acc[rr]));
            *reinterpret_cast<f32x2*>(M + (size_t)rr * d_phi + c) = m[rr];
            *reinterpret_cast<f32x2*>(S + (size_t)rr * d_phi + c) = sv[rr];
        }
    };
    if constexpr (WN) {
        // Variant 1 (weight-normalised rows): the whole row is in registers (d_phi <=
        // 128 NPRE); the new row is rescaled to the norm of the given one before it is
        // written, and the readout takes the same factor
        float n_old[RW], n_new[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) n_old[rr] = n_new[rr] = 0.0f;
#pragma unroll
        for (int it = 0; it < NPRE; ++it) {
            const int c = c0 + 128 * it;
            if (c < d_phi) {
                const float pk0 = sPk[c], pk1 = sPk[c + 1], pq0 = sPq[c], pq1 = sPq[c + 1];
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    f32x2& m = m0[it][rr];
                    f32x2& sv = s0[it][rr];
                    n_old[rr] = fmaf(sv[0], sv[0], fmaf(sv[1], sv[1], n_old[rr]));
                    m[0] = fmaf(beta, m[0], ev[rr] * pk0);
                    m[1] = fmaf(beta, m[1], ev[rr] * pk1);
                    sv[0] += m[0];
                    sv[1] += m[1];
                    n_new[rr] = fmaf(sv[0], sv[0], fmaf(sv[1], sv[1], n_new[rr]));
                    acc[rr] = fmaf(sv[0], pq0, fmaf(sv[1], pq1, acc[rr]));
                }
            }
        }
        float fac[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                n_old[rr] += __shfl_xor(n_old[rr], off, 64);
                n_new[rr] += __shfl_xor(n_new[rr], off, 64);
            }
            fac[rr] = n_new[rr] > 0.0f ? sqrtf(n_old[rr] / n_new[rr]) : 0.0f;
        }
#pragma unroll
        for (int it = 0; it < NPRE; ++it) {
            const int c = c0 + 128 * it;
            if (c < d_phi) {
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    *reinterpret_cast<f32x2*>(M + (size_t)rr * d_phi + c) = m0[it][rr];
                    *reinterpret_cast<f32x2*>(S + (size_t)rr * d_phi + c) =
                        f32x2{fac[rr] * s0[it][rr][0], fac[rr] * s0[it][rr][1]};
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) acc[rr] *= fac[rr];   // reduced below like the plain step
    } else if constexpr (RULE == ROW_MSE) {
        // the residual v - S phi(k) of each row at the given S (the whole row is in
        // registers: d_phi <= 128 NPRE), reduced across the wave, is the value
        // factor of the plain step that follows
        float pr[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) pr[rr] = 0.0f;
#pragma unroll
        for (int it = 0; it < NPRE; ++it) {
            const int c = c0 + 128 * it;
            if (c < d_phi) {
                const float pk0 = sPk[c], pk1 = sPk[c + 1];
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) pr[rr] = fmaf(s0[it][rr][0], pk0, fmaf(s0[it][rr][1], pk1, pr[rr]));
            }
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) pr[rr] += __shfl_xor(pr[rr], off, 64);
            ev[rr] = fmaf(-et, pr[rr], ev[rr]);    // eta (v - S phi(k))
        }
#pragma unroll
        for (int it = 0; it < NPRE; ++it)
            if (c0 + 128 * it < d_phi) row_step(c0 + 128 * it, m0[it], s0[it]);
    } else {
#pragma unroll
    for (int it = 0; it < NPRE; ++it)
        if (c0 + 128 * it < d_phi) row_step(c0 + 128 * it, m0[it], s0[it]);
    for (int c = c0 + 128 * NPRE; c < d_phi; c += 128) {
        f32x2 m[RW], sv[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            m[rr] = *reinterpret_cast<const f32x2*>(M + (size_t)rr * d_phi + c);
            sv[rr] = *reinterpret_cast<const f32x2*>(S + (size_t)rr * d_phi + c);
        }
        row_step(c, m, sv);
    }
    }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        float a = acc[rr];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
        if (lane == 0) store_from_f32(o, row0 + rr, a);
    }
}

}  // namespace

bool step_row_in_registers(const Shape& s) { return s.d_phi <= (s.swiglu ? 512 : 128); }

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
    const int sr = (s.swiglu && s.d_v % SR_SWIGLU == 0) ? SR_SWIGLU : SR_PLAIN;
    p.n_rblk = s.d_v / sr;
    const size_t smem = step_smem_bytes(s);
    const dim3 grid((unsigned)(s.n_seq() * p.n_rblk)), block(STHREADS);
    void* args[] = {&p};
    if ((a.weight_norm || a.mse) && !step_row_in_registers(s)) return hipErrorInvalidValue;
    if (a.weight_norm && a.mse) return hipErrorInvalidValue;
    const int rule = a.weight_norm ? ROW_WN : (a.mse ? ROW_MSE : ROW_PLAIN);
    const bool wide_rows = s.swiglu && sr == SR_SWIGLU;
    const void* fn = nullptr;
    auto pick = [&](auto tag) {
        constexpr int R = decltype(tag)::value;
        if (wide_rows)
            fn = s.bf16 ? (const void*)step_kernel<uint16_t, true, SR_SWIGLU, R>
                        : (const void*)step_kernel<float, true, SR_SWIGLU, R>;
        else if (s.swiglu)
            fn = s.bf16 ? (const void*)step_kernel<uint16_t, true, SR_PLAIN, R>
                        : (const void*)step_kernel<float, true, SR_PLAIN, R>;
        else
            fn = s.bf16 ? (const void*)step_kernel<uint16_t, false, SR_PLAIN, R>
                        : (const void*)step_kernel<float, false, SR_PLAIN, R>;
    };
    if (rule == ROW_WN) pick(std::integral_constant<int, ROW_WN>{});
    else if (rule == ROW_MSE) pick(std::integral_constant<int, ROW_MSE>{});
    else pick(std::integral_constant<int, ROW_PLAIN>{});
    return hipExtLaunchKernel(fn, grid, block, args, smem, a.stream, ev_begin, ev_end, 0);
}

}  // namespace ttt
