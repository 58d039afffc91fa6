// Delta-rule forward for gfx950: the layer with the mean-squared binding loss.
//
// With l_t(S) = 1/2 ||S k_t - v_t||^2 (the MSE inner-loop loss that the Modular TTT
// abstract on the mlsanity.com page sets beside the inner-product loss) one descent
// step per token, no momentum, is
//     S_t = S_{t-1} - eta_t (S_{t-1} k_t - v_t) k_t^T,      o_t = S_t q_t,
// the delta rule of "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length" (cited by the same page).  S is d_v x d_k, reset per sequence.
//
// Chunk form (tokens as rows; a chunk of C tokens entered with S0).  Writing each
// step as S_t = S_{t-1} + u_t k_t^T with u_t = eta_t (v_t - S_{t-1} k_t) and
// unrolling S_{t-1} = S0 + sum_{j<t} u_j k_j^T:
//     u_t = eta_t r_t - sum_{j<t} N_tj u_j,   r_t = v_t - S0 k_t,  N_tj = eta_t (k_t . k_j)
//     O   = Q S0^T + tril(Q K^T) U,           S_C = S0 + U^T K
// R = V - K S0^T, the scores and the update are dense products on the matrix cores;
// the C-step solve for U runs in fp32 with one thread per value column.
//
// One workgroup (four waves) walks one sequence in chunks of 32 tokens and keeps
// its fp32 S in registers as 16x16 MFMA result tiles (wave w: value rows
// 32w .. 32w+31 at d = 128, 16w .. 16w+15 at d = 64).  A bf16 copy of S in LDS
// serves as the operand of K S0^T and Q S0^T.
//
// Register layouts of v_mfma_f32_16x16x32_bf16 (lane l, c16 = l % 16, g = l / 16):
//   A operand  A[m = c16][k = 8g .. 8g+7]      B operand  B[k = 8g .. 8g+7][n = c16]
//   D result   D[m = 4g .. 4g+3][n = c16]
// Operands whose contraction runs along the features are 16-byte row reads of the
// swizzled tiles; those whose contraction runs over tokens (U^T, K, U) are
// transpose reads.

#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_tiles.h"

namespace ttt {
namespace {

constexpr int DC = 32;         // tokens per chunk
constexpr int DTH = 256;       // threads: four waves
constexpr int NSTR = DC + 4;   // row stride (floats) of N
constexpr int PSTR = 40;       // row stride (bf16) of the masked scores: 16 rows read at one
                               // column fall on distinct banks

struct DeltaParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* eta;
    uint16_t* o;
    float eta_scalar;
    int eta_kind;
    int T;
};

template <int D>
__global__ void __launch_bounds__(DTH, 1) delta_forward(DeltaParams p) {
    constexpr int NT = D / 16;                // 16-wide tiles across d
    constexpr int SRT = D / 64;               // value-row tiles of S per wave
    constexpr int OTB = NT / 4;               // value tiles of R and O per wave
    __shared__ __attribute__((aligned(16))) uint16_t sQ[DC * D];
    __shared__ __attribute__((aligned(16))) uint16_t sK[DC * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[DC * D];
    __shared__ __attribute__((aligned(16))) uint16_t sU[DC * D];
    __shared__ __attribute__((aligned(16))) uint16_t sS[D * D];
    __shared__ __attribute__((aligned(16))) float sR[DC * D];
    __shared__ __attribute__((aligned(16))) float sN[DC * NSTR];
    __shared__ __attribute__((aligned(16))) uint16_t sP[DC * PSTR];
    __shared__ float sE[DC];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4, q4 = lane & 3;
    const int T = p.T;
    const size_t row0 = (size_t)blockIdx.x * T;
    const int vr0 = wv * 16 * SRT;            // first value row of this wave's S tiles

    f32x4 St[SRT][NT];
#pragma unroll
    for (int a = 0; a < SRT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) St[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int e = tid; e < D * D / 8; e += DTH) *reinterpret_cast<u32x4*>(sS + 8 * e) = u32x4{0u, 0u, 0u, 0u};

    const int n_chunks = (T + DC - 1) / DC;
    for (int c = 0; c < n_chunks; ++c) {
        const int t0 = c * DC;
        const int n = min(DC, T - t0);

        // ---- stage q, k, v rows of the chunk (zero past T) and the rates ----
        for (int e = tid; e < DC * D / 8; e += DTH) {
            const int r = e / (D / 8), col = 8 * (e % (D / 8));
            u32x4 xq = {0u, 0u, 0u, 0u}, xk = xq, xv = xq;
            if (r < n) {
                const size_t off = (row0 + t0 + r) * D + col;
                xq = *reinterpret_cast<const u32x4*>(p.q + off);
                xk = *reinterpret_cast<const u32x4*>(p.k + off);
                xv = *reinterpret_cast<const u32x4*>(p.v + off);
            }
            const int s = swz<D>(r, col);
            *reinterpret_cast<u32x4*>(sQ + s) = xq;
            *reinterpret_cast<u32x4*>(sK + s) = xk;
            *reinterpret_cast<u32x4*>(sV + s) = xv;
        }
        if (tid < DC) sE[tid] = tid < n ? eta_at(p.eta_kind, p.eta, p.eta_scalar, row0 + t0 + tid) : 0.0f;
        __syncthreads();

        // ---- R = V - K S0^T and O = Q S0^T (wave: value tiles OTB w .. OTB w + OTB - 1) ----
        f32x4 Oacc[2][OTB];
#pragma unroll
        for (int ta = 0; ta < 2; ++ta)
#pragma unroll
            for (int j = 0; j < OTB; ++j) {
                const int tb = OTB * wv + j;
                f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = ks;
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    const bf16x8 bS = as_bf16x8(lds_read16(sS + swz<D>(16 * tb + c16, 32 * kk + 8 * g)));
                    ks = mfma16(as_bf16x8(lds_read16(sK + swz<D>(16 * ta + c16, 32 * kk + 8 * g))), bS, ks);
                    qs = mfma16(as_bf16x8(lds_read16(sQ + swz<D>(16 * ta + c16, 32 * kk + 8 * g))), bS, qs);
                }
                Oacc[ta][j] = qs;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ta + 4 * g + r, col = 16 * tb + c16;
                    sR[t * D + col] = bf16_bits_to_f32(sV[swz<D>(t, col)]) - ks[r];
                }
            }
        // ---- N = diag(eta) strictly-lower(K K^T) and P = tril(Q K^T): the 2x2 tiles of 16
        //      tokens; waves 0..2 take the tiles (0,0), (1,0), (1,1), wave 3 zeroes (0,1) ----
        {
            const int ti = wv == 0 ? 0 : 1, tj = wv == 2 ? 1 : 0;
            if (wv < 3) {
                f32x4 gk = {0.f, 0.f, 0.f, 0.f}, gq = gk;
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    const bf16x8 bK = as_bf16x8(lds_read16(sK + swz<D>(16 * tj + c16, 32 * kk + 8 * g)));
                    gk = mfma16(as_bf16x8(lds_read16(sK + swz<D>(16 * ti + c16, 32 * kk + 8 * g))), bK, gk);
                    gq = mfma16(as_bf16x8(lds_read16(sQ + swz<D>(16 * ti + c16, 32 * kk + 8 * g))), bK, gq);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ti + 4 * g + r, j = 16 * tj + c16;
                    sN[t * NSTR + j] = j < t ? sE[t] * gk[r] : 0.0f;
                    sP[t * PSTR + j] = f32_to_bf16_bits(j <= t ? gq[r] : 0.0f);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * g + r, j = 16 + c16;
                    sN[t * NSTR + j] = 0.0f;
                    sP[t * PSTR + j] = 0;
                }
            }
        }
        __syncthreads();

        // ---- U: forward substitution, one thread per value column ----
        if (tid < D) {
            float u[DC];
#pragma unroll
            for (int t = 0; t < DC; ++t) {
                float acc = sE[t] * sR[t * D + tid];
#pragma unroll
                for (int j4 = 0; j4 < t; j4 += 4) {
                    const f32x4 nr = *reinterpret_cast<const f32x4*>(sN + t * NSTR + j4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (j4 + e < t) acc = fmaf(-nr[e], u[j4 + e], acc);
                }
                u[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < DC; ++t) sU[swz<D>(t, tid)] = f32_to_bf16_bits(u[t]);
        }
        __syncthreads();

        // ---- O += tril(Q K^T) U, written out ----
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            const bf16x8 aP = as_bf16x8(*reinterpret_cast<const u32x4*>(sP + (16 * ta + c16) * PSTR + 8 * g));
#pragma unroll
            for (int j = 0; j < OTB; ++j) {
                const int tb = OTB * wv + j;
                const f32x4 o = mfma16(aP, as_bf16x8(tr_read8<D>(sU, 8 * g, 16 * tb + 4 * q4)), Oacc[ta][j]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ta + 4 * g + r;
                    if (t < n) p.o[(row0 + t0 + t) * D + 16 * tb + c16] = f32_to_bf16_bits(o[r]);
                }
            }
        }
        // ---- S += U^T K, and its bf16 copy for the next chunk ----
#pragma unroll
        for (int a = 0; a < SRT; ++a) {
            const bf16x8 aU = as_bf16x8(tr_read8<D>(sU, 8 * g, vr0 + 16 * a + 4 * q4));
#pragma unroll
            for (int b = 0; b < NT; ++b) {
                St[a][b] = mfma16(aU, as_bf16x8(tr_read8<D>(sK, 8 * g, 16 * b + 4 * q4)), St[a][b]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sS[swz<D>(vr0 + 16 * a + 4 * g + r, 16 * b + c16)] = f32_to_bf16_bits(St[a][b][r]);
            }
        }
        __syncthreads();
    }
}

}  // namespace

bool delta_supported(const Shape& s) {
    return s.bf16 && !s.swiglu && s.d_k == s.d_v && s.d_phi == s.d_k && (s.d_k == 64 || s.d_k == 128);
}

hipError_t launch_delta(const Shape& s, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (!delta_supported(s) || a.bidirectional || a.beta != 0.0f || a.S0 || a.M0 || a.S_T || a.M_T || a.reverse)
        return hipErrorInvalidValue;
    DeltaParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.eta = a.eta;
    p.o = static_cast<uint16_t*>(a.o);
    p.eta_scalar = a.eta_scalar;
    p.eta_kind = a.eta_kind;
    p.T = s.T;
    const dim3 grid((unsigned)s.n_seq()), block(DTH);
    const void* fn = s.d_k == 128 ? reinterpret_cast<const void*>(delta_forward<128>)
                                  : reinterpret_cast<const void*>(delta_forward<64>);
    if (ev_begin || ev_end) {
        void* args[] = {&p};
        return hipExtLaunchKernel(fn, grid, block, args, 0, a.stream, ev_begin, ev_end, 0);
    }
    if (s.d_k == 128) hipLaunchKernelGGL(delta_forward<128>, grid, block, 0, a.stream, p);
    else hipLaunchKernelGGL(delta_forward<64>, grid, block, 0, a.stream, p);
    return hipGetLastError();
}

}  // namespace ttt
