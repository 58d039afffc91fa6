// One-pass fp32 forward for short sequences, from the closed form of the recurrence.
//
// One momentum-SGD step per token on the dot-product binding loss,
//     M_t = beta M_{t-1} + eta_t v_t k_t^T,   S_t = S_{t-1} + M_t,   o_t = S_t q_t,
// unrolls to
//     o_t = sum_{s <= t} eta_s w(t - s) (q_t . k_s) v_s,    w(n) = sum_{u <= n} beta^u,
// and, with every token updating before any readout (o_t = S_{T-1} q_t), to the
// weight w(T - 1 - s) on every key s.  That is linear attention written as a masked
// T x T product (the parallel form the kualia.ai blog, "The Linear Attention
// Equivalence", describes), with the per-token rate and momentum options of
// Variants 3-5 (Table 2 of the thelatestinai.com page).
//
// For a short sequence this costs less time than walking the tokens in order: a
// workgroup owns 16 query rows and 64 value columns of one sequence and sweeps the
// keys in tiles of 64 (causal: up to its last query).  Both products run on the fp32
// matrix instructions (16x16x4), with their operands loaded straight into registers;
// the weighted scores pass through LDS from the waves that form them (one per 16
// keys) to the waves that use them (one per 16 value columns).  The next key tile is
// loaded while the current one is used.

#include <hip/hip_ext.h>

#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace ttt {
namespace {

constexpr int RQ = 16;     // query rows per workgroup
constexpr int RK = 64;     // keys per tile
constexpr int RV = 64;     // value columns per workgroup
constexpr int RTH = 256;   // threads
constexpr int RMAX_T = 1024;
constexpr int RKP = RK + 4;  // row stride of the weighted scores (16-byte rows, spread over banks)

typedef float f4 __attribute__((ext_vector_type(4)));

#define TTT_INLINE __attribute__((always_inline))

struct ShortParams {
    const float* q;
    const float* k;
    const float* v;
    const float* eta;
    float* o;
    float eta_scalar;
    float beta;
    int eta_kind;
    int bidir;
    int T, d_v, n_qt, n_vb;
};

// v_mfma_f32_16x16x4_f32: D[16x16] += A[16x4] B[4x16] in fp32.  Lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16] in
// element r of its accumulator.  The contraction index may be permuted freely as
// long as A and B agree: here lane group g = l / 16 walks its own contiguous block of
// the contracted dimension, one MFMA per element, so every operand a lane needs is
// contiguous in memory.
__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK>
__global__ void __launch_bounds__(RTH) short_forward(ShortParams p) {
    constexpr int DG = DK / 4;   // features per lane group in the score products
    __shared__ __attribute__((aligned(16))) float sP[2][RQ * RKP];   // weighted scores, two buffers
    __shared__ float sW[RMAX_T];                                      // w(n), n < T

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    int blk = blockIdx.x;
    const int vb = blk % p.n_vb;
    blk /= p.n_vb;
    const int qt = blk % p.n_qt;
    const size_t seq = blk / p.n_qt;
    const int T = p.T, d_v = p.d_v;
    const int t0 = qt * RQ;
    const size_t row0 = seq * T;
    const float* q = p.q + row0 * DK;
    const float* k = p.k + row0 * DK;
    const float* v = p.v + row0 * d_v + vb * RV;

    const int last_key = p.bidir ? T - 1 : min(T, t0 + RQ) - 1;
    const int n_kt = last_key / RK + 1;

    // score A operands: q[t0 + l16][g DG .. g DG + DG)
    float qa[DG];
    {
        const int tq = t0 + l16;
#pragma unroll
        for (int e = 0; e < DG / 4; ++e) {
            const f4 x = tq < T ? *reinterpret_cast<const f4*>(q + (size_t)tq * DK + g * DG + 4 * e)
                                : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) qa[4 * e + c] = x[c];
        }
    }
    // w(n) = (1 - beta^{n+1}) / (1 - beta) = -expm1((n+1) log(beta)) / (1 - beta): 1 - beta is
    // exact for beta >= 1/2 and log(beta) = log1p(-(1 - beta)), so no digits cancel
    if (p.beta == 0.0f) {
        for (int n = tid; n < T; n += RTH) sW[n] = 1.0f;
    } else {
        const float omb = 1.0f - p.beta, lb = log1pf(-omb);
        for (int n = tid; n < T; n += RTH) sW[n] = -expm1f((float)(n + 1) * lb) / omb;
    }

    // per key tile, in registers (two sets: the next tile loads while this one is used):
    //   kb: score B operands k[s0 + 16 wv + l16][g DG + s]   (wave wv: keys 16 wv .. +15)
    //   vv: output B operands v[s0 + 16 g + s][16 wv + l16]  (wave wv: value columns 16 wv .. +15)
    //   eb: rate of key s0 + 16 wv + l16
    float kb[2][DG], vv[2][16], eb[2];
    auto fetch = [&](int kt, int b) TTT_INLINE {
        const int s0 = kt * RK;
        const int key = s0 + 16 * wv + l16;
#pragma unroll
        for (int e = 0; e < DG / 4; ++e) {
            const f4 x = key <= last_key ? *reinterpret_cast<const f4*>(k + (size_t)key * DK + g * DG + 4 * e)
                                         : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) kb[b][4 * e + c] = x[c];
        }
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int r = s0 + 16 * g + s;
            vv[b][s] = r <= last_key ? v[(size_t)r * d_v + 16 * wv + l16] : 0.0f;
        }
        eb[b] = key <= last_key ? eta_at(p.eta_kind, p.eta, p.eta_scalar, row0 + key) : 0.0f;
    };

    f4 acc = {0.f, 0.f, 0.f, 0.f};
    auto use_tile = [&](int kt, int b) TTT_INLINE {
        const int s0 = kt * RK;
        f4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DG; ++s) sc = mfma4(qa[s], kb[b][s], sc);
        // lane holds the scores of queries t0 + 4g + r and key s0 + 16 wv + l16
        const int key = s0 + 16 * wv + l16;
        float* P = sP[kt & 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * g + r;
            float w = 0.0f;
            if (t < T && key < T) {
                if (p.bidir) w = sW[T - 1 - key];
                else if (key <= t) w = sW[t - key];
            }
            P[(4 * g + r) * RKP + 16 * wv + l16] = sc[r] * (eb[b] * w);
        }
        __syncthreads();
        // output A operands: weighted scores of query t0 + l16 and keys s0 + 16 g + s
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f4 pa = *reinterpret_cast<const f4*>(P + l16 * RKP + 16 * g + 4 * e);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc = mfma4(pa[c], vv[b][4 * e + c], acc);
        }
    };

    fetch(0, 0);
    __syncthreads();   // the rate weights are in LDS
    for (int kt = 0; kt < n_kt; kt += 2) {
        if (kt + 1 < n_kt) fetch(kt + 1, 1);
        use_tile(kt, 0);
        if (kt + 1 >= n_kt) break;
        if (kt + 2 < n_kt) fetch(kt + 2, 0);
        use_tile(kt + 1, 1);
    }
    // lane holds o[t0 + 4g + r][16 wv + l16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * g + r;
        if (t < T) p.o[(row0 + t) * d_v + vb * RV + 16 * wv + l16] = acc[r];
    }
}

}  // namespace

bool short_supported(const Shape& s) {
    return !s.bf16 && !s.swiglu && (s.d_k == 64 || s.d_k == 128) && s.d_phi == s.d_k && s.d_v % RV == 0 &&
           s.T <= RMAX_T;
}

int short_grid(const Shape& s) { return s.n_seq() * ((s.T + RQ - 1) / RQ) * (s.d_v / RV); }

hipError_t launch_short(const Shape& s, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (!short_supported(s) || a.S0 || a.M0 || a.S_T || a.M_T || a.reverse) return hipErrorInvalidValue;
    ShortParams p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.eta = a.eta;
    p.o = static_cast<float*>(a.o);
    p.eta_scalar = a.eta_scalar;
    p.beta = a.beta;
    p.eta_kind = a.eta_kind;
    p.bidir = a.bidirectional ? 1 : 0;
    p.T = s.T;
    p.d_v = s.d_v;
    p.n_qt = (s.T + RQ - 1) / RQ;
    p.n_vb = s.d_v / RV;
    const dim3 grid((unsigned)short_grid(s)), block(RTH);
    const void* fn = s.d_k == 64 ? reinterpret_cast<const void*>(short_forward<64>)
                                 : reinterpret_cast<const void*>(short_forward<128>);
    if (ev_begin || ev_end) {
        void* args[] = {&p};
        return hipExtLaunchKernel(fn, grid, block, args, 0, a.stream, ev_begin, ev_end, 0);
    }
    if (s.d_k == 64) hipLaunchKernelGGL(short_forward<64>, grid, block, 0, a.stream, p);
    else hipLaunchKernelGGL(short_forward<128>, grid, block, 0, a.stream, p);
    return hipGetLastError();
}

}  // namespace ttt
