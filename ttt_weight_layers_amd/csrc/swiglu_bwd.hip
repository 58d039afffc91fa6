// Backward of the SwiGLU feature map (Variant 2 of Table 2, thelatestinai.com page:
// a two-layer MLP fast weight of which only the last layer is updated, so the first
// layer phi(x) = silu(W1 x) * (W3 x) is a slow weight trained through the outer loop).
//
// The layer is linear attention on the features phi(q), phi(k); its backward in
// feature space (forwards on permuted operands, api.hip) gives dphi(q) and dphi(k).
// The chain rule through phi, with u = W1 x and g = W3 x, is
//     du = dphi * g * silu'(u),   dg = dphi * silu(u),   silu'(u) = s (1 + u (1 - s)), s = sigmoid(u)
//     dx = W1^T du + W3^T dg,      dW1 = sum over tokens of du x^T,   dW3 = sum of dg x^T
// for x = q and x = k (both through the same W1, W3).  Kernels (bf16 operands,
// v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   gate_kernel<FEATURES>  phi = silu(X W1^T) * (X W3^T) for one 128-feature slice,
//                          written slice-major [slice][seq][T][128] (the operand layout
//                          of the feature-space forwards)
//   gate_kernel<GRADS>     du, dg from the same products and dphi (optionally scaled per
//                          token), written side by side as [seq][T][2 d_phi]
//   dx_kernel              dx = [du | dg] [W1 ; W3]: contraction over 2 d_phi
//   dw_kernel              [dW1 ; dW3] = sum over q, k, batch and tokens of [du | dg]^T x:
//                          fp32 partial sums over token ranges, then dw_reduce adds
//                          them in a fixed order (the result does not depend on
//                          scheduling)
//   wcat_kernel            [W1 ; W3]^T per head, the K-contiguous operand of dx_kernel
//
// Register layouts (lane l, c16 = l % 16, g = l / 16): A operand A[m = c16][k = 8g ..
// 8g+7], B operand B[k = 8g .. 8g+7][n = c16], D result D[m = 4g .. 4g+3][n = c16].
// K-contiguous operands are 16-byte row reads of swizzled LDS tiles; token-contracted
// ones (dw_kernel) are transpose reads.

#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_tiles.h"

namespace ttt {
namespace {

constexpr int GT = 64;     // tokens per tile
constexpr int GW = 128;    // input width d_k and feature slice width
constexpr int GTH = 256;   // threads

enum GateMode : int { G_FEATURES = 0, G_GRADS = 1 };

__device__ __forceinline__ float sigmoid_f32(float u) { return 1.0f / (1.0f + __expf(-u)); }

struct GateParams {
    const uint16_t* x;       // [seq][T][128] raw inputs (q or k)
    const uint16_t* w1;      // [H][d_phi][128]
    const uint16_t* w3;
    uint16_t* phi;           // FEATURES: [P][seq][T][128]
    const uint16_t* dphi;    // GRADS: [P][seq][T][128]
    uint16_t* dg;            // GRADS: [seq][T][2 d_phi]: du in columns < d_phi, dg after
    // GRADS: dphi of token t is scaled by eta_t c_t when scale_eta is set (c_t = 1
    // causal, (1 - beta^{T-t}) / (1 - beta) bidirectional), else taken as is
    const float* eta;
    float eta_scalar, beta;
    int eta_kind, scale_eta, bidir;
    int T, H, d_phi, n_seq, n_tiles;
};

constexpr int GTPW = 8;    // token tiles per workgroup of gate_kernel (the weights stay in LDS)

template <int MODE>
__global__ void __launch_bounds__(GTH) gate_kernel(GateParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sX[GT * GW];
    __shared__ __attribute__((aligned(16))) uint16_t sW1[GW * GW];
    __shared__ __attribute__((aligned(16))) uint16_t sW3[GW * GW];
    __shared__ __attribute__((aligned(16))) uint16_t sD[MODE == G_GRADS ? GT * GW : 8];
    __shared__ float sScale[GT];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int n_groups = (p.n_tiles + GTPW - 1) / GTPW;
    const int grp = blockIdx.x % n_groups;
    const int seq = blockIdx.x / n_groups;
    const int sl = blockIdx.y;                 // feature slice
    const int h = seq % p.H;
    const size_t slice_rows = (size_t)p.n_seq * p.T;
    const uint16_t* w1 = p.w1 + ((size_t)h * p.d_phi + sl * GW) * GW;
    const uint16_t* w3 = p.w3 + ((size_t)h * p.d_phi + sl * GW) * GW;

    for (int e = tid; e < GW * GW / 8; e += GTH) {
        const int r = e / (GW / 8), col = 8 * (e % (GW / 8));
        *reinterpret_cast<u32x4*>(sW1 + swz<GW>(r, col)) = *reinterpret_cast<const u32x4*>(w1 + r * GW + col);
        *reinterpret_cast<u32x4*>(sW3 + swz<GW>(r, col)) = *reinterpret_cast<const u32x4*>(w3 + r * GW + col);
    }
    const int tile_end = min(p.n_tiles, (grp + 1) * GTPW);
    for (int tile = grp * GTPW; tile < tile_end; ++tile) {
        const int t0 = tile * GT;
        const int n = min(GT, p.T - t0);
        const size_t row0 = (size_t)seq * p.T + t0;
        for (int e = tid; e < GT * GW / 8; e += GTH) {
            const int r = e / (GW / 8), col = 8 * (e % (GW / 8));
            u32x4 x = {0u, 0u, 0u, 0u}, d = x;
            if (r < n) {
                x = *reinterpret_cast<const u32x4*>(p.x + (row0 + r) * GW + col);
                if constexpr (MODE == G_GRADS)
                    d = *reinterpret_cast<const u32x4*>(p.dphi + (sl * slice_rows + row0 + r) * GW + col);
            }
            *reinterpret_cast<u32x4*>(sX + swz<GW>(r, col)) = x;
            if constexpr (MODE == G_GRADS) *reinterpret_cast<u32x4*>(sD + swz<GW>(r, col)) = d;
        }
        if (MODE == G_GRADS && tid < GT) {
            float sc = 1.0f;
            if (p.scale_eta && tid < n) {
                const int t = t0 + tid;
                sc = eta_at(p.eta_kind, p.eta, p.eta_scalar, (size_t)seq * p.T + t);
                if (p.bidir && p.beta != 0.0f) sc *= (1.0f - powf(p.beta, (float)(p.T - t))) / (1.0f - p.beta);
            }
            sScale[tid] = sc;
        }
        __syncthreads();

        // wave wv: tokens 16 wv .. +15, all eight 16-feature tiles of the slice
        f32x4 U[8], G[8];
#pragma unroll
        for (int tb = 0; tb < 8; ++tb) U[tb] = G[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < GW / 32; ++kk) {
            const bf16x8 a = as_bf16x8(lds_read16(sX + swz<GW>(16 * wv + c16, 32 * kk + 8 * g)));
#pragma unroll
            for (int tb = 0; tb < 8; ++tb) {
                U[tb] = mfma16(a, as_bf16x8(lds_read16(sW1 + swz<GW>(16 * tb + c16, 32 * kk + 8 * g))), U[tb]);
                G[tb] = mfma16(a, as_bf16x8(lds_read16(sW3 + swz<GW>(16 * tb + c16, 32 * kk + 8 * g))), G[tb]);
            }
        }
        // results of the tile into LDS (phi or du over the staged x, dg over the staged dphi:
        // each lane overwrites only entries it alone has read), then 16-byte stores
        __syncthreads();   // every wave is done reading sX for its products
#pragma unroll
        for (int tb = 0; tb < 8; ++tb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * wv + 4 * g + r, f = 16 * tb + c16;
                const float u = U[tb][r], gg = G[tb][r];
                const float sg = sigmoid_f32(u);
                if constexpr (MODE == G_FEATURES) {
                    sX[swz<GW>(t, f)] = f32_to_bf16_bits(u * sg * gg);
                } else {
                    const float d = bf16_bits_to_f32(sD[swz<GW>(t, f)]) * sScale[t];
                    sX[swz<GW>(t, f)] = f32_to_bf16_bits(d * gg * sg * (1.0f + u * (1.0f - sg)));
                    sD[swz<GW>(t, f)] = f32_to_bf16_bits(d * u * sg);
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < GT * GW / 8; e += GTH) {
            const int r = e / (GW / 8), col = 8 * (e % (GW / 8));
            if (r >= n) continue;
            const u32x4 a = *reinterpret_cast<const u32x4*>(sX + swz<GW>(r, col));
            if constexpr (MODE == G_FEATURES) {
                *reinterpret_cast<u32x4*>(p.phi + (sl * slice_rows + row0 + r) * GW + col) = a;
            } else {
                const size_t o = (row0 + r) * (size_t)(2 * p.d_phi) + sl * GW + col;
                *reinterpret_cast<u32x4*>(p.dg + o) = a;
                *reinterpret_cast<u32x4*>(p.dg + o + p.d_phi) = *reinterpret_cast<const u32x4*>(sD + swz<GW>(r, col));
            }
        }
        __syncthreads();   // the tile's LDS is used up
    }
}

struct DxParams {
    const uint16_t* dg;      // [seq][T][K], K = 2 d_phi
    const uint16_t* wcat;    // [H][128][K]
    uint16_t* dx;            // [seq][T][128]
    int T, H, K, n_tiles;
};

constexpr int DXK = 64;      // contraction panel

// dx[t][n] = sum_k dg[t][k] wcat[h][n][k]
__global__ void __launch_bounds__(GTH) dx_kernel(DxParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[GT * DXK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[GW * DXK];
    __shared__ __attribute__((aligned(16))) uint16_t sO[GT * GW];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int tile = blockIdx.x % p.n_tiles;
    const int seq = blockIdx.x / p.n_tiles;
    const int h = seq % p.H;
    const int t0 = tile * GT;
    const int n = min(GT, p.T - t0);
    const size_t row0 = (size_t)seq * p.T + t0;
    const uint16_t* wc = p.wcat + (size_t)h * GW * p.K;

    f32x4 acc[8];
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.K; k0 += DXK) {
        for (int e = tid; e < GT * DXK / 8; e += GTH) {
            const int r = e / (DXK / 8), col = 8 * (e % (DXK / 8));
            u32x4 a = {0u, 0u, 0u, 0u};
            if (r < n) a = *reinterpret_cast<const u32x4*>(p.dg + (row0 + r) * p.K + k0 + col);
            *reinterpret_cast<u32x4*>(sA + swz<DXK>(r, col)) = a;
        }
        for (int e = tid; e < GW * DXK / 8; e += GTH) {
            const int r = e / (DXK / 8), col = 8 * (e % (DXK / 8));
            *reinterpret_cast<u32x4*>(sB + swz<DXK>(r, col)) =
                *reinterpret_cast<const u32x4*>(wc + (size_t)r * p.K + k0 + col);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < DXK / 32; ++kk) {
            const bf16x8 a = as_bf16x8(lds_read16(sA + swz<DXK>(16 * wv + c16, 32 * kk + 8 * g)));
#pragma unroll
            for (int tb = 0; tb < 8; ++tb)
                acc[tb] = mfma16(a, as_bf16x8(lds_read16(sB + swz<DXK>(16 * tb + c16, 32 * kk + 8 * g))), acc[tb]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[swz<GW>(16 * wv + 4 * g + r, 16 * tb + c16)] = f32_to_bf16_bits(acc[tb][r]);
    __syncthreads();
    for (int e = tid; e < GT * GW / 8; e += GTH) {
        const int r = e / (GW / 8), col = 8 * (e % (GW / 8));
        if (r < n)
            *reinterpret_cast<u32x4*>(p.dx + (row0 + r) * GW + col) = *reinterpret_cast<const u32x4*>(sO + swz<GW>(r, col));
    }
}

struct DwParams {
    const uint16_t* dg_q;    // [seq][T][K]
    const uint16_t* dg_k;
    const uint16_t* x_q;     // [seq][T][128]
    const uint16_t* x_k;
    float* part;             // [n_parts][H][K][128] partial sums
    int B, H, T, K, n_split; // n_split: token ranges per (b, h)
};

constexpr int DWT = 64;      // tokens per panel
constexpr int DWM = 64;      // output rows (of 2 d_phi) per workgroup

// part[pi][h][m][n] = sum over (q, k) and the tokens t of part pi = (b, range) of
// dg[b,h,t][m] x[b,h,t][n]; the next panel loads into registers while this one is used
__global__ void __launch_bounds__(GTH) dw_kernel(DwParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[DWT * DWM];
    __shared__ __attribute__((aligned(16))) uint16_t sB[DWT * GW];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4, q4 = lane & 3;
    const int n_mt = p.K / DWM;
    int blk = blockIdx.x;
    const int mt = blk % n_mt;
    blk /= n_mt;
    const int h = blk % p.H;
    const int pi = blk / p.H;                  // b * n_split + range
    const int b = pi / p.n_split, rg = pi % p.n_split;
    const int m0 = mt * DWM;
    const int span = (p.T + p.n_split - 1) / p.n_split;
    const int t_begin = rg * span, t_end = min(p.T, t_begin + span);
    const size_t srow = ((size_t)b * p.H + h) * p.T;
    const int n_panels = t_end > t_begin ? (t_end - t_begin + DWT - 1) / DWT : 0;

    u32x4 ra[2], rb[4];   // one panel: dg 64 x 64 (2 loads a thread), x 64 x 128 (4 loads)
    auto fetch = [&](int i) {
        const int src = i % 2, t0 = t_begin + (i / 2) * DWT;
        const uint16_t* dgm = src == 0 ? p.dg_q : p.dg_k;
        const uint16_t* xm = src == 0 ? p.x_q : p.x_k;
#pragma unroll
        for (int l = 0; l < 2; ++l) {
            const int e = tid + l * GTH, r = e / (DWM / 8), col = 8 * (e % (DWM / 8));
            ra[l] = t0 + r < t_end ? *reinterpret_cast<const u32x4*>(dgm + (srow + t0 + r) * p.K + m0 + col)
                                   : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int e = tid + l * GTH, r = e / (GW / 8), col = 8 * (e % (GW / 8));
            rb[l] = t0 + r < t_end ? *reinterpret_cast<const u32x4*>(xm + (srow + t0 + r) * GW + col)
                                   : u32x4{0u, 0u, 0u, 0u};
        }
    };

    f32x4 acc[8];
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int n_it = 2 * n_panels;             // (q, k) alternating, panel by panel
    if (n_it > 0) fetch(0);
    for (int i = 0; i < n_it; ++i) {
#pragma unroll
        for (int l = 0; l < 2; ++l) {
            const int e = tid + l * GTH, r = e / (DWM / 8), col = 8 * (e % (DWM / 8));
            *reinterpret_cast<u32x4*>(sA + swz<DWM>(r, col)) = ra[l];
        }
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int e = tid + l * GTH, r = e / (GW / 8), col = 8 * (e % (GW / 8));
            *reinterpret_cast<u32x4*>(sB + swz<GW>(r, col)) = rb[l];
        }
        __syncthreads();
        if (i + 1 < n_it) fetch(i + 1);
#pragma unroll
        for (int kk = 0; kk < DWT / 32; ++kk) {
            const bf16x8 a = as_bf16x8(tr_read8<DWM>(sA, 32 * kk + 8 * g, 16 * wv + 4 * q4));
#pragma unroll
            for (int tb = 0; tb < 8; ++tb)
                acc[tb] = mfma16(a, as_bf16x8(tr_read8<GW>(sB, 32 * kk + 8 * g, 16 * tb + 4 * q4)), acc[tb]);
        }
        __syncthreads();
    }
    // lane holds rows m0 + 16 wv + 4g + r, columns 16 tb + c16
    float* dst = p.part + ((size_t)pi * p.H + h) * p.K * GW;
#pragma unroll
    for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(m0 + 16 * wv + 4 * g + r) * GW + 16 * tb + c16] = acc[tb][r];
}

// dW1, dW3 = the partial sums added in part order
__global__ void __launch_bounds__(GTH) dw_reduce(const float* part, float* dw1, float* dw3, int n_parts, int H,
                                                 int d_phi) {
    const size_t K = 2 * (size_t)d_phi;
    const size_t per = (size_t)H * K * GW;
    const size_t e = (size_t)blockIdx.x * GTH + threadIdx.x;
    if (e >= per) return;
    float s = 0.0f;
    for (int i = 0; i < n_parts; ++i) s += part[(size_t)i * per + e];
    const size_t nn = e % GW, m = (e / GW) % K, h = e / (GW * K);
    if (m < (size_t)d_phi) dw1[(h * d_phi + m) * GW + nn] = s;
    else dw3[(h * d_phi + (m - d_phi)) * GW + nn] = s;
}

// wcat[h][n][k] = W1[h][k][n] for k < d_phi, W3[h][k - d_phi][n] after
__global__ void __launch_bounds__(GTH) wcat_kernel(const uint16_t* w1, const uint16_t* w3, uint16_t* wcat, int H,
                                                   int d_phi) {
    const size_t K = 2 * (size_t)d_phi;
    const size_t total = (size_t)H * GW * K;
    for (size_t e = (size_t)blockIdx.x * GTH + threadIdx.x; e < total; e += (size_t)gridDim.x * GTH) {
        const size_t k = e % K, nn = (e / K) % GW, h = e / (K * GW);
        wcat[e] = k < (size_t)d_phi ? w1[(h * d_phi + k) * GW + nn] : w3[(h * d_phi + (k - d_phi)) * GW + nn];
    }
}

}  // namespace

bool swiglu_backward_supported(const Shape& s) {
    return s.bf16 && s.swiglu && s.d_k == GW && s.d_v == GW && s.d_phi % GW == 0 && s.d_phi <= 512;
}

hipError_t launch_swiglu_gate(const Shape& s, bool grads, const void* x, void* phi, const void* dphi, void* dg,
                              const float* eta, float eta_scalar, float beta, int eta_kind, bool scale_eta,
                              bool bidir, hipStream_t st) {
    GateParams p{};
    p.x = static_cast<const uint16_t*>(x);
    p.w1 = static_cast<const uint16_t*>(s.w1);
    p.w3 = static_cast<const uint16_t*>(s.w3);
    p.phi = static_cast<uint16_t*>(phi);
    p.dphi = static_cast<const uint16_t*>(dphi);
    p.dg = static_cast<uint16_t*>(dg);
    p.eta = eta;
    p.eta_scalar = eta_scalar;
    p.beta = beta;
    p.eta_kind = eta_kind;
    p.scale_eta = scale_eta ? 1 : 0;
    p.bidir = bidir ? 1 : 0;
    p.T = s.T;
    p.H = s.H;
    p.d_phi = s.d_phi;
    p.n_seq = s.n_seq();
    p.n_tiles = (s.T + GT - 1) / GT;
    const dim3 grid((unsigned)(s.n_seq() * ((p.n_tiles + GTPW - 1) / GTPW)), (unsigned)(s.d_phi / GW));
    if (grads) hipLaunchKernelGGL(gate_kernel<G_GRADS>, grid, dim3(GTH), 0, st, p);
    else hipLaunchKernelGGL(gate_kernel<G_FEATURES>, grid, dim3(GTH), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_swiglu_dx(const Shape& s, const void* dg, const void* wcat, void* dx, hipStream_t st) {
    DxParams p{};
    p.dg = static_cast<const uint16_t*>(dg);
    p.wcat = static_cast<const uint16_t*>(wcat);
    p.dx = static_cast<uint16_t*>(dx);
    p.T = s.T;
    p.H = s.H;
    p.K = 2 * s.d_phi;
    p.n_tiles = (s.T + GT - 1) / GT;
    hipLaunchKernelGGL(dx_kernel, dim3((unsigned)(s.n_seq() * p.n_tiles)), dim3(GTH), 0, st, p);
    return hipGetLastError();
}

// token ranges per (b, h) of dw_kernel: enough workgroups to fill the device
int swiglu_dw_split(const Shape& s) {
    const int n_mt = 2 * s.d_phi / DWM;
    const int n_panels = (s.T + DWT - 1) / DWT;
    int split = 1;
    while ((long)s.B * s.H * n_mt * split < 1024 && 2 * split <= n_panels) split *= 2;
    return split;
}

size_t swiglu_dw_partial_bytes(const Shape& s) {
    return (size_t)s.B * swiglu_dw_split(s) * s.H * (2 * s.d_phi) * GW * sizeof(float);
}

hipError_t launch_swiglu_dw(const Shape& s, const void* dg_q, const void* dg_k, const void* x_q, const void* x_k,
                            float* part, float* dw1, float* dw3, hipStream_t st) {
    DwParams p{};
    p.dg_q = static_cast<const uint16_t*>(dg_q);
    p.dg_k = static_cast<const uint16_t*>(dg_k);
    p.x_q = static_cast<const uint16_t*>(x_q);
    p.x_k = static_cast<const uint16_t*>(x_k);
    p.part = part;
    p.B = s.B;
    p.H = s.H;
    p.T = s.T;
    p.K = 2 * s.d_phi;
    p.n_split = swiglu_dw_split(s);
    const int n_parts = s.B * p.n_split;
    hipLaunchKernelGGL(dw_kernel, dim3((unsigned)(n_parts * s.H * (p.K / DWM))), dim3(GTH), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t per = (size_t)s.H * p.K * GW;
    hipLaunchKernelGGL(dw_reduce, dim3((unsigned)((per + GTH - 1) / GTH)), dim3(GTH), 0, st, part, dw1, dw3, n_parts,
                       s.H, s.d_phi);
    return hipGetLastError();
}

hipError_t launch_swiglu_wcat(const Shape& s, void* wcat, hipStream_t st) {
    hipLaunchKernelGGL(wcat_kernel, dim3(256), dim3(GTH), 0, st, static_cast<const uint16_t*>(s.w1),
                       static_cast<const uint16_t*>(s.w3), static_cast<uint16_t*>(wcat), s.H, s.d_phi);
    return hipGetLastError();
}

}  // namespace ttt
