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
//   gate_kernel      phi = silu(X W1^T) * (X W3^T) for one 128-feature slice, written
//                    slice-major [slice][seq][T][128] (the operand layout of the
//                    feature-space forwards)
//   chain_dx_kernel  dx from x and dphi: u, g, du and dg of a 32-feature block in
//                    registers, contracted with the block's W rows at once
//   chain_dw_kernel  [dW1 ; dW3] of a 32-feature block = sum over q, k, batch and tokens
//                    of [du | dg]^T x, recomputing du and dg the same way: fp32 partial
//                    sums over token ranges, then dw_reduce adds them in a fixed order
//                    (the result does not depend on scheduling)
// Nothing of size tokens x d_phi besides phi and dphi themselves is written.
//
// Register layouts (lane l, c16 = l % 16, g = l / 16): A operand A[m = c16][k = 8g ..
// 8g+7], B operand B[k = 8g .. 8g+7][n = c16], D result D[m = 4g .. 4g+3][n = c16].
// K-contiguous operands are 16-byte row reads of swizzled LDS tiles; the others are
// transpose reads (four rows of one column a lane).

#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_tiles.h"

namespace ttt {
namespace {

constexpr int GT = 64;     // tokens per tile
constexpr int GW = 128;    // input width d_k and feature slice width
constexpr int GTH = 256;   // threads

// 1 / (1 + e^-u) with the hardware exp2 and reciprocal (about 1 ulp each; the results
// are rounded to bf16)
__device__ __forceinline__ float sigmoid_f32(float u) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * 1.4426950408889634f));
}

struct GateParams {
    const uint16_t* x;       // [seq][T][128] raw inputs (q or k)
    const uint16_t* w1;      // [H][d_phi][128]
    const uint16_t* w3;
    uint16_t* phi;           // [P][seq][T][128]
    int T, H, d_phi, n_seq, n_tiles;
};

constexpr int GTPW = 8;    // token tiles per workgroup of gate_kernel (the weights stay in LDS)

// phi = silu(X W1^T) * (X W3^T) for one 128-feature slice (blockIdx.y) and GTPW tiles of
// 64 tokens of one sequence
__global__ void __launch_bounds__(GTH) gate_kernel(GateParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sX[GT * GW];
    __shared__ __attribute__((aligned(16))) uint16_t sW1[GW * GW];
    __shared__ __attribute__((aligned(16))) uint16_t sW3[GW * GW];

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
    // x of a tile: thread tid copies 16-byte pieces tid + 256 i; the next tile's are
    // loaded while this one is used
    u32x4 xp[4];
    auto fetch_x = [&](int tile) {
        const int t0 = tile * GT, n = min(GT, p.T - t0);
        const size_t row0 = (size_t)seq * p.T + t0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + GTH * i, r = e >> 4, col = 8 * (e & 15);
            xp[i] = r < n ? *reinterpret_cast<const u32x4*>(p.x + (row0 + r) * GW + col) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (grp * GTPW < tile_end) fetch_x(grp * GTPW);
    for (int tile = grp * GTPW; tile < tile_end; ++tile) {
        const int t0 = tile * GT;
        const int n = min(GT, p.T - t0);
        const size_t row0 = (size_t)seq * p.T + t0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + GTH * i, r = e >> 4, col = 8 * (e & 15);
            *reinterpret_cast<u32x4*>(sX + swz<GW>(r, col)) = xp[i];
        }
        __syncthreads();   // the tile's x (and, the first time, the weights)
        if (tile + 1 < tile_end) fetch_x(tile + 1);

        // wave wv: tokens 16 wv .. +15, all eight 16-feature tiles of the slice, as
        // U^T = W1 X^T and G^T: lane (c16, g) ends with features 16 tb + 4g .. +3 of
        // token 16 wv + c16
        f32x4 U[8], G[8];
#pragma unroll
        for (int tb = 0; tb < 8; ++tb) U[tb] = G[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < GW / 32; ++kk) {
            const bf16x8 xb = as_bf16x8(lds_read16(sX + swz<GW>(16 * wv + c16, 32 * kk + 8 * g)));
#pragma unroll
            for (int tb = 0; tb < 8; ++tb) {
                U[tb] = mfma16(as_bf16x8(lds_read16(sW1 + swz<GW>(16 * tb + c16, 32 * kk + 8 * g))), xb, U[tb]);
                G[tb] = mfma16(as_bf16x8(lds_read16(sW3 + swz<GW>(16 * tb + c16, 32 * kk + 8 * g))), xb, G[tb]);
            }
        }
        // the features into LDS over the staged x (8 bytes a lane and tile), then
        // 16-byte stores
        __syncthreads();   // every wave is done reading sX for its products
#pragma unroll
        for (int tb = 0; tb < 8; ++tb) {
            float ph[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ph[r] = U[tb][r] * sigmoid_f32(U[tb][r]) * G[tb][r];
            *reinterpret_cast<u32x2*>(sX + swz<GW>(16 * wv + c16, 16 * tb + 4 * g)) =
                u32x2{pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3])};
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + GTH * i, r = e >> 4, col = 8 * (e & 15);
            if (r < n)
                *reinterpret_cast<u32x4*>(p.phi + (sl * slice_rows + row0 + r) * GW + col) =
                    *reinterpret_cast<const u32x4*>(sX + swz<GW>(r, col));
        }
        __syncthreads();   // the tile's LDS is used up
    }
}

// ---- the chain rule without [du | dg] in memory ----------------------------------
//
// chain_dx_kernel: dx = W1^T du + W3^T dg for 128 tokens a workgroup (32 a wave),
// all d_phi features in blocks of 32.  Per block a wave forms U^T = W1 X^T and
// G^T = W3 X^T (features x its tokens: the W rows of the block, staged in LDS, are
// the A operands, its x rows the B operands held in registers), then du and dg in
// registers, and adds du W1 + dg W3 of the block to its dx tile.  The product
// leaves lane (c16, g) with features 4g .. 4g+3 and 16+4g .. 16+4g+3 of token
// c16: that is an A operand of the dx product as it stands, with the contraction
// index in that order, so the B operand (W of the block, feature-contracted) is
// read in the same order by two transpose reads of four rows.
// chain_dw_kernel: dW1 = sum du x^T, dW3 = sum dg x^T over every token of q and k,
// for one head and one block of 32 features a workgroup (the W rows of the block
// stay in LDS).  Per panel of 128 tokens each wave forms du and dg of its 32 tokens
// as above and puts them and the tokens' x rows in LDS; then each wave contracts
// the whole panel for its own 32 columns of dW (A = du^T, B = x, both transpose
// reads).  dphi and the x rows are read once per feature block; nothing of size
// tokens x d_phi is written.

constexpr int CT = 128;    // chain_dx_kernel: tokens per workgroup
constexpr int CF = 32;     // features per block

struct ChainParams {
    const uint16_t* x;       // [seq][T][128] (chain_dw: q; x2 = k)
    const uint16_t* x2;
    const uint16_t* w1;      // [H][d_phi][128]
    const uint16_t* w3;
    const uint16_t* dphi;    // [P][seq][T][128] (chain_dw: of q; dphi2 of k)
    const uint16_t* dphi2;
    uint16_t* dx;            // chain_dx: [seq][T][128]
    float* part;             // chain_dw: [n_parts][H][2 d_phi][128] partial sums
    // dphi of token t is scaled by eta_t c_t (gate_kernel's rule) when scale_eta is set;
    // chain_dw scales the second input's only (the keys')
    const float* eta;
    float eta_scalar, beta;
    int eta_kind, scale_eta, bidir;
    int B, T, H, d_phi, n_seq, n_tiles, n_split;
};

// the scale of token t from its raw rate a (eta[row], or anything for a scalar rate)
__device__ __forceinline__ float chain_scale_of(const ChainParams& p, float a, int t) {
    float sc = p.eta_kind == ETA_SCALAR ? p.eta_scalar : (p.eta_kind == ETA_SOFTPLUS ? softplus_f32(a) : a);
    if (p.bidir && p.beta != 0.0f) sc *= (1.0f - powf(p.beta, (float)(p.T - t))) / (1.0f - p.beta);
    return sc;
}

__device__ __forceinline__ float chain_scale(const ChainParams& p, size_t row, int t) {
    return chain_scale_of(p, p.eta_kind == ETA_SCALAR ? 0.0f : p.eta[row], t);
}

// U^T and G^T of one block for 32 tokens (xop(tt, kk): the B operand x[16 tt + c16][32 kk
// + 8g ..]), and from them du and dg as A operands (k slot 8g + j = feature 4g + j for
// j < 4, 16 + 4g + j - 4 after)
template <typename XOp>
__device__ __forceinline__ void chain_block(const uint16_t* W1s, const uint16_t* W3s, XOp xop,
                                            const u32x2 (&dd)[2][2], const float (&scl)[2], int c16, int g,
                                            bf16x8 (&adu)[2], bf16x8 (&adg)[2]) {
    f32x4 U[2][2], G[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) U[mt][tt] = G[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < GW / 32; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 a1 = as_bf16x8(lds_read16(W1s + swz<GW>(16 * mt + c16, 32 * kk + 8 * g)));
            const bf16x8 a3 = as_bf16x8(lds_read16(W3s + swz<GW>(16 * mt + c16, 32 * kk + 8 * g)));
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 xb = as_bf16x8(xop(tt, kk));
                U[mt][tt] = mfma16(a1, xb, U[mt][tt]);
                G[mt][tt] = mfma16(a3, xb, G[mt][tt]);
            }
        }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        float du[8], dg[8];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t wd = dd[mt][tt][r >> 1];
                const float d = __uint_as_float((r & 1) ? (wd & 0xffff0000u) : (wd << 16)) * scl[tt];
                const float u = U[mt][tt][r], gg = G[mt][tt][r];
                const float sg = sigmoid_f32(u);
                du[4 * mt + r] = d * gg * sg * (1.0f + u * (1.0f - sg));
                dg[4 * mt + r] = d * u * sg;
            }
        adu[tt] = as_bf16x8(u32x4{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]), pack_bf16x2(du[4], du[5]),
                                  pack_bf16x2(du[6], du[7])});
        adg[tt] = as_bf16x8(u32x4{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]), pack_bf16x2(dg[4], dg[5]),
                                  pack_bf16x2(dg[6], dg[7])});
    }
}

__global__ void __launch_bounds__(GTH, 2) chain_dx_kernel(ChainParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sW[2 * 2 * CF * GW];   // [buffer][W1, W3][32 x 128]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4, q4 = lane & 3;
    // XCD-aware: consecutive units (the tiles of one sequence, which read the same W)
    // share an XCD's L2
    const int u = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_seq * p.n_tiles) return;
    const int tile = u % p.n_tiles;
    const int seq = u / p.n_tiles;
    const int h = seq % p.H;
    const size_t srow = (size_t)seq * p.T;
    const size_t slice_rows = (size_t)p.n_seq * p.T;
    const int tw = tile * CT + 32 * wv;           // first token of the wave
    const uint16_t* w1 = p.w1 + (size_t)h * p.d_phi * GW;
    const uint16_t* w3 = p.w3 + (size_t)h * p.d_phi * GW;
    const int n_blocks = p.d_phi / CF;

    // x rows of the wave as B operands: lane (c16, g) holds x[tw + 16 tt + c16][32 kk + 8g ..]
    u32x4 xf[2][4];
    float scl[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = tw + 16 * tt + c16;
        const bool ok = t < p.T;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            xf[tt][kk] = ok ? *reinterpret_cast<const u32x4*>(p.x + (srow + t) * GW + 32 * kk + 8 * g)
                            : u32x4{0u, 0u, 0u, 0u};
        scl[tt] = ok ? (p.scale_eta ? chain_scale(p, srow + t, t) : 1.0f) : 0.0f;
    }
    // W rows of a block: thread tid copies 16-byte pieces tid and tid + 256 of each matrix
    u32x4 wr[4];
    auto fetch_w = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + GTH * (i & 1), r = e >> 4, col = 8 * (e & 15);
            wr[i] = *reinterpret_cast<const u32x4*>(((i >> 1) ? w3 : w1) + (size_t)(b * CF + r) * GW + col);
        }
    };
    auto put_w = [&](uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + GTH * (i & 1), r = e >> 4, col = 8 * (e & 15);
            *reinterpret_cast<u32x4*>(dst + (i >> 1) * CF * GW + swz<GW>(r, col)) = wr[i];
        }
    };
    // dphi of the block in the layout of the U^T product: 4 features of one token a load
    u32x2 dr[2][2];
    auto fetch_d = [&](int b) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int f = b * CF + 16 * mt + 4 * g, t = tw + 16 * tt + c16;
                dr[mt][tt] = t < p.T ? *reinterpret_cast<const u32x2*>(
                                           p.dphi + ((size_t)(f >> 7) * slice_rows + srow + t) * GW + (f & (GW - 1)))
                                     : u32x2{0u, 0u};
            }
    };

    f32x4 acc[2][8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch_w(0);
    fetch_d(0);
    for (int b = 0; b < n_blocks; ++b) {
        uint16_t* W1s = sW + (b & 1) * 2 * CF * GW;
        const uint16_t* W3s = W1s + CF * GW;
        put_w(W1s);
        u32x2 dd[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) dd[mt][tt] = dr[mt][tt];
        __syncthreads();   // the block's W rows (the buffer was last read two blocks ago)
        if (b + 1 < n_blocks) {
            fetch_w(b + 1);
            fetch_d(b + 1);
        }
        bf16x8 adu[2], adg[2];
        chain_block(W1s, W3s, [&](int tt, int kk) { return xf[tt][kk]; }, dd, scl, c16, g, adu, adg);
        // dx += du W1 + dg W3: B[k][n] = W[feature of slot k][16 nt + c16]
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const bf16x8 b1 = join8(tr_read<GW>(W1s, 4 * g, 16 * nt + 4 * q4), tr_read<GW>(W1s, 16 + 4 * g, 16 * nt + 4 * q4));
            const bf16x8 b3 = join8(tr_read<GW>(W3s, 4 * g, 16 * nt + 4 * q4), tr_read<GW>(W3s, 16 + 4 * g, 16 * nt + 4 * q4));
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                acc[tt][nt] = mfma16(adu[tt], b1, acc[tt][nt]);
                acc[tt][nt] = mfma16(adg[tt], b3, acc[tt][nt]);
            }
        }
    }
    // acc[tt][nt] = dx[tw + 16 tt + 4g + r][16 nt + c16]: through LDS (the wave's 32 rows)
    // to 16-byte stores
    __syncthreads();   // every wave is done with the W buffers
    uint16_t* sO = sW + wv * 32 * GW;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sO[swz<GW>(16 * tt + 4 * g + r, 16 * nt + c16)] = f32_to_bf16_bits(acc[tt][nt][r]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i, r = e >> 4, col = 8 * (e & 15);
        const int t = tw + r;
        if (t < p.T)
            *reinterpret_cast<u32x4*>(p.dx + (srow + t) * GW + col) = *reinterpret_cast<const u32x4*>(sO + swz<GW>(r, col));
    }
}

// grid: (n_parts = B x n_split) x H x (d_phi / 32); part pi = (b, token range).  Per
// panel of 128 tokens (q's, then k's): wave wv forms du and dg of tokens 32 wv .. +31 and
// puts them and the tokens' x rows in LDS; after a barrier it adds the panel's
// contribution to dW1 and dW3 columns 32 wv .. 32 wv + 31 (all 32 features of the
// block), contracting over the 128 tokens.
__global__ void __launch_bounds__(GTH, 2) chain_dw_kernel(ChainParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sW[2 * CF * GW];   // W1, W3 rows of the block
    __shared__ __attribute__((aligned(16))) uint16_t sX[CT * GW];       // x rows of the panel
    __shared__ __attribute__((aligned(16))) uint16_t sD[CT * 2 * CF];   // [t][du 32 | dg 32]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4, q4 = lane & 3;
    const int n_fb = p.d_phi / CF;
    // XCD-aware: the feature blocks of one (part, head), which read the same x rows and
    // dphi lines, share an XCD's L2
    int blk = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (blk >= p.B * p.n_split * p.H * n_fb) return;
    const int fb = blk % n_fb;
    blk /= n_fb;
    const int h = blk % p.H;
    const int pi = blk / p.H;
    const int b = pi / p.n_split, rg = pi % p.n_split;
    const int span = (p.T + p.n_split - 1) / p.n_split;
    const int t_begin = rg * span, t_end = min(p.T, t_begin + span);
    const size_t srow = ((size_t)b * p.H + h) * p.T;
    const size_t slice_rows = (size_t)p.n_seq * p.T;
    const int f0 = fb * CF;

    {
        const uint16_t* w1 = p.w1 + ((size_t)h * p.d_phi + f0) * GW;
        const uint16_t* w3 = p.w3 + ((size_t)h * p.d_phi + f0) * GW;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + GTH * (i & 1), r = e >> 4, col = 8 * (e & 15);
            *reinterpret_cast<u32x4*>(sW + (i >> 1) * CF * GW + swz<GW>(r, col)) =
                *reinterpret_cast<const u32x4*>(((i >> 1) ? w3 : w1) + (size_t)r * GW + col);
        }
    }
    const uint16_t* W1s = sW;
    const uint16_t* W3s = sW + CF * GW;

    // acc[m][mt][nt]: dW_m rows f0 + 16 mt + 4g + r, columns 32 wv + 16 nt + c16
    f32x4 acc[2][2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[m][mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int n_pan = t_end > t_begin ? (t_end - t_begin + CT - 1) / CT : 0;
    // the x rows, dphi and raw rates of the wave's tokens in the next panel are loaded
    // while this one is used
    u32x4 xr[2][4];
    u32x2 dr[2][2];
    float ar[2];
    const bool rates = p.scale_eta && p.eta_kind != ETA_SCALAR;
    auto fetch = [&](int i) {
        const int src = i / n_pan;
        const int tw = t_begin + CT * (i % n_pan) + 32 * wv;
        const uint16_t* xm = src ? p.x2 : p.x;
        const uint16_t* dm = src ? p.dphi2 : p.dphi;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = tw + 16 * tt + c16;
            const bool ok = t < t_end;
            ar[tt] = (rates && src && ok) ? p.eta[srow + t] : 0.0f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                xr[tt][kk] = ok ? *reinterpret_cast<const u32x4*>(xm + (srow + t) * GW + 32 * kk + 8 * g)
                                : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int f = f0 + 16 * mt + 4 * g;
                dr[mt][tt] = ok ? *reinterpret_cast<const u32x2*>(
                                      dm + ((size_t)(f >> 7) * slice_rows + srow + t) * GW + (f & (GW - 1)))
                                : u32x2{0u, 0u};
            }
        }
    };
    if (n_pan > 0) fetch(0);
    __syncthreads();   // the W rows
    for (int i = 0; i < 2 * n_pan; ++i) {
        const int src = i / n_pan;
        const int tw = t_begin + CT * (i % n_pan) + 32 * wv;
        const bool scale = src && p.scale_eta;
        u32x4 xf[2][4];
        u32x2 dd[2][2];
        float scl[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = tw + 16 * tt + c16;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                xf[tt][kk] = xr[tt][kk];
                *reinterpret_cast<u32x4*>(sX + swz<GW>(32 * wv + 16 * tt + c16, 32 * kk + 8 * g)) = xf[tt][kk];
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) dd[mt][tt] = dr[mt][tt];
            scl[tt] = t < t_end ? (scale ? chain_scale_of(p, ar[tt], t) : 1.0f) : 0.0f;
        }
        if (i + 1 < 2 * n_pan) fetch(i + 1);
        bf16x8 adu[2], adg[2];
        chain_block(W1s, W3s, [&](int tt, int kk) { return xf[tt][kk]; }, dd, scl, c16, g, adu, adg);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 uu = __builtin_bit_cast(u32x4, adu[tt]), gv = __builtin_bit_cast(u32x4, adg[tt]);
            const int row = 32 * wv + 16 * tt + c16;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                *reinterpret_cast<u32x2*>(sD + swz<2 * CF>(row, 16 * mt + 4 * g)) = u32x2{uu[2 * mt], uu[2 * mt + 1]};
                *reinterpret_cast<u32x2*>(sD + swz<2 * CF>(row, CF + 16 * mt + 4 * g)) = u32x2{gv[2 * mt], gv[2 * mt + 1]};
            }
        }
        lds_barrier();   // the panel's x, du and dg rows
        // dW[f][d] += sum over the panel's 128 tokens: A[m = f][k = t] = du^T, B[k = t][n = d] = x
#pragma unroll
        for (int ks = 0; ks < CT / 32; ++ks) {
            bf16x8 bx[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) bx[nt] = as_bf16x8(tr_read8<GW>(sX, 32 * ks + 8 * g, 32 * wv + 16 * nt + 4 * q4));
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const bf16x8 a = as_bf16x8(tr_read8<2 * CF>(sD, 32 * ks + 8 * g, m * CF + 16 * mt + 4 * q4));
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) acc[m][mt][nt] = mfma16(a, bx[nt], acc[m][mt][nt]);
                }
        }
        lds_barrier();   // every wave is done with the panel's rows
    }
    float* dst = p.part + ((size_t)pi * p.H + h) * (size_t)(2 * p.d_phi) * GW;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(m * p.d_phi + f0 + 16 * mt + 4 * g + r) * GW + 32 * wv + 16 * nt + c16] = acc[m][mt][nt][r];
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

}  // namespace

bool swiglu_backward_supported(const Shape& s) {
    return s.bf16 && s.swiglu && s.d_k == GW && s.d_v == GW && s.d_phi % GW == 0 && s.d_phi <= 512;
}

hipError_t launch_swiglu_features(const Shape& s, const void* x, void* phi, hipStream_t st) {
    GateParams p{};
    p.x = static_cast<const uint16_t*>(x);
    p.w1 = static_cast<const uint16_t*>(s.w1);
    p.w3 = static_cast<const uint16_t*>(s.w3);
    p.phi = static_cast<uint16_t*>(phi);
    p.T = s.T;
    p.H = s.H;
    p.d_phi = s.d_phi;
    p.n_seq = s.n_seq();
    p.n_tiles = (s.T + GT - 1) / GT;
    const dim3 grid((unsigned)(s.n_seq() * ((p.n_tiles + GTPW - 1) / GTPW)), (unsigned)(s.d_phi / GW));
    hipLaunchKernelGGL(gate_kernel, grid, dim3(GTH), 0, st, p);
    return hipGetLastError();
}

static ChainParams chain_params(const Shape& s, const float* eta, float eta_scalar, float beta, int eta_kind,
                                 bool scale_eta, bool bidir) {
    ChainParams p{};
    p.w1 = static_cast<const uint16_t*>(s.w1);
    p.w3 = static_cast<const uint16_t*>(s.w3);
    p.eta = eta;
    p.eta_scalar = eta_scalar;
    p.beta = beta;
    p.eta_kind = eta_kind;
    p.scale_eta = scale_eta ? 1 : 0;
    p.bidir = bidir ? 1 : 0;
    p.B = s.B;
    p.T = s.T;
    p.H = s.H;
    p.d_phi = s.d_phi;
    p.n_seq = s.n_seq();
    return p;
}

hipError_t launch_swiglu_chain_dx(const Shape& s, const void* x, const void* dphi, void* dx, const float* eta,
                                  float eta_scalar, float beta, int eta_kind, bool scale_eta, bool bidir,
                                  hipStream_t st) {
    ChainParams p = chain_params(s, eta, eta_scalar, beta, eta_kind, scale_eta, bidir);
    p.x = static_cast<const uint16_t*>(x);
    p.dphi = static_cast<const uint16_t*>(dphi);
    p.dx = static_cast<uint16_t*>(dx);
    p.n_tiles = (s.T + CT - 1) / CT;
    hipLaunchKernelGGL(chain_dx_kernel, dim3((unsigned)((s.n_seq() * p.n_tiles + 7) / 8 * 8)), dim3(GTH), 0, st, p);
    return hipGetLastError();
}

// token ranges per (b, h) of chain_dw_kernel: enough workgroups to fill the device twice
int swiglu_chain_dw_split(const Shape& s) {
    const int n_fb = s.d_phi / CF;
    const int n_pan = (s.T + CT - 1) / CT;
    int split = 1;
    while ((long)s.B * s.H * n_fb * split < 1024 && 2 * split <= n_pan) split *= 2;
    return split;
}

size_t swiglu_chain_dw_partial_bytes(const Shape& s) {
    return (size_t)s.B * swiglu_chain_dw_split(s) * s.H * (2 * s.d_phi) * GW * sizeof(float);
}

hipError_t launch_swiglu_chain_dw(const Shape& s, const void* x_q, const void* x_k, const void* dphi_q,
                                  const void* dphi_k, const float* eta, float eta_scalar, float beta, int eta_kind,
                                  bool bidir, float* part, float* dw1, float* dw3, hipStream_t st) {
    ChainParams p = chain_params(s, eta, eta_scalar, beta, eta_kind, true, bidir);
    p.x = static_cast<const uint16_t*>(x_q);
    p.x2 = static_cast<const uint16_t*>(x_k);
    p.dphi = static_cast<const uint16_t*>(dphi_q);
    p.dphi2 = static_cast<const uint16_t*>(dphi_k);
    p.part = part;
    p.n_split = swiglu_chain_dw_split(s);
    const int n_parts = s.B * p.n_split;
    hipLaunchKernelGGL(chain_dw_kernel, dim3((unsigned)((n_parts * s.H * (s.d_phi / CF) + 7) / 8 * 8)), dim3(GTH), 0,
                       st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t per = (size_t)s.H * 2 * s.d_phi * GW;
    hipLaunchKernelGGL(dw_reduce, dim3((unsigned)((per + GTH - 1) / GTH)), dim3(GTH), 0, st, part, dw1, dw3, n_parts,
                       s.H, s.d_phi);
    return hipGetLastError();
}

}  // namespace ttt
