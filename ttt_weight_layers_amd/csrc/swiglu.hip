// SwiGLU feature-map forward (Variant 2 of Table 2 on the thelatestinai.com
// page: the two-layer MLP fast weight with only its last layer updated) on
// 32x32x16 bf16 MFMA tiles, for d_k = d_v = 128 and d_phi a multiple of 128.
//
// The frozen first layer is the feature map phi(x) = silu(W1 x) * (W3 x),
// silu(u) = u / (1 + e^-u); the updated last layer is the fp32 state
// S in R^{d_v x d_phi}.  With the features in place of q and k the layer is the
// same chunked linear attention as the identity map (kualia.ai blog, "The
// Linear Attention Equivalence"): per chunk of n tokens entered with the
// T-form state (T = S + beta/(1-beta) M),
//   o_i = T phi(q_i) - beta^{i+2}/(1-beta) M phi(q_i)
//         + sum_{j<=i} eta_j c_{i-j} (phi(q_i) . phi(k_j)) v_j
//   T  <- T + sum_j eta_j v_j phi(k_j)^T / (1 - beta)
//   M  <- beta^n M + sum_j eta_j beta^{n-1-j} v_j phi(k_j)^T.
//
// Work split.  The state of one sequence (T and M: 2 x 128 x 512 fp32 for
// d_phi = 512) is larger than the register file of a compute unit, so the
// feature dimension is split into slices of 128: one workgroup per (sequence,
// slice) keeps T and M of its 128 features, computes those features of phi(q)
// and phi(k) from the raw q and k rows, and produces the slice's part of every
// output row; o is the sum of the slices' parts (both the readout and the
// intra-chunk scores are sums over features).  Each slice reads q, k and v in
// full: the workgroups of one sequence are launched on one XCD, so the repeated
// reads are served by its L2.
//
// Inside a workgroup: eight waves in two roles, one of each on every SIMD, so
// that the vector-ALU work of one (the silu of the feature map) overlaps the
// matrix-core work of the other.
//   State waves w = 0..3 own value columns 32w .. 32w+31 of the slice's T^T and
//   M^T (4 feature tiles of 32 x 32 each, in the feature order sigma described
//   in chunk_wide.hip, so that the state is the A operand of the readout without
//   data movement): readout, intra-chunk product, partial output, update.
//   Feature waves w = 0..3 compute features 32w .. 32w+31 of the slice for the
//   next chunk: W1 and W3 rows of those features are held as MFMA A operands (8
//   k-steps each), the raw rows of q and k are the B operands (16-byte row
//   reads), and the products land with every lane holding 16 features of one
//   token in two runs of 8 consecutive ones (the same sigma order on the rows of
//   W), which go to LDS as two 16-byte stores.  Three of them also form the
//   causal score tiles of the current chunk.
//
// LDS pools (separate __shared__ objects, so that reads of one are never made
// to wait for copies into another): the features of two chunks (the current
// one, read by the state waves; the next one, being written), raw q and k of
// two chunks (the next one, being read; the one after, in flight), v of the
// current chunk, score fragments and per-token weights.  Per chunk c:
//   state waves:   readout from phi(c), v fragments | P | copy v of chunk c+1,
//                  intra-chunk term, partial output, update | wait | S
//   feature waves: copy raw rows of chunk c+2, score tiles of chunk c, phi(q)
//                  of chunk c+1 | P | phi(k) of chunk c+1 (it takes the weights
//                  of chunk c+1, formed before P) | wait | S
// where P and S are the two workgroup barriers of the step.

#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "internal.h"
#include "lds_tiles.h"

#define TTT_INLINE __attribute__((always_inline))

namespace ttt {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int SC = 64;       // tokens per chunk
constexpr int SD = 128;      // d_k = d_v = features per slice
constexpr int SNW = 4;       // waves
constexpr int SNT = SNW * 64;
constexpr int SFT = SD / 32; // feature tiles of a wave's state
constexpr int SKB = SC / 16; // 16-token contraction blocks per chunk
constexpr int SKS = SD / 16; // k-steps of the feature map (d_k / 16)
constexpr int STILE = SC * SD;

struct SwigluParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* eta;
    const uint16_t* w1;     // [H][d_phi][128]
    const uint16_t* w3;
    float* partial;         // each slice's part of o, bf16 in register order (see store)
    float eta_scalar;
    float beta;
    int eta_kind;
    int T, H, d_phi, slices, n_units, n_seq, n_chunks;
    size_t n_rows;          // B * H * T
};

__device__ __forceinline__ f32x16 smfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// accumulator registers 8 kh .. 8 kh + 7 of a 32x32 tile as one bf16 operand
__device__ __forceinline__ bf16x8 half_operand(const f32x16& x, int kh) {
    const int b = 8 * kh;
    u32x4 u = {pack_bf16x2(x[b + 0], x[b + 1]), pack_bf16x2(x[b + 2], x[b + 3]),
               pack_bf16x2(x[b + 4], x[b + 5]), pack_bf16x2(x[b + 6], x[b + 7])};
    return as_bf16x8(u);
}

// 8 packed bf16 times one fp32 factor, re-rounded to bf16
__device__ __forceinline__ bf16x8 scale8u(const u32x4& raw, float f) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        u[e] = pack_bf16x2(__uint_as_float(raw[e] << 16) * f, __uint_as_float(raw[e] & 0xffff0000u) * f);
    return as_bf16x8(u);
}

// silu(u) * g with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float swiglu_f32(float u, float g) {
    const float e = __builtin_amdgcn_exp2f(-u * 1.4426950408889634f);
    return u * __builtin_amdgcn_rcpf(1.0f + e) * g;
}

// Transpose read of a swizzled 128-wide tile (see lds_tiles.h tr_read)
__device__ __forceinline__ u32x2 tr_rd(const uint16_t* tile, int r0, int col_q, int l16) {
    const uint16_t* p = tile + swz<SD>(r0 + (l16 >> 2), col_q);
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TTT_LDS bf16x4_t*)(p));
    return __builtin_bit_cast(u32x2, x);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

constexpr int SWAVES = 2 * SNW;          // four state waves, four feature waves
constexpr int SNT2 = SWAVES * 64;

template <bool MOM, bool ETAV>
__global__ void __launch_bounds__(SNT2, 1) swiglu_kernel(SwigluParams p) {
    // The compiler lays LDS objects out by decreasing size, then in declaration
    // order.  The features are read most, with several offsets per lane, so they
    // come first: below 64 KiB their base fits the offset field of the ds
    // instructions and an access needs no address register of its own.
    __shared__ __attribute__((aligned(16))) uint16_t phq0[STILE];   // phi(q), phi(k) of even chunks
    __shared__ __attribute__((aligned(16))) uint16_t phk0[STILE];
    __shared__ __attribute__((aligned(16))) uint16_t phq1[STILE];   // ... of odd chunks
    __shared__ __attribute__((aligned(16))) uint16_t phk1[STILE];
    __shared__ __attribute__((aligned(16))) uint16_t vt[STILE];     // v of the chunk in work
    __shared__ __attribute__((aligned(16))) uint16_t xq0[STILE];    // raw q, k of even chunks
    __shared__ __attribute__((aligned(16))) uint16_t xk0[STILE];
    __shared__ __attribute__((aligned(16))) uint16_t xq1[STILE];    // ... of odd chunks
    __shared__ __attribute__((aligned(16))) uint16_t xk1[STILE];
    __shared__ __attribute__((aligned(16))) uint16_t pfrag[3 * 2 * 64 * 8];
    // per-token weights of the two chunk parities (w_T, M factor), c_r, beta^r, score coefficients
    __shared__ __attribute__((aligned(16))) float sF[4 * SC + 2 * (SC + 1) + 2 + 2 * SC];
    __shared__ __attribute__((aligned(16))) float seta[2 * SC];     // rates of two chunks (by parity)
    float* const w_a = sF;
    float* const w_b = sF + 2 * SC;
    float* sC = sF + 4 * SC;
    float* sBP = sC + SC + 1;
    float* sK = sBP + SC + 1 + 2;
    auto s_wt = [](float* w) TTT_INLINE { return w; };         // eta_j / (1 - beta)
    auto s_wm = [](float* w) TTT_INLINE { return w + SC; };    // (1 - beta) beta^{n-1-j} / rho'
    u32x4* const P_lds = reinterpret_cast<u32x4*>(pfrag);

    // ---- unit: (sequence, feature slice); the slices of a sequence on one XCD ----
    const int G = gridDim.x;
    const int u = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_units) return;
    const int fs = u % p.slices;
    const int seq = u / p.slices;
    const int head = seq % p.H;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const bool feat_wave = wave >= SNW;          // workgroup-uniform per wave
    const int wv = wave & (SNW - 1);             // index within the wave's role
    const int n32 = lane & 31, hh = lane >> 5;
    const int g16 = (lane >> 4) & 1;
    const int q4 = lane & 3;
    const int l16 = lane & 15;
    const float beta = p.beta;
    const float inv1mb = 1.0f / (1.0f - beta);
    const int t_end = p.T;
    const int n_chunks = (t_end + SC - 1) / SC;
    const size_t seq_row = (size_t)seq * p.T;

    // element offsets of this lane's 16-byte row reads: row n32, columns 16 kb + 8 hh
    // (row 32 + n32 is 4096 elements further)
    int offr[SKS];
#pragma unroll
    for (int kb = 0; kb < SKS; ++kb) offr[kb] = swz<SD>(n32, 16 * kb + 8 * hh);

    // ---- asynchronous staging (buffer loads straight into LDS, see chunk_wide.hip):
    // each role's wave wv copies row groups wv, wv+4, wv+8, wv+12 of its tiles ----
    const int wv_s = __builtin_amdgcn_readfirstlane(wv);
    const int lane_row = lane >> 4;
    const int lane_col = 8 * ((lane & 15) ^ (4 * lane_row + wv));
    int voff[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) voff[gi] = 2 * ((4 * (wv + 4 * gi) + lane_row) * SD + lane_col);
    auto copy_start = [&](int t) TTT_INLINE { return t < t_end ? t : t_end - 1; };
    auto copy = [&](uint16_t* dst, const uint16_t* tensor, int t0, int gi) TTT_INLINE {
        const int n = min(SC, t_end - t0);
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)(tensor + (seq_row + t0) * SD), (short)0, n * SD * 2, 0x00020000);
        const int grp = wv_s + 4 * gi;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TTT_LDS void*)(dst + grp * 4 * SD), 16, voff[gi], 0, 0, 0);
    };

    if (wave == 0) coefficient_scan<SC>(beta, sC, sBP);
    __syncthreads();   // coefficient tables
    const float k0 = 1.0f - beta;   // the phi(k) rows carry eta / (1 - beta)
    if (tid < 2 * SC) sK[tid] = tid >= SC ? k0 * sC[tid - SC] : 0.0f;

    if (feat_wave) {
        // =================== feature waves: phi of the next chunk ===================
        // this wave's 32 features of W1 and W3 as A operands (rows in sigma order)
        bf16x8 w1f[SKS], w3f[SKS];
        {
            const int m = n32;
            const int sig = 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
            const size_t row = (size_t)head * p.d_phi + (size_t)fs * SD + 32 * wv + sig;
            const uint16_t* r1 = p.w1 + row * SD + 8 * hh;
            const uint16_t* r3 = p.w3 + row * SD + 8 * hh;
#pragma unroll
            for (int s = 0; s < SKS; ++s) {
                w1f[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(r1 + 16 * s));
                w3f[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(r3 + 16 * s));
            }
        }
        auto stage_x = [&](uint16_t* dq, uint16_t* dk, int t0) TTT_INLINE {   // 8 copies
            const int t = copy_start(t0);
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                copy(dq, p.q, t, gi);
                copy(dk, p.k, t, gi);
            }
        };
        // Features 32 wv .. 32 wv + 31 of one 32-token tile (rows 32I .. 32I+31 staged in
        // X): two independent accumulation chains, W1 x and W3 x.  Lane (n32, hh) ends
        // with 16 features of token 32I + n32 in two runs of 8 (the sigma order of the W
        // rows).
        auto chain = [&](const uint16_t* X, int I, f32x16& u1, f32x16& u3) TTT_INLINE {
            u1 = f32x16{};
            u3 = f32x16{};
#pragma unroll
            for (int s = 0; s < SKS; ++s) {
                const bf16x8 b = as_bf16x8(lds_read16(X + offr[s] + 4096 * I));
                u1 = smfma(w1f[s], b, u1);
                u3 = smfma(w3f[s], b, u3);
            }
        };
        // silu(W1 x) * (W3 x) of a finished tile to dst; phi(k) rows (wt) take the weight
        // w_T of their token, so that the scores and the T update take v as it is.  With
        // a next tile, its chain is issued in the same loop as this arithmetic and the
        // compiler interleaves the two (a fixed pattern of one product per six vector
        // instructions ran 2% slower).
        auto finish = [&](const f32x16& c1, f32x16 c3, uint16_t* dst, int I, float* wt, const uint16_t* Xn, int In,
                          f32x16* n1, f32x16* n3) TTT_INLINE {
            if (wt) {
                const float wj = s_wt(wt)[32 * I + n32];
#pragma unroll
                for (int r = 0; r < 16; ++r) c3[r] *= wj;
            }
            u32x4 half[2];
            if (n1) {
                *n1 = f32x16{};
                *n3 = f32x16{};
            }
#pragma unroll
            for (int s = 0; s < SKS; ++s) {
                if (n1) {
                    const bf16x8 b = as_bf16x8(lds_read16(Xn + offr[s] + 4096 * In));
                    *n1 = smfma(w1f[s], b, *n1);
                    *n3 = smfma(w3f[s], b, *n3);
                }
                half[s >> 2][s & 3] = pack_bf16x2(swiglu_f32(c1[2 * s], c3[2 * s]), swiglu_f32(c1[2 * s + 1], c3[2 * s + 1]));
            }
            *reinterpret_cast<u32x4*>(dst + swz<SD>(32 * I + n32, 32 * wv + 8 * hh)) = half[0];
            *reinterpret_cast<u32x4*>(dst + swz<SD>(32 * I + n32, 32 * wv + 16 + 8 * hh)) = half[1];
        };

        stage_x(xq0, xk0, 0);
        stage_x(xq1, xk1, SC);
        wait_vm0();
        lds_barrier();   // B0: raw rows of chunk 0, v of chunk 0, weights of chunk 0
        {
            f32x16 a1, a3, b1, b3;
            chain(xq0, 0, a1, a3);
            finish(a1, a3, phq0, 0, nullptr, xq0, 1, &b1, &b3);
            finish(b1, b3, phq0, 1, nullptr, xk0, 0, &a1, &a3);
            finish(a1, a3, phk0, 0, w_a, xk0, 1, &b1, &b3);
            finish(b1, b3, phk0, 1, w_a, nullptr, 0, nullptr, nullptr);
        }
        lds_barrier();   // B1: features of chunk 0

        // score tile of feature waves 0..2: (J, I) = (0,0), (0,1), (1,1); register r holds
        // j = 32 sJ + 8 (r / 4) + 4h + r % 4 of token i = 32 sI + n
        const int sJ = (wv >= 2) ? 1 : 0;
        const int sI = (wv == 0) ? 0 : 1;
        const float* coef = sK + (SC + 32 * (sI - sJ) + n32 - 4 * hh);
        // S^T = K Q^T of chunk (PQ, PK), scaled by c_{i-j} (1 - beta) (the rate is in the
        // phi(k) rows), to LDS as ready B fragments of the intra-chunk product
        auto scores = [&](const uint16_t* PQ, const uint16_t* PK) TTT_INLINE {
            if (wv < 3) {
                f32x16 acc = f32x16{};
#pragma unroll
                for (int kb = 0; kb < SKS; ++kb)
                    acc = smfma(as_bf16x8(lds_read16(PK + offr[kb] + 4096 * sJ)),
                                as_bf16x8(lds_read16(PQ + offr[kb] + 4096 * sI)), acc);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] *= coef[-(8 * (r >> 2) + (r & 3))];
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
                    P_lds[(wv * 2 + kh) * 64 + lane] = __builtin_bit_cast(u32x4, half_operand(acc, kh));
            }
        };

        // step c: the score tiles of chunk c (features in (cq, ck)); the raw rows of chunk
        // c+2 go to (fq, fk) (those of chunk c are done); the features of chunk c+1 are
        // formed from (nq, nk) into (dq, dk): phi(q) before the middle barrier, phi(k)
        // after it (it needs the chunk's weights)
        auto step = [&](int c, const uint16_t* cq, const uint16_t* ck, uint16_t* fq, uint16_t* fk,
                        const uint16_t* nq, const uint16_t* nk, uint16_t* dq, uint16_t* dk,
                        float* wn) TTT_INLINE -> bool {
            const bool has_next = c + 1 < n_chunks;
            if (has_next) stage_x(fq, fk, (c + 2) * SC);
            scores(cq, ck);
            // tiles q0, q1, k0, k1 of chunk c+1 in a software pipeline; the weights of
            // chunk c+1 (needed from k0's arithmetic on) are published by the middle
            // barrier, so q1's products are held across it
            f32x16 a1, a3, b1, b3;
            if (has_next) {
                chain(nq, 0, a1, a3);
                finish(a1, a3, dq, 0, nullptr, nq, 1, &b1, &b3);
            }
            lds_barrier();   // P (placed so that both roles bring about equal work to it)
            if (!has_next) return false;
            finish(b1, b3, dq, 1, nullptr, nk, 0, &a1, &a3);
            finish(a1, a3, dk, 0, wn, nk, 1, &b1, &b3);
            finish(b1, b3, dk, 1, wn, nullptr, 0, nullptr, nullptr);
            wait_vm0();      // raw rows of chunk c+2
            lds_barrier();   // S
            return true;
        };
        for (int c = 0;; c += 2) {
            if (!step(c, phq0, phk0, xq0, xk0, xq1, xk1, phq1, phk1, w_b)) break;
            if (!step(c + 1, phq1, phk1, xq1, xk1, xq0, xk0, phq0, phk0, w_a)) break;
        }
        wait_vm0();   // the last (empty) copies
        return;
    }

    // ===================== state waves: the slice's T and M =====================
    const int w = wv;   // value columns 32 w .. 32 w + 31
    f32x16 Ts[SFT], Ms[MOM ? SFT : 1];
#pragma unroll
    for (int ft = 0; ft < SFT; ++ft) Ts[ft] = f32x16{};
#pragma unroll
    for (int ft = 0; ft < (MOM ? SFT : 1); ++ft) Ms[ft] = f32x16{};
    // momentum M = rho Ms with a workgroup-uniform scale (see chunk_wide.hip)
    constexpr float RHO_MIN = 0x1p-60f;
    float rho = 1.0f;
    auto rho_step = [&](float r0, int n) TTT_INLINE {
        const float r = r0 * sBP[n];
        return r < RHO_MIN ? 1.0f : r;
    };
    const int col_v = 32 * w + 16 * (q4 & 1) + 8 * g16 + 4 * (q4 >> 1);
    auto col_k = [&](int ft) TTT_INLINE { return 32 * ft + 16 * g16 + 8 * (q4 & 1) + 4 * (q4 >> 1); };

    auto stage_v = [&](int t0) TTT_INLINE {   // 4 copies
        const int t = copy_start(t0);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) copy(vt, p.v, t, gi);
    };
    // Rates of the chunk at t0 copied into seta[parity]: one 4-byte copy a lane, tokens
    // past the end read as zero (past the last chunk: a copy of the last token into a
    // buffer nobody reads).  Every state wave issues the same copy, without a branch, so
    // that all of them count the same number of memory operations; it goes out together
    // with the copy of v, and the wait for v covers it.
    auto stage_eta = [&](int t0, int parity) TTT_INLINE {
        if (ETAV) {
            t0 = copy_start(t0);
            const int n = min(SC, t_end - t0);
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc((void*)(p.eta + seq_row + t0), (short)0, n * 4, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TTT_LDS void*)(seta + SC * parity), 4, 4 * lane, 0, 0, 0);
        }
    };
    auto eta_of = [&](int parity) TTT_INLINE { return ETAV ? seta[SC * parity + lane] : p.eta_scalar; };
    // Per-token weights of a chunk of n tokens entered with momentum scale r0: w_T =
    // eta_j / (1 - beta) (carried by the phi(k) rows) and the factor that turns it
    // into the M weight eta_j beta^{n-1-j} / rho', i.e. (1 - beta) beta^{n-1-j} / rho'
    // (applied to v in the M update).
    auto put_weights = [&](float* wts, float et, int n, float r0) TTT_INLINE {
        if (w == 3) {
            float wm = 0.0f;
            if constexpr (MOM) wm = (1.0f - beta) * sBP[max(n - 1 - lane, 0)] * __builtin_amdgcn_rcpf(rho_step(r0, n));
            if (ETAV && p.eta_kind == ETA_SOFTPLUS) et = softplus_f32(et);
            if (lane >= n) et = 0.0f;
            s_wt(wts)[lane] = et * inv1mb;
            if constexpr (MOM) s_wm(wts)[lane] = lane < n ? wm : 0.0f;
        }
    };
    auto weights8 = [&](const float* wp, int b, float* out) TTT_INLINE {
        const f32x4 a = *reinterpret_cast<const f32x4*>(wp + 16 * b + 4 * hh);
        const f32x4 c = *reinterpret_cast<const f32x4*>(wp + 16 * b + 8 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[e] = a[e];
            out[4 + e] = c[e];
        }
    };
    // v fragments: lane holds v[16b + slot(h, e)][32 w + pi(n)]
    u32x4 vf[SKB];
    auto read_v = [&]() TTT_INLINE {
#pragma unroll
        for (int b = 0; b < SKB; ++b) {
            const u32x2 lo = tr_rd(vt, 16 * b + 4 * hh, col_v, l16);
            const u32x2 hi = tr_rd(vt, 16 * b + 8 + 4 * hh, col_v, l16);
            vf[b] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    // update with phi(k) (rows already weighted by w_T) and the v fragments:
    // T += K^T v, M = beta^n M + K^T (m v), four 16-token blocks
    auto update = [&](const uint16_t* K, float* wts, int n) TTT_INLINE {
        if constexpr (MOM) {
            const float r = rho * sBP[n];
            if (r < RHO_MIN) {
#pragma unroll
                for (int ft = 0; ft < SFT; ++ft) Ms[ft] *= r;
                rho = 1.0f;
            } else {
                rho = r;
            }
        }
        // one 16-token block at a time: the feature wave on the same SIMD covers the
        // latency of the transpose reads
#pragma unroll
        for (int b = 0; b < SKB; ++b) {
            u32x4 kf[SFT];
#pragma unroll
            for (int ft = 0; ft < SFT; ++ft) {
                const u32x2 lo = tr_rd(K, 16 * b + 4 * hh, col_k(ft), l16);
                const u32x2 hi = tr_rd(K, 16 * b + 8 + 4 * hh, col_k(ft), l16);
                kf[ft] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
            bf16x8 bm;
            if constexpr (MOM) {
                float x[8];
                weights8(s_wm(wts), b, x);
                bm = scale8(vf[b], x);
            }
#pragma unroll
            for (int ft = 0; ft < SFT; ++ft) {
                const bf16x8 a = as_bf16x8(kf[ft]);
                Ts[ft] = smfma(a, as_bf16x8(vf[b]), Ts[ft]);
                if constexpr (MOM) Ms[ft] = smfma(a, bm, Ms[ft]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // This slice's part of output rows, in bf16 and in register order: lane (n, h) holds
    // o[32I + n][32 wv + 16h + r], r = 0..15, stored as two 16-byte pieces (r = 0..7, 8..15)
    // at [slice][sequence][chunk][wv][I][piece][lane].  Each store instruction then writes
    // 1 KiB of consecutive bytes (row-order stores of 16 bytes a lane scatter over 32 rows
    // and cost several times as long to issue); slice_sum reads this order back.  Past
    // the end of the sequence the pieces go to the padding of the last chunk.
    auto store = [&](const f32x16& o, int I, int c) TTT_INLINE {
        uint16_t* base = reinterpret_cast<uint16_t*>(p.partial) +
                         (((size_t)fs * p.n_seq + seq) * p.n_chunks + c) * (size_t)(SC * SD) + (size_t)(wv * 2 + I) * 1024;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 pk = {pack_bf16x2(o[8 * h + 0], o[8 * h + 1]), pack_bf16x2(o[8 * h + 2], o[8 * h + 3]),
                              pack_bf16x2(o[8 * h + 4], o[8 * h + 5]), pack_bf16x2(o[8 * h + 6], o[8 * h + 7])};
            *reinterpret_cast<u32x4*>(base + (size_t)h * 512 + 8 * lane) = pk;
        }
    };

    float gam[2];
#pragma unroll
    for (int I = 0; I < 2; ++I) gam[I] = MOM ? -beta * beta * sBP[32 * I + n32] * inv1mb : 0.0f;

    stage_v(0);
    stage_eta(0, 0);
    stage_eta(SC, 1);
    wait_vm0();
    put_weights(w_a, eta_of(0), min(SC, t_end), rho);
    lds_barrier();   // B0
    lds_barrier();   // B1: the feature waves formed phi of chunk 0

    // chunk c with its features in (PQ, PK) and its weights in wc; the weights of
    // chunk c+1 go to wn
    auto step = [&](int c, const uint16_t* PQ, const uint16_t* PK, float* wc, float* wn) TTT_INLINE -> bool {
        const int t0 = c * SC;
        const int n = min(SC, t_end - t0);
        const size_t row0 = seq_row + t0;
        const bool has_next = c + 1 < n_chunks;

        // readout T phi(q_i) + g_i rho Ms phi(q_i), g_i = -beta^{i+2}/(1-beta) (lane n holds
        // token 32I + n): the momentum part first, scaled per token in its accumulator,
        // then the T part accumulated onto it
        f32x16 o[2] = {f32x16{}, f32x16{}};
        if constexpr (MOM) {
#pragma unroll
            for (int ft = 0; ft < SFT; ++ft)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const int kb = 2 * ft + kh;
                    const bf16x8 aM = half_operand(Ms[ft], kh);
                    o[0] = smfma(aM, as_bf16x8(lds_read16(PQ + offr[kb])), o[0]);
                    o[1] = smfma(aM, as_bf16x8(lds_read16(PQ + offr[kb] + 4096)), o[1]);
                    if (kh) __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                const float gI = gam[I] * rho;
#pragma unroll
                for (int r = 0; r < 16; ++r) o[I][r] *= gI;
            }
        }
#pragma unroll
        for (int ft = 0; ft < SFT; ++ft)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const int kb = 2 * ft + kh;
                const bf16x8 aT = half_operand(Ts[ft], kh);
                o[0] = smfma(aT, as_bf16x8(lds_read16(PQ + offr[kb])), o[0]);
                o[1] = smfma(aT, as_bf16x8(lds_read16(PQ + offr[kb] + 4096)), o[1]);
                if (kh) __builtin_amdgcn_sched_barrier(0);
            }
        read_v();
        if (has_next) put_weights(wn, eta_of((c + 1) & 1), min(SC, t_end - (t0 + SC)), rho_step(rho, n));
        lds_barrier();   // P: score fragments (feature waves), weights of chunk c+1; every state
                         // wave has its v fragments
        if (has_next) {
            stage_v(t0 + SC);
            stage_eta(t0 + 2 * SC, c & 1);   // chunk c+2 takes the parity of chunk c
        }
        u32x4 pf[6];
#pragma unroll
        for (int f = 0; f < 6; ++f) pf[f] = P_lds[f * 64 + lane];
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            // blocks 0, 1 from tile (0, I); blocks 2, 3 from tile (1, 1)
#pragma unroll
            for (int b = 0; b < 2 * (I + 1); ++b) {
                const int tile = (b < 2) ? I : 2;
                o[I] = smfma(as_bf16x8(vf[b]), as_bf16x8(pf[tile * 2 + (b & 1)]), o[I]);
            }
            store(o[I], I, c);
        }
        update(PK, wc, n);
        if (!has_next) return false;
        // v of chunk c+1 (and the rates of chunk c+2) landed: those copies were issued
        // before the 4 stores of this chunk's partial output, which may still be in
        // flight (the counter retires in issue order)
        __builtin_amdgcn_s_waitcnt(0x0F70 | 4);   // vmcnt(4)
        lds_barrier();   // S: v of chunk c+1, features of chunk c+1
        return true;
    };
    for (int c = 0;; c += 2) {
        if (!step(c, phq0, phk0, w_a, w_b)) break;
        if (!step(c + 1, phq1, phk1, w_b, w_a)) break;
    }
    wait_vm0();
}

// o = bf16(sum over slices of the slices' parts), fixed order.  One thread per 16-byte
// piece of the register-order layout of swiglu_kernel's store: it reads the piece of
// every slice (consecutive threads read consecutive bytes) and writes the 8 columns
// 32w + 16h + 8 piece .. +7 of row 32I + n of its chunk.
__global__ void __launch_bounds__(256) slice_sum(const uint16_t* partial, uint16_t* o, int n_seq, int n_chunks, int T,
                                                 int n_split) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;   // piece
    const size_t per_slice = (size_t)n_seq * n_chunks * (SC * SD / 8);
    if (idx >= per_slice) return;
    const int lane = (int)(idx & 63), piece = (int)((idx >> 6) & 1), wI = (int)((idx >> 7) & 7);
    const size_t chunk_all = idx >> 10;                       // sequence * n_chunks + chunk
    const int c = (int)(chunk_all % n_chunks);
    const size_t seq = chunk_all / n_chunks;
    const int I = wI & 1, w = wI >> 1, n = lane & 31, h = lane >> 5;
    const int t = c * SC + 32 * I + n;
    if (t >= T) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_split; ++s) {
        const u32x4 x = reinterpret_cast<const u32x4*>(partial)[(size_t)s * per_slice + idx];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(x[e] << 16);
            acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
        }
    }
    const u32x4 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                      pack_bf16x2(acc[6], acc[7])};
    *reinterpret_cast<u32x4*>(o + (seq * T + t) * SD + 32 * w + 16 * h + 8 * piece) = pk;
}

template <bool MOM, bool ETAV>
hipError_t launch_swiglu_one(const SwigluParams& sp, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
    const int grid = (sp.n_units + 7) / 8 * 8;
    if (eb || ee) {
        SwigluParams a = sp;
        void* args[] = {&a};
        return hipExtLaunchKernel(reinterpret_cast<const void*>(swiglu_kernel<MOM, ETAV>), dim3(grid), dim3(SNT2),
                                  args, 0, st, eb, ee, 0);
    }
    hipLaunchKernelGGL((swiglu_kernel<MOM, ETAV>), dim3(grid), dim3(SNT2), 0, st, sp);
    return hipGetLastError();
}

}  // namespace

bool swiglu_supported(const Shape& s) {
    return s.bf16 && s.swiglu && s.d_k == SD && s.d_v == SD && s.d_phi % SD == 0 && s.d_phi <= 4 * SD;
}

size_t swiglu_partial_bytes(const Shape& s) {
    // bf16 parts of whole chunks (the last one padded)
    const size_t n_chunks = (size_t)(s.T + SC - 1) / SC;
    return (size_t)(s.d_phi / SD) * s.n_seq() * n_chunks * SC * SD * 2;
}

hipError_t launch_swiglu(const Shape& s, void* workspace, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end,
                         int* n_kernels) {
    if (a.bidirectional || a.reverse || a.S0 || a.M0 || a.S_T || a.M_T) return hipErrorInvalidValue;
    SwigluParams sp{};
    sp.q = static_cast<const uint16_t*>(a.q);
    sp.k = static_cast<const uint16_t*>(a.k);
    sp.v = static_cast<const uint16_t*>(a.v);
    sp.eta = a.eta;
    sp.w1 = static_cast<const uint16_t*>(s.w1);
    sp.w3 = static_cast<const uint16_t*>(s.w3);
    sp.partial = static_cast<float*>(workspace);
    sp.eta_scalar = a.eta_scalar;
    sp.beta = a.beta;
    sp.eta_kind = a.eta_kind;
    sp.T = s.T;
    sp.H = s.H;
    sp.d_phi = s.d_phi;
    sp.slices = s.d_phi / SD;
    sp.n_units = s.n_seq() * sp.slices;
    sp.n_seq = s.n_seq();
    sp.n_chunks = (s.T + SC - 1) / SC;
    sp.n_rows = (size_t)s.n_seq() * s.T;
    const bool mom = a.beta != 0.0f;
    const bool etav = a.eta_kind != ETA_SCALAR;
    hipStream_t st = a.stream;
    hipError_t e = mom ? (etav ? launch_swiglu_one<true, true>(sp, st, ev_begin, ev_end)
                               : launch_swiglu_one<true, false>(sp, st, ev_begin, ev_end))
                       : (etav ? launch_swiglu_one<false, true>(sp, st, ev_begin, ev_end)
                               : launch_swiglu_one<false, false>(sp, st, ev_begin, ev_end));
    if (e != hipSuccess) return e;
    const size_t pieces = (size_t)sp.n_seq * sp.n_chunks * (SC * SD / 8);
    hipLaunchKernelGGL(slice_sum, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(sp.partial), static_cast<uint16_t*>(a.o), sp.n_seq,
                       sp.n_chunks, s.T, sp.slices);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (n_kernels) *n_kernels = 2;
    return hipSuccess;
}

}  // namespace ttt
