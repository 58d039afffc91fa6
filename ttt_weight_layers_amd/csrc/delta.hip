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
// the C-step solve for U runs in fp32, four lanes per value column.
//
// A workgroup (four waves) walks one sequence in chunks of 32 tokens for 64 of its
// value columns (the rows of S evolve independently: row i only meets column i of
// v), keeps those 64 rows of S in fp32 registers as 16x16 MFMA result tiles (wave
// w: rows 16w .. 16w+15) and a bf16 copy of S^T in LDS as the operand of K S0^T and
// Q S0^T (written four entries at a time, read back by transpose reads).  The next chunk's rows load into registers while the current one is used;
// the LDS tiles of q, k, v are double-buffered.  Waves exchange data through LDS only,
// so the barriers inside the chunk loop wait for LDS traffic alone (lds_barrier), not
// for the prefetch loads or the output stores in flight.
//
// Register layouts of v_mfma_f32_16x16x32_bf16 (lane l, c16 = l % 16, g = l / 16):
//   A operand  A[m = c16][k = 8g .. 8g+7]      B operand  B[k = 8g .. 8g+7][n = c16]
//   D result   D[m = 4g .. 4g+3][n = c16]
// Operands whose contraction runs along the features are 16-byte row reads of the
// swizzled tiles; those whose contraction runs over tokens (U^T, K, U) or over the
// rows of the S^T copy are transpose reads.

#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_tiles.h"

#define TTT_INLINE __attribute__((always_inline))

namespace ttt {
namespace {

constexpr int DC = 32;         // tokens per chunk
constexpr int DTH = 256;       // threads: four waves
constexpr int DVW = 64;        // value columns per workgroup
constexpr int NSTR = DC + 4;   // row stride (floats) of N
constexpr int PSTR = 40;       // row stride (bf16) of the masked scores: 16 rows read at one
                               // column fall on distinct banks

// x of lane OWNER of each group of four lanes, in all four (one DPP move)
template <int OWNER>
__device__ __forceinline__ float quad_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), OWNER | (OWNER << 2) | (OWNER << 4) |
                                                                               (OWNER << 6),
                                                      0xF, 0xF, false));
}

struct DeltaParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* eta;
    uint16_t* o;
    float eta_scalar;
    int eta_kind;
    int T;
    int n_vsplit;              // workgroups per sequence (value columns DVW each)
    int n_units;               // sequences x n_vsplit (the grid is rounded up to a multiple of 8)
};

// DK = d_k = d_v.  Rows of the state evolve independently under the delta rule (row i
// of S only meets v's column i), so a workgroup owns DVW value columns of one sequence.
template <int DK>
__global__ void __launch_bounds__(DTH, 1) delta_forward(DeltaParams p) {
    constexpr int NT = DK / 16;                  // 16-wide feature tiles
    constexpr int QL = DC * DK / 8 / DTH;        // 16-byte loads per thread of a q or k chunk
    __shared__ __attribute__((aligned(16))) uint16_t sQ[2][DC * DK];
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][DC * DK];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][DC * DVW];
    __shared__ __attribute__((aligned(16))) uint16_t sU[DC * DVW];
    __shared__ __attribute__((aligned(16))) uint16_t sST[DK * DVW];  // S^T in bf16: row = feature
    __shared__ __attribute__((aligned(16))) float sR[DC * DVW];
    __shared__ __attribute__((aligned(16))) float sN[DC * NSTR];   // N^T: row j holds N[4m + i][j] at 8i + m
    __shared__ __attribute__((aligned(16))) uint16_t sP[DC * PSTR];
    __shared__ float sE[2][DC];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4, q4 = lane & 3;
    const int T = p.T;
    // unit u: the value splits of a sequence are consecutive units, and consecutive units
    // sit on one XCD (workgroups go to the XCDs in turn), so they share q and k in its L2
    const int G = gridDim.x;
    const int u = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_units) return;
    const int seq = u / p.n_vsplit;
    const int vc0 = (u % p.n_vsplit) * DVW;   // first value column of the workgroup
    const size_t row0 = (size_t)seq * T;
    const int vr0 = 16 * wv;                         // this wave's value rows of S (local)
    const int dv = DK;                               // row length of v and o

    f32x4 St[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) St[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int e = tid; e < DVW * DK / 8; e += DTH) *reinterpret_cast<u32x4*>(sST + 8 * e) = u32x4{0u, 0u, 0u, 0u};

    // next chunk's rows in registers (zero past T)
    u32x4 rq[QL], rk[QL], rv;
    float re = 0.0f;
    bool re_valid = false;
    auto fetch = [&](int c) {
        const int t0 = c * DC, n = min(DC, T - t0);
#pragma unroll
        for (int l = 0; l < QL; ++l) {
            const int e = tid + l * DTH, r = e / (DK / 8), col = 8 * (e % (DK / 8));
            rq[l] = rk[l] = u32x4{0u, 0u, 0u, 0u};
            if (r < n) {
                rq[l] = *reinterpret_cast<const u32x4*>(p.q + (row0 + t0 + r) * DK + col);
                rk[l] = *reinterpret_cast<const u32x4*>(p.k + (row0 + t0 + r) * DK + col);
            }
        }
        {
            const int r = tid / (DVW / 8), col = 8 * (tid % (DVW / 8));
            rv = r < n ? *reinterpret_cast<const u32x4*>(p.v + (row0 + t0 + r) * dv + vc0 + col)
                       : u32x4{0u, 0u, 0u, 0u};
        }
        // the raw rate only: its softplus waits until commit, when the load has landed
        re_valid = tid < n;
        if (tid < DC) re = re_valid ? (p.eta_kind == ETA_SCALAR ? p.eta_scalar : p.eta[row0 + t0 + tid]) : 0.0f;
    };
    auto commit = [&](int b) {
#pragma unroll
        for (int l = 0; l < QL; ++l) {
            const int e = tid + l * DTH, r = e / (DK / 8), col = 8 * (e % (DK / 8));
            *reinterpret_cast<u32x4*>(sQ[b] + swz<DK>(r, col)) = rq[l];
            *reinterpret_cast<u32x4*>(sK[b] + swz<DK>(r, col)) = rk[l];
        }
        {
            const int r = tid / (DVW / 8), col = 8 * (tid % (DVW / 8));
            *reinterpret_cast<u32x4*>(sV[b] + swz<DVW>(r, col)) = rv;
        }
        if (tid < DC) sE[b][tid] = !re_valid ? 0.0f : (p.eta_kind == ETA_SOFTPLUS ? softplus_f32(re) : re);
    };

    const int n_chunks = (T + DC - 1) / DC;
    fetch(0);
    commit(0);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
        const int b = c & 1;
        const int t0 = c * DC;
        const int n = min(DC, T - t0);
        const uint16_t* Q = sQ[b];
        const uint16_t* K = sK[b];
        const uint16_t* V = sV[b];
        const float* E = sE[b];
        if (c + 1 < n_chunks) fetch(c + 1);

        // ---- R = V - K S0^T and O = Q S0^T: tiles (token tile ta, value tile wv) ----
        f32x4 Oacc[2];
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = ks;
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                const bf16x8 bS = as_bf16x8(tr_read8<DVW>(sST, 32 * kk + 8 * g, 16 * wv + 4 * q4));
                ks = mfma16(as_bf16x8(lds_read16(K + swz<DK>(16 * ta + c16, 32 * kk + 8 * g))), bS, ks);
                qs = mfma16(as_bf16x8(lds_read16(Q + swz<DK>(16 * ta + c16, 32 * kk + 8 * g))), bS, qs);
            }
            Oacc[ta] = qs;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ta + 4 * g + r, col = 16 * wv + c16;
                sR[t * DVW + col] = bf16_bits_to_f32(V[swz<DVW>(t, col)]) - ks[r];
            }
        }
        // ---- N = diag(eta) strictly-lower(K K^T) and P = tril(Q K^T) on the 2x2 tiles of
        //      16 tokens: waves 0..2 take (0,0), (1,0), (1,1), wave 3 zeroes (0,1) ----
        {
            const int ti = wv == 0 ? 0 : 1, tj = wv == 2 ? 1 : 0;
            f32x4 gk = {0.f, 0.f, 0.f, 0.f}, gq = gk;
            if (wv < 3) {
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk) {
                    const bf16x8 bK = as_bf16x8(lds_read16(K + swz<DK>(16 * tj + c16, 32 * kk + 8 * g)));
                    gk = mfma16(as_bf16x8(lds_read16(K + swz<DK>(16 * ti + c16, 32 * kk + 8 * g))), bK, gk);
                    gq = mfma16(as_bf16x8(lds_read16(Q + swz<DK>(16 * ti + c16, 32 * kk + 8 * g))), bK, gq);
                }
            }
            const int i0 = wv < 3 ? 16 * ti : 0, j0 = wv < 3 ? 16 * tj : 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = i0 + 4 * g + r, j = j0 + c16;
                const float nv = (wv < 3 && j < t) ? E[t] * gk[r] : 0.0f;
                sN[j * NSTR + 8 * (t & 3) + (t >> 2)] = nv;
                sP[t * PSTR + j] = f32_to_bf16_bits((wv < 3 && j <= t) ? gq[r] : 0.0f);
            }
        }
        lds_barrier();

        // ---- (I + N) U = diag(eta) R by forward substitution, column by column of N: lane i
        //      of a quad keeps the running sums of the tokens t = 4m + i of its value
        //      column; token j is final once columns 0 .. j-1 are applied, its owner's
        //      value is broadcast to the quad (DPP) and column j applied to the rest.
        //      N[t][j] = 0 for t <= j, so finished sums stay untouched. ----
        {
            const int col = tid >> 2, i = tid & 3;
            float acc[DC / 4];
#pragma unroll
            for (int m = 0; m < DC / 4; ++m) acc[m] = E[4 * m + i] * sR[(4 * m + i) * DVW + col];
            // N^T rows of four steps in registers, the next four loading meanwhile
            f32x4 nb[2][8];
            auto load_n = [&](int j4, f32x4* dst) TTT_INLINE {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    dst[2 * s4] = *reinterpret_cast<const f32x4*>(sN + (j4 + s4) * NSTR + 8 * i);
                    dst[2 * s4 + 1] = *reinterpret_cast<const f32x4*>(sN + (j4 + s4) * NSTR + 8 * i + 4);
                }
            };
            auto apply = [&](const f32x4& n0, const f32x4& n1, float uj) TTT_INLINE {
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = fmaf(-n0[m], uj, acc[m]);
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[4 + m] = fmaf(-n1[m], uj, acc[4 + m]);
            };
            load_n(0, nb[0]);
#pragma unroll
            for (int j4 = 0; j4 < DC; j4 += 4) {
                const f32x4* cur = nb[(j4 >> 2) & 1];
                if (j4 + 4 < DC) load_n(j4 + 4, nb[((j4 >> 2) + 1) & 1]);
                apply(cur[0], cur[1], quad_bcast<0>(acc[j4 >> 2]));
                apply(cur[2], cur[3], quad_bcast<1>(acc[j4 >> 2]));
                apply(cur[4], cur[5], quad_bcast<2>(acc[j4 >> 2]));
                if (j4 + 3 < DC - 1) apply(cur[6], cur[7], quad_bcast<3>(acc[j4 >> 2]));
            }
#pragma unroll
            for (int m = 0; m < DC / 4; ++m) sU[swz<DVW>(4 * m + i, col)] = f32_to_bf16_bits(acc[m]);
        }
        lds_barrier();

        // ---- S += U^T K, and its bf16 copy for the next chunk ----
        {
            const bf16x8 aU = as_bf16x8(tr_read8<DVW>(sU, 8 * g, vr0 + 4 * q4));
#pragma unroll
            for (int bt = 0; bt < NT; ++bt) {
                St[bt] = mfma16(aU, as_bf16x8(tr_read8<DK>(K, 8 * g, 16 * bt + 4 * q4)), St[bt]);
                // lane holds S[vr0 + 4g + r][16 bt + c16], r = 0..3: four consecutive entries of
                // one row of S^T
                *reinterpret_cast<u32x2*>(sST + swz<DVW>(16 * bt + c16, vr0 + 4 * g)) =
                    u32x2{pack_bf16x2(St[bt][0], St[bt][1]), pack_bf16x2(St[bt][2], St[bt][3])};
            }
        }
        // the next chunk's rows go to LDS before this chunk's outputs are stored: the wait
        // for the loads (vector-memory counter) then does not include the stores
        if (c + 1 < n_chunks) commit(b ^ 1);
        // ---- O += tril(Q K^T) U, written out ----
        {
            const bf16x8 bU = as_bf16x8(tr_read8<DVW>(sU, 8 * g, 16 * wv + 4 * q4));
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const bf16x8 aP = as_bf16x8(*reinterpret_cast<const u32x4*>(sP + (16 * ta + c16) * PSTR + 8 * g));
                const f32x4 o = mfma16(aP, bU, Oacc[ta]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ta + 4 * g + r;
                    if (t < n) p.o[(row0 + t0 + t) * dv + vc0 + 16 * wv + c16] = f32_to_bf16_bits(o[r]);
                }
            }
        }
        lds_barrier();
    }
}


// ---- two-pass form -------------------------------------------------------------
// (I + N) depends on the keys and rates of a chunk only, not on the state, so its
// inverse can leave the sequential walk: a first pass over all chunks at once
// writes A = (I + N)^{-1} diag(eta) for every chunk, and the walk then takes
// U = A R as a product on the matrix cores (fp32 operands, v_mfma_f32_16x16x4_f32)
// instead of a 32-step substitution: the chunk form above with the triangular
// inverse made explicit and formed for every chunk before the walk starts.
//
// A of one chunk is lower triangular; its three non-zero 16 x 16 blocks (token
// tiles (0,0), (1,0), (1,1)) are stored in operand order: the f32x4 at index
// 16 g + c16 of block (to, ts) holds A[16 to + c16][16 ts + 4 g .. 16 ts + 4 g + 3],
// exactly what lane (c16, g) feeds the fp32 product over four k steps.
constexpr int ABLK = 256;          // floats of one 16 x 16 block
constexpr int ACH = 3 * ABLK;      // floats of one chunk's blocks
constexpr int NSTR2 = DC + 4;      // row stride (floats) of N and A in the first pass

struct DeltaPrepParams {
    const uint16_t* k;
    const float* eta;
    float* a;                  // [sequence][chunk][ACH]
    float eta_scalar;
    int eta_kind;
    int T;
    int n_chunks;              // chunks per sequence
    int n_units;               // sequences x n_chunks
};

// One wave per two chunks.  For each chunk the 2 x 2 tiles of K K^T come from
// 16-byte row loads of the keys (no staging: each key row is an operand row as it
// stands in memory) and N goes to the chunk's LDS rows; then each half of the wave
// takes one chunk and finds the columns of its A by forward substitution, lane j
// owning column j (A[t][j] = eta_j [t == j] - sum_{i<t} N[t][i] A[i][j]; the lanes of
// a half read the same row of N, an LDS broadcast); A goes back out through the same
// LDS rows in operand order.
template <int DK>
__global__ void __launch_bounds__(256) delta_prep(DeltaPrepParams p) {
    constexpr int KK = DK / 32;
    __shared__ __attribute__((aligned(16))) float sN[4][2][DC * NSTR2];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int unit0 = 2 * (blockIdx.x * 4 + wv);
    if (unit0 >= p.n_units) return;   // waves share no data: no barrier below
    const int half = lane >> 5, j = lane & (DC - 1);

    // N of chunk unit0 + h into sN[wv][h]
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // a missing second chunk reads no keys and writes nothing: its N is zero
        const int unit = unit0 + h;
        const bool live = unit < p.n_units;
        const int seq = unit / p.n_chunks, c = unit % p.n_chunks;
        const int t0 = c * DC, n = live ? min(DC, p.T - t0) : 0;
        const size_t row0 = (size_t)seq * p.T + t0;
        float* N = sN[wv][h];
        u32x4 kr[2][KK];
#pragma unroll
        for (int ta = 0; ta < 2; ++ta)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int r = 16 * ta + c16;
                kr[ta][kk] = r < n ? *reinterpret_cast<const u32x4*>(p.k + (row0 + r) * DK + 32 * kk + 8 * g)
                                   : u32x4{0u, 0u, 0u, 0u};
            }
        // G tiles (ti, tj): lane holds G[16 ti + 4 g + r][16 tj + c16]
        f32x4 g00 = {0.f, 0.f, 0.f, 0.f}, g10 = g00, g11 = g00;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 k0 = as_bf16x8(kr[0][kk]), k1 = as_bf16x8(kr[1][kk]);
            g00 = mfma16(k0, k0, g00);
            g10 = mfma16(k1, k0, g10);
            g11 = mfma16(k1, k1, g11);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            const float e0 = t < n ? eta_at(p.eta_kind, p.eta, p.eta_scalar, row0 + t) : 0.0f;
            const float e1 = 16 + t < n ? eta_at(p.eta_kind, p.eta, p.eta_scalar, row0 + 16 + t) : 0.0f;
            N[t * NSTR2 + c16] = c16 < t ? e0 * g00[r] : 0.0f;
            N[(16 + t) * NSTR2 + c16] = e1 * g10[r];
            N[(16 + t) * NSTR2 + 16 + c16] = c16 < t ? e1 * g11[r] : 0.0f;
        }
    }
    // column j of the A of chunk unit0 + half
    const int unit = unit0 + half;
    const int seq = unit / p.n_chunks, c = unit % p.n_chunks;
    const int t0 = c * DC, n = unit < p.n_units ? min(DC, p.T - t0) : 0;
    const float ej = j < n ? eta_at(p.eta_kind, p.eta, p.eta_scalar, (size_t)seq * p.T + t0 + j) : 0.0f;
    float* N = sN[wv][half];
    float x[DC];
#pragma unroll
    for (int t = 0; t < DC; ++t) {
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
        for (int i4 = 0; i4 < t / 4; ++i4) {
            const f32x4 nr = *reinterpret_cast<const f32x4*>(N + t * NSTR2 + 4 * i4);
            s0 = fmaf(nr[0], x[4 * i4], s0);
            s1 = fmaf(nr[1], x[4 * i4 + 1], s1);
            s2 = fmaf(nr[2], x[4 * i4 + 2], s2);
            s3 = fmaf(nr[3], x[4 * i4 + 3], s3);
        }
#pragma unroll
        for (int i = 4 * (t / 4); i < t; ++i) s0 = fmaf(N[t * NSTR2 + i], x[i], s0);
        x[t] = (t == j ? ej : 0.0f) - ((s0 + s1) + (s2 + s3));
    }
    // A over N (the wave's reads of N are all issued before these writes)
#pragma unroll
    for (int t = 0; t < DC; ++t) N[t * NSTR2 + j] = x[t];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (unit0 + h >= p.n_units) break;
        const float* A = sN[wv][h];
        float* dst = p.a + (size_t)(unit0 + h) * ACH + 4 * lane;
        *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(A + c16 * NSTR2 + 4 * g);
        *reinterpret_cast<f32x4*>(dst + ABLK) = *reinterpret_cast<const f32x4*>(A + (16 + c16) * NSTR2 + 4 * g);
        *reinterpret_cast<f32x4*>(dst + 2 * ABLK) =
            *reinterpret_cast<const f32x4*>(A + (16 + c16) * NSTR2 + 16 + 4 * g);
    }
}

struct DeltaWalkParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* a;            // the first pass's blocks
    uint16_t* o;
    const float* S0;           // entry state, fp32 [seq][d_v][d_k] (null: zero)
    float* S_T;                // state after the last token (null: not written)
    int T;
    int n_chunks;
    int n_vsplit;
    int n_units;               // sequences x n_vsplit (grid rounded up to a multiple of 8)
};

// The walk.  Workgroup and state as in delta_forward (64 value columns of one
// sequence, wave w keeps rows 16w .. 16w+15 of S and writes its own columns of the
// bf16 S^T copy), but now every wave's chain touches only its own columns: per chunk
//   R = V - K S0^T, O0^T = S0 Q^T         (the S^T fragment serves both products)
//   U = A R                               (fp32 products: lane (c16, g) holds R of
//                                          tokens 4g + r and 16 + 4g + r, which are
//                                          exactly the k index of step r)
//   S += U^T K,  O^T = O0^T + U^T P^T     (the U tiles, packed to bf16, are the A
//                                          operand with the contraction over tokens
//                                          4g .. 4g+3, 16+4g .. 16+4g+3; the matching
//                                          rows of K come from two transpose reads and
//                                          those of P^T = K Q^T straight from its tiles)
// so the waves meet only at the one barrier that hands over the staged q, k, v.
template <int DK>
__global__ void __launch_bounds__(DTH, 1) delta_walk(DeltaWalkParams p) {
    constexpr int NT = DK / 16;
    constexpr int KK = DK / 32;
    constexpr int QL = DC * DK / 8 / DTH;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[2][DC * DK];
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][DC * DK];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][DC * DVW];
    __shared__ __attribute__((aligned(16))) uint16_t sST[DK * DVW];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4, q4 = lane & 3;
    const int T = p.T;
    const int G = gridDim.x;
    const int u = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_units) return;
    const int seq = u / p.n_vsplit;
    const int vc0 = (u % p.n_vsplit) * DVW;
    const size_t row0 = (size_t)seq * T;
    const int vr0 = 16 * wv;
    const float* Ablk = p.a + (size_t)seq * p.n_chunks * ACH + 4 * lane;

    // the lane's entries of S: row vc0 + vr0 + 4g + r, column 16 bt + c16 (the entry
    // state, or zero), and this wave's columns of the bf16 copy of S^T
    const size_t srow = ((size_t)seq * DK + vc0 + vr0 + 4 * g) * DK + c16;
    f32x4 St[NT];
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) St[bt][r] = p.S0 ? p.S0[srow + (size_t)r * DK + 16 * bt] : 0.0f;
        *reinterpret_cast<u32x2*>(sST + swz<DVW>(16 * bt + c16, vr0 + 4 * g)) =
            u32x2{pack_bf16x2(St[bt][0], St[bt][1]), pack_bf16x2(St[bt][2], St[bt][3])};
    }

    u32x4 rq[QL], rk[QL], rv;
    f32x4 an[3];
    auto fetch = [&](int c) TTT_INLINE {
        const int t0 = c * DC, n = min(DC, T - t0);
#pragma unroll
        for (int l = 0; l < QL; ++l) {
            const int e = tid + l * DTH, r = e / (DK / 8), col = 8 * (e % (DK / 8));
            rq[l] = rk[l] = u32x4{0u, 0u, 0u, 0u};
            if (r < n) {
                rq[l] = *reinterpret_cast<const u32x4*>(p.q + (row0 + t0 + r) * DK + col);
                rk[l] = *reinterpret_cast<const u32x4*>(p.k + (row0 + t0 + r) * DK + col);
            }
        }
        {
            const int r = tid / (DVW / 8), col = 8 * (tid % (DVW / 8));
            rv = r < n ? *reinterpret_cast<const u32x4*>(p.v + (row0 + t0 + r) * DK + vc0 + col)
                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int b = 0; b < 3; ++b) an[b] = *reinterpret_cast<const f32x4*>(Ablk + (size_t)c * ACH + b * ABLK);
    };
    auto commit = [&](int b) TTT_INLINE {
#pragma unroll
        for (int l = 0; l < QL; ++l) {
            const int e = tid + l * DTH, r = e / (DK / 8), col = 8 * (e % (DK / 8));
            *reinterpret_cast<u32x4*>(sQ[b] + swz<DK>(r, col)) = rq[l];
            *reinterpret_cast<u32x4*>(sK[b] + swz<DK>(r, col)) = rk[l];
        }
        const int r = tid / (DVW / 8), col = 8 * (tid % (DVW / 8));
        *reinterpret_cast<u32x4*>(sV[b] + swz<DVW>(r, col)) = rv;
    };

    const int n_chunks = p.n_chunks;
    fetch(0);
    commit(0);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
        const int b = c & 1;
        const int t0 = c * DC;
        const int n = min(DC, T - t0);
        const uint16_t* Q = sQ[b];
        const uint16_t* K = sK[b];
        const uint16_t* V = sV[b];
        const f32x4 a00 = an[0], a10 = an[1], a11 = an[2];
        if (c + 1 < n_chunks) fetch(c + 1);

        // ---- K S0^T, S0 Q^T and the score tiles K Q^T (jb, ta) = (0,0), (0,1), (1,1) ----
        f32x4 ks0 = {0.f, 0.f, 0.f, 0.f}, ks1 = ks0, ot0 = ks0, ot1 = ks0, p00 = ks0, p01 = ks0, p11 = ks0;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 bS = as_bf16x8(tr_read8<DVW>(sST, 32 * kk + 8 * g, vr0 + 4 * q4));
            const bf16x8 k0 = as_bf16x8(lds_read16(K + swz<DK>(c16, 32 * kk + 8 * g)));
            const bf16x8 k1 = as_bf16x8(lds_read16(K + swz<DK>(16 + c16, 32 * kk + 8 * g)));
            const bf16x8 q0 = as_bf16x8(lds_read16(Q + swz<DK>(c16, 32 * kk + 8 * g)));
            const bf16x8 q1 = as_bf16x8(lds_read16(Q + swz<DK>(16 + c16, 32 * kk + 8 * g)));
            ks0 = mfma16(k0, bS, ks0);
            ks1 = mfma16(k1, bS, ks1);
            ot0 = mfma16(bS, q0, ot0);
            ot1 = mfma16(bS, q1, ot1);
            p00 = mfma16(k0, q0, p00);
            p01 = mfma16(k0, q1, p01);
            p11 = mfma16(k1, q1, p11);
        }
        // ---- R = V - K S0^T (lane: tokens 4g + r and 16 + 4g + r of column vr0 + c16) ----
        float r0[4], r1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            r0[r] = bf16_bits_to_f32(V[swz<DVW>(4 * g + r, vr0 + c16)]) - ks0[r];
            r1[r] = bf16_bits_to_f32(V[swz<DVW>(16 + 4 * g + r, vr0 + c16)]) - ks1[r];
        }
        // ---- U = A R in fp32 ----
        f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = u0;
#pragma unroll
        for (int r = 0; r < 4; ++r) u0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a00[r], r0[r], u0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) u1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a10[r], r0[r], u1, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) u1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a11[r], r1[r], u1, 0, 0, 0);
        const bf16x8 aU = as_bf16x8(u32x4{pack_bf16x2(u0[0], u0[1]), pack_bf16x2(u0[2], u0[3]),
                                          pack_bf16x2(u1[0], u1[1]), pack_bf16x2(u1[2], u1[3])});
        // ---- S += U^T K, and its bf16 copy (this wave's columns) ----
#pragma unroll
        for (int bt = 0; bt < NT; ++bt) {
            const bf16x8 bK = join8(tr_read<DK>(K, 4 * g, 16 * bt + 4 * q4), tr_read<DK>(K, 16 + 4 * g, 16 * bt + 4 * q4));
            St[bt] = mfma16(aU, bK, St[bt]);
            *reinterpret_cast<u32x2*>(sST + swz<DVW>(16 * bt + c16, vr0 + 4 * g)) =
                u32x2{pack_bf16x2(St[bt][0], St[bt][1]), pack_bf16x2(St[bt][2], St[bt][3])};
        }
        if (c + 1 < n_chunks) commit(b ^ 1);
        // ---- O^T = S0 Q^T + U^T P^T; P = tril(Q K^T), lane (c16, g) of tile (jb, ta) holds
        //      P[16 ta + c16][16 jb + 4 g + r] ----
        {
            const bool keep[4] = {4 * g <= c16, 4 * g + 1 <= c16, 4 * g + 2 <= c16, 4 * g + 3 <= c16};
            float m00[4], m11[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                m00[r] = keep[r] ? p00[r] : 0.0f;
                m11[r] = keep[r] ? p11[r] : 0.0f;
            }
            const bf16x8 bP0 = as_bf16x8(u32x4{pack_bf16x2(m00[0], m00[1]), pack_bf16x2(m00[2], m00[3]), 0u, 0u});
            const bf16x8 bP1 = as_bf16x8(u32x4{pack_bf16x2(p01[0], p01[1]), pack_bf16x2(p01[2], p01[3]),
                                               pack_bf16x2(m11[0], m11[1]), pack_bf16x2(m11[2], m11[3])});
            const f32x4 o0 = mfma16(aU, bP0, ot0);
            const f32x4 o1 = mfma16(aU, bP1, ot1);
            // lane holds O[t = 16 ta + c16][vr0 + 4g .. vr0 + 4g + 3]
            if (c16 < n)
                *reinterpret_cast<u32x2*>(p.o + (row0 + t0 + c16) * DK + vc0 + vr0 + 4 * g) =
                    u32x2{pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3])};
            if (16 + c16 < n)
                *reinterpret_cast<u32x2*>(p.o + (row0 + t0 + 16 + c16) * DK + vc0 + vr0 + 4 * g) =
                    u32x2{pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
        }
        lds_barrier();
    }
    if (p.S_T) {
#pragma unroll
        for (int bt = 0; bt < NT; ++bt)
#pragma unroll
            for (int r = 0; r < 4; ++r) p.S_T[srow + (size_t)r * DK + 16 * bt] = St[bt][r];
    }
}

}  // namespace

bool delta_supported(const Shape& s) {
    return s.bf16 && !s.swiglu && s.d_k == s.d_v && s.d_phi == s.d_k && (s.d_k == 64 || s.d_k == 128);
}

size_t delta_workspace_bytes(const Shape& s) {
    if (!delta_supported(s)) return 0;
    return (size_t)s.n_seq() * (size_t)((s.T + DC - 1) / DC) * ACH * sizeof(float);
}

hipError_t launch_delta(const Shape& s, const FwdArgs& a, void* workspace, size_t workspace_bytes,
                        hipEvent_t ev_begin, hipEvent_t ev_end) {
    // the carried state is S alone (no momentum); only the two-pass form takes it
    if (!delta_supported(s) || a.bidirectional || a.beta != 0.0f || a.M0 || a.M_T || a.reverse)
        return hipErrorInvalidValue;
    const size_t need = delta_workspace_bytes(s);
    const dim3 block(DTH);
    const bool two_pass = workspace && need > 0 && need <= workspace_bytes;
    if (!two_pass && (a.S0 || a.S_T)) return hipErrorInvalidValue;
    if (two_pass) {
        // two passes: the chunk inverses, then the walk (which carries the timing events)
        const int n_chunks = (s.T + DC - 1) / DC;
        DeltaPrepParams pp;
        pp.k = static_cast<const uint16_t*>(a.k);
        pp.eta = a.eta;
        pp.a = static_cast<float*>(workspace);
        pp.eta_scalar = a.eta_scalar;
        pp.eta_kind = a.eta_kind;
        pp.T = s.T;
        pp.n_chunks = n_chunks;
        pp.n_units = s.n_seq() * n_chunks;
        const dim3 pgrid((unsigned)((pp.n_units + 7) / 8));   // two chunks a wave, four waves
        if (s.d_k == 128) hipLaunchKernelGGL(delta_prep<128>, pgrid, block, 0, a.stream, pp);
        else hipLaunchKernelGGL(delta_prep<64>, pgrid, block, 0, a.stream, pp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        DeltaWalkParams wp;
        wp.q = static_cast<const uint16_t*>(a.q);
        wp.k = static_cast<const uint16_t*>(a.k);
        wp.v = static_cast<const uint16_t*>(a.v);
        wp.a = static_cast<const float*>(workspace);
        wp.o = static_cast<uint16_t*>(a.o);
        wp.S0 = a.S0;
        wp.S_T = a.S_T;
        wp.T = s.T;
        wp.n_chunks = n_chunks;
        wp.n_vsplit = s.d_v / DVW;
        wp.n_units = s.n_seq() * wp.n_vsplit;
        const dim3 grid((unsigned)((wp.n_units + 7) / 8 * 8));
        if (ev_begin || ev_end) {
            const void* fn = s.d_k == 128 ? reinterpret_cast<const void*>(delta_walk<128>)
                                          : reinterpret_cast<const void*>(delta_walk<64>);
            void* args[] = {&wp};
            return hipExtLaunchKernel(fn, grid, block, args, 0, a.stream, ev_begin, ev_end, 0);
        }
        if (s.d_k == 128) hipLaunchKernelGGL(delta_walk<128>, grid, block, 0, a.stream, wp);
        else hipLaunchKernelGGL(delta_walk<64>, grid, block, 0, a.stream, wp);
        return hipGetLastError();
    }
    // one pass, no workspace: the substitution runs inside the walk
    DeltaParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.eta = a.eta;
    p.o = static_cast<uint16_t*>(a.o);
    p.eta_scalar = a.eta_scalar;
    p.eta_kind = a.eta_kind;
    p.T = s.T;
    p.n_vsplit = s.d_v / DVW;
    p.n_units = s.n_seq() * p.n_vsplit;
    const dim3 grid((unsigned)((p.n_units + 7) / 8 * 8));
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
