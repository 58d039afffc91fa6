// bf16 MFMA chunk kernels for gfx950: the hot path of the TTT forward.
//
// The layer (one momentum-SGD step per token on the dot-product binding loss,
// fast weight reset per sequence, readout after the update) unrolls, for a
// chunk of n tokens entered with fp32 state (S, M), into
//
//   o_i = S phi(q_i) + g_i M phi(q_i) + sum_{j<=i} c_{i-j} eta_j (phi(q_i).phi(k_j)) v_j
//   S  <- S + g_{n-1} M + sum_j eta_j c_{n-1-j} v_j phi(k_j)^T
//   M  <- beta^n M + sum_j eta_j beta^{n-1-j} v_j phi(k_j)^T
//
// with c_r = sum_{u<=r} beta^u and g_i = beta c_i: dense causal blocks inside
// a chunk and a fixed-size state carried between chunks, the parallel form of
// the outer-product accumulation that the kualia.ai blog ("The Linear Attention
// Equivalence") identifies with linear attention, (phi(Q) phi(K)^T) V.  The
// per-token learning rate, momentum and SwiGLU feature map are the inner-loop
// options of Table 2 on the thelatestinai.com page (Variants 2-4).
//
// Carried state.  Instead of (S, M) the kernels carry (T, M) with
// T = S + kappa M, kappa = beta / (1 - beta).  Substituting into the chunk step
// above gives
//   T <- T + (1 / (1 - beta)) sum_j eta_j v_j phi(k_j)^T           (no decay)
//   M <- beta^n M + sum_j eta_j beta^{n-1-j} v_j phi(k_j)^T
//   o_i = T phi(q_i) - (beta^{i+2} / (1 - beta)) M phi(q_i) + intra-chunk part
// so T is a plain accumulation: it needs no per-chunk transition and, for a
// scalar step size, no per-token weights (T is kept as sum_j v_j phi(k_j)^T
// and scaled by eta / (1 - beta) when read).  S = T - kappa M is formed only
// where the bidirectional readout needs it.  beta = 0 gives T = S, no M.
//
// Kernels (bf16 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation and state):
//   chunk_kernel<OUTPUT>   one workgroup per (sequence, segment, feature slice,
//                          value slice); walks its segment chunk by chunk, keeps
//                          its slice of (S, M) in registers, writes o.
//   chunk_kernel<SUMMARY>  the same walk without readout: the zero-entry state
//                          change of every segment but the last.
//   segment_scan           composes those summaries into entry states.
//   chunk_kernel<BIDIR>    bidirectional: all updates, then every query reads S_T.
//   partial_reduce         sums fp32 partial outputs of feature slices (SwiGLU).
//
// Staging.  Every chunk's q, k (or raw SwiGLU inputs) and v rows are fetched
// with 16-byte global loads into registers one chunk ahead, then written to
// row-major LDS tiles whose 16-byte chunks are XOR-swizzled per row, so that
// both row reads (16 B per lane) and gfx950 transpose reads (ds_read_b64_tr_b16,
// 4 rows x 16 columns per 16-lane group) avoid bank conflicts.  Operands whose
// contraction runs over tokens (K^T, V^T) come from the transpose read; no
// transposed copy is stored.
//
// Register layouts (lane l of a 64-wide wave, c16 = l % 16, g = l / 16):
//   MFMA A operand  lane holds A[m = c16][k = 8g .. 8g+7]
//   MFMA B operand  lane holds B[k = 8g .. 8g+7][n = c16]
//   MFMA D result   lane holds D[m = 4g .. 4g+3][n = c16]
// The state is kept transposed, S^T[f][dv], as D tiles.  Tile ft covers the
// features 32(ft/2) + 8a + 4(ft%2) + b (a, b = 0..3), so lane (g, c16) holds
// S^T[32(ft/2) + 8g + 4(ft%2) + r][dv0 + c16]: the two tiles ft = 2s, 2s+1
// together give each lane 8 consecutive features 32s + 8g .. +7, i.e. without
// any data movement the A operand of O^T = S Q^T whose B operand is one
// 16-byte row read of Q.  The update builds the tiles in that order by pointing
// the transpose reads of K at the matching column groups.

#include <algorithm>
#include <cmath>

#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"
#include "lds_tiles.h"

namespace ttt {
namespace {

enum Kind : int { K_OUTPUT = 0, K_SUMMARY = 1, K_BIDIR = 2 };

constexpr int CH = 64;   // tokens per chunk

struct ChunkParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* eta;
    const uint16_t* w1;
    const uint16_t* w3;
    uint16_t* o;         // bf16 output (phi_split == 1)
    float* o_partial;    // [phi_split][B*H*T][d_v] fp32 (phi_split > 1)
    float* state;        // summaries / entry states
    float eta_scalar;
    float beta;
    int eta_kind;
    int T, H, d_k, d_v, d_phi;
    int dv_split, phi_split, seg_count, seg_len;
    int n_units;
    size_t n_rows;       // B * H * T
};

// bf16x8 built from two D tiles (4 floats each): elements 0..3 from x, 4..7 from y
__device__ __forceinline__ bf16x8 pack8(const f32x4& x, const f32x4& y) {
    u32x4 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
               pack_bf16x2(y[2], y[3])};
    return as_bf16x8(u);
}

// LDS layout of one workgroup (bf16 elements, then floats).  The staged tiles
// (q or raw q, k or raw k, v) and the score tiles are double-buffered so that
// one barrier per chunk suffices: chunk c is written into buffer c & 1 while
// other waves may still be finishing the deferred work of chunk c - 1.
template <int D, int DK, int NW, bool SWIGLU>
struct Lds {
    static constexpr int DVWG = 16 * NW;                 // value columns of one workgroup
    static constexpr int WX = SWIGLU ? DK : D;           // width of the staged q/k rows
    static constexpr int TX = CH * WX, TV = CH * DVWG;
    static constexpr int STAGE = 2 * TX + TV;            // one buffer: x_q, x_k, v
    static constexpr int OFF_PHI = 2 * STAGE;            // SwiGLU features phi(q), phi(k): [CH][D] each
    static constexpr int OFF_A = OFF_PHI + (SWIGLU ? 2 * CH * D : 0);   // 2 x [CH][CH] scores
    static constexpr int N_BF16 = OFF_A + 2 * CH * CH;
    // floats: 2 x (eta, eta/(1-beta), eta beta^{n-1-j}) [CH each], c[CH+1], beta^r[CH+1]
    static constexpr int N_F32 = 6 * CH + 2 * (CH + 1);
    static constexpr int BYTES = 2 * N_BF16 + 4 * N_F32;
    // The bidirectional kernel stages k (pass 0) and q (pass 1) in the same place,
    // never both at once, and has no score tiles: its floats follow the staged tiles.
    static constexpr int stage(bool bidir) { return bidir ? TX + TV : STAGE; }
    static constexpr int off_phi(bool bidir) { return 2 * stage(bidir); }
    static constexpr int n_bf16(bool bidir) { return bidir ? off_phi(true) + (SWIGLU ? 2 * CH * D : 0) : N_BF16; }
    static constexpr int bytes(bool bidir) { return 2 * n_bf16(bidir) + 4 * N_F32; }
    // workgroups that share a CU (160 KiB of LDS): three for the d = 64
    // bidirectional kernel without momentum (its registers fit in 168 a lane; four
    // would leave 128 and spill), otherwise up to two
    static constexpr int per_cu(bool bidir, bool mom) {
        constexpr int lds = 160 * 1024;
        const bool small = bidir && !mom && D == 64 && !SWIGLU;
        return (small && 3 * bytes(true) <= lds) ? 3 : 2 * bytes(bidir) <= lds ? 2 : 1;
    }
};

// Global -> register prefetch of one chunk: each thread owns 16-byte pieces of
// the x (q or raw q), y (k or raw k) and v tiles plus one eta value.
template <int WX, int DVWG, int NT>
struct Prefetch {
    static constexpr int PX = CH * WX / 8 / NT;       // pieces of a q/k tile per thread
    static constexpr int PV = CH * DVWG / 8 / NT;     // pieces of the v tile per thread
    static_assert(PX * NT * 8 == CH * WX && PV * NT * 8 == CH * DVWG, "tile split");
    u32x4 x[PX], y[PX], v[PV];
    float eta;
};

// NW waves of 64 lanes; each wave owns DVT tiles of 16 value columns (and the
// matching d_phi x 16 DVT slice of T and M in registers).  DV is the value
// width of the layer; DV / (16 NW DVT) workgroups share one sequence segment.
// ETAV: the step size varies per token (otherwise it is the scalar eta).
template <int D, int DK, int DV, int NW, int DVT, bool MOM, bool ETAV, bool SWIGLU, int KIND>
__global__ void __launch_bounds__(NW * 64, (NW == 4 ? Lds<D, DK, NW, SWIGLU>::per_cu(KIND == K_BIDIR, MOM) : 1))
chunk_kernel(ChunkParams p) {
    static_assert(DVT == 1, "one 16-column value tile per wave");
    using L = Lds<D, DK, NW, SWIGLU>;
    constexpr int NT = NW * 64;
    constexpr int DVWG = L::DVWG;
    constexpr int WX = L::WX;
    constexpr int NFT = D / 16;           // feature tiles of the state slice
    constexpr int NS = D / 32;            // contraction steps over features
    constexpr int NI = CH / 16;           // token blocks per chunk
    constexpr int NJS = CH / 32;          // contraction steps over tokens

    constexpr bool BI = KIND == K_BIDIR;
    constexpr int NB16 = L::n_bf16(BI);
    __shared__ __attribute__((aligned(16))) uint16_t smem16[NB16 + 2 * L::N_F32];
    float* sF = reinterpret_cast<float*>(smem16 + NB16);
    float* sC = sF + 6 * CH;        // c_r, r = 0..CH
    float* sBP = sC + CH + 1;       // beta^r, r = 0..CH
    constexpr int STG = L::stage(BI);
    auto stage_x = [&](int buf) { return smem16 + buf * STG; };
    auto stage_y = [&](int buf) { return smem16 + buf * STG + (BI ? 0 : L::TX); };
    auto stage_v = [&](int buf) { return smem16 + buf * STG + (BI ? 1 : 2) * L::TX; };
    auto tile_a = [&](int buf) { return smem16 + L::OFF_A + buf * CH * CH; };
    auto s_eta = [&](int buf) { return sF + buf * 3 * CH; };
    auto s_wt = [&](int buf) { return sF + buf * 3 * CH + CH; };    // eta_j / (1 - beta)
    auto s_wm = [&](int buf) { return sF + buf * 3 * CH + 2 * CH; }; // eta_j beta^{n-1-j}
    // feature rows read by the contractions: the staged rows (identity) or phi (SwiGLU)
    auto tile_q = [&](int buf) { return SWIGLU ? smem16 + L::off_phi(BI) : stage_x(buf); };
    auto tile_k = [&](int buf) { return SWIGLU ? smem16 + L::off_phi(BI) + CH * D : stage_y(buf); };

    // ---- unit of work (XCD-aware: consecutive units land on one XCD) --------
    const int G = gridDim.x;
    const int u = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_units) return;
    const int vs = u % p.dv_split;
    const int fs = (u / p.dv_split) % p.phi_split;
    const int rest = u / (p.dv_split * p.phi_split);
    const int nseg = (KIND == K_SUMMARY) ? p.seg_count - 1 : (KIND == K_BIDIR ? 1 : p.seg_count);
    const int seg = rest % nseg;
    const int seq = rest / nseg;
    const int h = seq % p.H;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    const int dvw = wave * 16;            // wave's first value column inside the slice
    const int dv_base = vs * DVWG;        // workgroup's first value column
    const float beta = p.beta;
    const float inv1mb = 1.0f / (1.0f - beta);
    // scale applied to the stored T when it is read: eta / (1 - beta) for a scalar step
    const float t_scale = ETAV ? 1.0f : p.eta_scalar * inv1mb;

    const int t_begin = (KIND == K_BIDIR) ? 0 : seg * p.seg_len;
    const int t_end = (KIND == K_BIDIR) ? p.T : min(p.T, t_begin + p.seg_len);
    const size_t seq_row = (size_t)seq * p.T;

    if (wave == 0) coefficient_scan<CH>(beta, sC, sBP);

    // zero the score tiles above the diagonal that the token-pair steps read
    if (KIND == K_OUTPUT) {
        for (int idx = tid; idx < 2 * (NI / 2) * 16 * 4; idx += NT) {
            const int buf = idx / ((NI / 2) * 64), w = idx % ((NI / 2) * 64);
            const int I = 2 * (w / 64), rr = (w / 4) % 16, q4 = w % 4;
            *reinterpret_cast<u32x2*>(tile_a(buf) + swz<CH>(16 * I + rr, 16 * (I + 1) + 4 * q4)) = u32x2{0u, 0u};
        }
    }

    // SwiGLU: this wave's rows of W1/W3 (feature slice fs) as MFMA A operands
    constexpr int FPW = SWIGLU ? D / NW : 16;       // features computed per wave
    constexpr int NFW = SWIGLU ? FPW / 16 : 1;
    constexpr int NSK = SWIGLU ? DK / 32 : 1;
    bf16x8 w1f[NFW][NSK];
    bf16x8 w3f[NFW][NSK];
    if constexpr (SWIGLU) {
        const size_t wrow0 = (size_t)h * p.d_phi + (size_t)fs * D + wave * FPW;
#pragma unroll
        for (int a = 0; a < NFW; ++a)
#pragma unroll
            for (int s = 0; s < NSK; ++s) {
                const size_t off = (wrow0 + 16 * a + c16) * DK + 32 * s + 8 * g;
                w1f[a][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(p.w1 + off));
                w3f[a][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(p.w3 + off));
            }
    }

    // ---- state slice in registers ------------------------------------------
    f32x4 St[NFT], M[MOM ? NFT : 1];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) St[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ft = 0; ft < (MOM ? NFT : 1); ++ft) M[ft] = f32x4{0.f, 0.f, 0.f, 0.f};

    // summaries / entry states: [slot][wave][ft][lane] f32x4, T then M
    constexpr size_t SLICE_F4 = (size_t)NW * NFT * 64;
    const size_t slice_units = (size_t)p.phi_split * p.dv_split;
    const size_t slot_stride = SLICE_F4 * 2;
    if (KIND == K_OUTPUT && seg > 0) {
        const size_t slot = ((size_t)seq * (p.seg_count - 1) + (seg - 1)) * slice_units + (size_t)fs * p.dv_split + vs;
        const f32x4* src = reinterpret_cast<const f32x4*>(p.state) + slot * slot_stride;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) St[ft] = src[((size_t)wave * NFT + ft) * 64 + lane];
        if constexpr (MOM) {
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) M[ft] = src[SLICE_F4 + ((size_t)wave * NFT + ft) * 64 + lane];
        }
    }

    using PF = Prefetch<WX, DVWG, NT>;
    constexpr int XCH = WX / 8;     // 16-byte pieces per q/k row
    constexpr int VCH = DVWG / 8;   // 16-byte pieces per v row

    // issue the global loads of the chunk starting at t0 into registers
    auto fetch = [&](PF& f, int t0, bool want_q, bool want_k, bool want_v, bool want_eta) {
        const int n = min(CH, t_end - t0);
        const size_t row0 = seq_row + t0;
        // the rate first: its address may have to come back from a register spill,
        // and waiting for that reload must not mean waiting for the chunk's loads
        f.eta = 0.0f;
        if (want_eta && tid < n) f.eta = ETAV ? p.eta[row0 + tid] : p.eta_scalar;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < PF::PX; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / XCH, c = idx % XCH;
            const size_t off = (row0 + r) * WX + 8 * c;
            f.x[i] = (want_q && r < n) ? *reinterpret_cast<const u32x4*>(p.q + off) : u32x4{0u, 0u, 0u, 0u};
            f.y[i] = (want_k && r < n) ? *reinterpret_cast<const u32x4*>(p.k + off) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < PF::PV; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / VCH, c = idx % VCH;
            const size_t off = (row0 + r) * DV + dv_base + 8 * c;
            f.v[i] = (want_v && r < n) ? *reinterpret_cast<const u32x4*>(p.v + off) : u32x4{0u, 0u, 0u, 0u};
        }
    };

    // write a prefetched chunk into buffer buf of the swizzled LDS tiles (and its token weights)
    auto commit = [&](const PF& f, int buf, int n, bool want_q, bool want_k, bool want_v, bool want_eta) {
#pragma unroll
        for (int i = 0; i < PF::PX; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / XCH, c = idx % XCH;
            if (want_q) *reinterpret_cast<u32x4*>(stage_x(buf) + swz<WX>(r, 8 * c)) = f.x[i];
            if (want_k) *reinterpret_cast<u32x4*>(stage_y(buf) + swz<WX>(r, 8 * c)) = f.y[i];
        }
        if (want_v) {
#pragma unroll
            for (int i = 0; i < PF::PV; ++i) {
                const int idx = tid + i * NT;
                const int r = idx / VCH, c = idx % VCH;
                *reinterpret_cast<u32x4*>(stage_v(buf) + swz<DVWG>(r, 8 * c)) = f.v[i];
            }
        }
        if (want_eta && tid < CH) {
            float et = tid < n ? f.eta : 0.0f;
            if (ETAV && p.eta_kind == ETA_SOFTPLUS && tid < n) et = softplus_f32(et);
            s_eta(buf)[tid] = et;
            s_wt(buf)[tid] = tid < n ? et * inv1mb : 0.0f;                // eta_j / (1 - beta)
            s_wm(buf)[tid] = tid < n ? et * sBP[n - 1 - tid] : 0.0f;      // eta_j beta^{n-1-j}
        }
    };

    // SwiGLU feature prologue: phi = silu(W1 x) * (W3 x) of the staged rows
    auto features = [&](int buf, bool do_q, bool do_k) {
        if constexpr (SWIGLU) {
#pragma unroll
            for (int a = 0; a < NFW; ++a) {
                const int f0 = wave * FPW + 16 * a;       // feature tile inside the slice
#pragma unroll
                for (int which = 0; which < 2; ++which) {
                    if (which == 0 && !do_q) continue;
                    if (which == 1 && !do_k) continue;
                    const uint16_t* X = which == 0 ? stage_x(buf) : stage_y(buf);
                    uint16_t* dst = which == 0 ? tile_q(buf) : tile_k(buf);
#pragma unroll
                    for (int I = 0; I < NI; ++I) {
                        f32x4 u1 = {0.f, 0.f, 0.f, 0.f}, u3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < NSK; ++s) {
                            bf16x8 xb = as_bf16x8(lds_read16(X + swz<DK>(16 * I + c16, 32 * s + 8 * g)));
                            u1 = mfma16(w1f[a][s], xb, u1);
                            u3 = mfma16(w3f[a][s], xb, u3);
                        }
                        // lane: features f0 + 4g + r of token 16I + c16
                        f32x4 ph;
#pragma unroll
                        for (int r = 0; r < 4; ++r) ph[r] = silu_f32(u1[r]) * u3[r];
                        u32x2 pk = {pack_bf16x2(ph[0], ph[1]), pack_bf16x2(ph[2], ph[3])};
                        *reinterpret_cast<u32x2*>(dst + swz<D>(16 * I + c16, f0 + 4 * g)) = pk;
                    }
                }
            }
        }
    };

    // readout of buffer buf from the current state into oacc (T part) and yacc (M part)
    f32x4 oacc[NI], yacc[MOM ? NI : 1];
    auto readout = [&](int buf, float scale, bool with_m) {
        const uint16_t* Q = tile_q(buf);
#pragma unroll
        for (int I = 0; I < NI; ++I) {
            oacc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (MOM) yacc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8 aS = pack8(St[2 * s], St[2 * s + 1]);
            bf16x8 aM;
            if constexpr (MOM) {
                if (with_m) aM = pack8(M[2 * s], M[2 * s + 1]);
            }
#pragma unroll
            for (int I = 0; I < NI; ++I) {
                const bf16x8 b = as_bf16x8(lds_read16(Q + swz<D>(16 * I + c16, 32 * s + 8 * g)));
                oacc[I] = mfma16(aS, b, oacc[I]);
                if constexpr (MOM) {
                    if (with_m) yacc[I] = mfma16(aM, b, yacc[I]);
                }
            }
        }
        if (scale != 1.0f) {
#pragma unroll
            for (int I = 0; I < NI; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[I][r] *= scale;
        }
    };

    // one output tile: lane holds O[row0 + 16I + c16][dv_base + dvw + 4g + r]
    auto store = [&](const f32x4& o, int I, int n, size_t row0) {
        const int i = 16 * I + c16;
        if (i < n) {
            const size_t orow = row0 + i;
            const int col = dv_base + dvw + 4 * g;
            if (p.phi_split == 1) {
                u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                *reinterpret_cast<u32x2*>(p.o + orow * DV + col) = pk;
            } else {
                float* dst = p.o_partial + ((size_t)fs * p.n_rows + orow) * DV + col;
                *reinterpret_cast<f32x4*>(dst) = o;
            }
        }
    };

    // v^T fragments of buffer buf: tokens 32t + 8g .. +7 of this wave's 16 columns
    u32x4 vt[NJS];
    auto read_vt = [&](int buf) {
#pragma unroll
        for (int t = 0; t < NJS; ++t) vt[t] = tr_read8<DVWG>(stage_v(buf), 32 * t + 8 * g, dvw + 4 * (lane & 3));
    };

    // state update with chunk buf (n tokens): T += K^T (w_T v), M = beta^n M + K^T (w_M v)
    auto update = [&](int buf, int n) {
        if constexpr (MOM) {
            const float bn = sBP[n];             // beta^n
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) M[ft][r] *= bn;
        }
        const uint16_t* K = tile_k(buf);
#pragma unroll
        for (int t = 0; t < NJS; ++t) {
            float wt[8], wm[8];
            if constexpr (ETAV) {
#pragma unroll
                for (int e = 0; e < 8; ++e) wt[e] = s_wt(buf)[32 * t + 8 * g + e];
            }
            if constexpr (MOM) {
#pragma unroll
                for (int e = 0; e < 8; ++e) wm[e] = s_wm(buf)[32 * t + 8 * g + e];
            }
            // rows beyond the chunk end are zero in the v tile
            const bf16x8 bT = ETAV ? scale8(vt[t], wt) : as_bf16x8(vt[t]);
            bf16x8 bM;
            if constexpr (MOM) bM = scale8(vt[t], wm);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
                const int colq = 32 * (ft >> 1) + 8 * (lane & 3) + 4 * (ft & 1);
                const bf16x8 a = as_bf16x8(tr_read8<D>(K, 32 * t + 8 * g, colq));
                St[ft] = mfma16(a, bT, St[ft]);
                if constexpr (MOM) M[ft] = mfma16(a, bM, M[ft]);
            }
        }
    };

    // scores of chunk buf: A = (P o Gamma) diag(eta), P = Phi_Q Phi_K^T, into tile_a(buf)
    auto scores = [&](int buf, int n) {
        constexpr int NTILE = NI * (NI + 1) / 2;
        const uint16_t* Q = tile_q(buf);
        const uint16_t* K = tile_k(buf);
        const float* eta = s_eta(buf);
        for (int ti = wave; ti < NTILE; ti += NW) {
            int I = 0, rem = ti;
            while (rem > I) { rem -= I + 1; ++I; }
            const int J = rem;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8 a = as_bf16x8(lds_read16(K + swz<D>(16 * J + c16, 32 * s + 8 * g)));
                bf16x8 b = as_bf16x8(lds_read16(Q + swz<D>(16 * I + c16, 32 * s + 8 * g)));
                acc = mfma16(a, b, acc);
            }
            // acc[r] = P[i = 16I + c16][j = 16J + 4g + r]
            const int i = 16 * I + c16;
            float val[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * J + 4 * g + r;
                val[r] = (j <= i && i < n) ? acc[r] * sC[max(i - j, 0)] * eta[j] : 0.0f;
            }
            u32x2 pk = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
            *reinterpret_cast<u32x2*>(tile_a(buf) + swz<CH>(i, 16 * J + 4 * g)) = pk;
        }
    };

    // intra-chunk term of chunk buf (scores and v^T fragments ready), combine, store
    auto intra_and_store = [&](int buf, int n, size_t row0) {
#pragma unroll
        for (int I = 0; I < NI; ++I) {
#pragma unroll
            for (int t = 0; t <= I / 2; ++t) {
                bf16x8 b = as_bf16x8(lds_read16(tile_a(buf) + swz<CH>(16 * I + c16, 32 * t + 8 * g)));
                oacc[I] = mfma16(as_bf16x8(vt[t]), b, oacc[I]);
            }
            f32x4 o = oacc[I];
            if constexpr (MOM) {
                const float gi = -beta * beta * sBP[16 * I + c16] * inv1mb;   // -beta^{i+2} / (1 - beta)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = fmaf(gi, yacc[I][r], o[r]);
            }
            store(o, I, n, row0);
        }
    };

    __syncthreads();   // coefficient tables and zeroed score tiles are visible

    if constexpr (KIND == K_OUTPUT) {
        // chunk c is staged in buffer c & 1; its intra-chunk term and store run in
        // the next iteration, after the one barrier that also publishes its scores
        PF pf;
        if (t_begin < t_end) fetch(pf, t_begin, true, true, true, true);
        int buf = 0, n_prev = 0;
        size_t row_prev = 0;
        for (int t0 = t_begin; t0 < t_end; t0 += CH) {
            const int n = min(CH, t_end - t0);
            const size_t row0 = seq_row + t0;
            commit(pf, buf, n, true, true, true, true);
            __syncthreads();
            if (t0 + CH < t_end) fetch(pf, t0 + CH, true, true, true, true);   // in flight during compute
            if (t0 > t_begin) intra_and_store(buf ^ 1, n_prev, row_prev);
            if constexpr (SWIGLU) {
                features(buf, true, true);
                lds_barrier();
            }
            scores(buf, n);
            readout(buf, t_scale, true);
            read_vt(buf);
            update(buf, n);
            n_prev = n;
            row_prev = row0;
            buf ^= 1;
        }
        __syncthreads();
        if (t_begin < t_end) intra_and_store(buf ^ 1, n_prev, row_prev);
    } else if constexpr (KIND == K_SUMMARY) {
        PF pf;
        if (t_begin < t_end) fetch(pf, t_begin, false, true, true, true);
        int buf = 0;
        for (int t0 = t_begin; t0 < t_end; t0 += CH) {
            const int n = min(CH, t_end - t0);
            commit(pf, buf, n, false, true, true, true);
            __syncthreads();
            if (t0 + CH < t_end) fetch(pf, t0 + CH, false, true, true, true);
            if constexpr (SWIGLU) {
                features(buf, false, true);
                lds_barrier();
            }
            read_vt(buf);
            update(buf, n);
            buf ^= 1;
        }
        const size_t slot = ((size_t)seq * (p.seg_count - 1) + seg) * slice_units + (size_t)fs * p.dv_split + vs;
        f32x4* dst = reinterpret_cast<f32x4*>(p.state) + slot * slot_stride;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) dst[((size_t)wave * NFT + ft) * 64 + lane] = St[ft];
        if constexpr (MOM) {
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) dst[SLICE_F4 + ((size_t)wave * NFT + ft) * 64 + lane] = M[ft];
        }
    } else {
        // bidirectional: pass 0 accumulates the state over all tokens, then every
        // query reads the final S = t_scale T - kappa M
        const float kappa = beta * inv1mb;
        auto final_state = [&]() {
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = St[ft][r] * t_scale;
                    if constexpr (MOM) v = fmaf(-kappa, M[ft][r], v);
                    St[ft][r] = v;
                }
        };
        // d = 64 sequences of at most NCB chunks (a ViT's patch rows): the loads of
        // the whole sequence are in flight together, 64 registers a thread.  The
        // loads take no branch (rows past the end read the last row and are zeroed
        // when staged), so that none of them waits for another.
        constexpr int NCB = 4;
        if constexpr (D == 64 && !SWIGLU) {
            if (t_end > 0 && t_end <= NCB * CH) {
                const size_t last = seq_row + t_end - 1;
                auto fetch_rows = [&](PF& f, int t0, bool kv) {
                    if (kv) f.eta = ETAV ? p.eta[min(seq_row + t0 + tid, last)] : p.eta_scalar;
#pragma unroll
                    for (int i = 0; i < PF::PX; ++i) {
                        const int idx = tid + i * NT;
                        const size_t off = min(seq_row + t0 + idx / XCH, last) * WX + 8 * (idx % XCH);
                        if (kv) f.y[i] = *reinterpret_cast<const u32x4*>(p.k + off);
                        else f.x[i] = *reinterpret_cast<const u32x4*>(p.q + off);
                    }
                    if (kv) {
#pragma unroll
                        for (int i = 0; i < PF::PV; ++i) {
                            const int idx = tid + i * NT;
                            const size_t off = min(seq_row + t0 + idx / VCH, last) * DV + dv_base + 8 * (idx % VCH);
                            f.v[i] = *reinterpret_cast<const u32x4*>(p.v + off);
                        }
                    }
                };
                // stages rows below n, zeros in the rest
                auto commit_rows = [&](const PF& f, int buf, int n, bool kv) {
                    PF m;
                    m.eta = f.eta;
#pragma unroll
                    for (int i = 0; i < PF::PX; ++i) {
                        const bool in = (tid + i * NT) / XCH < n;
                        m.x[i] = (!kv && in) ? f.x[i] : u32x4{0u, 0u, 0u, 0u};
                        m.y[i] = (kv && in) ? f.y[i] : u32x4{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int i = 0; i < PF::PV; ++i)
                        m.v[i] = (kv && (tid + i * NT) / VCH < n) ? f.v[i] : u32x4{0u, 0u, 0u, 0u};
                    commit(m, buf, n, !kv, kv, kv, kv);
                };
                // k and v of every chunk first; the q loads of a chunk go out once
                // its k and v are staged, into the registers they leave
                PF pk[NCB], pq[NCB];
#pragma unroll
                for (int c = 0; c < NCB; ++c) fetch_rows(pk[c], c * CH, true);
                int buf = 0;
#pragma unroll
                for (int c = 0; c < NCB; ++c) {
                    const int n = min(CH, t_end - c * CH);
                    if (n <= 0) break;
                    commit_rows(pk[c], buf, n, true);
                    fetch_rows(pq[c], c * CH, false);
                    __syncthreads();
                    read_vt(buf);
                    update(buf, n);
                    buf ^= 1;
                }
                final_state();
                __syncthreads();
                buf = 0;
#pragma unroll
                for (int c = 0; c < NCB; ++c) {
                    const int n = min(CH, t_end - c * CH);
                    if (n <= 0) break;
                    commit_rows(pq[c], buf, n, false);
                    __syncthreads();
                    readout(buf, 1.0f, false);
#pragma unroll
                    for (int I = 0; I < NI; ++I) store(oacc[I], I, n, seq_row + c * CH);
                    buf ^= 1;
                }
                return;
            }
        }
        PF pf;
        fetch(pf, 0, false, true, true, true);
        int buf = 0;
        for (int t0 = 0; t0 < t_end; t0 += CH) {
            const int n = min(CH, t_end - t0);
            commit(pf, buf, n, false, true, true, true);
            __syncthreads();
            // the next chunk's k and v; during the last chunk the first chunk's q
            if (t0 + CH < t_end) fetch(pf, t0 + CH, false, true, true, true);
            else fetch(pf, 0, true, false, false, false);
            if constexpr (SWIGLU) {
                features(buf, false, true);
                lds_barrier();
            }
            read_vt(buf);
            update(buf, n);
            buf ^= 1;
        }
        final_state();
        __syncthreads();
        buf = 0;
        for (int t0 = 0; t0 < t_end; t0 += CH) {
            const int n = min(CH, t_end - t0);
            const size_t row0 = seq_row + t0;
            commit(pf, buf, n, true, false, false, false);
            __syncthreads();
            if (t0 + CH < t_end) fetch(pf, t0 + CH, true, false, false, false);
            if constexpr (SWIGLU) {
                features(buf, true, false);
                lds_barrier();
            }
            readout(buf, 1.0f, false);
#pragma unroll
            for (int I = 0; I < NI; ++I) store(oacc[I], I, n, row0);
            buf ^= 1;
        }
    }
}

// Composes segment summaries into entry states, in place, for the (T, M) state:
//   T <- T + dT_p,  M <- beta^L M + dM_p,  slot p <- (T, M) = entry of segment p + 1
// (L = segment length).  Slots are [seq][step][slice] and hold T then M
// (slice_f4 float4s each).  One thread per float4 of a slice.
__global__ void segment_scan(float* state, size_t n_threads, int n_slices, int n_steps, int slice_f4, float bL,
                             int mom) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_threads) return;
    const size_t e_per_seq = (size_t)n_slices * slice_f4;
    const size_t seqi = idx / e_per_seq;
    const size_t within = idx % e_per_seq;
    const size_t sl = within / slice_f4, e = within % slice_f4;
    f32x4* base = reinterpret_cast<f32x4*>(state);
    f32x4 T = {0.f, 0.f, 0.f, 0.f}, M = {0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step < n_steps; ++step) {
        const size_t slot = (seqi * n_steps + step) * n_slices + sl;
        f32x4* ps = base + slot * 2 * slice_f4 + e;
        const f32x4 dT = ps[0];
#pragma unroll
        for (int r = 0; r < 4; ++r) T[r] += dT[r];
        ps[0] = T;
        if (mom) {
            const f32x4 dM = ps[slice_f4];
#pragma unroll
            for (int r = 0; r < 4; ++r) M[r] = fmaf(bL, M[r], dM[r]);
            ps[slice_f4] = M;
        }
    }
}

// o[row][c] = bf16( sum_{s < n_split} partial[s][row][c] ), fixed order
__global__ void partial_reduce(const float* partial, uint16_t* o, size_t n_elem4, int n_split) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_elem4) return;
    const f32x4* src = reinterpret_cast<const f32x4*>(partial);
    f32x4 acc = src[idx];
    for (int s = 1; s < n_split; ++s) {
        f32x4 x = src[(size_t)s * n_elem4 + idx];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += x[r];
    }
    u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    reinterpret_cast<u32x2*>(o)[idx] = pk;
}

}  // namespace

// ---------------------------------------------------------------------------
// plan and launches
// ---------------------------------------------------------------------------

bool fast_supported(const Shape& s, int chunk) {
    if (!s.bf16) return false;
    if (s.d_k != 64 && s.d_k != 128) return false;
    if (s.d_v != 64 && s.d_v != 128) return false;
    if (s.swiglu) {
        if (s.d_phi % 128 != 0 || s.d_phi > 512) return false;
    } else if (s.d_phi != s.d_k) {
        return false;
    }
    return chunk == 0 || chunk == 64 || chunk == 128;
}

FastPlan fast_plan(const Shape& s, int /*chunk*/, int segments, int value_split, int launch) {
    FastPlan p{};
    if (wide_supported(s) && value_split != 2) {
        // one workgroup of four waves per sequence segment (chunk_wide.hip)
        p.wide = true;
        p.chunk = CH;
        p.nwaves = 4;
        p.dvt = 2;
        p.dv_split = 1;
        p.phi_split = 1;
        const int n_chunks = (s.T + CH - 1) / CH;
        int S = 1;
        if (segments > 0) {
            S = std::min(std::min(segments, n_chunks), wide_max_segments());
        } else {
            while ((long)s.n_seq() * S < 256 && n_chunks >= 8 * S && 2 * S <= wide_max_segments()) S *= 2;
        }
        const int seg_chunks = (n_chunks + S - 1) / S;
        p.seg_len = seg_chunks * CH;
        p.segments = (n_chunks + seg_chunks - 1) / seg_chunks;
        p.partial_bytes = 0;
        p.zero_bytes = wide_zero_bytes(s);
        if (launch == TTT_LA_LAUNCH_PREFIX) {
            p.prefix = true;
            wide_prefix_bounds(s.T, p.segments, p.bounds);
            p.summary_bytes = 0;
            p.zero_bytes = 0;
            return p;
        }
        // one launch, on request, when every workgroup of the grid can be resident at once
        const long grid = ((long)s.n_seq() * p.segments + 7) / 8 * 8;
        p.fused = launch == TTT_LA_LAUNCH_SINGLE && p.segments > 1 && grid <= wide_fused_capacity();
        // two segments whose one summary would leave half the CUs idle: summarise the
        // halves of segment 0 (an even number of chunks, at least 8 each)
        p.sum_split = (!p.fused && p.segments == 2 && 2L * s.n_seq() <= 256 && seg_chunks % 2 == 0 &&
                       seg_chunks >= 16)
                          ? 2
                          : 1;
        p.summary_bytes = wide_summary_bytes(s, p.segments + (p.sum_split == 2 ? 1 : 0));
        return p;
    }
    if (swiglu_supported(s)) {
        // causal: one workgroup per (sequence, 128-feature slice) over the whole
        // sequence (swiglu.hip); bidirectional: the 16x16-tile kernel below with the
        // same slices and the same partial-output area
        p.swiglu32 = true;
        p.chunk = CH;
        p.phi_split = s.d_phi / 128;
        p.dvt = 1;
        p.dv_split = 1;
        p.nwaves = s.d_v / 16;
        p.segments = 1;
        p.seg_len = s.T;
        p.summary_bytes = 0;
        // the mode is a per-call choice: room for either kernel's parts (bf16 whole
        // chunks for the causal kernel, fp32 rows for the bidirectional one)
        p.partial_bytes = std::max(swiglu_partial_bytes(s), (size_t)p.phi_split * s.n_seq() * s.T * s.d_v * sizeof(float));
        return p;
    }
    // The chunk length is a tiling choice (results differ only by rounding);
    // this path always tiles at 64 tokens.
    p.chunk = CH;
    p.phi_split = s.swiglu ? s.d_phi / 128 : 1;
    // one wave per 16 value columns; identity maps with d = 128 may split the
    // value columns over two workgroups of four waves
    p.dvt = 1;
    p.dv_split = (value_split == 2 && !s.swiglu && s.d_k == 128 && s.d_v == 128) ? 2 : 1;
    p.nwaves = s.d_v / (16 * p.dv_split);
    const int D = s.swiglu ? 128 : s.d_k;
    const int n_chunks = (s.T + CH - 1) / CH;
    const long base = (long)s.n_seq() * p.phi_split * p.dv_split;
    int S = 1;
    if (segments > 0) {
        S = std::min(segments, n_chunks);
    } else {
        // enough workgroups for 256 CUs, segments of at least 4 chunks
        const long target = p.nwaves == 8 ? 256 : 512;
        while (base * S < target && n_chunks >= 8 * S) S *= 2;
    }
    const int seg_chunks = (n_chunks + S - 1) / S;
    p.seg_len = seg_chunks * CH;
    p.segments = (n_chunks + seg_chunks - 1) / seg_chunks;
    const size_t slice_floats = (size_t)p.nwaves * (D / 16) * p.dvt * 64 * 4;
    p.summary_bytes = p.segments > 1
        ? (size_t)s.n_seq() * (p.segments - 1) * p.phi_split * p.dv_split * slice_floats * 2 * sizeof(float)
        : 0;
    p.partial_bytes = p.phi_split > 1 ? (size_t)p.phi_split * s.n_seq() * s.T * s.d_v * sizeof(float) : 0;
    return p;
}

namespace {

// With events, the launch carries them (hipExtLaunchKernel): they take their
// timestamps at the start and end of the kernel itself, not around its dispatch.
template <int D, int DK, int DV, int NW, bool MOM, bool ETAV, bool SW, int KIND>
hipError_t launch_one(const ChunkParams& cp, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
    const int grid = (cp.n_units + 7) / 8 * 8;
    if (eb || ee) {
        ChunkParams a = cp;
        void* args[] = {&a};
        return hipExtLaunchKernel(reinterpret_cast<const void*>(chunk_kernel<D, DK, DV, NW, 1, MOM, ETAV, SW, KIND>),
                                  dim3(grid), dim3(NW * 64), args, 0, st, eb, ee, 0);
    }
    hipLaunchKernelGGL((chunk_kernel<D, DK, DV, NW, 1, MOM, ETAV, SW, KIND>), dim3(grid), dim3(NW * 64), 0, st,
                       cp);
    return hipGetLastError();
}

template <int D, int DK, int DV, int NW, bool MOM, bool ETAV, bool SW>
hipError_t launch_k(int kind, const ChunkParams& cp, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
    if (kind == K_OUTPUT) return launch_one<D, DK, DV, NW, MOM, ETAV, SW, K_OUTPUT>(cp, st, eb, ee);
    if (kind == K_SUMMARY) return launch_one<D, DK, DV, NW, MOM, ETAV, SW, K_SUMMARY>(cp, st, eb, ee);
    return launch_one<D, DK, DV, NW, MOM, ETAV, SW, K_BIDIR>(cp, st, eb, ee);
}

template <int D, int DK, int DV, int NW, bool SW>
hipError_t launch_kind(int kind, bool mom, bool etav, const ChunkParams& cp, hipStream_t st, hipEvent_t eb,
                       hipEvent_t ee) {
    if (mom) {
        return etav ? launch_k<D, DK, DV, NW, true, true, SW>(kind, cp, st, eb, ee)
                    : launch_k<D, DK, DV, NW, true, false, SW>(kind, cp, st, eb, ee);
    }
    return etav ? launch_k<D, DK, DV, NW, false, true, SW>(kind, cp, st, eb, ee)
                : launch_k<D, DK, DV, NW, false, false, SW>(kind, cp, st, eb, ee);
}

// one wave per 16 value columns of the workgroup; DV / (16 NW) workgroups per sequence
hipError_t launch_chunk(const Shape& s, const FastPlan& p, int kind, bool mom, bool etav, const ChunkParams& cp,
                        hipStream_t st, hipEvent_t eb = nullptr, hipEvent_t ee = nullptr) {
    if (!s.swiglu) {
        if (s.d_k == 128) {
            if (s.d_v == 128) {
                return p.nwaves == 8 ? launch_kind<128, 128, 128, 8, false>(kind, mom, etav, cp, st, eb, ee)
                                     : launch_kind<128, 128, 128, 4, false>(kind, mom, etav, cp, st, eb, ee);
            }
            return launch_kind<128, 128, 64, 4, false>(kind, mom, etav, cp, st, eb, ee);
        }
        return s.d_v == 128 ? launch_kind<64, 64, 128, 8, false>(kind, mom, etav, cp, st, eb, ee)
                            : launch_kind<64, 64, 64, 4, false>(kind, mom, etav, cp, st, eb, ee);
    }
    if (s.d_k == 128) {
        return s.d_v == 128 ? launch_kind<128, 128, 128, 8, true>(kind, mom, etav, cp, st, eb, ee)
                            : launch_kind<128, 128, 64, 4, true>(kind, mom, etav, cp, st, eb, ee);
    }
    return s.d_v == 128 ? launch_kind<128, 64, 128, 8, true>(kind, mom, etav, cp, st, eb, ee)
                        : launch_kind<128, 64, 64, 4, true>(kind, mom, etav, cp, st, eb, ee);
}

}  // namespace

hipError_t launch_fast(const Shape& s, const FastPlan& p, void* workspace, const FwdArgs& a, hipEvent_t ev_begin,
                       hipEvent_t ev_end, int* n_kernels) {
    if (p.wide) return launch_wide(s, p, workspace, a, ev_begin, ev_end, n_kernels);
    if (p.swiglu32 && !a.bidirectional) return launch_swiglu(s, workspace, a, ev_begin, ev_end, n_kernels);
    if (a.reverse) return hipErrorInvalidValue;   // time reversal: 32x32-tile kernels only
    ChunkParams cp{};
    cp.q = static_cast<const uint16_t*>(a.q);
    cp.k = static_cast<const uint16_t*>(a.k);
    cp.v = static_cast<const uint16_t*>(a.v);
    cp.eta = a.eta;
    cp.w1 = static_cast<const uint16_t*>(s.w1);
    cp.w3 = static_cast<const uint16_t*>(s.w3);
    cp.o = static_cast<uint16_t*>(a.o);
    cp.state = static_cast<float*>(workspace);
    cp.o_partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.summary_bytes);
    cp.eta_scalar = a.eta_scalar;
    cp.beta = a.beta;
    cp.eta_kind = a.eta_kind;
    cp.T = s.T;
    cp.H = s.H;
    cp.d_k = s.d_k;
    cp.d_v = s.d_v;
    cp.d_phi = s.d_phi;
    cp.dv_split = p.dv_split;
    cp.phi_split = p.phi_split;
    cp.n_rows = (size_t)s.n_seq() * s.T;
    const bool mom = a.beta != 0.0f;
    const bool etav = a.eta_kind != ETA_SCALAR;
    const int slice_units = p.phi_split * p.dv_split;
    hipStream_t st = a.stream;
    int nk = 0;
    hipError_t e = hipSuccess;

    if (a.bidirectional) {
        cp.seg_count = 1;
        cp.seg_len = s.T;
        cp.n_units = s.n_seq() * slice_units;
        if ((e = launch_chunk(s, p, K_BIDIR, mom, etav, cp, st, ev_begin, ev_end)) != hipSuccess) return e;
        ++nk;
    } else {
        cp.seg_count = p.segments;
        cp.seg_len = p.seg_len;
        if (p.segments > 1) {
            cp.n_units = s.n_seq() * (p.segments - 1) * slice_units;
            if ((e = launch_chunk(s, p, K_SUMMARY, mom, etav, cp, st)) != hipSuccess) return e;
            ++nk;
            if (p.segments > 2) {
                // with two segments the one summary already is the entry state
                const int D = s.swiglu ? 128 : s.d_k;
                const int slice_f4 = p.nwaves * (D / 16) * p.dvt * 64;
                const size_t n_threads = (size_t)s.n_seq() * slice_units * slice_f4;
                const double bL = std::pow((double)a.beta, (double)p.seg_len);   // beta^L
                hipLaunchKernelGGL(segment_scan, dim3((unsigned)((n_threads + 255) / 256)), dim3(256), 0, st,
                                   cp.state, n_threads, slice_units, p.segments - 1, slice_f4, (float)bL,
                                   mom ? 1 : 0);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                ++nk;
            }
        }
        cp.n_units = s.n_seq() * p.segments * slice_units;
        if ((e = launch_chunk(s, p, K_OUTPUT, mom, etav, cp, st, ev_begin, ev_end)) != hipSuccess) return e;
        ++nk;
    }
    if (p.phi_split > 1) {
        const size_t n4 = (size_t)s.n_seq() * s.T * s.d_v / 4;
        hipLaunchKernelGGL(partial_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, cp.o_partial,
                           static_cast<uint16_t*>(a.o), n4, p.phi_split);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        ++nk;
    }
    if (n_kernels) *n_kernels = nk;
    return hipSuccess;
}

}  // namespace ttt
