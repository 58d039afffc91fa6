// Wide-tile bf16 MFMA chunk kernels for gfx950: the TTT forward for the
// identity feature map with d_k = d_v = 128 (Variants 3-5 of Table 2 on the
// thelatestinai.com page), one workgroup of four waves per sequence segment.
//
// Same chunk algebra as the 16x16 kernels (chunk_mfma.hip): within a chunk of
// n tokens entered with the carried state (T, M), T = S + beta/(1-beta) M,
//   o_i = T q_i - beta^{i+2}/(1-beta) M q_i + sum_{j<=i} eta_j c_{i-j} (q_i . k_j) v_j
//   T  <- T + sum_j eta_j v_j k_j^T / (1 - beta)
//   M  <- beta^n M + sum_j eta_j beta^{n-1-j} v_j k_j^T
// with c_r = sum_{u<=r} beta^u: dense causal blocks inside the chunk and a
// fixed-size fp32 state between chunks, the parallel evaluation of the
// outer-product accumulation that the kualia.ai blog ("The Linear Attention
// Equivalence") identifies with linear attention.
//
// Why a second kernel family.  On gfx950 the LDS delivers about 128 bytes per
// clock per CU to 16-byte reads and less to transpose reads, while one
// v_mfma_f32_16x16x32_bf16 consumes 2 KiB of operands per 16 K flops.  With
// v_mfma_f32_32x32x16_bf16 the same operand bytes feed twice the flops, and a
// wave owning 32 value rows of the state reads each staged q and k row once
// per 32 rows instead of once per 16.  Each of the four waves keeps T and M for
// its 32 value columns (4 tiles of 32 features x 32 values each, 128 fp32
// registers) and issues the readout, the update and its share of the score
// tiles; the workgroup needs one barrier per chunk.
//
// Register layouts of v_mfma_f32_32x32x16_bf16 (lane l, n = l % 32, h = l / 32):
//   A operand  lane holds A[m = n][k = 8h .. 8h+7]
//   B operand  lane holds B[k = 8h .. 8h+7][n]
//   D result   lane holds D[m = 8(r/4) + 4h + r%4][n], r = 0..15
// The state is kept as D tiles of T^T (features x values).  The A-operand rows
// of the update (features) are permuted by sigma(m) = 16(q/2) + 8h + 4(q%2) + r'
// for m = 8q + 4h + r', so that accumulator registers 8k .. 8k+7 of a tile
// hold 8 consecutive features: the state feeds the readout directly as an A
// operand whose B operand is one 16-byte row read of q.  The value columns
// (the n index of the update, taken from the transpose read of v) are permuted
// by pi(m) = 16h + 4q + r', so that after the readout each lane holds 16
// consecutive output columns of one token (two 16-byte stores).  Inside a
// 16-token contraction block the lanes of half h take tokens 4h .. 4h+3 and
// 8+4h .. 8+4h+3, which is exactly how a 32x32 score tile S^T = K Q^T leaves
// them in its accumulators; the scaled score tiles therefore go to LDS as ready
// B-operand fragments (16 bytes per lane, no swizzle) and come back with
// conflict-free 16-byte reads.

#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "internal.h"
#include "lds_tiles.h"

// every helper lambda of the kernels is inlined: a lambda left as a call keeps the
// state it captures by reference in scratch memory
#define TTT_INLINE __attribute__((always_inline))

namespace ttt {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

enum WideKind : int { W_OUTPUT = 0, W_SUMMARY = 1, W_BIDIR = 2, W_FUSED = 3, W_PREFIX = 4 };

constexpr int WC = 64;     // tokens per chunk
constexpr int WD = 128;    // features (d_k = d_phi) and values (d_v)
constexpr int WNW = 4;     // waves per workgroup; wave w owns value columns 32w .. 32w+31
constexpr int WNT = WNW * 64;
constexpr int WFT = WD / 32;    // feature tiles of the state per wave
constexpr int WKB = WC / 16;    // 16-token contraction blocks per chunk

struct WideParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* eta;
    uint16_t* o;
    float* state;        // segment summaries / entry states
    float eta_scalar;
    float beta;
    int eta_kind;
    int T;
    int seg_count, seg_len;
    int slot_count;     // workspace slots per sequence
    int entry_split;    // summary slots per segment: segment j enters with slot j entry_split
    float beta_seg;      // beta^seg_len
    int n_units;
    // cooperative (fused) launch only: per-sequence arrival counters (two per
    // sequence), this launch's epoch, a bound on each wait, and a flag set when a
    // wait gave up
    unsigned* counters;
    unsigned epoch;
    unsigned spin_limit;
    unsigned* wait_failed;
    // W_PREFIX: first token of each segment, bounds[seg_count] = T
    int bounds[17];
    // carried state in the caller's layout, fp32 [seq][d_v][d_phi] (W_OUTPUT):
    // the entry state of segment 0 (has_init; with several segments the scan
    // copies it into slot 0 first) and the state after the last token (either
    // output may be null)
    const float* S0;
    const float* M0;
    float* S_T;
    float* M_T;
    int has_init;
    int reverse;        // time-reversed rows (see FwdArgs::reverse)
};

// The caller's state layout [seq][d_v][d_phi] against the register tiles: lane l
// of wave w holds value column vcol(w, l) of the fast weight, and the f32x4 group
// r4 of feature tile ft holds the four consecutive features user_f0(ft, r4, l).
__device__ __forceinline__ int user_vcol(int w, int l) {
    return 32 * w + 16 * ((l >> 2) & 1) + 8 * ((l >> 4) & 1) + 4 * ((l >> 3) & 1) + (l & 3);
}
__device__ __forceinline__ int user_f0(int ft, int r4, int l) {
    return 32 * ft + 16 * (r4 >> 1) + 8 * (l >> 5) + 4 * (r4 & 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// accumulator registers 8 kh .. 8 kh + 7 of a 32x32 tile as one bf16 operand
__device__ __forceinline__ bf16x8 pack_half(const f32x16& x, int kh) {
    const int b = 8 * kh;
    u32x4 u = {pack_bf16x2(x[b + 0], x[b + 1]), pack_bf16x2(x[b + 2], x[b + 3]),
               pack_bf16x2(x[b + 4], x[b + 5]), pack_bf16x2(x[b + 6], x[b + 7])};
    return as_bf16x8(u);
}

// LDS of one workgroup.  Stage buffers hold the 64 x 128 bf16 tiles of one
// chunk (XOR-swizzled rows): q, k, v for the output pass, k, v for the
// summary pass and the first pass of the bidirectional kernel, q for its
// second pass.  Three buffers: the copy of chunk c + 2 is in flight while
// chunk c is computed.  Each buffer is a separate __shared__ object and the chunk
// loop is unrolled over the ring, so that in every step the buffer being
// filled by global_load_lds and the buffers being read are distinct objects:
// the compiler then knows that the transpose reads cannot alias the copies in
// flight and does not make them wait.  Besides: the score fragments of the
// current chunk (3 tiles x 2 halves x 64 lanes x 16 bytes) and floats: the
// per-token weights of every buffer, c_r, beta^r, and the score coefficients
// k0 c_d at index 64 + d (zero for d < 0).
struct WideLds {
    static constexpr int TILE = WC * WD;
    static constexpr int P_FRAG = 3 * 2 * 64 * 8;
    static constexpr int N_F32 = 4 * 2 * WC + 2 * (WC + 1) + 2 + 2 * WC;
};
template <int KIND>
struct WideRing {
    static constexpr bool QKV = KIND == W_OUTPUT || KIND == W_FUSED || KIND == W_PREFIX;
    static constexpr int NB = 3;                                  // buffers
    static constexpr int TILES = QKV ? 3 : 2;                     // tiles per buffer
    static constexpr int SIZE = TILES * WideLds::TILE;
    static constexpr int K_OFF = QKV ? WideLds::TILE : 0;
    static constexpr int V_OFF = QKV ? 2 * WideLds::TILE : WideLds::TILE;
    static constexpr int BYTES = 2 * NB * SIZE + 2 * WideLds::P_FRAG + 4 * WideLds::N_F32;
};
static_assert(WideRing<W_OUTPUT>::BYTES <= 160 * 1024 && WideRing<W_SUMMARY>::BYTES <= 160 * 1024, "LDS budget");

// s_waitcnt immediate for vmcnt(k) alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
constexpr int vmcnt_imm(int k) { return (k & 15) | ((k >> 4) << 14) | 0x0F70; }

// Arrival barrier of the workgroups of one sequence (W_FUSED only; the
// cooperative launch makes them co-resident).  Every workgroup adds 1 to
// *counter and waits until it reaches target = epoch x workgroups per
// sequence; counters only grow, so nothing is reset between launches.  The
// release makes this workgroup's global writes visible device-wide before it
// arrives.  Polling uses relaxed atomic loads (an acquire on every poll would
// invalidate the caches the other workgroups of the XCD are using); one
// acquire fence follows the last poll.  The wait is bounded: after spin_limit
// polls it sets *failed and returns, so the kernel always terminates.
__device__ __forceinline__ void seq_sync(unsigned* counter, unsigned target, unsigned spin_limit, unsigned* failed) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        unsigned polls = 0;
        while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++polls > spin_limit) {
                __hip_atomic_store(failed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

template <bool MOM, bool ETAV, int KIND>
__global__ void __launch_bounds__(WNT, 1) wide_kernel(WideParams p) {
    using L = WideLds;
    using R = WideRing<KIND>;
    __shared__ __attribute__((aligned(16))) uint16_t stage_a[R::SIZE];
    __shared__ __attribute__((aligned(16))) uint16_t stage_b[R::SIZE];
    __shared__ __attribute__((aligned(16))) uint16_t stage_c[R::SIZE];
    __shared__ __attribute__((aligned(16))) uint16_t pfrag[R::QKV ? L::P_FRAG : 8];
    __shared__ __attribute__((aligned(16))) float sF[L::N_F32];
    float* const w_a = sF;               // per-token weights of the chunk in stage_a
    float* const w_b = sF + 2 * WC;      // ... stage_b
    float* const w_c = sF + 4 * WC;      // ... stage_c
    float* sC = sF + 8 * WC;             // c_r, r = 0..WC
    float* sBP = sC + WC + 1;            // beta^r, r = 0..WC
    float* sK = sBP + WC + 1 + 2;        // k0 c_{x - 64} for x >= 64, 0 below (x = 0..127)
    auto tq = [](uint16_t* st) TTT_INLINE { return st; };
    auto tk = [](uint16_t* st) TTT_INLINE { return st + R::K_OFF; };
    auto tv = [](uint16_t* st) TTT_INLINE { return st + R::V_OFF; };
    auto s_wt = [](float* w) TTT_INLINE { return w; };          // eta_j / (1 - beta)
    auto s_wm = [](float* w) TTT_INLINE { return w + WC; };     // eta_j beta^{n-1-j}
    u32x4* const P_lds = reinterpret_cast<u32x4*>(pfrag);

    // ---- unit of work (XCD-aware: consecutive units land on one XCD) --------
    const int G = gridDim.x;
    const int u = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (u >= p.n_units) return;
    const int nseg = (KIND == W_SUMMARY) ? p.seg_count - 1 : (KIND == W_BIDIR ? 1 : p.seg_count);
    // the workgroups of one sequence must be co-resident for W_FUSED; the launch guarantees it
    const int seg = u % nseg;
    const int seq = u / nseg;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const int g16 = (lane >> 4) & 1;     // which half of n the lane's 16-lane group covers
    const int q4 = lane & 3;             // column quartet a lane points at in a transpose read
    const float beta = p.beta;
    const float inv1mb = 1.0f / (1.0f - beta);
    const float t_scale = ETAV ? 1.0f : p.eta_scalar * inv1mb;

    // token range of the pass being run (the prefix kernel runs two passes)
    int t_begin = (KIND == W_BIDIR) ? 0 : (KIND == W_PREFIX ? p.bounds[seg] : seg * p.seg_len);
    int t_end = (KIND == W_BIDIR) ? p.T : (KIND == W_PREFIX ? p.bounds[seg + 1] : min(p.T, t_begin + p.seg_len));
    const size_t seq_row = (size_t)seq * p.T;

    if (wave == 0) coefficient_scan<WC>(beta, sC, sBP);

    // ---- state: T^T and M^T tiles (features x this wave's 32 value columns) --
    f32x16 Ts[WFT], Ms[MOM ? WFT : 1];
#pragma unroll
    for (int ft = 0; ft < WFT; ++ft) Ts[ft] = f32x16{};
#pragma unroll
    for (int ft = 0; ft < (MOM ? WFT : 1); ++ft) Ms[ft] = f32x16{};
    // The momentum is M = rho Ms with a workgroup-uniform scale rho: the decay
    // beta^n of a chunk multiplies rho instead of the 64 accumulator registers, and
    // the chunk's M weights are divided by the new rho.  Ms absorbs rho (one pass
    // over the registers) only when rho would fall below RHO_MIN; so rho stays in
    // [RHO_MIN, 1] and the weights within a factor 1 / RHO_MIN of their value.
    constexpr float RHO_MIN = 0x1p-60f;
    float rho = 1.0f;
    // rho after a chunk of n tokens entered with rho = r0 (without renormalisation
    // if it stays >= RHO_MIN); the update takes the same step
    auto rho_step = [&](float r0, int n) TTT_INLINE {
        const float r = r0 * sBP[n];
        return r < RHO_MIN ? 1.0f : r;
    };

    // workspace slots: [slot][T | M][wave][ft][r4][lane] f32x4 (16 floats per lane per tile)
    constexpr size_t TILE_F4 = 4 * 64;
    constexpr size_t HALF_F4 = (size_t)WNW * WFT * TILE_F4;
    // seg_count slots per sequence: slot j (j >= 1) receives the summary of segment
    // j - 1 and, after the scan, holds the entry state of segment j; slot 0 holds
    // the carried entry state of segment 0 (when the call has one)
    auto slot_ptr = [&](int s) TTT_INLINE {
        return reinterpret_cast<f32x4*>(p.state) + ((size_t)seq * p.slot_count + s) * 2 * HALF_F4;
    };

    // transpose-read columns: value columns in pi order, feature columns in sigma order
    const int col_v = 32 * wave + 16 * (q4 & 1) + 8 * g16 + 4 * (q4 >> 1);
    auto col_k = [&](int ft) TTT_INLINE { return 32 * ft + 16 * g16 + 8 * (q4 & 1) + 4 * (q4 >> 1); };

    // Asynchronous staging: buffer loads straight into LDS, 16 bytes per lane.
    // Wave w copies the row groups 4g .. 4g+3 with g = w, w+4, w+8, w+12 of each
    // tile: one instruction fills 1 KiB of LDS, lane L landing at byte 16 L =
    // row L / 16, physical piece L % 16, so the lane reads the logical piece
    // (L % 16) ^ f(row) of its row; f(row) = 4 (row % 4) + (row / 4) % 4 is
    // 4 (L / 16) + w for every group this wave copies.  Each copy goes through a
    // buffer resource spanning exactly the chunk's n valid rows: rows past the
    // end of the sequence read as zero (range check), and the lane offsets are
    // the same for every chunk (four registers).
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int lane_row = lane >> 4;
    const int lane_col = 8 * ((lane & 15) ^ (4 * lane_row + wave));
    int voff[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) voff[gi] = 2 * ((4 * (wave + 4 * gi) + lane_row) * WD + lane_col);
    auto chunk_rsrc = [&](const uint16_t* tensor, size_t row0, int n) TTT_INLINE {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(tensor + row0 * WD), (short)0, n * WD * 2, 0x00020000);
    };
    // copies of row group gi of this wave (one instruction per tensor)
    // (the resources are bound to locals before use: passed as temporaries straight
    // into the builtin they make the host pass drop the kernels without a diagnostic)
    // Every step issues the same number of copies, so that the waits can count them:
    // a copy of a chunk past the end of the range reads only the range's last row
    // (the other lanes are out of range) into a buffer nobody reads.  t0 < t_end.
    // (The resources are bound to locals: passed as temporaries straight into the
    // copy builtin they make the host pass drop the kernels without a diagnostic.)
    auto stage_group = [&](uint16_t* st, int t0, int gi, bool want_q, bool want_k, bool want_v) TTT_INLINE {
        const int n = min(WC, t_end - t0);
        // reversed: the chunk's rows are tensor rows T-t0-n .. T-t0-1, row r of the
        // chunk at n-1-r of the range (r >= n wraps far past it and reads zero)
        const size_t row0 = p.reverse ? seq_row + (p.T - t0 - n) : seq_row + t0;
        const int vo = p.reverse ? voff[gi] + 2 * (n - 1 - 2 * (4 * (wave_s + 4 * gi) + lane_row)) * WD : voff[gi];
        const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(p.q, row0, n);
        const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(p.k, row0, n);
        const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(p.v, row0, n);
        const int grp = wave_s + 4 * gi;
        if (want_q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (TTT_LDS void*)(tq(st) + grp * 4 * WD), 16, vo, 0, 0, 0);
        if (want_k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (TTT_LDS void*)(tk(st) + grp * 4 * WD), 16, vo, 0, 0, 0);
        if (want_v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (TTT_LDS void*)(tv(st) + grp * 4 * WD), 16, vo, 0, 0, 0);
    };
    // first row of a copy that starts at t (t_end - 1 past the end of the range)
    auto copy_start = [&](int t) TTT_INLINE { return t < t_end ? t : t_end - 1; };
    auto stage = [&](uint16_t* st, int t0, bool want_q, bool want_k, bool want_v) TTT_INLINE {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) stage_group(st, copy_start(t0), gi, want_q, want_k, want_v);
    };
    // The per-token weights of a chunk are formed by one wave (owner), lane j for
    // token j: the output pass gives the job to its fourth wave in the middle of
    // the step (it has no score tile of its own), the summary pass to wave 0.
    // rate of token `lane` of the chunk at t0
    auto load_eta = [&](int t0) TTT_INLINE {
        const int n = min(WC, t_end - t0);
        float et = p.eta_scalar;
        if (ETAV)
            et = lane < n ? (p.eta ? p.eta[seq_row + (p.reverse ? p.T - 1 - (t0 + lane) : t0 + lane)] : p.eta_scalar)
                          : 0.0f;
        return et;
    };
    // per-token weights of a chunk of n tokens entered with momentum scale r0
    auto put_weights = [&](float* w, float et, int n, float r0, int owner) TTT_INLINE {
        if (wave == owner) {
            // the table reads come before the stores
            float wm = 0.0f;
            if constexpr (MOM) wm = sBP[max(n - 1 - lane, 0)] * __builtin_amdgcn_rcpf(rho_step(r0, n));
            if (ETAV && p.eta_kind == ETA_SOFTPLUS) et = softplus_f32(et);
            if (lane >= n) et = 0.0f;
            s_wt(w)[lane] = et * inv1mb;
            if constexpr (MOM) s_wm(w)[lane] = et * wm;
        }
    };
    // the stage copies this wave issued have landed (the barrier that follows publishes them)
    auto wait_stage = [&]() TTT_INLINE { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

    // per-token weights of contraction block b in this lane's token order
    auto weights8 = [&](const float* w, int b, float* out) TTT_INLINE {
        const f32x4 a = *reinterpret_cast<const f32x4*>(w + 16 * b + 4 * hh);
        const f32x4 c = *reinterpret_cast<const f32x4*>(w + 16 * b + 8 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[e] = a[e];
            out[4 + e] = c[e];
        }
    };

    // v fragments: lane holds v[16b + slot(h, e)][32 wave + pi(n)]
    u32x4 vf[WKB];
    auto read_v = [&](uint16_t* st) TTT_INLINE {
#pragma unroll
        for (int b = 0; b < WKB; ++b) {
            const u32x2 lo = tr_read<WD>(tv(st), 16 * b + 4 * hh, col_v);
            const u32x2 hi = tr_read<WD>(tv(st), 16 * b + 8 + 4 * hh, col_v);
            vf[b] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };

    // T-part value operands w_T v (the raw fragments for a scalar rate)
    u32x4 bT[WKB];
    auto value_weights = [&](float* w) TTT_INLINE {
#pragma unroll
        for (int b = 0; b < WKB; ++b) {
            if constexpr (ETAV) {
                float x[8];
                weights8(s_wt(w), b, x);
                bT[b] = __builtin_bit_cast(u32x4, scale8(vf[b], x));
            } else {
                bT[b] = vf[b];
            }
        }
    };

    // update with the chunk in st (after read_v, value_weights):
    // T += K^T (w_T v), M = beta^n M + K^T (w_M v), as a software pipeline over the
    // four 16-token blocks: while block b's eight products run, the K fragments and
    // the M-weighted value operand of block b + 1 are prepared and a quarter of the
    // copy of the chunk at t_far into far is issued.  The copy is issued in every
    // step (far is always a free buffer); rows past the end of the segment have a
    // zero-length range and read nothing.
    auto update = [&](uint16_t* st, float* w, int n, uint16_t* far, int t_far, bool far_q) TTT_INLINE {
        if constexpr (MOM) {
            const float r = rho * sBP[n];
            if (r < RHO_MIN) {
#pragma unroll
                for (int ft = 0; ft < WFT; ++ft) Ms[ft] *= r;
                rho = 1.0f;
            } else {
                rho = r;
            }
        }
        const uint16_t* K = tk(st);
        u32x4 kf[2][WFT];
        bf16x8 bm[2];
        auto load_k = [&](int b, u32x4* dst) TTT_INLINE {
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft) {
                const u32x2 lo = tr_read<WD>(K, 16 * b + 4 * hh, col_k(ft));
                const u32x2 hi = tr_read<WD>(K, 16 * b + 8 + 4 * hh, col_k(ft));
                dst[ft] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        };
        // the M weights of all four blocks are read up front (one LDS wait)
        f32x4 wm[MOM ? WKB : 1][2];
        if constexpr (MOM) {
#pragma unroll
            for (int b = 0; b < WKB; ++b) {
                wm[b][0] = *reinterpret_cast<const f32x4*>(s_wm(w) + 16 * b + 4 * hh);
                wm[b][1] = *reinterpret_cast<const f32x4*>(s_wm(w) + 16 * b + 8 + 4 * hh);
            }
        }
        auto m_operand = [&](int b) TTT_INLINE {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = wm[b][0][e];
                x[4 + e] = wm[b][1][e];
            }
            return scale8(vf[b], x);
        };
        const int t_src = copy_start(t_far);
        load_k(0, kf[0]);
        if constexpr (MOM) bm[0] = m_operand(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < WKB; ++b) {
            if (b + 1 < WKB) {
                load_k(b + 1, kf[(b + 1) & 1]);
                if constexpr (MOM) bm[(b + 1) & 1] = m_operand(b + 1);
            }
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft) {
                const bf16x8 a = as_bf16x8(kf[b & 1][ft]);
                Ts[ft] = mfma32(a, as_bf16x8(bT[b]), Ts[ft]);
                if constexpr (MOM) Ms[ft] = mfma32(a, bm[b & 1], Ms[ft]);
            }
            // interleave: each product followed by LDS reads and vector work of the next block
            if (b + 1 < WKB) {
#pragma unroll
                for (int i = 0; i < (MOM ? 8 : 4); ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, MOM ? 2 : 3, 0);   // LDS reads
                    __builtin_amdgcn_sched_group_barrier(0x002, MOM ? 3 : 1, 0);   // VALU
                }
            }
            // the copy instructions end a scheduling region: issue them after the block
            stage_group(far, t_src, b, far_q, true, true);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // q fragment: B operand Q^T[feature 16 kb + 8h + e][token 32 I + n]
    auto q_frag = [&](uint16_t* st, int I, int kb) TTT_INLINE {
        return as_bf16x8(lds_read16(tq(st) + swz<WD>(32 * I + n32, 16 * kb + 8 * hh)));
    };

    // readout of the chunk's queries from the state entering it
    auto readout = [&](uint16_t* st, f32x16* oT, f32x16* oM, bool with_m) TTT_INLINE {
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            oT[I] = f32x16{};
            if constexpr (MOM) oM[I] = f32x16{};
        }
#pragma unroll
        for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8 b0 = q_frag(st, 0, 2 * ft + kh);
                const bf16x8 b1 = q_frag(st, 1, 2 * ft + kh);
                const bf16x8 aT = pack_half(Ts[ft], kh);
                oT[0] = mfma32(aT, b0, oT[0]);
                oT[1] = mfma32(aT, b1, oT[1]);
                if constexpr (MOM) {
                    if (with_m) {
                        const bf16x8 aM = pack_half(Ms[ft], kh);
                        oM[0] = mfma32(aM, b0, oM[0]);
                        oM[1] = mfma32(aM, b1, oM[1]);
                    }
                }
            }
    };

    // one output tile: lane holds o[i = 32I + n][32 wave + 16h + r], r = 0..15
    auto store = [&](const f32x16& o, int I, int n, size_t row0) TTT_INLINE {
        const int i = 32 * I + n32;
        if (i < n) {
            // row0 = seq_row + t0; reversed: tensor row T-1-(t0+i)
            const size_t orow = p.reverse ? 2 * seq_row + (p.T - 1) - row0 - i : row0 + i;
            uint16_t* dst = p.o + orow * WD + 32 * wave + 16 * hh;
            const u32x4 lo = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])};
            const u32x4 hi = {pack_bf16x2(o[8], o[9]), pack_bf16x2(o[10], o[11]), pack_bf16x2(o[12], o[13]),
                              pack_bf16x2(o[14], o[15])};
            *reinterpret_cast<u32x4*>(dst) = lo;
            *reinterpret_cast<u32x4*>(dst + 8) = hi;
        }
    };

    __syncthreads();   // coefficient tables

    // ---- output pass over the segment from its entry state (slot seg - 1) ----
    auto output_pass = [&]() TTT_INLINE {
        // score coefficients: c_{i-j} times (1 - beta) when the rate is folded into
        // the value operand, else times the scalar rate; 0 above the diagonal
        const float k0 = ETAV ? (1.0f - beta) : p.eta_scalar;
        if (tid < 2 * WC) sK[tid] = tid >= WC ? k0 * sC[tid - WC] : 0.0f;
        // score tile of waves 0..2: (J, I) = (0,0), (0,1), (1,1); the fourth wave repeats (1,1).
        // Register r holds j = 32 sJ + 8 (r / 4) + 4h + r % 4 of token i = 32 sI + n.
        const int sJ = (wave >= 2) ? 1 : 0;
        const int sI = (wave == 0) ? 0 : 1;
        // one offset added to the array base: the compiler tags an LDS access with its
        // array only through a short chain of address steps, and an untagged read has
        // to wait for every copy in flight
        const float* coef = sK + (WC + 32 * (sI - sJ) + n32 - 4 * hh);   // coef[-off_r]
        // M readout weight of token i: -beta^{i+2} / (1 - beta)
        float gam[2];
#pragma unroll
        for (int I = 0; I < 2; ++I) gam[I] = MOM ? -beta * beta * sBP[32 * I + n32] * inv1mb : 0.0f;

        // prologue: chunk 0, the entry state, then chunk 1 (the first step waits for
        // everything but chunk 1)
        const bool two = t_begin + WC < t_end;
        stage(stage_a, t_begin, true, true, true);
        const float et0 = load_eta(t_begin);
        // the rate of chunk c + 1 is loaded a step ahead, before the copies of that
        // step, so that reading it never waits for a copy in flight
        float et_ahead = two ? load_eta(t_begin + WC) : 0.0f;
        const bool slot_entry = KIND != W_PREFIX && (seg > 0 || (p.has_init && p.seg_count > 1));
        if (slot_entry) {
            const f32x4* src = slot_ptr(seg * p.entry_split);
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 t = src[(((size_t)wave * WFT + ft) * 4 + r4) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) Ts[ft][4 * r4 + e] = t[e];
                    if constexpr (MOM) {
                        const f32x4 m = src[HALF_F4 + (((size_t)wave * WFT + ft) * 4 + r4) * 64 + lane];
#pragma unroll
                        for (int e = 0; e < 4; ++e) Ms[ft][4 * r4 + e] = m[e];
                    }
                }
        } else if (KIND == W_OUTPUT && p.has_init) {
            // one segment: the entry state straight from the caller's layout,
            // T = S0 + kappa M0 (the carried-state calls use the per-token weights
            // of the value operand, t_scale = 1)
            const float kappa = beta * inv1mb;
            const float* s0 = p.S0 ? p.S0 + (size_t)seq * WD * WD + (size_t)user_vcol(wave, lane) * WD : nullptr;
            const float* m0 = p.M0 ? p.M0 + (size_t)seq * WD * WD + (size_t)user_vcol(wave, lane) * WD : nullptr;
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int f0 = user_f0(ft, r4, lane);
                    const f32x4 sv = s0 ? *reinterpret_cast<const f32x4*>(s0 + f0) : f32x4{0.f, 0.f, 0.f, 0.f};
                    const f32x4 mv = m0 ? *reinterpret_cast<const f32x4*>(m0 + f0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Ts[ft][4 * r4 + e] = fmaf(kappa, mv[e], sv[e]);
                        if constexpr (MOM) Ms[ft][4 * r4 + e] = mv[e];
                    }
                }
        }
        if (two) stage(stage_b, t_begin + WC, true, true, true);
        put_weights(w_a, et0, min(WC, t_end - t_begin), rho, 3);
        if (two) __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); else wait_stage();   // chunk 0 landed
        lds_barrier();

        // Chunk c, staged in cur with weights wc.  Chunk c + 1 is in flight (its
        // weights go to wn before the middle barrier); the copy of chunk c + 2 into
        // far is issued during the update.
        auto step = [&](uint16_t* cur, float* wc, float* wn, uint16_t* far, int t0) TTT_INLINE -> bool {
            const int n = min(WC, t_end - t0);
            const size_t row0 = seq_row + t0;
            const bool has_next = t0 + WC < t_end;
            const bool has_far = t0 + 2 * WC < t_end;
            float cf[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) cf[r] = coef[-(8 * (r >> 2) + (r & 3))];
            const float et_next = et_ahead;
            et_ahead = has_far ? load_eta(t0 + 2 * WC) : 0.0f;

            // Score tile S^T = K Q^T of this wave and the readout from the entering
            // state, in one loop: the score products (a chain on one accumulator) are
            // spread between the 32 independent readout products.  The fourth wave
            // computes the third wave's tile too (it would wait at the barrier
            // anyway) and does not write it.
            f32x16 o[2];
            {
                f32x16 oT[2], oM[2], acc = f32x16{};
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    oT[I] = f32x16{};
                    if constexpr (MOM) oM[I] = f32x16{};
                }
#pragma unroll
                for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {
                        const int kb = 2 * ft + kh;
                        const bf16x8 b0 = q_frag(cur, 0, kb);
                        const bf16x8 b1 = q_frag(cur, 1, kb);
                        const bf16x8 bs = q_frag(cur, sI, kb);
                        const bf16x8 ks = as_bf16x8(lds_read16(tk(cur) + swz<WD>(32 * sJ + n32, 16 * kb + 8 * hh)));
                        const bf16x8 aT = pack_half(Ts[ft], kh);
                        oT[0] = mfma32(aT, b0, oT[0]);
                        oT[1] = mfma32(aT, b1, oT[1]);
                        acc = mfma32(ks, bs, acc);
                        if constexpr (MOM) {
                            const bf16x8 aM = pack_half(Ms[ft], kh);
                            oM[0] = mfma32(aM, b0, oM[0]);
                            oM[1] = mfma32(aM, b1, oM[1]);
                        }
                    }
                // scaled score fragments to LDS; readout combined:
                // t_scale T q - beta^{i+2}/(1-beta) M q
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] *= cf[r];
                if (wave < 3) {
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh)
                        P_lds[(wave * 2 + kh) * 64 + lane] = __builtin_bit_cast(u32x4, pack_half(acc, kh));
                }
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    const float gI = gam[I] * rho;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float x = oT[I][r] * t_scale;
                        if constexpr (MOM) x = fmaf(gI, oM[I][r], x);
                        o[I][r] = x;
                    }
                }
            }
            // the weighted value fragments do not depend on the scores
            read_v(cur);
            value_weights(wc);
            // the weights of the next chunk (its buffer's previous chunk is long done),
            // published by the barrier below; the momentum scale they divide by is rho
            // after this chunk's update and the next one's, predicted the way the
            // update takes it
            if (has_next) put_weights(wn, et_next, min(WC, t_end - (t0 + WC)), rho_step(rho, n), 3);
            lds_barrier();   // every wave's score fragments

            // intra-chunk term with the weighted value fragments (every score
            // fragment read first), then the store
            u32x4 pf[6];
#pragma unroll
            for (int f = 0; f < 6; ++f) pf[f] = P_lds[f * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                // blocks 0, 1 from tile (0, I); blocks 2, 3 from tile (1, 1)
#pragma unroll
                for (int b = 0; b < 2 * (I + 1); ++b) {
                    const int tile = (b < 2) ? I : 2;
                    o[I] = mfma32(as_bf16x8(bT[b]), as_bf16x8(pf[tile * 2 + (b & 1)]), o[I]);
                }
                store(o[I], I, n, row0);
            }
            __builtin_amdgcn_sched_barrier(0);
            update(cur, wc, n, far, t0 + 2 * WC, true);
            if (!has_next) return false;
            // chunk c + 1 landed; the 12 copies of chunk c + 2 may still be in flight
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
            lds_barrier();
            return true;
        };
        for (int t0 = t_begin;; t0 += 3 * WC) {
            if (!step(stage_a, w_a, w_b, stage_c, t0)) break;
            if (!step(stage_b, w_b, w_c, stage_a, t0 + WC)) break;
            if (!step(stage_c, w_c, w_a, stage_b, t0 + 2 * WC)) break;
        }
        wait_stage();   // the last (empty) copies
    };

    // ---- summary pass: three stage buffers, k, v copied two chunks ahead ----
    auto summary_pass = [&]() TTT_INLINE {
        auto issue_kv = [&](uint16_t* st, int t0) TTT_INLINE { stage(st, t0, false, true, true); };   // 8 copies
        // chunk t0 + WC landed; the copies of chunk t0 + 2 WC (8, some possibly empty) may
        // still be in flight
        auto wait_kv = [&]() TTT_INLINE { __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); };
        issue_kv(stage_a, t_begin);
        issue_kv(stage_b, t_begin + WC);
        put_weights(w_a, load_eta(t_begin), min(WC, t_end - t_begin), rho, 0);
        wait_kv();
        lds_barrier();
        auto step = [&](uint16_t* cur, float* wc, float* wn, uint16_t* far, int t0) TTT_INLINE -> bool {
            const int n = min(WC, t_end - t0);
            const bool has_next = t0 + WC < t_end;
            const float et_next = has_next ? load_eta(t0 + WC) : 0.0f;
            read_v(cur);
            value_weights(wc);
            update(cur, wc, n, far, t0 + 2 * WC, false);
            if (!has_next) return false;
            put_weights(wn, et_next, min(WC, t_end - (t0 + WC)), rho, 0);
            wait_kv();
            lds_barrier();
            return true;
        };
        for (int t0 = t_begin;; t0 += 3 * WC) {
            if (!step(stage_a, w_a, w_b, stage_c, t0)) break;
            if (!step(stage_b, w_b, w_c, stage_a, t0 + WC)) break;
            if (!step(stage_c, w_c, w_a, stage_b, t0 + 2 * WC)) break;
        }
        wait_stage();   // the last (empty) copies
    };

    auto write_summary = [&](f32x4* dst) TTT_INLINE {
#pragma unroll
        for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                dst[(((size_t)wave * WFT + ft) * 4 + r4) * 64 + lane] =
                    f32x4{Ts[ft][4 * r4], Ts[ft][4 * r4 + 1], Ts[ft][4 * r4 + 2], Ts[ft][4 * r4 + 3]};
                if constexpr (MOM)
                    dst[HALF_F4 + (((size_t)wave * WFT + ft) * 4 + r4) * 64 + lane] =
                        f32x4{rho * Ms[ft][4 * r4], rho * Ms[ft][4 * r4 + 1], rho * Ms[ft][4 * r4 + 2],
                              rho * Ms[ft][4 * r4 + 3]};
            }
    };

    if constexpr (KIND == W_OUTPUT) {
        output_pass();
        if (seg == p.seg_count - 1 && (p.S_T || p.M_T)) {
            // the state after the last token in the caller's layout:
            // S = t_scale T - kappa M, M = rho Ms
            const float kappa = beta * inv1mb;
            const size_t row = (size_t)seq * WD * WD + (size_t)user_vcol(wave, lane) * WD;
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int f0 = user_f0(ft, r4, lane);
                    f32x4 sv, mv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        mv[e] = MOM ? rho * Ms[ft][4 * r4 + e] : 0.0f;
                        sv[e] = fmaf(-kappa, mv[e], t_scale * Ts[ft][4 * r4 + e]);
                    }
                    if (p.S_T) *reinterpret_cast<f32x4*>(p.S_T + row + f0) = sv;
                    if (p.M_T) *reinterpret_cast<f32x4*>(p.M_T + row + f0) = mv;
                }
        }
    } else if constexpr (KIND == W_PREFIX) {
        // entry state from zero over all earlier tokens (an update-only pass), then
        // the segment's outputs
        const int s0 = t_begin, s1 = t_end;
        if (s0 > 0) {
            t_begin = 0;
            t_end = s0;
            summary_pass();
            __syncthreads();   // every wave is done with the stage buffers and weights
            t_begin = s0;
            t_end = s1;
        }
        output_pass();
    } else if constexpr (KIND == W_FUSED) {
        // 1. zero-entry summary of this segment (every segment but the last)
        if (seg < p.seg_count - 1) {
            summary_pass();
            write_summary(slot_ptr(seg + 1));
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft) Ts[ft] = f32x16{};
#pragma unroll
            for (int ft = 0; ft < (MOM ? WFT : 1); ++ft) Ms[ft] = f32x16{};
            rho = 1.0f;
        }
        // 2. the sequence's summaries are written: scan them, each workgroup one slice
        unsigned* cnt = p.counters + 2 * (size_t)seq;
        const unsigned target = p.epoch * (unsigned)p.seg_count;
        seq_sync(cnt, target, p.spin_limit, p.wait_failed);
        {
            // this workgroup's slice of the float4s of a slot (T, then M with momentum),
            // every step's summary loaded before the first add: at most 32 loads per thread
            const int steps = p.seg_count - 1;
            const int total = (MOM ? 2 : 1) * (int)HALF_F4;
            const int per = (total + p.seg_count - 1) / p.seg_count;
            const int e0 = seg * per, e1 = min(total, e0 + per);
            const int n_el = (e1 - e0 + WNT - 1) / WNT;          // elements per thread
            const float bL = p.beta_seg;
            f32x4* base = slot_ptr(1);
            constexpr int MAXL = 32;
            const int batch = max(1, MAXL / steps);               // elements per round of loads
            for (int eb = 0; eb < n_el; eb += batch) {
            f32x4 d[MAXL];
#pragma unroll
            for (int j = 0; j < MAXL; ++j) {
                const int ei = eb + j / steps, st = j % steps;
                const int e = e0 + tid + ei * WNT;
                // unconditional loads (an unused one reads element e0), so that all of
                // them are in flight together instead of one branch at a time
                const bool ok = j / steps < batch && ei < n_el && e < e1;
                d[j] = base[(size_t)st * 2 * HALF_F4 + (ok ? e : e0)];
            }
#pragma unroll
            for (int j = 0; j < MAXL; ++j) {
                const int ei = eb + j / steps, st = j % steps;
                const int e = e0 + tid + ei * WNT;
                if (j / steps < batch && ei < n_el && e < e1) {
                    // running prefix of element ei lives in d[j]: add the previous step's
                    if (st > 0) {
                        if (e >= (int)HALF_F4) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) d[j][r] = fmaf(bL, d[j - 1][r], d[j][r]);
                        } else {
                            d[j] += d[j - 1];
                        }
                    }
                    base[(size_t)st * 2 * HALF_F4 + e] = d[j];
                }
            }
            }
        }
        // 3. entry states are complete: the output pass
        seq_sync(cnt + 1, target, p.spin_limit, p.wait_failed);
        output_pass();
    } else {
        // SUMMARY: zero-entry state change of the segment.  BIDIR: the same over
        // the whole sequence, then every query reads S = t_scale T - kappa M.
        summary_pass();
        if constexpr (KIND == W_SUMMARY) {
            f32x4* dst = slot_ptr(seg + 1);
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    dst[(((size_t)wave * WFT + ft) * 4 + r4) * 64 + lane] =
                        f32x4{Ts[ft][4 * r4], Ts[ft][4 * r4 + 1], Ts[ft][4 * r4 + 2], Ts[ft][4 * r4 + 3]};
                    if constexpr (MOM)
                        dst[HALF_F4 + (((size_t)wave * WFT + ft) * 4 + r4) * 64 + lane] =
                            f32x4{rho * Ms[ft][4 * r4], rho * Ms[ft][4 * r4 + 1], rho * Ms[ft][4 * r4 + 2],
                                  rho * Ms[ft][4 * r4 + 3]};
                }
        } else {
            const float kappa = beta * inv1mb * rho;
#pragma unroll
            for (int ft = 0; ft < WFT; ++ft)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = Ts[ft][r] * t_scale;
                    if constexpr (MOM) x = fmaf(-kappa, Ms[ft][r], x);
                    Ts[ft][r] = x;
                }
            __syncthreads();   // every wave is done with the stage buffers
            // queries: three buffers, copies two chunks ahead (4 per chunk and wave)
            auto issue_q = [&](uint16_t* st, int t0) TTT_INLINE { if (t0 < t_end) stage(st, t0, true, false, false); };
            auto wait_q = [&](int t0) TTT_INLINE {
                if (t0 + 2 * WC < t_end) __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); else wait_stage();
            };
            issue_q(stage_a, 0);
            issue_q(stage_b, WC);
            wait_q(-WC);
            lds_barrier();
            auto qstep = [&](uint16_t* cur, uint16_t* far, int t0) TTT_INLINE -> bool {
                const int n = min(WC, t_end - t0);
                const size_t row0 = seq_row + t0;
                const bool has_next = t0 + WC < t_end;
                issue_q(far, t0 + 2 * WC);
                f32x16 oT[2], oM[2];
                readout(cur, oT, oM, false);
#pragma unroll
                for (int I = 0; I < 2; ++I) store(oT[I], I, n, row0);
                if (!has_next) return false;
                wait_q(t0);
                lds_barrier();
                return true;
            };
            for (int t0 = 0;; t0 += 3 * WC) {
                if (!qstep(stage_a, stage_c, t0)) break;
                if (!qstep(stage_b, stage_a, t0 + WC)) break;
                if (!qstep(stage_c, stage_b, t0 + 2 * WC)) break;
            }
        }
    }
}

// Composes segment summaries into entry states, in place, per sequence:
//   (T, M) = entry state of segment 0 (the carried state if has_init, else 0),
//   then for s = 1 .. n_slots - 1:  T <- T + dT,  M <- beta^L M + dM,
//   slot s <- (T, M) = entry state of segment s.
// With has_init the carried state is read from the caller's layout, put in the
// T-form T = S0 + kappa M0 and also written to slot 0 (so that the output kernel
// never reads S0, M0: they may be the buffers the final state goes to).  One
// thread per float4 of one sequence's state; all summaries are loaded before
// the first store so that the loads overlap.
// mmode: 0 no momentum; 1 compose M; 2 beta^L is below 2^-30, so the carried
// term beta^L M is below the fp32 resolution of dM and every entry M is the
// previous segment's dM, already in its slot (only a carried M0 is written).
template <int MAXS>
__global__ void __launch_bounds__(256) wide_scan(float* state, int n_seq, int n_slots, float bL, int mmode,
                                                 const float* S0, const float* M0, float kappa, int has_init) {
    const bool mom = mmode == 1;
    constexpr int HALF = WNW * WFT * 4 * 64;       // float4s of T (and of M) per slot
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n_seq * HALF) return;
    const size_t seqi = idx / HALF;
    const int e = (int)(idx % HALF);
    f32x4* base = reinterpret_cast<f32x4*>(state) + seqi * n_slots * 2 * HALF + e;
    const int n_steps = n_slots - 1;
    f32x4 dT[MAXS], dM[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        if (s < n_steps) {
            dT[s] = base[(size_t)(s + 1) * 2 * HALF];
            if (mom) dM[s] = base[(size_t)(s + 1) * 2 * HALF + HALF];
        }
    }
    f32x4 T = {0.f, 0.f, 0.f, 0.f}, M = {0.f, 0.f, 0.f, 0.f};
    if (has_init) {
        // element e = ((wave * WFT + ft) * 4 + r4) * 64 + lane of the register tiles
        const int lane = e & 63, r4 = (e >> 6) & 3, ft = (e >> 8) % WFT, w = (e >> 8) / WFT;
        const size_t off = seqi * WD * WD + (size_t)user_vcol(w, lane) * WD + user_f0(ft, r4, lane);
        const f32x4 sv = S0 ? *reinterpret_cast<const f32x4*>(S0 + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (M0) M = *reinterpret_cast<const f32x4*>(M0 + off);
#pragma unroll
        for (int r = 0; r < 4; ++r) T[r] = fmaf(kappa, M[r], sv[r]);
        base[0] = T;
        if (mmode != 0) base[HALF] = M;
    }
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        if (s < n_steps) {
            T += dT[s];
            base[(size_t)(s + 1) * 2 * HALF] = T;
            if (mom) {
#pragma unroll
                for (int r = 0; r < 4; ++r) M[r] = fmaf(bL, M[r], dM[s][r]);
                base[(size_t)(s + 1) * 2 * HALF + HALF] = M;
            }
        }
    }
}

// With events, the launch carries them (hipExtLaunchKernel): they take their
// timestamps at the start and end of the kernel itself, not around its dispatch.
template <bool MOM, bool ETAV, int KIND>
hipError_t launch_wide_one(const WideParams& wp, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
    const int grid = (wp.n_units + 7) / 8 * 8;
    if (ev_begin || ev_end) {
        WideParams a = wp;
        void* args[] = {&a};
        return hipExtLaunchKernel(reinterpret_cast<const void*>(wide_kernel<MOM, ETAV, KIND>), dim3(grid), dim3(WNT),
                                  args, 0, st, ev_begin, ev_end, 0);
    }
    hipLaunchKernelGGL((wide_kernel<MOM, ETAV, KIND>), dim3(grid), dim3(WNT), 0, st, wp);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_wide_kind(bool mom, bool etav, const WideParams& wp, hipStream_t st, hipEvent_t ev_begin = nullptr,
                            hipEvent_t ev_end = nullptr) {
    if (mom)
        return etav ? launch_wide_one<true, true, KIND>(wp, st, ev_begin, ev_end)
                    : launch_wide_one<true, false, KIND>(wp, st, ev_begin, ev_end);
    return etav ? launch_wide_one<false, true, KIND>(wp, st, ev_begin, ev_end)
                : launch_wide_one<false, false, KIND>(wp, st, ev_begin, ev_end);
}

}  // namespace

int wide_fused_capacity() {
    static int cached = -1;
    if (cached >= 0) return cached;
    int dev = 0, coop = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, wide_kernel<true, true, W_FUSED>, WNT, 0) !=
            hipSuccess) {
        (void)hipGetLastError();
        return cached = 0;
    }
    return cached = coop ? per_cu * cus : 0;
}

// The scan over n_slots slots per sequence of summaries of seg_len tokens each
// (slot 0: the carried state when has_init).
static hipError_t launch_scan(const Shape& s, float* state, int n_slots, int seg_len, const FwdArgs& a, bool mom,
                              int has_init, hipStream_t st) {
    constexpr int HALF = WNW * WFT * 4 * 64;
    const size_t n_threads = (size_t)s.n_seq() * HALF;
    const float bL = (float)std::pow((double)a.beta, (double)seg_len);
    const float kappa = a.beta / (1.0f - a.beta);
    const int mmode = !mom ? 0 : (bL < 0x1p-30f ? 2 : 1);
    const dim3 grid((unsigned)((n_threads + 255) / 256));
    if (n_slots - 1 <= 7)
        hipLaunchKernelGGL(wide_scan<7>, grid, dim3(256), 0, st, state, s.n_seq(), n_slots, bL, mmode, a.S0, a.M0,
                           kappa, has_init);
    else
        hipLaunchKernelGGL(wide_scan<15>, grid, dim3(256), 0, st, state, s.n_seq(), n_slots, bL, mmode, a.S0, a.M0,
                           kappa, has_init);
    return hipGetLastError();
}

size_t wide_zero_bytes(const Shape& s) {
    // two counters per sequence and the wait-failed flag
    return ((size_t)(2 * s.n_seq() + 1) * sizeof(unsigned) + 255) / 256 * 256;
}

size_t wide_flag_offset(const Shape& s, const FastPlan& p) {
    return p.summary_bytes + (size_t)2 * s.n_seq() * sizeof(unsigned);
}

bool wide_supported(const Shape& s) {
    return s.bf16 && !s.swiglu && s.d_k == WD && s.d_v == WD && s.d_phi == WD;
}

size_t wide_summary_bytes(const Shape& s, int segments) {
    // one slot per segment: the summaries of segments 0 .. S-2 (then the entry
    // states of segments 1 .. S-1) and the carried entry state of segment 0
    if (segments <= 1) return 0;
    return (size_t)s.n_seq() * segments * 2 * WD * WD * sizeof(float);
}

int wide_max_segments() { return 16; }

void wide_prefix_bounds(int T, int S, int* bounds) {
    // equal chunk-aligned segments
    const int n_chunks = (T + WC - 1) / WC;
    const int per = (n_chunks + S - 1) / S;
    for (int i = 0; i <= S; ++i) bounds[i] = std::min(T, i * per * WC);
}

hipError_t launch_wide(const Shape& s, const FastPlan& p, void* workspace, const FwdArgs& a, hipEvent_t ev_begin,
                       hipEvent_t ev_end, int* n_kernels) {
    WideParams wp{};
    wp.q = static_cast<const uint16_t*>(a.q);
    wp.k = static_cast<const uint16_t*>(a.k);
    wp.v = static_cast<const uint16_t*>(a.v);
    wp.eta = a.eta;
    wp.o = static_cast<uint16_t*>(a.o);
    wp.state = static_cast<float*>(workspace);
    wp.eta_scalar = a.eta_scalar;
    wp.beta = a.beta;
    wp.eta_kind = a.eta_kind;
    wp.T = s.T;
    // A carried state (in or out) takes the kernels with per-token value weights
    // (a scalar rate is then read as a constant per-token rate, so that the state
    // needs no 1 / eta), and the momentum kernels whenever M_T is asked for.
    const bool state_io = a.S0 || a.M0 || a.S_T || a.M_T;
    const bool mom = a.beta != 0.0f || a.M_T;
    const bool etav = a.eta_kind != ETA_SCALAR || state_io;
    wp.S0 = a.S0;
    wp.M0 = a.M0;
    wp.S_T = a.S_T;
    wp.M_T = a.M_T;
    wp.has_init = (a.S0 || a.M0) ? 1 : 0;
    wp.reverse = a.reverse ? 1 : 0;
    if (a.reverse && (state_io || a.bidirectional)) return hipErrorInvalidValue;
    wp.beta_seg = (float)std::pow((double)a.beta, (double)p.seg_len);
    wp.slot_count = p.segments;
    wp.entry_split = 1;
    hipStream_t st = a.stream;
    hipError_t e = hipSuccess;
    int nk = 0;
    if (!a.bidirectional && p.fused && !state_io) {
        char* z = static_cast<char*>(workspace) + p.summary_bytes;
        wp.seg_count = p.segments;
        wp.seg_len = p.seg_len;
        wp.n_units = s.n_seq() * p.segments;
        wp.counters = reinterpret_cast<unsigned*>(z);
        wp.wait_failed = wp.counters + 2 * s.n_seq();
        wp.epoch = a.epoch;
        wp.spin_limit = 1u << 20;
        const int grid = (wp.n_units + 7) / 8 * 8;
        void* args[] = {&wp};
        const void* fn = mom ? (etav ? (const void*)wide_kernel<true, true, W_FUSED>
                                     : (const void*)wide_kernel<true, false, W_FUSED>)
                             : (etav ? (const void*)wide_kernel<false, true, W_FUSED>
                                     : (const void*)wide_kernel<false, false, W_FUSED>);
        if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
        e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(WNT), args, 0, st);
        if (e == hipSuccess) {
            if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
            if (n_kernels) *n_kernels = 1;
            return hipSuccess;
        }
        // Only "the grid cannot be made resident right now" sends the caller to the
        // three-kernel path (it then does not advance the epoch: no workgroup of this
        // launch ran); any other launch error is the caller's error.
        (void)hipGetLastError();
        return e;
    }
    if (!a.bidirectional && p.prefix && !state_io) {
        wp.seg_count = p.segments;
        wp.seg_len = p.seg_len;
        for (int i = 0; i <= p.segments; ++i) wp.bounds[i] = p.bounds[i];
        wp.n_units = s.n_seq() * p.segments;
        if ((e = launch_wide_kind<W_PREFIX>(mom, etav, wp, st, ev_begin, ev_end)) != hipSuccess) return e;
        if (n_kernels) *n_kernels = 1;
        return hipSuccess;
    }
    if (a.bidirectional) {
        wp.seg_count = 1;
        wp.seg_len = s.T;
        wp.n_units = s.n_seq();
        if ((e = launch_wide_kind<W_BIDIR>(mom, etav, wp, st, ev_begin, ev_end)) != hipSuccess) return e;
        ++nk;
    } else {
        wp.seg_count = p.segments;
        wp.seg_len = p.seg_len;
        if (p.segments == 2 && p.sum_split == 2) {
            // summaries of the two halves of segment 0 into slots 1 and 2 (three slots
            // per sequence, slot 0 the carried state), scanned over the half length:
            // segment 1 enters with slot 2
            WideParams sp = wp;
            sp.seg_count = 3;
            sp.seg_len = p.seg_len / 2;
            sp.slot_count = 3;
            sp.n_units = s.n_seq() * 2;
            if ((e = launch_wide_kind<W_SUMMARY>(mom, etav, sp, st)) != hipSuccess) return e;
            if ((e = launch_scan(s, wp.state, 3, sp.seg_len, a, mom, wp.has_init, st)) != hipSuccess) return e;
            nk += 2;
            wp.slot_count = 3;
            wp.entry_split = 2;
        } else if (p.segments > 1) {
            wp.n_units = s.n_seq() * (p.segments - 1);
            if ((e = launch_wide_kind<W_SUMMARY>(mom, etav, wp, st)) != hipSuccess) return e;
            ++nk;
            // with two segments and no carried state the one summary already is the
            // entry state of segment 1
            if (p.segments > 2 || wp.has_init) {
                if ((e = launch_scan(s, wp.state, p.segments, p.seg_len, a, mom, wp.has_init, st)) != hipSuccess)
                    return e;
                ++nk;
            }
        }
        wp.n_units = s.n_seq() * p.segments;
        if ((e = launch_wide_kind<W_OUTPUT>(mom, etav, wp, st, ev_begin, ev_end)) != hipSuccess) return e;
        ++nk;
    }
    if (n_kernels) *n_kernels = nk;
    return hipSuccess;
}

}  // namespace ttt
