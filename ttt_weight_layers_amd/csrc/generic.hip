// Generic chunked TTT / linear-attention forward with fp32 arithmetic.
//
// One workgroup owns one sequence (b, h) and 16 value columns of its fast
// weight (a d_phi x 16 slice of S and M, kept in LDS), and walks the sequence
// chunk by chunk (16 tokens).  Per chunk of n tokens entered with (S, M):
//
//   o_i = S phi(q_i) + g_i M phi(q_i) + sum_{j<=i} c_{i-j} eta_j (phi(q_i).phi(k_j)) v_j
//   S  <- S + g_{n-1} M + sum_j eta_j c_{n-1-j} v_j phi(k_j)^T
//   M  <- beta^n M + sum_j eta_j beta^{n-1-j} v_j phi(k_j)^T
//
// with c_r = sum_{u<=r} beta^u and g_i = beta c_i.  This is the unrolled form
// of one momentum-SGD step per token on the dot-product binding loss, i.e.
// the outer-product accumulation that the kualia.ai blog ("The Linear
// Attention Equivalence") equates with linear attention and says can be
// computed in parallel; the per-token learning rate and momentum are the
// Variant 3/4 inner-loop options of Table 2 on the thelatestinai.com page.
//
// This path serves fp32 inputs (where bf16 tensor-core arithmetic would not
// meet an fp32 error budget) and any shape the MFMA path does not cover.
// It is plain vector-ALU code: correctness first, adequate speed.

#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace ttt {
namespace {

constexpr int GC = 16;        // tokens per chunk
constexpr int GDV = 16;       // value columns per workgroup
constexpr int GTHREADS = 256; // GC * GDV

struct GenericParams {
    const void* q;
    const void* k;
    const void* v;
    const float* eta;
    const void* w1;
    const void* w3;
    void* o;
    float eta_scalar;
    float beta;
    int eta_kind;
    int T, H, d_k, d_v, d_phi;
    int n_dvblk;
    // carried state, fp32 [seq][d_v][d_phi] (causal only; null: zero entry state /
    // final state not written).  A workgroup reads and writes only its own 16
    // value rows, so the final state may overwrite the entry state in place.
    const float* S0;
    const float* M0;
    float* S_T;
    float* M_T;
};

// LDS layout (floats):
//   S[d_phi][GDV], M[d_phi][GDV], Pq[GC][d_phi], Pk[GC][d_phi], Xq[GC][d_k], Xk[GC][d_k],
//   V[GC][GDV], A[GC][GC], eta[GC], wS[GC], wM[GC], c[GC], bp[GC + 1]
__host__ __device__ inline size_t generic_smem_floats(int d_k, int d_phi, bool swiglu) {
    size_t n = 2 * (size_t)d_phi * GDV + 2 * (size_t)GC * d_phi + (size_t)GC * GDV + GC * GC + 5 * GC + 1;
    if (swiglu) n += 2 * (size_t)GC * d_k;
    return n;
}

// Loads the features of rows [t0, t0 + n) of x (sequence seq) into P[GC][d_phi]
// (rows >= n are zero).  For SwiGLU the raw rows are staged in X first.
template <typename TI, bool SWIGLU>
__device__ void load_features(const TI* x, const TI* w1, const TI* w3, float* P, float* X, size_t row0,
                              int n, int d_k, int d_phi) {
    const int tid = threadIdx.x;
    if (!SWIGLU) {
        for (int idx = tid; idx < GC * d_phi; idx += GTHREADS) {
            int r = idx / d_phi, f = idx % d_phi;
            P[idx] = r < n ? load_as_f32(x, (row0 + r) * d_k + f) : 0.0f;
        }
        return;
    }
    for (int idx = tid; idx < GC * d_k; idx += GTHREADS) {
        int r = idx / d_k, d = idx % d_k;
        X[idx] = r < n ? load_as_f32(x, (row0 + r) * d_k + d) : 0.0f;
    }
    __syncthreads();
    for (int idx = tid; idx < GC * d_phi; idx += GTHREADS) {
        int r = idx / d_phi, f = idx % d_phi;
        float u = 0.0f, g = 0.0f;
        if (r < n) {
            const float* xr = X + r * d_k;
            for (int d = 0; d < d_k; ++d) {
                float xv = xr[d];
                u = fmaf(load_as_f32(w1, (size_t)f * d_k + d), xv, u);
                g = fmaf(load_as_f32(w3, (size_t)f * d_k + d), xv, g);
            }
        }
        P[idx] = r < n ? silu_f32(u) * g : 0.0f;
    }
}

template <typename TI, bool SWIGLU>
__global__ void __launch_bounds__(GTHREADS) generic_forward(GenericParams p) {
    extern __shared__ float smem[];
    const int d_phi = p.d_phi, d_k = p.d_k;
    float* sS = smem;
    float* sM = sS + d_phi * GDV;
    float* sPq = sM + d_phi * GDV;
    float* sPk = sPq + GC * d_phi;
    float* sV = sPk + GC * d_phi;
    float* sA = sV + GC * GDV;
    float* sEta = sA + GC * GC;
    float* sWS = sEta + GC;
    float* sWM = sWS + GC;
    float* sC = sWM + GC;
    float* sBP = sC + GC;          // GC + 1 entries
    float* sXq = sBP + GC + 1;     // SwiGLU staging
    float* sXk = sXq + GC * d_k;

    const int tid = threadIdx.x;
    const int seq = blockIdx.x / p.n_dvblk;
    const int dv0 = (blockIdx.x % p.n_dvblk) * GDV;
    const int h = seq % p.H;
    const int T = p.T;
    const float beta = p.beta;

    const TI* q = static_cast<const TI*>(p.q);
    const TI* k = static_cast<const TI*>(p.k);
    const TI* v = static_cast<const TI*>(p.v);
    TI* o = static_cast<TI*>(p.o);
    const TI* w1 = SWIGLU ? static_cast<const TI*>(p.w1) + (size_t)h * d_phi * d_k : nullptr;
    const TI* w3 = SWIGLU ? static_cast<const TI*>(p.w3) + (size_t)h * d_phi * d_k : nullptr;

    // momentum coefficient tables: c_r = 1 + beta c_{r-1}, beta^r
    if (tid == 0) {
        float c = 0.0f, bp = 1.0f;
        for (int r = 0; r < GC; ++r) {
            c = 1.0f + beta * c;
            sC[r] = c;
            sBP[r] = bp;
            bp *= beta;
        }
        sBP[GC] = bp;
    }
    {
        const size_t sbase = ((size_t)seq * p.d_v + dv0) * d_phi;
        for (int idx = tid; idx < d_phi * GDV; idx += GTHREADS) {
            const int f = idx / GDV, e = idx % GDV;
            sS[idx] = p.S0 ? p.S0[sbase + (size_t)e * d_phi + f] : 0.0f;
            sM[idx] = p.M0 ? p.M0[sbase + (size_t)e * d_phi + f] : 0.0f;
        }
    }
    __syncthreads();

    const size_t seq_row0 = (size_t)seq * T;
    const int n_chunks = (T + GC - 1) / GC;
    const bool causal = !(p.eta_kind & 0x100);   // bit 8 carries the bidirectional flag
    const int eta_kind = p.eta_kind & 0xff;

    // Identity map: the rows of chunk ch + 1 (k, q, this workgroup's v columns, the
    // rates) are loaded into registers while chunk ch is computed, every load of a
    // chunk issued before any is waited for.  d_phi = d_k <= 128: at most 8 feature
    // values of q and of k a thread.
    constexpr int PL = 8;
    float rk[PL], rq[PL], rv = 0.0f, re = 0.0f;
    auto fetch = [&](int ch) {
        const int t0 = ch * GC;
        const int n = min(GC, T - t0);
        const size_t row0 = seq_row0 + t0;
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int idx = tid + u * GTHREADS;
            const int r = idx / d_phi, f = idx - r * d_phi;
            const bool ok = idx < GC * d_phi && r < n;
            rk[u] = ok ? load_as_f32(k, (row0 + r) * d_k + f) : 0.0f;
            rq[u] = ok && causal ? load_as_f32(q, (row0 + r) * d_k + f) : 0.0f;
        }
        const int j = tid / GDV, e = tid % GDV;
        rv = j < n ? load_as_f32(v, (row0 + j) * p.d_v + dv0 + e) : 0.0f;
        re = tid < n ? eta_at(eta_kind, p.eta, p.eta_scalar, row0 + tid) : 0.0f;
    };
    if constexpr (!SWIGLU) {
        if (n_chunks > 0) fetch(0);
    }

    // ---- pass 1: state updates (causal: interleaved with the readout) -------
    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * GC;
        const int n = min(GC, T - t0);
        const size_t row0 = seq_row0 + t0;

        float et = 0.0f;
        if constexpr (SWIGLU) {
            load_features<TI, SWIGLU>(k, w1, w3, sPk, sXk, row0, n, d_k, d_phi);
            if (causal) load_features<TI, SWIGLU>(q, w1, w3, sPq, sXq, row0, n, d_k, d_phi);
            const int j = tid / GDV, e = tid % GDV;
            sV[tid] = j < n ? load_as_f32(v, (row0 + j) * p.d_v + dv0 + e) : 0.0f;
            et = tid < n ? eta_at(eta_kind, p.eta, p.eta_scalar, row0 + tid) : 0.0f;
        } else {
#pragma unroll
            for (int u = 0; u < PL; ++u) {
                const int idx = tid + u * GTHREADS;
                if (idx < GC * d_phi) {
                    sPk[idx] = rk[u];
                    if (causal) sPq[idx] = rq[u];
                }
            }
            sV[tid] = rv;
            et = re;
        }
        if (tid < GC) {
            sEta[tid] = et;
            sWS[tid] = tid < n ? et * sC[n - 1 - tid] : 0.0f;     // eta_j c_{n-1-j}
            sWM[tid] = tid < n ? et * sBP[n - 1 - tid] : 0.0f;    // eta_j beta^{n-1-j}
        }
        __syncthreads();
        if constexpr (!SWIGLU) {
            if (ch + 1 < n_chunks) fetch(ch + 1);   // in flight during this chunk
        }

        if (causal) {
            // A_ij = c_{i-j} eta_j phi(q_i).phi(k_j) for j <= i
            {
                int i = tid / GC, j = tid % GC;
                float acc = 0.0f;
                if (j <= i && i < n) {
                    const float* a = sPq + i * d_phi;
                    const float* b = sPk + j * d_phi;
                    for (int f = 0; f < d_phi; ++f) acc = fmaf(a[f], b[f], acc);
                    acc *= sC[i - j] * sEta[j];
                }
                sA[tid] = acc;
            }
            __syncthreads();
            // o_i = phi(q_i) (S + g_i M) + sum_j A_ij v_j
            {
                int i = tid / GDV, e = tid % GDV;
                if (i < n) {
                    const float gi = beta * sC[i];
                    const float* a = sPq + i * d_phi;
                    float acc = 0.0f, accm = 0.0f;
                    for (int f = 0; f < d_phi; ++f) {
                        acc = fmaf(a[f], sS[f * GDV + e], acc);
                        accm = fmaf(a[f], sM[f * GDV + e], accm);
                    }
                    acc = fmaf(gi, accm, acc);
                    for (int j = 0; j <= i; ++j) acc = fmaf(sA[i * GC + j], sV[j * GDV + e], acc);
                    store_from_f32(o, (row0 + i) * p.d_v + dv0 + e, acc);
                }
            }
            __syncthreads();
        }

        // state update
        {
            const float gl = beta * sC[n - 1];
            const float bn = sBP[n];
            for (int idx = tid; idx < d_phi * GDV; idx += GTHREADS) {
                int f = idx / GDV, e = idx % GDV;
                float s = sS[idx], m = sM[idx];
                s = fmaf(gl, m, s);
                m *= bn;
                for (int j = 0; j < n; ++j) {
                    float vk = sV[j * GDV + e] * sPk[j * d_phi + f];
                    s = fmaf(sWS[j], vk, s);
                    m = fmaf(sWM[j], vk, m);
                }
                sS[idx] = s;
                sM[idx] = m;
            }
        }
        __syncthreads();
    }

    if (causal) {
        if (p.S_T || p.M_T) {
            const size_t sbase = ((size_t)seq * p.d_v + dv0) * d_phi;
            for (int idx = tid; idx < d_phi * GDV; idx += GTHREADS) {
                const int e = idx / d_phi, f = idx % d_phi;   // coalesced along the features
                if (p.S_T) p.S_T[sbase + idx] = sS[f * GDV + e];
                if (p.M_T) p.M_T[sbase + idx] = sM[f * GDV + e];
            }
        }
        return;
    }

    // ---- pass 2 (bidirectional): every query reads the final state ---------
    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * GC;
        const int n = min(GC, T - t0);
        const size_t row0 = seq_row0 + t0;
        load_features<TI, SWIGLU>(q, w1, w3, sPq, sXq, row0, n, d_k, d_phi);
        __syncthreads();
        int i = tid / GDV, e = tid % GDV;
        if (i < n) {
            const float* a = sPq + i * d_phi;
            float acc = 0.0f;
            for (int f = 0; f < d_phi; ++f) acc = fmaf(a[f], sS[f * GDV + e], acc);
            store_from_f32(o, (row0 + i) * p.d_v + dv0 + e, acc);
        }
        __syncthreads();
    }
}

}  // namespace

size_t generic_smem_bytes(const Shape& s) {
    return generic_smem_floats(s.d_k, s.d_phi, s.swiglu) * sizeof(float);
}

hipError_t launch_generic(const Shape& s, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end) {
    GenericParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.eta = a.eta;
    p.w1 = s.w1;
    p.w3 = s.w3;
    p.o = a.o;
    p.eta_scalar = a.eta_scalar;
    p.beta = a.beta;
    p.eta_kind = a.eta_kind | (a.bidirectional ? 0x100 : 0);
    p.T = s.T;
    p.H = s.H;
    p.d_k = s.d_k;
    p.d_v = s.d_v;
    p.d_phi = s.d_phi;
    p.n_dvblk = s.d_v / GDV;
    p.S0 = a.S0;
    p.M0 = a.M0;
    p.S_T = a.S_T;
    p.M_T = a.M_T;
    const size_t smem = generic_smem_bytes(s);
    dim3 grid((unsigned)(s.n_seq() * p.n_dvblk)), block(GTHREADS);
    hipError_t e = hipSuccess;
#define TTT_GENERIC_LAUNCH(TI, SW)                                                                      \
    do {                                                                                                \
        e = hipFuncSetAttribute((const void*)generic_forward<TI, SW>,                                   \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);                 \
        if (e != hipSuccess) return e;                                                                  \
        if (ev_begin || ev_end) {                                                                       \
            void* args[] = {&p};                                                                        \
            return hipExtLaunchKernel(reinterpret_cast<const void*>(generic_forward<TI, SW>), grid, block, \
                                      args, smem, a.stream, ev_begin, ev_end, 0);                       \
        }                                                                                               \
        hipLaunchKernelGGL((generic_forward<TI, SW>), grid, block, smem, a.stream, p);                  \
    } while (0)
    if (s.bf16) {
        if (s.swiglu) TTT_GENERIC_LAUNCH(uint16_t, true);
        else TTT_GENERIC_LAUNCH(uint16_t, false);
    } else {
        if (s.swiglu) TTT_GENERIC_LAUNCH(float, true);
        else TTT_GENERIC_LAUNCH(float, false);
    }
#undef TTT_GENERIC_LAUNCH
    return hipGetLastError();
}

}  // namespace ttt
