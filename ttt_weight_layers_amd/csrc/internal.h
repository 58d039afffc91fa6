// Host-side interface between the C ABI (api.hip) and the kernel translation
// units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ttt_la.h"

namespace ttt {

// Arguments of one forward call after validation.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* eta;
    float eta_scalar;
    float beta;
    int eta_kind;      // EtaKind
    bool bidirectional;
    void* o;
    hipStream_t stream;
    unsigned epoch;    // 1, 2, 3, ... per forward of a handle whose plan is fused
    // carried state, fp32 [B, H, d_v, d_phi] in the caller's layout (null: zero
    // entry state / final state not written)
    const float* S0 = nullptr;
    const float* M0 = nullptr;
    float* S_T = nullptr;
    float* M_T = nullptr;
    // time-reversed causal forward (32x32-tile plans of three launches, no carried
    // state): step t of the recurrence reads row T-1-t of q, k, v and the rates and
    // writes row T-1-t of o
    bool reverse = false;
};

// Shape of one layer (copied from the descriptor).
struct Shape {
    int B, H, T, d_k, d_v, d_phi;
    bool bf16;
    bool swiglu;
    const void* w1;
    const void* w3;
    int n_seq() const { return B * H; }
};

// ---- generic path: fp32 arithmetic on the vector ALUs ----------
// Handles every supported shape and mode, fp32 or bf16 inputs.
size_t generic_smem_bytes(const Shape& s);
// ev_begin/ev_end (may be null) take the kernel's start and end timestamps
hipError_t launch_generic(const Shape& s, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end);

// ---- bf16 MFMA path --------------------------------------------------------
struct FastPlan {
    int chunk;        // C
    int nwaves;       // waves per workgroup
    int dvt;          // 16-column value tiles per wave
    int dv_split;     // value-column slices per sequence
    int phi_split;    // 128-wide feature slices per sequence (SwiGLU)
    int segments;     // segments per sequence
    int seg_len;      // tokens per segment (multiple of chunk)
    size_t summary_bytes;   // segment summaries / entry states
    size_t partial_bytes;   // fp32 partial outputs when phi_split > 1
    bool wide;              // 32x32-tile kernels (chunk_wide.hip)
    bool fused;             // wide causal path as one cooperative launch (summary, scan, output)
    size_t zero_bytes;      // zeroed tail of the workspace (cleared once at create): the
                            // counters of the single-launch path
    bool prefix;            // wide causal path as one kernel whose segments rebuild their
                            // entry states from the earlier tokens
    int bounds[17];         // prefix path: first token of each segment, bounds[segments] = T
    int sum_split;          // two segments: summaries over halves of segment 0 (2) or all
                            // of it (1); the halves put twice the workgroups on the summary
    bool swiglu32;          // SwiGLU map, d_k = d_v = 128: causal forwards on the 32x32-tile
                            // kernel of swiglu.hip (one workgroup per sequence and 128-feature
                            // slice); bidirectional ones on the 16x16-tile kernels
};

bool fast_supported(const Shape& s, int chunk);
// launch: TTT_LA_LAUNCH_*
FastPlan fast_plan(const Shape& s, int chunk, int segments, int value_split, int launch);
// 32x32-tile kernels: identity map, d_k = d_v = 128, bf16
bool wide_supported(const Shape& s);
size_t wide_summary_bytes(const Shape& s, int segments);
int wide_max_segments();
// prefix path: chunk-aligned segment starts for T tokens and S segments, bounds[S] = T
void wide_prefix_bounds(int T, int S, int* bounds);
// workgroups the fused cooperative kernel can keep resident at once (0 if the
// device cannot launch cooperatively)
int wide_fused_capacity();
size_t wide_zero_bytes(const Shape& s);
// offset of the fused path's wait-failed flag inside the workspace
size_t wide_flag_offset(const Shape& s, const FastPlan& p);
hipError_t launch_wide(const Shape& s, const FastPlan& p, void* workspace, const FwdArgs& a, hipEvent_t ev_begin,
                       hipEvent_t ev_end, int* n_kernels);

// ---- SwiGLU feature map on 32x32 tiles (swiglu.hip) ----------------------------
// fp32 one-pass masked product for short sequences (short_f32.hip): identity map,
// d_k in {64, 128}, d_v a multiple of 64, T <= 1024, no carried state
bool short_supported(const Shape& s);
int short_grid(const Shape& s);
hipError_t launch_short(const Shape& s, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end);

// delta rule (mean-squared binding loss, no momentum, causal; delta.hip): bf16,
// identity map, d_k = d_v in {64, 128}
// identity map, d_k = d_v in {64, 128}.  With a workspace of delta_workspace_bytes
// (3 KiB per chunk of 32 tokens: the chunk inverses) two passes, else the one-pass walk.
bool delta_supported(const Shape& s);
size_t delta_workspace_bytes(const Shape& s);
hipError_t launch_delta(const Shape& s, const FwdArgs& a, void* workspace, size_t workspace_bytes,
                        hipEvent_t ev_begin, hipEvent_t ev_end);

// weight-normalised recurrent forward (wn.hip): causal, entry state required; bf16 or
// fp32 identity map (d_k = d_phi), or the bf16 SwiGLU map with d_k = 128; d_v a
// multiple of 16, d_phi in {64, 128, 256, 512}
bool wn_supported(const Shape& s);
size_t wn_workspace_bytes(const Shape& s);
hipError_t launch_wn(const Shape& s, void* workspace, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end);

// backward through the SwiGLU feature map (swiglu_bwd.hip): d_k = d_v = 128, bf16
bool swiglu_backward_supported(const Shape& s);
// phi(x) of every 128-feature slice, slice-major [P][B H T][128]
hipError_t launch_swiglu_features(const Shape& s, const void* x, void* phi, hipStream_t st);
// the chain rule through phi without [du | dg] in memory: dx of one input, and dW1, dW3
// from both (the keys' dphi scaled per token when eta is given)
hipError_t launch_swiglu_chain_dx(const Shape& s, const void* x, const void* dphi, void* dx, const float* eta,
                                  float eta_scalar, float beta, int eta_kind, bool scale_eta, bool bidir,
                                  hipStream_t st);
int swiglu_chain_dw_split(const Shape& s);
size_t swiglu_chain_dw_partial_bytes(const Shape& s);
hipError_t launch_swiglu_chain_dw(const Shape& s, const void* x_q, const void* x_k, const void* dphi_q,
                                  const void* dphi_k, const float* eta, float eta_scalar, float beta, int eta_kind,
                                  bool bidir, float* part, float* dw1, float* dw3, hipStream_t st);

bool swiglu_supported(const Shape& s);
// fp32 parts of o of the feature slices: [d_phi / 128][B * H * T][128]
size_t swiglu_partial_bytes(const Shape& s);
// causal forward without carried state; ev_begin/ev_end take the feature kernel's timestamps
hipError_t launch_swiglu(const Shape& s, void* workspace, const FwdArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end,
                         int* n_kernels);

// ---- recurrent step (decode.hip) ----------------------------------------------
struct StepArgs {
    const void* q;       // [B, H, d_k]
    const void* k;
    const void* v;       // [B, H, d_v]
    const float* eta;    // [B, H] or null
    float eta_scalar;
    float beta;
    int eta_kind;        // EtaKind
    float* S;            // fp32 [B, H, d_v, d_phi], updated in place
    float* M;
    void* o;             // [B, H, d_v]
    hipStream_t stream;
    bool weight_norm = false;   // rows of the new S rescaled to the norms of the given S
    bool mse = false;           // mean-squared loss: value factor v - S phi(k) at the given S
};
size_t step_smem_bytes(const Shape& s);
// the weight-normalised and the mean-squared step keep a whole row of S in registers
bool step_row_in_registers(const Shape& s);
// ev_begin/ev_end (may be null) take the step kernel's start and end timestamps
hipError_t launch_step(const Shape& s, const StepArgs& a, hipEvent_t ev_begin, hipEvent_t ev_end);

// ---- backward helpers (backward.hip) ----------------------------------------------
// dst[i][seq, t, :] = src[i][seq, T-1-t, :] for count <= 4 tensors of rows of row_bytes
// (a multiple of 16)
hipError_t launch_reverse(const void* const* src, void* const* dst, int count, size_t n_seq, int T, size_t row_bytes,
                          hipStream_t st);
struct BackArgs {
    const void* u;       // rate-1 forward outputs [n_seq, T, d]
    const void* w;
    bool uw_reversed;    // causal: u, w are stored reversed in time
    const void* v;
    const float* eta;
    void* dk;
    void* dv;
    float* deta;         // [n_seq, T] or null
    float eta_scalar;
    float beta;
    int eta_kind;
    bool causal;
    hipStream_t stream;
};
hipError_t launch_finalize_grads(const Shape& s, const BackArgs& a);

// Enqueues the whole forward (all kernels).  If ev_begin/ev_end are non-null
// they take the start and end timestamps of the output kernel.
hipError_t launch_fast(const Shape& s, const FastPlan& p, void* workspace, const FwdArgs& a,
                       hipEvent_t ev_begin, hipEvent_t ev_end, int* n_kernels);

}  // namespace ttt
