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
hipError_t launch_generic(const Shape& s, const FwdArgs& a);

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
};

bool fast_supported(const Shape& s, int chunk);
FastPlan fast_plan(const Shape& s, int chunk, int segments, int value_split);
// Enqueues the whole forward (all kernels).  If ev_begin/ev_end are non-null
// they are recorded around the output kernel.
hipError_t launch_fast(const Shape& s, const FastPlan& p, void* workspace, const FwdArgs& a,
                       hipEvent_t ev_begin, hipEvent_t ev_end, int* n_kernels);

}  // namespace ttt
