/*
 * ttt_la.h - C ABI of libttt_la.so: the forward pass of a test-time-training
 * (TTT) layer with key-value binding, computed as learned linear attention on
 * one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes.  The five web pages about "Test-Time Training with
 * KV Binding Is Secretly Linear Attention" describe the layer as a fixed-size
 * fast-weight matrix that takes one gradient step per sequence entry and is
 * reset for every new sequence (wpnews.pro, "Test Time Training"), whose
 * update is the outer-product accumulation of linear attention, computable
 * either as a recurrence or in parallel (kualia.ai blog, "The Linear Attention
 * Equivalence"), with the inner-loop options removed one by one in the
 * ablation of the thelatestinai.com page (Table 2: Variant 2 SwiGLU feature
 * map; Variant 3 per-token learning rate and momentum; Variant 4 no per-token
 * lr; Variant 5 no momentum).  With the readings adopted here (dot-product
 * binding loss, zero initial state, readout after the update, heavy-ball
 * momentum with the step inside the buffer), for every sequence (b, h):
 *
 *     M_t = beta * M_{t-1} + eta_t * v_t phi(k_t)^T        (M_{-1} = 0)
 *     S_t = S_{t-1} + M_t                                   (S_{-1} = 0)
 *     o_t = S_t phi(q_t)              causal mode
 *     o_t = S_{T-1} phi(q_t)          bidirectional mode
 *
 * with S, M in R^{d_v x d_phi} kept in fp32 and phi the identity
 * (d_phi = d_k) or the frozen SwiGLU map phi(x) = silu(W1 x) * (W3 x),
 * silu(u) = u / (1 + e^-u).  The library evaluates this in its chunked
 * parallel form (dense causal blocks inside a chunk, fp32 state carried from
 * chunk to chunk); the result equals the recurrence up to rounding.  Gradient
 * ascent in the inner loop (Table 1 of the same page) is eta -> -eta.
 *
 * Conventions for every entry point:
 *   - Device buffers are plain device pointers owned by the caller.  The
 *     library never frees them and keeps none of them after a call returns,
 *     except W1/W3, which are borrowed at create and must outlive the handle.
 *   - Every call returns a ttt_la_status; no call aborts, throws or prints.
 *   - Arguments are validated on the host before any HIP call.
 *   - ttt_la_forward allocates nothing and does not synchronise: it enqueues
 *     kernels on the given stream and returns.  Device-side faults surface at
 *     the caller's next synchronisation.  One handle serves one stream at a
 *     time (its workspace is reused by every call).
 */
#ifndef TTT_LA_H
#define TTT_LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ttt_la_s* ttt_la_t; /* opaque handle */

typedef enum {
    TTT_LA_OK = 0,
    TTT_LA_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad size, bad mode bit, beta or eta out of range, overlap */
    TTT_LA_ERR_UNSUPPORTED = -2, /* well-formed request outside the supported shapes */
    TTT_LA_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
    TTT_LA_ERR_OOM = -4,         /* workspace allocation failed */
    TTT_LA_ERR_TOO_LARGE = -5    /* ttt_la_forward_noalloc: the plan needs more scratch than
                                    TTT_LA_NOALLOC_SCRATCH_BYTES */
} ttt_la_status;

typedef enum { TTT_LA_F32 = 0, TTT_LA_BF16 = 1 } ttt_la_dtype; /* q, k, v, o, W1, W3 */

typedef enum {
    TTT_LA_PHI_IDENTITY = 0, /* phi(x) = x, d_phi = d_k (Variants 3-5) */
    TTT_LA_PHI_SWIGLU = 1    /* phi(x) = silu(W1 x) * (W3 x) (Variant 2) */
} ttt_la_phi;

/* Mode bits for ttt_la_forward.  At most one of the ETA bits may be set. */
enum {
    TTT_LA_CAUSAL = 0u,              /* o_t = S_t phi(q_t) */
    TTT_LA_BIDIRECTIONAL = 1u << 0,  /* o_t = S_{T-1} phi(q_t): all tokens update before any readout */
    TTT_LA_ETA_SCALAR = 0u,          /* eta_t = eta_scalar; the eta pointer must be NULL */
    TTT_LA_ETA_PER_TOKEN = 1u << 1,  /* eta_t = eta[b,h,t] */
    TTT_LA_ETA_SOFTPLUS = 1u << 2,   /* eta_t = softplus(eta[b,h,t]) = ln(1 + e^a) (Table 2, Variant 3) */
    TTT_LA_LOSS_MSE = 1u << 3,       /* binding loss 1/2 ||S phi(k_t) - v_t||^2 instead of -<S phi(k_t), v_t>:
                                        the delta rule S_t = S_{t-1} - eta_t (S_{t-1} k_t - v_t) k_t^T
                                        (mlsanity.com page: Modular TTT abstract, MSE and inner-product
                                        losses; "Builds on": the delta-rule parallelisation paper).
                                        ttt_la_forward and ttt_la_forward_state: bf16, identity map,
                                        d_k = d_v in {64, 128}, causal, beta = 0; anything else
                                        TTT_LA_ERR_UNSUPPORTED.  The carried state is S alone: S0 and
                                        S_T as for the other losses, M0 and M_T must be NULL
                                        (TTT_LA_ERR_INVALID_ARG).  On a handle the per-chunk inverses
                                        (I + N)^-1 diag(eta), 3 KiB per 32 tokens of each sequence, go
                                        to the handle's workspace (sized for them at creation).
                                        ttt_la_step: M <- beta M + eta (v - S phi(k)) phi(k)^T,
                                        S <- S + M, o = S phi(q) (momentum allowed), for every dtype and
                                        feature map with d_phi <= 128 (identity) or <= 512 (SwiGLU),
                                        else TTT_LA_ERR_UNSUPPORTED; with TTT_LA_WEIGHT_NORM
                                        TTT_LA_ERR_INVALID_ARG */
    TTT_LA_WEIGHT_NORM = 1u << 4     /* Variant 1 of Table 2 (thelatestinai.com page): the updated layer
                                        is weight-normalised, recurrent implementation only.  The pages
                                        do not define the normalisation; here, after each token's update,
                                        every row of S (one value column: its weights over the features)
                                        is rescaled to the Euclidean norm that row has in S0, and M is
                                        not rescaled (a row with a zero S0 norm stays zero).
                                        ttt_la_forward_state, with S0 given (else
                                        TTT_LA_ERR_INVALID_ARG, as with the bidirectional or MSE bits),
                                        and ttt_la_step (each row of the new S rescaled to the norm of
                                        the same row of the given S, which a weight-normalised run
                                        keeps at its entry-state norm); ttt_la_forward and the
                                        backward: TTT_LA_ERR_INVALID_ARG;
                                        d_v a multiple of 16, d_phi in {64, 128, 256, 512}, identity map
                                        (bf16 or fp32, d_k = d_phi) or bf16 SwiGLU map with d_k = 128,
                                        else TTT_LA_ERR_UNSUPPORTED.  One workgroup per 16 rows of S
                                        walks the tokens in order; the SwiGLU features of q and k go to
                                        the handle's workspace first (TTT_LA_ERR_UNSUPPORTED if it is
                                        smaller than 4 B H T d_phi bytes). */
};

typedef struct {
    int32_t B, H, T;           /* batch, heads, sequence length: B, H, T >= 1 */
    int32_t d_k, d_v, d_phi;   /* key/query width, value width, feature width */
    int32_t dtype;             /* ttt_la_dtype of q, k, v, o (and W1, W3) */
    int32_t phi;               /* ttt_la_phi */
    int32_t chunk;             /* tile length along T: 0 = auto, else 64 or 128 (bf16); it changes
                                  the result only by rounding */
    const void* w1;            /* SWIGLU: device [H, d_phi, d_k] (out x in) in dtype; else NULL */
    const void* w3;            /* SWIGLU: device [H, d_phi, d_k] in dtype; else NULL */
} ttt_la_desc;

/* Launch choice for a causal forward split into segments (ttt_la_hints.launch). */
enum {
    TTT_LA_LAUNCH_AUTO = 0,      /* the library's choice (currently: separate kernels) */
    TTT_LA_LAUNCH_SEPARATE = 1,  /* segment summaries, their scan and the outputs as three kernels */
    TTT_LA_LAUNCH_SINGLE = 2,    /* one cooperative kernel whose workgroups exchange the segment
                                    summaries through device memory, when the device can keep the
                                    whole grid resident (32x32-tile path only); else as SEPARATE */
    TTT_LA_LAUNCH_PREFIX = 3     /* one kernel, no exchange: the workgroup of each segment first
                                    rebuilds its entry state from the keys and values of all earlier
                                    tokens (32x32-tile path only; else as SEPARATE) */
};

/* Optional kernel-plan hints for ttt_la_create_hinted.  They choose how the
 * work is tiled and launched, never what is computed: results differ only by
 * rounding.  All-zero = the library's choice (what ttt_la_create takes). */
typedef struct {
    int32_t segments;          /* sequence segments scanned in parallel: 0 = auto, else >= 1 (bf16 causal) */
    int32_t value_split;       /* workgroups sharing one segment's value columns: 0 = auto, 1 or 2
                                  (2 is used for d_k = d_v = 128 with the identity map) */
    int32_t launch;            /* TTT_LA_LAUNCH_*: how a segmented causal forward is launched */
} ttt_la_hints;

/* Supported shapes (anything else well-formed returns TTT_LA_ERR_UNSUPPORTED):
 *   d_k, d_v in {64, 128}
 *   identity: d_phi == d_k;  SwiGLU: d_phi in {128, 256, 384, 512}
 *   B * H * T * max(d_k, d_v, d_phi) < 2^31, except on the 32x32-tile plan (bf16,
 *   identity map, d_k = d_v = 128, no value-split hint): there B * H * T < 2^31, and
 *   past 2^31 elements a tensor only the forwards with the dot-product loss run
 *   (ttt_la_forward, ttt_la_forward_state, ttt_la_forward_noalloc; weight
 *   normalisation, the mean-squared loss and the backward return
 *   TTT_LA_ERR_UNSUPPORTED)
 *
 * Layout: q, k are [B, H, T, d_k]; v and o are [B, H, T, d_v]; eta is
 * [B, H, T] fp32; all C-contiguous.  Pointers to q, k, v, o, W1, W3 must be
 * 16-byte aligned, eta 4-byte aligned. */

/* Creates a handle for one layer shape.  Validates *desc, picks the kernel
 * plan for the shape and allocates the workspace (hipMalloc on the current
 * device), once.  On any error *out is set to NULL. */
int ttt_la_create(const ttt_la_desc* desc, ttt_la_t* out);

/* ttt_la_create with kernel-plan hints (hints may be NULL: all automatic).
 * TTT_LA_ERR_INVALID_ARG for a negative segment count, a value split other
 * than 0, 1, 2 or an unknown launch value, before any HIP call. */
int ttt_la_create_hinted(const ttt_la_desc* desc, const ttt_la_hints* hints, ttt_la_t* out);

/* Enqueues one forward pass on hip_stream (a hipStream_t; NULL = the null
 * stream).
 *   q, k, v  device inputs as above.  q may alias k ("Replace Q with K",
 *            Table 1): inputs are only read.
 *   eta      NULL for TTT_LA_ETA_SCALAR, else device [B, H, T] fp32.
 *   eta_scalar  the step size when no ETA bit is set; must be finite.
 *   beta     momentum in [0, 1); 0 turns momentum off (Variant 5).
 *   mode     TTT_LA_* bits above.
 *   o        device output [B, H, T, d_v] in dtype; must not overlap any input.
 * Returns TTT_LA_ERR_INVALID_ARG without any HIP call for bad arguments and
 * TTT_LA_ERR_HIP if a launch fails. */
int ttt_la_forward(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta,
                   float eta_scalar, float beta, uint32_t mode, void* o, void* hip_stream);

/* Size of the static device scratch of ttt_la_forward_noalloc (one copy per
 * device, held until the process ends). */
#define TTT_LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* ttt_la_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  No
 * handle: the kernel plan is taken from *desc and *hints (hints may be NULL) on
 * every call, exactly as ttt_la_create_hinted would take it, and the
 * workspace of that plan (segment summaries, per-slice partial outputs) lives in
 * a static device array of TTT_LA_NOALLOC_SCRATCH_BYTES instead.  The call makes
 * no hipMalloc, hipFree or other allocating call; the first call on a device
 * resolves that device's copy of the array (hipGetSymbolAddress).
 *   desc, hints  as for ttt_la_create_hinted; q, k, v, eta, eta_scalar, beta,
 *            mode, o, hip_stream as for ttt_la_forward.  The inputs and o are
 *            the caller's and stay so.
 * Results equal those of ttt_la_forward on a handle created from the same desc
 * and hints.  TTT_LA_LAUNCH_SINGLE runs as three launches here (the single
 * launch keeps counters from call to call of one handle).
 * All calls on one device share its scratch and leave their contents in it:
 * calls that overlap in time on one device (streams that are not ordered with
 * each other) race and their results are undefined.
 * With TTT_LA_LOSS_MSE the per-chunk inverses use the scratch when they fit
 * (3 KiB per 32 tokens of each sequence); beyond that the call runs the one-pass
 * delta-rule kernel, which needs no workspace (same results within rounding, not
 * bit for bit).
 * Errors: as ttt_la_create_hinted and ttt_la_forward (all before any HIP call),
 * and TTT_LA_ERR_TOO_LARGE, before any HIP call, when the plan's workspace
 * exceeds TTT_LA_NOALLOC_SCRATCH_BYTES (for instance B*H*T*d_phi*2 bytes of
 * SwiGLU partials above 64 MiB; fewer segments shrink the summaries). */
int ttt_la_forward_noalloc(const ttt_la_desc* desc, const ttt_la_hints* hints, const void* q, const void* k,
                           const void* v, const float* eta, float eta_scalar, float beta, uint32_t mode, void* o,
                           void* hip_stream);

/* Causal forward from a carried state.  Table 2 of the thelatestinai.com page
 * lists a recurrent implementation of every variant beside the parallel one:
 * the recurrent form keeps the fast weight (S, M) from one call to the next.
 * Same as ttt_la_forward in the causal mode, except that the state before the
 * first token is (S0, M0) instead of zero, and that the state after the last
 * token is written to (S_T, M_T):
 *   S0, M0, S_T, M_T  device fp32 [B, H, d_v, d_phi] (row r = value column r
 *            of the fast weight, column = feature), C-contiguous, 16-byte
 *            aligned.  Any may be NULL: a NULL S0 or M0 reads as zero, a NULL
 *            S_T or M_T is not written.  S_T may be S0 and M_T may be M0 (the
 *            state is then updated in place); apart from that the outputs must
 *            not overlap each other or any input, and S0, M0 must not overlap
 *            q, k, v, eta or o.
 * With TTT_LA_LOSS_MSE (the delta rule, no momentum) only S0 and S_T are
 * taken; M0 and M_T must be NULL.
 * Errors: as ttt_la_forward, and TTT_LA_ERR_INVALID_ARG for the bidirectional
 * mode bit, a misaligned or overlapping state pointer, or M0 / M_T with
 * TTT_LA_LOSS_MSE.
 * TTT_LA_ERR_UNSUPPORTED for a handle created with TTT_LA_LAUNCH_PREFIX on the
 * 32x32-tile plan (that plan has no workspace for the entry state; the delta
 * rule is not affected). */
int ttt_la_forward_state(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta,
                         float eta_scalar, float beta, uint32_t mode, const float* S0, const float* M0,
                         void* o, float* S_T, float* M_T, void* hip_stream);

/* One recurrent step (decode) for every (b, h), the recurrent implementation
 * of Table 2 applied to a single new token:
 *   M <- beta M + eta v phi(k)^T,   S <- S + M,   o = S phi(q)
 *   q, k     device [B, H, 1, d_k] in dtype; v, o: [B, H, 1, d_v] in dtype.
 *   eta      NULL for TTT_LA_ETA_SCALAR, else device [B, H] fp32 (the rate or
 *            the softplus argument of this token).
 *   S, M     device fp32 [B, H, d_v, d_phi] as in ttt_la_forward_state,
 *            updated in place; they must not overlap each other or any other
 *            argument.
 *   mode     rate bits, and TTT_LA_WEIGHT_NORM (Variant 1's step) or
 *            TTT_LA_LOSS_MSE (the delta-rule step, value factor v - S phi(k) at
 *            the given S): see the mode bits; TTT_LA_BIDIRECTIONAL is invalid here.
 * The handle's T is ignored; its B, H, widths, dtype and feature map (W1, W3)
 * apply.  Allocates nothing, does not synchronise; errors as ttt_la_forward. */
int ttt_la_step(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                float beta, uint32_t mode, float* S, float* M, void* o, void* hip_stream);

/* Gradients of the forward.  Figure 4 of the thelatestinai.com page trains the
 * parallel form end to end; with L = sum(o * dO) for the o that ttt_la_forward
 * returns on the same q, k, v, eta, eta_scalar, beta and mode:
 *   dO       device [B, H, T, d_v] in dtype (the gradient of L with respect to o).
 *   dQ, dK   device [B, H, T, d_k] in dtype;  dV: [B, H, T, d_v] in dtype.
 *   dEta     NULL, or device [B, H, T] fp32: dL/deta_t for TTT_LA_ETA_PER_TOKEN,
 *            dL/da_t (the softplus argument) for TTT_LA_ETA_SOFTPLUS, and for a
 *            scalar rate the per-token terms whose sum is dL/deta_scalar.
 *   workspace, workspace_bytes  caller-owned device memory, 16-byte aligned, at
 *            least ttt_la_backward_workspace() bytes (may be NULL when that is 0).
 * Identity feature map (TTT_LA_ERR_UNSUPPORTED for SwiGLU: see ttt_la_backward_swiglu);
 * d_k and d_v may differ (dQ, dK are d_k wide, dV is d_v wide).
 * Runs three forwards of the layer on permuted operands (two over the sequence
 * reversed in time; those giving dq and dk have queries and keys of width d_v and
 * values of width d_k) and one to three small kernels, enqueued on hip_stream; no
 * device memory is allocated and nothing is synchronised with the host.  On the
 * bf16 d = 128 plans of three launches the two reversed forwards read their rows
 * in reverse order and run beside the first one on two streams of the handle,
 * which start after the work already on hip_stream and which hip_stream waits
 * for; their segment summaries live in the workspace.  The first such call on a
 * handle creates those two streams (default priority) and three events; if that
 * fails, everything runs on hip_stream.  Like the forward, one handle serves one
 * stream at a time.
 * The outputs must not overlap each other, any input or the workspace.
 * Errors: as ttt_la_forward, and TTT_LA_ERR_INVALID_ARG for a missing, misaligned,
 * overlapping or too small buffer. */
int ttt_la_backward(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                    float beta, uint32_t mode, const void* dO, void* dQ, void* dK, void* dV, float* dEta,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* Gradients of a SwiGLU layer (Variant 2 of Table 2 on the thelatestinai.com page:
 * only the last layer of the fast-weight MLP is updated by the inner loop, so W1
 * and W3 are slow weights, trained through the outer loop as Figure 4 trains the
 * parallel form end to end).  With L = sum(o * dO) for the o of ttt_la_forward on
 * the same arguments:
 *   dQ, dK, dV, dEta  as for ttt_la_backward (dQ and dK through phi)
 *   dW1, dW3  device fp32 [H, d_phi, d_k], 16-byte aligned: dL/dW1, dL/dW3 summed
 *            over the batch (overwritten, not accumulated)
 *   workspace  caller-owned device memory, 256-byte aligned, at least
 *            ttt_la_backward_workspace(h, mode) bytes
 * bf16, d_k = d_v = 128 (TTT_LA_ERR_UNSUPPORTED otherwise, and for
 * TTT_LA_LOSS_MSE).  Causal and bidirectional.  Runs, on hip_stream: the features
 * phi(q), phi(k); for each 128-feature slice a forward of the d = 128 identity plan
 * giving dL/dphi(q) and one (rate 1, over the sequence reversed in time when
 * causal) giving dL/dphi(k); one SwiGLU forward of (k, q, dO) at rate 1 giving
 * dV and dEta; the chain rule through phi (du = dphi g silu'(u), dg = dphi silu(u))
 * and the products dq = W1^T du + W3^T dg, dW1 = sum du x^T, dW3 = sum dg x^T,
 * with fixed-order sums.  No device memory is allocated.  The outputs must not
 * overlap each other, any input or the workspace.
 * Errors: as ttt_la_backward. */
int ttt_la_backward_swiglu(ttt_la_t h, const void* q, const void* k, const void* v, const float* eta,
                           float eta_scalar, float beta, uint32_t mode, const void* dO, void* dQ, void* dK, void* dV,
                           float* dEta, float* dW1, float* dW3, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/* Bytes of workspace ttt_la_backward needs on handle h for the given mode bits:
 * the outputs of the two rate-1 forwards ([B, H, T, d_v] and [B, H, T, d_k]),
 * plus in causal mode either two segment-summary areas of the handle's plan (bf16
 * d = 128 plans of three launches) or the four time-reversed operands, plus for
 * d_k != d_v the segment-summary area of the plan with the widths swapped.  For a SwiGLU
 * handle: the workspace of ttt_la_backward_swiglu.  Host only;
 * TTT_LA_ERR_UNSUPPORTED if the handle's shape has no backward. */
int ttt_la_backward_workspace(ttt_la_t h, uint32_t mode, size_t* bytes);

/* Releases the workspace and the handle.  NULL-safe. */
void ttt_la_destroy(ttt_la_t h);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* ttt_la_status_string(int status);

/* Host-only validation of a descriptor and of the arguments of one forward
 * call, exactly as ttt_la_create / ttt_la_forward perform it, without any HIP
 * call (pointers are only compared, never dereferenced).  Pass q == NULL to
 * check the descriptor alone.  Returns the status create/forward would return
 * for these arguments before touching the device. */
int ttt_la_check(const ttt_la_desc* desc, const void* q, const void* k, const void* v,
                 const float* eta, float eta_scalar, float beta, uint32_t mode, const void* o);

/* The same for the state-carrying calls: call = 0 checks the arguments of
 * ttt_la_forward_state (s_in = S0, m_in = M0, s_out = S_T, m_out = M_T),
 * call = 1 those of ttt_la_step (s_in = s_out = S, m_in = m_out = M).  The
 * descriptor is checked first; q must not be NULL. */
int ttt_la_check_state(const ttt_la_desc* desc, int32_t call, const void* q, const void* k, const void* v,
                       const float* eta, float eta_scalar, float beta, uint32_t mode, const float* s_in,
                       const float* m_in, const void* o, const float* s_out, const float* m_out);

/* Host-only validation of plan hints, as ttt_la_create_hinted performs it (NULL is valid). */
int ttt_la_check_hints(const ttt_la_hints* hints);

/* The same for ttt_la_backward (the descriptor and the hints, NULL = automatic,
 * stand for the handle: the workspace size depends on the plan). */
int ttt_la_check_backward(const ttt_la_desc* desc, const ttt_la_hints* hints, const void* q, const void* k, const void* v, const float* eta,
                          float eta_scalar, float beta, uint32_t mode, const void* dO, const void* dQ,
                          const void* dK, const void* dV, const float* dEta, const void* workspace,
                          size_t workspace_bytes);

/* Kernel plan chosen at create, for tests and measurement. */
typedef struct {
    int32_t path;          /* 0 = generic fp32-accumulate kernels, 1 = bf16 16x16-tile MFMA chunk
                              kernels, 2 = bf16 32x32-tile MFMA chunk kernels (identity map, d = 128),
                              3 = bf16 32x32-tile SwiGLU kernel (d_k = d_v = 128; causal forwards,
                              bidirectional ones as path 1), 4 = fp32 one-pass masked T x T product
                              (identity map, d_k in {64, 128}, d_v a multiple of 64, T <= 1024;
                              calls with a carried state as path 0) */
    int32_t chunk;         /* tokens per chunk */
    int32_t segments;      /* sequence segments per (b, h) scanned in parallel (1 = none) */
    int32_t seg_len;       /* tokens per segment (last one may be shorter) */
    int32_t dv_split;      /* value-column slices per (b, h) */
    int32_t phi_split;     /* feature slices per (b, h) (partial outputs summed) */
    int32_t grid_main;     /* workgroups of the output kernel */
    int32_t n_kernels;     /* kernels enqueued by one causal forward */
    size_t workspace_bytes;
} ttt_la_plan;

/* Fills *plan for handle h.  Host only. */
int ttt_la_get_plan(ttt_la_t h, ttt_la_plan* plan);

/* Diagnostic of the single-launch causal path (path 2 with n_kernels == 1):
 * the workgroups of one sequence wait for each other twice per forward, each
 * wait bounded so that a kernel always terminates.  *failed is set to 1 if any
 * wait of a forward on h since the previous call gave up (that output is then
 * invalid), else 0; reading a 1 clears the flag.  Always 0 for other plans.
 * Synchronises with the device (a blocking copy). */
int ttt_la_wait_status(ttt_la_t h, int32_t* failed);

/* Measurement hook.  When n_slots > 0, every following ttt_la_forward,
 * ttt_la_forward_state or ttt_la_step passes a pair of HIP events (created
 * here, not device memory) to the launch of its output kernel (the step
 * kernel for ttt_la_step), which takes the kernel's start and end timestamps,
 * cycling through n_slots pairs; ttt_la_kernel_times then
 * returns the elapsed milliseconds of the last min(calls, n_slots) pairs
 * (oldest first) after synchronising on them.  n_slots = 0 turns it off. */
int ttt_la_enable_kernel_timing(ttt_la_t h, int32_t n_slots);
int ttt_la_kernel_times(ttt_la_t h, float* ms, int32_t capacity, int32_t* count);

/* The same hook on one call in `every` (>= 1): the first following call and
 * every `every`-th one after it carry the events, the others launch without
 * them (an event pair around a kernel costs the stream some time of its own).
 * ttt_la_enable_kernel_timing(h, n) is ttt_la_enable_kernel_timing_every(h, n, 1).
 * TTT_LA_ERR_INVALID_ARG for a null handle, n_slots < 0 or every < 1. */
int ttt_la_enable_kernel_timing_every(ttt_la_t h, int32_t n_slots, int32_t every);

#ifdef __cplusplus
}
#endif

#endif /* TTT_LA_H */
