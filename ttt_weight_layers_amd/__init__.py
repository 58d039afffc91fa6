"""MI355X-native forward of a TTT layer with KV binding, as learned linear attention.

The compute lives in ``libttt_la.so`` (hand-written HIP for gfx950, C ABI in
``include/ttt_la.h``); this package is its thin ctypes binding.  The library is
loaded on first use and its absence is an error, never a fallback.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, TTTError, TTTLinearAttention, load_library, make_desc, make_hints, mode_bits,
    ttt_la_hints, ttt_la_create_hinted, ttt_la_check_hints,
    ttt_la_check, ttt_la_create, ttt_la_desc, ttt_la_destroy, ttt_la_enable_kernel_timing,
    ttt_la_enable_kernel_timing_every,
    ttt_la_forward, ttt_la_forward_noalloc, ttt_la_forward_state, ttt_la_step, ttt_la_check_state, ttt_la_get_plan,
    ttt_la_backward, ttt_la_backward_swiglu, ttt_la_backward_workspace, ttt_la_check_backward,
    ttt_la_kernel_times, ttt_la_plan, ttt_la_status_string,
    ttt_la_wait_status,
    TTT_LA_OK, TTT_LA_ERR_INVALID_ARG, TTT_LA_ERR_UNSUPPORTED, TTT_LA_ERR_HIP, TTT_LA_ERR_OOM,
    TTT_LA_ERR_TOO_LARGE, TTT_LA_NOALLOC_SCRATCH_BYTES,
    TTT_LA_F32, TTT_LA_BF16, TTT_LA_PHI_IDENTITY, TTT_LA_PHI_SWIGLU, TTT_LA_CAUSAL,
    TTT_LA_BIDIRECTIONAL, TTT_LA_ETA_SCALAR, TTT_LA_ETA_PER_TOKEN, TTT_LA_ETA_SOFTPLUS, TTT_LA_LOSS_MSE, TTT_LA_WEIGHT_NORM,
    TTT_LA_LAUNCH_AUTO, TTT_LA_LAUNCH_SEPARATE, TTT_LA_LAUNCH_SINGLE, TTT_LA_LAUNCH_PREFIX,
)
