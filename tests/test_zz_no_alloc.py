"""ttt_la_forward_noalloc: the handle-less forward whose workspace is the
library's static device scratch.  Each case makes two calls in a row through
the C ABI, the second on a smaller input (so it runs over what the first left in
the scratch), and checks both against ttt_la_forward on a handle of the same
shape and plan hints (same kernels: equal bit for bit) and against the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
import ttt_weight_layers_amd as tla
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, run_gpu, run_oracle, to_device


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _desc(w, d):
    return tla.make_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.d_phi, dtype=w.dtype, phi=w.phi, chunk=w.chunk,
                         w1=d["w1"], w3=d["w3"])


def _noalloc(w, d, hints):
    import torch
    o = torch.empty(d["q"].shape[:-1] + (w.d_v,), dtype=d["v"].dtype, device=d["v"].device)
    eta = d["a"] if w.eta_mode != "scalar" else None
    st = tla.ttt_la_forward_noalloc(_desc(w, d), hints, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                    None if eta is None else eta.data_ptr(), w.eta_scalar, w.beta,
                                    tla.mode_bits(w.eta_mode, w.causal, w.loss), o.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == tla.TTT_LA_OK, tla.ttt_la_status_string(st)
    torch.cuda.synchronize()
    return from_device(o, w.dtype)


# (base workload, settings, first shape, second shape, plan hints)
CASES = {
    "wide_segments": ("v4_momentum_4x8x2048_d128", dict(eta_mode="softplus", beta=0.9),
                      dict(B=2, H=4, T=2048 - 37), dict(B=1, H=3, T=700), dict(segments=4)),
    "wide_sum_split": ("v3_softplus_8x16x4096_d128", dict(),
                       dict(B=1, H=4, T=2048 + 5), dict(B=1, H=2, T=1100), dict(segments=2)),
    "wide_bidir": ("v4_momentum_4x8x2048_d128", dict(causal=False),
                   dict(B=1, H=4, T=600), dict(B=1, H=2, T=130), dict()),
    "wide_single_hint": ("v4_momentum_4x8x2048_d128", dict(),
                         dict(B=1, H=4, T=1500), dict(B=1, H=2, T=800), dict(segments=4, launch="single")),
    "tile_d64_segments": ("bidir_vit_256x6x196_d64", dict(causal=True, eta_mode="per_token", beta=0.5),
                          dict(B=1, H=3, T=900), dict(B=1, H=2, T=300), dict(segments=3)),
    "swiglu_d128": ("v2_swiglu_4x16x8192_d128_f512", dict(d_phi=256),
                    dict(B=1, H=2, T=64 * 5 + 11), dict(B=1, H=1, T=100), dict()),
    "swiglu_d128_bidir": ("v2_swiglu_4x16x8192_d128_f512", dict(d_phi=256, causal=False),
                          dict(B=1, H=2, T=64 * 3 + 7), dict(B=1, H=1, T=90), dict()),
    "swiglu_d64_slices": ("v2_swiglu_4x16x8192_d128_f512", dict(d_k=64, d_v=64, d_phi=256),
                          dict(B=1, H=2, T=300), dict(B=1, H=1, T=70), dict()),
    "f32": ("v5_f32_1x1x256_d64", dict(), dict(B=1, H=2, T=256), dict(B=1, H=1, T=100), dict()),
    # delta rule: the chunk inverses in the scratch, then the walk
    "delta": ("v3_softplus_8x16x4096_d128", dict(loss="mse", beta=0.0, l2norm=True),
              dict(B=1, H=4, T=32 * 7 + 5), dict(B=1, H=2, T=100), dict()),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_handle_forward(name):
    base, settings, first, second, hint_kw = CASES[name]
    hints = tla.make_hints(**hint_kw)
    for i, shape in enumerate((first, second)):
        w = WORKLOADS[base].with_shape(**shape).with_settings(**settings)
        say(f"[noalloc] {name} call {i + 1}: {w.B}x{w.H}x{w.T} d_k={w.d_k} d_v={w.d_v} d_phi={w.d_phi} "
            f"causal={w.causal} hints={hint_kw}")
        x = make_inputs(w)
        d = to_device(x)
        got = _noalloc(w, d, hints)
        # the single-launch hint runs as three launches here: compare with those
        launch = hint_kw.get("launch", "auto")
        lay = make_layer(w, d, segments=hint_kw.get("segments", 0), launch="separate" if launch == "single" else launch)
        want = run_gpu(w, d, layer=lay)
        assert np.array_equal(got, want)
        assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


# aligned, far-apart stand-in addresses: the calls below return before any HIP call
Q, K, V, O, W1, W3 = (i << 40 for i in range(1, 7))


def test_noalloc_rejects_scratch_beyond_maximum():
    # Variant 2 at 4 x 16 x 8192 with 512 features: 4 slices of bf16 partial
    # outputs, 512 MiB, far above the static maximum
    d = tla.make_desc(4, 16, 8192, 128, 128, 512, dtype="bf16", phi="swiglu", w1=W1, w3=W3)
    st = tla.ttt_la_forward_noalloc(d, None, Q, K, V, None, 0.1, 0.9, tla.TTT_LA_CAUSAL, O, None)
    assert st == tla.TTT_LA_ERR_TOO_LARGE
    assert "static maximum" in tla.ttt_la_status_string(st)


def test_noalloc_argument_errors_before_any_hip_call():
    d = tla.make_desc(1, 2, 256, 64, 64)
    args = (Q, K, V, None, 0.1, 0.9, tla.TTT_LA_CAUSAL, O, None)
    assert tla.ttt_la_forward_noalloc(d, tla.make_hints(value_split=3), *args) == tla.TTT_LA_ERR_INVALID_ARG
    bad = list(args)
    bad[5] = 1.0   # beta out of [0, 1)
    assert tla.ttt_la_forward_noalloc(d, None, *bad) == tla.TTT_LA_ERR_INVALID_ARG
    bad = list(args)
    bad[7] = Q     # o on top of q
    assert tla.ttt_la_forward_noalloc(d, None, *bad) == tla.TTT_LA_ERR_INVALID_ARG
    assert tla.ttt_la_forward_noalloc(tla.make_desc(1, 2, 256, 96, 64, 96), None, *args) == \
        tla.TTT_LA_ERR_UNSUPPORTED
