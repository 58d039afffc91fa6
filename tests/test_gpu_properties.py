"""GPU invariants and edge cases of the HIP path (each against the oracle or
against a property the pages fix)."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, **kw):
    return WORKLOADS[name].with_shape(**kw)


def test_gradient_ascent_negates_output():
    # thelatestinai.com Table 1 'Gradient Ascent': ascent == eta -> -eta
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=200)
    say(f"[ascent] {w.name}")
    d = to_device(make_inputs(w))
    a = run_gpu(w, d)
    b = run_gpu(w, d, eta_sign=-1.0)
    assert oracle.rel_err(b, -a) <= 1e-6


def test_ascent_with_per_token_rate():
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=150).with_settings(eta_mode="per_token")
    say(f"[ascent-per-token] {w.name}")
    x = make_inputs(w)
    d = to_device(x)
    a = run_gpu(w, d)
    b = run_gpu(w, d, eta_sign=-1.0)
    assert oracle.rel_err(b, -a) <= 1e-6
    ref = run_oracle(w, x)
    assert oracle.rel_err(a, ref) <= TOL[w.dtype]


def test_query_replaced_by_key():
    # thelatestinai.com Table 1 'Replace Q with K': q aliases k
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=170)
    say(f"[q=k] {w.name}")
    x = make_inputs(w)
    d = to_device(x)
    got = run_gpu(w, d, q_override=d["k"])
    ref = run_oracle(w, x, q64=x.k64)
    assert oracle.rel_err(got, ref) <= TOL[w.dtype]


def test_linear_in_values_exactly_for_power_of_two():
    w = small("v4_momentum_4x8x2048_d128", B=1, H=1, T=130)
    say(f"[linearity] {w.name}")
    d = to_device(make_inputs(w))
    a = run_gpu(w, d)
    b = run_gpu(w, d, v_scale=2.0)
    np.testing.assert_array_equal(b, 2.0 * a)


def test_deterministic_run_to_run():
    w = small("v3_softplus_8x16x4096_d128", B=2, H=2, T=333)
    say(f"[determinism] {w.name}")
    d = to_device(make_inputs(w))
    a = run_gpu(w, d)
    b = run_gpu(w, d)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 129])
def test_short_and_ragged_sequences(T):
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=T)
    say(f"[ragged] T={T}")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x))
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


def test_zero_step_gives_zero_output():
    w = small("v4_momentum_4x8x2048_d128", B=1, H=1, T=100).with_settings(eta_scalar=0.0)
    say("[eta=0]")
    got = run_gpu(w, to_device(make_inputs(w)))
    assert np.all(got == 0.0)


@pytest.mark.parametrize("eta_mode", ["per_token", "softplus"])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_bidirectional_with_rates_and_momentum(eta_mode, beta):
    w = small("bidir_vit_256x6x196_d64", B=2, H=2, T=150).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[bidir] {eta_mode} beta={beta}")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x))
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


@pytest.mark.parametrize("d_k,d_v", [(64, 128), (128, 64), (64, 64)])
def test_mixed_widths(d_k, d_v):
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=140).with_settings(d_k=d_k, d_v=d_v, d_phi=d_k)
    say(f"[widths] d_k={d_k} d_v={d_v}")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x))
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


def test_fp32_momentum_softplus_and_bidirectional():
    for causal in (True, False):
        w = small("v5_f32_1x1x256_d64", B=2, H=2, T=90).with_settings(
            eta_mode="softplus", beta=0.9, causal=causal, d_v=128)
        say(f"[fp32] causal={causal}")
        x = make_inputs(w)
        got = run_gpu(w, to_device(x))
        assert oracle.rel_err(got, run_oracle(w, x)) <= TOL["f32"]


def test_fp32_swiglu():
    w = small("v5_f32_1x1x256_d64", B=1, H=2, T=40).with_settings(
        phi="swiglu", d_k=128, d_v=64, d_phi=256, eta_mode="softplus", beta=0.9)
    say("[fp32 swiglu]")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x))
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL["f32"]


def test_swiglu_small_feature_width_and_bidirectional():
    for causal in (True, False):
        w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=100).with_settings(d_phi=256, causal=causal)
        say(f"[swiglu d_phi=256] causal={causal}")
        x = make_inputs(w)
        got = run_gpu(w, to_device(x))
        assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("segments", [1, 2, 3, 5])
@pytest.mark.parametrize("value_split", [1, 2])
def test_tiling_does_not_change_the_result(chunk, segments, value_split):
    # chunk, segment count and value split are tiling choices: results agree with the oracle
    w = small("v3_long_1x16x65536_d128", B=1, H=2, T=1000)
    say(f"[tiling] chunk={chunk} segments={segments} value_split={value_split}")
    x = make_inputs(w)
    d = to_device(x)
    got = run_gpu(w, d, chunk=chunk, segments=segments, value_split=value_split)
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


def test_forward_rejects_bad_arguments_without_launching():
    import torch
    import ttt_weight_layers_amd as tla
    w = small("v4_momentum_4x8x2048_d128", B=1, H=1, T=64)
    d = to_device(make_inputs(w))
    lay = make_layer(w, d)
    o = torch.full_like(d["v"], 7.0)
    st = tla.ttt_la_forward(lay.handle, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), None,
                            0.1, 1.5, 0, o.data_ptr(), None)
    assert st == tla.TTT_LA_ERR_INVALID_ARG
    st = tla.ttt_la_forward(lay.handle, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), None,
                            0.1, 0.5, 0, d["q"].data_ptr(), None)
    assert st == tla.TTT_LA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
