"""GPU invariants and edge cases of the HIP path (each against the oracle or
against a property the pages fix)."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, run_gpu, run_oracle, select_heads, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, **kw):
    return WORKLOADS[name].with_shape(**kw)


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_negated(b, a):
    """b == -a up to one bf16 rounding step per element.  Negating the rate
    negates every operand the kernels feed to the matrix cores; the fp32
    accumulation inside a matrix instruction is not guaranteed to round
    symmetrically, so an output that lands next to a bf16 rounding boundary
    may round to the neighbouring value."""
    diff = np.abs(b + a)
    assert np.all(diff <= bf16_ulp(a) * 1.0001), f"max |b + a| = {diff.max():.3e}"
    assert np.mean(diff == 0) >= 0.999


def oracle_ascent(w, x):
    """The oracle's gradient-ascent inner loop (its own sign flag, not a negated rate)."""
    return oracle.forward(x.q64, x.k64, x.v64, eta_mode=w.eta_mode, eta=x.a32, eta_scalar=w.eta_scalar,
                          beta=w.beta, causal=w.causal, phi=w.phi, w1=x.w1_64, w3=x.w3_64, ascent=True)


@pytest.mark.parametrize("name,kw,settings", [
    ("v4_momentum_4x8x2048_d128", dict(B=1, H=2, T=200), {}),
    ("v5_long_1x16x65536_d128", dict(B=1, H=2, T=64 * 7 + 3), {}),
    ("bidir_vit_256x6x196_d64", dict(B=2, H=2, T=196), {}),
    ("v5_f32_1x1x256_d64", dict(B=1, H=2, T=100), {}),
    ("v2_swiglu_4x16x8192_d128_f512", dict(B=1, H=2, T=64 * 2 + 9), dict(eta_mode="per_token")),
])
def test_gradient_ascent(name, kw, settings):
    # thelatestinai.com Table 1 'Gradient Ascent': the library runs ascent as the
    # rate -eta; the result is checked against the oracle's ascent loop, and
    # against the descent output negated
    w = small(name, **kw).with_settings(**settings)
    say(f"[ascent] {w.name} {kw} {settings}")
    x = make_inputs(w)
    d = to_device(x)
    a = run_gpu(w, d)
    b = run_gpu(w, d, eta_sign=-1.0)
    assert oracle.rel_err(b, oracle_ascent(w, x)) <= TOL[w.dtype]
    if w.dtype == "f32":
        np.testing.assert_allclose(b, -a, rtol=0, atol=1e-6 * np.max(np.abs(a)))
    elif w.phi == "identity":
        assert_negated(b, a)


def test_ascent_with_per_token_rate():
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=150).with_settings(eta_mode="per_token")
    say(f"[ascent-per-token] {w.name}")
    x = make_inputs(w)
    d = to_device(x)
    a = run_gpu(w, d)
    b = run_gpu(w, d, eta_sign=-1.0)
    assert_negated(b, a)
    assert oracle.rel_err(a, run_oracle(w, x)) <= TOL[w.dtype]
    assert oracle.rel_err(b, oracle_ascent(w, x)) <= TOL[w.dtype]


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


@pytest.mark.parametrize("T", [1, 63, 64, 129, 256, 257, 700])
@pytest.mark.parametrize("eta_mode,beta", [("scalar", 0.0), ("softplus", 0.5)])
def test_bidirectional_lengths(T, eta_mode, beta):
    # d = 64: up to 256 tokens every load of a sequence is issued at once (rows past
    # the end are zeroed when staged); longer sequences stream chunk by chunk
    w = small("bidir_vit_256x6x196_d64", B=1, H=3, T=T).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[bidir lengths] T={T} {eta_mode} beta={beta}")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x))
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


@pytest.mark.parametrize("eta_mode", ["scalar", "softplus"])
@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_bidirectional_wide_tiles(eta_mode, beta):
    # d = 128 with the identity map runs the 32x32-tile kernels
    w = small("v3_softplus_8x16x4096_d128", B=1, H=3, T=64 * 3 + 29).with_settings(
        eta_mode=eta_mode, beta=beta, causal=False)
    say(f"[bidir d=128] {eta_mode} beta={beta}")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x))
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


@pytest.mark.parametrize("eta_mode", ["scalar", "per_token", "softplus"])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_causal_wide_tiles_all_rate_modes(eta_mode, beta):
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=64 * 9 + 3).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[causal d=128] {eta_mode} beta={beta}")
    x = make_inputs(w)
    got = run_gpu(w, to_device(x), segments=4)
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]


@pytest.mark.parametrize("eta_mode,beta", [("scalar", 0.9), ("softplus", 0.9), ("scalar", 0.0)])
@pytest.mark.parametrize("segments", [8, 16])
def test_single_and_three_launch_paths(eta_mode, beta, segments):
    # 32 sequences, single launch requested: 8 segments make a 256-workgroup grid that
    # runs as one cooperative launch; 16 segments (512 workgroups) cannot be co-resident
    # and take three launches
    w = small("v4_momentum_4x8x2048_d128", T=2048 - 37).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[launch paths] segments={segments} {eta_mode} beta={beta}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=segments, launch="single")
    plan = lay.plan()
    assert plan.path == 2 and plan.segments == segments
    assert plan.n_kernels == (1 if segments == 8 else 3)
    heads = [0, 9, 31]
    got = run_gpu(w, d, layer=lay)
    got2 = run_gpu(w, d, layer=lay)          # a second launch on the same handle (next epoch)
    assert lay.wait_failed() == 0
    np.testing.assert_array_equal(got, got2)
    ref = run_oracle(w, x, heads=heads)
    assert oracle.rel_err(select_heads(got, w, heads), ref) <= TOL[w.dtype]


@pytest.mark.parametrize("eta_mode,beta", [("softplus", 0.9), ("per_token", 0.999), ("scalar", 0.0)])
def test_two_segments_with_split_summary(eta_mode, beta):
    # two segments of 20 chunks and few sequences: segment 0 is summarised in two
    # halves and the output kernel of segment 1 combines them (beta^(L/2) M_a + M_b;
    # with beta = 0.999 that term matters, with 0.9 it is below 2^-30)
    w = small("v4_momentum_4x8x2048_d128", B=1, H=3, T=64 * 40 - 13).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[split summary] {eta_mode} beta={beta}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=2)
    plan = lay.plan()
    assert plan.path == 2 and plan.segments == 2
    got = run_gpu(w, d, layer=lay)
    assert lay.plan().n_kernels == 3
    ref = run_oracle(w, x)
    assert oracle.rel_err(got, ref) <= TOL[w.dtype]


def test_timing_hook_between_single_launches():
    # the measurement hook switched on (one call in two) and off between forwards of
    # the single-launch plan: the arrival counters keep their targets, so every
    # forward waits as it should and gives the same output
    import ttt_weight_layers_amd as tla
    w = small("v4_momentum_4x8x2048_d128", T=1024 + 29)
    say("[timing hook / single launch]")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=8, launch="single")
    assert lay.plan().n_kernels == 1
    first = run_gpu(w, d, layer=lay)
    run_gpu(w, d, layer=lay)
    assert tla.ttt_la_enable_kernel_timing_every(lay.handle, 4, 2) == tla.TTT_LA_OK
    outs = [run_gpu(w, d, layer=lay) for _ in range(4)]
    times = tla.ttt_la_kernel_times(lay.handle, 4)
    assert len(times) == 2 and all(t > 0 for t in times)
    assert tla.ttt_la_enable_kernel_timing(lay.handle, 0) == tla.TTT_LA_OK
    outs.append(run_gpu(w, d, layer=lay))
    assert lay.wait_failed() == 0
    for o in outs:
        np.testing.assert_array_equal(o, first)
    heads = [0, 17, 31]
    ref = run_oracle(w, x, heads=heads)
    assert oracle.rel_err(select_heads(first, w, heads), ref) <= TOL[w.dtype]


@pytest.mark.parametrize("eta_mode,beta,segments", [("scalar", 0.9, 8), ("softplus", 0.9, 5), ("per_token", 0.0, 16)])
def test_prefix_launch(eta_mode, beta, segments):
    # one kernel: each segment's workgroup rebuilds its entry state from the earlier
    # tokens; a ragged last chunk and segment counts that do not divide the chunks
    w = small("v4_momentum_4x8x2048_d128", T=2048 - 37).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[prefix launch] segments={segments} {eta_mode} beta={beta}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=segments, launch="prefix")
    plan = lay.plan()
    # the plan itself keeps no workspace; the handle holds only the delta rule's chunk
    # inverses (3 KiB per 32 tokens of each sequence) for a mean-squared-loss forward
    assert plan.path == 2 and plan.n_kernels == 1
    assert plan.workspace_bytes == w.B * w.H * -(-w.T // 32) * 3072
    heads = [0, 13, 31]
    got = run_gpu(w, d, layer=lay)
    ref = run_oracle(w, x, heads=heads)
    assert oracle.rel_err(select_heads(got, w, heads), ref) <= TOL[w.dtype]


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


@pytest.mark.parametrize("T", [7, 64 * 3 + 11])
def test_swiglu_workspace_serves_both_modes(T):
    # one handle, causal then bidirectional calls: the causal kernel keeps each
    # slice's part as bf16 whole chunks, the bidirectional one as fp32 rows, and
    # the handle's workspace must hold the larger of the two
    w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=T).with_settings(d_phi=256)
    say(f"[swiglu workspace] T={T}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    plan = lay.plan()
    slices, n_seq, chunks = w.d_phi // 128, w.B * w.H, -(-T // 64)
    assert plan.path == 3
    assert plan.workspace_bytes >= max(slices * n_seq * T * 128 * 4, slices * n_seq * chunks * 64 * 128 * 2)
    for causal in (True, False):
        wc = w.with_settings(causal=causal)
        got = run_gpu(wc, d, layer=lay)
        assert oracle.rel_err(got, run_oracle(wc, x)) <= TOL[w.dtype]


@pytest.mark.parametrize("T,path", [(1024, 4), (1025, 0)])
def test_fp32_short_kernel_boundary(T, path):
    # up to 1024 tokens the fp32 forward is one masked product; beyond, the chunked walk
    w = small("v5_f32_1x1x256_d64", B=1, H=2, T=T).with_settings(eta_mode="softplus", beta=0.9)
    say(f"[fp32 boundary] T={T}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    assert lay.plan().path == path
    got = run_gpu(w, d, layer=lay)
    assert oracle.rel_err(got, run_oracle(w, x)) <= TOL[w.dtype]
