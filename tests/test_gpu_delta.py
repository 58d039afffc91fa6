"""GPU parity of the delta rule (TTT_LA_LOSS_MSE: mean-squared binding loss, no
momentum) against the oracle's loop with loss="mse", at the bf16 bar.

The workload is the Variant-3 shape (8 x 16 x 4096, d = 128, rate softplus(a))
with momentum off and L2-normalised tokens, so that every step
S (I - eta k k^T) + eta v k^T is a contraction in the direction of k
(0 < eta < 2); reduced shapes cover d = 64, the three rate modes, ragged and
sub-chunk lengths.
"""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, head_subset, make_inputs
from _gpu import TOL, make_layer, run_gpu, run_oracle, select_heads, to_device

pytestmark = pytest.mark.gpu

DELTA = WORKLOADS["v3_softplus_8x16x4096_d128"].with_settings(
    name="v3_delta_8x16x4096_d128", loss="mse", beta=0.0, l2norm=True)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("d,eta_mode,eta_scalar,B,H,T", [
    (128, "softplus", 0.0, 2, 2, 300),
    (128, "scalar", 0.5, 1, 3, 32 * 3 + 5),
    (128, "per_token", 0.0, 1, 2, 31),
    (128, "softplus", 0.0, 1, 1, 1),
    (64, "softplus", 0.0, 2, 2, 250),
    (64, "scalar", 1.0, 1, 2, 64),
])
def test_delta_parity_reduced(d, eta_mode, eta_scalar, B, H, T):
    w = DELTA.with_shape(B=B, H=H, T=T).with_settings(d_k=d, d_v=d, d_phi=d, eta_mode=eta_mode,
                                                      eta_scalar=eta_scalar)
    say(f"[delta] d={d} {eta_mode} {B}x{H}x{T}")
    x = make_inputs(w)
    d_ = to_device(x)
    got = run_gpu(w, d_)
    ref = run_oracle(w, x)
    err = oracle.rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL[w.dtype]


def test_delta_parity_full_shape():
    w = DELTA
    heads = head_subset(w, 8)
    say(f"[delta full] heads {heads}")
    x = make_inputs(w)
    d_ = to_device(x)
    got = select_heads(run_gpu(w, d_), w, heads)
    ref = run_oracle(w, x, heads=heads)
    err = oracle.rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL[w.dtype]


def test_delta_is_not_the_dot_product_layer():
    # same inputs, the two losses give different outputs after the first token
    w = DELTA.with_shape(B=1, H=1, T=70)
    x = make_inputs(w)
    d_ = to_device(x)
    mse = run_gpu(w, d_)
    dot = run_gpu(w.with_settings(loss="dot"), d_)
    np.testing.assert_allclose(mse[0, 0, 0], dot[0, 0, 0], rtol=0, atol=1e-6 * np.max(np.abs(dot)))
    assert np.max(np.abs(mse[0, 0, 40:] - dot[0, 0, 40:])) > 0.1 * np.max(np.abs(dot[0, 0, 40:]))


def test_delta_one_pass_beyond_the_noalloc_scratch():
    """ttt_la_forward_noalloc at a shape whose chunk inverses (3 KiB per 32 tokens of
    each sequence: 72 MiB here) exceed the 64 MiB scratch runs the one-pass kernel;
    sampled heads against the oracle."""
    import torch
    import ttt_weight_layers_amd as tla
    from _gpu import from_device
    w = DELTA.with_shape(B=1, H=12, T=65536).with_settings(d_k=64, d_v=64, d_phi=64)
    assert w.B * w.H * (w.T // 32) * 3072 > tla.TTT_LA_NOALLOC_SCRATCH_BYTES
    heads = [0, 7]
    say(f"[delta one-pass] {w.B}x{w.H}x{w.T} d=64 heads {heads}")
    x = make_inputs(w)
    d_ = to_device(x)
    desc = tla.make_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.d_phi, dtype=w.dtype, phi=w.phi, chunk=w.chunk)
    o = torch.empty_like(d_["v"])
    st = tla.ttt_la_forward_noalloc(desc, None, d_["q"].data_ptr(), d_["k"].data_ptr(), d_["v"].data_ptr(),
                                    d_["a"].data_ptr(), w.eta_scalar, w.beta, tla.mode_bits(w.eta_mode, True, "mse"),
                                    o.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == tla.TTT_LA_OK, tla.ttt_la_status_string(st)
    torch.cuda.synchronize()
    got = select_heads(from_device(o, w.dtype), w, heads)
    ref = run_oracle(w, x, heads=heads)
    err = oracle.rel_err(got, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL[w.dtype]

