"""GPU parity of ttt_la_backward_swiglu (gradients through the SwiGLU feature map,
and of W1, W3) against the oracle's backward on the same seeded inputs and output
gradient, at the Variant-2 shape (d = 128) with reduced lengths."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, to_device
from test_gpu_backward import grad_output

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("d_phi,eta_mode,beta,causal,B,H,T", [
    (512, "softplus", 0.9, True, 1, 2, 64 * 3 + 11),
    (256, "per_token", 0.0, True, 2, 2, 130),
    (256, "scalar", 0.5, False, 2, 1, 100),
    (128, "softplus", 0.9, True, 1, 2, 37),
    (512, "softplus", 0.0, False, 1, 2, 64 * 2 + 5),
    # dW over several token ranges of 138 tokens (ragged 32-token panels) per sequence
    (512, "softplus", 0.9, True, 1, 1, 1100),
])
def test_swiglu_backward_parity(d_phi, eta_mode, beta, causal, B, H, T):
    import torch
    w = WORKLOADS["v2_swiglu_4x16x8192_d128_f512"].with_shape(B=B, H=H, T=T).with_settings(
        d_phi=d_phi, eta_mode=eta_mode, beta=beta, causal=causal,
        eta_scalar=0.3 if eta_mode == "scalar" else 0.0)
    say(f"[swiglu backward] d_phi={d_phi} {eta_mode} beta={beta} causal={causal} {B}x{H}x{T}")
    x = make_inputs(w)
    d = to_device(x)
    dO, dO64 = grad_output(w, 41)
    lay = make_layer(w, d)
    dq, dk, dv, de, dw1, dw3 = lay.backward(d["q"], d["k"], d["v"], dO, eta=d["a"], eta_scalar=w.eta_scalar,
                                            beta=w.beta, eta_mode=w.eta_mode, causal=w.causal)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q64, x.k64, x.v64, dO64, eta_mode=w.eta_mode, eta=x.a32, eta_scalar=w.eta_scalar,
                          beta=w.beta, causal=w.causal, phi="swiglu", w1=x.w1_64, w3=x.w3_64)
    got = {"dq": from_device(dq, "bf16"), "dk": from_device(dk, "bf16"), "dv": from_device(dv, "bf16"),
           "dW1": dw1.cpu().numpy().astype(np.float64), "dW3": dw3.cpu().numpy().astype(np.float64)}
    want = {"dq": ref[0], "dk": ref[1], "dv": ref[2], "dW1": ref[4], "dW3": ref[5]}
    for name in got:
        assert np.all(np.isfinite(got[name])), name
        err = oracle.rel_err(got[name], want[name])
        say(f"  {name} rel err {err:.2e}")
        assert err <= TOL["bf16"], name
    de_np = de.cpu().numpy().astype(np.float64)
    if w.eta_mode == "scalar":
        assert abs(de_np.sum() - ref[3]) <= TOL["bf16"] * max(1.0, np.abs(de_np).sum())
    else:
        err = oracle.rel_err(de_np, ref[3])
        say(f"  deta rel err {err:.2e}")
        assert err <= TOL["bf16"]
