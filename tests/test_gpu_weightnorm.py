"""GPU parity of the weight-normalised recurrence (TTT_LA_WEIGHT_NORM through
ttt_la_forward_state; Variant 1 of Table 2, thelatestinai.com page, with the reading
the oracle documents) against the oracle on seeded inputs: outputs, final state and
momentum buffer, for the identity map (bf16 and fp32) and the SwiGLU map, feature
widths 64 to 512, ragged 16-token chunks, in-place state and zero rows."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


BASE = WORKLOADS["v1_weightnorm_4x16x8192_d128_f512"]

CASES = [
    # (phi, dtype, d_k, d_v, d_phi, eta_mode, beta, B, H, T, with_m0)
    ("identity", "bf16", 128, 128, 128, "softplus", 0.9, 1, 2, 100, True),
    ("identity", "f32", 64, 64, 64, "scalar", 0.0, 2, 1, 37, False),
    ("identity", "bf16", 64, 128, 64, "per_token", 0.5, 1, 1, 45, True),
    ("identity", "f32", 128, 64, 128, "softplus", 0.9, 1, 1, 33, False),
    ("swiglu", "bf16", 128, 128, 512, "softplus", 0.9, 1, 2, 16 * 4 + 9, True),
    ("swiglu", "bf16", 128, 64, 256, "per_token", 0.5, 2, 1, 50, False),
    ("swiglu", "bf16", 128, 64, 128, "scalar", 0.0, 1, 2, 17, True),
]


def _case(phi, dtype, d_k, d_v, d_phi, eta_mode, beta, B, H, T):
    return BASE.with_shape(B=B, H=H, T=T).with_settings(
        phi=phi, dtype=dtype, d_k=d_k, d_v=d_v, d_phi=d_phi, eta_mode=eta_mode, beta=beta,
        eta_scalar=0.4 if eta_mode == "scalar" else 0.0,
        name=f"wn_{phi}_{dtype}_{d_k}x{d_v}x{d_phi}_{eta_mode}_b{beta}_{B}x{H}x{T}")


@pytest.mark.parametrize("phi,dtype,d_k,d_v,d_phi,eta_mode,beta,B,H,T,with_m0", CASES)
def test_weight_norm_parity(phi, dtype, d_k, d_v, d_phi, eta_mode, beta, B, H, T, with_m0):
    import torch
    w = _case(phi, dtype, d_k, d_v, d_phi, eta_mode, beta, B, H, T)
    say(f"[weight norm] {w.name} M0={with_m0}")
    x = make_inputs(w)
    d = to_device(x)
    rng = np.random.default_rng(77)
    M0 = (0.05 * rng.standard_normal((B, H, d_v, d_phi))).astype(np.float32) if with_m0 else None
    S0 = x.S0.copy()
    S0[0, 0, 1] = 0.0                                   # a zero row stays zero
    lay = make_layer(w, d)
    S0_d = torch.from_numpy(S0).cuda()
    M0_d = torch.from_numpy(M0).cuda() if with_m0 else None
    S_T = torch.empty_like(S0_d)
    M_T = torch.empty_like(S0_d)
    o = lay.forward_state(d["q"], d["k"], d["v"], eta=d["a"], eta_scalar=w.eta_scalar, beta=w.beta,
                          eta_mode=w.eta_mode, S0=S0_d, M0=M0_d, S_T=S_T, M_T=M_T, weight_norm=True)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_M = oracle.forward(x.q64, x.k64, x.v64, eta_mode=w.eta_mode, eta=x.a32,
                                         eta_scalar=w.eta_scalar, beta=w.beta, phi=w.phi, w1=x.w1_64,
                                         w3=x.w3_64, S0=S0.astype(np.float64),
                                         M0=None if M0 is None else M0.astype(np.float64),
                                         return_state=True, weight_norm=True)
    got_o = from_device(o, w.dtype)
    got_S = S_T.cpu().numpy().astype(np.float64)
    got_M = M_T.cpu().numpy().astype(np.float64)
    tol = TOL[w.dtype]
    for name, got, ref in (("o", got_o, ref_o), ("S_T", got_S, ref_S), ("M_T", got_M, ref_M)):
        assert np.all(np.isfinite(got)), name
        err = oracle.rel_err(got, ref)
        say(f"  {name} rel err {err:.2e}")
        assert err <= tol, name
    # the normalisation's invariant on the GPU's own final state (fp32 arithmetic)
    n0 = np.linalg.norm(S0.astype(np.float64), axis=-1)
    nT = np.linalg.norm(got_S, axis=-1)
    np.testing.assert_allclose(nT, n0, rtol=2e-5, atol=1e-30)
    assert np.all(got_S[0, 0, 1] == 0.0) and np.all(got_o[0, 0, :, 1] == 0.0)


def test_weight_norm_state_in_place():
    import torch
    w = _case("swiglu", "bf16", 128, 64, 256, "softplus", 0.9, 1, 2, 40)
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    S = torch.from_numpy(x.S0).cuda()
    M = torch.zeros_like(S)
    ref_S, ref_M = S.clone(), M.clone()
    o1 = lay.forward_state(d["q"], d["k"], d["v"], eta=d["a"], beta=w.beta, eta_mode=w.eta_mode, S0=ref_S,
                           M0=ref_M, S_T=torch.empty_like(S), M_T=torch.empty_like(M), weight_norm=True)
    o2 = lay.forward_state(d["q"], d["k"], d["v"], eta=d["a"], beta=w.beta, eta_mode=w.eta_mode, S0=S, M0=M,
                           S_T=S, M_T=M, weight_norm=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    _, want_S, want_M = oracle.forward(x.q64, x.k64, x.v64, eta_mode=w.eta_mode, eta=x.a32, beta=w.beta,
                                       phi=w.phi, w1=x.w1_64, w3=x.w3_64, S0=x.S0.astype(np.float64),
                                       return_state=True, weight_norm=True)
    assert oracle.rel_err(S.cpu().numpy().astype(np.float64), want_S) <= TOL["bf16"]
    assert oracle.rel_err(M.cpu().numpy().astype(np.float64), want_M) <= TOL["bf16"]


def test_weight_norm_needs_the_entry_state():
    import torch
    import ttt_weight_layers_amd as tla
    w = _case("identity", "bf16", 128, 128, 128, "scalar", 0.0, 1, 1, 20)
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    with pytest.raises(tla.TTTError):
        lay.forward_state(d["q"], d["k"], d["v"], eta_scalar=0.5, weight_norm=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("phi,dtype,d_k,d_v,d_phi", [
    ("identity", "bf16", 128, 128, 128), ("identity", "f32", 64, 64, 64), ("swiglu", "bf16", 128, 128, 512),
    ("swiglu", "bf16", 128, 64, 256),
])
def test_weight_norm_steps_follow_the_oracle(phi, dtype, d_k, d_v, d_phi):
    # T decode steps from S0 against the oracle's weight-normalised forward
    import torch
    w = _case(phi, dtype, d_k, d_v, d_phi, "softplus", 0.9, 2, 2, 12)
    say(f"[weight norm step] {w.name}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    S = torch.from_numpy(x.S0).cuda()
    M = torch.zeros_like(S)
    outs = []
    for t in range(w.T):
        sl = lambda a: a[:, :, t:t + 1].contiguous()
        outs.append(lay.step(sl(d["q"]), sl(d["k"]), sl(d["v"]), S, M, eta=d["a"][:, :, t].contiguous(),
                             beta=w.beta, eta_mode=w.eta_mode, weight_norm=True))
    torch.cuda.synchronize()
    got_o = np.concatenate([from_device(o, w.dtype) for o in outs], axis=2)
    ref_o, ref_S, ref_M = oracle.forward(x.q64, x.k64, x.v64, eta_mode=w.eta_mode, eta=x.a32, beta=w.beta,
                                         phi=w.phi, w1=x.w1_64, w3=x.w3_64, S0=x.S0.astype(np.float64),
                                         return_state=True, weight_norm=True)
    tol = TOL[w.dtype]
    for name, got, ref in (("o", got_o, ref_o), ("S", S.cpu().numpy().astype(np.float64), ref_S),
                           ("M", M.cpu().numpy().astype(np.float64), ref_M)):
        err = oracle.rel_err(got, ref)
        say(f"  {name} rel err {err:.2e}")
        assert err <= tol, name
