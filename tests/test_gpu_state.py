"""GPU parity of the state-carrying calls against the oracle: the causal forward
from an entry state (S0, M0) with the final state written out, and the
one-token recurrent step (decode).  Every expectation comes from the fp64
oracle on the same seeded inputs."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, to_device

pytestmark = pytest.mark.gpu

STATE_TOL = {"f32": 1e-4, "bf16": 2e-2}     # max |gpu - oracle| / max |oracle| of S_T, M_T


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, **kw):
    return WORKLOADS[name].with_shape(**kw)


def entry_state(w, seed, scale=0.05):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((w.B, w.H, w.d_v, w.d_phi)) * scale
    M0 = rng.standard_normal((w.B, w.H, w.d_v, w.d_phi)) * scale
    return S0.astype(np.float32), M0.astype(np.float32)


def dev32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def oracle_state(w, x, S0=None, M0=None, T0=0, T1=None):
    sl = lambda t: None if t is None else t[:, :, T0:T1]
    return oracle.forward(sl(x.q64), sl(x.k64), sl(x.v64), eta_mode=w.eta_mode, eta=sl(x.a32),
                          eta_scalar=w.eta_scalar, beta=w.beta, phi=w.phi, w1=x.w1_64, w3=x.w3_64,
                          S0=None if S0 is None else S0.astype(np.float64),
                          M0=None if M0 is None else M0.astype(np.float64), return_state=True)


def forward_state(lay, w, d, S0=None, M0=None, S_T=None, M_T=None, T0=0, T1=None):
    import torch
    sl = lambda t: None if t is None else t[:, :, T0:T1].contiguous()
    o = lay.forward_state(sl(d["q"]), sl(d["k"]), sl(d["v"]), eta=sl(d["a"]), eta_scalar=w.eta_scalar,
                          beta=w.beta, eta_mode=w.eta_mode, S0=S0, M0=M0, S_T=S_T, M_T=M_T)
    torch.cuda.synchronize()
    return from_device(o, w.dtype)


@pytest.mark.parametrize("eta_mode,beta,segments", [("scalar", 0.9, 4), ("softplus", 0.9, 3),
                                                    ("per_token", 0.0, 1), ("scalar", 0.9, 1)])
def test_forward_state_wide_tiles(eta_mode, beta, segments):
    # d = 128 identity map: the 32x32-tile kernels; ragged last chunk
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=64 * 9 + 3).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[state wide] {eta_mode} beta={beta} segments={segments}")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=segments)
    assert lay.plan().path == 2
    S0, M0 = entry_state(w, 5)
    S_T = dev32(np.zeros_like(S0))
    M_T = dev32(np.zeros_like(M0))
    got = forward_state(lay, w, d, dev32(S0), dev32(M0), S_T, M_T)
    o, S, M = oracle_state(w, x, S0, M0)
    assert oracle.rel_err(got, o) <= TOL[w.dtype]
    assert oracle.rel_err(S_T.cpu().numpy(), S) <= STATE_TOL[w.dtype]
    assert oracle.rel_err(M_T.cpu().numpy(), M) <= STATE_TOL[w.dtype]


def test_forward_state_split_summary():
    # two segments of 20 chunks on two sequences: segment 0 is summarised in two
    # halves, the scan starts from the carried state in slot 0
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=64 * 40 - 13).with_settings(eta_mode="softplus", beta=0.9)
    say("[state split summary]")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=2)
    assert lay.plan().path == 2 and lay.plan().segments == 2
    S0, M0 = entry_state(w, 9)
    S_T = dev32(np.zeros_like(S0))
    M_T = dev32(np.zeros_like(M0))
    got = forward_state(lay, w, d, dev32(S0), dev32(M0), S_T, M_T)
    o, S, M = oracle_state(w, x, S0, M0)
    assert oracle.rel_err(got, o) <= TOL[w.dtype]
    assert oracle.rel_err(S_T.cpu().numpy(), S) <= STATE_TOL[w.dtype]
    assert oracle.rel_err(M_T.cpu().numpy(), M) <= STATE_TOL[w.dtype]


def test_forward_state_in_place_and_chained():
    # the final state overwrites the entry state; two calls over the halves of a
    # sequence equal one call over all of it
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=64 * 8 + 17).with_settings(eta_mode="softplus")
    say("[state chain]")
    x = make_inputs(w)
    d = to_device(x)
    cut = 64 * 5 + 9
    # a handle is bound to one sequence length: one per part
    lay1 = make_layer(w.with_shape(T=cut), d, segments=4)
    lay2 = make_layer(w.with_shape(T=w.T - cut), d, segments=2)
    S = dev32(np.zeros((w.B, w.H, w.d_v, w.d_phi)))
    M = dev32(np.zeros((w.B, w.H, w.d_v, w.d_phi)))
    o1 = forward_state(lay1, w, d, None, None, S, M, 0, cut)
    o2 = forward_state(lay2, w, d, S, M, S, M, cut, None)
    o, S_ref, M_ref = oracle_state(w, x)
    assert oracle.rel_err(np.concatenate([o1, o2], axis=2), o) <= TOL[w.dtype]
    assert oracle.rel_err(S.cpu().numpy(), S_ref) <= STATE_TOL[w.dtype]
    assert oracle.rel_err(M.cpu().numpy(), M_ref) <= STATE_TOL[w.dtype]


@pytest.mark.parametrize("case", ["f32_d64", "bf16_swiglu", "bf16_d64"])
def test_forward_state_other_shapes(case):
    if case == "f32_d64":
        w = small("v5_f32_1x1x256_d64", B=1, H=2, T=90).with_settings(eta_mode="softplus", beta=0.5)
    elif case == "bf16_swiglu":
        w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=70).with_settings(d_phi=256)
    else:
        w = small("bidir_vit_256x6x196_d64", B=1, H=2, T=75).with_settings(causal=True, beta=0.9)
    say(f"[state {case}]")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    S0, M0 = entry_state(w, 6)
    S_T = dev32(np.zeros_like(S0))
    M_T = dev32(np.zeros_like(M0))
    got = forward_state(lay, w, d, dev32(S0), dev32(M0), S_T, M_T)
    o, S, M = oracle_state(w, x, S0, M0)
    assert oracle.rel_err(got, o) <= TOL[w.dtype]
    assert oracle.rel_err(S_T.cpu().numpy(), S) <= STATE_TOL[w.dtype]
    assert oracle.rel_err(M_T.cpu().numpy(), M) <= STATE_TOL[w.dtype]


def test_forward_state_zero_entry_equals_forward():
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=300)
    say("[state zero entry]")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=2)
    got = forward_state(lay, w, d)
    assert oracle.rel_err(got, oracle_state(w, x)[0]) <= TOL[w.dtype]


def test_forward_state_unsupported_on_prefix_plan():
    import ttt_weight_layers_amd as tla
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=256)
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=2, launch="prefix")
    with pytest.raises(tla.TTTError) as e:
        forward_state(lay, w, d)
    assert e.value.status == tla.TTT_LA_ERR_UNSUPPORTED


def run_steps(lay, w, d, S, M, t0, t1):
    """Decode tokens t0 .. t1-1 one at a time; returns [B, H, t1-t0, d_v] fp64."""
    import torch
    outs = []
    for t in range(t0, t1):
        tok = lambda a: a[:, :, t:t + 1].contiguous()
        eta = None if d["a"] is None else d["a"][:, :, t].contiguous()
        o = lay.step(tok(d["q"]), tok(d["k"]), tok(d["v"]), S, M, eta=eta, eta_scalar=w.eta_scalar,
                     beta=w.beta, eta_mode=w.eta_mode)
        outs.append(o)
    torch.cuda.synchronize()
    return np.concatenate([from_device(o, w.dtype) for o in outs], axis=2)


@pytest.mark.parametrize("case", ["bf16_d128_momentum", "f32_d64_softplus", "bf16_swiglu_per_token",
                                  "bf16_swiglu_dk64", "f32_swiglu"])
def test_step_matches_recurrence(case):
    if case == "bf16_d128_momentum":
        w = small("v4_momentum_4x8x2048_d128", B=2, H=2, T=6)
    elif case == "f32_d64_softplus":
        w = small("v5_f32_1x1x256_d64", B=2, H=2, T=6).with_settings(eta_mode="softplus", beta=0.9)
    elif case == "bf16_swiglu_dk64":
        # the matrix-core features with four k-steps; d_v = 64 takes 32 rows a workgroup
        w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=4).with_settings(d_k=64, d_v=64, d_phi=256)
    elif case == "f32_swiglu":
        # fp32 features as dot products
        w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=4).with_settings(dtype="f32", d_phi=128)
    else:
        w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=5).with_settings(eta_mode="per_token")
    say(f"[step {case}]")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    S0, M0 = entry_state(w, 7)
    S, M = dev32(S0), dev32(M0)
    got = run_steps(lay, w, d, S, M, 0, w.T)
    o, S_ref, M_ref = oracle_state(w, x, S0, M0)
    assert oracle.rel_err(got, o) <= TOL[w.dtype]
    # fp32 arithmetic on the exact inputs: the state itself is fp32-accurate
    assert oracle.rel_err(S.cpu().numpy(), S_ref) <= 1e-4
    assert oracle.rel_err(M.cpu().numpy(), M_ref) <= 1e-4


def test_prefill_then_decode():
    # chunked forward over the prompt with the final state written out, then the
    # remaining tokens decoded one by one, equals the recurrence over everything
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=64 * 6 + 5)
    say("[prefill -> decode]")
    x = make_inputs(w)
    d = to_device(x)
    cut = w.T - 4
    lay = make_layer(w.with_shape(T=cut), d, segments=2)
    S = dev32(np.zeros((w.B, w.H, w.d_v, w.d_phi)))
    M = dev32(np.zeros((w.B, w.H, w.d_v, w.d_phi)))
    o1 = forward_state(lay, w, d, None, None, S, M, 0, cut)
    o2 = run_steps(lay, w, d, S, M, cut, w.T)
    o, S_ref, M_ref = oracle_state(w, x)
    assert oracle.rel_err(np.concatenate([o1, o2], axis=2), o) <= TOL[w.dtype]
    assert oracle.rel_err(S.cpu().numpy(), S_ref) <= STATE_TOL[w.dtype]
    assert oracle.rel_err(M.cpu().numpy(), M_ref) <= STATE_TOL[w.dtype]


def test_step_full_width_batch():
    # the decode shape of the 4x8 momentum workload: every (b, h), two steps
    w = small("v4_momentum_4x8x2048_d128", T=2)
    say("[step full batch]")
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    S0, M0 = entry_state(w, 8)
    S, M = dev32(S0), dev32(M0)
    got = run_steps(lay, w, d, S, M, 0, 2)
    o, S_ref, M_ref = oracle_state(w, x, S0, M0)
    assert oracle.rel_err(got, o) <= TOL[w.dtype]
    assert oracle.rel_err(S.cpu().numpy(), S_ref) <= 1e-4
