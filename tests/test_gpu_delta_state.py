"""GPU parity of the delta rule's carried state (TTT_LA_LOSS_MSE through
ttt_la_forward_state: S0 in, S_T out) and of its one-token recurrent step
(ttt_la_step with TTT_LA_LOSS_MSE, momentum allowed) against the oracle's
loss="mse" recurrence and step on seeded inputs: outputs at the bf16 or fp32
bar, final states, in-place state, a chunk-ragged prefill cut and prefill ->
decode."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, to_device

pytestmark = pytest.mark.gpu

STATE_TOL = {"f32": 1e-4, "bf16": 2e-2}

# the Variant-3 shape with momentum off and L2-normalised tokens (every step a
# contraction along k), as the delta-rule forward parity uses
DELTA = WORKLOADS["v3_softplus_8x16x4096_d128"].with_settings(
    name="v3_delta_8x16x4096_d128", loss="mse", beta=0.0, l2norm=True)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def entry_state(B, H, d_v, d_phi, seed, scale):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, d_v, d_phi)) * scale).astype(np.float32)


def delta_case(d, eta_mode, eta_scalar, B, H, T):
    return DELTA.with_shape(B=B, H=H, T=T).with_settings(d_k=d, d_v=d, d_phi=d, eta_mode=eta_mode,
                                                        eta_scalar=eta_scalar)


def sl(t, T0, T1):
    return None if t is None else t[:, :, T0:T1].contiguous()


def gpu_forward_state(lay, w, d, S0, S_T, T0=0, T1=None):
    import torch
    o = lay.forward_state(sl(d["q"], T0, T1), sl(d["k"], T0, T1), sl(d["v"], T0, T1), eta=sl(d["a"], T0, T1),
                          eta_scalar=w.eta_scalar, beta=0.0, eta_mode=w.eta_mode, S0=S0, S_T=S_T, loss="mse")
    torch.cuda.synchronize()
    return from_device(o, w.dtype)


def oracle_delta(w, x, S0, T0=0, T1=None):
    s = lambda t: None if t is None else t[:, :, T0:T1]
    return oracle.forward(s(x.q64), s(x.k64), s(x.v64), eta_mode=w.eta_mode, eta=s(x.a32),
                          eta_scalar=w.eta_scalar, beta=0.0, S0=None if S0 is None else S0.astype(np.float64),
                          loss="mse", return_state=True)


@pytest.mark.parametrize("d,eta_mode,eta_scalar,B,H,T,with_s0,with_st", [
    (128, "softplus", 0.0, 2, 2, 300, True, True),
    (64, "scalar", 0.5, 1, 3, 32 * 3 + 5, True, True),
    (128, "per_token", 0.0, 1, 2, 31, False, True),
    (64, "softplus", 0.0, 2, 1, 1, True, False),
    (128, "scalar", 1.0, 1, 1, 64, True, True),
])
def test_delta_forward_state_parity(d, eta_mode, eta_scalar, B, H, T, with_s0, with_st):
    import torch
    w = delta_case(d, eta_mode, eta_scalar, B, H, T)
    say(f"[delta state] d={d} {eta_mode} {B}x{H}x{T} S0={with_s0} S_T={with_st}")
    x = make_inputs(w)
    dd = to_device(x)
    lay = make_layer(w, dd)
    S0 = entry_state(B, H, d, d, 31 + T, 1.0 / np.sqrt(d)) if with_s0 else None
    S_T = torch.full((B, H, d, d), float("nan"), device="cuda") if with_st else None
    got = gpu_forward_state(lay, w, dd, None if S0 is None else dev32(S0), S_T)
    ref_o, ref_S, _ = oracle_delta(w, x, S0)
    err = oracle.rel_err(got, ref_o)
    say(f"  o rel err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL[w.dtype]
    if with_st:
        got_S = S_T.cpu().numpy().astype(np.float64)
        err_s = oracle.rel_err(got_S, ref_S)
        say(f"  S_T rel err {err_s:.3e}")
        assert np.all(np.isfinite(got_S)) and err_s <= STATE_TOL[w.dtype]
    if not with_s0:
        # a zero entry state is the plain forward, bit for bit
        plain = lay.forward(dd["q"], dd["k"], dd["v"], eta=dd["a"], eta_scalar=w.eta_scalar, beta=0.0,
                            eta_mode=w.eta_mode, loss="mse")
        torch.cuda.synchronize()
        assert np.array_equal(from_device(plain, w.dtype), got)


def test_delta_state_in_place():
    w = delta_case(128, "softplus", 0.0, 1, 2, 32 * 4 + 9)
    say("[delta state in place]")
    x = make_inputs(w)
    dd = to_device(x)
    lay = make_layer(w, dd)
    S0 = entry_state(w.B, w.H, 128, 128, 5, 1.0 / np.sqrt(128))
    out_of_place = dev32(np.zeros_like(S0))
    o1 = gpu_forward_state(lay, w, dd, dev32(S0), out_of_place)
    S = dev32(S0)
    o2 = gpu_forward_state(lay, w, dd, S, S)
    assert np.array_equal(o1, o2)
    assert np.array_equal(S.cpu().numpy(), out_of_place.cpu().numpy())


def test_delta_prefill_cut_then_decode():
    # a prompt cut off the chunk grid, prefilled in two calls that carry S, then
    # decoded token by token with the delta-rule step: the oracle's recurrence
    # over the whole sequence from the same entry state
    import torch
    w = delta_case(128, "softplus", 0.0, 2, 2, 32 * 5 + 11)
    say("[delta prefill -> decode]")
    x = make_inputs(w)
    dd = to_device(x)
    cut1, cut2 = 32 * 2 + 3, w.T - 5
    lay1 = make_layer(w.with_shape(T=cut1), dd)
    lay2 = make_layer(w.with_shape(T=cut2 - cut1), dd)
    S0 = entry_state(w.B, w.H, 128, 128, 9, 1.0 / np.sqrt(128))
    S = dev32(S0)
    M = dev32(np.zeros_like(S0))
    o1 = gpu_forward_state(lay1, w, dd, S, S, 0, cut1)
    o2 = gpu_forward_state(lay2, w, dd, S, S, cut1, cut2)
    outs = []
    for t in range(cut2, w.T):
        tok = lambda a: a[:, :, t:t + 1].contiguous()
        o = lay2.step(tok(dd["q"]), tok(dd["k"]), tok(dd["v"]), S, M, eta=dd["a"][:, :, t].contiguous(),
                      eta_scalar=w.eta_scalar, beta=0.0, eta_mode=w.eta_mode, loss="mse")
        outs.append(from_device(o, w.dtype))
    torch.cuda.synchronize()
    got = np.concatenate([o1, o2] + outs, axis=2)
    ref_o, ref_S, _ = oracle_delta(w, x, S0)
    err = oracle.rel_err(got, ref_o)
    say(f"  o rel err {err:.3e}")
    assert err <= TOL[w.dtype]
    assert oracle.rel_err(S.cpu().numpy().astype(np.float64), ref_S) <= STATE_TOL[w.dtype]


STEP_CASES = [
    # (name, base workload, settings, beta, eta_mode)
    ("bf16_d128_momentum", "delta", dict(d_k=128, d_v=128, d_phi=128), 0.9, "softplus"),
    ("f32_d64_plain", "delta", dict(dtype="f32", d_k=64, d_v=64, d_phi=64), 0.0, "scalar"),
    ("bf16_dk64_dv128", "delta", dict(d_k=64, d_v=128, d_phi=64), 0.5, "per_token"),
    ("bf16_swiglu_512", "swiglu", dict(), 0.9, "softplus"),
    ("f32_swiglu_128", "swiglu", dict(dtype="f32", d_phi=128), 0.9, "scalar"),
]


@pytest.mark.parametrize("name,base,settings,beta,eta_mode", STEP_CASES)
def test_delta_step_parity(name, base, settings, beta, eta_mode):
    import torch
    n_steps = 6
    src = DELTA if base == "delta" else WORKLOADS["v2_swiglu_4x16x8192_d128_f512"]
    w = src.with_shape(B=2, H=2, T=n_steps).with_settings(beta=beta, eta_mode=eta_mode, eta_scalar=0.4,
                                                          **settings)
    say(f"[delta step {name}]")
    x = make_inputs(w)
    dd = to_device(x)
    lay = make_layer(w, dd)
    S0 = entry_state(w.B, w.H, w.d_v, w.d_phi, 13, 0.3)
    M0 = entry_state(w.B, w.H, w.d_v, w.d_phi, 14, 0.05) if beta else np.zeros_like(S0)
    S, M = dev32(S0), dev32(M0)
    Sr, Mr = S0.astype(np.float64), M0.astype(np.float64)
    for t in range(n_steps):
        tok = lambda a: a[:, :, t:t + 1].contiguous()
        eta = None if dd["a"] is None else dd["a"][:, :, t].contiguous()
        o = lay.step(tok(dd["q"]), tok(dd["k"]), tok(dd["v"]), S, M, eta=eta, eta_scalar=w.eta_scalar,
                     beta=beta, eta_mode=w.eta_mode, loss="mse")
        torch.cuda.synchronize()
        e_t = None if x.a32 is None else x.a32[:, :, t]
        o_ref, Sr, Mr = oracle.step(x.q64[:, :, t], x.k64[:, :, t], x.v64[:, :, t], Sr, Mr, eta_mode=w.eta_mode,
                                    eta=e_t, eta_scalar=w.eta_scalar, beta=beta, phi=w.phi, w1=x.w1_64,
                                    w3=x.w3_64, loss="mse")
        got = from_device(o, w.dtype)[:, :, 0]
        err = oracle.rel_err(got, o_ref)
        assert np.all(np.isfinite(got)) and err <= TOL[w.dtype], (t, err)
    # fp32 arithmetic on the exact inputs: the state is fp32-accurate
    err_s = oracle.rel_err(S.cpu().numpy().astype(np.float64), Sr)
    err_m = oracle.rel_err(M.cpu().numpy().astype(np.float64), Mr)
    say(f"  S rel err {err_s:.2e}, M rel err {err_m:.2e}")
    assert err_s <= 1e-4 and err_m <= 1e-4
    # the dot-product step of the same kernel family from the same state still follows its own rule
    Sd, Md = dev32(S0), dev32(M0)
    eta0 = None if dd["a"] is None else dd["a"][:, :, 0].contiguous()
    tok0 = lambda a: a[:, :, 0:1].contiguous()
    lay.step(tok0(dd["q"]), tok0(dd["k"]), tok0(dd["v"]), Sd, Md, eta=eta0, eta_scalar=w.eta_scalar,
             beta=beta, eta_mode=w.eta_mode)
    _, Sd_ref, _ = oracle.step(x.q64[:, :, 0], x.k64[:, :, 0], x.v64[:, :, 0], S0.astype(np.float64),
                               M0.astype(np.float64), eta_mode=w.eta_mode,
                               eta=None if x.a32 is None else x.a32[:, :, 0], eta_scalar=w.eta_scalar,
                               beta=beta, phi=w.phi, w1=x.w1_64, w3=x.w3_64)
    torch.cuda.synchronize()
    assert oracle.rel_err(Sd.cpu().numpy().astype(np.float64), Sd_ref) <= 1e-4


def test_delta_state_rejects_momentum_buffers():
    import torch
    import ttt_weight_layers_amd as tla
    w = delta_case(64, "scalar", 0.5, 1, 1, 40)
    x = make_inputs(w)
    dd = to_device(x)
    lay = make_layer(w, dd)
    Z = torch.zeros((1, 1, 64, 64), device="cuda")
    with pytest.raises(tla.TTTError) as e:
        lay.forward_state(dd["q"], dd["k"], dd["v"], eta_scalar=0.5, S0=Z, M0=Z.clone(), loss="mse")
    assert e.value.status == tla.TTT_LA_ERR_INVALID_ARG
    with pytest.raises(tla.TTTError) as e:
        lay.forward_state(dd["q"], dd["k"], dd["v"], eta_scalar=0.5, beta=0.5, S0=Z, loss="mse")
    assert e.value.status == tla.TTT_LA_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_delta_forward_state_full_shape():
    # the 8 x 16 x 4096 workload from a drawn entry state, eight heads (the first
    # and the last among them) against the oracle at full T, outputs and final state
    import torch
    from ttt_workloads import head_subset
    w = DELTA
    heads = head_subset(w, 8)
    say(f"[delta state full] heads {heads}")
    x = make_inputs(w)
    dd = to_device(x)
    lay = make_layer(w, dd)
    S0 = entry_state(w.B, w.H, 128, 128, 3, 1.0 / np.sqrt(128))
    S_T = torch.full_like(dev32(S0), float("nan"))
    got = gpu_forward_state(lay, w, dd, dev32(S0), S_T)
    got_S = S_T.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got_S))
    for n in heads:
        b, h = divmod(n, w.H)
        sub = lambda t: None if t is None else t[b:b + 1, h:h + 1]
        ref_o, ref_S, _ = oracle.forward(sub(x.q64), sub(x.k64), sub(x.v64), eta_mode=w.eta_mode, eta=sub(x.a32),
                                         beta=0.0, S0=S0[b:b + 1, h:h + 1].astype(np.float64), loss="mse",
                                         return_state=True)
        e_o = oracle.rel_err(got[b:b + 1, h:h + 1], ref_o)
        e_s = oracle.rel_err(got_S[b:b + 1, h:h + 1], ref_S)
        say(f"  head ({b},{h}): o {e_o:.2e}, S_T {e_s:.2e}")
        assert e_o <= TOL[w.dtype] and e_s <= STATE_TOL[w.dtype]
