"""Seeded sweeps of the state-carrying calls against the oracle: the causal
forward from an entry state with the final state written out (which state
pointers are given, in place or not, varies per case), and the one-token
recurrent step over a few tokens.  The case lists are drawn once from fixed
seeds; each case's id names its settings."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, to_device

pytestmark = pytest.mark.gpu

STATE_TOL = {"f32": 1e-4, "bf16": 2e-2}


def _shape(rng, kind, t_max):
    c = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), T=int(rng.integers(1, t_max)),
             eta_mode=str(rng.choice(["scalar", "per_token", "softplus"])),
             beta=float(rng.choice([0.0, 0.5, 0.9, 0.99])))
    if kind == "wide":
        c.update(base="v4_momentum_4x8x2048_d128", d_k=128, d_v=128, d_phi=128, phi="identity", dtype="bf16")
    elif kind == "tile":
        d_k, d_v = [int(x) for x in rng.choice([64, 128], size=2)]
        c.update(base="bidir_vit_256x6x196_d64", d_k=d_k, d_v=d_v, d_phi=d_k, phi="identity", dtype="bf16")
    elif kind == "swiglu":
        d_k, d_v = [int(x) for x in rng.choice([64, 128], size=2)]
        c.update(base="v2_swiglu_4x16x8192_d128_f512", d_k=d_k, d_v=d_v, d_phi=int(rng.choice([128, 256])),
                 phi="swiglu", dtype=str(rng.choice(["bf16", "f32"])), T=min(c["T"], 300))
    else:
        c.update(base="v5_f32_1x1x256_d64", d_k=64, d_v=64, d_phi=64, phi="identity", dtype="f32",
                 T=min(c["T"], 200))
    return c


def _forward_cases(n=40, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kind = str(rng.choice(["wide", "wide", "tile", "swiglu", "f32"]))
        c = _shape(rng, kind, 700)
        c["segments"] = int(rng.choice([0, 1, 2, 3, 5])) if kind in ("wide", "tile") else 0
        c["io"] = str(rng.choice(["full", "in_place", "no_m0", "out_only"]))
        out.append(c)
    return out


def _step_cases(n=24, seed=20261205):
    rng = np.random.default_rng(seed)
    return [_shape(rng, str(rng.choice(["wide", "tile", "swiglu", "f32"])), 6) for _ in range(n)]


def _id(c):
    s = (f"{c['dtype']}_{c['phi'][:2]}{c['d_k']}x{c['d_v']}f{c['d_phi']}_{c['B']}x{c['H']}x{c['T']}"
         f"_{c['eta_mode'][:4]}_b{c['beta']}")
    if "io" in c:
        s += f"_s{c['segments']}_{c['io']}"
    return s


FORWARD_CASES = _forward_cases()
STEP_CASES = _step_cases()


def _workload(c):
    base = WORKLOADS[c["base"]]
    return base.with_shape(B=c["B"], H=c["H"], T=c["T"]).with_settings(
        d_k=c["d_k"], d_v=c["d_v"], d_phi=c["d_phi"], phi=c["phi"], dtype=c["dtype"], eta_mode=c["eta_mode"],
        beta=c["beta"], causal=True, eta_scalar=0.3 if c["eta_mode"] == "scalar" else base.eta_scalar)


def _entry(w, seed):
    rng = np.random.default_rng(seed)
    shape = (w.B, w.H, w.d_v, w.d_phi)
    return (rng.standard_normal(shape) * 0.05).astype(np.float32), (rng.standard_normal(shape) * 0.05).astype(
        np.float32)


def _dev32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def _oracle(w, x, S0, M0, loss="dot"):
    return oracle.forward(x.q64, x.k64, x.v64, eta_mode=w.eta_mode, eta=x.a32, eta_scalar=w.eta_scalar,
                          beta=w.beta, phi=w.phi, w1=x.w1_64, w3=x.w3_64,
                          S0=None if S0 is None else S0.astype(np.float64),
                          M0=None if M0 is None else M0.astype(np.float64), return_state=True, loss=loss)


@pytest.mark.parametrize("c", FORWARD_CASES, ids=[_id(c) for c in FORWARD_CASES])
def test_forward_state_sweep(c):
    import torch
    w = _workload(c)
    print(f"[state sweep] {_id(c)}", flush=True)
    sys.stdout.flush()
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d, segments=c["segments"])
    S0, M0 = _entry(w, 11)
    io = c["io"]
    if io == "out_only":
        S0 = M0 = None
    elif io == "no_m0":
        M0 = None
    s0 = None if S0 is None else _dev32(S0)
    m0 = None if M0 is None else _dev32(M0)
    zeros = np.zeros((w.B, w.H, w.d_v, w.d_phi), np.float32)
    s_t, m_t = (s0, m0) if io == "in_place" else (_dev32(zeros), _dev32(zeros))
    o = lay.forward_state(d["q"], d["k"], d["v"], eta=d["a"], eta_scalar=w.eta_scalar, beta=w.beta,
                          eta_mode=w.eta_mode, S0=s0, M0=m0, S_T=s_t, M_T=m_t)
    torch.cuda.synchronize()
    ref_o, ref_S, ref_M = _oracle(w, x, S0, M0)
    assert oracle.rel_err(from_device(o, w.dtype), ref_o) <= TOL[w.dtype]
    assert oracle.rel_err(s_t.cpu().numpy(), ref_S) <= STATE_TOL[w.dtype]
    assert oracle.rel_err(m_t.cpu().numpy(), ref_M) <= STATE_TOL[w.dtype]


@pytest.mark.parametrize("c", STEP_CASES, ids=[_id(c) for c in STEP_CASES])
def test_step_sweep(c):
    _step_sweep(c, "dot")


# the delta-rule step (mean-squared loss) over the same space of shapes, rates and momentum
MSE_STEP_CASES = _step_cases(n=16, seed=20261206)


@pytest.mark.parametrize("c", MSE_STEP_CASES, ids=[_id(c) for c in MSE_STEP_CASES])
def test_step_sweep_mse(c):
    _step_sweep(c, "mse")


def _step_sweep(c, loss):
    import torch
    w = _workload(c)
    print(f"[step sweep {loss}] {_id(c)}", flush=True)
    sys.stdout.flush()
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    S0, M0 = _entry(w, 12)
    S, M = _dev32(S0), _dev32(M0)
    outs = []
    for t in range(w.T):
        tok = lambda a: a[:, :, t:t + 1].contiguous()
        eta = None if d["a"] is None else d["a"][:, :, t].contiguous()
        outs.append(lay.step(tok(d["q"]), tok(d["k"]), tok(d["v"]), S, M, eta=eta, eta_scalar=w.eta_scalar,
                             beta=w.beta, eta_mode=w.eta_mode, loss=loss))
    torch.cuda.synchronize()
    got = np.concatenate([from_device(o, w.dtype) for o in outs], axis=2)
    ref_o, ref_S, ref_M = _oracle(w, x, S0, M0, loss)
    assert oracle.rel_err(got, ref_o) <= TOL[w.dtype]
    # fp32 arithmetic on the exact inputs: the state is fp32-accurate
    assert oracle.rel_err(S.cpu().numpy(), ref_S) <= 1e-4
    assert oracle.rel_err(M.cpu().numpy(), ref_M) <= 1e-4
