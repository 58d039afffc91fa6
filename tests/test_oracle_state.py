"""Pins of the oracle's carried state: an entry state (S0, M0), the final state,
and the one-token recurrent step (the recurrent implementation that Table 2 of
the thelatestinai.com page lists beside the parallel one).

Each compares the oracle with an independent computation: a hand-worked
example, closed forms of the geometric sums, and the invariance of the result
under splitting a sequence into calls.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import ttt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, B, H, T, dk, dv):
    return (rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk)),
            rng.standard_normal((B, H, T, dv)))


def test_state_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_state_T2.json")))
    sh = (1, 1, 2, 1)
    q = np.array(g["q"], float).reshape(sh)
    k = np.array(g["k"], float).reshape(sh)
    v = np.array(g["v"], float).reshape(sh)
    eta = np.array(g["eta"], float).reshape(1, 1, 2)
    S0 = np.full((1, 1, 1, 1), g["S0"], float)
    M0 = np.full((1, 1, 1, 1), g["M0"], float)
    o, S, M = oracle.forward(q, k, v, eta_mode="per_token", eta=eta, beta=g["beta"], S0=S0, M0=M0,
                             return_state=True)
    np.testing.assert_array_equal(o.ravel(), g["o"])
    assert S.item() == g["S_T"] and M.item() == g["M_T"]
    # the same by two steps
    Sx, Mx = S0, M0
    for t in range(2):
        ot, Sx, Mx = O.step(q[:, :, t], k[:, :, t], v[:, :, t], Sx, Mx, eta_mode="per_token",
                            eta=eta[:, :, t], beta=g["beta"])
        assert ot.item() == g["o"][t]
    assert Sx.item() == g["S_T"] and Mx.item() == g["M_T"]


@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9])
def test_entry_state_alone_is_a_geometric_readout(beta):
    # with v = 0 no token changes the fast weight's momentum input, so
    # M_t = beta^{t+1} M0 and S_t = S0 + g_t M0 with g_t = beta + ... + beta^{t+1}
    rng = np.random.default_rng(11)
    B, H, T, d = 2, 3, 9, 4
    q, k, _ = _rand(rng, B, H, T, d, d)
    v = np.zeros((B, H, T, 5))
    S0 = rng.standard_normal((B, H, 5, d))
    M0 = rng.standard_normal((B, H, 5, d))
    o, S, M = oracle.forward(q, k, v, eta_scalar=0.7, beta=beta, S0=S0, M0=M0, return_state=True)
    g = np.cumsum(beta ** np.arange(1, T + 1))          # g_t, t = 0..T-1
    ref = np.einsum("bhvf,bhtf->bhtv", S0, q) + g[None, None, :, None] * np.einsum("bhvf,bhtf->bhtv", M0, q)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S0 + g[-1] * M0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M, beta ** T * M0, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_final_state_closed_form(beta):
    # S_T = sum_j eta_j c_{T-1-j} v_j k_j^T, M_T = sum_j eta_j beta^{T-1-j} v_j k_j^T
    rng = np.random.default_rng(12)
    B, H, T, dk, dv = 1, 2, 13, 3, 4
    q, k, v = _rand(rng, B, H, T, dk, dv)
    a = rng.standard_normal((B, H, T))
    _, S, M = oracle.forward(q, k, v, eta_mode="softplus", eta=a, beta=beta, return_state=True)
    eta = np.log1p(np.exp(a))
    back = T - 1 - np.arange(T)
    c = np.array([sum(beta ** u for u in range(r + 1)) for r in back])
    w_s = eta * c[None, None, :]
    w_m = eta * (beta ** back)[None, None, :]
    np.testing.assert_allclose(S, np.einsum("bht,bhtv,bhtf->bhvf", w_s, v, k), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M, np.einsum("bht,bhtv,bhtf->bhvf", w_m, v, k), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("phi,eta_mode,beta", [("identity", "scalar", 0.9), ("identity", "softplus", 0.5),
                                               ("swiglu", "per_token", 0.9), ("identity", "per_token", 0.0)])
def test_split_calls_equal_one_call(phi, eta_mode, beta):
    # carrying (S, M) from one call to the next gives the single-call result
    rng = np.random.default_rng(13)
    B, H, T, dk, dv = 2, 2, 17, 4, 3
    q, k, v = _rand(rng, B, H, T, dk, dv)
    eta = rng.standard_normal((B, H, T)) if eta_mode != "scalar" else None
    kw = dict(eta_mode=eta_mode, eta_scalar=0.3, beta=beta, phi=phi)
    if phi == "swiglu":
        kw.update(w1=rng.standard_normal((H, 6, dk)) / 2, w3=rng.standard_normal((H, 6, dk)) / 2)
    o, S, M = oracle.forward(q, k, v, eta=eta, return_state=True, **kw)
    for cut in (1, 7, 16):
        sl = lambda x, a, b: None if x is None else x[:, :, a:b]
        o1, S1, M1 = oracle.forward(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], eta=sl(eta, 0, cut),
                                    return_state=True, **kw)
        o2, S2, M2 = oracle.forward(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], eta=sl(eta, cut, T),
                                    return_state=True, S0=S1, M0=M1, **kw)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S2, S, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(M2, M, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("phi,eta_mode,beta", [("identity", "scalar", 0.9), ("swiglu", "softplus", 0.9),
                                               ("identity", "per_token", 0.0)])
def test_steps_equal_forward(phi, eta_mode, beta):
    rng = np.random.default_rng(14)
    B, H, T, dk, dv = 2, 2, 6, 4, 3
    q, k, v = _rand(rng, B, H, T, dk, dv)
    eta = rng.standard_normal((B, H, T)) if eta_mode != "scalar" else None
    kw = dict(eta_mode=eta_mode, eta_scalar=0.4, beta=beta, phi=phi)
    if phi == "swiglu":
        kw.update(w1=rng.standard_normal((H, 5, dk)) / 2, w3=rng.standard_normal((H, 5, dk)) / 2)
    S0 = rng.standard_normal((B, H, dv, 5 if phi == "swiglu" else dk))
    M0 = rng.standard_normal(S0.shape)
    o, S, M = oracle.forward(q, k, v, eta=eta, S0=S0, M0=M0, return_state=True, **kw)
    Sx, Mx = S0, M0
    for t in range(T):
        ot, Sx, Mx = O.step(q[:, :, t], k[:, :, t], v[:, :, t], Sx, Mx,
                            eta=None if eta is None else eta[:, :, t], **kw)
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sx, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Mx, M, rtol=1e-12, atol=1e-12)


def test_entry_state_is_rejected_bidirectionally():
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 1, 1, 3, 2, 2)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, causal=False, S0=np.zeros((1, 1, 2, 2)))


@pytest.mark.parametrize("mistake", ["readout_before_update", "no_decay", "state_not_carried"])
def test_planted_step_mistakes_fail_a_pin(monkeypatch, mistake):
    orig = O.step

    def bad(q1, k1, v1, S, M, **kw):
        if mistake == "readout_before_update":
            o, S2, M2 = orig(q1, k1, v1, S, M, **kw)
            return np.einsum("bhvf,bhf->bhv", np.asarray(S, float), np.asarray(q1, float)), S2, M2
        if mistake == "no_decay":
            return orig(q1, k1, v1, S, M, **dict(kw, beta=1.0))
        return orig(q1, k1, v1, np.zeros_like(np.asarray(S, float)), M, **kw)

    test_state_hand_example()
    monkeypatch.setattr(O, "step", bad)
    with pytest.raises(AssertionError):
        test_state_hand_example()
