"""Pins of the oracle's weight-normalised recurrence (Variant 1 of Table 2 on the
thelatestinai.com page; the pages do not define the normalisation, and the reading
is: after each token's update every row of S is rescaled to the norm it has in the
entry state S0, the momentum buffer untouched).  Each test checks the oracle against
something it does not compute itself: a hand-worked example, the norm invariant, the
closed form of a zero rate, the scale and rotation symmetries the reading implies,
and the momentum buffer of the unnormalised recurrence.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(seed, B=1, H=2, T=9, d_k=6, d_v=4, phi="identity", d_phi=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d_k))
    k = rng.standard_normal((B, H, T, d_k))
    v = rng.standard_normal((B, H, T, d_v))
    a = rng.standard_normal((B, H, T)) - 1.0
    kw = {}
    dphi = d_k
    if phi == "swiglu":
        dphi = d_phi
        kw = dict(w1=rng.standard_normal((H, d_phi, d_k)) / np.sqrt(d_k),
                  w3=rng.standard_normal((H, d_phi, d_k)) / np.sqrt(d_k))
    S0 = rng.standard_normal((B, H, d_v, dphi))
    M0 = 0.1 * rng.standard_normal((B, H, d_v, dphi))
    return q, k, v, a, S0, M0, kw


def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_weightnorm_T2.json")))
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    S0 = np.array(g["S0"])[None, None]
    o, S, M = oracle.forward(q, k, v, eta_scalar=g["eta"], beta=g["beta"], S0=S0, return_state=True,
                             weight_norm=True)
    np.testing.assert_allclose(o[0, 0], np.array(g["o"]), rtol=1e-13)
    np.testing.assert_allclose(S[0, 0], np.array(g["S_T"]), rtol=1e-13)
    np.testing.assert_allclose(M[0, 0], np.array(g["M_T"]), atol=1e-13)
    o2 = oracle.forward(q, k, v, eta_scalar=g["eta"], beta=g["beta"], S0=S0)
    np.testing.assert_allclose(o2[0, 0], np.array(g["o_without_norm"]), rtol=1e-13)


@pytest.mark.parametrize("phi,d_phi", [("identity", None), ("swiglu", 12)])
@pytest.mark.parametrize("eta_mode,beta", [("scalar", 0.0), ("softplus", 0.9), ("per_token", 0.5)])
def test_row_norms_stay_those_of_the_entry_state(phi, d_phi, eta_mode, beta):
    q, k, v, a, S0, M0, kw = _inputs(1, phi=phi, d_phi=d_phi)
    for T in (1, 2, 5, 9):
        _, S, _ = oracle.forward(q[:, :, :T], k[:, :, :T], v[:, :, :T], eta_mode=eta_mode, eta=a[:, :, :T],
                                 eta_scalar=0.7, beta=beta, phi=phi, S0=S0, M0=M0, return_state=True,
                                 weight_norm=True, **kw)
        np.testing.assert_allclose(np.linalg.norm(S, axis=-1), np.linalg.norm(S0, axis=-1), rtol=1e-12)


def test_zero_rate_reads_the_entry_state():
    q, k, v, a, S0, _, _ = _inputs(2)
    o, S, M = oracle.forward(q, k, v, eta_scalar=0.0, S0=S0, return_state=True, weight_norm=True)
    np.testing.assert_allclose(o, np.einsum("bhvf,bhtf->bhtv", S0, q), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S0, rtol=1e-12)
    assert np.all(M == 0.0)


def test_scaling_the_entry_state_and_the_rates_scales_everything():
    q, k, v, a, S0, M0, _ = _inputs(3)
    c = 2.5
    o1, S1, M1 = oracle.forward(q, k, v, eta_mode="per_token", eta=np.exp(a), beta=0.8, S0=S0, M0=M0,
                                return_state=True, weight_norm=True)
    o2, S2, M2 = oracle.forward(q, k, v, eta_mode="per_token", eta=c * np.exp(a), beta=0.8, S0=c * S0,
                                M0=c * M0, return_state=True, weight_norm=True)
    np.testing.assert_allclose(o2, c * o1, rtol=1e-11)
    np.testing.assert_allclose(S2, c * S1, rtol=1e-11)
    np.testing.assert_allclose(M2, c * M1, rtol=1e-11)


def test_rotating_the_feature_space_leaves_the_outputs():
    # the row norms are invariant under an orthogonal map of the features; a
    # normalisation over the other axis of S would not be
    q, k, v, a, S0, M0, _ = _inputs(4)
    R, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((6, 6)))
    o1, S1, M1 = oracle.forward(q, k, v, eta_mode="softplus", eta=a, beta=0.9, S0=S0, M0=M0, return_state=True,
                                weight_norm=True)
    o2, S2, M2 = oracle.forward(q @ R, k @ R, v, eta_mode="softplus", eta=a, beta=0.9, S0=S0 @ R, M0=M0 @ R,
                                return_state=True, weight_norm=True)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S2, S1 @ R, rtol=1e-10, atol=1e-10)


def test_momentum_buffer_is_that_of_the_plain_recurrence():
    # with the dot-product loss the gradient does not depend on S, so the buffer
    # does not see the normalisation
    q, k, v, a, S0, M0, _ = _inputs(6)
    _, _, M1 = oracle.forward(q, k, v, eta_mode="softplus", eta=a, beta=0.9, S0=S0, M0=M0, return_state=True,
                              weight_norm=True)
    _, _, M2 = oracle.forward(q, k, v, eta_mode="softplus", eta=a, beta=0.9, S0=np.zeros_like(S0), M0=M0,
                              return_state=True)
    np.testing.assert_allclose(M1, M2, rtol=1e-13)


def test_zero_rows_stay_zero_and_errors():
    q, k, v, a, S0, _, _ = _inputs(7)
    S0[0, 1, 2] = 0.0
    o, S, _ = oracle.forward(q, k, v, eta_scalar=0.5, S0=S0, return_state=True, weight_norm=True)
    assert np.all(S[0, 1, 2] == 0.0) and np.all(o[0, 1, :, 2] == 0.0)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, weight_norm=True)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, S0=S0, causal=False, weight_norm=True)


@pytest.mark.parametrize("phi,d_phi", [("identity", None), ("swiglu", 12)])
def test_steps_give_the_forward(phi, d_phi):
    # the step rescales to the norms of the state it is given, which a weight-normalised
    # run keeps at the entry-state norms: T steps are the forward
    q, k, v, a, S0, M0, kw = _inputs(8, phi=phi, d_phi=d_phi)
    o_ref, S_ref, M_ref = oracle.forward(q, k, v, eta_mode="softplus", eta=a, beta=0.9, phi=phi, S0=S0, M0=M0,
                                         return_state=True, weight_norm=True, **kw)
    S, M = S0.copy(), M0.copy()
    for t in range(q.shape[2]):
        o, S, M = oracle.step(q[:, :, t], k[:, :, t], v[:, :, t], S, M, eta_mode="softplus", eta=a[:, :, t],
                              beta=0.9, phi=phi, weight_norm=True, **kw)
        np.testing.assert_allclose(o, o_ref[:, :, t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11)
    np.testing.assert_allclose(M, M_ref, rtol=1e-11)
