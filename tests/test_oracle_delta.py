"""Pins of the oracle's mean-squared binding loss (the delta rule).

The loss is l(S) = 1/2 ||S phi(k) - v||^2 (the MSE inner-loop loss named in the
Modular TTT abstract on the mlsanity.com page; the same page cites the delta-rule
parallelisation paper among the works the paper builds on).  Each test compares
the oracle with something computed independently: finite differences, a
hand-worked example, pure-Python loops over the explicit delta-rule product
form, an exact-memorisation invariant.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import ttt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_mse_gradient_matches_central_finite_difference():
    rng = np.random.default_rng(11)
    S = rng.standard_normal((3, 4))
    pk = rng.standard_normal(4)
    v = rng.standard_normal(3)
    g = oracle.mse_loss_grad(S, pk, v)
    h = 1e-6
    fd = np.zeros_like(S)
    for i in range(3):
        for j in range(4):
            Sp, Sm = S.copy(), S.copy()
            Sp[i, j] += h
            Sm[i, j] -= h
            fd[i, j] = (oracle.mse_loss(Sp, pk, v) - oracle.mse_loss(Sm, pk, v)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-7, atol=1e-8)


def test_mse_loss_value():
    # 1/2 ||S k - v||^2 at a point worked by hand: S k = (3, 1), v = (1, 1) -> 1/2 (4 + 0) = 2
    S = np.array([[1.0, 2.0], [1.0, 0.0]])
    assert oracle.mse_loss(S, np.array([1.0, 1.0]), np.array([1.0, 1.0])) == 2.0


def test_delta_hand_example():
    g = _load("hand_delta_T2.json")
    q, k, v = (np.array(g[n], float)[None, None] for n in "qkv")
    got = oracle.forward(q, k, v, eta_scalar=g["eta"], loss="mse")
    np.testing.assert_allclose(got[0, 0], np.array(g["o_causal"]), rtol=0, atol=1e-14)
    dot = oracle.forward(q, k, v, eta_scalar=g["eta"])
    np.testing.assert_allclose(dot[0, 0], np.array(g["o_dot_causal"]), rtol=0, atol=1e-14)


def _delta_product_form(q, k, v, eta, beta=0.0):
    """Pure-Python loops: S_t = S_{t-1} (I - eta_t k_t k_t^T) + eta_t v_t k_t^T for beta = 0; with
    momentum the buffer M_t = beta M_{t-1} + eta_t (v_t - S_{t-1} k_t) k_t^T, S_t = S_{t-1} + M_t."""
    T, dk = len(k), len(k[0])
    dv = len(v[0])
    S = [[0.0] * dk for _ in range(dv)]
    M = [[0.0] * dk for _ in range(dv)]
    out = []
    for t in range(T):
        if beta == 0.0:
            # S (I - eta k k^T) + eta v k^T, entry by entry
            new = [[0.0] * dk for _ in range(dv)]
            for i in range(dv):
                for j in range(dk):
                    acc = 0.0
                    for m in range(dk):
                        ident = 1.0 if m == j else 0.0
                        acc += S[i][m] * (ident - eta[t] * k[t][m] * k[t][j])
                    new[i][j] = acc + eta[t] * v[t][i] * k[t][j]
            S = new
        else:
            err = [sum(S[i][m] * k[t][m] for m in range(dk)) - v[t][i] for i in range(dv)]
            for i in range(dv):
                for j in range(dk):
                    M[i][j] = beta * M[i][j] - eta[t] * err[i] * k[t][j]
            for i in range(dv):
                for j in range(dk):
                    S[i][j] += M[i][j]
        out.append([sum(S[i][m] * q[t][m] for m in range(dk)) for i in range(dv)])
    return np.array(out)


@pytest.mark.parametrize("beta", [0.0, 0.6])
def test_delta_matches_pure_python_product_form(beta):
    rng = np.random.default_rng(12)
    T, dk, dv = 7, 3, 2
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk)) * 0.5
    v = rng.standard_normal((T, dv))
    eta = rng.uniform(0.1, 0.9, size=T)
    got = oracle.forward(q[None, None], k[None, None], v[None, None], eta_mode="per_token", eta=eta[None, None],
                         beta=beta, loss="mse")
    want = _delta_product_form(q.tolist(), k.tolist(), v.tolist(), eta.tolist(), beta)
    np.testing.assert_allclose(got[0, 0], want, rtol=1e-12, atol=1e-12)


def test_delta_memorises_exactly_with_unit_keys_and_unit_rate():
    # with ||k_t|| = 1 and eta = 1 the step makes S_t k_t = v_t exactly
    rng = np.random.default_rng(13)
    T, d = 6, 4
    k = rng.standard_normal((T, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, d))
    o = oracle.forward(k[None, None], k[None, None], v[None, None], eta_scalar=1.0, loss="mse")
    np.testing.assert_allclose(o[0, 0], v, rtol=0, atol=1e-12)


def test_first_step_is_shared_with_the_dot_product_loss():
    # from the reset state S = 0 the two gradients coincide (-v k^T)
    rng = np.random.default_rng(14)
    q, k, v = (rng.standard_normal((1, 2, 1, 5)) for _ in range(3))
    np.testing.assert_allclose(oracle.forward(q, k, v, eta_scalar=0.3, loss="mse"),
                               oracle.forward(q, k, v, eta_scalar=0.3), rtol=0, atol=1e-15)


def test_delta_bidirectional_reads_the_final_state():
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((1, 1, 5, 3)) * 0.5 for _ in range(3))
    causal, S, _ = oracle.forward(q, k, v, eta_scalar=0.4, loss="mse", return_state=True)
    bi = oracle.forward(q, k, v, eta_scalar=0.4, loss="mse", causal=False)
    np.testing.assert_allclose(bi[0, 0], q[0, 0] @ S[0, 0].T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(causal[0, 0, -1], bi[0, 0, -1], rtol=1e-13, atol=1e-13)


def test_unknown_loss_is_rejected():
    with pytest.raises(ValueError):
        oracle.forward(np.zeros((1, 1, 1, 2)), np.zeros((1, 1, 1, 2)), np.zeros((1, 1, 1, 2)), loss="l1")


def _delta_pins_pass():
    try:
        test_mse_gradient_matches_central_finite_difference()
        test_delta_hand_example()
        test_delta_matches_pure_python_product_form(0.0)
        test_delta_memorises_exactly_with_unit_keys_and_unit_rate()
    except (AssertionError, ValueError):   # a wrong formula may also fail on shapes
        return False
    return True


@pytest.mark.parametrize("mistake", ["residual_sign", "missing_state_term", "transposed_outer"])
def test_planted_mistakes_fail_a_delta_pin(monkeypatch, mistake):
    assert _delta_pins_pass()
    if mistake == "residual_sign":
        monkeypatch.setattr(O, "mse_loss_grad", lambda S, pk, v: np.einsum(
            "...v,...f->...vf", v - np.einsum("...vf,...f->...v", S, pk), pk))
    elif mistake == "missing_state_term":
        monkeypatch.setattr(O, "mse_loss_grad", lambda S, pk, v: np.einsum("...v,...f->...vf", -v, pk))
    elif mistake == "transposed_outer":
        # (S k - v) k^T with S's transpose in the residual (square shapes only)
        monkeypatch.setattr(O, "mse_loss_grad", lambda S, pk, v: np.einsum(
            "...v,...f->...vf", np.einsum("...fv,...f->...v", S, pk) - v, pk))
    monkeypatch.setattr(oracle, "mse_loss_grad", O.mse_loss_grad)
    assert not _delta_pins_pass()


# ---- the recurrent step (decode) of the delta rule ----

def test_delta_step_hand_example():
    g = _load("hand_delta_step.json")
    q, k, v = (np.array(g[n], float)[None, None] for n in "qkv")
    S = np.array(g["S"], float)[None, None]
    M = np.array(g["M"], float)[None, None]
    o, S1, M1 = oracle.step(q, k, v, S, M, eta_scalar=g["eta"], beta=g["beta"], loss="mse")
    np.testing.assert_allclose(o[0, 0], g["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S1[0, 0], g["S_new"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(M1[0, 0], g["M_new"], rtol=0, atol=1e-15)
    od, Sd, _ = oracle.step(q, k, v, S, M, eta_scalar=g["eta"], beta=g["beta"])
    np.testing.assert_allclose(od[0, 0], g["o_dot"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Sd[0, 0], g["S_new_dot"], rtol=0, atol=1e-15)


def test_delta_step_from_zero_state_is_the_dot_step():
    # at S = 0 the residual is v itself, so both losses take the same step
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((2, 2, 3, 8))
    v = rng.standard_normal((2, 3, 6))
    M = rng.standard_normal((2, 3, 6, 8))
    S = np.zeros((2, 3, 6, 8))
    a = oracle.step(q, k, v, S, M, eta_scalar=0.3, beta=0.7, loss="mse")
    b = oracle.step(q, k, v, S, M, eta_scalar=0.3, beta=0.7)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_delta_step_leaves_an_exact_binding_alone():
    # S k = v: the gradient vanishes and only the momentum moves S
    rng = np.random.default_rng(22)
    S = rng.standard_normal((1, 2, 5, 4))
    k = rng.standard_normal((1, 2, 4))
    v = np.einsum("bhvf,bhf->bhv", S, k)
    q = rng.standard_normal((1, 2, 4))
    M = rng.standard_normal((1, 2, 5, 4))
    o, S1, M1 = oracle.step(q, k, v, S, M, eta_scalar=0.9, beta=0.6, loss="mse")
    np.testing.assert_allclose(M1, 0.6 * M, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, S + 0.6 * M, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o, np.einsum("bhvf,bhf->bhv", S + 0.6 * M, q), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("beta,eta_mode", [(0.0, "scalar"), (0.9, "softplus"), (0.5, "per_token")])
def test_delta_steps_match_the_forward_from_an_entry_state(beta, eta_mode):
    # T steps from (S0, M0) against the token loop of forward(loss="mse")
    rng = np.random.default_rng(23)
    B, H, T, d = 2, 2, 7, 5
    q, k, v = rng.standard_normal((3, B, H, T, d)) / np.sqrt(d)
    a = rng.standard_normal((B, H, T)) - 1.0
    eta = None if eta_mode == "scalar" else (np.abs(a) if eta_mode == "per_token" else a)
    S0 = rng.standard_normal((B, H, d, d))
    M0 = rng.standard_normal((B, H, d, d)) if beta else np.zeros((B, H, d, d))
    o_ref, S_ref, M_ref = oracle.forward(q, k, v, eta_mode=eta_mode, eta=eta, eta_scalar=0.4, beta=beta,
                                         S0=S0, M0=M0, loss="mse", return_state=True)
    S, M = S0, M0
    for t in range(T):
        e_t = None if eta is None else eta[:, :, t]
        o, S, M = oracle.step(q[:, :, t], k[:, :, t], v[:, :, t], S, M, eta_mode=eta_mode, eta=e_t,
                              eta_scalar=0.4, beta=beta, loss="mse")
        np.testing.assert_allclose(o, o_ref[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M, M_ref, rtol=1e-12, atol=1e-12)


def test_delta_step_rejects_weight_norm_and_unknown_losses():
    z = np.zeros((1, 1, 2))
    Z = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.step(z, z, z, Z, Z, loss="mse", weight_norm=True)
    with pytest.raises(ValueError):
        oracle.step(z, z, z, Z, Z, loss="l1")
