"""CPU checks (fp64) of the identities the HIP kernels are built on, against the
oracle's token-by-token recurrence.  They use no GPU and no kernel code: each
identity is written out here from its derivation and compared with
``oracle.forward``.

T-form of the momentum state (kappa = beta / (1 - beta), T = S + kappa M):
  T_t = T_{t-1} + eta_t v_t k_t^T / (1 - beta)     (no transition)
  M_t = beta M_{t-1} + eta_t v_t k_t^T
Chunk step with entry (T, M), local index i, chunk length n:
  o_i = T q_i - beta^{i+2}/(1-beta) M q_i + sum_{j<=i} eta_j c_{i-j} (q_i.k_j) v_j
  T'  = T + sum_j eta_j v_j k_j^T / (1 - beta)
  M'  = beta^n M + sum_j eta_j beta^{n-1-j} v_j k_j^T
with c_r = (1 - beta^{r+1}) / (1 - beta).  Segments of length L compose as
T += dT, M = beta^L M + dM.  Bidirectional: S_{T-1} = T_{T-1} - kappa M_{T-1}.
"""
import numpy as np
import pytest

import oracle


def _inputs(T, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((T, dv))
    eta = np.exp(rng.standard_normal(T) * 0.3 - 1.0)
    return q, k, v, eta


def _ref(q, k, v, eta, beta, causal=True):
    o = oracle.forward(q[None, None], k[None, None], v[None, None], eta_mode="per_token",
                       eta=eta[None, None], beta=beta, causal=causal)
    return o[0, 0]


def _chunk_step(Tst, M, q, k, v, eta, beta):
    n = q.shape[0]
    idx = np.arange(n)
    diff = idx[:, None] - idx[None, :]
    c = np.where(diff >= 0, (1.0 - beta ** (np.maximum(diff, 0) + 1)) / (1.0 - beta), 0.0)
    scores = (q @ k.T) * c * eta[None, :]
    o = q @ Tst.T - (beta ** (idx + 2) / (1.0 - beta))[:, None] * (q @ M.T) + scores @ v
    Tn = Tst + (v * eta[:, None]).T @ k / (1.0 - beta)
    Mn = beta ** n * M + (v * (eta * beta ** (n - 1 - idx))[:, None]).T @ k
    return o, Tn, Mn


@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9, 0.99])
@pytest.mark.parametrize("chunk", [1, 7, 16])
def test_t_form_chunk_step_equals_recurrence(beta, chunk):
    q, k, v, eta = _inputs(45, 6, 5, 11)
    ref = _ref(q, k, v, eta, beta)
    Tst = np.zeros((5, 6))
    M = np.zeros((5, 6))
    out = []
    for s in range(0, 45, chunk):
        o, Tst, M = _chunk_step(Tst, M, q[s:s + chunk], k[s:s + chunk], v[s:s + chunk], eta[s:s + chunk], beta)
        out.append(o)
    got = np.concatenate(out)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_segment_summaries_compose(beta):
    # entry state of segment s from the zero-entry summaries of segments < s
    q, k, v, eta = _inputs(60, 4, 3, 12)
    L = 12
    ref = _ref(q, k, v, eta, beta)
    summaries = []
    for s in range(0, 60, L):
        _, dT, dM = _chunk_step(np.zeros((3, 4)), np.zeros((3, 4)), q[s:s + L], k[s:s + L], v[s:s + L],
                                eta[s:s + L], beta)
        summaries.append((dT, dM))
    Tst = np.zeros((3, 4))
    M = np.zeros((3, 4))
    out = []
    for i, s in enumerate(range(0, 60, L)):
        o, _, _ = _chunk_step(Tst, M, q[s:s + L], k[s:s + L], v[s:s + L], eta[s:s + L], beta)
        out.append(o)
        dT, dM = summaries[i]
        Tst = Tst + dT
        M = beta ** L * M + dM
    got = np.concatenate(out)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9])
def test_bidirectional_state_from_t_form(beta):
    q, k, v, eta = _inputs(30, 4, 3, 13)
    ref = _ref(q, k, v, eta, beta, causal=False)
    _, Tst, M = _chunk_step(np.zeros((3, 4)), np.zeros((3, 4)), q, k, v, eta, beta)
    S = Tst - beta / (1.0 - beta) * M
    got = q @ S.T
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_t_form_is_not_the_plain_state():
    # a dropped kappa M term must be visible: T differs from S when beta > 0
    q, k, v, eta = _inputs(20, 4, 3, 14)
    beta = 0.9
    ref = _ref(q, k, v, eta, beta, causal=False)
    _, Tst, _ = _chunk_step(np.zeros((3, 4)), np.zeros((3, 4)), q, k, v, eta, beta)
    assert np.max(np.abs(q @ Tst.T - ref)) > 1e-3


# ----------------------------------------------------------------------------
# backward as forward passes on permuted, time-reversed operands (the library
# computes the gradients this way); checked in fp64 against the oracle backward
# ----------------------------------------------------------------------------

def _rev(x):
    return x[:, :, ::-1]


@pytest.mark.parametrize("eta_mode", ["scalar", "per_token", "softplus"])
@pytest.mark.parametrize("beta", [0.0, 0.8])
def test_backward_as_reversed_forwards_causal(eta_mode, beta):
    rng = np.random.default_rng(31)
    B, H, T, d = 1, 2, 11, 4
    q, k, v, dO = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    a = rng.standard_normal((B, H, T))
    eta = None if eta_mode == "scalar" else a
    kw = dict(eta_mode=eta_mode, eta=eta, eta_scalar=0.6, beta=beta)
    dq, dk, dv, de = oracle.backward(q, k, v, dO, **kw)
    e = oracle.learning_rates(eta_mode, T, B * H, eta, 0.6).reshape(B, H, T)
    # dq: the causal forward with (q, k, v) -> (dO, v, k)
    np.testing.assert_allclose(oracle.forward(dO, v, k, **kw), dq, rtol=1e-10, atol=1e-10)
    # dv, dk, deta: unit-rate forwards over the reversed sequence
    u = _rev(oracle.forward(_rev(k), _rev(q), _rev(dO), eta_scalar=1.0, beta=beta))
    w = _rev(oracle.forward(_rev(v), _rev(dO), _rev(q), eta_scalar=1.0, beta=beta))
    np.testing.assert_allclose(e[..., None] * u, dv, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(e[..., None] * w, dk, rtol=1e-10, atol=1e-10)
    d_eta = np.einsum("bhtd,bhtd->bht", v, u)
    if eta_mode == "per_token":
        np.testing.assert_allclose(d_eta, de, rtol=1e-10, atol=1e-10)
    elif eta_mode == "softplus":
        np.testing.assert_allclose(d_eta / (1 + np.exp(-a)), de, rtol=1e-10, atol=1e-10)
    else:
        assert abs(d_eta.sum() - de) <= 1e-9 * max(1.0, abs(de))


@pytest.mark.parametrize("beta", [0.0, 0.8])
def test_backward_as_forwards_bidirectional(beta):
    rng = np.random.default_rng(32)
    B, H, T, d = 1, 2, 9, 4
    q, k, v, dO = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    a = rng.standard_normal((B, H, T))
    kw = dict(eta_mode="softplus", eta=a, beta=beta, causal=False)
    dq, dk, dv, de = oracle.backward(q, k, v, dO, **kw)
    e = np.log1p(np.exp(a))
    c = np.array([sum(beta ** r for r in range(T - s)) for s in range(T)])     # c_{T-1-s}
    np.testing.assert_allclose(oracle.forward(dO, v, k, **kw), dq, rtol=1e-10, atol=1e-10)
    u = oracle.forward(k, q, dO, eta_scalar=1.0, causal=False)
    w = oracle.forward(v, dO, q, eta_scalar=1.0, causal=False)
    np.testing.assert_allclose((e * c)[..., None] * u, dv, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose((e * c)[..., None] * w, dk, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(c * np.einsum("bhtd,bhtd->bht", v, u) / (1 + np.exp(-a)), de, rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------
# delta rule (mean-squared binding loss, beta = 0): chunk form
#
# Within a chunk entered with S0 (d_v x d_k), write the step of token t as
# S_t = S_{t-1} + u_t k_t^T with u_t = eta_t (v_t - S_{t-1} k_t).  Unrolling S_{t-1}
# = S0 + sum_{j<t} u_j k_j^T gives, with rows = tokens,
#   (I + diag(eta) L) U = diag(eta) (V - K S0^T),  L = strictly lower part of K K^T
# so U = A (V - K S0^T) with A = (I + diag(eta) L)^{-1} diag(eta), and
#   O = Q S0^T + tril(Q K^T) U,     S_n = S0 + U^T K.
# ----------------------------------------------------------------------------

def _delta_chunked(q, k, v, eta, chunk):
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk))
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        Q, K, V, e = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk], eta[c0:c0 + chunk]
        n = len(K)
        L = np.tril(K @ K.T, -1)
        # unit lower-triangular inverse by forward substitution, row by row
        X = np.zeros((n, n))
        Nm = e[:, None] * L
        for t in range(n):
            X[t, t] = 1.0
            for j in range(t):
                X[t] -= Nm[t, j] * X[j]
        A = X * e[None, :]
        U = A @ (V - K @ S.T)
        o[c0:c0 + n] = Q @ S.T + np.tril(Q @ K.T) @ U
        S = S + U.T @ K
    return o, S


@pytest.mark.parametrize("chunk", [1, 5, 16, 32, 64])
def test_delta_chunk_form_equals_recurrence(chunk):
    q, k, v, eta = _inputs(150, 8, 6, 31)
    got, S = _delta_chunked(q, k, v, eta, chunk)
    ref, Sref, _ = oracle.forward(q[None, None], k[None, None], v[None, None], eta_mode="per_token",
                                  eta=eta[None, None], loss="mse", return_state=True)
    np.testing.assert_allclose(got, ref[0, 0], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S, Sref[0, 0], rtol=1e-10, atol=1e-10)
