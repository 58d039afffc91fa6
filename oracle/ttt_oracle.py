"""Plain, slow fp64 CPU oracle of the TTT-with-KV-binding forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
product path (the HIP library and its Python binding) never does, and this
module shares no code with it.

What it computes (sources are the five web pages about "Test-Time Training with
KV Binding Is Secretly Linear Attention"; readings are marked READING):

* The layer keeps a fixed-size fast-weight matrix per sequence, takes one
  gradient step on it for every entry of the sequence, and starts every new
  sequence from a reset state (wpnews.pro "Test Time Training" commentary).
  READING: the reset state is zero.
* The step binds the key to the value.  READING: the binding loss is the
  negative dot product  l_t(S) = -<S phi(k_t), v_t>,  whose gradient
  -v_t phi(k_t)^T does not depend on S.  A descent step therefore adds the
  outer product eta_t v_t phi(k_t)^T, i.e. the outer-product accumulation the
  kualia.ai blog ("The Linear Attention Equivalence") identifies with the
  numerator of linear attention (phi(Q) phi(K)^T) V.  READING: no denominator.
* Optional SGD momentum and a per-token learning rate are the inner-loop
  options that Table 2 of the thelatestinai.com page removes one by one
  (Variant 3 keeps both, Variant 4 drops the per-token lr, Variant 5 drops
  momentum).  READING: heavy-ball momentum with the step inside the buffer,
  M_t = beta M_{t-1} - eta_t G_t,  S_t = S_{t-1} + M_t, no dampening, no
  Nesterov; per-token lr eta_t = softplus(a_t).
* Variant 2 of Table 2 keeps a two-layer MLP fast weight and updates only its
  last layer: the first layer is a frozen feature map.  READING: SwiGLU
  features phi(x) = silu(W1 x) * (W3 x) with silu(u) = u / (1 + e^-u).
* Variant 1 of Table 2 is Variant 2 with weight normalisation of the updated
  layer, and has a recurrent implementation only.  The pages do not define the
  normalisation.  READING (``weight_norm=True``): after every token's update each
  row of S (one output unit: its weights over the features) is rescaled to the
  Euclidean norm that row has in the entry state S0, the initial fast weight,
  which must be given; the momentum buffer is not rescaled.  A row whose entry
  norm is zero stays zero.
* READING: the readout of token t uses the state after token t's own update,
  o_t = S_t phi(q_t).  In the bidirectional (ViT) mode every token updates the
  state first and every query reads the final state.
* The mean-squared binding loss (``loss="mse"``) is the other inner-loop loss
  the pages name: the Modular TTT abstract on the mlsanity.com page compares MSE
  and inner-product losses, and the same page lists "Parallelizing Linear
  Transformers with the Delta Rule over Sequence Length" among the works the
  paper builds on.  READING: l_t(S) = 1/2 ||S phi(k_t) - v_t||^2, gradient
  (S phi(k_t) - v_t) phi(k_t)^T, taken through the same inner loop (rate,
  momentum, readout after the update).  With beta = 0 a descent step is the
  delta rule S_t = S_{t-1} - eta_t (S_{t-1} phi(k_t) - v_t) phi(k_t)^T.

``forward`` is the definition, a token-by-token loop.  ``forward_closed_form``
and ``forward_chunked`` are the parallel forms the blog says the recurrence can
be rewritten into ("The Cracks in the Memorization Hypothesis": closed form;
"The Linear Attention Equivalence": sequential or parallel); the tests use them
only to check that those forms agree with the loop.

Every function here is pinned by a test in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "softplus", "silu", "silu_grad", "swiglu_features", "features", "learning_rates",
    "binding_loss", "binding_loss_grad", "mse_loss", "mse_loss_grad", "forward", "forward_closed_form",
    "forward_chunked", "rel_err",
]


# ----------------------------------------------------------------------------
# elementary functions
# ----------------------------------------------------------------------------

def softplus(a):
    """softplus(a) = ln(1 + e^a), evaluated as max(a,0) + log1p(e^-|a|).

    Per-token learnable learning rate of Variant 3 (thelatestinai.com,
    Table 2).  READING: eta_t = softplus(a_t) with a_t given per token.
    """
    a = np.asarray(a, dtype=np.float64)
    return np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a)))


def silu(u):
    """silu(u) = u * sigmoid(u) = u / (1 + e^-u)  (gate of the SwiGLU MLP)."""
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


def swiglu_features(x, w1, w3):
    """phi(x) = silu(W1 x) * (W3 x) for rows x of ``x``.

    x: [..., d_k];  w1, w3: [d_phi, d_k] (out x in).  Returns [..., d_phi].
    Frozen first layer of Variant 2's two-layer MLP fast weight
    (thelatestinai.com, Table 2, Variant 2 vs Variant 3).
    """
    x = np.asarray(x, dtype=np.float64)
    return silu(x @ np.asarray(w1, np.float64).T) * (x @ np.asarray(w3, np.float64).T)


def features(x, phi: str, w1=None, w3=None):
    """Kernel feature map phi applied to the last axis of x ([N, T, d_k])."""
    if phi == "identity":
        return np.asarray(x, dtype=np.float64)
    if phi == "swiglu":
        # w1, w3 are per sequence here: [N, d_phi, d_k]
        x = np.asarray(x, dtype=np.float64)
        u = np.einsum("ntd,nfd->ntf", x, w1)
        g = np.einsum("ntd,nfd->ntf", x, w3)
        return silu(u) * g
    raise ValueError(f"unknown feature map {phi!r}")


def learning_rates(eta_mode: str, T: int, N: int, eta=None, eta_scalar: float = 1.0):
    """Per-token step sizes, shape [N, T], fp64.

    scalar: eta_scalar for every token; per_token: eta given; softplus:
    eta = softplus(a) with the logits a given (fp32 values upcast exactly).
    """
    if eta_mode == "scalar":
        return np.full((N, T), float(eta_scalar), dtype=np.float64)
    e = np.asarray(eta, dtype=np.float64).reshape(N, T)
    if eta_mode == "per_token":
        return e.copy()
    if eta_mode == "softplus":
        return softplus(e)
    raise ValueError(f"unknown eta mode {eta_mode!r}")


# ----------------------------------------------------------------------------
# binding loss and its explicit gradient
# ----------------------------------------------------------------------------

def binding_loss(S, phik, v):
    """l(S) = -<S phi(k), v>: the dot-product key->value binding loss.

    S: [..., d_v, d_phi], phik: [..., d_phi], v: [..., d_v].  READING of
    "a training step to bind them together" (kualia.ai blog, "The Cracks in
    the Memorization Hypothesis").
    """
    return -np.einsum("...v,...vf,...f->...", v, S, phik)


def binding_loss_grad(S, phik, v):
    """Gradient of ``binding_loss`` with respect to S: -v phi(k)^T.

    The loss is linear in S, so the gradient is the same at every S (the shape
    of S is only used to broadcast).
    """
    g = -np.einsum("...v,...f->...vf", v, phik)
    return np.broadcast_to(g, np.shape(S)).copy()


def mse_loss(S, phik, v):
    """l(S) = 1/2 ||S phi(k) - v||^2: the mean-squared key->value binding loss.

    S: [..., d_v, d_phi], phik: [..., d_phi], v: [..., d_v].  READING of the MSE
    inner-loop loss the mlsanity.com page names (Modular TTT abstract).
    """
    r = np.einsum("...vf,...f->...v", S, phik) - v
    return 0.5 * np.einsum("...v,...v->...", r, r)


def mse_loss_grad(S, phik, v):
    """Gradient of ``mse_loss`` with respect to S: (S phi(k) - v) phi(k)^T."""
    r = np.einsum("...vf,...f->...v", S, phik) - v
    return np.einsum("...v,...f->...vf", r, phik)


# ----------------------------------------------------------------------------
# the definition: token-by-token recurrence
# ----------------------------------------------------------------------------

def _flatten(x, d):
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(-1, x.shape[-2], d)


def forward(q, k, v, *, eta_mode: str = "scalar", eta=None, eta_scalar: float = 1.0,
            beta: float = 0.0, causal: bool = True, phi: str = "identity",
            w1=None, w3=None, ascent: bool = False, inner_steps: int = 1,
            return_state: bool = False, S0=None, M0=None, loss: str = "dot", weight_norm: bool = False):
    """Recurrent TTT forward, fp64, one gradient step per token.

    q, k: [B, H, T, d_k]; v: [B, H, T, d_v]; eta / a: [B, H, T] (per_token /
    softplus modes); w1, w3: [H, d_phi, d_k] for the SwiGLU feature map.
    Returns o: [B, H, T, d_v] (and the final (S, M) if ``return_state``).
    ``S0``, ``M0`` ([B, H, d_v, d_phi], causal only) replace the reset state:
    the recurrent form carries (S, M) from one call to the next (Table 2 lists
    a recurrent implementation of every variant); None reads as zero.

    For every sequence (b, h) independently:
      S = S0 or 0, M = M0 or 0                       (reset per sequence)
      for t = 0 .. T-1:
        G   = grad_S l_t(S)  = -v_t phi(k_t)^T        (explicit gradient; loss="mse":
                             = (S phi(k_t) - v_t) phi(k_t)^T)
        M   = beta M - eta_t G      (ascent: + eta_t G)
        S   = S + M
        weight_norm: S[i, :] *= ||S0[i, :]|| / ||S[i, :]||  (per row; 0 if either is 0)
        o_t = S phi(q_t)                              (causal readout)
      bidirectional: o_t = S_T phi(q_t) for all t.
    ``inner_steps`` > 1 repeats the (momentum-free) step on the same token,
    the "more inner-loop iterations" manipulation of Figure 1; it requires
    beta == 0.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, T, d_k = q.shape
    d_v = np.shape(v)[-1]
    N = B * H
    qf = _flatten(q, d_k)
    kf = _flatten(k, d_k)
    vf = _flatten(v, d_v)
    if phi == "swiglu":
        w1n = np.broadcast_to(np.asarray(w1, np.float64)[None], (B,) + np.shape(w1)).reshape(N, -1, d_k)
        w3n = np.broadcast_to(np.asarray(w3, np.float64)[None], (B,) + np.shape(w3)).reshape(N, -1, d_k)
        pq = features(qf, phi, w1n, w3n)
        pk = features(kf, phi, w1n, w3n)
    else:
        pq = features(qf, phi)
        pk = features(kf, phi)
    d_phi = pk.shape[-1]
    lr = learning_rates(eta_mode, T, N, eta, eta_scalar)
    if inner_steps != 1 and beta != 0.0:
        raise ValueError("inner_steps > 1 is defined here for beta == 0 only")
    sign = 1.0 if ascent else -1.0
    if loss not in ("dot", "mse"):
        raise ValueError(f"unknown binding loss {loss!r}")
    loss_grad = binding_loss_grad if loss == "dot" else mse_loss_grad

    if (S0 is not None or M0 is not None) and not causal:
        raise ValueError("an entry state is defined for the causal mode only")
    S = np.zeros((N, d_v, d_phi)) if S0 is None else np.array(S0, dtype=np.float64).reshape(N, d_v, d_phi)
    M = np.zeros((N, d_v, d_phi)) if M0 is None else np.array(M0, dtype=np.float64).reshape(N, d_v, d_phi)
    if weight_norm:
        if S0 is None or not causal or loss != "dot":
            raise ValueError("weight normalisation is defined here for the causal dot-product layer "
                             "with a given entry state")
        row_norm0 = np.sqrt(np.sum(S * S, axis=2))          # [N, d_v]
    o = np.zeros((N, T, d_v))
    for t in range(T):
        for _ in range(inner_steps):
            G = loss_grad(S, pk[:, t], vf[:, t])
            M = beta * M + sign * lr[:, t, None, None] * G
            S = S + M
            if weight_norm:
                norm = np.sqrt(np.sum(S * S, axis=2))
                factor = np.divide(row_norm0, norm, out=np.zeros_like(norm), where=norm > 0)
                S = S * factor[:, :, None]
        if causal:
            o[:, t] = np.einsum("nvf,nf->nv", S, pq[:, t])
    if not causal:
        o = np.einsum("nvf,ntf->ntv", S, pq)
    o = o.reshape(B, H, T, d_v)
    if return_state:
        return o, S.reshape(B, H, d_v, d_phi), M.reshape(B, H, d_v, d_phi)
    return o


def step(q1, k1, v1, S, M, *, eta_mode: str = "scalar", eta=None, eta_scalar: float = 1.0,
         beta: float = 0.0, phi: str = "identity", w1=None, w3=None, weight_norm: bool = False,
         loss: str = "dot"):
    """One recurrent step (decode) for every sequence: the token q1, k1, v1
    ([B, H, d]) with rate eta ([B, H], per_token / softplus modes) updates the
    carried state (S, M) ([B, H, d_v, d_phi]) and is read out after its update:

      M' = beta M + eta v phi(k)^T,   S' = S + M',   o = S' phi(q).

    ``loss="mse"``: the step of the mean-squared binding loss 1/2 ||S phi(k) - v||^2
    (the MSE inner-loop loss of the Modular TTT abstract on the mlsanity.com page),
    whose gradient at the given S is (S phi(k) - v) phi(k)^T, so that

      M' = beta M + eta (v - S phi(k)) phi(k)^T,   S' = S + M',   o = S' phi(q)

    (the delta rule of the paper that page cites, with heavy-ball momentum).

    ``weight_norm``: Variant 1's step (the reading in ``forward``): each row of S'
    is rescaled to the norm of the same row of S (which a weight-normalised run
    keeps at its entry-state norm), 0 if either norm is 0.

    Returns (o [B, H, d_v], S', M').  The step is written out on its own (it is
    the loop body of ``forward``); the tests check T steps against ``forward``.
    """
    q1 = np.asarray(q1, dtype=np.float64)
    B, H, d_k = q1.shape
    N = B * H
    v1 = np.asarray(v1, dtype=np.float64).reshape(N, -1)
    if phi == "swiglu":
        w1n = np.broadcast_to(np.asarray(w1, np.float64)[None], (B,) + np.shape(w1)).reshape(N, -1, d_k)
        w3n = np.broadcast_to(np.asarray(w3, np.float64)[None], (B,) + np.shape(w3)).reshape(N, -1, d_k)
        pq = features(q1.reshape(N, 1, d_k), phi, w1n, w3n)[:, 0]
        pk = features(np.asarray(k1, np.float64).reshape(N, 1, d_k), phi, w1n, w3n)[:, 0]
    else:
        pq = q1.reshape(N, d_k)
        pk = np.asarray(k1, np.float64).reshape(N, d_k)
    if eta_mode == "scalar":
        e = np.full(N, float(eta_scalar))
    elif eta_mode == "per_token":
        e = np.asarray(eta, np.float64).reshape(N)
    elif eta_mode == "softplus":
        e = softplus(np.asarray(eta, np.float64).reshape(N))
    else:
        raise ValueError(eta_mode)
    d_v, d_phi = v1.shape[1], pk.shape[1]
    S = np.asarray(S, np.float64).reshape(N, d_v, d_phi)
    M = np.asarray(M, np.float64).reshape(N, d_v, d_phi)
    if loss == "dot":
        target = v1                                      # -grad = v phi(k)^T for -<S phi(k), v>
    elif loss == "mse":
        if weight_norm:
            raise ValueError("weight normalisation is defined here for the dot-product loss only")
        target = v1 - np.einsum("nvf,nf->nv", S, pk)     # -grad = (v - S phi(k)) phi(k)^T at the given S
    else:
        raise ValueError(f"unknown binding loss {loss!r}")
    M_new = beta * M + e[:, None, None] * target[:, :, None] * pk[:, None, :]
    S_new = S + M_new
    if weight_norm:
        target = np.sqrt(np.sum(S * S, axis=2))
        norm = np.sqrt(np.sum(S_new * S_new, axis=2))
        S_new = S_new * np.divide(target, norm, out=np.zeros_like(norm), where=norm > 0)[:, :, None]
    o = np.einsum("nvf,nf->nv", S_new, pq)
    return o.reshape(B, H, d_v), S_new.reshape(B, H, d_v, d_phi), M_new.reshape(B, H, d_v, d_phi)


def silu_grad(u):
    """d silu(u) / du = sigmoid(u) (1 + u (1 - sigmoid(u)))."""
    u = np.asarray(u, dtype=np.float64)
    sg = 1.0 / (1.0 + np.exp(-u))
    return sg * (1.0 + u * (1.0 - sg))


def backward(q, k, v, dO, *, eta_mode: str = "scalar", eta=None, eta_scalar: float = 1.0,
             beta: float = 0.0, causal: bool = True, phi: str = "identity", w1=None, w3=None):
    """Gradients of sum(o * dO), fp64.

    phi="swiglu": the recurrence below runs on the features phi(q), phi(k)
    (it gives dphi(q), dphi(k) in place of dq, dk), then the chain rule through
    phi(x) = silu(u) * g, u = W1 x, g = W3 x:
      du = dphi * g * silu'(u),  dg = dphi * silu(u)
      dx = W1^T du + W3^T dg,    dW1[h] = sum over b, t of du x^T (q and k both), dW3 alike.
    Returns (dq, dk, dv, deta, dW1, dW3) for SwiGLU.

    The plain reverse-mode derivative of ``forward`` (backpropagation through
    the token loop).  With G_t = dL/dS_t and H_t = dL/dM_t:
      causal:   G_t = dO_t q_t^T + G_{t+1},         G_T = 0
      bidir.:   G_t = sum_s dO_s q_s^T  for every t (only S_{T-1} is read)
                H_t = G_t + beta H_{t+1},           H_T = 0
      dq_t = S_t^T dO_t   (bidirectional: S_{T-1}^T dO_t)
      dv_t = eta_t H_t k_t,  dk_t = eta_t H_t^T v_t,  deta_t = v_t^T H_t k_t
    The rate gradient is returned per token for the per_token mode, as d a_t =
    deta_t * sigmoid(a_t) for softplus, and summed over every token for the
    scalar mode.  Returns (dq, dk, dv, deta).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, T, d_in = q.shape
    d_v = np.shape(v)[-1]
    N = B * H
    xq, xk, vf = _flatten(q, d_in), _flatten(k, d_in), _flatten(v, d_v)
    if phi == "swiglu":
        w1n = np.broadcast_to(np.asarray(w1, np.float64)[None], (B,) + np.shape(w1)).reshape(N, -1, d_in)
        w3n = np.broadcast_to(np.asarray(w3, np.float64)[None], (B,) + np.shape(w3)).reshape(N, -1, d_in)
        qf, kf = features(xq, phi, w1n, w3n), features(xk, phi, w1n, w3n)
    elif phi == "identity":
        qf, kf = xq, xk
    else:
        raise ValueError(f"unknown feature map {phi!r}")
    d_k = qf.shape[-1]
    gf = _flatten(dO, d_v)
    lr = learning_rates(eta_mode, T, N, eta, eta_scalar)
    # forward states S_t (the readout needs them)
    S = np.zeros((N, d_v, d_k))
    M = np.zeros((N, d_v, d_k))
    S_all = np.zeros((T, N, d_v, d_k))
    for t in range(T):
        M = beta * M + lr[:, t, None, None] * vf[:, t, :, None] * kf[:, t, None, :]
        S = S + M
        S_all[t] = S
    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    de = np.zeros((N, T))
    G = np.zeros((N, d_v, d_k))
    if not causal:
        G = np.einsum("ntv,ntf->nvf", gf, qf)
    Hm = np.zeros((N, d_v, d_k))
    for t in range(T - 1, -1, -1):
        if causal:
            G = G + gf[:, t, :, None] * qf[:, t, None, :]
            dq[:, t] = np.einsum("nvf,nv->nf", S_all[t], gf[:, t])
        else:
            dq[:, t] = np.einsum("nvf,nv->nf", S_all[T - 1], gf[:, t])
        Hm = G + beta * Hm
        Hk = np.einsum("nvf,nf->nv", Hm, kf[:, t])
        dv[:, t] = lr[:, t, None] * Hk
        dk[:, t] = lr[:, t, None] * np.einsum("nvf,nv->nf", Hm, vf[:, t])
        de[:, t] = np.einsum("nv,nv->n", vf[:, t], Hk)
    shape = lambda x, d: x.reshape(B, H, T, d)
    if eta_mode == "per_token":
        deta = de.reshape(B, H, T)
    elif eta_mode == "softplus":
        a = np.asarray(eta, np.float64).reshape(N, T)
        deta = (de / (1.0 + np.exp(-a))).reshape(B, H, T)
    else:
        deta = float(de.sum())
    if phi != "swiglu":
        return shape(dq, d_k), shape(dk, d_k), shape(dv, d_v), deta
    # chain rule through the feature map, for q and for k
    dW1 = np.zeros(np.shape(w1))
    dW3 = np.zeros(np.shape(w3))
    dx = []
    for x, dphi in ((xq, dq), (xk, dk)):
        u = np.einsum("nfd,ntd->ntf", w1n, x)
        g = np.einsum("nfd,ntd->ntf", w3n, x)
        du = dphi * g * silu_grad(u)
        dg = dphi * silu(u)
        dx.append(np.einsum("nfd,ntf->ntd", w1n, du) + np.einsum("nfd,ntf->ntd", w3n, dg))
        dW1 += np.einsum("ntf,ntd->nfd", du, x).reshape(B, H, -1, d_in).sum(axis=0)
        dW3 += np.einsum("ntf,ntd->nfd", dg, x).reshape(B, H, -1, d_in).sum(axis=0)
    return shape(dx[0], d_in), shape(dx[1], d_in), shape(dv, d_v), deta, dW1, dW3


# ----------------------------------------------------------------------------
# parallel forms (used by tests to check the equivalence the pages state)
# ----------------------------------------------------------------------------

def _momentum_weights(beta: float, n: int):
    """c_r = sum_{s=0..r} beta^s, r = 0..n-1 (weight of a token r steps back)."""
    c = np.empty(n)
    acc = 0.0
    p = 1.0
    for r in range(n):
        acc += p
        c[r] = acc
        p *= beta
    return c


def forward_closed_form(q, k, v, *, eta_mode="scalar", eta=None, eta_scalar=1.0,
                        beta=0.0, causal=True, phi="identity", w1=None, w3=None):
    """Closed form: O = (Gamma o (Phi_Q Phi_K^T)) diag(eta) V.

    Unrolling the momentum recurrence gives
      S_t = sum_{s<=t} eta_s c_{t-s} v_s phi(k_s)^T,  c_r = sum_{u=0..r} beta^u,
    so the causal output is a masked, reweighted product of the feature
    matrices (Gamma_ts = c_{t-s} for s <= t); bidirectionally every query reads
    S_{T-1}, i.e. Gamma_ts = c_{T-1-s}.  With beta = 0 and eta = 1 this is the
    plain causal linear attention of the blog's "(phi(Q) phi(K)^T) V".
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, T, d_k = q.shape
    d_v = np.shape(v)[-1]
    N = B * H
    qf, kf, vf = _flatten(q, d_k), _flatten(k, d_k), _flatten(v, d_v)
    if phi == "swiglu":
        w1n = np.broadcast_to(np.asarray(w1, np.float64)[None], (B,) + np.shape(w1)).reshape(N, -1, d_k)
        w3n = np.broadcast_to(np.asarray(w3, np.float64)[None], (B,) + np.shape(w3)).reshape(N, -1, d_k)
        pq, pk = features(qf, phi, w1n, w3n), features(kf, phi, w1n, w3n)
    else:
        pq, pk = features(qf, phi), features(kf, phi)
    lr = learning_rates(eta_mode, T, N, eta, eta_scalar)
    c = _momentum_weights(beta, T)
    t_idx = np.arange(T)[:, None]
    s_idx = np.arange(T)[None, :]
    if causal:
        gamma = np.where(s_idx <= t_idx, c[np.clip(t_idx - s_idx, 0, T - 1)], 0.0)
    else:
        gamma = np.broadcast_to(c[T - 1 - s_idx], (T, T))
    scores = np.einsum("ntf,nsf->nts", pq, pk) * gamma[None] * lr[:, None, :]
    o = np.einsum("nts,nsv->ntv", scores, vf)
    return o.reshape(B, H, T, d_v)


def forward_chunked(q, k, v, *, chunk: int, eta_mode="scalar", eta=None, eta_scalar=1.0,
                    beta=0.0, causal=True, phi="identity", w1=None, w3=None):
    """Chunked form: dense blocks inside a chunk, (S, M) carried between chunks.

    For a chunk of n tokens entered with state (S, M) and local indices i, j:
      o_i = S phi(q_i) + g_i M phi(q_i) + sum_{j<=i} c_{i-j} eta_j (phi(q_i).phi(k_j)) v_j
      S'  = S + g_{n-1} M + sum_j eta_j c_{n-1-j} v_j phi(k_j)^T
      M'  = beta^n M + sum_j eta_j beta^{n-1-j} v_j phi(k_j)^T
    with c_r = sum_{u=0..r} beta^u and g_i = sum_{u=1..i+1} beta^u.
    Bidirectional: run the state update over all chunks, then o_t = S phi(q_t).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, T, d_k = q.shape
    d_v = np.shape(v)[-1]
    N = B * H
    qf, kf, vf = _flatten(q, d_k), _flatten(k, d_k), _flatten(v, d_v)
    if phi == "swiglu":
        w1n = np.broadcast_to(np.asarray(w1, np.float64)[None], (B,) + np.shape(w1)).reshape(N, -1, d_k)
        w3n = np.broadcast_to(np.asarray(w3, np.float64)[None], (B,) + np.shape(w3)).reshape(N, -1, d_k)
        pq, pk = features(qf, phi, w1n, w3n), features(kf, phi, w1n, w3n)
    else:
        pq, pk = features(qf, phi), features(kf, phi)
    d_phi = pk.shape[-1]
    lr = learning_rates(eta_mode, T, N, eta, eta_scalar)
    S = np.zeros((N, d_v, d_phi))
    M = np.zeros((N, d_v, d_phi))
    o = np.zeros((N, T, d_v))
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        c = _momentum_weights(beta, n)
        g = beta * c                                   # g_i = beta * c_i
        bp = beta ** np.arange(n)                      # beta^r
        PQ, PK, V, E = pq[:, t0:t0 + n], pk[:, t0:t0 + n], vf[:, t0:t0 + n], lr[:, t0:t0 + n]
        if causal:
            ii = np.arange(n)[:, None]
            jj = np.arange(n)[None, :]
            gam = np.where(jj <= ii, c[np.clip(ii - jj, 0, n - 1)], 0.0)
            A = np.einsum("nif,njf->nij", PQ, PK) * gam[None] * E[:, None, :]
            o[:, t0:t0 + n] = (np.einsum("nvf,nif->niv", S, PQ)
                               + g[None, :, None] * np.einsum("nvf,nif->niv", M, PQ)
                               + np.einsum("nij,njv->niv", A, V))
        wS = E * c[::-1][None, :]                      # eta_j c_{n-1-j}
        wM = E * bp[::-1][None, :]                     # eta_j beta^{n-1-j}
        S = S + g[n - 1] * M + np.einsum("nj,njv,njf->nvf", wS, V, PK)
        M = (beta ** n) * M + np.einsum("nj,njv,njf->nvf", wM, V, PK)
    if not causal:
        o = np.einsum("nvf,ntf->ntv", S, pq)
    return o.reshape(B, H, T, d_v)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over every element (0/0 -> 0)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den
