"""Helpers shared by the GPU parity tests: device upload, library call, oracle.

Expected values always come from ``oracle`` (fp64 CPU) on the same seeded
inputs; nothing here feeds a GPU result back into an expectation.
"""
from __future__ import annotations

import numpy as np

import oracle
from ttt_workloads import Inputs, Workload, bf16_bits_to_f64

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max |gpu - oracle| / max |oracle|


def torch_mod():
    import torch
    return torch


def to_device(x: Inputs):
    torch = torch_mod()
    w = x.workload

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if w.dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.to("cuda")

    out = {"q": dev(x.q_dev), "k": dev(x.k_dev), "v": dev(x.v_dev)}
    out["a"] = torch.from_numpy(x.a32).to("cuda") if x.a32 is not None else None
    out["w1"] = dev(x.w1_dev) if x.w1_dev is not None else None
    out["w3"] = dev(x.w3_dev) if x.w3_dev is not None else None
    out["S0"] = torch.from_numpy(x.S0).to("cuda") if x.S0 is not None else None
    return out


def from_device(t, dtype: str) -> np.ndarray:
    torch = torch_mod()
    if dtype == "bf16":
        return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def make_layer(w: Workload, d, chunk=None, segments=0, value_split=0, launch="auto"):
    import ttt_weight_layers_amd as tla
    return tla.TTTLinearAttention(w.B, w.H, w.T, w.d_k, w.d_v, w.d_phi, dtype=w.dtype, phi=w.phi,
                                  chunk=w.chunk if chunk is None else chunk, segments=segments,
                                  w1=d["w1"], w3=d["w3"], value_split=value_split, launch=launch)


def run_gpu(w: Workload, d, chunk=None, segments=0, eta_sign=1.0, q_override=None, v_scale=None,
            layer=None, value_split=0):
    """Runs the library once on device tensors d; returns o as fp64 numpy."""
    torch = torch_mod()
    lay = layer or make_layer(w, d, chunk, segments, value_split)
    eta = None
    eta_scalar = w.eta_scalar * eta_sign
    if w.eta_mode != "scalar":
        eta = d["a"] if eta_sign == 1.0 else None
        if eta is None:
            if w.eta_mode == "softplus":
                raise ValueError("negating a softplus rate needs per-token eta")
            eta = -d["a"]
    q = d["q"] if q_override is None else q_override
    v = d["v"] if v_scale is None else (d["v"] * v_scale).contiguous()
    if w.weight_norm:
        o = lay.forward_state(q, d["k"], v, eta=eta, eta_scalar=eta_scalar, beta=w.beta, eta_mode=w.eta_mode,
                              S0=d["S0"], weight_norm=True)
    else:
        o = lay.forward(q, d["k"], v, eta=eta, eta_scalar=eta_scalar, beta=w.beta, eta_mode=w.eta_mode,
                        causal=w.causal, loss=w.loss)
    torch.cuda.synchronize()
    return from_device(o, w.dtype)


def run_oracle(w: Workload, x: Inputs, heads=None, q64=None):
    """Oracle output for all heads, or for flat head indices ``heads``."""
    q = x.q64 if q64 is None else q64
    k, v = x.k64, x.v64
    a = x.a32
    w1, w3 = x.w1_64, x.w3_64
    if heads is not None:
        B, H = w.B, w.H
        bs = [hh // H for hh in heads]
        hs = [hh % H for hh in heads]
        sel = lambda t: t[bs, hs][:, None]          # [n, 1, T, d]
        q, k, v = sel(q), sel(k), sel(v)
        if a is not None:
            a = a[bs, hs][:, None]
        if w1 is not None:
            # per-sequence weights: run head by head
            outs = []
            for i, h in enumerate(hs):
                outs.append(oracle.forward(q[i:i + 1], k[i:i + 1], v[i:i + 1], eta_mode=w.eta_mode,
                                           eta=None if a is None else a[i:i + 1],
                                           eta_scalar=w.eta_scalar, beta=w.beta, causal=w.causal,
                                           phi=w.phi, w1=w1[h:h + 1], w3=w3[h:h + 1], loss=w.loss,
                                           **_wn(w, x, [bs[i]], [h])))
            return np.concatenate(outs, axis=0)
        return oracle.forward(q, k, v, eta_mode=w.eta_mode, eta=a, eta_scalar=w.eta_scalar, beta=w.beta,
                              causal=w.causal, phi=w.phi, w1=w1, w3=w3, loss=w.loss, **_wn(w, x, bs, hs))
    return oracle.forward(q, k, v, eta_mode=w.eta_mode, eta=a, eta_scalar=w.eta_scalar, beta=w.beta,
                          causal=w.causal, phi=w.phi, w1=w1, w3=w3, loss=w.loss, **_wn(w, x))


def _wn(w: Workload, x: Inputs, bs=None, hs=None):
    """Oracle arguments of a weight-normalised workload (the entry state of the
    selected sequences, as [n, 1, d_v, d_phi])."""
    if not w.weight_norm:
        return {}
    S0 = x.S0.astype(np.float64)
    if bs is not None:
        S0 = S0[bs, hs][:, None]
    return {"S0": S0, "weight_norm": True}


def select_heads(o: np.ndarray, w: Workload, heads):
    bs = [hh // w.H for hh in heads]
    hs = [hh % w.H for hh in heads]
    return o[bs, hs][:, None]
