"""Seeded synthetic inputs for the TTT-as-linear-attention forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds the workload shapes and the recipe that draws q, k, v,
the learning-rate logits a and the frozen feature-map weights W1, W3.  It does
none of the layer's arithmetic: no feature map, no learning rate, no state.

The workloads stand in for the activations of the LLM and ViT models that the
ablation of "Test-Time Training with KV Binding Is Secretly Linear Attention"
measures (page thelatestinai.com, Table 2): those models, their datasets and
their trained weights are not available, so seeded Gaussian tensors of the same
shapes are used instead.

Recipe (per workload, numpy PCG64 ``default_rng(seed)``):
  1. q, k, v drawn in that order as full C-order fp64 ``standard_normal``
     tensors of shape [B, H, T, d], then scaled by 1/sqrt(d).
  2. Workloads marked ``l2norm``: each token of q, k and v is divided by its
     Euclidean norm (in fp64).
  3. Cast to the workload dtype: fp64 -> fp32 (round to nearest even), and for
     bf16 a further fp32 -> bf16 round to nearest even.
  4. If the learning rate is per token: a ~ N(-2, 1) of shape [B, H, T], kept
     as fp32 (one more ``standard_normal`` draw, shifted by -2).
  5. If the feature map is SwiGLU: W1 then W3 ~ N(0, 1)/sqrt(128), shape
     [H, d_phi, d_k] (out x in), cast like q.
  6. Workloads with a weight-normalised fast weight (Variant 1): the entry
     state S0 ~ N(0, 1)/sqrt(d_phi), shape [B, H, d_v, d_phi], fp32 (the
     stand-in for the learned initial fast weight whose row norms the
     normalisation keeps).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "Inputs", "make_inputs", "f64_to_bf16_bits",
           "bf16_bits_to_f64", "round_to_dtype"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and settings of one synthetic workload."""
    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    d_phi: int
    dtype: str            # "f32" or "bf16" (q, k, v, o and W1, W3)
    phi: str              # "identity" or "swiglu"
    eta_mode: str         # "scalar", "per_token" or "softplus"
    eta_scalar: float     # used when eta_mode == "scalar"
    beta: float           # momentum; 0 disables it
    causal: bool
    chunk: int            # tiling hint passed to the library (0 = auto)
    l2norm: bool          # per-token L2 normalisation of q, k, v
    seed: int
    note: str = ""
    loss: str = "dot"     # binding loss: "dot" (linear attention) or "mse" (delta rule)
    weight_norm: bool = False   # Variant 1: rows of S kept at their entry-state norms

    @property
    def n_seq(self) -> int:
        return self.B * self.H

    @property
    def tokens(self) -> int:
        """Positions per forward: B*T, all heads (one token = one position)."""
        return self.B * self.T

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T

    def with_shape(self, B: Optional[int] = None, H: Optional[int] = None,
                   T: Optional[int] = None, name: Optional[str] = None) -> "Workload":
        """Same settings at another shape (reduced sizes for parity tests)."""
        B = self.B if B is None else B
        H = self.H if H is None else H
        T = self.T if T is None else T
        nm = name or f"{self.name}@{B}x{H}x{T}"
        return dataclasses.replace(self, B=B, H=H, T=T, name=nm)

    def with_settings(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The synthetic workloads.  Seeds 1001..1009 in this order.
WORKLOADS = {
    # Plain causal linear attention (the last row of the ablation, Table 2, with a
    # constant unit step and no momentum), fp32.
    "v5_f32_1x1x256_d64": Workload(
        "v5_f32_1x1x256_d64", B=1, H=1, T=256, d_k=64, d_v=64, d_phi=64,
        dtype="f32", phi="identity", eta_mode="scalar", eta_scalar=1.0, beta=0.0,
        causal=True, chunk=0, l2norm=False, seed=1001,
        note="V5, eta=1, no momentum, fp32"),
    # Momentum SGD, constant step 0.1, L2-normalised tokens.
    "v4_momentum_4x8x2048_d128": Workload(
        "v4_momentum_4x8x2048_d128", B=4, H=8, T=2048, d_k=128, d_v=128, d_phi=128,
        dtype="bf16", phi="identity", eta_mode="scalar", eta_scalar=0.1, beta=0.9,
        causal=True, chunk=64, l2norm=True, seed=1002,
        note="V4, eta=0.1, beta=0.9, chunk 64"),
    # Per-token learning rate eta_t = softplus(a_t) plus momentum.
    "v3_softplus_8x16x4096_d128": Workload(
        "v3_softplus_8x16x4096_d128", B=8, H=16, T=4096, d_k=128, d_v=128, d_phi=128,
        dtype="bf16", phi="identity", eta_mode="softplus", eta_scalar=0.0, beta=0.9,
        causal=True, chunk=64, l2norm=False, seed=1003,
        note="V3, eta=softplus(a), a~N(-2,1), beta=0.9, chunk 64"),
    # Frozen two-layer SwiGLU fast-weight MLP, last layer updated.
    "v2_swiglu_4x16x8192_d128_f512": Workload(
        "v2_swiglu_4x16x8192_d128_f512", B=4, H=16, T=8192, d_k=128, d_v=128, d_phi=512,
        dtype="bf16", phi="swiglu", eta_mode="softplus", eta_scalar=0.0, beta=0.9,
        causal=True, chunk=64, l2norm=False, seed=1004,
        note="V2, SwiGLU phi 128->512, eta=softplus(a), beta=0.9, chunk 64"),
    # Long-context prefill, plain linear attention.
    "v5_long_1x16x65536_d128": Workload(
        "v5_long_1x16x65536_d128", B=1, H=16, T=65536, d_k=128, d_v=128, d_phi=128,
        dtype="bf16", phi="identity", eta_mode="scalar", eta_scalar=1.0, beta=0.0,
        causal=True, chunk=128, l2norm=False, seed=1005,
        note="V5 at 64k, eta=1, no momentum, chunk 128"),
    # Long-context prefill, per-token lr and momentum.
    "v3_long_1x16x65536_d128": Workload(
        "v3_long_1x16x65536_d128", B=1, H=16, T=65536, d_k=128, d_v=128, d_phi=128,
        dtype="bf16", phi="identity", eta_mode="softplus", eta_scalar=0.0, beta=0.9,
        causal=True, chunk=128, l2norm=False, seed=1006,
        note="V3 at 64k, eta=softplus(a), beta=0.9, chunk 128"),
    # ViT-shaped bidirectional run: every token updates the state before any readout.
    "bidir_vit_256x6x196_d64": Workload(
        "bidir_vit_256x6x196_d64", B=256, H=6, T=196, d_k=64, d_v=64, d_phi=64,
        dtype="bf16", phi="identity", eta_mode="scalar", eta_scalar=1.0, beta=0.0,
        causal=False, chunk=0, l2norm=False, seed=1007,
        note="bidirectional, eta=1, no momentum"),
    # The mean-squared binding loss (delta rule) at the Variant-3 shape: per-token rate,
    # no momentum, L2-normalised tokens (each step is then a contraction along k).
    "v3_delta_8x16x4096_d128": Workload(
        "v3_delta_8x16x4096_d128", B=8, H=16, T=4096, d_k=128, d_v=128, d_phi=128,
        dtype="bf16", phi="identity", eta_mode="softplus", eta_scalar=0.0, beta=0.0,
        causal=True, chunk=0, l2norm=True, seed=1008,
        note="delta rule (MSE loss), eta=softplus(a), no momentum", loss="mse"),
    # Variant 1: the Variant 2 layer with its updated layer weight-normalised
    # (recurrent implementation only), from a drawn entry state.
    "v1_weightnorm_4x16x8192_d128_f512": Workload(
        "v1_weightnorm_4x16x8192_d128_f512", B=4, H=16, T=8192, d_k=128, d_v=128, d_phi=512,
        dtype="bf16", phi="swiglu", eta_mode="softplus", eta_scalar=0.0, beta=0.9,
        causal=True, chunk=0, l2norm=False, seed=1009,
        note="V1, V2 with weight-normalised rows of S, recurrent", weight_norm=True),
}


@dataclasses.dataclass
class Inputs:
    """One drawn input set.

    Arrays ending in ``64`` hold the exact values the device receives, upcast to
    fp64 (so the oracle consumes what the kernels consume).  ``*_dev`` arrays
    hold the device representation: float32, or uint16 bf16 bit patterns.
    """
    workload: Workload
    q64: np.ndarray
    k64: np.ndarray
    v64: np.ndarray
    q_dev: np.ndarray
    k_dev: np.ndarray
    v_dev: np.ndarray
    a32: Optional[np.ndarray] = None        # [B,H,T] fp32 logits (softplus mode)
    w1_64: Optional[np.ndarray] = None
    w3_64: Optional[np.ndarray] = None
    w1_dev: Optional[np.ndarray] = None
    w3_dev: Optional[np.ndarray] = None
    S0: Optional[np.ndarray] = None         # [B,H,d_v,d_phi] fp32 entry state (weight_norm)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE) bit patterns as uint16."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    # round to nearest even on the 16 dropped bits; NaN is kept quiet
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(f)
    out = r.astype(np.uint16)
    if nan.any():
        out = np.where(nan, np.uint16(0x7FC0), out)
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    u = (b.astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


def round_to_dtype(x: np.ndarray, dtype: str):
    """Returns (device array, exact fp64 copy of it)."""
    if dtype == "f32":
        d = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
        return d, d.astype(np.float64)
    if dtype == "bf16":
        d = f64_to_bf16_bits(x)
        return d, bf16_bits_to_f64(d)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draws one input set for workload ``w`` (seed defaults to ``w.seed``)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp_k = (w.B, w.H, w.T, w.d_k)
    shp_v = (w.B, w.H, w.T, w.d_v)
    raw = {}
    for name, shp, d in (("q", shp_k, w.d_k), ("k", shp_k, w.d_k), ("v", shp_v, w.d_v)):
        x = rng.standard_normal(shp) / np.sqrt(d)
        if w.l2norm:
            x = x / np.linalg.norm(x, axis=-1, keepdims=True)
        raw[name] = round_to_dtype(x, w.dtype)
        del x
    a32 = None
    if w.eta_mode in ("per_token", "softplus"):
        a32 = (rng.standard_normal((w.B, w.H, w.T)) - 2.0).astype(np.float32)
    w1_64 = w3_64 = w1_dev = w3_dev = None
    if w.phi == "swiglu":
        s = 1.0 / np.sqrt(128.0)
        w1_dev, w1_64 = round_to_dtype(rng.standard_normal((w.H, w.d_phi, w.d_k)) * s, w.dtype)
        w3_dev, w3_64 = round_to_dtype(rng.standard_normal((w.H, w.d_phi, w.d_k)) * s, w.dtype)
    S0 = None
    if w.weight_norm:
        S0 = (rng.standard_normal((w.B, w.H, w.d_v, w.d_phi)) / np.sqrt(w.d_phi)).astype(np.float32)
    return Inputs(workload=w,
                  q64=raw["q"][1], k64=raw["k"][1], v64=raw["v"][1],
                  q_dev=raw["q"][0], k_dev=raw["k"][0], v_dev=raw["v"][0],
                  a32=a32, w1_64=w1_64, w3_64=w3_64, w1_dev=w1_dev, w3_dev=w3_dev, S0=S0)


def head_subset(w: Workload, n: int = 8, seed: Optional[int] = None):
    """A fixed subset of (b, h) pairs for oracle checks at full T.

    Always contains (0, 0) and (B-1, H-1); the rest are drawn with the
    workload seed.  Returns a sorted list of flat indices b*H + h.
    """
    total = w.B * w.H
    if total <= n:
        return list(range(total))
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    chosen = {0, total - 1}
    while len(chosen) < n:
        chosen.add(int(rng.integers(0, total)))
    return sorted(chosen)
