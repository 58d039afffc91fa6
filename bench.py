#!/usr/bin/env python3
"""Throughput of the TTT-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full forward of the layer (every kernel of the chunked path:
segment summaries, segment scan, output pass; the SwiGLU feature map where the
workload has it) over one batch of seeded synthetic q, k, v already resident in
HBM.  Without --workload every workload of DEFAULT_ORDER is run in turn and
prints its own JSON line; the last line is the Variant 2 SwiGLU workload
(B=4, H=16, T=8192, d=128 -> 512 features: the most work per step and the only
one bound by the matrix cores; thelatestinai.com page, Table 2).  Input sets are
rotated so that the working set of the timed loop exceeds the 256 MB
last-level cache.

Each line carries tokens/s (tokens = B*T positions), the roofline of the
dominant kernel (its duration measured with HIP events on the stream it runs
on, during the timed loop) and of the whole step (algorithmic work / time per
step), and the CPU oracle's tokens/s on a bounded sample of the same workload,
timed over worker processes forked before the first GPU call.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TTT-layer fwd tokens/sec (1 GPU) + % MFMA/HBM roofline, Variants 2–5"
DEFAULT_WORKLOAD = "v4_momentum_4x8x2048_d128"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6   # dense bf16, 256 CU x 2.4 GHz x 4096 flop/clk
F32_PEAK_TFLOPS = 157.3          # fp32 vector (and matrix) peak
# The output kernel of one timed step in TIMING_EVERY carries a pair of HIP events:
# an event pair costs the stream a little time of its own, which would otherwise
# show up in every step of the throughput figure.
TIMING_EVERY = 8


def timed_calls(steps: int) -> int:
    """Timed launches among `steps` calls when the first and every TIMING_EVERY-th one are timed."""
    return max(1, (steps + TIMING_EVERY - 1) // TIMING_EVERY)
MALL_BYTES = 256 * 2 ** 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "ttt_weight_layers_amd", "csrc", "chunk_mfma.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="one workload (default: every workload of DEFAULT_ORDER, one line each, "
                         "the SwiGLU case last)")
    ap.add_argument("--segments", type=int, default=0, help="plan override: sequence segments (0 = auto)")
    ap.add_argument("--value-split", type=int, default=0, help="plan override: workgroups per value width")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--launch", default="auto", choices=["auto", "separate", "single", "prefix"],
                    help="how a segmented causal forward is launched")
    ap.add_argument("--decode", action="store_true",
                    help="time the one-token recurrent step (ttt_la_step) at the workload's B, H and widths "
                         "instead of the forward; prints its own JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="time ttt_la_backward (gradients of the forward) on the workload instead of the forward; "
                         "prints its own JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device copy of MIB mebibytes (counter calibration) and exit")
    return ap.parse_args()


def algorithmic_bytes_per_ht(w) -> int:
    """q, k, v read once and o written once (+ 4 B of per-token eta / logits)."""
    e = 4 if w.dtype == "f32" else 2
    b = (2 * w.d_k + w.d_v) * e + w.d_v * e
    if w.eta_mode != "scalar":
        b += 4
    return b


# tokens per chunk of the delta-rule kernel
DELTA_CHUNK = 32


def algorithmic_flops_per_ht(w, chunk: int) -> int:
    """Causal intra-chunk triangle + state readout and update (x2 with momentum)
    + SwiGLU feature map for q and k.  Delta rule (loss "mse"): K S^T, Q S^T and
    the update U^T K (3 d_k d_v multiply-adds) plus the half triangles of K K^T,
    Q K^T, tril(Q K^T) U and the solve for U (C/2 (2 d_k + 2 d_v))."""
    if w.loss == "mse":
        return 2 * (3 * w.d_k * w.d_v + DELTA_CHUNK // 2 * (2 * w.d_k + 2 * w.d_v))
    if w.weight_norm:
        # the recurrence: per state entry and token, the momentum and state updates and
        # the two row sums (norm and readout), four multiply-adds; fp32 vector work
        return 8 * w.d_v * w.d_phi
    if not w.causal:
        return 4 * w.d_phi * w.d_v
    f = (chunk + 1) * (w.d_phi + w.d_v) + 4 * w.d_phi * w.d_v * (2 if w.beta != 0.0 else 1)
    if w.phi == "swiglu":
        f += 8 * w.d_k * w.d_phi
    return f


def source_hash(kernel: str) -> str:
    """Hash of the code that compiles into `kernel`: the source file whose
    __global__ function carries its name, and the headers that file includes,
    followed through their own includes."""
    csrc = os.path.dirname(KERNEL_SOURCE)
    inc = os.path.join(ROOT, "include")
    base = kernel.split("<")[0]
    pat = re.compile(r"__global__[^;{]*?\b" + re.escape(base) + r"\s*\(")
    srcs = [n for n in sorted(os.listdir(csrc)) if n.endswith(".hip")
            and pat.search(open(os.path.join(csrc, n)).read())]
    if len(srcs) != 1:
        return ""
    todo, seen = [os.path.join(csrc, srcs[0])], []
    while todo:
        path = todo.pop()
        if path in seen:
            continue
        seen.append(path)
        text = open(path).read()
        for name in re.findall(r'^#include "([^"]+)"', text, re.M):
            for d in (csrc, inc):
                if os.path.exists(os.path.join(d, name)):
                    todo.append(os.path.join(d, name))
                    break
    h = hashlib.sha256()
    for path in sorted(seen):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the timed kernel from the committed counter runs,
    or None if they were taken on another kernel or on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_hash") != source_hash(kernel) or e.get("kernel") != kernel:
        return None
    return e.get("bytes_per_launch")


# Workloads of the default run, in the order their lines are printed: the
# Variant 2 SwiGLU case, the one bound by the matrix cores and the most work per
# step, comes last.
DEFAULT_ORDER = (
    "v5_f32_1x1x256_d64",
    "v4_momentum_4x8x2048_d128",
    "v3_softplus_8x16x4096_d128",
    "v5_long_1x16x65536_d128",
    "v3_long_1x16x65536_d128",
    "bidir_vit_256x6x196_d64",
    "v3_delta_8x16x4096_d128",
    "v1_weightnorm_4x16x8192_d128_f512",
    "v2_swiglu_4x16x8192_d128_f512",
)
# Worker processes of the oracle timing: the host cores this process may use,
# at most 16 (the CPU share of one GPU).
MAX_ORACLE_WORKERS = 16


def oracle_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(MAX_ORACLE_WORKERS, n))


def make_oracle_pool(n: int):
    """A pool of n forked worker processes.  Created before the first GPU call
    of the process (a child forked after it would share the parent's device
    state); each worker runs the oracle with one BLAS thread."""
    import multiprocessing as mp
    return mp.get_context("fork").Pool(processes=n, initializer=_oracle_worker_init)


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass


def _oracle_task(task):
    """One sampled sequence in a worker: (workload, q, k, v, a, w1, w3, S0) fp64
    slices of one (b, h) -> (o [1, 1, T, d_v], seconds)."""
    import oracle
    w, q, k, v, a, w1, w3, S0 = task
    t0 = time.perf_counter()
    extra = {"S0": S0, "weight_norm": True} if w.weight_norm else {}
    o = oracle.forward(q, k, v, eta_mode=w.eta_mode, eta=a, eta_scalar=w.eta_scalar, beta=w.beta,
                       causal=w.causal, phi=w.phi, w1=w1, w3=w3, loss=w.loss, **extra)
    return o, time.perf_counter() - t0


def baseline_heads(w, n_workers: int):
    """The sampled (b, h) sequences at full T: every sequence when there are at
    most 2 n_workers of them, else n_workers of them (at least 8), always with
    (0, 0) and (B-1, H-1)."""
    from ttt_workloads import head_subset
    total = w.B * w.H
    if total <= 2 * n_workers:
        return list(range(total))
    return head_subset(w, max(8, n_workers))


def cpu_baseline(w, x, pool=None, n_workers: int = 1):
    """Times the fp64 oracle (the recurrence of ``oracle.forward``, untuned) on a
    bounded sample of the workload: whole sequences at full T, one per worker
    task, spread over ``n_workers`` processes of ``pool`` (in this process when
    pool is None).  Returns (baseline dict, oracle outputs [n, 1, T, d_v], heads)."""
    import numpy as np
    heads = baseline_heads(w, n_workers if pool is not None else 1)
    tasks = []
    for hh in heads:
        b, h = hh // w.H, hh % w.H
        sl = lambda t: np.ascontiguousarray(t[b:b + 1, h:h + 1])
        tasks.append((w, sl(x.q64), sl(x.k64), sl(x.v64),
                      None if x.a32 is None else np.ascontiguousarray(x.a32[b:b + 1, h:h + 1]),
                      None if x.w1_64 is None else x.w1_64[h:h + 1],
                      None if x.w3_64 is None else x.w3_64[h:h + 1],
                      None if x.S0 is None else sl(x.S0).astype(np.float64)))
    t0 = time.perf_counter()
    if pool is None:
        res = [_oracle_task(t) for t in tasks]
        cores = 1
    else:
        res = pool.map(_oracle_task, tasks, chunksize=1)
        cores = min(n_workers, len(tasks))
    wall = time.perf_counter() - t0
    o = np.concatenate([r[0] for r in res], axis=0)
    cpu_s = sum(r[1] for r in res)
    head_tokens_per_s = len(heads) * w.T / wall
    return {
        "value": round(head_tokens_per_s / w.H, 1),   # tokens = positions, all heads
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{len(heads)} of {w.B * w.H} (b,h) sequences at full T={w.T}, fp64 numpy recurrence, "
                  f"one sequence per task over {cores} worker processes (one BLAS thread each): "
                  f"{wall:.1f} s wall, {cpu_s:.1f} s of CPU; head-tokens/s={head_tokens_per_s:.4g}",
    }, o, heads


def step_bytes(w) -> int:
    """Algorithmic bytes of one recurrent step: S and M read and written once (fp32),
    q, k, v read and o written for one token per (b, h) (+4 B of rate)."""
    e = 4 if w.dtype == "f32" else 2
    n = w.B * w.H
    b = n * (2 * 2 * w.d_v * w.d_phi * 4 + (2 * w.d_k + 2 * w.d_v) * e)
    if w.eta_mode != "scalar":
        b += n * 4
    return b


def run_decode(args, w):
    """K one-token steps of every (b, h) of workload w, the fp32 state resident in
    HBM; the states are rotated over enough sets to exceed the last-level cache."""
    import numpy as np
    import torch

    import ttt_weight_layers_amd as tla
    from ttt_workloads import make_inputs

    n_tok = 16
    x = make_inputs(w.with_shape(T=n_tok))
    dev = torch.device("cuda:0")

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).to(dev)

    q, k, v = up(x.q_dev), up(x.k_dev), up(x.v_dev)
    toks = [(q[:, :, t:t + 1].contiguous(), k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous(),
             None if x.a32 is None else torch.from_numpy(x.a32[:, :, t].copy()).to(dev)) for t in range(n_tok)]
    w1 = up(x.w1_dev) if x.w1_dev is not None else None
    w3 = up(x.w3_dev) if x.w3_dev is not None else None
    lay = tla.TTTLinearAttention(w.B, w.H, 1, w.d_k, w.d_v, w.d_phi, dtype=w.dtype, phi=w.phi, w1=w1, w3=w3)
    state_bytes = 2 * w.B * w.H * w.d_v * w.d_phi * 4
    n_sets = max(1, min(64, -(-2 * MALL_BYTES // state_bytes)))
    g = torch.Generator(device=dev).manual_seed(w.seed)
    states = [(torch.randn((w.B, w.H, w.d_v, w.d_phi), generator=g, device=dev) * 0.05,
               torch.randn((w.B, w.H, w.d_v, w.d_phi), generator=g, device=dev) * 0.05) for _ in range(n_sets)]
    outs = [torch.empty((w.B, w.H, 1, w.d_v), dtype=v.dtype, device=dev) for _ in range(n_tok)]
    stream = torch.cuda.current_stream()
    # the workload's own step: the mean-squared loss and the weight normalisation included
    mode = tla.mode_bits(w.eta_mode, True, w.loss, weight_norm=w.weight_norm)

    def step(i):
        qt, kt, vt, et = toks[i % n_tok]
        S, M = states[i % n_sets]
        st = tla.ttt_la_step(lay.handle, qt.data_ptr(), kt.data_ptr(), vt.data_ptr(),
                             None if et is None else et.data_ptr(), w.eta_scalar, w.beta, mode,
                             S.data_ptr(), M.data_ptr(), outs[i % n_tok].data_ptr(), stream.cuda_stream)
        if st != 0:
            raise tla.TTTError(st, "ttt_la_step")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_timed = timed_calls(args.steps)
    if tla.ttt_la_enable_kernel_timing_every(lay.handle, n_timed, TIMING_EVERY) != 0:
        raise RuntimeError("could not create timing events")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    kms = float(np.mean(tla.ttt_la_kernel_times(lay.handle, n_timed)))
    tla.ttt_la_enable_kernel_timing(lay.handle, 0)
    nbytes = step_bytes(w)
    achieved = nbytes / (kms * 1e-3) / 1e9
    return {
        "metric": "TTT-layer decode tokens/sec (1 GPU, one recurrent step per token) + % HBM roofline",
        "value": round(w.B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 state, " + w.dtype + " tokens", "data": "synthetic",
        "config": {"workload": w.name + " (decode)", "B": w.B, "H": w.H, "d_k": w.d_k, "d_v": w.d_v,
                   "d_phi": w.d_phi, "phi": w.phi, "eta": w.eta_mode if w.eta_mode != "scalar" else w.eta_scalar,
                   "beta": w.beta, "loss": w.loss, "weight_norm": w.weight_norm, "state_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "step_kernel",
                     "kernel_ms": round(kms, 5), "bytes_per_step": nbytes},
        "cpu_baseline": None,
    }


def run_backward(args, w):
    """K backward passes over the workload (inputs and the output gradient resident
    in HBM, rotated over sets like the forward).  Bytes of the roofline: q, k, v, dO
    read once and dq, dk, dv written once (+ the rate and its gradient)."""
    import numpy as np
    import torch

    import ttt_weight_layers_amd as tla
    from ttt_workloads import make_inputs

    x = make_inputs(w)
    dev = torch.device("cuda:0")

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).to(dev)

    q0, k0, v0 = up(x.q_dev), up(x.k_dev), up(x.v_dev)
    a0 = torch.from_numpy(x.a32).to(dev) if x.a32 is not None else None
    g = torch.Generator(device=dev).manual_seed(w.seed)
    dO0 = torch.randn(v0.shape, generator=g, device=dev).to(v0.dtype)
    e = 4 if w.dtype == "f32" else 2
    nbytes = w.head_tokens * ((2 * w.d_k + 2 * w.d_v) * e + (2 * w.d_k + w.d_v) * e)
    if w.eta_mode != "scalar":
        nbytes += w.head_tokens * 8
    n_sets = max(1, min(8, -(-2 * MALL_BYTES // nbytes)))
    sets = [dict(q=q0.clone(), k=k0.clone(), v=v0.clone(), dO=dO0.clone(), a=None if a0 is None else a0.clone())
            for _ in range(n_sets)]
    w1 = up(x.w1_dev) if x.w1_dev is not None else None
    w3 = up(x.w3_dev) if x.w3_dev is not None else None
    swiglu = w.phi == "swiglu"
    if swiglu:
        nbytes += 2 * w.H * w.d_phi * w.d_k * (e + 4)     # W1, W3 read, dW1, dW3 written (fp32)
    lay = tla.TTTLinearAttention(w.B, w.H, w.T, w.d_k, w.d_v, w.d_phi, dtype=w.dtype, phi=w.phi, chunk=w.chunk,
                                 segments=args.segments, w1=w1, w3=w3)
    mode = tla.mode_bits(w.eta_mode, w.causal)
    st, ws_bytes = tla.ttt_la_backward_workspace(lay.handle, mode)
    if st != 0:
        raise tla.TTTError(st, "ttt_la_backward_workspace")
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    outs = dict(dq=torch.empty_like(q0), dk=torch.empty_like(k0), dv=torch.empty_like(v0),
                de=torch.empty(q0.shape[:-1], dtype=torch.float32, device=dev))
    if swiglu:
        outs["dw1"] = torch.empty((w.H, w.d_phi, w.d_k), dtype=torch.float32, device=dev)
        outs["dw3"] = torch.empty_like(outs["dw1"])
    stream = torch.cuda.current_stream()

    def step(i):
        s_ = sets[i % n_sets]
        args_ = (lay.handle, s_["q"].data_ptr(), s_["k"].data_ptr(), s_["v"].data_ptr(),
                 None if s_["a"] is None else s_["a"].data_ptr(), w.eta_scalar, w.beta, mode,
                 s_["dO"].data_ptr(), outs["dq"].data_ptr(), outs["dk"].data_ptr(),
                 outs["dv"].data_ptr(), outs["de"].data_ptr())
        if swiglu:
            r = tla.ttt_la_backward_swiglu(*args_, outs["dw1"].data_ptr(), outs["dw3"].data_ptr(), ws.data_ptr(),
                                           ws_bytes, stream.cuda_stream)
        else:
            r = tla.ttt_la_backward(*args_, ws.data_ptr(), ws_bytes, stream.cuda_stream)
        if r != 0:
            raise tla.TTTError(r, "ttt_la_backward")

    for i in range(args.warmup):
        step(i)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {
        "metric": "TTT-layer backward tokens/sec (1 GPU) + % HBM roofline of the whole backward",
        "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name + " (backward)", "B": w.B, "H": w.H, "T": w.T, "d_k": w.d_k, "d_v": w.d_v,
                   "d_phi": w.d_phi, "phi": w.phi,
                   "eta": w.eta_mode if w.eta_mode != "scalar" else w.eta_scalar, "beta": w.beta,
                   "causal": w.causal, "segments": lay.plan().segments, "input_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": ("whole backward (features, 2 P + 1 forwards, chain rule through phi, dW)" if swiglu
                                else "whole backward (3 forwards + reversal + finalize)"),
                     "bytes_per_step": nbytes},
        "cpu_baseline": None,
    }


def roofline_of(w, chunk: int, seconds: float):
    """Roofline object for the algorithmic work of one forward done in `seconds`:
    bf16 work is priced against the dense bf16 MFMA peak, fp32 work (vector ALU)
    against the fp32 vector peak; below the ridge of that peak and HBM it is
    HBM-bound."""
    bpht = algorithmic_bytes_per_ht(w)
    flops_ht = algorithmic_flops_per_ht(w, chunk)
    peak_flops, bound = ((MFMA_BF16_PEAK_TFLOPS, "mfma") if w.dtype == "bf16" and not w.weight_norm
                         else (F32_PEAK_TFLOPS, "alu"))
    ridge = peak_flops * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops_ht / bpht < ridge:
        achieved = w.head_tokens * bpht / seconds / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = w.head_tokens * flops_ht / seconds / 1e12
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak_flops, "unit": "TFLOP/s",
            "frac": round(achieved / peak_flops, 4)}


def timed_kernel_name(plan, w, launch: str) -> str:
    """The kernel that carries the timing events (the output pass of the plan)."""
    if w.loss == "mse":
        return "delta_walk"
    if w.weight_norm:
        return "wn_forward"
    if plan.path == 3:
        # the bidirectional SwiGLU pass runs on the 16x16-tile kernel
        return "chunk_kernel<BIDIR>" if not w.causal else "swiglu_kernel<OUTPUT>"
    if plan.path == 2:
        if not w.causal:
            return "wide_kernel<BIDIR>"
        if plan.n_kernels == 1 and plan.segments > 1:
            return "wide_kernel<FUSED>" if launch == "single" else "wide_kernel<PREFIX>"
        return "wide_kernel<OUTPUT>"
    if plan.path == 1:
        return "chunk_kernel<BIDIR>" if not w.causal else "chunk_kernel<OUTPUT>"
    if plan.path == 4:
        return "short_forward"
    return "generic_forward"


def run_forward(args, w, pool=None, n_workers: int = 1):
    """K timed forwards of workload w; returns the JSON object of its line."""
    import numpy as np
    import torch

    import ttt_weight_layers_amd as tla
    from ttt_workloads import make_inputs, bf16_bits_to_f64

    x = make_inputs(w)
    dev = torch.device("cuda:0")

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).to(dev)

    q0, k0, v0 = up(x.q_dev), up(x.k_dev), up(x.v_dev)
    a0 = torch.from_numpy(x.a32).to(dev) if x.a32 is not None else None
    w1 = up(x.w1_dev) if x.w1_dev is not None else None
    w3 = up(x.w3_dev) if x.w3_dev is not None else None
    bpht = algorithmic_bytes_per_ht(w)
    set_bytes = w.head_tokens * bpht
    n_sets = max(1, min(16, -(-2 * MALL_BYTES // set_bytes)))
    sets = []
    for i in range(n_sets):
        s = dict(q=q0 if i == 0 else q0.clone(), k=k0 if i == 0 else k0.clone(),
                 v=v0 if i == 0 else v0.clone(), a=None if a0 is None else (a0 if i == 0 else a0.clone()),
                 o=torch.empty_like(v0))
        sets.append(s)

    layer = tla.TTTLinearAttention(w.B, w.H, w.T, w.d_k, w.d_v, w.d_phi, dtype=w.dtype, phi=w.phi,
                                   chunk=w.chunk, segments=args.segments, w1=w1, w3=w3,
                                   value_split=args.value_split, launch=args.launch)
    plan = layer.plan()
    stream = torch.cuda.current_stream()
    mode = tla.mode_bits(w.eta_mode, w.causal, w.loss, weight_norm=w.weight_norm)
    chunk = DELTA_CHUNK if w.loss == "mse" else plan.chunk
    # the weight-normalised recurrence starts from the drawn entry state (no final state)
    S0 = torch.from_numpy(x.S0).to(dev) if w.weight_norm else None

    def step(i):
        s = sets[i % n_sets]
        a_ptr = None if s["a"] is None else s["a"].data_ptr()
        if w.weight_norm:
            st = tla.ttt_la_forward_state(layer.handle, s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(),
                                          a_ptr, w.eta_scalar, w.beta, mode, S0.data_ptr(), None,
                                          s["o"].data_ptr(), None, None, stream.cuda_stream)
        else:
            st = tla.ttt_la_forward(layer.handle, s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(),
                                    a_ptr, w.eta_scalar, w.beta, mode, s["o"].data_ptr(), stream.cuda_stream)
        if st != 0:
            raise tla.TTTError(st, "ttt_la_forward")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed loop; HIP events around the output kernel of one forward in TIMING_EVERY
    n_timed = timed_calls(args.steps)
    if tla.ttt_la_enable_kernel_timing_every(layer.handle, n_timed, TIMING_EVERY) != 0:
        raise RuntimeError("could not create timing events")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    kernel_ms = tla.ttt_la_kernel_times(layer.handle, n_timed)
    tla.ttt_la_enable_kernel_timing(layer.handle, 0)
    if plan.n_kernels == 1 and plan.segments > 1 and args.launch == "single" and layer.wait_failed():
        raise RuntimeError("a bounded wait of the single-launch path gave up: its outputs are invalid")
    ms_per_step = total_ms / args.steps
    tokens_per_s = w.tokens / (ms_per_step * 1e-3)
    k_avg_ms = float(np.mean(kernel_ms)) if kernel_ms else float("nan")

    roof = roofline_of(w, chunk, k_avg_ms * 1e-3)
    roof["kernel"] = timed_kernel_name(plan, w, args.launch)
    roof["traffic"] = measured_traffic(w.name, roof["kernel"])
    roof["kernel_ms"] = round(k_avg_ms, 5)
    step_roof = roofline_of(w, chunk, ms_per_step * 1e-3)
    roof["step_achieved"] = step_roof["achieved"]
    roof["step_frac"] = step_roof["frac"]

    # parity of the first input set's output against the oracle on the sampled heads
    cpu = None
    check = None
    if not args.no_cpu_baseline:
        step(0)
        torch.cuda.synchronize()
        o_gpu = sets[0]["o"]
        got = (bf16_bits_to_f64(o_gpu.view(torch.int16).cpu().numpy().view(np.uint16))
               if w.dtype == "bf16" else o_gpu.cpu().numpy().astype(np.float64))
        cpu, o_ref, heads = cpu_baseline(w, x, pool, n_workers)
        import oracle
        sel = got[[h // w.H for h in heads], [h % w.H for h in heads]][:, None]
        check = {"rel_err_vs_oracle": float(f"{oracle.rel_err(sel, o_ref):.3e}"), "heads": len(heads)}
    layer.close()
    del sets, q0, k0, v0, a0
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d_k": w.d_k, "d_v": w.d_v, "d_phi": w.d_phi,
            "phi": w.phi, "eta": w.eta_mode if w.eta_mode != "scalar" else w.eta_scalar, "beta": w.beta,
            "causal": w.causal, "loss": w.loss, "chunk": chunk,
            "segments": 1 if (w.loss == "mse" or w.weight_norm) else plan.segments, "dv_split": plan.dv_split,
            "phi_split": plan.phi_split, "launch": args.launch,
            "kernels_per_step": 2 if w.loss == "mse" else (3 if w.weight_norm else plan.n_kernels),
            "weight_norm": w.weight_norm,
            "input_sets": n_sets,
            "head_tokens_per_s": round(w.head_tokens / (ms_per_step * 1e-3), 1),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if check is not None:
        out["check"] = check
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the layer shards over (b, h) with no communication)", file=sys.stderr)
        sys.exit(2)

    names = [args.workload] if args.workload else list(DEFAULT_ORDER)
    forward_run = not (args.calibrate_copy or args.decode or args.backward)
    # the oracle's worker processes are forked before anything touches the GPU
    pool, n_workers = None, 1
    if forward_run and not args.no_cpu_baseline:
        n_workers = oracle_workers()
        pool = make_oracle_pool(n_workers)

    import torch

    import ttt_weight_layers_amd as tla
    from ttt_workloads import WORKLOADS

    if args.calibrate_copy:
        n = args.calibrate_copy * 2 ** 20
        # an elementwise kernel that reads n bytes and writes n bytes
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return

    tla.load_library()
    if args.decode:
        print(json.dumps(run_decode(args, WORKLOADS[names[0] if args.workload else DEFAULT_WORKLOAD])))
        return
    if args.backward:
        print(json.dumps(run_backward(args, WORKLOADS[names[0] if args.workload else DEFAULT_WORKLOAD])))
        return
    try:
        for name in names:
            print(json.dumps(run_forward(args, WORKLOADS[name], pool, n_workers)), flush=True)
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()


if __name__ == "__main__":
    main()
