"""GPU parity of ttt_la_backward against the oracle's adjoint recurrence on the
same seeded inputs and output gradient (identity feature map, d_k = d_v)."""
import sys

import numpy as np
import pytest

import oracle
from ttt_workloads import WORKLOADS, make_inputs
from _gpu import TOL, from_device, make_layer, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name, **kw):
    return WORKLOADS[name].with_shape(**kw)


def grad_output(w, seed):
    """A seeded output gradient, rounded to the workload dtype like the inputs."""
    import torch
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((w.B, w.H, w.T, w.d_v))
    t = torch.from_numpy(g).to(torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    g64 = t.to(torch.float64).numpy()
    return t.to("cuda").contiguous(), g64


def run_case(w, segments=0, seed=40, launch=None):
    import torch
    x = make_inputs(w)
    d = to_device(x)
    dO, dO64 = grad_output(w, seed)
    lay = make_layer(w, d, segments=segments, launch=launch or "auto")
    dq, dk, dv, de = lay.backward(d["q"], d["k"], d["v"], dO, eta=d["a"], eta_scalar=w.eta_scalar, beta=w.beta,
                                  eta_mode=w.eta_mode, causal=w.causal)
    torch.cuda.synchronize()
    ref = oracle.backward(x.q64, x.k64, x.v64, dO64, eta_mode=w.eta_mode, eta=x.a32, eta_scalar=w.eta_scalar,
                          beta=w.beta, causal=w.causal)
    got = (from_device(dq, w.dtype), from_device(dk, w.dtype), from_device(dv, w.dtype))
    for name, g, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        err = oracle.rel_err(g, r)
        say(f"  {name} rel err {err:.2e}")
        assert err <= TOL[w.dtype], name
    de_np = de.cpu().numpy().astype(np.float64)
    if w.eta_mode == "scalar":
        assert abs(de_np.sum() - ref[3]) <= TOL[w.dtype] * max(1.0, np.abs(de_np).sum())
    else:
        err = oracle.rel_err(de_np, ref[3])
        say(f"  deta rel err {err:.2e}")
        assert err <= TOL[w.dtype]
    return lay


@pytest.mark.parametrize("eta_mode,beta,segments", [("scalar", 0.9, 4), ("softplus", 0.9, 2),
                                                    ("per_token", 0.0, 1)])
def test_backward_wide_tiles(eta_mode, beta, segments):
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=64 * 4 + 7).with_settings(eta_mode=eta_mode, beta=beta)
    say(f"[backward wide] {eta_mode} beta={beta} segments={segments}")
    lay = run_case(w, segments)
    assert lay.plan().path == 2


def test_backward_two_segments_split_summary():
    # two segments of 20 chunks on two sequences: the forwards inside the backward
    # (two of them reading in reverse time order) summarise segment 0 in two halves
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=64 * 40 - 13).with_settings(eta_mode="softplus", beta=0.9)
    say("[backward split summary]")
    lay = run_case(w, 2)
    assert lay.plan().path == 2 and lay.plan().segments == 2


@pytest.mark.parametrize("launch", ["prefix", "single"])
def test_backward_wide_other_launches(launch):
    # these plans take reversed copies of the inputs instead of reading them in
    # reverse order
    w = small("v4_momentum_4x8x2048_d128", B=1, H=2, T=64 * 5 + 11).with_settings(eta_mode="softplus", beta=0.9)
    say(f"[backward wide launch={launch}]")
    lay = run_case(w, 3, launch=launch)
    assert lay.plan().path == 2


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_backward_bidirectional(beta):
    w = small("v3_softplus_8x16x4096_d128", B=1, H=2, T=64 * 3 + 5).with_settings(causal=False, beta=beta)
    say(f"[backward bidir d=128] beta={beta}")
    run_case(w)


@pytest.mark.parametrize("case", ["f32_causal", "f32_bidir", "bf16_d64_causal", "bf16_d64_bidir"])
def test_backward_other_shapes(case):
    if case.startswith("f32"):
        w = small("v5_f32_1x1x256_d64", B=1, H=2, T=70).with_settings(eta_mode="softplus", beta=0.5,
                                                                       causal=case == "f32_causal")
    else:
        w = small("bidir_vit_256x6x196_d64", B=2, H=2, T=90).with_settings(causal=case == "bf16_d64_causal",
                                                                          beta=0.9, eta_mode="per_token")
    say(f"[backward {case}]")
    run_case(w)


@pytest.mark.parametrize("base,d_k,d_v,causal,eta_mode,beta", [
    ("v3_softplus_8x16x4096_d128", 64, 128, True, "softplus", 0.9),
    ("v3_softplus_8x16x4096_d128", 128, 64, True, "per_token", 0.0),
    ("v3_softplus_8x16x4096_d128", 64, 128, False, "scalar", 0.5),
    ("v3_softplus_8x16x4096_d128", 128, 64, False, "softplus", 0.0),
    ("v5_f32_1x1x256_d64", 64, 128, True, "softplus", 0.9),
    ("v5_f32_1x1x256_d64", 128, 64, False, "scalar", 0.0),
])
def test_backward_unequal_widths(base, d_k, d_v, causal, eta_mode, beta):
    # dq and dk come from forwards with queries and keys of width d_v and values of width d_k
    w = small(base, B=1, H=2, T=150).with_settings(d_k=d_k, d_v=d_v, d_phi=d_k, causal=causal, eta_mode=eta_mode,
                                                    beta=beta, eta_scalar=0.4 if eta_mode == "scalar" else 0.0)
    say(f"[backward widths] {w.dtype} d_k={d_k} d_v={d_v} causal={causal} {eta_mode} beta={beta}")
    run_case(w)


def test_backward_entry_points_for_swiglu():
    import torch
    import ttt_weight_layers_amd as tla
    # d = 128: the workspace query answers for ttt_la_backward_swiglu; ttt_la_backward itself
    # (no place for dW1, dW3) refuses a SwiGLU handle
    w = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=64).with_settings(d_phi=128)
    x = make_inputs(w)
    d = to_device(x)
    lay = make_layer(w, d)
    st, nbytes = tla.ttt_la_backward_workspace(lay.handle, tla.TTT_LA_ETA_SOFTPLUS)
    assert st == tla.TTT_LA_OK and nbytes > 0
    dO = torch.zeros_like(d["v"])
    outs = [torch.empty_like(d["q"]) for _ in range(3)]
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = tla.ttt_la_backward(lay.handle, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["a"].data_ptr(),
                             0.0, 0.9, tla.TTT_LA_ETA_SOFTPLUS, dO.data_ptr(), *(o.data_ptr() for o in outs), None,
                             ws.data_ptr(), nbytes, None)
    assert st == tla.TTT_LA_ERR_UNSUPPORTED
    # d = 64: no SwiGLU backward
    w64 = small("v2_swiglu_4x16x8192_d128_f512", B=1, H=2, T=64).with_settings(d_k=64, d_v=64, d_phi=128)
    x64 = make_inputs(w64)
    d64 = to_device(x64)
    lay64 = make_layer(w64, d64)
    st, _ = tla.ttt_la_backward_workspace(lay64.handle, 0)
    assert st == tla.TTT_LA_ERR_UNSUPPORTED
    with pytest.raises(tla.TTTError) as e:
        lay64.backward(d64["q"], d64["k"], d64["v"], torch.zeros_like(d64["v"]), eta=d64["a"], eta_mode="softplus",
                       beta=0.9)
    assert e.value.status == tla.TTT_LA_ERR_UNSUPPORTED


def _backward_cases(n=40, seed=20261206):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        kind = str(rng.choice(["wide", "wide", "d64", "f32"]))
        c = dict(kind=kind, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                 T=int(rng.integers(1, 500 if kind != "f32" else 150)),
                 eta_mode=str(rng.choice(["scalar", "per_token", "softplus"])),
                 beta=float(rng.choice([0.0, 0.5, 0.9])), causal=bool(rng.random() < 0.75),
                 segments=int(rng.choice([0, 1, 2, 3])) if kind != "f32" else 0, launch="auto")
        if kind == "wide" and c["causal"]:
            c["launch"] = str(rng.choice(["auto", "auto", "separate", "single", "prefix"]))
        cases.append(c)
    return cases


BACKWARD_CASES = _backward_cases()


@pytest.mark.parametrize("c", BACKWARD_CASES, ids=[
    f"{c['kind']}_{c['B']}x{c['H']}x{c['T']}_{c['eta_mode'][:4]}_b{c['beta']}_{'c' if c['causal'] else 'bi'}"
    f"_s{c['segments']}_{c['launch']}" for c in BACKWARD_CASES])
def test_backward_sweep(c):
    # seeded sweep of shapes, modes and plans (the case list is drawn once from a fixed seed)
    base = {"wide": "v4_momentum_4x8x2048_d128", "d64": "bidir_vit_256x6x196_d64",
            "f32": "v5_f32_1x1x256_d64"}[c["kind"]]
    w = small(base, B=c["B"], H=c["H"], T=c["T"]).with_settings(
        eta_mode=c["eta_mode"], beta=c["beta"], causal=c["causal"],
        eta_scalar=0.3 if c["eta_mode"] == "scalar" else WORKLOADS[base].eta_scalar)
    say(f"[backward sweep] {c}")
    run_case(w, c["segments"], launch=c["launch"])
