"""The C ABI on the host: symbols, status codes, argument validation (no GPU).

Every check here runs before the library makes any HIP call, so it works in a
container without a GPU.
"""
import ctypes
import math
import os
import re

import pytest

import ttt_weight_layers_amd as tla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt_la.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tla.LIB_PATH),
                                reason="libttt_la.so not built (run ttt_weight_layers_amd.build)")

# fake, 16-byte aligned, non-overlapping "device" addresses: only compared
Q, K, V, O, ETA, W1, W3 = (0x10000000 * (i + 1) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_la_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = tla.load_library()
    names = declared_functions()
    assert set(names) == set(tla.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert tla.ttt_la_status_string(0) == "ok"
    assert tla.ttt_la_status_string(-1) == "invalid argument"
    assert tla.ttt_la_status_string(-2).startswith("unsupported")
    assert tla.ttt_la_status_string(-3).startswith("HIP")
    assert tla.ttt_la_status_string(-4).startswith("out of")
    assert "static maximum" in tla.ttt_la_status_string(-5)
    assert tla.ttt_la_status_string(12345) == "unknown status"


def desc(**kw):
    base = dict(B=2, H=3, T=100, d_k=128, d_v=128, d_phi=None, dtype="bf16", phi="identity", chunk=0)
    base.update(kw)
    return tla.make_desc(**base)


def test_descriptor_layout_is_the_documented_one():
    # B, H, T, d_k, d_v, d_phi, dtype, phi, chunk (nine int32), then the two weight pointers
    names = [f[0] for f in tla.ttt_la_desc._fields_]
    assert names == ["B", "H", "T", "d_k", "d_v", "d_phi", "dtype", "phi", "chunk", "w1", "w3"]
    assert tla.ttt_la_desc.w1.offset == 40 and tla.ttt_la_desc.w3.offset == 48
    assert ctypes.sizeof(tla.ttt_la_desc) == 56
    text = open(HEADER).read()
    body = text[text.index("typedef struct {\n    int32_t B, H, T;"):text.index("} ttt_la_desc;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b(B, H, T|d_k, d_v, d_phi|dtype|phi|chunk|w1|w3);", body)
    assert fields == ["B, H, T", "d_k, d_v, d_phi", "dtype", "phi", "chunk", "w1", "w3"]


def check(d=None, q=Q, k=K, v=V, eta=None, eta_scalar=0.5, beta=0.0, mode=0, o=O):
    return tla.ttt_la_check(d or desc(), q, k, v, eta, eta_scalar, beta, mode, o)


def test_valid_arguments_pass():
    assert check() == tla.TTT_LA_OK
    assert check(eta=ETA, mode=tla.TTT_LA_ETA_SOFTPLUS, beta=0.9) == tla.TTT_LA_OK
    assert check(eta=ETA, mode=tla.TTT_LA_ETA_PER_TOKEN | tla.TTT_LA_BIDIRECTIONAL) == tla.TTT_LA_OK
    assert check(d=desc(dtype="f32", d_k=64, d_v=64)) == tla.TTT_LA_OK


def test_query_may_alias_key():
    # thelatestinai.com Table 1 'Replace Q with K'
    assert check(q=K) == tla.TTT_LA_OK


@pytest.mark.parametrize("field,value", [("B", 0), ("H", 0), ("T", 0), ("T", -5), ("d_k", 0),
                                         ("d_v", -1), ("dtype", 7), ("phi", 3), ("chunk", -1)])
def test_bad_descriptor_fields(field, value):
    d = desc()
    setattr(d, field, value)
    assert check(d=d, q=None) == tla.TTT_LA_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [("segments", -2), ("value_split", 3), ("value_split", -1),
                                         ("launch", 4), ("launch", -1)])
def test_bad_plan_hints(field, value):
    h = tla.make_hints()
    setattr(h, field, value)
    assert tla.ttt_la_check_hints(h) == tla.TTT_LA_ERR_INVALID_ARG
    # create rejects them before any HIP call
    st, handle = tla.ttt_la_create_hinted(desc(), h)
    assert st == tla.TTT_LA_ERR_INVALID_ARG and not handle.value


def test_good_plan_hints():
    assert tla.ttt_la_check_hints(None) == tla.TTT_LA_OK
    assert tla.ttt_la_check_hints(tla.make_hints(segments=4, value_split=2, launch="prefix")) == tla.TTT_LA_OK


@pytest.mark.parametrize("kw", [dict(d_k=96, d_v=128), dict(d_k=128, d_v=32), dict(d_k=256, d_v=128),
                                dict(chunk=32), dict(chunk=100)])
def test_unsupported_shapes(kw):
    assert check(d=desc(**kw), q=None) == tla.TTT_LA_ERR_UNSUPPORTED


def test_identity_requires_dphi_equal_dk_and_no_weights():
    assert check(d=desc(d_phi=64), q=None) == tla.TTT_LA_ERR_INVALID_ARG
    d = desc()
    d.w1 = W1
    assert check(d=d, q=None) == tla.TTT_LA_ERR_INVALID_ARG


def test_swiglu_descriptor():
    assert check(d=desc(phi="swiglu", d_phi=512, w1=W1, w3=W3), q=None) == tla.TTT_LA_OK
    assert check(d=desc(phi="swiglu", d_phi=512, w1=W1, w3=None), q=None) == tla.TTT_LA_ERR_INVALID_ARG
    assert check(d=desc(phi="swiglu", d_phi=200, w1=W1, w3=W3), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(phi="swiglu", d_phi=1024, w1=W1, w3=W3), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(phi="swiglu", d_phi=512, w1=W1 + 8, w3=W3), q=None) == tla.TTT_LA_ERR_INVALID_ARG


def test_size_limit():
    # 2^32 tokens: past the token-count limit on every plan
    assert check(d=desc(B=1024, H=64, T=65536), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    # past 2^31 elements a tensor: the 32x32-tile plan (bf16, identity, d = 128) only
    big = dict(B=1, H=16, T=(1 << 20) + 96)
    assert check(d=desc(**big), q=None) == tla.TTT_LA_OK
    assert check(d=desc(**big, chunk=128), q=None) == tla.TTT_LA_OK
    assert check(d=desc(B=1, H=16, T=(1 << 21) + 96, d_k=64, d_v=64), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(**big, d_v=64), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(**big, dtype="f32"), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(**big, phi="swiglu", d_phi=128, w1=W1, w3=W3), q=None) == tla.TTT_LA_ERR_UNSUPPORTED
    # and there only the forwards with the dot-product loss (pointers far apart: no overlap)
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40)
    assert check(d=desc(**big), **far) == tla.TTT_LA_OK
    assert check(d=desc(**big), **far, mode=tla.TTT_LA_LOSS_MSE) == tla.TTT_LA_ERR_UNSUPPORTED
    assert tla.ttt_la_check_backward(desc(**big), None, 1 << 40, 2 << 40, 3 << 40, None, 0.5, 0.9, 0, 5 << 40,
                                     6 << 40, 7 << 40, 8 << 40, None, 9 << 40, 1 << 44) == tla.TTT_LA_ERR_UNSUPPORTED
    # just below 2^31 elements every plan is open
    assert check(d=desc(B=1, H=16, T=(1 << 21) - 1, d_k=64, d_v=64), q=None) == tla.TTT_LA_OK


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_null_and_misaligned_pointers(which):
    if which != "q":             # q == NULL asks ttt_la_check for the descriptor alone
        kw = {which: None}
        assert check(**kw) == tla.TTT_LA_ERR_INVALID_ARG
    kw = {which: {"q": Q, "k": K, "v": V, "o": O}[which] + 2}
    assert check(**kw) == tla.TTT_LA_ERR_INVALID_ARG


def test_mode_bits():
    assert check(mode=1 << 5) == tla.TTT_LA_ERR_INVALID_ARG
    both = tla.TTT_LA_ETA_PER_TOKEN | tla.TTT_LA_ETA_SOFTPLUS
    assert check(eta=ETA, mode=both) == tla.TTT_LA_ERR_INVALID_ARG
    # a per-token mode needs a pointer; the scalar mode forbids one
    assert check(eta=None, mode=tla.TTT_LA_ETA_SOFTPLUS) == tla.TTT_LA_ERR_INVALID_ARG
    assert check(eta=ETA, mode=tla.TTT_LA_ETA_SCALAR) == tla.TTT_LA_ERR_INVALID_ARG
    assert check(eta=ETA + 2, mode=tla.TTT_LA_ETA_PER_TOKEN) == tla.TTT_LA_ERR_INVALID_ARG


@pytest.mark.parametrize("beta", [-0.1, 1.0, 1.5, math.nan, math.inf])
def test_beta_range(beta):
    assert check(beta=beta) == tla.TTT_LA_ERR_INVALID_ARG


@pytest.mark.parametrize("eta", [math.nan, math.inf, -math.inf])
def test_non_finite_eta_scalar(eta):
    assert check(eta_scalar=eta) == tla.TTT_LA_ERR_INVALID_ARG


def test_negative_eta_is_gradient_ascent_and_allowed():
    assert check(eta_scalar=-0.5) == tla.TTT_LA_OK


def test_output_must_not_overlap_inputs():
    n = 2 * 3 * 100 * 128 * 2                       # bytes of one bf16 tensor
    assert check(o=Q) == tla.TTT_LA_ERR_INVALID_ARG
    assert check(o=K + n - 16) == tla.TTT_LA_ERR_INVALID_ARG
    assert check(o=V - n + 16) == tla.TTT_LA_ERR_INVALID_ARG
    assert check(o=V + n) == tla.TTT_LA_OK               # adjacent is fine
    assert check(o=ETA, eta=ETA, mode=tla.TTT_LA_ETA_PER_TOKEN) == tla.TTT_LA_ERR_INVALID_ARG


def test_create_rejects_bad_descriptor_before_device_work():
    d = desc(T=0)
    st, h = tla.ttt_la_create(d)
    assert st == tla.TTT_LA_ERR_INVALID_ARG and not h.value
    st, h = tla.ttt_la_create(desc(d_k=96))
    assert st == tla.TTT_LA_ERR_UNSUPPORTED and not h.value


def test_null_handle_calls():
    tla.ttt_la_destroy(None)                      # NULL-safe
    lib = tla.load_library()
    assert lib.ttt_la_forward(None, Q, K, V, None, 1.0, 0.0, 0, O, None) == tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_get_plan(None, None) == tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_enable_kernel_timing(None, 4) == tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_enable_kernel_timing_every(None, 4, 2) == tla.TTT_LA_ERR_INVALID_ARG
    n = ctypes.c_int32(0)
    assert lib.ttt_la_kernel_times(None, None, 0, ctypes.byref(n)) == tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_create(None, None) == tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_wait_status(None, ctypes.byref(n)) == tla.TTT_LA_ERR_INVALID_ARG


def test_binding_refuses_missing_library(tmp_path):
    from ttt_weight_layers_amd import _binding
    saved = _binding._lib
    _binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            _binding.load_library(str(tmp_path / "nope.so"))
    finally:
        _binding._lib = saved


# ----------------------------------------------------------------------------
# state-carrying calls: ttt_la_forward_state (call 0) and ttt_la_step (call 1)
# ----------------------------------------------------------------------------

S0, M0, ST, MT = (0x10000000 * (i + 8) for i in range(4))
SB = 2 * 3 * 128 * 128 * 4                          # bytes of one fp32 state [B, H, d_v, d_phi]


def check_fs(d=None, q=Q, k=K, v=V, eta=None, eta_scalar=0.5, beta=0.9, mode=0, s0=S0, m0=M0, o=O, st=ST, mt=MT):
    return tla.ttt_la_check_state(d or desc(), 0, q, k, v, eta, eta_scalar, beta, mode, s0, m0, o, st, mt)


def check_step(d=None, q=Q, k=K, v=V, eta=None, eta_scalar=0.5, beta=0.9, mode=0, s=S0, m=M0, o=O):
    return tla.ttt_la_check_state(d or desc(), 1, q, k, v, eta, eta_scalar, beta, mode, s, m, o, s, m)


def test_forward_state_valid_arguments():
    assert check_fs() == tla.TTT_LA_OK
    assert check_fs(s0=None, m0=None) == tla.TTT_LA_OK               # zero entry state
    assert check_fs(st=None, mt=None) == tla.TTT_LA_OK               # no final state
    assert check_fs(st=S0, mt=M0) == tla.TTT_LA_OK                   # in place
    assert check_fs(eta=ETA, mode=tla.TTT_LA_ETA_SOFTPLUS) == tla.TTT_LA_OK
    assert check_fs(d=desc(dtype="f32", d_k=64, d_v=64)) == tla.TTT_LA_OK


def test_forward_state_rejections():
    bad = tla.TTT_LA_ERR_INVALID_ARG
    assert check_fs(mode=tla.TTT_LA_BIDIRECTIONAL) == bad           # causal only
    assert check_fs(s0=S0 + 8) == bad                                # misaligned
    assert check_fs(mt=MT + 4) == bad
    assert check_fs(st=MT) == bad                                    # S_T and M_T overlap
    assert check_fs(st=S0 + 16) == bad                               # partial overlap with S0
    assert check_fs(st=M0) == bad                                    # S_T over M0
    assert check_fs(mt=S0) == bad
    assert check_fs(s0=Q) == bad                                     # state over an input
    assert check_fs(st=O + 16) == bad                                # state over the output
    assert check_fs(st=ST + SB, mt=MT) == tla.TTT_LA_OK              # disjoint elsewhere
    assert check_fs(beta=1.0) == bad
    assert check_fs(q=None) == bad


def test_step_arguments():
    bad = tla.TTT_LA_ERR_INVALID_ARG
    assert check_step() == tla.TTT_LA_OK
    assert check_step(eta=ETA, mode=tla.TTT_LA_ETA_PER_TOKEN) == tla.TTT_LA_OK
    assert check_step(d=desc(phi="swiglu", d_phi=512, w1=W1, w3=W3)) == tla.TTT_LA_OK
    assert check_step(s=None) == bad
    assert check_step(m=None) == bad
    assert check_step(s=S0 + 4) == bad
    assert check_step(m=S0 + 256) == bad                             # S and M overlap
    assert check_step(mode=tla.TTT_LA_BIDIRECTIONAL) == bad
    assert check_step(mode=tla.TTT_LA_ETA_SOFTPLUS) == bad           # rate pointer missing
    assert check_step(eta=ETA) == bad                                # pointer without a mode bit
    assert check_step(o=Q) == bad
    assert check_step(s=O) == bad
    # step and forward_state check different extents: one token per (b, h)
    assert check_step(o=V + 2 * 3 * 128 * 2) == tla.TTT_LA_OK
    # call 1 requires the state outputs to be the inputs; unknown call numbers fail
    assert tla.ttt_la_check_state(desc(), 1, Q, K, V, None, 0.5, 0.9, 0, S0, M0, O, ST, MT) == bad
    assert tla.ttt_la_check_state(desc(), 2, Q, K, V, None, 0.5, 0.9, 0, S0, M0, O, S0, M0) == bad


def test_state_calls_with_null_handle():
    lib = tla.load_library()
    assert lib.ttt_la_forward_state(None, Q, K, V, None, 1.0, 0.0, 0, S0, M0, O, ST, MT, None) == \
        tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_step(None, Q, K, V, None, 1.0, 0.0, 0, S0, M0, O, None) == tla.TTT_LA_ERR_INVALID_ARG


# ----------------------------------------------------------------------------
# ttt_la_backward
# ----------------------------------------------------------------------------

DO, DQ, DK, DV, DE, WS = (0x10000000 * (i + 12) for i in range(6))
TB = 2 * 3 * 100 * 128 * 2                         # one bf16 [B, H, T, d] tensor


def check_bw(d=None, q=Q, k=K, v=V, eta=None, beta=0.9, mode=0, dO=DO, dq=DQ, dk=DK, dv=DV, de=DE, ws=WS,
             wsb=6 * TB, hints=None):
    return tla.ttt_la_check_backward(d or desc(), hints, q, k, v, eta, 0.5, beta, mode, dO, dq, dk, dv, de, ws,
                                     wsb)


def test_backward_arguments():
    bad = tla.TTT_LA_ERR_INVALID_ARG
    assert check_bw() == tla.TTT_LA_OK
    assert check_bw(de=None) == tla.TTT_LA_OK
    assert check_bw(mode=tla.TTT_LA_BIDIRECTIONAL, wsb=2 * TB) == tla.TTT_LA_OK   # the two outputs
    # bf16 d = 128, one segment: the two outputs and no summaries
    assert check_bw(wsb=2 * TB) == tla.TTT_LA_OK
    assert check_bw(wsb=2 * TB - 16) == bad                                      # too small
    # two segments of 8 chunks: plus a summary area of 6 sequences x 2 slots x 128 KiB
    # for each reversed forward
    d2, h2 = desc(T=1024), tla.make_hints(segments=2)
    tb2 = 2 * 3 * 1024 * 128 * 2
    need2 = 2 * tb2 + 2 * (6 * 2 * 128 * 128 * 2 * 4)
    assert check_bw(d=d2, hints=h2, wsb=need2) == tla.TTT_LA_OK
    assert check_bw(d=d2, hints=h2, wsb=need2 - 16) == bad
    # the single-launch plan and the 16x16-tile shapes take reversed copies of
    # q, k, v, dO: six tensors
    single = tla.make_hints(launch="single")
    assert check_bw(hints=single, wsb=6 * TB - 16) == bad
    assert check_bw(hints=single, wsb=6 * TB) == tla.TTT_LA_OK
    tb64 = 2 * 3 * 100 * 64 * 2
    assert check_bw(d=desc(d_k=64, d_v=64), wsb=6 * tb64 - 16) == bad
    assert check_bw(d=desc(d_k=64, d_v=64), wsb=6 * tb64) == tla.TTT_LA_OK
    assert check_bw(ws=None) == bad
    assert check_bw(ws=WS + 8) == bad
    assert check_bw(dO=None) == bad
    assert check_bw(dk=DQ) == bad                                                # outputs overlap
    assert check_bw(dv=Q) == bad                                                 # output over an input
    assert check_bw(dq=DO) == bad
    assert check_bw(ws=DO) == bad                                                # workspace over dO
    assert check_bw(de=DE + 2) == bad
    assert check_bw(eta=ETA, mode=tla.TTT_LA_ETA_SOFTPLUS, de=ETA) == bad
    # d_k != d_v: reversed q, k (d_k wide) and v, dO (d_v wide), the two rate-1 outputs, then the
    # swapped plan's summary area
    kb, vb = 2 * 3 * 100 * 128 * 2, 2 * 3 * 100 * 64 * 2
    assert check_bw(d=desc(d_v=64), wsb=3 * (kb + vb) - 16) == bad
    assert check_bw(d=desc(d_v=64), wsb=1 << 30) == tla.TTT_LA_OK
    assert check_bw(d=desc(phi="swiglu", d_phi=256, w1=W1, w3=W3)) == tla.TTT_LA_ERR_UNSUPPORTED


def test_backward_null_handle():
    lib = tla.load_library()
    n = ctypes.c_size_t(0)
    assert lib.ttt_la_backward_workspace(None, 0, ctypes.byref(n)) == tla.TTT_LA_ERR_INVALID_ARG
    assert lib.ttt_la_backward(None, Q, K, V, None, 1.0, 0.0, 0, DO, DQ, DK, DV, None, WS, 0, None) == \
        tla.TTT_LA_ERR_INVALID_ARG


def test_mse_loss_mode():
    # the delta rule: bf16 identity map, d_k = d_v in {64, 128}, causal, beta = 0
    mse = tla.TTT_LA_LOSS_MSE
    assert check(mode=mse) == tla.TTT_LA_OK
    assert check(d=desc(d_k=64, d_v=64), eta=ETA, mode=mse | tla.TTT_LA_ETA_SOFTPLUS) == tla.TTT_LA_OK
    assert check(mode=mse, beta=0.5) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(mode=mse | tla.TTT_LA_BIDIRECTIONAL) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(dtype="f32", d_k=64, d_v=64), mode=mse) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(d_k=64, d_v=128), mode=mse) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check(d=desc(phi="swiglu", d_phi=512, w1=W1, w3=W3), mode=mse) == tla.TTT_LA_ERR_UNSUPPORTED
    # carried state: S alone (the delta rule runs without momentum)
    assert check_fs(mode=mse, beta=0.0, m0=None, mt=None) == tla.TTT_LA_OK
    assert check_fs(mode=mse, beta=0.0, m0=None, mt=None, st=S0) == tla.TTT_LA_OK      # in place
    assert check_fs(mode=mse, beta=0.0, s0=None, m0=None, mt=None) == tla.TTT_LA_OK    # zero entry state
    assert check_fs(mode=mse, beta=0.0) == tla.TTT_LA_ERR_INVALID_ARG                  # M0 and M_T given
    assert check_fs(mode=mse, beta=0.0, m0=None) == tla.TTT_LA_ERR_INVALID_ARG
    assert check_fs(mode=mse, beta=0.0, mt=None) == tla.TTT_LA_ERR_INVALID_ARG
    assert check_fs(mode=mse, beta=0.5, m0=None, mt=None) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check_fs(d=desc(dtype="f32", d_k=64, d_v=64), mode=mse, beta=0.0, m0=None, mt=None) == \
        tla.TTT_LA_ERR_UNSUPPORTED
    # the step: momentum allowed, every dtype and feature map while a row of S fits the registers
    assert check_step(mode=mse, beta=0.9) == tla.TTT_LA_OK
    assert check_step(d=desc(dtype="f32", d_k=64, d_v=64), mode=mse, beta=0.0) == tla.TTT_LA_OK
    assert check_step(d=desc(phi="swiglu", d_phi=512, w1=W1, w3=W3), mode=mse | tla.TTT_LA_ETA_SOFTPLUS,
                      eta=ETA, beta=0.9) == tla.TTT_LA_OK
    assert check_step(mode=mse | tla.TTT_LA_WEIGHT_NORM) == tla.TTT_LA_ERR_INVALID_ARG
    assert tla.mode_bits("softplus", True, "mse") == tla.TTT_LA_ETA_SOFTPLUS | mse


def test_weight_norm_mode():
    # Variant 1's weight-normalised recurrence: ttt_la_forward_state with an entry state
    wn = tla.TTT_LA_WEIGHT_NORM
    assert check_fs(mode=wn) == tla.TTT_LA_OK
    assert check_fs(mode=wn, m0=None, st=None, mt=None) == tla.TTT_LA_OK
    assert check_fs(eta=ETA, mode=wn | tla.TTT_LA_ETA_SOFTPLUS) == tla.TTT_LA_OK
    assert check_fs(d=desc(phi="swiglu", d_phi=512, w1=W1, w3=W3), mode=wn) == tla.TTT_LA_OK
    assert check_fs(d=desc(dtype="f32", d_k=64, d_v=64), mode=wn) == tla.TTT_LA_OK
    bad = tla.TTT_LA_ERR_INVALID_ARG
    assert check_fs(mode=wn, s0=None) == bad                          # the target norms come from S0
    assert check_fs(mode=wn | tla.TTT_LA_LOSS_MSE, beta=0.0) == bad
    assert check(mode=wn) == bad                                     # plain forward: no entry state
    # widths the kernel does not take
    assert check_fs(d=desc(d_v=120), mode=wn) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check_fs(d=desc(d_k=96, d_v=96), mode=wn) == tla.TTT_LA_ERR_UNSUPPORTED
    assert check_fs(d=desc(d_k=64, phi="swiglu", d_phi=256, w1=W1, w3=W3), mode=wn) == tla.TTT_LA_ERR_UNSUPPORTED
    # the weight-normalised step (same widths)
    assert check_step(mode=wn) == tla.TTT_LA_OK
    assert check_step(d=desc(phi="swiglu", d_phi=384, w1=W1, w3=W3), mode=wn) == tla.TTT_LA_ERR_UNSUPPORTED
    assert tla.mode_bits("softplus", True, weight_norm=True) == tla.TTT_LA_ETA_SOFTPLUS | wn
    assert wn == 1 << 4
