"""The binding's tensor checks (no GPU): every call's tensors are checked against
the handle's descriptor before a raw pointer reaches the C ABI, which cannot see
sizes.  CPU tensors of the right shape and dtype reach the last check (the
device) and are rejected there."""
import pytest
import torch

import ttt_weight_layers_amd as tla
from ttt_weight_layers_amd._binding import check_tensors

B, H, T, D = 2, 3, 40, 128


def desc(dtype="bf16", phi="identity", d_phi=None):
    return tla.make_desc(B, H, T, D, D, d_phi, dtype=dtype, phi=phi)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def fwd(**kw):
    base = dict(q=t(B, H, T, D), k=t(B, H, T, D), v=t(B, H, T, D), eta=None, out=None)
    base.update(kw)
    mode = kw.pop("mode", 0) if "mode" in kw else 0
    base.pop("mode", None)
    return base, mode


def expect(msg, call, mode, d=None, **tensors):
    with pytest.raises(ValueError, match=msg):
        check_tensors(d or desc(), call, mode, **tensors)


def test_well_formed_cpu_tensors_stop_at_the_device_check():
    tens, mode = fwd()
    expect("device tensor", "forward", mode, **tens)


@pytest.mark.parametrize("name,bad", [("q", t(B, H, T - 1, D)), ("k", t(B, H, T, 64)), ("v", t(B, H + 1, T, D)),
                                      ("out", t(B, H, T, D, 1))])
def test_wrong_shapes(name, bad):
    tens, mode = fwd(**{name: bad})
    expect("shape", "forward", mode, **tens)


def test_wrong_dtype_for_the_handle():
    tens, mode = fwd(v=t(B, H, T, D, dtype=torch.float32))
    expect("dtype", "forward", mode, **tens)
    tens, mode = fwd(q=t(B, H, T, D, dtype=torch.bfloat16))
    expect("dtype", "forward", mode, d=desc(dtype="f32"), **tens)


def test_rates():
    soft = tla.TTT_LA_ETA_SOFTPLUS
    tens, _ = fwd()
    expect("needs eta", "forward", soft, **tens)
    tens, _ = fwd(eta=t(B, H, T, dtype=torch.float32))
    expect("must be None", "forward", 0, **tens)
    tens, _ = fwd(eta=t(B, H, T, dtype=torch.bfloat16))
    expect("dtype", "forward", soft, **tens)
    tens, _ = fwd(eta=t(B, H, T + 1, dtype=torch.float32))
    expect("shape", "forward", soft, **tens)
    tens, _ = fwd(eta=torch.zeros((B, T, H), dtype=torch.float32).transpose(1, 2))
    expect("contiguous", "forward", soft, **tens)


def test_state_tensors():
    f32 = torch.float32
    d = desc(phi="swiglu", d_phi=512)
    base = dict(q=t(B, H, T, D), k=t(B, H, T, D), v=t(B, H, T, D))
    expect("S0 has shape", "forward_state", 0, d=d, S0=t(B, H, D, D, dtype=f32), **base)
    expect("M_T has dtype", "forward_state", 0, d=d, M_T=t(B, H, D, 512), **base)
    expect("device tensor", "forward_state", 0, d=d, S0=t(B, H, D, 512, dtype=f32), **base)


def test_step_shapes():
    f32 = torch.float32
    one = dict(q=t(B, H, 1, D), k=t(B, H, 1, D), v=t(B, H, 1, D))
    S, M = t(B, H, D, D, dtype=f32), t(B, H, D, D, dtype=f32)
    expect("device tensor", "step", 0, S=S, M=M, **one)
    expect("q has shape", "step", 0, S=S, M=M, **dict(one, q=t(B, H, 2, D)))
    soft = tla.TTT_LA_ETA_SOFTPLUS
    expect("device tensor", "step", soft, S=S, M=M, eta=t(B, H, dtype=f32), **one)
    expect("device tensor", "step", soft, S=S, M=M, eta=t(B, H, 1, dtype=f32), **one)
    expect("eta has shape", "step", soft, S=S, M=M, eta=t(B, H, T, dtype=f32), **one)


def test_backward_gradient_of_the_output():
    tens, _ = fwd()
    tens.pop("out")
    expect("dO has shape", "backward", 0, dO=t(B, H, T, 64), **tens)
