"""The forward at the size limits, checked on sampled outputs against a closed
form: B * H * T * d just below 2^31 elements (one sequence of 2^24 - 37 tokens,
d = 128: 4 GiB per bf16 tensor), the bound of every plan, and past it (2^24 +
4099 tokens), where only the 32x32-tile plan (bf16, identity map, d = 128) runs.

With q = k = e_0 every score phi(k_s) . phi(q_t) is exactly 1, so column j of
the output is the heavy-ball recurrence of column j of v alone:
    m_t = beta m_{t-1} + eta v_t[j],   s_t = s_{t-1} + m_t,   o_t[j] = s_t
(the update rule and readout of the layer with a unit key and query), which an
IIR filter and a cumulative sum give exactly in fp64 over the whole sequence.
v repeats with period 5 in t: columns below 64 have zero mean (the state stays
small, so rounding is small next to every entry and the check is strict),
columns from 64 on have mean 1 (the state grows with t, so an entry state lost
at a segment boundary shows as an error of the size of the whole prefix)."""
import sys

import numpy as np
import pytest
from scipy.signal import lfilter

import oracle
from _gpu import TOL

pytestmark = pytest.mark.gpu

T_MAX = (1 << 24) - 37            # 128 T < 2^31
T_BIG = (1 << 24) + 4099          # 128 T > 2^31
COLS = [0, 5, 63, 64, 100, 127]


def v_block():
    r = np.arange(5)[:, None]
    j = np.arange(128)[None, :]
    return ((7 * r + j) % 5) - 2 + (j >= 64)


def expected(T, t_rows, eta, beta):
    t = np.arange(T)
    out = np.empty((len(t_rows), len(COLS)))
    for c, j in enumerate(COLS):
        vj = (((7 * t + j) % 5) - 2 + (j >= 64)).astype(np.float64)
        s = np.cumsum(lfilter([eta], [1.0, -beta], vj))
        out[:, c] = s[t_rows]
    return out


@pytest.mark.parametrize("T", [T_MAX, T_BIG])
@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_forward_at_size_limits(T, beta):
    import torch
    import ttt_weight_layers_amd as tla
    eta = 0.1
    print(f"[max size] T={T} ({128 * T / 2 ** 31:.4f} x 2^31 elements) beta={beta}", flush=True)
    sys.stdout.flush()
    qk = torch.zeros((1, 1, T, 128), dtype=torch.bfloat16, device="cuda")
    qk[..., 0] = 1.0
    blk = torch.from_numpy(v_block()).to(torch.bfloat16)
    v = blk.to("cuda").repeat((T + 4) // 5, 1)[:T].reshape(1, 1, T, 128).contiguous()
    lay = tla.TTTLinearAttention(1, 1, T, 128, 128, 128, dtype="bf16")
    plan = lay.plan()
    assert plan.path == 2
    o = lay.forward(qk, qk, v, eta_scalar=eta, beta=beta, eta_mode="scalar", causal=True)
    torch.cuda.synchronize()
    # rows: both ends, both sides of every segment boundary, and a seeded sample
    rng = np.random.default_rng(31)
    rows = [np.arange(256), np.arange(T - 256, T), rng.integers(0, T, 4096)]
    for b in range(plan.seg_len, T, plan.seg_len):
        rows.append(np.arange(b - 70, min(b + 70, T)))
    rows = np.unique(np.concatenate(rows))
    idx = torch.from_numpy(rows).to("cuda")
    got = o[0, 0].index_select(0, idx)[:, COLS].float().cpu().numpy().astype(np.float64)
    want = expected(T, rows, eta, beta)
    zero_mean = [c for c, j in enumerate(COLS) if j < 64]
    drift = [c for c, j in enumerate(COLS) if j >= 64]
    assert oracle.rel_err(got[:, zero_mean], want[:, zero_mean]) <= TOL["bf16"]
    assert oracle.rel_err(got[:, drift], want[:, drift]) <= TOL["bf16"]


def bidir_expected(phase, T, eta, beta, cols, half=32):
    """o_t[j] = s_{T-1}[j] for every t: the recurrence over the whole sequence,
    rows starting at `phase` of the period-5 pattern (columns >= half drift)."""
    r = phase + np.arange(T)
    out = []
    for j in cols:
        vj = (((7 * r + j) % 5) - 2 + (j >= half)).astype(np.float64)
        out.append(np.cumsum(lfilter([eta], [1.0, -beta], vj))[-1])
    return np.array(out)


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_bidirectional_at_maximum_size(beta):
    # 171000 sequences of 196 tokens, d = 64: 2.145e9 elements a tensor (< 2^31)
    import torch
    import ttt_weight_layers_amd as tla
    B, H, T, eta = 171, 1000, 196, 0.1
    print(f"[max size bidir] {B}x{H}x{T} beta={beta}", flush=True)
    sys.stdout.flush()
    n_rows = B * H * T
    qk = torch.zeros((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
    qk[..., 0] = 1.0
    r = np.arange(5)[:, None]
    j = np.arange(64)[None, :]
    blk = torch.from_numpy(((7 * r + j) % 5) - 2 + (j >= 32)).to(torch.bfloat16).to("cuda")
    v = blk.repeat((n_rows + 4) // 5, 1)[:n_rows].reshape(B, H, T, 64).contiguous()
    lay = tla.TTTLinearAttention(B, H, T, 64, 64, 64, dtype="bf16")
    o = lay.forward(qk, qk, v, eta_scalar=eta, beta=beta, eta_mode="scalar", causal=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    seqs = np.unique(np.concatenate([[0, 1, B * H - 2, B * H - 1], rng.integers(0, B * H, 60)]))
    cols = [0, 7, 31, 32, 50, 63]
    flat = o.view(B * H, T, 64)
    got = flat.index_select(0, torch.from_numpy(seqs).to("cuda"))[:, :, cols].float().cpu().numpy()
    # sequence n starts at row 196 n, phase (196 n) mod 5 = n mod 5
    want = np.stack([np.broadcast_to(bidir_expected(int(n % 5), T, eta, beta, cols), (T, len(cols)))
                     for n in seqs])
    assert oracle.rel_err(got[..., :3].astype(np.float64), want[..., :3]) <= TOL["bf16"]
    assert oracle.rel_err(got[..., 3:].astype(np.float64), want[..., 3:]) <= TOL["bf16"]


def test_bidirectional_past_2_31_elements():
    # 16384 sequences of 1025 tokens, d = 128: 2.149e9 elements a tensor (> 2^31), on the
    # 32x32-tile plan
    import torch
    import ttt_weight_layers_amd as tla
    B, H, T, eta, beta = 1024, 16, 1025, 0.1, 0.5
    assert B * H * T * 128 > 1 << 31
    print(f"[past 2^31 bidir] {B}x{H}x{T} beta={beta}", flush=True)
    sys.stdout.flush()
    n_rows = B * H * T
    qk = torch.zeros((B, H, T, 128), dtype=torch.bfloat16, device="cuda")
    qk[..., 0] = 1.0
    blk = torch.from_numpy(v_block()).to(torch.bfloat16).to("cuda")
    v = blk.repeat((n_rows + 4) // 5, 1)[:n_rows].reshape(B, H, T, 128).contiguous()
    lay = tla.TTTLinearAttention(B, H, T, 128, 128, 128, dtype="bf16")
    assert lay.plan().path == 2
    o = lay.forward(qk, qk, v, eta_scalar=eta, beta=beta, eta_mode="scalar", causal=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    seqs = np.unique(np.concatenate([[0, 1, B * H - 2, B * H - 1], rng.integers(0, B * H, 60)]))
    flat = o.view(B * H, T, 128)
    got = flat.index_select(0, torch.from_numpy(seqs).to("cuda"))[:, :, COLS].float().cpu().numpy()
    # sequence n starts at row 1025 n, phase (1025 n) mod 5 = 0
    want = np.stack([np.broadcast_to(bidir_expected(int(1025 * n % 5), T, eta, beta, COLS, half=64),
                                     (T, len(COLS))) for n in seqs])
    assert oracle.rel_err(got[..., :3].astype(np.float64), want[..., :3]) <= TOL["bf16"]
    assert oracle.rel_err(got[..., 3:].astype(np.float64), want[..., 3:]) <= TOL["bf16"]



def test_state_and_noalloc_forwards_past_2_31_elements():
    # the carried-state forward (zero entry state; the state after the last token against
    # the closed form too) and the no-allocation forward (bit for bit the handle's)
    import torch
    import ttt_weight_layers_amd as tla
    T, eta, beta = T_BIG, 0.1, 0.9
    print(f"[past 2^31 state/noalloc] T={T} beta={beta}", flush=True)
    sys.stdout.flush()
    qk = torch.zeros((1, 1, T, 128), dtype=torch.bfloat16, device="cuda")
    qk[..., 0] = 1.0
    blk = torch.from_numpy(v_block()).to(torch.bfloat16)
    v = blk.to("cuda").repeat((T + 4) // 5, 1)[:T].reshape(1, 1, T, 128).contiguous()
    lay = tla.TTTLinearAttention(1, 1, T, 128, 128, 128, dtype="bf16")
    S_T = torch.empty((1, 1, 128, 128), dtype=torch.float32, device="cuda")
    M_T = torch.empty_like(S_T)
    o_fs = lay.forward_state(qk, qk, v, eta_scalar=eta, beta=beta, S_T=S_T, M_T=M_T)
    torch.cuda.synchronize()
    rng = np.random.default_rng(34)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(T - 256, T), rng.integers(0, T, 4096)]))
    idx = torch.from_numpy(rows).to("cuda")
    got = o_fs[0, 0].index_select(0, idx)[:, COLS].float().cpu().numpy().astype(np.float64)
    want = expected(T, rows, eta, beta)
    assert oracle.rel_err(got[:, :3], want[:, :3]) <= TOL["bf16"]
    assert oracle.rel_err(got[:, 3:], want[:, 3:]) <= TOL["bf16"]
    # with k = e_0 the state's column 0 carries the recurrence: S_T[j, 0] = s_{T-1}[j]
    s_last = S_T[0, 0, COLS, 0].cpu().numpy().astype(np.float64)
    assert oracle.rel_err(s_last[None], expected(T, np.array([T - 1]), eta, beta)) <= 1e-3
    del o_fs
    o = lay.forward(qk, qk, v, eta_scalar=eta, beta=beta, eta_mode="scalar", causal=True)
    o_na = torch.empty_like(o)
    desc = tla.make_desc(1, 1, T, 128, 128, 128, dtype="bf16")
    st = tla.ttt_la_forward_noalloc(desc, None, qk.data_ptr(), qk.data_ptr(), v.data_ptr(), None, eta, beta,
                                    tla.mode_bits("scalar", True), o_na.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == tla.TTT_LA_OK, tla.ttt_la_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_na)
