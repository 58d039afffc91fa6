"""ctypes binding of libttt_la.so (argument marshalling only).

The function names match the C ABI in include/ttt_la.h.  Every step of the
forward runs in the library's HIP kernels; this module only converts Python
and torch objects to pointers, sizes and status codes.  There is no fallback:
if the library is missing or fails to load, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# TTT_LA_LIBRARY names another build of the same sources (the host-sanitized
# one of build_sanitized.py, for the host-only tests)
LIB_PATH = os.environ.get("TTT_LA_LIBRARY") or os.path.join(_PKG, "libttt_la.so")

# status codes
TTT_LA_OK = 0
TTT_LA_ERR_INVALID_ARG = -1
TTT_LA_ERR_UNSUPPORTED = -2
TTT_LA_ERR_HIP = -3
TTT_LA_ERR_OOM = -4
TTT_LA_ERR_TOO_LARGE = -5
TTT_LA_NOALLOC_SCRATCH_BYTES = 64 << 20

TTT_LA_F32 = 0
TTT_LA_BF16 = 1
TTT_LA_PHI_IDENTITY = 0
TTT_LA_PHI_SWIGLU = 1

TTT_LA_LAUNCH_AUTO = 0
TTT_LA_LAUNCH_SEPARATE = 1
TTT_LA_LAUNCH_SINGLE = 2
TTT_LA_LAUNCH_PREFIX = 3
_LAUNCH = {"auto": TTT_LA_LAUNCH_AUTO, "separate": TTT_LA_LAUNCH_SEPARATE, "single": TTT_LA_LAUNCH_SINGLE,
           "prefix": TTT_LA_LAUNCH_PREFIX}

TTT_LA_CAUSAL = 0
TTT_LA_BIDIRECTIONAL = 1 << 0
TTT_LA_ETA_SCALAR = 0
TTT_LA_ETA_PER_TOKEN = 1 << 1
TTT_LA_ETA_SOFTPLUS = 1 << 2
TTT_LA_LOSS_MSE = 1 << 3
TTT_LA_WEIGHT_NORM = 1 << 4


class ttt_la_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("d_phi", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("phi", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p),
    ]


class ttt_la_hints(ctypes.Structure):
    _fields_ = [("segments", ctypes.c_int32), ("value_split", ctypes.c_int32), ("launch", ctypes.c_int32)]


class ttt_la_plan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32), ("chunk", ctypes.c_int32), ("segments", ctypes.c_int32),
        ("seg_len", ctypes.c_int32), ("dv_split", ctypes.c_int32), ("phi_split", ctypes.c_int32),
        ("grid_main", ctypes.c_int32), ("n_kernels", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


EXPORTS = ("ttt_la_create", "ttt_la_create_hinted", "ttt_la_check_hints", "ttt_la_forward", "ttt_la_forward_state", "ttt_la_step", "ttt_la_backward",
           "ttt_la_backward_workspace", "ttt_la_destroy",
           "ttt_la_status_string", "ttt_la_check", "ttt_la_check_state", "ttt_la_check_backward", "ttt_la_get_plan",
           "ttt_la_wait_status", "ttt_la_enable_kernel_timing", "ttt_la_kernel_times",
           "ttt_la_enable_kernel_timing_every", "ttt_la_forward_noalloc", "ttt_la_backward_swiglu")

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libttt_la.so once and declares the signatures.  Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libttt_la.so is not built ({path}); run "
                           "`python -m ttt_weight_layers_amd.build` (the HIP library is required, "
                           "there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, u32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    lib.ttt_la_create.argtypes = [ctypes.POINTER(ttt_la_desc), ctypes.POINTER(vp)]
    lib.ttt_la_create.restype = ctypes.c_int
    lib.ttt_la_create_hinted.argtypes = [ctypes.POINTER(ttt_la_desc), ctypes.POINTER(ttt_la_hints),
                                         ctypes.POINTER(vp)]
    lib.ttt_la_create_hinted.restype = ctypes.c_int
    lib.ttt_la_check_hints.argtypes = [ctypes.POINTER(ttt_la_hints)]
    lib.ttt_la_check_hints.restype = ctypes.c_int
    lib.ttt_la_forward.argtypes = [vp, vp, vp, vp, vp, f32, f32, u32, vp, vp]
    lib.ttt_la_forward.restype = ctypes.c_int
    lib.ttt_la_forward_noalloc.argtypes = [ctypes.POINTER(ttt_la_desc), ctypes.POINTER(ttt_la_hints), vp, vp, vp,
                                           vp, f32, f32, u32, vp, vp]
    lib.ttt_la_forward_noalloc.restype = ctypes.c_int
    lib.ttt_la_forward_state.argtypes = [vp, vp, vp, vp, vp, f32, f32, u32, vp, vp, vp, vp, vp, vp]
    lib.ttt_la_forward_state.restype = ctypes.c_int
    lib.ttt_la_step.argtypes = [vp, vp, vp, vp, vp, f32, f32, u32, vp, vp, vp, vp]
    lib.ttt_la_step.restype = ctypes.c_int
    lib.ttt_la_check_state.argtypes = [ctypes.POINTER(ttt_la_desc), i32, vp, vp, vp, vp, f32, f32, u32, vp, vp,
                                       vp, vp, vp]
    lib.ttt_la_check_state.restype = ctypes.c_int
    lib.ttt_la_backward.argtypes = [vp, vp, vp, vp, vp, f32, f32, u32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ttt_la_backward.restype = ctypes.c_int
    lib.ttt_la_backward_swiglu.argtypes = [vp, vp, vp, vp, vp, f32, f32, u32, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_size_t, vp]
    lib.ttt_la_backward_swiglu.restype = ctypes.c_int
    lib.ttt_la_check_backward.argtypes = [ctypes.POINTER(ttt_la_desc), ctypes.POINTER(ttt_la_hints), vp, vp, vp, vp, f32, f32, u32, vp, vp, vp, vp,
                                          vp, vp, ctypes.c_size_t]
    lib.ttt_la_check_backward.restype = ctypes.c_int
    lib.ttt_la_backward_workspace.argtypes = [vp, u32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_la_backward_workspace.restype = ctypes.c_int
    lib.ttt_la_destroy.argtypes = [vp]
    lib.ttt_la_destroy.restype = None
    lib.ttt_la_status_string.argtypes = [ctypes.c_int]
    lib.ttt_la_status_string.restype = ctypes.c_char_p
    lib.ttt_la_check.argtypes = [ctypes.POINTER(ttt_la_desc), vp, vp, vp, vp, f32, f32, u32, vp]
    lib.ttt_la_check.restype = ctypes.c_int
    lib.ttt_la_get_plan.argtypes = [vp, ctypes.POINTER(ttt_la_plan)]
    lib.ttt_la_get_plan.restype = ctypes.c_int
    lib.ttt_la_wait_status.argtypes = [vp, ctypes.POINTER(i32)]
    lib.ttt_la_wait_status.restype = ctypes.c_int
    lib.ttt_la_enable_kernel_timing.argtypes = [vp, i32]
    lib.ttt_la_enable_kernel_timing.restype = ctypes.c_int
    lib.ttt_la_kernel_times.argtypes = [vp, ctypes.POINTER(f32), i32, ctypes.POINTER(i32)]
    lib.ttt_la_kernel_times.restype = ctypes.c_int
    lib.ttt_la_enable_kernel_timing_every.argtypes = [vp, i32, i32]
    lib.ttt_la_enable_kernel_timing_every.restype = ctypes.c_int
    _lib = lib
    return lib


class TTTError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ttt_la_status_string(status)} ({status})")


def ttt_la_status_string(status: int) -> str:
    return load_library().ttt_la_status_string(int(status)).decode()


def ttt_la_create(desc: ttt_la_desc):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = load_library().ttt_la_create(ctypes.byref(desc), ctypes.byref(h))
    return st, h


def ttt_la_create_hinted(desc: ttt_la_desc, hints: Optional[ttt_la_hints]):
    """Returns (status, handle); hints None = all automatic."""
    h = ctypes.c_void_p()
    st = load_library().ttt_la_create_hinted(ctypes.byref(desc), None if hints is None else ctypes.byref(hints),
                                             ctypes.byref(h))
    return st, h


def ttt_la_check_hints(hints: Optional[ttt_la_hints]) -> int:
    return load_library().ttt_la_check_hints(None if hints is None else ctypes.byref(hints))


def ttt_la_forward_noalloc(desc: ttt_la_desc, hints: Optional[ttt_la_hints], q: int, k: int, v: int,
                           eta: Optional[int], eta_scalar: float, beta: float, mode: int, o: int,
                           stream: Optional[int]) -> int:
    """The handle-less forward whose workspace is the library's static device scratch."""
    return load_library().ttt_la_forward_noalloc(ctypes.byref(desc), None if hints is None else ctypes.byref(hints),
                                                 q, k, v, eta, float(eta_scalar), float(beta), int(mode), o, stream)


def ttt_la_forward(h, q: int, k: int, v: int, eta: Optional[int], eta_scalar: float, beta: float,
                   mode: int, o: int, stream: Optional[int]) -> int:
    return load_library().ttt_la_forward(h, q, k, v, eta, float(eta_scalar), float(beta),
                                         int(mode), o, stream)


def ttt_la_forward_state(h, q: int, k: int, v: int, eta: Optional[int], eta_scalar: float, beta: float,
                         mode: int, S0: Optional[int], M0: Optional[int], o: int, S_T: Optional[int],
                         M_T: Optional[int], stream: Optional[int]) -> int:
    return load_library().ttt_la_forward_state(h, q, k, v, eta, float(eta_scalar), float(beta), int(mode),
                                               S0, M0, o, S_T, M_T, stream)


def ttt_la_step(h, q: int, k: int, v: int, eta: Optional[int], eta_scalar: float, beta: float, mode: int,
                S: int, M: int, o: int, stream: Optional[int]) -> int:
    return load_library().ttt_la_step(h, q, k, v, eta, float(eta_scalar), float(beta), int(mode), S, M, o,
                                      stream)


def ttt_la_check_state(desc: ttt_la_desc, call: int, q=None, k=None, v=None, eta=None, eta_scalar=1.0,
                       beta=0.0, mode=0, s_in=None, m_in=None, o=None, s_out=None, m_out=None) -> int:
    return load_library().ttt_la_check_state(ctypes.byref(desc), int(call), q, k, v, eta, float(eta_scalar),
                                             float(beta), int(mode), s_in, m_in, o, s_out, m_out)


def ttt_la_backward(h, q: int, k: int, v: int, eta: Optional[int], eta_scalar: float, beta: float, mode: int,
                    dO: int, dQ: int, dK: int, dV: int, dEta: Optional[int], workspace: Optional[int],
                    workspace_bytes: int, stream: Optional[int]) -> int:
    return load_library().ttt_la_backward(h, q, k, v, eta, float(eta_scalar), float(beta), int(mode), dO, dQ, dK,
                                          dV, dEta, workspace, int(workspace_bytes), stream)


def ttt_la_check_backward(desc: ttt_la_desc, hints: Optional[ttt_la_hints] = None, q=None, k=None, v=None, eta=None,
                          eta_scalar=1.0, beta=0.0, mode=0, dO=None, dQ=None, dK=None, dV=None, dEta=None,
                          workspace=None, workspace_bytes=0) -> int:
    return load_library().ttt_la_check_backward(ctypes.byref(desc), None if hints is None else ctypes.byref(hints),
                                                q, k, v, eta, float(eta_scalar), float(beta),
                                                int(mode), dO, dQ, dK, dV, dEta, workspace, int(workspace_bytes))


def ttt_la_backward_swiglu(h, q: int, k: int, v: int, eta: Optional[int], eta_scalar: float, beta: float,
                           mode: int, dO: int, dQ: int, dK: int, dV: int, dEta: Optional[int], dW1: int, dW3: int,
                           workspace: Optional[int], workspace_bytes: int, stream: Optional[int]) -> int:
    return load_library().ttt_la_backward_swiglu(h, q, k, v, eta, float(eta_scalar), float(beta), int(mode), dO, dQ,
                                                 dK, dV, dEta, dW1, dW3, workspace, int(workspace_bytes), stream)


def ttt_la_backward_workspace(h, mode: int):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = load_library().ttt_la_backward_workspace(h, int(mode), ctypes.byref(n))
    return st, n.value


def ttt_la_destroy(h) -> None:
    load_library().ttt_la_destroy(h)


def ttt_la_check(desc: ttt_la_desc, q=None, k=None, v=None, eta=None, eta_scalar=1.0, beta=0.0,
                 mode=0, o=None) -> int:
    return load_library().ttt_la_check(ctypes.byref(desc), q, k, v, eta, float(eta_scalar),
                                       float(beta), int(mode), o)


def ttt_la_get_plan(h) -> ttt_la_plan:
    p = ttt_la_plan()
    st = load_library().ttt_la_get_plan(h, ctypes.byref(p))
    if st != TTT_LA_OK:
        raise TTTError(st, "ttt_la_get_plan")
    return p


def ttt_la_wait_status(h) -> int:
    """1 if a bounded wait of the single-launch path gave up on h, else 0."""
    f = ctypes.c_int32(0)
    st = load_library().ttt_la_wait_status(h, ctypes.byref(f))
    if st != TTT_LA_OK:
        raise TTTError(st, "ttt_la_wait_status")
    return f.value


def ttt_la_enable_kernel_timing(h, n_slots: int) -> int:
    return load_library().ttt_la_enable_kernel_timing(h, int(n_slots))


def ttt_la_enable_kernel_timing_every(h, n_slots: int, every: int) -> int:
    return load_library().ttt_la_enable_kernel_timing_every(h, int(n_slots), int(every))


def ttt_la_kernel_times(h, capacity: int):
    buf = (ctypes.c_float * max(1, capacity))()
    n = ctypes.c_int32(0)
    st = load_library().ttt_la_kernel_times(h, buf, int(capacity), ctypes.byref(n))
    if st != TTT_LA_OK:
        raise TTTError(st, "ttt_la_kernel_times")
    return [buf[i] for i in range(n.value)]


# ----------------------------------------------------------------------------
# torch-facing convenience wrapper (still marshalling only)
# ----------------------------------------------------------------------------

_DTYPES = {"f32": TTT_LA_F32, "bf16": TTT_LA_BF16}
_PHIS = {"identity": TTT_LA_PHI_IDENTITY, "swiglu": TTT_LA_PHI_SWIGLU}
_ETA = {"scalar": TTT_LA_ETA_SCALAR, "per_token": TTT_LA_ETA_PER_TOKEN, "softplus": TTT_LA_ETA_SOFTPLUS}


def make_desc(B, H, T, d_k, d_v, d_phi=None, dtype="bf16", phi="identity", chunk=0,
              w1=None, w3=None) -> ttt_la_desc:
    d = ttt_la_desc()
    d.B, d.H, d.T, d.d_k, d.d_v = int(B), int(H), int(T), int(d_k), int(d_v)
    d.d_phi = int(d_k if d_phi is None else d_phi)
    d.dtype = _DTYPES[dtype]
    d.phi = _PHIS[phi]
    d.chunk = int(chunk)
    d.w1 = _ptr(w1)
    d.w3 = _ptr(w3)
    return d


def make_hints(segments=0, value_split=0, launch="auto") -> ttt_la_hints:
    h = ttt_la_hints()
    h.segments = int(segments)
    h.value_split = int(value_split)
    h.launch = _LAUNCH[launch] if isinstance(launch, str) else int(launch)
    return h


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


_LOSS = {"dot": 0, "mse": TTT_LA_LOSS_MSE}


def mode_bits(eta_mode: str = "scalar", causal: bool = True, loss: str = "dot", weight_norm: bool = False) -> int:
    return (_ETA[eta_mode] | (0 if causal else TTT_LA_BIDIRECTIONAL) | _LOSS[loss]
            | (TTT_LA_WEIGHT_NORM if weight_norm else 0))


_TORCH_DTYPES = {"f32": "float32", "bf16": "bfloat16"}


def check_tensors(desc: ttt_la_desc, call: str, mode: int, **tensors) -> None:
    """Host-side check of the torch tensors of one library call against the
    handle's descriptor, before any pointer reaches the C ABI (which takes raw
    pointers and cannot see sizes): shape, dtype, contiguity, one CUDA device.

    call: "forward", "forward_state", "step" or "backward".  Tensors that are
    None are skipped (optional arguments).  Raises ValueError."""
    import torch
    B, H, T = desc.B, desc.H, desc.T
    dk, dv, dphi = desc.d_k, desc.d_v, desc.d_phi
    io = getattr(torch, _TORCH_DTYPES["f32" if desc.dtype == TTT_LA_F32 else "bf16"])
    tok = 1 if call == "step" else T
    per_token = (mode & (TTT_LA_ETA_PER_TOKEN | TTT_LA_ETA_SOFTPLUS)) != 0
    want = {
        "q": ((B, H, tok, dk), io), "k": ((B, H, tok, dk), io), "v": ((B, H, tok, dv), io),
        "out": ((B, H, tok, dv), io), "dO": ((B, H, tok, dv), io),
        "eta": ((B, H) if call == "step" else (B, H, T), torch.float32),
    }
    for name in ("S0", "M0", "S_T", "M_T", "S", "M"):
        want[name] = ((B, H, dv, dphi), torch.float32)
    device = None
    for name, t in tensors.items():
        if name == "eta" and not per_token:
            if t is not None:
                raise ValueError("eta must be None for a scalar rate")
            continue
        if t is None:
            if name == "eta":
                raise ValueError("a per-token rate needs eta")
            continue
        shape, dtype = want[name]
        if name == "eta" and call == "step" and tuple(t.shape) == (B, H, 1):
            shape = (B, H, 1)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, the handle expects {shape}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, the handle expects {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    # devices last, once every shape and dtype is known to be right
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")


def _launch_stream(t, stream):
    """(stream handle for the C call, torch stream object or None).  Tensors this
    binding allocates for a call on another stream are recorded on that stream,
    so that the caching allocator does not hand their memory out again while the
    call's kernels may still use it."""
    import torch
    cur = torch.cuda.current_stream(t.device)
    if stream is None or int(stream) == cur.cuda_stream:
        return cur.cuda_stream, None
    return int(stream), torch.cuda.ExternalStream(int(stream), device=t.device)


def _record(ext, *ts):
    if ext is None:
        return
    for t in ts:
        if t is not None:
            t.record_stream(ext)


class TTTLinearAttention:
    """One layer shape bound to a library handle.

    ``forward(q, k, v, ...)`` takes contiguous device tensors shaped
    [B, H, T, d] (torch.float32 or torch.bfloat16) and writes o.
    """

    def __init__(self, B, H, T, d_k, d_v, d_phi=None, dtype="bf16", phi="identity", chunk=0,
                 segments=0, w1=None, w3=None, value_split=0, launch="auto"):
        self._keep = (w1, w3)         # W1/W3 are borrowed by the handle
        self.desc = make_desc(B, H, T, d_k, d_v, d_phi, dtype, phi, chunk, w1, w3)
        self.hints = make_hints(segments, value_split, launch)
        self.dtype = dtype
        st, h = ttt_la_create_hinted(self.desc, self.hints)
        if st != TTT_LA_OK:
            raise TTTError(st, "ttt_la_create_hinted")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            ttt_la_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def plan(self) -> ttt_la_plan:
        return ttt_la_get_plan(self.handle)

    def wait_failed(self) -> int:
        return ttt_la_wait_status(self.handle)

    def forward(self, q, k, v, eta=None, eta_scalar=1.0, beta=0.0, eta_mode="scalar", causal=True,
                out=None, stream=None, loss="dot"):
        """One forward; loss "mse" runs the delta rule (TTT_LA_LOSS_MSE)."""
        import torch
        mode = mode_bits(eta_mode, causal, loss)
        check_tensors(self.desc, "forward", mode, q=q, k=k, v=v, eta=eta, out=out)
        s, ext = _launch_stream(q, stream)
        fresh = out is None
        if fresh:
            out = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=v.dtype, device=v.device)
        st = ttt_la_forward(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), eta_scalar, beta, mode, _ptr(out), s)
        if st != TTT_LA_OK:
            raise TTTError(st, "ttt_la_forward")
        if fresh:
            _record(ext, out)
        return out

    def forward_state(self, q, k, v, eta=None, eta_scalar=1.0, beta=0.0, eta_mode="scalar", S0=None, M0=None,
                      out=None, S_T=None, M_T=None, stream=None, weight_norm=False, loss="dot"):
        """Causal forward from the carried state (S0, M0) (None = zero); writes the state
        after the last token to S_T, M_T when given (fp32 [B, H, d_v, d_phi]).
        weight_norm: the weight-normalised recurrence (TTT_LA_WEIGHT_NORM; S0 required).
        loss "mse": the delta rule (TTT_LA_LOSS_MSE), whose state is S alone (M0, M_T None)."""
        import torch
        mode = mode_bits(eta_mode, True, loss, weight_norm=weight_norm)
        check_tensors(self.desc, "forward_state", mode, q=q, k=k, v=v, eta=eta, out=out, S0=S0, M0=M0, S_T=S_T,
                      M_T=M_T)
        s, ext = _launch_stream(q, stream)
        fresh = out is None
        if fresh:
            out = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=v.dtype, device=v.device)
        st = ttt_la_forward_state(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), eta_scalar, beta, mode,
                                  _ptr(S0), _ptr(M0), _ptr(out), _ptr(S_T), _ptr(M_T), s)
        if st != TTT_LA_OK:
            raise TTTError(st, "ttt_la_forward_state")
        if fresh:
            _record(ext, out)
        return out

    def step(self, q, k, v, S, M, eta=None, eta_scalar=1.0, beta=0.0, eta_mode="scalar", out=None, stream=None,
             weight_norm=False, loss="dot"):
        """One recurrent step: q, k, v [B, H, 1, d]; S, M fp32 [B, H, d_v, d_phi] updated in place.
        weight_norm: Variant 1's step (TTT_LA_WEIGHT_NORM); loss "mse": the delta-rule step."""
        import torch
        mode = mode_bits(eta_mode, True, loss, weight_norm=weight_norm)
        if S is None or M is None:
            raise ValueError("the step needs the state S and M")
        check_tensors(self.desc, "step", mode, q=q, k=k, v=v, eta=eta, out=out, S=S, M=M)
        s, ext = _launch_stream(q, stream)
        fresh = out is None
        if fresh:
            out = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=v.dtype, device=v.device)
        st = ttt_la_step(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), eta_scalar, beta, mode, _ptr(S),
                         _ptr(M), _ptr(out), s)
        if st != TTT_LA_OK:
            raise TTTError(st, "ttt_la_step")
        if fresh:
            _record(ext, out)
        return out

    def backward(self, q, k, v, dO, eta=None, eta_scalar=1.0, beta=0.0, eta_mode="scalar", causal=True,
                 stream=None, want_eta=True):
        """Gradients (dq, dk, dv, deta) of sum(o * dO), and (dW1, dW3) for a SwiGLU layer;
        the workspace is a device tensor allocated here (the library itself allocates
        nothing)."""
        import torch
        mode = mode_bits(eta_mode, causal)
        check_tensors(self.desc, "backward", mode, q=q, k=k, v=v, eta=eta, dO=dO)
        st, nbytes = ttt_la_backward_workspace(self.handle, mode)
        if st != TTT_LA_OK:
            raise TTTError(st, "ttt_la_backward_workspace")
        s, ext = _launch_stream(q, stream)
        ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        de = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if want_eta else None
        if self.desc.phi == TTT_LA_PHI_SWIGLU:
            # also the gradients of the feature map's weights (fp32 [H, d_phi, d_k])
            wshape = (self.desc.H, self.desc.d_phi, self.desc.d_k)
            dw1 = torch.empty(wshape, dtype=torch.float32, device=q.device)
            dw3 = torch.empty(wshape, dtype=torch.float32, device=q.device)
            st = ttt_la_backward_swiglu(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), eta_scalar, beta, mode,
                                        _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(de), _ptr(dw1), _ptr(dw3),
                                        _ptr(ws), nbytes, s)
            if st != TTT_LA_OK:
                raise TTTError(st, "ttt_la_backward_swiglu")
            _record(ext, ws, dq, dk, dv, de, dw1, dw3)
            return dq, dk, dv, de, dw1, dw3
        st = ttt_la_backward(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), eta_scalar, beta, mode, _ptr(dO),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(de), _ptr(ws), nbytes, s)
        if st != TTT_LA_OK:
            raise TTTError(st, "ttt_la_backward")
        _record(ext, ws, dq, dk, dv, de)
        return dq, dk, dv, de
