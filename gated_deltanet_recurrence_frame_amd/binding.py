"""Thin ctypes binding over libgdn's C ABI (include/gdn.h).

Argument marshalling only: every tensor argument is checked for device,
dtype, shape and contiguity before the C entry point is called, outputs and
workspace are allocated with torch on the tensors' device, and the entry
point runs on torch's current stream.  Every step of the computation runs in
the HIP kernels of libgdn.so; if the library is missing the first call
raises.

``POISON``: when true, every output, state and workspace buffer the binding
allocates is filled with all-ones bytes (NaN in bf16 and fp32) before the
library sees it, so that an element a kernel fails to write shows up as NaN
instead of a stale value from the caching allocator.  The parity tests turn
it on.
"""

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gdn.h")

GDN_BF16, GDN_FP32 = 0, 1
GDN_OP_FORWARD, GDN_OP_STEP, GDN_OP_BACKWARD = 0, 1, 2
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL_POINTER", 2: "GDN_ERR_BAD_SHAPE",
          3: "GDN_ERR_BAD_DTYPE", 4: "GDN_ERR_MISALIGNED",
          5: "GDN_ERR_WORKSPACE_TOO_SMALL", 6: "GDN_ERR_UNSUPPORTED",
          7: "GDN_ERR_HIP", 8: "GDN_ERR_ALIASING", 9: "GDN_ERR_SCRATCH_TOO_SMALL"}


ABI_VERSION = 4   # GDN_ABI_VERSION of include/gdn.h that GdnProblem mirrors
NOALLOC_SCRATCH_BYTES = 192 << 20   # GDN_NOALLOC_SCRATCH_BYTES


class GdnProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("N", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("key_scale", ctypes.c_float),
                ("scan_chunk", ctypes.c_int32), ("algorithm", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        self.name = STATUS.get(code, str(code))
        super().__init__("%s failed: %s (%s)" % (where, self.name, _status_string(code)))


_lib = None
_VP = ctypes.c_void_p
POISON = False


def _empty(shape, dtype, device):
    """torch.empty, filled with NaN bytes when POISON is set."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if POISON and t.numel():
        t.view(torch.uint8).fill_(255)
    return t


def lib():
    """Load libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(GdnProblem)
    L.gdn_abi_version.restype = ctypes.c_int
    L.gdn_abi_version.argtypes = []
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_status_string.argtypes = [ctypes.c_int]
    L.gdn_workspace_size.restype = ctypes.c_int
    L.gdn_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.gdn_saved_size.restype = ctypes.c_int
    L.gdn_saved_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    L.gdn_forward.restype = ctypes.c_int
    L.gdn_forward.argtypes = [P] + [_VP] * 10 + [ctypes.c_size_t, _VP]
    L.gdn_forward_events.restype = ctypes.c_int
    L.gdn_forward_events.argtypes = [P] + [_VP] * 10 + [ctypes.c_size_t, _VP,
                                                         ctypes.POINTER(_VP)]
    L.gdn_forward_noalloc.restype = ctypes.c_int
    L.gdn_forward_noalloc.argtypes = [P] + [_VP] * 10
    L.gdn_step.restype = ctypes.c_int
    L.gdn_step.argtypes = [P] + [_VP] * 8 + [ctypes.c_size_t, _VP]
    L.gdn_backward.restype = ctypes.c_int
    L.gdn_backward.argtypes = [P] + [_VP] * 16 + [ctypes.c_size_t, _VP]
    if L.gdn_abi_version() != ABI_VERSION:
        raise RuntimeError("libgdn.so has ABI version %d, this binding expects %d; rebuild it"
                           % (L.gdn_abi_version(), ABI_VERSION))
    _lib = L
    return L


def _status_string(code):
    try:
        return lib().gdn_status_string(int(code)).decode()
    except Exception:  # library not loadable: fall back to the name
        return STATUS.get(code, "?")


def header_functions():
    """Names of the functions include/gdn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:gdn_status|int|const char\*)\s+(gdn_\w+)\s*\(",
                                 text, re.M)))


def _check(code, where):
    if code != 0:
        raise GdnError(code, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


ALGORITHMS = {"auto": 0, "frame": 1, "token": 2, "direct": 3}
GDN_FLAG_NORMALIZE_QK, GDN_FLAG_GATE_LOGITS = 1, 2


def flags_of(normalize_qk=False, gate_logits=False):
    return ((GDN_FLAG_NORMALIZE_QK if normalize_qk else 0) |
            (GDN_FLAG_GATE_LOGITS if gate_logits else 0))


def make_problem(B, H, T, N, D, io="bf16", key_scale=0.0, scan_chunk=0, algorithm="auto",
                 flags=0):
    """gdn_problem; `flags` is an OR of GDN_FLAG_* (see flags_of)."""
    return GdnProblem(int(B), int(H), int(T), int(N), int(D), int(D),
                      GDN_BF16 if io == "bf16" else GDN_FP32, float(key_scale),
                      int(scan_chunk), ALGORITHMS[algorithm], int(flags))


def workspace_size(prob, op):
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_size(ctypes.byref(prob), int(op), ctypes.byref(n)),
           "gdn_workspace_size")
    return n.value


def saved_size(prob):
    n = ctypes.c_size_t(0)
    _check(lib().gdn_saved_size(ctypes.byref(prob), ctypes.byref(n)), "gdn_saved_size")
    return n.value


def _io_of(t):
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "fp32"
    raise TypeError("io tensors must be bfloat16 or float32, got %s" % t.dtype)


def _need(t, name, dtype, shape, dev):
    if t is None:
        raise ValueError("%s is required" % name)
    if t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _shapes(q, k, v, gamma, beta, n):
    if q.dim() != 4:
        raise ValueError("q must be [B, L, H, D]")
    B, L, H, D = q.shape
    if n < 1 or L % n:
        raise ValueError("L = %d is not a whole number of frames of N = %d" % (L, n))
    T = L // n
    dev, io = q.device, q.dtype
    _need(q, "q", io, (B, L, H, D), dev)
    _need(k, "k", io, (B, L, H, D), dev)
    _need(v, "v", io, (B, L, H, D), dev)
    _need(gamma, "gamma", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, L, H), dev)
    return B, L, H, D, T, dev


class ForwardPlan:
    """Preallocated outputs and workspace for repeated gdn_forward calls on
    one problem shape (used by the benchmark to keep allocation out of the
    timed region)."""

    def __init__(self, B, H, T, N, D, io, device, key_scale=0.0, scan_chunk=0, saved=False,
                 algorithm="auto", flags=0):
        self.prob = make_problem(B, H, T, N, D, io, key_scale, scan_chunk, algorithm, flags)
        dt = torch.bfloat16 if io == "bf16" else torch.float32
        device = torch.device(device)
        self.o = _empty((B, T * N, H, D), dt, device)
        self.state_out = _empty((B, H, D, D), torch.float32, device)
        self.ws = _empty(max(16, workspace_size(self.prob, GDN_OP_FORWARD)), torch.uint8, device)
        self.saved = _empty(saved_size(self.prob), torch.uint8, device) if saved else None
        self.device = device
        self.dtype = dt
        self.dims = (B, H, T, N, D)

    def check(self, q, k, v, gamma, beta, state_in=None, state_out=None):
        """Raise unless every tensor matches the plan's device, dtype, shape
        and layout (nothing is launched on a mismatch)."""
        B, H, T, N, D = self.dims
        dev, dt = self.device, self.dtype
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            _need(t, name, dt, (B, T * N, H, D), dev)
        _need(gamma, "gamma", torch.float32, (B, T, H), dev)
        _need(beta, "beta", torch.float32, (B, T * N, H), dev)
        for t, name in ((state_in, "state_in"), (state_out, "state_out")):
            if t is not None:
                _need(t, name, torch.float32, (B, H, D, D), dev)

    def __call__(self, q, k, v, gamma, beta, state_in=None, events=None, state_out=None):
        """events: None, or 4 raw hipEvent_t handles (ints) recorded around
        the Gram/write, scan and output kernels (gdn_forward_events).
        state_out: None (the plan's own buffer), or a [B, H, D, D] fp32
        tensor, which may be state_in itself (the state carried in place
        from one call to the next)."""
        self.check(q, k, v, gamma, beta, state_in, state_out)
        so = self.state_out if state_out is None else state_out
        args = (ctypes.byref(self.prob), _p(q), _p(k), _p(v), _p(gamma), _p(beta),
                _p(state_in), _p(self.o), _p(so), _p(self.saved), _p(self.ws),
                self.ws.numel(), _stream(self.device))
        if events is None:
            _check(lib().gdn_forward(*args), "gdn_forward")
        else:
            ev = (_VP * 4)(*[_VP(int(e)) for e in events])
            _check(lib().gdn_forward_events(*args, ev), "gdn_forward_events")
        return self.o, so


def forward(q, k, v, gamma, beta, n, state_in=None, key_scale=0.0, scan_chunk=0,
            return_saved=False, algorithm="auto", normalize_qk=False, gate_logits=False):
    """o, state_out (and the saved A_t / S_t buffer) of gdn_forward.
    normalize_qk / gate_logits: the block's prologue (GDN_FLAG_*)."""
    B, L, H, D, T, dev = _shapes(q, k, v, gamma, beta, n)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, D, D), dev)
    plan = ForwardPlan(B, H, T, n, D, _io_of(q), dev, key_scale, scan_chunk, return_saved,
                       algorithm, flags_of(normalize_qk, gate_logits))
    o, st = plan(q, k, v, gamma, beta, state_in)
    if return_saved:
        return o, st, plan.saved
    return o, st


class StepPlan:
    """Preallocated problem, output and workspace for repeated gdn_step calls
    on one frame shape (streaming: one call per latent frame, the state
    carried in place).  Call with q, k, v [B, N, H, D], gamma [B, 1, H],
    beta [B, N, H] and the state [B, H, D, D] fp32; returns the plan's
    output buffer [B, N, H, D] (overwritten by the next call)."""

    def __init__(self, B, H, N, D, io, device, key_scale=0.0, algorithm="auto", flags=0):
        self.prob = make_problem(B, H, 1, N, D, io, key_scale, 0, algorithm, flags)
        dt = torch.bfloat16 if io == "bf16" else torch.float32
        device = torch.device(device)
        self.o = _empty((B, N, H, D), dt, device)
        self.ws = _empty(max(16, workspace_size(self.prob, GDN_OP_STEP)), torch.uint8, device)
        self.device = device
        self.dtype = dt
        self.shape = (B, N, H, D)

    def check(self, q, k, v, gamma, beta, state):
        """Raise unless every tensor matches the plan (nothing is launched on
        a mismatch)."""
        B, N, H, D = self.shape
        dev, dt = self.device, self.dtype
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            _need(t, name, dt, (B, N, H, D), dev)
        _need(gamma, "gamma", torch.float32, (B, 1, H), dev)
        _need(beta, "beta", torch.float32, (B, N, H), dev)
        _need(state, "state", torch.float32, (B, H, D, D), dev)

    def __call__(self, q, k, v, gamma, beta, state):
        self.check(q, k, v, gamma, beta, state)
        _check(lib().gdn_step(ctypes.byref(self.prob), _p(q), _p(k), _p(v), _p(gamma), _p(beta),
                              _p(state), _p(self.o), _p(self.ws), self.ws.numel(),
                              _stream(self.device)), "gdn_step")
        return self.o


def step(q, k, v, gamma, beta, state, key_scale=0.0, out=None, workspace=None,
         normalize_qk=False, gate_logits=False, algorithm="auto"):
    """One streaming frame: q, k, v [B, N, H, D], gamma [B, 1, H], beta
    [B, N, H]; `state` [B, H, D, D] fp32 is updated in place.  Returns o."""
    B, N, H, D, T, dev = _shapes(q, k, v, gamma, beta, q.shape[1])
    _need(state, "state", torch.float32, (B, H, D, D), dev)
    prob = make_problem(B, H, 1, N, D, _io_of(q), key_scale, 0, algorithm,
                        flags=flags_of(normalize_qk, gate_logits))
    if out is not None:
        _need(out, "out", q.dtype, tuple(v.shape), dev)
    o = out if out is not None else _empty(tuple(v.shape), q.dtype, dev)
    if workspace is None:
        workspace = _empty(max(16, workspace_size(prob, GDN_OP_STEP)), torch.uint8, dev)
    else:
        _need(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    _check(lib().gdn_step(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(gamma), _p(beta),
                          _p(state), _p(o), _p(workspace), workspace.numel(), _stream(dev)),
           "gdn_step")
    return o


def backward(q, k, v, gamma, beta, n, d_o, state_in=None, d_state_out=None, saved=None,
             key_scale=0.0, workspace=None, scan_chunk=0, normalize_qk=False,
             gate_logits=False):
    """Gradients dict (dq, dk, dv, dgamma, dbeta, dstate_in) of gdn_backward
    (with the prologue flags: with respect to the raw q, k, gate logits)."""
    B, L, H, D, T, dev = _shapes(q, k, v, gamma, beta, n)
    _need(d_o, "d_o", q.dtype, (B, L, H, D), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, D, D), dev)
    if d_state_out is not None:
        _need(d_state_out, "d_state_out", torch.float32, (B, H, D, D), dev)
    prob = make_problem(B, H, T, n, D, _io_of(q), key_scale, scan_chunk,
                        flags=flags_of(normalize_qk, gate_logits))
    if saved is not None:
        _need(saved, "saved", torch.uint8, (saved_size(prob),), dev)
    dq, dk, dv = (_empty(tuple(t.shape), t.dtype, dev) for t in (q, k, v))
    dgamma = _empty(tuple(gamma.shape), torch.float32, dev)
    dbeta = _empty(tuple(beta.shape), torch.float32, dev)
    dstate = _empty((B, H, D, D), torch.float32, dev)
    if workspace is None:
        workspace = _empty(max(16, workspace_size(prob, GDN_OP_BACKWARD)), torch.uint8, dev)
    else:
        _need(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    _check(lib().gdn_backward(ctypes.byref(prob), _p(q), _p(k), _p(v), _p(gamma), _p(beta),
                              _p(state_in), _p(d_o), _p(d_state_out), _p(saved), _p(dq),
                              _p(dk), _p(dv), _p(dgamma), _p(dbeta), _p(dstate),
                              _p(workspace), workspace.numel(), _stream(dev)),
           "gdn_backward")
    return {"dq": dq, "dk": dk, "dv": dv, "dgamma": dgamma, "dbeta": dbeta,
            "dstate_in": dstate}
