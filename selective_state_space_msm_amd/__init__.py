"""Momentum-Mamba selective scan on AMD MI355X (gfx950): thin Python binding of libmsm.so.

The functions here have the names of the C entry points declared in ``include/msm.h`` and do
argument marshalling only: every step of the scan runs in the library's HIP kernels.  PyTorch
provides device memory and the current HIP stream.  If ``libmsm.so`` has not been built (see
``selective_state_space_msm_amd.build``) every call raises ``MsmLibraryMissing``; there is no
fallback implementation.

    y = msm_scan_fwd(x, delta, A, B, C, beta=0.9, alpha=1.0)             # (Bt, L, D)
    y, last_h, last_v = msm_scan_fwd(..., return_last_state=True)
    grads = msm_scan_bwd(x, delta, A, B, C, dy, beta=0.9, alpha=1.0)     # dict of tensors
    # the full operation: delta bias + softplus, SiLU output gate, initial state
    y = msm_selective_scan_fwd(x, delta, A, B, C, 0.9, 1.0, Dskip, z=z, delta_bias=bias,
                               delta_softplus=True)
    grads = msm_selective_scan_bwd(x, delta, A, B, C, dy, 0.9, 1.0, Dskip, z=z, delta_bias=bias,
                                   delta_softplus=True)        # also dz, ddelta_bias
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MsmError", "MsmLibraryMissing", "MSM_F32", "MSM_BF16", "library_path", "load_library",
    "msm_version", "msm_status_string", "msm_scan_fwd_workspace_bytes",
    "msm_scan_bwd_workspace_bytes", "msm_scan_fwd_plan", "msm_scan_bwd_plan", "msm_scan_fwd",
    "msm_scan_bwd", "msm_selective_scan_fwd", "msm_selective_scan_bwd", "msm_scan_step",
    "msm_scan_complex_fwd", "msm_scan_complex_bwd", "msm_scan_complex_bwd_workspace_bytes",
    "msm_scan_fwd_noalloc", "EXPORTED_SYMBOLS",
]

MSM_F32 = 0
MSM_BF16 = 1
_STATUS = {0: "MSM_OK", 1: "MSM_ERR_INVALID_ARG", 2: "MSM_ERR_UNSUPPORTED",
           3: "MSM_ERR_WORKSPACE", 4: "MSM_ERR_LAUNCH"}
EXPORTED_SYMBOLS = [
    "msm_version", "msm_status_string", "msm_scan_fwd_workspace_bytes",
    "msm_scan_bwd_workspace_bytes", "msm_scan_fwd_plan", "msm_scan_bwd_plan", "msm_scan_fwd",
    "msm_scan_fwd_with_plan", "msm_scan_bwd", "msm_scan_bwd_with_plan", "msm_scan_fwd_state",
    "msm_scan_bwd_state", "msm_selective_scan_fwd", "msm_selective_scan_bwd", "msm_scan_step",
    "msm_scan_complex_fwd", "msm_scan_complex_bwd_workspace_bytes", "msm_scan_complex_bwd",
    "msm_scan_fwd_noalloc",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmsm.so")
_lib = None


class MsmError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s" % (what, _STATUS.get(status, "status %d" % status)))


class MsmLibraryMissing(RuntimeError):
    pass


class _Plan(ctypes.Structure):
    _fields_ = [("states_per_wave", ctypes.c_int32), ("chunks", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmsm.so (once).  Raises MsmLibraryMissing when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MsmLibraryMissing(
            "libmsm.so not found at %s; build it with `python -m selective_state_space_msm_amd.build`"
            " (or __graft_entry__.build())" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, F, I32, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32,
                          ctypes.c_size_t)
    lib.msm_version.argtypes = []
    lib.msm_version.restype = I32
    lib.msm_status_string.argtypes = [ctypes.c_int]
    lib.msm_status_string.restype = ctypes.c_char_p
    for name in ("msm_scan_fwd_workspace_bytes", "msm_scan_bwd_workspace_bytes"):
        fn = getattr(lib, name)
        fn.argtypes = [I64, I64, I64, I64, ctypes.c_int]
        fn.restype = SZ
    for name in ("msm_scan_fwd_plan", "msm_scan_bwd_plan"):
        fn = getattr(lib, name)
        fn.argtypes = [I64, I64, I64, I64, ctypes.c_int, F, ctypes.POINTER(_Plan)]
        fn.restype = ctypes.c_int
    fwd = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, F, F, ctypes.c_int, P, SZ, P]
    lib.msm_scan_fwd.argtypes = fwd
    lib.msm_scan_fwd.restype = ctypes.c_int
    lib.msm_scan_fwd_with_plan.argtypes = fwd + [ctypes.POINTER(_Plan)]
    lib.msm_scan_fwd_with_plan.restype = ctypes.c_int
    lib.msm_scan_fwd_noalloc.argtypes = [P] * 9 + [I64, I64, I64, I64, F, F, ctypes.c_int, P]
    lib.msm_scan_fwd_noalloc.restype = ctypes.c_int
    bwd = [P, P, P, P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, F, F, ctypes.c_int, P, SZ, P]
    lib.msm_scan_bwd.argtypes = bwd
    lib.msm_scan_bwd.restype = ctypes.c_int
    lib.msm_scan_bwd_with_plan.argtypes = bwd + [ctypes.POINTER(_Plan)]
    lib.msm_scan_bwd_with_plan.restype = ctypes.c_int
    lib.msm_scan_fwd_state.argtypes = ([P] * 11 + [I64, I64, I64, I64, F, F, ctypes.c_int, P, SZ, P,
                                                   ctypes.POINTER(_Plan)])
    lib.msm_scan_fwd_state.restype = ctypes.c_int
    lib.msm_scan_bwd_state.argtypes = ([P] * 19 + [I64, I64, I64, I64, F, F, ctypes.c_int, P, SZ, P,
                                                   ctypes.POINTER(_Plan)])
    lib.msm_scan_bwd_state.restype = ctypes.c_int
    tail = [I64, I64, I64, I64, F, F, ctypes.c_int, P, SZ, P, ctypes.POINTER(_Plan)]
    lib.msm_selective_scan_fwd.argtypes = [P] * 8 + [I32, I32] + [P] * 5 + tail
    lib.msm_selective_scan_fwd.restype = ctypes.c_int
    lib.msm_selective_scan_bwd.argtypes = [P] * 8 + [I32, I32] + [P] * 15 + tail
    lib.msm_selective_scan_bwd.restype = ctypes.c_int
    lib.msm_scan_step.argtypes = ([P] * 8 + [I32, I32] + [P] * 3
                                  + [I64, I64, I64, F, F, ctypes.c_int, P])
    lib.msm_scan_step.restype = ctypes.c_int
    lib.msm_scan_complex_fwd.argtypes = [P] * 11 + [I64, I64, I64, I64, F, F, ctypes.c_int, P]
    lib.msm_scan_complex_fwd.restype = ctypes.c_int
    lib.msm_scan_complex_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, ctypes.c_int]
    lib.msm_scan_complex_bwd_workspace_bytes.restype = SZ
    lib.msm_scan_complex_bwd.argtypes = [P] * 19 + [I64, I64, I64, I64, F, F, ctypes.c_int, P, SZ,
                                                    P]
    lib.msm_scan_complex_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def msm_version() -> int:
    return int(load_library().msm_version())


def msm_status_string(status: int) -> str:
    return load_library().msm_status_string(int(status)).decode()


def _io_code(io) -> int:
    if io in (MSM_F32, "f32", "fp32", "float32"):
        return MSM_F32
    if io in (MSM_BF16, "bf16", "bfloat16"):
        return MSM_BF16
    import torch
    if io == torch.float32:
        return MSM_F32
    if io == torch.bfloat16:
        return MSM_BF16
    raise ValueError("unsupported io dtype %r" % (io,))


def msm_scan_fwd_workspace_bytes(Bt, L, D, N, io) -> int:
    return int(load_library().msm_scan_fwd_workspace_bytes(Bt, L, D, N, _io_code(io)))


def msm_scan_bwd_workspace_bytes(Bt, L, D, N, io) -> int:
    return int(load_library().msm_scan_bwd_workspace_bytes(Bt, L, D, N, _io_code(io)))


def _plan_call(fn, Bt, L, D, N, io, beta):
    pl = _Plan()
    st = fn(Bt, L, D, N, _io_code(io), float(beta), ctypes.byref(pl))
    if st != 0:
        raise MsmError(st, fn.__name__)
    return {"states_per_wave": pl.states_per_wave, "chunks": pl.chunks}


def msm_scan_fwd_plan(Bt, L, D, N, io, beta) -> dict:
    return _plan_call(load_library().msm_scan_fwd_plan, Bt, L, D, N, io, beta)


def msm_scan_bwd_plan(Bt, L, D, N, io, beta) -> dict:
    return _plan_call(load_library().msm_scan_bwd_plan, Bt, L, D, N, io, beta)


# ----------------------------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_handle(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class _Owned:
    """The tensors the binding allocates for one call (workspace, outputs the caller did not
    pass).  They are allocated on the current stream; when the call is enqueued on another
    stream, done() records each of them on that stream (Tensor.record_stream), so the caching
    allocator hands their memory to no other work until the call's kernels have finished."""

    def __init__(self, stream):
        self.stream = stream
        self.tensors = []

    def empty(self, shape, dtype, device):
        import torch
        t = torch.empty(shape, dtype=dtype, device=device)
        self.tensors.append(t)
        return t

    def done(self):
        if self.stream is not None:
            for t in self.tensors:
                t.record_stream(self.stream)


def _workspace(nbytes, workspace, device, own):
    import torch
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = own.empty(nbytes, torch.uint8, device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise MsmError(3, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _plan_arg(plan):
    if plan is None:
        return None
    return ctypes.byref(_Plan(int(plan.get("states_per_wave", 0)), int(plan.get("chunks", 0))))


def msm_scan_fwd(x, delta, A, B, C, beta, alpha, Dskip=None, *, y=None, last_h=None,
                 last_v=None, return_last_state=False, workspace=None, stream=None, plan=None,
                 h0=None, v0=None):
    """Forward scan.  x, delta: (Bt, L, D); A: (D, N) fp32; B, C: (Bt, L, N); Dskip: (D,) fp32.

    x, delta, B, C share one dtype (float32 or bfloat16), which is also the dtype of y.
    h0, v0: optional (Bt, D, N) fp32 initial state (msm_scan_fwd_state), e.g. the last state of
    a previous call over the first part of the sequence.
    Returns y, or (y, last_h, last_v) when return_last_state is true.
    """
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev = x.device
    Bt, L, D = x.shape
    N = A.shape[1]
    io = _io_code(x.dtype)
    _check(x, "x", (Bt, L, D), x.dtype, dev)
    _check(delta, "delta", (Bt, L, D), x.dtype, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(B, "B", (Bt, L, N), x.dtype, dev)
    _check(C, "C", (Bt, L, N), x.dtype, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    if y is None:
        y = own.empty((Bt, L, D), x.dtype, dev)
    _check(y, "y", (Bt, L, D), x.dtype, dev)
    if return_last_state:
        if last_h is None:
            last_h = own.empty((Bt, D, N), torch.float32, dev)
        if last_v is None:
            last_v = own.empty((Bt, D, N), torch.float32, dev)
    for t, nm in ((last_h, "last_h"), (last_v, "last_v"), (h0, "h0"), (v0, "v0")):
        if t is not None:
            _check(t, nm, (Bt, D, N), torch.float32, dev)
    nbytes = int(lib.msm_scan_fwd_workspace_bytes(Bt, L, D, N, io))
    ws, wsb = _workspace(nbytes, workspace, dev, own)
    tail = (Bt, L, D, N, float(beta), float(alpha), io, _ptr(ws), wsb, _stream_handle(stream, dev))
    if h0 is not None or v0 is not None:
        st = lib.msm_scan_fwd_state(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip),
                                    _ptr(h0), _ptr(v0), _ptr(y), _ptr(last_h), _ptr(last_v),
                                    *tail, _plan_arg(plan))
    else:
        args = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(y),
                _ptr(last_h), _ptr(last_v)) + tail
        if plan is None:
            st = lib.msm_scan_fwd(*args)
        else:
            st = lib.msm_scan_fwd_with_plan(*args, _plan_arg(plan))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_scan_fwd")
    if return_last_state:
        return y, last_h, last_v
    return y


def msm_scan_fwd_noalloc(x, delta, A, B, C, beta, alpha, Dskip=None, *, y, last_h=None,
                         last_v=None, stream=None):
    """Allocation-free forward (msm_scan_fwd_noalloc): msm_scan_fwd without a workspace, for
    callers that cannot allocate.  Every output is passed by the caller (y, and last_h / last_v
    when wanted); neither this function nor the library allocates.  Calls on one GPU share the
    library's static scratch and must not overlap.  Returns y."""
    import torch
    lib = load_library()
    dev = x.device
    Bt, L, D = x.shape
    N = A.shape[1]
    io = _io_code(x.dtype)
    for t, nm, shp in ((x, "x", (Bt, L, D)), (delta, "delta", (Bt, L, D)), (B, "B", (Bt, L, N)),
                       (C, "C", (Bt, L, N)), (y, "y", (Bt, L, D))):
        _check(t, nm, shp, x.dtype, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    for t, nm in ((last_h, "last_h"), (last_v, "last_v")):
        if t is not None:
            _check(t, nm, (Bt, D, N), torch.float32, dev)
    st = lib.msm_scan_fwd_noalloc(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip),
                                  _ptr(y), _ptr(last_h), _ptr(last_v), Bt, L, D, N, float(beta),
                                  float(alpha), io, _stream_handle(stream, dev))
    if st != 0:
        raise MsmError(st, "msm_scan_fwd_noalloc")
    return y


def msm_scan_bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=None, *, out=None, workspace=None,
                 stream=None, plan=None, h0=None, v0=None, dlast_h=None, dlast_v=None,
                 state_grads=False):
    """Gradients of sum(dy * y).  Returns a dict: dx, ddelta (Bt, L, D) and dB, dC (Bt, L, N)
    in the I/O dtype; dA (D, N) and dDskip (D,) (None without Dskip) in float32.

    With an initial state h0, v0 and/or adjoints dlast_h, dlast_v of the final state (all
    (Bt, D, N) fp32; msm_scan_bwd_state), the loss also holds <dlast_h, last_h> +
    <dlast_v, last_v>; with state_grads the dict also holds dh0, dv0 (fp32 (Bt, D, N)).
    """
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev = x.device
    Bt, L, D = x.shape
    N = A.shape[1]
    io = _io_code(x.dtype)
    for t, nm, shp in ((x, "x", (Bt, L, D)), (delta, "delta", (Bt, L, D)), (B, "B", (Bt, L, N)),
                       (C, "C", (Bt, L, N)), (dy, "dy", (Bt, L, D))):
        _check(t, nm, shp, x.dtype, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    o = dict(out or {})
    if "dx" not in o:
        o["dx"] = own.empty((Bt, L, D), x.dtype, dev)
    if "ddelta" not in o:
        o["ddelta"] = own.empty((Bt, L, D), x.dtype, dev)
    if "dA" not in o:
        o["dA"] = own.empty((D, N), torch.float32, dev)
    if "dB" not in o:
        o["dB"] = own.empty((Bt, L, N), x.dtype, dev)
    if "dC" not in o:
        o["dC"] = own.empty((Bt, L, N), x.dtype, dev)
    if Dskip is not None:
        if "dDskip" not in o:
            o["dDskip"] = own.empty((D,), torch.float32, dev)
    else:
        o["dDskip"] = None
    states = (h0, v0, dlast_h, dlast_v)
    for t, nm in zip(states, ("h0", "v0", "dlast_h", "dlast_v")):
        if t is not None:
            _check(t, nm, (Bt, D, N), torch.float32, dev)
    if state_grads:
        if "dh0" not in o:
            o["dh0"] = own.empty((Bt, D, N), torch.float32, dev)
        if "dv0" not in o:
            o["dv0"] = own.empty((Bt, D, N), torch.float32, dev)
    nbytes = int(lib.msm_scan_bwd_workspace_bytes(Bt, L, D, N, io))
    ws, wsb = _workspace(nbytes, workspace, dev, own)
    tail = (Bt, L, D, N, float(beta), float(alpha), io, _ptr(ws), wsb, _stream_handle(stream, dev))
    grads = (_ptr(o["dx"]), _ptr(o["ddelta"]), _ptr(o["dA"]), _ptr(o["dB"]), _ptr(o["dC"]),
             _ptr(o["dDskip"]))
    ins = (_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(dy))
    if state_grads or any(t is not None for t in states):
        st = lib.msm_scan_bwd_state(*ins, *(_ptr(t) for t in states), *grads,
                                    _ptr(o.get("dh0")), _ptr(o.get("dv0")), *tail,
                                    _plan_arg(plan))
    elif plan is None:
        st = lib.msm_scan_bwd(*ins, *grads, *tail)
    else:
        st = lib.msm_scan_bwd_with_plan(*ins, *grads, *tail, _plan_arg(plan))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_scan_bwd")
    return o


def _check_extras(x, z, delta_bias, dev):
    import torch
    Bt, L, D = x.shape
    if z is not None:
        _check(z, "z", (Bt, L, D), x.dtype, dev)
    if delta_bias is not None:
        _check(delta_bias, "delta_bias", (D,), torch.float32, dev)


def msm_selective_scan_fwd(x, delta, A, B, C, beta, alpha, Dskip=None, *, z=None,
                           delta_bias=None, delta_softplus=False, zero_order_hold=False, h0=None,
                           v0=None, y=None, last_h=None, last_v=None, return_last_state=False,
                           workspace=None, stream=None, plan=None):
    """The full forward (msm_selective_scan_fwd): the scan on softplus(delta + delta_bias) (or
    delta + delta_bias), output times silu(z); zero_order_hold selects the exact discretisation
    of the write.  z: (Bt, L, D) in the I/O dtype; delta_bias: (D,) fp32; other arguments as
    msm_scan_fwd.  Returns y, or (y, last_h, last_v)."""
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev = x.device
    Bt, L, D = x.shape
    N = A.shape[1]
    io = _io_code(x.dtype)
    for t, nm, shp in ((x, "x", (Bt, L, D)), (delta, "delta", (Bt, L, D)), (B, "B", (Bt, L, N)),
                       (C, "C", (Bt, L, N))):
        _check(t, nm, shp, x.dtype, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    _check_extras(x, z, delta_bias, dev)
    if y is None:
        y = own.empty((Bt, L, D), x.dtype, dev)
    _check(y, "y", (Bt, L, D), x.dtype, dev)
    if return_last_state:
        if last_h is None:
            last_h = own.empty((Bt, D, N), torch.float32, dev)
        if last_v is None:
            last_v = own.empty((Bt, D, N), torch.float32, dev)
    for t, nm in ((last_h, "last_h"), (last_v, "last_v"), (h0, "h0"), (v0, "v0")):
        if t is not None:
            _check(t, nm, (Bt, D, N), torch.float32, dev)
    nbytes = int(lib.msm_scan_fwd_workspace_bytes(Bt, L, D, N, io))
    ws, wsb = _workspace(nbytes, workspace, dev, own)
    st = lib.msm_selective_scan_fwd(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(delta_bias),
        int(bool(delta_softplus)), int(bool(zero_order_hold)), _ptr(h0), _ptr(v0), _ptr(y),
        _ptr(last_h), _ptr(last_v), Bt,
        L, D, N, float(beta), float(alpha), io, _ptr(ws), wsb, _stream_handle(stream, dev),
        _plan_arg(plan))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_selective_scan_fwd")
    if return_last_state:
        return y, last_h, last_v
    return y


def msm_selective_scan_bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=None, *, z=None,
                           delta_bias=None, delta_softplus=False, zero_order_hold=False, h0=None,
                           v0=None, dlast_h=None, dlast_v=None, state_grads=False, out=None,
                           workspace=None, stream=None, plan=None):
    """Gradients of the full operation (msm_selective_scan_bwd).  Returns the dict of
    msm_scan_bwd, where ddelta is the gradient of the raw delta, plus dz (I/O dtype, None
    without z), ddelta_bias (fp32 (D,), None without delta_bias) and, with state_grads, dh0 and
    dv0."""
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev = x.device
    Bt, L, D = x.shape
    N = A.shape[1]
    io = _io_code(x.dtype)
    for t, nm, shp in ((x, "x", (Bt, L, D)), (delta, "delta", (Bt, L, D)), (B, "B", (Bt, L, N)),
                       (C, "C", (Bt, L, N)), (dy, "dy", (Bt, L, D))):
        _check(t, nm, shp, x.dtype, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    _check_extras(x, z, delta_bias, dev)
    states = (h0, v0, dlast_h, dlast_v)
    for t, nm in zip(states, ("h0", "v0", "dlast_h", "dlast_v")):
        if t is not None:
            _check(t, nm, (Bt, D, N), torch.float32, dev)
    o = dict(out or {})
    for k, shp, dt in (("dx", (Bt, L, D), x.dtype), ("ddelta", (Bt, L, D), x.dtype),
                       ("dA", (D, N), torch.float32), ("dB", (Bt, L, N), x.dtype),
                       ("dC", (Bt, L, N), x.dtype)):
        if k not in o:
            o[k] = own.empty(shp, dt, dev)
    for k, given, shp, dt in (("dDskip", Dskip, (D,), torch.float32), ("dz", z, (Bt, L, D), x.dtype),
                              ("ddelta_bias", delta_bias, (D,), torch.float32)):
        if given is not None:
            if k not in o:
                o[k] = own.empty(shp, dt, dev)
        else:
            o[k] = None
    if state_grads:
        if "dh0" not in o:
            o["dh0"] = own.empty((Bt, D, N), torch.float32, dev)
        if "dv0" not in o:
            o["dv0"] = own.empty((Bt, D, N), torch.float32, dev)
    nbytes = int(lib.msm_scan_bwd_workspace_bytes(Bt, L, D, N, io))
    ws, wsb = _workspace(nbytes, workspace, dev, own)
    st = lib.msm_selective_scan_bwd(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(delta_bias),
        int(bool(delta_softplus)), int(bool(zero_order_hold)), _ptr(dy),
        *(_ptr(t) for t in states), _ptr(o["dx"]),
        _ptr(o["ddelta"]), _ptr(o["dA"]), _ptr(o["dB"]), _ptr(o["dC"]), _ptr(o["dDskip"]),
        _ptr(o["dz"]), _ptr(o["ddelta_bias"]), _ptr(o.get("dh0")), _ptr(o.get("dv0")), Bt, L, D,
        N, float(beta), float(alpha), io, _ptr(ws), wsb, _stream_handle(stream, dev),
        _plan_arg(plan))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_selective_scan_bwd")
    return o


def msm_scan_step(x, delta, A, B, C, h, v, beta, alpha, Dskip=None, *, z=None, delta_bias=None,
                  delta_softplus=False, zero_order_hold=False, y=None, stream=None):
    """One decode step (msm_scan_step): x, delta, z (Bt, D) and B, C (Bt, N) in the I/O dtype;
    h, v (Bt, D, N) fp32 states, updated in place.  Returns y (Bt, D)."""
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev = x.device
    Bt, D = x.shape
    N = A.shape[1]
    io = _io_code(x.dtype)
    for t, nm, shp in ((x, "x", (Bt, D)), (delta, "delta", (Bt, D)), (B, "B", (Bt, N)),
                       (C, "C", (Bt, N))):
        _check(t, nm, shp, x.dtype, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    for t, nm in ((h, "h"), (v, "v")):
        _check(t, nm, (Bt, D, N), torch.float32, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    if z is not None:
        _check(z, "z", (Bt, D), x.dtype, dev)
    if delta_bias is not None:
        _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
    if y is None:
        y = own.empty((Bt, D), x.dtype, dev)
    _check(y, "y", (Bt, D), x.dtype, dev)
    st = lib.msm_scan_step(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z),
                           _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zero_order_hold)),
                           _ptr(h), _ptr(v), _ptr(y),
                           Bt, D, N, float(beta), float(alpha), io, _stream_handle(stream, dev))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_scan_step")
    return y


# ----------------------------------------------------------------------------------------------
# complex-valued scan: complex arrays are passed as real tensors with a trailing dimension of 2
# (torch.view_as_real of a complex64 tensor for float32 I/O)
# ----------------------------------------------------------------------------------------------

def msm_scan_complex_bwd_workspace_bytes(Bt, L, D, N, io) -> int:
    return int(load_library().msm_scan_complex_bwd_workspace_bytes(Bt, L, D, N, _io_code(io)))


def _complex_inputs(x, delta, A, B, C, Dskip):
    import torch
    dev = x.device
    Bt, L, D = x.shape
    N = A.shape[1]
    for t, nm, shp in ((x, "x", (Bt, L, D)), (delta, "delta", (Bt, L, D)),
                       (B, "B", (Bt, L, N, 2)), (C, "C", (Bt, L, N, 2))):
        _check(t, nm, shp, x.dtype, dev)
    _check(A, "A", (D, N, 2), torch.float32, dev)
    if Dskip is not None:
        _check(Dskip, "Dskip", (D,), torch.float32, dev)
    return dev, Bt, L, D, N, _io_code(x.dtype)


def msm_scan_complex_fwd(x, delta, A, B, C, beta, alpha, Dskip=None, *, h0=None, v0=None, y=None,
                         last_h=None, last_v=None, return_last_state=False, stream=None):
    """Complex forward (msm_scan_complex_fwd).  x, delta: (Bt, L, D); A: (D, N, 2) fp32;
    B, C: (Bt, L, N, 2) in the dtype of x; h0, v0: optional (Bt, D, N, 2) fp32.  Returns y
    (Bt, L, D), or (y, last_h, last_v)."""
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev, Bt, L, D, N, io = _complex_inputs(x, delta, A, B, C, Dskip)
    if y is None:
        y = own.empty((Bt, L, D), x.dtype, dev)
    _check(y, "y", (Bt, L, D), x.dtype, dev)
    if return_last_state:
        if last_h is None:
            last_h = own.empty((Bt, D, N, 2), torch.float32, dev)
        if last_v is None:
            last_v = own.empty((Bt, D, N, 2), torch.float32, dev)
    for t, nm in ((last_h, "last_h"), (last_v, "last_v"), (h0, "h0"), (v0, "v0")):
        if t is not None:
            _check(t, nm, (Bt, D, N, 2), torch.float32, dev)
    st = lib.msm_scan_complex_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip),
                                  _ptr(h0), _ptr(v0), _ptr(y), _ptr(last_h), _ptr(last_v), Bt, L,
                                  D, N, float(beta), float(alpha), io, _stream_handle(stream, dev))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_scan_complex_fwd")
    if return_last_state:
        return y, last_h, last_v
    return y


def msm_scan_complex_bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=None, *, h0=None, v0=None,
                         dlast_h=None, dlast_v=None, state_grads=False, out=None, workspace=None,
                         stream=None):
    """Gradients of the complex scan's real loss (msm_scan_complex_bwd).  Returns a dict: dx,
    ddelta (Bt, L, D) and dB, dC (Bt, L, N, 2) in the I/O dtype, dA (D, N, 2) and dDskip (D,)
    (None without Dskip) in float32, and with state_grads dh0, dv0 (Bt, D, N, 2) fp32.  Complex
    gradients hold dL/dRe and dL/dIm in their last dimension."""
    import torch
    lib = load_library()
    own = _Owned(stream)
    dev, Bt, L, D, N, io = _complex_inputs(x, delta, A, B, C, Dskip)
    _check(dy, "dy", (Bt, L, D), x.dtype, dev)
    for t, nm in ((h0, "h0"), (v0, "v0"), (dlast_h, "dlast_h"), (dlast_v, "dlast_v")):
        if t is not None:
            _check(t, nm, (Bt, D, N, 2), torch.float32, dev)
    o = dict(out or {})
    for k, shp, dt in (("dx", (Bt, L, D), x.dtype), ("ddelta", (Bt, L, D), x.dtype),
                       ("dA", (D, N, 2), torch.float32), ("dB", (Bt, L, N, 2), x.dtype),
                       ("dC", (Bt, L, N, 2), x.dtype)):
        if k not in o:
            o[k] = own.empty(shp, dt, dev)
    if Dskip is not None:
        if "dDskip" not in o:
            o["dDskip"] = own.empty((D,), torch.float32, dev)
    else:
        o["dDskip"] = None
    if state_grads:
        if "dh0" not in o:
            o["dh0"] = own.empty((Bt, D, N, 2), torch.float32, dev)
        if "dv0" not in o:
            o["dv0"] = own.empty((Bt, D, N, 2), torch.float32, dev)
    nbytes = int(lib.msm_scan_complex_bwd_workspace_bytes(Bt, L, D, N, io))
    ws, wsb = _workspace(nbytes, workspace, dev, own)
    st = lib.msm_scan_complex_bwd(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(h0), _ptr(v0), _ptr(dy),
        _ptr(dlast_h), _ptr(dlast_v), _ptr(o["dx"]), _ptr(o["ddelta"]), _ptr(o["dA"]),
        _ptr(o["dB"]), _ptr(o["dC"]), _ptr(o["dDskip"]), _ptr(o.get("dh0")), _ptr(o.get("dv0")),
        Bt, L, D, N, float(beta), float(alpha), io, _ptr(ws), wsb, _stream_handle(stream, dev))
    own.done()
    if st != 0:
        raise MsmError(st, "msm_scan_complex_bwd")
    return o
