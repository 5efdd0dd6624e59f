"""fp64 CPU oracle for the Momentum-Mamba selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product library (``selective_state_space_msm_amd``) never imports it,
and it imports nothing from the product.  It shares no code with the HIP path.

The arithmetic lives in ``msm_oracle.c`` (plain double-precision loops; its header gives the
equations and the pages they follow).  This module only builds that file with gcc, loads it
with ctypes and widens numpy inputs to float64 (exact for fp32 and bf16 values).

Pinned by ``tests/test_oracle_pins.py``: worked examples printed on the pages, closed forms,
the materialised matrix form, the convolution form, finite differences and scaling identities.
``tests/test_oracle_mutants.py`` compiles deliberately broken copies of the C file and checks
that the pins reject each of them.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "msm_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libmsm_oracle.so")

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
             "-std=c11", "-Wall"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C file into a shared library with the oracle's fixed gcc flags."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile msm_oracle.c (always).  Returns the .so path."""
    return compile_source(SOURCE, _LIB_PATH)


def _f64(a):
    """Widen to a C-contiguous float64 array (exact for fp32 / bf16-valued inputs)."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shapes(x, A, B):
    Bt, L, D = x.shape
    D2, N = A.shape
    if D2 != D or B.shape != (Bt, L, N):
        raise ValueError("inconsistent shapes: x %s A %s B %s" % (x.shape, A.shape, B.shape))
    return Bt, L, D, N


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I64, Dbl, Int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        lib.msm_oracle_fwd.argtypes = [P, P, P, P, P, P, P, P, Dbl, Dbl, I64, I64, I64, I64, P, P, P,
                                       Int]
        lib.msm_oracle_fwd.restype = Int
        lib.msm_oracle_fwd_plain.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, P, Int]
        lib.msm_oracle_fwd_plain.restype = Int
        lib.msm_oracle_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, Dbl, Dbl, I64, I64, I64,
                                       I64, P, P, P, P, P, P, P, P, Int]
        lib.msm_oracle_bwd.restype = Int
        lib.msm_oracle_fused_fwd.argtypes = [P, P, P, P, P, P, P, P, Int, Int, P, P, Dbl, Dbl, I64,
                                             I64, I64, I64, P, P, P, P, Int]
        lib.msm_oracle_fused_fwd.restype = Int
        lib.msm_oracle_fused_bwd.argtypes = [P, P, P, P, P, P, P, P, Int, Int, P, P, P, P, P, Dbl,
                                             Dbl, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P,
                                             Int]
        lib.msm_oracle_fused_bwd.restype = Int
        lib.msm_oracle_complex_fwd.argtypes = lib.msm_oracle_fwd.argtypes
        lib.msm_oracle_complex_fwd.restype = Int
        lib.msm_oracle_complex_bwd.argtypes = lib.msm_oracle_bwd.argtypes
        lib.msm_oracle_complex_bwd.restype = Int
        lib.msm_oracle_max_threads.argtypes = []
        lib.msm_oracle_max_threads.restype = Int
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.msm_oracle_max_threads())

    def fwd(self, x, delta, A, B, C, beta, alpha, Dskip=None, threads=0, h0=None, v0=None):
        """Momentum recurrence forward in fp64.  Returns (y, last_h, last_v) as float64.

        x, delta: (Bt, L, D); A: (D, N); B, C: (Bt, L, N); Dskip: (D,) or None;
        h0, v0: (Bt, D, N) initial state or None (zero).
        """
        x, delta, A, B, C = (_f64(a) for a in (x, delta, A, B, C))
        Ds = None if Dskip is None else _f64(Dskip)
        Bt, L, D, N = _shapes(x, A, B)
        if delta.shape != x.shape or C.shape != B.shape or (Ds is not None and Ds.shape != (D,)):
            raise ValueError("inconsistent shapes")
        h0, v0 = (None if a is None else _f64(a) for a in (h0, v0))
        for a in (h0, v0):
            if a is not None and a.shape != (Bt, D, N):
                raise ValueError("initial state shape %s" % (a.shape,))
        y = np.empty((Bt, L, D), np.float64)
        last_h = np.empty((Bt, D, N), np.float64)
        last_v = np.empty((Bt, D, N), np.float64)
        rc = self.lib.msm_oracle_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Ds),
                                     _ptr(h0), _ptr(v0), float(beta), float(alpha), Bt, L, D, N,
                                     _ptr(y), _ptr(last_h), _ptr(last_v), int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_fwd failed (%d)" % rc)
        return y, last_h, last_v

    def fwd_plain(self, x, delta, A, B, C, Dskip=None, threads=0):
        """Standard (velocity-free) Mamba recurrence in fp64.  Returns (y, last_h)."""
        x, delta, A, B, C = (_f64(a) for a in (x, delta, A, B, C))
        Ds = None if Dskip is None else _f64(Dskip)
        Bt, L, D, N = _shapes(x, A, B)
        y = np.empty((Bt, L, D), np.float64)
        last_h = np.empty((Bt, D, N), np.float64)
        rc = self.lib.msm_oracle_fwd_plain(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                           _ptr(Ds), Bt, L, D, N, _ptr(y), _ptr(last_h),
                                           int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_fwd_plain failed (%d)" % rc)
        return y, last_h

    def bwd(self, x, delta, A, B, C, dy, beta, alpha, Dskip=None, threads=0, h0=None, v0=None,
            dlast_h=None, dlast_v=None):
        """Gradients of sum(dy * y) (+ <dlast_h, last_h> + <dlast_v, last_v>) in fp64, for the
        scan started at (h0, v0) (None: zero).

        Returns a dict with dx, ddelta (Bt, L, D), dA (D, N), dB, dC (Bt, L, N), dDskip (D,)
        (None when Dskip is None) and dh0, dv0 (Bt, D, N).
        """
        x, delta, A, B, C, dy = (_f64(a) for a in (x, delta, A, B, C, dy))
        Ds = None if Dskip is None else _f64(Dskip)
        Bt, L, D, N = _shapes(x, A, B)
        if dy.shape != x.shape:
            raise ValueError("dy shape")
        st = [None if a is None else _f64(a) for a in (h0, v0, dlast_h, dlast_v)]
        for a in st:
            if a is not None and a.shape != (Bt, D, N):
                raise ValueError("state shape %s" % (a.shape,))
        out = dict(dx=np.empty((Bt, L, D)), ddelta=np.empty((Bt, L, D)), dA=np.empty((D, N)),
                   dB=np.empty((Bt, L, N)), dC=np.empty((Bt, L, N)),
                   dDskip=None if Ds is None else np.empty((D,)),
                   dh0=np.empty((Bt, D, N)), dv0=np.empty((Bt, D, N)))
        rc = self.lib.msm_oracle_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Ds),
                                     _ptr(dy), _ptr(st[0]), _ptr(st[1]), _ptr(st[2]), _ptr(st[3]),
                                     float(beta), float(alpha), Bt, L, D, N,
                                     _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
                                     _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dDskip"]),
                                     _ptr(out["dh0"]), _ptr(out["dv0"]), int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_bwd failed (%d)" % rc)
        return out

    def fused_fwd(self, x, delta, A, B, C, beta, alpha, Dskip=None, z=None, delta_bias=None,
                  delta_softplus=False, h0=None, v0=None, threads=0, zoh=False):
        """The fused op forward: delta_eff = softplus(delta + delta_bias) (or delta + delta_bias),
        the momentum scan on delta_eff (zoh: zero-order-hold write coefficient), then
        y = y_raw * silu(z).

        Returns (y, y_raw, last_h, last_v) as float64; y_raw is the output before the gate.
        """
        x, delta, A, B, C = (_f64(a) for a in (x, delta, A, B, C))
        Bt, L, D, N = _shapes(x, A, B)
        Ds, zz, db, h0, v0 = (None if a is None else _f64(a) for a in (Dskip, z, delta_bias, h0, v0))
        if zz is not None and zz.shape != x.shape:
            raise ValueError("z shape %s" % (zz.shape,))
        if db is not None and db.shape != (D,):
            raise ValueError("delta_bias shape %s" % (db.shape,))
        y, y_raw = np.empty((Bt, L, D)), np.empty((Bt, L, D))
        last_h, last_v = np.empty((Bt, D, N)), np.empty((Bt, D, N))
        rc = self.lib.msm_oracle_fused_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                           _ptr(Ds), _ptr(zz), _ptr(db), int(bool(delta_softplus)),
                                           int(bool(zoh)), _ptr(h0), _ptr(v0), float(beta), float(alpha), Bt, L,
                                           D, N, _ptr(y), _ptr(y_raw), _ptr(last_h), _ptr(last_v),
                                           int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_fused_fwd failed (%d)" % rc)
        return y, y_raw, last_h, last_v

    def fused_bwd(self, x, delta, A, B, C, dy, beta, alpha, Dskip=None, z=None, delta_bias=None,
                  delta_softplus=False, h0=None, v0=None, dlast_h=None, dlast_v=None, threads=0,
                  zoh=False):
        """Gradients of the fused op.  Returns the dict of ``bwd`` (ddelta is the gradient of
        the raw delta) plus dz (None without z) and ddelta_bias (None without delta_bias)."""
        x, delta, A, B, C, dy = (_f64(a) for a in (x, delta, A, B, C, dy))
        Bt, L, D, N = _shapes(x, A, B)
        Ds, zz, db = (None if a is None else _f64(a) for a in (Dskip, z, delta_bias))
        st = [None if a is None else _f64(a) for a in (h0, v0, dlast_h, dlast_v)]
        out = dict(dx=np.empty((Bt, L, D)), ddelta=np.empty((Bt, L, D)), dA=np.empty((D, N)),
                   dB=np.empty((Bt, L, N)), dC=np.empty((Bt, L, N)),
                   dDskip=None if Ds is None else np.empty((D,)),
                   dz=None if zz is None else np.empty((Bt, L, D)),
                   ddelta_bias=None if db is None else np.empty((D,)),
                   dh0=np.empty((Bt, D, N)), dv0=np.empty((Bt, D, N)))
        rc = self.lib.msm_oracle_fused_bwd(
            _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Ds), _ptr(zz), _ptr(db),
            int(bool(delta_softplus)), int(bool(zoh)), _ptr(dy), _ptr(st[0]), _ptr(st[1]), _ptr(st[2]),
            _ptr(st[3]), float(beta), float(alpha), Bt, L, D, N, _ptr(out["dx"]),
            _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
            _ptr(out["dDskip"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]),
            _ptr(out["dv0"]), int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_fused_bwd failed (%d)" % rc)
        return out

    def step(self, x, delta, A, B, C, h, v, beta, alpha, Dskip=None, z=None, delta_bias=None,
             delta_softplus=False, zoh=False):
        """One decode step (the README's ``step``: one token, the ssm and velocity states
        carried in and out).  x, delta, z: (Bt, D); B, C: (Bt, N); h, v: (Bt, D, N).  It is the
        fused forward over a sequence of length one started at (h, v).
        Returns (y (Bt, D), h_new, v_new) as float64."""
        x, delta, B, C = (_f64(a) for a in (x, delta, B, C))
        Bt, D = x.shape
        N = B.shape[1]
        y, _, hn, vn = self.fused_fwd(x.reshape(Bt, 1, D), delta.reshape(Bt, 1, D), A,
                                      B.reshape(Bt, 1, N), C.reshape(Bt, 1, N), beta, alpha,
                                      Dskip=Dskip,
                                      z=None if z is None else _f64(z).reshape(Bt, 1, D),
                                      delta_bias=delta_bias, delta_softplus=delta_softplus,
                                      h0=h, v0=v, zoh=zoh)
        return y.reshape(Bt, D), hn, vn

    def complex_fwd(self, x, delta, A, B, C, beta, alpha, Dskip=None, h0=None, v0=None,
                    threads=0):
        """Complex-valued SSM forward in fp64: A (D, N), B, C (Bt, L, N), h0, v0 (Bt, D, N)
        complex; x, delta (Bt, L, D) real.  y = Re(sum_n C h) (+ Dskip x).  Returns (y real,
        last_h, last_v complex)."""
        x, delta = _f64(x), _f64(delta)
        cz = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a, np.complex128))
        A, B, C, h0, v0 = (cz(a) for a in (A, B, C, h0, v0))
        Bt, L, D = x.shape
        N = A.shape[1]
        if A.shape != (D, N) or B.shape != (Bt, L, N) or C.shape != B.shape:
            raise ValueError("inconsistent shapes")
        Ds = None if Dskip is None else _f64(Dskip)
        y = np.empty((Bt, L, D))
        lh, lv = np.empty((Bt, D, N), np.complex128), np.empty((Bt, D, N), np.complex128)
        rc = self.lib.msm_oracle_complex_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                             _ptr(Ds), _ptr(h0), _ptr(v0), float(beta),
                                             float(alpha), Bt, L, D, N, _ptr(y), _ptr(lh),
                                             _ptr(lv), int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_complex_fwd failed (%d)" % rc)
        return y, lh, lv

    def complex_bwd(self, x, delta, A, B, C, dy, beta, alpha, Dskip=None, h0=None, v0=None,
                    dlast_h=None, dlast_v=None, threads=0):
        """Gradients of the complex-valued SSM (real loss; each complex gradient is
        dl/d(re) + i dl/d(im)).  Returns dx, ddelta, dDskip real and dA, dB, dC, dh0, dv0
        complex."""
        x, delta, dy = _f64(x), _f64(delta), _f64(dy)
        cz = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a, np.complex128))
        A, B, C, h0, v0, dlh, dlv = (cz(a) for a in (A, B, C, h0, v0, dlast_h, dlast_v))
        Bt, L, D = x.shape
        N = A.shape[1]
        Ds = None if Dskip is None else _f64(Dskip)
        out = dict(dx=np.empty((Bt, L, D)), ddelta=np.empty((Bt, L, D)),
                   dA=np.empty((D, N), np.complex128), dB=np.empty((Bt, L, N), np.complex128),
                   dC=np.empty((Bt, L, N), np.complex128),
                   dDskip=None if Ds is None else np.empty((D,)),
                   dh0=np.empty((Bt, D, N), np.complex128), dv0=np.empty((Bt, D, N), np.complex128))
        rc = self.lib.msm_oracle_complex_bwd(
            _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Ds), _ptr(dy), _ptr(h0),
            _ptr(v0), _ptr(dlh), _ptr(dlv), float(beta), float(alpha), Bt, L, D, N,
            _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
            _ptr(out["dC"]), _ptr(out["dDskip"]), _ptr(out["dh0"]), _ptr(out["dv0"]),
            int(threads))
        if rc != 0:
            raise RuntimeError("msm_oracle_complex_bwd failed (%d)" % rc)
        return out


_default = None


def default() -> Oracle:
    """The oracle built from msm_oracle.c (compiled on first use if no library is present)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def fwd(*args, **kw):
    return default().fwd(*args, **kw)


def fwd_plain(*args, **kw):
    return default().fwd_plain(*args, **kw)


def bwd(*args, **kw):
    return default().bwd(*args, **kw)


def fused_fwd(*args, **kw):
    return default().fused_fwd(*args, **kw)


def fused_bwd(*args, **kw):
    return default().fused_bwd(*args, **kw)


def step(*args, **kw):
    return default().step(*args, **kw)


def complex_fwd(*args, **kw):
    return default().complex_fwd(*args, **kw)


def complex_bwd(*args, **kw):
    return default().complex_bwd(*args, **kw)


def max_threads() -> int:
    return default().max_threads()
