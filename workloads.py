"""Seeded synthetic inputs for the Momentum-Mamba selective scan.

This module is shared by the tests, the bench and the smoke check.  It only *draws* inputs: it
holds none of the scan's arithmetic (no recurrence, no exp of delta*A, no gradient).  Both the
fp64 oracle and the HIP library receive the arrays it returns.

Distributions (one recipe per named workload):

* ``tiny``   Bt=1, L=64,    D=4,    N=4,  fp32 I/O, beta=0.9 (also beta=0), alpha=1.
             x ~ N(0,1); delta log-uniform on [1e-3, 1e-1] (the dt_min/dt_max defaults of the
             Mamba module); A[d,n] = -(n+1) (S4D-real); B, C ~ N(0,1).
* ``m130m``  Bt=8, L=2048,  D=1536, N=16, fp32 I/O, beta in {0, 0.9}, alpha=1 (forward).
             delta = softplus(N(-4, 1)); otherwise as ``tiny``.
* ``m1p4b``  Bt=4, L=4096,  D=4096, N=16, bf16 I/O with fp32 state, beta=0.9, alpha=1 (forward).
* ``long``   Bt=1, L=65536, D=2048, N=16, bf16 I/O, beta=0.95, alpha=0.5, Dskip ~ N(0,1)
             (forward; long enough that the sequence is split into chunks).
* ``bwd``    Bt=4, L=2048,  D=2048, N=16, fp32 I/O, beta=0.9, alpha=1, plus dy ~ N(0,1)
             (backward).
* ``pages``  Bt=2, L=512, D=256, N=16, fp32 I/O, beta in {0, 0.9}, alpha=1: the shape of the
             benchmark table in the Momentum Mamba README (batch 2, dim 256, seqlen 512,
             dstate 16; its precision is not stated), distributions as ``m130m``.  Context only.
* ``decode`` Bt=1024, L=1,  D=4096, N=16, bf16 I/O, beta=0.9, alpha=1, Dskip ~ N(0,1): one
             token of the Mamba-1.4B layer shape for a serving batch of 1024 sequences, with
             (Bt, D, N) fp32 ssm / velocity states ~ N(0,1) (``make_state``) and the fused op's
             extras (``make_fused_extras``).  Large enough that the states (2 x 268 MB) do not
             stay in the last-level cache between steps.

* ``complex`` Bt=4, L=2048, D=2048, N=16 complex states, fp32 I/O, beta=0.9, alpha=1 (the
             complex scan, forward and backward; ``make_complex_inputs``): A[d, n] = -1/2 + i pi n
             (the S4D-Lin initialisation named on the complextorch page), B, C complex with
             independent N(0, 1/2) real and imaginary parts (unit variance), x ~ N(0, 1),
             delta = softplus(N(-4, 1)), dy ~ N(0, 1).

Draws are made in float64 with ``numpy.random.Generator(PCG64(seed))``, cast to float32, and for
bf16 workloads rounded once to bfloat16 (round-to-nearest-even) on the host.  Arrays are always
returned as float32 numpy arrays whose values are exactly representable in the I/O dtype, so the
oracle (which widens to float64) and the GPU see the same numbers.  A and Dskip stay float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_complex_inputs", "make_complex_state",
           "round_to_bf16", "bf16_bits"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    Bt: int
    L: int
    D: int
    N: int
    io: str            # "f32" or "bf16"
    beta: float
    alpha: float
    dskip: bool
    direction: str     # "fwd", "bwd" or "step" (one decode token)
    delta_dist: str    # "loguniform" or "softplus"
    seed: int

    @property
    def updates(self) -> int:
        return self.Bt * self.L * self.D * self.N

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 4, 4, "f32", 0.9, 1.0, False, "fwd", "loguniform", 1001),
    "m130m": Workload("m130m", 8, 2048, 1536, 16, "f32", 0.9, 1.0, False, "fwd", "softplus", 1002),
    "m1p4b": Workload("m1p4b", 4, 4096, 4096, 16, "bf16", 0.9, 1.0, False, "fwd", "softplus", 1003),
    "long": Workload("long", 1, 65536, 2048, 16, "bf16", 0.95, 0.5, True, "fwd", "softplus", 1004),
    "bwd": Workload("bwd", 4, 2048, 2048, 16, "f32", 0.9, 1.0, False, "bwd", "softplus", 1005),
    "pages": Workload("pages", 2, 512, 256, 16, "f32", 0.9, 1.0, False, "fwd", "softplus", 1007),
    "decode": Workload("decode", 1024, 1, 4096, 16, "bf16", 0.9, 1.0, True, "step", "softplus",
                       1006),
    "complex": Workload("complex", 4, 2048, 2048, 16, "f32", 0.9, 1.0, False, "fwd", "softplus",
                        1008),
}


def round_to_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    # leave NaN/Inf bit patterns alone (none are drawn here; kept for completeness)
    special = (u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)
    r = np.where(special, (u & np.uint64(0xFFFF0000)).astype(np.uint32), r)
    return r.view(np.float32).reshape(f.shape)


def bf16_bits(a) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable (as uint16)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _softplus(z):
    # input recipe only (the scan takes delta as given): log(1 + e^z), computed stably
    return np.logaddexp(0.0, z)


def make_inputs(w: Workload, *, a_kind: str = "s4d", with_dy: bool | None = None,
                seed: int | None = None) -> dict:
    """Draw the inputs of workload ``w``.

    a_kind: "s4d"    -> A[d, n] = -(n+1)  (the configs' S4D-real initialisation)
            "random" -> A[d, n] = -exp(U(ln 0.5, ln 16))  (no structure across n or d)
    Returns a dict of float32 numpy arrays: x, delta, A, B, C, Dskip (or None), dy (or None),
    plus the scalars beta, alpha and the io string.  beta and alpha are rounded to float32,
    the precision in which the library receives them, so both sides see the same values.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    Bt, L, D, N = w.Bt, w.L, w.D, w.N
    x = rng.standard_normal((Bt, L, D)).astype(np.float32)
    if w.delta_dist == "loguniform":
        delta = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(Bt, L, D))).astype(np.float32)
    elif w.delta_dist == "softplus":
        delta = _softplus(rng.normal(-4.0, 1.0, size=(Bt, L, D))).astype(np.float32)
    else:
        raise ValueError(w.delta_dist)
    B = rng.standard_normal((Bt, L, N)).astype(np.float32)
    C = rng.standard_normal((Bt, L, N)).astype(np.float32)
    if a_kind == "s4d":
        A = np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)).copy()
    elif a_kind == "random":
        A = (-np.exp(rng.uniform(np.log(0.5), np.log(16.0), size=(D, N)))).astype(np.float32)
    else:
        raise ValueError(a_kind)
    Dskip = rng.standard_normal(D).astype(np.float32) if w.dskip else None
    need_dy = (w.direction == "bwd") if with_dy is None else with_dy
    dy = None
    if need_dy:
        rng_dy = np.random.Generator(np.random.PCG64((w.seed if seed is None else seed) + 1000))
        dy = rng_dy.standard_normal((Bt, L, D)).astype(np.float32)
    if w.io == "bf16":
        x, delta, B, C = (round_to_bf16(a) for a in (x, delta, B, C))
        if dy is not None:
            dy = round_to_bf16(dy)
    return dict(x=x, delta=delta, A=A, B=B, C=C, Dskip=Dskip, dy=dy,
                beta=float(np.float32(w.beta)), alpha=float(np.float32(w.alpha)), io=w.io)


def make_state(w: Workload, seed: int, scale: float = 1.0):
    """A seeded (Bt, D, N) float32 pair ~ N(0, scale^2): an initial state (h0, v0), or the
    adjoints (dlast_h, dlast_v) of a final state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = (scale * rng.standard_normal((w.Bt, w.D, w.N))).astype(np.float32)
    b = (scale * rng.standard_normal((w.Bt, w.D, w.N))).astype(np.float32)
    return a, b


def make_fused_extras(w: Workload, seed: int, softplus: bool = True) -> dict:
    """Inputs of the fused op for workload ``w``: a raw delta that replaces ``delta``, the
    per-channel delta bias and the gate z (float32 numpy; raw delta and z bf16-representable
    when w.io == "bf16").

    With softplus the bias is the inverse softplus of a log-uniform step in [1e-3, 1e-1] (the
    usual initialisation of a Mamba layer's step bias) and the raw delta is N(0, 0.5^2)
    projection noise around it, so softplus(delta + bias) covers the same range as the
    workload's own delta.  Without softplus the raw delta is the workload's delta distribution
    and the bias a small positive shift U(0, 0.02), keeping delta + bias positive.
    z ~ N(0, 1), the gate branch's activations.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    Bt, L, D = w.Bt, w.L, w.D
    if softplus:
        dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=D))
        bias = np.log(np.expm1(dt)).astype(np.float32)
        raw = (0.5 * rng.standard_normal((Bt, L, D))).astype(np.float32)
    else:
        bias = rng.uniform(0.0, 0.02, size=D).astype(np.float32)
        raw = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(Bt, L, D))).astype(np.float32)
    z = rng.standard_normal((Bt, L, D)).astype(np.float32)
    if w.io == "bf16":
        raw, z = round_to_bf16(raw), round_to_bf16(z)
    return dict(delta_raw=raw, delta_bias=bias, z=z, softplus=softplus)


def make_step_inputs(w: Workload, seed: int | None = None, softplus: bool = True) -> dict:
    """Inputs of one decode step for workload ``w`` (L is ignored): x, raw delta, z (Bt, D);
    B, C (Bt, N); A, Dskip, delta_bias; states h, v (Bt, D, N) ~ N(0, 1).  Recipes as in
    ``make_inputs``, ``make_fused_extras`` and ``make_state``."""
    s0 = w.seed if seed is None else seed
    w1 = w.replace(L=1)
    inp = make_inputs(w1, a_kind="s4d", seed=s0, with_dy=False)
    ex = make_fused_extras(w1, s0 + 11, softplus=softplus)
    h, v = make_state(w1, s0 + 13)
    return dict(x=inp["x"][:, 0], delta=ex["delta_raw"][:, 0], z=ex["z"][:, 0], B=inp["B"][:, 0],
                C=inp["C"][:, 0], A=inp["A"], Dskip=inp["Dskip"], delta_bias=ex["delta_bias"],
                softplus=softplus, h=h, v=v, beta=inp["beta"], alpha=inp["alpha"], io=w.io)


def make_complex_inputs(w: Workload, *, a_kind: str = "s4d_lin", with_dy: bool | None = None,
                        seed: int | None = None) -> dict:
    """Inputs of the complex scan for workload ``w``: x, delta, dy (Bt, L, D) and Dskip as in
    ``make_inputs``; A (D, N, 2) float32 and B, C (Bt, L, N, 2) as interleaved (re, im) pairs.

    a_kind: "s4d_lin" -> A[d, n] = -1/2 + i pi n
            "random"  -> Re A = -exp(U(ln 0.3, ln 3)), Im A ~ U(-10, 10)  (no structure)
    """
    s = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(s))
    Bt, L, D, N = w.Bt, w.L, w.D, w.N
    x = rng.standard_normal((Bt, L, D)).astype(np.float32)
    if w.delta_dist == "loguniform":
        delta = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(Bt, L, D))).astype(np.float32)
    else:
        delta = _softplus(rng.normal(-4.0, 1.0, size=(Bt, L, D))).astype(np.float32)
    B = (rng.standard_normal((Bt, L, N, 2)) * np.sqrt(0.5)).astype(np.float32)
    C = (rng.standard_normal((Bt, L, N, 2)) * np.sqrt(0.5)).astype(np.float32)
    A = np.empty((D, N, 2), np.float32)
    if a_kind == "s4d_lin":
        A[..., 0] = -0.5
        A[..., 1] = (np.pi * np.arange(N)).astype(np.float32)
    elif a_kind == "random":
        A[..., 0] = -np.exp(rng.uniform(np.log(0.3), np.log(3.0), size=(D, N)))
        A[..., 1] = rng.uniform(-10.0, 10.0, size=(D, N))
    else:
        raise ValueError(a_kind)
    Dskip = rng.standard_normal(D).astype(np.float32) if w.dskip else None
    need_dy = (w.direction == "bwd") if with_dy is None else with_dy
    dy = None
    if need_dy:
        rng_dy = np.random.Generator(np.random.PCG64(s + 1000))
        dy = rng_dy.standard_normal((Bt, L, D)).astype(np.float32)
    if w.io == "bf16":
        x, delta, B, C = (round_to_bf16(a) for a in (x, delta, B, C))
        if dy is not None:
            dy = round_to_bf16(dy)
    return dict(x=x, delta=delta, A=A, B=B, C=C, Dskip=Dskip, dy=dy,
                beta=float(np.float32(w.beta)), alpha=float(np.float32(w.alpha)), io=w.io)


def make_complex_state(w: Workload, seed: int, scale: float = 1.0):
    """A seeded (Bt, D, N, 2) float32 pair of complex states (or adjoints), independent
    N(0, scale^2 / 2) real and imaginary parts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = (w.Bt, w.D, w.N, 2)
    h = (rng.standard_normal(shp) * scale * np.sqrt(0.5)).astype(np.float32)
    v = (rng.standard_normal(shp) * scale * np.sqrt(0.5)).astype(np.float32)
    return h, v
