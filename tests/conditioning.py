"""How far the exact result moves when the inputs move by one fp32 rounding.

Some outputs are ill-conditioned: for large steps delta with A near 0 the state has a long
memory, h grows like a sum over many steps, and the parameter gradient dA = sum_t delta a h gh is
a sum of large terms of mixed sign.  There, rounding each input element once to fp32 (a relative
change of at most 2^-24) already moves the exact dA by more than the fp32 bound
rtol 1e-5 / atol 1e-4.  Any implementation whose arithmetic rounds to fp32 (the state, the
write delta*x*B) makes errors of that kind, so it cannot be held to the plain bound there.

`spread` measures that movement on the oracle itself: it perturbs every element of the named
inputs by an independent random relative +-2^-24 and records, element by element, the largest
change of each output over a few trials.  Tests of such regimes then allow
atol + rtol |want| + 2 * spread (assert_close_cond).  The factor 2 is margin over a CPU
emulation of the backward's fp32 arithmetic (correctly rounded exp2, which the hardware exp2 is
to within 0.8 ulp), whose excess over the plain bound stayed below 0.72 spread over 20 seeds.

Only the oracle is called here; no GPU result enters the bound.
"""
from __future__ import annotations

import numpy as np

from gpu_util import TOL

ULP32 = 2.0 ** -24


def perturbed(inp, keys, rng):
    """A copy of inp with every element of inp[k] (k in keys) scaled by 1 +- 2^-24."""
    out = dict(inp)
    for k in keys:
        if inp.get(k) is None:
            continue
        a = np.asarray(inp[k], np.float64)
        out[k] = a * (1.0 + rng.choice([-1.0, 1.0], size=a.shape) * ULP32)
    return out


def spread(fn, inp, keys, outputs, trials=4, seed=11):
    """Element-wise largest |fn(perturbed)[o] - fn(inp)[o]| over `trials` perturbations of the
    inputs named in keys, for each output name o.  fn maps an input dict to an output dict."""
    rng = np.random.default_rng(seed)
    ref = fn(inp)
    sp = {o: np.zeros_like(np.asarray(ref[o], np.float64)) for o in outputs if ref.get(o) is not None}
    for _ in range(trials):
        got = fn(perturbed(inp, keys, rng))
        for o in sp:
            sp[o] = np.maximum(sp[o], np.abs(np.asarray(got[o], np.float64) - ref[o]))
    return ref, sp


def assert_close_cond(got, want, sp, io, what):
    """|got - want| <= atol + rtol |want| + 2 spread, element-wise; reports how many elements
    needed the spread term."""
    rtol, atol = TOL[io]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - want)
    plain = atol + rtol * np.abs(want)
    lim = plain + 2.0 * sp
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d of %d past the conditioned bound; worst at %s: got %.9g want "
                             "%.9g (err %.3g, plain bound %.3g, spread %.3g)"
                             % (what, bad.sum(), bad.size, i, got[i], want[i], err[i], plain[i],
                                sp[i]))
    return int((err > plain).sum())
