"""Checks that pin the fp64 oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees.  ``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on deliberately broken copies and expects at least one pin to fail for each.

None of these checks calls the oracle's own formula a second time: they compare it with values
printed on the pages (``tests/golden``), closed forms, a materialised matrix form, a library
convolution / IIR filter, finite differences, or exact invariances of the recurrence.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.signal
import scipy.integrate
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def num(v):
    """Golden values are numbers or strings "lnX" meaning log(X)."""
    if isinstance(v, str):
        assert v.startswith("ln")
        return math.log(float(v[2:]))
    return float(v)


def close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    bad = err > atol + rtol * np.abs(b)
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - rtol * np.abs(b)), err.shape) if err.ndim else ()
        raise AssertionError("%s mismatch: got %r want %r (max err %.3e at %s)"
                             % (what, a[i] if err.ndim else a, b[i] if err.ndim else b,
                                float(err.max()), i))


def seq(values):
    """(L,) list -> (1, L, 1) array for a single channel."""
    return np.asarray(values, np.float64).reshape(1, -1, 1)


def seqn(rows):
    """(L, N) nested list -> (1, L, N)."""
    a = np.asarray(rows, np.float64)
    return a.reshape(1, a.shape[0], a.shape[1])


def run_single(orc, deltas, xs, A_row, B_rows, C_rows, beta=0.0, alpha=1.0, plain=False):
    """One batch row, one channel: returns (y (L,), last_h (N,), last_v (N,) or None)."""
    x = seq(xs)
    delta = seq(deltas)
    A = np.asarray(A_row, np.float64).reshape(1, -1)
    B = seqn(B_rows)
    C = seqn(C_rows)
    if plain:
        y, lh = orc.fwd_plain(x, delta, A, B, C)
        return y[0, :, 0], lh[0, 0], None
    y, lh, lv = orc.fwd(x, delta, A, B, C, beta, alpha)
    return y[0, :, 0], lh[0, 0], lv[0, 0]


# ---------------------------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------------------------

def pin_retention_fig2(orc):
    """A = ln 0.5: state 2 retained to 1 (Delta=1) or 0.5 (Delta=2); writes 2 and 4."""
    g = golden("retention_fig2.json")
    A = num(g["A"])
    prev = g["prev_state"]
    for plain in (False, True):
        for case in g["retention"]:
            # step 0 writes the previous state from zero (Delta=1, B=1, x=prev); step 1 writes
            # nothing (B=0, x=0) so only the retained part is left.
            y, lh, _ = run_single(orc, [1.0, case["delta"]], [prev, 0.0], [A], [[1.0], [0.0]],
                                  [[1.0], [1.0]], plain=plain)
            close(y[0], prev, what="primed state")
            close(y[1], case["state"], what="Fig.2 retention")
            close(lh[0], case["state"], what="Fig.2 last state")
        for case in g["write"]["cases"]:
            y, lh, _ = run_single(orc, [case["delta"]], [g["write"]["u"]], [A],
                                  [[g["write"]["B"]]], [[1.0]], plain=plain)
            close(lh[0], case["write"], what="Fig.2 write")


def pin_write_ratio_fig3(orc):
    g = golden("write_ratio_fig3.json")
    for case in g["cases"]:
        y, lh, lv = run_single(orc, [case["delta"]], [g["u"]], [math.log(0.5), math.log(0.8)],
                               [g["B"]], [[1.0, 1.0]])
        close(lh, case["write"], what="Fig.3 write ratio")
        close(lv, case["write"], what="Fig.3 velocity equals the write at the first step")


def pin_two_updates_fig5(orc):
    g = golden("two_updates_fig5.json")
    A = [num(a) for a in g["A"]]
    for plain in (False, True):
        for case in g["cases"]:
            # step 0 writes the start state from zero: Delta=1, x=1, B=start_state
            y, lh, _ = run_single(orc, [1.0, case["delta"]], [1.0, g["u"]], A,
                                  [g["start_state"], case["B"]], [[1.0, 1.0], case["C"]],
                                  plain=plain)
            close(y[0], sum(g["start_state"]), what="Fig.5 primed read")
            close(lh, case["state"], what="Fig.5 %s state" % case["name"])
            close(y[1], case["y"], what="Fig.5 %s read" % case["name"])


def pin_retention_gate_table(orc):
    """Scalar ZOH gate written through the first-order recurrence with B = (1-e^-D)/D."""
    g = golden("retention_gate_table.json")
    A = g["A"]
    for case in g["cases"]:
        dlt = num(case["delta"])
        B1 = (1.0 - math.exp(A * dlt)) / dlt
        close(math.exp(A * dlt), case["old_weight"], what="gate old-state weight")
        close(dlt * B1, case["input_weight"], what="gate input weight")
        y, lh, _ = run_single(orc, [1.0, dlt], [g["prev_state"], g["held_input"]], [A],
                              [[1.0], [B1]], [[1.0], [1.0]])
        close(lh[0], case["state"], what="retention gate table state")


# ---------------------------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------------------------

def _const_run(orc, L, a, beta, w):
    """Constant coefficients: delta=1, A=ln a, B=1, x=w (alpha=1), C=1 -> y_t = h_t."""
    y, lh, lv = run_single(orc, [1.0] * L, [w] * L, [math.log(a)], [[1.0]] * L, [[1.0]] * L,
                           beta=beta, alpha=1.0)
    return y, lv


def closed_form_h(t, a, beta, w):
    if beta == 0.0:
        return w * (1.0 - a ** (t + 1)) / (1.0 - a)
    geo = (1.0 - a ** (t + 1)) / (1.0 - a)
    if abs(a - beta) < 1e-15:
        cross = (t + 1) * beta ** (t + 1)
    else:
        cross = beta * (a ** (t + 1) - beta ** (t + 1)) / (a - beta)
    return w / (1.0 - beta) * (geo - cross)


def pin_closed_form(orc):
    # hand-computed: beta = a = 0.5, w = 2 -> h = 2, 4, 5.5
    y, _ = _const_run(orc, 3, 0.5, 0.5, 2.0)
    close(y, [2.0, 4.0, 5.5], what="hand-computed momentum steps")
    for (a, beta, w) in [(0.8, 0.9, 0.3), (0.95, 0.5, -1.25), (0.6, 0.0, 0.7), (0.7, 0.7, 1.0)]:
        L = 120
        y, _ = _const_run(orc, L, a, beta, w)
        want = [closed_form_h(t, a, beta, w) for t in range(L)]
        close(y, want, rtol=1e-11, atol=1e-13, what="closed form a=%g beta=%g" % (a, beta))
        for Lv in (1, 2, 5, 17):
            _, lv = _const_run(orc, Lv, a, beta, w)
            close(lv[0], w * (1.0 - beta ** Lv) / (1.0 - beta), rtol=1e-12,
                  what="velocity geometric sum")


# ---------------------------------------------------------------------------------------------
# Materialised matrix form (lower-triangular L_ij of the Mamba-2 page, extended to momentum)
# ---------------------------------------------------------------------------------------------

def matrix_form_y(x, delta, A, B, C, beta, alpha, Dskip=None):
    """y_i = sum_{m<=i} sum_n C_{i,n} K_{i,m,n} w_{m,n} + Dskip x_i, with
    K_{i,m,n} = sum_{j=m..i} (prod_{k=j+1..i} a_{k,n}) beta^(j-m) and w = alpha delta B x.
    For beta = 0 only j = m survives: K = prod_{k=m+1..i} a_k (the semiseparable L_ij)."""
    Bt, L, D = x.shape
    N = A.shape[1]
    y = np.zeros((Bt, L, D))
    for b in range(Bt):
        for d in range(D):
            a = np.exp(delta[b, :, d, None] * A[d][None, :])
            w = alpha * delta[b, :, d, None] * B[b] * x[b, :, d, None]
            for i in range(L):
                acc = 0.0
                for m in range(i + 1):
                    K = np.zeros(N)
                    for j in range(m, i + 1):
                        K += np.prod(a[j + 1:i + 1], axis=0) * beta ** (j - m)
                    acc += float(np.sum(C[b, i] * K * w[m]))
                y[b, i, d] = acc + (0.0 if Dskip is None else Dskip[d] * x[b, i, d])
    return y


def semiseparable_y(x, delta, A, B, C):
    """beta = 0 reading straight from L_ij = C_i^T (A_i ... A_{j+1}) Bbar_j, y = L x."""
    Bt, L, D = x.shape
    y = np.zeros((Bt, L, D))
    for b in range(Bt):
        for d in range(D):
            Abar = np.exp(delta[b, :, d, None] * A[d][None, :])        # (L, N)
            Bbar = delta[b, :, d, None] * B[b]                         # (L, N)
            Lmat = np.zeros((L, L))
            for i in range(L):
                for j in range(i + 1):
                    Lmat[i, j] = np.sum(C[b, i] * np.prod(Abar[j + 1:i + 1], axis=0) * Bbar[j])
            y[b, :, d] = Lmat @ x[b, :, d]
    return y


def _rand_problem(rng, Bt, L, D, N, dskip):
    x = rng.standard_normal((Bt, L, D))
    delta = np.exp(rng.uniform(np.log(1e-2), np.log(0.5), size=(Bt, L, D)))
    A = -np.exp(rng.uniform(np.log(0.3), np.log(3.0), size=(D, N)))
    B = rng.standard_normal((Bt, L, N))
    C = rng.standard_normal((Bt, L, N))
    Ds = rng.standard_normal(D) if dskip else None
    return x, delta, A, B, C, Ds


def pin_matrix_form(orc):
    rng = np.random.default_rng(7)
    x, delta, A, B, C, Ds = _rand_problem(rng, 2, 12, 3, 3, True)
    y0, _, _ = orc.fwd(x, delta, A, B, C, 0.0, 1.0)
    close(y0, semiseparable_y(x, delta, A, B, C), rtol=1e-11, atol=1e-12,
          what="beta=0 semiseparable matrix form")
    for beta, alpha in [(0.9, 1.0), (0.5, 0.7), (0.99, 2.0)]:
        y, _, _ = orc.fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds)
        close(y, matrix_form_y(x, delta, A, B, C, beta, alpha, Ds), rtol=1e-11, atol=1e-12,
              what="momentum matrix form beta=%g" % beta)


# ---------------------------------------------------------------------------------------------
# Time-invariant special case: convolution / IIR filter (library routines)
# ---------------------------------------------------------------------------------------------

def pin_convolution(orc):
    rng = np.random.default_rng(11)
    L, N = 50, 3
    xs = rng.standard_normal(L)
    dlt = 0.3
    A = np.array([-0.5, -1.3, -2.2])
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    for beta, alpha in [(0.0, 1.0), (0.8, 0.6)]:
        a = np.exp(dlt * A)
        K = np.zeros(L)
        for l in range(L):
            inner = sum(a ** (l - j) * beta ** j for j in range(l + 1))
            K[l] = np.sum(Cv * alpha * dlt * Bv * inner)
        want = np.convolve(xs, K)[:L]
        y, _, _ = orc.fwd(xs.reshape(1, L, 1), np.full((1, L, 1), dlt), A.reshape(1, N),
                          np.tile(Bv, (1, L, 1)), np.tile(Cv, (1, L, 1)), beta, alpha)
        close(y[0, :, 0], want, rtol=1e-11, atol=1e-12, what="LTI convolution beta=%g" % beta)
    # A = 0 (no decay): beta = 0 gives a running sum; beta > 0 gives an IIR-filtered velocity
    # integrated by the running sum.
    dl = np.exp(rng.uniform(-3, -1, size=L))
    Bs = rng.standard_normal((L, 1))
    wseq = 0.4 * dl * Bs[:, 0] * xs
    for beta in (0.0, 0.7):
        v = scipy.signal.lfilter([1.0], [1.0, -beta], wseq)
        want = np.cumsum(v)
        y, lh, lv = orc.fwd(xs.reshape(1, L, 1), dl.reshape(1, L, 1), np.zeros((1, 1)),
                            Bs.reshape(1, L, 1), np.ones((1, L, 1)), beta, 0.4)
        close(y[0, :, 0], want, rtol=1e-12, atol=1e-13, what="A=0 filter beta=%g" % beta)
        close(lv[0, 0, 0], v[-1], rtol=1e-12, atol=1e-13, what="A=0 last velocity")


# ---------------------------------------------------------------------------------------------
# beta = 0 reduces to the standard recurrence
# ---------------------------------------------------------------------------------------------

def pin_beta0_equivalence(orc):
    rng = np.random.default_rng(3)
    x, delta, A, B, C, Ds = _rand_problem(rng, 2, 40, 5, 4, True)
    y, lh, lv = orc.fwd(x, delta, A, B, C, 0.0, 1.0, Dskip=Ds)
    yp, lhp = orc.fwd_plain(x, delta, A, B, C, Dskip=Ds)
    assert np.array_equal(y, yp), "beta=0, alpha=1 must equal the standard recurrence bitwise"
    assert np.array_equal(lh, lhp)
    # with beta = 0 the velocity is just the last write alpha*delta*B*x
    close(lv, 1.0 * delta[:, -1, :, None] * B[:, -1, None, :] * x[:, -1, :, None], rtol=1e-15,
          what="beta=0 velocity")


# ---------------------------------------------------------------------------------------------
# Structure: linearity, causality, alpha-homogeneity
# ---------------------------------------------------------------------------------------------

def pin_structure(orc):
    rng = np.random.default_rng(5)
    x, delta, A, B, C, Ds = _rand_problem(rng, 2, 30, 4, 3, True)
    x2 = rng.standard_normal(x.shape)
    beta, alpha = 0.85, 1.3
    y1, _, _ = orc.fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds)
    y2, _, _ = orc.fwd(x2, delta, A, B, C, beta, alpha, Dskip=Ds)
    y12, _, _ = orc.fwd(x + x2, delta, A, B, C, beta, alpha, Dskip=Ds)
    close(y12, y1 + y2, rtol=1e-11, atol=1e-12, what="linearity in x")
    # causality: a change at t' leaves every earlier output bitwise unchanged
    tp = 17
    xp = x.copy()
    xp[:, tp, :] += 1.0
    yp, _, _ = orc.fwd(xp, delta, A, B, C, beta, alpha, Dskip=Ds)
    assert np.array_equal(yp[:, :tp], y1[:, :tp]), "causality"
    assert not np.allclose(yp[:, tp:], y1[:, tp:]), "a change must reach later outputs"
    # alpha enters only the write: y(alpha) - Dx = alpha * (y(1) - Dx)
    ya, _, _ = orc.fwd(x, delta, A, B, C, beta, 1.0, Dskip=Ds)
    close(y1 - Ds * x, alpha * (ya - Ds * x), rtol=1e-11, atol=1e-12, what="alpha homogeneity")


# ---------------------------------------------------------------------------------------------
# Backward: central finite differences and scaling identities
# ---------------------------------------------------------------------------------------------

def _loss(orc, p, dy, beta, alpha):
    y, _, _ = orc.fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], beta, alpha, Dskip=p["Dskip"])
    return float(np.sum(dy * y))


def pin_finite_differences(orc, shape=(2, 7, 3, 2), beta=0.9, alpha=0.7, dskip=True, seed=13,
                           max_per_input=None):
    rng = np.random.default_rng(seed)
    Bt, L, D, N = shape
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, dskip)
    dy = rng.standard_normal((Bt, L, D))
    p = dict(x=x, delta=delta, A=A, B=B, C=C, Dskip=Ds)
    g = orc.bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds)
    names = [("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC")]
    if dskip:
        names.append(("Dskip", "dDskip"))
    eps = 1e-6
    for pname, gname in names:
        arr = p[pname]
        idx = list(np.ndindex(arr.shape))
        if max_per_input is not None and len(idx) > max_per_input:
            sel = rng.choice(len(idx), max_per_input, replace=False)
            idx = [idx[i] for i in sel]
        for i in idx:
            orig = arr[i]
            arr[i] = orig + eps
            lp = _loss(orc, p, dy, beta, alpha)
            arr[i] = orig - eps
            lm = _loss(orc, p, dy, beta, alpha)
            arr[i] = orig
            fd = (lp - lm) / (2 * eps)
            an = g[gname][i]
            if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                raise AssertionError("finite difference mismatch for %s%s: fd %.9g analytic %.9g"
                                     % (gname, i, fd, an))


def pin_scaling_identities(orc):
    rng = np.random.default_rng(17)
    x, delta, A, B, C, Ds = _rand_problem(rng, 2, 48, 5, 3, True)
    dy = rng.standard_normal(x.shape)
    beta, alpha = 0.9, 0.8
    y, _, _ = orc.fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds)
    g = orc.bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds)
    lp = float(np.sum(dy * (y - Ds * x)))            # loss without the skip term
    ip = lambda a, b: float(np.sum(a * b))
    close(ip(g["dx"] - Ds * dy, x), lp, rtol=1e-10, what="<dx - D dy, x>")
    close(ip(g["dB"], B), lp, rtol=1e-10, what="<dB, B>")
    close(ip(g["dC"], C), lp, rtol=1e-10, what="<dC, C>")
    close(ip(g["ddelta"], delta) - ip(g["dA"], A), lp, rtol=1e-10, what="<ddelta,delta>-<dA,A>")
    close(ip(g["dx"], x), float(np.sum(dy * y)), rtol=1e-10, what="<dx, x>")
    close(ip(g["dDskip"], Ds), float(np.sum(dy * Ds * x)), rtol=1e-12, what="<dDskip, Dskip>")


def pin_bwd_beta0_alpha0(orc):
    """alpha = 0 writes nothing: the state stays zero, y is the skip term, and every gradient
    except dx (= Dskip * dy) is zero."""
    rng = np.random.default_rng(19)
    x, delta, A, B, C, Ds = _rand_problem(rng, 1, 9, 2, 2, True)
    dy = rng.standard_normal(x.shape)
    y, lh, lv = orc.fwd(x, delta, A, B, C, 0.5, 0.0, Dskip=Ds)
    close(y, Ds * x, rtol=0, atol=0, what="alpha=0 output")
    g = orc.bwd(x, delta, A, B, C, dy, 0.5, 0.0, Dskip=Ds)
    for k in ("ddelta", "dA", "dB", "dC"):
        close(g[k], 0.0, rtol=0, atol=0, what="alpha=0 %s" % k)
    close(g["dx"], Ds * dy, rtol=1e-15, atol=0, what="alpha=0 dx")


# ---------------------------------------------------------------------------------------------
# Initial state and continuation (the README's last_state outputs fed back into the scan)
# ---------------------------------------------------------------------------------------------

def _rand_state(rng, Bt, D, N):
    return rng.standard_normal((Bt, D, N)), rng.standard_normal((Bt, D, N))


def pin_initial_state_filter(orc):
    """Constant coefficients from a non-zero start: v and h are first-order IIR filters whose
    initial conditions are the initial state (scipy.signal.lfilter with zi)."""
    rng = np.random.default_rng(23)
    L, N = 40, 3
    A = np.array([-0.4, -1.1, 0.0])
    dlt = 0.25
    xs = rng.standard_normal(L)
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    h0, v0 = rng.standard_normal((1, 1, N)), rng.standard_normal((1, 1, N))
    for beta, alpha in [(0.0, 1.0), (0.85, 0.7)]:
        want_y = np.zeros(L)
        want_h, want_v = np.zeros(N), np.zeros(N)
        for n in range(N):
            a = math.exp(dlt * A[n])
            w = alpha * dlt * Bv[n] * xs
            v, _ = scipy.signal.lfilter([1.0], [1.0, -beta], w, zi=[beta * v0[0, 0, n]])
            h, _ = scipy.signal.lfilter([1.0], [1.0, -a], v, zi=[a * h0[0, 0, n]])
            want_y += Cv[n] * h
            want_h[n], want_v[n] = h[-1], v[-1]
        y, lh, lv = orc.fwd(xs.reshape(1, L, 1), np.full((1, L, 1), dlt), A.reshape(1, N),
                            np.tile(Bv, (1, L, 1)), np.tile(Cv, (1, L, 1)), beta, alpha,
                            h0=h0, v0=v0)
        close(y[0, :, 0], want_y, rtol=1e-11, atol=1e-12, what="initial-state filter beta=%g" % beta)
        close(lh[0, 0], want_h, rtol=1e-11, atol=1e-12, what="initial-state last h")
        close(lv[0, 0], want_v, rtol=1e-11, atol=1e-12, what="initial-state last v")


def pin_continuation(orc):
    """Scanning L1 steps, then continuing from the state reached, equals scanning L1 + L2 steps
    at once (bitwise: the same operations in the same order)."""
    rng = np.random.default_rng(29)
    Bt, L, D, N, L1 = 2, 23, 3, 4, 9
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    h0, v0 = _rand_state(rng, Bt, D, N)
    beta, alpha = 0.8, 0.9
    y, lh, lv = orc.fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds, h0=h0, v0=v0)
    s1 = (slice(None), slice(0, L1))
    s2 = (slice(None), slice(L1, L))
    y1, lh1, lv1 = orc.fwd(x[s1], delta[s1], A, B[s1], C[s1], beta, alpha, Dskip=Ds, h0=h0, v0=v0)
    y2, lh2, lv2 = orc.fwd(x[s2], delta[s2], A, B[s2], C[s2], beta, alpha, Dskip=Ds, h0=lh1,
                           v0=lv1)
    close(np.concatenate([y1, y2], axis=1), y, rtol=0, atol=0, what="continued y")
    close(lh2, lh, rtol=0, atol=0, what="continued last h")
    close(lv2, lv, rtol=0, atol=0, what="continued last v")


def _state_loss(orc, p, dy, dlh, dlv, beta, alpha):
    y, lh, lv = orc.fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], beta, alpha,
                        Dskip=p["Dskip"], h0=p["h0"], v0=p["v0"])
    return float(np.sum(dy * y) + np.sum(dlh * lh) + np.sum(dlv * lv))


def pin_state_finite_differences(orc):
    """Central differences of sum(dy y) + <dlast_h, last_h> + <dlast_v, last_v> for a scan
    started at a non-zero state: the initial-state adjoints and every input gradient."""
    rng = np.random.default_rng(31)
    Bt, L, D, N = 2, 6, 2, 3
    beta, alpha = 0.7, 0.8
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    h0, v0 = _rand_state(rng, Bt, D, N)
    dy = rng.standard_normal((Bt, L, D))
    dlh, dlv = _rand_state(rng, Bt, D, N)
    p = dict(x=x, delta=delta, A=A, B=B, C=C, Dskip=Ds, h0=h0, v0=v0)
    g = orc.bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds, h0=h0, v0=v0, dlast_h=dlh,
                dlast_v=dlv)
    eps = 1e-6
    for pname, gname in [("h0", "dh0"), ("v0", "dv0"), ("x", "dx"), ("delta", "ddelta"),
                         ("A", "dA"), ("B", "dB"), ("C", "dC"), ("Dskip", "dDskip")]:
        arr = p[pname]
        for i in np.ndindex(arr.shape):
            orig = arr[i]
            arr[i] = orig + eps
            lp = _state_loss(orc, p, dy, dlh, dlv, beta, alpha)
            arr[i] = orig - eps
            lm = _state_loss(orc, p, dy, dlh, dlv, beta, alpha)
            arr[i] = orig
            fd = (lp - lm) / (2 * eps)
            an = g[gname][i]
            if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                raise AssertionError("finite difference mismatch for %s%s: fd %.9g analytic %.9g"
                                     % (gname, i, fd, an))
    # no sequence: the initial-state adjoints are the terminal adjoints
    g0 = orc.bwd(x[:, :0], delta[:, :0], A, B[:, :0], C[:, :0], dy[:, :0], beta, alpha, h0=h0,
                 v0=v0, dlast_h=dlh, dlast_v=dlv)
    close(g0["dh0"], dlh, rtol=0, atol=0, what="L=0 dh0")
    close(g0["dv0"], dlv, rtol=0, atol=0, what="L=0 dv0")


def pin_bwd_continuation(orc):
    """The backward of a scan split in two: the second part's initial-state adjoints are the
    first part's terminal adjoints, and the pieces add up to the backward of the whole."""
    rng = np.random.default_rng(37)
    Bt, L, D, N, L1 = 2, 17, 3, 2, 7
    beta, alpha = 0.9, 0.6
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    h0, v0 = _rand_state(rng, Bt, D, N)
    dy = rng.standard_normal((Bt, L, D))
    g = orc.bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds, h0=h0, v0=v0)
    s1 = (slice(None), slice(0, L1))
    s2 = (slice(None), slice(L1, L))
    _, lh1, lv1 = orc.fwd(x[s1], delta[s1], A, B[s1], C[s1], beta, alpha, h0=h0, v0=v0)
    g2 = orc.bwd(x[s2], delta[s2], A, B[s2], C[s2], dy[s2], beta, alpha, Dskip=Ds, h0=lh1, v0=lv1)
    g1 = orc.bwd(x[s1], delta[s1], A, B[s1], C[s1], dy[s1], beta, alpha, Dskip=Ds, h0=h0, v0=v0,
                 dlast_h=g2["dh0"], dlast_v=g2["dv0"])
    for k in ("dx", "ddelta", "dB", "dC"):
        close(np.concatenate([g1[k], g2[k]], axis=1), g[k], rtol=1e-10, atol=1e-12,
              what="split %s" % k)
    for k in ("dA", "dDskip"):
        close(g1[k] + g2[k], g[k], rtol=1e-10, atol=1e-12, what="split %s" % k)
    close(g1["dh0"], g["dh0"], rtol=1e-10, atol=1e-12, what="split dh0")
    close(g1["dv0"], g["dv0"], rtol=1e-10, atol=1e-12, what="split dv0")



# ---------------------------------------------------------------------------------------------
# The fused op: delta bias + softplus before the scan, the SiLU gate after it (the README's
# selective-scan function arguments; the gate branch of the Mamba block on the Mamba page)
# ---------------------------------------------------------------------------------------------

def pin_fused_delta_transform(orc):
    """softplus(delta + bias) feeds the scan: a raw delta chosen as log(e^c - 1) - bias (numpy's
    expm1 / log) must give the plain scan run on c; without softplus, delta = c - bias must.
    The targets include large values (the overflow-free branch of softplus) and ln 2 = softplus(0)."""
    rng = np.random.default_rng(41)
    Bt, L, D, N = 2, 9, 4, 3
    x, dstar, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    dstar[0, 0, 0] = 30.0                       # softplus far in its linear regime
    dstar[1, 2, 1] = math.log(2.0)              # softplus(0)
    bias = rng.standard_normal(D)
    beta, alpha = 0.8, 0.9
    want, wlh, wlv = orc.fwd(x, dstar, A, B, C, beta, alpha, Dskip=Ds)
    raw = np.log(np.expm1(dstar)) - bias
    raw[1, 2, 1] = -bias[1]                     # exactly zero after the bias
    y, y_raw, lh, lv = orc.fused_fwd(x, raw, A, B, C, beta, alpha, Dskip=Ds, delta_bias=bias,
                                     delta_softplus=True)
    close(y, want, rtol=1e-9, atol=1e-12, what="softplus(delta + bias)")
    close(y_raw, want, rtol=1e-9, atol=1e-12, what="ungated output")
    close(lh, wlh, rtol=1e-9, atol=1e-12, what="softplus last h")
    y, _, lh, _ = orc.fused_fwd(x, dstar - bias, A, B, C, beta, alpha, Dskip=Ds,
                                delta_bias=bias, delta_softplus=False)
    close(y, want, rtol=1e-12, atol=1e-12, what="delta + bias")
    y, _, _, _ = orc.fused_fwd(x, dstar, A, B, C, beta, alpha, Dskip=Ds)
    close(y, want, rtol=0, atol=0, what="no extras")


def pin_fused_gate(orc):
    """y = y_raw * z * logistic(z) (scipy.special.expit), the skip term included in y_raw;
    z = 0 closes the gate."""
    rng = np.random.default_rng(43)
    Bt, L, D, N = 2, 8, 3, 2
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    z = 3.0 * rng.standard_normal((Bt, L, D))
    z[0, 1, :] = 0.0
    z[1, 3, 0] = 40.0
    z[1, 4, 1] = -40.0
    beta, alpha = 0.9, 0.5
    want_raw, _, _ = orc.fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds)
    y, y_raw, _, _ = orc.fused_fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds, z=z)
    close(y_raw, want_raw, rtol=0, atol=0, what="gate: output before the gate")
    close(y, want_raw * z * scipy.special.expit(z), rtol=1e-13, atol=1e-300, what="gated output")
    assert np.all(y[0, 1, :] == 0.0), "z = 0 must close the gate"


def _fused_loss(orc, p, dy, dlh, dlv, beta, alpha, softplus):
    y, _, lh, lv = orc.fused_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], beta, alpha,
                                 Dskip=p["Dskip"], z=p["z"], delta_bias=p["bias"],
                                 delta_softplus=softplus, h0=p["h0"], v0=p["v0"])
    return float(np.sum(dy * y) + np.sum(dlh * lh) + np.sum(dlv * lv))


def pin_fused_finite_differences(orc):
    """Central differences of the fused op's loss for every input: raw delta, its bias, the gate
    z, the scan's inputs and the initial state; with and without softplus."""
    rng = np.random.default_rng(47)
    Bt, L, D, N = 2, 5, 3, 2
    beta, alpha = 0.75, 0.8
    for softplus, with_z in [(True, True), (False, True), (True, False)]:
        x, _, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
        raw = rng.normal(-2.0, 1.0, size=(Bt, L, D)) if softplus else \
            np.exp(rng.uniform(np.log(1e-2), np.log(0.5), size=(Bt, L, D)))
        bias = 0.3 * rng.standard_normal(D)
        z = 2.0 * rng.standard_normal((Bt, L, D)) if with_z else None
        h0, v0 = _rand_state(rng, Bt, D, N)
        dy = rng.standard_normal((Bt, L, D))
        dlh, dlv = _rand_state(rng, Bt, D, N)
        p = dict(x=x, delta=raw, A=A, B=B, C=C, Dskip=Ds, z=z, bias=bias, h0=h0, v0=v0)
        g = orc.fused_bwd(x, raw, A, B, C, dy, beta, alpha, Dskip=Ds, z=z, delta_bias=bias,
                          delta_softplus=softplus, h0=h0, v0=v0, dlast_h=dlh, dlast_v=dlv)
        eps = 1e-6
        names = [("x", "dx"), ("delta", "ddelta"), ("bias", "ddelta_bias"), ("A", "dA"),
                 ("B", "dB"), ("C", "dC"), ("Dskip", "dDskip"), ("h0", "dh0"), ("v0", "dv0")]
        if with_z:
            names.append(("z", "dz"))
        else:
            assert g["dz"] is None
        for pname, gname in names:
            arr = p[pname]
            for i in np.ndindex(arr.shape):
                orig = arr[i]
                arr[i] = orig + eps
                lp = _fused_loss(orc, p, dy, dlh, dlv, beta, alpha, softplus)
                arr[i] = orig - eps
                lm = _fused_loss(orc, p, dy, dlh, dlv, beta, alpha, softplus)
                arr[i] = orig
                fd = (lp - lm) / (2 * eps)
                an = g[gname][i]
                if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                    raise AssertionError("fused finite difference mismatch for %s%s "
                                         "(softplus=%s): fd %.9g analytic %.9g"
                                         % (gname, i, softplus, fd, an))



def pin_step_sequence(orc):
    """L decode steps, each fed the state the previous one returned, reproduce the fused forward
    over the whole sequence (y row by row and the final state), bit for bit: the step is one
    iteration of the same recurrence."""
    rng = np.random.default_rng(53)
    Bt, L, D, N = 2, 7, 3, 4
    beta, alpha = 0.85, 0.7
    x, _, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    raw = rng.normal(-2.0, 1.0, size=(Bt, L, D))
    bias = 0.3 * rng.standard_normal(D)
    z = rng.standard_normal((Bt, L, D))
    h, v = _rand_state(rng, Bt, D, N)
    want, _, wh, wv = orc.fused_fwd(x, raw, A, B, C, beta, alpha, Dskip=Ds, z=z, delta_bias=bias,
                                    delta_softplus=True, h0=h, v0=v)
    for t in range(L):
        y, h, v = orc.step(x[:, t], raw[:, t], A, B[:, t], C[:, t], h, v, beta, alpha, Dskip=Ds,
                           z=z[:, t], delta_bias=bias, delta_softplus=True)
        close(y, want[:, t], rtol=0, atol=0, what="step %d y" % t)
    close(h, wh, rtol=0, atol=0, what="stepped h")
    close(v, wv, rtol=0, atol=0, what="stepped v")
    # one step of a single state from zero with beta = 0, alpha = 1: h = delta B x
    y, h1, v1 = orc.step(np.array([[2.0]]), np.array([[0.5]]), np.array([[-1.0]]),
                         np.array([[3.0]]), np.array([[1.5]]), np.zeros((1, 1, 1)),
                         np.zeros((1, 1, 1)), 0.0, 1.0)
    close(h1[0, 0, 0], 3.0, what="single write")
    close(y[0, 0], 4.5, what="single readout")



# ---------------------------------------------------------------------------------------------
# Zero-order hold: Bbar = (Abar - 1) A^{-1} B (glossary page; complextorch, "The diagonal SSM")
# ---------------------------------------------------------------------------------------------

def pin_zoh_ode(orc):
    """beta = 0, alpha = 1 with the zero-order hold samples the continuous system
    h' = A h + B_t x_t exactly when the input is held over each step: a high-accuracy ODE
    integration (scipy.integrate.solve_ivp, DOP853) over the same piecewise-constant input."""
    rng = np.random.default_rng(59)
    L, N = 7, 3
    A = np.array([-0.7, -2.5, 0.3])
    dts = np.exp(rng.uniform(np.log(0.05), np.log(0.8), size=L))
    xs = rng.standard_normal(L)
    Bm, Cm = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    h0 = rng.standard_normal(N)
    h = h0.copy()
    want = np.zeros(L)
    for t in range(L):
        sol = scipy.integrate.solve_ivp(lambda _s, hh, t=t: A * hh + Bm[t] * xs[t], (0.0, dts[t]), h,
                                        method="DOP853", rtol=1e-13, atol=1e-14)
        h = sol.y[:, -1]
        want[t] = Cm[t] @ h
    y, _, lh, _ = orc.fused_fwd(xs.reshape(1, L, 1), dts.reshape(1, L, 1), A.reshape(1, N),
                                Bm.reshape(1, L, N), Cm.reshape(1, L, N), 0.0, 1.0, zoh=True,
                                h0=h0.reshape(1, 1, N), v0=np.zeros((1, 1, N)))
    close(y[0, :, 0], want, rtol=1e-9, atol=1e-11, what="zero-order hold vs ODE")
    close(lh[0, 0], h, rtol=1e-9, atol=1e-11, what="zero-order hold final state")


def pin_zoh_retention_gate_table(orc):
    """The glossary's retention-gate table with the zero-order hold itself (A = -1, B = 1, a
    state of 1 carried in, x = 3): delta = ln 2 gives 2, delta = ln 4 gives 2.5."""
    g = golden("retention_gate_table.json")
    for case in g["cases"]:
        dt = num(case["delta"])
        _, _, lh, _ = orc.fused_fwd(np.full((1, 1, 1), float(g["held_input"])),
                                    np.full((1, 1, 1), dt), np.full((1, 1), float(g["A"])),
                                    np.ones((1, 1, 1)), np.ones((1, 1, 1)), 0.0, 1.0, zoh=True,
                                    h0=np.full((1, 1, 1), float(g["prev_state"])),
                                    v0=np.zeros((1, 1, 1)))
        close(lh[0, 0, 0], case["state"], rtol=1e-12, atol=1e-12,
              what="zero-order hold table row %s" % case["delta"])


def pin_zoh_limit(orc):
    """A = 0 makes the zero-order hold coefficient delta exactly (the first-order form); a tiny
    A differs from it only at second order."""
    rng = np.random.default_rng(61)
    Bt, L, D, N = 2, 9, 3, 2
    x, delta, _, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    A0 = np.zeros((D, N))
    y0, _, _, _ = orc.fused_fwd(x, delta, A0, B, C, 0.8, 0.9, Dskip=Ds, zoh=True)
    y1, _, _ = orc.fwd(x, delta, A0, B, C, 0.8, 0.9, Dskip=Ds)
    close(y0, y1, rtol=0, atol=0, what="zero-order hold at A = 0")
    At = np.full((D, N), -1e-9)
    y2, _, _, _ = orc.fused_fwd(x, delta, At, B, C, 0.8, 0.9, Dskip=Ds, zoh=True)
    close(y2, y1, rtol=1e-7, atol=1e-9, what="zero-order hold at tiny A")


def pin_zoh_finite_differences(orc):
    """Central differences of the zero-order-hold loss for every input, including steps where
    delta A is small enough for the series form of dg/dA."""
    rng = np.random.default_rng(67)
    Bt, L, D, N = 2, 5, 3, 2
    beta, alpha = 0.7, 0.9
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    A[0, 0] = -3e-4                    # delta A below 1e-3: the series branch
    h0, v0 = _rand_state(rng, Bt, D, N)
    dy = rng.standard_normal((Bt, L, D))
    dlh, dlv = _rand_state(rng, Bt, D, N)
    p = dict(x=x, delta=delta, A=A, B=B, C=C, Dskip=Ds, z=None, bias=None, h0=h0, v0=v0)
    g = orc.fused_bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds, h0=h0, v0=v0, dlast_h=dlh,
                      dlast_v=dlv, zoh=True)

    def loss():
        y, _, lh, lv = orc.fused_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], beta, alpha,
                                     Dskip=p["Dskip"], h0=p["h0"], v0=p["v0"], zoh=True)
        return float(np.sum(dy * y) + np.sum(dlh * lh) + np.sum(dlv * lv))

    eps = 1e-6
    for pname, gname in [("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                         ("Dskip", "dDskip"), ("h0", "dh0"), ("v0", "dv0")]:
        arr = p[pname]
        for i in np.ndindex(arr.shape):
            orig = arr[i]
            arr[i] = orig + eps
            lp = loss()
            arr[i] = orig - eps
            lm = loss()
            arr[i] = orig
            fd = (lp - lm) / (2 * eps)
            an = g[gname][i]
            if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                raise AssertionError("zero-order hold finite difference mismatch for %s%s: "
                                     "fd %.9g analytic %.9g" % (gname, i, fd, an))



# ---------------------------------------------------------------------------------------------
# Complex-valued SSM (README, "Complex Number Support"; complextorch, "The diagonal SSM")
# ---------------------------------------------------------------------------------------------

def _rand_complex_problem(rng, Bt, L, D, N):
    x = rng.standard_normal((Bt, L, D))
    delta = np.exp(rng.uniform(np.log(1e-2), np.log(0.5), size=(Bt, L, D)))
    A = (-np.exp(rng.uniform(np.log(0.3), np.log(3.0), size=(D, N)))
         + 1j * rng.uniform(-4.0, 4.0, size=(D, N)))
    B = rng.standard_normal((Bt, L, N)) + 1j * rng.standard_normal((Bt, L, N))
    C = rng.standard_normal((Bt, L, N)) + 1j * rng.standard_normal((Bt, L, N))
    return x, delta, A, B, C


def pin_complex_real_case(orc):
    """With every imaginary part zero the complex scan is the real one: same y, states and
    gradients, and zero imaginary gradients."""
    rng = np.random.default_rng(71)
    Bt, L, D, N = 2, 9, 3, 4
    x, delta, A, B, C, Ds = _rand_problem(rng, Bt, L, D, N, True)
    h0, v0 = _rand_state(rng, Bt, D, N)
    dy = rng.standard_normal((Bt, L, D))
    dlh, dlv = _rand_state(rng, Bt, D, N)
    beta, alpha = 0.8, 0.7
    y, lh, lv = orc.fwd(x, delta, A, B, C, beta, alpha, Dskip=Ds, h0=h0, v0=v0)
    yc, lhc, lvc = orc.complex_fwd(x, delta, A + 0j, B + 0j, C + 0j, beta, alpha, Dskip=Ds,
                                   h0=h0 + 0j, v0=v0 + 0j)
    close(yc, y, rtol=1e-13, atol=1e-14, what="complex real-case y")
    close(lhc.real, lh, rtol=1e-13, atol=1e-14, what="complex real-case h")
    close(lvc.imag, 0.0 * lv, rtol=0, atol=0, what="complex real-case v imaginary part")
    g = orc.bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds, h0=h0, v0=v0, dlast_h=dlh,
                dlast_v=dlv)
    gc = orc.complex_bwd(x, delta, A + 0j, B + 0j, C + 0j, dy, beta, alpha, Dskip=Ds,
                         h0=h0 + 0j, v0=v0 + 0j, dlast_h=dlh + 0j, dlast_v=dlv + 0j)
    for k in ("dx", "ddelta", "dDskip"):
        close(gc[k], g[k], rtol=1e-12, atol=1e-13, what="complex real-case %s" % k)
    for k in ("dA", "dB", "dC", "dh0", "dv0"):
        close(gc[k].real, g[k], rtol=1e-12, atol=1e-13, what="complex real-case %s" % k)
        close(gc[k].imag, 0.0 * g[k], rtol=0, atol=1e-15, what="complex real-case Im %s" % k)


def pin_complex_convolution(orc):
    """beta = 0 with constant coefficients: y is the real part of the convolution of x with the
    complex kernel K_k = sum_n C_n a_n^k delta B_n (numpy's complex powers and np.convolve), the
    convolution view of the complextorch page's diagonal SSM."""
    rng = np.random.default_rng(73)
    L, N = 30, 4
    A = np.array([-0.5 + 3.1j, -0.9 - 1.2j, -0.2 + 0.4j, -1.5 + 0.0j])
    dlt = 0.3
    xs = rng.standard_normal(L)
    Bv = rng.standard_normal(N) + 1j * rng.standard_normal(N)
    Cv = rng.standard_normal(N) + 1j * rng.standard_normal(N)
    a = np.exp(dlt * A)
    K = np.array([np.sum(Cv * a ** k * dlt * Bv) for k in range(L)])
    want = np.convolve(xs, K.real)[:L]
    y, _, _ = orc.complex_fwd(xs.reshape(1, L, 1), np.full((1, L, 1), dlt), A.reshape(1, N),
                              np.tile(Bv, (1, L, 1)), np.tile(Cv, (1, L, 1)), 0.0, 1.0)
    close(y[0, :, 0], want, rtol=1e-11, atol=1e-12, what="complex convolution")


def pin_complex_conjugate_pairs(orc):
    """States in conjugate pairs (A, B, C and their conjugates) give twice the real part of one
    of them: y(pair) = 2 y(single) - the convention S4D uses to keep half the states."""
    rng = np.random.default_rng(79)
    Bt, L, D, N = 1, 12, 2, 3
    x, delta, A, B, C = _rand_complex_problem(rng, Bt, L, D, N)
    y1, _, _ = orc.complex_fwd(x, delta, A, B, C, 0.6, 1.0)
    y2, _, _ = orc.complex_fwd(x, delta, np.concatenate([A, A.conj()], 1),
                               np.concatenate([B, B.conj()], 2), np.concatenate([C, C.conj()], 2),
                               0.6, 1.0)
    close(y2, 2 * y1, rtol=1e-12, atol=1e-13, what="conjugate pairs")


def pin_complex_finite_differences(orc):
    """Central differences of the complex scan's real loss for every input, real and imaginary
    parts separately, with an initial state and terminal adjoints."""
    rng = np.random.default_rng(83)
    Bt, L, D, N = 2, 5, 2, 2
    beta, alpha = 0.7, 0.9
    x, delta, A, B, C = _rand_complex_problem(rng, Bt, L, D, N)
    Ds = rng.standard_normal(D)
    h0 = rng.standard_normal((Bt, D, N)) + 1j * rng.standard_normal((Bt, D, N))
    v0 = rng.standard_normal((Bt, D, N)) + 1j * rng.standard_normal((Bt, D, N))
    dy = rng.standard_normal((Bt, L, D))
    dlh = rng.standard_normal((Bt, D, N)) + 1j * rng.standard_normal((Bt, D, N))
    dlv = rng.standard_normal((Bt, D, N)) + 1j * rng.standard_normal((Bt, D, N))
    p = dict(x=x, delta=delta, A=A, B=B, C=C, Dskip=Ds, h0=h0, v0=v0)
    g = orc.complex_bwd(x, delta, A, B, C, dy, beta, alpha, Dskip=Ds, h0=h0, v0=v0, dlast_h=dlh,
                        dlast_v=dlv)

    def loss():
        y, lh, lv = orc.complex_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], beta, alpha,
                                    Dskip=p["Dskip"], h0=p["h0"], v0=p["v0"])
        return float(np.sum(dy * y) + np.sum(dlh.real * lh.real + dlh.imag * lh.imag)
                     + np.sum(dlv.real * lv.real + dlv.imag * lv.imag))

    eps = 1e-6
    for pname, gname in [("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                         ("Dskip", "dDskip"), ("h0", "dh0"), ("v0", "dv0")]:
        arr = p[pname]
        parts = [1.0, 1j] if np.iscomplexobj(arr) else [1.0]
        for i in np.ndindex(arr.shape):
            for u in parts:
                orig = arr[i]
                arr[i] = orig + eps * u
                lp = loss()
                arr[i] = orig - eps * u
                lm = loss()
                arr[i] = orig
                fd = (lp - lm) / (2 * eps)
                an = g[gname][i]
                an = an.real if u == 1.0 else an.imag
                if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                    raise AssertionError("complex finite difference mismatch for %s%s %s: fd %.9g "
                                         "analytic %.9g" % (gname, i, "re" if u == 1.0 else "im",
                                                            fd, an))


ALL_PINS = [pin_retention_fig2, pin_write_ratio_fig3, pin_two_updates_fig5,
            pin_retention_gate_table, pin_closed_form, pin_matrix_form, pin_convolution,
            pin_beta0_equivalence, pin_structure, pin_finite_differences,
            pin_scaling_identities, pin_bwd_beta0_alpha0, pin_initial_state_filter,
            pin_continuation, pin_state_finite_differences, pin_bwd_continuation,
            pin_fused_delta_transform, pin_fused_gate, pin_fused_finite_differences,
            pin_step_sequence, pin_zoh_ode, pin_zoh_retention_gate_table, pin_zoh_limit,
            pin_zoh_finite_differences, pin_complex_real_case, pin_complex_convolution,
            pin_complex_conjugate_pairs, pin_complex_finite_differences]
