"""The conditioning of the backward's outputs, on the CPU: where the plain fp32 bound applies and
where it cannot.

At large steps (delta in [0.4, 1.3]) with A near 0 the states keep a long memory and dA is a
sum of large terms of mixed sign.  There, rounding the inputs once to fp32 moves the exact dA
(the fp64 oracle) by more than atol 1e-4 + rtol 1e-5 |dA|: no implementation that rounds its
arithmetic to fp32 can be held to that bound, and the GPU tests of that regime add the
oracle's own spread under such perturbations (tests/conditioning.py).  An fp32 model of the
backward's arithmetic (fp32 states and write, correctly rounded exp2, fp64 adjoints, as the
kernel computes them) misses the plain bound there but stays within the conditioned one.  At
the workloads' steps (softplus(N(-4, 1)), median 0.018) the spread stays below half the plain
bound, and those tests keep it.
"""
import numpy as np
import pytest

import oracle
import workloads
from conditioning import spread

W = workloads.WORKLOADS
F32 = np.float32
KEYS = ("x", "delta", "B", "C", "dy")


def _bwd(inp):
    return oracle.bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"],
                      inp["beta"], inp["alpha"], Dskip=inp.get("Dskip"))


def long_memory_case(seed, L=37, D=70, Bt=2):
    w = W["bwd"].replace(Bt=Bt, L=L, D=D, N=16)
    inp = workloads.make_inputs(w, a_kind="random", seed=seed, with_dy=True)
    cols = np.array([0.0, -1e-4, -0.06, -0.11] * 4, dtype=np.float32)
    inp["A"] = np.ascontiguousarray(np.tile(cols, (D, 1)))
    rng = np.random.default_rng(seed + 1)
    inp["delta"] = rng.uniform(0.4, 1.3, size=inp["delta"].shape).astype(np.float32)
    return inp


def fp32_backward_model(inp):
    """dA and ddelta as the backward kernel forms them: fp32 write c = delta x, w = c (alpha B),
    fp32 velocity and hidden-state FMAs, a = exp2(fp32(delta * fp32(A log2 e))) correctly
    rounded to fp32, fp64 adjoints gh, gv, and the products leaving the recurrence rounded to
    fp32.  (A model of the kernel's rounding, not a reference for the method.)"""
    x, dl, A, B, C, dy = (inp[k] for k in ("x", "delta", "A", "B", "C", "dy"))
    beta, alpha = np.float64(inp["beta"]), np.float64(inp["alpha"])
    Bt, L, D = x.shape
    N = A.shape[1]
    A2 = (A.astype(F32) * F32(1.4426950408889634)).astype(F32)
    bs = (B.astype(F32) * F32(alpha)).astype(F32)
    dA = np.zeros((D, N))
    ddelta = np.zeros((Bt, L, D))

    def fma32(a, b, c):
        return (np.float64(a) * np.float64(b) + np.float64(c)).astype(F32)

    for b in range(Bt):
        v = np.zeros((D, N), F32)
        h = np.zeros((D, N), F32)
        hs, av = [h], []
        for t in range(L):
            arg = (dl[b, t][:, None].astype(F32) * A2).astype(F32)
            a = np.exp2(np.float64(arg)).astype(F32)
            c = (dl[b, t] * x[b, t]).astype(F32)[:, None]
            w = (c * bs[b, t][None, :]).astype(F32)
            v = fma32(F32(beta), v, w)
            h = fma32(a, h, v)
            hs.append(h)
            av.append(a)
        ghn = np.zeros((D, N))
        gvp = np.zeros((D, N))
        for t in range(L - 1, -1, -1):
            gh = np.float64(C[b, t])[None, :] * np.float64(dy[b, t])[:, None] + ghn
            gv = beta * gvp + gh
            ghn = np.float64(av[t]) * gh
            gvp = gv
            gg = (ghn.astype(F32) * hs[t]).astype(F32)
            dA += np.float64(dl[b, t])[:, None] * np.float64(gg)
            p1 = (np.float64(bs[b, t])[None, :] * np.float64(gv.astype(F32))).sum(1)
            ddelta[b, t] = np.float64(x[b, t]) * p1 + (np.float64(A) * np.float64(gg)).sum(1)
    return {"dA": dA, "ddelta": ddelta}


def plain_bound(want):
    return 1e-4 + 1e-5 * np.abs(want)


@pytest.mark.parametrize("seed", [541, 7, 15])
def test_long_memory_dA_moves_past_the_fp32_bound_under_one_rounding(seed):
    inp = long_memory_case(seed)
    ref, sp = spread(_bwd, inp, KEYS, ("dA", "ddelta"))
    ratio = (sp["dA"] / plain_bound(ref["dA"])).max()
    assert ratio > 1.0, ratio


def test_fp32_model_needs_and_meets_the_conditioned_bound():
    misses = 0
    for seed in (541, 7, 15, 4):
        inp = long_memory_case(seed)
        ref, sp = spread(_bwd, inp, KEYS, ("dA", "ddelta"))
        got = fp32_backward_model(inp)
        for k in ("dA", "ddelta"):
            err = np.abs(got[k] - ref[k])
            assert np.all(err <= plain_bound(ref[k]) + 2.0 * sp[k]), (seed, k)
        misses += int((np.abs(got["dA"] - ref["dA"]) > plain_bound(ref["dA"])).any())
    # the plain bound alone fails for this fp32 arithmetic on some of the seeds
    assert misses >= 1


def test_workload_regime_is_well_conditioned():
    # the backward workload's distributions on a slice: one rounding of the inputs moves every
    # output by less than half the plain bound (ddelta comes closest, at about 0.4: its terms
    # x B gv and A a h gh are large and cancel), so the GPU tests hold that bound there
    w = W["bwd"].replace(Bt=2, L=300, D=40, N=16)
    inp = workloads.make_inputs(w, seed=3, with_dy=True)
    ref, sp = spread(_bwd, inp, KEYS, ("dx", "ddelta", "dA", "dB", "dC"))
    for k, s in sp.items():
        assert (s / plain_bound(ref[k])).max() < 0.5, k


def fp32_forward_model(inp):
    """y as a sequential fp32 scan forms it (fp32 write, velocity and hidden-state FMAs,
    correctly rounded exp2; the readout summed exactly).  A model of fp32 state, not a
    reference for the method."""
    x, dl, A, B, C = inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"]
    beta = F32(inp["beta"])
    Bt, L, D = x.shape
    A2 = (A.astype(F32) * F32(1.4426950408889634)).astype(F32)
    y = np.zeros((Bt, L, D))

    def fma32(a, b, c):
        return (np.float64(a) * np.float64(b) + np.float64(c)).astype(F32)

    for b in range(Bt):
        v = np.zeros(A.shape, F32)
        h = np.zeros(A.shape, F32)
        for t in range(L):
            a = np.exp2(np.float64((dl[b, t][:, None] * A2).astype(F32))).astype(F32)
            w = ((dl[b, t] * x[b, t]).astype(F32)[:, None] * B[b, t][None, :]).astype(F32)
            v = fma32(beta, v, w)
            h = fma32(a, h, v)
            y[b, t] = (np.float64(C[b, t][None, :]) * np.float64(h)).sum(1)
    return y


@pytest.mark.parametrize("beta,within", [(0.995, True), (0.999, False)])
def test_fp32_state_with_velocity_decay_near_one(beta, within):
    """With beta near 1 the velocity sums about 1 / (1 - beta) writes, and each step's fp32
    rounding of v (about 2^-24 |v|, hundreds of times the write) accumulates: over 8000 steps
    with delta = softplus(N(-2, 1)) an fp32 state stays within the bound at beta = 0.995 and
    misses it at beta = 0.999, by far more than the oracle's spread under one fp32 rounding of
    the inputs.  The library's state is fp32, so parity at beta = 0.999 holds over shorter
    sequences only (test_parity_fwd.test_momentum_edge_cases)."""
    w = W["m130m"].replace(Bt=1, L=8000, D=12, N=16, beta=beta)
    inp = workloads.make_inputs(w, a_kind="random", seed=160)
    rng = np.random.default_rng(161)
    inp["delta"] = np.log1p(np.exp(rng.normal(-2.0, 1.0, size=inp["delta"].shape))).astype(F32)
    want = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["beta"],
                      inp["alpha"])[0]
    err = np.abs(fp32_forward_model(inp) - want)
    assert bool(np.all(err <= plain_bound(want))) == within, (err / plain_bound(want)).max()
