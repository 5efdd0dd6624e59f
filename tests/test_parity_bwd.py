"""Backward parity: gradients from the HIP library (through the C ABI) against the fp64
oracle, plus the scaling identities of the backward at full size."""
import numpy as np
import pytest

import oracle
import workloads
from conditioning import assert_close_cond, spread
from gpu_util import (assert_close, host, inputs_to_device, log, run_bwd, run_fwd,
                      sample_channels, sub_problem)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
NAMES = ("dx", "ddelta", "dA", "dB", "dC", "dDskip")


def oracle_bwd(inp):
    return oracle.bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"],
                      inp["beta"], inp["alpha"], Dskip=inp["Dskip"])


def check_full(inp, plan=None, tag=""):
    io = inp["io"]
    log("bwd %s shape=%s io=%s beta=%g alpha=%g plan=%s" % (tag, inp["x"].shape, io, inp["beta"],
                                                           inp["alpha"], plan))
    got = run_bwd(inp, plan=plan)
    # gradients are differences of large per-state terms: each is held to the fp32 bound plus the
    # oracle's own spread under one fp32 rounding of the inputs (tests/conditioning.py), which
    # is far below the bound except for the rare ill-conditioned element
    outs = tuple(k for k in NAMES if not (k == "dDskip" and inp["Dskip"] is None))
    want, sp = spread(oracle_bwd, inp, ("x", "delta", "B", "C", "dy"), outs)
    for k in NAMES:
        if k not in outs:
            assert got[k] is None
            continue
        # dA and dDskip are fp32 outputs in every I/O mode
        n = assert_close_cond(host(got[k]), want[k], sp[k],
                              "f32" if k in ("dA", "dDskip") and io == "f32" else io,
                              "%s %s" % (k, tag))
        if n:
            log("  %s %s: %d elements needed the conditioning term" % (k, tag, n))


@pytest.mark.parametrize("beta", [0.9, 0.0])
@pytest.mark.parametrize("K", [1, 2])
def test_tiny_workload(beta, K):
    inp = workloads.make_inputs(W["tiny"].replace(beta=beta), with_dy=True)
    check_full(inp, plan={"states_per_wave": K}, tag="tiny")


SMALL = W["bwd"].replace(Bt=2, L=100, D=70, N=16)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 4])
@pytest.mark.parametrize("beta,alpha,dskip", [(0.9, 1.0, False), (0.0, 1.0, True),
                                              (0.6, 0.7, True)])
def test_small_ragged(io, K, beta, alpha, dskip):
    inp = workloads.make_inputs(SMALL.replace(io=io, beta=beta, alpha=alpha, dskip=dskip),
                                a_kind="random", seed=31)
    check_full(inp, plan={"states_per_wave": K}, tag="small")


@pytest.mark.parametrize("N", [16, 4])
@pytest.mark.parametrize("K", [1, 2])
@pytest.mark.parametrize("L", [31, 32, 33, 64, 65, 96, 97, 193, 320])
def test_forward_pass_step_boundaries(N, K, L):
    # the backward's forward pass stages 64 rows (two 32-row checkpoint tiles at one state per
    # lane, four 16-row tiles at two) per step when a workgroup has four or more wavefronts:
    # one tile short of, at and one row past a 32-row tile, whole steps, one row past a step,
    # an odd tile count, a ragged last tile in a fourth step, and an odd number of whole steps
    # (4 states: one checkpoint tile per step, the workgroup has one or two wavefronts)
    inp = workloads.make_inputs(SMALL.replace(L=L, D=40, N=N, dskip=True), a_kind="random",
                                seed=90 + L)
    check_full(inp, plan={"states_per_wave": K}, tag="N=%d L=%d" % (N, L))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,dskip", [(33, True), (48, False), (64, True)])
def test_64_states_in_halves(io, N, dskip):
    # 33-64 states by default: two launches of the 32-state plan, the second adding the first's
    # dx / ddelta sums
    inp = workloads.make_inputs(SMALL.replace(io=io, L=53, D=45, N=N, dskip=dskip),
                                a_kind="random", seed=70 + N)
    check_full(inp, tag="N=%d halves" % N)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_64_states_in_halves_beta0(io):
    # the beta = 0 build of both halves (velocity equals the write), with terminal adjoints
    inp = workloads.make_inputs(SMALL.replace(io=io, L=61, D=37, N=64, beta=0.0, dskip=True),
                                a_kind="random", seed=88)
    check_full(inp, tag="N=64 halves beta=0")


@pytest.mark.parametrize("N", [33, 64])
def test_many_states(N):
    # with 4 states per lane N pads to 64 states: the full-wavefront backward (16 wavefronts)
    inp = workloads.make_inputs(SMALL.replace(L=37, D=45, N=N, dskip=True), a_kind="random",
                                seed=54 + N)
    check_full(inp, plan={"states_per_wave": 4}, tag="N=%d" % N)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,dskip", [(17, True), (24, False), (32, True)])
def test_32_states(io, N, dskip):
    # 17-32 states pad to 32: the half-wavefront backward with 8 wavefronts of 2 states
    inp = workloads.make_inputs(SMALL.replace(io=io, L=53, D=45, N=N, dskip=dskip),
                                a_kind="random", seed=60 + N)
    check_full(inp, tag="N=%d" % N)


@pytest.mark.skip(reason="64 padded states in one half-wavefront launch (K=2: 16 wavefronts) "
                         "need 172 KB of LDS, above the 160 KB of an MI355X workgroup, so the "
                         "build has no such instantiation; a build of it once stopped with an "
                         "illegal memory access (uncommitted, no out-of-bounds index found in the "
                         "nearest committed form). 64 states run as two launches of the 32-state "
                         "plan (test_64_states_in_halves) or in the full-wavefront kernel "
                         "(test_many_states)")
@pytest.mark.parametrize("K", [2, 4])
@pytest.mark.parametrize("N", [33, 64])
def test_half_wave_64_states(N, K):
    inp = workloads.make_inputs(SMALL.replace(L=37, D=45, N=N, dskip=True), a_kind="random",
                                seed=50 + N + K)
    check_full(inp, plan={"states_per_wave": K}, tag="N=%d" % N)


@pytest.mark.parametrize("N", [1, 3, 5, 17])
def test_state_counts(N):
    inp = workloads.make_inputs(SMALL.replace(L=40, D=33, N=N, dskip=True), a_kind="random",
                                seed=40 + N)
    check_full(inp, tag="N=%d" % N)


@pytest.mark.parametrize("shape", [(1, 1, 1, 16), (2, 17, 1, 4), (1, 16, 64, 16), (3, 5, 65, 2)])
def test_degenerate_shapes(shape):
    Bt, L, D, N = shape
    inp = workloads.make_inputs(SMALL.replace(Bt=Bt, L=L, D=D, N=N, dskip=True), seed=3)
    check_full(inp, tag="shape=%s" % (shape,))


def test_deterministic_across_runs():
    inp = workloads.make_inputs(SMALL.replace(dskip=True), seed=4)
    g = inputs_to_device(inp)
    a = run_bwd(inp, g)
    b = run_bwd(inp, g)
    for k in NAMES:
        assert np.array_equal(host(a[k]), host(b[k])), k


def test_long_memory_large_delta():
    """delta ~ U[0.4, 1.3] with A in {0, -1e-4, -0.06, -0.11}: states with memories as long as
    the sequence, where dA and ddelta are ill-conditioned (one fp32 rounding of the inputs moves
    the exact dA past the fp32 bound, tests/test_conditioning.py).  Every output against the
    oracle with the bound plus the oracle's own spread under such perturbations."""
    for io in ("f32", "bf16"):
        w = SMALL.replace(io=io, L=37, D=70, N=16)
        inp = workloads.make_inputs(w, a_kind="random", seed=541, with_dy=True)
        cols = np.array([0.0, -1e-4, -0.06, -0.11] * 4, dtype=np.float32)
        inp["A"] = np.ascontiguousarray(np.tile(cols, (w.D, 1)))
        rng = np.random.default_rng(542)
        dl = rng.uniform(0.4, 1.3, size=inp["delta"].shape).astype(np.float32)
        inp["delta"] = dl if io == "f32" else workloads.round_to_bf16(dl)
        got = run_bwd(inp)
        want, sp = spread(oracle_bwd, inp, ("x", "delta", "B", "C", "dy"), NAMES[:5])
        for k in NAMES[:5]:
            tol = "f32" if k == "dA" and io == "f32" else io
            n = assert_close_cond(host(got[k]), want[k], sp[k], tol, "%s %s" % (k, io))
            log("  %s %s: %d of %d elements needed the conditioning term"
                % (k, io, n, want[k].size))


def test_full_size_backward():
    w = W["bwd"]
    log("full-size bwd: drawing inputs")
    inp = workloads.make_inputs(w)
    g = inputs_to_device(inp)
    got = {k: (None if v is None else host(v)) for k, v in run_bwd(inp, g).items()}
    # (1) every output of every batch row and channel against the oracle on the whole workload.
    #     Its steps are in the well-conditioned regime (tests/test_conditioning.py), yet among
    #     16.7M ddelta elements a few cancel far enough that one fp32 rounding of the inputs
    #     moves them by about the bound: the bound adds the oracle's own spread (two perturbed
    #     runs), and the test logs how many elements needed it.
    log("  oracle on the whole workload (and two perturbed runs)")
    want, sp = spread(oracle_bwd, inp, ("x", "delta", "B", "C", "dy"), NAMES[:5], trials=2)
    for k in ("dx", "ddelta", "dA", "dB", "dC"):
        n = assert_close_cond(got[k], want[k], sp[k], w.io, "%s full" % k)
        log("  %s: %d of %d elements needed the conditioning term" % (k, n, want[k].size))
    del want, sp
    # (2) scaling identities on the whole output (fp64 inner products on the host):
    #     <dB,B> = <dC,C> = <dx,x> = <ddelta,delta> - <dA,A> = <dy,y>  (no skip term here)
    y = host(run_fwd(inp, g)[0])
    ip = lambda a, b: float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))
    ref = ip(inp["dy"], y)
    vals = {"<dB,B>": ip(got["dB"], inp["B"]), "<dC,C>": ip(got["dC"], inp["C"]),
            "<dx,x>": ip(got["dx"], inp["x"]),
            "<dd,d>-<dA,A>": ip(got["ddelta"], inp["delta"]) - ip(got["dA"], inp["A"])}
    log("  <dy,y> = %.9g; %s" % (ref, vals))
    for k, v in vals.items():
        assert abs(v - ref) <= 1e-4 * abs(ref) + 1e-2, (k, v, ref)


def test_rows_beyond_32bit_offsets():
    """The backward over one batch row of 2^19 + 37 steps x 1024 fp32 channels (2.1 GB per
    array): dx, ddelta and dA on sampled channels against the oracle, and the scaling identity
    <dB,B> = <dC,C> = <dx,x> = <ddelta,delta> - <dA,A> = <dy,y> over the whole output."""
    import torch
    import selective_state_space_msm_amd as msm
    from test_parity_fwd import _device_inputs
    Bt, L, D, N = 1, (1 << 19) + 37, 1024, 16
    log("backward rows beyond 32-bit offsets: L=%d D=%d fp32" % (L, D))
    x, delta, A, B, C = _device_inputs(Bt, L, D, N, 81)
    dy = torch.randn((Bt, L, D), generator=torch.Generator(device="cuda").manual_seed(82),
                     device="cuda")
    got = msm.msm_scan_bwd(x, delta, A, B, C, dy, 0.9, 1.0)
    torch.cuda.synchronize()
    dsel = sample_channels(D, 6, seed=83)
    sub = dict(x=host(x[:, :, dsel]), delta=host(delta[:, :, dsel]), A=host(A[dsel]), B=host(B),
               C=host(C), dy=host(dy[:, :, dsel]), beta=0.9, alpha=1.0, Dskip=None)
    # over 2^19 steps a few states keep memories of thousands of steps, and ddelta, a difference
    # of per-state terms of order 1e2, is ill-conditioned for a few elements in 1e7: the bound
    # adds the oracle's own spread under one fp32 rounding of the inputs (tests/conditioning.py)
    od, sp = spread(oracle_bwd, sub, ("x", "delta", "B", "C", "dy"), ("dx", "ddelta", "dA"),
                    trials=2)
    for k in ("dx", "ddelta"):
        n = assert_close_cond(host(got[k][:, :, dsel]), od[k], sp[k], "f32", k + " sampled")
        log("  %s: %d elements needed the conditioning term" % (k, n))
    assert_close_cond(host(got["dA"][dsel]), od["dA"], sp["dA"], "f32", "dA sampled")
    y = msm.msm_scan_fwd(x, delta, A, B, C, 0.9, 1.0)
    ip = lambda a, b: float(torch.sum(a.double() * b.double()))
    ref = ip(dy, y)
    vals = {"<dB,B>": ip(got["dB"], B), "<dC,C>": ip(got["dC"], C), "<dx,x>": ip(got["dx"], x),
            "<dd,d>-<dA,A>": ip(got["ddelta"], delta) - ip(got["dA"], A)}
    log("  <dy,y> = %.9g; %s" % (ref, vals))
    for k, v in vals.items():
        assert abs(v - ref) <= 1e-4 * abs(ref) + 1e-2, (k, v, ref)
