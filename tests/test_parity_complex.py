"""The complex-valued scan on the GPU (msm_scan_complex_fwd / msm_scan_complex_bwd through the C
ABI) against the fp64 oracle: small shapes with ragged tiles, channel blocks and state groups
for every plan (4, 16, 32 and 64 padded states) and both I/O dtypes, then every output of the
full-size workload, continuation across calls, and the degenerate cases."""
import numpy as np
import pytest

import oracle
import workloads
from conditioning import assert_close_cond, spread
from gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
CW = W["complex"]
SMALL = CW.replace(Bt=2, L=100, D=70)


def cx(a):
    """(..., 2) interleaved float array -> complex128 (None passes through)."""
    if a is None:
        return None
    a = np.asarray(a, np.float64)
    return a[..., 0] + 1j * a[..., 1]


def ri(z):
    """complex array -> (..., 2) float64."""
    return np.stack([np.real(z), np.imag(z)], axis=-1)


def to_dev(inp):
    io = inp["io"]
    g = dict(x=dev(inp["x"], io), delta=dev(inp["delta"], io), A=dev(inp["A"]),
             B=dev(inp["B"], io), C=dev(inp["C"], io),
             Dskip=None if inp["Dskip"] is None else dev(inp["Dskip"]))
    if inp.get("dy") is not None:
        g["dy"] = dev(inp["dy"], io)
    return g


def opt(a):
    return None if a is None else dev(a)


def run_fwd(inp, h0=None, v0=None):
    import torch
    import selective_state_space_msm_amd as msm
    g = to_dev(inp)
    y, lh, lv = msm.msm_scan_complex_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], inp["beta"],
                                         inp["alpha"], g["Dskip"], h0=opt(h0), v0=opt(v0),
                                         return_last_state=True)
    torch.cuda.synchronize()
    return y, lh, lv


def run_bwd(inp, h0=None, v0=None, dlh=None, dlv=None):
    import torch
    import selective_state_space_msm_amd as msm
    g = to_dev(inp)
    out = msm.msm_scan_complex_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"],
                                   inp["beta"], inp["alpha"], g["Dskip"], h0=opt(h0), v0=opt(v0),
                                   dlast_h=opt(dlh), dlast_v=opt(dlv), state_grads=True)
    torch.cuda.synchronize()
    return out


def oracle_fwd(inp, h0=None, v0=None):
    return oracle.complex_fwd(inp["x"], inp["delta"], cx(inp["A"]), cx(inp["B"]), cx(inp["C"]),
                              inp["beta"], inp["alpha"], Dskip=inp["Dskip"], h0=cx(h0), v0=cx(v0))


def oracle_bwd(inp, h0=None, v0=None, dlh=None, dlv=None):
    return oracle.complex_bwd(inp["x"], inp["delta"], cx(inp["A"]), cx(inp["B"]), cx(inp["C"]),
                              inp["dy"], inp["beta"], inp["alpha"], Dskip=inp["Dskip"], h0=cx(h0),
                              v0=cx(v0), dlast_h=cx(dlh), dlast_v=cx(dlv))


def check_fwd(inp, h0=None, v0=None, tag=""):
    io = inp["io"]
    log("complex fwd %s shape=%s N=%d io=%s" % (tag, inp["x"].shape, inp["A"].shape[1], io))
    y, lh, lv = run_fwd(inp, h0, v0)
    oy, olh, olv = oracle_fwd(inp, h0, v0)
    assert_close(host(y), oy, io, "y " + tag)
    assert_close(host(lh), ri(olh), "f32" if io == "f32" else io, "last_h " + tag)
    assert_close(host(lv), ri(olv), "f32" if io == "f32" else io, "last_v " + tag)


def check_bwd(inp, h0=None, v0=None, dlh=None, dlv=None, tag=""):
    io = inp["io"]
    log("complex bwd %s shape=%s N=%d io=%s" % (tag, inp["x"].shape, inp["A"].shape[1], io))
    got = run_bwd(inp, h0, v0, dlh, dlv)
    outs = ("dx", "ddelta", "dA", "dB", "dC", "dh0", "dv0") + (("dDskip",) if inp["Dskip"] is not None
                                                               else ())

    def fn(q):
        o = oracle_bwd(q, h0, v0, dlh, dlv)
        return {k: (o[k] if k in ("dx", "ddelta", "dDskip") else ri(o[k])) for k in outs}

    # gradients held to the bound plus the oracle's own spread under one fp32 rounding of the
    # inputs (tests/conditioning.py)
    want, sp = spread(fn, inp, ("x", "delta", "B", "C", "dy"), outs)
    for k in outs:
        n = assert_close_cond(host(got[k]), want[k], sp[k], io, "%s %s" % (k, tag))
        if n:
            log("  %s %s: %d elements needed the conditioning term" % (k, tag, n))


# ---- small shapes: every plan, ragged tiles / channel blocks / states, both dtypes ----

@pytest.mark.parametrize("beta", [0.9, 0.0])
@pytest.mark.parametrize("N", [4, 16])
def test_fwd_tiny(beta, N):
    w = W["tiny"].replace(beta=beta, N=N)
    check_fwd(workloads.make_complex_inputs(w, seed=301), tag="tiny")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [3, 16, 24, 40, 64])
@pytest.mark.parametrize("a_kind", ["s4d_lin", "random"])
def test_fwd_small_ragged(io, N, a_kind):
    w = SMALL.replace(io=io, N=N, dskip=True, beta=0.8, alpha=0.7)
    inp = workloads.make_complex_inputs(w, a_kind=a_kind, seed=311)
    h0, v0 = workloads.make_complex_state(w, 312)
    check_fwd(inp, h0, v0, tag="small")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [3, 16, 29, 40])
@pytest.mark.parametrize("dskip", [True, False])
def test_bwd_small_ragged(io, N, dskip):
    w = SMALL.replace(io=io, N=N, dskip=dskip, beta=0.8, alpha=0.7, direction="bwd")
    inp = workloads.make_complex_inputs(w, a_kind="random", seed=321)
    h0, v0 = workloads.make_complex_state(w, 322)
    dlh, dlv = workloads.make_complex_state(w, 323)
    check_bwd(inp, h0, v0, dlh, dlv, tag="small")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_64_states_beta0(io):
    # 64 padded states: four launches of 16 states adding their dx / ddelta sums, beta = 0
    w = SMALL.replace(io=io, N=64, dskip=True, beta=0.0, alpha=1.3, direction="bwd")
    inp = workloads.make_complex_inputs(w, a_kind="random", seed=327)
    h0, v0 = workloads.make_complex_state(w, 328)
    dlh, dlv = workloads.make_complex_state(w, 329)
    check_bwd(inp, h0, v0, dlh, dlv, tag="N=64 beta=0")


@pytest.mark.parametrize("beta", [0.9, 0.0])
def test_bwd_tiny_no_state(beta):
    w = W["tiny"].replace(beta=beta, N=4, direction="bwd")
    check_bwd(workloads.make_complex_inputs(w, seed=331), tag="tiny")


# ---- degenerate cases ----

def test_single_step_and_channel():
    w = CW.replace(Bt=1, L=1, D=1, N=1, dskip=True, direction="bwd")
    inp = workloads.make_complex_inputs(w, a_kind="random", seed=341)
    h0, v0 = workloads.make_complex_state(w, 342)
    check_fwd(inp, h0, v0, tag="L=D=N=1")
    check_bwd(inp, h0, v0, *workloads.make_complex_state(w, 343), tag="L=D=N=1")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_many_turns_per_step(io):
    """Rotations of up to about 50 turns per step (|Im A| up to 1000, delta up to 0.3): the
    quarter-turn reduction of the fp32 readout and of the fp64 training path far from the
    first turn, both signs of Im A."""
    w = SMALL.replace(io=io, L=61, N=16, dskip=True, direction="bwd")
    inp = workloads.make_complex_inputs(w, a_kind="random", seed=361)
    rng = np.random.default_rng(362)
    inp["A"] = inp["A"].copy()
    inp["A"][..., 0] = -0.5
    inp["A"][..., 1] = rng.uniform(-1000.0, 1000.0, size=inp["A"].shape[:2]).astype(np.float32)
    inp["delta"] = rng.uniform(0.05, 0.3, size=inp["delta"].shape).astype(np.float32)
    if io == "bf16":
        inp["delta"] = workloads.round_to_bf16(inp["delta"])
    turns = np.abs(inp["delta"][..., None] * inp["A"][None, None, :, :, 1]) / (2 * np.pi)
    assert turns.max() > 40
    h0, v0 = workloads.make_complex_state(w, 363)
    dlh, dlv = workloads.make_complex_state(w, 364)
    check_fwd(inp, h0, v0, tag="many turns")
    check_bwd(inp, h0, v0, dlh, dlv, tag="many turns")


def test_real_inputs_match_real_scan():
    """Zero imaginary parts: the complex kernels give the real scan's outputs (the real
    kernels' results through the real entry point, to the parity tolerance of each)."""
    w = SMALL.replace(N=16, dskip=True, direction="bwd")
    inp = workloads.make_complex_inputs(w, a_kind="random", seed=351)
    for k in ("A", "B", "C"):
        inp[k] = inp[k].copy()
        inp[k][..., 1] = 0.0
    y, _, _ = run_fwd(inp)
    oy, _, _ = oracle.fwd(inp["x"], inp["delta"], inp["A"][..., 0], inp["B"][..., 0],
                          inp["C"][..., 0], inp["beta"], inp["alpha"], Dskip=inp["Dskip"])
    assert_close(host(y), oy, "f32", "y (real inputs)")
    got = run_bwd(inp)
    want = oracle.bwd(inp["x"], inp["delta"], inp["A"][..., 0], inp["B"][..., 0], inp["C"][..., 0],
                      inp["dy"], inp["beta"], inp["alpha"], Dskip=inp["Dskip"])
    for k in ("dx", "ddelta", "dDskip"):
        assert_close(host(got[k]), want[k], "f32", k + " (real inputs)")
    for k in ("dA", "dB", "dC"):
        assert_close(host(got[k])[..., 0], want[k], "f32", k + " (real inputs)")
        assert_close(host(got[k])[..., 1], 0.0 * want[k], "f32", "Im " + k + " (real inputs)")


def test_argument_errors():
    import torch
    import selective_state_space_msm_amd as msm
    w = CW.replace(Bt=1, L=8, D=4, N=4, direction="bwd")
    g = to_dev(workloads.make_complex_inputs(w, seed=361))
    with pytest.raises(ValueError):  # A without its (re, im) dimension
        msm.msm_scan_complex_fwd(g["x"], g["delta"], g["A"][..., 0].contiguous(), g["B"], g["C"],
                                 0.9, 1.0)
    with pytest.raises(msm.MsmError):  # beta out of range
        msm.msm_scan_complex_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], 1.5, 1.0)
    with pytest.raises(msm.MsmError):  # N beyond 64
        A = torch.zeros((4, 65, 2), dtype=torch.float32, device="cuda")
        B = torch.zeros((1, 8, 65, 2), dtype=torch.float32, device="cuda")
        msm.msm_scan_complex_fwd(g["x"], g["delta"], A, B, B, 0.9, 1.0)
    with pytest.raises(msm.MsmError):  # workspace too small
        msm.msm_scan_complex_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"], 0.9, 1.0,
                                 workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))


# ---- the full-size workload (Bt=4, L=2048, D=2048, N=16) ----

@pytest.fixture(scope="module")
def full():
    w = CW.replace(direction="bwd")
    inp = workloads.make_complex_inputs(w)
    return inp, to_dev(inp)


def test_full_size_fwd(full):
    import torch
    import selective_state_space_msm_amd as msm
    inp, g = full
    log("complex fwd full size %s" % (inp["x"].shape,))
    y, lh, lv = msm.msm_scan_complex_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], inp["beta"],
                                         inp["alpha"], g["Dskip"], return_last_state=True)
    torch.cuda.synchronize()
    oy, olh, olv = oracle_fwd(inp)
    assert_close(host(y), oy, "f32", "y")
    assert_close(host(lh), ri(olh), "f32", "last_h")
    assert_close(host(lv), ri(olv), "f32", "last_v")


def test_full_size_bwd(full):
    """Every gradient of every batch row and channel against the oracle on the whole workload.
    ddelta holds Re(conj(gh) A a h) terms a factor |A| (up to 47) above the states, which cancel:
    among its 16.7M elements a few move by about the fp32 bound under one fp32 rounding of the
    inputs, so the bound adds the oracle's own spread (two perturbed runs,
    tests/conditioning.py) and the test logs how many elements needed it."""
    inp, g = full
    log("complex bwd full size %s" % (inp["x"].shape,))
    got = run_bwd(inp)

    def fn(q):
        o = oracle_bwd(q)
        return {k: (ri(v) if k in ("dA", "dB", "dC") else v) for k, v in o.items()
                if k in ("dx", "ddelta", "dA", "dB", "dC")}

    want, sp = spread(fn, inp, ("x", "delta", "B", "C", "dy"), ("dx", "ddelta", "dA", "dB", "dC"),
                      trials=2)
    for k in ("dx", "ddelta", "dA", "dB", "dC"):
        n = assert_close_cond(host(got[k]), want[k], sp[k], "f32", k)
        log("  %s: %d of %d elements needed the conditioning term" % (k, n, want[k].size))


# ---- continuation: a sequence in two calls equals one call ----

def _split(inp, t):
    a = dict(inp, x=inp["x"][:, :t], delta=inp["delta"][:, :t], B=inp["B"][:, :t],
             C=inp["C"][:, :t])
    b = dict(inp, x=inp["x"][:, t:], delta=inp["delta"][:, t:], B=inp["B"][:, t:],
             C=inp["C"][:, t:])
    if inp.get("dy") is not None:
        a["dy"], b["dy"] = inp["dy"][:, :t], inp["dy"][:, t:]
    return a, b


@pytest.mark.parametrize("N", [16, 40])
def test_forward_continuation(N):
    """Scanning the first 1000 steps and continuing from the returned (last_h, last_v) over the
    rest gives the outputs and final states of one scan over all 2048 steps (the oracle's)."""
    w = CW.replace(Bt=2, L=2048, D=96, N=N, dskip=True)
    inp = workloads.make_complex_inputs(w, seed=391)
    oy, olh, olv = oracle_fwd(inp)
    a, b = _split(inp, 1000)
    ya, lha, lva = run_fwd(a)
    yb, lhb, lvb = run_fwd(b, host(lha).astype(np.float32), host(lva).astype(np.float32))
    assert_close(np.concatenate([host(ya), host(yb)], axis=1), oy, "f32", "y (continued)")
    assert_close(host(lhb), ri(olh), "f32", "last_h (continued)")
    assert_close(host(lvb), ri(olv), "f32", "last_v (continued)")


@pytest.mark.parametrize("N", [16, 40])
def test_backward_continuation(N):
    """The backward of a sequence in two parts: the second part first, from the first part's
    final state, then the first with the second's (dh0, dv0) as its terminal adjoints.  Each
    part runs on the GPU and in the oracle from the same inputs: the state at the split is the
    oracle's forward over the first part rounded to fp32, and the first part's terminal adjoints
    are the oracle's (dh0, dv0) of the second part rounded to fp32.  Every output of both parts,
    including the adjoints of the initial state, is held to the fp32 bound plus the oracle's own
    spread under one fp32 rounding of the inputs (ddelta's terms carry |A| up to 47 and cancel;
    tests/conditioning.py)."""
    w = CW.replace(Bt=2, L=2048, D=96, N=N, dskip=False, direction="bwd")
    inp = workloads.make_complex_inputs(w, seed=397)
    a, b = _split(inp, 1000)
    _, lha, lva = oracle_fwd(a)
    h1, v1 = ri(lha).astype(np.float32), ri(lva).astype(np.float32)
    outs = ("dx", "ddelta", "dA", "dB", "dC", "dh0", "dv0")

    def as_ri(o):
        return {k: (o[k] if k in ("dx", "ddelta") else ri(o[k])) for k in outs}

    gb = run_bwd(b, h1, v1)
    ob, spb = spread(lambda q: as_ri(oracle_bwd(q, h1, v1)), b, ("x", "delta", "B", "C", "dy"),
                     outs)
    dlh, dlv = ob["dh0"].astype(np.float32), ob["dv0"].astype(np.float32)
    ga = run_bwd(a, dlh=dlh, dlv=dlv)
    oa, spa = spread(lambda q: as_ri(oracle_bwd(q, dlh=dlh, dlv=dlv)), a,
                     ("x", "delta", "B", "C", "dy"), outs)
    for tag, got, want, sp in (("second part", gb, ob, spb), ("first part", ga, oa, spa)):
        for k in outs:
            n = assert_close_cond(host(got[k]), want[k], sp[k], "f32", "%s %s" % (k, tag))
            if n:
                log("  %s %s: %d elements needed the conditioning term" % (k, tag, n))
