"""Helpers for the GPU parity tests: move seeded inputs to the device, run the library through
its C ABI, and compare with the fp64 oracle element by element."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances: |got - want| <= atol + rtol * |want|, elementwise, for every output.
#   fp32 I/O: rtol 1e-5, atol 1e-4.
#   bf16 I/O (fp32 state): rtol 2e-2, with the fp32 atol of 1e-4 kept for values near zero.
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, 1e-4)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(io):
    import torch
    return torch.float32 if io == "f32" else torch.bfloat16


def dev(a, io=None):
    """numpy float32 array (bf16-representable when io == "bf16") -> device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    if io is not None:
        t = t.to(torch_dtype(io))
    return t


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def inputs_to_device(inp):
    io = inp["io"]
    out = dict(x=dev(inp["x"], io), delta=dev(inp["delta"], io), A=dev(inp["A"]),
               B=dev(inp["B"], io), C=dev(inp["C"], io),
               Dskip=None if inp["Dskip"] is None else dev(inp["Dskip"]))
    if inp.get("dy") is not None:
        out["dy"] = dev(inp["dy"], io)
    return out


def run_fwd(inp, d_inp=None, plan=None, beta=None, alpha=None):
    import torch
    import selective_state_space_msm_amd as msm
    g = d_inp if d_inp is not None else inputs_to_device(inp)
    b = inp["beta"] if beta is None else beta
    a = inp["alpha"] if alpha is None else alpha
    y, lh, lv = msm.msm_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], b, a, g["Dskip"],
                                 return_last_state=True, plan=plan)
    torch.cuda.synchronize()
    return y, lh, lv


def run_bwd(inp, d_inp=None, plan=None):
    import torch
    import selective_state_space_msm_amd as msm
    g = d_inp if d_inp is not None else inputs_to_device(inp)
    out = msm.msm_scan_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"], inp["beta"],
                           inp["alpha"], g["Dskip"], plan=plan)
    torch.cuda.synchronize()
    return out


def assert_close(got, want, io, what):
    rtol, atol = TOL[io]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.all(np.isfinite(got)):
        bad = np.argwhere(~np.isfinite(got))[0]
        raise AssertionError("%s: non-finite output at %s" % (what, tuple(bad)))
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    excess = err - lim
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    nbad = int(np.sum(excess > 0))
    if nbad:
        raise AssertionError(
            "%s: %d of %d elements out of tolerance (rtol %g, atol %g); worst at %s: got %.9g "
            "want %.9g (|err| %.3g, allowed %.3g)" % (what, nbad, err.size, rtol, atol,
                                                      tuple(worst), got[worst], want[worst],
                                                      err[worst], lim[worst]))
    return float(err.max()) if err.size else 0.0


def sub_problem(inp, dsel=None, bsel=None):
    """Slice channels (d) and/or batch rows (b) out of a workload's inputs.  Channels are
    independent in the forward, so the oracle on the slice gives those outputs exactly."""
    out = dict(inp)
    if bsel is not None:
        for k in ("x", "delta", "B", "C", "dy", "z"):
            if out.get(k) is not None:
                out[k] = out[k][bsel]
    if dsel is not None:
        for k in ("x", "delta", "dy", "z"):
            if out.get(k) is not None:
                out[k] = out[k][:, :, dsel]
        out["A"] = out["A"][dsel]
        for k in ("Dskip", "delta_bias"):
            if out.get(k) is not None:
                out[k] = out[k][dsel]
    return out


def sample_channels(D, k, seed):
    rng = np.random.default_rng(seed)
    edge = [0, 1, 63, 64, D // 2, D - 2, D - 1]
    pick = rng.choice(D, size=min(k, D), replace=False).tolist()
    return np.array(sorted(set(int(c) for c in edge + pick if 0 <= c < D)))
