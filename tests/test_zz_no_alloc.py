"""The allocation-free forward (msm_scan_fwd_noalloc, static device scratch) against the
workspace forward (msm_scan_fwd) and the fp64 oracle, through the C ABI: two calls in a row on
chunked shapes, the second smaller, so the scratch's reuse across calls is exercised."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, host, inputs_to_device, log

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _noalloc(g, inp, y, lh, lv):
    import torch
    import selective_state_space_msm_amd as msm
    lib = msm.load_library()
    P = ctypes.c_void_p
    ptr = lambda t: None if t is None else P(t.data_ptr())
    Bt, L, D = inp["x"].shape
    N = inp["A"].shape[1]
    st = lib.msm_scan_fwd_noalloc(ptr(g["x"]), ptr(g["delta"]), ptr(g["A"]), ptr(g["B"]),
                                  ptr(g["C"]), ptr(g["Dskip"]), ptr(y), ptr(lh), ptr(lv), Bt, L, D,
                                  N, ctypes.c_float(inp["beta"]), ctypes.c_float(inp["alpha"]),
                                  0 if inp["io"] == "f32" else 1,
                                  P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, msm.msm_status_string(st)
    torch.cuda.synchronize()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_noalloc_matches_workspace_forward(io):
    import torch
    import selective_state_space_msm_amd as msm
    shapes = [dict(Bt=2, L=3000, D=200, N=16), dict(Bt=1, L=2000, D=70, N=13)]
    for i, shp in enumerate(shapes):
        w = W["m130m"].replace(io=io, beta=0.9, alpha=0.8, dskip=True, **shp)
        inp = workloads.make_inputs(w, a_kind="random", seed=900 + i)
        plan = msm.msm_scan_fwd_plan(w.Bt, w.L, w.D, w.N, io, w.beta)
        log("noalloc call %d: %s io=%s plan=%s" % (i, shp, io, plan))
        assert plan["chunks"] > 1  # the scratch holds chunk summaries
        g = inputs_to_device(inp)
        y = torch.empty_like(g["x"])
        lh = torch.empty((w.Bt, w.D, w.N), dtype=torch.float32, device="cuda")
        lv = torch.empty_like(lh)
        _noalloc(g, inp, y, lh, lv)
        ry, rh, rv = msm.msm_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], inp["beta"],
                                      inp["alpha"], g["Dskip"], return_last_state=True)
        torch.cuda.synchronize()
        # the same kernels and plan: identical results
        for a, b, nm in ((y, ry, "y"), (lh, rh, "last_h"), (lv, rv, "last_v")):
            assert np.array_equal(host(a), host(b)), nm
        oy, oh, ov = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["beta"],
                                inp["alpha"], Dskip=inp["Dskip"])
        assert_close(host(y), oy, io, "noalloc y")
        assert_close(host(lh), oh, "f32", "noalloc last_h")
        assert_close(host(lv), ov, "f32", "noalloc last_v")
