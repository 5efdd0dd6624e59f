"""C-ABI checks that need no GPU: the library loads, exports every function msm.h declares,
and rejects bad arguments before anything reaches the device."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_msm_amd as msm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msm.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return msm.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(msm.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", msm.library_path()], check=True,
                         capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code, word in [(0, "MSM_OK"), (1, "INVALID_ARG"), (2, "UNSUPPORTED"), (3, "WORKSPACE"),
                       (4, "LAUNCH"), (99, "UNKNOWN")]:
        assert word in msm.msm_status_string(code)
    assert msm.msm_version() >= 10000


def test_workspace_queries(lib):
    assert msm.msm_scan_fwd_workspace_bytes(0, 10, 10, 4, "f32") == 0
    assert msm.msm_scan_fwd_workspace_bytes(1, 10, 10, 65, "f32") == 0
    assert msm.msm_scan_bwd_workspace_bytes(1, -1, 10, 4, "bf16") == 0
    # the large-batch headline shape needs no chunk summaries; the long sequence does
    plan = msm.msm_scan_fwd_plan(4, 4096, 4096, 16, "bf16", 0.9)
    assert plan["chunks"] == 1
    plan = msm.msm_scan_fwd_plan(1, 65536, 2048, 16, "bf16", 0.95)
    assert plan["chunks"] > 1
    assert msm.msm_scan_fwd_workspace_bytes(1, 65536, 2048, 16, "bf16") > 0
    assert msm.msm_scan_bwd_workspace_bytes(4, 2048, 2048, 16, "f32") > 0


def _fwd(lib, *, x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, y=0x100000,
         lh=None, lv=None, Bt=1, L=8, D=4, N=4, beta=0.5, alpha=1.0, io=0, ws=None, wsb=0,
         plan=None):
    P = ctypes.c_void_p
    args = [P(x), P(delta), P(A), P(B), P(C), P(Dskip), P(y), P(lh), P(lv), Bt, L, D, N,
            ctypes.c_float(beta), ctypes.c_float(alpha), io, P(ws), wsb, None]
    if plan is None:
        return lib.msm_scan_fwd(*args)
    return lib.msm_scan_fwd_with_plan(*args, ctypes.byref(plan))


def test_fwd_argument_validation_never_launches(lib):
    # every call below must be rejected by the host checks (no GPU in this container)
    assert _fwd(lib, x=None) == INVALID
    assert _fwd(lib, y=None) == INVALID
    assert _fwd(lib, Bt=0) == INVALID
    assert _fwd(lib, L=0) == INVALID
    assert _fwd(lib, D=-3) == INVALID
    assert _fwd(lib, N=0) == INVALID
    assert _fwd(lib, N=65) == UNSUPPORTED
    assert _fwd(lib, io=7) == UNSUPPORTED
    assert _fwd(lib, beta=1.0) == INVALID
    assert _fwd(lib, beta=-0.1) == INVALID
    assert _fwd(lib, beta=float("nan")) == INVALID
    assert _fwd(lib, alpha=-1.0) == INVALID
    assert _fwd(lib, alpha=float("inf")) == INVALID
    assert _fwd(lib, alpha=float("nan")) == INVALID
    # output overlapping an input
    assert _fwd(lib, y=0x1000 + 16) == INVALID
    assert _fwd(lib, lh=0x4000) == INVALID
    # chunked shape without the workspace it needs
    need = lib.msm_scan_fwd_workspace_bytes(1, 65536, 64, 16, 0)
    assert need > 0
    big = dict(x=0x10000000, delta=0x20000000, A=0x30000000, B=0x40000000, C=0x50000000,
               y=0x60000000, Bt=1, L=65536, D=64, N=16)
    assert _fwd(lib, **big) == WORKSPACE
    assert _fwd(lib, ws=0x70000000, wsb=need - 1, **big) == WORKSPACE
    # workspace overlapping an input
    assert _fwd(lib, ws=0x10000000, wsb=need, **big) == INVALID
    # explicit plans outside what the build supports
    bad = msm._Plan(3, 1)
    assert _fwd(lib, plan=bad) == UNSUPPORTED
    bad = msm._Plan(4, 1000)
    assert _fwd(lib, plan=bad) == INVALID


def test_bwd_argument_validation_never_launches(lib):
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, dy=0x6000,
                 dx=0x100000, ddelta=0x200000, dA=0x300000, dB=0x400000, dC=0x500000,
                 dDskip=None, Bt=1, L=8, D=4, N=4, beta=0.5, alpha=1.0, io=0, ws=0x900000,
                 wsb=1 << 30)
        plan = kw.pop("plan", None)
        a.update(kw)
        args = [P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]), P(a["Dskip"]),
                P(a["dy"]), P(a["dx"]), P(a["ddelta"]), P(a["dA"]), P(a["dB"]), P(a["dC"]),
                P(a["dDskip"]), a["Bt"], a["L"], a["D"], a["N"], ctypes.c_float(a["beta"]),
                ctypes.c_float(a["alpha"]), a["io"], P(a["ws"]), a["wsb"], None]
        if plan is None:
            return lib.msm_scan_bwd(*args)
        return lib.msm_scan_bwd_with_plan(*args, ctypes.byref(plan))

    assert call(dy=None) == INVALID
    assert call(dA=None) == INVALID
    assert call(Dskip=0x7000) == INVALID          # Dskip without dDskip
    assert call(dDskip=0x700000) == INVALID       # dDskip without Dskip
    assert call(beta=1.5) == INVALID
    assert call(N=100) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(dx=0x6000) == INVALID             # gradient aliasing dy
    assert call(dB=0x100000 + 4) == INVALID       # two outputs overlapping
    # explicit plans: N=4 pads to 4 states, two per wavefront half at most
    assert call(plan=msm._Plan(4, 1)) == UNSUPPORTED
    assert call(plan=msm._Plan(3, 1)) == UNSUPPORTED
    assert call(plan=msm._Plan(2, 2)) == UNSUPPORTED  # the backward is never chunked
    # one tile's checkpoints ([2][N][D] fp32) sit behind one buffer resource of at most
    # 2^31 - 1 bytes: larger shapes are refused up to 32 states instead of losing their high
    # states' checkpoints
    assert call(N=32, D=1 << 23) == UNSUPPORTED
    assert call(N=17, D=(1 << 31) // (8 * 17) + 1) == UNSUPPORTED
    assert call(N=16, D=1 << 24) == UNSUPPORTED
    assert call(N=32, D=(1 << 23) - 64, plan=msm._Plan(2, 1)) == WORKSPACE  # within the limit
    # rows and tiles of a sequence are indexed in 32 bits: L below 2^30
    assert call(L=1 << 30) == UNSUPPORTED
    assert call(L=(1 << 30) - 1, wsb=16) == WORKSPACE
    # its forward pass addresses 64 rows of (Bt, L, D) arrays with 32-bit offsets
    assert call(N=4, D=1 << 23) == UNSUPPORTED
    assert call(N=4, D=1 << 23, io=1, wsb=16) == WORKSPACE


def test_state_entry_points_validation_never_launches(lib):
    P = ctypes.c_void_p

    def fwd(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, h0=None,
                 v0=None, y=0x100000, lh=None, lv=None, Bt=1, L=8, D=4, N=4)
        a.update(kw)
        return lib.msm_scan_fwd_state(
            P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]), P(a["Dskip"]), P(a["h0"]),
            P(a["v0"]), P(a["y"]), P(a["lh"]), P(a["lv"]), a["Bt"], a["L"], a["D"], a["N"],
            ctypes.c_float(0.5), ctypes.c_float(1.0), 0, None, 0, None, None)

    def bwd(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, dy=0x6000,
                 h0=None, v0=None, dlh=None, dlv=None, dx=0x100000, ddelta=0x200000,
                 dA=0x300000, dB=0x400000, dC=0x500000, dDskip=None, dh0=None, dv0=None, Bt=1,
                 L=8, D=4, N=4)
        a.update(kw)
        return lib.msm_scan_bwd_state(
            P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]), P(a["Dskip"]), P(a["dy"]),
            P(a["h0"]), P(a["v0"]), P(a["dlh"]), P(a["dlv"]), P(a["dx"]), P(a["ddelta"]),
            P(a["dA"]), P(a["dB"]), P(a["dC"]), P(a["dDskip"]), P(a["dh0"]), P(a["dv0"]),
            a["Bt"], a["L"], a["D"], a["N"], ctypes.c_float(0.5), ctypes.c_float(1.0), 0,
            P(0x900000), 1 << 30, None, None)

    # a state of 1*4*4 floats = 64 bytes
    assert fwd(h0=0x100000 + 8) == INVALID        # y written over h0
    assert fwd(lh=0x7000, h0=0x7000 + 32) == INVALID  # last_h written over h0 (in place)
    assert fwd(lv=0x7000, v0=0x7000) == INVALID
    assert fwd(lh=0x7000, lv=0x7000 + 32) == INVALID  # the two last states overlapping
    assert fwd(L=0, h0=0x7000) == INVALID
    assert bwd(dh0=0x100000) == INVALID           # dh0 over dx
    assert bwd(dh0=0x8000, dlh=0x8000) == INVALID  # dh0 over its own terminal adjoint
    assert bwd(dv0=0x8000, h0=0x8000 + 60) == INVALID
    assert bwd(dh0=0x8000, dv0=0x8000 + 16) == INVALID
    assert bwd(dx=None) == INVALID


def test_fused_entry_points_validation_never_launches(lib):
    P = ctypes.c_void_p

    def fwd(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, z=None,
                 bias=None, sp=0, zoh=0, h0=None, v0=None, y=0x100000, lh=None, lv=None, N=4)
        a.update(kw)
        return lib.msm_selective_scan_fwd(
            P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]), P(a["Dskip"]), P(a["z"]),
            P(a["bias"]), a["sp"], a["zoh"], P(a["h0"]), P(a["v0"]), P(a["y"]), P(a["lh"]),
            P(a["lv"]), 1,
            8, 4, a["N"], ctypes.c_float(0.5), ctypes.c_float(1.0), 0, None, 0, None, None)

    def bwd(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, z=None,
                 bias=None, sp=0, zoh=0, dy=0x6000, dx=0x100000, ddelta=0x200000, dA=0x300000,
                 dB=0x400000, dC=0x500000, dDskip=None, dz=None, dbias=None, N=4)
        a.update(kw)
        return lib.msm_selective_scan_bwd(
            P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]), P(a["Dskip"]), P(a["z"]),
            P(a["bias"]), a["sp"], a["zoh"], P(a["dy"]), None, None, None, None, P(a["dx"]),
            P(a["ddelta"]), P(a["dA"]), P(a["dB"]), P(a["dC"]), P(a["dDskip"]), P(a["dz"]),
            P(a["dbias"]), None, None, 1, 8, 4, a["N"], ctypes.c_float(0.5),
            ctypes.c_float(1.0), 0, P(0x900000), 1 << 30, None, None)

    # x, y: 1*8*4 floats = 128 bytes; bias: 16 bytes
    assert fwd(sp=2) == INVALID                   # softplus flag is 0 or 1
    assert fwd(z=0x100000 + 64) == INVALID        # the gate overlapping y
    assert fwd(bias=0x100000) == INVALID          # the bias overlapping y
    assert bwd(z=0x7000) == INVALID               # z without dz
    assert bwd(dz=0x700000) == INVALID            # dz without z
    assert bwd(bias=0x7000) == INVALID            # bias without its gradient
    assert bwd(dbias=0x700000) == INVALID
    assert bwd(z=0x7000, dz=0x7000 + 8) == INVALID  # dz over z
    assert bwd(bias=0x7000, dbias=0x100000 + 4) == INVALID  # bias gradient over dx
    assert bwd(sp=-1) == INVALID
    assert fwd(zoh=2) == INVALID
    assert bwd(zoh=-1) == INVALID
    assert bwd(N=65, sp=1) == UNSUPPORTED


def test_step_validation_never_launches(lib):
    P = ctypes.c_void_p

    def step(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, z=None,
                 bias=None, sp=0, zoh=0, h=0x100000, v=0x200000, y=0x300000, Bt=2, D=4, N=4)
        a.update(kw)
        return lib.msm_scan_step(P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]),
                                 P(a["Dskip"]), P(a["z"]), P(a["bias"]), a["sp"], a["zoh"], P(a["h"]),
                                 P(a["v"]), P(a["y"]), a["Bt"], a["D"], a["N"],
                                 ctypes.c_float(0.5), ctypes.c_float(1.0), 0, None)

    # states: 2*4*4 floats = 128 bytes
    assert step(h=None) == INVALID
    assert step(y=None) == INVALID
    assert step(Bt=0) == INVALID
    assert step(N=65) == UNSUPPORTED
    assert step(sp=3) == INVALID
    assert step(zoh=5) == INVALID
    assert step(v=0x100000 + 64) == INVALID        # h and v overlapping
    assert step(h=0x1000) == INVALID               # a state over an input
    assert step(y=0x200000 + 8) == INVALID         # y over a state
    assert step(z=0x100000) == INVALID             # the gate over a state


def test_workspace_covers_the_offset_limit(lib):
    # one batch row of 2^20 fp32 channels over 1024 steps is 4 GiB per array: the forward must
    # cut it into chunks below 2 GiB even when the plan asks for one, and the workspace query
    # must leave room for those chunks' summaries
    assert lib.msm_scan_fwd_workspace_bytes(1, 1024, 1 << 20, 16, 0) > 0
    # a batch row beyond 64 chunks of 2 GiB is rejected
    assert lib.msm_scan_fwd_workspace_bytes(1, 1 << 25, 1 << 20, 16, 0) == 0
    big = dict(x=1 << 44, delta=2 << 44, A=3 << 44, B=4 << 44, C=5 << 44, y=6 << 44, Bt=1,
               L=1 << 25, D=1 << 20, N=16)
    assert _fwd(lib, ws=7 << 44, wsb=1 << 40, **big) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(msm, "_lib", None)
    monkeypatch.setattr(msm, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(msm.MsmLibraryMissing):
        msm.load_library()


def test_bwd_plan_choice():
    # Bt * D / 32 workgroups; two states per lane only once that still gives 2048 wavefronts
    assert msm.msm_scan_bwd_plan(4, 2048, 2048, 16, "f32", 0.9) == {"states_per_wave": 1,
                                                                     "chunks": 1}
    assert msm.msm_scan_bwd_plan(8, 2048, 4096, 16, "f32", 0.9)["states_per_wave"] == 2
    assert msm.msm_scan_bwd_plan(1, 64, 64, 16, "f32", 0.9)["states_per_wave"] == 1
    assert msm.msm_scan_bwd_plan(1, 64, 64, 4, "f32", 0.9)["states_per_wave"] == 1
    # 64 padded states: two halves of the 32-state plan, 2 states per lane (4 selects the
    # full-wavefront backward)
    assert msm.msm_scan_bwd_plan(1, 64, 64, 64, "f32", 0.9)["states_per_wave"] == 2
    assert msm.msm_scan_bwd_plan(1, 64, 1 << 23, 64, "f32", 0.9)["states_per_wave"] == 4
    # the split halves keep the 64-state checkpoint layout: 8 N D must stay below 2^31 bytes
    assert msm.msm_scan_bwd_plan(1, 64, (1 << 22) - 64, 64, "f32", 0.9)["states_per_wave"] == 2
    assert msm.msm_scan_bwd_plan(1, 64, 1 << 22, 64, "f32", 0.9)["states_per_wave"] == 4
    assert msm.msm_scan_bwd_plan(1, 64, (1 << 22) + 64, 48, "f32", 0.9)["states_per_wave"] == 2
    # 17-32 states: the half-wavefront backward with 2 states per lane
    assert msm.msm_scan_bwd_plan(1, 64, 64, 17, "f32", 0.9)["states_per_wave"] == 2
    assert msm.msm_scan_bwd_plan(4, 2048, 2048, 32, "f32", 0.9)["states_per_wave"] == 2
    assert msm.msm_scan_fwd_plan(4, 2048, 2048, 32, "f32", 0.9)["states_per_wave"] == 4


def test_complex_workspace_query(lib):
    align = lambda v: (v + 255) // 256 * 256
    Bt, L, D, N = 4, 2048, 2048, 16
    ncb, NP = (D + 31) // 32, 16
    want = (align(8 * Bt * (L + 1) * N * D) + align(16 * Bt * ncb * L * NP) + align(8 * Bt * D * N)
            + align(4 * Bt * D))
    assert msm.msm_scan_complex_bwd_workspace_bytes(Bt, L, D, N, "f32") == want
    # more than 16 states: launches of 16 states add up dx, ddelta in fp64 ([Bt][L][2][D])
    N2, NP2 = 24, 32
    want2 = (align(8 * Bt * (L + 1) * N2 * D) + align(16 * Bt * ncb * L * NP2)
             + align(8 * Bt * D * N2) + align(4 * Bt * D) + align(16 * Bt * L * D))
    assert msm.msm_scan_complex_bwd_workspace_bytes(Bt, L, D, N2, "f32") == want2
    assert msm.msm_scan_complex_bwd_workspace_bytes(0, L, D, N, "f32") == 0
    assert msm.msm_scan_complex_bwd_workspace_bytes(1, L, D, 65, "f32") == 0
    # 17 history rows of N * D complex fp32 values must stay below 2^31 bytes
    assert msm.msm_scan_complex_bwd_workspace_bytes(1, 16, 1 << 21, 64, "bf16") == 0
    assert msm.msm_scan_complex_bwd_workspace_bytes(1, 16, 1 << 19, 16, "bf16") > 0


def test_complex_validation_never_launches(lib):
    P = ctypes.c_void_p
    F = ctypes.c_float

    def fwd(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, h0=None,
                 v0=None, y=0x100000, lh=None, lv=None, Bt=2, L=8, D=4, N=4, beta=0.5, io=0)
        a.update(kw)
        return lib.msm_scan_complex_fwd(P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]),
                                        P(a["Dskip"]), P(a["h0"]), P(a["v0"]), P(a["y"]), P(a["lh"]),
                                        P(a["lv"]), a["Bt"], a["L"], a["D"], a["N"], F(a["beta"]),
                                        F(1.0), a["io"], None)

    # x, delta, y: 2*8*4 fp32 = 256 bytes; B, C: 2*8*4 complex = 512 bytes
    assert fwd(x=None) == INVALID
    assert fwd(y=None) == INVALID
    assert fwd(Bt=0) == INVALID
    assert fwd(N=65) == UNSUPPORTED
    assert fwd(beta=1.0) == INVALID
    assert fwd(io=7) == UNSUPPORTED
    assert fwd(y=0x1000 + 128) == INVALID          # y over x
    assert fwd(lh=0x4000 + 256) == INVALID         # a final state over B
    assert fwd(D=1 << 21, N=64) == INVALID         # history rows past 32-bit offsets
    assert fwd(L=1 << 30) == UNSUPPORTED           # rows and tiles indexed in 32 bits
    assert fwd(B=0x4000 + 4) == INVALID            # B not aligned to a complex fp32 pair
    assert fwd(C=0x5000 + 2, io=1) == INVALID      # C not aligned to a complex bf16 pair

    def bwd(ws_bytes=1 << 30, **kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, h0=None,
                 v0=None, dy=0x6000, dlh=None, dlv=None, dx=0x100000, dd=0x200000, dA=0x300000,
                 dB=0x400000, dC=0x500000, dDskip=None, dh0=None, dv0=None, ws=0x10000000, Bt=2,
                 L=8, D=4, N=4)
        a.update(kw)
        return lib.msm_scan_complex_bwd(
            P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]), P(a["Dskip"]), P(a["h0"]),
            P(a["v0"]), P(a["dy"]), P(a["dlh"]), P(a["dlv"]), P(a["dx"]), P(a["dd"]), P(a["dA"]),
            P(a["dB"]), P(a["dC"]), P(a["dDskip"]), P(a["dh0"]), P(a["dv0"]), a["Bt"], a["L"],
            a["D"], a["N"], F(0.5), F(1.0), 0, P(a["ws"]), ws_bytes, None)

    assert bwd(dy=None) == INVALID
    assert bwd(dC=None) == INVALID
    assert bwd(Dskip=0x7000) == INVALID            # Dskip without dDskip
    assert bwd(dDskip=0x7000) == INVALID           # dDskip without Dskip
    assert bwd(ws_bytes=16) == WORKSPACE
    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws=0x10000000 + 8) == INVALID       # workspace not 16-byte aligned
    assert bwd(dx=0x2000) == INVALID               # dx over delta
    assert bwd(dB=0x10000000) == INVALID           # dB inside the workspace
    assert bwd(dh0=0x6000) == INVALID              # dh0 over dy


def test_noalloc_forward_validation_never_launches(lib):
    # the allocation-free forward checks its arguments like msm_scan_fwd, and refuses shapes whose
    # chunk summaries exceed its static scratch before touching the device
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, Dskip=None, y=0x100000,
                 lh=None, lv=None, Bt=1, L=8, D=4, N=4, beta=0.5, alpha=1.0, io=0)
        a.update(kw)
        return lib.msm_scan_fwd_noalloc(P(a["x"]), P(a["delta"]), P(a["A"]), P(a["B"]), P(a["C"]),
                                        P(a["Dskip"]), P(a["y"]), P(a["lh"]), P(a["lv"]), a["Bt"],
                                        a["L"], a["D"], a["N"], ctypes.c_float(a["beta"]),
                                        ctypes.c_float(a["alpha"]), a["io"], None)

    assert call(x=None) == INVALID
    assert call(beta=1.0) == INVALID
    assert call(N=65) == UNSUPPORTED
    assert call(y=0x1000 + 16) == INVALID
    # two batch rows of 2^20 steps x 4096 fp32 channels at 64 states: 9 chunks of < 2 GiB per
    # row, whose summaries (about 57 MB) exceed the 32 MiB scratch
    big = dict(x=1 << 44, delta=2 << 44, A=3 << 44, B=4 << 44, C=5 << 44, y=6 << 44, Bt=2,
               L=1 << 20, D=4096, N=64)
    assert call(**big) == WORKSPACE


def test_binding_records_owned_tensors_on_the_launch_stream():
    # tensors the binding allocates are recorded on the stream the call is enqueued on, so the
    # caching allocator cannot reuse their memory while the kernels still run
    calls = []

    class FakeTensor:
        def record_stream(self, s):
            calls.append(s)

    own = msm._Owned("side-stream")
    own.tensors = [FakeTensor(), FakeTensor()]
    own.done()
    assert calls == ["side-stream", "side-stream"]
    calls.clear()
    own = msm._Owned(None)  # the current stream: nothing to record
    own.tensors = [FakeTensor()]
    own.done()
    assert calls == []
