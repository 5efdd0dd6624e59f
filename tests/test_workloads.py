"""Host-side input generation: seeded, exact bf16 rounding, recipe shapes (CPU only)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0, 1e-30, 3.4e38],
                 np.float32),  # exact ties round to even
    ])
    ours = workloads.round_to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = workloads.bf16_bits(ours)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), ours)


def test_inputs_are_seeded_and_shaped():
    w = workloads.WORKLOADS["tiny"]
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for k in ("x", "delta", "A", "B", "C"):
        assert np.array_equal(a[k], b[k])
        assert a[k].dtype == np.float32
    assert a["x"].shape == (1, 64, 4) and a["B"].shape == (1, 64, 4) and a["A"].shape == (4, 4)
    assert np.all(a["delta"] >= 1e-3 * (1 - 1e-6)) and np.all(a["delta"] <= 1e-1 * (1 + 1e-6))
    assert np.array_equal(a["A"][0], -np.arange(1, 5, dtype=np.float32))
    c = workloads.make_inputs(w.replace(Bt=2, L=16, D=8, N=3, io="bf16", delta_dist="softplus",
                                        dskip=True), a_kind="random", with_dy=True)
    for k in ("x", "delta", "B", "C", "dy"):
        assert np.array_equal(workloads.round_to_bf16(c[k]), c[k])
    assert np.all(c["delta"] > 0) and np.all(c["A"] < 0) and c["Dskip"].shape == (8,)
