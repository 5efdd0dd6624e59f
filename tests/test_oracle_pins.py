"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_finite_differences_tiny_workload_shape(orc):
    # the tiny workload's shape (Bt=1, L=64, D=4, N=4), beta = 0.9 and beta = 0, sampled
    for beta in (0.9, 0.0):
        pins.pin_finite_differences(orc, shape=(1, 64, 4, 4), beta=beta, alpha=1.0, dskip=False,
                                    seed=23, max_per_input=12)


def test_thread_count_does_not_change_results(orc):
    rng = np.random.default_rng(29)
    x, delta, A, B, C, Ds = pins._rand_problem(rng, 3, 33, 7, 5, True)
    dy = rng.standard_normal(x.shape)
    y1 = orc.fwd(x, delta, A, B, C, 0.9, 1.0, Dskip=Ds, threads=1)
    y4 = orc.fwd(x, delta, A, B, C, 0.9, 1.0, Dskip=Ds, threads=4)
    for a, b in zip(y1, y4):
        assert np.array_equal(a, b)
    g1 = orc.bwd(x, delta, A, B, C, dy, 0.9, 1.0, Dskip=Ds, threads=1)
    g4 = orc.bwd(x, delta, A, B, C, dy, 0.9, 1.0, Dskip=Ds, threads=3)
    for k in g1:
        assert np.array_equal(g1[k], g4[k]), k


def test_single_step_and_empty_batch(orc):
    # L = 1: h_0 = alpha delta B x, v_0 = the same, y = C.h (+ Dskip x)
    rng = np.random.default_rng(31)
    x, delta, A, B, C, Ds = pins._rand_problem(rng, 2, 1, 3, 4, True)
    y, lh, lv = orc.fwd(x, delta, A, B, C, 0.6, 1.7, Dskip=Ds)
    w = 1.7 * delta[:, 0, :, None] * B[:, 0, None, :] * x[:, 0, :, None]
    pins.close(lh, w, rtol=1e-15, what="L=1 state")
    pins.close(lv, w, rtol=1e-15, what="L=1 velocity")
    pins.close(y[:, 0], np.sum(C[:, 0, None, :] * w, axis=-1) + Ds * x[:, 0], rtol=1e-14,
               what="L=1 output")
    # empty batch: nothing to do, nothing fails
    e = np.zeros((0, 5, 3))
    y, lh, lv = orc.fwd(e, e, np.zeros((3, 2)), np.zeros((0, 5, 2)), np.zeros((0, 5, 2)), 0.9, 1.0)
    assert y.shape == (0, 5, 3)
