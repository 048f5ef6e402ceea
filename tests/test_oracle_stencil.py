"""Pins for the stencil oracle (CPU only): brute force against an independent
numpy formulation, fixed points, the max principle and an exact mass identity."""

import itertools

import numpy as np
import pytest

import oracle
from cross_core_barrier_amd import inputs


def _numpy_step(x):
    # Edge padding gives the clamped ends; slices give the neighbours.
    p = np.pad(x.astype(np.int64), 1, mode="edge")
    return ((p[:-2] + 2 * p[1:-1] + p[2:]) // 4).astype(np.int32)


def _numpy_iter(x, iters):
    for _ in range(iters):
        x = _numpy_step(x)
    return x


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_bruteforce_small(n):
    for vals in itertools.product(range(4), repeat=n):
        x = np.array(vals, dtype=np.int32)
        for iters in (0, 1, 2, 3):
            np.testing.assert_array_equal(oracle.stencil(x, iters), _numpy_iter(x, iters))


@pytest.mark.parametrize("n,iters", [(1000, 1), (4097, 5), (65536 * 3 + 17, 4)])
def test_random_vs_numpy(n, iters):
    x = inputs.stencil_input(2, n)
    np.testing.assert_array_equal(oracle.stencil(x, iters), _numpy_iter(x, iters))


def test_constant_fixed_point():
    x = np.full(1001, 777, dtype=np.int32)
    np.testing.assert_array_equal(oracle.stencil(x, 7), x)


def test_ramp_interior_fixed_point():
    n = 50
    x = np.arange(n, dtype=np.int32)
    y = oracle.stencil(x, 1)
    np.testing.assert_array_equal(y[:-1], x[:-1])
    assert y[-1] == n - 2  # (n-2 + 2(n-1) + (n-1)) >> 2


def test_max_principle_and_mass_identity():
    x = inputs.stencil_input(2, 10_000)
    y = oracle.stencil(x, 1)
    assert x.min() <= y.min() and y.max() <= x.max()
    # Sum over i of the clamped 3-point sums is exactly 4 * sum(x); the shift
    # drops the low two bits of each, so 4*sum(y) + sum(low bits) == 4*sum(x).
    p = np.pad(x.astype(np.int64), 1, mode="edge")
    s = p[:-2] + 2 * p[1:-1] + p[2:]
    assert 4 * int(y.astype(np.int64).sum()) + int((s & 3).sum()) == 4 * int(x.astype(np.int64).sum())


def test_iteration_parity_of_result_buffer():
    x = inputs.stencil_input(5, 333)
    np.testing.assert_array_equal(oracle.stencil(x, 2), _numpy_step(_numpy_step(x)))
    np.testing.assert_array_equal(oracle.stencil(x, 3), _numpy_iter(x, 3))
