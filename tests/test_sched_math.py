"""The split scheduler replaces 64-bit integer divisions by floor(a / b) of one correctly
rounded fp64 division, claiming exactness for 0 <= a < 2^53, b > 0.  Its operands are
below 2^47 (block positions < 2^31 times item counts <= 65535).  Checked here with the
same IEEE division on the host, over random and adversarial operands."""

import numpy as np


def _floordiv_f64(a, b):
    return np.floor(a.astype(np.float64) / b.astype(np.float64)).astype(np.int64)


def test_random_operands_below_2_47():
    rng = np.random.default_rng(7)
    a = rng.integers(0, 1 << 47, size=200_000, dtype=np.int64)
    b = rng.integers(1, 1 << 31, size=200_000, dtype=np.int64)
    assert np.array_equal(_floordiv_f64(a, b), a // b)


def test_quotients_just_below_an_integer():
    # a = k*b - 1: the quotient is k - 1/b, the case a rounding error would push up to k
    rng = np.random.default_rng(8)
    b = rng.integers(2, 1 << 31, size=100_000, dtype=np.int64)
    k = rng.integers(1, (1 << 47) // b, dtype=np.int64)
    a = k * b - 1
    assert np.array_equal(_floordiv_f64(a, b), k - 1)
    assert np.array_equal(_floordiv_f64(a + 1, b), k)


def test_scheduler_shapes():
    # the exact expressions the scheduler evaluates, at the largest sizes it accepts
    T = (1 << 31) - 1
    for n in (1, 7, 256, 65535):
        for pos in (0, 1, T // 3, T - 1):
            a = np.array([(pos + 1) * n + T - 1], dtype=np.int64)
            assert _floordiv_f64(a, np.array([T]))[0] == ((pos + 1) * n + T - 1) // T
        for k in (0, 1, n // 2, n - 1):
            a = np.array([k * T], dtype=np.int64)
            assert _floordiv_f64(a, np.array([n]))[0] == (k * T) // n
