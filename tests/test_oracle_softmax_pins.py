"""Pins of the CPU oracle's row softmax ("Triton from zero, Lesson 4: Block
Pointers", homework 4) to facts that do not come from the oracle itself:
closed forms, the formula's IEEE special values, invariants, scipy's
independent implementation, and numpy's rounding to the output dtype."""

import numpy as np
import pytest
import scipy.special

import oracle
import workloads as W


def _sm(x64, in_dtype="f32", out_dtype="f32"):
    x64 = np.atleast_2d(np.asarray(x64, dtype=np.float64))
    M, N = x64.shape
    bits = oracle.encode(x64, in_dtype).reshape(-1)
    return oracle.softmax(M, N, bits, 0, N, 1, in_dtype, out_dtype)


def test_closed_forms():
    """exp(ln k) / sum = k / sum; equal entries give 1/N; one entry gives 1."""
    for n in [1, 2, 3, 4, 7, 64]:
        y, _ = _sm([np.log(np.arange(1, n + 1, dtype=np.float64))])
        want = np.arange(1, n + 1) / (n * (n + 1) / 2)
        np.testing.assert_allclose(y[0], want, rtol=2.0 ** -20)  # inputs rounded to fp32
    for n in [1, 5, 1000]:
        y, _ = _sm([[2.5] * n])
        assert (y == 1.0 / n).all()
    y, _ = _sm([[-7.0]])
    assert y[0, 0] == 1.0


def test_max_is_subtracted():
    """Large equal entries do not overflow: without the shift exp(1000) = inf
    and the row would be NaN."""
    y, _ = _sm([[1000.0, 1000.0], [1000.0, 0.0], [-1000.0, -1000.0]])
    assert y.tolist() == [[0.5, 0.5], [1.0, 0.0], [0.5, 0.5]]


def test_special_values():
    """-inf entries give exact zeros; a row of -inf, a +inf entry or a NaN
    makes the row NaN, as the formula's own arithmetic does."""
    inf, nan = np.inf, np.nan
    y, _ = _sm([[0.0, -inf, 0.0, -inf], [-inf, -inf, -inf, -inf], [1.0, inf, 0.0, 2.0],
                [1.0, nan, 0.0, 2.0], [-inf, 3.0, -inf, -inf]])
    assert y[0].tolist() == [0.5, 0.0, 0.5, 0.0]
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isnan(y[3]).all()
    assert y[4].tolist() == [0.0, 1.0, 0.0, 0.0]


def test_rows_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(7)
    for dtype in ["f32", "f16", "bf16"]:
        x = rng.normal(0.0, 4.0, size=(37, 301))
        y, _ = _sm(x, dtype, "f32")
        xr = oracle.decode(oracle.encode(x, dtype), dtype)
        want = scipy.special.softmax(xr, axis=1)
        np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=1e-13)


def test_shift_invariance_and_order():
    """softmax(x + c) == softmax(x) for exactly representable shifts, and
    permuting a row permutes its result."""
    rng = np.random.default_rng(8)
    x = np.round(rng.normal(0.0, 2.0, size=(5, 64)) * 64) / 64
    y0, _ = _sm(x)
    y1, _ = _sm(x + 8.0)
    np.testing.assert_allclose(y0, y1, rtol=1e-13)
    perm = rng.permutation(64)
    y2, _ = _sm(x[:, perm])
    np.testing.assert_allclose(y2, y0[:, perm], rtol=1e-13)


def test_strided_views():
    """A transposed view and a negative row stride read the same rows as a
    contiguous copy."""
    rng = np.random.default_rng(9)
    x = rng.normal(0.0, 2.0, size=(6, 9))
    want, _ = _sm(x)
    xt = oracle.encode(x.T.copy(), "f32").reshape(-1)  # storage 9 x 6
    got, _ = oracle.softmax(6, 9, xt, 0, 1, 6, "f32", "f32")
    assert (got == want).all()
    xf = oracle.encode(x[::-1].copy(), "f32").reshape(-1)  # rows stored in reverse
    got, _ = oracle.softmax(6, 9, xf, 5 * 9, -9, 1, "f32", "f32")
    assert (got == want).all()


@pytest.mark.parametrize("out", ["f16", "f32"])
def test_output_rounding_matches_numpy(out):
    rng = np.random.default_rng(10)
    x = rng.normal(0.0, 5.0, size=(20, 513))
    y, yo = _sm(x, "f32", out)
    npd = {"f16": np.float16, "f32": np.float32}[out]
    assert (oracle.decode(yo, out) == y.astype(npd).astype(np.float64)).all()


def test_bf16_output_is_the_nearest_bf16():
    """The bf16 output is within half a bf16 ulp of the fp64 value (the
    definition of round-to-nearest; values here are normal)."""
    rng = np.random.default_rng(11)
    x = rng.normal(0.0, 5.0, size=(20, 513))
    y, yo = _sm(x, "f32", "bf16")
    got = oracle.decode(yo, "bf16")
    nz = y > 2.0 ** -120
    ulp = 2.0 ** (np.floor(np.log2(y[nz])) - 7)
    assert (np.abs(got[nz] - y[nz]) <= ulp / 2).all()


def test_degenerate_shapes():
    y, yo = oracle.softmax(0, 5, np.zeros(1, np.uint32), 0, 5, 1, "f32", "f32")
    assert y.shape == (0, 5)
    y, yo = oracle.softmax(3, 0, np.zeros(1, np.uint32), 0, 0, 1, "f32", "f32")
    assert y.shape == (3, 0)


def test_workloads_hold_the_stated_mask_fraction():
    p = W.softmax_problem(200, 300, "bf16", "bf16", ("normal", 0.0, 3.0), 5, masked=0.1)
    x = oracle.decode(p.X.logical_bits(), "bf16")
    assert 0.08 < np.isneginf(x).mean() < 0.12 and not np.isnan(x).any()
