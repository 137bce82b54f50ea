"""Host checks of bench.py's result check: the CPU-oracle leg compares the
GPU's first rows with the oracle's fp64 rows at the per-element tolerance
of the fp32-accumulated product (Chapter 13 section 13.3, Worked Example
13.3.1).  Here the "GPU rows" are the oracle's own rounded output, with and
without a planted error, so no GPU is needed."""
import numpy as np

import bench
import oracle
import workloads as W


def _rows(p, R):
    c64, cout = oracle.gemm_problem(bench._first_rows(p, R))
    return c64, cout


def test_first_rows_match_full_problem():
    p = W.random_problem(40, 24, 72, "bf16", "bf16", ("normal", 0.0, 1.0), 7, "T", "N")
    full, _ = oracle.gemm_problem(p)
    part, _ = _rows(p, 13)
    assert part.shape == (13, 24)
    assert np.array_equal(part, full[:13])
    # magnitudes: |A||B| bounds |AB| elementwise
    ab, _ = oracle.gemm_problem(bench._first_rows(p, 13, absolute=True))
    assert (ab >= np.abs(part)).all()


def test_check_passes_on_rounded_oracle_output():
    p = W.random_problem(48, 32, 96, "bf16", "bf16", ("normal", 0.0, 1.0), 11)
    c64, cout = _rows(p, 20)
    chk = bench.result_check(p, c64, cout, threads=1)
    assert chk["ok"] and chk["elements_over_tol"] == 0
    assert chk["rows"] == 20 and chk["of_rows"] == 48
    # only the final rounding to bf16 separates them: within half an ulp,
    # far inside the fp32-accumulation bound
    assert chk["max_err_over_tol"] < 0.5
    assert chk["higham_ratio"] <= 1.0


def test_check_flags_a_planted_error():
    p = W.random_problem(32, 16, 64, "f16", "f32", ("uniform", -1.0, 1.0), 3)
    c64, cout = _rows(p, 32)
    bad = cout.copy()
    v = oracle.decode(bad[5:6, 7:8], "f32") + 1.0  # one element off by 1
    bad[5, 7] = oracle.encode(v, "f32")[0, 0]
    chk = bench.result_check(p, c64, bad, threads=1)
    assert not chk["ok"] and chk["elements_over_tol"] == 1
    assert chk["higham_ratio"] > 1.0


def test_check_flags_nan():
    p = W.random_problem(16, 16, 32, "f16", "f16", ("uniform", -1.0, 1.0), 5)
    c64, cout = _rows(p, 16)
    bad = cout.copy()
    bad[0, 0] = 0x7E00  # an f16 NaN
    chk = bench.result_check(p, c64, bad, threads=1)
    assert chk["nan"] and not chk["ok"]


def test_oracle_rows_keeps_the_timed_result():
    p = W.random_problem(24, 8, 16, "f32", "f32", ("normal", 0.0, 1.0), 9)
    keep = []
    R, t = bench._oracle_rows(p, 5.0, 1, keep)
    assert R == p.M and t >= 0 and len(keep) == 1
    full, _ = oracle.gemm_problem(p)
    assert np.array_equal(keep[0], full)
