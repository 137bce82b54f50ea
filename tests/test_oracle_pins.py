"""Pins for the CPU oracle: checks against what the pages print and what the
mathematics fixes, never against the oracle itself or the HIP path.

Each test names the passage or the fact it pins.  Together they are chosen so
that a plausible slip in the oracle (a dropped term, a swapped index or
stride, a transposed operand, an fp32 accumulator, a wrong rounding) fails at
least one of them; ``test_oracle_mutants.py`` checks that claim by planting
such slips in copies of the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

from conftest import read_golden


def _f(p, out_dtype=None):
    c64, cout = oracle.gemm_problem(p, out_dtype)
    return c64, oracle.decode(cout, out_dtype or p.out_dtype)


# ---------------------------------------------------------------- the pages


def test_worked_2x2():
    """Chapter 13 opening list: the Chapter 11 single-tile product is
    [[19, 22], [43, 50]]."""
    g = read_golden("worked_2x2.txt")
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    C = np.array(g["C"], dtype=np.float64)
    p = W.Problem(2, 2, 2, W.dense(W.to_bits(A, "f32"), "f32"), W.dense(W.to_bits(B, "f32"), "f32"),
                  "f32", "f32")
    c64, cout = _f(p)
    assert np.array_equal(c64, C)
    assert np.array_equal(cout, C)


def test_sentinel_table_correct():
    """Section 13.2, Worked Example 13.2.2: the K-masked result on the
    sentinel-padded views matches the printed 4x4 table (4 decimals)."""
    g = read_golden("sentinel_4x5x4.txt")
    want = np.array(g["CORRECT"], dtype=np.float64)
    c64, cout = _f(W.sentinel_problem(999.0))
    assert np.abs(cout - want).max() < 5e-5 + 1e-6
    assert np.abs(c64 - want).max() < 5e-5 + 1e-6


def test_sentinel_nan_is_never_read():
    """Section 13.2: only k < K may be read.  With NaN in every slot outside the
    views the result must be finite and identical to the 999.0 version."""
    c_999, _ = _f(W.sentinel_problem(999.0))
    c_nan, _ = _f(W.sentinel_problem(float("nan")))
    assert np.isfinite(c_nan).all()
    assert np.array_equal(c_999, c_nan)


def test_sentinel_without_k_mask_matches_printed_buggy_table():
    """Section 13.2, Worked Example 13.2.2: summing k up to 8 over the padded
    buffers adds 3 * 999^2 per element; the printed buggy table agrees to within
    its fp32 summation-order noise (spacing 0.25 near 3e6)."""
    g = read_golden("sentinel_4x5x4.txt")
    want = np.array(g["NO_K_MASK"], dtype=np.float64)
    p = W.sentinel_problem(999.0)
    # the same storage read with K = 8: the padded columns/rows become real
    c64, _ = oracle.gemm(4, 4, 8, p.A.bits, 0, 8, 1, p.B.bits, 0, 4, 1, "f32", "f32")
    correct, _ = _f(p)
    assert np.allclose(c64 - correct, 3 * 999.0 ** 2, atol=1e-6)
    assert np.abs(c64 - want).max() <= 1.0


def test_accumulation_seed0_fp32acc():
    """Section 13.3, Worked Example 13.3.1: fp32 accumulation with a single
    fp16 cast at the store is 9.737179152580211e-05 from the fp64 truth."""
    g = read_golden("accumulation_seed0.txt")
    want = float(g["_"][4][1])
    p = W.seed0_fp16_problem()
    c64, c16 = _f(p)  # out dtype fp16: one rounding of the fp64 sum
    assert float(np.abs(c16 - c64).max()) == want


def test_accumulation_seed0_fp16acc():
    """Section 13.3, Worked Example 13.3.1: the fp16 accumulator over 128
    K-chunks of 8 is 0.001974425897060428 from the fp64 truth."""
    g = read_golden("accumulation_seed0.txt")
    bk = int(g["_"][3][1])
    want = float(g["_"][5][1])
    p = W.seed0_fp16_problem()
    c64, _ = _f(p)
    c16 = oracle.decode(oracle.gemm_fp16acc_problem(p, bk), "f16")
    assert float(np.abs(c16 - c64).max()) == want
    # BLOCK_K matters: a different chunking gives a different error
    c16_4 = oracle.decode(oracle.gemm_fp16acc_problem(p, 4), "f16")
    assert float(np.abs(c16_4 - c64).max()) != want


@pytest.mark.parametrize("M,K,N", [(8, 8, 8), (5, 7, 6)])
def test_small_fp32_against_torch_within_printed_diff(M, K, N):
    """Worked Examples 13.1.1 / 13.2.1: the tiled kernel and torch's matmul
    differ by at most the printed max abs diff (one fp32 spacing at the
    largest entry).  The oracle's single rounding must sit at least that close
    to torch's fp32 matmul."""
    rows = read_golden("tiled_small_fp32.txt")["_"]
    row = [r for r in rows if (int(r[0]), int(r[1]), int(r[2])) == (M, K, N)][0]
    bound = float(row[6])
    p = W.arange_problem(M, K, N, scale=0.1)
    _, cout = _f(p)
    a = torch.arange(M * K, dtype=torch.float32).reshape(M, K) * 0.1
    b = torch.arange(K * N, dtype=torch.float32).reshape(K, N) * 0.1
    ref = (a @ b).double().numpy()
    assert np.abs(cout - ref).max() <= bound


# ------------------------------------------------------------ closed forms


def _arange_closed_form(M, K, N):
    """sum_k (i*K + k) * (k*N + j) = K*N*S1*i + K^2*i*j + N*S2 + S1*j with
    S1 = sum k = K(K-1)/2 and S2 = sum k^2 = (K-1)K(2K-1)/6."""
    i = np.arange(M, dtype=object)[:, None]
    j = np.arange(N, dtype=object)[None, :]
    S1 = K * (K - 1) // 2
    S2 = (K - 1) * K * (2 * K - 1) // 6
    return K * N * S1 * i + K * K * i * j + N * S2 + S1 * j


@pytest.mark.parametrize("M,K,N", [(8, 8, 8), (5, 7, 6), (4, 5, 4), (33, 17, 65), (3, 129, 2)])
def test_arange_closed_form_exact(M, K, N):
    """Integer arange inputs (the pages' operands without the 0.1 factor): the
    fp64 sum is exact and equals the closed form; the fp32 output is its
    correctly rounded value."""
    p = W.arange_problem(M, K, N, scale=1.0)
    c64, cout = _f(p)
    want = _arange_closed_form(M, K, N)
    assert np.array_equal(c64.astype(np.int64), want.astype(np.int64))
    assert np.array_equal(c64, want.astype(np.float64))
    assert np.array_equal(cout, want.astype(np.float64).astype(np.float32).astype(np.float64))


def test_scaled_arange_is_hundredth_of_closed_form():
    """The pages' 0.1*arange operands give C close to closed_form/100 (the
    operands are fp32-rounded multiples of 0.1)."""
    for (M, K, N) in [(8, 8, 8), (5, 7, 6), (4, 5, 4)]:
        c64, _ = _f(W.arange_problem(M, K, N, scale=0.1))
        want = _arange_closed_form(M, K, N).astype(np.float64) / 100.0
        assert np.abs(c64 - want).max() <= 1e-6 * max(1.0, np.abs(want).max())


# -------------------------------------------------------------- invariants


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_identity_and_zero(in_dtype, out_dtype):
    """A.I = A, I.B = B, A.0 = 0, and K = 0 gives an all-zero C."""
    rng = np.random.default_rng(7)
    M, K, N = 6, 9, 5
    # integers small enough to be exact in every dtype
    a = rng.integers(-16, 17, size=(M, K)).astype(np.float64)
    b = rng.integers(-16, 17, size=(K, N)).astype(np.float64)
    A = W.dense(W.to_bits(a, in_dtype), in_dtype)
    B = W.dense(W.to_bits(b, in_dtype), in_dtype)
    IK = W.dense(W.to_bits(np.eye(K), in_dtype), in_dtype)
    IM = W.dense(W.to_bits(np.eye(M), in_dtype), in_dtype)
    Z = W.dense(W.to_bits(np.zeros((K, N)), in_dtype), in_dtype)
    _, c = _f(W.Problem(M, K, K, A, IK, in_dtype, out_dtype))
    assert np.array_equal(c, a)
    _, c = _f(W.Problem(M, N, M, IM, W.dense(W.to_bits(b[:M], in_dtype), in_dtype), in_dtype,
                        out_dtype))
    assert np.array_equal(c, b[:M])
    c64, c = _f(W.Problem(M, N, K, A, Z, in_dtype, out_dtype))
    assert not c64.any() and not c.any()
    c64, c = oracle.gemm(M, N, 0, A.bits, 0, K, 1, B.bits, 0, N, 1, in_dtype, out_dtype)
    assert not c64.any() and not c.any()


def test_empty_shapes():
    a = np.zeros(4, dtype=np.uint32)
    c64, c = oracle.gemm(0, 3, 2, a, 0, 2, 1, a, 0, 3, 1, "f32", "f32")
    assert c64.shape == (0, 3)
    c64, c = oracle.gemm(3, 0, 2, a, 0, 2, 1, a, 0, 0, 1, "f32", "f32")
    assert c64.shape == (3, 0)


# ---------------------------------------------------- exact integer results


def _numpy_round(x64, dtype):
    """Reference rounding of exact values through library conversions."""
    if dtype == "f32":
        return x64.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x64.astype(np.float16).astype(np.float64)
    t = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16)  # exact f32 values here
    return t.double().numpy()


def _view(bits2d, layout, rng, dtype):
    """Materialise a logical matrix under one of several storage layouts."""
    R, C = bits2d.shape
    if layout == "N":
        return W.dense(bits2d, dtype)
    if layout == "T":
        return W.transposed_view(bits2d.T.copy(), dtype)
    if layout == "pad":  # leading dimension larger than the row, non-zero offset
        ld = C + 3
        store = rng.integers(0, 2 ** 15, size=(R + 1) * ld + 5).astype(bits2d.dtype)
        store[5 + np.arange(R)[:, None] * ld + np.arange(C)[None, :]] = bits2d
        return W.Operand(store, dtype, R, C, 5, ld, 1)
    if layout == "neg":  # rows stored bottom-up: negative row stride
        store = np.ascontiguousarray(bits2d[::-1]).reshape(-1)
        return W.Operand(store, dtype, R, C, (R - 1) * C, -C, 1)
    raise ValueError(layout)


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_integer_brute_force_vs_numpy_int64(in_dtype, out_dtype):
    """Integer-valued inputs: the exact result is numpy's int64 matmul of the
    logical matrices; the oracle's fp64 sum equals it and its output is the
    library rounding of it.  Shapes include 0 and 1 and non-square ones so a
    swapped index or a transposed operand cannot pass; layouts cover
    transposed, padded (offset + leading dim) and negative-stride views."""
    rng = np.random.default_rng(11)
    R = 16 if in_dtype == "bf16" else 64
    layouts = ["N", "T", "pad", "neg"]
    for trial in range(40):
        M, N, K = (int(x) for x in rng.integers(0, 10, size=3))
        a = rng.integers(-R, R + 1, size=(M, K)).astype(np.float64)
        b = rng.integers(-R, R + 1, size=(K, N)).astype(np.float64)
        la, lb = layouts[trial % 4], layouts[(trial // 4) % 4]
        if M == 0 or K == 0:
            la = "N"
        if K == 0 or N == 0:
            lb = "N"
        A = _view(W.to_bits(a, in_dtype).reshape(M, K), la, rng, in_dtype)
        B = _view(W.to_bits(b, in_dtype).reshape(K, N), lb, rng, in_dtype)
        p = W.Problem(M, N, K, A, B, in_dtype, out_dtype)
        c64, c = _f(p)
        exact = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64)
        assert np.array_equal(c64, exact), (trial, M, N, K, la, lb)
        assert np.array_equal(c, _numpy_round(exact, out_dtype)), (trial, M, N, K)


def test_strided_view_equals_contiguous_copy():
    """A view and numpy's contiguous copy of it give identical fp64 results,
    for non-integer values too (the stride rule of Lesson 4, homework 2: the
    transpose of a row-major (N,K) buffer read as (K,N) has strides (1, K))."""
    rng = np.random.default_rng(3)
    M, N, K = 13, 7, 29
    for dt in ["f32", "f16", "bf16"]:
        a = W.to_bits(rng.normal(size=(M, K)), dt).reshape(M, K)
        b = W.to_bits(rng.normal(size=(K, N)), dt).reshape(K, N)
        base, _ = _f(W.Problem(M, N, K, W.dense(a, dt), W.dense(b, dt), dt, "f32"))
        for la in ["T", "pad", "neg"]:
            for lb in ["T", "pad", "neg"]:
                A = _view(a, la, rng, dt)
                B = _view(b, lb, rng, dt)
                assert np.array_equal(A.logical_bits(), a) and np.array_equal(B.logical_bits(), b)
                got, _ = _f(W.Problem(M, N, K, A, B, dt, "f32"))
                assert np.array_equal(got, base), (dt, la, lb)


def test_broadcast_zero_stride():
    """A zero stride repeats one row/column: C's rows are then all equal."""
    rng = np.random.default_rng(5)
    K, N = 11, 6
    row = W.to_bits(rng.normal(size=K), "f32")
    b = W.to_bits(rng.normal(size=(K, N)), "f32")
    A = W.Operand(row, "f32", 4, K, 0, 0, 1)
    c64, _ = _f(W.Problem(4, N, K, A, W.dense(b.reshape(K, N), "f32"), "f32", "f32"))
    assert (c64 == c64[0]).all()


# ------------------------------------------------------- fp64 accumulation


def test_fp64_sum_is_accurate():
    """The running sum is fp64: against the correctly rounded exact sum
    (math.fsum over the exact products) the error stays within the textbook
    bound K*u*sum|a*b| with u = 2^-53, far below what an fp32 sum reaches."""
    rng = np.random.default_rng(9)
    M, N, K = 3, 4, 4096
    a = W.to_bits(rng.normal(size=(M, K)), "f32").reshape(M, K)
    b = W.to_bits(rng.normal(size=(K, N)), "f32").reshape(K, N)
    c64, _ = _f(W.Problem(M, N, K, W.dense(a, "f32"), W.dense(b, "f32"), "f32", "f32"))
    af = a.view(np.float32).astype(np.float64)
    bf = b.view(np.float32).astype(np.float64)
    for i in range(M):
        for j in range(N):
            prods = af[i] * bf[:, j]
            exact = math.fsum(prods)
            bound = K * 2.0 ** -53 * np.abs(prods).sum()
            assert abs(c64[i, j] - exact) <= bound
    # the fp64 sum is not accidentally an fp32 one: an fp32 running sum is
    # typically ~1e-6 relative off, four orders of magnitude above this bound
    s32 = np.float32(0)
    for p in (af[0] * bf[:, 0]).astype(np.float32):
        s32 = np.float32(s32 + p)
    assert abs(float(s32) - math.fsum(af[0] * bf[:, 0])) > 100 * abs(
        c64[0, 0] - math.fsum(af[0] * bf[:, 0]))


# ------------------------------------------------------------------ codecs


def test_decode_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_f32_sampled():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:6] = [0, 0x80000000, 1, 0x007FFFFF, 0x7F800000, 0xFF800000]
    got = oracle.decode(bits, "f32")
    want = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_encode_f16_and_f32_vs_numpy():
    """Round-to-nearest-even from double, against numpy's double->half and
    double->single conversions (both correctly rounded), including subnormals,
    overflow and exact ties."""
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.normal(size=100000) * 10.0 ** rng.integers(-9, 6, size=100000),
        (np.arange(-70000, 70000, 0.5)),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 1e300, -1e-300, np.inf, -np.inf],
    ])
    for dt, npdt, ubits in [("f16", np.float16, np.uint16), ("f32", np.float32, np.uint32)]:
        with np.errstate(over="ignore"):
            want = x.astype(npdt).view(ubits)
        got = oracle.encode(x, dt)
        assert np.array_equal(got, want), dt
    assert oracle.encode(np.array([np.nan]), "f16")[0] & 0x7C00 == 0x7C00


def test_encode_bf16():
    """bf16 rounding: against torch's float->bf16 on fp32-representable values,
    plus ties and sticky bits below fp32 precision that a detour through fp32
    would lose (direct rounding from double is required)."""
    rng = np.random.default_rng(4)
    x = (rng.normal(size=200000) * 10.0 ** rng.integers(-30, 30, size=200000)).astype(np.float32)
    x = np.concatenate([x, np.array([3.3895313892515355e38, 3.4e38, 1e-40, -0.0],
                                    dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode(x.astype(np.float64), "bf16")
    assert np.array_equal(got, want)
    one = 0x3F80
    cases = {
        1.0 + 2.0 ** -8: one,                    # exact tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: one + 2,            # tie between odd and even -> even
        1.0 + 2.0 ** -8 + 2.0 ** -40: one + 1,   # just above the tie -> up
        1.0 + 2.0 ** -8 - 2.0 ** -40: one,       # just below -> down
        2.0 ** 128 * (1 - 2.0 ** -9): 0x7F80,    # halfway above max finite -> inf
        2.0 ** -134: 0x0000,                     # half the smallest subnormal -> 0
        3 * 2.0 ** -135: 0x0001,                 # 0.75 of it -> smallest subnormal
    }
    got = oracle.encode(np.array(list(cases)), "bf16")
    assert list(got) == list(cases.values())


def test_tolerance_formula():
    """The per-element bounds used by every parity test."""
    assert oracle.tolerance("f32", 193, 2.0, 3.0) == pytest.approx(1e-5 * 193 * 6.0)
    assert oracle.tolerance("f16", 4096, 1.0, 1.0) == pytest.approx(4e-3 * 64)
    assert oracle.tolerance("bf16", 8192, 0.5, 2.0) == pytest.approx(4e-3 * math.sqrt(8192))
