"""CPU oracle for the blocked GEMM C = A·B and the row softmax (ctypes
wrapper over liboracle.so).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

What it computes follows "Chapter 13: The Blocked Matmul Kernel" (sections
13.1-13.3): ``C[i][j] = sum_k A[i][k]*B[k][j]`` with k ascending and an fp64
running sum over the exact decoded inputs, then one round-to-nearest-even
conversion to the output dtype; plus section 13.3's fp16-accumulator variant
as an emulation.  The row softmax follows "Triton from zero, Lesson 4: Block
Pointers", homework 4, in fp64.  See ``oracle_gemm.c`` for the arithmetic.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_ITEM = {"f32": 4, "f16": 2, "bf16": 2}
_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}

_lib = None


def load_library(path: str):
    """Open an oracle shared library at ``path`` and declare its signatures."""
    L = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.oracle_gemm.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, i32, i32, vp, vp,
                              i32]
    L.oracle_gemm.restype = i32
    L.oracle_gemm_fp16acc.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, i32, i64,
                                      vp]
    L.oracle_gemm_fp16acc.restype = i32
    L.oracle_softmax.argtypes = [i64, i64, vp, i64, i64, i32, i32, vp, vp, i32]
    L.oracle_softmax.restype = i32
    L.oracle_decode_array.argtypes = [vp, i64, i32, vp]
    L.oracle_decode_array.restype = i32
    L.oracle_encode_array.argtypes = [vp, i64, i32, vp]
    L.oracle_encode_array.restype = i32
    return L


def lib():
    """Load liboracle.so, building it first only if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load_library(_build.LIB)
    return _lib


def _ptr(bits: np.ndarray, offset: int) -> int:
    assert bits.flags["C_CONTIGUOUS"]
    return bits.ctypes.data + offset * bits.itemsize if bits.size else 0


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of raw ``dtype`` bits."""
    b = np.ascontiguousarray(bits, dtype=_BITS[dtype])
    out = np.empty(b.shape, dtype=np.float64)
    rc = lib().oracle_decode_array(_ptr(b, 0), b.size, _CODE[dtype], out.ctypes.data)
    assert rc == 0
    return out


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (nearest, ties to even) and return bits."""
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=_BITS[dtype])
    rc = lib().oracle_encode_array(v.ctypes.data, v.size, _CODE[dtype], _ptr(out, 0))
    assert rc == 0
    return out


def gemm(M, N, K, a_bits, a_offset, stride_am, stride_ak, b_bits, b_offset, stride_bk,
         stride_bn, in_dtype, out_dtype, threads: int = 0):
    """Return ``(C64, Cout_bits)``: the fp64 sums and their rounding to out_dtype.

    ``a_bits``/``b_bits`` are flat storage arrays of raw bits; the (0,0) element
    sits at ``*_offset`` and strides are in elements (they may be zero or
    negative).  Both results are dense row-major M x N.
    """
    a = np.ascontiguousarray(a_bits, dtype=_BITS[in_dtype]).reshape(-1)
    b = np.ascontiguousarray(b_bits, dtype=_BITS[in_dtype]).reshape(-1)
    c64 = np.zeros((M, N), dtype=np.float64)
    cout = np.zeros((M, N), dtype=_BITS[out_dtype])
    rc = lib().oracle_gemm(M, N, K, _ptr(a, a_offset), stride_am, stride_ak, _ptr(b, b_offset),
                           stride_bk, stride_bn, _CODE[in_dtype], _CODE[out_dtype],
                           c64.ctypes.data, _ptr(cout, 0), threads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed with {rc}")
    return c64, cout


def gemm_problem(p, out_dtype=None, threads: int = 0):
    """``gemm`` on a ``workloads.Problem``."""
    od = out_dtype or p.out_dtype
    return gemm(p.M, p.N, p.K, p.A.bits, p.A.offset, p.A.stride_r, p.A.stride_c, p.B.bits,
                p.B.offset, p.B.stride_r, p.B.stride_c, p.in_dtype, od, threads)


def gemm_fp16acc(M, N, K, a_bits, a_offset, stride_am, stride_ak, b_bits, b_offset, stride_bk,
                 stride_bn, in_dtype, block_k):
    """Section 13.3's fp16-accumulator variant; returns fp16 bits (M x N)."""
    a = np.ascontiguousarray(a_bits, dtype=_BITS[in_dtype]).reshape(-1)
    b = np.ascontiguousarray(b_bits, dtype=_BITS[in_dtype]).reshape(-1)
    out = np.zeros((M, N), dtype=np.uint16)
    rc = lib().oracle_gemm_fp16acc(M, N, K, _ptr(a, a_offset), stride_am, stride_ak,
                                   _ptr(b, b_offset), stride_bk, stride_bn, _CODE[in_dtype],
                                   block_k, out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_fp16acc failed with {rc}")
    return out


def gemm_fp16acc_problem(p, block_k):
    return gemm_fp16acc(p.M, p.N, p.K, p.A.bits, p.A.offset, p.A.stride_r, p.A.stride_c,
                        p.B.bits, p.B.offset, p.B.stride_r, p.B.stride_c, p.in_dtype, block_k)


def tolerance(in_dtype: str, K: int, max_abs_a: float, max_abs_b: float) -> float:
    """Per-element error bound for a result computed with an fp32 accumulator.

    fp32 inputs: 1e-5*K*max|a|*max|b|; fp16/bf16 inputs: 4e-3*sqrt(K)*max|a|*max|b|,
    both relative to this oracle's fp64 result on the same rounded inputs.
    """
    if in_dtype == "f32":
        return 1e-5 * K * max_abs_a * max_abs_b
    return 4e-3 * float(np.sqrt(K)) * max_abs_a * max_abs_b


def softmax(M, N, x_bits, x_offset, stride_xm, stride_xn, in_dtype, out_dtype, threads: int = 0):
    """Row softmax of the M x N view; returns ``(Y64, Yout_bits)``, both dense
    row-major M x N (fp64 values and their rounding to out_dtype)."""
    x = np.ascontiguousarray(x_bits, dtype=_BITS[in_dtype]).reshape(-1)
    y64 = np.zeros((M, N), dtype=np.float64)
    yout = np.zeros((M, N), dtype=_BITS[out_dtype])
    rc = lib().oracle_softmax(M, N, _ptr(x, x_offset), stride_xm, stride_xn, _CODE[in_dtype],
                              _CODE[out_dtype], y64.ctypes.data, _ptr(yout, 0), threads)
    if rc != 0:
        raise RuntimeError(f"oracle_softmax failed with {rc}")
    return y64, yout


def softmax_problem(p, out_dtype=None, threads: int = 0):
    """``softmax`` on a ``workloads.SoftmaxProblem``."""
    X = p.X
    return softmax(p.M, p.N, X.bits, X.offset, X.stride_r, X.stride_c, p.in_dtype,
                   out_dtype or p.out_dtype, threads)


def softmax_tolerance(x64_row_minus_max: np.ndarray, y64: np.ndarray, n: int) -> np.ndarray:
    """Per-element bound on |Y - Y64| for a row softmax of row length ``n``
    computed in fp32 (unit roundoff u = 2^-24) from the same inputs, fixed
    in advance from the formula alone, whatever the order of the sum:

    * the shifted argument d = x - max rounded once and scaled by log2(e)
      once: a relative error of at most 2|d|u in exp(d);
    * the exponential itself: 4u (a few ulps);
    * the sum of the row's n exponentials, with any rescaling of partial
      sums by exp(m_old - m_new) and the argument errors of the other terms:
      bounded probabilistically (Higham & Mary, "A new approach to
      probabilistic rounding error analysis", 2019: rounding errors behave
      as independent, mean-zero, so n of them grow as sqrt(n), not n) by
      lambda * sqrt(4n) u with lambda = 8 (a failure probability below
      1e-13 per element under that model);
    * the reciprocal of the sum and the product with it: 2u;
    * exponentials below 2^-126 may flush to zero: an absolute 2^-125
      (the sum is at least 1, the maximum's own term).

    Returns the bounds elementwise: |Y64| * (2|d| + 6 + 16 sqrt(n)) u + 2^-125."""
    d = np.abs(np.nan_to_num(x64_row_minus_max, nan=0.0, neginf=0.0))
    rel = (2.0 * d + 6.0 + 16.0 * np.sqrt(float(max(n, 1)))) * 2.0 ** -24
    return np.abs(y64) * rel + 2.0 ** -125
