"""Seeded synthetic inputs for the blocked GEMM C = A·B and the row softmax.

This module is shared by the HIP path's tests and bench and by the CPU oracle's
tests.  It holds no part of the GEMM itself: it only draws numbers, rounds them
to the storage dtype of the operands, and describes the operand views (shape,
strides, storage offset).  Both sides then read the same bits.

Distributions, shapes and layouts follow the five workloads the library is
measured and checked on (integer-valued fp32 8x8x8, a ragged fp32 problem with
a transposed A view, fp16 4096^3, bf16 8192^3 and a long-K fp16 skinny
problem).  Values are drawn in float64 from numpy's PCG64 generator with seed
``1000*workload + 0`` for A and ``+1`` for B, then rounded to the input dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}
BITS_NP = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def draw(shape, dist, seed: int) -> np.ndarray:
    """Draw float64 values of ``shape``.

    ``dist`` is one of ``("int", lo, hi)`` (integers, both ends inclusive),
    ``("uniform", lo, hi)`` or ``("normal", mean, std)``.
    """
    rng = np.random.default_rng(seed)
    kind = dist[0]
    if kind == "int":
        return rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float64)
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape)
    raise ValueError(f"unknown distribution {dist!r}")


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` storage and return the raw bits.

    fp32 and fp16 use numpy's own conversions; bf16 goes through torch's CPU
    conversion from fp32.  Whatever the rounding of this step, both sides of a
    comparison consume the bits it returns.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).view(np.uint32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Operand:
    """A strided 2-D view into flat storage (bits), strides in elements."""

    bits: np.ndarray  # flat storage, uint16 or uint32
    dtype: str
    rows: int
    cols: int
    offset: int  # element index of (0, 0) in ``bits``
    stride_r: int
    stride_c: int

    def logical_bits(self) -> np.ndarray:
        """The rows x cols matrix of bits seen through the view (a copy)."""
        if self.rows == 0 or self.cols == 0:
            return np.zeros((self.rows, self.cols), dtype=self.bits.dtype)
        r = np.arange(self.rows, dtype=np.int64)[:, None] * self.stride_r
        c = np.arange(self.cols, dtype=np.int64)[None, :] * self.stride_c
        return self.bits[self.offset + r + c]


@dataclass
class Problem:
    M: int
    N: int
    K: int
    A: Operand
    B: Operand
    in_dtype: str
    out_dtype: str
    name: str = ""
    meta: dict = field(default_factory=dict)


def dense(bits2d: np.ndarray, dtype: str) -> Operand:
    """Row-major contiguous operand over a 2-D bits array."""
    r, c = bits2d.shape
    return Operand(np.ascontiguousarray(bits2d).reshape(-1), dtype, r, c, 0, c, 1)


def transposed_view(bits_t: np.ndarray, dtype: str) -> Operand:
    """Operand whose storage is the contiguous transpose ``bits_t`` (cols x rows).

    Element (r, c) of the view lives at ``c*rows + r``: strides (1, rows).
    """
    c, r = bits_t.shape
    return Operand(np.ascontiguousarray(bits_t).reshape(-1), dtype, r, c, 0, 1, r)


def random_problem(M, N, K, in_dtype, out_dtype, dist, seed, a_layout="N", b_layout="N",
                   name="") -> Problem:
    """A problem with operands drawn from ``dist``.

    ``a_layout``/``b_layout`` of "N" give a row-major view, "T" a view of a
    contiguous transpose (the column-major case).
    """
    a64 = draw((M, K), dist, seed)
    b64 = draw((K, N), dist, seed + 1)
    if a_layout == "N":
        A = dense(to_bits(a64, in_dtype).reshape(M, K), in_dtype)
    else:
        A = transposed_view(to_bits(a64.T.copy(), in_dtype).reshape(K, M), in_dtype)
    if b_layout == "N":
        B = dense(to_bits(b64, in_dtype).reshape(K, N), in_dtype)
    else:
        B = transposed_view(to_bits(b64.T.copy(), in_dtype).reshape(N, K), in_dtype)
    return Problem(M, N, K, A, B, in_dtype, out_dtype, name=name)


# The measured / checked workloads.  ``index`` is the seed base.
WORKLOADS = {
    "int8x8x8_f32": dict(index=0, M=8, N=8, K=8, in_dtype="f32", out_dtype="f32",
                         dist=("int", -4, 4), a_layout="N", b_layout="N"),
    "ragged257x129x193_f32_At": dict(index=1, M=257, N=129, K=193, in_dtype="f32",
                                     out_dtype="f32", dist=("normal", 0.0, 1.0),
                                     a_layout="T", b_layout="N"),
    "f16_4096_f32out": dict(index=2, M=4096, N=4096, K=4096, in_dtype="f16",
                            out_dtype="f32", dist=("uniform", -1.0, 1.0),
                            a_layout="N", b_layout="N"),
    "bf16_8192_bf16out": dict(index=3, M=8192, N=8192, K=8192, in_dtype="bf16",
                              out_dtype="bf16", dist=("normal", 0.0, 1.0),
                              a_layout="N", b_layout="N"),
    "f16_skinny512x512x65536_f32out": dict(index=4, M=512, N=512, K=65536, in_dtype="f16",
                                           out_dtype="f32", dist=("uniform", 0.0, 1.0),
                                           a_layout="N", b_layout="N"),
    # the two other size/dtype pairings of the measured shapes (extras)
    "f16_8192_f32out": dict(index=5, M=8192, N=8192, K=8192, in_dtype="f16",
                            out_dtype="f32", dist=("uniform", -1.0, 1.0),
                            a_layout="N", b_layout="N"),
    "bf16_4096_bf16out": dict(index=6, M=4096, N=4096, K=4096, in_dtype="bf16",
                              out_dtype="bf16", dist=("normal", 0.0, 1.0),
                              a_layout="N", b_layout="N"),
    # fp32 inputs on the fp32 matrix cores at a size where they dominate
    "f32_4096_f32out": dict(index=7, M=4096, N=4096, K=4096, in_dtype="f32",
                            out_dtype="f32", dist=("normal", 0.0, 1.0),
                            a_layout="N", b_layout="N"),
}


def workload(name: str) -> Problem:
    w = WORKLOADS[name]
    p = random_problem(w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["dist"],
                       1000 * w["index"], w["a_layout"], w["b_layout"], name=name)
    p.meta = dict(w)
    return p


def worked_2x2() -> Problem:
    """[[1,2],[3,4]] times [[5,6],[7,8]] in fp32."""
    a = to_bits(np.array([[1.0, 2.0], [3.0, 4.0]]), "f32")
    b = to_bits(np.array([[5.0, 6.0], [7.0, 8.0]]), "f32")
    return Problem(2, 2, 2, dense(a, "f32"), dense(b, "f32"), "f32", "f32", name="2x2")


def arange_problem(M, K, N, scale=1.0, dtype="f32") -> Problem:
    """A = arange(M*K).reshape(M,K)*scale, B = arange(K*N).reshape(K,N)*scale.

    Computed in fp32 (``arange`` then one fp32 multiply) as the Triton pages
    build them, then stored as ``dtype``.
    """
    a = (np.arange(M * K, dtype=np.float32).reshape(M, K) * np.float32(scale)).astype(np.float64)
    b = (np.arange(K * N, dtype=np.float32).reshape(K, N) * np.float32(scale)).astype(np.float64)
    return Problem(M, N, K, dense(to_bits(a, dtype), dtype), dense(to_bits(b, dtype), dtype),
                   dtype, "f32", name=f"arange{M}x{K}x{N}")


def sentinel_problem(sentinel: float = 999.0, dtype="f32") -> Problem:
    """The 4x5x4 sentinel case: A is the first 5 columns of a 4x8 buffer and B
    the first 5 rows of an 8x4 buffer; the rest of both buffers is ``sentinel``.
    Real entries are ``0.1*arange`` in fp32."""
    M, K, N = 4, 5, 4
    ab = np.full((M, 8), sentinel, dtype=np.float64)
    ab[:, :K] = (np.arange(M * K, dtype=np.float32).reshape(M, K) * np.float32(0.1))
    bb = np.full((8, N), sentinel, dtype=np.float64)
    bb[:K, :] = (np.arange(K * N, dtype=np.float32).reshape(K, N) * np.float32(0.1))
    A = Operand(to_bits(ab, dtype).reshape(-1), dtype, M, K, 0, 8, 1)
    B = Operand(to_bits(bb, dtype).reshape(-1), dtype, K, N, 0, N, 1)
    return Problem(M, N, K, A, B, dtype, "f32", name="sentinel4x5x4")


def seed0_fp16_problem() -> Problem:
    """torch.manual_seed(0); A = (randn(4,1024)*0.1).half(); B = (randn(1024,4)*0.1).half()."""
    import torch

    g = torch.Generator().manual_seed(0)
    a = (torch.randn(4, 1024, generator=g) * 0.1).to(torch.float16)
    b = (torch.randn(1024, 4, generator=g) * 0.1).to(torch.float16)
    A = dense(a.view(torch.int16).numpy().view(np.uint16).copy(), "f16")
    B = dense(b.view(torch.int16).numpy().view(np.uint16).copy(), "f16")
    return Problem(4, 4, 1024, A, B, "f16", "f16", name="seed0_4x1024x4")


# ----------------------------------------------------------------- row softmax


@dataclass
class SoftmaxProblem:
    M: int
    N: int
    X: Operand
    in_dtype: str
    out_dtype: str
    name: str = ""
    meta: dict = field(default_factory=dict)


def softmax_problem(M, N, in_dtype, out_dtype, dist, seed, layout="N", masked=0.0,
                    name="") -> SoftmaxProblem:
    """Rows drawn from ``dist``; a fraction ``masked`` of the entries (chosen
    with seed+1) set to -inf, as an attention-style mask would.  Layout "N"
    is a row-major view, "T" a view of a contiguous transpose."""
    x64 = draw((M, N), dist, seed)
    if masked > 0.0:
        rng = np.random.default_rng(seed + 1)
        x64[rng.random((M, N)) < masked] = -np.inf
    if layout == "N":
        X = dense(to_bits(x64, in_dtype).reshape(M, N), in_dtype)
    else:
        X = transposed_view(to_bits(x64.T.copy(), in_dtype).reshape(N, M), in_dtype)
    return SoftmaxProblem(M, N, X, in_dtype, out_dtype, name=name)


# Softmax workloads (synthetic; the pages give no sizes).  ``index`` is the
# seed base, after the GEMM workloads'.
SOFTMAX_WORKLOADS = {
    "softmax_f32_4096x4096": dict(index=10, M=4096, N=4096, in_dtype="f32", out_dtype="f32",
                                  dist=("normal", 0.0, 3.0), masked=0.0),
    "softmax_bf16_8192x8192_masked": dict(index=11, M=8192, N=8192, in_dtype="bf16",
                                          out_dtype="bf16", dist=("normal", 0.0, 3.0),
                                          masked=0.1),
    "softmax_f16_32768x1024": dict(index=12, M=32768, N=1024, in_dtype="f16", out_dtype="f16",
                                   dist=("normal", 0.0, 3.0), masked=0.0),
    "softmax_f32_256x65536": dict(index=13, M=256, N=65536, in_dtype="f32", out_dtype="f32",
                                  dist=("normal", 0.0, 3.0), masked=0.0),
}


def softmax_workload(name: str) -> SoftmaxProblem:
    w = SOFTMAX_WORKLOADS[name]
    p = softmax_problem(w["M"], w["N"], w["in_dtype"], w["out_dtype"], w["dist"],
                        1000 * w["index"], masked=w["masked"], name=name)
    p.meta = dict(w)
    return p
