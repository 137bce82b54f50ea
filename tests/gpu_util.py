"""Helpers for GPU parity tests: operands of a workloads.Problem on the device,
a GEMM through the C ABI (raw pointers, so any strides work, including
negative ones), and the comparison with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dense_tiled_matrix_amd as dtm
import oracle

CODE = {"f32": dtm.DTM_F32, "f16": dtm.DTM_F16, "bf16": dtm.DTM_BF16}
ITEM = {"f32": 4, "f16": 2, "bf16": 2}
INT = {"f32": np.int32, "f16": np.int16, "bf16": np.int16}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_storage(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """Raw bits on cuda:0 (int32 or int16 tensor)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(INT[dtype]).copy()).to("cuda:0")


def sentinel_bits(value: float, dtype: str):
    return oracle.encode(np.array([value]), dtype).view(INT[dtype])[0]


class CBuf:
    """An output view (M x N, strides scm/scn, element offset) inside a
    device buffer pre-filled with a sentinel.  The offset defaults to 3
    elements when the leading dimension is padded (a misaligned view), else
    0."""

    def __init__(self, M, N, dtype, layout="N", sentinel=float("nan"), pad=0, offset=None):
        self.M, self.N, self.dtype = M, N, dtype
        if layout == "N":
            self.scm, self.scn = N + pad, 1
        elif layout == "T":
            self.scm, self.scn = 1, M + pad
        else:
            raise ValueError(layout)
        self.offset = (3 if pad else 0) if offset is None else offset
        size = self.offset + max(M * self.scm, N * self.scn, 1) + pad + 4
        self.sentinel = sentinel_bits(sentinel, dtype)
        self.buf = torch.full((size,), int(self.sentinel), dtype=torch.int32 if dtype == "f32"
                              else torch.int16, device="cuda:0")
        self.ptr = self.buf.data_ptr() + self.offset * ITEM[dtype]

    def read(self):
        """(view bits M x N, outside-of-view bits untouched?)"""
        host = self.buf.cpu().numpy()
        idx = (self.offset + np.arange(self.M)[:, None] * self.scm +
               np.arange(self.N)[None, :] * self.scn)
        mask = np.ones(host.shape, dtype=bool)
        mask[idx.reshape(-1)] = False
        untouched = bool((host[mask] == self.sentinel).all())
        u = np.uint32 if self.dtype == "f32" else np.uint16
        return host[idx].view(u), untouched


def run(p, out_dtype=None, config=None, c_layout="N", c_pad=0, stream=None, expect=0,
        plan=None, c_offset=None):
    """GEMM of problem ``p`` on the GPU; returns (C bits M x N, untouched).
    A dict passed as ``plan`` receives the plan of the call."""
    od = out_dtype or p.out_dtype
    sa = dev_storage(p.A.bits, p.in_dtype) if p.A.bits.size else None
    sb = dev_storage(p.B.bits, p.in_dtype) if p.B.bits.size else None
    a_ptr = sa.data_ptr() + p.A.offset * ITEM[p.in_dtype] if sa is not None else 0
    b_ptr = sb.data_ptr() + p.B.offset * ITEM[p.in_dtype] if sb is not None else 0
    c = CBuf(p.M, p.N, od, c_layout, pad=c_pad, offset=c_offset)
    s = torch.cuda.current_stream() if stream is None else stream
    if plan is not None:
        pst, pd = dtm.gemm_plan_raw(p.M, p.N, p.K, a_ptr, p.A.stride_r, p.A.stride_c, b_ptr,
                                    p.B.stride_r, p.B.stride_c, c.ptr, c.scm, c.scn,
                                    CODE[p.in_dtype], CODE[od], config=config)
        plan.update(pd, status=pst)
    st = dtm.gemm_ex_raw(p.M, p.N, p.K, a_ptr, p.A.stride_r, p.A.stride_c, b_ptr, p.B.stride_r,
                         p.B.stride_c, c.ptr, c.scm, c.scn, CODE[p.in_dtype], CODE[od],
                         config=config, stream=s.cuda_stream)
    assert st == expect, (dtm.STATUS.get(st, st), dtm.gemm_status_string(st))
    torch.cuda.synchronize()
    return c.read()


def maxabs(op):
    if op.rows == 0 or op.cols == 0:
        return 0.0
    v = oracle.decode(op.logical_bits(), op.dtype)
    return float(np.abs(v).max())


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of ``dtype`` at |x| (the most one final rounding adds)."""
    if dtype == "f32":
        mant, emin = 23, -126
    elif dtype == "f16":
        mant, emin = 10, -14
    else:
        mant, emin = 7, -126
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    return 0.5 * np.exp2(e - mant)


def compare(p, cbits, out_dtype=None, exact=False, c64=None, cout=None, label=""):
    """Check the GPU result against the oracle.  ``exact``: value-equal to the
    oracle's rounded output.  Otherwise per element
    |C - C64| <= tol(in_dtype, K, max|a|, max|b|) + half an output ulp."""
    od = out_dtype or p.out_dtype
    if c64 is None:
        c64, cout = oracle.gemm_problem(p, od)
    got = oracle.decode(cbits, od)
    assert not np.isnan(got).any(), f"{label}: NaN in GPU result"
    if exact:
        want = oracle.decode(cout, od)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{label}: {len(bad)} mismatches, first {bad[:3].tolist()}: " \
                              f"got {got[tuple(bad[0])]}, want {want[tuple(bad[0])]}"
        return 0.0, 0.0
    tol = oracle.tolerance(p.in_dtype, p.K, maxabs(p.A), maxabs(p.B))
    allowed = tol + (half_ulp(c64, od) if od != "f32" else 0.0)
    err = np.abs(got - c64)
    worst = float(err.max()) if err.size else 0.0
    over = np.argwhere(err > allowed)
    assert over.size == 0, f"{label}: {len(over)} elements over tolerance; max err {worst} " \
                           f"tol {tol}; first at {over[:3].tolist()}"
    return worst, tol


def _abs_operand(op):
    """The operand with every element's sign bit cleared (|x|, exactly)."""
    import workloads as W

    mask = 0x7FFFFFFF if op.dtype == "f32" else 0x7FFF
    bits = (np.asarray(op.bits).astype(np.uint64) & mask).astype(op.bits.dtype)
    return W.Operand(bits, op.dtype, op.rows, op.cols, op.offset, op.stride_r, op.stride_c)


def higham_ratio(p, cbits, c64, out_dtype=None):
    """max over C of |C - C64| / (gamma_K * (|A||B|)_ij + half an output ulp
    of C64), gamma_K = K u' / (1 - K u') with u' = 2 * 2^-24: the worst-case
    error of any order of K fp32 additions of the products (the textbook
    bound, with twice the fp32 unit roundoff as headroom for the matrix
    cores' internal adds).  At most 1 for fp32 accumulation; inputs rounded
    below fp32 precision on the way in would exceed it."""
    import workloads as W

    od = out_dtype or p.out_dtype
    absp = W.Problem(p.M, p.N, p.K, _abs_operand(p.A), _abs_operand(p.B), p.in_dtype, od)
    ab64, _ = oracle.gemm_problem(absp)
    u = 2.0 * 2.0 ** -24
    gamma = p.K * u / (1 - p.K * u)
    bound = gamma * ab64 + (half_ulp(c64, od) if od != "f32" else 0.0)
    got = oracle.decode(cbits, od)
    err = np.abs(got - c64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / bound)
    return float(r.max()) if r.size else 0.0
