"""GPU parity of the row softmax ("Triton from zero, Lesson 4: Block Pointers",
homework 4) through the C ABI against the CPU oracle.

Bar: the device computes in fp32 from the exactly decoded inputs, the oracle
in fp64.  Per element |Y - Y64| <= oracle.softmax_tolerance(d, Y64, N)
(d = x - row max, N the row length: a bound fixed from the formula, not from
the launched form), plus half an output ulp for fp16/bf16 outputs; where the
oracle gives NaN
(rows of -inf, +inf or NaN entries) the device must too, and exact zeros
(-inf entries in finite rows) must be exact zeros.
"""
import numpy as np
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import oracle
import workloads as W
from gpu_util import CBuf, dev_storage, half_ulp, note

pytestmark = pytest.mark.gpu

CODE = {"f32": dtm.DTM_F32, "f16": dtm.DTM_F16, "bf16": dtm.DTM_BF16}
ITEM = {"f32": 4, "f16": 2, "bf16": 2}


def run_softmax(p, out_dtype=None, layout="N", pad=0, plan=None, in_place=False):
    """Row softmax of problem ``p`` on the GPU; returns (Y bits M x N, untouched)."""
    od = out_dtype or p.out_dtype
    sx = dev_storage(p.X.bits, p.in_dtype) if p.X.bits.size else None
    x_ptr = sx.data_ptr() + p.X.offset * ITEM[p.in_dtype] if sx is not None else 0
    if in_place:
        assert od == p.in_dtype or ITEM[od] == ITEM[p.in_dtype]
        y_ptr, sym, syn = x_ptr, p.X.stride_r, p.X.stride_c
        c = None
    else:
        c = CBuf(p.M, p.N, od, layout, pad=pad)
        y_ptr, sym, syn = c.ptr, c.scm, c.scn
    if plan is not None:
        st, pd = dtm.row_softmax_plan_raw(p.M, p.N, x_ptr, p.X.stride_r, p.X.stride_c, y_ptr,
                                          sym, syn, CODE[p.in_dtype], CODE[od])
        plan.update(pd, status=st)
    st = dtm.row_softmax_raw(p.M, p.N, x_ptr, p.X.stride_r, p.X.stride_c, y_ptr, sym, syn,
                             CODE[p.in_dtype], CODE[od],
                             stream=torch.cuda.current_stream().cuda_stream)
    assert st == 0, (dtm.STATUS.get(st, st),)
    torch.cuda.synchronize()
    if in_place:
        host = sx.cpu().numpy().view(W.BITS_NP[od])
        idx = p.X.offset + np.arange(p.M)[:, None] * p.X.stride_r + \
            np.arange(p.N)[None, :] * p.X.stride_c
        return host[idx], True
    return c.read()


def check(p, ybits, plan, out_dtype=None, label=""):
    od = out_dtype or p.out_dtype
    y64, _ = oracle.softmax_problem(p, od)
    got = oracle.decode(ybits, od)
    x = oracle.decode(p.X.logical_bits(), p.in_dtype)
    with np.errstate(invalid="ignore"):
        m = np.max(np.where(np.isnan(x), -np.inf, x), axis=1, keepdims=True) if p.N else x
        d = x - m
    nan = np.isnan(y64)
    assert (np.isnan(got) == nan).all(), f"{label}: NaN pattern differs"
    zero = (y64 == 0.0)
    tol = oracle.softmax_tolerance(d, y64, p.N)
    if od != "f32":
        tol = tol + half_ulp(y64, od)
    err = np.where(nan, 0.0, np.abs(got - y64))
    over = np.argwhere(err > tol)
    assert over.size == 0, f"{label}: {len(over)} over tolerance, first {over[:3].tolist()}: " \
                           f"got {got[tuple(over[0])]} want {y64[tuple(over[0])]}"
    assert (got[zero & np.isneginf(x)] == 0.0).all(), f"{label}: -inf entries not exact zeros"
    worst = float(err.max()) if err.size else 0.0
    rel = float(np.max(np.where(nan | (y64 == 0), 0.0, err / np.where(y64 == 0, 1, y64)))) \
        if err.size else 0.0
    return worst, rel


@pytest.mark.parametrize("name", list(W.SOFTMAX_WORKLOADS))
def test_softmax_workloads(name):
    """The four softmax workloads at full size in the launch configuration the
    bench times, compared in full."""
    p = W.softmax_workload(name)
    note(f"{name}: {p.M}x{p.N} {p.in_dtype}->{p.out_dtype}")
    plan = {}
    y, untouched = run_softmax(p, plan=plan)
    worst, rel = check(p, y, plan, label=name)
    note(f"{name}: form {plan['form_name']} x{plan['chunks']} vec {plan['vectorized']}: "
         f"max abs err {worst:.3e}, max rel err {rel:.3e}")
    assert untouched


ROW_LENGTHS = [1, 2, 3, 7, 63, 64, 65, 255, 256, 257, 1000, 1023, 1024, 1025, 2047, 2049,
               4095, 4097, 8191, 16385, 32769, 65537, 100003]


@pytest.mark.parametrize("ind,outd", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                      ("f16", "f32"), ("f32", "bf16")])
def test_softmax_row_length_sweep(ind, outd):
    """Every form and chunk count: row lengths around each capacity (wave,
    workgroup, online), including partial 16-byte chunks, with a few rows;
    -inf masked entries; NaN sentinel around the output view."""
    for n, N in enumerate(ROW_LENGTHS):
        M = [1, 3, 5, 17, 2049][n % 5] if N <= 4097 else [1, 3, 5][n % 3]
        p = W.softmax_problem(M, N, ind, outd, ("normal", 0.0, 4.0), seed=900 + n,
                              masked=0.05 if n % 2 else 0.0)
        plan = {}
        y, untouched = run_softmax(p, plan=plan, pad=3 if n % 3 == 0 else 0)
        check(p, y, plan, label=f"{ind}->{outd} {M}x{N} {plan['form_name']}")
        assert untouched


def test_softmax_block_form_many_chunks():
    """Rows held whole in a 1024-thread workgroup's registers: 8 and 16 chunks
    per thread (fp32), 8 (16-bit), ragged lengths, -inf masks, an
    element-wise (transposed) view, in and out of every dtype."""
    cases = [(256, 65536, "f32", "f32", "N"), (300, 65532, "f32", "bf16", "N"),
             (257, 30004, "f32", "f32", "N"), (260, 60000, "bf16", "bf16", "N"),
             (256, 49160, "f16", "f32", "N"), (300, 13000, "f32", "f16", "T")]
    for n, (M, N, ind, outd, layout) in enumerate(cases):
        p = W.softmax_problem(M, N, ind, outd, ("normal", 0.0, 3.0), seed=1050 + n,
                              layout=layout, masked=0.05 if n % 2 else 0.0)
        plan = {}
        y, untouched = run_softmax(p, plan=plan)
        assert plan["form_name"] == "block" and plan["chunks"] in (8, 16), (M, N, plan)
        check(p, y, plan, label=f"block x{plan['chunks']} {ind}->{outd} {M}x{N}")
        assert untouched


def test_softmax_many_rows_wave_form():
    """Many short rows so the wave form runs with several chunk counts."""
    for n, N in enumerate([100, 512, 1024, 2048, 4096]):
        p = W.softmax_problem(4099, N, "bf16", "f32", ("normal", 0.0, 3.0), seed=950 + n)
        plan = {}
        y, untouched = run_softmax(p, plan=plan)
        assert plan["form_name"] == "wave", plan
        check(p, y, plan, label=f"wave {N}")
        assert untouched


@pytest.mark.parametrize("layout", ["T", "N"])
def test_softmax_strided_views(layout):
    """Transposed input views and transposed or padded output views (the
    element-wise path), and an input misaligned by one element."""
    for n, (M, N) in enumerate([(37, 300), (129, 5000), (5, 70000)]):
        p = W.softmax_problem(M, N, "f32", "f16", ("normal", 0.0, 3.0), seed=970 + n,
                              layout=layout)
        plan = {}
        y, untouched = run_softmax(p, plan=plan, layout="T" if n % 2 else "N", pad=1)
        assert plan["vectorized"] == 0
        check(p, y, plan, label=f"strided {layout} {M}x{N}")
        assert untouched
    # misaligned row-major view: offset by one element inside a larger buffer
    p = W.softmax_problem(64, 1001, "bf16", "bf16", ("normal", 0.0, 3.0), seed=975)
    bits = np.concatenate([np.zeros(1, p.X.bits.dtype), p.X.bits])
    q = W.SoftmaxProblem(64, 1001, W.Operand(bits, "bf16", 64, 1001, 1, 1001, 1), "bf16", "bf16")
    plan = {}
    y, untouched = run_softmax(q, plan=plan)
    assert plan["vectorized"] == 0
    check(q, y, plan, label="misaligned")


def test_softmax_special_values():
    """-inf entries give exact zeros, a row of -inf or one with +inf or NaN is
    NaN, huge finite entries do not overflow (the max is subtracted) -- in
    every form."""
    for N in [50, 3000, 20000, 70000]:
        rng = np.random.default_rng(N)
        x = rng.normal(0.0, 3.0, size=(8, N))
        x[0, ::3] = -np.inf
        x[1, :] = -np.inf
        x[2, N // 2] = np.inf
        x[3, N // 3] = np.nan
        x[4, :] = 1.0e4
        x[4, ::7] = 1.0e4 - 1.0
        x[5, :] = -np.inf
        x[5, N - 1] = 2.5   # only the last column is finite
        x[6, :] = -1.0e4
        bits = W.to_bits(x, "f32").reshape(8, N)
        p = W.SoftmaxProblem(8, N, W.dense(bits, "f32"), "f32", "f32")
        plan = {}
        y, untouched = run_softmax(p, plan=plan)
        check(p, y, plan, label=f"special {N} {plan['form_name']}")
        got = oracle.decode(y, "f32")
        assert np.isnan(got[1:4]).all() and (got[5, :-1] == 0).all() and got[5, -1] == 1.0
        assert untouched


def test_softmax_split_form():
    """Few long rows split over several workgroups: per-part (max, sum) pairs
    merged in a fixed order, so results match the oracle and repeat bit for
    bit; parts that are wholly -inf, and a row of -inf, behave as in the
    other forms."""
    for n, (M, N, dt) in enumerate([(2, 300001, "f32"), (64, 65536, "bf16"), (9, 131073, "f16")]):
        p = W.softmax_problem(M, N, dt, dt, ("normal", 0.0, 3.0), seed=1010 + n,
                              masked=0.02)
        x = oracle.decode(p.X.logical_bits(), dt)
        if n == 0:  # a whole part of row 0 masked, and row 1 all -inf
            x[0, :100000] = -np.inf
            x[1, :] = -np.inf
            p = W.SoftmaxProblem(M, N, W.dense(W.to_bits(x, dt).reshape(M, N), dt), dt, dt)
        plan = {}
        y1, untouched = run_softmax(p, plan=plan)
        assert plan["form_name"] == "split" and plan["parts"] > 1, plan
        check(p, y1, plan, label=f"split {M}x{N} parts {plan['parts']}")
        y2, _ = run_softmax(p)
        assert (y1 == y2).all()
        assert untouched


def test_softmax_in_place():
    """Y the same view as X (the listing stores through the input's block
    pointer): every form."""
    for n, (M, N, dt) in enumerate([(300, 777, "f32"), (64, 9000, "bf16"), (3, 80000, "f16")]):
        p = W.softmax_problem(M, N, dt, dt, ("normal", 0.0, 3.0), seed=990 + n)
        plan = {}
        y, _ = run_softmax(p, plan=plan, in_place=True)
        check(p, y, plan, label=f"in place {M}x{N} {plan['form_name']}")


def test_softmax_deterministic_and_torch_binding():
    """Repeated calls give identical bits; the tensor binding handles views
    and allocates the output."""
    x = torch.randn(1000, 3000, device="cuda:0") * 3
    y1 = dtm.row_softmax(x)
    y2 = dtm.row_softmax(x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = torch.softmax(x.double(), dim=1)
    assert float((y1.double() - ref).abs().max()) < 1e-6
    xt = x.t()  # a transposed view: 3000 rows of 1000
    yt = dtm.row_softmax(xt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert yt.dtype == torch.bfloat16 and tuple(yt.shape) == (3000, 1000)
    assert float((yt.double() - torch.softmax(xt.double(), dim=1)).abs().max()) < 2 ** -8


def test_softmax_empty_shapes():
    assert dtm.row_softmax_raw(0, 5, 0, 5, 1, 0, 5, 1, 0, 0) == 0
    assert dtm.row_softmax_raw(5, 0, 0, 0, 1, 0, 0, 1, 0, 0) == 0
