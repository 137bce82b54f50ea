"""Operands and results past 2^31 and 2^32 bytes through the C ABI: every
address on the GEMM and softmax paths is 64-bit, and the range-checked
pipelined form (32-bit buffer offsets) hands views over 2^31 bytes to the
register-staged kernel.

The inputs are drawn on the device by torch's seeded generator (copying
gigabytes of host-drawn values would dominate the test), as small integers
for the GEMM, which every dtype holds exactly, so the products are exact in
fp32 and the oracle's rounded output must match bit for bit.  Rows on both
sides of the 2^31- and 2^32-byte marks, the first and the last rows are
pulled back and recomputed by the oracle.
"""
import numpy as np
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import oracle
import workloads as W
from gpu_util import note
from test_softmax_gpu import check as softmax_check

pytestmark = pytest.mark.gpu


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _rows_past(row_bytes: int, M: int):
    """Rows whose start crosses 2^31 and 2^32 bytes, plus the ends."""
    rows = {0, 1, M // 2, M - 2, M - 1}
    for mark in (1 << 31, 1 << 32):
        r = mark // row_bytes
        rows.update(x for x in (r - 1, r, r + 1) if 0 <= x < M)
    return sorted(rows)


@pytest.mark.parametrize("M,N,K,kernel_bk,ragged", [
    (69632, 256, 32768, 32, 0),   # A is 4.25 GiB: the pipelined kernel's interior form
    (69633, 248, 32768, 64, 1),   # ragged, A over 2^31 bytes: the register-staged kernel
])
def test_gemm_past_4gib(M, N, K, kernel_bk, ragged):
    note(f"gemm {M}x{N}x{K} bf16: A {M * K * 2 / 2**30:.2f} GiB")
    g = torch.Generator(device="cuda").manual_seed(4242 + M)
    a = torch.randint(-2, 3, (M, K), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    b = torch.randint(-2, 3, (K, N), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    plan = dtm.gemm_plan(a, b, out_dtype=torch.bfloat16)
    assert (plan["kernel_name"], plan["block_k"], plan["ragged"]) == \
        ("mfma_f16", kernel_bk, ragged), plan
    c = dtm.gemm(a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _rows_past(K * 2, M)
    idx = torch.tensor(rows, device="cuda")
    a_rows = _bits16(a.index_select(0, idx))
    got = _bits16(c.index_select(0, idx))
    del a, c
    p = W.Problem(len(rows), N, K, W.dense(a_rows, "bf16"), W.dense(_bits16(b), "bf16"),
                  "bf16", "bf16")
    _, want = oracle.gemm_problem(p)
    assert (got == want).all(), f"rows {rows}: {np.argwhere(got != want)[:3].tolist()}"
    # the C view ends past 2^25 elements; its last rows were among those checked
    note(f"checked rows {rows}")


def test_softmax_past_4gib():
    """A 300000 x 8192 bf16 row softmax (4.6 GiB each way) in the wave form."""
    M, N = 300000, 8192
    g = torch.Generator(device="cuda").manual_seed(4343)
    x = (torch.randn(M, N, generator=g, device="cuda") * 3).to(torch.bfloat16)
    y = torch.empty_like(x)
    plan = dtm.row_softmax_plan(x, out=y)
    assert plan["form_name"] == "wave", plan
    dtm.row_softmax(x, out=y)
    torch.cuda.synchronize()
    rows = _rows_past(N * 2, M)
    idx = torch.tensor(rows, device="cuda")
    x_rows = _bits16(x.index_select(0, idx))
    got = _bits16(y.index_select(0, idx))
    del x, y
    p = W.SoftmaxProblem(len(rows), N, W.dense(x_rows, "bf16"), "bf16", "bf16")
    softmax_check(p, got, plan, label=f"softmax {M}x{N} rows {rows}")
    note(f"checked rows {rows}")
