"""The optional pointer checks (gemm_set_pointer_checks) on the device:
views inside device allocations of the current device run and give the
right result; a view in pinned host memory is refused with DTM_ERR_POINTER
and nothing is written.  (A view running past its allocation is refused by
the same range test; no case here would touch memory outside a mapped
allocation if a check let it through.)"""
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import workloads as W
from gpu_util import CODE, run, compare

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks_on():
    prev = dtm.set_pointer_checks(True)
    yield
    dtm.set_pointer_checks(prev)


def test_checked_calls_run(checks_on):
    # the pipelined kernel, the generic kernel (transposed fp32 A) and split-K
    for p, cfg in [(W.random_problem(512, 384, 256, "bf16", "f32", ("int", -3, 3), 900), None),
                   (W.random_problem(65, 33, 47, "f32", "f32", ("int", -3, 3), 901, "T", "N"),
                    None),
                   (W.random_problem(256, 256, 2048, "f16", "f16", ("int", -2, 2), 902),
                    dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=128, block_n=128, block_k=32,
                         split_k=4))]:
        c, untouched = run(p, config=cfg)
        compare(p, c, exact=True, label=f"checked {p.name}")
        assert untouched
    x = torch.randn(64, 1000, device="cuda")
    y = dtm.row_softmax(x)
    torch.testing.assert_close(y, torch.softmax(x, dim=1), rtol=1e-5, atol=1e-6)


def test_host_memory_refused(checks_on):
    M = N = K = 64
    a = torch.ones(M, K, dtype=torch.bfloat16, device="cuda")
    b_host = torch.ones(K, N, dtype=torch.bfloat16).pin_memory()
    c = torch.full((M, N), -7.0, device="cuda")
    st = dtm.gemm_raw(M, N, K, a.data_ptr(), K, 1, b_host.data_ptr(), N, 1, c.data_ptr(), N, 1,
                      CODE["bf16"], CODE["f32"], stream=torch.cuda.current_stream().cuda_stream)
    assert st == dtm.DTM_ERR_POINTER, dtm.STATUS.get(st, st)
    x_host = torch.randn(8, 64).pin_memory()
    y = torch.full((8, 64), -7.0, device="cuda")
    st = dtm.row_softmax_raw(8, 64, x_host.data_ptr(), 64, 1, y.data_ptr(), 64, 1,
                             CODE["f32"], CODE["f32"],
                             stream=torch.cuda.current_stream().cuda_stream)
    assert st == dtm.DTM_ERR_POINTER, dtm.STATUS.get(st, st)
    torch.cuda.synchronize()
    assert (c == -7.0).all() and (y == -7.0).all()
    # the same calls with device memory go through
    b = b_host.to("cuda")
    st = dtm.gemm_raw(M, N, K, a.data_ptr(), K, 1, b.data_ptr(), N, 1, c.data_ptr(), N, 1,
                      CODE["bf16"], CODE["f32"], stream=torch.cuda.current_stream().cuda_stream)
    assert st == dtm.DTM_OK
    torch.cuda.synchronize()
    assert (c == float(K)).all()
