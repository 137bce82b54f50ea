"""The MFMA fragment-layout probe (gemm_mfma_probe): one 16 x 16 x 32
matrix-core product through the LDS staging, fragment reads and epilogue lane
map of the fp16/bf16 kernels, in every operand layout and both staging row
widths, on integer-valued inputs (every sum exact in fp32), compared value
for value with the oracle.  A wrong lane <-> element map of A, B or C
permutes or mixes products and fails it."""
import numpy as np
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import oracle
from gpu_util import CODE, INT

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("paired", [0, 1])
@pytest.mark.parametrize("layout", [0, 1, 2, 3])
@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_fragment_layout_probe(ind, layout, paired):
    rng = np.random.default_rng(100 * layout + 10 * paired + (ind == "bf16"))
    for trial in range(3):
        if trial == 0:
            # distinct rows and columns: A[i][k] = i + 1 on one k per row, B[k][j] = k * 16 + j
            a = np.zeros((16, 32))
            a[np.arange(16), rng.permutation(32)[:16]] = np.arange(1, 17)
            b = np.arange(32 * 16, dtype=np.float64).reshape(32, 16) % 61 - 30
        else:
            a = rng.integers(-8, 9, size=(16, 32)).astype(np.float64)
            b = rng.integers(-8, 9, size=(32, 16)).astype(np.float64)
        a_store = a.T if layout & dtm.DTM_LAYOUT_A_M_CONTIG else a
        b_store = b.T if layout & dtm.DTM_LAYOUT_B_K_CONTIG else b
        ta = torch.from_numpy(np.ascontiguousarray(oracle.encode(a_store, ind)).view(INT[ind]))
        tb = torch.from_numpy(np.ascontiguousarray(oracle.encode(b_store, ind)).view(INT[ind]))
        ta, tb = ta.to("cuda:0"), tb.to("cuda:0")
        c = torch.full((16, 16), float("nan"), device="cuda:0")
        st = dtm.gemm_mfma_probe_raw(CODE[ind], layout, paired, ta.data_ptr(), tb.data_ptr(),
                                     c.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, dtm.STATUS.get(st, st)
        torch.cuda.synchronize()
        a_bits = oracle.encode(a, ind).reshape(-1)
        b_bits = oracle.encode(b, ind).reshape(-1)
        c64, _ = oracle.gemm(16, 16, 32, a_bits, 0, 32, 1, b_bits, 0, 16, 1, ind, "f32")
        got = c.cpu().numpy().astype(np.float64)
        bad = np.argwhere(got != c64)
        assert bad.size == 0, f"trial {trial}: {len(bad)} wrong, first {bad[:4].tolist()}"


def test_probe_rejects_bad_arguments():
    t = torch.zeros(512, dtype=torch.int16, device="cuda:0")
    c = torch.zeros(256, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    assert dtm.gemm_mfma_probe_raw(CODE["f32"], 0, 0, t.data_ptr(), t.data_ptr(), c.data_ptr(),
                                   s) == dtm.DTM_ERR_DTYPE
    assert dtm.gemm_mfma_probe_raw(CODE["f16"], 4, 0, t.data_ptr(), t.data_ptr(), c.data_ptr(),
                                   s) == dtm.DTM_ERR_CONFIG
    assert dtm.gemm_mfma_probe_raw(CODE["f16"], 0, 0, t.data_ptr() + 2, t.data_ptr(),
                                   c.data_ptr(), s) == dtm.DTM_ERR_STRIDE
    assert dtm.gemm_mfma_probe_raw(CODE["f16"], 0, 0, 0, t.data_ptr(), c.data_ptr(),
                                   s) == dtm.DTM_ERR_NULL_POINTER
