"""GPU parity of the wave-K kernel (128 x 128 x 32 tiles whose 4 waves each
accumulate the whole tile over every fourth 32-deep chunk of the K loop of
"Chapter 13: The Blocked Matmul Kernel", section 13.1, and sum the four
partial tiles in LDS), forced through gemm_ex, against the CPU oracle.

Bar: value-exact on integer-valued inputs (every partial sum an integer
below 2^24); on random inputs within the stated tolerance and the
Higham-style bound gamma_K (|A| |B|) of the oracle's fp64 product."""
import numpy as np
import pytest

import dense_tiled_matrix_amd as dtm
import oracle
import workloads as W
from gpu_util import compare, higham_ratio, note, run
from test_gpu_parity import LAYOUT_BITS, padded_int_problem

pytestmark = pytest.mark.gpu

WK = dtm.DTM_KERNEL_MFMA_F16_WAVEK


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_wavek_layouts_exact(ind, layout):
    """1, 2, 3 and many 128-deep regions per slice (the loop's odd and even
    trip counts, with and without split-K: the five LDS slots' rotation from
    its first state), several grids, padded leading dimensions, every output
    dtype: value-exact."""
    shapes = [(128, 128, 128, 1), (256, 128, 256, 1), (128, 384, 384, 1), (384, 256, 2048, 1),
              (512, 512, 8192, 4), (256, 256, 4096, 8), (256, 384, 640, 1),
              (256, 256, 512, 4), (256, 128, 1024, 4), (128, 256, 1536, 4)]
    for n, (M, N, K, S) in enumerate(shapes):
        outd = ["f32", "f16", "bf16"][n % 3]
        p = padded_int_problem(M, N, K, ind, outd, 8 if K <= 512 else 2, seed=900 + n,
                               extra=8 * (n % 2), a_layout=layout[0], b_layout=layout[1])
        cfg = dict(kernel=WK, split_k=S)
        plan = {}
        c, untouched = run(p, config=cfg, c_pad=4 if n % 2 else 0, plan=plan)
        assert plan["status"] == 0 and plan["kernel"] == WK and plan["split_k"] == S, plan
        assert plan["layout"] == LAYOUT_BITS[layout], plan
        compare(p, c, exact=True, label=f"wave-K {layout} {ind} {M}x{N}x{K} S{S}->{outd}")
        assert untouched


def test_wavek_long_k_random():
    """The long-K workload (512 x 512 x 65536 fp16 U[0,1] -> fp32) forced on
    the wave-K kernel with K split 16 ways: every element within the stated
    tolerance and the Higham bound; two calls give identical bits."""
    p = W.workload("f16_skinny512x512x65536_f32out")
    cfg = dict(kernel=WK, split_k=16)
    c, untouched = run(p, config=cfg)
    c2, _ = run(p, config=cfg)
    assert np.array_equal(c, c2)
    c64, cout = oracle.gemm_problem(p)
    err, tol = compare(p, c, c64=c64, cout=cout, label="wave-K long K")
    ratio = higham_ratio(p, c, c64)
    note(f"wave-K {p.name}: err/tol {err / tol:.2e}; Higham ratio {ratio:.3f}")
    assert ratio <= 1.0
    assert untouched


@pytest.mark.parametrize("layout", ["NN", "NT"])
def test_wavek_random_bf16(layout):
    """N(0,1) bf16 -> bf16, 1024 x 768 x 4096 with K split 2 ways, against
    the oracle within the stated tolerance."""
    p = W.random_problem(1024, 768, 4096, "bf16", "bf16", ("normal", 0.0, 1.0), seed=930,
                         a_layout=layout[0], b_layout=layout[1])
    c, untouched = run(p, config=dict(kernel=WK, split_k=2))
    err, tol = compare(p, c, label=f"wave-K {layout} bf16 1024x768x4096")
    note(f"wave-K {layout}: max err {err:.3e} tol {tol:.3e}")
    assert untouched


def test_wavek_selector_random():
    """1536 x 1536 x 8192 bf16 N(0,1) -> bf16 through the selector's plan
    (the wave-K kernel unsplit: 144 tiles of 128 with an 8192-long K loop),
    compared in full with the oracle within the stated tolerance and the
    Higham bound."""
    p = W.random_problem(1536, 1536, 8192, "bf16", "bf16", ("normal", 0.0, 1.0), seed=940)
    plan = {}
    c, untouched = run(p, plan=plan)
    assert plan["kernel"] == WK and plan["split_k"] == 1 and plan["block_m"] == 128, plan
    c64, cout = oracle.gemm_problem(p)
    err, tol = compare(p, c, c64=c64, cout=cout, label="wave-K selector 1536x1536x8192")
    ratio = higham_ratio(p, c, c64)
    note(f"wave-K selector 1536x1536x8192: err/tol {err / tol:.2e}; Higham ratio {ratio:.3f}")
    assert ratio <= 1.0
    assert untouched
