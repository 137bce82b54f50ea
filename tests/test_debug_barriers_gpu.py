"""A/B race check: every LDS-staged GEMM kernel form against the debug build
of the same sources (libdtm_gemm_debug.so, built with DTM_DEBUG_BARRIERS=1),
which waits for all outstanding loads and LDS accesses and then for the
whole workgroup at the top of every K iteration.  The arithmetic and its
order are the same in both builds, so any difference in the output bits
means a wait or barrier is missing in the normal build (the blocked loop of
"Chapter 13: The Blocked Matmul Kernel", section 13.1, must read each chunk
only after the whole chunk has landed).

Inputs are random (seeded), so an element read from a stage before its load
landed, or after the next chunk overwrote it, changes the result."""
import os

import pytest
import torch

import dense_tiled_matrix_amd as dtm

pytestmark = pytest.mark.gpu

MF16, MF32 = dtm.DTM_KERNEL_MFMA_F16, dtm.DTM_KERNEL_MFMA_F32
WK, GEN = dtm.DTM_KERNEL_MFMA_F16_WAVEK, dtm.DTM_KERNEL_GENERIC
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# (label, M, N, K, in dtype, out dtype, layout, config)
CASES = [
    ("pair 256 x 4 waves", 1024, 768, 2048, "bf16", "bf16", "NN",
     dict(kernel=MF16, block_m=256, block_n=256, block_k=32, threads=256)),
    ("pair 256 x 4 waves NT", 512, 1024, 1536, "f16", "f32", "NT",
     dict(kernel=MF16, block_m=256, block_n=256, block_k=32, threads=256)),
    ("pair 256 x 4 waves TT", 768, 512, 1024, "bf16", "f32", "TT",
     dict(kernel=MF16, block_m=256, block_n=256, block_k=32, threads=256)),
    ("pair 256 x 8 waves TN", 768, 768, 1024, "f16", "f16", "TN",
     dict(kernel=MF16, block_m=256, block_n=256, block_k=32, threads=512)),
    ("pair 192", 576, 384, 1024, "bf16", "bf16", "NN",
     dict(kernel=MF16, block_m=192, block_n=192, block_k=32)),
    ("four-stage 128", 512, 384, 1024, "f16", "f32", "NT",
     dict(kernel=MF16, block_m=128, block_n=128, block_k=32)),
    ("four-stage 128 ragged", 1000, 776, 1000, "bf16", "f32", "NN",
     dict(kernel=MF16, block_m=128, block_n=128, block_k=32)),
    ("split-K 128 x 4", 384, 256, 4096, "f16", "f32", "NN",
     dict(kernel=MF16, block_m=128, block_n=128, block_k=32, split_k=4)),
    ("wave-K", 256, 384, 4096, "bf16", "f32", "TN", dict(kernel=WK)),
    ("wave-K split 4", 512, 512, 8192, "f16", "f32", "NN", dict(kernel=WK, split_k=4)),
    ("register-staged 256", 512, 512, 1024, "f16", "f32", "NT",
     dict(kernel=MF16, block_m=256, block_n=256, block_k=64)),
    ("register-staged 128 ragged", 296, 200, 776, "bf16", "bf16", "TN",
     dict(kernel=MF16, block_m=128, block_n=128, block_k=64)),
    ("fp32 MFMA 256", 1024, 512, 512, "f32", "f32", "NN",
     dict(kernel=MF32, block_m=256, block_n=256, block_k=16)),
    ("fp32 MFMA 256 x 32 TT", 768, 512, 1024, "f32", "f32", "TT",
     dict(kernel=MF32, block_m=256, block_n=256, block_k=32)),
    ("fp32 MFMA 256 x 32 ragged", 600, 520, 1000, "f32", "f32", "NN",
     dict(kernel=MF32, block_m=256, block_n=256, block_k=32)),
    ("fp32 MFMA 192 ragged", 400, 580, 1000, "f32", "bf16", "NT",
     dict(kernel=MF32, block_m=192, block_n=192, block_k=32)),
    ("fp32 MFMA 128 ragged", 300, 260, 200, "f32", "f32", "NT",
     dict(kernel=MF32, block_m=128, block_n=128, block_k=16)),
    ("generic", 200, 136, 300, "f32", "f32", "TN",
     dict(kernel=GEN, block_m=64, block_n=64, block_k=16)),
]


def _operand(rows, cols, dtype, transposed, gen):
    """rows x cols values of `dtype`; `transposed` makes the view a transpose
    of a contiguous cols x rows array."""
    if transposed:
        return torch.randn(cols, rows, generator=gen).to(TD[dtype]).to("cuda:0").t()
    return torch.randn(rows, cols, generator=gen).to(TD[dtype]).to("cuda:0")


@pytest.fixture(scope="module")
def debug():
    if not os.path.exists(dtm.DEBUG_LIB_PATH):
        pytest.skip("libdtm_gemm_debug.so is not built "
                    "(python -m dense_tiled_matrix_amd.build)")
    if os.path.getmtime(dtm.DEBUG_LIB_PATH) < os.path.getmtime(dtm.LIB_PATH) - 600:
        pytest.skip("libdtm_gemm_debug.so is older than libdtm_gemm.so: rebuild both "
                    "(python -m dense_tiled_matrix_amd.build)")
    return dtm.debug_lib()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_same_bits_as_extra_barrier_build(case, debug):
    label, M, N, K, ind, outd, layout, cfg = case
    gen = torch.Generator().manual_seed(M * 7 + N * 3 + K)
    a = _operand(M, K, ind, layout[0] == "T", gen)
    b = _operand(K, N, ind, layout[1] == "T", gen)
    plan = dtm.gemm_plan(a, b, out_dtype=TD[outd], config=cfg)
    assert plan["kernel"] == cfg["kernel"], (label, plan)
    assert all(plan[k] == v for k, v in cfg.items() if k.startswith("block")), (label, plan)
    ws = torch.empty(max(plan["workspace_bytes"], 16) // 4, dtype=torch.float32,
                     device="cuda:0")
    c0 = torch.full((M, N), float("nan"), dtype=TD[outd], device="cuda:0")
    c1 = torch.full((M, N), float("nan"), dtype=TD[outd], device="cuda:0")
    dtm.gemm_ex(a, b, out=c0, config=cfg, workspace=ws)
    dtm.gemm_ex(a, b, out=c1, config=cfg, workspace=ws, library=debug)
    torch.cuda.synchronize()
    ibits = torch.int32 if outd == "f32" else torch.int16
    same = torch.equal(c0.view(ibits), c1.view(ibits))
    assert not torch.isnan(c0).any(), label
    assert same, f"{label}: {int((c0.view(ibits) != c1.view(ibits)).sum())} elements differ"
