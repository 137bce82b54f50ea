"""gemm_ex_noalloc, the entry point for callers that cannot allocate: its
split-K partials live in the library's fixed device array.  Two calls in a
row, the second with a smaller problem, each equal bit for bit to gemm_ex
with a caller's workspace running the same plan (and within the oracle's
tolerance); no call changes the device's free memory; a forced split that
needs more than the array holds is refused with nothing written."""
import numpy as np
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import workloads as W
from gpu_util import CODE, compare, dev_storage, note

pytestmark = pytest.mark.gpu


def _problem_on_device(p):
    sa, sb = dev_storage(p.A.bits, p.in_dtype), dev_storage(p.B.bits, p.in_dtype)
    return sa, sb


def _args(p, sa, sb, c):
    return (p.M, p.N, p.K, sa.data_ptr(), p.A.stride_r, p.A.stride_c, sb.data_ptr(),
            p.B.stride_r, p.B.stride_c, c.data_ptr(), p.N, 1, CODE[p.in_dtype],
            CODE[p.out_dtype])


def test_noalloc_matches_gemm_ex_twice():
    scratch = dtm.gemm_noalloc_scratch_bytes()
    assert scratch == 32 << 20
    stream = torch.cuda.current_stream().cuda_stream
    big = W.workload("f16_skinny512x512x65536_f32out")  # K split 16 ways: 16 MiB of partials
    small = W.random_problem(256, 384, 8192, "bf16", "bf16", ("normal", 0.0, 1.0), seed=4242)
    first = True
    for n, p in enumerate([big, small]):
        sa, sb = _problem_on_device(p)
        TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
        c = torch.full((p.M, p.N), float("nan"), dtype=TD[p.out_dtype], device="cuda:0")
        ref = torch.full_like(c, float("nan"))
        st, plan = dtm.gemm_plan_raw(*_args(p, sa, sb, c), config=dict(workspace_limit=scratch))
        assert st == 0 and plan["split_k"] > 1, plan
        note(f"call {n + 1}: {p.M}x{p.N}x{p.K} {p.in_dtype}->{p.out_dtype}, "
             f"split {plan['split_k']}, {plan['workspace_bytes']} bytes of scratch")
        ws = torch.empty(plan["workspace_bytes"] // 4, dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        # gemm_ex first: the runtime loads a kernel's code on its first launch
        # in a process and takes device memory for it (4 MiB when this test
        # runs alone), which no gemm_ex_noalloc call must be blamed for; the
        # array keeps the previous no-alloc call's contents meanwhile
        free_warm = torch.cuda.mem_get_info()[0]
        st = dtm.gemm_ex_raw(*_args(p, sa, sb, ref), config=dict(split_k=plan["split_k"],
                                                                 kernel=plan["kernel"],
                                                                 block_m=plan["block_m"],
                                                                 block_n=plan["block_n"],
                                                                 block_k=plan["block_k"]),
                             workspace=ws.data_ptr(), workspace_bytes=plan["workspace_bytes"],
                             stream=stream)
        assert st == 0, dtm.STATUS.get(st, st)
        torch.cuda.synchronize()
        note(f"call {n + 1}: gemm_ex changed free device memory by "
             f"{torch.cuda.mem_get_info()[0] - free_warm} bytes")
        if first:
            # the first call on the device finds its copy of the array
            assert dtm.gemm_ex_noalloc_raw(*_args(p, sa, sb, c), stream=stream) == 0
            torch.cuda.synchronize()
            first = False
        # every tensor of this round is allocated and every kernel loaded: the
        # call alone must not change the device's free memory
        free_before = torch.cuda.mem_get_info()[0]
        st = dtm.gemm_ex_noalloc_raw(*_args(p, sa, sb, c), stream=stream)
        assert st == 0, dtm.STATUS.get(st, st)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free_before
        bits = np.uint32 if p.out_dtype == "f32" else np.uint16
        ints = torch.int32 if p.out_dtype == "f32" else torch.int16
        got = c.view(ints).cpu().numpy().view(bits)
        want = ref.view(ints).cpu().numpy().view(bits)
        assert np.array_equal(got, want), f"call {n + 1}: differs from gemm_ex"
        err, tol = compare(p, got, label=f"noalloc call {n + 1}")
        note(f"call {n + 1}: equal to gemm_ex; max err {err:.3e} tol {tol:.3e}")


def test_noalloc_refuses_a_split_beyond_the_array():
    p = W.random_problem(1024, 1024, 65536 // 4, "f16", "f32", ("uniform", 0.0, 1.0), seed=99)
    sa, sb = _problem_on_device(p)
    c = torch.full((p.M, p.N), 7.0, device="cuda:0")
    cfg = dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=128, block_n=128, block_k=32, split_k=16)
    st, plan = dtm.gemm_plan_raw(*_args(p, sa, sb, c), config=cfg)
    assert st == 0 and plan["workspace_bytes"] == 16 * 1024 * 1024 * 4 > (32 << 20)
    st = dtm.gemm_ex_noalloc_raw(*_args(p, sa, sb, c), config=cfg,
                                 stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == dtm.DTM_ERR_SCRATCH, dtm.STATUS.get(st, st)
    assert "scratch" in dtm.gemm_status_string(st)
    assert bool((c == 7.0).all())
    # the selector's own plan for the same problem fits the array and runs
    st = dtm.gemm_ex_noalloc_raw(*_args(p, sa, sb, c),
                                 stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    compare(p, c.cpu().numpy().view(np.uint32), label="noalloc selector plan")
