"""The call boundary on the device: gemm() allocates and frees nothing and
does not wait for the GPU, even on a plan that splits K (its partials live in
the workspace reserved beforehand for the stream); calls on one stream from
several host threads queue their launches one call at a time.  The long-K
skinny workload (512 x 512 x 65536 fp16 -> fp32) is the split plan used."""
import threading
import time

import numpy as np
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import oracle
import workloads as W
from gpu_util import CODE, compare, dev_storage, note

pytestmark = pytest.mark.gpu


def _skinny_on_device():
    p = W.workload("f16_skinny512x512x65536_f32out")
    sa, sb = dev_storage(p.A.bits, "f16"), dev_storage(p.B.bits, "f16")
    return p, sa, sb


def _raw_gemm(p, sa, sb, c, stream):
    return dtm.gemm_raw(p.M, p.N, p.K, sa.data_ptr(), p.K, 1, sb.data_ptr(), p.N, 1, c.data_ptr(),
                        p.N, 1, CODE["f16"], CODE["f32"], stream=stream)


def test_split_plan_allocates_nothing_and_does_not_wait():
    """With the workspace reserved, the skinny workload's gemm() (K split 16
    ways, 16 MiB of partials) leaves the device's free memory unchanged and
    returns while earlier work on its stream is still running."""
    p, sa, sb = _skinny_on_device()
    stream = torch.cuda.current_stream()
    assert dtm.workspace_reserved() >= 16 * 512 * 512 * 4
    a_big = torch.randn(8192, 8192, device="cuda:0").to(torch.bfloat16)
    c_big = torch.empty(8192, 8192, dtype=torch.bfloat16, device="cuda:0")
    c = torch.empty(p.M, p.N, dtype=torch.float32, device="cuda:0")
    # first calls: the runtime loads each kernel's code object on its first
    # launch (the skinny plan's kernels and the big GEMM's live in different
    # ones), so nothing lazy is left inside the measured window
    assert _raw_gemm(p, sa, sb, c, stream.cuda_stream) == 0
    dtm.gemm(a_big, a_big, out=c_big)
    torch.cuda.synchronize()
    ref = c.clone()
    free0, _ = torch.cuda.mem_get_info()
    # about 10 ms of earlier work on the stream
    for _ in range(12):
        dtm.gemm(a_big, a_big, out=c_big)
    t0 = time.perf_counter()
    st = _raw_gemm(p, sa, sb, c, stream.cuda_stream)
    host_s = time.perf_counter() - t0
    done = torch.cuda.Event()
    done.record(stream)
    still_running = not done.query()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    note(f"split gemm(): {host_s * 1e6:.1f} us on the host; earlier work still running: "
         f"{still_running}; free memory change {free1 - free0} bytes")
    assert st == 0
    assert still_running and host_s < 2e-3
    assert free1 == free0
    assert torch.equal(c, ref)
    plan = dtm.gemm_plan(torch.empty(p.M, p.K, dtype=torch.float16, device="cuda:0"),
                         torch.empty(p.K, p.N, dtype=torch.float16, device="cuda:0"),
                         out_dtype=torch.float32)
    assert plan["split_k"] == 16, plan


def test_stream_without_workspace_runs_unsplit():
    """On a stream with nothing reserved the same call plans no split (it
    cannot allocate one) and gives a result within tolerance; after a
    reservation on that stream it splits, bit-identical to the default
    stream's split result."""
    p, sa, sb = _skinny_on_device()
    s = torch.cuda.Stream()
    assert dtm.workspace_reserved(stream=s) == 0
    c = torch.empty(p.M, p.N, dtype=torch.float32, device="cuda:0")
    free0, _ = torch.cuda.mem_get_info()
    assert _raw_gemm(p, sa, sb, c, s.cuda_stream) == 0
    s.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    c64, cout = oracle.gemm_problem(p)
    err, tol = compare(p, c.cpu().numpy().view(np.uint32), c64=c64, cout=cout,
                       label="skinny unsplit")
    note(f"skinny on a stream without workspace (unsplit): max err {err:.3e} tol {tol:.3e}")
    dtm.reserve_workspace(16 * 512 * 512 * 4, stream=s)
    c2 = torch.empty_like(c)
    assert _raw_gemm(p, sa, sb, c2, s.cuda_stream) == 0
    s.synchronize()
    c3 = torch.empty_like(c)
    assert _raw_gemm(p, sa, sb, c3, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(c2, c3)
    dtm.release_workspace(stream=s)
    assert dtm.workspace_reserved(stream=s) == 0


def test_threads_sharing_a_stream():
    """Four host threads call the split plan on the default stream at once,
    each with its own inputs and output: every result equals that input's
    result computed alone, bit for bit (the partial products of one call are
    summed before another call's partials can overwrite the workspace)."""
    M = N = 512
    K = 16384
    torch.manual_seed(3)
    ins = [(torch.randn(M, K, device="cuda:0").half(), torch.randn(K, N, device="cuda:0").half())
           for _ in range(4)]
    plan = dtm.gemm_plan(ins[0][0], ins[0][1], out_dtype=torch.float32)
    assert plan["split_k"] > 1, plan
    refs = [dtm.gemm(a, b, out_dtype=torch.float32) for a, b in ins]
    torch.cuda.synchronize()
    outs = [[torch.empty(M, N, device="cuda:0") for _ in range(25)] for _ in range(4)]
    errors = []
    stream = torch.cuda.current_stream()

    def worker(t):
        try:
            torch.cuda.set_device(0)
            a, b = ins[t]
            for c in outs[t]:
                st = dtm.gemm_raw(M, N, K, a.data_ptr(), K, 1, b.data_ptr(), N, 1, c.data_ptr(),
                                  N, 1, CODE["f16"], CODE["f32"], stream=stream.cuda_stream)
                if st != 0:
                    errors.append((t, st))
        except Exception as e:  # reported below
            errors.append((t, repr(e)))

    th = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(4):
        for c in outs[t]:
            assert torch.equal(c, refs[t]), t
    note(f"4 threads x 25 split-K calls (S = {plan['split_k']}) on one stream: all equal")
