"""The calls inside a captured HIP graph: gemm() and row_softmax() are
captured on a stream (after one eager call of each plan, so the code objects
are loaded) and the graph is replayed several times, with eager work and
synchronisation between the replays; every replay must give the eager
result bit for bit.  The calls allocate nothing and record no memset, so a
replay repeats exactly the launches of the eager call (the blocked product
of "Chapter 13: The Blocked Matmul Kernel", section 13.1, split K included,
and the row softmax of "Triton from zero, Lesson 4: Block Pointers")."""
import pytest
import torch

import dense_tiled_matrix_amd as dtm

pytestmark = pytest.mark.gpu

# (label, M, N, K, in dtype, out dtype, expected kernel)
CASES = [
    ("bf16 paired stages", 1024, 1024, 2048, torch.bfloat16, torch.bfloat16, "mfma_f16"),
    ("fp16 long K, wave-K split 16 + reduce", 512, 512, 65536, torch.float16, torch.float32,
     "mfma_f16_wavek"),
    ("fp32 ragged", 1000, 600, 300, torch.float32, torch.float32, "mfma_f32"),
]


def _bits(t):
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gemm_graph_replays_match_eager(case):
    label, M, N, K, dt, od, kernel = case
    s = torch.cuda.Stream()
    dtm.reserve_workspace(stream=s)
    gen = torch.Generator().manual_seed(M + N + K)
    a = torch.randn(M, K, generator=gen).to(dt).to("cuda:0")
    b = torch.randn(K, N, generator=gen).to(dt).to("cuda:0")
    c = torch.empty(M, N, dtype=od, device="cuda:0")
    plan = dtm.gemm_plan(a, b, out=c)
    assert plan["kernel_name"] == kernel, (label, plan)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dtm.gemm(a, b, out=c, stream=s)  # eager: loads the code objects
    s.synchronize()
    ref = c.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dtm.gemm(a, b, out=c, stream=s)
    for r in range(3):
        c.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(c), _bits(ref)), f"{label}: replay {r} differs"
    assert plan["split_k"] == (16 if "split" in label else 1)


def test_softmax_graph_replays_match_eager():
    s = torch.cuda.Stream()
    dtm.reserve_workspace(stream=s)
    gen = torch.Generator().manual_seed(7)
    x = torch.randn(4096, 4096, generator=gen).to("cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dtm.row_softmax(x, out=y, stream=s)
    s.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dtm.row_softmax(x, out=y, stream=s)
    for r in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(ref)), f"softmax: replay {r} differs"
