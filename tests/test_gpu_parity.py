"""GPU parity: the HIP kernels through the C ABI against the CPU oracle.

Bar: value-exact for integer-valued inputs (every partial sum is an integer
below 2^24, so fp32 accumulation is exact in any order and only the final
round-to-nearest-even conversion remains); otherwise per element
|C - C64| <= 1e-5*K*max|a|*max|b| (fp32 inputs) or 4e-3*sqrt(K)*max|a|*max|b|
(fp16/bf16 inputs), plus half an output ulp for fp16/bf16 outputs, with C64
the oracle's fp64 result on the same rounded inputs.
"""
import numpy as np
import pytest
import torch

import dense_tiled_matrix_amd as dtm
import oracle
import workloads as W
from conftest import read_golden
from gpu_util import compare, dev_storage, higham_ratio, note, run

pytestmark = pytest.mark.gpu

GEN = dtm.DTM_KERNEL_GENERIC
MF16 = dtm.DTM_KERNEL_MFMA_F16
ACC16 = dtm.DTM_KERNEL_GENERIC_FP16ACC
T444 = dict(kernel=GEN, block_m=4, block_n=4, block_k=4)
LAYOUT_BITS = {"NN": 0, "TN": dtm.DTM_LAYOUT_A_M_CONTIG, "NT": dtm.DTM_LAYOUT_B_K_CONTIG,
               "TT": dtm.DTM_LAYOUT_A_M_CONTIG | dtm.DTM_LAYOUT_B_K_CONTIG}


def int_problem(M, N, K, ind, outd, R, seed, la="N", lb="N"):
    return W.random_problem(M, N, K, ind, outd, ("int", -R, R), seed, la, lb,
                            name=f"int{M}x{N}x{K}")


def padded_int_problem(M, N, K, ind, outd, R, seed, extra=0, a_layout="N", b_layout="N"):
    """Integer-valued operands whose leading dimensions are rounded up to a
    multiple of 8 elements (16 bytes), plus ``extra``; the padding holds NaN,
    which must never be read.  Layout "N" stores an operand row-major (A
    K-contiguous, B N-contiguous); "T" stores its transpose row-major, so the
    view has stride 1 along M (A) or K (B)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-R, R + 1, size=(M, K))
    b = rng.integers(-R, R + 1, size=(K, N))

    def store(x, layout, name):
        rows, cols = x.shape
        if layout == "T":
            x = x.T
        ld = -(-x.shape[1] // 8) * 8 + extra
        buf = np.full((x.shape[0], ld), np.nan)
        buf[:, :x.shape[1]] = x
        strides = (ld, 1) if layout == "N" else (1, ld)
        return W.Operand(W.to_bits(buf, ind).reshape(-1), ind, rows, cols, 0, *strides)

    A = store(a, a_layout, "A")
    B = store(b, b_layout, "B")
    return W.Problem(M, N, K, A, B, ind, outd, name=f"pad{a_layout}{b_layout}{M}x{N}x{K}")


# ----------------------------------------------------------- the pages' cases


def test_worked_2x2_forced_4x4x4():
    """The 2x2 single-tile product through one ragged 4x4x4 tile."""
    p = W.worked_2x2()
    c, untouched = run(p, config=T444)
    assert oracle.decode(c, "f32").tolist() == [[19.0, 22.0], [43.0, 50.0]]
    assert untouched


def test_int8x8x8_forced_4x4x4_grid_2x2():
    """Integer-valued fp32 8x8x8 with 4x4x4 tiles: a (2, 2) grid and two
    K-iterations per tile (Worked Example 13.1.1's launch); exact."""
    p = W.workload("int8x8x8_f32")
    a = torch.empty(8, 8, device="cuda:0")
    assert dtm.gemm_plan(a, a, config=T444)["k_iters"] == 2
    c, untouched = run(p, config=T444)
    compare(p, c, exact=True, label="int8x8x8")
    assert untouched


@pytest.mark.parametrize("M,K,N", [(8, 8, 8), (5, 7, 6)])
def test_pages_arange_cases(M, K, N):
    """Worked Examples 13.1.1 and 13.2.1 (0.1*arange inputs, fp32, 4x4x4)."""
    p = W.arange_problem(M, K, N, scale=0.1)
    c, _ = run(p, config=T444)
    compare(p, c, label=f"arange{M}x{K}x{N}")
    c, _ = run(p)  # the selector's own choice
    compare(p, c, label=f"arange{M}x{K}x{N} default")


@pytest.mark.parametrize("sentinel", [999.0, float("nan"), float("inf")])
@pytest.mark.parametrize("config", [T444, None])
def test_sentinel_views(sentinel, config):
    """Worked Example 13.2.2: A and B are views into buffers whose other slots
    hold a sentinel.  The result must equal the K-masked table; C sits inside
    a NaN-filled buffer whose other slots must stay untouched."""
    p = W.sentinel_problem(sentinel)
    c, untouched = run(p, config=config, c_pad=3)
    want = oracle.gemm_problem(W.sentinel_problem(999.0))
    compare(p, c, c64=want[0], cout=want[1], label=f"sentinel {sentinel}")
    assert untouched


@pytest.mark.parametrize("ind", ["f16", "bf16"])
@pytest.mark.parametrize("sentinel", [999.0, float("nan")])
def test_sentinel_views_mfma(ind, sentinel):
    """The sentinel construction on the MFMA kernel: A is the first K columns
    of a wider buffer, B the first K rows and N columns of a larger one, both
    with 16-byte-aligned leading dimensions; every other slot is a sentinel."""
    M, K, N, ldA, ldB = 40, 37, 50, 64, 72
    rng = np.random.default_rng(1)
    abuf = np.full((M, ldA), sentinel)
    abuf[:, :K] = rng.integers(-8, 9, size=(M, K))
    bbuf = np.full((K + 9, ldB), sentinel)
    bbuf[:K, :N] = rng.integers(-8, 9, size=(K, N))
    A = W.Operand(W.to_bits(abuf, ind).reshape(-1), ind, M, K, 0, ldA, 1)
    B = W.Operand(W.to_bits(bbuf, ind).reshape(-1), ind, K, N, 0, ldB, 1)
    p = W.Problem(M, N, K, A, B, ind, "f32")
    cfg = dict(kernel=MF16, block_m=128, block_n=128, block_k=64)
    c, untouched = run(p, config=cfg, c_pad=5)
    compare(p, c, exact=True, label=f"sentinel mfma {ind} {sentinel}")
    assert untouched


def test_seed0_accumulation_fp16_out():
    """Section 13.3's inputs (4x1024x4 fp16, fp16 output): the fp32
    accumulator keeps the result at one final rounding of the exact sum, so
    its max error against the fp64 truth matches the printed fp32-accumulator
    figure, far below the fp16-accumulator one."""
    p = W.seed0_fp16_problem()
    c64, c16 = oracle.gemm_problem(p)
    fp16acc = oracle.decode(oracle.gemm_fp16acc_problem(p, 8), "f16")
    for config in [dict(kernel=GEN, block_m=4, block_n=4, block_k=4), None]:
        c, _ = run(p, config=config)
        got = oracle.decode(c, "f16")
        err = float(np.abs(got - c64).max())
        note(f"fp32-acc err {err!r} vs fp16-acc err {float(np.abs(fp16acc - c64).max())!r}")
        # equal to rne16(C64) except where the fp32 sum falls on the other side
        # of an fp16 rounding boundary
        assert (got != oracle.decode(c16, "f16")).sum() <= 2
        assert err <= 9.737179152580211e-05 * 1.01
        assert err * 10 < float(np.abs(fp16acc - c64).max())


# --------------------------------------- the fp16-accumulator negative control


def _fp16acc_against_emulation(p, cfg, label):
    """The on-device fp16-accumulator kernel against the oracle's emulation
    of section 13.3 with the same BLOCK_K.  The two differ only in how a
    chunk's tile product is formed before its rounding to fp16: an fp32 FMA
    chain on the device, the exact sum in the oracle.  They round to
    different fp16 values only when the exact sum lies within the fp32
    chain's error (about sqrt(BLOCK_K) * 2^-24 relative) of an fp16 rounding
    boundary, an event of probability ~2^-12 per chunk; each such event moves
    the fp16 accumulator by about one fp16 ulp, and fp16 additions of the
    same later chunk values keep that offset.  Bound: a few ulps at the
    result's magnitude, on a small fraction of the outputs."""
    c, untouched = run(p, out_dtype="f16", config=cfg)
    emu = oracle.gemm_fp16acc_problem(p, cfg["block_k"])
    got, want = oracle.decode(c, "f16"), oracle.decode(emu, "f16")
    top = max(float(np.abs(want).max()), 2.0 ** -14)
    ulp = 2.0 ** (np.floor(np.log2(top)) - 10)
    ndiff = int((c != emu).sum())
    maxd = float(np.abs(got - want).max())
    note(f"{label}: {ndiff} of {c.size} outputs differ from the emulation, max {maxd:.3e} "
         f"(fp16 ulp at |C| {ulp:.3e})")
    assert untouched
    assert maxd <= 4 * ulp
    assert ndiff <= max(2, c.size // 20)
    return got


@pytest.mark.parametrize("bk", [8, 4])
def test_fp16acc_control_seed0(bk):
    """Worked Example 13.3.1 on the device with the fp16 accumulator: the
    max error against the fp64 truth is the printed fp16-accumulator figure
    (up to the fp32-versus-exact chunk product), more than 10x the fp32
    accumulator's printed figure."""
    g = {t[0]: t[1] for t in read_golden("accumulation_seed0.txt")["_"]}
    p = W.seed0_fp16_problem()
    cfg = dict(kernel=ACC16, block_m=128, block_n=128, block_k=8) if bk == 8 else \
        dict(kernel=ACC16, block_m=4, block_n=4, block_k=4)
    got = _fp16acc_against_emulation(p, cfg, f"seed0 BLOCK_K {bk}")
    c64, _ = oracle.gemm_problem(p)
    err = float(np.abs(got - c64).max())
    note(f"seed0 BLOCK_K {bk}: fp16-acc max error {err!r} (printed for BLOCK_K 8: "
         f"{g['fp16acc_max_abs_diff']!r})")
    assert err > 10 * float(g["fp32acc_max_abs_diff"])
    if bk == 8:
        assert abs(err - float(g["fp16acc_max_abs_diff"])) <= 2 * 2.0 ** -16


def test_fp16acc_control_long_k():
    """The long-K workload's 64 x 64 corner (fp16 U[0,1], K = 65536) with the
    fp16 accumulator on the device: it follows the emulation, and its error
    against the fp64 truth is over 100x that of the fp32-accumulating
    split-K path on the same corner."""
    w = W.workload("f16_skinny512x512x65536_f32out")
    A2, B2 = w.A.bits.reshape(w.M, w.K), w.B.bits.reshape(w.K, w.N)
    p = W.Problem(64, 64, w.K, W.dense(np.ascontiguousarray(A2[:64]), "f16"),
                  W.dense(np.ascontiguousarray(B2[:, :64]), "f16"), "f16", "f32",
                  name="skinny corner")
    got = _fp16acc_against_emulation(p, dict(kernel=ACC16, block_m=64, block_n=64, block_k=16),
                                     "long-K corner BLOCK_K 16")
    c64, _ = oracle.gemm_problem(p)
    c32, _ = run(p, out_dtype="f32")
    err16 = float(np.abs(got - c64).max())
    err32 = float(np.abs(oracle.decode(c32, "f32") - c64).max())
    note(f"long-K corner: fp16-acc max error {err16:.4g}, fp32-acc {err32:.3e}")
    assert err16 > 100 * err32


# ------------------------------------------------------ the measured workloads


def test_ragged_f32_transposed_a():
    """257x129x193 fp32, A a transposed view (strides (1, 257)), N(0,1)."""
    p = W.workload("ragged257x129x193_f32_At")
    assert (p.A.stride_r, p.A.stride_c) == (1, 257)
    c, untouched = run(p)
    c64, cout = oracle.gemm_problem(p)
    err, tol = compare(p, c, c64=c64, cout=cout, label="ragged257")
    ratio = higham_ratio(p, c, c64)
    note(f"ragged257x129x193 f32: max err {err:.3e} tol {tol:.3e} (err/tol {err / tol:.2e}); "
         f"Higham ratio {ratio:.3f}")
    assert ratio <= 1.0
    assert untouched


def _big_check(p, tile, threads=None, kernel="mfma_f16"):
    """Full-size run in the launch configuration the bench times, compared
    with the oracle on every element of C (Worked Example 13.3.1's method:
    the fp64 truth from the same rounded inputs), and the Higham ratio of
    the error against the worst-case fp32 accumulation bound."""
    note(f"{p.name}: {p.M}x{p.N}x{p.K} {p.in_dtype}->{p.out_dtype}")
    sa, sb = dev_storage(p.A.bits, p.in_dtype), dev_storage(p.B.bits, p.in_dtype)
    TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    a = sa.view(TD[p.in_dtype]).view(p.M, p.K)
    b = sb.view(TD[p.in_dtype]).view(p.K, p.N)
    plan = dtm.gemm_plan(a, b, out_dtype=TD[p.out_dtype])
    assert plan["kernel_name"] == kernel and plan["block_m"] == tile, plan
    assert threads is None or plan["threads"] == threads, plan
    c = dtm.gemm(a, b, out_dtype=TD[p.out_dtype])
    torch.cuda.synchronize()
    cb = c.view(torch.int32 if p.out_dtype == "f32" else torch.int16).cpu().numpy()
    cb = cb.view(np.uint32 if p.out_dtype == "f32" else np.uint16)
    del c, a, b, sa, sb
    c64, cout = oracle.gemm_problem(p)
    err, tol = compare(p, cb, c64=c64, cout=cout, label=p.name)
    ratio = higham_ratio(p, cb, c64)
    note(f"{p.name}: max err {err:.3e} tol {tol:.3e} (err/tol {err / tol:.2e}); "
         f"Higham ratio {ratio:.3f}")
    assert ratio <= 1.0
    return err, tol


def test_f16_4096_f32out():
    _big_check(W.workload("f16_4096_f32out"), 256, threads=256)


def test_bf16_8192_bf16out():
    _big_check(W.workload("bf16_8192_bf16out"), 256, threads=256)


def test_f16_8192_f32out():
    """Extra: fp16 8192^3 with fp32 output (the 4-wave form)."""
    _big_check(W.workload("f16_8192_f32out"), 256, threads=256)


def test_bf16_4096_bf16out():
    """Extra: bf16 4096^3 with bf16 output (one tile per CU, 4 waves)."""
    _big_check(W.workload("bf16_4096_bf16out"), 256, threads=256)


def test_f32_4096_f32out():
    """Extra: fp32 4096^3 on the fp32 matrix cores (256-wide tiles, one per
    CU), compared on every element, with its Higham ratio."""
    _big_check(W.workload("f32_4096_f32out"), 256, threads=256, kernel="mfma_f32")


def test_f16_skinny_long_k():
    """512x512x65536 fp16 U[0,1] -> fp32 through the selector's split-K plan
    (16 slices of 4096 on the pipelined kernel's 128-wide tiles): full
    comparison, plus the
    accumulation-error report against section 13.3's fp16 accumulator
    (emulated by the oracle on a 64x64 corner with the kernel's BLOCK_K)."""
    p = W.workload("f16_skinny512x512x65536_f32out")
    note(f"{p.name}: {p.M}x{p.N}x{p.K}")
    a = torch.empty(p.M, p.K, dtype=torch.float16, device="cuda:0")
    b = torch.empty(p.K, p.N, dtype=torch.float16, device="cuda:0")
    plan = dtm.gemm_plan(a, b, out_dtype=torch.float32)
    assert (plan["split_k"], plan["block_k"], plan["block_m"]) == (16, 32, 128), plan
    c, untouched = run(p)
    c64, cout = oracle.gemm_problem(p)
    err, tol = compare(p, c, c64=c64, cout=cout, label=p.name)
    ratio = higham_ratio(p, c, c64)
    note(f"{p.name}: err/tol {err / tol:.2e}; Higham ratio {ratio:.3f}")
    assert ratio <= 1.0
    plan_bk = 32
    A2, B2 = p.A.bits.reshape(p.M, p.K), p.B.bits.reshape(p.K, p.N)
    corner = oracle.gemm_fp16acc(64, 64, p.K, np.ascontiguousarray(A2[:64]), 0, p.K, 1,
                                 np.ascontiguousarray(B2[:, :64]), 0, 64, 1, "f16", plan_bk)
    err16 = float(np.abs(oracle.decode(corner, "f16") - c64[:64, :64]).max())
    gerr = float(np.abs(oracle.decode(c, "f32")[:64, :64] - c64[:64, :64]).max())
    note(f"long-K: fp32-acc max err {err:.3e} (corner {gerr:.3e}) vs fp16-acc emulation "
         f"{err16:.3e} (BLOCK_K {plan_bk}); tol {tol:.3e}")
    assert gerr * 100 < err16
    assert untouched


# ------------------------------------------------------------ ragged sweeps

EDGE = [1, 2, 3, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _sweep_shapes(n, seed):
    rng = np.random.default_rng(seed)
    shapes = [(1, 1, 1), (257, 257, 257), (129, 1, 65), (1, 300, 1), (64, 64, 1)]
    while len(shapes) < n:
        shapes.append(tuple(int(x) for x in rng.choice(EDGE, size=3)))
    return shapes


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("ind", ["f16", "bf16"])
@pytest.mark.parametrize("tile", [128, 256])
def test_mfma_ragged_sweep_exact(ind, tile, layout):
    """Integer-valued inputs on the register-staged MFMA kernel at edge sizes
    around the tile (both tiles), every output dtype, in each operand layout
    (a transposed operand is loaded along its contiguous axis and transposed
    in registers): value-exact."""
    cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=64)
    shapes = _sweep_shapes(14 if layout == "NN" else 8, seed=tile + len(ind) + 7 * len(layout))
    for n, (M, N, K) in enumerate(shapes):
        outd = ["f32", "f16", "bf16"][n % 3]
        p = padded_int_problem(M, N, K, ind, outd, 8, seed=100 + n, extra=8 * (n % 2),
                               a_layout=layout[0], b_layout=layout[1])
        plan = {}
        c, untouched = run(p, config=cfg, c_pad=2 if n % 2 else 0, plan=plan)
        assert plan["layout"] == LAYOUT_BITS[layout], plan
        compare(p, c, exact=True, label=f"{layout} {ind} {tile} {M}x{N}x{K}->{outd}")
        assert untouched


@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_mfma_pipelined_exact(ind):
    """The 256x256x32 pipelined kernel (global->LDS DMA, 4 stages) at every
    trip count of its pipeline (1, 2, 3, 4 and many K-chunks) and several
    grid shapes: value-exact on integer-valued inputs, all output dtypes."""
    cfg = dict(kernel=MF16, block_m=256, block_n=256, block_k=32)
    shapes = [(256, 256, 32), (256, 256, 64), (512, 256, 96), (256, 512, 128),
              (768, 512, 160), (512, 1024, 2048), (1280, 256, 4096)]
    for n, (M, N, K) in enumerate(shapes):
        outd = ["f32", "f16", "bf16"][n % 3]
        R = 8 if K <= 256 else 2
        p = padded_int_problem(M, N, K, ind, outd, R, seed=400 + n, extra=8 * (n % 2))
        c, untouched = run(p, config=cfg, c_pad=4 if n % 2 else 0)
        compare(p, c, exact=True, label=f"pipelined {ind} {M}x{N}x{K}->{outd}")
        assert untouched


@pytest.mark.parametrize("tile,threads", [(256, 512), (256, 256), (192, 256), (128, 256)])
@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_pipelined_layouts_exact(ind, layout, tile, threads):
    """Every operand layout on the pipelined kernel: 256-wide tiles with 8
    and with 4 waves, 192- and 128-wide tiles with 4 (A M-contiguous and/or
    B K-contiguous, staged as stored and read with transposing LDS reads):
    pipeline depths 1, 3, 5 and many chunks, several grids, padded leading
    dimensions, split-K; value-exact on integer-valued inputs."""
    u = 192 if tile == 192 else 256  # shapes in whole tiles of 192, else of 256
    shapes = [(u, u, 32, 1), (2 * u, u, 96, 1), (u, 3 * u, 160, 1), (3 * u, 2 * u, 2048, 1),
              (2 * u, 2 * u, 4096, 8), (u, u, 1024, 4)]
    for n, (M, N, K, S) in enumerate(shapes):
        outd = ["f32", "f16", "bf16"][n % 3]
        p = padded_int_problem(M, N, K, ind, outd, 8 if K <= 256 else 2, seed=600 + n,
                               extra=8 * (n % 2), a_layout=layout[0], b_layout=layout[1])
        cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=32, split_k=S,
                   threads=threads)
        plan = {}
        c, untouched = run(p, config=cfg, c_pad=4 if n % 2 else 0, plan=plan)
        assert plan["status"] == 0 and plan["block_k"] == 32 and plan["block_m"] == tile, plan
        assert plan["layout"] == LAYOUT_BITS[layout] and plan["split_k"] == S, plan
        assert plan["threads"] == threads and plan["ragged"] == 0, plan
        compare(p, c, exact=True,
                label=f"pipelined {tile} x{threads} {layout} {ind} {M}x{N}x{K} S{S}->{outd}")
        assert untouched


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
def test_pipelined_layouts_random(layout):
    """N(0,1) bf16 and U[-1,1] fp16 operands in every layout through the
    selector's plan, against the oracle within the stated tolerance."""
    for n, (ind, outd, dist) in enumerate([("bf16", "bf16", ("normal", 0.0, 1.0)),
                                          ("f16", "f32", ("uniform", -1.0, 1.0))]):
        p = W.random_problem(1024, 768, 1536, ind, outd, dist, seed=700 + n,
                             a_layout=layout[0], b_layout=layout[1])
        plan = {}
        c, untouched = run(p, plan=plan)
        assert plan["layout"] == LAYOUT_BITS[layout] and plan["block_k"] == 32, plan
        err, tol = compare(p, c, label=f"{layout} {ind} 1024x768x1536")
        note(f"{layout} {ind}->{outd}: max err {err:.3e} tol {tol:.3e}")
        assert untouched


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
def test_four_wave_selector_random(layout):
    """192 tiles of 256 and a 3072-long K loop: the selector's 4-wave form
    of the pipelined kernel, N(0,1) bf16 in every layout, compared in full
    within the stated tolerance."""
    p = W.random_problem(4096, 3072, 3072, "bf16", "bf16", ("normal", 0.0, 1.0), seed=720,
                         a_layout=layout[0], b_layout=layout[1])
    plan = {}
    c, untouched = run(p, plan=plan)
    assert (plan["block_m"], plan["block_k"], plan["threads"], plan["ragged"]) == \
        (256, 32, 256, 0), plan
    assert plan["layout"] == LAYOUT_BITS[layout], plan
    err, tol = compare(p, c, label=f"4 waves {layout} 4096x3072x3072")
    note(f"4 waves {layout}: max err {err:.3e} tol {tol:.3e}")
    assert untouched


@pytest.mark.parametrize("layout", ["NN", "TT"])
def test_192_selector_random(layout):
    """Shapes whose 256-wide tiles leave a round of the CUs part-empty: the
    selector's 192-wide tiles, interior (3072 x 3072 x 1024) and
    range-checked (3000 x 3000 x 1000), N(0,1) bf16 compared in full within
    the stated tolerance."""
    for M, N, K, ragged, seed in [(3072, 3072, 1024, 0, 730), (3000, 3000, 1000, 1, 731)]:
        p = W.random_problem(M, N, K, "bf16", "bf16", ("normal", 0.0, 1.0), seed=seed,
                             a_layout=layout[0], b_layout=layout[1])
        plan = {}
        c, untouched = run(p, plan=plan)
        assert (plan["block_m"], plan["block_k"], plan["threads"], plan["ragged"]) == \
            (192, 32, 256, ragged), plan
        err, tol = compare(p, c, label=f"192 {layout} {M}x{N}x{K}")
        note(f"192 {layout} {M}x{N}x{K}: max err {err:.3e} tol {tol:.3e}")
        assert untouched


@pytest.mark.parametrize("layout", ["NN", "TT", "NT"])
def test_unsplit_rows_exact(layout):
    """Plans whose top rows run unsplit and whose lower rows run with K split
    (forced): interior and range-checked lower parts, tiles of 256, 192 and
    128, every output dtype.  Value-exact on integer-valued inputs; C
    outside the view untouched."""
    cases = [(768, 512, 2048, 4, 512, 256), (1000, 520, 1000, 3, 512, 256),
             (960, 576, 2048, 4, 576, 192), (640, 384, 4096, 2, 384, 128),
             (520, 264, 2056, 8, 256, 256)]
    for n, (M, N, K, S, dp, tile) in enumerate(cases):
        if layout[0] == "T":
            M = _round8(M)
        if layout[1] == "N":
            N = _round8(N)
        outd = ["f32", "bf16", "f16", "f32", "bf16"][n]
        p = padded_int_problem(M, N, K, "bf16" if n % 2 else "f16", outd, 2, seed=880 + n,
                               a_layout=layout[0], b_layout=layout[1])
        cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=32, split_k=S, dp_rows=dp)
        plan = {}
        c, untouched = run(p, config=cfg, c_pad=3 if n % 2 else 0, plan=plan)
        assert plan["status"] == 0 and (plan["split_k"], plan["dp_rows"]) == (S, dp), plan
        compare(p, c, exact=True, label=f"unsplit rows {layout} {M}x{N}x{K} S{S} dp{dp}->{outd}")
        assert untouched


def test_unsplit_rows_selector_random():
    """4096 x 5120 x 4096 has 320 tiles of 256 for 256 CUs: the selector runs
    the top 12 tile-rows unsplit and the 4 below with K in 2 slices; N(0,1)
    bf16 compared in full within the stated tolerance."""
    p = W.random_problem(4096, 5120, 4096, "bf16", "bf16", ("normal", 0.0, 1.0), seed=890)
    plan = {}
    c, untouched = run(p, plan=plan)
    assert (plan["block_m"], plan["split_k"], plan["dp_rows"]) == (256, 2, 3072), plan
    err, tol = compare(p, c, label="unsplit rows 4096x5120x4096")
    note(f"unsplit rows 4096x5120x4096: max err {err:.3e} tol {tol:.3e}")
    assert untouched


def test_uneven_split_selector_random():
    """36 tiles of 128 and a 32768-long K: the selector splits K seven ways
    (252 work units, range-checked slices of 4704 and a shorter last one);
    U[-1,1] fp16 -> fp32 compared in full within the stated tolerance."""
    p = W.random_problem(768, 768, 32768, "f16", "f32", ("uniform", -1.0, 1.0), seed=895)
    plan = {}
    c, untouched = run(p, plan=plan)
    assert (plan["block_m"], plan["split_k"], plan["ragged"]) == (128, 7, 1), plan
    err, tol = compare(p, c, label="split 7 768x768x32768")
    note(f"split 7 768x768x32768: max err {err:.3e} tol {tol:.3e}")
    assert untouched


def _round8(x):
    return -(-x // 8) * 8


@pytest.mark.parametrize("tile", [256, 192, 128])
@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_pipelined_ragged_exact(ind, layout, tile):
    """The pipelined kernel's range-checked form at shapes its tile does not
    divide (M, N of any size -- multiples of 8 along a contiguous M or N --
    and K a multiple of 8, including K < 32 and K not a multiple of 32):
    chunks outside the views must arrive as exact zeros, the NaN padding
    beyond each leading dimension must never be read, and C outside M x N
    must stay untouched.  Value-exact on integer-valued inputs."""
    cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=32)
    shapes = [(300, 264, 104), (256, 520, 8), (513, 777, 1000), (8, 8, 8), (777, 255, 64),
              (1000, 1001, 2048), (257, 300, 24), (384, 640, 96)]
    for n, (M, N, K) in enumerate(shapes):
        if layout[0] == "T":
            M = _round8(M)
        if layout[1] == "N":
            N = _round8(N)
        outd = ["f32", "f16", "bf16"][n % 3]
        p = padded_int_problem(M, N, K, ind, outd, 8 if K <= 256 else 2, seed=800 + n,
                               extra=8 * (n % 2), a_layout=layout[0], b_layout=layout[1])
        plan = {}
        c, untouched = run(p, config=cfg, c_pad=3 if n % 2 else 0, plan=plan)
        assert plan["status"] == 0 and plan["block_k"] == 32 and plan["block_m"] == tile, plan
        assert plan["ragged"] == (1 if (M % tile or N % tile or K % 32) else 0), plan
        compare(p, c, exact=True,
                label=f"pipelined {tile} ragged {layout} {ind} {M}x{N}x{K}->{outd}")
        assert untouched


@pytest.mark.parametrize("tile", [256, 192, 128])
def test_pipelined_output_views(tile):
    """The pipelined kernel's store of C through views of every kind: rows
    4-element aligned with N not a multiple of 4 (whole 4-column groups
    written at once, the group across N element by element), a column-major
    C, and row strides or base addresses that rule out the wide store.
    Value-exact on integer-valued inputs; C outside the view untouched."""
    cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=32)
    # (M, N, K, C layout, pad, offset): B is K-contiguous, so N may be any size
    cases = [(300, 250, 96, "N", 6, 0), (512, 256, 64, "N", 4, 4), (264, 258, 160, "N", 2, 0),
             (256, 512, 64, "T", 0, 0), (520, 256, 32, "N", 4, 2), (256, 254, 64, "N", 2, 8)]
    for n, (M, N, K, cl, pad, off) in enumerate(cases):
        for outd in ("f32", "f16", "bf16"):
            p = padded_int_problem(M, N, K, "bf16" if n % 2 else "f16", outd, 4, seed=870 + n,
                                   b_layout="T")
            plan = {}
            c, untouched = run(p, config=cfg, c_layout=cl, c_pad=pad, c_offset=off, plan=plan)
            assert plan["status"] == 0 and plan["block_m"] == tile, plan
            label = f"output view {tile} {M}x{N}x{K} C {cl} pad {pad} offset {off} -> {outd}"
            compare(p, c, exact=True, label=label)
            assert untouched, label


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
def test_pipelined_ragged_random_selector(layout):
    """A large ragged bf16 problem (4000 x 4008 x 520, N(0,1)) through the
    selector's plan -- the pipelined kernel's range-checked form -- against
    the oracle within tolerance."""
    p = W.random_problem(4000, 4008, 520, "bf16", "bf16", ("normal", 0.0, 1.0), seed=820,
                         a_layout=layout[0], b_layout=layout[1])
    plan = {}
    c, untouched = run(p, plan=plan)
    assert (plan["block_k"], plan["ragged"], plan["layout"]) == (32, 1, LAYOUT_BITS[layout]), plan
    err, tol = compare(p, c, label=f"ragged {layout} 4000x4008x520")
    note(f"ragged {layout} 4000x4008x520: max err {err:.3e} tol {tol:.3e}")
    assert untouched


@pytest.mark.parametrize("tile", [256, 192, 128])
@pytest.mark.parametrize("layout", ["NN", "TT"])
def test_split_k_ragged_exact(layout, tile):
    """Split-K on the range-checked pipelined kernel: ragged M and N, slices
    of cdiv(K, S) rounded up to 32 with a shorter last slice, K a multiple of
    8 only; value-exact on integer-valued inputs (every partial sum is an
    integer, so the slice order cannot change the result)."""
    cases = [(500, 264, 1000, 4), (300, 256, 4104, 8), (264, 520, 2056, 3), (8, 8, 2048, 64)]
    for n, (M, N, K, S) in enumerate(cases):
        if layout[0] == "T":
            M = _round8(M)
        outd = ["f32", "bf16", "f16", "f32"][n]
        cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=32, split_k=S)
        p = padded_int_problem(M, N, K, "bf16" if n % 2 else "f16", outd, 2, seed=840 + n,
                               a_layout=layout[0], b_layout=layout[1])
        plan = {}
        c, untouched = run(p, config=cfg, c_pad=3 if n % 2 else 0, plan=plan)
        assert (plan["split_k"], plan["ragged"]) == (S, 1), plan
        compare(p, c, exact=True, label=f"split-K ragged {layout} S{S} {M}x{N}x{K}->{outd}")
        assert untouched


def test_ragged_selector_split():
    """Few tiles through the selector on the range-checked pipelined kernel:
    bf16 2000^3 (64 tiles of 256, so 256 of 128) and 1000 x 1000 x 8200
    (16 of 256: 64 of 128, K split in 4); N(0,1) values within tolerance."""
    for M, N, K, S, seed in [(2000, 2000, 2000, 1, 860), (1000, 1000, 8200, 4, 861)]:
        p = W.random_problem(M, N, K, "bf16", "f32", ("normal", 0.0, 1.0), seed=seed)
        plan = {}
        c, untouched = run(p, plan=plan)
        assert (plan["block_m"], plan["block_k"], plan["split_k"], plan["ragged"]) == \
            (128, 32, S, 1), plan
        err, tol = compare(p, c, label=f"ragged {M}x{N}x{K}")
        note(f"ragged {M}x{N}x{K} S{S}: max err {err:.3e} tol {tol:.3e}")
        assert untouched


@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_split_k_exact(ind):
    """Split-K on the pipelined kernel (forced splits, fp32 partials summed
    in slice order by a second pass): value-exact on integer-valued inputs,
    with the library's workspace."""
    shapes = [(256, 256, 64, 2), (512, 256, 1024, 4), (256, 768, 4096, 16), (512, 512, 8192, 64)]
    for n, (M, N, K, S) in enumerate(shapes):
        outd = ["f32", "bf16", "f16", "f32"][n]
        cfg = dict(kernel=MF16, block_m=256, block_n=256, block_k=32, split_k=S)
        p = padded_int_problem(M, N, K, ind, outd, 2, seed=500 + n)
        c, untouched = run(p, config=cfg, c_pad=3 if n % 2 else 0)
        compare(p, c, exact=True, label=f"split-K {S} {ind} {M}x{N}x{K}->{outd}")
        assert untouched


@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_many_tiles_exact(ind):
    """More 256x256 (and 192x192) work units than compute units on the
    pipelined kernel (several tiles per CU in turn): 1-, 2-, 3- and 5-chunk
    units, and split-K with more (tile, slice) units than CUs.  Value-exact
    on integer-valued inputs."""
    cases = [(4352, 4352, 32, 1, 256), (4352, 4352, 64, 1, 256), (4096, 4608, 96, 1, 256),
             (2560, 2560, 1024, 4, 256), (4608, 4608, 64, 1, 192), (4032, 4608, 160, 1, 192)]
    for n, (M, N, K, S, tile) in enumerate(cases):
        outd = ["bf16", "f32", "f16", "f32", "bf16", "f16"][n]
        cfg = dict(kernel=MF16, block_m=tile, block_n=tile, block_k=32, split_k=S)
        p = padded_int_problem(M, N, K, ind, outd, 4, seed=700 + n)
        note(f"many tiles {ind} {M}x{N}x{K} tile {tile} split {S}")
        c, untouched = run(p, config=cfg)
        compare(p, c, exact=True, label=f"many tiles {ind} {M}x{N}x{K} tile {tile} split {S}")
        assert untouched


def test_split_k_caller_workspace():
    """gemm_ex with a caller-owned workspace: same result as the library's;
    a workspace smaller than the plan needs is rejected before any launch."""
    M, N, K, S = 512, 512, 2048, 8
    p = padded_int_problem(M, N, K, "f16", "f32", 4, seed=77)
    cfg = dict(kernel=MF16, block_m=256, block_n=256, block_k=32, split_k=S)
    ref, _ = run(p, config=cfg)
    sa, sb = dev_storage(p.A.bits, "f16"), dev_storage(p.B.bits, "f16")
    c = torch.empty(M, N, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(S * M * N, dtype=torch.float32, device="cuda:0")
    st = dtm.gemm_ex_raw(M, N, K, sa.data_ptr(), p.A.stride_r, 1, sb.data_ptr(), p.B.stride_r, 1,
                         c.data_ptr(), N, 1, dtm.DTM_F16, dtm.DTM_F32, config=cfg,
                         workspace=ws.data_ptr(), workspace_bytes=ws.numel() * 4)
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(c.cpu().numpy().view(np.uint32), ref)
    c2 = torch.full((M, N), 7.0, device="cuda:0")
    st = dtm.gemm_ex_raw(M, N, K, sa.data_ptr(), p.A.stride_r, 1, sb.data_ptr(), p.B.stride_r, 1,
                         c2.data_ptr(), N, 1, dtm.DTM_F16, dtm.DTM_F32, config=cfg,
                         workspace=ws.data_ptr(), workspace_bytes=ws.numel() * 4 - 4)
    torch.cuda.synchronize()
    assert st == dtm.DTM_ERR_WORKSPACE
    assert bool((c2 == 7.0).all())
    # unsplit top rows: the workspace covers only the rows below them
    M2, dp = 768, 512
    p = padded_int_problem(M2, N, K, "f16", "f32", 4, seed=78)
    cfg = dict(kernel=MF16, block_m=256, block_n=256, block_k=32, split_k=S, dp_rows=dp)
    plan = {}
    ref, _ = run(p, config=cfg, plan=plan)
    assert plan["workspace_bytes"] == S * (M2 - dp) * N * 4, plan
    sa, sb = dev_storage(p.A.bits, "f16"), dev_storage(p.B.bits, "f16")
    c = torch.empty(M2, N, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(S * (M2 - dp) * N, dtype=torch.float32, device="cuda:0")
    for nbytes, want in [(ws.numel() * 4 - 16, dtm.DTM_ERR_WORKSPACE), (ws.numel() * 4, 0)]:
        st = dtm.gemm_ex_raw(M2, N, K, sa.data_ptr(), p.A.stride_r, 1, sb.data_ptr(),
                             p.B.stride_r, 1, c.data_ptr(), N, 1, dtm.DTM_F16, dtm.DTM_F32,
                             config=cfg, workspace=ws.data_ptr(), workspace_bytes=nbytes)
        torch.cuda.synchronize()
        assert st == want, (nbytes, st)
    assert np.array_equal(c.cpu().numpy().view(np.uint32), ref)


def _padded_f32_problem(M, N, K, outd, seed, a_layout, b_layout):
    """Integer-valued fp32 operands, leading dimensions rounded up to 4
    elements (16 bytes) with NaN padding; layouts as padded_int_problem."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-16, 17, size=(M, K))
    b = rng.integers(-16, 17, size=(K, N))

    def store(x, layout):
        rows, cols = x.shape
        if layout == "T":
            x = x.T
        ld = -(-x.shape[1] // 4) * 4
        buf = np.full((x.shape[0], ld), np.nan)
        buf[:, :x.shape[1]] = x
        strides = (ld, 1) if layout == "N" else (1, ld)
        return W.Operand(W.to_bits(buf, "f32").reshape(-1), "f32", rows, cols, 0, *strides)

    return W.Problem(M, N, K, store(a, a_layout), store(b, b_layout), "f32", outd,
                     name=f"f32{a_layout}{b_layout}{M}x{N}x{K}")


def _unaligned_f32_problem(M, N, K, outd, seed, a_layout, b_layout, ld_extra, offset,
                           ind="f32"):
    """As _padded_f32_problem, but leading dimensions of cols + ld_extra
    elements (off 16-byte boundaries unless ld_extra * item size is a
    multiple of 16) and each view starting `offset` elements into its
    NaN-filled buffer; `ind` the operands' dtype."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-16, 17, size=(M, K))
    b = rng.integers(-16, 17, size=(K, N))

    def store(x, layout):
        rows, cols = x.shape
        if layout == "T":
            x = x.T
        ld = x.shape[1] + ld_extra
        if ind != "f32":
            # 16-bit views: an even leading dimension off a multiple of 8
            ld += ld % 2
            ld += 2 if ld % 8 == 0 else 0
        buf = np.full(offset + x.shape[0] * ld + 8, np.nan)
        view = buf[offset:offset + x.shape[0] * ld].reshape(x.shape[0], ld)
        view[:, :x.shape[1]] = x
        strides = (ld, 1) if layout == "N" else (1, ld)
        return W.Operand(W.to_bits(buf, ind), ind, rows, cols, offset, *strides)

    return W.Problem(M, N, K, store(a, a_layout), store(b, b_layout), ind, outd,
                     name=f"{ind}u{a_layout}{b_layout}{M}x{N}x{K}")


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
def test_mfma16_views_off_16_bytes_exact(layout):
    """fp16/bf16 views whose chunks start on 4-byte but not 16-byte
    boundaries (even leading dimensions off a multiple of 8 elements, views
    starting 0, 2 or 6 elements into their buffers) on the register-staged
    kernel's range-checked form, 16-byte copies at 4-byte alignment: value-
    exact on integer-valued inputs, nothing outside the views read (NaN
    padding), at both tiles and through the selector."""
    cases = [(128, 128, 64, 2, 2), (257, 129, 200, 6, 2), (300, 260, 1000, 2, 6),
             (64, 500, 78, 6, 6), (512, 256, 96, 2, 0), (1000, 776, 520, 2, 2)]
    for n, (M, N, K, extra, off) in enumerate(cases):
        ind = ["bf16", "f16"][n % 2]
        outd = ["f32", "bf16", "f16"][n % 3]
        p = _unaligned_f32_problem(M, N, K, outd, 700 + n, layout[0], layout[1], extra, off,
                                   ind=ind)
        for cfg in (dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=128, block_n=128, block_k=64),
                    dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=256, block_n=256, block_k=64),
                    None):
            plan = {}
            c, untouched = run(p, config=cfg, c_pad=2 if n % 2 else 0, plan=plan)
            assert plan["status"] == 0 and plan["kernel_name"] == "mfma_f16", plan
            assert (plan["block_k"], plan["ragged"]) == (64, 1), plan
            assert plan["layout"] == LAYOUT_BITS[layout], plan
            compare(p, c, exact=True, label=f"mfma_f16 4-byte views {layout} {M}x{N}x{K}"
                    f"+{extra}@{off} {ind}->{outd} {cfg and cfg['block_m']}")
            assert untouched


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
def test_mfma_f32_unaligned_exact(layout):
    """fp32 views off 16-byte boundaries (leading dimensions of cols + 1 or
    + 3 elements, views starting 1 or 3 elements into their buffers) on the
    fp32 matrix cores' range-checked form with element loads, both tile
    sizes: value-exact on integer-valued inputs, nothing outside the views
    read (NaN padding)."""
    MF32 = dtm.DTM_KERNEL_MFMA_F32
    cases = [(128, 128, 16, 1, 0), (257, 129, 193, 1, 1), (300, 260, 1000, 3, 3),
             (64, 500, 77, 2, 1), (512, 256, 96, 1, 2)]
    for n, (M, N, K, extra, off) in enumerate(cases):
        outd = ["f32", "f16", "bf16"][n % 3]
        p = _unaligned_f32_problem(M, N, K, outd, 660 + n, layout[0], layout[1], extra, off)
        for tile, bk in ((128, 16), (192, 32), (256, 16), (256, 32)):
            plan = {}
            c, untouched = run(p, config=dict(kernel=MF32, block_m=tile, block_n=tile, block_k=bk),
                               c_pad=2 if n % 2 else 0, plan=plan)
            assert plan["status"] == 0 and plan["layout"] == LAYOUT_BITS[layout], plan
            compare(p, c, exact=True, label=f"mfma_f32 unaligned {tile}x{bk} {layout} "
                    f"{M}x{N}x{K}+{extra}@{off}->{outd}")
            assert untouched


@pytest.mark.parametrize("layout", ["NN", "TN", "NT", "TT"])
def test_mfma_f32_exact_and_random(layout):
    """fp32 inputs on the fp32 matrix cores in each operand layout:
    value-exact on integer-valued inputs at ragged and interior sizes (every
    output dtype), and within the fp32 tolerance on N(0,1) inputs."""
    MF32 = dtm.DTM_KERNEL_MFMA_F32
    for n, (M, N, K) in enumerate([(128, 128, 16), (256, 384, 512), (129, 257, 33), (1, 1, 1),
                                   (300, 200, 1000), (127, 129, 17)]):
        outd = ["f32", "f16", "bf16"][n % 3]
        p = _padded_f32_problem(M, N, K, outd, 600 + n, layout[0], layout[1])
        plan = {}
        c, untouched = run(p, config=dict(kernel=MF32), c_pad=2 if n % 2 else 0, plan=plan)
        assert plan["layout"] == LAYOUT_BITS[layout], plan
        compare(p, c, exact=True, label=f"mfma_f32 {layout} {M}x{N}x{K}->{outd}")
        assert untouched
    # the 256-wide tile (the selector's choice for large full rounds), forced,
    # with 16- and 32-deep chunks, and the 192-wide tile
    for n, (M, N, K) in enumerate([(256, 256, 16), (512, 768, 96), (257, 513, 49),
                                   (300, 260, 1000), (256, 512, 32), (512, 256, 80),
                                   (384, 576, 64), (385, 193, 40)]):
        outd = ["f32", "bf16", "f16"][n % 3]
        p = _padded_f32_problem(M, N, K, outd, 640 + n, layout[0], layout[1])
        for tile, bk in ((256, 16), (256, 32), (192, 32)):
            plan = {}
            c, untouched = run(p, config=dict(kernel=MF32, block_m=tile, block_n=tile, block_k=bk),
                               c_pad=2 if n % 2 else 0, plan=plan)
            assert (plan["block_m"], plan["block_k"]) == (tile, bk), plan
            assert plan["layout"] == LAYOUT_BITS[layout], plan
            compare(p, c, exact=True, label=f"mfma_f32 {tile}x{bk} {layout} {M}x{N}x{K}->{outd}")
            assert untouched
    for n, (M, N, K) in enumerate([(1024, 1024, 1024), (1000, 600, 776), (3000, 2900, 200)]):
        p = W.random_problem(M, N, K, "f32", "f32", ("normal", 0.0, 1.0), seed=650 + n,
                             a_layout=layout[0], b_layout=layout[1])
        plan = {}
        c, _ = run(p, plan=plan)
        assert plan["kernel_name"] == "mfma_f32" and plan["layout"] == LAYOUT_BITS[layout], plan
        err, tol = compare(p, c, label=f"mfma_f32 {layout} random {M}x{N}x{K}")
        note(f"mfma_f32 {layout} {M}x{N}x{K}: max err {err:.3e} tol {tol:.3e}")


@pytest.mark.parametrize("layout", ["TN", "NT", "TT"])
@pytest.mark.parametrize("ind", ["f16", "bf16"])
def test_register_kernel_layouts_random(ind, layout):
    """Random values, sizes ragged against the tiles (multiples of 8, so
    every leading dimension is a 16-byte multiple), transposed operands on
    the register-staged MFMA kernel (both tiles): within tolerance."""
    for n, (M, N, K) in enumerate([(296, 200, 152), (1000, 520, 776), (504, 264, 1032)]):
        p = W.random_problem(M, N, K, ind, "f32", ("normal", 0.0, 1.0), seed=680 + n,
                             a_layout=layout[0], b_layout=layout[1])
        tile = 128 if n % 2 else 256
        plan = {}
        c, _ = run(p, plan=plan, config=dict(kernel=MF16, block_m=tile, block_n=tile,
                                             block_k=64))
        assert plan["block_k"] == 64 and plan["layout"] == LAYOUT_BITS[layout], plan
        err, tol = compare(p, c, label=f"{layout} {ind} {M}x{N}x{K}")
        note(f"{layout} {ind} {M}x{N}x{K}: max err {err:.3e} tol {tol:.3e}")


@pytest.mark.parametrize("layout", ["NN", "NT", "TN", "TT"])
@pytest.mark.parametrize("ind", ["f32", "f16", "bf16"])
def test_generic_layouts_sweep_exact(layout, ind):
    """All four transpose combinations on the generic kernel, ragged sizes,
    each of its tile shapes: value-exact on integer-valued inputs."""
    cfgs = [dict(kernel=GEN, block_m=b, block_n=b, block_k=k)
            for b, k in [(4, 4), (16, 16), (32, 16), (64, 16), (128, 8)]]
    R = 16 if ind == "bf16" else 32
    for n, (M, N, K) in enumerate(_sweep_shapes(8, seed=len(layout) + len(ind))):
        outd = ["f32", "f16", "bf16"][n % 3]
        p = int_problem(M, N, K, ind, outd, R, seed=200 + n, la=layout[0], lb=layout[1])
        c, untouched = run(p, config=cfgs[n % len(cfgs)], c_layout="T" if n % 2 else "N")
        compare(p, c, exact=True, label=f"{layout} {ind} {M}x{N}x{K}")
        assert untouched


@pytest.mark.parametrize("ind", ["f32", "f16", "bf16"])
def test_random_values_default_plan(ind):
    """N(0,1) inputs at ragged sizes through the selector's own plan."""
    for n, (M, N, K) in enumerate([(300, 200, 150), (1000, 513, 777), (64, 4097, 33),
                                   (511, 257, 1025)]):
        p = W.random_problem(M, N, K, ind, "f32", ("normal", 0.0, 1.0), seed=300 + n)
        c, _ = run(p)
        err, tol = compare(p, c, label=f"{ind} {M}x{N}x{K}")
        note(f"{ind} {M}x{N}x{K}: max err {err:.3e} tol {tol:.3e}")


def test_negative_and_zero_strides():
    """Negative row strides and a broadcast (zero-stride) row: through the
    selector's plan (the fp32 matrix cores' range-checked form, K being the
    unit-stride axis) and forced onto the generic kernel; exact."""
    rng = np.random.default_rng(9)
    M, N, K = 33, 21, 17
    a = rng.integers(-9, 10, size=(M, K)).astype(np.float64)
    b = rng.integers(-9, 10, size=(K, N)).astype(np.float64)
    A = W.Operand(W.to_bits(a[::-1].copy(), "f32").reshape(-1), "f32", M, K, (M - 1) * K, -K, 1)
    B = W.dense(W.to_bits(b, "f32"), "f32")
    p = W.Problem(M, N, K, A, B, "f32", "f32")
    assert np.array_equal(A.logical_bits(), W.to_bits(a, "f32"))
    row = W.Operand(W.to_bits(a[0], "f32"), "f32", M, K, 0, 0, 1)
    p2 = W.Problem(M, N, K, row, B, "f32", "f32")
    for cfg, kernel in [(None, "mfma_f32"), (dict(kernel=GEN), "generic")]:
        for prob, label in [(p, "negative stride"), (p2, "broadcast")]:
            plan = {}
            c, _ = run(prob, config=cfg, plan=plan)
            assert plan["kernel_name"] == kernel, plan
            compare(prob, c, exact=True, label=f"{label} {kernel}")


# ------------------------------------------------------------ semantics


@pytest.mark.parametrize("outd", ["f32", "f16", "bf16"])
def test_k_zero_writes_zeros(outd):
    p = W.Problem(37, 19, 0, W.Operand(np.zeros(1, np.uint16), "f16", 37, 0, 0, 0, 1),
                  W.Operand(np.zeros(1, np.uint16), "f16", 0, 19, 0, 19, 1), "f16", outd)
    c, untouched = run(p, c_pad=3)
    assert not oracle.decode(c, outd).any()
    assert untouched


def test_m_or_n_zero_writes_nothing():
    for (M, N) in [(0, 7), (7, 0)]:
        buf = torch.full((64,), 12345, dtype=torch.int32, device="cuda:0")
        a = torch.ones(max(M, 1), 5, device="cuda:0")
        st = dtm.gemm_raw(M, N, 5, a.data_ptr(), 5, 1, a.data_ptr(), 7, 1, buf.data_ptr(), 7, 1,
                          dtm.DTM_F32, dtm.DTM_F32)
        torch.cuda.synchronize()
        assert st == 0 and bool((buf == 12345).all())


def test_deterministic():
    p = W.random_problem(1024, 768, 2048, "bf16", "f32", ("normal", 0.0, 1.0), seed=17)
    c1, _ = run(p)
    c2, _ = run(p)
    assert np.array_equal(c1, c2)
    q = W.random_problem(200, 300, 500, "f32", "f32", ("normal", 0.0, 1.0), seed=18,
                         a_layout="T")
    assert np.array_equal(run(q)[0], run(q)[0])


def test_non_default_stream_ordering():
    """The work is enqueued on the caller's stream: it sees writes made
    earlier on that stream and is complete after that stream synchronises."""
    s = torch.cuda.Stream()
    M = N = K = 512
    with torch.cuda.stream(s):
        a = torch.zeros(M, K, dtype=torch.float16, device="cuda:0")
        b = torch.zeros(K, N, dtype=torch.float16, device="cuda:0")
        a.fill_(1.0)  # ordered before the GEMM on s
        b.fill_(2.0)
        c = dtm.gemm(a, b, stream=s)
    s.synchronize()
    assert bool((c == 2.0 * K).all())


def test_tensor_binding_views():
    """The torch-level binding: strides and storage offsets of views pass
    through unchanged."""
    base = torch.randn(300, 400, device="cuda:0")
    a = base[10:210, 5:105].t()  # 100 x 200, column-major view with offset
    b = torch.randn(200, 50, device="cuda:0")[:, ::2]  # stride 2 columns
    out = torch.empty(100, 25, device="cuda:0")
    dtm.gemm(a, b, out=out)
    torch.cuda.synchronize()
    p = W.Problem(100, 25, 200,
                  W.Operand(a.contiguous().cpu().numpy().view(np.uint32).reshape(-1), "f32", 100,
                            200, 0, 200, 1),
                  W.Operand(b.contiguous().cpu().numpy().view(np.uint32).reshape(-1), "f32", 200,
                            25, 0, 25, 1), "f32", "f32")
    compare(p, out.cpu().numpy().view(np.uint32), label="torch views")
