"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/dtm_gemm.h declares, plans launches ("Chapter 13: The
Blocked Matmul Kernel", Worked Example 13.1.1: an 8x8x8 product with 4x4x4
tiles runs a (2, 2) grid with 2 K-iterations per tile) and rejects bad
arguments before anything is launched."""
import ctypes
import os

import pytest

import dense_tiled_matrix_amd as dtm

F32, F16, BF16 = dtm.DTM_F32, dtm.DTM_F16, dtm.DTM_BF16
# fake, 256-byte-aligned, far-apart addresses: gemm_plan only reads pointer values
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000


def plan(M, N, K, A=PA, sam=None, sak=1, B=PB, sbk=None, sbn=1, C=PC, scm=None, scn=1,
         ind=F16, outd=F32, config=None):
    sam = K if sam is None else sam
    sbk = N if sbk is None else sbk
    scm = N if scm is None else scm
    return dtm.gemm_plan_raw(M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, ind, outd, config)


def test_library_exports_every_declared_function():
    names = dtm.header_functions()
    assert {"gemm", "gemm_plan", "gemm_ex", "gemm_status_string", "gemm_kernel_name"} <= set(names)
    L = dtm.lib()
    for n in names:
        assert hasattr(L, n), n
        assert isinstance(getattr(L, n), ctypes._CFuncPtr)


def test_status_strings():
    for code, name in dtm.STATUS.items():
        s = dtm.gemm_status_string(code)
        assert s and s != "unknown status", name
    assert dtm.gemm_status_string(999) == "unknown status"
    assert dtm.gemm_kernel_name(dtm.DTM_KERNEL_MFMA_F16) == "mfma_f16"


def test_plan_worked_example_grid():
    """8x8x8 with forced 4x4x4 tiles: grid (2, 2), 2 K-iterations."""
    st, p = plan(8, 8, 8, ind=F32, config=dict(kernel=dtm.DTM_KERNEL_GENERIC, block_m=4, block_n=4,
                                                 block_k=4))
    assert st == 0
    assert (p["grid_m"], p["grid_n"], p["k_iters"]) == (2, 2, 2)
    assert p["kernel_name"] == "generic" and p["threads"] == 16 and p["ragged"] == 0


def test_plan_ragged_awkward_dims():
    """Worked Example 13.2.1: M, K, N = 5, 7, 6 with 4x4x4 tiles -> grid (2, 2),
    2 K-iterations, and every dimension ragged."""
    st, p = plan(5, 6, 7, ind=F32, config=dict(kernel=dtm.DTM_KERNEL_GENERIC, block_m=4, block_n=4,
                                                 block_k=4))
    assert st == 0 and (p["grid_m"], p["grid_n"], p["k_iters"]) == (2, 2, 2) and p["ragged"] == 1
    st, p = plan(2, 2, 2, ind=F32, config=dict(kernel=dtm.DTM_KERNEL_GENERIC, block_m=4, block_n=4,
                                                 block_k=4))
    assert st == 0 and (p["grid_m"], p["grid_n"], p["k_iters"]) == (1, 1, 1) and p["ragged"] == 1


def test_selector_measured_workloads():
    st, p = plan(4096, 4096, 4096, ind=F16, outd=F32)
    assert st == 0 and p["kernel_name"] == "mfma_f16" and p["fast_path"] == 1
    assert (p["block_m"], p["block_n"], p["block_k"]) == (256, 256, 32)
    assert (p["grid_m"], p["grid_n"], p["k_iters"], p["ragged"]) == (16, 16, 128, 0)
    st, p = plan(8192, 8192, 8192, ind=BF16, outd=BF16)
    assert st == 0 and p["kernel_name"] == "mfma_f16"
    assert (p["grid_m"], p["grid_n"], p["k_iters"]) == (32, 32, 256)
    # large ragged shapes with K % 8 == 0: the pipelined kernel's
    # range-checked form
    st, p = plan(4000, 4000, 4000, ind=BF16, outd=BF16)
    assert st == 0 and (p["block_m"], p["block_k"], p["ragged"], p["threads"]) == \
        (256, 32, 1, 512)
    assert (p["grid_m"], p["grid_n"], p["k_iters"]) == (16, 16, 125)
    # K % 8 != 0: the 64-deep register-staged kernel
    st, p = plan(4096, 4096, 4100, sam=4104, ind=F16, outd=F32)
    assert st == 0 and (p["block_m"], p["block_k"], p["ragged"]) == (256, 64, 1)
    # long-K skinny: 4 tiles of 256 x 256 -> 16 of 128 x 128, K split into
    # 16 slices of 4096, each tile's K loop split across its 4 waves
    st, p = plan(512, 512, 65536, ind=F16, outd=F32)
    assert st == 0 and p["kernel_name"] == "mfma_f16_wavek" and p["split_k"] == 16
    assert (p["block_m"], p["block_k"], p["k_iters"], p["threads"]) == (128, 32, 128, 256)
    assert p["workspace_bytes"] == 16 * 512 * 512 * 4
    # few 256-wide tiles: 128-wide ones, split only with K long enough;
    # 192-wide ones where they fill the 256 CUs' rounds enough better
    for M, N, K, tile, S in [(2048, 2048, 2048, 128, 1), (1024, 1024, 8192, 128, 4),
                             (1024, 1024, 1024, 128, 1), (8192, 1024, 8192, 128, 1),
                             (2560, 2560, 2560, 128, 1), (3072, 3072, 3072, 192, 1),
                             (4096, 4096, 1024, 256, 1), (2000, 2000, 2000, 128, 1),
                             (6144, 6144, 6144, 192, 1), (6144, 6144, 2048, 192, 1),
                             (3072, 3072, 1024, 192, 1), (3000, 3000, 3000, 192, 1),
                             (3840, 3840, 3840, 256, 1),
                             (5120, 5120, 5120, 256, 1),
                             (8192, 8192, 8192, 256, 1), (12288, 12288, 1024, 256, 1),
                             (4096, 3072, 2048, 256, 1)]:
        st, p = plan(M, N, K, A=1 << 40, B=2 << 40, C=3 << 40, ind=BF16, outd=BF16)
        assert st == 0 and (p["block_m"], p["block_k"], p["split_k"]) == (tile, 32, S), \
            (M, N, K, p)
        if tile != 256:
            assert p["threads"] == 256, (M, N, K, p)
        assert p["ragged"] == (1 if (M % tile or N % tile) else 0), (M, N, K, p)
        assert p["dp_rows"] == 0, (M, N, K, p)
        # 128-wide interior tiles with a K loop of 8192 or more: wave-K
        wk = tile == 128 and not p["ragged"] and K // S >= 8192
        assert p["kernel_name"] == ("mfma_f16_wavek" if wk else "mfma_f16"), (M, N, K, p)
    # 256-wide tiles that leave the last round part-empty: the top tile-rows
    # in whole rounds unsplit, the rest with K split so that tiles x S nearly
    # fills one round (partials: S x rows below x N x 4 bytes)
    for M, N, K, S, dp_rows, ragged in [(4096, 5120, 4096, 2, 3072, 0),
                                        (5120, 4096, 4096, 3, 4096, 1),
                                        (4608, 4608, 4608, 3, 3584, 0),
                                        (6000, 6000, 6000, 3, 5376, 1),
                                        (7000, 7000, 7000, 5, 6912, 1),
                                        (4096, 5120, 8192, 3, 3072, 1),
                                        (7168, 7168, 7168, 5, 6912, 1)]:
        st, p = plan(M, N, K, A=1 << 40, B=2 << 40, C=3 << 40, ind=BF16, outd=BF16)
        assert st == 0 and (p["block_m"], p["block_k"], p["split_k"], p["dp_rows"]) == \
            (256, 32, S, dp_rows), (M, N, K, p)
        assert p["ragged"] == ragged and p["k_iters"] == -(-(-(-K // S)) // 32), (M, N, K, p)
        assert p["workspace_bytes"] == S * (M - dp_rows) * N * 4, (M, N, K, p)
        gm, gn = -(-M // 256), -(-N // 256)
        assert (dp_rows // 256) * gn <= 256 * (gm * gn // 256) < (dp_rows // 256 + 1) * gn
        assert (gm - dp_rows // 256) * gn * S <= 256
    # fewer 128-wide tiles than CUs: S up to min(256 / tiles, K / 2048), a
    # power of two when that reaches 3/4 of it
    for M, N, K, S, ragged in [(768, 768, 32768, 7, 1), (384, 384, 65536, 28, 1),
                               (896, 896, 16384, 4, 0), (640, 640, 32768, 8, 0),
                               (256, 256, 65536, 32, 0), (1024, 1024, 4096, 2, 0)]:
        st, p = plan(M, N, K, A=1 << 40, B=2 << 40, C=3 << 40, ind=F16, outd=F32)
        assert st == 0 and (p["block_m"], p["split_k"], p["ragged"]) == (128, S, ragged), \
            (M, N, K, p)
        # split interior tiles: wave-K for slices of 4096 or more
        wk = not ragged and K % (128 * S) == 0 and K // S >= 4096
        assert p["kernel_name"] == ("mfma_f16_wavek" if wk else "mfma_f16"), (M, N, K, p)
    # enough tiles: no split
    st, p = plan(4096, 4096, 65536, A=1 << 40, B=2 << 40, C=3 << 40, ind=F16, outd=F32)
    assert st == 0 and p["split_k"] == 1 and p["workspace_bytes"] == 0
    # fp32 with a transposed A view whose leading dimension (257 floats) is
    # off a 16-byte boundary: the fp32 matrix cores' range-checked form
    st, p = plan(257, 129, 193, sam=1, sak=257, ind=F32, outd=F32)
    assert st == 0 and p["kernel_name"] == "mfma_f32" and p["fast_path"] == 1 and p["ragged"] == 1
    assert p["layout"] == dtm.DTM_LAYOUT_A_M_CONTIG


@pytest.mark.parametrize("kw,why", [
    (dict(sak=2), "A not K-contiguous"),
    (dict(sbn=3), "B not N-contiguous"),
    (dict(A=PA + 2), "A base not 4-byte aligned"),
    (dict(B=PB + 6), "B base not 4-byte aligned"),
    (dict(sam=1001), "A leading dimension odd"),
    (dict(sbk=999), "B leading dimension odd"),
])
def test_fast_path_predicate_falls_back_to_generic(kw, why):
    st, p = plan(1024, 1024, 1000, **kw)
    assert st == 0, why
    assert p["fast_path"] == 0 and p["kernel_name"] == "generic", why
    # forcing the MFMA kernel on such a layout is a configuration error
    st, _ = plan(1024, 1024, 1000, config=dict(kernel=dtm.DTM_KERNEL_MFMA_F16), **kw)
    assert st == dtm.DTM_ERR_CONFIG


@pytest.mark.parametrize("kw,bits", [
    (dict(B=PB + 8), 0), (dict(A=PA + 4), 0), (dict(sam=1002), 0), (dict(sbk=1006), 0),
    (dict(sam=1, sak=1026), dtm.DTM_LAYOUT_A_M_CONTIG),
    (dict(sbk=1, sbn=1010), dtm.DTM_LAYOUT_B_K_CONTIG),
])
def test_fp16_views_off_16_bytes_take_the_register_staged_kernel(kw, bits):
    """fp16/bf16 views whose chunks start on 4-byte but not 16-byte
    boundaries run on the register-staged kernel's range-checked form (never
    on the pipelined or wave-K kernels, whose loads need 16-byte chunks)."""
    st, p = plan(1024, 1024, 1000, **kw)
    assert st == 0 and p["kernel_name"] == "mfma_f16" and p["fast_path"] == 1, (kw, p)
    assert (p["block_k"], p["ragged"], p["split_k"], p["layout"]) == (64, 1, 1, bits), (kw, p)
    st, p = plan(1024, 1024, 1024, **kw)
    assert st == 0 and (p["kernel_name"], p["block_k"], p["ragged"]) == ("mfma_f16", 64, 1)
    for cfg in [dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=128, block_n=128, block_k=32),
                dict(kernel=dtm.DTM_KERNEL_MFMA_F16, split_k=4),
                dict(kernel=dtm.DTM_KERNEL_MFMA_F16_WAVEK)]:
        st, _ = plan(1024, 1024, 1024, config=cfg, **kw)
        assert st == dtm.DTM_ERR_CONFIG, (kw, cfg)
    st, p = plan(1024, 1024, 1024, config=dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=128,
                                                block_n=128, block_k=64), **kw)
    assert st == 0 and (p["block_m"], p["ragged"]) == (128, 1), (kw, p)


def test_selector_transposed_layouts():
    """A M-contiguous and/or B K-contiguous views run on the MFMA kernels with
    the layout bits in the plan: the pipelined kernel when its tile divides
    the problem, the register-staged one for ragged shapes, the fp32 one for
    fp32; views whose other stride is not a 16-byte multiple run on the
    generic kernel."""
    LA, LB = dtm.DTM_LAYOUT_A_M_CONTIG, dtm.DTM_LAYOUT_B_K_CONTIG
    big = dict(A=1 << 40, B=2 << 40, C=3 << 40)
    cases = {0: dict(), LA: dict(sam=1, sak=4096), LB: dict(sbk=1, sbn=4096),
             LA | LB: dict(sam=1, sak=4096, sbk=1, sbn=4096)}
    for bits, kw in cases.items():
        st, p = plan(4096, 4096, 4096, ind=BF16, outd=BF16, **big, **kw)
        assert st == 0 and p["kernel_name"] == "mfma_f16" and p["fast_path"] == 1, kw
        assert (p["block_m"], p["block_k"], p["layout"], p["split_k"]) == (256, 32, bits, 1), kw
        assert p["threads"] == 256  # 4096-long K loop: 4 waves
        # ragged: the register-staged kernel, same layout bits
        rk = {0: dict(sam=4104, sbk=4104), LA: dict(sam=1, sak=4104, sbk=4104),
              LB: dict(sam=4104, sbk=1, sbn=4104), LA | LB: dict(sam=1, sak=4104, sbk=1,
                                                                 sbn=4104)}[bits]
        st, p = plan(4095, 4097, 4100, ind=F16, outd=F32, **big, **rk)
        assert st == 0 and p["kernel_name"] == "mfma_f16" and p["layout"] == bits, kw
        assert (p["block_m"], p["block_k"], p["ragged"], p["threads"]) == (256, 64, 1, 256), kw
        # fp32
        st, p = plan(1000, 1000, 1000, ind=F32, outd=F32, **big,
                     **{k: (1000 if v == 4096 else v) for k, v in kw.items()})
        assert st == 0 and p["kernel_name"] == "mfma_f32" and p["layout"] == bits, kw
    # few tiles and a transposed operand: the pipelined kernel with split K
    st, p = plan(512, 512, 65536, sam=1, sak=512, ind=F16, outd=F32)
    assert st == 0 and p["layout"] == LA and p["split_k"] == 16 and p["block_k"] == 32
    # a small transposed problem: the pipelined kernel as well ...
    st, p = plan(256, 256, 64, sbk=1, sbn=64, ind=F16, outd=F32)
    assert st == 0 and p["layout"] == LB and p["block_k"] == 32 and p["ragged"] == 0
    # ... unless K % 8 != 0: then the register-staged kernel
    st, p = plan(256, 256, 60, sam=64, sbk=1, sbn=64, ind=F16, outd=F32)
    assert st == 0 and p["layout"] == LB and p["block_k"] == 64 and p["block_m"] == 128
    # other stride not a 16-byte multiple: fp16/bf16 on the register-staged
    # kernel's range-checked form when it is even, else on the generic kernel;
    # fp32 on the fp32 matrix cores' range-checked form
    for M, N, K, kw, ind, bits in [(4096, 4096, 4096, dict(sam=1, sak=4100), F16, LA),
                                   (4096, 4096, 4096, dict(sbk=1, sbn=4092), BF16, LB)]:
        st, p = plan(M, N, K, ind=ind, **big, **kw)
        assert st == 0 and p["kernel_name"] == "mfma_f16" and p["layout"] == bits, (M, N, K, kw)
        assert (p["block_k"], p["ragged"]) == (64, 1), (M, N, K, kw, p)
    for M, N, K, kw, ind in [(4096, 4096, 4096, dict(sam=1, sak=4099), F16),
                             (4096, 4096, 4096, dict(sbk=1, sbn=4093), BF16)]:
        st, p = plan(M, N, K, ind=ind, **big, **kw)
        assert st == 0 and p["kernel_name"] == "generic" and p["layout"] == 0, (M, N, K, kw)
    for M, N, K, kw, bits in [(257, 129, 193, dict(sam=1, sak=257), LA),
                              (1024, 1024, 1024, dict(sbk=1, sbn=1026), LB)]:
        st, p = plan(M, N, K, ind=F32, **big, **kw)
        assert st == 0 and p["kernel_name"] == "mfma_f32" and p["layout"] == bits, (M, N, K, kw)
    # forced tiles accept every layout
    for cfg in [dict(block_m=256, block_n=256, block_k=64), dict(block_m=128, block_n=128,
                                                                 block_k=64),
                dict(block_m=256, block_n=256, block_k=32, split_k=4)]:
        st, p = plan(4096, 4096, 4096, sam=1, sak=4096, ind=F16, **big,
                     config=dict(kernel=dtm.DTM_KERNEL_MFMA_F16, **cfg))
        assert st == 0 and p["layout"] == LA and p["block_k"] == cfg["block_k"], cfg


def test_fp32_selector():
    """fp32 with a unit stride along one axis of each operand runs on the
    fp32 matrix cores, on or off 16-byte boundaries; views with no unit
    stride on the generic kernel."""
    st, p = plan(1024, 1024, 1000, ind=F32, sam=1000)
    assert st == 0 and p["kernel_name"] == "mfma_f32" and p["fast_path"] == 1
    assert (p["block_m"], p["block_n"], p["block_k"], p["ragged"]) == (128, 128, 16, 1)
    for kw in [dict(sam=1001), dict(A=PA + 4), dict(sbk=1002), dict(B=PB + 8),
               dict(sam=1, sak=1001), dict(sbk=1, sbn=1003)]:
        st, p = plan(1024, 1024, 1000, ind=F32, **kw)
        assert st == 0 and p["kernel_name"] == "mfma_f32" and p["fast_path"] == 1, kw
    for kw in [dict(sak=2), dict(sbn=3), dict(sam=2, sak=2048)]:
        st, p = plan(1024, 1024, 1000, ind=F32, **kw)
        assert st == 0 and p["kernel_name"] == "generic" and p["fast_path"] == 0, kw
    st, p = plan(1024, 1024, 1000, ind=F32, config=dict(kernel=dtm.DTM_KERNEL_MFMA_F16))
    assert st == dtm.DTM_ERR_CONFIG
    st, p = plan(1024, 1024, 1000, ind=F16, config=dict(kernel=dtm.DTM_KERNEL_MFMA_F32))
    assert st == dtm.DTM_ERR_CONFIG
    # the tile whose rounds over the 256 CUs cost least: 256 and 192 wide run
    # one workgroup per CU, 128 wide up to three
    big = dict(A=1 << 40, B=2 << 40, C=3 << 40)
    for M, N, K, tile in [(4096, 4096, 4096, 256), (8192, 8192, 8192, 256), (3000, 3000, 3000, 192),
                          (1024, 1024, 1024, 128), (4096, 8192, 2048, 256), (2048, 2048, 8192, 128),
                          (6000, 6000, 6000, 128), (4608, 4608, 4608, 128), (3072, 3072, 512, 192),
                          (2900, 3000, 1000, 192)]:
        st, p = plan(M, N, K, ind=F32, outd=F32, **big)
        assert st == 0 and p["kernel_name"] == "mfma_f32" and p["block_m"] == tile, (M, N, K, p)
        assert (p["grid_m"], p["grid_n"]) == (-(-M // tile), -(-N // tile))
    for bm, bk, ok in [(256, 16, True), (256, 32, True), (192, 32, True), (192, 16, False),
                       (128, 16, True), (128, 32, False), (64, 16, False), (256, 64, False)]:
        st, p = plan(1000, 1000, 1000, ind=F32, config=dict(kernel=dtm.DTM_KERNEL_MFMA_F32,
                                                            block_m=bm, block_n=bm, block_k=bk))
        assert (st == 0) == ok and (not ok or (p["block_m"], p["block_k"]) == (bm, bk)), \
            (bm, bk, st, p)
    # chunk depth: 32 at 192 x 192, and at 256 x 256 when K is a multiple of
    # 32; else 16
    for M, N, K, tile, bk, ragged in [(4096, 4096, 4096, 256, 32, 0), (8192, 8192, 8192, 256, 32, 0),
                                      (4096, 4096, 4112, 256, 16, 0), (4096, 4096, 4100, 256, 16, 1),
                                      (3000, 3000, 3008, 192, 32, 1), (3072, 3072, 4112, 192, 32, 1),
                                      (3072, 3072, 4096, 192, 32, 0), (1024, 1024, 1024, 128, 16, 0)]:
        st, p = plan(M, N, K, ind=F32, outd=F32, **big)
        assert st == 0 and (p["block_m"], p["block_k"], p["ragged"]) == (tile, bk, ragged), \
            (M, N, K, p)
        assert p["k_iters"] == -(-K // bk)


def test_fp16acc_control_is_forced_only():
    """The fp16-accumulator negative control runs only when forced, on fp16
    inputs, on the generic kernel's tiles, without split-K."""
    ACC = dtm.DTM_KERNEL_GENERIC_FP16ACC
    for M, N, K, kw in [(4, 4, 1024, dict(ind=F16, outd=F16)),
                        (1024, 1024, 1024, dict(ind=F16, outd=F32))]:
        st, p = plan(M, N, K, **kw)
        assert st == 0 and p["kernel"] != ACC
    st, p = plan(4, 4, 1024, ind=F16, outd=F16,
                 config=dict(kernel=ACC, block_m=128, block_n=128, block_k=8))
    assert st == 0 and p["kernel"] == ACC and p["kernel_name"] == "generic_fp16acc"
    assert (p["block_k"], p["k_iters"], p["threads"]) == (8, 128, 256)
    assert dtm.gemm_kernel_name(ACC) == "generic_fp16acc"
    st, p = plan(300, 200, 150, ind=F16, outd=F32, config=dict(kernel=ACC))
    assert st == 0 and p["kernel"] == ACC
    for kw in [dict(ind=BF16), dict(ind=F32, sam=1024)]:
        st, _ = plan(256, 256, 1024, config=dict(kernel=ACC), **kw)
        assert st == dtm.DTM_ERR_CONFIG, kw
    st, _ = plan(256, 256, 1024, ind=F16, config=dict(kernel=ACC, block_m=256, block_n=256,
                                                      block_k=32))
    assert st == dtm.DTM_ERR_CONFIG
    st, _ = plan(256, 256, 1024, ind=F16, config=dict(kernel=ACC, split_k=4))
    assert st == dtm.DTM_ERR_CONFIG


def test_degenerate_shapes():
    st, p = plan(0, 5, 7)
    assert st == 0 and p["kernel_name"] == "none"
    st, p = plan(5, 0, 7, A=0, B=0, C=0)  # nothing to do: pointers are not needed
    assert st == 0 and p["kernel_name"] == "none"
    st, p = plan(5, 6, 0, A=0, B=0)  # K == 0: zeros into C, A and B never read
    assert st == 0 and p["kernel_name"] == "zero_fill"


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), "DTM_ERR_INVALID_DIM"),
    (dict(K=-5), "DTM_ERR_INVALID_DIM"),
    (dict(N=2 ** 31), "DTM_ERR_INVALID_DIM"),
    (dict(ind=7), "DTM_ERR_DTYPE"),
    (dict(outd=-1), "DTM_ERR_DTYPE"),
    (dict(A=0), "DTM_ERR_NULL_POINTER"),
    (dict(B=0), "DTM_ERR_NULL_POINTER"),
    (dict(C=0), "DTM_ERR_NULL_POINTER"),
    (dict(scm=-64), "DTM_ERR_STRIDE"),
    (dict(scm=0), "DTM_ERR_STRIDE"),
    (dict(scm=32), "DTM_ERR_STRIDE"),           # rows overlap: 32 < N = 64
    (dict(scm=1, scn=32), "DTM_ERR_STRIDE"),    # columns overlap: 32 < M = 48
    (dict(C=PA + 64), "DTM_ERR_ALIAS"),         # C inside A
    (dict(C=PB - 100), "DTM_ERR_ALIAS"),        # C runs into B
    (dict(sam=2 ** 62), "DTM_ERR_STRIDE"),      # A's address range overflows
])
def test_validation_errors(kw, status):
    args = dict(M=48, N=64, K=32)
    for k in ("M", "N", "K"):
        if k in kw:
            args[k] = kw.pop(k)
    st, p = plan(args["M"], args["N"], args["K"], **kw)
    assert dtm.STATUS[st] == status
    assert p["kernel"] == 0


def test_c_strides_accepted():
    # column-major C, padded C, and a single row / column with any stride
    assert plan(48, 64, 32, scm=1, scn=48)[0] == 0
    assert plan(48, 64, 32, scm=100, scn=1)[0] == 0
    assert plan(1, 64, 32, scm=0, scn=1)[0] == 0
    assert plan(48, 1, 32, scm=1, scn=0)[0] == 0


def test_a_and_b_may_alias_each_other_and_broadcast():
    # A and B may overlap (both are only read) and may have zero strides
    assert plan(48, 64, 32, B=PA)[0] == 0
    st, p = plan(48, 64, 32, sam=0, ind=F32)
    assert st == 0  # a broadcast row is a valid layout for every kernel that reads rows
    st, p = plan(48, 64, 32, sam=-32, A=PA + 48 * 32 * 2, ind=F32)
    assert st == 0


def test_forced_configs():
    gen = dtm.DTM_KERNEL_GENERIC
    assert plan(64, 64, 64, config=dict(kernel=gen, block_m=4, block_n=4, block_k=4))[0] == 0
    assert plan(64, 64, 64, config=dict(kernel=gen, block_m=5, block_n=4, block_k=4))[0] == \
        dtm.DTM_ERR_CONFIG
    mf = dtm.DTM_KERNEL_MFMA_F16
    st, p = plan(64, 64, 64, config=dict(kernel=mf, block_m=128, block_n=128, block_k=64))
    assert st == 0 and p["grid_m"] == 1 and p["ragged"] == 1
    assert plan(64, 64, 64, config=dict(kernel=mf, block_m=64, block_n=64, block_k=64))[0] == \
        dtm.DTM_ERR_CONFIG
    # the 32-deep pipelined tile: interior when M, N are multiples of 256
    # and K of 32; its range-checked form needs K % 8 == 0 and, for an
    # N-contiguous B, N % 8 == 0 (an M-contiguous A: M % 8 == 0)
    dma = dict(kernel=mf, block_m=256, block_n=256, block_k=32)
    st, p = plan(512, 256, 96, config=dma)
    assert st == 0 and p["ragged"] == 0
    st, p = plan(500, 256, 96, config=dma)
    assert st == 0 and p["ragged"] == 1 and (p["grid_m"], p["k_iters"]) == (2, 3)
    st, p = plan(512, 256, 104, sam=104, config=dma)
    assert st == 0 and p["ragged"] == 1 and p["k_iters"] == 4
    assert plan(512, 256, 100, sam=104, config=dma)[0] == dtm.DTM_ERR_CONFIG
    assert plan(500, 250, 96, sbk=256, config=dma)[0] == dtm.DTM_ERR_CONFIG
    assert plan(500, 250, 96, sbk=1, sbn=96, config=dma)[0] == 0  # B K-contiguous
    assert plan(500, 256, 96, sam=1, sak=504, config=dma)[0] == dtm.DTM_ERR_CONFIG
    assert plan(504, 256, 96, sam=1, sak=504, config=dma)[0] == 0
    # negative strides or views over 2^31 bytes: not on the range-checked form
    assert plan(500, 256, 96, sam=-96, A=PA + 600 * 96 * 2, config=dma)[0] == \
        dtm.DTM_ERR_CONFIG
    assert plan(40000, 256, 32768, A=1 << 40, B=2 << 40, C=3 << 40, config=dma)[0] == \
        dtm.DTM_ERR_CONFIG
    assert plan(64, 64, 64, config=dict(kernel=99))[0] == dtm.DTM_ERR_CONFIG
    # forced split-K: only on the pipelined tile, K divisible by 32 * split
    st, p = plan(512, 256, 1024, config=dict(dma, split_k=4))
    assert st == 0 and p["split_k"] == 4 and p["k_iters"] == 8
    assert p["workspace_bytes"] == 4 * 512 * 256 * 4
    # uneven slices (256, 256, 256, 232) on the range-checked form
    st, p = plan(512, 256, 1000, sam=1000, config=dict(dma, split_k=4))
    assert st == 0 and p["ragged"] == 1 and p["k_iters"] == 8
    assert plan(512, 256, 1004, sam=1008, config=dict(dma, split_k=4))[0] == dtm.DTM_ERR_CONFIG
    # a split that would leave a slice empty
    assert plan(512, 256, 96, config=dict(dma, split_k=4))[0] == dtm.DTM_ERR_CONFIG
    assert plan(512, 256, 1024, config=dict(kernel=mf, block_m=128, block_n=128, block_k=64,
                                            split_k=2))[0] == dtm.DTM_ERR_CONFIG
    assert plan(512, 256, 1024, ind=F32, config=dict(kernel=gen, split_k=2))[0] == \
        dtm.DTM_ERR_CONFIG


def test_pipelined_wave_count():
    """The 256-wide pipelined tile runs 4 waves (256 threads) on its interior
    form when each tile's K loop is at least 3072 long, else 8 (512
    threads); the 192- and 128-wide tiles run 4; a forced size must be one
    the form has, and only that tile takes one."""
    big = dict(A=1 << 40, B=2 << 40, C=3 << 40)
    for (M, N, K, kw, threads) in [
            (8192, 8192, 8192, dict(), 256),
            (8192, 8192, 8192, dict(sam=1, sak=8192, sbk=1, sbn=8192), 256),
            (4096, 4096, 4096, dict(), 256),
            (4096, 4096, 3072, dict(), 256),
            (4096, 4096, 3040, dict(), 512),                       # K loop under 3072
            (4096, 4096, 2048, dict(), 512),
            (16384, 16384, 1024, dict(), 512),
            (4096, 8192, 64, dict(), 512),
            (8000, 8000, 8000, dict(), 512),                       # range-checked form
            (512, 512, 65536, dict(), 256)]:                       # 128-wide tiles
        st, p = plan(M, N, K, ind=BF16, outd=BF16, **big, **kw)
        assert st == 0 and p["block_k"] == 32 and p["threads"] == threads, (M, N, K, kw, p)
    dma = dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=256, block_n=256, block_k=32)
    for t in (256, 512):
        st, p = plan(512, 256, 96, config=dict(dma, threads=t))
        assert st == 0 and p["threads"] == t and p["ragged"] == 0
        st, p = plan(512, 256, 1024, config=dict(dma, threads=t, split_k=4))
        assert st == 0 and p["threads"] == t and p["split_k"] == 4
    st, p = plan(500, 256, 96, config=dict(dma, threads=512))
    assert st == 0 and p["ragged"] == 1
    # the range-checked form has 8 waves only
    assert plan(500, 256, 96, config=dict(dma, threads=256))[0] == dtm.DTM_ERR_CONFIG
    # 128-wide tiles: 4 waves, both forms, split-K too
    d128 = dict(dma, block_m=128, block_n=128)
    for M, N, K, ragged in [(512, 256, 96, 0), (500, 256, 96, 1), (384, 640, 104, 1)]:
        st, p = plan(M, N, K, sam=K + (-K % 8), config=d128)
        assert st == 0 and (p["block_m"], p["threads"], p["ragged"]) == (128, 256, ragged), p
        assert (p["grid_m"], p["grid_n"]) == (-(-M // 128), -(-N // 128))
    st, p = plan(512, 256, 1024, config=dict(d128, split_k=4))
    assert st == 0 and p["split_k"] == 4 and p["k_iters"] == 8 and p["block_m"] == 128
    assert plan(512, 256, 96, config=dict(d128, threads=512))[0] == dtm.DTM_ERR_CONFIG
    # 192-wide tiles: 4 waves, both forms, split-K too
    d192 = dict(dma, block_m=192, block_n=192)
    for M, N, K, ragged in [(384, 576, 96, 0), (500, 256, 96, 1), (3072, 3072, 4096, 0)]:
        st, p = plan(M, N, K, sam=K + (-K % 8), config=d192)
        assert st == 0 and (p["block_m"], p["threads"], p["ragged"]) == (192, 256, ragged), p
        assert (p["grid_m"], p["grid_n"]) == (-(-M // 192), -(-N // 192))
    st, p = plan(384, 384, 1024, config=dict(d192, split_k=4))
    assert st == 0 and p["split_k"] == 4 and p["k_iters"] == 8 and p["block_m"] == 192
    assert plan(384, 384, 96, config=dict(d192, threads=512))[0] == dtm.DTM_ERR_CONFIG
    assert plan(384, 384, 96, config=dict(dma, block_m=192))[0] == dtm.DTM_ERR_CONFIG
    assert plan(512, 256, 96, config=dict(dma, block_m=128))[0] == dtm.DTM_ERR_CONFIG
    assert plan(512, 256, 96, config=dict(dma, block_m=64, block_n=64))[0] == dtm.DTM_ERR_CONFIG
    for t in (128, 320, 1024, 100):
        assert plan(512, 256, 96, config=dict(dma, threads=t))[0] == dtm.DTM_ERR_CONFIG, t
    assert plan(512, 256, 96, config=dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=256,
                                          block_n=256, block_k=64, threads=256))[0] == \
        dtm.DTM_ERR_CONFIG
    # with the tile left to the selector, the size must suit the tile it picks
    # (128 x 128 here: 4 waves)
    st, p = plan(64, 64, 64, config=dict(threads=256))
    assert st == 0 and (p["block_m"], p["threads"]) == (128, 256)
    assert plan(64, 64, 64, config=dict(threads=512))[0] == dtm.DTM_ERR_CONFIG
    st, p = plan(8192, 8192, 64, A=1 << 40, B=2 << 40, C=3 << 40, config=dict(threads=512))
    assert st == 0 and (p["block_m"], p["threads"]) == (256, 512)
    assert plan(64, 64, 64, ind=F32, outd=F32, config=dict(threads=512))[0] == \
        dtm.DTM_ERR_CONFIG


def test_gemm_rejects_before_touching_a_device():
    """Argument errors come back from gemm() itself without any GPU."""
    assert dtm.gemm_raw(-1, 4, 4, PA, 4, 1, PB, 4, 1, PC, 4, 1, F32, F32) == \
        dtm.DTM_ERR_INVALID_DIM
    assert dtm.gemm_raw(4, 4, 4, PA, 4, 1, PB, 4, 1, PA, 4, 1, F32, F32) == dtm.DTM_ERR_ALIAS
    assert dtm.gemm_raw(0, 4, 4, 0, 4, 1, 0, 4, 1, 0, 4, 1, F32, F32) == dtm.DTM_OK


def test_pointer_check_switch():
    """gemm_set_pointer_checks returns the previous setting; the checks are
    off unless DTM_CHECK_POINTERS (other than "0") is set when the library
    loads; argument errors still come first with them on."""
    import subprocess
    import sys
    prev = dtm.set_pointer_checks(True)
    try:
        assert dtm.set_pointer_checks(True) is True
        assert dtm.gemm_raw(-1, 4, 4, PA, 4, 1, PB, 4, 1, PC, 4, 1, F32, F32) == \
            dtm.DTM_ERR_INVALID_DIM
        assert dtm.set_pointer_checks(False) is True
        assert dtm.set_pointer_checks(False) is False
    finally:
        dtm.set_pointer_checks(prev)
    probe = "import dense_tiled_matrix_amd as d; print(int(d.set_pointer_checks(False)))"
    for env, want in [(None, "0"), ("1", "1"), ("0", "0"), ("yes", "1")]:
        e = {k: v for k, v in os.environ.items() if k != "DTM_CHECK_POINTERS"}
        if env is not None:
            e["DTM_CHECK_POINTERS"] = env
        out = subprocess.run([sys.executable, "-c", probe], env=e, capture_output=True,
                             text=True, check=True).stdout.strip()
        assert out == want, (env, out)


def test_forced_unsplit_rows():
    """dp_rows in a forced configuration: the top rows run unsplit and only the
    rows below them in split_k slices; it must be a multiple of the tile,
    below M, and come with a split on the pipelined kernel."""
    dma = dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=256, block_n=256, block_k=32)
    st, p = plan(1024, 512, 4096, config=dict(dma, split_k=4, dp_rows=512))
    assert st == 0 and (p["split_k"], p["dp_rows"], p["k_iters"], p["ragged"]) == (4, 512, 32, 0)
    assert p["workspace_bytes"] == 4 * 512 * 512 * 4
    st, p = plan(1000, 520, 1000, sam=1000, sbk=520, scm=520,
                 config=dict(dma, split_k=3, dp_rows=512))
    assert st == 0 and (p["split_k"], p["dp_rows"], p["ragged"]) == (3, 512, 1), p
    st, p = plan(960, 576, 2048, config=dict(dma, block_m=192, block_n=192, split_k=4,
                                                dp_rows=576))
    assert st == 0 and (p["block_m"], p["dp_rows"], p["threads"]) == (192, 576, 256), p
    for bad in [dict(split_k=4, dp_rows=300), dict(split_k=4, dp_rows=1024),
                dict(split_k=4, dp_rows=-256), dict(dp_rows=512), dict(split_k=1, dp_rows=512)]:
        assert plan(1024, 512, 4096, config=dict(dma, **bad))[0] == dtm.DTM_ERR_CONFIG, bad
    assert plan(1024, 512, 4096, config=dict(kernel=dtm.DTM_KERNEL_GENERIC, block_m=64,
                                             block_n=64, block_k=16, dp_rows=512))[0] == \
        dtm.DTM_ERR_CONFIG


def test_selector_splits_only_within_the_workspace():
    """gemm() plans within the workspace reserved for its stream; the
    workspace_limit field shows that plan on the host.  The long-K skinny
    case wants 16 slices (16 MiB of fp32 partials); with room for fewer it
    takes the largest split that fits, and with room for none it runs
    unsplit (S up to the cap: the selector's rule takes the cap itself when
    the largest power of two below it is under 3/4 of it).  A forced split
    is not capped."""
    big = dict(A=1 << 40, B=2 << 40, C=3 << 40, ind=F16, outd=F32)
    slice_bytes = 512 * 512 * 4
    for limit, S in [(0, 16), (16 * slice_bytes, 16), (16 * slice_bytes - 1, 15),
                     (9 * slice_bytes, 8), (8 * slice_bytes, 8), (3 * slice_bytes, 3),
                     (2 * slice_bytes, 2), (2 * slice_bytes - 1, 1), (1, 1)]:
        st, p = plan(512, 512, 65536, config=dict(workspace_limit=limit), **big)
        assert st == 0 and p["split_k"] == S, (limit, p)
        assert p["workspace_bytes"] == (S * slice_bytes if S > 1 else 0), (limit, p)
        assert limit == 0 or p["workspace_bytes"] <= limit
    # the split of the last tile-rows (S x rows x N x 4 bytes) likewise
    st, p = plan(7168, 7168, 7168, A=1 << 40, B=2 << 40, C=3 << 40, ind=BF16, outd=BF16)
    assert (p["split_k"], p["dp_rows"]) == (5, 6912), p
    row_bytes = (7168 - 6912) * 7168 * 4
    st, p = plan(7168, 7168, 7168, A=1 << 40, B=2 << 40, C=3 << 40, ind=BF16, outd=BF16,
                 config=dict(workspace_limit=3 * row_bytes))
    assert st == 0 and p["split_k"] <= 3 and p["workspace_bytes"] <= 3 * row_bytes, p
    st, p = plan(7168, 7168, 7168, A=1 << 40, B=2 << 40, C=3 << 40, ind=BF16, outd=BF16,
                 config=dict(workspace_limit=row_bytes))
    assert st == 0 and p["split_k"] == 1 and p["dp_rows"] == 0 and p["workspace_bytes"] == 0, p
    # a forced split reports what it needs, whatever the limit
    cfg = dict(kernel=dtm.DTM_KERNEL_MFMA_F16, block_m=128, block_n=128, block_k=32, split_k=4,
               workspace_limit=1)
    st, p = plan(512, 512, 65536, config=cfg, **big)
    assert st == 0 and p["split_k"] == 4 and p["workspace_bytes"] == 4 * slice_bytes


def test_softmax_plan_split_form_within_budget():
    """row_softmax_plan reports the split form's part count with room for it;
    the host logic that caps it to the stream's workspace is what gemm uses
    (the same lease); here only the unbounded plan is visible."""
    st, p = dtm.row_softmax_plan_raw(64, 262144, PA, 262144, 1, PC, 262144, 1, BF16, BF16)
    assert st == 0 and p["form_name"] == "split" and p["parts"] >= 2, p


def test_tensor_binding_rejects_host_and_mixed_devices():
    """dtm.gemm / gemm_ex / row_softmax raise ValueError, before any library
    call, for host tensors or tensors on different devices: a host pointer
    handed to a kernel would fault the GPU rather than fail."""
    import torch

    a = torch.zeros(64, 32, dtype=torch.float16)
    b = torch.zeros(32, 48, dtype=torch.float16)
    with pytest.raises(ValueError, match="CUDA"):
        dtm.gemm(a, b)
    with pytest.raises(ValueError, match="CUDA"):
        dtm.gemm_ex(a, b, config=dict(kernel=dtm.DTM_KERNEL_GENERIC))
    with pytest.raises(ValueError, match="CUDA"):
        dtm.row_softmax(a)
    meta_a = torch.empty(64, 32, dtype=torch.float16, device="meta")
    with pytest.raises(ValueError, match="different devices"):
        dtm.gemm(meta_a, b, out=torch.empty(64, 48))
    with pytest.raises(ValueError, match="different devices"):
        dtm.row_softmax(a, out=torch.empty(64, 32, dtype=torch.float16, device="meta"))


def test_wave_k_selector():
    """The selector's 128-wide interior plans take the wave-K kernel when
    each tile's K loop (per slice when split) is 4096 or more; shorter loops
    keep the 4-wave form."""
    big = dict(A=1 << 40, B=2 << 40, C=3 << 40)
    for M, N, K, kernel in [(2048, 2048, 8192, "mfma_f16_wavek"), (1536, 1536, 8192, "mfma_f16_wavek"),
                            (8192, 1024, 8192, "mfma_f16_wavek"), (1024, 8192, 8192, "mfma_f16_wavek"),
                            (512, 512, 65536, "mfma_f16_wavek"), (1024, 1024, 16384, "mfma_f16_wavek"),
                            (1024, 1024, 32768, "mfma_f16_wavek"), (640, 640, 32768, "mfma_f16_wavek"),
                            (896, 896, 16384, "mfma_f16_wavek"), (1536, 1536, 4096, "mfma_f16_wavek"),
                            (1024, 1024, 8192, "mfma_f16"), (2048, 2048, 2048, "mfma_f16"),
                            (256, 256, 65536, "mfma_f16"), (1024, 1024, 4096, "mfma_f16")]:
        st, p = plan(M, N, K, ind=BF16, outd=BF16, **big)
        assert st == 0 and p["kernel_name"] == kernel and p["block_m"] == 128, (M, N, K, p)


def test_forced_wave_k_kernel():
    """The wave-K kernel (128 x 128 x 32 tiles whose 4 waves split the K
    loop) is planned when forced on an interior shape: M and N multiples of
    128, K of 128 * split_k, fp16/bf16 inputs; anything else is refused."""
    wk = dtm.DTM_KERNEL_MFMA_F16_WAVEK
    assert dtm.gemm_kernel_name(wk) == "mfma_f16_wavek"
    st, p = plan(512, 384, 1024, config=dict(kernel=wk))
    assert st == 0 and p["kernel"] == wk and (p["block_m"], p["block_n"], p["block_k"]) == \
        (128, 128, 32)
    assert (p["grid_m"], p["grid_n"], p["split_k"], p["threads"], p["k_iters"]) == \
        (4, 3, 1, 256, 32)
    assert p["workspace_bytes"] == 0 and p["ragged"] == 0
    st, p = plan(512, 512, 65536, config=dict(kernel=wk, split_k=16))
    assert st == 0 and p["split_k"] == 16 and p["workspace_bytes"] == 16 * 512 * 512 * 4
    assert p["k_iters"] == 128
    # every layout
    assert plan(256, 256, 256, sam=1, sak=256, config=dict(kernel=wk))[0] == 0
    assert plan(256, 256, 256, sbk=1, sbn=256, config=dict(kernel=wk))[0] == 0
    # explicit tile and workgroup size: only the ones it has
    assert plan(256, 256, 256, config=dict(kernel=wk, block_m=128, block_n=128, block_k=32,
                                           threads=256))[0] == 0
    for bad in (dict(block_m=256, block_n=256, block_k=32), dict(threads=512)):
        assert plan(256, 256, 256, config=dict(kernel=wk, **bad))[0] == dtm.DTM_ERR_CONFIG
    # shapes it does not run: ragged M or N, K not a whole number of
    # 128-deep regions per slice, fp32 inputs, unsplit top rows
    err = dtm.DTM_ERR_CONFIG
    assert plan(200, 256, 256, config=dict(kernel=wk))[0] == err
    assert plan(256, 136, 256, config=dict(kernel=wk))[0] == err
    assert plan(256, 256, 96, config=dict(kernel=wk))[0] == err
    assert plan(256, 256, 1024, config=dict(kernel=wk, split_k=16))[0] == err
    assert plan(256, 256, 256, ind=F32, config=dict(kernel=wk))[0] == err
    assert plan(512, 256, 1024, config=dict(kernel=wk, split_k=2, dp_rows=256))[0] == err


def _plan_with_env(force_env, code):
    """Runs `code` (which prints a result) in a fresh interpreter whose
    DTM_GEMM_FORCE is `force_env` (the library reads it once, at load)."""
    import subprocess
    import sys

    env = dict(os.environ)
    env["DTM_GEMM_FORCE"] = force_env
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prog = ("import sys; sys.path.insert(0, %r); import dense_tiled_matrix_amd as dtm; "
            "PA, PB, PC = 0x10000000, 0x20000000, 0x30000000; " % root) + code
    r = subprocess.run([sys.executable, "-c", prog], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.strip()


_PLAN_4096 = ("st, p = dtm.gemm_plan_raw(4096, 4096, 4096, PA, 4096, 1, PB, 4096, 1, PC, 4096, 1, "
              "dtm.DTM_F16, dtm.DTM_F32{cfg}); "
              "print(st, p['kernel_name'], p['block_m'], p['block_n'], p['block_k'], "
              "p['split_k'])")


def test_env_force_tile_and_split():
    """DTM_GEMM_FORCE gives calls without a configuration of their own a
    forced tile (and split), as gemm_ex's force argument would."""
    out = _plan_with_env("128x128x32,split=4", _PLAN_4096.format(cfg=""))
    assert out == "0 mfma_f16 128 128 32 4"
    out = _plan_with_env("kernel=generic,64x64x16", _PLAN_4096.format(cfg=""))
    assert out == "0 generic 64 64 16 1"
    out = _plan_with_env("kernel=2,64x64x16", _PLAN_4096.format(cfg=""))
    assert out == "0 generic 64 64 16 1"


def test_env_force_yields_to_an_explicit_config():
    cfg = ", {'kernel': dtm.DTM_KERNEL_MFMA_F16, 'block_m': 256, 'block_n': 256, 'block_k': 32}"
    out = _plan_with_env("kernel=generic,64x64x16", _PLAN_4096.format(cfg=cfg))
    assert out == "0 mfma_f16 256 256 32 1"


def test_env_force_unparsable_is_a_config_error():
    for bad in ("128x128", "tile=3", "kernel=nope", "128x128x32,", "split=-1"):
        out = _plan_with_env(bad, _PLAN_4096.format(cfg=""))
        assert out.split()[0] == str(dtm.DTM_ERR_CONFIG), (bad, out)


def test_env_force_empty_is_off():
    out = _plan_with_env("", _PLAN_4096.format(cfg=""))
    _, p = plan(4096, 4096, 4096)
    assert out == f"0 {p['kernel_name']} {p['block_m']} {p['block_n']} {p['block_k']} " \
                  f"{p['split_k']}"
