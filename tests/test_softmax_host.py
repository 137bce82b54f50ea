"""Host-side checks of the row-softmax C ABI (no GPU): exported symbols,
validation before any launch, and the launch plan."""
import dense_tiled_matrix_amd as dtm

F32, F16, BF16 = dtm.DTM_F32, dtm.DTM_F16, dtm.DTM_BF16
PX, PY = 1 << 40, 2 << 40


def plan(M, N, X=PX, sxm=None, sxn=1, Y=PY, sym=None, syn=1, ind=F32, outd=None):
    sxm = N if sxm is None else sxm
    sym = N if sym is None else sym
    return dtm.row_softmax_plan_raw(M, N, X, sxm, sxn, Y, sym, syn, ind,
                                    ind if outd is None else outd)


def test_symbols_exported():
    L = dtm.lib()
    for n in ["row_softmax", "row_softmax_plan"]:
        assert n in dtm.header_functions() and hasattr(L, n)


def test_forms_by_row_length():
    """A wave per row while the row fits in a wave's registers (16 chunks per
    lane) and rows are many; a workgroup per row up to 16 chunks per thread
    for fp32 rows, 8 for 16-bit ones, past 4 only when the row fills at
    least 3/4 of its chunks; beyond that the two-pass online form.  16-byte
    chunks: 4 fp32 or 8 fp16/bf16 elements."""
    cases = [
        (32768, 1024, F16, "wave", 2, 8, 1),
        (32768, 4096, F16, "wave", 8, 8, 1),
        (4096, 2048, F32, "wave", 8, 4, 1),
        (4096, 4096, F32, "wave", 16, 4, 1),
        (8192, 8192, BF16, "wave", 16, 8, 1),
        (1024, 8192, BF16, "block", 1, 8, 1),   # fewer rows: a workgroup per row
        (256, 16384, F32, "block", 4, 4, 1),
        (256, 65536, F32, "block", 16, 4, 1),
        (256, 49152, F32, "block", 16, 4, 1),  # 75% of 16 chunks
        (256, 49148, F32, "online", 2, 4, 2),
        (256, 40000, F32, "online", 2, 4, 2),
        (300, 60000, BF16, "block", 8, 8, 1),
        (300, 65544, BF16, "online", 2, 8, 2),  # 16-bit rows: at most 8 chunks
        (256, 16388, F32, "online", 2, 4, 2),   # 50% of 8 chunks
        (256, 24576, F32, "block", 8, 4, 1),
        (256, 65540, F32, "online", 2, 4, 2),
        (128, 2048, F32, "block", 1, 4, 1),  # few rows: a workgroup per row
        (64, 512, F32, "wave", 2, 4, 1),
    ]
    for M, N, ind, form, ch, e, passes in cases:
        st, p = plan(M, N, ind=ind)
        assert st == 0, (M, N)
        assert (p["form_name"], p["chunks"], p["chunk_elems"], p["passes"]) == \
            (form, ch, e, passes), (M, N, p)
        assert p["vectorized"] == 1 and p["parts"] == 1
        assert p["grid"] == (-(-M // 4) if form == "wave" else M)
        assert p["threads"] == (256 if form == "wave" else 1024)


def test_split_form_for_few_long_rows():
    """Fewer than 128 rows that a wave cannot hold: each row is split over
    about 256 / M workgroups, parts of whole tiles (2048 chunks), none
    empty."""
    for M, N, ind, parts in [(64, 262144, BF16, 4), (8, 1048576, F32, 32), (1, 100003, F32, 13),
                             (100, 65536, F32, 3), (127, 16384, F32, 2), (64, 2048, F32, 1)]:
        st, p = plan(M, N, ind=ind)
        assert st == 0
        e = 4 if ind == F32 else 8
        tile = 1024 * 2 * e
        assert p["parts"] == parts, (M, N, p)
        if parts > 1:
            assert p["form_name"] == "split" and p["passes"] == 2 and p["grid"] == M * parts
            length = -(-(-(-N // parts)) // tile) * tile
            assert (parts - 1) * length < N <= parts * length
        else:
            assert p["form_name"] != "split"


def test_vectorization_conditions():
    """16-byte loads need unit column strides, a 16-byte aligned X row and a Y
    row aligned to one chunk's output."""
    assert plan(100, 1000)[1]["vectorized"] == 1
    assert plan(100, 1000, sxm=1001)[1]["vectorized"] == 0      # row stride not 16 B
    assert plan(100, 1000, X=PX + 4)[1]["vectorized"] == 0      # base not 16 B
    assert plan(100, 1000, sxn=2, sxm=2000)[1]["vectorized"] == 0
    assert plan(100, 1000, sym=1, syn=100)[1]["vectorized"] == 0  # transposed output
    st, p = plan(100, 1000, ind=F32, outd=F16, sym=1004)         # 8-byte output chunks
    assert st == 0 and p["vectorized"] == 1
    assert plan(100, 1000, ind=F32, outd=F16, sym=1002)[1]["vectorized"] == 0
    st, p = plan(100, 1000, sxn=1, sxm=1000, sym=1, syn=100)
    assert st == 0 and p["vectorized"] == 0 and p["chunk_elems"] == 1


def test_validation_before_launch():
    S = dtm.STATUS
    inv = {v: k for k, v in S.items()}
    assert plan(-1, 5)[0] == inv["DTM_ERR_INVALID_DIM"]
    assert plan(5, 1 << 31)[0] == inv["DTM_ERR_INVALID_DIM"]
    assert plan(5, 5, ind=7)[0] == inv["DTM_ERR_DTYPE"]
    assert plan(5, 5, outd=9)[0] == inv["DTM_ERR_DTYPE"]
    assert plan(5, 5, X=0)[0] == inv["DTM_ERR_NULL_POINTER"]
    assert plan(5, 5, Y=0)[0] == inv["DTM_ERR_NULL_POINTER"]
    assert plan(5, 5, sym=2)[0] == inv["DTM_ERR_STRIDE"]        # output rows overlap
    assert plan(5, 5, sym=-5)[0] == inv["DTM_ERR_STRIDE"]
    # in place: the identical view is allowed, any other overlap is not
    assert plan(5, 5, Y=PX)[0] == 0
    assert plan(5, 5, Y=PX + 8)[0] == inv["DTM_ERR_ALIAS"]
    assert plan(5, 5, Y=PX, ind=F32, outd=F16)[0] == inv["DTM_ERR_ALIAS"]
    # X may be broadcast or reversed
    assert plan(5, 5, sxm=0)[0] == 0
    assert plan(5, 5, sxm=-5, X=PX + 100)[0] == 0
    # empty shapes are no-ops, even with null pointers
    st, p = plan(0, 5, X=0, Y=0)
    assert st == 0 and p["form_name"] == "none"
    st, p = plan(5, 0, X=0, Y=0)
    assert st == 0 and p["form_name"] == "none"


def test_row_softmax_rejects_before_touching_a_device():
    inv = {v: k for k, v in dtm.STATUS.items()}
    assert dtm.row_softmax_raw(-1, 4, PX, 4, 1, PY, 4, 1, F32, F32) == inv["DTM_ERR_INVALID_DIM"]
    assert dtm.row_softmax_raw(4, 4, PX, 4, 1, PX + 4, 4, 1, F32, F32) == inv["DTM_ERR_ALIAS"]
    assert dtm.row_softmax_raw(0, 4, 0, 4, 1, 0, 4, 1, F32, F32) == 0
