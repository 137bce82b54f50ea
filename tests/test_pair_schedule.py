"""Event model of the paired-stage schedule of the pipelined GEMM kernel
(gemm_mfma16_pair_kernel): two LDS regions each holding a pair of 32-deep
chunks, refilled in odd iterations, with a wait and a barrier only in odd
iterations.  The model restates the kernel's schedule formulas and checks,
for every even chunk count, that

- every fragment read finds its pair in the region, loaded, waited for by
  the wave that loaded it (vmcnt completes loads in issue order) and
  published to all waves by a barrier before the read's barrier epoch, and
  not overwritten by a load issued in the same or an earlier epoch;
- every refill writes a region whose previous pair all waves have finished
  reading in an earlier epoch (a refill of the same pair, past the end of
  K, writes identical data).

Waves run freely between barriers, so events in one epoch may interleave in
any order across waves; events of different epochs are ordered.
"""
import pytest

NREG = 2  # regions of the kernel


def _schedule(nk, nreg=NREG, even_sync=False):
    np_ = nk // 2
    loads, reads = [], []
    epoch = 0

    def load(region, pair):
        loads.append({"r": region, "j": pair, "ie": epoch, "done": None, "pe": None})

    def wait(outstanding_groups):
        pend = [l for l in loads if l["done"] is None]
        for l in pend[: len(pend) - outstanding_groups]:
            l["done"] = epoch

    def barrier():
        nonlocal epoch
        for l in loads:
            if l["done"] is not None and l["pe"] is None:
                l["pe"] = epoch + 1
        epoch += 1

    def read(chunk):
        reads.append({"r": (chunk >> 1) % nreg, "x": chunk, "e": epoch})

    # prologue: pair r into region r; wait for pair 0; chunk 0's fragments
    for r in range(nreg):
        load(r, r if r < np_ else np_ - 1)
    wait(nreg - 1)
    barrier()
    read(0)
    read(1)  # iteration 0 (even) reads chunk 1
    c = 1
    while c + 1 < nk:
        # odd iteration c: wait, barrier, read chunk c + 1, refill the region of pair (c - 1) / 2
        wait(nreg - 2)
        barrier()
        read(c + 1)
        load(((c - 1) >> 1) % nreg, min((c - 1) // 2 + nreg, np_ - 1))
        # even iteration c + 1: reads chunk c + 2, no wait or barrier
        if even_sync:
            wait(nreg - 1)
            barrier()
        read(c + 2)
        c += 2
    wait(0)
    return loads, reads


def _hazards(loads, reads):
    out = []
    for rd in reads:
        cand = [l for l in loads if l["r"] == rd["r"] and l["ie"] <= rd["e"]]
        last = cand[-1]
        if last["j"] != rd["x"] // 2:
            out.append(("wrong pair", rd, last))
        elif last["pe"] is None or last["pe"] > rd["e"]:
            out.append(("not published", rd, last))
    for i, l in enumerate(loads):
        prev = [q for q in loads[:i] if q["r"] == l["r"]]
        if not prev:
            continue
        pj = prev[-1]["j"]
        for rd in reads:
            if rd["r"] == l["r"] and rd["x"] // 2 == pj and rd["e"] >= l["ie"] and l["j"] != pj:
                out.append(("overwritten while read", rd, l))
    return out


@pytest.mark.parametrize("nk", range(2, 130, 2))
def test_pair_schedule_has_no_hazard(nk):
    loads, reads = _schedule(nk)
    assert _hazards(loads, reads) == []
    # every chunk is read exactly once, in order
    assert [rd["x"] for rd in reads] == list(range(nk))


def test_model_catches_a_missing_odd_barrier():
    """Plant a mistake in the model: refill before the barrier that shows the
    region read (the refill moved into the even iteration)."""
    nk = 16
    np_ = nk // 2
    loads, reads = [], []
    epoch = 0
    # prologue as the kernel
    for r in range(NREG):
        loads.append({"r": r, "j": r, "ie": epoch, "done": epoch, "pe": epoch + 1})
    epoch = 1
    reads.append({"r": 0, "x": 0, "e": epoch})
    # even iteration 0 refills region 0 while chunk 1 is still read from it
    loads.append({"r": 0, "j": min(NREG, np_ - 1), "ie": epoch, "done": None, "pe": None})
    reads.append({"r": 0, "x": 1, "e": epoch})
    assert any(h[0] == "overwritten while read" or h[0] == "wrong pair" for h in _hazards(loads, reads))


def test_model_catches_a_short_wait():
    """Plant a mistake in the model: odd iterations wait for all but one
    refill, so the pair read next may not have landed."""
    nk = 12
    loads, reads = _schedule(nk, nreg=NREG)
    # redo with the wait one group too short
    np_ = nk // 2
    loads2, reads2 = [], []
    epoch = 0

    def load(region, pair):
        loads2.append({"r": region, "j": pair, "ie": epoch, "done": None, "pe": None})

    def wait(k):
        pend = [l for l in loads2 if l["done"] is None]
        for l in pend[: max(len(pend) - k, 0)]:
            l["done"] = epoch

    def barrier():
        nonlocal epoch
        for l in loads2:
            if l["done"] is not None and l["pe"] is None:
                l["pe"] = epoch + 1
        epoch += 1

    for r in range(NREG):
        load(r, r)
    wait(NREG - 1)
    barrier()
    reads2.append({"r": 0, "x": 0, "e": epoch})
    reads2.append({"r": 0, "x": 1, "e": epoch})
    c = 1
    while c + 1 < nk:
        wait(NREG - 1)  # one refill too many left outstanding
        barrier()
        reads2.append({"r": ((c + 1) >> 1) % NREG, "x": c + 1, "e": epoch})
        load(((c - 1) >> 1) % NREG, min((c - 1) // 2 + NREG, np_ - 1))
        reads2.append({"r": ((c + 2) >> 1) % NREG, "x": c + 2, "e": epoch})
        c += 2
    assert _hazards(loads, reads) == []
    assert any(h[0] == "not published" for h in _hazards(loads2, reads2))


def test_even_barrier_is_also_hazard_free():
    """The variant with a wait and barrier in every iteration (the build
    option) is hazard-free too."""
    for nk in range(2, 40, 2):
        assert _hazards(*_schedule(nk, even_sync=True)) == []
