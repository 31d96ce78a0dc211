"""CPU model of the grouped GEMMs' load/wait protocol (gemm.hip, gemm_fp8.hip).

The kernels stream K tiles global -> LDS through rings of NA (A) and NB (B) stages with direct
loads whose completion is tracked by hand: `s_waitcnt vmcnt(N)` lets at most the N most recent
loads of a wave stay in flight (loads retire in issue order).  This model replays one wave's
issue order for every K length and checks, at every wait, that

  * the tile the next barrier publishes (all of its A and B loads) has landed, and
  * no load overwrites a stage before the barrier after which no wave reads its old tile
    (tile t is read between the barriers of iterations t - 1 and t).

The issue orders restate the kernels' loops: a change there must be mirrored here.
"""

import itertools

import pytest


class Wave:
    def __init__(self, NA, NB, nk, loads_a=True):
        self.NA, self.NB, self.nk = NA, NB, nk
        self.issued = []          # (operand, tile) per load, in issue order
        self.last_barrier = -1    # iteration whose barrier was passed last (-1: the prologue's)
        self.needs = {"A", "B"} if loads_a else {"B"}  # operands this wave loads for every tile

    def load(self, op, tile, count):
        ring = self.NA if op == "A" else self.NB
        # the stage's previous tile (tile - ring) is read up to the barrier of its own iteration
        assert tile - ring <= self.last_barrier, (op, tile, self.last_barrier)
        self.issued.extend([(op, tile)] * count)

    def wait(self, n, tile):
        """s_waitcnt vmcnt(n): every load but the n newest has landed; `tile` must be complete."""
        done = len(self.issued) - n
        assert done >= 0
        ops = set()
        for i, (op, t) in enumerate(self.issued):
            if t == tile:
                assert i < done, ("tile in flight", tile, op, n)
                ops.add(op)
        assert ops == self.needs, ("tile never loaded", tile, ops)


def bf16_kernel(NA, NB, AR, BR, nk, dead=0, place=0):
    """gemm_bf16_kernel: prologue groups -NB..-1 (A tile j+NA, B tile j+NB); in iteration kt the
    B loads of tile kt-1+NB go out in k-steps 1 and 2 (place 0), the wait for tile kt+1 and the
    barrier follow k-step 2, and the A loads of tile kt+NA take the last slots of the last k-step,
    followed there by the B loads of tile kt+NB with place 2.  A wave skips `dead` of its AR A
    loads per tile (the rounds past the tile's last live row block); its waits allow (NA - 1) and
    (NA - 2) groups of AR - dead + BR loads."""
    ar = AR - dead
    w = Wave(NA, NB, nk, loads_a=ar > 0)
    RPT = ar + BR
    after = BR if NB > NA else 0

    def group(j):
        if 0 <= j + NA < nk and ar:
            w.load("A", j + NA, ar)
        if j + NB < nk:
            w.load("B", j + NB, BR)

    for j in range(-NB, 0):
        group(j)
    w.wait(after + (NA - 1) * RPT if NB <= nk else 0, 0)
    w.last_barrier = -1
    for kt in range(nk):
        tb = kt - 1 + NB
        if place == 0 and kt >= 1 and tb < nk:
            w.load("B", tb, BR // 2)           # k-step 1
            w.load("B", tb, BR - BR // 2)      # k-step 2
        if kt + 1 < nk:
            w.wait(after + (NA - 2) * RPT if kt + NB <= nk else 0, kt + 1)
            w.last_barrier = kt
        if kt + 1 < nk and kt + NA < nk and ar:
            w.load("A", kt + NA, ar)           # last k-step
        if place == 2 and kt + 1 < nk and kt + NB < nk:
            w.load("B", kt + NB, BR)           # last k-step, after the A loads
    return w


def fp8_kernel(NA, NB, AR, BR, nk, scale_load, mx):
    """gemm_fp8_kernel: prologue groups -max(NA,NB)..-1 (A tile j+NA with its scale load on the
    scale-gathering waves, then B tile j+NB).  MX: in iteration kt the B loads of tile kt-1+NB
    take the last slots of the first sub-step, the wait and barrier follow, and the A loads (+
    scale) of tile kt+NA the last slots of the second.  General variant: group kt whole, right
    after the barrier."""
    w = Wave(NA, NB, nk)
    AR1 = AR + scale_load
    RPT = AR + BR
    NM, GM = max(NA, NB), min(NA, NB)
    after = BR if NB > NA else 0

    def wait_count(full, G):
        return after + G * (RPT + scale_load) if full else 0

    def a_part(j):
        if 0 <= j + NA < nk:
            w.load("A", j + NA, AR1)

    def group(j):
        a_part(j)
        if 0 <= j + NB < nk:
            w.load("B", j + NB, BR)

    for j in range(-NM, 0):
        group(j)
    w.wait(wait_count(NM <= nk, GM - 1), 0)
    for kt in range(nk):
        if mx:
            tb = kt - 1 + NB
            if kt >= 1 and tb < nk:
                w.load("B", tb, BR)
        if kt + 1 < nk:
            w.wait(wait_count(kt + NM <= nk, GM - 2), kt + 1)
            w.last_barrier = kt
            if mx:
                a_part(kt)
            else:
                group(kt)
    return w


# ring depths and loads per wave per tile of the instantiated kernels
BF16 = {"BM 320": (2, 2, 5, 4, 2), "BM 256": (2, 3, 4, 4, 0), "BM 128": (3, 3, 2, 4, 0)}
FP8 = {"MX, BM 192": (2, 3, 3, 4, True), "general, BM 128": (3, 3, 2, 4, False)}


@pytest.mark.parametrize("name", list(BF16))
def test_bf16_ring_protocol(name):
    NA, NB, AR, BR, place = BF16[name]
    for nk, dead in itertools.product(range(1, 80), range(AR + 1)):
        bf16_kernel(NA, NB, AR, BR, nk, dead, place)



def test_dead_rounds_need_the_reduced_counts():
    """With skipped A loads the unreduced wait count is too permissive for the deeper A ring (the
    tile's B loads may still be in flight), so the reduction is what keeps the protocol correct."""
    NA, NB, AR, BR, _ = BF16["BM 128"]
    nk, dead = 8, 1
    w = Wave(NA, NB, nk)
    ar = AR - dead
    for j in range(-NB, 0):
        if 0 <= j + NA < nk:
            w.load("A", j + NA, ar)
        w.load("B", j + NB, BR)
    with pytest.raises(AssertionError):
        w.wait((NA - 1) * (AR + BR), 0)   # the count without the skipped loads
    w.wait((NA - 1) * (ar + BR), 0)


@pytest.mark.parametrize("name", list(FP8))
def test_fp8_ring_protocol(name):
    NA, NB, AR, BR, mx = FP8[name]
    for nk, scale_load in itertools.product(range(1, 80), (0, 1)):
        fp8_kernel(NA, NB, AR, BR, nk, scale_load, mx)


def test_model_catches_a_short_wait():
    """The model is not vacuous: one load fewer allowed in flight passes, one more fails."""
    NA, NB, AR, BR, _ = BF16["BM 256"]
    w = Wave(NA, NB, 10)
    w.load("A", 0, AR)
    w.load("B", 0, BR)
    w.load("B", 1, BR)
    w.wait(BR, 0)
    with pytest.raises(AssertionError):
        w.wait(BR + 1, 0)


def test_model_catches_an_early_overwrite():
    w = Wave(2, 3, 10)
    with pytest.raises(AssertionError):
        w.load("A", 2, 1)  # the stage of A tile 0, before the barrier of iteration 0
    w.last_barrier = 0
    w.load("A", 2, 1)
