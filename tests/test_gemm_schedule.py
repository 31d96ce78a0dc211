"""CPU model of the grouped GEMMs' load/wait protocol (gemm.hip, gemm_fp8.hip).

The kernels stream K tiles global -> LDS through rings of NA (A) and NB (B) stages with direct
loads whose completion is tracked by hand: `s_waitcnt vmcnt(N)` lets at most the N most recent
loads of a wave stay in flight (loads retire in issue order).  This model replays one wave's
issue order for every K length and checks, at every wait, that

  * the tile the next barrier publishes (all of its A and B loads) has landed, and
  * no load overwrites a stage before the barrier after which no wave reads its old tile
    (tile t is read between the barriers of iterations t - 1 and t).

The issue orders restate the kernels' loops.  test_compiled_waits_match_the_model ties them to
the code that runs: it compiles the GEMM sources to gfx950 assembly with the library's own flags
and requires every instantiated kernel's set of `s_waitcnt vmcnt` counts to be exactly the set
the model's replay waits with, so a change of ring depth, load rounds or wait counts in a kernel
that is not made here as well fails.
"""

import concurrent.futures
import itertools
import os
import re
import subprocess
import tempfile

import pytest


class Wave:
    def __init__(self, NA, NB, nk, loads_a=True):
        self.NA, self.NB, self.nk = NA, NB, nk
        self.issued = []          # (operand, tile) per load, in issue order
        self.last_barrier = -1    # iteration whose barrier was passed last (-1: the prologue's)
        self.needs = {"A", "B"} if loads_a else {"B"}  # operands this wave loads for every tile
        self.waits = set()        # every vmcnt count the replay waited with

    def load(self, op, tile, count):
        ring = self.NA if op == "A" else self.NB
        # the stage's previous tile (tile - ring) is read up to the barrier of its own iteration
        assert tile - ring <= self.last_barrier, (op, tile, self.last_barrier)
        self.issued.extend([(op, tile)] * count)

    def wait(self, n, tile):
        """s_waitcnt vmcnt(n): every load but the n newest has landed; `tile` must be complete."""
        self.waits.add(n)
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


def fp4_kernel(AR, BR, BSR, nk, scale_load):
    """gemm_fp4_kernel: one ring of three stages, each holding a K stage of A, B and both operands'
    scale bytes; the prologue issues stages 0 and 1; in iteration kt the wave waits for stage kt
    (all but the next stage's loads landed), meets the barrier that publishes it, and issues stage
    kt + 2 into the slot stage kt - 1 left.  Waves that gather A scales issue one more load per
    stage."""
    w = Wave(3, 3, nk)

    def issue(kt):
        if kt < nk:
            w.load("A", kt, AR + scale_load)
            w.load("B", kt, BR + BSR)

    issue(0)
    issue(1)
    for kt in range(nk):
        w.wait(AR + BR + BSR + scale_load if kt + 1 < nk else 0, kt)
        w.last_barrier = kt - 1  # the barrier publishing stage kt frees stage kt - 1
        issue(kt + 2)
    return w


# ring depths and loads per wave per tile of the instantiated kernels
BF16 = {"BM 320": (2, 2, 5, 4, 2), "BM 256": (2, 3, 4, 4, 0), "BM 128": (3, 3, 2, 4, 0)}
FP8 = {"MX, BM 192": (2, 3, 3, 4, True), "general, BM 128": (3, 3, 2, 4, False)}
FP4 = {"BM 128": (2, 4, 1)}  # A rounds, B rounds, B scale rounds per wave per stage


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


@pytest.mark.parametrize("name", list(FP4))
def test_fp4_ring_protocol(name):
    AR, BR, BSR = FP4[name]
    for nk, scale_load in itertools.product(range(1, 80), (0, 1)):
        fp4_kernel(AR, BR, BSR, nk, scale_load)


# ---- the model against the compiled kernels

def _model_waits():
    """vmcnt counts of the model's replays, per kernel family and tile height (mangled BM)."""
    out = {}
    for name, (NA, NB, AR, BR, place) in BF16.items():
        s = set()
        for nk, dead in itertools.product(range(1, 80), range(AR + 1)):
            s |= bf16_kernel(NA, NB, AR, BR, nk, dead, place).waits
        out[("gemm_bf16_kernel", int(name.split()[-1]))] = s
    for name, (NA, NB, AR, BR, mx) in FP8.items():
        s = set()
        for nk, scale_load in itertools.product(range(1, 80), (0, 1)):
            s |= fp8_kernel(NA, NB, AR, BR, nk, scale_load, mx).waits
        out[("gemm_fp8_kernel", int(name.split()[-1]))] = s
    for name, (AR, BR, BSR) in FP4.items():
        s = set()
        for nk, scale_load in itertools.product(range(1, 80), (0, 1)):
            s |= fp4_kernel(AR, BR, BSR, nk, scale_load).waits
        out[("gemm_fp4_kernel", int(name.split()[-1]))] = s
    return out


@pytest.fixture(scope="module")
def compiled_asm():
    from mixture_experts_layer_fp32_amd import build
    try:
        cc = build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    srcs = ["gemm.hip", "gemm_fp8.hip", "gemm_fp4.hip"]
    with tempfile.TemporaryDirectory() as d:
        def one(src):
            out = os.path.join(d, src + ".s")
            cmd = [cc] + build._flags() + ["--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
            res = subprocess.run(cmd, capture_output=True, text=True)
            assert res.returncode == 0, res.stderr[-2000:]
            with open(out) as f:
                return f.read()
        with concurrent.futures.ThreadPoolExecutor(len(srcs)) as ex:
            return "\n".join(ex.map(one, srcs))


def test_compiled_waits_match_the_model(compiled_asm):
    """Every instantiated GEMM kernel waits with exactly the vmcnt counts the model's replay of its
    ring configuration uses (the kernels' only vmcnt waits are the protocol's)."""
    model = _model_waits()
    seen = set()
    for m in re.finditer(r"^(_ZN\S*?(gemm_(?:bf16|fp8|fp4)_kernel)ILi(\d+)E\S*):\s*(?:;.*)?$", compiled_asm, re.M):
        sym, fam, bm = m.group(1), m.group(2), int(m.group(3))
        end = compiled_asm.find(".Lfunc_end", m.end())
        waits = {int(v) for v in re.findall(r"s_waitcnt vmcnt\((\d+)\)", compiled_asm[m.end():end])}
        assert (fam, bm) in model, f"{sym}: no model for this tile height"
        assert waits == model[(fam, bm)], (sym, sorted(waits), sorted(model[(fam, bm)]))
        seen.add((fam, bm))
    assert seen == set(model), ("configurations modelled but not compiled", set(model) - seen)


@pytest.mark.parametrize("fam,key,wrong", [
    ("bf16", "BM 256", (2, 3, 3, 4, 0)),           # one A round fewer than the kernel loads
    ("bf16", "BM 320", (2, 3, 5, 4, 0)),           # a third B stage the kernel does not have
    ("fp8", "MX, BM 192", (2, 2, 3, 4, True)),     # a B ring one stage shallower
    ("fp4", "BM 128", (2, 4, 2)),                  # twice the B scale loads
])
def test_compiled_check_detects_a_changed_ring(compiled_asm, monkeypatch, fam, key, wrong):
    """The comparison is not vacuous: a model one step off the kernel's configuration fails it."""
    table = {"bf16": BF16, "fp8": FP8, "fp4": FP4}[fam]
    monkeypatch.setitem(table, key, wrong)
    with pytest.raises(AssertionError):
        test_compiled_waits_match_the_model(compiled_asm)
