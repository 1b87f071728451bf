"""Host model of the GEMM kernel's vector-memory wait accounting (CPU only).

The grouped-GEMM kernel (csrc/gmm.hip, gmm_kernel) moves operand tiles into
LDS with LDS-DMA loads and orders them by hand: every wait names how many of
the wave's vector-memory operations may still be in flight.  One counter
covers loads and stores, and a store may retire before older loads; loads
retire in issue order among themselves.  The model below replays, per wave,
the main loop's issue order -- NS - 1 stages loaded ahead, LPS transfers per
k-step, the fp8 epilogue's scale loads at the top of an item's last k-step,
NST stores per epilogue -- and checks every wait against the worst
retirement that order allows (every store first, then the oldest loads),
for all the kernel's stage counts and many item-length mixes.

Checked at each wait:
  * top of a k-step: the stage it reads has landed;
  * an epilogue: (fp8) the tile's scale loads have landed, and the stage the
    next k-step reads has landed before any store is issued -- which is what
    lets the next top-of-k-step wait allow for the stores.
"""
import itertools

import pytest


def _worst_case_wait(outstanding, n):
    """Retire stores first, then the oldest loads, until at most n remain."""
    loads = [op for op in outstanding if op[0] != "S"]
    keep = min(n, len(loads))
    return loads[len(loads) - keep:] if keep else []


def simulate(items, NS, LPS, NST, scaled, nsc, epi_waits_for_stage=True):
    """Replay one wave's issue order over work items of the given k-step
    counts; returns a list of violations (empty when every wait is safe)."""
    epi_vm_stages = (NS - 2) * LPS
    epi_vm = min(epi_vm_stages, LPS) if scaled else epi_vm_stages
    top_after_epi = (NS - 2) * LPS + NST
    out, bad = [], []

    def wait(n, need, where):
        nonlocal out
        out = _worst_case_wait(out, n)
        still = [op for op in out if op in need]
        if still:
            bad.append((where, still[0]))

    nxt = 0   # k-step whose stage the next load fills
    for _ in range(NS - 1):
        out += [("L", nxt)] * LPS
        nxt += 1
    j, epi_prev = 0, False
    for it, nsteps in enumerate(items):
        for s in range(nsteps):
            wait(top_after_epi if epi_prev else (NS - 2) * LPS, {("L", j)}, ("top", it, s))
            epi_prev = False
            if scaled and s == nsteps - 1:
                out += [("C", it)] * nsc
            out += [("L", nxt)] * LPS
            nxt += 1
            j += 1
        need = {("C", it)} if scaled else set()
        if epi_waits_for_stage:
            need.add(("L", j))
            wait(epi_vm, need, ("epilogue", it))
        elif scaled:
            wait(epi_vm, need, ("epilogue", it))
        out += [("S", it)] * NST
        epi_prev = True
    return bad


_ITEMS = [[1] * 6, [2, 1, 1, 3], [1, 5, 1], [12, 1, 1, 12], [3] * 4, [1, 2] * 3]


@pytest.mark.parametrize("NS", [2, 3])
@pytest.mark.parametrize("scaled", [False, True])
def test_every_wait_is_safe_under_out_of_order_stores(NS, scaled):
    for LPS, NST, nsc, items in itertools.product([2, 4, 6, 8, 16], [4, 8, 16], [0, 1], _ITEMS):
        if not scaled and nsc:
            continue
        assert simulate(items, NS, LPS, NST, scaled, nsc) == [], (LPS, NST, nsc, items)


def test_model_catches_an_epilogue_without_the_stage_wait():
    """Without the epilogue's wait for the next stage, the top-of-k-step
    wait that allows for the stores can pass with that stage in flight once
    stores retire early (NST >= LPS): the model must report it."""
    bad = simulate([1, 1, 1], 3, 6, 8, False, 0, epi_waits_for_stage=False)
    assert bad and bad[0][0][0] == "top"
    # in the fp8 form the scale wait already covers the stage (NS = 3)
    assert simulate([1, 1, 1], 3, 6, 8, True, 1, epi_waits_for_stage=False) == []


def test_model_catches_scales_issued_after_the_transfers():
    """If an item's scale loads followed its last k-step's transfers, the
    epilogue's wait (at most LPS loads in flight) would not cover them."""
    def late_scales(items, NS, LPS, NST):
        out, bad, nxt = [], [], 0
        for _ in range(NS - 1):
            out += [("L", nxt)] * LPS
            nxt += 1
        for it, nsteps in enumerate(items):
            for s in range(nsteps):
                out = _worst_case_wait(out, (NS - 2) * LPS + NST)
                out += [("L", nxt)] * LPS
                nxt += 1
                if s == nsteps - 1:
                    out += [("C", it)]
            out = _worst_case_wait(out, min((NS - 2) * LPS, LPS))
            if ("C", it) in out:
                bad.append(it)
            out += [("S", it)] * NST
        return bad
    assert late_scales([1, 2, 1], 3, 6, 8)
