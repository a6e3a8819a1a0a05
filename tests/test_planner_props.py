"""Properties of the planner's row blocks, long-context split and launch
order (steps P6-P8), checked on the library's host-only plans of the five
workloads and of random trees (CPU only).

These follow from what the pages ask of the steps, not from the rule the
planner uses to meet it:

* multi-stage query tiling (FastTree review, kernel design): a group's rows
  are cut into as few blocks as the tile limit allows, and the blocks are
  even, so no block is a nearly empty tile;
* long-context splitting (FastTree review, section 3.3): the launch should
  fill the GPU and its last wave should not be left to a few long units.
  Checked here as: chunks cut a segment into equal pieces (a shorter last
  one at most); a larger machine never gets longer chunks; when the tree
  holds enough work, the launch has at least as many units as the machine
  has compute units; and no unit is longer than a few fair shares of the
  streaming work per wave slot (or its group's floor for partial traffic);
* the launch order is longest-first: a list schedule of the units in launch
  order on the machine's slots then meets Graham's bound for the
  longest-processing-time rule, makespan <= (4/3) x max(mean load, longest
  unit), on the planner's own cost estimate.

Constants (rb, split alignment, waves per CU, the chunk floor) are the
library's own; the pages print none (parity unpinned for their values).
"""
import heapq

import numpy as np
import pytest

import synth
from tree_structured_shared_amd import Plan

RB, ALIGN, WAVES, FLOOR_F, STREAM_ROWS = 128, 128, 5, 4, 16


def _plan(inst, **kw):
    p = Plan.for_instance(inst, host_only=True, **kw)
    t = {k: p.export(k) for k in ("params", "groups", "chunks", "items")}
    p.close()
    return t


def _cases():
    for k in (1, 2, 3, 4, 5):
        yield f"config{k}", synth.make_config(k, tensors=False)
    for seed in range(25):
        yield f"rand{seed}", synth.random_small_tree(seed, max_nodes=40, max_len=3000, tensors=False)


CASES = list(_cases())


@pytest.mark.parametrize("name,inst", CASES, ids=[c[0] for c in CASES])
def test_row_blocks_are_minimal_and_even(name, inst):
    t = _plan(inst)
    g = inst.n_qheads // inst.n_kvheads
    groups, items = t["groups"], t["items"]
    blocks = {}
    for gi, r0, nr, ci, cls in items:
        blocks.setdefault((int(gi), int(ci)), []).append((int(r0), int(nr), int(cls)))
    for (gi, ci), bl in blocks.items():
        rows = int(groups[gi][3]) * g
        bl.sort()
        # the blocks partition [0, rows) in order
        assert bl[0][0] == 0 and sum(b[1] for b in bl) == rows
        assert all(bl[x][0] + bl[x][1] == bl[x + 1][0] for x in range(len(bl) - 1))
        sizes = [b[1] for b in bl]
        if bl[0][2] == 0:   # a single-wave item holds the whole (small) group
            assert len(bl) == 1 and rows <= STREAM_ROWS
        else:               # as few blocks as the limit allows, even in 16-row tiles
            assert max(sizes) <= RB and len(bl) == -(-rows // RB)
            tiles = [-(-n // 16) for n in sizes]
            assert max(tiles) - min(tiles) <= 1
            assert all(n % 16 == 0 for n in sizes[:-1])  # only the last block ends in a partial tile


@pytest.mark.parametrize("name,inst", CASES, ids=[c[0] for c in CASES])
def test_chunks_are_even_and_shrink_with_the_machine(name, inst):
    prev = None
    for ncu in (64, 256, 1024):
        t = _plan(inst, ncu=ncu)
        longest = {}
        for gi, G in enumerate(t["groups"]):
            cs = t["chunks"][int(G[5]):int(G[5]) + int(G[6])]
            lens = cs[:, 2] - cs[:, 1]
            # equal pieces, 16-token aligned, a shorter last one at most
            assert (lens[:-1] == lens[0]).all() and lens[-1] <= lens[0] and (lens[:-1] % 16 == 0).all()
            longest[(int(G[0]), int(G[1]))] = int(lens[0])
        if prev is not None:   # the same groups (the grouping does not depend on ncu)
            assert prev.keys() == longest.keys()
            assert all(longest[k] <= prev[k] for k in longest), (ncu, name)
        prev = longest


def _units(inst, t):
    """Per unit (item x kv-head): streamed tokens, rows, class."""
    H = inst.n_kvheads
    out = []
    for gi, r0, nr, ci, cls in t["items"]:
        toks = int(t["chunks"][ci][2] - t["chunks"][ci][1])
        out += [(toks, int(nr), int(cls))] * H
    return out


@pytest.mark.parametrize("name,inst", CASES, ids=[c[0] for c in CASES])
def test_split_fills_the_machine_without_a_long_tail(name, inst):
    ncu = 256
    g = inst.n_qheads // inst.n_kvheads
    t = _plan(inst, ncu=ncu)
    units = _units(inst, t)
    # streaming work in wave-slot tokens: a workgroup unit's four waves share
    # one stream, a single-wave unit is one wave's stream
    slots = ncu * WAVES
    work = sum(tok for tok, _, _ in units)
    fair = work / slots
    groups = t["groups"]
    # the most units the chunk floors allow (the floor keeps a row's partial
    # results, written and read back, small against the K/V it streams: the
    # pages' intermediate-result cost)
    blocks = {}
    for gi, r0, nr, ci, c in t["items"]:
        blocks.setdefault(int(gi), set()).add(int(r0))
    most = 0
    for gi, G in enumerate(groups):
        rows = int(G[3]) * g
        floor = max(ALIGN, -(-FLOOR_F * min(rows, RB) // ALIGN) * ALIGN)
        most += inst.n_kvheads * len(blocks[gi]) * -(-int(G[2]) // floor)
    if work >= ncu * ALIGN:
        assert len(units) >= min(ncu, most), (name, len(units), most)
    for gi, r0, nr, ci, cls in t["items"]:
        toks = int(t["chunks"][ci][2] - t["chunks"][ci][1])
        rows = int(groups[gi][3]) * g
        floor = -(-FLOOR_F * min(rows, RB) // ALIGN) * ALIGN
        # a unit is at most a few fair shares long, or its group's floor
        assert toks <= max(3 * fair + ALIGN, floor), (name, toks, fair, floor)
    # without the split the longest unit of a long-context tree is a whole group
    if name == "config4":
        t0 = _plan(inst, ncu=ncu, split=False)
        assert max(tok for tok, _, _ in _units(inst, t0)) > 8 * max(tok for tok, _, _ in units)


@pytest.mark.parametrize("name,inst", CASES, ids=[c[0] for c in CASES])
def test_launch_order_meets_the_longest_first_bound(name, inst):
    """Graham's bound for longest-processing-time list scheduling, on the
    planner's cost estimate (chunk tokens x (256 + rows)) per unit, with the
    workgroup units first on the workgroup slots and the single-wave units
    after them."""
    ncu = 256
    t = _plan(inst, ncu=ncu)
    units = _units(inst, t)
    cls = [c for _, _, c in units]
    assert cls == sorted(cls, reverse=True)  # workgroup units first
    for c, m in ((1, 2 * ncu), (0, 8 * ncu)):
        jobs = [tok * (256 + nr) for tok, nr, cc in units if cc == c]
        if not jobs:
            continue
        free = [0] * min(m, len(jobs))
        heapq.heapify(free)
        span = 0
        for j in jobs:   # in launch order, each on the earliest free slot
            s = heapq.heappop(free)
            span = max(span, s + j)
            heapq.heappush(free, s + j)
        lower = max(sum(jobs) / m, max(jobs))
        assert span <= (4 / 3) * lower + 1e-9, (name, c, span / lower)
