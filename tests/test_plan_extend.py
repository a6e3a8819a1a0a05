"""Decode-loop plan reuse (tree_attn_plan_extend) on host-only plans: after
any sequence of leaf growths the extended plan's tables equal, bit for bit,
those of a fresh plan of the grown tree with the same (kept) edge assignment,
both from the library's planner and from the Python re-derivation; errors
leave the plan as it was."""
import numpy as np
import pytest

import synth
from oracle import planner_ref as pr
from tree_structured_shared_amd import Plan, TreeAttnError

EDGES_FORCED, EDGES_KEPT = 1, 2


def _tables_equal(got, ref, edges_mode):
    for name in pr.TABLE_NAMES:
        a, b = np.asarray(ref[name]), np.asarray(got[name])
        if name == "params":
            assert b[16] == edges_mode, ("params[16]", b[16], edges_mode)
            a, b = np.delete(a, 16), np.delete(b, 16)
        assert a.shape == b.shape, (name, a.shape, b.shape)
        assert np.array_equal(a, b), name


def _check_page_table(plan, inst):
    """The page table the kernels read: segment token t of each group is
    (page << 8) | slot of that token, taken from the instance's page lists."""
    seg_tok, bases, groups = plan.export("seg_tok"), plan.export("group_seg"), plan.export("groups")
    ps = inst.page_size
    for gi, (node, top, kv_len) in enumerate(groups[:, :3]):
        path = [int(node)]
        while path[-1] != top:
            path.append(int(inst.parent[path[-1]]))
        want = []
        for u in reversed(path):
            pages = inst.node_page_ids[inst.node_page_ptr[u]:inst.node_page_ptr[u + 1]]
            want += [(int(pages[t // ps]) << 8) | (t % ps) for t in range(int(inst.node_len[u]))]
        assert len(want) == kv_len
        got = seg_tok[bases[gi]:bases[gi] + kv_len]
        assert np.array_equal(got, want), f"group {gi}"
        # the words up to the next segment (the kernels read a few tiles past a
        # segment's end) name written tokens of this segment, at least 96 of them
        end = bases[gi + 1] if gi + 1 < len(bases) else len(seg_tok)
        assert end - (bases[gi] + kv_len) >= 96, f"group {gi}: short guard"
        assert set(seg_tok[bases[gi] + kv_len:end].tolist()) <= set(want), f"group {gi}: guard word"


def _check_against_fresh(plan, inst, edges_mode, **kw):
    _check_page_table(plan, inst)
    edges = plan.export("edges")
    got = plan.tables()
    fresh = Plan.for_instance(inst, host_only=True, force_edges=edges, **kw)
    _tables_equal(got, fresh.tables(), edges_mode)
    fresh.close()
    ref_kw = dict(kw)
    ref_kw.setdefault("ncu", 256)
    _tables_equal(got, pr.plan_instance(inst, force_edges=edges.tolist(), **ref_kw), edges_mode)


@pytest.mark.parametrize("seed", range(24))
def test_extend_random_trees(seed):
    inst = synth.random_small_tree(seed, max_nodes=20, max_len=120, tensors=False)
    rng = np.random.default_rng(seed + 77)
    kw = {}
    if seed % 3 == 1:
        kw = dict(ncu=8, ts_c=16, split_align=16)        # small chunks: growth changes chunk counts
    elif seed % 3 == 2:
        kw = dict(split=False)
    plan = Plan.for_instance(inst, host_only=True, **kw)
    for step in range(6):
        if step == 3:
            add = rng.integers(100, 400, size=inst.n_leaves)   # past the page-table slack
        else:
            add = rng.integers(0, 3, size=inst.n_leaves) * rng.integers(0, 20, size=inst.n_leaves)
        inst, new_pages = synth.grow_leaves(inst, add, seed=1000 * seed + step)
        plan.extend(add, new_pages)
        _check_against_fresh(plan, inst, EDGES_KEPT, **kw)
    plan.close()


@pytest.mark.parametrize("k", [2, 5])
def test_extend_decode_loop_configs(k):
    """Every leaf gains its queries' worth of tokens per step, as in a decode
    loop (40 steps), checked against a fresh plan every 10 steps."""
    inst = synth.make_config(k, tensors=False)
    plan = Plan.for_instance(inst, host_only=True)
    for step in range(1, 41):
        add = np.full(inst.n_leaves, inst.qpl)
        inst, new_pages = synth.grow_leaves(inst, add, seed=step)
        plan.extend(add, new_pages)
        if step % 10 == 0:
            _check_against_fresh(plan, inst, EDGES_KEPT)
    plan.close()


def test_extend_forced_plan_keeps_forced_mark():
    inst = synth.random_small_tree(3, max_nodes=12, tensors=False)
    fe = np.random.default_rng(3).integers(0, 2, inst.n_nodes)
    plan = Plan.for_instance(inst, host_only=True, force_edges=fe)
    add = np.arange(inst.n_leaves) % 5
    inst, new_pages = synth.grow_leaves(inst, add, seed=9)
    plan.extend(add, new_pages)
    _check_against_fresh(plan, inst, EDGES_FORCED)
    plan.close()


def test_extend_zero_growth_changes_nothing():
    inst = synth.make_config(5, tensors=False)
    plan = Plan.for_instance(inst, host_only=True)
    before = plan.tables()
    plan.extend(np.zeros(inst.n_leaves, np.int32), [])
    after = plan.tables()
    for name in pr.TABLE_NAMES:
        a, b = before[name], after[name]
        if name == "params":
            a, b = np.delete(a, 16), np.delete(b, 16)
        assert np.array_equal(a, b), name
    plan.close()


def test_extend_errors_leave_plan_unchanged():
    inst = synth.make_tree([-1, 0, 0], [40, 15, 16], page_size=16, qpl=1, seed=1)
    plan = Plan.for_instance(inst, host_only=True)
    before = plan.tables()
    bad = [
        (([1, 1], []), "the second leaf crosses into a new page: one page needed"),
        (([0, 1], [7, 8]), "one page needed, two given"),
        (([-1, 0], []), "negative growth"),
        (([0, 1], [1 << 23]), "page id out of range"),
        (([0, 1, 0], [5]), "one entry per leaf"),
    ]
    for (add, pages), why in bad:
        with pytest.raises(TreeAttnError):
            plan.extend(add, pages)
        after = plan.tables()
        for name in pr.TABLE_NAMES:
            assert np.array_equal(before[name], after[name]), (why, name)
    # then a valid growth still works
    grown, new_pages = synth.grow_leaves(inst, [1, 1], seed=4)
    plan.extend([1, 1], new_pages)
    _check_against_fresh(plan, grown, EDGES_KEPT)
    plan.close()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_page_table_of_fresh_plans(k):
    inst = synth.make_config(k, tensors=False)
    plan = Plan.for_instance(inst, host_only=True)
    _check_page_table(plan, inst)
    plan.close()
