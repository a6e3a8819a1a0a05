"""Pins of the planner re-derivation (CPU only): the pad closed forms, the
worked grouping example of the FastTree review, hand-computed costs for the
workloads, and structural invariants of every table."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import planner_ref as pr
from oracle.tree_attention import leaves_in_order, root_path

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pad_closed_forms():
    assert pr.pad(16, 1) == 15
    assert pr.pad(16, 16) == 0
    assert pr.pad(16, 17) == 15
    assert pr.pad(16, 0) == 0
    assert pr.pad(64, 64) == 0
    assert pr.pad(64, 32) == 32
    assert pr.pad(16, 8) == 8


def _two_child_tree(M, N, len_root, len_child):
    # root with two leaves; leaf i carries M (resp. N) query tokens
    assert M == N
    return dict(parent=[-1, 0, 0], node_len=[len_root, len_child, len_child], qpl=M)


def test_fasttree_grouping_example():
    with open(os.path.join(GOLDEN, "fasttree_grouping_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        t = _two_child_tree(c["M"], c["N"], c["len_root"], c["len_child"])
        lens = np.array(t["node_len"], np.int32)
        ptr = np.concatenate([[0], np.cumsum((lens + 15) // 16)]).astype(np.int32)
        ids = np.arange(ptr[-1], dtype=np.int32)
        plan = pr.build_plan(t["parent"], lens, ptr, ids, 16, t["qpl"], 4, 4, 128)
        assert plan["edges"][1:].tolist() == c["expected_edges"], c["name"]
        assert plan["nq"][0] == c["root_group_queries"], c["name"]


def test_case_costs_by_hand():
    # case 1 (child 256 tokens): C0 = 0 + 8*256 + 32*8 = 2304 ; C1 = 8*256 + 8*512 = 6144
    assert pr.split_kv_cost(16, 8, 256, 256, 16, 64, 32) == 2304
    assert pr.split_q_cost(16, 8, 256, 256, 16, 64) == 6144
    # a 64-token child: C0 = 8*64 + 32*8 = 768 ; C1 = 8*256 + 8*320 = 4608
    assert pr.split_kv_cost(16, 8, 64, 256, 16, 64, 32) == 768
    assert pr.split_q_cost(16, 8, 64, 256, 16, 64) == 4608
    # case 2: C0 = 32*128 = 4096 ; C1 = 0 (every tile full)
    assert pr.split_kv_cost(256, 128, 256, 256, 16, 64, 32) == 4096
    assert pr.split_q_cost(256, 128, 256, 256, 16, 64) == 0


def test_workload_costs_by_hand():
    # config 1: root 256 with 4 query tokens, leaf 32 with 1
    #   C0 = 12*256 + (15*32 + 1*32) + 32 = 3616 ; C1 = 13*256 + 15*288 = 7648
    assert pr.split_kv_cost(4, 1, 32, 256, 16, 64, 32) == 3616
    assert pr.split_q_cost(4, 1, 32, 256, 16, 64) == 7648
    # config 4: root 32000 with 10 queries, leaf 400 with 1
    #   C0 = 6*32000 + 15*400 + 32 = 198032 ; C1 = 7*32000 + 15*32400 = 710000
    assert pr.split_kv_cost(10, 1, 400, 32000, 16, 64, 32) == 198032
    assert pr.split_q_cost(10, 1, 400, 32000, 16, 64) == 710000


def test_default_intermediate_cost_scales_with_the_gqa_group():
    """The default gamma is 128 per q-head of a kv-head's group (nQ counts query
    tokens; each query leaves g partial rows per kv-head). Root of 256 tokens,
    two 64-token leaves with 2 query tokens each:
      first child:  C0 = CP(4, 256) + CP(2, 64) + 2 gamma = 3072 + 896 + 2 gamma
                    C1 = CP(2, 256) + CP(2, 320) = 3584 + 4480 = 8064
      g = 4  (gamma 512):  C0 = 4992 < 8064 -> 0, and the same for the second child;
      g = 16 (gamma 2048): C0 = 8064 >= 8064 -> 1 (the printed tie rule); then
      second child with cur = 2: C0 = 3584 + 896 + 4096 = 8576 >= CP(0, 256) +
      CP(2, 320) = 4480 -> 1, and the root keeps no queries."""
    lens = np.array([256, 64, 64], np.int32)
    ptr = np.concatenate([[0], np.cumsum((lens + 15) // 16)]).astype(np.int32)
    ids = np.arange(ptr[-1], dtype=np.int32)
    for hq, hk, edges, root_q, gamma in [(16, 4, [0, 0], 4, 512), (64, 4, [1, 1], 0, 2048)]:
        plan = pr.build_plan([-1, 0, 0], lens, ptr, ids, 16, 2, hq, hk, 128)
        assert plan["params"][10] == gamma
        assert plan["edges"][1:].tolist() == edges
        assert plan["nq"][0] == root_q
    assert pr.cost_pad(4, 256, 16, 64) == 3072 and pr.cost_pad(2, 64, 16, 64) == 896
    assert pr.cost_pad(2, 256, 16, 64) == 3584 and pr.cost_pad(2, 320, 16, 64) == 4480


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_simple_trees_aggregate_directly(k):
    """Simple trees keep every edge at 0 (the review's ablation: the greedy
    heuristic tends to aggregate directly on simple trees)."""
    inst = synth.make_config(k, tensors=False)
    plan = pr.plan_instance(inst)
    assert plan["edges"].sum() == 0
    assert plan["params"][18] == inst.n_nodes   # n_groups
    assert len(plan["groups"]) == inst.n_nodes


def check_invariants(inst, plan):
    P = plan["params"]
    n_q = int(P[2])
    g = inst.n_qheads // inst.n_kvheads
    groups = plan["groups"]
    qs, vis = plan["group_qs"], plan["group_vis"]
    lens = inst.node_len.astype(np.int64)
    leaves = leaves_in_order(inst.parent)
    # path length of each query's leaf
    path_len = {}
    for r, lf in enumerate(leaves):
        pl = sum(int(lens[u]) for u in root_path(inst.parent, lf))
        for j in range(inst.qpl):
            path_len[r * inst.qpl + j] = pl
    # (1) group segments of each query partition its path exactly
    covered = {q: 0 for q in range(n_q)}
    for G in groups:
        node, top, kv_len, nq, qptr = G[:5]
        assert nq > 0
        seg = root_path(inst.parent, node)
        seg = seg[seg.index(top):]
        assert sum(int(lens[u]) for u in seg) == kv_len
        for q in qs[qptr:qptr + nq]:
            covered[int(q)] += kv_len
            lf = leaves[int(q) // inst.qpl]
            assert node in root_path(inst.parent, lf)
    for q in range(n_q):
        assert covered[q] == path_len[q]
    # (2) sum kv_len * nQ = sum of path lengths
    assert int((groups[:, 2].astype(np.int64) * groups[:, 3]).sum()) == sum(path_len.values())
    # (3) chunks tile each group's segment
    chunks = plan["chunks"]
    for gi, G in enumerate(groups):
        cp, nch = G[5], G[6]
        cs = chunks[cp:cp + nch]
        assert (cs[:, 0] == gi).all()
        assert cs[0, 1] == 0 and cs[-1, 2] == G[2]
        assert (cs[1:, 1] == cs[:-1, 2]).all() and (cs[:, 2] > cs[:, 1]).all()
    # (4) items cover every (group, row, chunk) exactly once
    seen = set()
    for gi_, r0, nr, ci, _cls in plan["items"]:
        assert chunks[ci, 0] == gi_
        for r in range(r0, r0 + nr):
            key = (int(gi_), r, int(ci))
            assert key not in seen
            seen.add(key)
    total = sum(int(G[3]) * g * int(G[6]) for G in groups)
    assert len(seen) == total
    # (4b) classes: single-wave items are groups of at most stream_rows rows, in
    # one row block, except (tile_join) groups of a full 16-row tile in a plan
    # that has workgroup items; workgroup items come first in launch order
    srows, join = int(P[24]), int(P[27])
    cls = plan["items"][:, 4]
    assert (np.diff(cls) <= 0).all() and int(P[25]) == int((cls == 0).sum())
    has_wg = any(int(G[3]) * g > srows for G in groups)
    for gi_, r0, nr, ci, c in plan["items"]:
        rows_g = int(groups[gi_][3]) * g
        single = rows_g <= srows and not (join and has_wg and rows_g >= 16)
        assert c == (0 if single else 1)
        if c == 0:
            assert r0 == 0 and nr == rows_g
    # (5) slots are a bijection onto (group, chunk, query-in-group)
    sl = plan["q_slots"]
    assert sorted(sl.tolist()) == list(range(int(P[21])))
    # (6) page runs expand to exactly the pages of each chunk's segment tokens
    runs, rp = plan["runs"], plan["chunk_run_ptr"]
    ps = inst.page_size
    for ci, (gi, t0, t1) in enumerate(chunks):
        node, top = groups[gi][0], groups[gi][1]
        seg = root_path(inst.parent, node)
        seg = seg[seg.index(top):]
        expect = []
        for u in seg:
            for t in range(int(lens[u])):
                expect.append((int(inst.node_page_ids[inst.node_page_ptr[u] + t // ps]), t % ps))
        expect = expect[t0:t1]
        got = []
        for page, s0, nt in runs[rp[ci]:rp[ci + 1]]:
            assert 1 <= nt <= ps and s0 + nt <= ps
            got.extend((int(page), int(s0) + i) for i in range(nt))
        assert got == expect
    # (7) visible lengths: a leaf's own queries see its tokens up to their position
    for G in groups:
        node, kv_len, nq, qptr = G[0], G[2], G[3], G[4]
        for q, vv in zip(qs[qptr:qptr + nq], vis[qptr:qptr + nq]):
            lf = leaves[int(q) // inst.qpl]
            if lf == node:
                assert vv == kv_len - (inst.qpl - 1 - int(q) % inst.qpl)
            else:
                assert vv == kv_len


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_invariants_workloads(k):
    inst = synth.make_config(k, tensors=False)
    check_invariants(inst, pr.plan_instance(inst))


@pytest.mark.parametrize("seed", range(60))
def test_invariants_random(seed):
    inst = synth.random_small_tree(seed, tensors=False)
    rng = np.random.default_rng(seed)
    kw = {}
    if seed % 3 == 1:
        kw["force_edges"] = rng.integers(0, 2, size=inst.n_nodes).tolist()
    if seed % 4 == 2:
        kw["ncu"] = 4
        kw["ts_c"] = 16
    check_invariants(inst, pr.plan_instance(inst, **kw))


def test_forced_all_ones_is_query_separated():
    inst = synth.make_config(2, tensors=False)
    plan = pr.plan_instance(inst, force_edges=[1] * inst.n_nodes)
    groups = plan["groups"]
    assert len(groups) == 16 and (groups[:, 3] == 1).all()
    assert (groups[:, 2] == 2048 + 512 + 128).all()


def test_split_off_single_chunk():
    inst = synth.make_config(4, tensors=False)
    plan = pr.plan_instance(inst, split=0)
    assert len(plan["chunks"]) == len(plan["groups"])


def test_long_root_is_split():
    inst = synth.make_config(4, tensors=False)
    plan = pr.plan_instance(inst)
    root_group = plan["groups"][0]
    assert root_group[6] > 10  # the 32000-token root is cut into many chunks


def test_validation_errors():
    ok = dict(parent=[-1, 0], node_len=[4, 4], node_page_ptr=[0, 1, 2], node_page_ids=[0, 1],
              page_size=16, qpl=1, n_qheads=4, n_kvheads=4, head_dim=128)
    pr.build_plan(**ok)
    bad = [dict(parent=[-1, -1]), dict(parent=[1, 0]), dict(node_len=[4, 0]),
           dict(qpl=5), dict(n_qheads=6), dict(head_dim=96), dict(node_page_ptr=[0, 1, 1]),
           dict(parent=[-1, 5])]
    for b in bad:
        kw = dict(ok)
        kw.update(b)
        with pytest.raises(pr.PlanError):
            pr.build_plan(**kw)
