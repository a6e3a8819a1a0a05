"""CPU: the peaky-softmax GPU cases (tests/test_gpu_peaky.py) reach the
branches they are meant for. With the chunks the library's planner cuts
(host-only plan), some row of each case raises its running max in the middle
of a chunk by more than the kernels' lazy-rescale threshold, and some query
has partials whose maxima lie further apart than that threshold (the merge's
large-weight-ratio case). Scores here are plain fp64 dot products of the
instance's own Q and K rows."""
import numpy as np
import pytest
import torch

import synth
from oracle import tree_attention as ta
from tree_structured_shared_amd import Plan
from test_gpu_peaky import peaky_tree

RESCALE_LOG2 = 8.0  # the kernels raise the running max only past this many log2 units
TILE = 32


def _segments(inst):
    """Each group's token list (node, position) and chunk boundaries, from a
    host-only plan, plus the group queries and their visible lengths."""
    plan = Plan.for_instance(inst, host_only=True)
    groups, chunks = plan.export("groups"), plan.export("chunks")
    gqs, gvis = plan.export("group_qs"), plan.export("group_vis")
    lcum_nodes = []
    out = []
    for gi, G in enumerate(groups):
        node, top = int(G[0]), int(G[1])
        seg = ta.root_path(inst.parent, node)
        seg = seg[seg.index(top):]
        toks = [(u, t) for u in seg for t in range(int(inst.node_len[u]))]
        ch = [(int(c[1]), int(c[2])) for c in chunks[int(G[5]):int(G[5]) + int(G[6])]]
        qs = gqs[int(G[4]):int(G[4]) + int(G[3])]
        vis = gvis[int(G[4]):int(G[4]) + int(G[3])]
        out.append((toks, ch, qs, vis))
    plan.close()
    return out


def _rise_and_spread(inst):
    """(largest mid-chunk raise of a running max, largest spread of one
    query's partial maxima), both in log2 units at scale 1/sqrt(d)."""
    q = inst.q.to(torch.float64).numpy()
    g = inst.n_qheads // inst.n_kvheads
    c = np.log2(np.e) / np.sqrt(inst.head_dim)
    kcache = {}

    def krow(u, t):
        if (u, t) not in kcache:
            kcache[(u, t)] = ta.node_kv(inst.k_pool, u, inst.node_len, inst.node_page_ptr, inst.node_page_ids,
                                        inst.page_size)[t]
        return kcache[(u, t)]

    rise, part_max = 0.0, {}
    for toks, ch, qs, vis in _segments(inst):
        K = np.stack([krow(u, t) for u, t in toks])         # [T, H, d]
        for qi, nv in zip(qs, vis):
            for h in range(inst.n_qheads):
                s = K[:nv, h // g] @ q[qi, h] * c
                for a, b in ch:
                    b = min(b, nv)
                    if a >= b:
                        continue
                    m = s[a:min(b, a + TILE)].max()
                    for t0 in range(a + TILE, b, TILE):
                        mx = s[t0:min(b, t0 + TILE)].max()
                        rise = max(rise, mx - m)
                        if mx > m + RESCALE_LOG2:
                            m = mx
                    part_max.setdefault((int(qi), h), []).append(s[a:b].max())
    spread = max(max(v) - min(v) for v in part_max.values())
    return rise, spread


@pytest.mark.parametrize("cls", ["wave", "workgroup"])
def test_peaky_inputs_reach_the_rescale_and_merge_cases(cls):
    for kind in ("ramp", "late_spike"):
        inst = peaky_tree(cls, kind, torch.bfloat16, 128)
        rise, spread = _rise_and_spread(inst)
        assert rise > RESCALE_LOG2, (kind, cls, rise)
    inst = peaky_tree(cls, "sink", torch.bfloat16, 128)
    rise, spread = _rise_and_spread(inst)
    assert spread > 1.5 * RESCALE_LOG2, (cls, spread)


def test_flat_inputs_do_not_reach_the_rescale():
    """Why the peaky cases exist: N(0,1) inputs never raise the max mid-chunk."""
    inst = peaky_tree("workgroup", "none", torch.bfloat16, 128)
    rise, _ = _rise_and_spread(inst)
    assert rise < RESCALE_LOG2, rise


def _record_forms(inst):
    """(rows whose partial o / l stays inside (-1, 1), rows with a value of
    magnitude 1 or more): the two workspace forms the kernels choose between
    (fp16 o / l, fp32 o), from fp64 chunk softmaxes of the instance's own rows."""
    q = inst.q.to(torch.float64).numpy()
    g = inst.n_qheads // inst.n_kvheads
    c = 1.0 / np.sqrt(inst.head_dim)
    half = full = 0
    for toks, ch, qs, vis in _segments(inst):
        nodes = sorted({u for u, _ in toks})
        kv = {u: (ta.node_kv(inst.k_pool, u, inst.node_len, inst.node_page_ptr, inst.node_page_ids, inst.page_size),
                  ta.node_kv(inst.v_pool, u, inst.node_len, inst.node_page_ptr, inst.node_page_ids, inst.page_size))
              for u in nodes}
        K = np.stack([kv[u][0][t] for u, t in toks])
        V = np.stack([kv[u][1][t] for u, t in toks])
        for qi, nv in zip(qs, vis):
            for h in range(inst.n_qheads):
                s = K[:nv, h // g] @ q[qi, h] * c
                for a, b in ch:
                    b = min(b, nv)
                    if a >= b:
                        continue
                    w = np.exp(s[a:b] - s[a:b].max())
                    o = (w @ V[a:b, h // g]) / w.sum()
                    if np.abs(o).max() < 1.0:
                        half += 1
                    else:
                        full += 1
    return half, full


def test_both_partial_record_forms_occur():
    """N(0,1) inputs give partials that are weighted averages well inside
    (-1, 1) (fp16 records); a dominant key carries its own value, whose
    largest component exceeds 1 (fp32 records)."""
    half, full = _record_forms(peaky_tree("workgroup", "none", torch.bfloat16, 128))
    assert half > 0 and full <= 0.01 * (half + full), (half, full)
    half, full = _record_forms(peaky_tree("workgroup", "sink", torch.bfloat16, 128))
    assert half > 0 and full > 0, (half, full)
