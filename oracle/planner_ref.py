"""Plain-Python re-derivation of the host planner -- TEST INFRASTRUCTURE ONLY.

Only tests use this. It shares no code with the C++ planner in the library;
the tests compare every table the library exports against the ones built here,
element for element.

Sources (FastTree review, section 3 "technical architecture"):
* 3.1 "context-query grouping" and "binary edge assignment": an edge assigned
  1 joins a child to its parent in the virtual tree, 0 keeps it apart; each
  virtual node becomes one context-query group.
* 3.2 Algorithm 1 (greedy binary edge assignment) and its cost model:
  padding costs C_{P,q}(nQ, len) = Pad(TS_q, nQ) * len * d,
  C_{P,c}(nQ, len) = nQ * Pad(TS_c, min(len, TS_c)) * d,
  Pad(TS, N) = TS - ((N - 1) % TS + 1), and the intermediate-result cost
  SplitKVCost_R = gamma * nQ_l * d.
* 3.3 long-context splitting: nodes above a threshold are cut so the launch
  fills the GPU and the last waves are not nearly empty.

Readings taken where the page is silent or garbled (each is a choice, listed
with the reasons in the design notes):
* "for l in leaves(v)" means the children of v (the edge assigned is v -> l).
* A[v] counts the query tokens below v; L is cumulative along merged edges.
* BFS and child order are ascending node id; ties C_0 == C_1 assign 1.
* SplitKVCost = C_P(nQ_curr, len_v) + C_P(nQ_l, len_l) + gamma * nQ_l;
  SplitQCost  = C_P(nQ_curr - nQ_l, len_v) + C_P(nQ_l, len_l + len_v);
  C_P = C_{P,q} + C_{P,c}; the common factor d is dropped; Pad(TS, 0) = 0.
* Constants (not printed on the page): TS_q = 16, TS_c = 64, and gamma =
  128 g per query, g = n_qheads / n_kvheads: nQ counts query tokens, a query's
  partials are g rows of d fp32 values written and read back (8 g d bytes per
  kv-head) against d / 4 bytes per query-token of K/V shared by a 16-query
  tile (32 g in these units), times four as measured on the target GPU.
* Split rule, row blocks, work-item classes and order, slot numbering and
  page runs are this library's own, written out step by step below. Groups
  with at most ``stream_rows`` rows become single-wave stream items (one row
  block); larger groups become workgroup items (row blocks of ``rb``) whose
  four waves share the chunk. When a plan has workgroup items, the groups
  that fill a whole 16-row tile join them (``tile_join``): one launch then
  holds a single item class wherever the rows allow it. The split rule counts capacity in busy waves:
  a single-wave stream as one, a workgroup block as 8/3 (its four waves
  share each staged tile); chunk lengths are multiples of ``split_align``.

Parity unpinned: the constants and the split rule (the page prints no plan,
no cost value and no threshold); they are pinned only against this file.
"""
from __future__ import annotations

from collections import deque

import numpy as np

FORMAT_VERSION = 4
TILE_ROWS = 16          # rows of one MFMA row tile
BLOCK_WAVE_WEIGHT3 = 8   # split rule: a workgroup block counts as 8/3 busy waves
CHUNK_ALIGN = 16
ITEM_FIXED_COST = 256

# table ids (same numbering as the library's export call)
T_PARAMS, T_EDGES, T_NQ, T_LCUM, T_GROUPS, T_GROUP_QS, T_GROUP_VIS, T_CHUNKS, T_ITEMS, \
    T_Q_SLOT_PTR, T_Q_SLOTS, T_RUNS, T_CHUNK_RUN_PTR, T_BFS = range(14)
TABLE_NAMES = ["params", "edges", "nq", "lcum", "groups", "group_qs", "group_vis", "chunks",
               "items", "q_slot_ptr", "q_slots", "runs", "chunk_run_ptr", "bfs"]

DEFAULTS = dict(ts_q=16, ts_c=64, gamma=0, rb=128, waves=5, floor_f=4, ncu=256, split=1,
                stream_rows=16, split_align=128, tile_join=1)


class PlanError(ValueError):
    pass


def pad(ts, n):
    """Pad(TS, N) = TS - ((N - 1) % TS + 1); zero for N = 0 (no group)."""
    if n <= 0:
        return 0
    return ts - ((n - 1) % ts + 1)


def cost_pad(nq, length, ts_q, ts_c):
    """C_{P,q} + C_{P,c} without the factor d."""
    return pad(ts_q, nq) * length + nq * pad(ts_c, min(length, ts_c))


def split_kv_cost(nq_curr, nq_l, len_l, len_v, ts_q, ts_c, gamma):
    """Edge 0: v keeps all nq_curr queries over len_v, the child runs its own
    group over len_l, and the child's queries write one more partial result."""
    return (cost_pad(nq_curr, len_v, ts_q, ts_c) + cost_pad(nq_l, len_l, ts_q, ts_c)
            + gamma * nq_l)


def split_q_cost(nq_curr, nq_l, len_l, len_v, ts_q, ts_c):
    """Edge 1: the child's queries leave v's group and the child's group reads
    the parent's context as well (len_l + len_v)."""
    return (cost_pad(nq_curr - nq_l, len_v, ts_q, ts_c)
            + cost_pad(nq_l, len_l + len_v, ts_q, ts_c))


def _cdiv(a, b):
    return -(-a // b)


def _align_up(a, b):
    return _cdiv(a, b) * b


def build_plan(parent, node_len, node_page_ptr, node_page_ids, page_size, qpl,
               n_qheads, n_kvheads, head_dim, force_edges=None, **opts):
    """Return {table name: int32 numpy array}."""
    o = dict(DEFAULTS)
    for k, v in opts.items():
        if k not in o:
            raise TypeError(k)
        if v:
            o[k] = int(v)
    if "split" in opts:
        o["split"] = int(opts["split"])
    if "tile_join" in opts:
        o["tile_join"] = int(opts["tile_join"])
    o["stream_rows"] = max(0, o["stream_rows"])     # negative: no single-wave items
    if o["gamma"] == 0:   # the default: 128 per q-head of a kv-head's group
        o["gamma"] = min(2**31 - 1, 128 * (n_qheads // max(1, n_kvheads)))
    ts_q, ts_c, gamma, rb = o["ts_q"], o["ts_c"], o["gamma"], o["rb"]
    parent = [int(x) for x in parent]
    lens = [int(x) for x in node_len]
    n = len(parent)

    # ---- P0: validation
    if n < 1 or len(lens) != n:
        raise PlanError("EINVAL: empty tree")
    if qpl < 1 or n_kvheads < 1 or n_qheads < 1 or n_qheads % n_kvheads:
        raise PlanError("EINVAL: heads/qpl")
    if head_dim not in (64, 128):
        raise PlanError("EUNSUPPORTED: head_dim")
    if not (1 <= page_size <= 256):
        raise PlanError("EINVAL: page_size")
    if o["stream_rows"] > TILE_ROWS:   # a single-wave item computes one 16-row tile
        raise PlanError("EINVAL: stream_rows")
    roots = [v for v in range(n) if parent[v] == -1]
    if len(roots) != 1:
        raise PlanError("EINVAL: need exactly one root")
    root = roots[0]
    for v in range(n):
        if parent[v] != -1 and not (0 <= parent[v] < n) or parent[v] == v:
            raise PlanError("EINVAL: parent out of range")
    for v in range(n):            # every node reaches the root within n steps
        u, steps = v, 0
        while u != root:
            u = parent[u]
            steps += 1
            if steps > n:
                raise PlanError("EINVAL: cycle")
    children = [[] for _ in range(n)]
    for v in range(n):
        if parent[v] >= 0:
            children[parent[v]].append(v)
    # P1: children ascending (built in ascending v order already)
    for v in range(n):
        if lens[v] < 1:
            raise PlanError("EINVAL: node length < 1")
        if not children[v] and lens[v] < qpl:
            raise PlanError("EINVAL: leaf shorter than queries_per_leaf")
    if sum(lens) >= (1 << 30):
        raise PlanError("EINVAL: too many tokens")
    ptr = [int(x) for x in node_page_ptr]
    pid = [int(x) for x in node_page_ids]
    if len(ptr) != n + 1 or ptr[0] != 0:
        raise PlanError("EINVAL: page ptr")
    for v in range(n):
        if ptr[v + 1] - ptr[v] != _cdiv(lens[v], page_size):
            raise PlanError("EINVAL: page count")
    for x in pid[:ptr[n]]:
        if not (0 <= x < (1 << 23)):
            raise PlanError("EINVAL: page id")
    if force_edges is not None and len(force_edges) != n:
        raise PlanError("EINVAL: force_edges")

    leaves = [v for v in range(n) if not children[v]]
    leaf_rank = {v: i for i, v in enumerate(leaves)}
    n_q = len(leaves) * qpl
    g = n_qheads // n_kvheads
    H = n_kvheads

    # ---- P2: A[v] = query tokens below v
    A = [0] * n
    # ---- P3: BFS from the root, children pushed in ascending id
    bfs, dq = [], deque([root])
    while dq:
        v = dq.popleft()
        bfs.append(v)
        dq.extend(children[v])
    for v in reversed(bfs):
        A[v] = qpl if not children[v] else sum(A[c] for c in children[v])

    # ---- P4: greedy binary edge assignment (Algorithm 1)
    L = list(lens)
    f = [0] * n
    nQ = [0] * n
    for v in bfs:
        nq_curr = A[v]
        len_v = L[v]
        for l in children[v]:
            nq_l, len_l = A[l], L[l]
            if force_edges is not None:
                assign = 1 if force_edges[l] else 0
            else:
                c0 = split_kv_cost(nq_curr, nq_l, len_l, len_v, ts_q, ts_c, gamma)
                c1 = split_q_cost(nq_curr, nq_l, len_l, len_v, ts_q, ts_c)
                assign = 1 if c0 >= c1 else 0
            f[l] = assign
            if assign:
                nq_curr -= nq_l
                L[l] = len_l + len_v
        nQ[v] = nq_curr

    # ---- P5: virtual-tree groups in BFS order
    top = [0] * n
    for v in bfs:
        top[v] = v if (v == root or f[v] == 0) else top[parent[v]]

    def queries_of(v):
        qs = []
        if not children[v]:
            r = leaf_rank[v]
            qs.extend(range(r * qpl, r * qpl + qpl))
        for c in children[v]:
            if f[c] == 0:
                stack = [c]
                while stack:
                    u = stack.pop()
                    if not children[u]:
                        r = leaf_rank[u]
                        qs.extend(range(r * qpl, r * qpl + qpl))
                    stack.extend(children[u])
        return sorted(qs)

    groups = []   # dicts
    group_of_node = {}
    for v in bfs:
        if nQ[v] == 0:
            continue
        qs = queries_of(v)
        assert len(qs) == nQ[v]
        kv_len = L[v]
        seg = []
        u = v
        while True:
            seg.append(u)
            if u == top[v]:
                break
            u = parent[u]
        seg.reverse()
        assert sum(lens[u] for u in seg) == kv_len
        if not children[v]:
            vis = [kv_len - (qpl - 1 - (q % qpl)) for q in qs]
        else:
            vis = [kv_len] * len(qs)
        group_of_node[v] = len(groups)
        groups.append(dict(node=v, top=top[v], kv_len=kv_len, qs=qs, vis=vis, seg=seg,
                           rows=len(qs) * g))

    # ---- P6 / P7: item class, row blocks and KV chunks
    has_wg = any(G["rows"] > o["stream_rows"] for G in groups)
    for G in groups:
        # 0 = stream (one wave), 1 = workgroup
        single = G["rows"] <= o["stream_rows"] and not (o["tile_join"] and has_wg and G["rows"] >= TILE_ROWS)
        G["cls"] = 0 if single else 1
        if G["cls"] == 0:
            G["blocks"] = [(0, G["rows"])]
        else:
            # as few blocks of at most rb rows as possible, even in whole
            # tiles: the tiles of the group are dealt out so that the first
            # (tiles mod blocks) blocks hold one more; the last block ends
            # at the group's last row
            tile = TILE_ROWS if rb % TILE_ROWS == 0 else 1
            nb = _cdiv(G["rows"], rb)
            n_tiles = _cdiv(G["rows"], tile)
            G["blocks"] = []
            t0 = 0
            for b in range(nb):
                nt = n_tiles // nb + (1 if b < n_tiles % nb else 0)
                r0 = t0 * tile
                G["blocks"].append((r0, min(G["rows"], r0 + nt * tile) - r0))
                t0 += nt
        G["nblocks"] = len(G["blocks"])
        G["rb"] = max(nr for _, nr in G["blocks"])
    def chunking(G, c_glob):
        """(chunk length, chunk count) of group G under global chunk c_glob:
        at least the group's floor, then balanced pieces, 16-aligned."""
        kvl = G["kv_len"]
        cg = max(c_glob, _align_up(o["floor_f"] * min(G["rows"], G["rb"]), o["split_align"]))
        nch = _cdiv(kvl, cg)
        csz = _align_up(_cdiv(kvl, nch), CHUNK_ALIGN)
        return csz, _cdiv(kvl, csz)

    if o["split"]:
        W = H * sum((3 if G["cls"] == 0 else BLOCK_WAVE_WEIGHT3) * G["nblocks"] * G["kv_len"]
                    for G in groups)
        U = _cdiv(W, o["ncu"] * o["waves"] * 3)
        c_glob = max(o["split_align"], _align_up(U, o["split_align"]))
        # the launch fills the GPU (review 3.3): while it would hold fewer
        # units (item x kv-head) than compute units, the global chunk steps
        # down by one alignment
        while c_glob > o["split_align"] and \
                H * sum(G["nblocks"] * chunking(G, c_glob)[1] for G in groups) < o["ncu"]:
            c_glob -= o["split_align"]
    else:
        c_glob = 0
    chunks = []
    for gi, G in enumerate(groups):
        kvl = G["kv_len"]
        if o["split"]:
            csz, nch = chunking(G, c_glob)
        else:
            csz, nch = kvl, 1
        G["chunk_ptr"] = len(chunks)
        G["n_chunks"] = nch
        for i in range(nch):
            chunks.append((gi, i * csz, min(kvl, (i + 1) * csz)))

    # ---- P8: work items: workgroup items first, then stream items; each
    # class longest first (stable on (group, block, chunk))
    items = []
    for gi, G in enumerate(groups):
        for r0, nr in G["blocks"]:
            for c in range(G["n_chunks"]):
                ci = G["chunk_ptr"] + c
                est = (chunks[ci][2] - chunks[ci][1]) * (ITEM_FIXED_COST + nr)
                items.append((est, gi, r0, nr, ci, G["cls"]))
    items.sort(key=lambda t: (-t[5], -t[0]))   # Python's sort is stable
    n_stream = sum(1 for t in items if t[5] == 0)

    # ---- P9: slots
    slot_base = 0
    for G in groups:
        G["slot_base"] = slot_base
        slot_base += G["n_chunks"] * len(G["qs"])
    n_slots = slot_base
    q_lists = [[] for _ in range(n_q)]
    for lf in leaves:
        path = []
        u = lf
        while u != -1:
            path.append(u)
            u = parent[u]
        path.reverse()
        for k, u in enumerate(path):
            stop = (u == lf) or f[path[k + 1]] == 0
            if stop:
                G = groups[group_of_node[u]]
                r = leaf_rank[lf]
                for j in range(qpl):
                    q = r * qpl + j
                    jj = G["qs"].index(q)
                    for c in range(G["n_chunks"]):
                        q_lists[q].append(G["slot_base"] + c * len(G["qs"]) + jj)
    q_slot_ptr = [0]
    q_slots = []
    for q in range(n_q):
        q_slots.extend(q_lists[q])
        q_slot_ptr.append(len(q_slots))

    # ---- P10: page runs per chunk
    runs, chunk_run_ptr = [], [0]
    for (gi, t0, t1) in chunks:
        G = groups[gi]
        pos = 0
        last = None
        for u in G["seg"]:
            for t in range(lens[u]):
                if t0 <= pos < t1:
                    page = pid[ptr[u] + t // page_size]
                    slot = t % page_size
                    if last is not None and last[0] == page and last[1] + last[2] == slot and last[3] == u:
                        last[2] += 1
                    else:
                        if last is not None:
                            runs.append(last[:3])
                        last = [page, slot, 1, u]
                pos += 1
        runs.append(last[:3])
        chunk_run_ptr.append(len(runs))

    params = [FORMAT_VERSION, n, n_q, qpl, n_qheads, n_kvheads, head_dim, page_size,
              ts_q, ts_c, gamma, rb, o["waves"], o["floor_f"], o["ncu"], o["split"],
              1 if force_edges is not None else 0, CHUNK_ALIGN, len(groups), len(chunks),
              len(items), n_slots, c_glob, len(runs), o["stream_rows"], n_stream, o["split_align"],
              1 if o["tile_join"] else 0]
    gq, gv, gt = [], [], []
    for G in groups:
        gt.append([G["node"], G["top"], G["kv_len"], len(G["qs"]), len(gq), G["chunk_ptr"],
                   G["n_chunks"], G["slot_base"]])
        gq.extend(G["qs"])
        gv.extend(G["vis"])
    i32 = lambda a, shape=None: np.asarray(a, dtype=np.int32).reshape(shape if shape else -1)
    return {
        "params": i32(params),
        "edges": i32(f),
        "nq": i32(nQ),
        "lcum": i32(L),
        "groups": i32(gt, (-1, 8)) if gt else np.zeros((0, 8), np.int32),
        "group_qs": i32(gq),
        "group_vis": i32(gv),
        "chunks": i32([list(c) for c in chunks], (-1, 3)),
        "items": i32([[t[1], t[2], t[3], t[4], t[5]] for t in items], (-1, 5)),
        "q_slot_ptr": i32(q_slot_ptr),
        "q_slots": i32(q_slots),
        "runs": i32(runs, (-1, 3)),
        "chunk_run_ptr": i32(chunk_run_ptr),
        "bfs": i32(bfs),
    }


def plan_instance(inst, **kw):
    return build_plan(inst.parent, inst.node_len, inst.node_page_ptr, inst.node_page_ids,
                      inst.page_size, inst.qpl, inst.n_qheads, inst.n_kvheads, inst.head_dim, **kw)
