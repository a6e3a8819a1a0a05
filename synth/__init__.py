"""Seeded synthetic inputs for tree-structured decode attention.

This module only draws trees, page tables and Q/K/V tensors. It holds none of
the attention arithmetic and none of the planner: both the fp64 oracle and the
HIP path consume the same instance, each on its own.

Workload shapes follow the tree grid of the FastTree review (section 5, "kernel
benchmark": N nodes per level, C tokens per node, GQA 1/4/16, Llama-2-7B and
Mistral-7B head layouts). The datasets of that page's end-to-end benchmarks
are not available, so these seeded trees stand in for their shapes.

Conventions shared by both sides:
  * ``parent[v]`` is -1 for the root, otherwise the parent's node id.
  * Node ``v`` owns pages ``node_page_ids[node_page_ptr[v]:node_page_ptr[v+1]]``;
    token ``t`` of ``v`` sits in page ``t // page_size`` of that list at slot
    ``t % page_size``.
  * The K and V pools are ``[n_pages, page_size, n_kvheads, head_dim]``.
  * Queries are ordered by leaf rank (leaves sorted by node id), then by ``j``
    in ``[0, qpl)``; query ``j`` of leaf ``l`` is that leaf's token
    ``len(l) - qpl + j``. Q is ``[n_queries, n_qheads, head_dim]``.
  * Unused token slots and spare pages carry canaries (K = 0, V = 1e30) so an
    unmasked stray read is visible in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TREE_SEED_BASE = 2026_1000
TENSOR_SEED_BASE = 2026_2000
CANARY_V = 1.0e30

CONFIG_NAMES = {
    1: "tiny_2level_fp32",
    2: "multilevel_prompt_N1-4-16_C2048-512-128_gqa1",
    3: "wide_fanout_root4096_256x64_gqa4",
    4: "skewed_longctx_N1-10_C32000-400_gqa16",
    5: "random_radix_4level_qpl4_gqa4",
}


@dataclasses.dataclass
class TreeInstance:
    name: str
    parent: np.ndarray          # int32 [n]
    node_len: np.ndarray        # int32 [n]
    node_page_ptr: np.ndarray   # int32 [n+1]
    node_page_ids: np.ndarray   # int32 [sum pages]
    n_pages: int
    page_size: int
    qpl: int
    n_qheads: int
    n_kvheads: int
    head_dim: int
    dtype: torch.dtype          # torch.float32 or torch.bfloat16
    q: Optional[torch.Tensor] = None       # [n_q, Hq, d] CPU
    k_pool: Optional[torch.Tensor] = None  # [n_pages, ps, H, d] CPU
    v_pool: Optional[torch.Tensor] = None

    @property
    def n_nodes(self) -> int:
        return int(self.parent.shape[0])

    @property
    def n_leaves(self) -> int:
        has_child = np.zeros(self.n_nodes, dtype=bool)
        for v in range(self.n_nodes):
            if self.parent[v] >= 0:
                has_child[self.parent[v]] = True
        return int((~has_child).sum())

    @property
    def n_queries(self) -> int:
        return self.n_leaves * self.qpl

    @property
    def unique_kv_bytes(self) -> int:
        esize = 4 if self.dtype == torch.float32 else 2
        return int(self.node_len.astype(np.int64).sum()) * self.n_kvheads * self.head_dim * 2 * esize


def _assign_pages(node_len, page_size, rng, contiguous):
    n_pages_node = (node_len.astype(np.int64) + page_size - 1) // page_size
    ptr = np.zeros(len(node_len) + 1, dtype=np.int64)
    ptr[1:] = np.cumsum(n_pages_node)
    used = int(ptr[-1])
    if contiguous:
        pool = used
        ids = np.arange(used, dtype=np.int64)
    else:
        pool = used + int(math.ceil(0.05 * used))
        ids = rng.permutation(pool)[:used]
    return ptr.astype(np.int32), ids.astype(np.int32), pool


def _levels_tree(nodes_per_level, ctx_per_level):
    """Complete tree: level i has nodes_per_level[i] nodes, each level-(i-1)
    node has nodes_per_level[i] / nodes_per_level[i-1] children. Nodes are
    numbered level by level."""
    parent, length = [-1], [ctx_per_level[0]]
    prev = [0]
    for lvl in range(1, len(nodes_per_level)):
        fan = nodes_per_level[lvl] // nodes_per_level[lvl - 1]
        cur = []
        for p in prev:
            for _ in range(fan):
                cur.append(len(parent))
                parent.append(p)
                length.append(ctx_per_level[lvl])
        prev = cur
    return np.asarray(parent, np.int32), np.asarray(length, np.int32)


def _random_radix_tree(rng, levels=4, max_branch=8, median=256, sigma=0.8, lo=16, hi=4096):
    parent = [-1]
    frontier = [0]
    for _ in range(levels):
        nxt = []
        for p in frontier:
            b = int(rng.integers(1, max_branch + 1))
            for _ in range(b):
                nxt.append(len(parent))
                parent.append(p)
        frontier = nxt
    n = len(parent)
    z = rng.standard_normal(n)
    lens = np.floor(median * np.exp(sigma * z) + 0.5).astype(np.int64)
    lens = np.clip(lens, lo, hi)
    return np.asarray(parent, np.int32), lens.astype(np.int32)


def fill_tensors(inst: TreeInstance, seed: int) -> TreeInstance:
    """Draw Q, K, V as fp32 N(0,1) (in that order) from a CPU torch generator,
    plant canaries in unused slots, then cast to the instance dtype (bf16 casts
    round to nearest even)."""
    g = torch.Generator().manual_seed(seed)
    nq = inst.n_queries
    ps, H, d = inst.page_size, inst.n_kvheads, inst.head_dim
    q = torch.randn((nq, inst.n_qheads, d), generator=g, dtype=torch.float32)
    k = torch.randn((inst.n_pages, ps, H, d), generator=g, dtype=torch.float32)
    v = torch.randn((inst.n_pages, ps, H, d), generator=g, dtype=torch.float32)
    used = np.zeros((inst.n_pages, ps), dtype=bool)
    for u in range(inst.n_nodes):
        pages = inst.node_page_ids[inst.node_page_ptr[u]:inst.node_page_ptr[u + 1]]
        L = int(inst.node_len[u])
        for i, pg in enumerate(pages):
            n_in = min(ps, L - i * ps)
            used[pg, :n_in] = True
    unused = torch.from_numpy(~used)
    k[unused] = 0.0
    v[unused] = CANARY_V
    inst.q = q.to(inst.dtype).contiguous()
    inst.k_pool = k.to(inst.dtype).contiguous()
    inst.v_pool = v.to(inst.dtype).contiguous()
    return inst


def grow_leaves(inst: TreeInstance, leaf_add, seed: int):
    """One decode-loop step of the tree: leaf of rank r gains leaf_add[r]
    tokens at its end. The pages the growth needs are new pool pages (ids
    n_pages.. shuffled by ``seed``), handed out in leaf-rank order; existing
    K/V is kept, the new tokens' K and V are drawn as fp32 N(0,1) (K block
    then V block, leaf-rank order) and a fresh Q for every query follows; the
    new pages' unused slots carry the canaries. Returns (grown instance, new
    page ids in the order the leaves take them)."""
    leaf_add = np.asarray(leaf_add, np.int64)
    has_child = np.zeros(inst.n_nodes, dtype=bool)
    for v in range(inst.n_nodes):
        if inst.parent[v] >= 0:
            has_child[inst.parent[v]] = True
    leaves = np.flatnonzero(~has_child)
    assert len(leaf_add) == len(leaves) and (leaf_add >= 0).all()
    ps = inst.page_size
    rng = np.random.default_rng(seed)
    old_len = inst.node_len.astype(np.int64)
    new_len = old_len.copy()
    new_len[leaves] += leaf_add
    need = [int(-(-new_len[v] // ps) - (-(-old_len[v] // ps))) for v in leaves]
    n_new = int(sum(need))
    fresh = (inst.n_pages + rng.permutation(n_new)).astype(np.int32)
    pages = [list(inst.node_page_ids[inst.node_page_ptr[v]:inst.node_page_ptr[v + 1]]) for v in range(inst.n_nodes)]
    at = 0
    for v, k in zip(leaves, need):
        pages[v] += list(fresh[at:at + k])
        at += k
    ptr = np.zeros(inst.n_nodes + 1, np.int32)
    ptr[1:] = np.cumsum([len(x) for x in pages])
    ids = np.asarray([pg for x in pages for pg in x], np.int32)
    out = dataclasses.replace(inst, node_len=new_len.astype(np.int32), node_page_ptr=ptr, node_page_ids=ids,
                              n_pages=inst.n_pages + n_new, q=None, k_pool=None, v_pool=None)
    if inst.k_pool is not None:
        H, d = inst.n_kvheads, inst.head_dim
        g = torch.Generator().manual_seed(seed)
        n_tok = int(leaf_add.sum())
        k_new = torch.randn((n_tok, H, d), generator=g, dtype=torch.float32).to(inst.dtype)
        v_new = torch.randn((n_tok, H, d), generator=g, dtype=torch.float32).to(inst.dtype)
        q = torch.randn((out.n_queries, inst.n_qheads, d), generator=g, dtype=torch.float32)
        k = torch.zeros((n_new, ps, H, d), dtype=inst.dtype)
        v = torch.full((n_new, ps, H, d), CANARY_V, dtype=torch.float32).to(inst.dtype)
        k_pool = torch.cat([inst.k_pool, k]).contiguous()
        v_pool = torch.cat([inst.v_pool, v]).contiguous()
        x = 0
        for v_id in leaves:
            for t in range(int(old_len[v_id]), int(new_len[v_id])):
                pg = pages[v_id][t // ps]
                k_pool[pg, t % ps] = k_new[x]
                v_pool[pg, t % ps] = v_new[x]
                x += 1
        out.q = q.to(inst.dtype).contiguous()
        out.k_pool, out.v_pool = k_pool, v_pool
    return out, fresh


def make_tree(parent, node_len, *, page_size=16, qpl=1, n_qheads=4, n_kvheads=4, head_dim=64,
              dtype=torch.bfloat16, seed=0, contiguous=False, name="custom") -> TreeInstance:
    parent = np.asarray(parent, np.int32)
    node_len = np.asarray(node_len, np.int32)
    rng = np.random.default_rng(seed)
    ptr, ids, pool = _assign_pages(node_len, page_size, rng, contiguous)
    return TreeInstance(name, parent, node_len, ptr, ids, pool, page_size, qpl,
                        n_qheads, n_kvheads, head_dim, dtype)


def make_config(k: int, tensors: bool = True) -> TreeInstance:
    """The five seeded workloads (k = 1..5)."""
    rng = np.random.default_rng(TREE_SEED_BASE + k)
    if k == 1:
        parent, lens = _levels_tree([1, 4], [256, 32])
        kw = dict(qpl=1, n_qheads=4, n_kvheads=4, head_dim=64, dtype=torch.float32, contiguous=True)
    elif k == 2:
        parent, lens = _levels_tree([1, 4, 16], [2048, 512, 128])
        kw = dict(qpl=1, n_qheads=32, n_kvheads=32, head_dim=128, dtype=torch.bfloat16, contiguous=False)
    elif k == 3:
        parent, lens = _levels_tree([1, 256], [4096, 64])
        kw = dict(qpl=1, n_qheads=32, n_kvheads=8, head_dim=128, dtype=torch.bfloat16, contiguous=False)
    elif k == 4:
        parent, lens = _levels_tree([1, 10], [32000, 400])
        kw = dict(qpl=1, n_qheads=64, n_kvheads=4, head_dim=128, dtype=torch.bfloat16, contiguous=False)
    elif k == 5:
        parent, lens = _random_radix_tree(rng)
        kw = dict(qpl=4, n_qheads=32, n_kvheads=8, head_dim=128, dtype=torch.bfloat16, contiguous=False)
    else:
        raise ValueError(f"unknown config {k}")
    contiguous = kw.pop("contiguous")
    ptr, ids, pool = _assign_pages(lens, 16, rng, contiguous)
    inst = TreeInstance(CONFIG_NAMES[k], parent, lens, ptr, ids, pool, 16, **kw)
    if tensors:
        fill_tensors(inst, TENSOR_SEED_BASE + k)
    return inst


def random_small_tree(seed: int, *, max_nodes=24, max_len=80, page_size=None, qpl=None,
                      heads=None, head_dim=None, dtype=None, tensors=True) -> TreeInstance:
    """A random small tree with shuffled node ids (any numbering is legal),
    for parity sweeps. Every knob not given is drawn from the seed."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, max_nodes + 1))
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    perm = rng.permutation(n)            # new id of old node i is perm[i]
    parent = np.full(n, -1, np.int32)
    for old in range(n):
        if par[old] >= 0:
            parent[perm[old]] = perm[par[old]]
    if qpl is None:
        qpl = int(rng.choice([1, 1, 2, 3, 4]))
    has_child = np.zeros(n, bool)
    for v in range(n):
        if parent[v] >= 0:
            has_child[parent[v]] = True
    lens = rng.integers(1, max_len + 1, size=n)
    lens = np.where(has_child, lens, np.maximum(lens, qpl)).astype(np.int32)
    if page_size is None:
        page_size = int(rng.choice([16, 16, 8, 1, 32]))
    if heads is None:
        heads = [(4, 4), (8, 2), (16, 1), (32, 8), (64, 4)][int(rng.integers(0, 5))]
    if head_dim is None:
        head_dim = int(rng.choice([64, 128]))
    if dtype is None:
        dtype = torch.bfloat16 if rng.integers(0, 3) else torch.float32
    ptr, ids, pool = _assign_pages(lens, page_size, rng, False)
    inst = TreeInstance(f"rand{seed}", parent, lens, ptr, ids, pool, page_size, qpl,
                        heads[0], heads[1], head_dim, dtype)
    if tensors:
        fill_tensors(inst, seed + 77)
    return inst


# ---------------------------------------------------------------------------
# Peaky logits. Real attention is rarely the flat softmax that N(0,1) inputs
# give (score std ~1): heads put most of their mass on a few tokens (a sink on
# the first token, a couple of dominant keys) and scores can rise along a
# path. These helpers reshape an instance whose tensors are already drawn, so
# that a test can make the softmax peaky on purpose. They only move Q/K/V
# values; no attention arithmetic happens here.

PEAK_KINDS = ("scaled_q", "ramp", "late_spike", "sink", "two_peaks", "two_peaks_antipodal")


def _token_slots(inst, u):
    """(page, slot) of every token of node u, in order."""
    ps = inst.page_size
    pages = inst.node_page_ids[inst.node_page_ptr[u]:inst.node_page_ptr[u + 1]]
    return [(int(pages[t // ps]), t % ps) for t in range(int(inst.node_len[u]))]


def plant_peaks(inst: TreeInstance, kind: str, seed: int, strength: float = 10.0) -> TreeInstance:
    """Plant logit structure into inst's Q/K/V (in place; returns inst).

    Every q-head of kv-head h gets a component sqrt(d) * u_h along a unit
    vector u_h drawn per kv-head, so a key with a component b * u_h scores
    about b higher (in natural-log units, after the 1/sqrt(d) scale) than
    an unplanted one for every query of that kv-head. ``strength`` is that b
    for the planted keys. Kinds:

    * ``scaled_q``: Q multiplied by strength / 2.5 (score std ~4 at the
      default strength), so many keys dominate and the running max rises
      from tile to tile.
    * ``ramp``: key t of the root gets (strength * 3 t / len) u_h (the
      score rises ~3 strength along the root) and key t of every other node
      strength * (0.5 + t / len) u_h: the running max is raised again and
      again mid-chunk.
    * ``late_spike``: three keys in the second half of the root and one in
      the second half of each leaf get strength * u_h.
    * ``sink``: the root's first key gets strength * u_h (an attention sink:
      most of every query's mass on one token).
    * ``two_peaks``: two root keys (positions len/3 and 5 len/6) get
      strength * u_h and (strength - 0.3) * u_h: two near-equal dominant
      keys with their own N(0,1) values.
    * ``two_peaks_antipodal``: as two_peaks, with the second key's value set
      to minus the first's (the largest value difference two N(0,1) rows
      give, the worst case for rounding the two weights apart).
    """
    if kind not in PEAK_KINDS:
        raise ValueError(f"unknown peak kind {kind}")
    rng = np.random.default_rng(seed)
    H, d = inst.n_kvheads, inst.head_dim
    g = inst.n_qheads // H
    u = rng.standard_normal((H, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u = torch.from_numpy(u).to(torch.float32)
    q = inst.q.to(torch.float32)
    k = inst.k_pool.to(torch.float32)
    v = inst.v_pool.to(torch.float32)
    if kind == "scaled_q":
        q = q * (strength / 2.5)
    else:
        q = q + math.sqrt(d) * u.repeat_interleave(g, dim=0)[None]
        root = int(np.flatnonzero(inst.parent < 0)[0])
        has_child = np.zeros(inst.n_nodes, bool)
        has_child[inst.parent[inst.parent >= 0]] = True

        def plant(node, t, b):
            pg, sl = _token_slots(inst, node)[t]
            k[pg, sl] += b * u

        L = int(inst.node_len[root])
        if kind == "ramp":
            for node in range(inst.n_nodes):
                n = int(inst.node_len[node])
                for t in range(n):
                    plant(node, t, strength * 3.0 * t / n if node == root else strength * (0.5 + t / n))
        elif kind == "late_spike":
            for t in (L // 2 + L // 7, (3 * L) // 4, L - 2):
                plant(root, max(0, t), strength)
            for node in np.flatnonzero(~has_child):
                n = int(inst.node_len[node])
                if node != root:
                    plant(int(node), n // 2 + int(rng.integers(0, max(1, n - n // 2 - 1))), strength)
        elif kind == "sink":
            plant(root, 0, strength)
        else:
            a, b = L // 3, (5 * L) // 6
            plant(root, a, strength)
            plant(root, b, strength - 0.3)
            if kind == "two_peaks_antipodal":
                pa, sa = _token_slots(inst, root)[a]
                pb, sb = _token_slots(inst, root)[b]
                v[pb, sb] = -v[pa, sa]
    inst.q = q.to(inst.dtype).contiguous()
    inst.k_pool = k.to(inst.dtype).contiguous()
    inst.v_pool = v.to(inst.dtype).contiguous()
    return inst
