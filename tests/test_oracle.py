"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test would fail for a plausible mistake in the oracle: a dropped ancestor
node, a wrong leaf mask offset, a wrong GQA head mapping, a missing scale, a
transposed operand or a softmax that does not normalise.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import tree_attention as ta

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dense_tree_mask_attention(inst):
    """Independent formulation: every token of the tree in one flat list, a
    dense visibility mask per query (ancestor-node tokens plus the query's own
    leaf tokens up to its position), one masked softmax per query and head."""
    ps = inst.page_size
    toks_k, toks_v, tok_node, tok_pos = [], [], [], []
    kp = inst.k_pool.to(torch.float64).numpy()
    vp = inst.v_pool.to(torch.float64).numpy()
    for u in range(inst.n_nodes):
        base = inst.node_page_ptr[u]
        for t in range(inst.node_len[u]):
            page = inst.node_page_ids[base + t // ps]
            toks_k.append(kp[page, t % ps])
            toks_v.append(vp[page, t % ps])
            tok_node.append(u)
            tok_pos.append(t)
    K = np.stack(toks_k)          # [N, H, d]
    V = np.stack(toks_v)
    tok_node = np.array(tok_node)
    tok_pos = np.array(tok_pos)
    is_parent = set(int(p) for p in inst.parent if p >= 0)
    leaves = [v for v in range(inst.n_nodes) if v not in is_parent]
    q = inst.q.to(torch.float64).numpy()
    nq, hq, d = q.shape
    g = hq // inst.n_kvheads
    out = np.zeros_like(q)
    for r, leaf in enumerate(leaves):
        anc = set()
        u = int(inst.parent[leaf])
        while u >= 0:
            anc.add(u)
            u = int(inst.parent[u])
        for j in range(inst.qpl):
            qi = r * inst.qpl + j
            limit = inst.node_len[leaf] - inst.qpl + j
            mask = np.array([(n in anc) or (n == leaf and p <= limit) for n, p in zip(tok_node, tok_pos)])
            for h in range(hq):
                s = (K[:, h // g, :] @ q[qi, h]) / np.sqrt(d)
                s = np.where(mask, s, -np.inf)
                w = np.exp(s - s.max())
                w /= w.sum()
                out[qi, h] = w @ V[:, h // g, :]
    return out


def _all_parent_vectors(n):
    """Every rooted tree on n labelled nodes with parent[i] < i (root 0)."""
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(choice)


def test_brute_force_tiny_trees():
    rng = np.random.default_rng(7)
    count = 0
    for n in range(1, 7):
        for par in _all_parent_vectors(n):
            qpl = int(rng.integers(1, 4))
            has_child = np.zeros(n, bool)
            for v in range(1, n):
                has_child[par[v]] = True
            lens = rng.integers(1, 6, size=n)
            lens = np.where(has_child, lens, np.maximum(lens, qpl))
            hq, h = [(2, 2), (4, 2), (4, 1)][count % 3]
            inst = synth.make_tree(par, lens, page_size=int(rng.choice([1, 2, 4])), qpl=qpl,
                                   n_qheads=hq, n_kvheads=h, head_dim=8, dtype=torch.float64,
                                   seed=count)
            synth.fill_tensors(inst, seed=1000 + count)
            ref = _dense_tree_mask_attention(inst)
            got = ta.decode_instance(inst)
            assert np.max(np.abs(ref - got)) < 1e-12, (par, lens.tolist(), qpl)
            count += 1
    assert count == 1 + 1 + 2 + 6 + 24 + 120


def test_brute_force_shuffled_ids_and_pages():
    for seed in range(20):
        inst = synth.random_small_tree(seed, max_nodes=9, max_len=12, head_dim=64,
                                       dtype=torch.float32)
        ref = _dense_tree_mask_attention(inst)
        got = ta.decode_instance(inst)
        assert np.max(np.abs(ref - got)) < 1e-12


@pytest.mark.parametrize("qpl,heads", [(1, (4, 4)), (3, (8, 2)), (4, (16, 1))])
def test_chain_tree_equals_sdpa(qpl, heads):
    lens = [37, 5, 22, 9]
    par = [-1, 0, 1, 2]
    hq, h = heads
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=hq, n_kvheads=h,
                           head_dim=64, dtype=torch.float64, seed=3)
    synth.fill_tensors(inst, seed=11)
    got = ta.decode_instance(inst)
    # concatenated path KV straight from the page table
    ks, vs = [], []
    for u in range(4):
        pages = inst.node_page_ids[inst.node_page_ptr[u]:inst.node_page_ptr[u + 1]]
        ks.append(inst.k_pool[torch.from_numpy(pages.astype(np.int64))].reshape(-1, h, 64)[:lens[u]])
        vs.append(inst.v_pool[torch.from_numpy(pages.astype(np.int64))].reshape(-1, h, 64)[:lens[u]])
    K = torch.cat(ks).transpose(0, 1).repeat_interleave(hq // h, dim=0)   # [Hq, T, d]
    V = torch.cat(vs).transpose(0, 1).repeat_interleave(hq // h, dim=0)
    T = K.shape[1]
    Q = inst.q.transpose(0, 1)                                             # [Hq, qpl, d]
    mask = torch.tensor([[t <= T - qpl + j for t in range(T)] for j in range(qpl)])
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
    ref = ref.transpose(0, 1).numpy()
    assert np.max(np.abs(ref - got)) < 1e-12


def test_closed_form_constant_v():
    inst = synth.random_small_tree(5, max_nodes=12, dtype=torch.float32, head_dim=64)
    c = 0.375
    inst.v_pool = torch.full_like(inst.v_pool, c)
    got = ta.decode_instance(inst)
    assert np.max(np.abs(got - c)) < 1e-12


def test_closed_form_zero_k_is_mean_of_visible_v():
    # root (3 tokens) with two leaves of 2 tokens, qpl = 1, hand-listed visibility
    inst = synth.make_tree([-1, 0, 0], [3, 2, 2], page_size=2, qpl=1, n_qheads=2, n_kvheads=1,
                           head_dim=64, dtype=torch.float64, seed=1)
    synth.fill_tensors(inst, seed=2)
    inst.k_pool = torch.zeros_like(inst.k_pool)
    got = ta.decode_instance(inst)
    vp = inst.v_pool.numpy()
    ids = inst.node_page_ids
    def tok(u, t):
        return vp[ids[inst.node_page_ptr[u] + t // 2], t % 2, 0]
    root = [tok(0, 0), tok(0, 1), tok(0, 2)]
    leaf1 = root + [tok(1, 0), tok(1, 1)]
    leaf2 = root + [tok(2, 0), tok(2, 1)]
    for qi, vis in enumerate([leaf1, leaf2]):
        mean = np.mean(vis, axis=0)
        for h in range(2):
            assert np.max(np.abs(got[qi, h] - mean)) < 1e-12


def test_closed_form_single_token_path():
    inst = synth.make_tree([-1], [1], page_size=16, qpl=1, n_qheads=4, n_kvheads=2, head_dim=64,
                           dtype=torch.float64, seed=1)
    synth.fill_tensors(inst, seed=9)
    got = ta.decode_instance(inst)
    page = inst.node_page_ids[0]
    for h in range(4):
        np.testing.assert_allclose(got[0, h], inst.v_pool[page, 0, h // 2].numpy(), atol=1e-15)


def test_first_query_of_leaf_sees_only_its_prefix():
    # qpl = 3 on a single node of 3 tokens: query 0 sees one token -> its V exactly
    inst = synth.make_tree([-1], [3], page_size=16, qpl=3, n_qheads=2, n_kvheads=2, head_dim=64,
                           dtype=torch.float64, seed=1)
    synth.fill_tensors(inst, seed=4)
    got = ta.decode_instance(inst)
    page = inst.node_page_ids[0]
    for h in range(2):
        np.testing.assert_allclose(got[0, h], inst.v_pool[page, 0, h].numpy(), atol=1e-15)


def test_softmax_rows_sum_to_one():
    inst = synth.random_small_tree(11, max_nodes=15, dtype=torch.float32, head_dim=64)
    _, w = ta.decode_instance(inst, return_weights=True)
    for p in w.values():
        assert abs(p.sum() - 1.0) < 1e-12
        assert (p >= 0).all()


def test_scale_is_inverse_sqrt_head_dim():
    # two tokens with scores 0 and sqrt(d)*x: weight ratio must be exp(x)
    d = 64
    inst = synth.make_tree([-1], [2], page_size=16, qpl=1, n_qheads=1, n_kvheads=1, head_dim=d,
                           dtype=torch.float64, seed=1)
    synth.fill_tensors(inst, seed=5)
    page = inst.node_page_ids[0]
    inst.q = torch.zeros_like(inst.q)
    inst.q[0, 0, 0] = 1.0
    inst.k_pool[page, 0, 0] = 0.0
    inst.k_pool[page, 1, 0] = 0.0
    inst.k_pool[page, 1, 0, 0] = np.sqrt(d) * 0.7
    _, w = ta.decode_instance(inst, return_weights=True)
    p = w[(0, 0)]
    assert abs(p[1] / p[0] - np.exp(0.7)) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_logsumexp_merge_identity(seed):
    rng = np.random.default_rng(seed)
    T, d = int(rng.integers(1, 200)), 16
    s = rng.standard_normal(T) * 3
    v = rng.standard_normal((T, d))
    full = np.exp(s - s.max())
    full = (full / full.sum()) @ v
    cuts = np.sort(rng.integers(0, T + 1, size=int(rng.integers(0, 6))))
    bounds = [0] + cuts.tolist() + [T, T]       # includes empty parts
    parts = [ta.partial_softmax(s[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    got = ta.logsumexp_merge(parts)
    assert np.max(np.abs(got - full)) < 1e-12


def test_config_shapes():
    """The five workloads have the shapes stated for them."""
    c1 = synth.make_config(1, tensors=False)
    assert c1.node_len.tolist() == [256, 32, 32, 32, 32] and c1.n_queries == 4
    c2 = synth.make_config(2, tensors=False)
    assert c2.n_nodes == 21 and c2.n_queries == 16 and c2.unique_kv_bytes == 100_663_296
    c3 = synth.make_config(3, tensors=False)
    assert c3.n_queries == 256 and c3.unique_kv_bytes == 83_886_080
    c4 = synth.make_config(4, tensors=False)
    assert c4.n_queries == 10 and c4.unique_kv_bytes == 73_728_000
    c5 = synth.make_config(5, tensors=False)
    assert c5.qpl == 4 and c5.node_len.min() >= 16 and c5.node_len.max() <= 4096
    depth = np.zeros(c5.n_nodes, int)
    for v in range(1, c5.n_nodes):
        depth[v] = depth[c5.parent[v]] + 1
    is_parent = set(c5.parent[c5.parent >= 0].tolist())
    assert all(depth[v] == 4 for v in range(c5.n_nodes) if v not in is_parent)
