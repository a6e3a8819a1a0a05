"""fp64 CPU oracle of tree-structured decode attention -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

What it computes (the plain definition, no grouping, no splitting):

* DeFT reading notes, "decoding tree" and "tree attention" definitions: the
  root holds the prompt, every other node holds a generated token run, and the
  last token(s) of each leaf are the decode step's inputs. The tree attention
  of a token n inside node u runs over the path P_root->n, i.e. every token of
  u's ancestors followed by u's own tokens up to and including n. The notes'
  wording ("sum of sequence attention outputs") is garbled; the only reading
  consistent with exact reconstruction by softmax reduction (same notes,
  "global reduction") is one softmax over the concatenated path.
* FastTree review, section 3, core formula: Attention(Q,K,V) =
  softmax(Q K^T / sqrt(d)) V with d the head dimension.
* Query placement: query j (0 <= j < qpl) of leaf l is l's token
  len(l) - qpl + j; it sees every ancestor token and l's tokens 0..len(l)-qpl+j
  (a causal mask inside the leaf only; with qpl = 1 nothing is masked).
* GQA: q-head h reads kv-head h // (n_qheads / n_kvheads).

Parity pins (tests/test_oracle.py): a dense token-level tree-mask brute force,
chain tree == torch scaled_dot_product_attention, closed forms (constant V,
zero K, single visible token), and softmax rows summing to one.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    """Upcast a numpy array or CPU torch tensor to a float64 numpy array."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def children_lists(parent):
    n = len(parent)
    ch = [[] for _ in range(n)]
    for v in range(n):
        p = int(parent[v])
        if p >= 0:
            ch[p].append(v)
    return ch


def leaves_in_order(parent):
    """Leaves ranked by ascending node id."""
    ch = children_lists(parent)
    return [v for v in range(len(parent)) if not ch[v]]


def root_path(parent, v):
    """Node ids from the root down to v."""
    path = []
    while v >= 0:
        path.append(int(v))
        v = int(parent[v])
    return path[::-1]


def node_kv(pool, u, node_len, node_page_ptr, node_page_ids, page_size):
    """Tokens of node u gathered from a paged pool [n_pages, ps, H, d] -> [len, H, d] (fp64)."""
    pages = np.asarray(node_page_ids[int(node_page_ptr[u]):int(node_page_ptr[u + 1])], dtype=np.int64)
    if hasattr(pool, "detach"):
        import torch
        blk = pool[torch.from_numpy(pages)]
    else:
        blk = pool[pages]
    blk = _f64(blk)
    L = int(node_len[u])
    return blk.reshape(-1, blk.shape[2], blk.shape[3])[:L]


def tree_decode_attention(parent, node_len, node_page_ptr, node_page_ids, page_size,
                          q, k_pool, v_pool, qpl, n_kvheads, scale=None,
                          leaves=None, return_weights=False):
    """Output [n_queries, n_qheads, d] in fp64.

    ``leaves``: optional subset of leaf ranks to evaluate (other rows stay NaN),
    so full-size instances can be checked on samples.
    ``return_weights``: also return {(query, q-head): softmax weights over that
    query's visible path tokens}.
    """
    parent = np.asarray(parent)
    q = _f64(q)
    n_q, hq, d = q.shape
    g = hq // n_kvheads
    assert g * n_kvheads == hq
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lv = leaves_in_order(parent)
    assert n_q == len(lv) * qpl
    out = np.full((n_q, hq, d), np.nan)
    weights = {}
    ranks = range(len(lv)) if leaves is None else leaves
    cache_k, cache_v = {}, {}

    def kv(u):
        if u not in cache_k:
            cache_k[u] = node_kv(k_pool, u, node_len, node_page_ptr, node_page_ids, page_size)
            cache_v[u] = node_kv(v_pool, u, node_len, node_page_ptr, node_page_ids, page_size)
        return cache_k[u], cache_v[u]

    for r in ranks:
        leaf = lv[r]
        path = root_path(parent, leaf)
        ks, vs = zip(*(kv(u) for u in path))
        k_path = np.concatenate(ks, axis=0)          # [T, H, d]
        v_path = np.concatenate(vs, axis=0)
        n_anc = k_path.shape[0] - int(node_len[leaf])
        for j in range(qpl):
            qi = r * qpl + j
            n_vis = n_anc + int(node_len[leaf]) - qpl + j + 1
            kk = k_path[:n_vis].transpose(1, 2, 0)   # [H, d, T]
            vv = v_path[:n_vis].transpose(1, 0, 2)   # [H, T, d]
            qq = q[qi].reshape(n_kvheads, g, d)      # q-head h = kvh * g + i
            s = scale * np.matmul(qq, kk)            # [H, g, T]
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            o = np.matmul(p, vv)                     # [H, g, d]
            out[qi] = o.reshape(hq, d)
            if return_weights:
                pw = p.reshape(hq, -1)
                for h in range(hq):
                    weights[(qi, h)] = pw[h]
    if return_weights:
        return out, weights
    return out


def decode_instance(inst, leaves=None, return_weights=False, scale=None):
    """Convenience wrapper over a synth.TreeInstance-like object."""
    return tree_decode_attention(inst.parent, inst.node_len, inst.node_page_ptr, inst.node_page_ids,
                                 inst.page_size, inst.q, inst.k_pool, inst.v_pool, inst.qpl,
                                 inst.n_kvheads, scale=scale, leaves=leaves,
                                 return_weights=return_weights)


def logsumexp_merge(parts):
    """Merge partial softmax results of one query/head over disjoint token sets.

    Each part is (m, l, o) with m the max score of the part, l = sum exp(s - m)
    and o = sum exp(s - m) v (unnormalised). Empty parts are (-inf, 0, 0).
    Returns the normalised output. This is the incremental softmax reduction
    the DeFT notes describe for rebuilding attention from per-group partials
    ("tree-topology-aware global reduction").
    """
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    M = ms.max()
    w = np.where(np.isfinite(ms), np.exp(ms - M), 0.0)
    num = sum(wi * np.asarray(p[2], np.float64) for wi, p in zip(w, parts))
    den = sum(wi * float(p[1]) for wi, p in zip(w, parts))
    return num / den


def partial_softmax(s, v):
    """(m, l, o) of one part: scores s [T] and values v [T, d] (fp64)."""
    s = np.asarray(s, np.float64)
    v = np.asarray(v, np.float64)
    if s.size == 0:
        return (-np.inf, 0.0, np.zeros(v.shape[-1]))
    m = s.max()
    e = np.exp(s - m)
    return (m, e.sum(), e @ v)
