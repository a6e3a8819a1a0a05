"""GPU: decode-loop plan reuse. After tree_attn_plan_extend (device tables
updated in place on the decode stream, or uploaded whole when they outgrow
their allocation) the decode of the grown tree matches the fp64 oracle, and
a decode captured in a HIP graph replays the grown tree while extend reports
no relaunch. Extends and decodes are enqueued back to back on one stream,
without host synchronisation between them."""
import numpy as np
import pytest
import torch

import synth
from oracle import tree_attention as ta
from parity_util import check as _check_np, log as _log
from tree_structured_shared_amd import Plan

pytestmark = pytest.mark.gpu


def _check(got, ref, what):
    _check_np(got.cpu().numpy().astype(np.float64), ref, what)


def _small_tree(dtype, qpl):
    par = [-1, 0, 0, 1, 1, 2, 0]
    lens = [300, 40, 70, 20, 33, 16, 5 + qpl]
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=16, n_kvheads=4, head_dim=128,
                           dtype=dtype, seed=qpl)
    return synth.fill_tensors(inst, seed=40 + qpl)


@pytest.mark.parametrize("dtype,qpl", [(torch.bfloat16, 1), (torch.bfloat16, 4), (torch.float32, 2)])
def test_extend_decode_matches_oracle(dtype, qpl):
    inst = _small_tree(dtype, qpl)
    plan = Plan.for_instance(inst, poison_workspace=True, ncu=64, ts_c=16, split_align=16)
    rng = np.random.default_rng(qpl)
    for step in range(7):
        if step == 4:
            add = rng.integers(200, 500, size=inst.n_leaves)     # outgrows the page-table slack
        else:
            add = np.full(inst.n_leaves, qpl) + (step % 2) * rng.integers(0, 40, size=inst.n_leaves)
        inst, new_pages = synth.grow_leaves(inst, add, seed=100 * qpl + step)
        relaunch = plan.extend(add, new_pages)
        out = plan.decode(inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda())
        _check(out, ta.decode_instance(inst), f"{dtype} qpl {qpl} step {step} relaunch {relaunch}")
    plan.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_extend_across_single_slot_queries(dtype):
    """Every edge joined on a small tree: each leaf's group is its whole path
    in one chunk, so every query has one slot (outputs written by the partial
    kernel, no reduction launch). Growing one leaf past the chunk length
    gives its queries several slots while the other leaf's keep one (mixed),
    then both: the slot table moves from the direct form to the partial
    records in place, and the reduction comes back."""
    par, lens = [-1, 0, 0], [50, 30, 40]
    inst = synth.make_tree(par, lens, page_size=16, qpl=2, n_qheads=16, n_kvheads=4, head_dim=128, dtype=dtype,
                           seed=5)
    inst = synth.fill_tensors(inst, seed=6)
    plan = Plan.for_instance(inst, poison_workspace=True, force_edges=[1, 1, 1])
    slots = np.diff(plan.export("q_slot_ptr"))
    assert (slots == 1).all()
    out = plan.decode(inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda())
    _check(out, ta.decode_instance(inst), f"{dtype} one slot per query")
    for step, add in enumerate(([300, 2], [2, 300], [2, 2])):
        add = np.asarray(add, np.int64)
        inst, new_pages = synth.grow_leaves(inst, add, seed=50 + step)
        plan.extend(add, new_pages)
        slots = np.diff(plan.export("q_slot_ptr"))
        out = plan.decode(inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda())
        _check(out, ta.decode_instance(inst), f"{dtype} step {step} slots per query {slots.tolist()}")
        if step == 0:
            assert (slots == 1).any() and (slots > 1).any()
        if step == 2:
            assert (slots > 1).all()
    plan.close()


def test_extend_config2_decode_loop():
    """The multi-level prompt workload, one token per leaf per step."""
    inst = synth.make_config(2)
    plan = Plan.for_instance(inst, poison_workspace=True)
    for step in range(3):
        add = np.ones(inst.n_leaves, np.int64)
        inst, new_pages = synth.grow_leaves(inst, add, seed=7 + step)
        plan.extend(add, new_pages)
        out = plan.decode(inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda())
        _check(out, ta.decode_instance(inst), f"config 2 step {step}")
    plan.close()


def test_extend_graph_replay():
    """Pools, Q and out live at fixed addresses (pools with spare pages); the
    captured decode replays the grown tree after every extend that reports
    no relaunch, and is captured again when one does."""
    inst = _small_tree(torch.bfloat16, 2)
    spare = 256
    shape = (inst.n_pages + spare,) + tuple(inst.k_pool.shape[1:])
    k_dev = torch.zeros(shape, dtype=inst.dtype, device="cuda")
    v_dev = torch.full(shape, synth.CANARY_V, dtype=torch.float32, device="cuda").to(inst.dtype)
    q_dev = torch.empty(inst.q.shape, dtype=inst.dtype, device="cuda")
    out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device="cuda")

    def load(x):
        k_dev[:x.n_pages].copy_(x.k_pool)
        v_dev[:x.n_pages].copy_(x.v_pool)
        q_dev.copy_(x.q)

    load(inst)
    plan = Plan.for_instance(inst)
    side = torch.cuda.Stream()

    def capture():
        g = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            plan.decode(q_dev, k_dev, v_dev, out=out)
            side.synchronize()
            with torch.cuda.graph(g, stream=side):
                plan.decode(q_dev, k_dev, v_dev, out=out)
        torch.cuda.synchronize()
        return g

    g = capture()
    replays = 0
    for step in range(6):
        add = np.ones(inst.n_leaves, np.int64) * (1 if step != 3 else 37)
        inst, new_pages = synth.grow_leaves(inst, add, seed=500 + step)
        assert inst.n_pages <= shape[0]
        load(inst)
        relaunch = plan.extend(add, new_pages)
        if relaunch:
            g = capture()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        replays += 0 if relaunch else 1
        eager = plan.decode(q_dev, k_dev, v_dev)
        torch.cuda.synchronize()
        assert torch.equal(replayed, eager), f"step {step}: replay differs from eager"
        _check(replayed, ta.decode_instance(inst), f"graph step {step} relaunch {relaunch}")
    assert replays >= 1, "no extend kept the captured graph valid"
    plan.close()


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128)])
def test_kv_append_scatter(dtype, d):
    """Rows land bit for bit where the page-table words say; destinations
    outside the pool are skipped."""
    from tree_structured_shared_amd import kv_append
    g = torch.Generator().manual_seed(d)
    n_pages, ps, h, n = 40, 16, 4, 300
    k_pool = torch.randn((n_pages, ps, h, d), generator=g).to(dtype)
    v_pool = torch.randn((n_pages, ps, h, d), generator=g).to(dtype)
    k_new = torch.randn((n, h, d), generator=g).to(dtype)
    v_new = torch.randn((n, h, d), generator=g).to(dtype)
    cells = torch.randperm(n_pages * ps, generator=g)[:n]
    page, slot = cells // ps, cells % ps
    dst = (page << 8) | slot
    dst[::37] = (n_pages + 3) << 8          # past the pool: skipped
    dst[5] = (2 << 8) | 200                 # slot past the page: skipped
    dst[6] = -1                             # negative word: skipped
    ok = (dst >= 0) & ((dst >> 8) < n_pages) & ((dst & 255) < ps)
    want_k, want_v = k_pool.clone(), v_pool.clone()
    want_k[page[ok], slot[ok]] = k_new[ok]
    want_v[page[ok], slot[ok]] = v_new[ok]
    kd, vd = k_pool.cuda(), v_pool.cuda()
    kv_append(kd, vd, k_new.cuda(), v_new.cuda(), dst.to(torch.int32).cuda())
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), want_k) and torch.equal(vd.cpu(), want_v)


def test_kv_appender_reuses_buffers():
    """A prepared appender writes each call's rows where that call's dst
    says (same result as kv_append), and checks dst on every call."""
    from tree_structured_shared_amd import TreeAttnError, kv_append, kv_appender
    g = torch.Generator().manual_seed(7)
    n_pages, ps, h, d, n = 24, 16, 2, 128, 40
    k_pool = torch.randn((n_pages, ps, h, d), generator=g).to(torch.bfloat16)
    v_pool = torch.randn((n_pages, ps, h, d), generator=g).to(torch.bfloat16)
    k_new = torch.randn((n, h, d), generator=g).to(torch.bfloat16).cuda()
    v_new = torch.randn((n, h, d), generator=g).to(torch.bfloat16).cuda()
    cells = torch.randperm(n_pages * ps, generator=g)[:2 * n]
    dsts = [((cells[x * n:(x + 1) * n] // ps) << 8 | cells[x * n:(x + 1) * n] % ps).to(torch.int32).cuda()
            for x in range(2)]
    ka, va = k_pool.cuda(), v_pool.cuda()
    kb, vb = k_pool.cuda(), v_pool.cuda()
    app = kv_appender(ka, va, k_new, v_new)
    for dst in dsts:
        app(dst)
        kv_append(kb, vb, k_new, v_new, dst)
    torch.cuda.synchronize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert not torch.equal(ka.cpu(), k_pool)
    with pytest.raises(TreeAttnError):
        app(dsts[0].to(torch.int64))


def test_decode_loop_append_extend_decode():
    """A decode loop through the library only: the new tokens' K/V go in with
    kv_append, the plan grows with extend, the decode matches the oracle on
    the grown tree; the device pools equal the grown instance's pools."""
    from tree_structured_shared_amd import kv_append
    inst = _small_tree(torch.bfloat16, 2)
    spare = 64
    kd = torch.zeros((inst.n_pages + spare,) + tuple(inst.k_pool.shape[1:]), dtype=inst.dtype, device="cuda")
    vd = torch.full(kd.shape, synth.CANARY_V, dtype=torch.float32, device="cuda").to(inst.dtype)
    kd[:inst.n_pages].copy_(inst.k_pool)
    vd[:inst.n_pages].copy_(inst.v_pool)
    plan = Plan.for_instance(inst, poison_workspace=True)
    has_child = np.zeros(inst.n_nodes, bool)
    has_child[inst.parent[inst.parent >= 0]] = True
    leaves = np.flatnonzero(~has_child)
    for step in range(5):
        add = np.full(inst.n_leaves, inst.qpl) + (step == 2) * 30
        grown, new_pages = synth.grow_leaves(inst, add, seed=900 + step)
        assert grown.n_pages <= kd.shape[0]
        # the new tokens, leaf-rank order, and where the grown tree puts them
        locs, rows_k, rows_v = [], [], []
        for v in leaves:
            pages = grown.node_page_ids[grown.node_page_ptr[v]:grown.node_page_ptr[v + 1]]
            for t in range(int(inst.node_len[v]), int(grown.node_len[v])):
                pg, sl = int(pages[t // grown.page_size]), t % grown.page_size
                locs.append((pg << 8) | sl)
                rows_k.append(grown.k_pool[pg, sl])
                rows_v.append(grown.v_pool[pg, sl])
        kv_append(kd, vd, torch.stack(rows_k).cuda().contiguous(), torch.stack(rows_v).cuda().contiguous(),
                  torch.tensor(locs, dtype=torch.int32, device="cuda"))
        plan.extend(add, new_pages)
        out = plan.decode(grown.q.cuda(), kd, vd)
        _check(out, ta.decode_instance(grown), f"append+extend step {step}")
        assert torch.equal(kd[:grown.n_pages].cpu(), grown.k_pool)
        assert torch.equal(vd[:grown.n_pages].cpu(), grown.v_pool)
        inst = grown
    plan.close()


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_fused_append_extend_matches_separate_calls(dtype, d):
    """tree_attn_plan_extend_append (one launch for the KV append and the
    table update) against tree_attn_kv_append + tree_attn_plan_extend on a
    twin plan and twin pools: the same pools, tables and (bit-identical)
    decode outputs every step, within the tolerance of the oracle; covers the
    first extend (tables uploaded whole), in-place updates, a step that
    outgrows a leaf's page-table slack and a step with no new tokens."""
    from tree_structured_shared_amd import kv_append, kv_appender
    if d == 128:
        inst = _small_tree(dtype, 2)
    else:
        inst = synth.make_tree([-1, 0, 0, 1, 1, 2, 0], [300, 40, 70, 20, 33, 16, 7], page_size=16, qpl=2,
                               n_qheads=16, n_kvheads=4, head_dim=d, dtype=dtype, seed=2)
        inst = synth.fill_tensors(inst, seed=42)
    spare = 96
    pools = []
    for _ in range(2):
        kd = torch.zeros((inst.n_pages + spare,) + tuple(inst.k_pool.shape[1:]), dtype=inst.dtype, device="cuda")
        vd = torch.full(kd.shape, synth.CANARY_V, dtype=torch.float32, device="cuda").to(inst.dtype)
        kd[:inst.n_pages].copy_(inst.k_pool)
        vd[:inst.n_pages].copy_(inst.v_pool)
        pools.append((kd, vd))
    plans = [Plan.for_instance(inst, poison_workspace=True) for _ in range(2)]
    has_child = np.zeros(inst.n_nodes, bool)
    has_child[inst.parent[inst.parent >= 0]] = True
    leaves = np.flatnonzero(~has_child)
    for step, extra in enumerate([0, 0, 300, 0, -1, 0]):
        add = np.zeros(inst.n_leaves, np.int64) if extra < 0 else np.full(inst.n_leaves, inst.qpl) + extra
        grown, new_pages = synth.grow_leaves(inst, add, seed=700 + step)
        assert grown.n_pages <= pools[0][0].shape[0]
        locs, rows_k, rows_v = [], [], []
        for v in leaves:
            pages = grown.node_page_ids[grown.node_page_ptr[v]:grown.node_page_ptr[v + 1]]
            for t in range(int(inst.node_len[v]), int(grown.node_len[v])):
                pg, sl = int(pages[t // grown.page_size]), t % grown.page_size
                locs.append((pg << 8) | sl)
                rows_k.append(grown.k_pool[pg, sl])
                rows_v.append(grown.v_pool[pg, sl])
        shape = (len(locs), inst.n_kvheads, inst.head_dim)
        k_new = torch.stack(rows_k).cuda().contiguous() if locs else torch.zeros(shape, dtype=inst.dtype, device="cuda")
        v_new = torch.stack(rows_v).cuda().contiguous() if locs else torch.zeros(shape, dtype=inst.dtype, device="cuda")
        dst = torch.tensor(locs, dtype=torch.int32, device="cuda")
        _log(f"fused append+extend step {step}: {len(locs)} new tokens")
        (ka, va), (kb, vb) = pools
        kv_append(ka, va, k_new, v_new, dst)
        ra = plans[0].extend(add, new_pages)
        rb = plans[1].extend(add, new_pages, append=(kv_appender(kb, vb, k_new, v_new), dst))
        assert ra == rb
        outs = [p.decode(grown.q.cuda(), k, v) for p, (k, v) in zip(plans, pools)]
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {step}: fused and separate outputs differ"
        _check(outs[1], ta.decode_instance(grown), f"fused append+extend step {step}")
        ta_, tb_ = plans[0].tables(), plans[1].tables()
        assert ta_.keys() == tb_.keys()
        for name in ta_:
            assert np.array_equal(ta_[name], tb_[name]), (step, name)
        assert torch.equal(kb, ka) and torch.equal(vb, va)
        assert torch.equal(kb[:grown.n_pages].cpu(), grown.k_pool)
        assert torch.equal(vb[:grown.n_pages].cpu(), grown.v_pool)
        inst = grown
    for p in plans:
        p.close()


def test_update_routes_write_identical_device_tables():
    """In-place table updates travel in the kernel arguments when they fit
    (at most 448 words) and through the pinned staging buffer otherwise.
    Twin plans, one forced onto the staging route, grow over steps whose
    updates fall under and over that size: their device tables (read back
    from the device) and decode outputs are identical every step, and the
    update counts show which route each step took."""
    n_leaf = 20
    inst = synth.make_tree([-1] + [0] * n_leaf, [400] + [20 + 3 * i for i in range(n_leaf)], page_size=16, qpl=1,
                           n_qheads=8, n_kvheads=2, head_dim=128, dtype=torch.bfloat16, seed=9)
    inst = synth.fill_tensors(inst, seed=10)
    spare = n_leaf * 8 * 4
    k = torch.zeros((inst.n_pages + spare,) + tuple(inst.k_pool.shape[1:]), dtype=inst.dtype, device="cuda")
    v = torch.full(k.shape, synth.CANARY_V, dtype=torch.float32, device="cuda").to(inst.dtype)
    k[:inst.n_pages].copy_(inst.k_pool)
    v[:inst.n_pages].copy_(inst.v_pool)
    plans = [Plan.for_instance(inst), Plan.for_instance(inst, force_staging=True)]
    seen_args = seen_staging = False
    # step 0 uploads whole; then one leaf gains a token (a small update: its
    # item, its visible length, one page-table word), then every leaf gains
    # 100 (a large one: 2,000 page-table words), alternating
    for step in range(6):
        add = np.zeros(inst.n_leaves, np.int64)
        if step == 0:
            add[:] = 1
        elif step % 2 == 1:
            add[step % inst.n_leaves] = 1
        else:
            add[:] = 100
        grown, new_pages = synth.grow_leaves(inst, add, seed=800 + step)
        assert grown.n_pages <= k.shape[0]
        k[inst.n_pages:grown.n_pages].copy_(grown.k_pool[inst.n_pages:])
        v[inst.n_pages:grown.n_pages].copy_(grown.v_pool[inst.n_pages:])
        for (pg, grown_pg) in ((k, grown.k_pool), (v, grown.v_pool)):
            pg[:grown.n_pages].copy_(grown_pg)
        before = [p.export("update_counts").copy() for p in plans]
        rel = [p.extend(add, new_pages) for p in plans]
        assert rel[0] == rel[1]
        after = [p.export("update_counts") for p in plans]
        d = [a - b for a, b in zip(after, before)]
        _log(f"route step {step}: default {d[0].tolist()} forced staging {d[1].tolist()}")
        assert d[1][0] == 0                      # the forced plan never uses the arguments
        if d[0][2] == 0:                         # an in-place step on both
            assert d[0].sum() == 1 and d[1].sum() == 1 and d[1][1] == 1
            seen_args |= bool(d[0][0])
            seen_staging |= bool(d[0][1])
        dt = [p.export("device_tables") for p in plans]
        assert dt[0].shape == dt[1].shape and np.array_equal(dt[0], dt[1]), f"step {step}: device tables differ"
        outs = [p.decode(grown.q.cuda(), k, v) for p in plans]
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {step}: outputs differ"
        _check(outs[0], ta.decode_instance(grown), f"update routes step {step}")
        inst = grown
    assert seen_args and seen_staging, (seen_args, seen_staging)
    for p in plans:
        p.close()
