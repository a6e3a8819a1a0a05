"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max-abs error <= 3e-3 against the oracle, fp32 accumulation, on the
exact bf16 / fp32 inputs the GPU sees. Every plan is built with the workspace
poisoned with NaN before each decode, so a partial the kernels fail to write
shows up as NaN in the output; unused KV slots hold V = 1e30 canaries, so an
unmasked stray read shows up as a huge value.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import tree_attention as ta
from parity_util import check as _check, dev as _dev, log as _log, run as _run
from tree_structured_shared_amd import Plan, TreeAttnError

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_full(k):
    _log(f"config {k}")
    inst = synth.make_config(k)
    ref = ta.decode_instance(inst)
    got = _run(inst)
    _check(got, ref, f"config {k}")


def test_workload5_full():
    _log("config 5")
    inst = synth.make_config(5)
    dev = _dev(inst)
    got = _run(inst, dev)
    ref = ta.decode_instance(inst)
    _check(got, ref, "config 5")


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_workload_bench_layout(k):
    """The full workloads with the pools laid out as bench.py times them
    (head-major storage, built by bench.py's own helper)."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    _log(f"config {k}, head-major pools")
    inst = synth.make_config(k)
    dev = (inst.q.cuda(), bench.head_major_pool(inst.k_pool, "cuda"), bench.head_major_pool(inst.v_pool, "cuda"))
    assert dev[1].stride(1) == inst.head_dim  # tokens of one kv-head's page adjacent
    got = _run(inst, dev)
    _check(got, ta.decode_instance(inst), f"config {k} head-major pools")


@pytest.mark.parametrize("k", [2, 5])
def test_plan_invariance(k):
    """Grouping and splitting change only summation order: forced all-0,
    all-1 and random edges, split off and other chunk sizes agree with the
    oracle too."""
    inst = synth.make_config(k)
    dev = _dev(inst)
    n = inst.n_nodes
    leaves = None if k == 2 else list(range(0, inst.n_leaves, 7))
    ref = ta.decode_instance(inst, leaves=leaves)
    rows = ~np.isnan(ref[:, 0, 0])
    rng = np.random.default_rng(k)
    variants = [dict(force_edges=[0] * n), dict(force_edges=[1] * n),
                dict(force_edges=rng.integers(0, 2, n).tolist()), dict(split=False),
                dict(ncu=1024, ts_c=16, split_align=16), dict(rb=32, floor_f=1), dict(waves=1, ncu=64),
                dict(waves=8, split_align=64), dict(tile_join=False)]
    for kw in variants:
        got = _run(inst, dev, **kw)
        _check(got[rows], ref[rows], f"config {k} {kw if 'force_edges' not in kw else 'forced'}")


@pytest.mark.parametrize("seed", range(40))
def test_random_trees(seed):
    inst = synth.random_small_tree(seed, max_nodes=30, max_len=300)
    _log(f"random tree {seed}: n={inst.n_nodes} qpl={inst.qpl} heads={inst.n_qheads}/{inst.n_kvheads} "
         f"d={inst.head_dim} ps={inst.page_size} {inst.dtype}")
    ref = ta.decode_instance(inst)
    kw = {}
    if seed % 3 == 0:
        kw = dict(ncu=512, ts_c=16, split_align=16)      # many small chunks, ragged tails
    _check(_run(inst, **kw), ref, f"random tree {seed}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.bfloat16, 128),
                                     (torch.float32, 64), (torch.float32, 128)])
@pytest.mark.parametrize("rows_case", ["gemv", "mid", "wide"])
def test_row_paths(dtype, d, rows_case):
    """Each row path of the partial kernel: GEMV-sized (1-4 rows), one MFMA
    pass (<= 64 rows) and several row passes (> 128 rows)."""
    hq, h, n_leaf, qpl = {"gemv": (4, 1, 1, 1), "mid": (8, 2, 5, 3), "wide": (16, 1, 12, 2)}[rows_case]
    par = [-1] + [0] * n_leaf
    lens = [517] + [40 + 7 * i for i in range(n_leaf)]
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=hq, n_kvheads=h, head_dim=d,
                           dtype=dtype, seed=3)
    synth.fill_tensors(inst, seed=21)
    ref = ta.decode_instance(inst)
    _check(_run(inst), ref, f"rows {rows_case} {dtype} d{d}")
    _check(_run(inst, rb=256, split=False), ref, f"rows {rows_case} {dtype} d{d} rb256 nosplit")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_reduction_pairs_per_wave(dtype):
    """The reduction packs 4, 2 or 1 (query, q-head) pairs per wave by the
    plan's largest slot count per query (at most 4, 8, or more), and loads
    batches of 4, 8 or 16 slots per lane group (one pair per wave with up to
    16, 32 or more slots). Cover every kernel variant, with pair counts that
    are not a multiple of the packing (the wave's last groups have no pair)."""
    cases = [
        # (parent, lens, qpl, n_qheads, n_kvheads, plan options)
        ([-1, 0, 0], [40, 20, 30], 1, 1, 1, {}),                                  # 2 pairs, <= 4 slots
        ([-1, 0, 0, 1, 1, 2], [70, 20, 30, 9, 17, 25], 2, 3, 1, {}),              # 18 pairs
        ([-1, 0, 0, 0], [900, 40, 70, 33], 1, 3, 3,
         dict(waves=2, ncu=8, floor_f=0, split_align=16)),                        # 9 pairs, 6 slots
        ([-1, 0, 1, 1], [300, 300, 40, 70], 1, 5, 5,
         dict(waves=2, ncu=32, floor_f=0, split_align=16)),                       # 10 pairs, 12 slots
        ([-1, 0, 1, 1], [300, 300, 40, 70], 1, 5, 5,
         dict(waves=4, ncu=32, floor_f=0, split_align=16)),                       # 22 slots
        ([-1, 0, 1, 1], [2000, 300, 40, 70], 1, 5, 5,
         dict(waves=64, floor_f=0, split_align=16)),                              # 10 pairs, long paths
    ]
    seen = set()
    for x, (parent, lens, qpl, hq, hk, kw) in enumerate(cases):
        inst = synth.make_tree(parent, lens, page_size=16, qpl=qpl, n_qheads=hq, n_kvheads=hk,
                               head_dim=128 if dtype == torch.bfloat16 else 64, dtype=dtype, seed=40 + x)
        synth.fill_tensors(inst, seed=50 + x)
        plan = Plan.for_instance(inst, host_only=True, **kw)
        ms = int(np.diff(plan.export("q_slot_ptr")).max())
        plan.close()
        variant = (4, 4) if ms <= 4 else (2, 4) if ms <= 8 else (1, 4) if ms <= 16 else (1, 8) if ms <= 32 else (1, 16)
        seen.add(variant)
        _log(f"case {x}: {inst.n_queries} queries x {hq} q-heads, max {ms} slots per query, "
             f"(pairs per wave, batch) {variant}")
        _check(_run(inst, **kw), ta.decode_instance(inst), f"pairs-per-wave case {x}")
    assert seen == {(4, 4), (2, 4), (1, 4), (1, 8), (1, 16)}, seen


def test_edge_cases():
    cases = [
        ([-1], [1], 1),                 # one node, one token
        ([-1], [5], 5),                 # first query sees one token only
        ([-1, 0], [1, 1], 1),           # one-token nodes
        ([-1, 0, 0, 1], [33, 17, 1, 64], 1),
    ]
    for ps in (1, 16, 256):
        for par, lens, qpl in cases:
            for dtype in (torch.bfloat16, torch.float32):
                inst = synth.make_tree(par, lens, page_size=ps, qpl=qpl, n_qheads=8, n_kvheads=2,
                                       head_dim=128, dtype=dtype, seed=1)
                synth.fill_tensors(inst, seed=2)
                ref = ta.decode_instance(inst)
                _check(_run(inst), ref, f"edge {par} {lens} qpl{qpl} ps{ps} {dtype}")


@pytest.mark.parametrize("qpl", [8, 32, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_speculative_trees(qpl, dtype):
    """Larger speculative trees: 8-64 query tokens per leaf under the
    leaf-local causal mask (a leaf's j-th query sees its leaf up to its own
    position), with a shared prompt and a middle level."""
    par = [-1, 0, 0, 1, 1, 2, 2, 2]
    lens = [300, 40, 90, qpl + 5, 2 * qpl, qpl, qpl + 33, 3 * qpl + 1]
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=16, n_kvheads=4, head_dim=128,
                           dtype=dtype, seed=qpl)
    synth.fill_tensors(inst, seed=100 + qpl)
    ref = ta.decode_instance(inst)
    _check(_run(inst), ref, f"qpl {qpl} {dtype}")
    _check(_run(inst, force_edges=[1] * inst.n_nodes), ref, f"qpl {qpl} {dtype} all-1")


@pytest.mark.parametrize("dtype,d,qpl", [(torch.bfloat16, 128, 4), (torch.bfloat16, 128, 32),
                                         (torch.bfloat16, 64, 32), (torch.float32, 128, 4)])
def test_single_slot_queries(dtype, d, qpl):
    """A query whose path is one partial (one group, one chunk) takes its
    output straight from the partial kernel, which normalises it; the
    reduction skips it, and is not launched when every query is such. Every
    edge joined without the split: one slot per query (no reduction launch);
    one leaf joined to the root and one not: single-slot and two-slot queries
    in one decode. Leaf groups of 16 rows (qpl 4) and of 128 rows (32-row
    tiles), and the fp32 path."""
    par, lens = [-1, 0, 0, 1], [300, 70, 90, 40]
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=8, n_kvheads=2, head_dim=d, dtype=dtype,
                           seed=11)
    synth.fill_tensors(inst, seed=12)
    ref = ta.decode_instance(inst)
    devt = _dev(inst)
    tag = f"{str(dtype)[6:]} d{d} qpl{qpl}"
    plan = Plan.for_instance(inst, force_edges=[1, 1, 1, 1], split=False, poison_workspace=True)
    slots = np.diff(plan.export("q_slot_ptr"))
    assert (slots == 1).all()
    plan.timing_enable(2)  # the record stays whole without a reduction launch
    out = plan.decode(*devt)
    torch.cuda.synchronize()
    pm, rm = plan.timing_read(2)
    assert len(pm) == 1 and len(rm) == 1 and pm[0] > 0 and rm[0] == 0  # no reduction kernel
    _check(out.cpu().numpy().astype(np.float64), ref, f"single-slot queries, every edge joined, {tag}")
    plan.close()
    kw = dict(force_edges=[0, 1, 0, 1], split=False)
    plan = Plan.for_instance(inst, **kw)
    slots = np.diff(plan.export("q_slot_ptr"))
    assert (slots == 1).any() and (slots > 1).any()
    plan.close()
    _check(_run(inst, devt, **kw), ref, f"single- and two-slot queries, {tag}")


def test_max_rows_per_item():
    """A group with many rows (root of 300 queries x GQA 8 = 2400 rows) spans
    several row blocks."""
    n_leaf = 300
    inst = synth.make_tree([-1] + [0] * n_leaf, [700] + [3] * n_leaf, page_size=16, qpl=1,
                           n_qheads=32, n_kvheads=4, head_dim=128, dtype=torch.bfloat16, seed=5)
    synth.fill_tensors(inst, seed=6)
    ref = ta.decode_instance(inst, leaves=list(range(0, n_leaf, 13)))
    got = _run(inst)
    rows = ~np.isnan(ref[:, 0, 0])
    _check(got[rows], ref[rows], "2400-row root")


def test_repeat_decodes_identical():
    inst = synth.make_config(3)
    q, k, v = _dev(inst)
    plan = Plan.for_instance(inst)
    a = plan.decode(q, k, v).clone()
    b = plan.decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    plan.close()


def test_decode_argument_errors():
    inst = synth.make_config(1)
    q, k, v = _dev(inst)
    plan = Plan.for_instance(inst)
    with pytest.raises(TreeAttnError):
        plan.decode(q.to(torch.bfloat16), k, v)           # dtype mismatch
    with pytest.raises(TreeAttnError):
        plan.decode(q, k[:2], v[:2])                      # pool smaller than the plan's pages
    with pytest.raises(TreeAttnError):
        plan.decode(q[:2], k, v)                          # wrong query count
    plan.close()


@pytest.mark.parametrize("k", [2, 5])
def test_timing_records(k):
    """Per-kernel timing records, on a plan with one item class (config 2)
    and one with both (config 5)."""
    inst = synth.make_config(k)
    q, k_, v = _dev(inst)
    plan = Plan.for_instance(inst)
    plan.timing_enable(4)
    for _ in range(3):
        plan.decode(q, k_, v)
    pm, rm = plan.timing_read(4)
    assert len(pm) == 3 and (pm > 0).all() and (rm > 0).all()
    assert len(plan.timing_read(4)[0]) == 0          # the read cleared the record
    plan.decode(q, k_, v)
    assert len(plan.timing_read(4)[0]) == 1
    plan.close()


def test_graph_capture_replays():
    """A decode captured in a HIP graph (through torch's graph capture, on a
    plan with both item classes) replays to the eager result, with eager
    decodes and synchronisations between the replays."""
    inst = synth.make_config(5)
    q, k, v = _dev(inst)
    plan = Plan.for_instance(inst)
    eager = plan.decode(q, k, v).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        plan.decode(q, k, v, out=out)        # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            plan.decode(q, k, v, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        other = plan.decode(q, k, v)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    plan.close()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_of_new_nodes(dtype):
    """Prefill of new nodes as tree attention: every token of a new leaf is a
    query (queries_per_leaf = its length), causal inside the leaf, over the
    shared ancestors (two new 256-token leaves under a 700-token prompt)."""
    qpl = 256
    par = [-1, 0, 1, 1]
    lens = [700, 90, qpl, qpl]
    inst = synth.make_tree(par, lens, page_size=16, qpl=qpl, n_qheads=16, n_kvheads=4, head_dim=128,
                           dtype=dtype, seed=11)
    synth.fill_tensors(inst, seed=12)
    ref = ta.decode_instance(inst)
    _check(_run(inst), ref, f"prefill {dtype}")


def _strided_pools(inst, layout):
    """The instance's pools in another layout, as [n_pages, page_size, H, d]
    views with head_dim contiguous."""
    if layout == "head_major":     # storage [pages, H, page_size, d]
        mk = lambda p: p.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    else:                          # each page padded to 16 MiB: byte offsets past 32 bits' fast path
        def mk(p):
            n_pages, ps, h, d = p.shape
            esz = p.element_size()
            pad_tokens = max(ps, (16 << 20) // (h * d * esz))
            big = torch.zeros((n_pages, pad_tokens, h, d), dtype=p.dtype, device="cuda")
            big[:, :ps].copy_(p)
            return big[:, :ps]
    return mk(inst.k_pool), mk(inst.v_pool)


@pytest.mark.parametrize("layout,dtype", [("head_major", torch.bfloat16), ("head_major", torch.float32),
                                          ("padded_pages", torch.bfloat16)])
def test_pool_layouts(layout, dtype):
    """Pools in any layout with head_dim contiguous: head-major pages, and
    pages 16 MiB apart (the kernels' 64-bit address path)."""
    par = [-1, 0, 0, 1, 2, 2]
    lens = [400, 50, 33, 20 + 16, 17, 64]
    inst = synth.make_tree(par, lens, page_size=16, qpl=2, n_qheads=8, n_kvheads=2, head_dim=128, dtype=dtype,
                           seed=21)
    synth.fill_tensors(inst, seed=22)
    ref = ta.decode_instance(inst)
    k, v = _strided_pools(inst, layout)
    plan = Plan.for_instance(inst, poison_workspace=True)
    got = plan.decode(inst.q.cuda(), k, v)
    torch.cuda.synchronize()
    _check(got.cpu().numpy().astype(np.float64), ref, f"pools {layout} {dtype}")
    plan.close()
