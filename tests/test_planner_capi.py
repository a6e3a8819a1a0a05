"""The library's C++ planner (host-only plans, no GPU) against the Python
re-derivation, table by table, bit for bit; plus the C-ABI surface and its
documented error codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import planner_ref as pr
from tree_structured_shared_amd import Plan, TreeAttnError, _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _compare(inst, **kw):
    ref = pr.plan_instance(inst, **kw)
    ref_kw = dict(kw)
    split = ref_kw.pop("split", 1)
    p = Plan.for_instance(inst, host_only=True, ncu=ref_kw.pop("ncu", 256), split=bool(split), **ref_kw)
    got = p.tables()
    for name in pr.TABLE_NAMES:
        a, b = ref[name], got[name]
        assert a.shape == b.shape, (name, a.shape, b.shape)
        assert np.array_equal(a, b), name
    p.close()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_plans_bit_exact(k):
    _compare(synth.make_config(k, tensors=False))


@pytest.mark.parametrize("k", [2, 5])
def test_workload_plans_variants_bit_exact(k):
    inst = synth.make_config(k, tensors=False)
    _compare(inst, split=0)
    _compare(inst, force_edges=[0] * inst.n_nodes)
    _compare(inst, force_edges=[1] * inst.n_nodes)
    _compare(inst, ts_c=128, gamma=8, rb=64, waves=2, floor_f=8, ncu=304)
    _compare(inst, tile_join=0)


def test_random_trees_bit_exact():
    for seed in range(1000):
        inst = synth.random_small_tree(seed, tensors=False)
        rng = np.random.default_rng(seed + 5)
        kw = {}
        r = seed % 5
        if r == 1:
            kw["force_edges"] = rng.integers(0, 2, size=inst.n_nodes).tolist()
        elif r == 2:
            kw.update(ncu=int(rng.integers(1, 9)), ts_c=16, rb=int(rng.choice([4, 16, 64])))
        elif r == 3:
            kw.update(split=0, ts_q=4, gamma=int(rng.integers(1, 200)))
        elif r == 4:
            kw.update(waves=int(rng.integers(1, 8)), floor_f=int(rng.integers(1, 16)), ncu=16,
                      split_align=int(rng.choice([16, 32, 48, 128])), tile_join=int(rng.integers(0, 2)),
                      stream_rows=int(rng.choice([4, 8, 16])))
        _compare(inst, **kw)


def test_fasttree_example_through_library():
    for qpl, expect in ((8, [0, 0]), (128, [1, 1])):
        p = Plan([-1, 0, 0], [256, 256, 256], [0, 16, 32, 48], np.arange(48), 16, qpl, 4, 4, 128,
                 host_only=True)
        assert p.export("edges")[1:].tolist() == expect


def test_exported_symbols_match_header():
    with open(os.path.join(ROOT, "include", "tree_attn.h")) as fh:
        hdr = fh.read()
    declared = set(re.findall(r"\b(tree_attn_\w+)\s*\(", hdr))
    assert declared == set(_capi.EXPORTED_SYMBOLS)
    L = _capi.lib()
    for name in declared:
        assert hasattr(L, name), name


def _plan_raw(parent, lens, ptr, ids, ps=16, qpl=1, hq=4, h=4, d=128, host_only=1, **opt):
    L = _capi.lib()
    a = [np.ascontiguousarray(np.asarray(x, np.int32)) for x in (parent, lens, ptr, ids)]
    P = [x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) for x in a]
    opts = _capi.PlanOpts(host_only=host_only, **opt)
    hnd = ctypes.c_void_p()
    st = L.tree_attn_plan(P[0], len(a[0]), P[1], P[2], P[3], ps, qpl, hq, h, d,
                          ctypes.byref(opts), ctypes.byref(hnd))
    return st, hnd


@pytest.mark.parametrize("case,status", [
    (dict(parent=[-1, -1]), _capi.TA_EINVAL),               # two roots
    (dict(parent=[1, 0]), _capi.TA_EINVAL),                 # no root / cycle
    (dict(parent=[-1, 1, 1]), _capi.TA_EINVAL),             # self parent
    (dict(parent=[-1, 2, 1]), _capi.TA_EINVAL),             # cycle off the root
    (dict(lens=[4, 0]), _capi.TA_EINVAL),                   # empty node
    (dict(qpl=5), _capi.TA_EINVAL),                         # leaf shorter than qpl
    (dict(hq=6), _capi.TA_EINVAL),                          # n_qheads % n_kvheads
    (dict(d=96), _capi.TA_EUNSUPPORTED),                    # head_dim
    (dict(ptr=[0, 1, 1]), _capi.TA_EINVAL),                 # page CSR size mismatch
    (dict(ids=[0, -3]), _capi.TA_EINVAL),                   # negative page id
    (dict(ps=0), _capi.TA_EINVAL),                          # page size
    (dict(split_align=24), _capi.TA_EINVAL),                # split alignment not a multiple of 16
    (dict(stream_rows=17), _capi.TA_EINVAL),                # a single-wave item holds one 16-row tile
    (dict(waves=-1), _capi.TA_EINVAL),                      # negative option
])
def test_plan_error_codes(case, status):
    kw = dict(parent=[-1, 0], lens=[4, 4], ptr=[0, 1, 2], ids=[0, 1])
    if "parent" in case and len(case["parent"]) == 3:
        kw.update(lens=[4, 4, 4], ptr=[0, 1, 2, 3], ids=[0, 1, 2])
    kw.update(case)
    st, hnd = _plan_raw(**kw)
    assert st == status
    assert not hnd.value
    assert len(_capi.lib().tree_attn_last_error()) > 0


def test_plan_ok_and_info():
    st, hnd = _plan_raw([-1, 0], [4, 4], [0, 1, 2], [0, 1])
    assert st == _capi.TA_OK and hnd.value
    L = _capi.lib()
    nq, ws, ni = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
    assert L.tree_attn_plan_info(hnd, ctypes.byref(nq), ctypes.byref(ws), ctypes.byref(ni)) == 0
    assert nq.value == 1 and ni.value >= 1 and ws.value > 0
    n = ctypes.c_int64()
    assert L.tree_attn_plan_export(hnd, 99, None, ctypes.byref(n)) == _capi.TA_EINVAL
    small = (ctypes.c_int32 * 1)()
    n.value = 1
    assert L.tree_attn_plan_export(hnd, 0, small, ctypes.byref(n)) == _capi.TA_EINVAL
    # decode on a host-only plan is refused without touching the GPU
    kv = _capi.PagedKV()
    assert L.tree_attn_decode(None, 1, ctypes.byref(kv), hnd, None, None) == _capi.TA_EINVAL
    L.tree_attn_plan_destroy(hnd)
    L.tree_attn_plan_destroy(None)


def test_python_wrapper_raises():
    with pytest.raises(TreeAttnError):
        Plan([-1, -1], [4, 4], [0, 1, 2], [0, 1], 16, 1, 4, 4, 128, host_only=True)
    p = Plan([-1, 0], [4, 4], [0, 1, 2], [0, 1], 16, 1, 4, 4, 128, host_only=True)
    with pytest.raises(TreeAttnError):
        p.decode(None, None, None)


def test_kv_append_argument_errors():
    """Argument checks of tree_attn_kv_append run before any HIP call."""
    L = _capi.lib()
    kv = _capi.PagedKV(k=256, v=512, dtype=_capi.TA_BF16, page_size=16, n_pages=4, stride_page=16 * 4 * 128,
                       stride_token=4 * 128, stride_head=128)
    def call(kvp, n=8, h=4, d=128, knew=1024, vnew=2048, dst=4096):
        return L.tree_attn_kv_append(kvp, knew, vnew, n, h, d, dst, None)
    assert call(None) == _capi.TA_EINVAL                                   # no pools
    assert call(ctypes.byref(kv), n=-1) == _capi.TA_EINVAL                 # negative count
    assert call(ctypes.byref(kv), knew=None) == _capi.TA_EINVAL            # missing rows
    assert call(ctypes.byref(kv), d=96) == _capi.TA_EUNSUPPORTED           # head_dim
    assert call(ctypes.byref(kv), h=0) == _capi.TA_EINVAL                  # kv-heads
    assert call(ctypes.byref(kv), knew=1032) == _capi.TA_EINVAL            # misaligned rows
    bad = _capi.PagedKV(k=256, v=512, dtype=_capi.TA_BF16, page_size=16, n_pages=4, stride_page=16 * 4 * 128,
                        stride_token=4 * 128, stride_head=100)
    assert call(ctypes.byref(bad)) == _capi.TA_EINVAL                      # stride not 16-byte
    assert call(ctypes.byref(kv), n=0) == _capi.TA_OK                      # nothing to do


def test_kv_appender_rejects_host_pools():
    """Host tensors never reach the kernel: the binding refuses them before
    any HIP call."""
    import torch
    from tree_structured_shared_amd import kv_appender
    pool = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16)
    rows = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TreeAttnError):
        kv_appender(pool, pool.clone(), rows, rows.clone())


def test_extend_append_argument_errors():
    """tree_attn_plan_extend_append refuses a NULL plan and a host-only plan
    before any HIP call, and leaves the plan as it was."""
    L = _capi.lib()
    kv = _capi.PagedKV(k=256, v=512, dtype=_capi.TA_BF16, page_size=16, n_pages=4, stride_page=16 * 4 * 128,
                       stride_token=4 * 128, stride_head=128)
    add = (ctypes.c_int32 * 1)(1)
    assert L.tree_attn_plan_extend_append(None, add, None, 0, ctypes.byref(kv), 1024, 2048, 1, 4096, None,
                                          None) == _capi.TA_EINVAL
    p = Plan([-1, 0], [4, 4], [0, 1, 2], [0, 1], 16, 1, 4, 4, 128, host_only=True)
    before = p.export("params").copy()
    assert L.tree_attn_plan_extend_append(p._handle, add, None, 0, ctypes.byref(kv), 1024, 2048, 1, 4096, None,
                                          None) == _capi.TA_EINVAL
    assert np.array_equal(p.export("params"), before)
    p.close()
