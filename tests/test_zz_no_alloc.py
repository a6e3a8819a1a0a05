"""GPU: tree_attn_decode_noalloc (partials in the library's static device
scratch, no allocation in the call) against tree_attn_decode (the plan's own
workspace), called through the C ABI. Two calls in a row on the same GPU,
the second on a smaller tree, each checked bit for bit against the plan
workspace's decode of the same inputs and against the fp64 oracle at the
3e-3 bar; a plan whose workspace exceeds the scratch is refused."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import tree_attention as ta
from parity_util import check, log
from tree_structured_shared_amd import Plan, _capi

pytestmark = pytest.mark.gpu


def _decode(fn, plan, q, k, v, out):
    dt = _capi.TA_BF16 if q.dtype == torch.bfloat16 else _capi.TA_F32
    kv = _capi.PagedKV(k=k.data_ptr(), v=v.data_ptr(), dtype=dt, page_size=plan.page_size, n_pages=k.shape[0],
                       stride_page=k.stride(0), stride_token=k.stride(1), stride_head=k.stride(2))
    stream = torch.cuda.current_stream().cuda_stream
    return fn(ctypes.c_void_p(q.data_ptr()), dt, ctypes.byref(kv), plan._handle, ctypes.c_void_p(out.data_ptr()),
              ctypes.c_void_p(stream))


def _case(inst, what, **plan_kw):
    L = _capi.lib()
    q, k, v = inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda()
    plan = Plan.for_instance(inst, poison_workspace=True, **plan_kw)
    ref_out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device="cuda")
    got = torch.empty_like(ref_out)
    assert _decode(L.tree_attn_decode, plan, q, k, v, ref_out) == _capi.TA_OK
    st = _decode(L.tree_attn_decode_noalloc, plan, q, k, v, got)
    assert st == _capi.TA_OK, L.tree_attn_last_error()
    torch.cuda.synchronize()
    log(f"{what}: workspace {plan.workspace_bytes} bytes")
    assert torch.equal(got, ref_out), f"{what}: static-scratch decode differs from the plan-workspace decode"
    check(got.cpu().numpy().astype(np.float64), ta.decode_instance(inst), f"noalloc {what}")
    plan.close()


def test_noalloc_matches_decode_twice_smaller_second():
    big = synth.make_config(5)                      # 28 MB of partials: over half the scratch
    _case(big, "random radix tree")
    small = synth.make_tree([-1, 0, 0, 1], [300, 40, 70, 9], page_size=16, qpl=2, n_qheads=16, n_kvheads=2,
                            head_dim=128, seed=1)
    synth.fill_tensors(small, seed=2)
    _case(small, "small tree after the large one")
    # every edge joined, no split: one slot per query, outputs straight from
    # the partial kernel and no reduction launch
    _case(small, "small tree, one slot per query", force_edges=[1, 1, 1, 1], split=False)


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    # 2,400 queries x 64 q-heads x a few chunks: far more partials than 48 MiB
    n_leaf = 600
    inst = synth.make_tree([-1] + [0] * n_leaf, [9000] + [4] * n_leaf, page_size=16, qpl=4, n_qheads=64,
                           n_kvheads=4, head_dim=128, seed=3)
    synth.fill_tensors(inst, seed=4)
    plan = Plan.for_instance(inst)
    assert plan.workspace_bytes > 48 << 20
    out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device="cuda")
    q, k, v = inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda()
    st = _decode(_capi.lib().tree_attn_decode_noalloc, plan, q, k, v, out)
    assert st == _capi.TA_EINVAL
    assert b"static scratch" in _capi.lib().tree_attn_last_error()
    plan.close()
