"""Host logic of bench.py (no GPU): the pool layout it times, the streamed-bytes
count, the HBM-traffic record lookup and the one-GPU guard."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import torch

import synth
from tree_structured_shared_amd import Plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_head_major_pool_is_the_same_tensor_in_head_major_storage():
    b = _bench()
    pool = torch.randn(5, 16, 3, 8)
    hm = b.head_major_pool(pool, "cpu")
    assert hm.shape == pool.shape and torch.equal(hm, pool)
    # storage [n_pages, n_kvheads, page_size, head_dim]: head_dim contiguous, then tokens, then heads
    assert hm.stride() == (3 * 16 * 8, 8, 16 * 8, 1)


def test_streamed_bytes_count_each_row_block_once_per_chunk():
    b = _bench()
    # a 300-token root shared by 2 leaves x 2 queries x GQA 64 = 256 rows: two 128-row
    # blocks, each streaming the root; each leaf group (128 rows) streams its own tokens once
    inst = synth.make_tree([-1, 0, 0], [300, 40, 50], page_size=16, qpl=2, n_qheads=64, n_kvheads=1,
                           head_dim=128, seed=3)
    # (a small intermediate-result cost keeps both edges split at this GQA)
    plan = Plan.for_instance(inst, host_only=True, split=False, gamma=32)
    assert not plan.export("edges").any()
    assert b.streamed_kv_bytes(plan, inst) == (2 * 300 + 40 + 50) * 1 * 128 * 2 * 2
    plan.close()


def test_traffic_record_only_for_its_sources_and_workload():
    b = _bench()
    with open(b.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert b._traffic("no_such_workload") is None
    assert rec["workloads"]
    for name, w in rec["workloads"].items():
        got = b._traffic(name)
        if rec["source_sha256"] != b.source_hash():
            assert got is None
        else:
            cal = rec["copy_calibration"]
            want = (w["fetch_size_kib"] * cal["bytes"] / cal["fetch_size_kib"]
                    + w["write_size_kib"] * cal["bytes"] / cal["write_size_kib"])
            assert abs(got - want) <= 1


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_algorithmic_flops_closed_form_and_oracle_counts():
    """4 d flops per visible token and q-head (QK^T and PV): a hand count on a
    chain, and on a random tree the oracle's own visible-token counts (the
    lengths of its softmax weight vectors)."""
    from oracle import tree_attention as ta
    b = _bench()
    # chain root 10 -> leaf 5, two queries per leaf: they see 10 + 4 and 10 + 5 tokens
    inst = synth.make_tree([-1, 0], [10, 5], page_size=4, qpl=2, n_qheads=2, n_kvheads=1, head_dim=8, seed=1)
    assert b.algorithmic_flops(inst) == (14 + 15) * 2 * 4 * 8
    inst = synth.make_tree([-1, 0, 0, 1, 1, 2], [20, 7, 9, 4, 6, 3], page_size=4, qpl=3, n_qheads=4, n_kvheads=2,
                           head_dim=16, dtype=torch.float32, seed=5)
    synth.fill_tensors(inst, seed=6)
    _, w = ta.decode_instance(inst, return_weights=True)
    visible = sum(len(p) for p in w.values())
    assert b.algorithmic_flops(inst) == visible * 4 * 16
