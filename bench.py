"""Benchmark: tree-structured decode attention, one decode step of one layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--extra-configs 2,3,4]

A step is one tree_attn_decode (partial-attention kernel + log-sum-exp
reduction) over the whole tree. The headline workload is the largest one, the
irregular random radix tree (root + 4 levels, branching U{1..8}, lognormal
node lengths, 4 query tokens per leaf under a leaf-local causal mask, 32
q-heads / 8 kv-heads, head_dim 128, bf16, page size 16: 0.31 GB of unique
K/V). The same run times the other bf16 workloads (multi-level shared
prompt, wide fan-out, skewed long context) with the same steps and reports
them under "configs". Every workload's inputs, plan and pools are prepared
first; the other workloads are then timed, and the headline right after them,
so that no idle spell (input generation, planning) lies between the device's
work and the headline's W warm-up and K timed steps. A device that has been
idle for a second runs its first steps several per cent slower whatever it
runs (its clocks ramp up again); the headline's steps after such an idle spell
are reported as "post_idle", beside the figures and never in place of them.

The KV pool is replicated into enough copies (>= 1 GiB together) that each
timed step reads a copy no cache level holds from the step before: the 256 MB
Infinity Cache would otherwise serve a whole tree. Inputs are resident in
HBM before the timed region. Prints one JSON line.
"""
import argparse
import gc
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X
METRIC = "tree-decode attn: µs/step + effective HBM GB/s (unique KV bytes) vs peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_kernel_traffic.json")


def source_hash():
    """sha256 over the sources that decide what the partial kernel moves:
    the kernels and the planner that cuts their work. The HBM counters
    recorded under profiles/ hold only for the sources they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_structured_shared_amd", "csrc")
    for name in ("kernels.hip", "kernels.h", "planner.cpp", "planner.h"):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic(workload):
    """HBM bytes per partial-kernel launch from the recorded FETCH_SIZE /
    WRITE_SIZE counters of this workload, each scaled by what the counter
    reads for a plain copy of known size; None when the record was taken on
    other sources or holds no such workload."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if rec.get("source_sha256") != source_hash() or w is None:
        return None
    cal = rec["copy_calibration"]
    f_scale = cal["bytes"] / (cal["fetch_size_kib"] * 1024.0)
    w_scale = cal["bytes"] / (cal["write_size_kib"] * 1024.0)
    return round(w["fetch_size_kib"] * 1024.0 * f_scale + w["write_size_kib"] * 1024.0 * w_scale)


def _copy_calibration(mib):
    """A plain device copy of known size, for scaling the HBM counters."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def _cpu_baseline(inst, budget_s=20.0, max_reps=20):
    """The fp64 oracle, untuned, on the host cores: whole decode steps of the
    same workload, repeated until ~budget_s of CPU work."""
    from oracle import tree_attention as oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:
        cores = 1
    times = []
    t_all = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_all) < budget_s:
        t0 = time.perf_counter()
        oracle.decode_instance(inst)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {
        "value": round(inst.unique_kv_bytes / med / 1e9, 4),
        "unit": "GB/s",
        "us_per_step": round(med * 1e6, 1),
        "cores": int(cores),
        "cpu": cpu,
        "kind": "oracle",
        "sample": f"{len(times)} full decode steps of the same tree (all {inst.n_queries} queries, "
                  f"fp64 numpy), median",
    }


def head_major_pool(pool, dev):
    """A device copy of a [n_pages, page_size, H, d] pool stored head-major,
    [n_pages, H, page_size, d] (one kv-head's page is one contiguous run),
    returned as a [n_pages, page_size, H, d] view: the layout the library is
    timed on (the C ABI takes any pool strides with head_dim contiguous)."""
    return pool.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)


def algorithmic_flops(inst):
    """Flops one decode step must do: every query's q-heads against every
    token it sees, QK^T and PV at 2 flops per multiply-add each (4 d per
    visible token and q-head). A leaf's last qpl tokens are its queries;
    query j sees its ancestors' tokens and the leaf's first L - qpl + 1 + j."""
    parent = [int(x) for x in inst.parent]
    lens = [int(x) for x in inst.node_len]
    n = len(parent)
    has_child = [False] * n
    for v in range(n):
        if parent[v] >= 0:
            has_child[parent[v]] = True
    total = 0
    for v in range(n):
        if has_child[v]:
            continue
        path, u = 0, parent[v]
        while u >= 0:
            path += lens[u]
            u = parent[u]
        for j in range(inst.qpl):
            total += path + lens[v] - inst.qpl + 1 + j
    return total * inst.n_qheads * 4 * inst.head_dim


def streamed_kv_bytes(plan, inst):
    """K/V bytes a plan's items stream: every item reads its chunk once per
    kv-head (a group with several row blocks streams its chunks once per
    block)."""
    items, chunks = plan.export("items"), plan.export("chunks")
    esize = 2 if str(inst.dtype).endswith("bfloat16") else 4
    toks = int((chunks[items[:, 3], 2] - chunks[items[:, 3], 1]).sum())
    return toks * inst.n_kvheads * inst.head_dim * 2 * esize


def _ablation(args, inst, q, ks, vs, dev):
    """The same kernels on the plan variants the pages compare: the greedy
    edge assignment (FastTree), every edge 0 (one group per node: DeFT's
    KV-guided grouping), every edge 1 (each leaf's queries stream their whole
    path: query-separated decode), and greedy without the long-context split.
    Each variant: wall time per step over the rotated KV copies."""
    import numpy as np
    import torch
    from tree_structured_shared_amd import Plan
    n = inst.n_nodes
    variants = [("greedy", {}), ("all_0_kv_guided", dict(force_edges=[0] * n)),
                ("all_1_query_separated", dict(force_edges=[1] * n)), ("greedy_no_split", dict(split=False))]
    out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    ref = None
    for name, kw in variants:
        plan = Plan.for_instance(inst, **kw)
        calls = [plan.launcher(q, ks[c], vs[c], out, stream.cuda_stream) for c in range(len(ks))]
        for s in range(args.warmup):
            calls[s % len(ks)]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            calls[s % len(ks)]()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / args.steps
        got = out.clone()
        if ref is None:
            ref = got
        P = plan.export("params")
        res[name] = {"us_per_step": round(us, 2),
                     "effective_GBs": round(inst.unique_kv_bytes / us / 1e3, 1),
                     "kv_bytes_streamed": streamed_kv_bytes(plan, inst),
                     "groups": int(P[18]), "items": int(P[20]), "slots": int(P[21]),
                     "edges_joined": int(plan.export("edges").sum()),
                     "max_abs_diff_vs_greedy": float((got - ref).abs().max())}
        plan.close()
    base = res["greedy"]["us_per_step"]
    for name in res:
        res[name]["speedup_of_greedy"] = round(res[name]["us_per_step"] / base, 3)
    print(json.dumps({"ablation": inst.name, "steps": args.steps, "unique_kv_bytes": inst.unique_kv_bytes,
                      "variants": res}), flush=True)


def _speculative(args, base, dev):
    """The headline tree as a speculative-decoding verification step: the
    last Q tokens of every leaf are queries (Q draft tokens per branch under
    the leaf-local causal mask), with the same tree, heads and layout; timed
    like the headline (same steps and warm-up) beside the headline's own
    queries per leaf. Each leaf must hold at least Q tokens."""
    import numpy as np

    import synth
    res = {}
    for qpl in dict.fromkeys((base.qpl, args.speculative)):
        if qpl != base.qpl:
            has_child = np.zeros(base.n_nodes, bool)
            has_child[base.parent[base.parent >= 0]] = True
            shortest = int(base.node_len[~has_child].min())
            if shortest < qpl:
                raise SystemExit(f"--speculative {qpl}: the shortest leaf holds {shortest} tokens")
            inst = synth.make_tree(base.parent, base.node_len, page_size=base.page_size, qpl=qpl,
                                   n_qheads=base.n_qheads, n_kvheads=base.n_kvheads, head_dim=base.head_dim,
                                   dtype=base.dtype, seed=synth.TREE_SEED_BASE + args.config,
                                   name=f"{base.name}_qpl{qpl}")
            synth.fill_tensors(inst, synth.TENSOR_SEED_BASE + args.config)
        else:
            inst = base
        w = _prepare(inst, _copies(inst, args.copies), dev)
        us, part, red, _, _ = _measure(inst, w["plan"], w["calls"], args.steps, args.warmup)
        r = dict(_workload_desc(inst, w["copies"]), **_rates(inst, us, part, red))
        r["query_tokens_per_s"] = round(inst.n_queries / (us * 1e-6), 1)
        r["plan"] = _plan_info(w["plan"], inst)
        w["plan"].close()
        w.clear()
        res[f"qpl_{qpl}"] = r
    print(json.dumps({"speculative": base.name, "steps": args.steps, "warmup": args.warmup, "variants": res}),
          flush=True)


def _decode_loop(args, inst, dev):
    """Decode-loop plan reuse: W + K steps in which every leaf gains its
    queries' worth of tokens (tree_attn_plan_extend, pages handed out from
    spare pool pages) followed by one decode on the same stream, no host
    synchronisation in between. Reports wall time per step, host time per
    extend, the same decodes without growth, and the host time of planning
    the grown tree from scratch (what each step would cost without reuse).
    Each step first writes the new tokens' K/V into the pools with
    tree_attn_kv_append (a prepared appender; fixed rows: this mode times, it
    does not check); the same loop is also timed, from a fresh plan and
    fresh pools, with tree_attn_plan_extend_append (append and table update
    in one launch). Extend host times are those of the separate calls."""
    import numpy as np
    import torch
    from tree_structured_shared_amd import Plan, kv_appender
    K, W = args.steps, args.warmup
    ps, qpl = inst.page_size, inst.qpl
    has_child = np.zeros(inst.n_nodes, bool)
    has_child[inst.parent[inst.parent >= 0]] = True
    leaves = np.flatnonzero(~has_child)
    lens = inst.node_len.astype(np.int64).copy()
    node_pages = [list(inst.node_page_ids[inst.node_page_ptr[v]:inst.node_page_ptr[v + 1]]) for v in leaves]
    next_page, sched, dsts = inst.n_pages, [], []
    for _ in range(W + K):
        pages, locs = [], []
        for x, v in enumerate(leaves):
            grow = -(-(lens[v] + qpl) // ps) - (-(-lens[v] // ps))
            fresh = list(range(next_page, next_page + grow))
            pages += fresh
            node_pages[x] += fresh
            next_page += grow
            for t in range(int(lens[v]), int(lens[v]) + qpl):
                locs.append((int(node_pages[x][t // ps]) << 8) | (t % ps))
            lens[v] += qpl
        sched.append(np.asarray(pages, np.int32))
        dsts.append(torch.tensor(locs, dtype=torch.int32, device=dev))
    shape = (next_page,) + tuple(inst.k_pool.shape[1:])
    q = inst.q.to(dev)
    out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device=dev)
    new_rows = len(leaves) * qpl
    k_new = torch.randn((new_rows, inst.n_kvheads, inst.head_dim), device=dev).to(inst.dtype)
    v_new = torch.randn((new_rows, inst.n_kvheads, inst.head_dim), device=dev).to(inst.dtype)
    stream = torch.cuda.current_stream(dev).cuda_stream
    add = np.full(len(leaves), qpl, np.int32)

    def loop(fused):
        # W + K steps from the original tree: fresh pools and plan
        k = torch.zeros(shape, dtype=inst.dtype, device=dev)
        v = torch.zeros(shape, dtype=inst.dtype, device=dev)
        k[:inst.n_pages].copy_(inst.k_pool)
        v[:inst.n_pages].copy_(inst.v_pool)
        plan = Plan.for_instance(inst)
        call = plan.launcher(q, k, v, out, stream)
        append = kv_appender(k, v, k_new, v_new, stream)

        def step(s):
            if fused:
                return int(plan.extend(add, sched[s], stream, append=(append, dsts[s])))
            append(dsts[s])
            return int(plan.extend(add, sched[s], stream))
        for s in range(W):
            step(s)
            call()
        torch.cuda.synchronize()
        t_ext, relaunches = [], 0
        gc.disable()
        t0 = time.perf_counter()
        for s in range(W, W + K):
            a = time.perf_counter()
            relaunches += step(s)
            t_ext.append(time.perf_counter() - a)
            call()
        torch.cuda.synchronize()
        loop_us = (time.perf_counter() - t0) * 1e6 / K
        gc.enable()
        return loop_us, t_ext, relaunches, plan, call

    fused = loop(True)
    fused_us = fused[0]
    fused[3].close()
    del fused
    loop_us, t_ext, relaunches, plan, call = loop(False)
    gc.disable()
    t0 = time.perf_counter()
    for s in range(K):
        call()
    torch.cuda.synchronize()
    static_us = (time.perf_counter() - t0) * 1e6 / K
    gc.enable()
    import dataclasses
    g_inst = dataclasses.replace(inst, node_len=lens.astype(np.int32), q=None, k_pool=None, v_pool=None)
    ptr = np.zeros(inst.n_nodes + 1, np.int32)
    ptr[1:] = np.cumsum(-(-lens // ps))
    g_inst.node_page_ptr = ptr
    g_inst.node_page_ids = np.arange(int(ptr[-1]), dtype=np.int32)
    t_fresh = []
    for _ in range(20):
        a = time.perf_counter()
        Plan.for_instance(g_inst, host_only=True).close()
        t_fresh.append(time.perf_counter() - a)
    P = plan.export("params")
    print(json.dumps({"decode_loop": inst.name, "steps": K, "warmup": W, "tokens_per_leaf_per_step": qpl,
                      "us_per_step_append_extend_decode": round(loop_us, 2),
                      "us_per_step_fused_append_extend_decode": round(fused_us, 2),
                      "us_per_step_no_growth": round(static_us, 2),
                      "extend_host_us_median": round(statistics.median(t_ext) * 1e6, 2),
                      "extend_host_us_p90": round(sorted(t_ext)[int(0.9 * (len(t_ext) - 1))] * 1e6, 2),
                      "extend_host_us_max": round(max(t_ext) * 1e6, 2),
                      "extends_needing_relaunch": relaunches,
                      "fresh_plan_host_us_median": round(statistics.median(t_fresh) * 1e6, 2),
                      "final_plan": {"items": int(P[20]), "slots": int(P[21]), "tokens": int(lens.sum())},
                      "kv_cache": "warm (one pool, no rotation)"}), flush=True)
    plan.close()


def _pools(inst, dev, copies):
    q = inst.q.to(dev)
    ks = [head_major_pool(inst.k_pool, dev) for _ in range(copies)]
    vs = [head_major_pool(inst.v_pool, dev) for _ in range(copies)]
    return q, ks, vs


def _copies(inst, requested):
    import torch
    esize = 2 if inst.dtype == torch.bfloat16 else 4
    pool_bytes = 2 * inst.k_pool.numel() * esize
    return requested or max(2, math.ceil((1 << 30) / pool_bytes) + 1)


def _measure(inst, plan, calls, K, W):
    """Wall time per step over K back-to-back steps (after W warm-up steps),
    then the same K steps with the library's per-kernel events."""
    import numpy as np
    import torch
    copies = len(calls)
    for s in range(W):
        calls[s % copies]()
    torch.cuda.synchronize()
    # timed region: K back-to-back decode steps, each on its own KV copy
    # (no collector pauses inside it)
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        calls[s % copies]()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    # per-kernel device time: the library launches each kernel with HIP
    # start/stop events stamped at that kernel's own start and end, on the
    # stream it runs on
    plan.timing_enable(K)
    for s in range(K):
        calls[s % copies]()
    torch.cuda.synchronize()
    pm, rm = plan.timing_read(K)
    plan.timing_enable(0)
    return wall * 1e6 / K, float(np.mean(pm)) * 1e3, float(np.mean(rm)) * 1e3, pm, rm


def _sustained(inst, plan, calls, settle=200, n=300):
    """The same workload once the device has been busy for a while: `settle`
    untimed steps, then `n` timed steps (wall and per-kernel events). The
    first ~100 steps after an idle spell run a few per cent slower (the clock
    ramp), which a short run's K steps fall into; this is reported beside the
    contract's figures, never in place of them."""
    import numpy as np
    import torch
    copies = len(calls)
    for s in range(settle):
        calls[s % copies]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(n):
        calls[s % copies]()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / n
    plan.timing_enable(n)
    for s in range(n):
        calls[s % copies]()
    torch.cuda.synchronize()
    pm, rm = plan.timing_read(n)
    plan.timing_enable(0)
    part, red = float(np.mean(pm)) * 1e3, float(np.mean(rm)) * 1e3
    return {"settle_steps": settle, "steps": n, "us_per_step": round(us, 2),
            "effective_GBs": round(inst.unique_kv_bytes / (us * 1e-6) / 1e9, 2),
            "frac_of_peak": round(inst.unique_kv_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels_us": {"partial_attn": round(part, 3), "lse_reduce": round(red, 3)},
            "partial_frac_of_peak": round(inst.unique_kv_bytes / (part * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def _rates(inst, us_step, part_us, red_us):
    """The metric's figures for one workload: effective GB/s over unique K/V
    bytes per step, the dominant kernel's roofline and the MFMA rate."""
    import torch
    unique = inst.unique_kv_bytes
    bf16 = inst.dtype == torch.bfloat16
    dominant = f"partial_kernel<{'bf16' if bf16 else 'f32'},{inst.head_dim}>"
    flops = algorithmic_flops(inst)
    achieved = unique / (part_us * 1e-6) / 1e9
    value = unique / (us_step * 1e-6) / 1e9
    return {
        "us_per_step": round(us_step, 2),
        "effective_GBs": round(value, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "kernels_us": {"partial_attn": round(part_us, 3), "lse_reduce": round(red_us, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic(inst.name), "traffic_unit": "bytes per launch",
                     "kernel": dominant, "kernel_us": round(part_us, 3),
                     "alg_bytes": unique},
        "mfma": {"alg_flops": flops, "achieved_tflops": round(flops / (part_us * 1e-6) / 1e12, 1),
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS if bf16 else None,
                 "frac": (round(flops / (part_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4) if bf16 else None),
                 "kernel": dominant},
    }


def _plan_info(plan, inst):
    P = plan.export("params")
    return {"groups": int(P[18]), "chunks": int(P[19]), "items": int(P[20]), "slots": int(P[21]),
            "units": int(P[20]) * inst.n_kvheads, "edges_joined": int(plan.export("edges").sum())}


def _workload_desc(inst, copies):
    return {"workload": inst.name, "n_nodes": inst.n_nodes, "n_queries": inst.n_queries,
            "queries_per_leaf": inst.qpl, "n_qheads": inst.n_qheads, "n_kvheads": inst.n_kvheads,
            "head_dim": inst.head_dim, "page_size": inst.page_size, "unique_kv_bytes": inst.unique_kv_bytes,
            "kv_copies_rotated": copies}


def _prepare(inst, copies, dev):
    """A workload's plan, KV pool copies, output and one launcher per copy."""
    import torch

    from tree_structured_shared_amd import Plan
    q, ks, vs = _pools(inst, dev, copies)
    plan = Plan.for_instance(inst)
    out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    calls = [plan.launcher(q, ks[c], vs[c], out, stream.cuda_stream) for c in range(copies)]
    return {"inst": inst, "copies": copies, "plan": plan, "calls": calls, "bufs": [q, ks, vs, out]}


def _extra_config(w, args):
    """One more (prepared) workload, timed like the headline (same steps and
    warm-up). Its plan and pools stay allocated: freeing device memory right
    before the headline's steps would slow their first ones."""
    inst, plan, calls = w["inst"], w["plan"], w["calls"]
    us, part, red, _, _ = _measure(inst, plan, calls, args.steps, args.warmup)
    res = dict(_workload_desc(inst, w["copies"]), **_rates(inst, us, part, red))
    res["sustained"] = _sustained(inst, plan, calls)
    res["plan"] = _plan_info(plan, inst)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--extra-configs", default="2,3,4",
                    help="comma-separated workloads timed before the headline one ('' for none)")
    ap.add_argument("--post-idle-s", type=float, default=1.5,
                    help="idle time before the post_idle measurement of the headline (0: none)")
    ap.add_argument("--copies", type=int, default=0, help="KV pool copies (0 = enough for 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB on the device three times (counter calibration)")
    ap.add_argument("--ablation", action="store_true",
                    help="time the plan variants (greedy / all-0 / all-1 / no split) instead")
    ap.add_argument("--decode-loop", action="store_true",
                    help="time decode steps with plan reuse (every leaf grows each step) instead")
    ap.add_argument("--speculative", type=int, default=0, metavar="Q",
                    help="time the workload's tree with Q query tokens per leaf (a speculative verification "
                         "step) beside its own queries per leaf, instead")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the method runs one layer's decode on one device "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        _copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import synth
    from tree_structured_shared_amd import Plan

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inst = synth.make_config(args.config)
    copies = _copies(inst, args.copies)

    if args.decode_loop:
        _decode_loop(args, inst, dev)
        return

    if args.speculative:
        _speculative(args, inst, dev)
        return

    if args.ablation:
        q, ks, vs = _pools(inst, dev, copies)
        _ablation(args, inst, q, ks, vs, dev)
        return

    # planner host time (tables only, then the full plan with its one upload)
    t_host = []
    for _ in range(20):
        t0 = time.perf_counter()
        Plan.for_instance(inst, host_only=True).close()
        t_host.append(time.perf_counter() - t0)
    t0 = time.perf_counter()
    plan = Plan.for_instance(inst)
    t_plan_full = time.perf_counter() - t0

    q, ks, vs = _pools(inst, dev, copies)
    out = torch.empty((inst.n_queries, inst.n_qheads, inst.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    calls = [plan.launcher(q, ks[c], vs[c], out, stream.cuda_stream) for c in range(copies)]
    K = args.steps

    # the other workloads, prepared now and timed back to back, the headline
    # right after them
    extra = [int(x) for x in args.extra_configs.split(",") if x.strip()] if args.extra_configs else []
    extra = [k for k in dict.fromkeys(extra) if k != args.config]
    prepared = [_prepare(inst_k, _copies(inst_k, args.copies), dev)
                for inst_k in (synth.make_config(k) for k in extra)]
    extra_res = {}
    for w in prepared:
        r = _extra_config(w, args)
        extra_res[r["workload"]] = r

    us_step, part_us, red_us, pm, rm = _measure(inst, plan, calls, K, args.warmup)
    ref_out = out.clone()
    sustained = _sustained(inst, plan, calls)

    # warm reference: the same copy every step (Infinity Cache may hold it)
    plan.timing_enable(K)
    for s in range(K):
        calls[0]()
    torch.cuda.synchronize()
    pm_w, rm_w = plan.timing_read(K)
    plan.timing_enable(0)

    # the same K steps captured once in a HIP graph (no host launch cost per step)
    graph_us = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gcalls = [plan.launcher(q, ks[c], vs[c], out, side.cuda_stream) for c in range(copies)]
            gcalls[0]()
            side.synchronize()
            with torch.cuda.graph(g, stream=side):
                for s in range(K):
                    gcalls[s % copies]()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref_out):
                raise RuntimeError("graph replay output differs from the eager output")
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) * 1e6 / K
        del g, gcalls
    except Exception as exc:  # reported, never silently folded into value
        graph_us = f"unavailable: {exc}"

    # the same K steps on pools in the token-major layout [n_pages, page_size, H, d]
    # (for comparison only; value is the head-major pools' rate)
    tk = [inst.k_pool.to(dev) for _ in range(copies)]
    tv = [inst.v_pool.to(dev) for _ in range(copies)]
    tcalls = [plan.launcher(q, tk[c], tv[c], out, stream.cuda_stream) for c in range(copies)]
    for s in range(args.warmup):
        tcalls[s % copies]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        tcalls[s % copies]()
    torch.cuda.synchronize()
    token_major_us = (time.perf_counter() - t0) * 1e6 / K
    if not torch.allclose(out, ref_out, rtol=0.0, atol=1e-5):
        raise RuntimeError("token-major pools give a different output")
    # the same W + K steps after an idle spell: the device's clocks ramp up
    # again over its first tens of milliseconds of work (beside the figures,
    # never in place of them)
    post_idle = None
    if args.post_idle_s > 0:
        torch.cuda.synchronize()
        time.sleep(args.post_idle_s)
        pi_us, pi_part, pi_red, _, _ = _measure(inst, plan, calls, K, args.warmup)
        if not torch.equal(out, ref_out):
            raise RuntimeError("the post-idle steps give a different output")
        pi = _rates(inst, pi_us, pi_part, pi_red)
        post_idle = {"idle_s": args.post_idle_s, "warmup": args.warmup, "steps": K,
                     "us_per_step": pi["us_per_step"], "effective_GBs": pi["effective_GBs"],
                     "frac_of_peak": pi["frac_of_peak"], "kernels_us": pi["kernels_us"],
                     "partial_frac_of_peak": pi["roofline"]["frac"]}
    plan_desc = _plan_info(plan, inst)
    plan.close()
    for w in prepared:
        w["plan"].close()
        w.clear()
    del prepared
    del tcalls, tk, tv, calls, ks, vs
    gc.collect()
    torch.cuda.empty_cache()

    rates = _rates(inst, us_step, part_us, red_us)
    value = rates["effective_GBs"]
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us_step * 1e-3, 5),
        "us_per_step": rates["us_per_step"],
        "frac_of_peak": rates["frac_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inst.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": dict(_workload_desc(inst, copies),
                       pool_layout="head-major pages: storage [n_pages, n_kvheads, page_size, head_dim]",
                       plan=plan_desc),
        "kernels_us": dict(rates["kernels_us"], device_step=round(float(np.mean(pm + rm)) * 1e3, 3),
                           partial_attn_warm=round(float(np.mean(pm_w)) * 1e3, 3),
                           lse_reduce_warm=round(float(np.mean(rm_w)) * 1e3, 3)),
        "roofline": rates["roofline"],
        "mfma": rates["mfma"],
        "sustained": sustained,
        "graph_us_per_step": round(graph_us, 3) if isinstance(graph_us, float) else graph_us,
        "token_major_pool_us_per_step": round(token_major_us, 2),
        "planner_host_ms": {"tables_median": round(statistics.median(t_host) * 1e3, 3),
                            "with_upload": round(t_plan_full * 1e3, 3)},
    }
    if extra_res:
        res["configs"] = extra_res
    res["measurement_order"] = list(extra_res) + [inst.name]
    if args.post_idle_s > 0:
        res["post_idle"] = post_idle
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline(inst)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
