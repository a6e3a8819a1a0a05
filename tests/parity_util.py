"""Shared helpers of the GPU parity tests: run a plan through the C ABI and
compare with the fp64 oracle at the 3e-3 max-abs bar.

Every check records its max-abs error; with TREE_ATTN_MARGINS=<path> set,
the session writes them all to that JSON file (the margins table)."""
import sys

import numpy as np

TOL = 3e-3
MARGINS = []


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(inst):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return inst.q.cuda(), inst.k_pool.cuda(), inst.v_pool.cuda()


def run(inst, devt=None, **plan_kw):
    """One decode of inst through a fresh plan (workspace poisoned with NaN
    before the decode unless asked otherwise); returns the fp64 output."""
    import torch
    from tree_structured_shared_amd import Plan
    q, k, v = devt if devt is not None else dev(inst)
    plan_kw.setdefault("poison_workspace", True)
    plan = Plan.for_instance(inst, **plan_kw)
    out = plan.decode(q, k, v)
    torch.cuda.synchronize()
    res = out.cpu().numpy().astype(np.float64)
    plan.close()
    return res


def check(got, ref, what, tol=TOL):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = float(np.nanmax(np.abs(got - ref)))
    MARGINS.append({"case": what, "max_abs_err": err, "tol": tol})
    log(f"{what}: max-abs err {err:.3e}")
    assert err <= tol, f"{what}: max-abs err {err:.3e}"
    return err
