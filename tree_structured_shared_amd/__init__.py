"""Tree-structured decode attention for MI355X (gfx950).

A thin binding over the C ABI of ``libtree_attn.so`` (include/tree_attn.h):
argument checks and marshalling only. Planning runs in the library's C++ host
code and every step of the decode runs in its HIP kernels; PyTorch supplies
device memory and the stream.

    plan = Plan(parent, node_kv_len, node_page_ptr, node_page_ids, page_size,
                queries_per_leaf, n_qheads, n_kvheads, head_dim)
    out = plan.decode(q, k_pool, v_pool)      # fp32 [n_queries, n_qheads, head_dim]
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._capi import (TA_BF16, TA_F32, TABLE_COLS, TABLE_IDS, PagedKV, PlanOpts, TreeAttnError,
                    check, lib)

__all__ = ["Plan", "TreeAttnError", "TABLE_IDS", "kv_append", "kv_appender"]


def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _i32_addr(a):
    """(array, address) of a contiguous int32 version of a; no copy (and no
    ctypes object) when a already is one."""
    if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
        a = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    return a, a.__array_interface__["data"][0]


def kv_appender(k_pool, v_pool, k_new, v_new, stream=None):
    """Check the pools and the new-row buffers once and return a callable
    append(dst) that enqueues tree_attn_kv_append for them (for loops that
    append into the same buffers every step): token r's rows k_new[r] /
    v_new[r] ([n_kvheads, head_dim]) go to page dst[r] >> 8, slot dst[r] &
    255; dst is a device int32 [n_tokens] tensor, checked per call.
    Destinations outside the pools are skipped."""
    import torch
    dt = {torch.float32: TA_F32, torch.bfloat16: TA_BF16}.get(k_pool.dtype)
    if dt is None:
        raise TreeAttnError(4, f"unsupported dtype {k_pool.dtype}")
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise TreeAttnError(1, "pools must be [n_pages, page_size, n_kvheads, head_dim] with equal strides")
    if not (k_pool.is_cuda and v_pool.is_cuda) or v_pool.dtype != k_pool.dtype:
        raise TreeAttnError(1, "pools must be device tensors of one dtype")
    n, h, d = k_new.shape[0], k_pool.shape[2], k_pool.shape[3]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (n, h, d) or t.dtype != k_pool.dtype or not t.is_contiguous() or not t.is_cuda:
            raise TreeAttnError(1, f"{name} must be a contiguous device [n_tokens, {h}, {d}] {k_pool.dtype} tensor")
    if k_pool.stride(3) != 1:
        raise TreeAttnError(1, "head_dim must be contiguous in the pools")
    kv = PagedKV(k=k_pool.data_ptr(), v=v_pool.data_ptr(), dtype=dt, page_size=k_pool.shape[1],
                 n_pages=k_pool.shape[0], stride_page=k_pool.stride(0), stride_token=k_pool.stride(1),
                 stride_head=k_pool.stride(2))
    if stream is None:
        stream = torch.cuda.current_stream(k_pool.device).cuda_stream
    fn = lib().tree_attn_kv_append
    head = (ctypes.byref(kv), ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
            int(n), int(h), int(d))
    tail = ctypes.c_void_p(stream)
    keep = (kv, k_pool, v_pool, k_new, v_new)
    i32 = torch.int32

    def append(dst, _fn=fn, _head=head, _tail=tail, _keep=keep):
        if dst.dtype != i32 or dst.shape != (n,) or not dst.is_cuda or not dst.is_contiguous():
            raise TreeAttnError(1, "dst must be a contiguous device int32 [n_tokens] tensor")
        check(_fn(*_head, ctypes.c_void_p(dst.data_ptr()), _tail))

    def fused_args(dst, _kv=kv, _keep=keep):
        # the append's half of tree_attn_plan_extend_append's arguments
        if dst.dtype != i32 or dst.shape != (n,) or not dst.is_cuda or not dst.is_contiguous():
            raise TreeAttnError(1, "dst must be a contiguous device int32 [n_tokens] tensor")
        return (ctypes.byref(_kv), ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()), int(n),
                ctypes.c_void_p(dst.data_ptr()))
    append.fused_args = fused_args
    append.stream = stream
    return append


def kv_append(k_pool, v_pool, k_new, v_new, dst, stream=None):
    """One tree_attn_kv_append (see kv_appender): token r's rows k_new[r] /
    v_new[r] ([n_kvheads, head_dim]) go to page dst[r] >> 8, slot dst[r] &
    255; dst is a device int32 tensor. Destinations outside the pools are
    skipped."""
    kv_appender(k_pool, v_pool, k_new, v_new, stream)(dst)


class Plan:
    """A decode plan for one tree (owns device tables and the partial workspace)."""

    def __init__(self, parent, node_kv_len, node_page_ptr, node_page_ids, page_size,
                 queries_per_leaf, n_qheads, n_kvheads, head_dim, *, force_edges=None,
                 host_only=False, scale=0.0, poison_workspace=False, ts_q=0, ts_c=0, gamma=0,
                 rb=0, waves=0, floor_f=0, ncu=0, split=True, stream_rows=0, split_align=0,
                 tile_join=True, fail_alloc_after=0, force_staging=False):
        L = lib()
        self._handle = ctypes.c_void_p()
        par, par_p = _i32(parent)
        lens, lens_p = _i32(node_kv_len)
        ptr, ptr_p = _i32(node_page_ptr)
        ids, ids_p = _i32(node_page_ids)
        if len(lens) != len(par) or len(ptr) != len(par) + 1:
            raise TreeAttnError(1, "parent / node_kv_len / node_page_ptr sizes disagree")
        if len(ids) < (int(ptr[-1]) if len(ptr) else 0):
            raise TreeAttnError(1, "node_page_ids shorter than node_page_ptr[-1]")
        opts = PlanOpts(ts_q=ts_q, ts_c=ts_c, gamma=gamma, rb=rb, waves=waves, floor_f=floor_f,
                        ncu=ncu, no_split=0 if split else 1, host_only=1 if host_only else 0,
                        scale=float(scale), poison_workspace=1 if poison_workspace else 0,
                        stream_rows=int(stream_rows), split_align=int(split_align),
                        no_tile_join=0 if tile_join else 1, fail_alloc_after=int(fail_alloc_after),
                        force_staging=1 if force_staging else 0)
        self._force = None
        if force_edges is not None:
            fe = np.ascontiguousarray(np.asarray(force_edges), dtype=np.int8)
            if len(fe) != len(par):
                raise TreeAttnError(1, "force_edges must have one entry per node")
            self._force = fe
            opts.force_edges = fe.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))
        check(L.tree_attn_plan(par_p, len(par), lens_p, ptr_p, ids_p, int(page_size),
                               int(queries_per_leaf), int(n_qheads), int(n_kvheads), int(head_dim),
                               ctypes.byref(opts), ctypes.byref(self._handle)))
        self.page_size = int(page_size)
        self.qpl = int(queries_per_leaf)
        self.n_qheads = int(n_qheads)
        self.n_kvheads = int(n_kvheads)
        self.head_dim = int(head_dim)
        self.host_only = bool(host_only)
        self._info()

    def _info(self):
        nq = ctypes.c_int32()
        ws = ctypes.c_int64()
        ni = ctypes.c_int32()
        check(lib().tree_attn_plan_info(self._handle, ctypes.byref(nq), ctypes.byref(ws), ctypes.byref(ni)))
        self.n_queries, self.workspace_bytes, self.n_items = nq.value, ws.value, ni.value

    @classmethod
    def for_instance(cls, inst, **kw):
        return cls(inst.parent, inst.node_len, inst.node_page_ptr, inst.node_page_ids,
                   inst.page_size, inst.qpl, inst.n_qheads, inst.n_kvheads, inst.head_dim, **kw)

    # -- tables ---------------------------------------------------------------
    def export(self, name):
        tid = TABLE_IDS[name] if isinstance(name, str) else int(name)
        n = ctypes.c_int64()
        check(lib().tree_attn_plan_export(self._handle, tid, None, ctypes.byref(n)))
        out = np.zeros(n.value, dtype=np.int32)
        check(lib().tree_attn_plan_export(self._handle, tid,
                                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                          ctypes.byref(n)))
        cols = TABLE_COLS.get(name if isinstance(name, str) else "")
        return out.reshape(-1, cols) if cols else out

    def tables(self):
        """The planner's tables (not the library's update counts or the
        device read-back)."""
        return {k: self.export(k) for k in TABLE_IDS if k not in ("update_counts", "device_tables")}

    # -- decode loop ----------------------------------------------------------
    def extend(self, leaf_add, new_pages=(), stream=None, append=None):
        """Leaf of rank r grows by leaf_add[r] tokens (their K/V already in the
        pools), taking the pages it needs from new_pages in leaf-rank order;
        the grouping is kept (tree_attn_plan_extend). With append=(appender,
        dst), appender from kv_appender, the new tokens' K/V are written in
        the same call (tree_attn_plan_extend_append: one launch for both
        device updates; the appender's stream is used when stream is None).
        Returns True when a captured decode graph must be captured again."""
        n_leaves = self.n_queries // self.qpl
        add, add_a = _i32_addr(leaf_add)
        pages, pages_a = _i32_addr(new_pages)
        if len(add) != n_leaves:
            raise TreeAttnError(1, f"leaf_add must have one entry per leaf ({n_leaves})")
        if stream is None and append is not None:
            stream = append[0].stream
        if stream is None and not self.host_only:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        relaunch = ctypes.c_int32()
        if append is not None:
            appender, dst = append
            check(lib().tree_attn_plan_extend_append(self._handle, add_a, pages_a if len(pages) else None,
                                                     len(pages), *appender.fused_args(dst), stream or None,
                                                     ctypes.byref(relaunch)))
        else:
            check(lib().tree_attn_plan_extend(self._handle, add_a, pages_a if len(pages) else None, len(pages),
                                              stream or None, ctypes.byref(relaunch)))
        if relaunch.value or self.host_only:
            self._info()
        return bool(relaunch.value)

    # -- decode ---------------------------------------------------------------
    def decode(self, q, k_pool, v_pool, out=None, stream=None, noalloc=False):
        """Enqueue one decode step; returns ``out`` (fp32 [n_queries, n_qheads, head_dim]).
        noalloc: tree_attn_decode_noalloc (partials in the library's static
        device scratch instead of the plan's workspace)."""
        call, out = self._prepare(q, k_pool, v_pool, out, stream, noalloc)
        call()
        return out

    def launcher(self, q, k_pool, v_pool, out, stream=None, noalloc=False):
        """Check the tensors once and return a zero-argument callable that
        enqueues tree_attn_decode (or tree_attn_decode_noalloc) with the
        prepared arguments (for loops that decode the same buffers
        repeatedly)."""
        return self._prepare(q, k_pool, v_pool, out, stream, noalloc)[0]

    def _prepare(self, q, k_pool, v_pool, out, stream, noalloc=False):
        import torch
        if self.host_only:
            raise TreeAttnError(1, "plan was built host_only")
        dt = {torch.float32: TA_F32, torch.bfloat16: TA_BF16}.get(q.dtype)
        if dt is None:
            raise TreeAttnError(4, f"unsupported dtype {q.dtype}")
        for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
            if not t.is_cuda:
                raise TreeAttnError(1, f"{name} must be a device tensor")
            if t.dtype != q.dtype:
                raise TreeAttnError(4, f"{name} dtype {t.dtype} differs from q's {q.dtype}")
        if tuple(q.shape) != (self.n_queries, self.n_qheads, self.head_dim) or not q.is_contiguous():
            raise TreeAttnError(1, f"q must be contiguous [{self.n_queries}, {self.n_qheads}, {self.head_dim}]")
        if k_pool.dim() != 4 or tuple(k_pool.shape[1:]) != (self.page_size, self.n_kvheads, self.head_dim):
            raise TreeAttnError(1, "k_pool must be [n_pages, page_size, n_kvheads, head_dim]")
        if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
            raise TreeAttnError(1, "k_pool and v_pool must have the same shape and strides")
        if k_pool.stride(3) != 1:
            raise TreeAttnError(1, "head_dim must be contiguous in the pools")
        if out is None:
            out = torch.empty((self.n_queries, self.n_qheads, self.head_dim), dtype=torch.float32,
                              device=q.device)
        elif (out.dtype != torch.float32 or not out.is_contiguous()
              or tuple(out.shape) != (self.n_queries, self.n_qheads, self.head_dim)):
            raise TreeAttnError(1, "out must be contiguous fp32 [n_queries, n_qheads, head_dim]")
        kv = PagedKV(k=k_pool.data_ptr(), v=v_pool.data_ptr(), dtype=dt, page_size=self.page_size,
                     n_pages=k_pool.shape[0], stride_page=k_pool.stride(0),
                     stride_token=k_pool.stride(1), stride_head=k_pool.stride(2))
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        fn = lib().tree_attn_decode_noalloc if noalloc else lib().tree_attn_decode
        args = (ctypes.c_void_p(q.data_ptr()), dt, ctypes.byref(kv), self._handle,
                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
        keep = (kv, q, k_pool, v_pool, out)

        def call(_fn=fn, _args=args, _keep=keep):
            check(_fn(*_args))
        return call, out

    # -- timing ---------------------------------------------------------------
    def timing_enable(self, capacity):
        check(lib().tree_attn_timing_enable(self._handle, int(capacity)))

    def timing_read(self, capacity):
        """Per-decode kernel milliseconds (partial, reduce), each kernel timed
        from its own start to its own end."""
        pm = (ctypes.c_float * max(1, capacity))()
        rm = (ctypes.c_float * max(1, capacity))()
        n = ctypes.c_int32()
        check(lib().tree_attn_timing_read(self._handle, pm, rm, ctypes.byref(n)))
        return np.array(pm[:n.value]), np.array(rm[:n.value])

    def close(self):
        if getattr(self, "_handle", None) and self._handle.value:
            lib().tree_attn_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
