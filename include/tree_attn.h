/*
 * tree_attn.h -- C ABI of the MI355X tree-structured decode attention library.
 *
 * What it computes. Every query token sits at a leaf of a decoding tree whose
 * root holds the prompt and whose other nodes hold generated token runs
 * (DeFT reading notes, "decoding tree definition"). A query attends, with one
 * softmax(Q K^T / sqrt(d)) V (FastTree review, section 3, core formula), to the
 * concatenated KV of every node on its root-to-leaf path (DeFT notes, "tree
 * attention definition"). Query j of a leaf with qpl queries is that leaf's
 * token len - qpl + j and sees the leaf's tokens up to itself only; ancestors
 * are fully visible. The result is exact: grouping and splitting change only
 * the order of floating-point summation.
 *
 * How. tree_attn_plan() runs on the host once per tree: the greedy binary edge
 * assignment of the FastTree review (section 3.2, Algorithm 1, with its
 * padding and intermediate-result cost model) turns the tree into KV-guided
 * context-query groups (DeFT notes, "KV-guided tree split"), long groups are
 * cut into KV chunks (FastTree review, section 3.3), and the resulting tables
 * are uploaded once. tree_attn_decode() then enqueues (up to) two HIP kernels on the
 * caller's stream: one partial-attention launch over every (group, row block,
 * KV chunk, kv-head) work item, which streams each chunk's paged KV from HBM
 * once for all the queries of the group, and one log-sum-exp reduction that
 * merges each query's partials along its path (DeFT notes, "tree-topology-aware
 * global reduction"). A query whose path is one partial (one group, one chunk)
 * gets its output from the partial-attention launch directly; when every
 * query is such, the reduction is not enqueued.
 *
 * Conventions (all calls):
 *  - Every call returns a ta_status; on failure tree_attn_last_error() gives a
 *    thread-local message, valid until the next call on the same thread. No
 *    C++ exception and no abort crosses this boundary.
 *  - The caller owns every array it passes; the library copies what it needs
 *    and keeps no caller pointer past the call (except device buffers handed
 *    to tree_attn_decode, which must stay valid until the enqueued work ends).
 *  - Node ids are 0..n_nodes-1 in any order. Leaves are ranked by ascending id.
 *    Query index = leaf_rank * queries_per_leaf + j.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ta_plan ta_plan; /* opaque; owned by the library */

typedef enum {
  TA_OK = 0,
  TA_EINVAL = 1,      /* malformed tree, sizes or arguments */
  TA_ENOMEM = 2,      /* host or device allocation failed */
  TA_EHIP = 3,        /* a HIP runtime call failed */
  TA_EUNSUPPORTED = 4 /* valid, but not supported (head_dim, dtype mix) */
} ta_status;

typedef enum { TA_F32 = 0, TA_BF16 = 1 } ta_dtype;

/* Planner options. Any field left 0 takes its default. */
typedef struct {
  int32_t ts_q;    /* query tile of the padding cost (default 16) */
  int32_t ts_c;    /* context tile of the padding cost (default 64) */
  int32_t gamma;   /* intermediate-result cost per query, in token units (default 128 x n_qheads / n_kvheads) */
  int32_t rb;      /* maximum rows (query x q-head-in-group) per work item (default 128) */
  int32_t waves;   /* target busy waves per CU for the split rule (default 5) */
  int32_t floor_f; /* chunk length floor, in tokens per row (default 4) */
  int32_t ncu;     /* compute units (default: the current device's count; 256 if host_only) */
  int32_t no_split;/* 1 = never cut a group into KV chunks (default 0: split on) */
  const int8_t* force_edges; /* NULL = greedy; else f[v] in {0,1} per node (root ignored) */
  int32_t host_only;         /* 1 = build tables only, no HIP call (plan cannot decode) */
  float scale;               /* softmax scale; 0 = 1/sqrt(head_dim) */
  int32_t poison_workspace;  /* 1 = fill the workspace with NaN before every decode (testing) */
  int32_t stream_rows;       /* groups with at most this many rows (query x q-head-in-group)
                                run as single-wave items, which compute one 16-row tile
                                (1..16, default 16; -1 = none; above 16: TA_EINVAL) */
  int32_t split_align;       /* the split's chunk length is a multiple of this many tokens
                                (a multiple of 16; default 128: four 32-token tiles) */
  int32_t no_tile_join;      /* 1 = groups of 16 or more rows stay single-wave items (when
                                at most stream_rows) even if the plan has workgroup items;
                                default 0: they join the workgroup items */
  int32_t fail_alloc_after;  /* testing: the plan's N-th allocation step fails with
                                TA_ENOMEM as if memory ran out (0 = never). Steps, in order:
                                1 the plan object, 2 the planner state, 3 its tables, then
                                (device plans) 4 the device tables, 5 the workspace; each
                                tree_attn_plan_extend adds one host step first, then its
                                device steps (staging, regrown tables and workspace) */
  int32_t force_staging;     /* testing: in-place table updates of tree_attn_plan_extend always go
                                through the pinned staging buffer, never the kernel arguments */
} ta_plan_opts;

/* Paged K/V pools on the device. Element strides; head_dim is contiguous.
 * Token t of page p, kv-head h starts at base + p*stride_page + t*stride_token
 * + h*stride_head. Default layout [n_pages, page_size, n_kvheads, head_dim]. */
typedef struct {
  const void* k;
  const void* v;
  ta_dtype dtype;
  int32_t page_size;
  int64_t n_pages;      /* pages in each pool; every page id of the plan must be < n_pages */
  int64_t stride_page;
  int64_t stride_token;
  int64_t stride_head;
} ta_paged_kv;

/* Build a plan for one tree (host work; one upload of its tables).
 *  parent[n_nodes]       : parent id, -1 for the single root. Must be acyclic.
 *  node_kv_len[n_nodes]  : tokens per node, >= 1; a leaf has >= queries_per_leaf.
 *  node_page_ptr[n+1], node_page_ids[]: CSR of each node's pages; node v has
 *                          ceil(len/page_size) pages, token t in page t/page_size
 *                          at slot t%page_size. Page ids in [0, 2^23).
 *  page_size             : 1..256.
 *  queries_per_leaf      : >= 1 (the leaf's last tokens are the queries).
 *  n_qheads % n_kvheads == 0; q-head h reads kv-head h / (n_qheads/n_kvheads).
 *  head_dim              : 64 or 128 (else TA_EUNSUPPORTED).
 *  opts                  : NULL for defaults.
 * On success *out_plan owns host tables, device tables and the fp32 partial
 * workspace (size from tree_attn_plan_info). */
ta_status tree_attn_plan(const int32_t* parent, int32_t n_nodes, const int32_t* node_kv_len,
                         const int32_t* node_page_ptr, const int32_t* node_page_ids,
                         int32_t page_size, int32_t queries_per_leaf, int32_t n_qheads,
                         int32_t n_kvheads, int32_t head_dim, const ta_plan_opts* opts,
                         ta_plan** out_plan);

/* Enqueue one decode step on hip_stream (a hipStream_t; NULL = null stream).
 *  q   : device [n_queries, n_qheads, head_dim], contiguous, q_dtype.
 *  kv  : paged pools, dtype must equal q_dtype, page_size must equal the plan's.
 *  out : device [n_queries, n_qheads, head_dim] fp32, contiguous.
 * Asynchronous: returns after enqueueing. One plan serves one decode in
 * flight at a time (its workspace is shared); the plan must outlive the work.
 * TA_EINVAL for null pointers, dtype/page mismatches or page ids >= n_pages,
 * and for a plan left unusable by a failed tree_attn_plan_extend. */
ta_status tree_attn_decode(const void* q, ta_dtype q_dtype, const ta_paged_kv* kv,
                           const ta_plan* plan, float* out, void* hip_stream);

/* tree_attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the partial results in a static device
 * array of 48 MiB (one per GPU, held until the process ends) instead of the
 * plan's workspace. The call allocates nothing. Arguments, layouts and
 * asynchrony as in tree_attn_decode. TA_EINVAL when the plan's partial
 * workspace (tree_attn_plan_info) exceeds 48 MiB. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (two streams, or a
 * second call before the first has run) race; calls in order on one stream
 * do not. Nothing in the array needs clearing: every partial a call reads
 * was written by that call. */
ta_status tree_attn_decode_noalloc(const void* q, ta_dtype q_dtype, const ta_paged_kv* kv,
                                   const ta_plan* plan, float* out, void* hip_stream);

/* Decode-loop update (plan reuse): after a decode step every leaf's new
 * tokens are appended to its KV, and the next step's queries are each leaf's
 * last queries_per_leaf tokens again. Leaf of rank r (ascending node id) grows
 * by leaf_add[r] >= 0 tokens (leaf_add has one entry per leaf); the pages the
 * growth needs, ceil(new_len / page_size) - ceil(old_len / page_size) per
 * leaf, are taken in leaf-rank order from the host array
 * new_pages[n_new_pages] (page ids of the pools, [0, 2^23); their K/V is
 * written by the caller, e.g. with tree_attn_kv_append). The edge assignment and
 * so the context-query grouping are kept (FastTree review, section 3.2: the
 * grouping is a per-tree decision; call tree_attn_plan again to regroup); the
 * length-dependent steps (chunks, work items, slots, page table) are redone,
 * and the exported tables then equal those of tree_attn_plan on the grown
 * tree with force_edges = this plan's edges, except TA_T_PARAMS[16], which is
 * 2 ("kept") where the plan was greedy.
 * Device tables are updated in place, in order on hip_stream: enqueue the
 * following decodes on the same stream. Only when the tables outgrow their
 * allocation (they keep headroom after the first extend) or the page table is
 * laid out afresh does the call wait for the device and upload them whole.
 * *relaunch (may be NULL) is set to 1 when the decode's launch shape or a
 * device address changed: a decode captured in a HIP graph must then be
 * captured again; with 0 the captured graph stays valid. Do not call while a
 * graph capture is in progress on hip_stream. host_only plans update their
 * tables only. All-or-nothing on TA_EINVAL (counts, page ids); a failed
 * update after the plan's tables have moved on (TA_EHIP, TA_ENOMEM) leaves
 * the plan unusable: later extends and decodes return TA_EINVAL, and
 * tree_attn_plan_destroy still frees it. */
ta_status tree_attn_plan_extend(ta_plan* plan, const int32_t* leaf_add, const int32_t* new_pages,
                                int64_t n_new_pages, void* hip_stream, int32_t* relaunch);

/* KV append, the step before a decode (the new tokens' K and V into the
 * paged pools). Token r's rows k_new[r, n_kvheads, head_dim] and
 * v_new[r, n_kvheads, head_dim] (device, contiguous, kv->dtype) are written to
 * page dst[r] >> 8, slot dst[r] & 255 of the pools (dst: device int32
 * [n_tokens], the encoding of TA_T_SEG_TOK). Asynchronous on hip_stream. A
 * destination outside the pools (page >= kv->n_pages, slot >= page_size, or a
 * negative word) is skipped, never written. Two tokens with the same
 * destination race. TA_EINVAL / TA_EUNSUPPORTED for bad sizes, strides or
 * alignment (the rules of tree_attn_decode); n_tokens == 0 does nothing. */
ta_status tree_attn_kv_append(const ta_paged_kv* kv, const void* k_new, const void* v_new, int64_t n_tokens,
                              int32_t n_kvheads, int32_t head_dim, const int32_t* dst, void* hip_stream);

/* One decode-loop step's two device updates in one call (plan reuse, as for
 * tree_attn_plan_extend: FastTree review, section 3.2): the KV append of
 * tree_attn_kv_append(kv, k_new, v_new, n_tokens, the plan's n_kvheads, the
 * plan's head_dim, dst) and the plan growth of tree_attn_plan_extend(plan,
 * leaf_add, new_pages, n_new_pages). When the tables are updated in place
 * (every extend after the first, until they outgrow their headroom) both
 * updates go to hip_stream as ONE kernel launch instead of two; otherwise the
 * append is enqueued after the table upload. Results equal the two calls'.
 * Arguments, ownership and asynchrony as in those calls; kv->page_size must be
 * the plan's. The append's arguments are checked before the plan changes, so
 * TA_EINVAL / TA_EUNSUPPORTED from either part leave pools and plan
 * untouched. host_only plans: TA_EINVAL. n_tokens == 0 extends only. */
ta_status tree_attn_plan_extend_append(ta_plan* plan, const int32_t* leaf_add, const int32_t* new_pages,
                                       int64_t n_new_pages, const ta_paged_kv* kv, const void* k_new,
                                       const void* v_new, int64_t n_tokens, const int32_t* dst, void* hip_stream,
                                       int32_t* relaunch);

/* Plan sizes. Any output pointer may be NULL. The plan owns its scratch (the
 * fp32 partial workspace) and reports its size here: a caller never supplies
 * or keeps scratch buffers whose size the API leaves unstated, one reason the
 * TGI PR "Move to FlashDecoding instead of PagedAttention kernel" gives for
 * passing over another paged-attention library. */
ta_status tree_attn_plan_info(const ta_plan* plan, int32_t* n_queries, int64_t* workspace_bytes,
                              int32_t* n_items);

/* Export one plan table as int32 (table ids below). With dst == NULL only
 * *len (element count) is written; otherwise dst must hold *len elements.
 * The tables are the plan's whole decision (the context-query groups of the
 * FastTree review, section 3.1, the edge assignment of its Algorithm 1, the
 * chunks of section 3.3), exported so that they can be checked against an
 * independent re-derivation bit for bit. They are built once per plan and
 * reused by every decode: in the same TGI PR, building the sequence-length
 * index tensors anew on every call cost enough to make the new path slower
 * than the old one. */
ta_status tree_attn_plan_export(const ta_plan* plan, int32_t table_id, int32_t* dst, int64_t* len);

/* Timing of the last decodes (testing and benchmarking). After
 * tree_attn_timing_enable(plan, capacity) every decode, for up to `capacity`
 * decodes, launches its kernels with HIP start/stop events that the
 * runtime stamps at the start and at the end of each kernel's own execution
 * (not at enqueue); capacity 0 turns timing off. Do not enable timing on a
 * decode that is being captured into a graph.
 * tree_attn_timing_read() waits for the recorded events and writes per-decode
 * milliseconds of the partial-attention kernel (partial_ms[x]) and of the
 * reduction kernel (reduce_ms[x]: 0 for a decode that launched none, every
 * query having one partial); either pointer may be NULL. *n gets the count
 * and the record is cleared. */
ta_status tree_attn_timing_enable(ta_plan* plan, int32_t capacity);
ta_status tree_attn_timing_read(ta_plan* plan, float* partial_ms, float* reduce_ms, int32_t* n);

/* Free a plan (synchronises the device first). NULL is a no-op. */
void tree_attn_plan_destroy(ta_plan* plan);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* tree_attn_last_error(void);

/* Table ids for tree_attn_plan_export (all int32, row-major). */
enum {
  TA_T_PARAMS = 0,        /* [28]: version, n_nodes, n_queries, qpl, n_qheads, n_kvheads,
                             head_dim, page_size, ts_q, ts_c, gamma, rb, waves, floor_f, ncu,
                             split, edges (0 greedy, 1 forced, 2 kept by an extend),
                             chunk_align, n_groups, n_chunks, n_items, n_slots,
                             c_glob, n_runs, stream_rows, n_stream_items, split_align,
                             tile_join */
  TA_T_EDGES = 1,         /* [n_nodes] f(parent -> v), 0 at the root */
  TA_T_NQ = 2,            /* [n_nodes] queries left in v's virtual node */
  TA_T_LCUM = 3,          /* [n_nodes] cumulative context length after merging */
  TA_T_GROUPS = 4,        /* [n_groups x 8] node, top, kv_len, n_q, q_ptr, chunk_ptr, n_chunks,
                             slot_base */
  TA_T_GROUP_QS = 5,      /* [sum n_q] query ids per group, ascending */
  TA_T_GROUP_VIS = 6,     /* [sum n_q] visible segment prefix per group query */
  TA_T_CHUNKS = 7,        /* [n_chunks x 3] group, tok0, tok1 (segment positions) */
  TA_T_ITEMS = 8,         /* [n_items x 5] group, row0, nrows, chunk, class (1 = workgroup
                             item, 0 = single-wave item); launch order, workgroup items first */
  TA_T_Q_SLOT_PTR = 9,    /* [n_queries + 1] */
  TA_T_Q_SLOTS = 10,      /* partial slots of each query, root side first, chunks ascending */
  TA_T_RUNS = 11,         /* [n_runs x 3] page id, first slot, tokens */
  TA_T_CHUNK_RUN_PTR = 12,/* [n_chunks + 1] */
  TA_T_BFS = 13,          /* [n_nodes] BFS order (children by ascending id) */
  TA_T_SEG_TOK = 14,      /* the page table the kernels read: word (page_id << 8) | slot of
                             segment token t of group i at TA_T_GROUP_SEG[i] + t, t < kv_len;
                             the words after it, up to the next group's offset (at least 96),
                             repeat tokens of the same segment (the kernels read ahead) */
  TA_T_GROUP_SEG = 15,    /* [n_groups] offset of each group's segment in TA_T_SEG_TOK */
  TA_T_UPDATE_COUNTS = 16,/* [3] device-table updates so far: in-place in the kernel arguments,
                             in-place through the pinned staging buffer, whole uploads */
  TA_T_DEVICE_TABLES = 17,/* the device copy of the kernels' tables (work items, group queries,
                             visible prefixes, page table, slot tables), read back from the
                             device; the call waits for the device. TA_EINVAL if host_only */
  TA_T_COUNT = 18
};

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
