// Host planner: tree -> KV-guided context-query groups -> KV chunks -> work
// items, slots and page runs. Pure C++ (no HIP), so it also runs host-only.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace ta {

struct PlanParams {
  // gamma 0: kGammaPerGroupHead * (n_qheads / n_kvheads), resolved by plan_init
  int32_t ts_q = 16, ts_c = 64, gamma = 0, rb = 128, waves = 5, floor_f = 4, ncu = 256;
  int32_t split_align = 128;  // chunk lengths of the split are multiples of this
  int32_t split = 1;
  int32_t stream_rows = 16;  // groups with at most this many rows run as one-wave items
  int32_t tile_join = 1;     // ... except groups of a full 16-row tile when the plan has workgroup items
  const int8_t* force_edges = nullptr;
};

constexpr int32_t kFormatVersion = 4;
// Default intermediate-result cost per query (greedy edge assignment), in the
// cost model's query-token units, per q-head of a kv-head's group: a query's
// partials are g rows of d fp32 values written and read back (8 g d bytes per
// kv-head) against d / 4 bytes per query-token of K/V streamed once for a
// 16-query tile, i.e. 32 g; measured on MI355X, a partial costs about four
// times its bytes (the reduction's second pass and its launch), so 128 g.
constexpr int32_t kGammaPerGroupHead = 128;
constexpr int32_t kTileRows = 16;       // rows of one MFMA row tile
constexpr int64_t kBlockWaveWeight3 = 8; // split rule: a workgroup block counts as 8/3 busy waves
constexpr int32_t kChunkAlign = 16;     // chunk lengths are multiples of the MFMA token block
constexpr int64_t kItemFixedCost = 256; // per-item cost proxy in row units (longest-first order)
constexpr int32_t kParamsLen = 28;
// Page-table words after each group's segment (and its slack) that repeat the
// segment's last token: the kernels may read a few tiles of words past a
// segment's end unconditionally, and every word they can reach names a token
// the caller has written.
constexpr int32_t kSegGuard = 96;
// How the edge assignment was made (exported in the params table):
constexpr int32_t kEdgesGreedy = 0;  // the greedy assignment on these lengths
constexpr int32_t kEdgesForced = 1;  // given by the caller
constexpr int32_t kEdgesKept = 2;    // kept from the plan's earlier lengths (decode-loop extend)

struct PlanTables {
  // exported (see include/tree_attn.h for the layouts)
  std::vector<int32_t> params, edges, nq, lcum, groups, group_qs, group_vis, chunks, items,
      q_slot_ptr, q_slots, runs, chunk_run_ptr, bfs;
  bool runs_valid = false;  // runs / chunk_run_ptr are expanded on demand (plan_runs)
  // kernel-side expansions
  std::vector<int32_t> seg_tok;        // per group segment: (page_id << 8) | slot, one per token;
                                       // each region ends in slack and kSegGuard words that
                                       // repeat an earlier token of the segment
  std::vector<int32_t> group_seg_base; // offset of each group's segment in seg_tok
  // what the last plan_layout changed in seg_tok: everything (laid out afresh) or
  // the word ranges [seg_dirty[2i], seg_dirty[2i + 1])
  bool seg_relaid = true;
  std::vector<int32_t> seg_dirty;
  int32_t n_queries = 0, n_groups = 0, n_chunks = 0, n_items = 0, n_slots = 0;
  int32_t n_stream_items = 0;  // items [n_items - n_stream_items, n_items) are one-wave items
  int32_t max_page_id = -1;
};

// One context-query group. Membership (node, top, segment, queries, rows and
// row blocks) depends only on the tree and the edge assignment; the rest on
// the node lengths.
struct PlanGroup {
  int32_t node = 0, top = 0, rows = 0, nblocks = 0, rb = 0, cls = 0;
  int32_t tile = 1;  // row blocks are made of whole tiles of this many rows
  bool grows = false;  // the segment ends at a leaf: the group grows in a decode loop
  std::vector<int32_t> qs, seg;
  int32_t kv_len = 0, chunk_ptr = 0, n_chunks = 0, slot_base = 0, q_ptr = 0;
  std::vector<int32_t> vis;
  int32_t seg_base = 0, seg_cap = 0, seg_filled = 0;  // region of the group in seg_tok
};

// Everything a plan keeps so that a decode-loop extend (leaves grow) can
// redo only the length-dependent steps.
struct PlanState {
  PlanParams p;  // force_edges is not kept (the edges are, in f)
  int32_t n = 0, root = -1, qpl = 1, n_qheads = 1, n_kvheads = 1, head_dim = 0, page_size = 1, g = 1;
  int32_t n_q = 0, edges_mode = kEdgesGreedy, max_page = -1;
  int64_t total_tokens = 0;
  bool extended = false;  // an extend happened: growing groups get slack in seg_tok
  std::vector<int32_t> parent, ch_ptr, ch, bfs, leaves, leaf_rank, f, nq, len;
  std::vector<int64_t> A, L;
  std::vector<std::vector<int32_t>> pages;  // page ids of each node
  std::vector<PlanGroup> groups;
  // groups on each leaf's path, root side first: (group, position of the
  // leaf's first query in the group's query list)
  std::vector<int32_t> path_ptr, path_group, path_jj;
};

// P0-P6 and the greedy edge assignment. Returns 0, else a ta_status code with *err set.
int plan_init(const int32_t* parent, int32_t n_nodes, const int32_t* node_len,
              const int32_t* node_page_ptr, const int32_t* node_page_ids, int32_t page_size,
              int32_t qpl, int32_t n_qheads, int32_t n_kvheads, int32_t head_dim,
              const PlanParams& p, PlanState* S, std::string* err);

// The length-dependent steps (P5 lengths, P7-P10) into *T. Only the page-table
// words of segments that grew are rewritten (T.seg_dirty) unless the table is
// laid out afresh (T.seg_relaid). Leaves T.runs invalid.
void plan_layout(PlanState& S, PlanTables& T);

// Expands the page runs of every chunk (T.runs, T.chunk_run_ptr).
void plan_runs(const PlanState& S, PlanTables& T);

// Decode-loop growth: leaf of rank r gains leaf_add[r] >= 0 tokens at its end;
// the pages this needs (ceil(new_len / page_size) - ceil(old_len / page_size)
// per leaf) are taken from new_pages in leaf-rank order and must number
// exactly n_new_pages. The edge assignment is kept. All-or-nothing: on error
// (0 else a ta_status code with *err set) the state is unchanged.
int plan_extend(PlanState& S, const int32_t* leaf_add, const int32_t* new_pages, int64_t n_new_pages,
                std::string* err);

}  // namespace ta
