// Host planner: tree -> KV-guided context-query groups -> KV chunks -> work
// items, slots and page runs. Pure C++ (no HIP), so it also runs host-only.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace ta {

struct PlanParams {
  int32_t ts_q = 16, ts_c = 64, gamma = 32, rb = 128, waves = 5, floor_f = 4, ncu = 256;
  int32_t split_align = 128;  // chunk lengths of the split are multiples of this
  int32_t split = 1;
  int32_t stream_rows = 16;  // groups with at most this many rows run as one-wave items
  const int8_t* force_edges = nullptr;
};

constexpr int32_t kFormatVersion = 3;
constexpr int32_t kWavesPerWG = 4;     // waves of a workgroup item
constexpr int64_t kBlockWaveWeight3 = 8; // split rule: a workgroup block counts as 8/3 busy waves
constexpr int32_t kChunkAlign = 16;     // chunk lengths are multiples of the MFMA token block
constexpr int64_t kItemFixedCost = 256; // per-item cost proxy in row units (longest-first order)
constexpr int32_t kParamsLen = 27;

struct PlanTables {
  // exported (see include/tree_attn.h for the layouts)
  std::vector<int32_t> params, edges, nq, lcum, groups, group_qs, group_vis, chunks, items,
      q_slot_ptr, q_slots, runs, chunk_run_ptr, bfs;
  // kernel-side expansions
  std::vector<int32_t> seg_tok;        // per group segment: (page_id << 8) | slot, one per token
  std::vector<int32_t> group_seg_base; // offset of each group's segment in seg_tok
  int32_t n_queries = 0, n_groups = 0, n_chunks = 0, n_items = 0, n_slots = 0;
  int32_t n_stream_items = 0;  // items [n_items - n_stream_items, n_items) are one-wave items
  int32_t max_page_id = -1;
};

// Returns 0 on success, else a ta_status code with *err set.
int build_plan(const int32_t* parent, int32_t n_nodes, const int32_t* node_len,
               const int32_t* node_page_ptr, const int32_t* node_page_ids, int32_t page_size,
               int32_t qpl, int32_t n_qheads, int32_t n_kvheads, int32_t head_dim,
               const PlanParams& p, PlanTables* out, std::string* err);

}  // namespace ta
