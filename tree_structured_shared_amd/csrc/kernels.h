// Device-side work description and kernel launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ta {

// One work item of the partial-attention launch (built from the plan's
// ITEMS/GROUPS/CHUNKS tables at plan time). Rows r in [row0, row0 + nrows) of
// the group map to group query r / g and q-head-in-group r % g.
struct WorkItem {
  int32_t q_ptr;     // offset of the group's queries in group_qs / group_vis
  int32_t row0;      // first row of the block
  int32_t nrows;     // rows in the block (<= rb)
  int32_t tok0;      // chunk start (segment position)
  int32_t tok1;      // chunk end (exclusive)
  int32_t seg_base;  // offset of the group's segment in seg_tok
  int32_t slot0;     // slot of the chunk's first group query: slot_base + chunk * n_q
  int32_t flags;     // reserved (0)
};

// LDS stages of the workgroup tile loop (17 KiB each at head_dim 128: K, V
// and page-table words of 32 tokens; the loop keeps kLdsStages - 1 tiles in
// flight while one is computed). Every page-table read of the kernels is
// clamped to its chunk's last token; the planner's per-segment guard words
// (kSegGuard, repeating a written token of the segment) are a margin beyond.
constexpr int kLdsStages = 3;

struct PartialArgs {
  const WorkItem* items;
  const int32_t* group_qs;
  const int32_t* group_vis;
  const int32_t* seg_tok;  // (page << 8) | slot per segment token; each segment ends in guard words
  const int32_t* slot_pos; // per partial slot two words: the workspace index of its q-head 0 and
                           // the stride between q-heads. Pair-major: the slots of one (query q,
                           // q-head h), in path order, are adjacent, at s0 * n_qheads + h * nsl +
                           // [0, nsl) with s0 = q_slot_ptr[q], nsl = q_slot_ptr[q + 1] - s0; a
                           // query's only slot (nsl = 1) holds -(q * n_qheads) - 1 and -1 instead
                           // (its rows write the output directly, see out)
  const void* q;
  const void* k;
  const void* v;
  int64_t stride_page, stride_token, stride_head;  // elements
  int64_t sp_bytes, st_bytes;   // page and token strides in bytes
  int32_t fast_addr;            // 1: every pool byte offset fits 32 bits and both
                                // byte strides fit 24 bits (24-bit multiplies)
  float* o_part;   // [n_slots (by position), n_qheads, D] records: o unnormalised in fp32, or
                   // (every |o| below l) o / l as D fp16 values in the record's first half
  float* m_part;   // [n_slots (by position), n_qheads] running max, base-2 scaled units
  float* l_part;   // [n_slots (by position), n_qheads] sum of exp2(s - m), negated for fp16 records
  float* out;      // [n_q, n_qheads, D]: rows of a query with a single partial slot (slot_pos holds
                   // -(q * n_qheads) - 1 and -1 for its slot, so the row's index is negative) write
                   // their normalised output here instead of a record
  int32_t n_qheads, n_kvheads, g;
  float scale_log2;  // softmax scale * log2(e)
};

struct ReduceArgs {
  const int32_t* q_slot_ptr;  // query q holds slots [q_slot_ptr[q], q_slot_ptr[q + 1]) (pair-major workspace);
                              // a query with one slot is skipped (the partial kernel wrote its output)
  const float* o_part;  // records as the partial kernel writes them (fp32 o, or fp16 o / l)
  const float* m_part;
  const float* l_part;  // negative (or -0) for an fp16 record
  float* out;  // [n_q, n_qheads, D]
  int32_t n_queries, n_qheads;
  int32_t max_slots;  // largest slot count of one query (sets the pairs per wave)
};

// Each launcher takes an optional pair of timing events (both null or both
// created with timing): they are stamped with the start and the end of that
// kernel's own execution (hipExtLaunchKernelGGL), not of the enqueue.
struct KernelTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};

// dtype: 0 = fp32, 1 = bf16 (Q, K and V share it). Items [0, n_block_items)
// are workgroup items (one workgroup per item x kv-head), the next
// n_wave_items single-wave items (one wave per item x kv-head); one launch.
hipError_t launch_partial(const PartialArgs& a, int32_t n_block_items, int32_t n_wave_items, int dtype,
                          int head_dim, hipStream_t s, KernelTimer t = {});
hipError_t launch_reduce(const ReduceArgs& a, int head_dim, hipStream_t s, KernelTimer t = {});
hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t s);

// KV append: token r's rows (n_kvheads x row_bytes, contiguous, r-major) of
// k_new / v_new go to pool page dst[r] >> 8, slot dst[r] & 255; element
// strides as in PartialArgs. Rows whose page is >= n_pages or whose slot is
// >= page_size are skipped.
struct AppendArgs {
  const char* k_new;
  const char* v_new;
  char* k;
  char* v;
  const int32_t* dst;
  int64_t n_tokens, n_pages;
  int64_t sp_bytes, st_bytes, sh_bytes;  // page, token and head strides in bytes
  int32_t n_kvheads, row_bytes, page_size;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
// Table update: stage holds n_desc descriptors (destination word, words,
// source word in stage) followed by the words; each range is copied into
// dst[0, dst_words). stage is pinned host memory the kernel reads in place
// (it must stay unchanged until the kernel has run). The host checks every
// range lies inside dst.
hipError_t launch_scatter(int32_t* dst, int64_t dst_words, const int32_t* stage, int32_t n_desc, hipStream_t s);
// launch_append and launch_scatter as one launch (their block ranges side by
// side in one grid); either part may be empty.
hipError_t launch_append_scatter(const AppendArgs& a, int32_t* dst, int64_t dst_words, const int32_t* stage,
                                 int32_t n_desc, hipStream_t s);
// A table update small enough to travel in the kernel arguments (descriptors
// and words as in launch_scatter, at most kArgStageWords words in all): the
// kernel reads them from its argument segment, with no read of host memory.
// app (may be NULL) is appended in the same launch.
constexpr int kArgStageWords = 448;
struct ArgStage {
  int32_t w[kArgStageWords];
};
hipError_t launch_update_args(const AppendArgs* app, int32_t* dst, int64_t dst_words, const ArgStage& stage,
                              int32_t n_desc, hipStream_t s);

}  // namespace ta
