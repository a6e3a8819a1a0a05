// C ABI of the tree-attention library: plan lifetime, table export, decode
// launches and kernel timing. Declared in include/tree_attn.h.
#include "tree_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "planner.h"

// The partial workspace of tree_attn_decode_noalloc: a static device array,
// one per GPU the library runs on, held until the process ends. Host code
// never uses its name as an address: each device's address comes from
// hipGetSymbolAddress (scratch_of).
constexpr size_t kScratchBytes = size_t(48) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of scratch on each device, once looked up

ta_status set_err(ta_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

ta_status hip_err(hipError_t e, const std::string& where) {
  return set_err(TA_EHIP, where + ": " + hipGetErrorString(e));
}

// Device address of the static scratch on device dev (the current device),
// looked up once per device with hipGetSymbolAddress.
ta_status scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return set_err(TA_EUNSUPPORTED, "static scratch: device id out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_err(e, "static scratch: hipGetSymbolAddress");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TA_OK;
}

int32_t max_slot_count(const std::vector<int32_t>& ptr) {
  int32_t m = 0;
  for (size_t x = 0; x + 1 < ptr.size(); ++x) m = std::max(m, ptr[x + 1] - ptr[x]);
  return m;
}

}  // namespace

struct ta_plan {
  ta::PlanState S;  // what a decode-loop extend reuses
  ta::PlanTables T;
  int32_t host_only = 0, head_dim = 0, n_qheads = 0, n_kvheads = 0, g = 1, page_size = 0, qpl = 0;
  float scale = 0.0f;
  int32_t poison = 0;
  int device = -1;
  // Device tables, one allocation of kRegions regions (word offsets / capacities):
  // work items, group query ids, visible prefixes, page table (guarded segments), slot CSR,
  // slot workspace indices (two words per slot).
  void* d_tables = nullptr;
  size_t reg_off[6] = {}, reg_cap[6] = {}, tables_words = 0;
  ta::WorkItem* d_items = nullptr;
  int32_t *d_group_qs = nullptr, *d_group_vis = nullptr, *d_seg_tok = nullptr;
  int32_t *d_q_slot_ptr = nullptr, *d_slot_pos = nullptr;
  // host copies of what the device holds in the item and slot-position regions
  std::vector<ta::WorkItem> h_items;
  std::vector<int32_t> h_slot_pos, h_vis, h_q_slot_ptr;
  int32_t max_slots = 0;  // largest slot count of one query in h_q_slot_ptr
  void* d_ws = nullptr;  // workspace: o_part | m_part | l_part
  float *d_o_part = nullptr, *d_m_part = nullptr, *d_l_part = nullptr;
  int64_t ws_bytes = 0, ws_cap = 0;
  // decode-loop updates: pinned host staging (two, alternating), read in place
  // by the table-scatter kernel; an event marks when that kernel has run
  int32_t* h_stage[2] = {nullptr, nullptr};
  size_t h_stage_cap[2] = {0, 0};
  hipEvent_t stage_done[2] = {nullptr, nullptr};
  bool stage_used[2] = {false, false};
  int32_t stage_next = 0;
  bool sized_for_growth = false;  // the first extend gave every region and the workspace headroom
  // 4 per timed decode: start/stop of the partial kernel and of the reduction
  std::vector<hipEvent_t> ev;
  std::vector<uint8_t> ev_reduced;  // per timed decode: 1 if it launched the reduction
  int32_t timing_cap = 0, timing_n = 0;
  // false after a device update failed part-way (the device tables or the
  // workspace may be gone): decode refuses the plan from then on
  bool usable = true;
  // testing (ta_plan_opts.fail_alloc_after): the plan's fail_after-th
  // allocation step fails as if out of memory; alloc_steps counts the steps
  int32_t fail_after = 0, alloc_steps = 0;
  // testing (ta_plan_opts.force_staging): in-place table updates always go
  // through the pinned staging buffer, never the kernel arguments
  int32_t force_staging = 0;
  // how each device-table update went: in the kernel arguments, through the
  // pinned staging buffer, or as a whole upload (TA_T_UPDATE_COUNTS)
  std::vector<int32_t> update_counts = std::vector<int32_t>(3, 0);
  std::vector<int32_t> device_copy;  // TA_T_DEVICE_TABLES, read back on export
};

namespace {

const std::vector<int32_t>* table_ptr(const ta_plan* p, int32_t id) {
  const ta::PlanTables& T = p->T;
  if ((id == TA_T_RUNS || id == TA_T_CHUNK_RUN_PTR) && !T.runs_valid) {
    ta_plan* mp = const_cast<ta_plan*>(p);  // page runs are expanded on first export
    ta::plan_runs(mp->S, mp->T);
  }
  switch (id) {
    case TA_T_PARAMS: return &T.params;
    case TA_T_EDGES: return &T.edges;
    case TA_T_NQ: return &T.nq;
    case TA_T_LCUM: return &T.lcum;
    case TA_T_GROUPS: return &T.groups;
    case TA_T_GROUP_QS: return &T.group_qs;
    case TA_T_GROUP_VIS: return &T.group_vis;
    case TA_T_CHUNKS: return &T.chunks;
    case TA_T_ITEMS: return &T.items;
    case TA_T_Q_SLOT_PTR: return &T.q_slot_ptr;
    case TA_T_Q_SLOTS: return &T.q_slots;
    case TA_T_RUNS: return &T.runs;
    case TA_T_CHUNK_RUN_PTR: return &T.chunk_run_ptr;
    case TA_T_BFS: return &T.bfs;
    case TA_T_SEG_TOK: return &T.seg_tok;
    case TA_T_GROUP_SEG: return &T.group_seg_base;
    case TA_T_UPDATE_COUNTS: return &p->update_counts;
    case TA_T_DEVICE_TABLES: return &p->device_copy;
    default: return nullptr;
  }
}

// One allocation step of a plan (plan object, planner state, tables, device
// tables, workspace, staging): true when the testing option asks this step
// to fail.
bool alloc_fails(ta_plan* p) { return p->fail_after > 0 && ++p->alloc_steps == p->fail_after; }

void free_device(ta_plan* p) {
  if (p->host_only) return;
  for (hipEvent_t e : p->ev) (void)hipEventDestroy(e);
  p->ev.clear();
  for (int x = 0; x < 2; ++x) {
    if (p->stage_done[x]) (void)hipEventDestroy(p->stage_done[x]);
    if (p->h_stage[x]) (void)hipHostFree(p->h_stage[x]);
    p->stage_done[x] = nullptr;
    p->h_stage[x] = nullptr;
  }
  if (p->d_tables) (void)hipFree(p->d_tables);
  if (p->d_ws) (void)hipFree(p->d_ws);
  p->d_tables = p->d_ws = nullptr;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t align64w(size_t words) { return (words + 63) & ~size_t(63); }  // 256-byte regions
constexpr int kWordsPerItem = int(sizeof(ta::WorkItem) / 4);

// Device forms of the plan's tables: work items in launch order and the
// workspace index of every slot (pair-major, so each (query, q-head)'s
// partials are contiguous in path order and the reduction needs no slot list).
void device_forms(ta_plan* p) {
  const ta::PlanTables& T = p->T;
  p->h_items.resize(T.n_items);
  for (int32_t x = 0; x < T.n_items; ++x) {
    const int32_t gi = T.items[5 * x], r0 = T.items[5 * x + 1], nr = T.items[5 * x + 2],
                  ci = T.items[5 * x + 3];
    const int32_t* G = &T.groups[8 * gi];
    ta::WorkItem w{};
    w.q_ptr = G[4];
    w.row0 = r0;
    w.nrows = nr;
    w.tok0 = T.chunks[3 * ci + 1];
    w.tok1 = T.chunks[3 * ci + 2];
    w.seg_base = T.group_seg_base[gi];
    w.slot0 = G[7] + (ci - G[5]) * G[3];
    w.flags = 0;
    p->h_items[x] = w;
  }
  // per slot: workspace index of its q-head 0 and the q-head stride, pair-major
  // (the slots of one (query, q-head) adjacent, so the reduction reads them in
  // one run); a query's only slot holds -(q * n_qheads) - 1 and -1, so its rows
  // find a negative index and write the query's output directly
  p->h_slot_pos.assign(2 * T.q_slots.size(), 0);
  for (int32_t q = 0; q < T.n_queries; ++q) {
    const int32_t s0 = T.q_slot_ptr[q], nsl = T.q_slot_ptr[q + 1] - s0;
    for (int32_t k = s0; k < s0 + nsl; ++k) {
      p->h_slot_pos[2 * size_t(T.q_slots[k])] = nsl == 1 ? -(q * p->n_qheads) - 1 : s0 * p->n_qheads + (k - s0);
      p->h_slot_pos[2 * size_t(T.q_slots[k]) + 1] = nsl == 1 ? -1 : nsl;
    }
  }
}

// Words each device region needs now.
void region_sizes(const ta_plan* p, size_t (&w)[6]) {
  const ta::PlanTables& T = p->T;
  w[0] = size_t(T.n_items) * kWordsPerItem;
  w[1] = T.group_qs.size();
  w[2] = T.group_vis.size();
  w[3] = T.seg_tok.size();  // every segment ends in the planner's guard words
  w[4] = T.q_slot_ptr.size();
  w[5] = 2 * T.q_slots.size();
}

int64_t workspace_need(const ta_plan* p) {
  const size_t n_pairs = size_t(p->T.n_slots) * p->n_qheads;
  return int64_t(align256(n_pairs * p->head_dim * 4) + 2 * align256(n_pairs * 4));
}

// The workspace at base: o_part, then m_part, then l_part, each 256-byte aligned.
void workspace_layout(const ta_plan* p, void* base, float** o, float** m, float** l) {
  const size_t n_pairs = size_t(p->T.n_slots) * p->n_qheads;
  const size_t sz_o = align256(n_pairs * p->head_dim * 4), sz_m = align256(n_pairs * 4);
  uint8_t* wb = static_cast<uint8_t*>(base);
  *o = reinterpret_cast<float*>(wb);
  *m = reinterpret_cast<float*>(wb + sz_o);
  *l = reinterpret_cast<float*>(wb + sz_o + sz_m);
}

void set_workspace_ptrs(ta_plan* p) { workspace_layout(p, p->d_ws, &p->d_o_part, &p->d_m_part, &p->d_l_part); }

// (Re)allocate the workspace when it no longer fits; growth keeps headroom.
// The caller has made sure no enqueued work uses the old one.
ta_status ensure_workspace(ta_plan* p, bool headroom, bool* moved) {
  p->ws_bytes = workspace_need(p);
  if (p->d_ws && p->ws_bytes <= p->ws_cap && !(headroom && p->ws_cap < 2 * p->ws_bytes)) {
    set_workspace_ptrs(p);
    return TA_OK;
  }
  if (p->d_ws) (void)hipFree(p->d_ws);
  p->d_ws = nullptr;
  const int64_t cap = headroom ? 2 * p->ws_bytes : p->ws_bytes;
  hipError_t e = alloc_fails(p) ? hipErrorOutOfMemory : hipMalloc(&p->d_ws, size_t(cap));
  if (e != hipSuccess) {
    p->d_ws = nullptr;
    p->ws_cap = 0;
    return set_err(TA_ENOMEM, std::string("tree_attn_plan: hipMalloc(workspace): ") + hipGetErrorString(e));
  }
  p->ws_cap = cap;
  *moved = true;
  set_workspace_ptrs(p);
  return TA_OK;
}

// Whole-table upload (plan creation, and an extend whose tables outgrew their
// regions or whose page table was laid out afresh). The caller has made sure
// no enqueued work reads the old tables.
ta_status upload_full(ta_plan* p, bool headroom, bool* moved) {
  const ta::PlanTables& T = p->T;
  if (int64_t(T.n_slots) * p->n_qheads >= int64_t(INT32_MAX))
    return set_err(TA_EINVAL, "tree_attn_plan: partial slots x q-heads exceed 32-bit workspace indices");
  device_forms(p);
  p->h_vis = T.group_vis;
  p->h_q_slot_ptr = T.q_slot_ptr;
  p->max_slots = max_slot_count(T.q_slot_ptr);
  size_t need[6];
  region_sizes(p, need);
  bool fits = p->d_tables != nullptr && !headroom;  // growth always re-sizes
  for (int x = 0; x < 6; ++x) fits = fits && need[x] <= p->reg_cap[x];
  if (!fits) {
    if (p->d_tables) (void)hipFree(p->d_tables);
    p->d_tables = nullptr;
    size_t total = 0;
    for (int x = 0; x < 6; ++x) {
      const bool grows = x == 0 || x == 3 || x == 5;  // items, page table, slots
      p->reg_cap[x] = align64w(std::max<size_t>(1, (headroom && grows) ? 2 * need[x] : need[x]));
      p->reg_off[x] = total;
      total += p->reg_cap[x];
    }
    hipError_t e = alloc_fails(p) ? hipErrorOutOfMemory : hipMalloc(&p->d_tables, total * 4);
    if (e != hipSuccess) {
      p->d_tables = nullptr;
      return set_err(TA_ENOMEM, std::string("tree_attn_plan: hipMalloc(tables): ") + hipGetErrorString(e));
    }
    p->tables_words = total;
    *moved = true;
  }
  std::vector<int32_t> host(p->tables_words, 0);
  const void* src[6] = {p->h_items.data(), T.group_qs.data(), T.group_vis.data(), T.seg_tok.data(),
                        T.q_slot_ptr.data(), p->h_slot_pos.data()};
  const size_t src_words[6] = {need[0], need[1], need[2], T.seg_tok.size(), need[4], need[5]};
  for (int x = 0; x < 6; ++x)
    if (src_words[x]) std::memcpy(host.data() + p->reg_off[x], src[x], src_words[x] * 4);
  hipError_t e = hipMemcpy(p->d_tables, host.data(), p->tables_words * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_err(e, "tree_attn_plan: hipMemcpy(tables)");
  int32_t* base = static_cast<int32_t*>(p->d_tables);
  p->d_items = reinterpret_cast<ta::WorkItem*>(base + p->reg_off[0]);
  p->d_group_qs = base + p->reg_off[1];
  p->d_group_vis = base + p->reg_off[2];
  p->d_seg_tok = base + p->reg_off[3];
  p->d_q_slot_ptr = base + p->reg_off[4];
  p->d_slot_pos = base + p->reg_off[5];
  return ensure_workspace(p, headroom, moved);
}

ta_status upload(ta_plan* p) {
  bool moved = false;
  return upload_full(p, false, &moved);
}

// Decode-loop update of the device tables in place: the regions that changed
// (and the page-table words of the grown segments) go through pinned staging
// and one copy, then one kernel scatters them, all in order on `s`.
// app (may be NULL): KV rows to append in the same launch as the table
// update; *app_done says whether they were enqueued here.
ta_status upload_incremental(ta_plan* p, hipStream_t s, const ta::AppendArgs* app, bool* app_done) {
  *app_done = false;
  const ta::PlanTables& T = p->T;
  if (int64_t(T.n_slots) * p->n_qheads >= int64_t(INT32_MAX))
    return set_err(TA_EINVAL, "tree_attn_plan_extend: partial slots x q-heads exceed 32-bit workspace indices");
  std::vector<ta::WorkItem> old_items;
  old_items.swap(p->h_items);
  std::vector<int32_t> old_pos;
  old_pos.swap(p->h_slot_pos);
  device_forms(p);
  // descriptors (dst word, words, src word) then the words themselves
  std::vector<int32_t> desc, data;
  auto add = [&](size_t dst, const int32_t* src, size_t n) {
    if (n == 0) return;
    desc.insert(desc.end(), {int32_t(dst), int32_t(n), int32_t(data.size())});
    data.insert(data.end(), src, src + n);
  };
  const size_t w_items = size_t(T.n_items) * kWordsPerItem;
  if (old_items.size() != p->h_items.size() ||
      std::memcmp(old_items.data(), p->h_items.data(), w_items * 4) != 0)
    add(p->reg_off[0], reinterpret_cast<const int32_t*>(p->h_items.data()), w_items);
  if (T.group_vis != p->h_vis) add(p->reg_off[2], T.group_vis.data(), T.group_vis.size());
  if (T.q_slot_ptr != p->h_q_slot_ptr) add(p->reg_off[4], T.q_slot_ptr.data(), T.q_slot_ptr.size());
  if (old_pos != p->h_slot_pos) add(p->reg_off[5], p->h_slot_pos.data(), p->h_slot_pos.size());
  if (T.seg_relaid)  // page table laid out afresh (a growing segment used up its slack)
    add(p->reg_off[3], T.seg_tok.data(), T.seg_tok.size());
  else
    for (size_t x = 0; x + 1 < T.seg_dirty.size(); x += 2)
      add(p->reg_off[3] + size_t(T.seg_dirty[x]), T.seg_tok.data() + T.seg_dirty[x],
          size_t(T.seg_dirty[x + 1] - T.seg_dirty[x]));
  p->h_vis = T.group_vis;
  p->h_q_slot_ptr = T.q_slot_ptr;
  p->max_slots = max_slot_count(T.q_slot_ptr);
  if (desc.empty()) return TA_OK;
  const int32_t n_desc = int32_t(desc.size() / 3);
  for (int32_t d = 0; d < n_desc; ++d) desc[3 * d + 2] += int32_t(desc.size());  // data after descriptors
  const size_t words = desc.size() + data.size();
  if (words >= size_t(INT32_MAX)) return set_err(TA_EINVAL, "tree_attn_plan_extend: update too large");
  hipError_t e;
  if (words <= size_t(ta::kArgStageWords) && !p->force_staging) {
    // small update: descriptors and words travel in the kernel arguments
    ta::ArgStage st{};
    std::memcpy(st.w, desc.data(), desc.size() * 4);
    std::memcpy(st.w + desc.size(), data.data(), data.size() * 4);
    if ((e = ta::launch_update_args(app, static_cast<int32_t*>(p->d_tables), int64_t(p->tables_words), st, n_desc,
                                    s)) != hipSuccess)
      return hip_err(e, "tree_attn_plan_extend: table update launch");
    *app_done = app != nullptr;
    ++p->update_counts[0];
    return TA_OK;
  }
  // pinned host staging, read by the scatter kernel in place: this buffer's
  // previous scatter must have run
  const int b = p->stage_next;
  if (p->stage_used[b] && (e = hipEventSynchronize(p->stage_done[b])) != hipSuccess)
    return hip_err(e, "tree_attn_plan_extend: hipEventSynchronize");
  if (words > p->h_stage_cap[b]) {
    if (p->h_stage[b]) (void)hipHostFree(p->h_stage[b]);
    p->h_stage[b] = nullptr;
    const size_t cap = align64w(std::max(2 * words, p->tables_words));
    e = alloc_fails(p) ? hipErrorOutOfMemory
                       : hipHostMalloc(reinterpret_cast<void**>(&p->h_stage[b]), cap * 4, hipHostMallocDefault);
    if (e != hipSuccess) {
      p->h_stage[b] = nullptr;
      p->h_stage_cap[b] = 0;
      return hip_err(e, "tree_attn_plan_extend: hipHostMalloc(staging)");
    }
    p->h_stage_cap[b] = cap;
  }
  if (!p->stage_done[b] &&
      (e = hipEventCreateWithFlags(&p->stage_done[b], hipEventDisableTiming)) != hipSuccess)
    return hip_err(e, "tree_attn_plan_extend: hipEventCreate");
  std::memcpy(p->h_stage[b], desc.data(), desc.size() * 4);
  std::memcpy(p->h_stage[b] + desc.size(), data.data(), data.size() * 4);
  e = app ? ta::launch_append_scatter(*app, static_cast<int32_t*>(p->d_tables), int64_t(p->tables_words),
                                      p->h_stage[b], n_desc, s)
          : ta::launch_scatter(static_cast<int32_t*>(p->d_tables), int64_t(p->tables_words), p->h_stage[b], n_desc, s);
  if (e != hipSuccess) return hip_err(e, "tree_attn_plan_extend: table update launch");
  *app_done = app != nullptr;
  if ((e = hipEventRecord(p->stage_done[b], s)) != hipSuccess)
    return hip_err(e, "tree_attn_plan_extend: hipEventRecord");
  p->stage_used[b] = true;
  p->stage_next = b ^ 1;
  ++p->update_counts[1];
  return TA_OK;
}

// tree_attn_plan_extend, with app (may be NULL) appended on the same stream:
// in the table update's launch when the tables are updated in place, else by
// a launch of its own after them.
ta_status extend_impl(ta_plan* plan, const int32_t* leaf_add, const int32_t* new_pages, int64_t n_new_pages,
                      void* hip_stream, int32_t* relaunch, const ta::AppendArgs* app) {
  bool changed = false;  // the plan's state has moved on: a failure from here leaves it unusable
  try {
    if (!plan->usable)
      return set_err(TA_EINVAL, "tree_attn_plan_extend: the plan is unusable after a failed update");
    if (!plan->host_only) {
      int dev = -1;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return hip_err(e, "tree_attn_plan_extend: hipGetDevice");
      if (dev != plan->device)
        return set_err(TA_EINVAL, "tree_attn_plan_extend: current device differs from the plan's");
    }
    if (alloc_fails(plan)) throw std::bad_alloc();  // testing: the host step (plan unchanged)
    const int32_t old_items = plan->T.n_items, old_stream = plan->T.n_stream_items, old_slots = plan->T.n_slots;
    std::string err;
    const int rc = ta::plan_extend(plan->S, leaf_add, new_pages, n_new_pages, &err);
    if (rc != 0) return set_err(ta_status(rc), err);
    changed = true;
    ta::plan_layout(plan->S, plan->T);
    if (plan->host_only) return TA_OK;
    size_t need[6];
    region_sizes(plan, need);
    bool fits = plan->sized_for_growth;
    for (int x = 0; x < 6; ++x) fits = fits && need[x] <= plan->reg_cap[x];
    fits = fits && workspace_need(plan) <= plan->ws_cap;
    bool moved = false, app_done = false;
    ta_status st;
    if (fits) {
      st = upload_incremental(plan, static_cast<hipStream_t>(hip_stream), app, &app_done);
      set_workspace_ptrs(plan);
      plan->ws_bytes = workspace_need(plan);
    } else {
      // first extend, or regions outgrown: wait for every enqueued use of the
      // old tables, then upload them whole with room to grow (2x)
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_err(e, "tree_attn_plan_extend: hipDeviceSynchronize");
      st = upload_full(plan, true, &moved);
      plan->sized_for_growth = true;
      if (st == TA_OK) ++plan->update_counts[2];
    }
    if (st != TA_OK) {
      plan->usable = false;
      return st;
    }
    if (app && !app_done) {
      const hipError_t e = ta::launch_append(*app, static_cast<hipStream_t>(hip_stream));
      if (e != hipSuccess) return hip_err(e, "tree_attn_plan_extend_append: append launch");
    }
    if (relaunch)
      *relaunch = (moved || plan->T.n_items != old_items || plan->T.n_stream_items != old_stream ||
                   plan->T.n_slots != old_slots) ? 1 : 0;
    return TA_OK;
  } catch (const std::bad_alloc&) {
    if (changed) plan->usable = false;
    return set_err(TA_ENOMEM, "tree_attn_plan_extend: host allocation failed");
  }
}

// Checks the arguments of a KV append (fn names the entry point in errors)
// and fills *a; a->n_tokens == 0 means nothing to append.
ta_status append_args(const char* fn, const ta_paged_kv* kv, const void* k_new, const void* v_new, int64_t n_tokens,
                      int32_t n_kvheads, int32_t head_dim, const int32_t* dst, ta::AppendArgs* a) {
  const std::string f(fn);
  if (!kv || !kv->k || !kv->v) return set_err(TA_EINVAL, f + ": NULL pool");
  if (n_tokens < 0) return set_err(TA_EINVAL, f + ": negative token count");
  if (n_tokens > 0 && (!k_new || !v_new || !dst)) return set_err(TA_EINVAL, f + ": NULL argument");
  if (kv->dtype != TA_F32 && kv->dtype != TA_BF16)
    return set_err(TA_EUNSUPPORTED, f + ": dtype must be TA_F32 or TA_BF16");
  if (head_dim != 64 && head_dim != 128) return set_err(TA_EUNSUPPORTED, f + ": head_dim must be 64 or 128");
  if (n_kvheads < 1 || kv->page_size < 1 || kv->page_size > 256 || kv->n_pages < 1)
    return set_err(TA_EINVAL, f + ": bad n_kvheads, page_size or n_pages");
  const int64_t es = kv->dtype == TA_BF16 ? 2 : 4, vec = 16 / es;
  if (kv->stride_page <= 0 || kv->stride_token <= 0 || kv->stride_head <= 0 ||
      kv->stride_page % vec || kv->stride_token % vec || kv->stride_head % vec)
    return set_err(TA_EINVAL, f + ": strides must be positive multiples of 16 bytes");
  if ((reinterpret_cast<uintptr_t>(kv->k) | reinterpret_cast<uintptr_t>(kv->v) |
       reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return set_err(TA_EINVAL, f + ": pointers must be 16-byte aligned");
  *a = ta::AppendArgs{};
  a->k_new = static_cast<const char*>(k_new);
  a->v_new = static_cast<const char*>(v_new);
  a->k = static_cast<char*>(const_cast<void*>(kv->k));
  a->v = static_cast<char*>(const_cast<void*>(kv->v));
  a->dst = dst;
  a->n_tokens = n_tokens;
  a->n_pages = kv->n_pages;
  a->sp_bytes = kv->stride_page * es;
  a->st_bytes = kv->stride_token * es;
  a->sh_bytes = kv->stride_head * es;
  a->n_kvheads = n_kvheads;
  a->row_bytes = int32_t(head_dim * es);
  a->page_size = kv->page_size;
  return TA_OK;
}

// One decode step (tree_attn_decode, tree_attn_decode_noalloc): argument
// checks, then the partial-attention and reduction launches on hip_stream.
// The partial results go to the plan's workspace, or, with ws_base, to the
// same layout at ws_base (the static scratch). fn names the entry point in
// errors.
ta_status decode_impl(const char* fn_name, const void* q, ta_dtype q_dtype, const ta_paged_kv* kv,
                      const ta_plan* plan, float* out, void* hip_stream, void* ws_base) {
  const std::string fn(fn_name);
  if (!plan) return set_err(TA_EINVAL, fn + ": plan is NULL");
  if (plan->host_only) return set_err(TA_EINVAL, fn + ": plan was built host_only");
  if (!plan->usable) return set_err(TA_EINVAL, fn + ": the plan is unusable after a failed update");
  if (!q || !kv || !out || !kv->k || !kv->v)
    return set_err(TA_EINVAL, fn + ": NULL pointer argument");
  if (q_dtype != TA_F32 && q_dtype != TA_BF16)
    return set_err(TA_EUNSUPPORTED, fn + ": dtype must be TA_F32 or TA_BF16");
  if (kv->dtype != q_dtype)
    return set_err(TA_EUNSUPPORTED, fn + ": Q and KV dtypes differ");
  if (kv->page_size != plan->page_size)
    return set_err(TA_EINVAL, fn + ": page_size differs from the plan's");
  if (kv->n_pages <= int64_t(plan->T.max_page_id))
    return set_err(TA_EINVAL, fn + ": the plan references pages beyond kv->n_pages");
  const int64_t vec = (q_dtype == TA_BF16) ? 8 : 4;  // elements per 16 bytes
  if (kv->stride_page <= 0 || kv->stride_token <= 0 || kv->stride_head <= 0 ||
      kv->stride_page % vec || kv->stride_token % vec || kv->stride_head % vec)
    return set_err(TA_EINVAL, fn + ": strides must be positive multiples of 16 bytes");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv->k) |
       reinterpret_cast<uintptr_t>(kv->v) | reinterpret_cast<uintptr_t>(out)) & 15)
    return set_err(TA_EINVAL, fn + ": pointers must be 16-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_err(e, fn + ": hipGetDevice");
  if (dev != plan->device) return set_err(TA_EINVAL, fn + ": current device differs from the plan's");

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  ta_plan* mp = const_cast<ta_plan*>(plan);
  const bool timed = mp->timing_cap > 0 && mp->timing_n < mp->timing_cap;
  if (mp->poison) {
    e = ta::launch_fill(ws_base ? static_cast<float*>(ws_base) : mp->d_o_part, mp->ws_bytes / 4, std::nanf(""), s);
    if (e != hipSuccess) return hip_err(e, fn + ": poison fill");
  }
  ta::KernelTimer t_part, t_red;
  if (timed) {
    hipEvent_t* ev = &mp->ev[4 * size_t(mp->timing_n)];
    t_part = {ev[0], ev[1]};
    t_red = {ev[2], ev[3]};
  }

  float *o_part = plan->d_o_part, *m_part = plan->d_m_part, *l_part = plan->d_l_part;
  if (ws_base) workspace_layout(plan, ws_base, &o_part, &m_part, &l_part);

  ta::PartialArgs a{};
  a.items = plan->d_items;
  a.group_qs = plan->d_group_qs;
  a.group_vis = plan->d_group_vis;
  a.seg_tok = plan->d_seg_tok;
  a.slot_pos = plan->d_slot_pos;
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.stride_page = kv->stride_page;
  a.stride_token = kv->stride_token;
  a.stride_head = kv->stride_head;
  {
    const int64_t es = (q_dtype == TA_BF16) ? 2 : 4;
    a.sp_bytes = kv->stride_page * es;
    a.st_bytes = kv->stride_token * es;
    const int64_t max_off = ((kv->n_pages - 1) * kv->stride_page + (kv->page_size - 1) * kv->stride_token +
                             int64_t(plan->n_kvheads - 1) * kv->stride_head + plan->head_dim) * es;
    a.fast_addr = (max_off < (int64_t(1) << 32) && a.sp_bytes < (1 << 24) && a.st_bytes < (1 << 24)) ? 1 : 0;
  }
  a.o_part = o_part;
  a.m_part = m_part;
  a.l_part = l_part;
  a.out = out;
  a.n_qheads = plan->n_qheads;
  a.n_kvheads = plan->n_kvheads;
  a.g = plan->g;
  a.scale_log2 = plan->scale * 1.4426950408889634f;
  const int dt = q_dtype == TA_BF16 ? 1 : 0;
  const int32_t n_block = plan->T.n_items - plan->T.n_stream_items, n_wave = plan->T.n_stream_items;
  if ((e = ta::launch_partial(a, n_block, n_wave, dt, plan->head_dim, s, t_part)) != hipSuccess)
    return hip_err(e, fn + ": partial-attention launch");

  ta::ReduceArgs r{};
  r.q_slot_ptr = plan->d_q_slot_ptr;
  r.o_part = o_part;
  r.m_part = m_part;
  r.l_part = l_part;
  r.out = out;
  r.n_queries = plan->T.n_queries;
  r.n_qheads = plan->n_qheads;
  r.max_slots = plan->max_slots;
  // with one slot per query the partial kernel wrote every output
  if (plan->max_slots > 1) {
    e = ta::launch_reduce(r, plan->head_dim, s, t_red);
    if (e != hipSuccess) return hip_err(e, fn + ": reduction launch");
  }
  if (timed) mp->ev_reduced[size_t(mp->timing_n)] = plan->max_slots > 1 ? 1 : 0;
  if (timed) ++mp->timing_n;
  return TA_OK;
}


// TREE_ATTN_LOG set (and not "0"): one line of plan statistics on stderr per
// tree_attn_plan: groups, joined edges, chunks, items by class, partial
// slots, the split's chunk length, workspace bytes, unique K/V tokens and the
// partial-result bytes one decode writes and reads back.
void log_plan(const ta_plan* p) {
  const char* env = std::getenv("TREE_ATTN_LOG");
  if (!env || !*env || std::strcmp(env, "0") == 0) return;
  const ta::PlanTables& T = p->T;
  int32_t joined = 0;
  for (size_t v = 0; v < T.edges.size(); ++v) joined += T.edges[v];
  const int64_t pair_bytes = int64_t(p->head_dim + 2) * 4;
  const int64_t partial = 2 * int64_t(T.n_slots) * p->n_qheads * pair_bytes;
  const int64_t ws = p->host_only ? int64_t(align256(size_t(T.n_slots) * p->n_qheads * p->head_dim * 4)) +
                                        2 * int64_t(align256(size_t(T.n_slots) * p->n_qheads * 4))
                                  : p->ws_bytes;
  std::fprintf(stderr,
               "tree_attn_plan: nodes %d queries %d groups %d edges_joined %d chunks %d items %d "
               "(workgroup %d single_wave %d) slots %d chunk_tokens %d workspace_bytes %lld "
               "kv_tokens %lld partial_bytes %lld\n",
               p->S.n, T.n_queries, T.n_groups, joined, T.n_chunks, T.n_items, T.n_items - T.n_stream_items,
               T.n_stream_items, T.n_slots, T.params.size() > 22 ? T.params[22] : 0, (long long)ws,
               (long long)p->S.total_tokens, (long long)partial);
}

}  // namespace

extern "C" {

ta_status tree_attn_plan(const int32_t* parent, int32_t n_nodes, const int32_t* node_kv_len,
                         const int32_t* node_page_ptr, const int32_t* node_page_ids,
                         int32_t page_size, int32_t queries_per_leaf, int32_t n_qheads,
                         int32_t n_kvheads, int32_t head_dim, const ta_plan_opts* opts,
                         ta_plan** out_plan) {
  g_err.clear();
  if (!out_plan) return set_err(TA_EINVAL, "tree_attn_plan: out_plan is NULL");
  *out_plan = nullptr;
  ta_plan* p = nullptr;
  try {
    ta::PlanParams pp;
    int32_t host_only = 0, poison = 0, force_staging = 0;
    float scale = 0.0f;
    if (opts) {
      if (opts->ts_q) pp.ts_q = opts->ts_q;
      if (opts->ts_c) pp.ts_c = opts->ts_c;
      if (opts->gamma) pp.gamma = opts->gamma;
      if (opts->rb) pp.rb = opts->rb;
      if (opts->waves) pp.waves = opts->waves;
      if (opts->floor_f) pp.floor_f = opts->floor_f;
      pp.split = opts->no_split ? 0 : 1;
      pp.force_edges = opts->force_edges;
      host_only = opts->host_only ? 1 : 0;
      poison = opts->poison_workspace ? 1 : 0;
      scale = opts->scale;
      if (opts->ncu) pp.ncu = opts->ncu;
      if (opts->stream_rows) pp.stream_rows = opts->stream_rows < 0 ? 0 : opts->stream_rows;
      if (opts->split_align) pp.split_align = opts->split_align;
      pp.tile_join = opts->no_tile_join ? 0 : 1;
      if (opts->fail_alloc_after < 0) return set_err(TA_EINVAL, "tree_attn_plan: negative fail_alloc_after");
      force_staging = opts->force_staging ? 1 : 0;
    }
    const int32_t fail_after = opts ? opts->fail_alloc_after : 0;
    if (fail_after == 1) return set_err(TA_ENOMEM, "tree_attn_plan: host allocation failed (plan)");
    int device = -1;
    if (!host_only) {
      hipError_t e = hipGetDevice(&device);
      if (e != hipSuccess) return hip_err(e, "tree_attn_plan: hipGetDevice");
      if (!(opts && opts->ncu)) {
        int ncu = 0;
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device);
        if (e != hipSuccess) return hip_err(e, "tree_attn_plan: hipDeviceGetAttribute");
        pp.ncu = ncu;
      }
    }
    if (!(scale >= 0.0f) || std::isinf(scale)) return set_err(TA_EINVAL, "tree_attn_plan: bad scale");
    p = new ta_plan;
    p->fail_after = fail_after;
    p->force_staging = force_staging;
    p->alloc_steps = 1;  // the plan object
    std::string err;
    if (alloc_fails(p)) throw std::bad_alloc();  // testing: the planner state
    const int rc = ta::plan_init(parent, n_nodes, node_kv_len, node_page_ptr, node_page_ids,
                                 page_size, queries_per_leaf, n_qheads, n_kvheads, head_dim, pp,
                                 &p->S, &err);
    if (rc != 0) {
      delete p;
      return set_err(ta_status(rc), err);
    }
    if (alloc_fails(p)) throw std::bad_alloc();  // testing: the tables
    ta::plan_layout(p->S, p->T);
    p->host_only = host_only;
    p->head_dim = head_dim;
    p->n_qheads = n_qheads;
    p->n_kvheads = n_kvheads;
    p->g = n_qheads / n_kvheads;
    p->page_size = page_size;
    p->qpl = queries_per_leaf;
    p->scale = scale > 0.0f ? scale : 1.0f / std::sqrt(float(head_dim));
    p->poison = poison;
    p->device = device;
    if (!host_only) {
      const ta_status s = upload(p);
      if (s != TA_OK) {
        free_device(p);
        delete p;
        return s;
      }
    }
    log_plan(p);
    *out_plan = p;
    return TA_OK;
  } catch (const std::bad_alloc&) {
    delete p;
    return set_err(TA_ENOMEM, "tree_attn_plan: host allocation failed");
  } catch (...) {
    delete p;
    return set_err(TA_EINVAL, "tree_attn_plan: unexpected failure");
  }
}


ta_status tree_attn_plan_extend(ta_plan* plan, const int32_t* leaf_add, const int32_t* new_pages,
                                int64_t n_new_pages, void* hip_stream, int32_t* relaunch) {
  g_err.clear();
  if (relaunch) *relaunch = 0;
  if (!plan) return set_err(TA_EINVAL, "tree_attn_plan_extend: plan is NULL");
  return extend_impl(plan, leaf_add, new_pages, n_new_pages, hip_stream, relaunch, nullptr);
}

ta_status tree_attn_plan_extend_append(ta_plan* plan, const int32_t* leaf_add, const int32_t* new_pages,
                                       int64_t n_new_pages, const ta_paged_kv* kv, const void* k_new,
                                       const void* v_new, int64_t n_tokens, const int32_t* dst, void* hip_stream,
                                       int32_t* relaunch) {
  g_err.clear();
  if (relaunch) *relaunch = 0;
  if (!plan) return set_err(TA_EINVAL, "tree_attn_plan_extend_append: plan is NULL");
  if (plan->host_only) return set_err(TA_EINVAL, "tree_attn_plan_extend_append: plan was built host_only");
  if (kv && kv->page_size != plan->page_size)
    return set_err(TA_EINVAL, "tree_attn_plan_extend_append: pool page_size differs from the plan's");
  ta::AppendArgs a;
  const ta_status st = append_args("tree_attn_plan_extend_append", kv, k_new, v_new, n_tokens, plan->n_kvheads,
                                   plan->head_dim, dst, &a);
  if (st != TA_OK) return st;
  return extend_impl(plan, leaf_add, new_pages, n_new_pages, hip_stream, relaunch, n_tokens > 0 ? &a : nullptr);
}

ta_status tree_attn_decode(const void* q, ta_dtype q_dtype, const ta_paged_kv* kv,
                           const ta_plan* plan, float* out, void* hip_stream) {
  g_err.clear();
  return decode_impl("tree_attn_decode", q, q_dtype, kv, plan, out, hip_stream, nullptr);
}

ta_status tree_attn_decode_noalloc(const void* q, ta_dtype q_dtype, const ta_paged_kv* kv,
                                   const ta_plan* plan, float* out, void* hip_stream) {
  g_err.clear();
  if (!plan) return set_err(TA_EINVAL, "tree_attn_decode_noalloc: plan is NULL");
  if (plan->host_only) return set_err(TA_EINVAL, "tree_attn_decode_noalloc: plan was built host_only");
  const int64_t need = workspace_need(plan);
  if (need > int64_t(kScratchBytes))
    return set_err(TA_EINVAL, "tree_attn_decode_noalloc: the plan's partial workspace (" + std::to_string(need) +
                                  " bytes) exceeds the static scratch (" + std::to_string(kScratchBytes) +
                                  " bytes)");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_err(e, "tree_attn_decode_noalloc: hipGetDevice");
  void* ws = nullptr;
  const ta_status st = scratch_of(dev, &ws);
  if (st != TA_OK) return st;
  return decode_impl("tree_attn_decode_noalloc", q, q_dtype, kv, plan, out, hip_stream, ws);
}

ta_status tree_attn_kv_append(const ta_paged_kv* kv, const void* k_new, const void* v_new, int64_t n_tokens,
                              int32_t n_kvheads, int32_t head_dim, const int32_t* dst, void* hip_stream) {
  g_err.clear();
  ta::AppendArgs a;
  const ta_status st = append_args("tree_attn_kv_append", kv, k_new, v_new, n_tokens, n_kvheads, head_dim, dst, &a);
  if (st != TA_OK || n_tokens == 0) return st;
  const hipError_t e = ta::launch_append(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_err(e, "tree_attn_kv_append: launch");
  return TA_OK;
}

ta_status tree_attn_plan_info(const ta_plan* plan, int32_t* n_queries, int64_t* workspace_bytes,
                              int32_t* n_items) {
  g_err.clear();
  if (!plan) return set_err(TA_EINVAL, "tree_attn_plan_info: plan is NULL");
  if (n_queries) *n_queries = plan->T.n_queries;
  if (workspace_bytes) {
    if (plan->host_only) {
      const int64_t pairs = int64_t(plan->T.n_slots) * plan->n_qheads;
      *workspace_bytes = int64_t(align256(size_t(pairs) * plan->head_dim * 4)) + 2 * int64_t(align256(size_t(pairs) * 4));
    } else {
      *workspace_bytes = plan->ws_bytes;
    }
  }
  if (n_items) *n_items = plan->T.n_items;
  return TA_OK;
}

ta_status tree_attn_plan_export(const ta_plan* plan, int32_t table_id, int32_t* dst, int64_t* len) {
  g_err.clear();
  if (!plan || !len) return set_err(TA_EINVAL, "tree_attn_plan_export: NULL plan or len");
  if (table_id == TA_T_DEVICE_TABLES) {  // the device copy, read back (waits for the device)
    if (plan->host_only) return set_err(TA_EINVAL, "tree_attn_plan_export: host_only plans have no device tables");
    try {
      ta_plan* mp = const_cast<ta_plan*>(plan);
      mp->device_copy.resize(plan->tables_words);
      hipError_t e = hipDeviceSynchronize();
      if (e == hipSuccess)
        e = hipMemcpy(mp->device_copy.data(), plan->d_tables, plan->tables_words * 4, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_err(e, "tree_attn_plan_export: device tables");
    } catch (const std::bad_alloc&) {
      return set_err(TA_ENOMEM, "tree_attn_plan_export: host allocation failed");
    }
  }
  const std::vector<int32_t>* t = table_ptr(plan, table_id);
  if (!t) return set_err(TA_EINVAL, "tree_attn_plan_export: unknown table id");
  if (dst) {
    if (*len < int64_t(t->size())) return set_err(TA_EINVAL, "tree_attn_plan_export: dst too small");
    if (!t->empty()) std::memcpy(dst, t->data(), t->size() * sizeof(int32_t));
  }
  *len = int64_t(t->size());
  return TA_OK;
}

ta_status tree_attn_timing_enable(ta_plan* plan, int32_t capacity) {
  g_err.clear();
  if (!plan) return set_err(TA_EINVAL, "tree_attn_timing_enable: plan is NULL");
  if (plan->host_only) return set_err(TA_EINVAL, "tree_attn_timing_enable: host_only plan");
  if (capacity < 0) return set_err(TA_EINVAL, "tree_attn_timing_enable: negative capacity");
  for (hipEvent_t e : plan->ev) (void)hipEventDestroy(e);
  plan->ev.clear();
  plan->timing_cap = 0;
  plan->timing_n = 0;
  try {
    plan->ev.resize(size_t(capacity) * 4);
    plan->ev_reduced.assign(size_t(capacity), 0);
  } catch (const std::bad_alloc&) {
    return set_err(TA_ENOMEM, "tree_attn_timing_enable: host allocation failed");
  }
  for (size_t x = 0; x < plan->ev.size(); ++x) {
    hipError_t e = hipEventCreate(&plan->ev[x]);
    if (e != hipSuccess) {
      plan->ev.resize(x);
      return hip_err(e, "tree_attn_timing_enable: hipEventCreate");
    }
  }
  plan->timing_cap = capacity;
  return TA_OK;
}

ta_status tree_attn_timing_read(ta_plan* plan, float* partial_ms, float* reduce_ms, int32_t* n) {
  g_err.clear();
  if (!plan || !n) return set_err(TA_EINVAL, "tree_attn_timing_read: NULL argument");
  const int32_t cnt = plan->timing_n;
  for (int32_t x = 0; x < cnt; ++x) {
    const hipEvent_t* ev = &plan->ev[4 * size_t(x)];
    const bool reduced = plan->ev_reduced[size_t(x)] != 0;  // else no reduction kernel ran: 0 ms
    hipError_t e = hipEventSynchronize(ev[1]);
    if (e == hipSuccess && reduced) e = hipEventSynchronize(ev[3]);
    if (e != hipSuccess) return hip_err(e, "tree_attn_timing_read: hipEventSynchronize");
    float t0 = 0.0f, t1 = 0.0f;
    if ((e = hipEventElapsedTime(&t0, ev[0], ev[1])) != hipSuccess ||
        (reduced && (e = hipEventElapsedTime(&t1, ev[2], ev[3])) != hipSuccess))
      return hip_err(e, "tree_attn_timing_read: hipEventElapsedTime");
    if (partial_ms) partial_ms[x] = t0;
    if (reduce_ms) reduce_ms[x] = t1;
  }
  *n = cnt;
  plan->timing_n = 0;
  return TA_OK;
}

void tree_attn_plan_destroy(ta_plan* plan) {
  if (!plan) return;
  if (!plan->host_only) (void)hipDeviceSynchronize();
  free_device(plan);
  delete plan;
}

const char* tree_attn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
