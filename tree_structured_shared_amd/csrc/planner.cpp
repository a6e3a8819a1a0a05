// Host planner for tree-structured decode attention.
//
// Steps (integer only, deterministic, so its tables can be compared exactly):
//  P0  validate the tree, lengths and page CSR.
//  P1  children of every node in ascending id; leaves ranked by ascending id.
//  P2  A[v] = query tokens below v.
//  P3  BFS from the root (FIFO, children ascending).
//  P4  greedy binary edge assignment -- FastTree review, section 3.2,
//      Algorithm 1: for each child l of v (BFS order) compare the cost of
//      keeping the edge split (SplitKVCost: padding of both groups plus the
//      intermediate result gamma * nQ_l) with joining it (SplitQCost: v keeps
//      nQ_curr - nQ_l queries, l reads len_l + len_v); assign 1 iff C0 >= C1.
//      Padding cost C_P(n, len) = Pad(TS_q, n) * len + n * Pad(TS_c, min(len, TS_c))
//      with Pad(TS, N) = TS - ((N - 1) % TS + 1) (section 3.2 cost model; the
//      common factor d dropped, Pad(TS, 0) = 0).
//  P5  one group per virtual node with queries left (DeFT notes, KV-guided
//      split: a node's KV grouped with every query that shares it).
//  P6  item class and row blocks: a group with at most stream_rows rows is
//      one single-wave stream block; a larger one is cut into balanced
//      workgroup blocks of at most rb rows (16-aligned when rb is). Row r =
//      (query r / g, q-head r % g).
//  P7  long-context split (FastTree review, section 3.3): a global chunk
//      length sized so the launch gives about ncu * waves busy waves (a
//      workgroup block counts as kBlockWaveWeight3 / 3 waves: its four waves
//      share each staged tile), a multiple of split_align, floored per group
//      at floor_f tokens per row; each group's chunks are then balanced and
//      16-aligned.
//  P8  work items: workgroup items first, then stream items, each class
//      longest first (stable).
//  P9  partial-result slots: group, then chunk, then query.
//  P10 page runs of every chunk and the per-token page table the kernel reads.
#include "planner.h"

#include <algorithm>
#include <cstdio>
#include <deque>

namespace ta {
namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

inline int64_t pad_tiles(int64_t ts, int64_t n) { return n <= 0 ? 0 : ts - ((n - 1) % ts + 1); }

inline int64_t pad_cost(int64_t nq, int64_t len, int64_t ts_q, int64_t ts_c) {
  return pad_tiles(ts_q, nq) * len + nq * pad_tiles(ts_c, std::min(len, ts_c));
}

struct Group {
  int32_t node, top, kv_len, rows, nblocks, chunk_ptr, n_chunks, slot_base, q_ptr, seg_base;
  int32_t cls, rb;  // cls 0 = stream (one wave), 1 = workgroup
  std::vector<int32_t> qs, vis, seg;
};

int fail(std::string* err, int code, const char* msg) {
  *err = msg;
  return code;
}

}  // namespace

int build_plan(const int32_t* parent, int32_t n, const int32_t* node_len,
               const int32_t* node_page_ptr, const int32_t* node_page_ids, int32_t page_size,
               int32_t qpl, int32_t n_qheads, int32_t n_kvheads, int32_t head_dim,
               const PlanParams& p, PlanTables* out, std::string* err) {
  const int EINVAL_ = 1, EUNSUP_ = 4;
  // ---- P0
  if (n < 1 || !parent || !node_len || !node_page_ptr || !node_page_ids)
    return fail(err, EINVAL_, "tree_attn_plan: empty tree or null array");
  if (qpl < 1 || n_qheads < 1 || n_kvheads < 1 || n_qheads % n_kvheads)
    return fail(err, EINVAL_, "tree_attn_plan: need qpl >= 1 and n_qheads % n_kvheads == 0");
  if (head_dim != 64 && head_dim != 128)
    return fail(err, EUNSUP_, "tree_attn_plan: head_dim must be 64 or 128");
  if (page_size < 1 || page_size > 256)
    return fail(err, EINVAL_, "tree_attn_plan: page_size must be in 1..256");
  if (p.ts_q < 1 || p.ts_c < 1 || p.gamma < 0 || p.rb < 1 || p.waves < 1 || p.floor_f < 0 ||
      p.ncu < 1 || p.stream_rows < 0 || p.split_align < 16 || p.split_align % 16)
    return fail(err, EINVAL_, "tree_attn_plan: invalid option value");
  int32_t root = -1;
  for (int32_t v = 0; v < n; ++v) {
    if (parent[v] == -1) {
      if (root != -1) return fail(err, EINVAL_, "tree_attn_plan: more than one root");
      root = v;
    } else if (parent[v] < 0 || parent[v] >= n || parent[v] == v) {
      return fail(err, EINVAL_, "tree_attn_plan: parent id out of range");
    }
  }
  if (root < 0) return fail(err, EINVAL_, "tree_attn_plan: no root");
  for (int32_t v = 0; v < n; ++v) {
    int32_t u = v, steps = 0;
    while (u != root) {
      u = parent[u];
      if (++steps > n) return fail(err, EINVAL_, "tree_attn_plan: parent array has a cycle");
    }
  }
  // ---- P1
  std::vector<std::vector<int32_t>> ch(n);
  for (int32_t v = 0; v < n; ++v)
    if (parent[v] >= 0) ch[parent[v]].push_back(v);
  int64_t total_tokens = 0;
  for (int32_t v = 0; v < n; ++v) {
    if (node_len[v] < 1) return fail(err, EINVAL_, "tree_attn_plan: node length < 1");
    if (ch[v].empty() && node_len[v] < qpl)
      return fail(err, EINVAL_, "tree_attn_plan: leaf shorter than queries_per_leaf");
    total_tokens += node_len[v];
  }
  if (total_tokens >= (int64_t(1) << 30)) return fail(err, EINVAL_, "tree_attn_plan: too many tokens");
  if (node_page_ptr[0] != 0) return fail(err, EINVAL_, "tree_attn_plan: node_page_ptr[0] != 0");
  for (int32_t v = 0; v < n; ++v)
    if (int64_t(node_page_ptr[v + 1]) - node_page_ptr[v] != cdiv(node_len[v], page_size))
      return fail(err, EINVAL_, "tree_attn_plan: node page count != ceil(len / page_size)");
  int32_t max_page = -1;
  for (int32_t i = 0; i < node_page_ptr[n]; ++i) {
    if (node_page_ids[i] < 0 || node_page_ids[i] >= (1 << 23))
      return fail(err, EINVAL_, "tree_attn_plan: page id out of range [0, 2^23)");
    max_page = std::max(max_page, node_page_ids[i]);
  }
  std::vector<int32_t> leaves, leaf_rank(n, -1);
  for (int32_t v = 0; v < n; ++v)
    if (ch[v].empty()) {
      leaf_rank[v] = int32_t(leaves.size());
      leaves.push_back(v);
    }
  const int32_t n_q = int32_t(leaves.size()) * qpl;
  const int32_t g = n_qheads / n_kvheads;
  const int64_t H = n_kvheads;

  // ---- P3 (BFS) then P2 (A, bottom-up over reversed BFS)
  std::vector<int32_t> bfs;
  bfs.reserve(n);
  {
    std::deque<int32_t> dq{root};
    while (!dq.empty()) {
      int32_t v = dq.front();
      dq.pop_front();
      bfs.push_back(v);
      for (int32_t c : ch[v]) dq.push_back(c);
    }
  }
  std::vector<int64_t> A(n, 0);
  for (auto it = bfs.rbegin(); it != bfs.rend(); ++it) {
    int32_t v = *it;
    if (ch[v].empty()) A[v] = qpl;
    else
      for (int32_t c : ch[v]) A[v] += A[c];
  }

  // ---- P4 greedy
  std::vector<int64_t> L(node_len, node_len + n);
  std::vector<int32_t> f(n, 0), nQ(n, 0);
  for (int32_t v : bfs) {
    int64_t nq_curr = A[v];
    const int64_t len_v = L[v];
    for (int32_t l : ch[v]) {
      const int64_t nq_l = A[l], len_l = L[l];
      int32_t assign;
      if (p.force_edges) {
        assign = p.force_edges[l] ? 1 : 0;
      } else {
        const int64_t c0 = pad_cost(nq_curr, len_v, p.ts_q, p.ts_c) +
                           pad_cost(nq_l, len_l, p.ts_q, p.ts_c) + int64_t(p.gamma) * nq_l;
        const int64_t c1 = pad_cost(nq_curr - nq_l, len_v, p.ts_q, p.ts_c) +
                           pad_cost(nq_l, len_l + len_v, p.ts_q, p.ts_c);
        assign = (c0 >= c1) ? 1 : 0;
      }
      f[l] = assign;
      if (assign) {
        nq_curr -= nq_l;
        L[l] = len_l + len_v;
      }
    }
    nQ[v] = int32_t(nq_curr);
  }

  // ---- P5 groups
  std::vector<int32_t> top(n, 0);
  for (int32_t v : bfs) top[v] = (v == root || f[v] == 0) ? v : top[parent[v]];
  std::vector<Group> groups;
  std::vector<int32_t> group_of(n, -1);
  for (int32_t v : bfs) {
    if (nQ[v] == 0) continue;
    Group G{};
    G.node = v;
    G.top = top[v];
    G.kv_len = int32_t(L[v]);
    // queries: the leaf's own, plus those below children kept apart (edge 0)
    if (ch[v].empty())
      for (int32_t j = 0; j < qpl; ++j) G.qs.push_back(leaf_rank[v] * qpl + j);
    std::vector<int32_t> stack;
    for (int32_t c : ch[v])
      if (f[c] == 0) stack.push_back(c);
    while (!stack.empty()) {
      int32_t u = stack.back();
      stack.pop_back();
      if (ch[u].empty())
        for (int32_t j = 0; j < qpl; ++j) G.qs.push_back(leaf_rank[u] * qpl + j);
      for (int32_t c : ch[u]) stack.push_back(c);
    }
    std::sort(G.qs.begin(), G.qs.end());
    if (int32_t(G.qs.size()) != nQ[v]) return fail(err, EINVAL_, "tree_attn_plan: internal query count");
    for (int32_t u = v;; u = parent[u]) {
      G.seg.push_back(u);
      if (u == G.top) break;
    }
    std::reverse(G.seg.begin(), G.seg.end());
    for (int32_t q : G.qs)
      G.vis.push_back(ch[v].empty() ? G.kv_len - (qpl - 1 - q % qpl) : G.kv_len);
    G.rows = int32_t(G.qs.size()) * g;
    group_of[v] = int32_t(groups.size());
    groups.push_back(std::move(G));
  }

  // ---- P6 / P7
  for (auto& G : groups) {
    G.cls = G.rows <= p.stream_rows ? 0 : 1;
    if (G.cls == 0) {
      G.nblocks = 1;
      G.rb = G.rows;
    } else {  // balanced blocks of at most rb rows, 16-aligned when rb is
      const int64_t nb = cdiv(G.rows, p.rb);
      G.rb = int32_t(align_up(cdiv(G.rows, nb), p.rb % 16 == 0 ? 16 : 1));
      G.nblocks = int32_t(cdiv(G.rows, G.rb));
    }
  }
  int64_t c_glob = 0;
  if (p.split) {
    int64_t W = 0;
    for (auto& G : groups) W += int64_t(G.cls == 0 ? 3 : kBlockWaveWeight3) * G.nblocks * G.kv_len;
    W *= H;
    const int64_t U = cdiv(W, int64_t(p.ncu) * p.waves * 3);
    c_glob = std::max<int64_t>(p.split_align, align_up(U, p.split_align));
  }
  struct Chunk { int32_t group, t0, t1; };
  std::vector<Chunk> chunks;
  for (int32_t gi = 0; gi < int32_t(groups.size()); ++gi) {
    Group& G = groups[gi];
    int64_t csz, nch;
    if (p.split) {
      const int64_t cg =
          std::max<int64_t>(c_glob, align_up(int64_t(p.floor_f) * std::min(G.rows, G.rb), p.split_align));
      nch = cdiv(G.kv_len, cg);
      csz = align_up(cdiv(G.kv_len, nch), kChunkAlign);
      nch = cdiv(G.kv_len, csz);
    } else {
      csz = G.kv_len;
      nch = 1;
    }
    G.chunk_ptr = int32_t(chunks.size());
    G.n_chunks = int32_t(nch);
    for (int64_t i = 0; i < nch; ++i)
      chunks.push_back({gi, int32_t(i * csz), int32_t(std::min<int64_t>(G.kv_len, (i + 1) * csz))});
  }

  // ---- P8 items (longest first; stable on natural order)
  struct Item { int64_t est; int32_t group, row0, nrows, chunk, cls; };
  std::vector<Item> items;
  for (int32_t gi = 0; gi < int32_t(groups.size()); ++gi) {
    const Group& G = groups[gi];
    for (int32_t b = 0; b < G.nblocks; ++b) {
      const int32_t r0 = b * G.rb;
      const int32_t nr = std::min(G.rows, r0 + G.rb) - r0;
      for (int32_t c = 0; c < G.n_chunks; ++c) {
        const Chunk& C = chunks[G.chunk_ptr + c];
        items.push_back(
            {int64_t(C.t1 - C.t0) * (kItemFixedCost + nr), gi, r0, nr, G.chunk_ptr + c, G.cls});
      }
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
    if (a.cls != b.cls) return a.cls > b.cls;
    return a.est > b.est;
  });
  int32_t n_stream = 0;
  for (const Item& I : items) n_stream += I.cls == 0 ? 1 : 0;

  // ---- P9 slots
  int32_t slot = 0;
  for (auto& G : groups) {
    G.slot_base = slot;
    slot += G.n_chunks * int32_t(G.qs.size());
  }
  const int32_t n_slots = slot;
  std::vector<std::vector<int32_t>> qsl(n_q);
  for (int32_t lf : leaves) {
    std::vector<int32_t> path;
    for (int32_t u = lf; u != -1; u = parent[u]) path.push_back(u);
    std::reverse(path.begin(), path.end());
    for (size_t k = 0; k < path.size(); ++k) {
      const int32_t u = path[k];
      const bool stop = (u == lf) || f[path[k + 1]] == 0;
      if (!stop) continue;
      const Group& G = groups[group_of[u]];
      for (int32_t j = 0; j < qpl; ++j) {
        const int32_t q = leaf_rank[lf] * qpl + j;
        const int32_t jj =
            int32_t(std::lower_bound(G.qs.begin(), G.qs.end(), q) - G.qs.begin());
        for (int32_t c = 0; c < G.n_chunks; ++c)
          qsl[q].push_back(G.slot_base + c * int32_t(G.qs.size()) + jj);
      }
    }
  }

  // ---- P10 page runs + per-token page table
  PlanTables& T = *out;
  T = PlanTables{};
  T.chunk_run_ptr.push_back(0);
  for (auto& G : groups) {
    G.seg_base = int32_t(T.seg_tok.size());
    T.group_seg_base.push_back(G.seg_base);
    for (int32_t u : G.seg)
      for (int32_t t = 0; t < node_len[u]; ++t) {
        const int32_t pg = node_page_ids[node_page_ptr[u] + t / page_size];
        T.seg_tok.push_back((pg << 8) | (t % page_size));
      }
  }
  for (const Chunk& C : chunks) {
    const Group& G = groups[C.group];
    int32_t pos = 0;
    int32_t cur_page = -1, cur_slot = -1, cur_n = 0, cur_node = -1;
    for (int32_t u : G.seg) {
      const int32_t lu = node_len[u];
      if (pos + lu <= C.t0 || pos >= C.t1) {
        pos += lu;
        continue;
      }
      for (int32_t t = std::max(0, C.t0 - pos); t < lu && pos + t < C.t1; ++t) {
        const int32_t pg = node_page_ids[node_page_ptr[u] + t / page_size];
        const int32_t sl = t % page_size;
        if (cur_n > 0 && pg == cur_page && cur_slot + cur_n == sl && cur_node == u) {
          ++cur_n;
        } else {
          if (cur_n > 0) {
            T.runs.push_back(cur_page);
            T.runs.push_back(cur_slot);
            T.runs.push_back(cur_n);
          }
          cur_page = pg;
          cur_slot = sl;
          cur_n = 1;
          cur_node = u;
        }
      }
      pos += lu;
    }
    T.runs.push_back(cur_page);
    T.runs.push_back(cur_slot);
    T.runs.push_back(cur_n);
    T.chunk_run_ptr.push_back(int32_t(T.runs.size() / 3));
  }

  // ---- export
  T.params = {kFormatVersion, n, n_q, qpl, n_qheads, n_kvheads, head_dim, page_size,
              p.ts_q, p.ts_c, p.gamma, p.rb, p.waves, p.floor_f, p.ncu, p.split ? 1 : 0,
              p.force_edges ? 1 : 0, kChunkAlign, int32_t(groups.size()), int32_t(chunks.size()),
              int32_t(items.size()), n_slots, int32_t(c_glob), int32_t(T.runs.size() / 3),
              p.stream_rows, n_stream, p.split_align};
  T.edges = f;
  T.nq = nQ;
  T.lcum.assign(n, 0);
  for (int32_t v = 0; v < n; ++v) T.lcum[v] = int32_t(L[v]);
  for (auto& G : groups) {
    G.q_ptr = int32_t(T.group_qs.size());
    T.groups.insert(T.groups.end(), {G.node, G.top, G.kv_len, int32_t(G.qs.size()), G.q_ptr,
                                     G.chunk_ptr, G.n_chunks, G.slot_base});
    T.group_qs.insert(T.group_qs.end(), G.qs.begin(), G.qs.end());
    T.group_vis.insert(T.group_vis.end(), G.vis.begin(), G.vis.end());
  }
  for (const Chunk& C : chunks) T.chunks.insert(T.chunks.end(), {C.group, C.t0, C.t1});
  for (const Item& I : items) T.items.insert(T.items.end(), {I.group, I.row0, I.nrows, I.chunk, I.cls});
  T.q_slot_ptr.push_back(0);
  for (int32_t q = 0; q < n_q; ++q) {
    T.q_slots.insert(T.q_slots.end(), qsl[q].begin(), qsl[q].end());
    T.q_slot_ptr.push_back(int32_t(T.q_slots.size()));
  }
  T.bfs = bfs;
  T.n_queries = n_q;
  T.n_groups = int32_t(groups.size());
  T.n_chunks = int32_t(chunks.size());
  T.n_items = int32_t(items.size());
  T.n_stream_items = n_stream;
  T.n_slots = n_slots;
  T.max_page_id = max_page;
  return 0;
}

}  // namespace ta
