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
//      intermediate result gamma * nQ_l, gamma = 128 g by default) with
//      joining it (SplitQCost: v keeps
//      nQ_curr - nQ_l queries, l reads len_l + len_v); assign 1 iff C0 >= C1.
//      Padding cost C_P(n, len) = Pad(TS_q, n) * len + n * Pad(TS_c, min(len, TS_c))
//      with Pad(TS, N) = TS - ((N - 1) % TS + 1) (section 3.2 cost model; the
//      common factor d dropped, Pad(TS, 0) = 0).
//  P5  one group per virtual node with queries left (DeFT notes, KV-guided
//      split: a node's KV grouped with every query that shares it).
//  P6  item class and row blocks: a group with at most stream_rows rows is
//      one single-wave stream block (unless tile_join and the plan has
//      workgroup items and the group fills a 16-row tile: then it joins
//      them, so a launch holds one item class where the rows allow); a
//      larger one is cut into balanced workgroup blocks of at most rb rows
//      (16-aligned when rb is). Row r = (query r / g, q-head r % g).
//  P7  long-context split (FastTree review, section 3.3): a global chunk
//      length sized so the launch gives about ncu * waves busy waves (a
//      workgroup block counts as kBlockWaveWeight3 / 3 waves: its four waves
//      share each staged tile), a multiple of split_align, stepped down while
//      the launch would hold fewer units than compute units, floored per
//      group at floor_f tokens per row; each group's chunks are then balanced
//      and 16-aligned.
//  P8  work items: workgroup items first, then stream items, each class
//      longest first (stable).
//  P9  partial-result slots: group, then chunk, then query.
//  P10 page runs of every chunk and the per-token page table the kernel reads.
//
// Group membership, rows and row blocks depend only on the tree and the edge
// assignment, so plan_init does P0-P6 once and plan_layout redoes the
// length-dependent steps; a decode loop (every leaf gains tokens each step)
// keeps the edges and only re-lays out (plan_extend + plan_layout).
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

int fail(std::string* err, int code, const char* msg) {
  *err = msg;
  return code;
}

constexpr int EINVAL_ = 1, EUNSUP_ = 4;
constexpr int64_t kMaxTokens = int64_t(1) << 30;
constexpr int32_t kMaxPageId = 1 << 23;

// Page-table slack of a growing group laid out after an extend: room for at
// least 256 more tokens (a quarter of the segment for long ones).
inline int64_t seg_slack(int64_t kv_len) { return align_up(std::max<int64_t>(256, kv_len / 4), 16); }

// Page-table words of positions [a, b) of group G's segment.
void fill_segment(const PlanState& S, const PlanGroup& G, int32_t a, int32_t b, std::vector<int32_t>& seg_tok) {
  const int32_t ps = S.page_size;
  int64_t pos = 0;
  for (int32_t u : G.seg) {
    const int32_t lu = S.len[u];
    if (pos + lu > a) {
      const std::vector<int32_t>& pg = S.pages[u];
      for (int32_t t = int32_t(std::max<int64_t>(0, a - pos)); t < lu && pos + t < b; ++t)
        seg_tok[size_t(G.seg_base + pos + t)] = (pg[t / ps] << 8) | (t % ps);
    }
    pos += lu;
    if (pos >= b) break;
  }
}

}  // namespace

int plan_init(const int32_t* parent, int32_t n, const int32_t* node_len,
              const int32_t* node_page_ptr, const int32_t* node_page_ids, int32_t page_size,
              int32_t qpl, int32_t n_qheads, int32_t n_kvheads, int32_t head_dim,
              const PlanParams& p, PlanState* out, std::string* err) {
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
      p.ncu < 1 || p.stream_rows < 0 || p.stream_rows > kTileRows || p.split_align < 16 || p.split_align % 16)
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
  PlanState S;
  S.p = p;
  S.p.force_edges = nullptr;
  if (S.p.gamma == 0)
    S.p.gamma = int32_t(std::min<int64_t>(INT32_MAX, int64_t(kGammaPerGroupHead) * (n_qheads / n_kvheads)));
  S.n = n;
  S.root = root;
  S.qpl = qpl;
  S.n_qheads = n_qheads;
  S.n_kvheads = n_kvheads;
  S.head_dim = head_dim;
  S.page_size = page_size;
  S.g = n_qheads / n_kvheads;
  S.edges_mode = p.force_edges ? kEdgesForced : kEdgesGreedy;
  S.parent.assign(parent, parent + n);
  S.len.assign(node_len, node_len + n);
  // ---- P1 (children as CSR, ascending id)
  S.ch_ptr.assign(size_t(n) + 1, 0);
  for (int32_t v = 0; v < n; ++v)
    if (parent[v] >= 0) ++S.ch_ptr[size_t(parent[v]) + 1];
  for (int32_t v = 0; v < n; ++v) S.ch_ptr[size_t(v) + 1] += S.ch_ptr[v];
  S.ch.assign(size_t(S.ch_ptr[n]), 0);
  {
    std::vector<int32_t> fill(S.ch_ptr.begin(), S.ch_ptr.end() - 1);
    for (int32_t v = 0; v < n; ++v)
      if (parent[v] >= 0) S.ch[size_t(fill[parent[v]]++)] = v;
  }
  auto is_leaf = [&S](int32_t v) { return S.ch_ptr[v] == S.ch_ptr[size_t(v) + 1]; };
  for (int32_t v = 0; v < n; ++v) {
    if (node_len[v] < 1) return fail(err, EINVAL_, "tree_attn_plan: node length < 1");
    if (is_leaf(v) && node_len[v] < qpl)
      return fail(err, EINVAL_, "tree_attn_plan: leaf shorter than queries_per_leaf");
    S.total_tokens += node_len[v];
  }
  if (S.total_tokens >= kMaxTokens) return fail(err, EINVAL_, "tree_attn_plan: too many tokens");
  if (node_page_ptr[0] != 0) return fail(err, EINVAL_, "tree_attn_plan: node_page_ptr[0] != 0");
  for (int32_t v = 0; v < n; ++v)
    if (int64_t(node_page_ptr[v + 1]) - node_page_ptr[v] != cdiv(node_len[v], page_size))
      return fail(err, EINVAL_, "tree_attn_plan: node page count != ceil(len / page_size)");
  for (int32_t i = 0; i < node_page_ptr[n]; ++i) {
    if (node_page_ids[i] < 0 || node_page_ids[i] >= kMaxPageId)
      return fail(err, EINVAL_, "tree_attn_plan: page id out of range [0, 2^23)");
    S.max_page = std::max(S.max_page, node_page_ids[i]);
  }
  S.pages.resize(size_t(n));
  for (int32_t v = 0; v < n; ++v)
    S.pages[v].assign(node_page_ids + node_page_ptr[v], node_page_ids + node_page_ptr[v + 1]);
  S.leaf_rank.assign(size_t(n), -1);
  for (int32_t v = 0; v < n; ++v)
    if (is_leaf(v)) {
      S.leaf_rank[v] = int32_t(S.leaves.size());
      S.leaves.push_back(v);
    }
  S.n_q = int32_t(S.leaves.size()) * qpl;

  // ---- P3 (BFS) then P2 (A, bottom-up over reversed BFS)
  S.bfs.reserve(size_t(n));
  {
    std::deque<int32_t> dq{root};
    while (!dq.empty()) {
      int32_t v = dq.front();
      dq.pop_front();
      S.bfs.push_back(v);
      for (int32_t x = S.ch_ptr[v]; x < S.ch_ptr[v + 1]; ++x) dq.push_back(S.ch[x]);
    }
  }
  S.A.assign(size_t(n), 0);
  for (auto it = S.bfs.rbegin(); it != S.bfs.rend(); ++it) {
    const int32_t v = *it;
    if (is_leaf(v)) S.A[v] = qpl;
    else
      for (int32_t x = S.ch_ptr[v]; x < S.ch_ptr[v + 1]; ++x) S.A[v] += S.A[S.ch[x]];
  }

  // ---- P4 greedy
  std::vector<int64_t> L(node_len, node_len + n);
  S.f.assign(size_t(n), 0);
  S.nq.assign(size_t(n), 0);
  for (int32_t v : S.bfs) {
    int64_t nq_curr = S.A[v];
    const int64_t len_v = L[v];
    for (int32_t x = S.ch_ptr[v]; x < S.ch_ptr[v + 1]; ++x) {
      const int32_t l = S.ch[x];
      const int64_t nq_l = S.A[l], len_l = L[l];
      int32_t assign;
      if (p.force_edges) {
        assign = p.force_edges[l] ? 1 : 0;
      } else {
        const int64_t c0 = pad_cost(nq_curr, len_v, p.ts_q, p.ts_c) +
                           pad_cost(nq_l, len_l, p.ts_q, p.ts_c) + int64_t(S.p.gamma) * nq_l;
        const int64_t c1 = pad_cost(nq_curr - nq_l, len_v, p.ts_q, p.ts_c) +
                           pad_cost(nq_l, len_l + len_v, p.ts_q, p.ts_c);
        assign = (c0 >= c1) ? 1 : 0;
      }
      S.f[l] = assign;
      if (assign) {
        nq_curr -= nq_l;
        L[l] = len_l + len_v;
      }
    }
    S.nq[v] = int32_t(nq_curr);
  }

  // ---- P5 group membership
  std::vector<int32_t> top(size_t(n), 0), group_of(size_t(n), -1);
  for (int32_t v : S.bfs) top[v] = (v == root || S.f[v] == 0) ? v : top[parent[v]];
  for (int32_t v : S.bfs) {
    if (S.nq[v] == 0) continue;
    PlanGroup G;
    G.node = v;
    G.top = top[v];
    G.grows = is_leaf(v);
    // queries: the leaf's own, plus those below children kept apart (edge 0)
    if (is_leaf(v))
      for (int32_t j = 0; j < qpl; ++j) G.qs.push_back(S.leaf_rank[v] * qpl + j);
    std::vector<int32_t> stack;
    for (int32_t x = S.ch_ptr[v]; x < S.ch_ptr[v + 1]; ++x)
      if (S.f[S.ch[x]] == 0) stack.push_back(S.ch[x]);
    while (!stack.empty()) {
      const int32_t u = stack.back();
      stack.pop_back();
      if (is_leaf(u))
        for (int32_t j = 0; j < qpl; ++j) G.qs.push_back(S.leaf_rank[u] * qpl + j);
      for (int32_t x = S.ch_ptr[u]; x < S.ch_ptr[u + 1]; ++x) stack.push_back(S.ch[x]);
    }
    std::sort(G.qs.begin(), G.qs.end());
    if (int32_t(G.qs.size()) != S.nq[v]) return fail(err, EINVAL_, "tree_attn_plan: internal query count");
    for (int32_t u = v;; u = parent[u]) {
      G.seg.push_back(u);
      if (u == G.top) break;
    }
    std::reverse(G.seg.begin(), G.seg.end());
    G.rows = int32_t(G.qs.size()) * S.g;
    group_of[v] = int32_t(S.groups.size());
    S.groups.push_back(std::move(G));
  }
  // ---- P6 item class and row blocks
  bool has_wg = false;
  for (const PlanGroup& G : S.groups) has_wg = has_wg || G.rows > p.stream_rows;
  for (PlanGroup& G : S.groups) {
    const bool single = G.rows <= p.stream_rows && !(p.tile_join && has_wg && G.rows >= kTileRows);
    G.cls = single ? 0 : 1;
    if (G.cls == 0) {
      G.nblocks = 1;
      G.rb = G.rows;
    } else {  // as few blocks of at most rb rows as possible, even in whole tiles
      G.tile = p.rb % kTileRows == 0 ? kTileRows : 1;
      G.nblocks = int32_t(cdiv(G.rows, p.rb));
      G.rb = int32_t(std::min<int64_t>(G.rows, cdiv(cdiv(G.rows, G.tile), G.nblocks) * G.tile));
    }
  }

  // ---- P9 structure: the groups each leaf's queries read, root side first
  S.path_ptr.push_back(0);
  for (int32_t lf : S.leaves) {
    std::vector<int32_t> path;
    for (int32_t u = lf; u != -1; u = parent[u]) path.push_back(u);
    std::reverse(path.begin(), path.end());
    for (size_t k = 0; k < path.size(); ++k) {
      const int32_t u = path[k];
      const bool stop = (u == lf) || S.f[path[k + 1]] == 0;
      if (!stop) continue;
      const PlanGroup& G = S.groups[group_of[u]];
      const int32_t q0 = S.leaf_rank[lf] * qpl;
      S.path_group.push_back(group_of[u]);
      S.path_jj.push_back(int32_t(std::lower_bound(G.qs.begin(), G.qs.end(), q0) - G.qs.begin()));
    }
    S.path_ptr.push_back(int32_t(S.path_group.size()));
  }
  *out = std::move(S);
  return 0;
}

// Row block b of a group: a workgroup group's rows in whole tiles of G.tile
// rows, spread over its blocks as evenly as the tiles allow (the first
// tiles % nblocks blocks take one tile more); the last block ends at the
// group's last row.
static void row_block(const PlanGroup& G, int32_t b, int32_t* r0, int32_t* nr) {
  if (G.cls == 0) {
    *r0 = 0;
    *nr = G.rows;
    return;
  }
  const int32_t T = int32_t(cdiv(G.rows, G.tile)), base = T / G.nblocks, extra = T % G.nblocks;
  const int32_t t0 = b * base + std::min(b, extra), nt = base + (b < extra ? 1 : 0);
  *r0 = t0 * G.tile;
  *nr = std::min(G.rows, *r0 + nt * G.tile) - *r0;
}

void plan_layout(PlanState& S, PlanTables& T) {
  const PlanParams& p = S.p;
  const int32_t n = S.n, qpl = S.qpl;
  const int64_t H = S.n_kvheads;
  // ---- P5 lengths: context along joined edges, visible prefixes
  S.L.assign(size_t(n), 0);
  for (int32_t v : S.bfs) S.L[v] = S.len[v] + ((v != S.root && S.f[v]) ? S.L[S.parent[v]] : 0);
  for (PlanGroup& G : S.groups) {
    G.kv_len = int32_t(S.L[G.node]);
    G.vis.resize(G.qs.size());
    for (size_t x = 0; x < G.qs.size(); ++x)
      G.vis[x] = G.grows ? G.kv_len - (qpl - 1 - G.qs[x] % qpl) : G.kv_len;
  }

  // ---- P7 chunks
  // a group's chunk length and count under global chunk cg_glob: at least the
  // group's floor, then balanced pieces, 16-aligned
  auto chunking = [&](const PlanGroup& G, int64_t cg_glob, int64_t* csz, int64_t* nch) {
    const int64_t cg =
        std::max<int64_t>(cg_glob, align_up(int64_t(p.floor_f) * std::min(G.rows, G.rb), p.split_align));
    *nch = cdiv(G.kv_len, cg);
    *csz = align_up(cdiv(G.kv_len, *nch), kChunkAlign);
    *nch = cdiv(G.kv_len, *csz);
  };
  int64_t c_glob = 0;
  if (p.split) {
    int64_t W = 0;
    for (const PlanGroup& G : S.groups) W += int64_t(G.cls == 0 ? 3 : kBlockWaveWeight3) * G.nblocks * G.kv_len;
    W *= H;
    const int64_t U = cdiv(W, int64_t(p.ncu) * p.waves * 3);
    c_glob = std::max<int64_t>(p.split_align, align_up(U, p.split_align));
    // the launch fills the GPU (review 3.3): while it would hold fewer units
    // (item x kv-head) than compute units, the global chunk steps down by one
    // alignment
    auto units = [&](int64_t cg_glob) {
      int64_t u = 0, csz, nch;
      for (const PlanGroup& G : S.groups) {
        chunking(G, cg_glob, &csz, &nch);
        u += int64_t(G.nblocks) * nch;
      }
      return u * H;
    };
    while (c_glob > p.split_align && units(c_glob) < p.ncu) c_glob -= p.split_align;
  }
  T.chunks.clear();
  for (int32_t gi = 0; gi < int32_t(S.groups.size()); ++gi) {
    PlanGroup& G = S.groups[gi];
    int64_t csz, nch;
    if (p.split) {
      chunking(G, c_glob, &csz, &nch);
    } else {
      csz = G.kv_len;
      nch = 1;
    }
    G.chunk_ptr = int32_t(T.chunks.size() / 3);
    G.n_chunks = int32_t(nch);
    for (int64_t i = 0; i < nch; ++i)
      T.chunks.insert(T.chunks.end(),
                      {gi, int32_t(i * csz), int32_t(std::min<int64_t>(G.kv_len, (i + 1) * csz))});
  }
  const int32_t n_chunks = int32_t(T.chunks.size() / 3);

  // ---- P8 items (longest first; stable on natural order)
  struct Item { int64_t est; int32_t group, row0, nrows, chunk, cls; };
  std::vector<Item> items;
  for (int32_t gi = 0; gi < int32_t(S.groups.size()); ++gi) {
    const PlanGroup& G = S.groups[gi];
    for (int32_t b = 0; b < G.nblocks; ++b) {
      int32_t r0, nr;
      row_block(G, b, &r0, &nr);
      for (int32_t c = 0; c < G.n_chunks; ++c) {
        const int32_t ci = G.chunk_ptr + c;
        items.push_back({int64_t(T.chunks[3 * ci + 2] - T.chunks[3 * ci + 1]) * (kItemFixedCost + nr), gi, r0, nr,
                         ci, G.cls});
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
  for (PlanGroup& G : S.groups) {
    G.slot_base = slot;
    slot += G.n_chunks * int32_t(G.qs.size());
  }
  const int32_t n_slots = slot;
  T.q_slot_ptr.assign(1, 0);
  T.q_slots.clear();
  for (size_t r = 0; r < S.leaves.size(); ++r)
    for (int32_t j = 0; j < qpl; ++j) {
      for (int32_t x = S.path_ptr[r]; x < S.path_ptr[r + 1]; ++x) {
        const PlanGroup& G = S.groups[S.path_group[x]];
        const int32_t jj = S.path_jj[x] + j;
        for (int32_t c = 0; c < G.n_chunks; ++c) T.q_slots.push_back(G.slot_base + c * int32_t(G.qs.size()) + jj);
      }
      T.q_slot_ptr.push_back(int32_t(T.q_slots.size()));
    }

  // ---- P10 per-token page table (each group's region; growing groups get
  // slack once the plan has been extended, so later steps append in place)
  bool relay = T.seg_tok.empty() || T.group_seg_base.size() != S.groups.size();
  for (const PlanGroup& G : S.groups) relay = relay || G.kv_len > G.seg_cap;
  T.seg_dirty.clear();
  T.seg_relaid = relay;
  if (relay) {
    int64_t pos = 0;
    for (PlanGroup& G : S.groups) {
      G.seg_base = int32_t(pos);
      G.seg_cap = int32_t(G.kv_len + ((S.extended && G.grows) ? seg_slack(G.kv_len) : 0));
      G.seg_filled = 0;
      pos += G.seg_cap + kSegGuard;
    }
    T.seg_tok.assign(size_t(pos), 0);
  }
  T.group_seg_base.resize(S.groups.size());
  for (size_t gi = 0; gi < S.groups.size(); ++gi) {
    PlanGroup& G = S.groups[gi];
    T.group_seg_base[gi] = G.seg_base;
    if (G.seg_filled < G.kv_len) {
      fill_segment(S, G, G.seg_filled, G.kv_len, T.seg_tok);
      if (!relay) T.seg_dirty.insert(T.seg_dirty.end(), {G.seg_base + G.seg_filled, G.seg_base + G.kv_len});
      G.seg_filled = G.kv_len;
    }
    if (relay) {  // slack and guard repeat the last token (growth overwrites the slack in place)
      const int32_t lastw = T.seg_tok[size_t(G.seg_base + G.kv_len - 1)];
      std::fill(T.seg_tok.begin() + G.seg_base + G.kv_len, T.seg_tok.begin() + G.seg_base + G.seg_cap + kSegGuard,
                lastw);
    }
  }
  // page runs per chunk: counted here (a run is the part of one page of one
  // node inside the chunk), expanded by plan_runs on demand
  int64_t n_runs = 0;
  for (int32_t ci = 0; ci < n_chunks; ++ci) {
    const PlanGroup& G = S.groups[T.chunks[3 * ci]];
    const int64_t t0 = T.chunks[3 * ci + 1], t1 = T.chunks[3 * ci + 2];
    int64_t pos = 0;
    for (int32_t u : G.seg) {
      const int64_t lu = S.len[u];
      const int64_t a = std::max<int64_t>(0, t0 - pos), b = std::min<int64_t>(lu, t1 - pos);
      if (a < b) n_runs += (b - 1) / S.page_size - a / S.page_size + 1;
      pos += lu;
    }
  }
  T.runs.clear();
  T.chunk_run_ptr.clear();
  T.runs_valid = false;

  // ---- export
  T.params = {kFormatVersion, n, S.n_q, qpl, S.n_qheads, S.n_kvheads, S.head_dim, S.page_size,
              p.ts_q, p.ts_c, p.gamma, p.rb, p.waves, p.floor_f, p.ncu, p.split ? 1 : 0,
              S.edges_mode, kChunkAlign, int32_t(S.groups.size()), n_chunks,
              int32_t(items.size()), n_slots, int32_t(c_glob), int32_t(n_runs),
              p.stream_rows, n_stream, p.split_align, p.tile_join ? 1 : 0};
  T.edges = S.f;
  T.nq = S.nq;
  T.lcum.resize(size_t(n));
  for (int32_t v = 0; v < n; ++v) T.lcum[v] = int32_t(S.L[v]);
  T.groups.clear();
  T.group_qs.clear();
  T.group_vis.clear();
  for (PlanGroup& G : S.groups) {
    G.q_ptr = int32_t(T.group_qs.size());
    T.groups.insert(T.groups.end(), {G.node, G.top, G.kv_len, int32_t(G.qs.size()), G.q_ptr,
                                     G.chunk_ptr, G.n_chunks, G.slot_base});
    T.group_qs.insert(T.group_qs.end(), G.qs.begin(), G.qs.end());
    T.group_vis.insert(T.group_vis.end(), G.vis.begin(), G.vis.end());
  }
  T.items.clear();
  for (const Item& I : items) T.items.insert(T.items.end(), {I.group, I.row0, I.nrows, I.chunk, I.cls});
  T.bfs = S.bfs;
  T.n_queries = S.n_q;
  T.n_groups = int32_t(S.groups.size());
  T.n_chunks = n_chunks;
  T.n_items = int32_t(items.size());
  T.n_stream_items = n_stream;
  T.n_slots = n_slots;
  T.max_page_id = S.max_page;
}

void plan_runs(const PlanState& S, PlanTables& T) {
  T.runs.clear();
  T.chunk_run_ptr.assign(1, 0);
  const int32_t ps = S.page_size;
  for (int32_t ci = 0; ci < T.n_chunks; ++ci) {
    const PlanGroup& G = S.groups[T.chunks[3 * ci]];
    const int32_t t0 = T.chunks[3 * ci + 1], t1 = T.chunks[3 * ci + 2];
    int32_t pos = 0;
    int32_t cur_page = -1, cur_slot = -1, cur_n = 0, cur_node = -1;
    for (int32_t u : G.seg) {
      const int32_t lu = S.len[u];
      if (pos + lu <= t0 || pos >= t1) {
        pos += lu;
        continue;
      }
      for (int32_t t = std::max(0, t0 - pos); t < lu && pos + t < t1; ++t) {
        const int32_t pg = S.pages[u][t / ps];
        const int32_t sl = t % ps;
        if (cur_n > 0 && pg == cur_page && cur_slot + cur_n == sl && cur_node == u) {
          ++cur_n;
        } else {
          if (cur_n > 0) T.runs.insert(T.runs.end(), {cur_page, cur_slot, cur_n});
          cur_page = pg;
          cur_slot = sl;
          cur_n = 1;
          cur_node = u;
        }
      }
      pos += lu;
    }
    T.runs.insert(T.runs.end(), {cur_page, cur_slot, cur_n});
    T.chunk_run_ptr.push_back(int32_t(T.runs.size() / 3));
  }
  T.runs_valid = true;
}

int plan_extend(PlanState& S, const int32_t* leaf_add, const int32_t* new_pages, int64_t n_new_pages,
                std::string* err) {
  const int32_t nl = int32_t(S.leaves.size());
  if (!leaf_add || (n_new_pages > 0 && !new_pages) || n_new_pages < 0)
    return fail(err, EINVAL_, "tree_attn_plan_extend: null array or negative page count");
  int64_t add_total = 0, need = 0;
  for (int32_t r = 0; r < nl; ++r) {
    if (leaf_add[r] < 0) return fail(err, EINVAL_, "tree_attn_plan_extend: negative token count");
    const int64_t old_len = S.len[S.leaves[r]], new_len = old_len + leaf_add[r];
    add_total += leaf_add[r];
    if (add_total >= kMaxTokens) return fail(err, EINVAL_, "tree_attn_plan_extend: too many tokens");
    need += cdiv(new_len, S.page_size) - cdiv(old_len, S.page_size);
  }
  if (S.total_tokens + add_total >= kMaxTokens) return fail(err, EINVAL_, "tree_attn_plan_extend: too many tokens");
  if (need != n_new_pages)
    return fail(err, EINVAL_, "tree_attn_plan_extend: new page count != pages the growth needs");
  for (int64_t i = 0; i < n_new_pages; ++i)
    if (new_pages[i] < 0 || new_pages[i] >= kMaxPageId)
      return fail(err, EINVAL_, "tree_attn_plan_extend: page id out of range [0, 2^23)");
  int64_t at = 0;
  for (int32_t r = 0; r < nl; ++r) {
    const int32_t v = S.leaves[r];
    const int64_t old_pages = cdiv(S.len[v], S.page_size);
    S.len[v] += leaf_add[r];
    const int64_t k = cdiv(S.len[v], S.page_size) - old_pages;
    for (int64_t x = 0; x < k; ++x) {
      S.pages[v].push_back(new_pages[at]);
      S.max_page = std::max(S.max_page, new_pages[at]);
      ++at;
    }
  }
  S.total_tokens += add_total;
  if (S.edges_mode == kEdgesGreedy) S.edges_mode = kEdgesKept;
  S.extended = true;
  return 0;
}

}  // namespace ta
