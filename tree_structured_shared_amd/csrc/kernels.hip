// HIP kernels for tree-structured decode attention on CDNA4 (gfx950).
//
// Partial attention. A work item is one KV chunk of one context-query group
// and a block of its rows (row = query x q-head-in-group). The item's chunk of
// paged K/V is streamed once for all its rows -- the KV-guided grouping of the
// DeFT reading notes and the single-launch kernel of the FastTree review
// (section 3, kernel design: every group dispatched to its own blocks of one
// launch) -- with a flash-style online softmax over 32-token tiles (DeFT
// notes, attention calculation; FastTree review, tile-by-tile online softmax).
// Each row ends in one partial (m, l, o) in the workspace: o unnormalised in
// fp32, or, when every |o / l| of the row is below 1, o / l as fp16 in the
// first half of the row's record with l stored negated (the reduction reads
// the sign). The fp16 form rounds each value by at most 2^-12, a convex
// combination of them moves the output by no more, and it halves the
// partial results written and read back. A query whose path is one partial
// (one group, one chunk) needs no merge: its rows write the normalised
// output directly and the reduction skips it.
//
// One launch (partial_kernel) holds both item classes, chosen per group by
// its row count (the review's multi-stage query tiling: small tiles near the
// leaves, large ones near the root):
//  * workgroup items (many rows): one workgroup per item x kv-head. bf16:
//    the workgroup streams each K/V tile once into LDS with direct loads
//    (kLdsStages stages, one barrier per tile); up to 64 rows, wave w
//    computes 16-row tile w from it, above that (up to 128 rows) one 32-row
//    tile each on the 32x32 matrix instruction. fp32: each wave runs the
//    GEMV path on row pairs.
//  * single-wave items (up to 16 rows): each wave is one item x kv-head and
//    streams its chunk alone with two tiles in flight.
// A plan holds one class where its rows allow (the planner's tile join), so
// most launches are of one kind.
//
// kv append: the new tokens' K/V rows scattered into their pool pages (the
// step before a decode).
// Row arithmetic:
//  * bf16: v_mfma_f32_16x16x32_bf16 on a transposed formulation, 16-row
//    tiles (padded for fewer rows: the items are bound by their K/V stream).
//    S^T = K Q^T: K rows are the A operand (straight from the pool, or from
//    LDS). O^T = V^T P^T: the score accumulators already sit in the B-operand
//    layout of P^T; V^T comes from a v_perm transpose of 16-byte V reads
//    (single-wave items) or from LDS transpose reads (workgroup items)
//    (stacking the queries that share KV turns the decode GEMV into a GEMM,
//    FastTree review, kernel design).
//  * fp32: wavefront dot products (GEMV), 8 lanes per token, DPP reductions,
//    per-lane online softmax.
//
// lse_reduce: per (query, q-head), merges that query's partials along its
// path (root-side group first, chunks ascending) by log-sum-exp -- the
// tree-topology-aware global reduction of the DeFT notes.
//
// Softmax runs in base 2: scores are scaled by scale * log2(e) and the
// workspace m is in those units. The running max is only raised when a new
// score exceeds it by more than 8 (log2 units), so rescaling is rare; l and o
// always stay relative to the stored m.
#include "kernels.h"
#include "planner.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

namespace ta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 256;
constexpr int kWaves = 4;
constexpr int kBlockRowTiles = 2; // rows per wave in a workgroup pass, in 16-row tiles
constexpr float kRescale = 8.0f;  // lazy-rescale threshold, log2 units
// a row tile's weights enter P V as a bf16 hi + lo pair when some row's
// largest weight of the tile exceeds this share of its running sum
// (including the tile)
constexpr float kLoFrac = 0.125f;
// initial running max of the MFMA path: finite, so exp2(s - m) of a masked
// score (-inf) is 0 even before any score was seen, with no extra guard;
// exp2(kMInit - anything finite) is 0, so the first real max replaces it.
constexpr float kMInit = -1.0e30f;
#define TA_NEG_INF (-__builtin_inff())

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte offset of a pool token from its page-table entry (page << 8 | slot).
// FA: every offset fits 32 bits and both byte strides fit 24 bits, so two
// full-rate 24-bit multiplies do it and loads take the uniform-base +
// 32-bit-offset addressing form.
template <bool FA>
struct TokOff;
template <>
struct TokOff<true> {
  typedef uint32_t type;
  static __device__ __forceinline__ uint32_t of(int32_t st, const PartialArgs& a) {
    return __umul24(uint32_t(st) >> 8, uint32_t(a.sp_bytes)) + __umul24(uint32_t(st) & 255u, uint32_t(a.st_bytes));
  }
};
template <>
struct TokOff<false> {
  typedef int64_t type;
  static __device__ __forceinline__ int64_t of(int32_t st, const PartialArgs& a) {
    return int64_t(st >> 8) * a.sp_bytes + int64_t(st & 255) * a.st_bytes;
  }
};

template <typename V, typename O>
__device__ __forceinline__ V load_at(const char* base, O off) {
  return *reinterpret_cast<const V*>(base + off);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (VALU only: DPP and the gfx950 permlane swaps).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// all-reduce sum over each aligned group of 8 lanes: quad_perm xor 1, xor 2,
// then row_half_mirror pairs the two quads of the group
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v;
}
// value of lane l ^ 8 (row_ror:8 inside each 16-lane row)
__device__ __forceinline__ float xor8(float v) { return dpp_mov<0x128>(v); }
// value of lane l ^ 16 / l ^ 32: each permlane swap returns the pair
// (x[l & ~16], x[l | 16]) (resp. 32) in lane l
__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// max / sum over lanes l, l^16, l^32, l^48
__device__ __forceinline__ float max4rows(float v) {
  // each swap returns the lane's own value and its partner's; v (already
  // quiet) leads a three-input max, which takes the swapped values as they are
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(fmaxf(v, __uint_as_float(a[0])), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(fmaxf(v, __uint_as_float(b[0])), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// weight of a partial with max m against a combined max M (0 for empty parts)
__device__ __forceinline__ float part_weight(float m, float M) {
  return (m == TA_NEG_INF) ? 0.0f : fast_exp2(m - M);
}

// ---------------------------------------------------------------------------
// Rows of a work item. Row rr of the item is group row row0 + rr = (group
// query qig, q-head-in-group hig); its partial goes to slot slot0 + qig, stored
// at that slot's workspace index for the row's q-head (pair-major layout):
// pi = slot_pos[2 s] + qh * slot_pos[2 s + 1], below 2^31 (the host checks
// slots x q-heads against it). The only slot of a query q holds -(q *
// n_qheads) - 1 and -1, so pi = -(q * n_qheads + qh) - 1 < 0: such rows write
// their normalised output to out[-pi - 1] and no record. Only vis, pi and ok
// stay live over the tile loop; gq and qh serve the Q load.
struct RowRef {
  int gq, vis, qh, pi;
  bool ok;
};

__device__ __forceinline__ RowRef row_ref(const PartialArgs& a, const WorkItem& it, int h, int rr) {
  RowRef r{0, 0, 0, 0, rr < it.nrows};
  if (r.ok) {
    const int grow = it.row0 + rr;
    const int qig = grow / a.g, hig = grow - qig * a.g;
    r.gq = a.group_qs[it.q_ptr + qig];
    r.vis = a.group_vis[it.q_ptr + qig];
    r.qh = h * a.g + hig;
    r.pi = a.slot_pos[2 * (it.slot0 + qig)] + r.qh * a.slot_pos[2 * (it.slot0 + qig) + 1];
  }
  return r;
}

__device__ __forceinline__ const char* pool_head(const void* pool, const PartialArgs& a, int h, int esize) {
  return reinterpret_cast<const char*>(pool) + int64_t(h) * a.stride_head * esize;
}

// ---------------------------------------------------------------------------
// GEMV path (fp32 inputs): up to R rows. A wave streams tokens with 8 lanes
// per token (each lane owns D/8 consecutive head-dim elements) and 2 tokens
// per 8-lane group per step; every 8-lane group keeps its own online-softmax
// state, merged across the wave at the end. bf16 items of one or two rows
// run the 16-row matrix tile instead: it keeps twice the bytes in flight,
// and this loop on bf16 measured slower on the multi-level prompt.
template <typename T, int EPL>
struct Slice {  // EPL elements of one token row, as 16-byte words
  static_assert(std::is_same<T, float>::value, "the GEMV path reads fp32 rows");
  static constexpr int kWords = EPL * int(sizeof(T)) / 16;
  u32x4 w[kWords];
  template <typename O>
  __device__ __forceinline__ void load(const char* base, O off) {
#pragma unroll
    for (int c = 0; c < kWords; ++c) w[c] = load_at<u32x4>(base, off + O(16 * c));
  }
  __device__ __forceinline__ void to_float(float* out) const {
#pragma unroll
    for (int c = 0; c < kWords; ++c)
#pragma unroll
      for (int x = 0; x < 4; ++x) out[4 * c + x] = __uint_as_float(w[c][x]);
  }
};

template <typename T, int D, int R>
struct ValuState {
  static constexpr int EPL = D / 8;
  float q[R][EPL];
  float m[R], l[R], o[R][EPL];
  RowRef row[R];
};

template <typename T, int D, int R>
__device__ __forceinline__ void valu_init(ValuState<T, D, R>& S, const PartialArgs& a, const WorkItem& it,
                                          int h, int rbeg) {
  constexpr int EPL = D / 8;
  const int e = threadIdx.x & 7;
  const char* qbase = reinterpret_cast<const char*>(a.q);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    S.row[r] = row_ref(a, it, h, rbeg + r);
    S.m[r] = TA_NEG_INF;
    S.l[r] = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      S.q[r][k] = 0.0f;
      S.o[r][k] = 0.0f;
    }
    if (S.row[r].ok) {
      Slice<T, EPL> sq;
      sq.load(qbase, ((int64_t(S.row[r].gq) * a.n_qheads + S.row[r].qh) * D + e * EPL) * int64_t(sizeof(T)));
      sq.to_float(S.q[r]);
    }
  }
}

template <typename T, int D, int R>
__device__ __forceinline__ void valu_step(ValuState<T, D, R>& S, const Slice<T, D / 8> (&kc)[2],
                                          const Slice<T, D / 8> (&vc)[2], const PartialArgs& a, int base,
                                          int we, int tg) {
  constexpr int EPL = D / 8;
  float kf[2][EPL], vf[2][EPL];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    kc[u].to_float(kf[u]);
    vc[u].to_float(vf[u]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) acc = __builtin_fmaf(S.q[r][k], kf[u][k], acc);
      acc = sum8(acc);
      const int t = base + u * 8 + tg;
      s[u] = (t < we && t < S.row[r].vis) ? acc * a.scale_log2 : TA_NEG_INF;
    }
    const float smax = fmaxf(s[0], s[1]);
    if (smax > S.m[r] + kRescale) {
      const float al = part_weight(S.m[r], smax);
      S.l[r] *= al;
#pragma unroll
      for (int k = 0; k < EPL; ++k) S.o[r][k] *= al;
      S.m[r] = smax;
    }
    const float p0 = (s[0] == TA_NEG_INF) ? 0.0f : fast_exp2(s[0] - S.m[r]);
    const float p1 = (s[1] == TA_NEG_INF) ? 0.0f : fast_exp2(s[1] - S.m[r]);
    S.l[r] += p0 + p1;
#pragma unroll
    for (int k = 0; k < EPL; ++k)
      S.o[r][k] = __builtin_fmaf(p1, vf[1][k], __builtin_fmaf(p0, vf[0][k], S.o[r][k]));
  }
}

// Steps of 16 tokens over [wb, we). Two buffers alternate with no register
// copies. Each step's page-table entries are requested before the K/V of the
// step ahead of it (loads retire in issue order for the wait counter), so
// two steps of K/V stay in flight while one is computed. Loads past the end
// clamp to the last token (cache-resident, unused).
template <typename T, int D, int R, bool FA>
__device__ __forceinline__ void valu_stream(ValuState<T, D, R>& S, const PartialArgs& a,
                                            const WorkItem& it, int h, int wb, int we) {
  typedef typename TokOff<FA>::type Off;
  constexpr int EPL = D / 8;
  if (wb >= we) return;
  const int lane = threadIdx.x & 63;
  const int tg = lane >> 3, e = lane & 7;
  const char* kb = pool_head(a.k, a, h, sizeof(T));
  const char* vb = pool_head(a.v, a, h, sizeof(T));
  const Off lane_off = Off(e * EPL * int(sizeof(T)));
  const int32_t* st = a.seg_tok + it.seg_base;
  const int last = we - 1;
  int32_t sA[2], sB[2];
  Slice<T, EPL> kA[2], vA[2], kB[2], vB[2];
  auto seg = [&](int32_t (&sg)[2], int b) {
#pragma unroll
    for (int u = 0; u < 2; ++u) sg[u] = st[min(b + u * 8 + tg, last)];
  };
  auto kv = [&](Slice<T, EPL> (&kk)[2], Slice<T, EPL> (&vv)[2], const int32_t (&sg)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const Off off = TokOff<FA>::of(sg[u], a) + lane_off;
      kk[u].load(kb, off);
      vv[u].load(vb, off);
    }
  };
  seg(sA, wb);
  seg(sB, wb + 16);
  kv(kA, vA, sA);
  seg(sA, wb + 32);
  kv(kB, vB, sB);
  seg(sB, wb + 48);
  // no exit inside the body (it would make the compiler drain every load
  // at the back edge): the second half is skipped wave-uniformly at the end
  for (int base = wb; base < we; base += 32) {
    valu_step(S, kA, vA, a, base, we, tg);
    kv(kA, vA, sA);
    seg(sA, base + 64);
    if (base + 16 < we) valu_step(S, kB, vB, a, base + 16, we, tg);
    kv(kB, vB, sB);
    seg(sB, base + 80);
  }
}

// merge the 8 token groups of a wave (lanes e, e+8, ..., e+56); afterwards
// every lane group holds the wave's state
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (X == 8) return xor8(v);
  else if constexpr (X == 16) return xor16(v);
  else return xor32(v);
}

template <int X, typename T, int D, int R>
__device__ __forceinline__ void valu_merge_step(ValuState<T, D, R>& S) {
  constexpr int EPL = D / 8;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float mo = lane_xor<X>(S.m[r]);
    const float lo = lane_xor<X>(S.l[r]);
    const float M = fmaxf(S.m[r], mo);
    const float as = part_weight(S.m[r], M), ao = part_weight(mo, M);
    S.l[r] = S.l[r] * as + lo * ao;
#pragma unroll
    for (int k = 0; k < EPL; ++k) S.o[r][k] = S.o[r][k] * as + lane_xor<X>(S.o[r][k]) * ao;
    S.m[r] = M;
  }
}

template <typename T, int D, int R>
__device__ __forceinline__ void valu_merge_lanes(ValuState<T, D, R>& S) {
  valu_merge_step<8>(S);
  valu_merge_step<16>(S);
  valu_merge_step<32>(S);
}

template <typename T, int D, int R>
__device__ __forceinline__ void valu_write(const ValuState<T, D, R>& S, const PartialArgs& a) {
  constexpr int EPL = D / 8;
  const int lane = threadIdx.x & 63;
  if (lane >= 8) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!S.row[r].ok) continue;
    int32_t pi32 = S.row[r].pi;
    asm volatile("" : "+v"(pi32));  // keep the 32-bit index live over the loop, widen here
    const int64_t pi = pi32;
    // a query with one partial: its normalised output, no record
    const bool direct = pi < 0;
    const float sc = direct ? 1.0f / S.l[r] : 1.0f;
    float* op = (direct ? a.out + (-pi - 1) * D : a.o_part + pi * D) + lane * EPL;
#pragma unroll
    for (int k4 = 0; k4 < EPL / 4; ++k4)
      *reinterpret_cast<f32x4*>(op + 4 * k4) = f32x4{S.o[r][4 * k4] * sc, S.o[r][4 * k4 + 1] * sc,
                                                     S.o[r][4 * k4 + 2] * sc, S.o[r][4 * k4 + 3] * sc};
    if (lane == 0 && !direct) {
      a.m_part[pi] = S.m[r];
      a.l_part[pi] = S.l[r];
    }
  }
}

// one wave: rows [rbeg, rbeg + R) over the whole chunk, written directly
template <typename T, int D, int R, bool FA>
__device__ __forceinline__ void valu_wave_item(const PartialArgs& a, const WorkItem& it, int h, int rbeg) {
  ValuState<T, D, R> S;
  valu_init(S, a, it, h, rbeg);
  valu_stream<T, D, R, FA>(S, a, it, h, it.tok0, it.tok1);
  valu_merge_lanes(S);
  valu_write(S, a);
}

// ---------------------------------------------------------------------------
// GEMM path (bf16): 16-row tiles, 32-token tiles, v_mfma_f32_16x16x32_bf16.
// Lane (i = lane % 16, j = lane / 16). In a 32-token tile the lane's P/V
// token set is tau(j, e) = 4j + e for e < 4 and 16 + 4j + (e - 4) otherwise:
// exactly the tokens its S^T accumulators hold for row i.
__device__ __forceinline__ int tau(int j, int e) { return (e < 4) ? 4 * j + e : 16 + 4 * j + (e - 4); }

template <int DPL>
struct VSlice;  // DPL bf16 values of one token (V^T operand source)
template <>
struct VSlice<8> {
  u32x4 w;
  template <typename O>
  __device__ __forceinline__ void load(const char* base, O off) { w = load_at<u32x4>(base, off); }
  __device__ __forceinline__ uint32_t word(int x) const { return w[x]; }
};
template <>
struct VSlice<4> {
  u32x2 w;
  template <typename O>
  __device__ __forceinline__ void load(const char* base, O off) { w = load_at<u32x2>(base, off); }
  __device__ __forceinline__ uint32_t word(int x) const { return w[x]; }
};

template <int D, int NRTW>
struct MfmaState {
  static constexpr int KK = D / 32, DPL = D / 16;
  bf16x8 qf[NRTW][KK];
  f32x4 O[NRTW][DPL];
  f32x4 L4[NRTW];  // l by MFMA (ones x P^T): every element of lane (i, j) is row i's l
  float m[NRTW], l[NRTW];
  // split threshold per row: log2 units, m + log2(kLoFrac l) as of the last
  // exact decision (-inf before the first); a tile whose row max stays at or
  // below it cannot hold a weight above kLoFrac of the running sum
  float thr[NRTW];
  RowRef row[NRTW];
  int vmin[NRTW];  // wave-uniform: smallest visible length over the tile's valid rows
  bool on[NRTW];   // wave-uniform: row tile k exists
};

// row tile k of this wave covers item rows (rt[k] * 16 + i)
template <int D, int NRTW>
__device__ __forceinline__ void mfma_init(MfmaState<D, NRTW>& S, const PartialArgs& a, const WorkItem& it,
                                          int h, const int (&rt)[NRTW], const bool (&on)[NRTW]) {
  constexpr int KK = D / 32, DPL = D / 16;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, j = lane >> 4;
  const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q);
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    S.on[k] = on[k];
    S.row[k] = row_ref(a, it, h, on[k] ? rt[k] * 16 + i : it.nrows);
    S.m[k] = kMInit;
    S.l[k] = 0.0f;
    S.thr[k] = TA_NEG_INF;
    S.L4[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int db = 0; db < DPL; ++db) S.O[k][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int x = 0; x < 8; ++x) S.qf[k][kk][x] = __bf16(0.0f);
    {
      // over the 16 rows of the tile (lanes i; the 4 lanes of a row agree)
      float v = S.row[k].ok ? float(S.row[k].vis) : 3.0e38f;
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) v = fminf(v, __shfl_xor(v, x, 64));
      S.vmin[k] = __builtin_amdgcn_readfirstlane(int(fminf(v, 2.0e9f)));
    }
    if (S.row[k].ok) {
      const __bf16* qp = qbase + (int64_t(S.row[k].gq) * a.n_qheads + S.row[k].qh) * D + j * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) S.qf[k][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 32);
    }
  }
}

// page-table entries of one 32-token tile: lane l holds token (l mod 32)'s
// entry (clamped to the chunk's last token past its end); the K and V loads
// fetch the entries they need from the owning lanes (ds_bpermute)
struct TileSeg {
  int32_t mine;
};

__device__ __forceinline__ void load_tile_seg(TileSeg& t, const int32_t* st, int base, int last, int, int) {
  t.mine = st[min(base + int(threadIdx.x & 31), last)];
}

__device__ __forceinline__ int32_t seg_of(const TileSeg& t, int tok) {
  return __builtin_amdgcn_ds_bpermute(tok << 2, t.mine);
}

// one 32-token K/V tile in MFMA operand order
template <int D>
struct TileKV {
  u32x4 k[2][D / 32];
  VSlice<D / 16> v[8];
};

template <int D, bool FA>
__device__ __forceinline__ void load_tile_kv(TileKV<D>& b, const TileSeg& sg, const char* kb, const char* vb,
                                             int j, int i, const PartialArgs& a) {
  typedef typename TokOff<FA>::type Off;
  constexpr int DPL = D / 16;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const Off off = TokOff<FA>::of(seg_of(sg, tb * 16 + i), a) + Off(j * 16);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) b.k[tb][kk] = load_at<u32x4>(kb, off + Off(kk * 64));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) b.v[e].load(vb, TokOff<FA>::of(seg_of(sg, tau(j, e)), a) + Off(i * DPL * 2));
}

// Softmax of one row tile's 32 scores.
//
// mfma_softmax_max: masks tokens at or past the row's limit (the score
// accumulators s0, s1 are rewritten in place; skipped, wave-uniformly, when
// the whole tile is visible to every row of the tile), raises the running
// max when needed (rescaling l and O) and returns the row's max of the tile
// (scaled, log2 units).
//
// mfma_softmax_weights<SPLIT>: the weights as MFMA B operands, each rounded
// once to bf16 (pb) or, SPLIT, as a bf16 pair pb + pl (~16 bits of P);
// without LMF it also adds to the lane-partial S.l the weights exactly as
// P V uses them (pb, or p when split), so the output stays a weighted
// average of V. (With LMF the caller sums l on the matrix cores, ones x P^T
// into S.L4.)
//
// Precision of the P V product. Rounding a weight w to bf16 moves the
// output by up to 2^-8 w |v - o| / L (L the row's final sum of weights).
// Weights that are each a small share of L round independently and their
// errors average out; a few dominant ones (an attention sink, two near-equal
// peaks) do not. So a row tile's weights enter P V split into hi + lo
// whenever some row's largest weight of the tile exceeds kLoFrac of that
// row's running sum l including the tile (split_needed): the sums only grow
// (in the scale of the current max), so every weight left single-rounded is
// at most kLoFrac of L. The decision is a ballot over the wave, exact only
// when a row's max passes a cached threshold (split_needed).
template <int D, int NRTW>
__device__ __forceinline__ float mfma_softmax_max(MfmaState<D, NRTW>& S, int k, f32x4& s0, f32x4& s1,
                                                  const PartialArgs& a, const WorkItem& it, int base, int j) {
  constexpr int DPL = D / 16;
  const float c = a.scale_log2;
  if (base + 32 > min(it.tok1, S.vmin[k])) {  // wave-uniform: some token of the tile is masked
    // tokens 4 j + x and 16 + 4 j + x of the tile against the row's limit
    const int lim = min(it.tok1, S.row[k].vis) - base - 4 * j;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (x >= lim) s0[x] = TA_NEG_INF;
      if (16 + x >= lim) s1[x] = TA_NEG_INF;
    }
  }
  // four three-input maxes (s0[0] enters twice to make nine operands):
  // v_max3_f32 takes the matrix-core results as they are, where a tree of
  // two-input maxes first quiets each operand with an instruction of its own
  float mx = fmaxf(fmaxf(s0[0], s0[1]), s0[2]);
  mx = fmaxf(fmaxf(mx, s0[3]), s1[0]);
  mx = fmaxf(fmaxf(mx, s1[1]), s1[2]);
  mx = fmaxf(fmaxf(mx, s1[3]), s0[0]);
  mx = max4rows(mx) * c;  // c > 0: the max of scaled scores
  const bool raise = mx > S.m[k] + kRescale;
  if (__builtin_amdgcn_ballot_w64(raise)) {  // rare after the first tiles
    const float al = raise ? fast_exp2(S.m[k] - mx) : 1.0f;
    S.l[k] *= al;
    S.L4[k] *= al;
#pragma unroll
    for (int db = 0; db < DPL; ++db) S.O[k][db] *= al;
    S.m[k] = raise ? mx : S.m[k];
  }
  return mx;
}

// The split decision of a row tile (wave-uniform), given each row's tile
// max mx (scaled) and its running sum l including the tile. The exact test
// (some row's largest weight exp2(mx - m) above kLoFrac l) costs an exp2, a
// compare and, in workgroup waves, a wait for the row-sum MFMA; it runs only
// when some row's mx exceeds its cached threshold thr = m + log2(kLoFrac l)
// (from the last exact test). Sums only grow and a rescale moves m and
// log2 l by the same amount, so a row at or below its threshold needs no
// split. The exact test refreshes the thresholds. l is passed as a function
// so the caller's sum is only formed when needed.
template <int D, int NRTW, typename LF>
__device__ __forceinline__ bool split_needed(MfmaState<D, NRTW>& S, int k, float mx, LF lsum) {
  if (!__builtin_amdgcn_ballot_w64(mx > S.thr[k])) return false;
  const float l = lsum();
  S.thr[k] = S.m[k] + __builtin_amdgcn_logf(kLoFrac * l);
  return __builtin_amdgcn_ballot_w64(fast_exp2(mx - S.m[k]) > kLoFrac * l) != 0;
}

template <int D, int NRTW, bool SPLIT, bool LMF = false>
__device__ __forceinline__ void mfma_softmax_weights(MfmaState<D, NRTW>& S, int k, const f32x4& s0,
                                                     const f32x4& s1, const PartialArgs& a, bf16x8& pb,
                                                     bf16x8& pl) {
  const float c = a.scale_log2, nm = -S.m[k];
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = fast_exp2(__builtin_fmaf(e < 4 ? s0[e] : s1[e - 4], c, nm));
    pb[e] = __bf16(p);
    if constexpr (SPLIT) {
      pl[e] = __bf16(p - float(pb[e]));
      if constexpr (!LMF) psum += p;
    } else if constexpr (!LMF) {
      psum += float(pb[e]);
    }
  }
  if constexpr (!LMF) S.l[k] += psum;
}

// O^T[db] += V^T[db] P^T
template <int D, int NRTW>
__device__ __forceinline__ void pv_update(MfmaState<D, NRTW>& S, int k, int db, const bf16x8& vt, const bf16x8& pb) {
  S.O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb, S.O[k][db], 0, 0, 0);
}

template <int D, int NRTW>
__device__ __forceinline__ void mfma_tile(MfmaState<D, NRTW>& S, const TileKV<D>& b, const PartialArgs& a,
                                          const WorkItem& it, int base, int j) {
  constexpr int KK = D / 32, DPL = D / 16;
  // V^T operands: A_db element e = V[tau(j, e)][DPL * i + db]; v_perm picks
  // the low (db even) or high (db odd) halves of two token words
  bf16x8 vt[DPL];
#pragma unroll
  for (int db = 0; db < DPL; ++db) {
    const uint32_t sel = (db & 1) ? 0x07060302u : 0x05040100u;
    u32x4 wv;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      wv[u] = __builtin_amdgcn_perm(b.v[2 * u + 1].word(db >> 1), b.v[2 * u].word(db >> 1), sel);
    vt[db] = __builtin_bit_cast(bf16x8, wv);
  }
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    if (!S.on[k]) continue;
    f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.k[0][kk]), S.qf[k][kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.k[1][kk]), S.qf[k][kk], s1, 0, 0, 0);
    }
    bf16x8 pb, pl;
    const float mx = mfma_softmax_max<D, NRTW>(S, k, s0, s1, a, it, base, j);
    const float l0 = S.l[k];
    mfma_softmax_weights<D, NRTW, false>(S, k, s0, s1, a, pb, pl);
    if (split_needed(S, k, mx, [&] { return sum4rows(S.l[k]); })) {  // again, split; l takes them unrounded
      S.l[k] = l0;
      mfma_softmax_weights<D, NRTW, true>(S, k, s0, s1, a, pb, pl);
#pragma unroll
      for (int db = 0; db < DPL; ++db)
        S.O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[db], pl, S.O[k][db], 0, 0, 0);
    }
#pragma unroll
    for (int db = 0; db < DPL; ++db) pv_update<D, NRTW>(S, k, db, vt[db], pb);
  }
}

// Stream the item's 32-token tiles. Two tile buffers alternate with no
// register copies. Memory loads complete in issue order as far as the wait
// counter is concerned, so every tile's page-table entries are requested
// before the K/V of the tile ahead of it: waiting for them then never waits
// for younger K/V data, and two tiles stay in flight while one is computed.
template <int D, int NRTW, bool FA>
__device__ __forceinline__ void mfma_stream(MfmaState<D, NRTW>& S, const PartialArgs& a, const WorkItem& it,
                                            int h, TileSeg sgA, TileSeg sgB) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, j = lane >> 4;
  const int ntiles = (it.tok1 - it.tok0 + 31) >> 5;
  const char* kb = pool_head(a.k, a, h, 2);
  const char* vb = pool_head(a.v, a, h, 2);
  const int32_t* st = a.seg_tok + it.seg_base;
  const int last = it.tok1 - 1;

  // issue order: seg 0, seg 1 (by the caller, beside the row and Q loads),
  // kv 0, seg 2, kv 1, seg 3, then per tile n: compute n, kv n + 2, seg n + 4
  TileKV<D> bA, bB;
  int base = it.tok0;
  load_tile_kv<D, FA>(bA, sgA, kb, vb, j, i, a);
  load_tile_seg(sgA, st, base + 64, last, i, j);
  load_tile_kv<D, FA>(bB, sgB, kb, vb, j, i, a);
  load_tile_seg(sgB, st, base + 96, last, i, j);
  // no exit inside the body (an exit between the two halves makes the
  // compiler drain every load at the back edge): the second half is skipped
  // wave-uniformly on an odd last tile
  for (int kt = 0; kt < ntiles; kt += 2, base += 64) {
    mfma_tile<D, NRTW>(S, bA, a, it, base, j);
    load_tile_kv<D, FA>(bA, sgA, kb, vb, j, i, a);
    load_tile_seg(sgA, st, base + 128, last, i, j);
    if (kt + 1 < ntiles) mfma_tile<D, NRTW>(S, bB, a, it, base + 32, j);
    load_tile_kv<D, FA>(bB, sgB, kb, vb, j, i, a);
    load_tile_seg(sgB, st, base + 160, last, i, j);
  }
}

// lane (i, j) holds O[k][db][c] = O[row i][d], with d = DPL * (4j + c) + db
// when V^T came from v_perm, d = 16 db + 4j + c when it came from LDS
// transpose reads (workgroup waves with two row tiles, TR). With LM (every
// workgroup wave) l comes whole from the ones x P^T accumulator; without it
// (single-wave items) l is lane-partial (its 8 tokens per tile) and is summed
// over the row's 4 lanes.
template <int D, int NRTW, bool TR = false, bool LM = TR>
__device__ __forceinline__ void mfma_write(MfmaState<D, NRTW>& S, const PartialArgs& a) {
  constexpr int DPL = D / 16;
  const int j = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    if (!S.on[k]) continue;
    const float l = LM ? S.L4[k][0] : sum4rows(S.l[k]);
    // the row's largest |o| over its four lanes, before any lane leaves
    float mx = 0.0f;
#pragma unroll
    for (int db = 0; db < DPL; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(S.O[k][db][c]));
    mx = max4rows(mx);
    const bool half = mx < l;  // every |o / l| below 1
    if (!S.row[k].ok) continue;
    int32_t pi32 = S.row[k].pi;
    asm volatile("" : "+v"(pi32));  // keep the 32-bit index live over the loop, widen here
    const int64_t pi = pi32;
    // a query with one partial: its normalised output in fp32, no record
    const bool direct = pi < 0;
    const float sc = direct ? 1.0f / l : 1.0f;
    float* const rec = direct ? a.out + (-pi - 1) * D : a.o_part + pi * D;
    if (half && !direct) {
      const float inv = 1.0f / l;
      if constexpr (TR) {
        // lane j holds the 4-runs d = 16 db + 4 j; lanes j and j ^ 1 (l ^ 16)
        // trade one run per pair of d blocks over permlane16, so even j
        // stores d = 16 db + 4 j + [0, 8) of the even block and odd j d = 16 db
        // + 4 (j - 1) + [0, 8) of the odd one, each as one 16-byte store (the
        // row's four lanes take the same half path)
        const bool odd = j & 1;
        _Float16* hp = reinterpret_cast<_Float16*>(a.o_part + pi * D) + 4 * (j & ~1);
#pragma unroll
        for (int q = 0; q < DPL / 2; ++q) {
          u32x2 run[2];  // blocks 2 q, 2 q + 1
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const f32x4& o4 = S.O[k][2 * q + e];
            const f16x4 hv4 = {_Float16(o4[0] * inv), _Float16(o4[1] * inv), _Float16(o4[2] * inv),
                               _Float16(o4[3] * inv)};
            run[e] = __builtin_bit_cast(u32x2, hv4);
          }
          const u32x2 send = odd ? run[0] : run[1];
          u32x2 got;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const auto r = __builtin_amdgcn_permlane16_swap(send[w], send[w], false, false);
            got[w] = (threadIdx.x & 16) ? r[0] : r[1];
          }
          const u32x4 out = odd ? u32x4{got[0], got[1], run[1][0], run[1][1]}
                                : u32x4{run[0][0], run[0][1], got[0], got[1]};
          *reinterpret_cast<u32x4*>(hp + 16 * (2 * q + (odd ? 1 : 0))) = out;
        }
      } else {
        _Float16* hp = reinterpret_cast<_Float16*>(a.o_part + pi * D) + 4 * j * DPL;
#pragma unroll
        for (int x8 = 0; x8 < DPL / 2; ++x8) {
          f16x8 v;
#pragma unroll
          for (int y = 0; y < 8; ++y) {
            const int x = 8 * x8 + y;  // local offset = c * DPL + db
            v[y] = _Float16(S.O[k][x % DPL][x / DPL] * inv);
          }
          *reinterpret_cast<f16x8*>(hp + 8 * x8) = v;
        }
      }
    } else if constexpr (TR) {
      float* op = rec + 4 * j;
#pragma unroll
      for (int db = 0; db < DPL; ++db) *reinterpret_cast<f32x4*>(op + 16 * db) = S.O[k][db] * sc;
    } else {
      float* op = rec + 4 * j * DPL;
#pragma unroll
      for (int x4 = 0; x4 < DPL; ++x4) {
        f32x4 v;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int x = 4 * x4 + y;  // local offset = c * DPL + db
          v[y] = S.O[k][x % DPL][x / DPL] * sc;
        }
        *reinterpret_cast<f32x4*>(op + 4 * x4) = v;
      }
    }
    if (j == 0 && !direct) {
      a.m_part[pi] = S.m[k];
      a.l_part[pi] = half ? -l : l;
    }
  }
}

template <int D, int NRTW, bool FA>
__device__ __forceinline__ void mfma_wave(const PartialArgs& a, const WorkItem& it, int h, const int (&rt)[NRTW],
                                          const bool (&on)[NRTW]) {
  // the first two tiles' page-table entries depend only on the item: they
  // are requested together with the row references, so the first K/V loads
  // can follow the Q loads instead of waiting one more round trip
  const int lane = threadIdx.x & 63;
  TileSeg sgA, sgB;
  load_tile_seg(sgA, a.seg_tok + it.seg_base, it.tok0, it.tok1 - 1, lane & 15, lane >> 4);
  load_tile_seg(sgB, a.seg_tok + it.seg_base, it.tok0 + 32, it.tok1 - 1, lane & 15, lane >> 4);
  MfmaState<D, NRTW> S;
  mfma_init(S, a, it, h, rt, on);
  mfma_stream<D, NRTW, FA>(S, a, it, h, sgA, sgB);
  mfma_write(S, a);
}

// ---------------------------------------------------------------------------
// Workgroup items, bf16: one workgroup per item x kv-head, K/V tiles shared
// through LDS. Each 32-token tile is loaded once by the whole workgroup with
// direct-to-LDS loads into one of kLdsStages stages (two tiles in flight while
// one is computed), and one barrier per tile hands a stage over. Token rows
// are stored with their 16-byte chunks XOR-swizzled by the token index, so the
// MFMA operand reads hit distinct banks (a half wave's 32 lanes read one
// 256-byte bank line per cycle). K rows are read 16 tokens x one chunk at a
// time: chunk c of token t sits at c ^ t. V rows are read by transpose reads,
// whose half waves take 8 tokens x 2 adjacent chunks (16-row tiles) or
// 4 tokens x 4 adjacent chunks (32-row tiles, chunks 4k .. 4k + 3). At 16
// chunks a row (D = 128) chunk c of token t sits at c ^ sv(t), sv(t) =
// 4 (t mod 4) + 2 (bit 2 of t): over 8 aligned tokens sv takes the 8 even
// values, and over 4 aligned tokens its bits 2 and 3 take all four values,
// so either read puts its 16 pieces of a half wave on 16 distinct 16-byte
// positions (c ^ 2t would leave the 4-token reads two-way conflicted);
// at 8 chunks a row two tokens share a 256-byte bank line and c ^ t already
// spreads them. A stage ends in each wave's page-table words for the tile two
// later.
template <int D>
struct LdsTile {
  static constexpr int CH = D / 8;         // 16-byte chunks per token row
  static constexpr int ROW = D * 2;        // bytes per token row
  static constexpr int PART = 32 * ROW;    // one K or V tile
  static constexpr int WORDS = 256;        // per wave: the page-table words of a later tile
  static constexpr int STAGE = 2 * PART + kWaves * WORDS;  // K, V, then the words
  // XOR applied to the chunk index of token t's row in part 0 (K) or 1 (V)
  static __device__ __forceinline__ int swz(int part, int t) {
    if (CH != 16) return t & (CH - 1);
    return part == 0 ? (t & 15) : (((t & 3) << 2) | ((t >> 1) & 2));
  }
  static __device__ __forceinline__ int off(int part, int t, int c) {
    return part * PART + t * ROW + ((c ^ swz(part, t)) << 4);
  }
};

// One direct-to-LDS load (global_load_lds_dwordx4): 16 bytes per lane from
// base + off to the wave-uniform LDS address lds + 16 lane. Written as inline
// asm so that the compiler does not track it: it would otherwise make every
// LDS transpose read wait for all direct loads in flight (the tile loop's own
// waits order the loads and the reads). M0 carries the LDS address and is
// restored, as the compiler expects it unchanged.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(lds), "v"(off), "s"(base)
      : "memory");
}
__device__ __forceinline__ void dma16(const char* base, int64_t off, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(lds), "v"(base + off)
      : "memory");
}

// One direct-to-LDS load of 4 bytes per lane (global_load_lds_dword): from
// base + off to lds + 4 lane; the same conventions as dma16.
__device__ __forceinline__ void dma4(const int32_t* base, uint32_t off, uint32_t lds) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(lds), "v"(off), "s"(base)
      : "memory");
}

// Direct-to-LDS tile loads (global_load_lds_dwordx4): lane l of one
// instruction writes 16 bytes at the wave-uniform LDS base + 16 l, so one
// instruction fills 1 KiB = RPK token rows. A tile's K and V take NI
// instructions, NIW per wave. Lane l of an instruction covers token
// t = blk * RPK + l / CH at LDS chunk position p = l % CH and fetches the
// global chunk p ^ LdsTile::swz(part, t): the swizzle of LdsTile::off, with
// no register staging.
template <int D, bool FA>
struct TileDma {
  typedef LdsTile<D> L;
  typedef typename TokOff<FA>::type Off;
  static constexpr int CH = L::CH;
  static constexpr int RPK = 1024 / L::ROW;           // token rows per instruction
  static constexpr int NI = 2 * L::PART / 1024;       // instructions per tile (K and V)
  static constexpr int NIW = NI / kWaves;             // per wave
  static_assert(NI % kWaves == 0, "tile instructions split evenly over the waves");
  static_assert(NIW * RPK == 16, "each wave moves the K or the V rows of 16 tokens");
  const char* kb;
  const char* vb;
  int wave;
  __device__ __forceinline__ void init(const PartialArgs& a, int h, int w) {
    kb = pool_head(a.k, a, h, 2);
    vb = pool_head(a.v, a, h, 2);
    wave = w;
  }
  // Wave w moves the K (w < 2) or V (w >= 2) rows of tokens 16 (w & 1) ..
  // + 15 of the tile; e[x] is the page-table word of the token the lane moves
  // with its x-th instruction (token x * RPK + lane / CH of those 16).
  __device__ __forceinline__ void issue(char* stage, const int32_t (&e)[NIW], const PartialArgs& a) const {
    typedef __attribute__((address_space(3))) char lds_char;
    const int lane = threadIdx.x & 63;
    const int r = lane / CH, p = lane % CH;
#pragma unroll
    for (int x = 0; x < NIW; ++x) {
      const int m = wave * NIW + x;            // wave-uniform
      const int part = m / (NI / 2), blk = m % (NI / 2);
      const int32_t sg = e[x];
      const int t = blk * RPK + r;
      const Off off = TokOff<FA>::of(sg, a) + Off(((p ^ L::swz(part, t)) << 4));
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          uint32_t(reinterpret_cast<uintptr_t>((lds_char*)(stage + part * L::PART + blk * 1024))));
      dma16(part ? vb : kb, off, dst);
    }
  }
};

// One tile for the wave's first NACT row tiles, operands read straight from
// an LDS stage: K one k-step at a time (the A operand of S^T for both token
// blocks), then V^T one 16-wide d-block at a time by transpose reads.
template <int D, int NRTW, int NACT>
__device__ __forceinline__ void lds_tile(MfmaState<D, NRTW>& S, const char* stage, const PartialArgs& a,
                                         const WorkItem& it, int base, int i, int j) {
  typedef LdsTile<D> L;
  constexpr int KK = D / 32, DPL = D / 16;
  f32x4 s0[NACT], s1[NACT];
#pragma unroll
  for (int k = 0; k < NACT; ++k) s0[k] = s1[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(stage + L::off(0, i, kk * 4 + j));
    const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(stage + L::off(0, 16 + i, kk * 4 + j));
#pragma unroll
    for (int k = 0; k < NACT; ++k) {
      s0[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, S.qf[k][kk], s0[k], 0, 0, 0);
      s1[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, S.qf[k][kk], s1[k], 0, 0, 0);
    }
  }
  // V^T operands by LDS transpose reads: within each 16-lane group, lane L of
  // a ds_read_b64_tr_b16 receives element k = the (L % 4)-th 16-bit value at
  // the address of lane 4k + L / 4. Lane (i, j) points at token
  // 16 r + 4 j + i / 4, d = 16 db + 4 (i % 4): it gets d = 16 db + i of tokens
  // 16 r + 4 j + k, k = 0..3 -- with r = 0, 1 the token order tau(j, e) of P.
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  typedef __attribute__((address_space(3))) char lds_b;
  const lds_b* vstage = (const lds_b*)stage + L::PART;
  auto vt_of = [&](int db) {
    v4s half[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = 16 * r + 4 * j + (i >> 2);
      const int c = 2 * db + ((i & 3) >> 1);
      half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(vstage + t * L::ROW + ((c ^ L::swz(1, t)) << 4) + 8 * (i & 1)));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Per row tile: the max, the weights and their row sums l on the matrix
  // cores (ones x P^T, so l is the sum of the weights P V uses, in fp32; the
  // VALU sum it replaces is 16 converts and adds per row tile), then the
  // split decision against l including this tile. A split tile adds its lo
  // halves to O and l right away (V^T read for it), so they never outlive
  // the branch; the hi halves of every row tile then share one pass of V^T
  // reads.
  const bf16x8 ones = {__bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f),
                       __bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f)};
  bf16x8 pb[NACT];
#pragma unroll
  for (int k = 0; k < NACT; ++k) {
    const float mx = mfma_softmax_max<D, NRTW>(S, k, s0[k], s1[k], a, it, base, j);
    bf16x8 pl;
    mfma_softmax_weights<D, NRTW, false, true>(S, k, s0[k], s1[k], a, pb[k], pl);
    S.L4[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[k], S.L4[k], 0, 0, 0);
    if (split_needed(S, k, mx, [&] { return S.L4[k][0]; })) {  // the weights again, split (pb as before)
      mfma_softmax_weights<D, NRTW, true, true>(S, k, s0[k], s1[k], a, pb[k], pl);
      S.L4[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pl, S.L4[k], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < DPL; ++db)
        S.O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt_of(db), pl, S.O[k][db], 0, 0, 0);
    }
  }
#pragma unroll
  for (int db = 0; db < DPL; ++db) {
    const bf16x8 vt = vt_of(db);
#pragma unroll
    for (int k = 0; k < NACT; ++k) pv_update<D, NRTW>(S, k, db, vt, pb[k]);
  }
}

// Workgroup waves of wide row blocks (more than 64 rows): one 32-row tile
// per wave on v_mfma_f32_32x32x16_bf16, so every K and V operand read from
// LDS feeds 32 rows and the per-tile softmax bookkeeping (max, rescale and
// split tests, addresses) is shared by 32 rows instead of 16. Same transposed
// formulation as the 16-row tiles: S^T = K Q^T and O^T = V^T P^T. Operand
// layouts (lane l, h = l / 32): A[i = l % 32][k = 8h + e], B[k = 8h + e][j =
// l % 32], D[i = 8 (v / 4) + 4h + v % 4][j = l % 32] for e < 8, v < 16. So
// lane l holds 16 of the 32 scores of row l % 32 (tokens 8 (v / 4) + 4h +
// v % 4), and the other 16 sit in lane l ^ 32. P V k-step s (tokens 16 s ..
// 16 s + 15) takes the lane's scores v = 8 s .. 8 s + 7 as its B operand as
// they stand; the V^T operand uses the same token order, tokens 16 s + 4h +
// [0, 4) and 16 s + 8 + 4h + [0, 4), read from LDS by two transpose reads.
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D>
struct WideState {
  static constexpr int KS = D / 16, DB = D / 32;
  bf16x8 qf[KS];  // Q^T: row l % 32, d = 16 kk + 8h + [0, 8)
  f32x16 O[DB];   // O^T: d = 32 db + 8 (v / 4) + 4h + v % 4, row l % 32
  f32x16 L;       // ones x P^T: every element is row l % 32's l
  float m, thr;   // running max and split threshold (as in MfmaState)
  RowRef row;
  int vmin;       // wave-uniform: smallest visible length over the tile's rows
};

// rows rbeg + [0, 32) of the item (those below it.nrows)
template <int D>
__device__ __forceinline__ void wide_init(WideState<D>& W, const PartialArgs& a, const WorkItem& it, int h,
                                          int rbeg) {
  constexpr int KS = D / 16, DB = D / 32;
  const int lane = threadIdx.x & 63;
  W.row = row_ref(a, it, h, rbeg + (lane & 31));
  W.m = kMInit;
  W.thr = TA_NEG_INF;
  W.L = f32x16{};
#pragma unroll
  for (int db = 0; db < DB; ++db) W.O[db] = f32x16{};
  {
    float v = W.row.ok ? float(W.row.vis) : 3.0e38f;
#pragma unroll
    for (int x = 1; x < 32; x <<= 1) v = fminf(v, __shfl_xor(v, x, 64));
    W.vmin = __builtin_amdgcn_readfirstlane(int(fminf(v, 2.0e9f)));
  }
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int x = 0; x < 8; ++x) W.qf[kk][x] = __bf16(0.0f);
  if (W.row.ok) {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (int64_t(W.row.gq) * a.n_qheads + W.row.qh) * D +
                       8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) W.qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
  }
}

// One 32-token tile of a 32-row tile, operands from an LDS stage (LdsTile
// layout: K chunk c of token t at c ^ t, V chunk c at c ^ sv(t), both mod 16
// at D = 128; the K reads of 8 consecutive tokens and each half wave's
// transpose reads of 4 tokens x 4 chunks then fall on distinct banks).
template <int D>
__device__ __forceinline__ void wide_tile(WideState<D>& W, const char* stage, const PartialArgs& a,
                                          const WorkItem& it, int base) {
  typedef LdsTile<D> L;
  constexpr int KS = D / 16, DB = D / 32;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, t32 = lane & 31;
  f32x16 sc = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(stage + L::off(0, t32, 2 * kk + h));
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, W.qf[kk], sc, 0, 0, 0);
  }
  const float c = a.scale_log2;
  if (base + 32 > min(it.tok1, W.vmin)) {  // wave-uniform: some token of the tile is masked
    const int lim = min(it.tok1, W.row.vis) - base - 4 * h;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (8 * (v >> 2) + (v & 3) >= lim) sc[v] = TA_NEG_INF;
  }
  // row max over the lane's 16 scores (three-input maxes, which take the
  // matrix-core results without quieting them first), then over lane l ^ 32
  float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
  mx = fmaxf(fmaxf(mx, sc[3]), sc[4]);
  mx = fmaxf(fmaxf(mx, sc[5]), sc[6]);
  mx = fmaxf(fmaxf(mx, sc[7]), sc[8]);
  mx = fmaxf(fmaxf(mx, sc[9]), sc[10]);
  mx = fmaxf(fmaxf(mx, sc[11]), sc[12]);
  mx = fmaxf(fmaxf(mx, sc[13]), sc[14]);
  mx = fmaxf(fmaxf(mx, sc[15]), sc[0]);
  {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(fmaxf(mx, __uint_as_float(b[0])), __uint_as_float(b[1])) * c;
  }
  const bool raise = mx > W.m + kRescale;
  if (__builtin_amdgcn_ballot_w64(raise)) {  // rare after the first tiles
    const float al = raise ? fast_exp2(W.m - mx) : 1.0f;
    W.L *= al;
#pragma unroll
    for (int db = 0; db < DB; ++db) W.O[db] *= al;
    W.m = raise ? mx : W.m;
  }
  // V^T operand of k-step ks and d block db: lane (16 G + x) of group G
  // points at token 16 ks + 8 half + 4 (G / 2) + x / 4, d = 32 db + 16 (G % 2)
  // + 4 (x % 4); a transpose read hands lane l the values at d = 32 db + l % 32
  // of tokens 16 ks + 8 half + 4h + [0, 4). The swizzle depends on the token
  // mod 8 only, so ks and half are immediate offsets.
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  typedef __attribute__((address_space(3))) char lds_b;
  const lds_b* vstage = (const lds_b*)stage + L::PART;
  const int G = lane >> 4, x = lane & 15;
  const int tv = 4 * (G >> 1) + (x >> 2);
  auto vt_of = [&](int ks, int db) {
    v4s part[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t = 16 * ks + 8 * half + tv;
      const int ch = 4 * db + 2 * (G & 1) + ((x & 3) >> 1);
      part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s*)(vstage + t * L::ROW + ((ch ^ L::swz(1, t)) << 4) + 8 * (x & 1)));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const bf16x8 ones = {__bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f),
                       __bf16(1.0f), __bf16(1.0f), __bf16(1.0f), __bf16(1.0f)};
  const float nm = -W.m;
  bf16x8 pb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[ks][e] = __bf16(fast_exp2(__builtin_fmaf(sc[8 * ks + e], c, nm)));
    W.L = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[ks], W.L, 0, 0, 0);
  }
  // the split decision (as split_needed: an exact test only when some row's
  // max passes its cached threshold); a split tile adds its lo halves to O
  // and l at once
  if (__builtin_amdgcn_ballot_w64(mx > W.thr)) {
    const float l = W.L[0];
    W.thr = W.m + __builtin_amdgcn_logf(kLoFrac * l);
    if (__builtin_amdgcn_ballot_w64(fast_exp2(mx - W.m) > kLoFrac * l)) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(__builtin_fmaf(sc[8 * ks + e], c, nm));
          pl[e] = __bf16(p - float(pb[ks][e]));
        }
        W.L = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pl, W.L, 0, 0, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          W.O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_of(ks, db), pl, W.O[db], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      W.O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_of(ks, db), pb[ks], W.O[db], 0, 0, 0);
}

// lane l writes the d values it holds of row l % 32: runs of 4 at
// 32 db + 8 u + 4h (u < 4); lanes of the first half write m and l
template <int D>
__device__ __forceinline__ void wide_write(const WideState<D>& W, const PartialArgs& a) {
  constexpr int DB = D / 32;
  const int h = (threadIdx.x & 63) >> 5;
  // the row's largest |o| (lanes l and l ^ 32 hold its two halves), before
  // any lane leaves
  const float l = W.L[0];
  float mx = 0.0f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, fabsf(W.O[db][v]));
  mx = fmaxf(mx, xor32(mx));
  const bool half = mx < l;  // every |o / l| below 1
  if (!W.row.ok) return;
  int32_t pi32 = W.row.pi;
  asm volatile("" : "+v"(pi32));
  const int64_t pi = pi32;
  // a query with one partial: its normalised output in fp32, no record
  const bool direct = pi < 0;
  if (half && !direct) {
    // lane h holds the 4-runs d = 32 db + 8 u + 4 h; for each pair of runs u
    // = 2 p, 2 p + 1 the lanes trade one run over permlane32, so lane h = 0
    // stores d = 32 db + 16 p + [0, 8) and lane h = 1 the next 8, each as one
    // 16-byte store (a row's two lanes take the same half path: one l, one mx)
    const float inv = 1.0f / l;
    _Float16* hp = reinterpret_cast<_Float16*>(a.o_part + pi * D) + 8 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        u32x2 run[2];  // runs u = 2 pp, 2 pp + 1 as packed halves
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int u = 2 * pp + q;
          const f16x4 hv4 = {_Float16(W.O[db][4 * u] * inv), _Float16(W.O[db][4 * u + 1] * inv),
                             _Float16(W.O[db][4 * u + 2] * inv), _Float16(W.O[db][4 * u + 3] * inv)};
          run[q] = __builtin_bit_cast(u32x2, hv4);
        }
        // h = 0 keeps run 0 and sends run 1; h = 1 keeps run 1 and sends run 0
        const u32x2 send = h ? run[0] : run[1];
        u32x2 got;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const auto r = __builtin_amdgcn_permlane32_swap(send[w], send[w], false, false);
          got[w] = h ? r[0] : r[1];
        }
        // h = 0: own d 8u..8u+3 of u = 2pp then the partner's 8u+4..8u+7;
        // h = 1: the partner's d 8u..8u+3 of u = 2pp+1 then its own 8u+4..8u+7
        const u32x4 out = h ? u32x4{got[0], got[1], run[1][0], run[1][1]}
                            : u32x4{run[0][0], run[0][1], got[0], got[1]};
        *reinterpret_cast<u32x4*>(hp + 32 * db + 16 * pp) = out;
      }
  } else {
    const float sc = direct ? 1.0f / l : 1.0f;
    float* op = (direct ? a.out + (-pi - 1) * D : a.o_part + pi * D) + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * u) = f32x4{W.O[db][4 * u] * sc, W.O[db][4 * u + 1] * sc,
                                                                 W.O[db][4 * u + 2] * sc, W.O[db][4 * u + 3] * sc};
  }
  if (h == 0 && !direct) {
    a.m_part[pi] = W.m;
    a.l_part[pi] = half ? -l : l;
  }
}

// The tile loop of a workgroup item: kLdsStages LDS stages filled by direct
// loads kLdsStages - 1 tiles ahead. Per tile: wait for this wave's own
// loads of the tile (explicit vmcnt: the direct loads are invisible to the
// compiler), one barrier (every wave's part of the tile has landed and every
// wave is done with the stage the next loads overwrite), the next loads, then
// the compute. The page-table words of tile t + AHEAD (AHEAD = kLdsStages -
// 1) travel with tile t: each wave's direct loads of a tile end with one
// 4-byte-per-lane load of the 16 words it needs AHEAD tiles later, into the
// stage's word area, so the words are in LDS when the tile has landed and no
// load latency other than the tiles' own is on the loop's path. Every
// page-table read is clamped to the chunk's last token (loads past the last
// tile fetch written K/V that the softmax never uses). NACT (row tiles this
// wave computes) is fixed per loop.

// The tile loop's body over its NS stages: stage S takes tile n + S (while
// there is one), with S a compile-time constant.
template <int S, int NS, typename F>
__device__ __forceinline__ void unroll_stages(int n, int ntiles, F& f) {
  if constexpr (S < NS) {
    if (S == 0 || n + S < ntiles) f(n + S, std::integral_constant<int, S>());
    unroll_stages<S + 1, NS>(n, ntiles, f);
  }
}

// s_waitcnt with vmcnt = n (< 16) and no wait on the other counters
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the LDS stages only: this wave's direct loads up to
// the last N and all its LDS accesses retire, then s_barrier. (__syncthreads
// also releases global memory, which waits for every direct load in flight.)
// The clobber keeps the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void lds_stage_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0x0 << 8));
  asm volatile("s_barrier" ::: "memory");
}

// body(stage, base): the compute of one tile (base = its first token), or
// nothing for a wave without rows
template <int D, bool FA, typename Body>
__device__ __forceinline__ void lds_stream(char* lds, const PartialArgs& a, const WorkItem& it, int h, Body body) {
  typedef TileDma<D, FA> Dma;
  typedef LdsTile<D> L;
  typedef __attribute__((address_space(3))) char lds_char;
  constexpr int ST = L::STAGE, NIW = Dma::NIW;
  const int ntiles = (it.tok1 - it.tok0 + 31) >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // Page-table words. Lane l of the words load fetches the word of token
  // u = (l mod NIW) * RPK + (l mod 16) / NIW of this wave's 16, so the NIW
  // words a lane needs for its direct loads (tokens x * RPK + lane / CH) are
  // adjacent in LDS at 4 NIW (lane / CH). Indices are clamped to the chunk's
  // last token: past it the loads fetch written K/V that the softmax masks.
  constexpr int NS = kLdsStages, AHEAD = NS - 1;  // loads (and the words they carry) run AHEAD tiles ahead
  static_assert(NS >= 3 && (AHEAD - 1) * (NIW + 1) < 16, "the loop's wait fits the vmcnt field");
  const int32_t* st = a.seg_tok;
  const int seg0 = __builtin_amdgcn_readfirstlane(it.seg_base);
  const int u = (lane % NIW) * Dma::RPK + (lane & 15) / NIW;
  const int first = __builtin_amdgcn_readfirstlane(it.tok0) + (wave & 1) * 16 + u;
  const int last = it.tok1 - 1;
  auto word_off = [&](int n) -> uint32_t { return uint32_t(seg0 + min(first + n * 32, last)) * 4u; };
  const int wpos = 2 * L::PART + wave * L::WORDS;           // this wave's word area in a stage
  const int rpos = wpos + 4 * NIW * (lane / Dma::CH);        // this lane's NIW words there
  auto lds_addr = [&](int stage_off) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lds_char*)(lds + stage_off))));
  };
  Dma dma;
  dma.init(a, h, wave);
  // tiles 0 .. AHEAD - 1 take their words from plain loads; each later
  // tile's come with the tile AHEAD before it
  int32_t e[AHEAD][NIW];
#pragma unroll
  for (int x = 0; x < NIW; ++x) {
    const int tk = x * Dma::RPK + lane / Dma::CH;
    const int b0 = __builtin_amdgcn_readfirstlane(it.tok0) + (wave & 1) * 16 + tk;
#pragma unroll
    for (int t = 0; t < AHEAD; ++t) e[t][x] = st[seg0 + min(b0 + 32 * t, last)];
  }
  // the unit's Q and row loads, these words (and the previous unit's
  // stores) retire here, so no register the loop reads waits on a vector load
  wait_vmcnt<0>();
#pragma unroll
  for (int t = 0; t < AHEAD; ++t) {
    dma.issue(lds + t * ST, e[t], a);
    dma4(st, word_off(t + AHEAD), lds_addr(t * ST + wpos));
  }
  // one tile in stage SG (a compile-time stage, so every LDS address below is
  // a loop-invariant lane offset plus an immediate)
  auto step = [&](int n, auto sg) {
    constexpr int SG = decltype(sg)::value;
    // this wave's loads of tile n (and the words of tile n + AHEAD) landed;
    // those of the next AHEAD - 1 tiles in flight
    lds_stage_barrier<(AHEAD - 1) * (NIW + 1)>();
    int32_t w[NIW];
    {
      const char* wp = lds + SG * ST + rpos;
      if constexpr (NIW == 4) {
        const i32x4 w4 = *reinterpret_cast<const i32x4*>(wp);
#pragma unroll
        for (int x = 0; x < NIW; ++x) w[x] = w4[x];
      } else {
#pragma unroll
        for (int x = 0; x < NIW; ++x) w[x] = reinterpret_cast<const int32_t*>(wp)[x];
      }
    }
    constexpr int SF = SG == 0 ? NS - 1 : SG - 1;  // the stage of tile n - 1, done by every wave
    dma.issue(lds + SF * ST, w, a);
    dma4(st, word_off(n + 2 * AHEAD), lds_addr(SF * ST + wpos));
    body(lds + SG * ST, it.tok0 + n * 32);
  };
  // wave-uniform: tile n sits in stage n mod NS
  for (int n = 0; n < ntiles; n += NS) unroll_stages<0, NS>(n, ntiles, step);
  // every wave's direct loads (the clamped ones past the end included) land
  // before the stages are reused
  lds_stage_barrier<0>();
}

template <int D, bool FA>
__device__ __forceinline__ void block_lds_item(const PartialArgs& a, char* lds, int blk) {
  const int item = blk / a.n_kvheads;
  const int h = blk - item * a.n_kvheads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, j = lane >> 4;
  const WorkItem it = a.items[item];
  const int nrt = (it.nrows + 15) >> 4;
  // row tiles beyond kWaves * kBlockRowTiles take further passes over the
  // chunk (the planner's row blocks keep this to one pass)
  for (int r0 = 0; r0 < nrt; r0 += kWaves * kBlockRowTiles) {
    // every wave takes part in the loads and barriers, computing or not
    auto idle = [](const char*, int) {};
    if (nrt - r0 > kWaves) {
      // more than 64 rows in this pass: wave w computes rows 32 w .. 32 w + 31
      // of the pass as one 32-row tile
      WideState<D> W;
      wide_init(W, a, it, h, (r0 + 2 * wave) * 16);
      if (2 * wave < nrt - r0)
        lds_stream<D, FA>(lds, a, it, h, [&](const char* st, int base) { wide_tile<D>(W, st, a, it, base); });
      else
        lds_stream<D, FA>(lds, a, it, h, idle);
      wide_write(W, a);
      continue;
    }
    // at most 64 rows: wave w computes 16-row tile w of the pass
    const int rt[1] = {r0 + wave};
    const bool on[1] = {r0 + wave < nrt};
    MfmaState<D, 1> S;
    mfma_init(S, a, it, h, rt, on);
    if (S.on[0])
      lds_stream<D, FA>(lds, a, it, h, [&](const char* st, int base) { lds_tile<D, 1, 1>(S, st, a, it, base, i, j); });
    else
      lds_stream<D, FA>(lds, a, it, h, idle);
    // V^T came from transpose reads (d = 16 db + 4j + c), l from the matrix cores
    mfma_write<D, 1, true>(S, a);
  }
}

// ---------------------------------------------------------------------------
// Workgroup items, fp32 (GEMV path): one workgroup per item x kv-head; wave
// w owns row pairs 2w, 2w + 8, ... over the whole chunk.
template <typename T, int D, bool FA>
__device__ __forceinline__ void block_valu_item(const PartialArgs& a, int blk) {
  const int item = blk / a.n_kvheads;
  const int h = blk - item * a.n_kvheads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const WorkItem it = a.items[item];
  for (int r = 2 * wave; r < it.nrows; r += 2 * kWaves) valu_wave_item<T, D, 2, FA>(a, it, h, r);
}

// Single-wave items (groups with few rows): each wave is one item x kv-head
// and streams its whole chunk alone.
template <typename T, int D, bool FA>
__device__ __forceinline__ void wave_item(const PartialArgs& a, int item0, int n_units, int wblk) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = wblk * int(blockDim.x >> 6) + wave;
  if (unit >= n_units) return;
  const int item = item0 + unit / a.n_kvheads;
  const int h = unit - (unit / a.n_kvheads) * a.n_kvheads;
  const WorkItem it = a.items[item];
  if constexpr (std::is_same<T, __bf16>::value) {
    // one 16-row MFMA tile even for one or two rows: the item is bound by
    // its K/V stream, and the tile loop keeps twice the bytes in flight of
    // the GEMV loop
    const int rt[1] = {0};
    const bool on[1] = {true};
    mfma_wave<D, 1, FA>(a, it, h, rt, on);
  } else if (it.nrows <= 1) {
    valu_wave_item<T, D, 1, FA>(a, it, h, 0);
  } else {
    for (int r = 0; r < it.nrows; r += 2) valu_wave_item<T, D, 2, FA>(a, it, h, r);
  }
}

// The partial-attention launch: workgroups [0, n_block_wgs) take the
// workgroup items (one per item x kv-head, longest items first as the
// planner sorts them), the rest take the single-wave items, four units per
// workgroup. One launch keeps both classes on the chip together without a
// second stream.
template <typename T, int D, bool FA>
__global__ __launch_bounds__(kBlock, 2) void partial_kernel(PartialArgs a, int n_block_wgs, int n_units) {
  constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  // the K/V stages of workgroup items (dynamic: launches without workgroup
  // items reserve none)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int blk = blockIdx.x;
  if (blk < n_block_wgs) {
    if constexpr (kBf16) block_lds_item<D, FA>(a, lds, blk);
    else block_valu_item<T, D, FA>(a, blk);
  } else {
    wave_item<T, D, FA>(a, n_block_wgs / a.n_kvheads, n_units, blk - n_block_wgs);
  }
}

// ---------------------------------------------------------------------------
// P (query, q-head) pairs per wave (P = 1, 2, 4): each pair gets 4 / P of the
// wave's 16-lane groups, which take every (4 / P)-th of the query's slots
// (each lane D/16 consecutive output elements), loading them in batches of B
// so the loads are in flight together; a pair's groups are then merged with
// permlane swaps and its first group writes the normalised output. The host
// picks P and B from the plan's largest slot count per query, so that one
// batch covers every pair where it can: short paths take a quarter of the
// waves, long ones keep all four groups on one pair with deeper batches.
constexpr int kReduceGroups = 4;

template <int D, int P, int B>
__global__ __launch_bounds__(kBlock) void lse_reduce_kernel(ReduceArgs a) {
  static_assert(P == 1 || P == 2 || P == 4, "pairs per wave");
  constexpr int kReduceBatch = B;
  constexpr int EPL = D / 16;         // output elements per lane
  constexpr int GP = kReduceGroups / P;  // lane groups per pair
  typedef _Float16 hv_t __attribute__((ext_vector_type(EPL)));
  const int64_t n_pairs = int64_t(a.n_queries) * a.n_qheads;
  const int64_t wave_id = int64_t(blockIdx.x) * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave_id * P >= n_pairs) return;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, sub = lane & 15;
  const int sg = g % GP;              // this group's place among its pair's groups
  const int64_t pair = wave_id * P + g / GP;
  const bool live = pair < n_pairs;   // the wave's last pairs may lie past the end
  const int q = live ? int(pair / a.n_qheads) : 0;
  const int hq = live ? int(pair - int64_t(q) * a.n_qheads) : 0;
  int s0 = a.q_slot_ptr[q];
  int s1 = live ? a.q_slot_ptr[q + 1] : s0;
  if constexpr (P == 1) {
    s0 = __builtin_amdgcn_readfirstlane(s0);
    s1 = __builtin_amdgcn_readfirstlane(s1);
  }
  // a query with a single slot has its output written by the partial kernel
  const bool single = s1 - s0 == 1;
  if (single) s1 = s0;
  float M = TA_NEG_INF, L = 0.0f;
  float acc[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) acc[x] = 0.0f;
  for (int b = s0 + sg; b < s1; b += GP * kReduceBatch) {
    int64_t pi[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u)
      pi[u] = int64_t(s0) * a.n_qheads + int64_t(hq) * (s1 - s0) + (min(b + GP * u, s1 - 1) - s0);
    // every slot's fp16 half-record is requested with its m and l; the slots
    // kept in fp32 (l not negated) are then read whole
    float mv[kReduceBatch], lv[kReduceBatch];
    hv_t hv[kReduceBatch];
    f32x4 ov[kReduceBatch][EPL / 4];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      mv[u] = (b + GP * u < s1) ? a.m_part[pi[u]] : TA_NEG_INF;
      lv[u] = a.l_part[pi[u]];
      hv[u] = *reinterpret_cast<const hv_t*>(reinterpret_cast<const _Float16*>(a.o_part + pi[u] * D) + sub * EPL);
    }
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u)
      if (!__builtin_signbit(lv[u]))
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c)
          ov[u][c] = *reinterpret_cast<const f32x4*>(a.o_part + pi[u] * D + sub * EPL + 4 * c);
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) Mn = fmaxf(Mn, mv[u]);
    const float wa = part_weight(M, Mn);
    L *= wa;
#pragma unroll
    for (int x = 0; x < EPL; ++x) acc[x] *= wa;
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      const float w = part_weight(mv[u], Mn);
      const bool half = __builtin_signbit(lv[u]);
      const float lu = fabsf(lv[u]);
      L += lu * w;
      const float sc = half ? lu * w : w;  // fp16 records hold o / l
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[4 * c + y] += (half ? float(hv[u][4 * c + y]) : ov[u][c][y]) * sc;
    }
    M = Mn;
  }
  // merge a pair's groups: lanes sub + 16 g over its GP groups (GP = 4: two
  // swaps; GP = 2: groups 2k and 2k + 1 by one swap)
#pragma unroll
  for (int step = 0; (1 << step) < GP; ++step) {
    const float Mo = step == 0 ? xor16(M) : xor32(M);
    const float Lo = step == 0 ? xor16(L) : xor32(L);
    const float Mn = fmaxf(M, Mo);
    const float ws = part_weight(M, Mn), wo = part_weight(Mo, Mn);
    L = L * ws + Lo * wo;
#pragma unroll
    for (int x = 0; x < EPL; ++x) {
      const float ao = step == 0 ? xor16(acc[x]) : xor32(acc[x]);
      acc[x] = acc[x] * ws + ao * wo;
    }
    M = Mn;
  }
  if (sg == 0 && live && !single) {
    const float inv = 1.0f / L;
    float* op = a.out + (int64_t(q) * a.n_qheads + hq) * D + sub * EPL;
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c)
      *reinterpret_cast<f32x4*>(op + 4 * c) =
          f32x4{acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv, acc[4 * c + 3] * inv};
  }
}

// One workgroup per descriptor (grid-stride over descriptors); the stage is
// pinned host memory, read over the bus.
// Table update by blocks [0, nb) of a launch (block b takes descriptors b,
// b + nb, ...).
__device__ __forceinline__ void scatter_blocks(int32_t* dst, int64_t dst_words, const int32_t* stage,
                                               int32_t n_desc, int32_t b, int32_t nb) {
  for (int32_t d = b; d < n_desc; d += nb) {
    const int64_t to = stage[3 * d], n = stage[3 * d + 1], from = stage[3 * d + 2];
    for (int64_t x = threadIdx.x; x < n; x += blockDim.x)
      if (to + x < dst_words) dst[to + x] = stage[from + x];
  }
}

// KV append by blocks [0, nb) of a launch: 16 lanes per 256-byte head row (16
// bytes each), block-stride over (token, kv-head) rows; a destination outside
// the pool is skipped.
__device__ __forceinline__ void append_blocks(const AppendArgs& a, int64_t b, int64_t nb) {
  const int64_t rows = a.n_tokens * a.n_kvheads;
  const int chunks = a.row_bytes >> 4;  // 16-byte pieces per head row
  const int64_t step = nb * blockDim.x;
  for (int64_t x = b * blockDim.x + threadIdx.x; x < rows * chunks; x += step) {
    const int64_t row = x / chunks;
    const int c = int(x - row * chunks);
    const int64_t r = row / a.n_kvheads;
    const int h = int(row - r * a.n_kvheads);
    const int32_t loc = a.dst[r];
    const int64_t page = loc >> 8;
    const int slot = loc & 255;
    if (loc < 0 || page >= a.n_pages || slot >= a.page_size) continue;
    const int64_t src = row * a.row_bytes + 16 * c;
    const int64_t off = page * a.sp_bytes + slot * a.st_bytes + h * a.sh_bytes + 16 * c;
    *reinterpret_cast<u32x4*>(a.k + off) = *reinterpret_cast<const u32x4*>(a.k_new + src);
    *reinterpret_cast<u32x4*>(a.v + off) = *reinterpret_cast<const u32x4*>(a.v_new + src);
  }
}

__global__ void scatter_kernel(int32_t* dst, int64_t dst_words, const int32_t* stage, int32_t n_desc) {
  scatter_blocks(dst, dst_words, stage, n_desc, int32_t(blockIdx.x), int32_t(gridDim.x));
}

__global__ void append_kernel(AppendArgs a) { append_blocks(a, blockIdx.x, gridDim.x); }

// Both updates of a decode-loop step in one launch: the first sb blocks
// update the tables, the rest append the new K/V rows (the two touch
// disjoint memory).
__global__ void update_kernel(AppendArgs a, int32_t* dst, int64_t dst_words, const int32_t* stage, int32_t n_desc,
                              int32_t sb) {
  if (int32_t(blockIdx.x) < sb)
    scatter_blocks(dst, dst_words, stage, n_desc, int32_t(blockIdx.x), sb);
  else
    append_blocks(a, int64_t(blockIdx.x) - sb, int64_t(gridDim.x) - sb);
}

// The same with the staged words in the kernel arguments (read in place from
// the argument segment). The whole argument list stays within 4 KiB.
// (explicit arguments, each 8-byte aligned at most, plus up to 256 bytes of
// the hidden arguments code-object v5 appends)
static_assert(sizeof(AppendArgs) + sizeof(int32_t*) + sizeof(int64_t) + sizeof(ArgStage) + 2 * sizeof(int32_t) +
                      6 * 8 + 256 <= 4096,
              "update_args_kernel's arguments fit a 4 KiB argument block");
__global__ void update_args_kernel(AppendArgs a, int32_t* dst, int64_t dst_words, ArgStage st, int32_t n_desc,
                                   int32_t sb) {
  if (int32_t(blockIdx.x) < sb)
    scatter_blocks(dst, dst_words, st.w, n_desc, int32_t(blockIdx.x), sb);
  else
    append_blocks(a, int64_t(blockIdx.x) - sb, int64_t(gridDim.x) - sb);
}

__global__ void fill_kernel(float* p, int64_t n, float value) {
  for (int64_t x = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; x < n; x += int64_t(gridDim.x) * blockDim.x)
    p[x] = value;
}

template <typename T, int D>
void launch_partial_t(const PartialArgs& a, int32_t n_block_items, int32_t n_wave_items, hipStream_t s,
                      KernelTimer t) {
  const int n_block_wgs = n_block_items * a.n_kvheads;
  const int n_units = n_wave_items * a.n_kvheads;
  // single-wave units go two per workgroup when there are no workgroup
  // items: the dispatcher then spreads them more evenly over the CUs
  const int wpb = n_block_wgs == 0 ? 2 : kWaves;
  const dim3 grid(unsigned(n_block_wgs + (n_units + wpb - 1) / wpb)), block(unsigned(wpb * 64));
  constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  const size_t lds = (kBf16 && n_block_wgs > 0) ? size_t(kLdsStages) * LdsTile<D>::STAGE : 0;
  if (a.fast_addr)
    hipExtLaunchKernelGGL((partial_kernel<T, D, true>), grid, block, lds, s, t.start, t.stop, 0, a, n_block_wgs,
                          n_units);
  else
    hipExtLaunchKernelGGL((partial_kernel<T, D, false>), grid, block, lds, s, t.start, t.stop, 0, a, n_block_wgs,
                          n_units);
}

template <int D, int P, int B>
void launch_reduce_t(const ReduceArgs& a, int64_t pairs, hipStream_t s, KernelTimer t) {
  const int64_t waves = (pairs + P - 1) / P;
  const dim3 grid(unsigned((waves + kWaves - 1) / kWaves)), block(kBlock);
  hipExtLaunchKernelGGL((lse_reduce_kernel<D, P, B>), grid, block, 0, s, t.start, t.stop, 0, a);
}

// one batch per group where the slots allow: up to 4 slots 4 pairs per
// wave, up to 8 two, then one pair with batches of 4, 8 or 16 slots per group
template <int D>
void launch_reduce_d(const ReduceArgs& a, int64_t pairs, hipStream_t s, KernelTimer t) {
  const int32_t m = a.max_slots;
  if (m <= 4) launch_reduce_t<D, 4, 4>(a, pairs, s, t);
  else if (m <= 8) launch_reduce_t<D, 2, 4>(a, pairs, s, t);
  else if (m <= 16) launch_reduce_t<D, 1, 4>(a, pairs, s, t);
  else if (m <= 32) launch_reduce_t<D, 1, 8>(a, pairs, s, t);
  else launch_reduce_t<D, 1, 16>(a, pairs, s, t);
}

}  // namespace

hipError_t launch_partial(const PartialArgs& a, int32_t n_block_items, int32_t n_wave_items, int dtype,
                          int head_dim, hipStream_t s, KernelTimer t) {
  if (n_block_items + n_wave_items <= 0) return hipSuccess;
  if (dtype == 1) {
    if (head_dim == 128) launch_partial_t<__bf16, 128>(a, n_block_items, n_wave_items, s, t);
    else launch_partial_t<__bf16, 64>(a, n_block_items, n_wave_items, s, t);
  } else {
    if (head_dim == 128) launch_partial_t<float, 128>(a, n_block_items, n_wave_items, s, t);
    else launch_partial_t<float, 64>(a, n_block_items, n_wave_items, s, t);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, hipStream_t s, KernelTimer t) {
  const int64_t pairs = int64_t(a.n_queries) * a.n_qheads;
  if (pairs <= 0) return hipSuccess;
  if (head_dim == 128) launch_reduce_d<128>(a, pairs, s, t);
  else launch_reduce_d<64>(a, pairs, s, t);
  return hipGetLastError();
}

hipError_t launch_scatter(int32_t* dst, int64_t dst_words, const int32_t* stage, int32_t n_desc, hipStream_t s) {
  if (n_desc <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel, dim3(unsigned(std::min(n_desc, 1024))), dim3(256), 0, s, dst, dst_words, stage,
                     n_desc);
  return hipGetLastError();
}

static int64_t append_grid(const AppendArgs& a) {
  const int64_t work = a.n_tokens * a.n_kvheads * (a.row_bytes >> 4);
  return work <= 0 ? 0 : std::min<int64_t>((work + 255) / 256, 8192);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t blocks = append_grid(a);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_update_args(const AppendArgs* app, int32_t* dst, int64_t dst_words, const ArgStage& stage,
                              int32_t n_desc, hipStream_t s) {
  AppendArgs a{};
  if (app) a = *app;  // else n_tokens = 0: no append blocks
  const int64_t ab = append_grid(a);
  const int32_t sb = std::max(0, std::min(n_desc, 64));
  if (sb + ab == 0) return hipSuccess;
  hipLaunchKernelGGL(update_args_kernel, dim3(unsigned(sb + ab)), dim3(256), 0, s, a, dst, dst_words, stage,
                     n_desc, sb);
  return hipGetLastError();
}

hipError_t launch_append_scatter(const AppendArgs& a, int32_t* dst, int64_t dst_words, const int32_t* stage,
                                 int32_t n_desc, hipStream_t s) {
  const int64_t ab = append_grid(a);
  if (ab == 0) return launch_scatter(dst, dst_words, stage, n_desc, s);
  if (n_desc <= 0) return launch_append(a, s);
  const int32_t sb = std::min(n_desc, 1024);
  hipLaunchKernelGGL(update_kernel, dim3(unsigned(sb + ab)), dim3(256), 0, s, a, dst, dst_words, stage, n_desc, sb);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace ta
