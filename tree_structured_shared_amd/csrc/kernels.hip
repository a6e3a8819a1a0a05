// HIP kernels for tree-structured decode attention on CDNA4 (gfx950).
//
// Partial attention: a work item is one KV chunk of one context-query group
// and a block of its rows (row = query x q-head-in-group); its kernel streams
// the chunk's paged K/V once for all those rows -- the KV-guided grouping of the DeFT reading notes and the
// single-launch, one-group-per-block-set kernel of the FastTree review
// (section 3, kernel design) -- and runs a flash-style online softmax over it
// (DeFT notes, attention calculation; FastTree review, tile-by-tile online
// softmax). It writes one unnormalised partial (m, l, o) per row. Groups with
// few rows run as single-wave items (wave_items_kernel: every wave of the
// launch is an independent item x kv-head); groups with many rows run as
// workgroup items (block_items_kernel: one item x kv-head per workgroup, the
// four waves split rows, or rows and tokens).
//
// Two row paths, chosen per item by its row count (the review's multi-stage
// query tiling: small tiles near the leaves, large ones near the root):
//  * GEMV-sized items (few rows, or fp32 inputs): wavefront dot products with
//    8 lanes per token, xor-shuffle reductions, and per-lane online softmax.
//  * GEMM-sized items (bf16): v_mfma_f32_16x16x32_bf16 on a transposed
//    formulation -- S^T = K Q^T (K rows are the A operand, loaded straight
//    from the paged pool) and O^T = V^T P^T, where the score accumulator
//    layout is already the B-operand layout of P, and V^T comes from an 8x8
//    register transpose of 16-byte V loads (stacking queries that share KV
//    turns the decode GEMV into a GEMM, FastTree review, kernel design).
//    No LDS and no barrier in the streaming loop: every wave runs alone.
//
// lse_reduce: per (query, q-head), merges that query's partials along its
// path (root-side group first, chunks ascending) by log-sum-exp -- the
// tree-topology-aware global reduction of the DeFT notes.
//
// Softmax runs in base 2: scores are scaled by scale * log2(e) and the
// workspace m is in those units. The running max is only raised when a new
// score exceeds it by more than 8 (in log2 units), so rescaling is rare; the
// stored (m, l, o) stay consistent because l and o are always relative to m.
#include "kernels.h"

#include <type_traits>

namespace ta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
constexpr int kWaves = 4;
constexpr int kValuMaxRows = 4;   // bf16 items with more rows take the MFMA path
constexpr float kRescale = 8.0f;  // lazy-rescale threshold, log2 units
#define TA_NEG_INF (-__builtin_inff())

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ int64_t tok_off(int32_t st, const PartialArgs& a) {
  return int64_t(st >> 8) * a.stride_page + int64_t(st & 255) * a.stride_token;
}

// weight of a partial with max m against a combined max M (0 for empty parts)
__device__ __forceinline__ float part_weight(float m, float M) {
  return (m == TA_NEG_INF) ? 0.0f : fast_exp2(m - M);
}

// ---------------------------------------------------------------------------
// raw per-lane slices of EPL elements, loaded as 16-byte words
template <typename T, int EPL>
struct Slice {
  static constexpr int kWords = EPL * int(sizeof(T)) / 16;
  u32x4 w[kWords];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int c = 0; c < kWords; ++c) w[c] = *reinterpret_cast<const u32x4*>(p + c * (16 / sizeof(T)));
  }
  __device__ __forceinline__ void to_float(float* out) const {
    if constexpr (std::is_same<T, float>::value) {
#pragma unroll
      for (int c = 0; c < kWords; ++c)
#pragma unroll
        for (int x = 0; x < 4; ++x) out[4 * c + x] = __uint_as_float(w[c][x]);
    } else {
#pragma unroll
      for (int c = 0; c < kWords; ++c)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          out[8 * c + 2 * x] = bf_lo(w[c][x]);
          out[8 * c + 2 * x + 1] = bf_hi(w[c][x]);
        }
    }
  }
};

// ---------------------------------------------------------------------------
// Rows of a work item. Row rr of the item is group row row0 + rr = (group
// query qig, q-head-in-group hig); its partial goes to slot slot0 + qig.
struct RowRef {
  int gq, vis, slot, qh;
  bool ok;
};

__device__ __forceinline__ RowRef row_ref(const PartialArgs& a, const WorkItem& it, int h, int rr) {
  RowRef r{0, 0, 0, 0, rr < it.nrows};
  if (r.ok) {
    const int grow = it.row0 + rr;
    const int qig = grow / a.g, hig = grow - qig * a.g;
    r.gq = a.group_qs[it.q_ptr + qig];
    r.vis = a.group_vis[it.q_ptr + qig];
    r.slot = it.slot0 + qig;
    r.qh = h * a.g + hig;
  }
  return r;
}

// ---------------------------------------------------------------------------
// GEMV path: up to R rows. A wave streams tokens with 8 lanes per token (each
// lane owns D/8 consecutive head-dim elements) and 2 tokens per 8-lane group
// per step; every 8-lane group keeps its own online-softmax state, merged
// across the wave at the end.
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
  const T* qbase = reinterpret_cast<const T*>(a.q);
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
      sq.load(qbase + (int64_t(S.row[r].gq) * a.n_qheads + S.row[r].qh) * D + e * EPL);
      sq.to_float(S.q[r]);
    }
  }
}

template <typename T, int D, int R>
__device__ __forceinline__ void valu_stream(ValuState<T, D, R>& S, const PartialArgs& a,
                                            const WorkItem& it, int h, int wb, int we) {
  constexpr int EPL = D / 8;
  if (wb >= we) return;
  const int lane = threadIdx.x & 63;
  const int tg = lane >> 3, e = lane & 7;
  const T* kb = reinterpret_cast<const T*>(a.k) + int64_t(h) * a.stride_head + e * EPL;
  const T* vb = reinterpret_cast<const T*>(a.v) + int64_t(h) * a.stride_head + e * EPL;
  const int32_t* st = a.seg_tok + it.seg_base;

  Slice<T, EPL> kc[2], vc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t off = tok_off(st[min(wb + u * 8 + tg, we - 1)], a);
    kc[u].load(kb + off);
    vc[u].load(vb + off);
  }
  for (int base = wb; base < we; base += 16) {
    Slice<T, EPL> kn[2], vn[2];
    const int nb = base + 16;
    if (nb < we) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t off = tok_off(st[min(nb + u * 8 + tg, we - 1)], a);
        kn[u].load(kb + off);
        vn[u].load(vb + off);
      }
    }
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
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 4, 64);
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
    if (nb < we) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        kc[u] = kn[u];
        vc[u] = vn[u];
      }
    }
  }
}

// merge the 8 token groups of a wave (lanes e, e+8, ..., e+56); afterwards
// every lane group holds the wave's state
template <typename T, int D, int R>
__device__ __forceinline__ void valu_merge_lanes(ValuState<T, D, R>& S) {
  constexpr int EPL = D / 8;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) {
      const float mo = __shfl_xor(S.m[r], x, 64);
      const float lo = __shfl_xor(S.l[r], x, 64);
      const float M = fmaxf(S.m[r], mo);
      const float as = part_weight(S.m[r], M), ao = part_weight(mo, M);
      S.l[r] = S.l[r] * as + lo * ao;
#pragma unroll
      for (int k = 0; k < EPL; ++k) S.o[r][k] = S.o[r][k] * as + __shfl_xor(S.o[r][k], x, 64) * ao;
      S.m[r] = M;
    }
  }
}

template <typename T, int D, int R>
__device__ __forceinline__ void valu_write(const ValuState<T, D, R>& S, const PartialArgs& a) {
  constexpr int EPL = D / 8;
  const int lane = threadIdx.x & 63;
  if (lane >= 8) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!S.row[r].ok) continue;
    const int64_t pi = int64_t(S.row[r].slot) * a.n_qheads + S.row[r].qh;
    float* op = a.o_part + pi * D + lane * EPL;
#pragma unroll
    for (int k4 = 0; k4 < EPL / 4; ++k4)
      *reinterpret_cast<f32x4*>(op + 4 * k4) =
          f32x4{S.o[r][4 * k4], S.o[r][4 * k4 + 1], S.o[r][4 * k4 + 2], S.o[r][4 * k4 + 3]};
    if (lane == 0) {
      a.m_part[pi] = S.m[r];
      a.l_part[pi] = S.l[r];
    }
  }
}

// single wave: rows [rbeg, rbeg + R) over the whole chunk, written directly
template <typename T, int D, int R>
__device__ __forceinline__ void valu_wave_item(const PartialArgs& a, const WorkItem& it, int h, int rbeg) {
  ValuState<T, D, R> S;
  valu_init(S, a, it, h, rbeg);
  valu_stream(S, a, it, h, it.tok0, it.tok1);
  valu_merge_lanes(S);
  valu_write(S, a);
}

// four waves split the chunk's tokens, merge through LDS, write
template <typename T, int D, int R>
__device__ void valu_block_item(const PartialArgs& a, const WorkItem& it, int h, int rbeg, float* lds) {
  constexpr int EPL = D / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tg = lane >> 3, e = lane & 7;
  ValuState<T, D, R> S;
  valu_init(S, a, it, h, rbeg);
  const int ntok = it.tok1 - it.tok0;
  const int per = (((ntok + kWaves - 1) / kWaves) + 7) & ~7;
  const int wb = it.tok0 + wave * per;
  valu_stream(S, a, it, h, wb, min(it.tok1, wb + per));
  valu_merge_lanes(S);
  // [wave][r][D + 2]
  constexpr int RS = D + 2;
  if (tg == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float* row = lds + (wave * R + r) * RS;
#pragma unroll
      for (int k = 0; k < EPL; ++k) row[e * EPL + k] = S.o[r][k];
      if (e == 0) {
        row[D] = S.m[r];
        row[D + 1] = S.l[r];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * D; idx += kBlock) {
    const int r = idx / D, d = idx - (idx / D) * D;
    RowRef rf{0, 0, 0, 0, false};
#pragma unroll
    for (int x = 0; x < R; ++x)
      if (x == r) rf = S.row[x];
    if (!rf.ok) continue;
    float M = TA_NEG_INF;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds[(w * R + r) * RS + D]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* row = lds + (w * R + r) * RS;
      const float wgt = (M == TA_NEG_INF) ? 0.0f : part_weight(row[D], M);
      acc += row[d] * wgt;
      lsum += row[D + 1] * wgt;
    }
    const int64_t pi = int64_t(rf.slot) * a.n_qheads + rf.qh;
    a.o_part[pi * D + d] = acc;
    if (d == 0) {
      a.m_part[pi] = M;
      a.l_part[pi] = lsum;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// GEMM path (bf16): 16-row tiles, 32-token tiles, v_mfma_f32_16x16x32_bf16.
// Lane (i = lane % 16, j = lane / 16). In a 32-token tile the lane's P/V
// token set is tau(j, e) = 4j + e for e < 4 and 16 + 4j + (e - 4) otherwise:
// exactly the tokens its S^T accumulators hold for row i.
__device__ __forceinline__ int tau(int j, int e) { return (e < 4) ? 4 * j + e : 16 + 4 * j + (e - 4); }

template <int DPL>
struct VSlice;  // DPL bf16 values of one token, V^T operand source
template <>
struct VSlice<8> {
  u32x4 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ uint32_t word(int x) const { return w[x]; }
};
template <>
struct VSlice<4> {
  u32x2 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ uint32_t word(int x) const { return w[x]; }
};

template <int D, int NRTW>
struct MfmaState {
  static constexpr int KK = D / 32, DPL = D / 16;
  bf16x8 qf[NRTW][KK];
  f32x4 O[NRTW][DPL];
  float m[NRTW], l[NRTW];
  RowRef row[NRTW];
  bool on[NRTW];  // wave-uniform: row tile k exists
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
    S.m[k] = TA_NEG_INF;
    S.l[k] = 0.0f;
#pragma unroll
    for (int db = 0; db < DPL; ++db) S.O[k][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int x = 0; x < 8; ++x) S.qf[k][kk][x] = __bf16(0.0f);
    if (S.row[k].ok) {
      const __bf16* qp = qbase + (int64_t(S.row[k].gq) * a.n_qheads + S.row[k].qh) * D + j * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) S.qf[k][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 32);
    }
  }
}

// stream 32-token tiles kt = kt0, kt0 + kstep, ... of the item's chunk
template <int D, int NRTW>
__device__ __forceinline__ void mfma_stream(MfmaState<D, NRTW>& S, const PartialArgs& a, const WorkItem& it,
                                            int h, int kt0, int kstep) {
  constexpr int KK = D / 32, DPL = D / 16;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, j = lane >> 4;
  const int ntiles = (it.tok1 - it.tok0 + 31) >> 5;
  if (kt0 >= ntiles) return;
  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + int64_t(h) * a.stride_head + j * 8;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + int64_t(h) * a.stride_head + i * DPL;
  const int32_t* st = a.seg_tok + it.seg_base;
  const int last = it.tok1 - 1;

  u32x4 kc[2][KK];
  VSlice<DPL> vc[8];
  {
    const int base = it.tok0 + kt0 * 32;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t off = tok_off(st[min(base + tb * 16 + i, last)], a);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kc[tb][kk] = *reinterpret_cast<const u32x4*>(kb + off + kk * 32);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vc[e].load(vb + tok_off(st[min(base + tau(j, e), last)], a));
  }
  for (int kt = kt0; kt < ntiles; kt += kstep) {
    const int base = it.tok0 + kt * 32;
    const int nbase = base + kstep * 32;
    const bool more = kt + kstep < ntiles;
    u32x4 kn[2][KK];
    VSlice<DPL> vn[8];
    if (more) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int64_t off = tok_off(st[min(nbase + tb * 16 + i, last)], a);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kn[tb][kk] = *reinterpret_cast<const u32x4*>(kb + off + kk * 32);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vn[e].load(vb + tok_off(st[min(nbase + tau(j, e), last)], a));
    }

    // V^T operands: A_db element e = V[tau(j, e)][DPL * i + db]
    bf16x8 vt[DPL];
#pragma unroll
    for (int db = 0; db < DPL; ++db) {
      u32x4 wv;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t x0 = vc[2 * u].word(db >> 1), x1 = vc[2 * u + 1].word(db >> 1);
        wv[u] = (db & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
      }
      vt[db] = __builtin_bit_cast(bf16x8, wv);
    }

#pragma unroll
    for (int k = 0; k < NRTW; ++k) {
      if (!S.on[k]) continue;
      f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[0][kk]), S.qf[k][kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[1][kk]), S.qf[k][kk], s1, 0, 0, 0);
      }
      float sv[8];
      const int vis = S.row[k].vis;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t0 = base + 4 * j + c, t1 = base + 16 + 4 * j + c;
        sv[c] = (t0 < it.tok1 && t0 < vis) ? s0[c] * a.scale_log2 : TA_NEG_INF;
        sv[4 + c] = (t1 < it.tok1 && t1 < vis) ? s1[c] * a.scale_log2 : TA_NEG_INF;
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (mx > S.m[k] + kRescale) {
        const float al = part_weight(S.m[k], mx);
        S.l[k] *= al;
#pragma unroll
        for (int db = 0; db < DPL; ++db) S.O[k][db] *= al;
        S.m[k] = mx;
      }
      // P = P_hi + P_lo, both bf16: the product keeps ~16 mantissa bits of P
      // (a single bf16 P would cost up to 2^-9 relative per weight, visible
      // when a query sees only a few tokens).
      bf16x8 pb, pl;
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = (sv[e] == TA_NEG_INF) ? 0.0f : fast_exp2(sv[e] - S.m[k]);
        psum += p;
        const __bf16 hi = __bf16(p);
        pb[e] = hi;
        pl[e] = __bf16(p - float(hi));
      }
      S.l[k] += psum;
#pragma unroll
      for (int db = 0; db < DPL; ++db) {
        S.O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[db], pb, S.O[k][db], 0, 0, 0);
        S.O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[db], pl, S.O[k][db], 0, 0, 0);
      }
    }

    if (more) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kc[tb][kk] = kn[tb][kk];
#pragma unroll
      for (int e = 0; e < 8; ++e) vc[e] = vn[e];
    }
  }
}

// l is lane-partial (its 8 tokens per tile); sum over the row's 4 lanes
template <int D, int NRTW>
__device__ __forceinline__ void mfma_finish(MfmaState<D, NRTW>& S) {
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    S.l[k] += __shfl_xor(S.l[k], 16, 64);
    S.l[k] += __shfl_xor(S.l[k], 32, 64);
  }
}

// lane (i, j) holds O[row i][d = DPL * (4j + c) + db] = O[k][db][c]
template <int D, int NRTW>
__device__ __forceinline__ void mfma_write(const MfmaState<D, NRTW>& S, const PartialArgs& a) {
  constexpr int DPL = D / 16;
  const int j = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    if (!S.row[k].ok) continue;
    const int64_t pi = int64_t(S.row[k].slot) * a.n_qheads + S.row[k].qh;
    float* op = a.o_part + pi * D + 4 * j * DPL;
#pragma unroll
    for (int x4 = 0; x4 < DPL; ++x4) {
      f32x4 v;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int x = 4 * x4 + y;  // local offset = c * DPL + db
        v[y] = S.O[k][x % DPL][x / DPL];
      }
      *reinterpret_cast<f32x4*>(op + 4 * x4) = v;
    }
    if (j == 0) {
      a.m_part[pi] = S.m[k];
      a.l_part[pi] = S.l[k];
    }
  }
}

// workgroup item, bf16: rows [16 * rt_base, ...) in nrt_pass row tiles. With
// few tiles the waves also split the tokens (WT > 1) and merge through LDS.
template <int D, int NRTW>
__device__ void mfma_block_pass(const PartialArgs& a, const WorkItem& it, int h, int rt_base, int nrt_pass,
                                float* lds) {
  constexpr int DPL = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, j = lane >> 4;
  const int WR = (nrt_pass <= 1) ? 1 : (nrt_pass <= 2) ? 2 : 4;
  const int WT = kWaves / WR;
  const int wr = wave % WR, wt = wave / WR;
  int rt[NRTW];
  bool on[NRTW];
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    on[k] = wr + k * WR < nrt_pass;
    rt[k] = rt_base + wr + k * WR;
  }
  MfmaState<D, NRTW> S;
  mfma_init(S, a, it, h, rt, on);
  mfma_stream(S, a, it, h, wt, WT);
  mfma_finish(S);

  constexpr int RS = D + 2;
  if (WT > 1) {  // then each wave has one row tile (k = 0)
    if (wt > 0 && S.on[0]) {
      float* buf = lds + ((wt - 1) * WR + wr) * 16 * RS + i * RS;
#pragma unroll
      for (int db = 0; db < DPL; ++db)
#pragma unroll
        for (int c = 0; c < 4; ++c) buf[DPL * (4 * j + c) + db] = S.O[0][db][c];
      if (j == 0) {
        buf[D] = S.m[0];
        buf[D + 1] = S.l[0];
      }
    }
    __syncthreads();
    if (wt == 0 && S.on[0]) {
      for (int w2 = 1; w2 < WT; ++w2) {
        const float* buf = lds + ((w2 - 1) * WR + wr) * 16 * RS + i * RS;
        const float mo = buf[D], lo = buf[D + 1];
        const float M = fmaxf(S.m[0], mo);
        const float as = part_weight(S.m[0], M), ao = part_weight(mo, M);
        S.l[0] = S.l[0] * as + lo * ao;
#pragma unroll
        for (int db = 0; db < DPL; ++db)
#pragma unroll
          for (int c = 0; c < 4; ++c) S.O[0][db][c] = S.O[0][db][c] * as + buf[DPL * (4 * j + c) + db] * ao;
        S.m[0] = M;
      }
    }
    __syncthreads();
  }
  if (wt == 0) mfma_write(S, a);
}

// ---------------------------------------------------------------------------
// Workgroup items (groups with many rows): one workgroup per item x kv-head.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void block_items_kernel(PartialArgs a) {
  __shared__ float lds[3 * 16 * (D + 2)];
  const int item = blockIdx.x / a.n_kvheads;
  const int h = blockIdx.x - item * a.n_kvheads;
  const WorkItem it = a.items[item];
  if constexpr (std::is_same<T, __bf16>::value) {
    const int nrt = (it.nrows + 15) >> 4;
    if (nrt <= 4) {
      mfma_block_pass<D, 1>(a, it, h, 0, nrt, lds);
    } else {
      for (int rb = 0; rb < nrt; rb += 8) mfma_block_pass<D, 2>(a, it, h, rb, min(8, nrt - rb), lds);
    }
  } else {
    for (int r = 0; r < it.nrows; r += 4) valu_block_item<T, D, 4>(a, it, h, r, lds);
  }
}

// Single-wave items (groups with few rows): each wave of the launch is one
// item x kv-head and streams its whole chunk alone -- no LDS, no barrier.
template <typename T, int D>
__global__ __launch_bounds__(kBlock, 2) void wave_items_kernel(PartialArgs a, int item0, int n_units) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kWaves + wave;
  if (unit >= n_units) return;
  const int item = item0 + unit / a.n_kvheads;
  const int h = unit - (unit / a.n_kvheads) * a.n_kvheads;
  const WorkItem it = a.items[item];
  if constexpr (std::is_same<T, __bf16>::value) {
    if (it.nrows > kValuMaxRows) {
      int rt[1] = {0};
      bool on[1] = {true};
      MfmaState<D, 1> S;
      mfma_init(S, a, it, h, rt, on);
      mfma_stream(S, a, it, h, 0, 1);
      mfma_finish(S);
      mfma_write(S, a);
      return;
    }
  }
  if (it.nrows <= 1) {
    valu_wave_item<T, D, 1>(a, it, h, 0);
  } else if (it.nrows <= 2) {
    valu_wave_item<T, D, 2>(a, it, h, 0);
  } else {
    for (int r = 0; r < it.nrows; r += 4) valu_wave_item<T, D, 4>(a, it, h, r);
  }
}

// ---------------------------------------------------------------------------
// One wave handles 64 / (D / 4) (query, q-head) pairs, D / 4 lanes each with
// a float4 of the output. Slots are read in batches of 8 so their loads are in
// flight together; each batch is folded into the running (M, L, acc).
constexpr int kReduceBatch = 8;

template <int D>
__global__ __launch_bounds__(64) void lse_reduce_kernel(ReduceArgs a) {
  constexpr int LP = D / 4;
  constexpr int PPW = 64 / LP;
  const int pair = blockIdx.x * PPW + threadIdx.x / LP;
  const int sub = threadIdx.x % LP;
  if (pair >= a.n_queries * a.n_qheads) return;
  const int q = pair / a.n_qheads;
  const int hq = pair - q * a.n_qheads;
  float M = TA_NEG_INF, L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int s0 = a.q_slot_ptr[q], s1 = a.q_slot_ptr[q + 1];
  for (int b = s0; b < s1; b += kReduceBatch) {
    int64_t pi[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) pi[u] = int64_t(a.q_slots[min(b + u, s1 - 1)]) * a.n_qheads + hq;
    float mv[kReduceBatch], lv[kReduceBatch];
    f32x4 ov[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      mv[u] = (b + u < s1) ? a.m_part[pi[u]] : TA_NEG_INF;
      lv[u] = a.l_part[pi[u]];
      ov[u] = *reinterpret_cast<const f32x4*>(a.o_part + pi[u] * D + sub * 4);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) Mn = fmaxf(Mn, mv[u]);
    const float wa = part_weight(M, Mn);
    acc *= wa;
    L *= wa;
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      const float w = part_weight(mv[u], Mn);
      acc += ov[u] * w;
      L += lv[u] * w;
    }
    M = Mn;
  }
  const float inv = 1.0f / L;
  *reinterpret_cast<f32x4*>(a.out + (int64_t(q) * a.n_qheads + hq) * D + sub * 4) = acc * inv;
}

__global__ void fill_kernel(float* p, int64_t n, float value) {
  for (int64_t x = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; x < n; x += int64_t(gridDim.x) * blockDim.x)
    p[x] = value;
}

}  // namespace

hipError_t launch_partial(const PartialArgs& a, int32_t n_block_items, int32_t n_wave_items, int dtype,
                          int head_dim, hipStream_t s) {
  const int H = a.n_kvheads;
  if (n_block_items > 0) {
    const dim3 grid(unsigned(n_block_items) * H), block(kBlock);
    if (dtype == 1) {
      if (head_dim == 128) hipLaunchKernelGGL((block_items_kernel<__bf16, 128>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((block_items_kernel<__bf16, 64>), grid, block, 0, s, a);
    } else {
      if (head_dim == 128) hipLaunchKernelGGL((block_items_kernel<float, 128>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((block_items_kernel<float, 64>), grid, block, 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_wave_items > 0) {
    const int n_units = n_wave_items * H;
    const dim3 grid(unsigned((n_units + kWaves - 1) / kWaves)), block(kBlock);
    if (dtype == 1) {
      if (head_dim == 128) hipLaunchKernelGGL((wave_items_kernel<__bf16, 128>), grid, block, 0, s, a, n_block_items, n_units);
      else hipLaunchKernelGGL((wave_items_kernel<__bf16, 64>), grid, block, 0, s, a, n_block_items, n_units);
    } else {
      if (head_dim == 128) hipLaunchKernelGGL((wave_items_kernel<float, 128>), grid, block, 0, s, a, n_block_items, n_units);
      else hipLaunchKernelGGL((wave_items_kernel<float, 64>), grid, block, 0, s, a, n_block_items, n_units);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, hipStream_t s) {
  const int64_t pairs = int64_t(a.n_queries) * a.n_qheads;
  if (pairs <= 0) return hipSuccess;
  const int ppw = 64 / (head_dim / 4);
  const dim3 grid(unsigned((pairs + ppw - 1) / ppw)), block(64);
  if (head_dim == 128) hipLaunchKernelGGL(lse_reduce_kernel<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(lse_reduce_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace ta
