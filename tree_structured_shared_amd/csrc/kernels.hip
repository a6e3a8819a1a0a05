// HIP kernels for tree-structured decode attention on CDNA4 (gfx950).
//
// partial_attn: one workgroup (4 x wave64) per work item x kv-head. A work item
// is one KV chunk of one context-query group and a block of its rows (row =
// query x q-head-in-group). The workgroup streams the chunk's paged K/V once
// for all its rows -- the KV-guided grouping of the DeFT reading notes and the
// single-launch, one-group-per-block-set kernel of the FastTree review
// (section 3, kernel design) -- and runs a flash-style online softmax over it
// (DeFT notes, attention calculation; FastTree review, tile-by-tile online
// softmax). It writes one unnormalised partial (m, l, o) per row.
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
// GEMV path: up to R rows, 8 lanes per token, 2 tokens per lane group per step.
template <typename T, int D, int R>
__device__ void valu_rows(const PartialArgs& a, const WorkItem& it, int h, int rbeg, float* lds) {
  constexpr int EPL = D / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tg = lane >> 3, e = lane & 7;

  float q[R][EPL];
  int vis[R], slot[R], qh[R];
  bool ok[R];
  const T* qbase = reinterpret_cast<const T*>(a.q);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = rbeg + r;
    ok[r] = rr < it.nrows;
    vis[r] = 0;
    slot[r] = 0;
    qh[r] = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) q[r][k] = 0.0f;
    if (ok[r]) {
      const int grow = it.row0 + rr;
      const int qig = grow / a.g, hig = grow - qig * a.g;
      const int gq = a.group_qs[it.q_ptr + qig];
      vis[r] = a.group_vis[it.q_ptr + qig];
      slot[r] = it.slot0 + qig;
      qh[r] = h * a.g + hig;
      Slice<T, EPL> sq;
      sq.load(qbase + (int64_t(gq) * a.n_qheads + qh[r]) * D + e * EPL);
      sq.to_float(q[r]);
    }
  }

  float m[R], l[R], o[R][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = TA_NEG_INF;
    l[r] = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) o[r][k] = 0.0f;
  }

  const int ntok = it.tok1 - it.tok0;
  const int per = (((ntok + kWaves - 1) / kWaves) + 7) & ~7;
  const int wb = it.tok0 + wave * per;
  const int we = min(it.tok1, wb + per);
  const T* kb = reinterpret_cast<const T*>(a.k) + int64_t(h) * a.stride_head + e * EPL;
  const T* vb = reinterpret_cast<const T*>(a.v) + int64_t(h) * a.stride_head + e * EPL;
  const int32_t* st = a.seg_tok + it.seg_base;

  if (wb < we) {
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
          for (int k = 0; k < EPL; ++k) acc = __builtin_fmaf(q[r][k], kf[u][k], acc);
          acc += __shfl_xor(acc, 1, 64);
          acc += __shfl_xor(acc, 2, 64);
          acc += __shfl_xor(acc, 4, 64);
          const int t = base + u * 8 + tg;
          s[u] = (t < we && t < vis[r]) ? acc * a.scale_log2 : TA_NEG_INF;
        }
        const float smax = fmaxf(s[0], s[1]);
        if (smax > m[r] + kRescale) {
          const float al = part_weight(m[r], smax);
          l[r] *= al;
#pragma unroll
          for (int k = 0; k < EPL; ++k) o[r][k] *= al;
          m[r] = smax;
        }
        const float p0 = (s[0] == TA_NEG_INF) ? 0.0f : fast_exp2(s[0] - m[r]);
        const float p1 = (s[1] == TA_NEG_INF) ? 0.0f : fast_exp2(s[1] - m[r]);
        l[r] += p0 + p1;
#pragma unroll
        for (int k = 0; k < EPL; ++k) o[r][k] = __builtin_fmaf(p1, vf[1][k], __builtin_fmaf(p0, vf[0][k], o[r][k]));
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

  // merge the 8 token groups of the wave (lanes e, e+8, ..., e+56)
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) {
      const float mo = __shfl_xor(m[r], x, 64);
      const float lo = __shfl_xor(l[r], x, 64);
      const float M = fmaxf(m[r], mo);
      const float as = part_weight(m[r], M), ao = part_weight(mo, M);
      l[r] = l[r] * as + lo * ao;
#pragma unroll
      for (int k = 0; k < EPL; ++k) o[r][k] = o[r][k] * as + __shfl_xor(o[r][k], x, 64) * ao;
      m[r] = M;
    }
  }
  // merge the 4 waves through LDS: [wave][r][D + 2]
  constexpr int RS = D + 2;
  if (tg == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float* row = lds + (wave * R + r) * RS;
#pragma unroll
      for (int k = 0; k < EPL; ++k) row[e * EPL + k] = o[r][k];
      if (e == 0) {
        row[D] = m[r];
        row[D + 1] = l[r];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * D; idx += kBlock) {
    const int r = idx / D, d = idx - (idx / D) * D;
    bool rok = false;
    int rs = 0, rq = 0;
#pragma unroll
    for (int x = 0; x < R; ++x)
      if (x == r) {
        rok = ok[x];
        rs = slot[x];
        rq = qh[x];
      }
    if (!rok) continue;
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
    const int64_t pi = int64_t(rs) * a.n_qheads + rq;
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
__device__ void mfma_rows(const PartialArgs& a, const WorkItem& it, int h, int rt_base, int nrt_pass,
                          float* lds) {
  constexpr int KK = D / 32;
  constexpr int DPL = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, j = lane >> 4;
  const int WR = (nrt_pass <= 1) ? 1 : (nrt_pass <= 2) ? 2 : 4;
  const int WT = kWaves / WR;
  const int wr = wave % WR, wt = wave / WR;

  const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q);
  bf16x8 qf[NRTW][KK];
  int vis[NRTW], slot[NRTW], qh[NRTW];
  bool tok_[NRTW], rok[NRTW];
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    const int rt_local = wr + k * WR;
    tok_[k] = rt_local < nrt_pass;  // wave-uniform: tile exists
    const int rr = (rt_base + rt_local) * 16 + i;
    rok[k] = tok_[k] && rr < it.nrows;
    vis[k] = 0;
    slot[k] = 0;
    qh[k] = 0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int x = 0; x < 8; ++x) qf[k][kk][x] = __bf16(0.0f);
    if (rok[k]) {
      const int grow = it.row0 + rr;
      const int qig = grow / a.g, hig = grow - qig * a.g;
      const int gq = a.group_qs[it.q_ptr + qig];
      vis[k] = a.group_vis[it.q_ptr + qig];
      slot[k] = it.slot0 + qig;
      qh[k] = h * a.g + hig;
      const __bf16* qp = qbase + (int64_t(gq) * a.n_qheads + qh[k]) * D + j * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[k][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 32);
    }
  }

  f32x4 O[NRTW][DPL];
  float m[NRTW], l[NRTW];
#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    m[k] = TA_NEG_INF;
    l[k] = 0.0f;
#pragma unroll
    for (int db = 0; db < DPL; ++db) O[k][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int ntok = it.tok1 - it.tok0;
  const int ntiles = (ntok + 31) >> 5;
  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + int64_t(h) * a.stride_head + j * 8;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + int64_t(h) * a.stride_head + i * DPL;
  const int32_t* st = a.seg_tok + it.seg_base;
  const int last = it.tok1 - 1;

  if (wt < ntiles) {
    u32x4 kc[2][KK];
    VSlice<DPL> vc[8];
    {
      const int base = it.tok0 + wt * 32;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int64_t off = tok_off(st[min(base + tb * 16 + i, last)], a);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kc[tb][kk] = *reinterpret_cast<const u32x4*>(kb + off + kk * 32);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vc[e].load(vb + tok_off(st[min(base + tau(j, e), last)], a));
    }
    for (int kt = wt; kt < ntiles; kt += WT) {
      const int base = it.tok0 + kt * 32;
      const int nbase = base + WT * 32;
      u32x4 kn[2][KK];
      VSlice<DPL> vn[8];
      if (kt + WT < ntiles) {
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
        if (!tok_[k]) continue;
        f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[0][kk]), qf[k][kk], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[1][kk]), qf[k][kk], s1, 0, 0, 0);
        }
        float sv[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int t0 = base + 4 * j + c, t1 = base + 16 + 4 * j + c;
          sv[c] = (t0 < it.tok1 && t0 < vis[k]) ? s0[c] * a.scale_log2 : TA_NEG_INF;
          sv[4 + c] = (t1 < it.tok1 && t1 < vis[k]) ? s1[c] * a.scale_log2 : TA_NEG_INF;
        }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (mx > m[k] + kRescale) {
          const float al = part_weight(m[k], mx);
          l[k] *= al;
#pragma unroll
          for (int db = 0; db < DPL; ++db) O[k][db] *= al;
          m[k] = mx;
        }
        // P = P_hi + P_lo, both bf16: the product keeps ~16 mantissa bits of P
        // (a single bf16 P would cost up to 2^-9 relative per weight, visible
        // when a query sees only a few tokens).
        bf16x8 pb, pl;
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = (sv[e] == TA_NEG_INF) ? 0.0f : fast_exp2(sv[e] - m[k]);
          psum += p;
          const __bf16 hi = __bf16(p);
          pb[e] = hi;
          pl[e] = __bf16(p - float(hi));
        }
        l[k] += psum;
#pragma unroll
        for (int db = 0; db < DPL; ++db) {
          O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[db], pb, O[k][db], 0, 0, 0);
          O[k][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[db], pl, O[k][db], 0, 0, 0);
        }
      }

      if (kt + WT < ntiles) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) kc[tb][kk] = kn[tb][kk];
#pragma unroll
        for (int e = 0; e < 8; ++e) vc[e] = vn[e];
      }
    }
  }

#pragma unroll
  for (int k = 0; k < NRTW; ++k) {
    l[k] += __shfl_xor(l[k], 16, 64);
    l[k] += __shfl_xor(l[k], 32, 64);
  }

  // token-split waves (WT > 1, one row tile each) merge into wt == 0 via LDS
  constexpr int RS = D + 2;
  if (WT > 1) {
    if (wt > 0 && tok_[0]) {
      float* buf = lds + ((wt - 1) * WR + wr) * 16 * RS + i * RS;
#pragma unroll
      for (int db = 0; db < DPL; ++db)
#pragma unroll
        for (int c = 0; c < 4; ++c) buf[DPL * (4 * j + c) + db] = O[0][db][c];
      if (j == 0) {
        buf[D] = m[0];
        buf[D + 1] = l[0];
      }
    }
    __syncthreads();
    if (wt == 0 && tok_[0]) {
      for (int w2 = 1; w2 < WT; ++w2) {
        const float* buf = lds + ((w2 - 1) * WR + wr) * 16 * RS + i * RS;
        const float mo = buf[D], lo = buf[D + 1];
        const float M = fmaxf(m[0], mo);
        const float as = part_weight(m[0], M), ao = part_weight(mo, M);
        l[0] = l[0] * as + lo * ao;
#pragma unroll
        for (int db = 0; db < DPL; ++db)
#pragma unroll
          for (int c = 0; c < 4; ++c) O[0][db][c] = O[0][db][c] * as + buf[DPL * (4 * j + c) + db] * ao;
        m[0] = M;
      }
    }
    __syncthreads();
  }

  if (wt == 0) {
#pragma unroll
    for (int k = 0; k < NRTW; ++k) {
      if (!rok[k]) continue;
      const int64_t pi = int64_t(slot[k]) * a.n_qheads + qh[k];
      float* op = a.o_part + pi * D + 4 * j * DPL;
#pragma unroll
      for (int x4 = 0; x4 < DPL; ++x4) {
        f32x4 v;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int x = 4 * x4 + y;  // local offset = c * DPL + db
          v[y] = O[k][x % DPL][x / DPL];
        }
        *reinterpret_cast<f32x4*>(op + 4 * x4) = v;
      }
      if (j == 0) {
        a.m_part[pi] = m[k];
        a.l_part[pi] = l[k];
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void partial_attn_kernel(PartialArgs a) {
  __shared__ float lds[3 * 16 * (D + 2)];
  const int item = blockIdx.x / a.n_kvheads;
  const int h = blockIdx.x - item * a.n_kvheads;
  const WorkItem it = a.items[item];
  if constexpr (std::is_same<T, __bf16>::value) {
    if (it.nrows > kValuMaxRows) {
      const int nrt = (it.nrows + 15) >> 4;
      if (nrt <= 4) {
        mfma_rows<D, 1>(a, it, h, 0, nrt, lds);
      } else {
        for (int rb = 0; rb < nrt; rb += 8) mfma_rows<D, 2>(a, it, h, rb, min(8, nrt - rb), lds);
      }
      return;
    }
  }
  if (it.nrows <= 1) {
    valu_rows<T, D, 1>(a, it, h, 0, lds);
  } else if (it.nrows <= 2) {
    valu_rows<T, D, 2>(a, it, h, 0, lds);
  } else {
    for (int r = 0; r < it.nrows; r += 4) valu_rows<T, D, 4>(a, it, h, r, lds);
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

hipError_t launch_partial(const PartialArgs& a, int32_t n_work, int dtype, int head_dim,
                          hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  const dim3 grid(n_work), block(kBlock);
  if (dtype == 1) {
    if (head_dim == 128) hipLaunchKernelGGL((partial_attn_kernel<__bf16, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((partial_attn_kernel<__bf16, 64>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((partial_attn_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((partial_attn_kernel<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
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
