// sv_presto.hip -- PRESTO prefix-aligned scoring and one priority expansion
// step on gfx950.
//
// PRESTO page §4.1: a drafted token's score is s = log q(t) + lambda_d *
// log rho(t) with rho = min(1, p/q), the log of the KL-regularised proxy
// p* ~ q rho^lambda (§4.4) up to its normaliser; a path's score is the sum of
// its tokens' scores (eq. 10).  §4.3, self-speculative form: the target's
// conditional rows of the tree are at hand, so rho is exact (no learned
// predictor).  §4.2: priority-based construction expands the best-scoring
// candidates; one step here proposes, from every leaf u, its k best tokens
// under the proxy and keeps the sequence's b best proposals by priority
// S_u + s_u(t).
//
// Three launches per call:
//  1. statistics: tree_stats_kernel over every node's row pair (leaves
//     included), which also gathers each child's logits under its parent's
//     rows.
//  2. expansion: a block per (node, row part); blocks of nodes with children
//     exit.  A leaf's block merges the node's row statistics, turns its part
//     of the row pair into proxy scores (in registers) and keeps each wave's
//     k best (sv_topk.hpp); the waves' lists merge into the part's list, and
//     the leaf's last part to finish merges the parts' lists into the leaf's
//     top k.
//  3. final: a block per sequence computes every node's s and S (level by
//     level from the root, so each S is summed in root-to-node order) and
//     ranks the leaves' proposals into the sequence's top b.
#include <cmath>

#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_topk.hpp"

namespace sv {

constexpr int kPNT = 256;   // expansion block
constexpr int kPFT = 1024;  // final block: one per sequence, on an otherwise idle device
constexpr int kStageE = 1024;  // proposal entries the final launch stages at once
constexpr int kMaxParts = 64;  // statistics parts per row (the plan caps it)
constexpr int kFinalParts = 2048;  // statistics parts the final launch stages in LDS (2 rows per node)
static_assert(kStageE <= kPFT, "a thread of the final launch prefetches at most one entry of the first chunk");
static_assert(SV_MAX_N % kPFT == 0 && kFinalParts % kPFT == 0, "whole loads per thread");
constexpr float kLn2 = 0.69314718055994531f;

hipError_t launch_tree_stats(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);

// log2 of a token's proxy weight q * rho^lambda from its two logits:
// log2 q = z_q c - offQ, log2 p = z_p c - offP (off = c * max + log2 S);
// -inf where q = 0, or where p = 0 and lambda > 0.
__device__ __forceinline__ float proxy_log2(float zp, float zq, float c, float offP, float offQ, float lam) {
  const float lq = __builtin_fmaf(zq, c, -offQ);
  if (lam == 0.f) return lq;
  const float lp = __builtin_fmaf(zp, c, -offP);
  // fminf drops a NaN (both logits -inf): lq is -inf there anyway
  return lq + lam * fminf(0.f, lp - lq);
}

// A leaf's row pair as a value source for the wave top-k scan.  It lists
// the proxy in logit units, y = z_q + lambda * min(0, z_p - z_q - delta)
// with delta = (offP - offQ) / c: log2 of the proxy weight is c * y - offQ,
// an increasing affine map, so the order (and every tie) is the same, and
// each token costs four operations after unpacking.  lambda = 0 lists z_q
// (LAM0: no 0 * -inf where p = 0).
template <int DT, bool LAM0>
struct ProxyValues {
  const void* rowP;
  const void* rowQ;
  int V;
  float delta, lam;
  struct Data {
    u32x4 p, q;
  };
  static constexpr bool kSkipNegInf = true;
  __device__ __forceinline__ Data load(int64_t v) const {
    if constexpr (LAM0) return Data{d_zero(), load_vec(rowQ, v)};
    return Data{load_vec(rowP, v), load_vec(rowQ, v)};
  }
  static __device__ __forceinline__ u32x4 d_zero() { return u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void values(const Data& d, int64_t v, float* x) const {
    constexpr int E = Fmt<DT>::kPerVec;
    unpack<DT>(d.q, x);
    if constexpr (!LAM0) {
      float zp[E];
      unpack<DT>(d.p, zp);
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __builtin_fmaf(lam, fminf(0.f, (zp[e] - x[e]) - delta), x[e]);
    }
    if ((v + 1) * E > V) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (v * E + e >= V) x[e] = kNegInf;
    }
  }
};

// Row statistic of a node's row `which` (0 target, 1 draft) as the offset
// c * max + log2 S (+inf for a row without a finite logit: every proxy
// weight of it is then -inf).
__device__ float row_offset(const PrestoParams& a, int64_t node_row, int which) {
  const RowStat st = merge_parts(static_cast<const Partial*>(a.part) + (node_row * 2 + which) * a.nch1, a.nch1, a.c);
  if (!(st.S > 0.0)) return __builtin_huge_valf();
  return (float)((double)st.cm + log2(st.S));
}

// The same offset from n parts staged in LDS (merge_parts' arithmetic, in
// part order).
__device__ float row_offset_staged(const Partial* pp, int n, float c) {
  float M = kNegInf;
  for (int i = 0; i < n; ++i) M = fmaxf(M, pp[i].m);
  if (M == kNegInf) return __builtin_huge_valf();
  const float cm = c * M;
  double S = 0.0;
  for (int i = 0; i < n; ++i)
    if (pp[i].m != kNegInf) S += pp[i].s * exp2_d((double)(c * pp[i].m) - (double)cm);
  if (!(S > 0.0)) return __builtin_huge_valf();
  return (float)((double)cm + log2(S));
}

// Lambda of a node at depth d >= 1.
__device__ __forceinline__ float lambda_at(const PrestoParams& a, int d) { return a.lam[(d < a.D ? d : a.D) - 1]; }

// Candidate order: priority descending, then node ascending, then token
// ascending; an empty entry (node kNoIdx) beats nothing.
__device__ __forceinline__ bool cand_better(float va, int32_t na, int32_t ta, float vb, int32_t nb, int32_t tb) {
  if (na == kNoIdx) return false;
  if (nb == kNoIdx) return true;
  if (va != vb) return va > vb;
  if (na != nb) return na < nb;
  return ta < tb;
}
template <int DT>
__global__ __launch_bounds__(kPNT) void presto_expand_kernel(PrestoParams a) {
  constexpr int E = Fmt<DT>::kPerVec;
  const int64_t bid = blockIdx.x;
  const int ch = (int)(bid % a.nch2);
  const int64_t rest = bid / a.nch2;
  const int b = (int)(rest % a.B);
  const int u = (int)(rest / a.B);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t rowbase = (int64_t)b * a.N;
  __shared__ int32_t s_par[SV_MAX_N];  // parents, each clamped below its node
  __shared__ int s_flag, s_depth;
  __shared__ Partial s_parts[2][kMaxParts];  // the node's row statistics parts (target, draft)
  __shared__ float s_offs[2];
  __shared__ float s_lamv[SV_MAX_N];  // lambda of depths 1..N
  // one round of loads: the parents, the node's parts of both rows, lambda
  for (int i = threadIdx.x; i < a.N; i += kPNT) {
    const int32_t p = a.parent[rowbase + i];
    s_par[i] = (i > 0 && p >= 0 && p < i) ? p : 0;
  }
  for (int i = threadIdx.x; i < a.N; i += kPNT) s_lamv[i] = a.lam[(i + 1 < a.D ? i + 1 : a.D) - 1];
  for (int i = threadIdx.x; i < 2 * a.nch1; i += kPNT)
    s_parts[i / a.nch1][i % a.nch1] =
        static_cast<const Partial*>(a.part)[((rowbase + u) * 2 + i / a.nch1) * a.nch1 + i % a.nch1];
  if (threadIdx.x == 0) s_flag = 0;
  lds_sync();
  for (int i = u + 1 + (int)threadIdx.x; i < a.N; i += kPNT)
    if (s_par[i] == u) s_flag = 1;
  if (threadIdx.x < 2) {
    // offset c * max + log2 S of row `which` (+inf for a row without a finite logit)
    const Partial* pp = s_parts[threadIdx.x];
    float M = kNegInf;
    for (int i = 0; i < a.nch1; ++i) M = fmaxf(M, pp[i].m);
    float off = __builtin_huge_valf();
    if (M != kNegInf) {
      const float cm = a.c * M;
      double S = 0.0;
      for (int i = 0; i < a.nch1; ++i)
        if (pp[i].m != kNegInf) S += pp[i].s * exp2_d((double)(a.c * pp[i].m) - (double)cm);
      if (S > 0.0) off = (float)((double)cm + log2(S));
    }
    s_offs[threadIdx.x] = off;
  }
  if (threadIdx.x == kWave) {
    int d = 0;
    for (int j = u; j > 0; j = s_par[j]) ++d;
    s_depth = d;
  }
  lds_sync();
  TopEntry* lists = static_cast<TopEntry*>(a.lists) + ((rowbase + u) * a.nch2 + ch) * a.k;
  if (!s_flag) {
    // a leaf: its k best proposals in this part of its row pair
    const float offP = s_offs[0];
    const float offQ = s_offs[1];
    const bool empty = offP == __builtin_huge_valf() || offQ == __builtin_huge_valf();
    if (ch == 0 && threadIdx.x == 0 && empty) set_error(a.err, SV_DERR_ROW);
    float lv = kNegInf;
    int32_t li = kNoIdx;
    const int64_t v0 = (int64_t)ch * a.vpc2;
    const int64_t v1 = v0 + a.vpc2 < a.nvec ? v0 + a.vpc2 : a.nvec;
    const float lam = s_lamv[s_depth];  // the proposals' depth is the leaf's + 1
    const void* rowP = row_ptr(a.tgt, rowbase + u, a.tgt_sb);
    const void* rowQ = row_ptr(a.drf, rowbase + u, a.drf_sb);
    if (!empty) {
      const TopPair t =
          lam == 0.f
              ? block_topk<kPNT, E, false>(ProxyValues<DT, true>{rowP, rowQ, a.V, 0.f, 0.f}, v0, v1, a.V, a.k)
              : block_topk<kPNT, E, false>(ProxyValues<DT, false>{rowP, rowQ, a.V, (offP - offQ) / a.c, lam},
                                              v0, v1, a.V, a.k);
      lv = t.v;
      li = t.i;
    }
    // wave 0 holds the part's list; logit units -> log2 of the proxy weight
    if (li != kNoIdx) lv = __builtin_fmaf(lv, a.c, -offQ);
    if (wave == 0) {
      if (a.nch2 == 1 && lane < a.k) put_entry(static_cast<TopEntry*>(a.leaf_lists) + (rowbase + u) * a.k + lane, lv, li);
      if (a.nch2 > 1 && lane < a.k) put_entry(lists + lane, lv, li);
    }
    // the leaf's last part to finish merges the parts' lists into the leaf's
    if (a.nch2 > 1 && arrive_last<kPNT>(&a.leaf_cnt[rowbase + u], (uint32_t)a.nch2) && wave == 0) {
      lv = kNegInf;
      li = kNoIdx;
      wave_merge_entries(static_cast<const TopEntry*>(a.lists) + (rowbase + u) * a.nch2 * a.k, a.nch2 * a.k, a.k, lv,
                         li, lane);
      if (lane < a.k) put_entry(static_cast<TopEntry*>(a.leaf_lists) + (rowbase + u) * a.k + lane, lv, li);
      if (lane == 0) __hip_atomic_store(&a.leaf_cnt[rowbase + u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Order key of a candidate at position pos of the ranking array: priority
// descending, then position ascending, as one unsigned compare (floats map
// to unsigned integers in their order, -0 as +0; -inf is above the empty
// key 0).
__device__ __forceinline__ uint64_t rank_key(float v, int pos) {
  const uint32_t bits = __float_as_uint(v == 0.f ? 0.f : v);
  const uint32_t o = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)pos);
}

// One block per sequence (after the expansion launch): every node's s and S,
// each leaf's part lists merged into its top k, and those into the
// sequence's top b.
__global__ __launch_bounds__(kPFT) void presto_final_kernel(PrestoParams a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t rowbase = (int64_t)b * a.N;
  __shared__ int32_t s_par[SV_MAX_N];  // parents, each clamped below its node
  __shared__ float s_off[2][SV_MAX_N];  // row offsets of the nodes with children (target, draft)
  __shared__ float s_s[SV_MAX_N], s_S[SV_MAX_N];
  __shared__ int s_dep[SV_MAX_N];
  __shared__ uint8_t s_leaf[SV_MAX_N];
  // the children's gathered logits and lambda per level, in LDS for the
  // level loop
  __shared__ float s_zt[SV_MAX_N], s_zd[SV_MAX_N], s_lam[SV_MAX_N];
  __shared__ Partial s_pp[kFinalParts];  // every row's statistics parts, when they fit
  const int np = 2 * a.N * a.nch1;
  const bool staged = np <= kFinalParts;  // block-uniform
  const int per_leaf = a.k;
  const int leaves_per_chunk = kStageE / per_leaf;
  const TopEntry* all = static_cast<const TopEntry*>(a.leaf_lists) + rowbase * a.k;
  // one round of loads, every one issued before any is used: the parents,
  // the children's gathered logits, lambda, the rows' statistics parts
  // (written two launches earlier) and this thread's entry of the first
  // chunk of proposals (whether its node is a leaf is known only later)
  constexpr int kPerThread = SV_MAX_N / kPFT;
  constexpr int kPartsPerThread = kFinalParts / kPFT;
  int32_t r_par[kPerThread];
  float r_zt[kPerThread], r_zd[kPerThread], r_lam[kPerThread];
  u32x4 r_pp[kPartsPerThread];
  const u32x4* gparts = reinterpret_cast<const u32x4*>(static_cast<const Partial*>(a.part) + rowbase * 2 * a.nch1);
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int i = (int)threadIdx.x + q * kPFT;
    const int ic = i < a.N ? i : a.N - 1;
    r_par[q] = a.parent[rowbase + ic];
    r_zt[q] = a.zc[rowbase + ic];
    r_zd[q] = a.zc[(int64_t)a.B * a.N + rowbase + ic];
    r_lam[q] = a.lam[(ic + 1 < a.D ? ic + 1 : a.D) - 1];  // depth i + 1
  }
  if (staged) {
#pragma unroll
    for (int q = 0; q < kPartsPerThread; ++q) {
      const int j = (int)threadIdx.x + q * kPFT;
      r_pp[q] = gparts[j < np ? j : np - 1];
    }
  }
  const int ne0 = (a.N < leaves_per_chunk ? a.N : leaves_per_chunk) * per_leaf;  // <= kStageE = kPFT
  const TopEntry pre = get_entry(all + ((int)threadIdx.x < ne0 ? (int)threadIdx.x : 0));
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int i = (int)threadIdx.x + q * kPFT;
    if (i < a.N) {
      const int32_t p = r_par[q];
      const bool ok = i == 0 || (p >= 0 && p < i);
      if (!ok) set_error(a.err, SV_DERR_TREE);
      s_par[i] = (i > 0 && ok) ? p : 0;
      s_leaf[i] = 1;
      s_dep[i] = i == 0 ? 0 : -1;
      s_zt[i] = r_zt[q];
      s_zd[i] = r_zd[q];
      s_lam[i] = r_lam[q];
    }
  }
  if (staged) {
#pragma unroll
    for (int q = 0; q < kPartsPerThread; ++q) {
      const int j = (int)threadIdx.x + q * kPFT;
      if (j < np) {
        s_pp[j].m = __uint_as_float(r_pp[q][0]);
        s_pp[j].pad = 0.f;
        s_pp[j].s = __longlong_as_double((long long)(((uint64_t)r_pp[q][3] << 32) | r_pp[q][2]));
      }
    }
  }
  lds_sync();
  for (int i = 1 + threadIdx.x; i < a.N; i += kPFT) s_leaf[s_par[i]] = 0;
  lds_sync();
  for (int i = threadIdx.x; i < 2 * a.N; i += kPFT) {
    const int node = i >> 1, which = i & 1;
    if (!s_leaf[node])
      s_off[which][node] = staged ? row_offset_staged(s_pp + (node * 2 + which) * a.nch1, a.nch1, a.c)
                                  : row_offset(a, rowbase + node, which);
  }
  lds_sync();
  // depth and path score, level by level (parents precede children), by
  // the first wave alone: its lanes' LDS accesses are performed in program
  // order, so a level needs no block barrier, only a vote on whether any
  // node was placed
  if (wave == 0) {
    if (lane == 0) {
      s_s[0] = 0.f;
      s_S[0] = 0.f;
    }
    for (int level = 1;; ++level) {
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");  // the previous level's writes first
      int placed = 0;
      for (int i = 1 + lane; i < a.N; i += kWave) {
        const int p = s_par[i];
        if (s_dep[i] < 0 && s_dep[p] == level - 1) {
          const float zp = s_zt[i], zq = s_zd[i];
          float sc;
          if (__builtin_isnan(zp) || __builtin_isnan(zq)) {
            set_error(a.err, SV_DERR_TOKEN);
            sc = kNegInf;
          } else {
            sc = proxy_log2(zp, zq, a.c, s_off[0][p], s_off[1][p], s_lam[level - 1]) * kLn2;
          }
          s_s[i] = sc;
          s_S[i] = s_S[p] + sc;
          s_dep[i] = level;
          placed = 1;
        }
      }
      if (!__any(placed)) break;
    }
  }
  lds_sync();
  for (int i = threadIdx.x; i < a.N; i += kPFT) {
    if (a.out_s) a.out_s[rowbase + i] = s_s[i];
    if (a.out_S) a.out_S[rowbase + i] = s_S[i];
  }
  // Proposals: every leaf's list of k (merged by the expansion launch),
  // staged in LDS in chunks of whole leaves with all loads in flight
  // together.  The current top b and the chunk's valid entries are laid out
  // in (node, token) order -- the top b first (earlier chunks hold smaller
  // nodes, and equal priorities among them are already in key order), then
  // each leaf's entries sorted by token -- so that the order (priority
  // descending, (node, token) ascending) is one 64-bit compare of
  // (ordered priority bits, inverted position).  Every candidate counts the
  // candidates that beat it; ranks are distinct, and those below b form the
  // new top b.
  __shared__ float c_v[kStageE];
  __shared__ int32_t c_t[kStageE];
  // candidates: the top b, then the chunk's kept entries, padded to a multiple of 8
  __shared__ float k_v[kStageE + SV_MAX_FANOUT + 8];
  __shared__ int64_t k_key[kStageE + SV_MAX_FANOUT + 8];
  __shared__ uint64_t k_ord[kStageE + SV_MAX_FANOUT + 16];  // 8 spare keys for the read-ahead
  __shared__ int s_rank[kStageE + SV_MAX_FANOUT + 8];  // each candidate's count of better keys
  __shared__ float top_v[SV_MAX_FANOUT];
  __shared__ int32_t top_n[SV_MAX_FANOUT], top_t[SV_MAX_FANOUT];
  __shared__ int s_nk;
  for (int j = threadIdx.x; j < a.b_top; j += kPFT) {
    top_v[j] = kNegInf;
    top_n[j] = kNoIdx;
    top_t[j] = kNoIdx;
  }
  for (int n0 = 0; n0 < a.N; n0 += leaves_per_chunk) {
    const int n1 = n0 + leaves_per_chunk < a.N ? n0 + leaves_per_chunk : a.N;
    const int ne = (n1 - n0) * per_leaf;
    lds_sync();  // the previous chunk is consumed
    for (int e = threadIdx.x; e < ne; e += kPFT) {
      TopEntry t;
      t.val = kNegInf;
      t.idx = kNoIdx;
      // the first chunk's entry was loaded with the tree (e is this thread's index there)
      if (s_leaf[n0 + e / per_leaf]) t = n0 == 0 ? pre : get_entry(all + (int64_t)n0 * per_leaf + e);
      c_v[e] = t.val;
      c_t[e] = t.idx;
    }
    if (threadIdx.x == 0) s_nk = 0;
    // the top b first (empty entries never win and are not ranked)
    for (int j = threadIdx.x; j < a.b_top; j += kPFT) {
      const bool top = top_n[j] != kNoIdx;
      k_v[j] = top_v[j];
      k_key[j] = top ? (((int64_t)top_n[j] << 32) | (uint32_t)top_t[j]) : INT64_MAX;
      k_ord[j] = top ? rank_key(top_v[j], j) : 0ull;
    }
    lds_sync();
    // the kept entries after them, each leaf's by token
    for (int e0 = 0; e0 < ne; e0 += kPFT) {
      const int e = e0 + (int)threadIdx.x;
      const int keep = (e < ne && c_t[e] != kNoIdx) ? 1 : 0;
      double before;
      const int total = (int)block_exclusive_scan<kPFT>((double)keep, &before);
      if (keep) {
        // within the leaf: kept entries before this one, and those with a smaller token
        const int l0 = e - e % per_leaf;
        int prior = 0, smaller = 0;
        for (int q = l0; q < l0 + per_leaf; ++q) {
          const int32_t tq = c_t[q];
          prior += (int)((q < e) & (tq != kNoIdx));
          smaller += (int)((tq != kNoIdx) & (tq < c_t[e]));
        }
        const int at = a.b_top + s_nk + (int)before - prior + smaller;
        const int node = n0 + e / per_leaf;
        const float v = s_S[node] + c_v[e] * kLn2;
        k_v[at] = v;
        k_key[at] = ((int64_t)node << 32) | (uint32_t)c_t[e];
        k_ord[at] = rank_key(v, at);
      }
      lds_sync();
      if (threadIdx.x == 0) s_nk += total;
      lds_sync();
    }
    const int nc = (a.b_top + s_nk + 7) & ~7;
    for (int j = a.b_top + s_nk + (int)threadIdx.x; j < nc; j += kPFT) {
      k_key[j] = INT64_MAX;
      k_ord[j] = 0ull;
    }
    for (int j = threadIdx.x; j < nc; j += kPFT) s_rank[j] = 0;
    lds_sync();
    // every candidate counts the keys above its own, in S segments of the
    // key array at once (S threads per candidate, so that the whole block
    // compares); a segment is a whole number of 8-key groups, and the next
    // eight keys are read while these are compared (the array has 8 spare
    // keys past nc)
    const int S = nc <= kPFT / 2 ? kPFT / nc : 1;
    const int L = ((nc + S - 1) / S + 7) & ~7;
    for (int t = threadIdx.x; t < nc * S; t += kPFT) {
      const int i = t % nc, seg = t / nc;
      const int j_lo = seg * L, j_hi = j_lo + L < nc ? j_lo + L : nc;
      if (k_key[i] == INT64_MAX || j_lo >= j_hi) continue;
      const uint64_t oi = k_ord[i];
      int rank = 0;
      uint64_t oj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) oj[q] = k_ord[j_lo + q];
      for (int j0 = j_lo; j0 < j_hi; j0 += 8) {
        uint64_t on[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) on[q] = k_ord[j0 + 8 + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) rank += (int)(oj[q] > oi);
#pragma unroll
        for (int q = 0; q < 8; ++q) oj[q] = on[q];
      }
      if (rank) atomicAdd(&s_rank[i], rank);
    }
    lds_sync();
    for (int i = threadIdx.x; i < nc; i += kPFT) {
      const int64_t ki = k_key[i];
      const int rank = s_rank[i];
      if (ki != INT64_MAX && rank < a.b_top) {
        top_v[rank] = k_v[i];
        top_n[rank] = (int32_t)(ki >> 32);
        top_t[rank] = (int32_t)(ki & 0xffffffff);
      }
    }
  }
  lds_sync();
  for (int j = threadIdx.x; j < a.b_top; j += kPFT) {
    const bool has = top_n[j] != kNoIdx;
    a.out_node[(int64_t)b * a.b_top + j] = has ? top_n[j] : -1;
    a.out_tok[(int64_t)b * a.b_top + j] = has ? top_t[j] : -1;
    if (a.out_score) a.out_score[(int64_t)b * a.b_top + j] = has ? top_v[j] : kNegInf;
  }
}

hipError_t launch_presto(const PrestoParams& p, const TreeParams& stats, sv_dtype dt, const Plan& plan,
                         hipStream_t s) {
  hipError_t e = launch_tree_stats(stats, dt, plan, s);
  if (e != hipSuccess) return e;
  if (dt == SV_BF16)
    presto_expand_kernel<SV_BF16><<<dim3((unsigned)plan.grid2), dim3(kPNT), 0, s>>>(p);
  else
    presto_expand_kernel<SV_F32><<<dim3((unsigned)plan.grid2), dim3(kPNT), 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  presto_final_kernel<<<dim3((unsigned)p.B), dim3(kPFT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
