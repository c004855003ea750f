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
// Two launches per call:
//  1. statistics: tree_stats_kernel over every node's row pair (leaves
//     included), which also gathers each child's logits under its parent's
//     rows.
//  2. expansion: a block per (node, row part).  Blocks of nodes with children
//     only arrive.  A leaf's block merges the node's row statistics, turns its
//     part of the row pair into proxy scores (base 2, in registers) and keeps
//     each wave's k best (sv_topk.hpp); the waves' lists merge into the
//     part's list.  The last block of a sequence to arrive computes every
//     node's s and S (level by level from the root, so each S is summed in
//     root-to-node order), merges each leaf's part lists into its top k, and
//     those into the sequence's top b.
#include <cmath>

#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_topk.hpp"

namespace sv {

constexpr int kPNT = 256;
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

// A leaf's row pair as a value source for the wave top-k scan.
template <int DT>
struct ProxyValues {
  const void* rowP;
  const void* rowQ;
  int V;
  float c, offP, offQ, lam;
  struct Data {
    u32x4 p, q;
  };
  static constexpr bool kSkipNegInf = true;
  __device__ __forceinline__ Data load(int64_t v) const { return Data{load_vec(rowP, v), load_vec(rowQ, v)}; }
  __device__ __forceinline__ void values(const Data& d, int64_t v, float* x) const {
    constexpr int E = Fmt<DT>::kPerVec;
    float zp[E];
    unpack<DT>(d.p, zp);
    unpack<DT>(d.q, x);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = proxy_log2(zp[e], x[e], c, offP, offQ, lam);
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

// Lambda of a node at depth d >= 1.
__device__ __forceinline__ float lambda_at(const PrestoParams& a, int d) { return a.lam[(d < a.D ? d : a.D) - 1]; }

// Insert (v, n, t) into a wave's sorted list of (priority desc, node asc,
// token asc); lane l holds entry l, lanes >= F the empty entry (node kNoIdx).
__device__ __forceinline__ bool cand_better(float va, int32_t na, int32_t ta, float vb, int32_t nb, int32_t tb) {
  if (na == kNoIdx) return false;
  if (nb == kNoIdx) return true;
  if (va != vb) return va > vb;
  if (na != nb) return na < nb;
  return ta < tb;
}
__device__ __forceinline__ void wave_insert3(float& lv, int32_t& ln, int32_t& lt, float v, int32_t n, int32_t t,
                                             int F, int lane) {
  const bool here = lane < F && cand_better(v, n, t, lv, ln, lt);
  const uint64_t m = __ballot(here);
  if (!m) return;
  const int pos = __builtin_ctzll(m);
  const float up_v = dpp_f<kWaveShr1, 0xF>(lv, lv);
  const int32_t up_n = dpp_i<kWaveShr1, 0xF>(ln, ln);
  const int32_t up_t = dpp_i<kWaveShr1, 0xF>(lt, lt);
  if (lane < F) {
    if (lane > pos) {
      lv = up_v;
      ln = up_n;
      lt = up_t;
    } else if (lane == pos) {
      lv = v;
      ln = n;
      lt = t;
    }
  }
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
  for (int i = threadIdx.x; i < a.N; i += kPNT) {
    const int32_t p = a.parent[rowbase + i];
    s_par[i] = (i > 0 && p >= 0 && p < i) ? p : 0;
  }
  if (threadIdx.x == 0) s_flag = 0;
  lds_sync();
  for (int i = u + 1 + (int)threadIdx.x; i < a.N; i += kPNT)
    if (s_par[i] == u) s_flag = 1;
  if (threadIdx.x == 0) {
    int d = 0;
    for (int j = u; j > 0; j = s_par[j]) ++d;
    s_depth = d;
  }
  lds_sync();
  TopEntry* lists = static_cast<TopEntry*>(a.lists) + ((rowbase + u) * a.nch2 + ch) * a.k;
  if (!s_flag) {
    // a leaf: its k best proposals in this part of its row pair
    const float offP = row_offset(a, rowbase + u, 0);
    const float offQ = row_offset(a, rowbase + u, 1);
    const ProxyValues<DT> src{row_ptr(a.tgt, rowbase + u, a.tgt_sb), row_ptr(a.drf, rowbase + u, a.drf_sb), a.V,
                              a.c, offP, offQ, lambda_at(a, s_depth + 1)};
    if (ch == 0 && threadIdx.x == 0 && (offP == __builtin_huge_valf() || offQ == __builtin_huge_valf()))
      set_error(a.err, SV_DERR_ROW);
    float lv = kNegInf;
    int32_t li = kNoIdx;
    const int64_t v0 = (int64_t)ch * a.vpc2;
    const int64_t v1 = v0 + a.vpc2 < a.nvec ? v0 + a.vpc2 : a.nvec;
    wave_topk_scan<kPNT, E>(src, v0, v1, a.V, a.k, lv, li);
    __shared__ TopEntry s_list[kPNT / kWave][SV_MAX_FANOUT];
    lds_sync();
    if (lane < SV_MAX_FANOUT) {
      s_list[wave][lane].val = lv;
      s_list[wave][lane].idx = li;
    }
    lds_sync();
    if (wave == 0) {
      for (int w = 1; w < kPNT / kWave; ++w)
        for (int e = 0; e < a.k; ++e) {
          const TopEntry t = s_list[w][e];
          const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), a.k - 1));
          const int32_t ti = __builtin_amdgcn_readlane(li, a.k - 1);
          if (t.idx == kNoIdx || (ti != kNoIdx && !top_better(t.val, t.idx, tv, ti))) break;
          wave_insert(lv, li, t.val, t.idx, a.k, lane);
        }
      if (lane < a.k) put_entry(lists + lane, lv, li);
    }
  }
  if (!arrive_last<kPNT>(&a.cnt[b], (uint32_t)(a.N * a.nch2))) return;

  // ---- the sequence's last block: scores, path scores, top b proposals
  __shared__ float s_off[2][SV_MAX_N];  // row offsets of the nodes with children (target, draft)
  __shared__ float s_s[SV_MAX_N], s_S[SV_MAX_N];
  __shared__ int s_dep[SV_MAX_N];
  __shared__ uint8_t s_leaf[SV_MAX_N];
  __shared__ int s_changed;
  for (int i = threadIdx.x; i < a.N; i += kPNT) {
    s_leaf[i] = 1;
    s_dep[i] = i == 0 ? 0 : -1;
  }
  lds_sync();
  if (threadIdx.x == 0) {
    for (int i = 1; i < a.N; ++i) {
      const int32_t p = a.parent[rowbase + i];
      if (p < 0 || p >= i) set_error(a.err, SV_DERR_TREE);
    }
  }
  for (int i = 1 + threadIdx.x; i < a.N; i += kPNT) s_leaf[s_par[i]] = 0;
  lds_sync();
  for (int i = threadIdx.x; i < 2 * a.N; i += kPNT) {
    const int node = i >> 1, which = i & 1;
    if (!s_leaf[node]) s_off[which][node] = row_offset(a, rowbase + node, which);
  }
  lds_sync();
  const float* zt = a.zc + rowbase;
  const float* zd = a.zc + (int64_t)a.B * a.N + rowbase;
  // depth and path score, level by level (parents precede children)
  if (threadIdx.x == 0) {
    s_s[0] = 0.f;
    s_S[0] = 0.f;
  }
  for (int level = 1;; ++level) {
    if (threadIdx.x == 0) s_changed = 0;
    lds_sync();
    for (int i = 1 + threadIdx.x; i < a.N; i += kPNT) {
      const int p = s_par[i];
      if (s_dep[i] < 0 && s_dep[p] == level - 1) {
        const float zp = zt[i], zq = zd[i];
        float sc;
        if (__builtin_isnan(zp) || __builtin_isnan(zq)) {
          set_error(a.err, SV_DERR_TOKEN);
          sc = kNegInf;
        } else {
          sc = proxy_log2(zp, zq, a.c, s_off[0][p], s_off[1][p], lambda_at(a, level)) * kLn2;
        }
        s_s[i] = sc;
        s_S[i] = s_S[p] + sc;
        s_dep[i] = level;
        s_changed = 1;
      }
    }
    lds_sync();
    if (!s_changed) break;
  }
  for (int i = threadIdx.x; i < a.N; i += kPNT) {
    if (a.out_s) a.out_s[rowbase + i] = s_s[i];
    if (a.out_S) a.out_S[rowbase + i] = s_S[i];
  }
  // every leaf's part lists -> its top k -> the wave's top b; waves take
  // leaves in turn
  float gv = kNegInf;
  int32_t gn = kNoIdx, gt = kNoIdx;
  const TopEntry* all = static_cast<const TopEntry*>(a.lists) + rowbase * a.nch2 * a.k;
  for (int leaf = wave; leaf < a.N; leaf += kPNT / kWave) {
    if (!s_leaf[leaf]) continue;
    float lv = kNegInf;
    int32_t li = kNoIdx;
    for (int c = 0; c < a.nch2; ++c)
      for (int e = 0; e < a.k; ++e) {
        const TopEntry t = get_entry(all + ((int64_t)leaf * a.nch2 + c) * a.k + e);
        const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), a.k - 1));
        const int32_t ti = __builtin_amdgcn_readlane(li, a.k - 1);
        if (t.idx == kNoIdx || (ti != kNoIdx && !top_better(t.val, t.idx, tv, ti))) break;
        wave_insert(lv, li, t.val, t.idx, a.k, lane);
      }
    // the leaf's list is sorted by score, so by priority: stop at the first
    // entry that does not enter the top b
    const float Su = s_S[leaf];
    for (int e = 0; e < a.k; ++e) {
      const int32_t t = __builtin_amdgcn_readlane(li, e);
      if (t == kNoIdx) break;
      const float pr = Su + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), e)) * kLn2;
      const float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), a.b_top - 1));
      const int32_t bn = __builtin_amdgcn_readlane(gn, a.b_top - 1);
      const int32_t bt = __builtin_amdgcn_readlane(gt, a.b_top - 1);
      if (!cand_better(pr, leaf, t, bv, bn, bt)) break;
      wave_insert3(gv, gn, gt, pr, leaf, t, a.b_top, lane);
    }
  }
  __shared__ float m_v[kPNT / kWave][SV_MAX_FANOUT];
  __shared__ int32_t m_n[kPNT / kWave][SV_MAX_FANOUT], m_t[kPNT / kWave][SV_MAX_FANOUT];
  if (lane < SV_MAX_FANOUT) {
    m_v[wave][lane] = gv;
    m_n[wave][lane] = gn;
    m_t[wave][lane] = gt;
  }
  lds_sync();
  if (wave == 0) {
    for (int w = 1; w < kPNT / kWave; ++w)
      for (int e = 0; e < a.b_top; ++e) {
        const float v = m_v[w][e];
        const int32_t n = m_n[w][e], t = m_t[w][e];
        const float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), a.b_top - 1));
        const int32_t bn = __builtin_amdgcn_readlane(gn, a.b_top - 1);
        const int32_t bt = __builtin_amdgcn_readlane(gt, a.b_top - 1);
        if (!cand_better(v, n, t, bv, bn, bt)) break;
        wave_insert3(gv, gn, gt, v, n, t, a.b_top, lane);
      }
    if (lane < a.b_top) {
      const bool has = gn != kNoIdx;
      a.out_node[(int64_t)b * a.b_top + lane] = has ? gn : -1;
      a.out_tok[(int64_t)b * a.b_top + lane] = has ? gt : -1;
      if (a.out_score) a.out_score[(int64_t)b * a.b_top + lane] = has ? gv : kNegInf;
    }
    if (lane == 0) __hip_atomic_store(&a.cnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  return hipGetLastError();
}

}  // namespace sv
