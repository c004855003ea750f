// sv_tree.hip -- token-tree verification on gfx950.
//
// PRESTO page §2.1: the target accepts tree candidates sequentially from the
// root until a mismatch.  At every child the draft-then-verify page's §2.1
// rule applies (accept with min(1, p/q)); after a rejected sibling the
// target distribution is replaced by its residual norm(max(0, p - q)) with the
// node's draft q kept (siblings tried in node order), which after i
// rejections is (p - c_i q)^+ / D_i with c_{i+1} = c_i + D_i and
// D_{i+1} = sum_v (p - c_{i+1} q)^+.  An accepted child becomes the current
// node; when all children are rejected the correction is drawn from the last
// residual; a node without children gives the bonus draw from its target row.
//
// Two launches per call:
//  1. stats: a block per (node, target|draft, row part) of every node that
//     has children (leaf rows are skipped), streaming each row once.
//  2. walk: G blocks per sequence replay the walk in lockstep: merge the
//     parts of the node they stand on, decide its children in order, and
//     split one pass over the node's row pair per rejection into slices; the
//     pass totals are exchanged, so the final draw only re-reads one slice.
#include "sv_device.hpp"
#include "sv_internal.h"

namespace sv {

constexpr int kTNT = 256;
constexpr int kTU = 4;

template <int DT>
__global__ __launch_bounds__(kTNT) void tree_stats_kernel(TreeParams a) {
  const int64_t per_node = 2 * (int64_t)a.nch;
  const int64_t per_seq = (int64_t)a.N * per_node;
  const int64_t bid = blockIdx.x;
  const int b = (int)(bid / per_seq);
  int64_t rem = bid - (int64_t)b * per_seq;
  const int u = (int)(rem / per_node);
  rem -= (int64_t)u * per_node;
  const int which = (int)(rem / a.nch);
  const int ch = (int)(rem - (int64_t)which * a.nch);
  int has_kids = 0;
  for (int i = u + 1 + threadIdx.x; i < a.N; i += kTNT) has_kids |= (a.parent[(int64_t)b * a.N + i] == u);
  if (!__syncthreads_or(has_kids)) return;
  const void* row = which ? row_ptr(a.drf, (int64_t)b * a.N + u, a.drf_sb) : row_ptr(a.tgt, (int64_t)b * a.N + u, a.tgt_sb);
  const int64_t v0 = (int64_t)ch * a.vpc;
  const int64_t v1 = v0 + a.vpc < a.nvec ? v0 + a.vpc : a.nvec;
  const Partial part = range_stats<DT, kTNT, kTU>(row, a.V, v0, v1, a.c);
  if (threadIdx.x == 0) put_partial(static_cast<Partial*>(a.part) + (((int64_t)b * a.N + u) * 2 + which) * a.nch + ch, part);
}

// ---------------------------------------------------------------------------
// Walk.  The G blocks of a sequence (G = 1 .. 64, at most one block per
// compute unit over the whole launch, so all of them are resident together)
// each own one slice of every row pass.  After a pass the blocks add
// (1 << 56) + round(slice sum * 2^54) into one 64-bit word of a 3-word ring
// per sequence: the top byte counts arrivals, the rest is the pass total in
// fixed point, so one device-scope atomic per block both delivers the sum and
// marks the arrival, and the total is the same bit pattern in every block
// whatever the arrival order.  Every decision is a deterministic function of
// global data and of these totals, so every block replays the identical walk.
// Slice sums also go to device-scope slots (read only for the final draw).
// Block 0 writes the per-child outputs; the owner of the slice holding the
// draw searches it.  Waits are bounded: a block that waits too long sets
// SV_DERR_TIMEOUT and goes on.
// ---------------------------------------------------------------------------
constexpr int kWNT = 256;  // walk block
constexpr int kMaxG = 64;  // walk blocks (slices) per sequence
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kMaxParts = 64;  // stats parts per row staged by the walk
constexpr int kRing = 3;       // pass-total words per sequence
constexpr double kFix = 18014398509481984.0;  // 2^54: totals up to 4 fit under the arrival byte
constexpr uint64_t kArrive = 1ull << 56;

struct WalkCtx {
  const TreeParams* a;
  int b, g, G;
  int64_t v0, v1;     // this block's slice of every row pass
  uint64_t* ring;     // [kRing] pass-total words of this sequence
  Partial* xch;       // [2][kMaxG] slice slots of this sequence
  int pass;           // exchanges so far
  bool late;          // a wait ran out: later exchanges do not wait
};

// Exchange this block's slice part.  Returns the fixed-point total of the
// parts' s (meaningful for residual passes, whose s is in [0, 1]); the parts
// themselves are left in the slots of this pass's parity.
__device__ double exchange(WalkCtx& w, const Partial& mine, bool sum) {
  __shared__ double s_total;
  Partial* slot = w.xch + (w.pass & 1) * kMaxG;
  // slice sums of a residual lie in [0, 1] (up to rounding); anything else
  // (a row error upstream) is clamped so it cannot reach the arrival byte
  const double s_in = sum && mine.s > 0.0 ? fmin(mine.s, 2.0) : 0.0;
  const uint64_t fixed = (uint64_t)llrint(s_in * kFix);
  if (w.G == 1) {
    if (threadIdx.x == 0) put_partial(slot, mine);
    __syncthreads();
    ++w.pass;
    return (double)fixed / kFix;
  }
  if (threadIdx.x == 0) put_partial(slot + w.g, mine);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* word = w.ring + (w.pass % kRing);
    __hip_atomic_fetch_add(word, kArrive + fixed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (!w.late && (v >> 56) < (uint64_t)w.G) {
      if (++spins > kSpinLimit) {
        set_error(w.a->err, SV_DERR_TIMEOUT);
        w.late = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_total = (double)(v & (kArrive - 1)) / kFix;
    // every block has now added to this pass's word, hence has finished
    // reading the previous one: block 0 clears it for reuse three passes on
    if (w.g == 0 && w.pass >= 1) {
      __hip_atomic_store(w.ring + ((w.pass - 1) % kRing), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  __syncthreads();
  const double t = s_total;
  __syncthreads();
  ++w.pass;
  return t;
}

// Read the G slice parts of pass `pass` into s_m / s_s.
__device__ void read_slices(const WalkCtx& w, int pass, float* s_m, double* s_s) {
  const Partial* slot = w.xch + (pass & 1) * kMaxG;
  if (threadIdx.x < w.G) {
    const Partial p = get_partial(slot + threadIdx.x);
    s_m[threadIdx.x] = p.m;
    s_s[threadIdx.x] = p.s;
  }
  __syncthreads();
}

// Draw from slice weights s_w (G of them, total `total`): locate the slice
// holding u * total; its owner block searches it and returns the token
// (-1 in the other blocks).
template <int DT>
__device__ int64_t slice_draw(const WalkCtx& w, const DrawSpec& sp, const double* s_w, double total, double u) {
  const double target = u * total;
  double cum = 0.0, cum_last = 0.0, loc = 0.0;
  int pick = -1, last = -1;
  for (int i = 0; i < w.G; ++i) {
    const double x = s_w[i];
    if (x > 0.0) {
      last = i;
      cum_last = cum;
    }
    if (pick < 0 && cum + x > target) {
      pick = i;
      loc = target - cum;
    }
    cum += x;
  }
  if (pick < 0) {
    pick = last < 0 ? 0 : last;
    loc = cum - cum_last;
  }
  if (pick != w.g) return -1;
  return block_search<DT, kWNT>(sp, w.a->V, w.v0, w.v1, loc);
}

template <int DT>
__global__ __launch_bounds__(kWNT) void tree_walk_kernel(TreeParams a) {
  WalkCtx w;
  w.a = &a;
  w.G = a.G;
  w.b = blockIdx.x / a.G;
  w.g = blockIdx.x - w.b * a.G;
  {
    const int64_t spv = (a.nvec + a.G - 1) / a.G;
    w.v0 = (int64_t)w.g * spv < a.nvec ? (int64_t)w.g * spv : a.nvec;
    w.v1 = w.v0 + spv < a.nvec ? w.v0 + spv : a.nvec;
  }
  w.ring = static_cast<uint64_t*>(a.ring) + (int64_t)w.b * kRing;
  w.xch = static_cast<Partial*>(a.xch) + (int64_t)w.b * 2 * kMaxG;
  w.pass = 0;
  w.late = false;
  const int b = w.b;
  const bool writer = (w.g == 0);
  const int64_t rowbase = (int64_t)b * a.N;
  const Partial* parts = static_cast<const Partial*>(a.part);
  __shared__ int32_t s_par[SV_MAX_N];
  __shared__ int32_t s_tok[SV_MAX_N];
  __shared__ int s_kids[SV_MAX_N];
  __shared__ int32_t s_path[SV_MAX_N];
  __shared__ float s_zp[SV_MAX_N], s_zq[SV_MAX_N];
  __shared__ float s_pm[2 * kMaxParts];
  __shared__ double s_ps[2 * kMaxParts];
  __shared__ RowStat s_P, s_Q;
  __shared__ float s_m[kMaxG];
  __shared__ double s_s[kMaxG];
  __shared__ int s_cnt;
  const double us = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);

  // the tree's shape and tokens, once
  for (int i = threadIdx.x; i < a.N; i += kWNT) {
    const int32_t pi = a.parent[rowbase + i];
    s_par[i] = pi;
    s_tok[i] = a.tok[rowbase + i];
    if (writer && i > 0 && (pi < 0 || pi >= i)) set_error(a.err, SV_DERR_TREE);
  }
  __syncthreads();

  int node = 0, depth = 0;
  int64_t t = -1;
  for (;;) {
    // children of `node` in increasing index (from LDS)
    if (threadIdx.x == 0) s_cnt = 0;
    __syncthreads();
    for (int base = node + 1; base < a.N; base += kWNT) {
      const int i = base + (int)threadIdx.x;
      const int flag = (i < a.N) && s_par[i] == node;
      double excl;
      const double tot = block_exclusive_scan<kWNT>((double)flag, &excl);
      if (flag) s_kids[s_cnt + (int)excl] = i;
      __syncthreads();
      if (threadIdx.x == 0) s_cnt += (int)tot;
      __syncthreads();
    }
    const int nk = s_cnt;
    const void* rowP = row_ptr(a.tgt, rowbase + node, a.tgt_sb);
    if (nk == 0 || depth >= a.max_depth) {
      if (nk > 0 && writer) set_error(a.err, SV_DERR_TREE);
      // bonus draw from P_node (not streamed by the stats pass): online slice
      // statistics, exchanged, then the draw with the merged shift
      const Partial st = range_stats<DT, kWNT, 4>(rowP, a.V, w.v0, w.v1, a.c);
      const int bp = w.pass;
      exchange(w, st, false);
      read_slices(w, bp, s_m, s_s);
      float M = kNegInf;
      for (int i = 0; i < w.G; ++i) M = fmaxf(M, s_m[i]);
      const float cm = a.c * M;
      double total = 0.0;
      __syncthreads();
      if (threadIdx.x < w.G)
        s_s[threadIdx.x] = s_m[threadIdx.x] == kNegInf ? 0.0
                                                       : s_s[threadIdx.x] * exp2((double)(a.c * s_m[threadIdx.x]) -
                                                                                 (double)cm);
      __syncthreads();
      for (int i = 0; i < w.G; ++i) total += s_s[i];
      if (M == kNegInf && writer && threadIdx.x == 0) set_error(a.err, SV_DERR_ROW);
      DrawSpec sp;
      sp.rowP = rowP;
      sp.rowQ = nullptr;
      sp.c = a.c;
      sp.cmP = cm;
      sp.invSP = 1.f;
      sp.cmQ = 0.f;
      sp.invSQ = 1.f;
      sp.coef = 0.f;
      t = slice_draw<DT>(w, sp, s_s, total, us);
      break;
    }
    const void* rowQ = row_ptr(a.drf, rowbase + node, a.drf_sb);
    // one round of loads: the node's stats parts and every child's logits
    const int np = a.nch <= kMaxParts ? a.nch : kMaxParts;
    const Partial* pn = parts + (rowbase + node) * 2 * a.nch;
    for (int i = threadIdx.x; i < 2 * np; i += kWNT) {
      const Partial pi = get_partial(pn + (i < np ? i : a.nch + (i - np)));
      s_pm[i] = pi.m;
      s_ps[i] = pi.s;
    }
    for (int k = threadIdx.x; k < nk; k += kWNT) {
      const int32_t x = s_tok[s_kids[k]];
      float zp = 0.f, zq = 0.f;
      if (x >= 0 && x < a.V) {
        zp = load_elem<DT>(rowP, x);
        zq = load_elem<DT>(rowQ, x);
      }
      s_zp[k] = zp;
      s_zq[k] = zq;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      const float* pm = s_pm + threadIdx.x * np;
      const double* ps = s_ps + threadIdx.x * np;
      float M = kNegInf;
      for (int i = 0; i < np; ++i) M = fmaxf(M, pm[i]);
      RowStat r;
      r.pad = 0.f;
      r.cm = M == kNegInf ? 0.f : a.c * M;
      double S = 0.0;
      if (M != kNegInf)
        for (int i = 0; i < np; ++i)
          if (pm[i] != kNegInf) S += ps[i] * exp2((double)(a.c * pm[i]) - (double)r.cm);
      r.S = S;
      if (threadIdx.x == 0) s_P = r; else s_Q = r;
    }
    __syncthreads();
    const RowStat P = s_P, Q = s_Q;
    if (writer && threadIdx.x == 0 && (!(P.S > 0.0) || !(Q.S > 0.0))) set_error(a.err, SV_DERR_ROW);
    DrawSpec sp;
    sp.rowP = rowP;
    sp.rowQ = rowQ;
    sp.c = a.c;
    sp.cmP = P.cm;
    sp.invSP = P.S > 0.0 ? (float)(1.0 / P.S) : 0.f;
    sp.cmQ = Q.cm;
    sp.invSQ = Q.S > 0.0 ? (float)(1.0 / Q.S) : 0.f;
    double c = 0.0, D = 1.0, total = 0.0;
    int sums_pass = -1;  // pass whose slice sums are those of the current residual
    int accepted = -1;
    for (int kk = 0; kk < nk; ++kk) {
      const int ch = s_kids[kk];
      const int32_t x = s_tok[ch];
      double pt = 0.0, qt = 0.0;
      if (x >= 0 && x < a.V) {
        pt = prob_of(s_zp[kk], a.c, P);
        qt = prob_of(s_zq[kk], a.c, Q);
      } else if (writer && threadIdx.x == 0) {
        set_error(a.err, SV_DERR_TOKEN);
      }
      if (writer && threadIdx.x == 0) {
        if (a.out_p) a.out_p[rowbase + ch] = (float)pt;
        if (a.out_q) a.out_q[rowbase + ch] = (float)qt;
      }
      const double pcur = fmax(0.0, pt - c * qt) / D;
      const double r = uniform24(a.seed, (uint32_t)ch, (uint32_t)b, 0, a.round, 0);
      if (r < accept_ratio(pcur, qt)) {
        accepted = ch;
        break;
      }
      const double cn = c + D;
      sp.coef = (float)cn;
      Partial mine;
      mine.m = 0.f;
      mine.pad = 0.f;
      mine.s = range_weight_sum<DT, kWNT>(sp, a.V, w.v0, w.v1);
      const int this_pass = w.pass;
      const double G = exchange(w, mine, true);
      if (G > 0.0) {
        c = cn;
        D = G;
        total = G;
        sums_pass = this_pass;
      } else {
        sums_pass = -1;  // residual mass rounded to 0: keep the previous residual
      }
    }
    if (accepted >= 0) {
      if (threadIdx.x == 0) s_path[depth] = accepted;
      ++depth;
      node = accepted;
      __syncthreads();
      continue;
    }
    // every child rejected: draw from (p - c q)^+
    sp.coef = (float)c;
    if (sums_pass < 0) {
      Partial mine;
      mine.m = 0.f;
      mine.pad = 0.f;
      mine.s = range_weight_sum<DT, kWNT>(sp, a.V, w.v0, w.v1);
      sums_pass = w.pass;
      total = exchange(w, mine, true);
    }
    read_slices(w, sums_pass, s_m, s_s);
    t = slice_draw<DT>(w, sp, s_s, total, us);
    break;
  }
  __syncthreads();
  if (writer) {
    for (int d = threadIdx.x; d < a.max_depth; d += kWNT)
      a.out_path[(int64_t)b * a.max_depth + d] = d < depth ? s_path[d] : -1;
    if (threadIdx.x == 0) a.out_len[b] = depth;
  }
  if (t >= 0 && threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
  // the last block of the sequence to leave clears the ring for the next call
  if (threadIdx.x == 0 && w.G > 1) {
    const uint32_t old = __hip_atomic_fetch_add(a.cnt2 + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)w.G - 1) {
      for (int i = 0; i < kRing; ++i) __hip_atomic_store(w.ring + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.cnt2 + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int DT>
hipError_t launch_tree_t(const TreeParams& p, const Plan& plan, hipStream_t s) {
  tree_stats_kernel<DT><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // B * G <= compute units (chosen by the caller): the walk's blocks are all
  // resident together on an otherwise idle device, and their waits are
  // bounded either way
  tree_walk_kernel<DT><<<dim3((unsigned)p.B * p.G), dim3(kWNT), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_tree(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  return dt == SV_BF16 ? launch_tree_t<SV_BF16>(p, plan, s) : launch_tree_t<SV_F32>(p, plan, s);
}

}  // namespace sv
