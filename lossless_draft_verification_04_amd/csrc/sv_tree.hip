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
//     make one pass over their held slices of the node's row pair per
//     rejection; the pass totals are exchanged, and the final draw searches
//     one held slice.
#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_walk.hpp"

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
  zero_slots(a.slots, (int64_t)a.B * 2 * a.G, bid, kTNT);  // for the walk launch
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
// Walk.  The G blocks of a sequence each own one slice of every row the walk
// draws from (sv_walk.hpp) and replay the walk in lockstep.  At each node a
// block loads its slice of the node's target and draft rows into registers
// once, together with the node's statistics parts and its children's
// logits; every rejection is then one pass over the held slice and one
// exchange of the slice sums.  Every decision is a deterministic function of
// global data and of the exchanged totals (the same bit pattern in every
// block), so every block walks the identical path.  Block 0 writes the
// per-child outputs; the owner of the slice holding the draw searches it.
// ---------------------------------------------------------------------------
constexpr int kWNT = 256;      // walk block
constexpr int kMaxParts = 64;  // stats parts per row staged by the walk

template <int DT, bool HELD>
__global__ __launch_bounds__(kWNT) void tree_walk_kernel(TreeParams a) {
  const int b = blockIdx.x / a.G;
  const int g = blockIdx.x - b * a.G;
  Exchange x = make_exchange(a.slots, a.err, b, a.G, g);
  const int64_t spv = (a.nvec + a.G - 1) / a.G;
  const int64_t v0 = (int64_t)g * spv < a.nvec ? (int64_t)g * spv : a.nvec;
  const int64_t v1 = v0 + spv < a.nvec ? v0 + spv : a.nvec;
  const bool writer = (g == 0);
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
  __shared__ uint64_t s_words[kMaxG];
  __shared__ double s_val[kMaxG];
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
  Slice<DT, kWNT, HELD> sl;
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
      // bonus draw from P_node (not streamed by the stats pass): the row's
      // maximum from the slices, then a plain draw with that shift
      sl.load(rowP, nullptr, v0, v1);
      const float M = exchange_max(x, sl.max_logit(a.c, a.V), s_words);
      if (M == kNegInf && writer && threadIdx.x == 0) set_error(a.err, SV_DERR_ROW);
      DrawSpec sp;
      sp.rowP = rowP;
      sp.rowQ = nullptr;
      sp.c = a.c;
      sp.cmP = M == kNegInf ? 0.f : a.c * M;
      sp.invSP = 1.f;
      sp.cmQ = 0.f;
      sp.invSQ = 1.f;
      sp.coef = 0.f;
      const double total = exchange_sum(x, sl.prepare(sp, a.V), s_words, s_val);
      int pick;
      double loc;
      slice_scan(s_val, x.G, us * total, &pick, &loc);
      if (pick == g) t = sl.search(sp, a.V, loc);
      break;
    }
    const void* rowQ = row_ptr(a.drf, rowbase + node, a.drf_sb);
    // one round of loads: the held slice of the node's rows, its stats parts
    // and every child's logits
    sl.load(rowP, rowQ, v0, v1);
    const int np = a.nch <= kMaxParts ? a.nch : kMaxParts;
    const Partial* pn = parts + (rowbase + node) * 2 * a.nch;
    for (int i = threadIdx.x; i < 2 * np; i += kWNT) {
      const Partial pi = get_partial(pn + (i < np ? i : a.nch + (i - np)));
      s_pm[i] = pi.m;
      s_ps[i] = pi.s;
    }
    for (int k = threadIdx.x; k < nk; k += kWNT) {
      const int32_t tk = s_tok[s_kids[k]];
      float zp = 0.f, zq = 0.f;
      if (tk >= 0 && tk < a.V) {
        zp = load_elem<DT>(rowP, tk);
        zq = load_elem<DT>(rowQ, tk);
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
    double c = 0.0, D = 1.0;
    bool sums_current = false;  // s_val holds the slice sums of the current residual
    int accepted = -1;
    for (int kk = 0; kk < nk; ++kk) {
      const int ch = s_kids[kk];
      const int32_t tk = s_tok[ch];
      double pt = 0.0, qt = 0.0;
      if (tk >= 0 && tk < a.V) {
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
      const double Dn = exchange_sum(x, sl.prepare(sp, a.V), s_words, s_val);
      if (Dn > 0.0) {
        c = cn;
        D = Dn;
        sums_current = true;
      } else {
        sums_current = false;  // residual mass rounded to 0: keep the previous residual
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
    if (!sums_current) D = exchange_sum(x, sl.prepare(sp, a.V), s_words, s_val);
    int pick;
    double loc;
    slice_scan(s_val, x.G, us * D, &pick, &loc);
    if (pick == g) t = sl.search(sp, a.V, loc);
    break;
  }
  __syncthreads();
  if (writer) {
    for (int d = threadIdx.x; d < a.max_depth; d += kWNT)
      a.out_path[(int64_t)b * a.max_depth + d] = d < depth ? s_path[d] : -1;
    if (threadIdx.x == 0) a.out_len[b] = depth;
  }
  if (t >= 0 && threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
}

template <int DT>
hipError_t launch_tree_t(const TreeParams& p, const Plan& plan, hipStream_t s) {
  tree_stats_kernel<DT><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // B * G <= the blocks the device holds at once (chosen by the caller): a
  // sequence's blocks are resident together on an otherwise idle device,
  // and their waits are bounded either way
  if (p.held)
    tree_walk_kernel<DT, true><<<dim3((unsigned)p.B * p.G), dim3(kWNT), 0, s>>>(p);
  else
    tree_walk_kernel<DT, false><<<dim3((unsigned)p.B * p.G), dim3(kWNT), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_tree(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  return dt == SV_BF16 ? launch_tree_t<SV_BF16>(p, plan, s) : launch_tree_t<SV_F32>(p, plan, s);
}

// Blocks of the walk kernel the device holds at once.
int tree_walk_capacity(sv_dtype dt, bool held) {
  static int cache[2][2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& c = cache[dt == SV_BF16][held][dev];
  if (c == 0) {
    const void* fn;
    if (dt == SV_BF16)
      fn = held ? reinterpret_cast<const void*>(&tree_walk_kernel<SV_BF16, true>)
                : reinterpret_cast<const void*>(&tree_walk_kernel<SV_BF16, false>);
    else
      fn = held ? reinterpret_cast<const void*>(&tree_walk_kernel<SV_F32, true>)
                : reinterpret_cast<const void*>(&tree_walk_kernel<SV_F32, false>);
    c = device_capacity(fn, kWNT, dev);
  }
  return c;
}

}  // namespace sv
