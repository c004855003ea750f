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
//  1. stats: a block per (k, sequence, target|draft, row part), where block
//     k of a sequence streams its k-th node with children (found from the
//     parent array in LDS).  The layout is k-major, so the blocks that stream
//     come first and spread evenly over the compute units; blocks past a
//     sequence's last node with children exit at once.  A working block
//     streams its part of the row once; the first part of a row also gathers
//     the row's logits at the node's children's tokens.
//  2. walk: G blocks per sequence replay the walk in lockstep.  Each stages
//     the tree, every node's row statistics and every child's logits in LDS
//     once and computes every child's p, q and uniform there; at a node it
//     tries the children in order and, at the first rejection, loads its
//     slice of the node's row pair into registers; each rejection is one
//     pass over that slice, the pass totals are exchanged, and the final
//     draw searches one held slice.
//
// Point-mass mode (SpecDiff-2 page, Core method: accept a drafted token with
// the verifier's probability, resample the residual on a rejection; read as
// the draft-then-verify page's §2.1 step with q a point mass at the child's
// token).  At a node the children are tried in index order against a running
// residual w = P_node with mass D = 1: child i is accepted iff
// r_i < w(x_i) / D; a rejection removes x_i (D -= w(x_i), w(x_i) = 0), so a
// repeated sibling token is rejected for sure.  Every decision is scalar
// arithmetic on the gathered p(x_i): no pass over V until the one final draw
// (P_node without the rejected tokens, or the bonus row).  Only target rows
// are streamed.  Exactly lossless for any sibling tokens, deterministic top-F
// ones included.
#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_walk.hpp"

namespace sv {

constexpr int kTNT = 512;
constexpr uint64_t kTimelineWalkBase = 16384;  // timeline records of the walk launch (the stats launch's start at 0)
constexpr int kTU = 4;
constexpr int kGather = SV_MAX_N / kTNT;  // candidate children per stats thread

template <int DT>
__global__ __launch_bounds__(kTNT) void tree_stats_kernel(TreeParams a) {
  const int64_t bid = blockIdx.x;
  const int ch = (int)(bid % a.nch);
  int64_t rest = bid / a.nch;
  const int nw = a.pm ? 1 : 2;  // rows per node: target (and draft)
  const int which = a.pm ? 0 : (int)(rest & 1);
  if (!a.pm) rest >>= 1;
  const int b = (int)(rest % a.B);
  const int k = (int)(rest / a.B);  // this block streams the k-th node with children of sequence b
  const int64_t rowbase = (int64_t)b * a.N;
  SV_STAMP_START(0);
  // the sequence's tree in LDS (one round of loads); blocks are laid out
  // k-major, so the blocks that stream come first and spread evenly over the
  // compute units, and the blocks past a sequence's last node with children
  // (the end of the grid, mostly) exit at once
  __shared__ int32_t s_par[SV_MAX_N], s_tok[SV_MAX_N];
  __shared__ int s_has[SV_MAX_N];
  __shared__ int s_u;
  for (int i = threadIdx.x; i < a.N; i += kTNT) {
    s_par[i] = a.parent[rowbase + i];
    s_tok[i] = a.tok[rowbase + i];
    s_has[i] = a.all_rows ? 1 : 0;
  }
  __syncthreads();
  if (!a.all_rows)
    for (int i = 1 + (int)threadIdx.x; i < a.N; i += kTNT) {
      const int pi = s_par[i];
      if (pi >= 0 && pi < i) s_has[pi] = 1;  // every writer stores the same value
    }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // the k-th flagged node in index order: one ballot per 64 nodes
    const int lane = threadIdx.x;
    int cnt = 0, found = -1;
    for (int base = 0; base < a.N && found < 0; base += kWave) {
      const int i = base + lane;
      uint64_t m = __ballot(i < a.N && s_has[i < a.N ? i : 0]);
      const int c = __popcll(m);
      if (k < cnt + c) {
        for (int r = k - cnt; r > 0; --r) m &= m - 1;
        found = base + __builtin_ctzll(m);
      }
      cnt += c;
    }
    if (lane == 0) s_u = found;
  }
  __syncthreads();
  const int u = s_u;
  if (u < 0) {
    zero_slots(a.slots, a.nzero, bid, kTNT);  // for the walk launch
    return;
  }
  const void* row = which ? row_ptr(a.drf, rowbase + u, a.drf_sb) : row_ptr(a.tgt, rowbase + u, a.tgt_sb);
  // children of u among the candidates i = u + 1 + tid + j * kTNT
  int32_t pk[kGather], xk[kGather];
#pragma unroll
  for (int j = 0; j < kGather; ++j) {
    const int i = u + 1 + (int)threadIdx.x + j * kTNT;
    const bool kid = i < a.N && s_par[i < a.N ? i : 0] == u;
    pk[j] = kid ? u : -1;
    xk[j] = kid ? s_tok[i] : 0;
  }
  // the first part of the row gathers its logits at the children's tokens
  // (NaN for a token outside the vocabulary); the loads are issued before the
  // stream and their bits used after it, so no wait precedes the stream.
  // Candidates that are not children all read element 0, so the block
  // issues no more distinct gathers than it has children.
  uint32_t zg[kGather];
  if (ch == 0) {  // block-uniform; the loads are unconditional (clamped token) so none waits for another
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const int32_t x = xk[j];
      zg[j] = load_bits<DT>(row, ((pk[j] >= 0) & (x >= 0) & (x < a.V)) ? x : 0);
    }
  }
  const int64_t v0 = (int64_t)ch * a.vpc;
  const int64_t v1 = v0 + a.vpc < a.nvec ? v0 + a.vpc : a.nvec;
  const Partial part = range_stats<DT, kTNT, kTU>(row, a.V, v0, v1, a.c);
  SV_STAMP(0, 1);
  SV_STAMP_TAG(0, 4, b);
  if (threadIdx.x == 0) put_partial(static_cast<Partial*>(a.part) + ((rowbase + u) * nw + which) * a.nch + ch, part);
  float* zc = a.zc + (int64_t)which * a.B * a.N + rowbase;
  if (ch == 0) {
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const int32_t x = xk[j];
      if (pk[j] >= 0)
        zc[u + 1 + (int)threadIdx.x + j * kTNT] = (x >= 0 && x < a.V) ? bits_value<DT>(zg[j]) : __builtin_nanf("");
    }
  }
  zero_slots(a.slots, a.nzero, bid, kTNT);  // for the walk launch
  SV_STAMP_FLUSH(0);
}

// ---------------------------------------------------------------------------
// Walk.  The G blocks of a sequence each own one slice of every row the walk
// draws from (sv_walk.hpp) and replay the walk in lockstep.  Every decision
// is a deterministic function of global data and of the exchanged totals
// (the same bits in every block), so every block walks the identical path.
// Block 0 writes the per-child outputs; the owner of the slice holding the
// draw searches it.
// ---------------------------------------------------------------------------
constexpr int kWNT = 256;  // walk block

// Staging of a walk block in one round of loads, for trees whose nodes and
// rows fit one per thread and whose rows have at most kStageParts parts:
// thread t loads node t's entries and row t's parts before it uses any, and
// draws child t's uniform while they travel.  (Otherwise a loop per kind of
// entry.)
constexpr int kStageParts = 4;

// A row's statistic (c max, S) from its n <= kStageParts parts in registers,
// merged in part order as the loop over parts in memory does.
__device__ __forceinline__ void merge_held(const Partial (&pv)[kStageParts], int n, float c, float* cm, double* S) {
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < kStageParts; ++i)
    if (i < n) M = fmaxf(M, pv[i].m);
  *cm = 0.f;
  *S = 0.0;
  if (M == kNegInf) return;
  *cm = c * M;
  if (n == 1) {
    *S = pv[0].s;
    return;
  }
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < kStageParts; ++i)
    if (i < n && pv[i].m != kNegInf) sum += pv[i].s * exp2_d((double)(c * pv[i].m) - (double)*cm);
  *S = sum;
}

// Children of `node` in increasing index (from the staged parent array) into
// s_kids; returns their count (the same in every thread).  The first wave
// finds them with one ballot per 64 candidates, so the block waits at one
// barrier; every wave has finished with the previous node's list (each
// node's processing ends at a barrier).
__device__ int node_children(int node, int N, const int32_t* s_par, int* s_kids, int* s_cnt) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int cnt = 0;
    for (int base = node + 1; base < N; base += kWave) {
      const int i = base + lane;
      const bool flag = (i < N) & (s_par[i < N ? i : N - 1] == node);
      const uint64_t m = __ballot(flag);
      if (flag) s_kids[cnt + __popcll(m & ((1ull << lane) - 1))] = i;
      cnt += __popcll(m);
    }
    if (lane == 0) *s_cnt = cnt;
  }
  lds_sync();
  return *s_cnt;
}

// Bonus draw from the row at rowP (a node without children, or at the depth
// limit; the row was not streamed by the stats pass): the slices' statistics
// in one exchange, then a plain draw under the row's shift.  Returns the
// token in the block whose slice holds the draw, -1 in the others.
template <int DT, bool HELD>
__device__ int64_t bonus_draw(const TreeParams& a, Exchange& x, Slice<DT, kWNT, HELD>& sl, const void* rowP,
                              int64_t v0, int64_t v1, double us, bool writer, uint64_t* s_w0, uint64_t* s_w1,
                              SliceSums& ss) {
  sl.load(rowP, nullptr, v0, v1);
  float M;
  const double total = exchange_stats(x, sl.row_stats(a.c, a.V), a.c, s_w0, s_w1, &ss, &M);
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
  sp.ex = nullptr;
  sp.nex = 0;
  int pick;
  double loc;
  pick_slice(ss, x.G, us * total, &pick, &loc);
  if (pick != x.g) return -1;
  sl.prepare(sp, a.V);
  return sl.search(sp, a.V, loc);
}

template <int DT, bool HELD>
__global__ __launch_bounds__(kWNT) void tree_walk_kernel(TreeParams a) {
  const int b = blockIdx.x / a.G;
  const int g = blockIdx.x - b * a.G;
  Exchange x = make_exchange(a.slots, a.err, a.knobs, b, a.G, g);
  const int64_t spv = (a.nvec + a.G - 1) / a.G;
  const int64_t v0 = (int64_t)g * spv < a.nvec ? (int64_t)g * spv : a.nvec;
  const int64_t v1 = v0 + spv < a.nvec ? v0 + spv : a.nvec;
  const bool writer = (g == 0);
  const int64_t rowbase = (int64_t)b * a.N;
  const Partial* parts = static_cast<const Partial*>(a.part);
  __shared__ int32_t s_par[SV_MAX_N];
  __shared__ int s_kids[SV_MAX_N];
  __shared__ int32_t s_path[SV_MAX_N];
  __shared__ float s_zp[SV_MAX_N], s_zq[SV_MAX_N];  // each child's logits under its parent's rows
  __shared__ float s_cm[2][SV_MAX_N];                // row statistics of the nodes with children
  __shared__ double s_S[2][SV_MAX_N];
  __shared__ double s_pt[SV_MAX_N], s_qt[SV_MAX_N];  // each child's p and q under its parent's rows
  __shared__ float s_r[SV_MAX_N];
  __shared__ int s_first[SV_MAX_N];  // each node's first child (N: none)
  __shared__ int s_tried[SV_MAX_N];  // children tried so far, in order (their outputs are stored at the end)
  __shared__ uint64_t s_w0[kMaxG], s_w1[kMaxG];
  SliceSums ss;  // the slices' values of the last exchange
  __shared__ int s_cnt;
  const double us = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);
  SV_STAMP_START(kTimelineWalkBase);
  SV_STAMP_TAG(kTimelineWalkBase, 5, b);
  Lap lp;        // rejection passes: summing the residual, exchanging the sums
  int npass = 0;

  // the tree, the gathered logits and every node's row statistic, in one
  // round of loads (parts and logits of nodes without children were not
  // written and are never used)
  const float* zc = a.zc + rowbase;
  const bool one_round = a.N <= kWNT && 2 * (a.N - 1) <= kWNT && a.nch <= kStageParts;  // block-uniform
  if (one_round) {
    const int t = threadIdx.x;
    int32_t par = 0;
    float zp = 0.f, zq = 0.f;
    Partial pv[kStageParts];
    if (t < a.N) {
      par = a.parent[rowbase + t];
      zp = zc[t];
      zq = zc[(int64_t)a.B * a.N + t];
    }
    if (t < 2 * (a.N - 1)) {
      const Partial* pr = parts + ((rowbase + (t >> 1)) * 2 + (t & 1)) * a.nch;  // written by the previous launch
#pragma unroll
      for (int i = 0; i < kStageParts; ++i) pv[i] = pr[i < a.nch ? i : a.nch - 1];
    }
    float r = 0.f;
    if (t >= 1 && t < a.N) r = (float)uniform24(a.seed, (uint32_t)t, (uint32_t)b, 0, a.round, 0);  // exact: 24-bit grid
    if (t < a.N) {
      s_par[t] = par;
      s_zp[t] = zp;
      s_zq[t] = zq;
      s_first[t] = a.N;
      s_r[t] = r;
    }
    if (t < 2 * (a.N - 1)) merge_held(pv, a.nch, a.c, &s_cm[t & 1][t >> 1], &s_S[t & 1][t >> 1]);
  }
  if (!one_round)
    for (int i = threadIdx.x; i < a.N; i += kWNT) {
      s_par[i] = a.parent[rowbase + i];
      s_zp[i] = zc[i];
      s_zq[i] = zc[(int64_t)a.B * a.N + i];
      s_first[i] = a.N;
    }
  for (int r = one_round ? kWNT : threadIdx.x; r < 2 * (a.N - 1); r += kWNT) {
    const int u = r >> 1, which = r & 1;
    const Partial* pr = parts + ((rowbase + u) * 2 + which) * a.nch;  // written by the previous launch
    float M = kNegInf;
    for (int i = 0; i < a.nch; ++i) M = fmaxf(M, pr[i].m);
    float cm = 0.f;
    double S = 0.0;
    if (M != kNegInf) {
      cm = a.c * M;
      if (a.nch == 1) {
        S = pr[0].s;
      } else {
        for (int i = 0; i < a.nch; ++i) {
          const Partial pi = pr[i];
          if (pi.m != kNegInf) S += pi.s * exp2_d((double)(a.c * pi.m) - (double)cm);
        }
      }
    }
    s_cm[which][u] = cm;
    s_S[which][u] = S;
  }
  lds_sync();
  if (writer)
    for (int i = 1 + threadIdx.x; i < a.N; i += kWNT)
      if (s_par[i] < 0 || s_par[i] >= i) set_error(a.err, SV_DERR_TREE);
  // every child's p and q under its parent's rows and its acceptance
  // uniform, once for the whole tree (indexed by node)
  for (int i = 1 + threadIdx.x; i < a.N; i += kWNT) {
    const int u = (s_par[i] >= 0 && s_par[i] < i) ? s_par[i] : 0;
    RowStat P, Q;
    P.cm = s_cm[0][u];
    P.S = s_S[0][u];
    Q.cm = s_cm[1][u];
    Q.S = s_S[1][u];
    P.pad = Q.pad = 0.f;
    const float zp = s_zp[i], zq = s_zq[i];
    double pt = 0.0, qt = 0.0;
    if (!__builtin_isnan(zp)) {
      pt = prob_of(zp, a.c, P);
      qt = prob_of(zq, a.c, Q);
    }
    s_pt[i] = pt;
    s_qt[i] = qt;
    if (!one_round) s_r[i] = (float)uniform24(a.seed, (uint32_t)i, (uint32_t)b, 0, a.round, 0);  // exact: 24-bit grid
    if (s_par[i] >= 0 && s_par[i] < i) atomicMin(&s_first[s_par[i]], i);
  }
  lds_sync();
  SV_STAMP(kTimelineWalkBase, 1);

  int node = 0, depth = 0;
  int ntried = 0;  // entries of s_tried (the same in every thread)
  int64_t t = -1;
  int nvisit = 0;  // (timeline builds) nodes entered
  Slice<DT, kWNT, HELD> sl;
  for (;;) {
    // a node whose first child is accepted at its first try needs no pass
    // over the logits: follow such nodes on the staged p, q and uniforms (the
    // test is the general loop's first iteration, with c = 0 and D = 1; an
    // accepted child has p > 0, so only the draft row can lack mass)
    for (;;) {
      const int fc = s_first[node];
      if (fc >= a.N || depth >= a.max_depth || !((double)s_r[fc] < accept_ratio(s_pt[fc], s_qt[fc]))) break;
      if (threadIdx.x == 0) {
        s_tried[ntried] = fc;
        s_path[depth] = fc;
        if (writer && !(s_S[1][node] > 0.0)) set_error(a.err, SV_DERR_ROW);
      }
      ++ntried;
      ++depth;
      node = fc;
    }
    const int nk = node_children(node, a.N, s_par, s_kids, &s_cnt);
    SV_STAMP(kTimelineWalkBase, 7 + (nvisit < 4 ? nvisit : 4));  // (timeline builds) a node's children are known
    ++nvisit;
    const void* rowP = row_ptr(a.tgt, rowbase + node, a.tgt_sb);
    if (nk == 0 || depth >= a.max_depth) {
      if (nk > 0 && writer) set_error(a.err, SV_DERR_TREE);
      t = bonus_draw<DT, HELD>(a, x, sl, rowP, v0, v1, us, writer, s_w0, s_w1, ss);
      break;
    }
    const void* rowQ = row_ptr(a.drf, rowbase + node, a.drf_sb);
    // the held slice of the node's row pair is loaded on entering the node,
    // so that the loads travel while the first children are tested
    sl.load(rowP, rowQ, v0, v1);
    bool loaded = true;
    RowStat P, Q;
    P.cm = s_cm[0][node];
    P.S = s_S[0][node];
    Q.cm = s_cm[1][node];
    Q.S = s_S[1][node];
    P.pad = Q.pad = 0.f;
    if (writer && threadIdx.x == 0 && (!(P.S > 0.0) || !(Q.S > 0.0))) set_error(a.err, SV_DERR_ROW);
    DrawSpec sp;
    sp.rowP = rowP;
    sp.rowQ = rowQ;
    sp.c = a.c;
    sp.cmP = P.cm;
    sp.invSP = P.S > 0.0 ? (float)(1.0 / P.S) : 0.f;
    sp.cmQ = Q.cm;
    sp.invSQ = Q.S > 0.0 ? (float)(1.0 / Q.S) : 0.f;
    sp.ex = nullptr;
    sp.nex = 0;
    double c = 0.0, D = 1.0;
    bool sums_current = false;  // the last exchange holds the slices' sums of the current residual
    int accepted = -1;
    for (int kk = 0; kk < nk; ++kk) {
      const int cn = s_kids[kk];
      const double pt = s_pt[cn], qt = s_qt[cn];
      if (threadIdx.x == 0) s_tried[ntried] = cn;
      ++ntried;
      const double pcur = fmax(0.0, pt - c * qt) / D;
      if ((double)s_r[cn] < accept_ratio(pcur, qt)) {
        accepted = cn;
        break;
      }
      const double cnext = c + D;
      sp.coef = (float)cnext;
      if (!loaded) {
        sl.load(rowP, rowQ, v0, v1);
        loaded = true;
      }
      lp.start();
      const double mine = sl.total(sp, a.V);
      lp.lap(0);
      const double Dn = exchange_sum(x, mine, s_w0, &ss);
      lp.lap(1);
      ++npass;
      if (Dn > 0.0) {
        c = cnext;
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
      lds_sync();
      continue;
    }
    // every child rejected: draw from (p - c q)^+; the rejection passes
    // exchanged only the slices' totals, so the searching block prepares its
    // slice's prefixes first
    sp.coef = (float)c;
    SV_STAMP(kTimelineWalkBase, 12);  // (timeline builds) every child rejected: the final draw starts
    if (!loaded) sl.load(rowP, rowQ, v0, v1);  // (not reached: the last child was rejected)
    if (!sums_current) D = exchange_sum(x, sl.total(sp, a.V), s_w0, &ss);
    int pick;
    double loc;
    pick_slice(ss, x.G, us * D, &pick, &loc);
    if (pick == g) {
      sl.prepare(sp, a.V);
      t = sl.search(sp, a.V, loc);
    }
    SV_STAMP(kTimelineWalkBase, 13);  // (timeline builds) the final draw is searched (its own block)
    break;
  }
  SV_STAMP_VAL(kTimelineWalkBase, 2, lp.sum[0]);
  SV_STAMP_VAL(kTimelineWalkBase, 3, lp.sum[1]);
  SV_STAMP_VAL(kTimelineWalkBase, 4, npass);
  SV_STAMP(kTimelineWalkBase, 5);
  SV_STAMP_VAL(kTimelineWalkBase, 6, depth);
  lds_sync();
  if (writer) {
    for (int d = threadIdx.x; d < a.max_depth; d += kWNT)
      a.out_path[(int64_t)b * a.max_depth + d] = d < depth ? s_path[d] : -1;
    if (threadIdx.x == 0) a.out_len[b] = depth;
    for (int k = threadIdx.x; k < ntried; k += kWNT) {
      const int cn = s_tried[k];
      if (__builtin_isnan(s_zp[cn])) set_error(a.err, SV_DERR_TOKEN);
      if (a.out_p) a.out_p[rowbase + cn] = (float)s_pt[cn];
      if (a.out_q) a.out_q[rowbase + cn] = (float)s_qt[cn];
    }
  }
  if (t >= 0 && threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
  SV_STAMP_FLUSH(kTimelineWalkBase);
}

// Point-mass walk.  The G blocks of a sequence replay the same scalar
// decisions; only the final draw touches the logits (one row, one exchange).
template <int DT, bool HELD>
__global__ __launch_bounds__(kWNT) void tree_pm_walk_kernel(TreeParams a) {
  const int b = blockIdx.x / a.G;
  const int g = blockIdx.x - b * a.G;
  Exchange x = make_exchange(a.slots, a.err, a.knobs, b, a.G, g);
  const int64_t spv = (a.nvec + a.G - 1) / a.G;
  const int64_t v0 = (int64_t)g * spv < a.nvec ? (int64_t)g * spv : a.nvec;
  const int64_t v1 = v0 + spv < a.nvec ? v0 + spv : a.nvec;
  constexpr int E = Fmt<DT>::kPerVec;
  const int64_t e0 = v0 * E, e1 = v1 * E;  // this block's token range
  const bool writer = (g == 0);
  const int64_t rowbase = (int64_t)b * a.N;
  const Partial* parts = static_cast<const Partial*>(a.part);
  __shared__ int32_t s_par[SV_MAX_N];
  __shared__ int32_t s_tok[SV_MAX_N];
  __shared__ int s_kids[SV_MAX_N];
  __shared__ int32_t s_path[SV_MAX_N];
  __shared__ float s_zp[SV_MAX_N];   // each child's logit under its parent's target row
  __shared__ float s_cm[SV_MAX_N];   // target row statistics of the nodes with children
  __shared__ double s_S[SV_MAX_N];
  __shared__ double s_pt[SV_MAX_N];  // each child's p under its parent's target row
  __shared__ double s_w[SV_MAX_N];   // the current node's children, in order: w(x_i) when child i is
                                     // tried (0 for a repeated token)
  __shared__ float s_r[SV_MAX_N];    // each child's acceptance uniform
  __shared__ int s_first[SV_MAX_N];  // each node's first child (N: none)
  __shared__ int s_tried[SV_MAX_N];  // children tried so far, in order (their outputs are stored at the end)
  __shared__ int32_t s_ex[SV_MAX_N];  // rejected tokens inside this block's slice
  __shared__ uint64_t s_w0[kMaxG], s_w1[kMaxG];
  SliceSums ss;  // the slices' values of the last exchange
  __shared__ int s_cnt;
  const double us = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);

  const float* zc = a.zc + rowbase;
  const bool one_round = a.N <= kWNT && a.nch <= kStageParts;  // block-uniform
  if (one_round) {
    const int t = threadIdx.x;
    int32_t par = 0, tok = 0;
    float zp = 0.f;
    Partial pv[kStageParts];
    if (t < a.N) {
      par = a.parent[rowbase + t];
      tok = a.tok[rowbase + t];
      zp = zc[t];
    }
    if (t < a.N - 1) {
      const Partial* pr = parts + (rowbase + t) * a.nch;  // written by the previous launch
#pragma unroll
      for (int i = 0; i < kStageParts; ++i) pv[i] = pr[i < a.nch ? i : a.nch - 1];
    }
    float r = 0.f;
    if (t >= 1 && t < a.N) r = (float)uniform24(a.seed, (uint32_t)t, (uint32_t)b, 0, a.round, 0);  // exact: 24-bit grid
    if (t < a.N) {
      s_par[t] = par;
      s_tok[t] = tok;
      s_zp[t] = zp;
      s_first[t] = a.N;
      s_r[t] = r;
    }
    if (t < a.N - 1) merge_held(pv, a.nch, a.c, &s_cm[t], &s_S[t]);
  }
  if (!one_round)
    for (int i = threadIdx.x; i < a.N; i += kWNT) {
      s_par[i] = a.parent[rowbase + i];
      s_tok[i] = a.tok[rowbase + i];
      s_zp[i] = zc[i];
      s_first[i] = a.N;
    }
  for (int u = one_round ? kWNT : threadIdx.x; u < a.N - 1; u += kWNT) {
    const Partial* pr = parts + (rowbase + u) * a.nch;  // written by the previous launch
    float M = kNegInf;
    for (int i = 0; i < a.nch; ++i) M = fmaxf(M, pr[i].m);
    float cm = 0.f;
    double S = 0.0;
    if (M != kNegInf) {
      cm = a.c * M;
      if (a.nch == 1) {
        S = pr[0].s;
      } else {
        for (int i = 0; i < a.nch; ++i) {
          const Partial pi = pr[i];
          if (pi.m != kNegInf) S += pi.s * exp2_d((double)(a.c * pi.m) - (double)cm);
        }
      }
    }
    s_cm[u] = cm;
    s_S[u] = S;
  }
  lds_sync();
  if (writer)
    for (int i = 1 + threadIdx.x; i < a.N; i += kWNT)
      if (s_par[i] < 0 || s_par[i] >= i) set_error(a.err, SV_DERR_TREE);
  // every child's p under its parent's target row and its uniform, once for
  // the whole tree (indexed by node)
  for (int i = 1 + threadIdx.x; i < a.N; i += kWNT) {
    const bool valid = s_par[i] >= 0 && s_par[i] < i;
    const int u = valid ? s_par[i] : 0;
    RowStat P;
    P.cm = s_cm[u];
    P.S = s_S[u];
    P.pad = 0.f;
    const float zp = s_zp[i];
    s_pt[i] = __builtin_isnan(zp) ? 0.0 : prob_of(zp, a.c, P);
    if (!one_round) s_r[i] = (float)uniform24(a.seed, (uint32_t)i, (uint32_t)b, 0, a.round, 0);  // exact: 24-bit grid
    if (valid) atomicMin(&s_first[u], i);
  }
  lds_sync();

  int node = 0, depth = 0;
  int ntried = 0;  // entries of s_tried (the same in every thread)
  int64_t t = -1;
  Slice<DT, kWNT, HELD> sl;
  for (;;) {
    // a node whose first child is accepted needs no list of its children:
    // follow such nodes on the staged p and uniforms (the test is the
    // general loop's first iteration, with D = 1; an accepted child has
    // p > 0, so its parent's row has mass)
    for (;;) {
      const int fc = s_first[node];
      if (fc >= a.N || depth >= a.max_depth || !((double)s_r[fc] < accept_ratio(s_pt[fc] / 1.0, 1.0))) break;
      if (threadIdx.x == 0) {
        s_tried[ntried] = fc;
        s_path[depth] = fc;
      }
      ++ntried;
      ++depth;
      node = fc;
    }
    const int nk = node_children(node, a.N, s_par, s_kids, &s_cnt);
    const void* rowP = row_ptr(a.tgt, rowbase + node, a.tgt_sb);
    if (nk == 0 || depth >= a.max_depth) {
      if (nk > 0 && writer) set_error(a.err, SV_DERR_TREE);
      t = bonus_draw<DT, HELD>(a, x, sl, rowP, v0, v1, us, writer, s_w0, s_w1, ss);
      break;
    }
    RowStat P;
    P.cm = s_cm[node];
    P.S = s_S[node];
    P.pad = 0.f;
    if (writer && threadIdx.x == 0 && !(P.S > 0.0)) set_error(a.err, SV_DERR_ROW);
    // every child's p, uniform and residual weight in parallel: all earlier
    // siblings are rejected when child i is tried, so w(x_i) is p(x_i) unless
    // an earlier sibling carries the same token
    for (int k = threadIdx.x; k < nk; k += kWNT) {
      const int cn = s_kids[k];
      const int32_t tk = s_tok[cn];
      bool repeated = false;
      for (int j = 0; j < k && !repeated; ++j) repeated = s_tok[s_kids[j]] == tk;
      s_w[k] = repeated ? 0.0 : s_pt[cn];
    }
    lds_sync();
    double D = 1.0;
    int accepted = -1, tried = nk;
    for (int kk = 0; kk < nk; ++kk) {
      const double w = s_w[kk];
      const double ar = D > 0.0 ? accept_ratio(w / D, 1.0) : 0.0;
      if ((double)s_r[s_kids[kk]] < ar) {
        accepted = s_kids[kk];
        tried = kk + 1;
        break;
      }
      D -= w;
    }
    for (int k = threadIdx.x; k < tried; k += kWNT) s_tried[ntried + k] = s_kids[k];
    ntried += tried;
    if (accepted >= 0) {
      if (threadIdx.x == 0) s_path[depth] = accepted;
      ++depth;
      node = accepted;
      lds_sync();
      continue;
    }
    // every child rejected: P_node without the children's tokens; this
    // block's list holds those inside its slice
    if (threadIdx.x == 0) s_cnt = 0;
    lds_sync();
    for (int base = 0; base < nk; base += kWNT) {
      const int k = base + (int)threadIdx.x;
      const int32_t tk = k < nk ? s_tok[s_kids[k]] : -1;
      const int flag = tk >= 0 && tk < a.V && tk >= e0 && tk < e1;
      double excl;
      const double tot = block_exclusive_scan<kWNT>((double)flag, &excl);
      if (flag) s_ex[s_cnt + (int)excl] = tk;
      lds_sync();
      if (threadIdx.x == 0) s_cnt += (int)tot;
      lds_sync();
    }
    DrawSpec sp;
    sp.rowP = rowP;
    sp.rowQ = nullptr;
    sp.c = a.c;
    sp.cmP = P.cm;
    sp.invSP = 1.f;
    sp.cmQ = 0.f;
    sp.invSQ = 1.f;
    sp.coef = 0.f;
    sp.ex = s_ex;
    sp.nex = s_cnt;
    sl.load(rowP, nullptr, v0, v1);
    double total = exchange_sum(x, sl.prepare(sp, a.V), s_w0, &ss);
    if (!(total > 0.0)) {
      // the row's mass sits on the rejected tokens (by rounding): draw from P_node
      sp.nex = 0;
      total = exchange_sum(x, sl.prepare(sp, a.V), s_w0, &ss);
    }
    int pick;
    double loc;
    pick_slice(ss, x.G, us * total, &pick, &loc);
    if (pick == g) t = sl.search(sp, a.V, loc);
    break;
  }
  lds_sync();
  if (writer) {
    for (int d = threadIdx.x; d < a.max_depth; d += kWNT)
      a.out_path[(int64_t)b * a.max_depth + d] = d < depth ? s_path[d] : -1;
    if (threadIdx.x == 0) a.out_len[b] = depth;
    for (int k = threadIdx.x; k < ntried; k += kWNT) {
      const int cn = s_tried[k];
      if (__builtin_isnan(s_zp[cn])) set_error(a.err, SV_DERR_TOKEN);
      if (a.out_p) a.out_p[rowbase + cn] = (float)s_pt[cn];
    }
  }
  if (t >= 0 && threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
}

// The statistics launch alone (also used by the PRESTO scoring call).
hipError_t launch_tree_stats(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16)
    tree_stats_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
  else
    tree_stats_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_tree_t(const TreeParams& p, const Plan& plan, hipStream_t s) {
  tree_stats_kernel<DT><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // B * G <= the blocks the device holds at once (chosen by the caller): a
  // sequence's blocks are resident together on an otherwise idle device,
  // and their waits are bounded either way
  const dim3 grid((unsigned)p.B * p.G);
  if (p.pm) {
    if (p.held)
      tree_pm_walk_kernel<DT, true><<<grid, dim3(kWNT), 0, s>>>(p);
    else
      tree_pm_walk_kernel<DT, false><<<grid, dim3(kWNT), 0, s>>>(p);
  } else {
    if (p.held)
      tree_walk_kernel<DT, true><<<grid, dim3(kWNT), 0, s>>>(p);
    else
      tree_walk_kernel<DT, false><<<grid, dim3(kWNT), 0, s>>>(p);
  }
  return hipGetLastError();
}

SV_TIMELINE_SETTER(timeline_set_tree)

hipError_t launch_tree(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  return dt == SV_BF16 ? launch_tree_t<SV_BF16>(p, plan, s) : launch_tree_t<SV_F32>(p, plan, s);
}

template <int DT>
const void* walk_fn(bool held, bool pm) {
  if (pm)
    return held ? reinterpret_cast<const void*>(&tree_pm_walk_kernel<DT, true>)
                : reinterpret_cast<const void*>(&tree_pm_walk_kernel<DT, false>);
  return held ? reinterpret_cast<const void*>(&tree_walk_kernel<DT, true>)
              : reinterpret_cast<const void*>(&tree_walk_kernel<DT, false>);
}

// Blocks of the walk kernel the device holds at once.
int tree_walk_capacity(sv_dtype dt, bool held, bool pm) {
  static int cache[2][2][2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& c = cache[dt == SV_BF16][held][pm][dev];
  if (c == 0) {
    const void* fn = dt == SV_BF16 ? walk_fn<SV_BF16>(held, pm) : walk_fn<SV_F32>(held, pm);
    c = device_capacity(fn, kWNT, dev);
  }
  return c;
}

}  // namespace sv
