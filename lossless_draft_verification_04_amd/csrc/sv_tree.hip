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
//  2. walk: one 512-thread block per sequence merges the parts of the node
//     it stands on, decides children in order, and makes one pass over the
//     node's row pair per rejection; the pass keeps per-tile weight sums in
//     LDS so the final draw only re-reads one tile.
#include "sv_device.hpp"
#include "sv_internal.h"

namespace sv {

constexpr int kTNT = 256;
constexpr int kTU = 4;
constexpr int kWNT = 512;        // walk block
constexpr int kMaxTiles = 8192;  // LDS tile sums of one row pass (tiles of kWNT vectors)
constexpr int kGroup = 8;        // tiles per pass step (vectors in flight per thread)

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
  if (threadIdx.x == 0) static_cast<Partial*>(a.part)[(((int64_t)b * a.N + u) * 2 + which) * a.nch + ch] = part;
}

// Per-tile sums of the draw weights over a whole row.  A tile is kWNT
// vectors (one per thread); kGroup tiles' loads are issued before any of
// them is reduced, so each thread keeps kGroup (x2 for a residual) 16-byte
// loads in flight.  Returns the total.
template <int DT>
__device__ double tile_pass(const DrawSpec& sp, int V, int64_t nvec, int ntiles, double* s_tiles) {
  constexpr int E = Fmt<DT>::kPerVec;
  __shared__ double red[kGroup][kWNT / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  double total = 0.0;
  for (int t0 = 0; t0 < ntiles; t0 += kGroup) {
    u32x4 dp[kGroup], dq[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int64_t v = (int64_t)(t0 + g) * kWNT + threadIdx.x;
      if (v < nvec) {
        dp[g] = load_vec(sp.rowP, v);
        if (sp.rowQ) dq[g] = load_vec(sp.rowQ, v);
      }
    }
    double own[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      own[g] = 0.0;
      const int64_t v = (int64_t)(t0 + g) * kWNT + threadIdx.x;
      if (v < nvec) {
        float w[E];
        draw_weights_from<DT>(sp, V, v, dp[g], dq[g], w);
#pragma unroll
        for (int e = 0; e < E; ++e) own[g] += (double)w[e];
      }
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) own[g] = wave_sum(own[g]);
    __syncthreads();
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < kGroup; ++g) red[g][wave] = own[g];
    }
    __syncthreads();
    if (threadIdx.x < kGroup && t0 + (int)threadIdx.x < ntiles) {
      double s = 0.0;
      for (int w = 0; w < kWNT / kWave; ++w) s += red[threadIdx.x][w];
      s_tiles[t0 + threadIdx.x] = s;
    }
    __syncthreads();
    for (int g = 0; g < kGroup && t0 + g < ntiles; ++g) total += s_tiles[t0 + g];
  }
  return total;
}

// Draw from the weights whose tile sums are in s_tiles (total `total`).
template <int DT>
__device__ int64_t tile_draw(const DrawSpec& sp, int V, int64_t nvec, int ntiles, const double* s_tiles, double total,
                             double u) {
  __shared__ int s_tile;
  __shared__ double s_loc;
  if (threadIdx.x == 0) {
    const double target = u * total;
    double cum = 0.0, cum_last = 0.0;
    int pick = -1, last = -1;
    for (int t = 0; t < ntiles; ++t) {
      const double w = s_tiles[t];
      if (w > 0.0) {
        last = t;
        cum_last = cum;
      }
      if (pick < 0 && cum + w > target) {
        pick = t;
        s_loc = target - cum;
      }
      cum += w;
    }
    if (pick < 0) {
      pick = last < 0 ? 0 : last;
      s_loc = cum - cum_last;
    }
    s_tile = pick;
  }
  __syncthreads();
  const int64_t v0 = (int64_t)s_tile * kWNT;
  const int64_t v1 = v0 + kWNT < nvec ? v0 + kWNT : nvec;
  return block_search<DT, kWNT>(sp, V, v0, v1, s_loc);
}

template <int DT>
__global__ __launch_bounds__(kWNT) void tree_walk_kernel(TreeParams a) {
  const int b = blockIdx.x;
  const int64_t rowbase = (int64_t)b * a.N;
  const Partial* parts = static_cast<const Partial*>(a.part);
  __shared__ int s_kids[SV_MAX_N];
  __shared__ int s_nkids;
  __shared__ RowStat s_P, s_Q;
  __shared__ int s_acc;
  __shared__ double s_tiles[kMaxTiles];
  __shared__ int32_t s_path[SV_MAX_N];

  const int ntiles = (int)((a.nvec + kWNT - 1) / kWNT);  // <= kMaxTiles (checked on the host)
  const double us = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);

  int node = 0, depth = 0;
  int64_t t = -1;
  for (;;) {
    // children of `node`, in increasing index
    const int i = node + 1 + (int)threadIdx.x;
    int flag = 0;
    if (i < a.N) {
      const int32_t pi = a.parent[rowbase + i];
      flag = (pi == node);
      if (pi < 0 || pi >= i) set_error(a.err, SV_DERR_TREE);
    }
    double excl;
    const double nk_d = block_exclusive_scan<kWNT>((double)flag, &excl);
    if (flag) s_kids[(int)excl] = i;
    const int nk = (int)nk_d;
    if (threadIdx.x == 0) s_nkids = nk;
    __syncthreads();

    const void* rowP = row_ptr(a.tgt, rowbase + node, a.tgt_sb);
    if (nk == 0 || depth >= a.max_depth) {
      if (nk > 0) set_error(a.err, SV_DERR_TREE);
      // bonus draw from P_node: its statistic first (leaf rows were not in
      // the stats pass), then tile sums with that shift, then the draw
      const Partial st = range_stats<DT, kWNT, 4>(rowP, a.V, 0, a.nvec, a.c);
      DrawSpec sp;
      sp.rowP = rowP;
      sp.rowQ = nullptr;
      sp.c = a.c;
      sp.cmP = a.c * st.m;
      sp.invSP = 1.f;
      sp.cmQ = 0.f;
      sp.invSQ = 1.f;
      sp.coef = 0.f;
      if (st.m == kNegInf) set_error(a.err, SV_DERR_ROW);
      const double total = tile_pass<DT>(sp, a.V, a.nvec, ntiles, s_tiles);
      t = tile_draw<DT>(sp, a.V, a.nvec, ntiles, s_tiles, total, us);
      break;
    }
    const void* rowQ = row_ptr(a.drf, rowbase + node, a.drf_sb);
    if (threadIdx.x == 0) {
      s_P = merge_parts(parts + ((rowbase + node) * 2 + 0) * a.nch, a.nch, a.c);
      s_Q = merge_parts(parts + ((rowbase + node) * 2 + 1) * a.nch, a.nch, a.c);
      if (!(s_P.S > 0.0) || !(s_Q.S > 0.0)) set_error(a.err, SV_DERR_ROW);
    }
    __syncthreads();
    const RowStat P = s_P, Q = s_Q;
    DrawSpec sp;
    sp.rowP = rowP;
    sp.rowQ = rowQ;
    sp.c = a.c;
    sp.cmP = P.cm;
    sp.invSP = P.S > 0.0 ? (float)(1.0 / P.S) : 0.f;
    sp.cmQ = Q.cm;
    sp.invSQ = Q.S > 0.0 ? (float)(1.0 / Q.S) : 0.f;
    double c = 0.0, D = 1.0, total = 0.0;
    bool tiles_ok = false;  // s_tiles hold the weights of the current residual
    int accepted = -1;
    for (int kk = 0; kk < nk; ++kk) {
      const int ch = s_kids[kk];
      if (threadIdx.x == 0) {
        const int32_t x = a.tok[rowbase + ch];
        double pt = 0.0, qt = 0.0;
        if (x >= 0 && x < a.V) {
          pt = prob_of(load_elem<DT>(rowP, x), a.c, P);
          qt = prob_of(load_elem<DT>(rowQ, x), a.c, Q);
        } else {
          set_error(a.err, SV_DERR_TOKEN);
        }
        if (a.out_p) a.out_p[rowbase + ch] = (float)pt;
        if (a.out_q) a.out_q[rowbase + ch] = (float)qt;
        const double pcur = fmax(0.0, pt - c * qt) / D;
        const double r = uniform24(a.seed, (uint32_t)ch, (uint32_t)b, 0, a.round, 0);
        s_acc = r < accept_ratio(pcur, qt);
      }
      __syncthreads();
      if (s_acc) {
        accepted = ch;
        break;
      }
      const double cn = c + D;
      sp.coef = (float)cn;
      const double G = tile_pass<DT>(sp, a.V, a.nvec, ntiles, s_tiles);
      if (G > 0.0) {
        c = cn;
        D = G;
        total = G;
        tiles_ok = true;
      } else {
        tiles_ok = false;  // residual mass rounded to 0: keep the previous residual
      }
      __syncthreads();
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
    if (!tiles_ok) total = tile_pass<DT>(sp, a.V, a.nvec, ntiles, s_tiles);
    t = tile_draw<DT>(sp, a.V, a.nvec, ntiles, s_tiles, total, us);
    break;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < a.max_depth; d += kWNT)
    a.out_path[(int64_t)b * a.max_depth + d] = d < depth ? s_path[d] : -1;
  if (threadIdx.x == 0) {
    a.out_len[b] = depth;
    a.out_tok[b] = (int32_t)t;
  }
}

hipError_t launch_tree(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16) {
    tree_stats_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
    tree_walk_kernel<SV_BF16><<<dim3((unsigned)plan.grid2), dim3(kWNT), 0, s>>>(p);
  } else {
    tree_stats_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kTNT), 0, s>>>(p);
    tree_walk_kernel<SV_F32><<<dim3((unsigned)plan.grid2), dim3(kWNT), 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace sv
