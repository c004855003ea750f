// sv_branch.hip -- SpecBranch branch resampling on gfx950.
//
// SpecBranch notes, key designs 2-3: the hybrid predictor's class s (an
// input here: the predictor is a trained network) places the branch point --
// s = 0: the round's first token; s = 1: the first drafted token whose draft
// probability falls below eps (the next round's first token when none does);
// s = 2: the next round's first token -- and k = max(1, floor(k_max *
// (1 - q(x_b)))) branches are forked with the top-k tokens of the draft
// distribution at the branch point.  At position gamma + 1 no token is
// drafted yet; x_b is read as the draft's most likely token there, so
// q(x_b) = max q_{gamma+1} = 1 / S of that row (its largest term is 1).
//
// Two launches per call:
//  1. statistics: a block per (draft row, part) of the gamma + 1 rows of every
//     sequence streams its part once into a mergeable (max, sum) and the
//     first part of row j < gamma also gathers the logit of x_{j+1} inside
//     the stream.
//  2. fork: a block per (sequence, part of the branch row).  Every block
//     merges the sequence's statistics and makes the same decisions (block 0
//     writes them), then scans its part of the branch row for the k largest
//     logits (sv_topk.hpp); the sequence's last block to finish merges the
//     parts' lists and writes the branches.
#include <cmath>

#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_topk.hpp"

namespace sv {

constexpr int kBNT = 256;
constexpr int kBU = 4;
constexpr int kBStage = 1024;  // statistics parts of one sequence staged in LDS

template <int DT>
__global__ __launch_bounds__(kBNT) void branch_stats_kernel(BranchParams a) {
  const int rows = a.gamma + 1;
  const int64_t per_seq = (int64_t)rows * a.nch1;
  const int64_t bid = blockIdx.x;
  const int b = (int)(bid / per_seq);
  const int64_t rem = bid - (int64_t)b * per_seq;
  const int j = (int)(rem / a.nch1);
  const int ch = (int)(rem - (int64_t)j * a.nch1);
  const void* row = row_ptr(a.drf, (int64_t)b * rows + j, a.sb);
  const bool gather = ch == 0 && j < a.gamma && threadIdx.x == 0;
  int32_t x = 0;
  if (gather) x = a.tok[(int64_t)b * a.gamma + j];
  const int64_t v0 = (int64_t)ch * a.vpc1;
  const int64_t v1 = v0 + a.vpc1 < a.nvec ? v0 + a.vpc1 : a.nvec;
  uint32_t zbits = 0;
  const Partial part = range_stats<DT, kBNT, kBU>(row, a.V, v0, v1, a.c, gather, x, &zbits);
  if (threadIdx.x == 0) put_partial(static_cast<Partial*>(a.part) + (int64_t)b * per_seq + (int64_t)j * a.nch1 + ch, part);
  if (gather) a.zq[(int64_t)b * a.gamma + j] = (x >= 0 && x < a.V) ? bits_value<DT>(zbits) : __builtin_nanf("");
}

// Row statistic j of the staged parts (or from global memory when the
// sequence has more parts than fit).
__device__ RowStat staged_stat(const Partial* st, bool staged, const Partial* gparts, int first, int n, float c) {
  if (!staged) return merge_parts(gparts + first, n, c);
  float M = kNegInf;
  for (int i = 0; i < n; ++i) M = fmaxf(M, st[first + i].m);
  RowStat r;
  r.pad = 0.f;
  r.cm = M == kNegInf ? 0.f : c * M;
  double S = 0.0;
  if (M != kNegInf)
    for (int i = 0; i < n; ++i)
      if (st[first + i].m != kNegInf) S += st[first + i].s * exp2_d((double)(c * st[first + i].m) - (double)r.cm);
  r.S = S;
  return r;
}

template <int DT>
__global__ __launch_bounds__(kBNT) void branch_fork_kernel(BranchParams a) {
  constexpr int E = Fmt<DT>::kPerVec;
  const int b = blockIdx.x / a.nch2;
  const int ch = blockIdx.x - b * a.nch2;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rows = a.gamma + 1;
  const int nparts = rows * a.nch1;
  const bool staged = nparts <= kBStage;
  const Partial* pb = static_cast<const Partial*>(a.part) + (int64_t)b * nparts;
  __shared__ Partial st[kBStage];
  __shared__ double s_q[SV_MAX_GAMMA];  // q_j(x_j)
  __shared__ int s_pos, s_k;
  __shared__ double s_qb;
  if (staged)
    for (int i = threadIdx.x; i < nparts; i += kBNT) st[i] = pb[i];  // written by the previous launch
  lds_sync();
  for (int j = threadIdx.x; j < a.gamma; j += kBNT) {
    const RowStat rs = staged_stat(st, staged, pb, j * a.nch1, a.nch1, a.c);
    const float z = a.zq[(int64_t)b * a.gamma + j];
    s_q[j] = __builtin_isnan(z) ? 0.0 : prob_of(z, a.c, rs);
  }
  lds_sync();
  if (threadIdx.x == 0) {
    int s = a.cls ? a.cls[b] : 1;
    const bool writer = ch == 0;
    if (s < 0 || s > 2) {
      if (writer) set_error(a.err, SV_DERR_TOKEN);
      s = 1;
    }
    if (writer)
      for (int j = 0; j < a.gamma; ++j)
        if (__builtin_isnan(a.zq[(int64_t)b * a.gamma + j])) set_error(a.err, SV_DERR_TOKEN);
    int pos = s == 0 ? 1 : a.gamma + 1;
    if (s == 1)
      for (int j = 1; j <= a.gamma; ++j)
        if (s_q[j - 1] < a.eps) {
          pos = j;
          break;
        }
    double qb;
    if (pos <= a.gamma) {
      qb = s_q[pos - 1];
    } else {
      const RowStat rs = staged_stat(st, staged, pb, a.gamma * a.nch1, a.nch1, a.c);
      if (writer && !(rs.S > 0.0)) set_error(a.err, SV_DERR_ROW);
      qb = rs.S > 0.0 ? 1.0 / rs.S : 0.0;  // the row's largest term is 2^0
    }
    const int k = (int)fmax(1.0, floor((double)a.k_max * (1.0 - qb)));
    s_pos = pos;
    s_k = k < a.k_max ? k : a.k_max;
    s_qb = qb;
    if (writer) {
      a.out_pos[b] = pos;
      if (a.out_qb) a.out_qb[b] = (float)qb;
      if (a.out_k) a.out_k[b] = s_k;
    }
  }
  lds_sync();
  const int k = s_k;
  const void* row = row_ptr(a.drf, (int64_t)b * rows + (s_pos - 1), a.sb);
  float lv = kNegInf;
  int32_t li = kNoIdx;
  const int64_t v0 = (int64_t)ch * a.vpc2;
  const int64_t v1 = v0 + a.vpc2 < a.nvec ? v0 + a.vpc2 : a.nvec;
  {
    const TopPair t = block_topk<kBNT, E>(RowValues<DT>{row, a.V}, v0, v1, a.V, k);
    lv = t.v;
    li = t.i;
  }
  // wave 0 holds the part's list
  TopEntry* lists = static_cast<TopEntry*>(a.lists) + (int64_t)b * a.nch2 * a.k_max;
  if (wave == 0 && lane < a.k_max)
    put_entry(lists + (int64_t)ch * a.k_max + lane, lane < k ? lv : kNegInf, lane < k ? li : kNoIdx);
  if (!arrive_last<kBNT>(&a.cnt[b], (uint32_t)a.nch2)) return;
  if (wave == 0) {
    float fv = kNegInf;
    int32_t fi = kNoIdx;
    wave_merge_entries(lists, a.nch2 * a.k_max, k, fv, fi, lane);
    if (lane < a.k_max) a.out_ids[(int64_t)b * a.k_max + lane] = (lane < k && fi != kNoIdx) ? fi : -1;
    if (lane == 0) __hip_atomic_store(&a.cnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_branch(const BranchParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16)
    branch_stats_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kBNT), 0, s>>>(p);
  else
    branch_stats_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kBNT), 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == SV_BF16)
    branch_fork_kernel<SV_BF16><<<dim3((unsigned)plan.grid2), dim3(kBNT), 0, s>>>(p);
  else
    branch_fork_kernel<SV_F32><<<dim3((unsigned)plan.grid2), dim3(kBNT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
