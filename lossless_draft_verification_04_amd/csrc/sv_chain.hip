// sv_chain.hip -- chain and multi-candidate verification on gfx950.
//
// Draft-then-verify page §1 steps 3-5 and §2.1 (accept with min(1, p/q),
// residual norm(max(0, p - q)), bonus row p_{gamma+1}); SpecDiff-2 page, Core
// method (K candidates over shared draft marginals, keep the longest streak).
//
// Three launches per call (back-to-back launches on one stream cost about
// nothing; a dependent pass inside one launch would cost a cross-block wait):
//  1. stats: one block per (row part); every needed logit row (target rows
//     1..gamma of every candidate, draft rows 1..gamma) is streamed once with
//     16-byte loads and reduced to a mergeable (max, sum 2^(z c - c max))
//     part.  The last block of a sequence to finish (arrival counter) merges
//     the parts, gathers p(x_j) and q(x_j), draws the acceptance uniforms,
//     finds each candidate's first rejection with a wave ballot, keeps the
//     best candidate and records which row(s) the final draw needs.
//  2. draw parts: blocks over parts of that row pair (or the bonus row) sum
//     the draw weights of their part.
//  3. draw finish: one block per sequence locates the part holding u * S and
//     searches inside it (one part re-read).
// The bonus row p_{gamma+1} is only read when every draft of the kept
// candidate is accepted.
#include "sv_device.hpp"
#include "sv_internal.h"

namespace sv {

constexpr int kNT = 256;
constexpr int kU = 4;
constexpr int kMaxSampleParts = 512;  // parts of the draw pass per sequence (host plan caps nch2)

struct Job {
  int64_t rowP;  // target row of the draw
  int64_t rowQ;  // draft row of a residual draw, -1 for the bonus draw
  float cmP, cmQ;
  double SP, SQ;
  double u;
};

// Parts of one sequence staged in LDS by the deciding block (all loads in
// flight together instead of one dependent load per part).
constexpr int kStage = 1024;

struct StagedParts {
  float m[kStage];
  double s[kStage];
};

// Row statistic from parts [first, first + n) of the staged set (or straight
// from global memory when the sequence has more parts than fit).
__device__ __forceinline__ RowStat merge_staged(const StagedParts& st, bool staged, const Partial* gparts, int first,
                                                int n, float c) {
  if (!staged) return merge_parts(gparts + first, n, c);
  float M = kNegInf;
  for (int i = 0; i < n; ++i) M = fmaxf(M, st.m[first + i]);
  RowStat r;
  r.pad = 0.f;
  if (M == kNegInf) {
    r.cm = 0.f;
    r.S = 0.0;
    return r;
  }
  r.cm = c * M;
  double S = 0.0;
  for (int i = 0; i < n; ++i)
    if (st.m[first + i] != kNegInf) S += st.s[first + i] * exp2((double)(c * st.m[first + i]) - (double)r.cm);
  r.S = S;
  return r;
}

template <int DT>
__device__ void chain_decide(const ChainParams& a, int b) {
  __shared__ StagedParts st;
  __shared__ RowStat sQ[SV_MAX_GAMMA];
  __shared__ int sN[SV_MAX_K];
  const int rows = (a.K + 1) * a.gamma;
  const int Kg = a.K * a.gamma;
  const int nparts = rows * a.nch1;
  const bool staged = nparts <= kStage;
  const Partial* pb = static_cast<const Partial*>(a.part1) + (int64_t)b * nparts;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  // Gathers of the first candidates' logits do not depend on any statistic:
  // issue them before waiting on the parts.
  float zp0 = 0.f, zq0 = 0.f;
  int32_t x0 = -1;
  if (wave < a.K && lane < a.gamma) {
    const int64_t o = ((int64_t)b * a.K + wave) * a.gamma + lane;
    x0 = a.tok[o];
    if (x0 >= 0 && x0 < a.V) {
      zp0 = load_elem<DT>(row_ptr(a.tgt, ((int64_t)b * a.K + wave) * (a.gamma + 1) + lane, a.tgt_sb), x0);
      zq0 = load_elem<DT>(row_ptr(a.drf, (int64_t)b * a.gamma + lane, a.drf_sb), x0);
    }
  }
  if (staged) {
    for (int i = threadIdx.x; i < nparts; i += kNT) {
      const Partial pi = get_partial(pb + i);
      st.m[i] = pi.m;
      st.s[i] = pi.s;
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.gamma; j += kNT)
    sQ[j] = merge_staged(st, staged, pb, (Kg + j) * a.nch1, a.nch1, a.c);
  __syncthreads();
  for (int k = wave; k < a.K; k += kNT / kWave) {
    bool acc = false;
    if (lane < a.gamma) {
      const int j = lane;
      const RowStat sp = merge_staged(st, staged, pb, (k * a.gamma + j) * a.nch1, a.nch1, a.c);
      const RowStat sq = sQ[j];
      const int64_t o = ((int64_t)b * a.K + k) * a.gamma + j;
      int32_t x;
      float zp, zq;
      if (k == wave) {
        x = x0;
        zp = zp0;
        zq = zq0;
      } else {
        x = a.tok[o];
        zp = zq = 0.f;
        if (x >= 0 && x < a.V) {
          zp = load_elem<DT>(row_ptr(a.tgt, ((int64_t)b * a.K + k) * (a.gamma + 1) + j, a.tgt_sb), x);
          zq = load_elem<DT>(row_ptr(a.drf, (int64_t)b * a.gamma + j, a.drf_sb), x);
        }
      }
      double p = 0.0, q = 0.0;
      if (x >= 0 && x < a.V) {
        p = prob_of(zp, a.c, sp);
        q = prob_of(zq, a.c, sq);
      } else {
        set_error(a.err, SV_DERR_TOKEN);
      }
      if (!(sp.S > 0.0) || !(sq.S > 0.0)) set_error(a.err, SV_DERR_ROW);
      const double r = uniform24(a.seed, (uint32_t)(j + 1), (uint32_t)b, (uint32_t)k, a.round, 0);
      acc = r < accept_ratio(p, q);
      if (a.out_p) a.out_p[o] = (float)p;
      if (a.out_q) a.out_q[o] = (float)q;
    }
    const uint64_t rejected = ~(uint64_t)__ballot(acc);
    int n = rejected ? __builtin_ctzll(rejected) : kWave;
    if (n > a.gamma) n = a.gamma;
    if (lane == 0) {
      sN[k] = n;
      if (a.out_n_cand) a.out_n_cand[(int64_t)b * a.K + k] = n;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    for (int k = 1; k < a.K; ++k)
      if (sN[k] > sN[best]) best = k;
    const int n = sN[best];
    a.out_n[b] = n;
    if (a.out_k) a.out_k[b] = best;
    Job jb;
    jb.rowP = ((int64_t)b * a.K + best) * (a.gamma + 1) + n;
    if (n < a.gamma) {
      const RowStat sp = merge_staged(st, staged, pb, (best * a.gamma + n) * a.nch1, a.nch1, a.c);
      jb.rowQ = (int64_t)b * a.gamma + n;
      jb.cmP = sp.cm;
      jb.SP = sp.S;
      jb.cmQ = sQ[n].cm;
      jb.SQ = sQ[n].S;
    } else {
      jb.rowQ = -1;
      jb.cmP = jb.cmQ = 0.f;
      jb.SP = jb.SQ = 0.0;
    }
    jb.u = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);
    static_cast<Job*>(a.jobs)[b] = jb;
    __hip_atomic_store(&a.cnt1[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int DT>
__global__ __launch_bounds__(kNT) void chain_stats_kernel(ChainParams a) {
  const int rows = (a.K + 1) * a.gamma;
  const int64_t per_seq = (int64_t)rows * a.nch1;
  const int64_t bid = blockIdx.x;
  const int b = (int)(bid / per_seq);
  const int64_t rem = bid - (int64_t)b * per_seq;
  const int lr = (int)(rem / a.nch1);
  const int ch = (int)(rem - (int64_t)lr * a.nch1);
  const int Kg = a.K * a.gamma;
  const void* row;
  if (lr < Kg) {
    const int k = lr / a.gamma, j = lr - k * a.gamma;
    row = row_ptr(a.tgt, ((int64_t)b * a.K + k) * (a.gamma + 1) + j, a.tgt_sb);
  } else {
    row = row_ptr(a.drf, (int64_t)b * a.gamma + (lr - Kg), a.drf_sb);
  }
  const int64_t v0 = (int64_t)ch * a.vpc1;
  const int64_t v1 = v0 + a.vpc1 < a.nvec ? v0 + a.vpc1 : a.nvec;
  const Partial part = range_stats<DT, kNT, kU>(row, a.V, v0, v1, a.c);
  if (threadIdx.x == 0) put_partial(static_cast<Partial*>(a.part1) + (int64_t)b * per_seq + (int64_t)lr * a.nch1 + ch, part);
  if (!arrive_last<kNT>(&a.cnt1[b], (uint32_t)per_seq)) return;
  chain_decide<DT>(a, b);
}

template <int DT>
__device__ DrawSpec job_spec(const ChainParams& a, const Job& jb, float cm_plain) {
  DrawSpec sp;
  sp.rowP = row_ptr(a.tgt, jb.rowP, a.tgt_sb);
  sp.c = a.c;
  sp.coef = 1.f;
  if (jb.rowQ >= 0) {
    sp.rowQ = row_ptr(a.drf, jb.rowQ, a.drf_sb);
    sp.cmP = jb.cmP;
    sp.invSP = (float)(1.0 / jb.SP);
    sp.cmQ = jb.cmQ;
    sp.invSQ = (float)(1.0 / jb.SQ);
  } else {
    sp.rowQ = nullptr;
    sp.cmP = cm_plain;
    sp.invSP = 1.f;
    sp.cmQ = 0.f;
    sp.invSQ = 1.f;
  }
  return sp;
}

// Draw pass, part sums: one block per (sequence, part) of the row pair of
// the draw (or of the bonus row), no cross-block hand-off.
template <int DT>
__global__ __launch_bounds__(kNT) void chain_draw_parts_kernel(ChainParams a) {
  const int b = blockIdx.x / a.nch2;
  const int ch = blockIdx.x - b * a.nch2;
  const Job jb = static_cast<const Job*>(a.jobs)[b];
  const int64_t v0 = (int64_t)ch * a.vpc2;
  const int64_t v1 = v0 + a.vpc2 < a.nvec ? v0 + a.vpc2 : a.nvec;
  const bool resid = jb.rowQ >= 0 && jb.SP > 0.0 && jb.SQ > 0.0;
  Partial part;
  if (resid) {
    const DrawSpec sp = job_spec<DT>(a, jb, 0.f);
    part.m = 0.f;
    part.pad = 0.f;
    part.s = range_weight_sum<DT, kNT>(sp, a.V, v0, v1);
  } else {
    part = range_stats<DT, kNT, kU>(row_ptr(a.tgt, jb.rowP, a.tgt_sb), a.V, v0, v1, a.c);
  }
  if (threadIdx.x == 0) static_cast<Partial*>(a.part2)[(int64_t)b * a.nch2 + ch] = part;
}

// Draw pass, finish: one block per sequence stages the part sums, locates
// the part holding u * S and searches inside it.
template <int DT>
__global__ __launch_bounds__(kNT) void chain_draw_finish_kernel(ChainParams a) {
  const int b = blockIdx.x;
  const Job jb = static_cast<const Job*>(a.jobs)[b];
  const bool resid = jb.rowQ >= 0 && jb.SP > 0.0 && jb.SQ > 0.0;
  const Partial* parts = static_cast<const Partial*>(a.part2) + (int64_t)b * a.nch2;
  __shared__ double s_w[kMaxSampleParts];
  __shared__ float s_pm[kMaxSampleParts];
  __shared__ double s_target;
  __shared__ int64_t s_v0, s_v1;
  __shared__ float s_cm;
  __shared__ int s_mode;  // 0 residual, 1 plain (bonus), 2 plain over P with the row statistic
  for (int i = threadIdx.x; i < a.nch2; i += kNT) {
    s_pm[i] = parts[i].m;
    s_w[i] = parts[i].s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double total = 0.0;
    float cm = 0.f;
    int mode = resid ? 0 : 1;
    if (resid) {
      for (int i = 0; i < a.nch2; ++i) total += s_w[i];
      if (!(total > 0.0)) mode = 2;  // residual mass rounded to 0: draw from p_{n+1}
    } else {
      float M = kNegInf;
      for (int i = 0; i < a.nch2; ++i) M = fmaxf(M, s_pm[i]);
      cm = a.c * M;
      for (int i = 0; i < a.nch2; ++i) {
        s_w[i] = s_pm[i] == kNegInf ? 0.0 : s_w[i] * exp2((double)(a.c * s_pm[i]) - (double)cm);
        total += s_w[i];
      }
    }
    if (mode == 2) {
      s_mode = 2;
      s_cm = jb.cmP;
      s_target = jb.u * jb.SP;
      s_v0 = 0;
      s_v1 = a.nvec;
    } else {
      const double target = jb.u * total;
      double cum = 0.0;
      int pick = -1, last_pos = -1;
      double cum_last = 0.0;
      for (int i = 0; i < a.nch2; ++i) {
        const double w = s_w[i];
        if (w > 0.0) {
          last_pos = i;
          cum_last = cum;
        }
        if (pick < 0 && cum + w > target) {
          pick = i;
          s_target = target - cum;
        }
        cum += w;
      }
      if (pick < 0) {  // rounding put u * S past the last part: take its end
        pick = last_pos < 0 ? 0 : last_pos;
        s_target = cum - cum_last;
      }
      s_mode = mode;
      s_cm = cm;
      s_v0 = (int64_t)pick * a.vpc2;
      s_v1 = s_v0 + a.vpc2 < a.nvec ? s_v0 + a.vpc2 : a.nvec;
    }
  }
  __syncthreads();
  DrawSpec sp = job_spec<DT>(a, jb, s_cm);
  if (s_mode != 0) {
    sp.rowQ = nullptr;
    sp.cmP = s_cm;
  }
  const int64_t t = block_search<DT, kNT>(sp, a.V, s_v0, s_v1, s_target);
  if (threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
}

hipError_t launch_chain(const ChainParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16) {
    chain_stats_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kNT), 0, s>>>(p);
    chain_draw_parts_kernel<SV_BF16><<<dim3((unsigned)plan.grid2), dim3(kNT), 0, s>>>(p);
    chain_draw_finish_kernel<SV_BF16><<<dim3((unsigned)p.B), dim3(kNT), 0, s>>>(p);
  } else {
    chain_stats_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kNT), 0, s>>>(p);
    chain_draw_parts_kernel<SV_F32><<<dim3((unsigned)plan.grid2), dim3(kNT), 0, s>>>(p);
    chain_draw_finish_kernel<SV_F32><<<dim3((unsigned)p.B), dim3(kNT), 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace sv
