// sv_chain.hip -- chain and multi-candidate verification on gfx950.
//
// Draft-then-verify page §1 steps 3-5 and §2.1 (accept with min(1, p/q),
// residual norm(max(0, p - q)), bonus row p_{gamma+1}); SpecDiff-2 page, Core
// method (K candidates over shared draft marginals, keep the longest streak).
//
// One launch per call, with two kinds of block.
//  - Statistics blocks (the first grid1): one per row part.  Every needed
//    logit row (target rows 1..gamma of every candidate, draft rows 1..gamma)
//    is streamed once with 16-byte loads and reduced to a mergeable
//    (max, sum 2^(z c - c max)) part; the first part of a row also gathers
//    the drafted tokens' logits in it.  The block then counts one arrival
//    for its sequence and exits (nothing waits).  When the batch is a
//    multiple of 8 sequences, all statistics blocks of a sequence sit on one
//    XCD (blocks are dealt to the 8 XCDs in turn), so sequences finish at
//    their XCD's pace and most draws run while other XCDs still stream.
//  - Draw blocks (the next B * G): G per sequence, spread over the XCDs.
//    Each waits until its sequence's parts have all arrived, merges them,
//    draws the acceptance uniforms, finds each candidate's first rejection
//    with a wave ballot and keeps the best candidate (the same decisions in
//    every block; one block stores them).  It then loads its slice of the
//    rows the final draw needs into registers, the slice sums are exchanged,
//    and the block whose slice holds u * S searches it (sv_walk.hpp).  The
//    bonus row p_{gamma+1} is only read when every draft of the kept
//    candidate is accepted.
// Each XCD places its blocks in index order, so every statistics block is
// placed before any draw block.  Draw blocks wait only on statistics blocks
// (which never wait) and on their own sequence's draw blocks, and the host
// keeps B * G within the blocks the device holds at once, so once the
// statistics blocks are done every draw block is resident.  Every wait is
// bounded.  The last draw block of a sequence to exit takes the arrivals
// back off the counter and clears the sequence's exchange slots, so both
// are zero when the next call starts (they live in the workspace's counter
// region, which every entry point leaves zero).
//
// Point-mass mode (SpecDiff-2 page, Core method: the chosen draft token is
// accepted with the verifier's own probability, the residual is resampled on
// a rejection; no drafter probabilities).  Read as the draft-then-verify
// page's §2.1 step with q a point mass at the drafted token: accept x_j iff
// r_j < p_j(x_j); the residual at a rejection is p_{n+1} with x_{n+1}
// removed.  Only target rows are streamed (no draft rows at all), and the
// draw is a plain draw from one row with one excluded token.
#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_walk.hpp"

namespace sv {

constexpr int kNT = 256;
constexpr int kU = 4;

__device__ __forceinline__ void st_dev32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Job {
  int64_t rowP;  // target row of the draw
  int64_t rowQ;  // draft row of a residual draw, -1 for the bonus draw
  float cmP, cmQ;
  double SP, SQ;
  double u;
  int32_t ex;  // point-mass residual: the rejected token (-1: none)
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
  if (n == 1) {  // one part: the part is the row statistic
    RowStat r;
    r.pad = 0.f;
    const float m = st.m[first];
    r.cm = m == kNegInf ? 0.f : c * m;
    r.S = m == kNegInf ? 0.0 : st.s[first];
    return r;
  }
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
    if (st.m[first + i] != kNegInf) S += st.s[first + i] * exp2_d((double)(c * st.m[first + i]) - (double)r.cm);
  r.S = S;
  return r;
}

// Parts per row that a lane merges straight from memory (more are staged in
// LDS by the whole block first): a lane loads the parts of two rows, or of
// one row in point-mass mode.
template <bool PM>
constexpr int direct_parts() {
  return PM ? 8 : 4;
}

// Parts [0, n) at gp, 1 <= n <= N, as 16-byte vectors, read with
// device-scope loads (written by other blocks of this launch): every load is
// issued at once and unconditionally (clamped indexes), so the merge waits
// for one round trip.
template <int N>
__device__ __forceinline__ void load_parts(const Partial* gp, int n, u32x4 (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint64_t* w = reinterpret_cast<const uint64_t*>(gp + (i < n ? i : n - 1));
    const uint64_t w0 = ld_dev(w), w1 = ld_dev(w + 1);
    v[i] = u32x4{(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
  }
}

// Row statistic from loaded parts (the arithmetic of merge_staged).
template <int N>
__device__ __forceinline__ RowStat merge_loaded(const u32x4 (&v)[N], int n, float c) {
  float m[N];
  double sum[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    m[i] = __uint_as_float(v[i][0]);
    sum[i] = __longlong_as_double((long long)(((uint64_t)v[i][3] << 32) | v[i][2]));
  }
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n) M = fmaxf(M, m[i]);
  RowStat r;
  r.pad = 0.f;
  if (M == kNegInf) {
    r.cm = 0.f;
    r.S = 0.0;
    return r;
  }
  r.cm = c * M;
  if (n == 1) {
    r.S = sum[0];
    return r;
  }
  double S = 0.0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < n && m[i] != kNegInf) S += sum[i] * exp2_d((double)(c * m[i]) - (double)r.cm);
  r.S = S;
  return r;
}

// Decisions of one sequence in LDS.  With at most one candidate per wave
// the per-position outputs wait in pq until after the draw's exchange, so
// that no block carries stores into the loads and exchange on the critical
// path (a wait for a load also waits for earlier stores here).
// What a draw block computes before it waits for the statistics: the draw
// uniform, and (wave k < K, lane j < gamma) candidate k's drafted token x_{k,j}
// and its acceptance uniform.
struct Early {
  double u;
  double r;
  int32_t x;
};

struct Decided {
  StagedParts st;
  int n[SV_MAX_K];  // first rejection (accepted count) per candidate
  Job job[SV_MAX_K];
  float2 pq[kNT / kWave][SV_MAX_GAMMA];  // (p, q) per (candidate, position) when deferred
  int best;
  bool deferred;
};

// Decisions of sequence b (identical in every block that makes them; parts
// and gathered logits were written by statistics blocks of this launch and
// are read with device-scope loads).  Wave
// k takes candidate k: lane j merges the statistics of its target and draft
// rows j, decides position j + 1, and the lane at the candidate's first
// rejection (lane 0 when every draft is accepted) writes the candidate's
// draw job, so the only block barrier is the one before the longest
// candidate is picked (plus the staging barrier when a row has more than
// direct_parts() parts).  The writer block reports errors and, unless the
// outputs are deferred (d.deferred), stores them; chain_outputs stores
// deferred ones.  Returns the kept candidate's job (in LDS).
template <int DT, bool PM>
__device__ const Job* chain_decide(const ChainParams& a, int b, bool writer, Decided& d, const Early& e) {
  StagedParts& st = d.st;
  int* sN = d.n;
  Job* sJob = d.job;
  const bool defer = a.K <= kNT / kWave;
  const int Kg = a.K * a.gamma;
  const int rows = PM ? Kg : Kg + a.gamma;
  const int nparts = rows * a.nch1;
  constexpr int kDP = direct_parts<PM>();
  const bool direct = a.nch1 <= kDP;
  const bool staged = !direct && nparts <= kStage;
  const Partial* pb = static_cast<const Partial*>(a.part1) + (int64_t)b * nparts;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  // the first candidate's gathered logits are loaded before the parts are
  // staged, so that both travel in one round of loads (its token came
  // before the wait)
  const int32_t x_pre = e.x;
  uint32_t zp_pre = 0, zq_pre = 0;
  if (wave < a.K && lane < a.gamma) {
    const int64_t o = ((int64_t)b * a.K + wave) * a.gamma + lane;
    zp_pre = ld_dev32(reinterpret_cast<const uint32_t*>(a.zg) + o);
    if (!PM) zq_pre = ld_dev32(reinterpret_cast<const uint32_t*>(a.zq) + o);
  }
  if (staged) {
    for (int i = threadIdx.x; i < nparts; i += kNT) {
      const Partial pi = get_partial(pb + i);
      st.m[i] = pi.m;
      st.s[i] = pi.s;
    }
  }
  if (!direct) lds_sync();  // block-uniform
  for (int k = wave; k < a.K; k += kNT / kWave) {
    bool acc = false;
    RowStat sp, sq;
    sp.cm = sq.cm = 0.f;
    sp.pad = sq.pad = 0.f;
    sp.S = 0.0;
    sq.S = 1.0;  // point mass: q(x) = 1
    int32_t x = -1;
    const double u = e.u;  // the draw uniform (only the job's lane uses it)
    if (lane < a.gamma) {
      const int j = lane;
      const int64_t o = ((int64_t)b * a.K + k) * a.gamma + j;
      const int first_p = (k * a.gamma + j) * a.nch1, first_q = (Kg + j) * a.nch1;
      const double r = k == wave ? e.r : uniform24(a.seed, (uint32_t)(j + 1), (uint32_t)b, (uint32_t)k, a.round, 0);
      // the drafted token, its gathered logits (stats pass) and the rows'
      // parts: one round of independent loads
      const bool pre = k == wave;
      x = pre ? x_pre : a.tok[o];
      const float zp = __uint_as_float(pre ? zp_pre : ld_dev32(reinterpret_cast<const uint32_t*>(a.zg) + o));
      const float zq =
          PM ? 0.f : __uint_as_float(pre ? zq_pre : ld_dev32(reinterpret_cast<const uint32_t*>(a.zq) + o));
      if (a.nch1 == 1) {  // whole rows: one part each
        u32x4 vp[1], vq[1];
        load_parts(pb + first_p, 1, vp);
        if constexpr (!PM) load_parts(pb + first_q, 1, vq);
        sp = merge_loaded(vp, 1, a.c);
        if constexpr (!PM) sq = merge_loaded(vq, 1, a.c);
      } else if (direct) {
        u32x4 vp[kDP], vq[PM ? 1 : kDP];
        load_parts(pb + first_p, a.nch1, vp);
        if constexpr (!PM) load_parts(pb + first_q, a.nch1, vq);
        sp = merge_loaded(vp, a.nch1, a.c);
        if constexpr (!PM) sq = merge_loaded(vq, a.nch1, a.c);
      } else {
        sp = merge_staged(st, staged, pb, first_p, a.nch1, a.c);
        if (!PM) sq = merge_staged(st, staged, pb, first_q, a.nch1, a.c);
      }
      double p = 0.0, q = PM ? 1.0 : 0.0;
      if (x >= 0 && x < a.V) {
        p = prob_of(zp, a.c, sp);
        if (!PM) q = prob_of(zq, a.c, sq);
      } else if (writer) {
        set_error(a.err, SV_DERR_TOKEN);
      }
      if (writer && (!(sp.S > 0.0) || !(sq.S > 0.0))) set_error(a.err, SV_DERR_ROW);
      acc = r < accept_ratio(p, q);
      if (defer) {
        d.pq[k][j] = make_float2((float)p, (float)q);
      } else if (writer) {
        if (a.out_p) a.out_p[o] = (float)p;
        if (!PM && a.out_q) a.out_q[o] = (float)q;
      }
    }
    const uint64_t rejected = ~(uint64_t)__ballot(acc);
    int n = rejected ? __builtin_ctzll(rejected) : kWave;
    if (n > a.gamma) n = a.gamma;
    if (lane == 0) {
      sN[k] = n;
      if (!defer && writer && a.out_n_cand) a.out_n_cand[(int64_t)b * a.K + k] = n;
    }
    if (lane == (n < a.gamma ? n : 0)) {
      Job jb;
      jb.rowP = ((int64_t)b * a.K + k) * (a.gamma + 1) + n;
      jb.ex = -1;
      if (n < a.gamma) {
        jb.cmP = sp.cm;
        jb.SP = sp.S;
        if (PM) {
          jb.ex = x >= 0 && x < a.V ? x : -1;
          jb.rowQ = -1;
          jb.cmQ = 0.f;
          jb.SQ = 0.0;
        } else {
          jb.rowQ = (int64_t)b * a.gamma + n;
          jb.cmQ = sq.cm;
          jb.SQ = sq.S;
        }
      } else {
        jb.rowQ = -1;
        jb.cmP = jb.cmQ = 0.f;
        jb.SP = jb.SQ = 0.0;
      }
      jb.u = u;
      sJob[k] = jb;
    }
  }
  lds_sync();
  int best = 0;
  for (int k = 1; k < a.K; ++k)
    if (sN[k] > sN[best]) best = k;
  d.best = best;
  d.deferred = defer;
  if (!defer && writer && threadIdx.x == 0) {
    a.out_n[b] = sN[best];
    if (a.out_k) a.out_k[b] = best;
  }
  return &sJob[best];
}

// The deferred outputs of sequence b (one block).
template <bool PM>
__device__ void chain_outputs(const ChainParams& a, int b, const Decided& d) {
  if (!d.deferred) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int k = threadIdx.x / kWave;
  if (k < a.K && lane < a.gamma) {
    const int64_t o = ((int64_t)b * a.K + k) * a.gamma + lane;
    if (a.out_p) a.out_p[o] = d.pq[k][lane].x;
    if (!PM && a.out_q) a.out_q[o] = d.pq[k][lane].y;
  }
  if (k < a.K && lane == 0 && a.out_n_cand) a.out_n_cand[(int64_t)b * a.K + k] = d.n[k];
  if (threadIdx.x == 0) {
    a.out_n[b] = d.n[d.best];
    if (a.out_k) a.out_k[b] = d.best;
  }
}

// Statistics block: one row part, then one arrival for its sequence.
template <int DT>
__device__ void stats_role(const ChainParams& a) {
  const int rows = a.pm ? a.K * a.gamma : (a.K + 1) * a.gamma;
  const int64_t per_seq = (int64_t)rows * a.nch1;
  SV_STAMP_START(0);
  const int64_t bid = blockIdx.x;
  int b;
  int64_t rem;
  if (a.xcd) {
    // blocks are dealt to the 8 XCDs in turn: XCD x streams sequences x, x + 8, ...
    const int64_t i = bid >> 3;
    b = (int)(bid & 7) + 8 * (int)(i / per_seq);
    rem = i % per_seq;
  } else {
    b = (int)(bid / per_seq);
    rem = bid - (int64_t)b * per_seq;
  }
  const int lr = (int)(rem / a.nch1);
  const int ch = (int)(rem - (int64_t)lr * a.nch1);
  const int Kg = a.K * a.gamma;
  const bool is_tgt = lr < Kg;
  const void* row;
  int j;
  if (is_tgt) {
    const int k = lr / a.gamma;
    j = lr - k * a.gamma;
    row = row_ptr(a.tgt, ((int64_t)b * a.K + k) * (a.gamma + 1) + j, a.tgt_sb);
  } else {
    j = lr - Kg;
    row = row_ptr(a.drf, (int64_t)b * a.gamma + j, a.drf_sb);
  }
  // the first part of a row also gathers the drafted tokens' logits in it
  // (target row (k, j): x_{k,j}; draft row j: x_{k,j} of every candidate k);
  // the token is loaded here and the logit inside the stream
  int64_t zo = -1;
  int32_t x = 0;
  if (ch == 0 && (int)threadIdx.x < (is_tgt ? 1 : a.K)) {
    const int k = is_tgt ? lr / a.gamma : (int)threadIdx.x;
    zo = ((int64_t)b * a.K + k) * a.gamma + j;
    x = a.tok[zo];
  }
  const int64_t v0 = (int64_t)ch * a.vpc1;
  const int64_t v1 = v0 + a.vpc1 < a.nvec ? v0 + a.vpc1 : a.nvec;
  uint32_t zbits = 0;
  const Partial part = range_stats<DT, kNT, kU>(row, a.V, v0, v1, a.c, zo >= 0, x, &zbits);
  SV_STAMP(0, 1);
  SV_STAMP_TAG(0, 1, b);
  // every store of this block is made by wave 0 (K <= 64 gathering threads)
  if (threadIdx.x < kWave) {
    if (threadIdx.x == 0) put_partial(static_cast<Partial*>(a.part1) + (int64_t)b * per_seq + (int64_t)lr * a.nch1 + ch, part);
    if (zo >= 0)
      st_dev32(reinterpret_cast<uint32_t*>(is_tgt ? a.zg : a.zq) + zo,
               __float_as_uint((x >= 0 && x < a.V) ? bits_value<DT>(zbits) : 0.f));
    __builtin_amdgcn_s_waitcnt(0);  // the wave's stores are complete (device-visible)
    if (threadIdx.x == 0) add_dev32(a.cnt + (int64_t)b * a.cstride, 1u);
  }
  SV_STAMP_FLUSH(0);
}

template <int DT>
__device__ DrawSpec job_spec(const ChainParams& a, const Job& jb, float cm_plain) {
  DrawSpec sp;
  sp.rowP = row_ptr(a.tgt, jb.rowP, a.tgt_sb);
  sp.c = a.c;
  sp.coef = 1.f;
  sp.ex = nullptr;
  sp.nex = 0;
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

// Wave 0 waits until every part of sequence b has arrived; false if the wait
// ran out.  Far from done (under half the parts in), polls are spaced about
// half a microsecond apart.
__device__ bool wait_parts(const ChainParams& a, int b, uint32_t limit) {
  const uint32_t* arrivals = a.cnt + (int64_t)b * a.cstride;
  const uint32_t total = (uint32_t)(a.pm ? a.K * a.gamma : (a.K + 1) * a.gamma) * (uint32_t)a.nch1;
  uint32_t spins = 0;
  for (;;) {
    uint32_t c = 0;
    if ((threadIdx.x & (kWave - 1)) == 0) c = ld_dev32(arrivals);
    c = __builtin_amdgcn_readfirstlane(c);
    if (c >= total) return true;
    const bool near = 2u * c >= total;
    spins += near ? 1u : 4u;
    if (spins > limit) return false;
    if (near)
      __builtin_amdgcn_s_sleep(2);
    else
      __builtin_amdgcn_s_sleep(16);
  }
}

// A draw block of sequence b is done with the sequence's counters and
// exchange slots, in two steps.  draw_exit_begin (thread 0) counts the exit
// once the block's slot stores are complete (wave 0 made them all) and
// keeps the old count; the counting atomic is then in flight while the
// block searches.  draw_exit_end (block-uniform) lets the last block of the
// sequence take the arrivals back off the counter (late ones, after a
// timed-out wait, bring it to zero too) and clear the exchange slots for the
// next call.
__device__ __forceinline__ uint32_t draw_exit_begin(const ChainParams& a, int b) {
  uint32_t old = 0;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    old = add_dev32(a.cnt + (int64_t)(a.B + b) * a.cstride, 1u);
  }
  return old;
}
__device__ void draw_exit_end(const ChainParams& a, int b, uint32_t old) {
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    s_last = old == (uint32_t)a.G - 1u;
    if (s_last) {
      st_dev32(a.cnt + (int64_t)(a.B + b) * a.cstride, 0u);
      const uint32_t total = (uint32_t)(a.pm ? a.K * a.gamma : (a.K + 1) * a.gamma) * (uint32_t)a.nch1;
      __hip_atomic_fetch_sub(a.cnt + (int64_t)b * a.cstride, total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  lds_sync();
  if (s_last && a.G > 1) {
    uint64_t* slots = static_cast<uint64_t*>(a.slots) + (int64_t)b * kSlotWords * a.G;
    for (int i = threadIdx.x; i < kSlotWords * a.G; i += kNT) st_dev(slots + i, 0ull);
  }
}
__device__ __forceinline__ void draw_exit(const ChainParams& a, int b) { draw_exit_end(a, b, draw_exit_begin(a, b)); }

template <int DT, bool HELD, bool PM>
__device__ void draw_body(const ChainParams& a, int b, int g, Exchange& x, Decided& dec, uint64_t* s_words,
                          uint64_t* s_w1, SliceSums& ss, const Early& e) {
  const Job* pj = chain_decide<DT, PM>(a, b, g == 0, dec, e);
  const Job jb = *pj;
  SV_STAMP(0, 2);
  const int64_t spv = (a.nvec + a.G - 1) / a.G;
  const int64_t v0 = (int64_t)g * spv < a.nvec ? (int64_t)g * spv : a.nvec;
  const int64_t v1 = v0 + spv < a.nvec ? v0 + spv : a.nvec;
  const bool resid = !PM && jb.rowQ >= 0 && jb.SP > 0.0 && jb.SQ > 0.0;
  const bool pm_resid = PM && jb.SP > 0.0;  // a rejection, in a row with mass
  DrawSpec sp = job_spec<DT>(a, jb, 0.f);
  Slice<DT, kNT, HELD> sl;
  sl.load(sp.rowP, resid ? sp.rowQ : nullptr, v0, v1);
  double total;
  bool plain = false;
  if (pm_resid) {
    // p_{n+1} without the rejected token, under the row's own shift
    sp.rowQ = nullptr;
    sp.cmP = jb.cmP;
    sp.invSP = 1.f;
    sp.ex = &pj->ex;
    sp.nex = jb.ex >= 0 ? 1 : 0;
    total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    if (!(total > 0.0)) {
      // the row is a point mass at the rejected token (by rounding): draw from it
      sp.nex = 0;
      total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    }
  } else if (resid) {
    const double mine = sl.prepare(sp, a.V);
    SV_STAMP(0, 3);
    total = exchange_sum(x, mine, s_words, &ss);
    if (!(total > 0.0)) {
      // residual mass rounded to 0: draw from p_{n+1} itself
      sp.rowQ = nullptr;
      total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    }
  } else {
    // bonus draw (or a row without mass): the row's statistics from the
    // slices in one exchange, then a plain draw with the row's shift
    float M;
    total = exchange_stats(x, sl.row_stats(a.c, a.V), a.c, s_words, s_w1, &ss, &M);
    if (g == 0 && threadIdx.x == 0 && M == kNegInf) set_error(a.err, SV_DERR_ROW);
    sp.rowQ = nullptr;
    sp.cmP = M == kNegInf ? 0.f : a.c * M;
    sp.invSP = 1.f;
    plain = true;
  }
  SV_STAMP(0, 4);
  int pick;
  double loc;
  pick_slice(ss, x.G, jb.u * total, &pick, &loc);
  // the slots are read no more (the search works on registers): the exit
  // counts while the block searches
  const uint32_t exits = draw_exit_begin(a, b);
  // a block other than the searching one stores the deferred outputs
  if (g == (x.G > 1 && pick == 0 ? 1 : 0)) chain_outputs<PM>(a, b, dec);
  if (pick == g) {
    if (plain) sl.prepare(sp, a.V);  // the owner's weights under the row's shift
    const int64_t t = sl.search(sp, a.V, loc);
    if (threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
    SV_STAMP(0, 5);
  }
  draw_exit_end(a, b, exits);
}

// Draw block g of sequence b: decides the sequence and owns one slice of the
// draw row(s).
template <int DT, bool HELD, bool PM>
__device__ void draw_role(const ChainParams& a, int d, Decided& dec) {
  // with sequences grouped by XCD, a sequence's draw blocks sit on the XCD
  // that streamed its rows (the grid before them is a multiple of 8 blocks,
  // so d and the block index agree mod 8): they start as that XCD's
  // statistics blocks end, whatever the other XCDs still stream
  int b, g;
  if (a.xcd) {
    const int i = d >> 3;
    b = (d & 7) + 8 * (i / a.G);
    g = i - (i / a.G) * a.G;
  } else {
    b = d / a.G;
    g = d - b * a.G;
  }
  __shared__ uint64_t s_words[kMaxG], s_w1[kMaxG];
  __shared__ int s_ok;
  SliceSums ss;  // the slices' values of the last exchange
  SV_STAMP_START(0);
  SV_STAMP_TAG(0, 2, b);
  Exchange x = make_exchange(a.slots, a.err, a.knobs, b, a.G, g);
  // everything that does not depend on the statistics, while they stream
  Early e;
  e.u = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);
  e.r = 1.0;
  e.x = 0;
  {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (wave < a.K && lane < a.gamma) {
      e.x = a.tok[((int64_t)b * a.K + wave) * a.gamma + lane];
      e.r = uniform24(a.seed, (uint32_t)(lane + 1), (uint32_t)b, (uint32_t)wave, a.round, 0);
    }
  }
  if (threadIdx.x < kWave) {
    const bool ok = wait_parts(a, b, x.limit);
    if (threadIdx.x == 0) {
      s_ok = ok;
      if (!ok) set_error(a.err, SV_DERR_TIMEOUT);
    }
  }
  __syncthreads();
  SV_STAMP(0, 1);
  if (s_ok) draw_body<DT, HELD, PM>(a, b, g, x, dec, s_words, s_w1, ss, e);  // counts the exit itself
  if (!s_ok) draw_exit(a, b);
  SV_STAMP(0, 6);
  SV_STAMP_FLUSH(0);
}

template <int DT, bool HELD, bool PM>
__global__ __launch_bounds__(kNT) void chain_kernel(ChainParams a) {
  __shared__ Decided dec;
  if ((int64_t)blockIdx.x < a.grid1)
    stats_role<DT>(a);
  else
    draw_role<DT, HELD, PM>(a, (int)((int64_t)blockIdx.x - a.grid1), dec);
}

template <int DT>
hipError_t launch_chain_t(const ChainParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.grid1 + (int64_t)p.B * p.G));
  if (p.pm) {
    if (p.held)
      chain_kernel<DT, true, true><<<grid, dim3(kNT), 0, s>>>(p);
    else
      chain_kernel<DT, false, true><<<grid, dim3(kNT), 0, s>>>(p);
  } else {
    if (p.held)
      chain_kernel<DT, true, false><<<grid, dim3(kNT), 0, s>>>(p);
    else
      chain_kernel<DT, false, false><<<grid, dim3(kNT), 0, s>>>(p);
  }
  return hipGetLastError();
}

SV_TIMELINE_SETTER(timeline_set_chain)

hipError_t launch_chain(const ChainParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  (void)plan;
  return dt == SV_BF16 ? launch_chain_t<SV_BF16>(p, s) : launch_chain_t<SV_F32>(p, s);
}

template <int DT, bool PM>
const void* chain_fn(bool held) {
  return held ? reinterpret_cast<const void*>(&chain_kernel<DT, true, PM>)
              : reinterpret_cast<const void*>(&chain_kernel<DT, false, PM>);
}

// Blocks of the chain kernel the device holds at once.
int chain_capacity(sv_dtype dt, bool held, bool pm) {
  static int cache[2][2][2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& c = cache[dt == SV_BF16][held][pm][dev];
  if (c == 0) {
    const void* fn;
    if (dt == SV_BF16)
      fn = pm ? chain_fn<SV_BF16, true>(held) : chain_fn<SV_BF16, false>(held);
    else
      fn = pm ? chain_fn<SV_F32, true>(held) : chain_fn<SV_F32, false>(held);
    c = device_capacity(fn, kNT, dev);
  }
  return c;
}

}  // namespace sv
