// sv_topk.hpp -- a block's top-F values of a range of 16-byte vectors
// (value descending, index ascending), shared by the fan-out, the SpecBranch
// fork and the PRESTO expansion.
//
// Lists live in registers, one entry per lane (lane i = i-th best).  The scan
// takes two passes (block_topk_scan): every thread first keeps only the best
// element of the vectors it owns, the block selects the F threads with the
// best such elements by F rounds of a wave-wide DPP reduction, and only
// those threads' vectors are looked at again and their qualifying values
// inserted with a lane shift.  Lists from other blocks are merged by the same
// selection rounds (wave_merge_entries).
#pragma once

#include "sv_device.hpp"

namespace sv {

struct TopEntry {
  float val;
  int32_t idx;
};

constexpr int32_t kNoIdx = 0x7fffffff;

__device__ __forceinline__ void put_entry(TopEntry* dst, float val, int32_t idx) {
  st_dev(reinterpret_cast<uint64_t*>(dst), (uint64_t)__float_as_uint(val) | ((uint64_t)(uint32_t)idx << 32));
}
__device__ __forceinline__ TopEntry get_entry(const TopEntry* src) {
  const uint64_t w = ld_dev(reinterpret_cast<const uint64_t*>(src));
  TopEntry t;
  t.val = __uint_as_float((uint32_t)w);
  t.idx = (int32_t)(uint32_t)(w >> 32);
  return t;
}

// (value desc, index asc), evaluated without branches.  An empty entry is
// (-inf, kNoIdx): it never beats any entry, and every entry with an index
// beats it.
__device__ __forceinline__ bool top_better(float va, int32_t ia, float vb, int32_t ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

// DPP data movement within a wave (one VALU instruction each; a lane whose
// source is outside the pattern keeps `old`).
template <int CTRL, int ROWS>
__device__ __forceinline__ int32_t dpp_i(int32_t old, int32_t v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
constexpr int kWaveShr1 = 0x138;  // lane l takes lane l - 1
constexpr int kRowShr = 0x110;    // + n: lane l takes lane l - n within its row of 16
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// (v, i) <- the better of itself and the pair DPP pattern CTRL brings in
// (selects, no branches).
template <int CTRL, int ROWS>
__device__ __forceinline__ void best_step(float& v, int32_t& i) {
  const float ov = dpp_f<CTRL, ROWS>(v, v);
  const int32_t oi = dpp_i<CTRL, ROWS>(i, i);
  const bool take = top_better(ov, oi, v, i);
  v = take ? ov : v;
  i = take ? oi : i;
}

// The wave's best pair (value desc, index asc; empty entries are
// (-inf, kNoIdx) and never win), in every lane: a reduction within rows of
// 16, then across rows, ending in lane 63.
__device__ __forceinline__ void wave_best(float& v, int32_t& i) {
  best_step<kRowShr + 1, 0xF>(v, i);
  best_step<kRowShr + 2, 0xF>(v, i);
  best_step<kRowShr + 4, 0xF>(v, i);
  best_step<kRowShr + 8, 0xF>(v, i);
  best_step<kRowBcast15, 0xA>(v, i);
  best_step<kRowBcast31, 0xC>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
  i = __builtin_amdgcn_readlane(i, kWave - 1);
}

// Insert (v, i) into the wave's sorted list (lane l holds entry l; lanes
// >= F hold the empty entry).  Wave-uniform arguments.
__device__ __forceinline__ void wave_insert(float& lv, int32_t& li, float v, int32_t i, int F, int lane) {
  const bool here = top_better(v, i, lv, li) & (lane < F);
  const uint64_t m = __ballot(here);
  if (!m) return;
  const int pos = __builtin_ctzll(m);
  const float up_v = dpp_f<kWaveShr1, 0xF>(lv, lv);
  const int32_t up_i = dpp_i<kWaveShr1, 0xF>(li, li);
  if (lane < F) {
    if (lane > pos) {
      lv = up_v;
      li = up_i;
    } else if (lane == pos) {
      lv = v;
      li = i;
    }
  }
}

// One logit row as a value source (elements past V read as -inf; -inf
// logits are listed like any other value).
template <int DT>
struct RowValues {
  const void* row;
  int V;
  using Data = u32x4;
  static constexpr bool kSkipNegInf = false;
  __device__ __forceinline__ Data load(int64_t v) const { return load_vec(row, v); }
  __device__ __forceinline__ void values(const Data& d, int64_t v, float* x) const {
    constexpr int E = Fmt<DT>::kPerVec;
    unpack<DT>(d, x);
    if ((v + 1) * E > V) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (v * E + e >= V) x[e] = kNegInf;
    }
  }
};

// Merge n entries (src[0..n), written by other blocks of the launch) into
// the wave's list (lv, li) of F entries: up to kMergeK entries per lane in
// one round of device-scope loads, then F rounds of a wave-wide selection
// over them and the list (no entry-by-entry insertion chain).
constexpr int kMergeK = 4;
__device__ __forceinline__ void wave_merge_entries(const TopEntry* src, int n, int F, float& lv, int32_t& li,
                                                   int lane) {
  for (int e0 = 0; e0 < n; e0 += kWave * kMergeK) {
    float cv[kMergeK + 1];
    int32_t ci[kMergeK + 1];
#pragma unroll
    for (int q = 0; q < kMergeK; ++q) {
      const int e = e0 + q * kWave + lane;
      TopEntry t;
      t.val = kNegInf;
      t.idx = kNoIdx;
      if (e < n) t = get_entry(src + e);
      cv[q] = t.val;
      ci[q] = t.idx;
    }
    cv[kMergeK] = lane < F ? lv : kNegInf;
    ci[kMergeK] = lane < F ? li : kNoIdx;
    uint32_t taken = 0;
    float nv = kNegInf;
    int32_t ni = kNoIdx;
    for (int k = 0; k < F; ++k) {
      float bv = kNegInf;
      int32_t bi = kNoIdx;
      int bq = -1;
#pragma unroll
      for (int q = 0; q <= kMergeK; ++q) {
        const bool t = (((taken >> q) & 1u) == 0u) & top_better(cv[q], ci[q], bv, bi);
        bv = t ? cv[q] : bv;
        bi = t ? ci[q] : bi;
        bq = t ? q : bq;
      }
      float wv = bv;
      int32_t wi = bi;
      wave_best(wv, wi);
      if (wi == kNoIdx) break;
      if (bi == wi && bq >= 0) taken |= 1u << bq;  // an index is held once, so only its holder matches
      if (lane == k) {
        nv = wv;
        ni = wi;
      }
    }
    lv = nv;
    li = ni;
  }
}

// A value source for the scans below provides
//   using Data = ...;                        one vector's raw data
//   Data load(int64_t v) const;              the loads of vector v
//   void values(const Data&, int64_t v, float* x) const;
//                                            its E values (-inf past V)
//   static constexpr bool kSkipNegInf;       -inf values are never listed
// A lane's entry of a wave's list (lane l holds the l-th best).
struct TopPair {
  float v;
  int32_t i;
};

// Insert the values of one vector per lane that `mine` flags (lane l's
// vector is vector vs of the range; x its E values) into the wave's list of
// F entries; *count is the number of entries held (wave-uniform).
template <int E>
__device__ __forceinline__ void insert_flagged(const float (&x)[E], uint32_t mine, int64_t vs, int F, float& lv,
                                               int32_t& li, int* count, int lane) {
  uint64_t cm = __ballot(mine != 0);
  while (cm) {
    const int sl = __builtin_ctzll(cm);
    cm &= cm - 1;
    uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)mine, sl);
    const int64_t v = readlane_i64(vs, sl);
    while (bits) {
      const int e = __builtin_ctz(bits);
      bits &= bits - 1;
      float xe = 0.f;
#pragma unroll
      for (int q = 0; q < E; ++q)
        if (q == e) xe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[q]), sl));
      const int32_t ie = (int32_t)(v * E + e);
      const float fv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), F - 1));
      const int32_t fi = __builtin_amdgcn_readlane(li, F - 1);
      if (*count < F || top_better(xe, ie, fv, fi)) {
        wave_insert(lv, li, xe, ie, F, lane);
        if (*count < F) ++*count;
      }
    }
  }
}

// The block's top F values of [v0, v1) as per-wave lists (F <= 64; every
// wave of the block calls it with the same arguments).  Block thread t owns
// the vectors v0 + t + k * NT.
//  Pass 1 streams the range once; each thread keeps only its best element
//  (value desc, then vector asc), about one max and one compare per vector.
//  The block's F best threads by that element are the only threads that can
//  own a top-F value: a value owned by any other thread is beaten by the F
//  selected threads' bests.  So
//  pass 2 looks again at just those threads' vectors -- still in registers
//  when every thread owns at most kWin of them, else re-read (F times the
//  range / NT vectors, mostly from L2) spread over the waves -- and each wave
//  lists the values of its share that reach the F-th selected best,
//  inserting each with a lane shift.
// Each wave returns its list (lane l = l-th best); the block's top F is the
// top F of the waves' lists.  (Keeping running top-F lists during the
// stream instead costs an insertion per new record, about F ln(n / F) per
// list, which dominated at F >= 4.)  MAY_HOLD = false drops the register
// path (it keeps kWin vectors live across the selection).
template <int NT, int E, bool MAY_HOLD, int KEEP, class Src>
__device__ TopPair block_topk_scan(const Src src, int64_t v0, int64_t v1, int V, int F) {
  constexpr int NW = NT / kWave;
  constexpr int kWin = 4;   // vectors in flight per thread
  constexpr int kKeep = KEEP > 0 ? KEEP : 1;  // best vectors a thread remembers for pass 2
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  __shared__ float s_m[NT];
  __shared__ int32_t s_mv[NT];
  __shared__ uint8_t s_pick[NT];
  __shared__ int32_t s_sel[kWave];
  __shared__ int32_t s_rr[kWave * kKeep];  // vectors pass 2 reads again (offsets in the range)
  __shared__ int s_nsel, s_nrr, s_full;
  __shared__ float s_tf;
  float lv = kNegInf;
  int32_t li = kNoIdx;
  if (F <= 0) return TopPair{lv, li};
  const int64_t span = v1 - v0;
  const int64_t nk = (span + NT - 1) / NT;  // vectors per thread at most
  const bool held = MAY_HOLD && nk <= kWin;  // block-uniform
  // pass 1: this thread's kKeep best vectors by their largest element, as
  // (value, vector offset), best first (equal values: lower offset first);
  // the first is the thread's best element
  float bm[kKeep];
  int32_t bo[kKeep];
#pragma unroll
  for (int i = 0; i < kKeep; ++i) {
    bm[i] = kNegInf;
    bo[i] = kNoIdx;
  }
  typename Src::Data d[kWin];
  if (span > 0) {  // block-uniform
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int64_t a = v0 + tid + (int64_t)u * NT;
      d[u] = src.load(a < v1 ? a : v1 - 1);  // clamped: every load is issued
    }
    for (int64_t v = v0 + tid; v < v1; v += (int64_t)kWin * NT) {
      typename Src::Data nx[kWin];
      if (!held) {
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
          const int64_t a = v + (int64_t)(kWin + u) * NT;
          nx[u] = src.load(a < v1 ? a : v1 - 1);
        }
      }
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t vu = v + (int64_t)u * NT;
        if (vu < v1) {
          float x[E];
          src.values(d[u], vu, x);
          float vm = x[0];
#pragma unroll
          for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[e]);
          // a vector always holds a listable element unless -inf is not listed
          const bool has = !Src::kSkipNegInf || vm > kNegInf;
          if (has) {
            // insertion by carrying the displaced entry down the list
            float cv = vm;
            int32_t co = (int32_t)(vu - v0);
#pragma unroll
            for (int i = 0; i < kKeep; ++i) {
              const bool t = (bo[i] == kNoIdx) | top_better(cv, co, bm[i], bo[i]);
              const float sv = bm[i];
              const int32_t so = bo[i];
              bm[i] = t ? cv : bm[i];
              bo[i] = t ? co : bo[i];
              cv = t ? sv : cv;
              co = t ? so : co;
            }
          }
        }
      }
      if (held) break;  // d stays for pass 2
#pragma unroll
      for (int u = 0; u < kWin; ++u) d[u] = nx[u];
    }
  }
  SV_STAMP(0, 2);  // (timeline builds) this thread's pass 1 is done
  const float m = bm[0];
  const int32_t mv = bo[0];
  s_m[tid] = m;
  s_mv[tid] = mv;
  s_pick[tid] = 0;
  if (tid == 0) {
    s_nrr = 0;
    s_full = 0;
  }
  lds_sync();
  SV_STAMP(0, 6);  // (timeline builds) every thread's pass 1 is done
  // the F best threads (wave 0: F rounds of a wave-wide selection over the
  // NW entries each lane holds)
  if (wave == 0) {
    float em[NW];
    int32_t ei[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      em[w] = s_m[w * kWave + lane];
      ei[w] = s_mv[w * kWave + lane];
    }
    uint32_t taken = 0;
    int n = 0;
    float tf = kNegInf;
    for (; n < F; ++n) {
      float bv = kNegInf;
      int32_t bi = kNoIdx;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const bool t = (((taken >> w) & 1u) == 0u) & top_better(em[w], ei[w], bv, bi);
        bv = t ? em[w] : bv;
        bi = t ? ei[w] : bi;
      }
      float wv = bv;
      int32_t wi = bi;
      wave_best(wv, wi);
      if (wi == kNoIdx) break;  // fewer than F threads hold an element
      const int owner = wi % NT;  // the thread whose vectors hold it
      if (lane == (owner & (kWave - 1))) taken |= 1u << (owner / kWave);
      if (lane == 0) {
        s_sel[n] = owner;
        s_pick[owner] = 1;
      }
      tf = wv;
    }
    if (lane == 0) {
      s_nsel = n;
      s_tf = n == F ? tf : kNegInf;  // fewer threads than F: every listable value qualifies
    }
  }
  lds_sync();
  SV_STAMP(0, 3);  // (timeline builds) the F best threads are selected
  const float tf = s_tf;
  int count = 0;
  if (MAY_HOLD && held) {
    // pass 2 from registers: the selected threads flag their own values
    const bool picked = s_pick[tid] != 0;
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int64_t vu = v0 + tid + (int64_t)u * NT;
      float x[E];
      uint32_t mine = 0;
      if (picked && vu < v1) {
        src.values(d[u], vu, x);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (x[e] >= tf && vu * E + e < V && (!Src::kSkipNegInf || x[e] > kNegInf)) mine |= 1u << e;
      }
      insert_flagged<E>(x, mine, vu, F, lv, li, &count, lane);
    }
    return TopPair{lv, li};
  }
  // pass 2 re-read, short form (KEEP > 0): each selected thread lists its
  // kept vectors whose largest element reaches the F-th selected best; only
  // a thread with more such vectors than it kept needs all its vectors read
  // again
  if (KEEP == 0 && tid == 0) s_full = 1;
  if (KEEP > 0 && s_pick[tid]) {
    if (nk > kKeep && bo[kKeep - 1] != kNoIdx && bm[kKeep - 1] >= tf) {
      s_full = 1;  // every writer stores the same value
    } else {
#pragma unroll
      for (int i = 0; i < kKeep; ++i)
        if (bo[i] != kNoIdx && bm[i] >= tf) s_rr[atomicAdd(&s_nrr, 1)] = bo[i];
    }
  }
  lds_sync();
  if (!s_full) {
    const int nrr = s_nrr;
    for (int base = 0; base < nrr; base += NT) {  // block-uniform
      const int t = base + tid;
      const int64_t vs = t < nrr ? v0 + s_rr[t] : -1;
      typename Src::Data dd;
      if (vs >= 0) dd = src.load(vs);
      float x[E];
      uint32_t mine = 0;
      if (vs >= 0) {
        src.values(dd, vs, x);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (x[e] >= tf && vs * E + e < V && (!Src::kSkipNegInf || x[e] > kNegInf)) mine |= 1u << e;
      }
      insert_flagged<E>(x, mine, vs, F, lv, li, &count, lane);
    }
    return TopPair{lv, li};
  }
  // pass 2 re-read, full form: the selected threads' vectors, kWin per thread at a time
  const int nsel = s_nsel;
  const int64_t total = (int64_t)nsel * nk;
  for (int64_t base = 0; base < total; base += (int64_t)kWin * NT) {
    int64_t vs[kWin];
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int64_t t = base + (int64_t)u * NT + tid;
      vs[u] = -1;
      if (t < total) {
        const int sidx = (int)(t / nk);
        const int64_t r = s_sel[sidx] + (t - (int64_t)sidx * nk) * NT;
        if (r < span) vs[u] = v0 + r;
      }
      d[u] = src.load(vs[u] >= 0 ? vs[u] : v0);
    }
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      float x[E];
      uint32_t mine = 0;
      if (vs[u] >= 0) {
        src.values(d[u], vs[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (x[e] >= tf && vs[u] * E + e < V && (!Src::kSkipNegInf || x[e] > kNegInf)) mine |= 1u << e;
      }
      insert_flagged<E>(x, mine, vs[u], F, lv, li, &count, lane);
    }
  }
  return TopPair{lv, li};
}

// Per-wave lists whose merge is the block's top F of [v0, v1).  KEEP > 0:
// every thread remembers its KEEP best vectors, so that pass 2 reads again
// only the vectors that can hold a top-F value (each 16-byte re-read costs a
// whole memory line); the bookkeeping costs pass 1 a few operations per
// vector, which pays where pass 2 would re-read a large share of the range.
template <int NT, int E, bool MAY_HOLD = true, int KEEP = 0, class Src>
__device__ TopPair wave_topk_scan(const Src src, int64_t v0, int64_t v1, int V, int F) {
  return block_topk_scan<NT, E, MAY_HOLD, KEEP>(src, v0, v1, V, F);
}

}  // namespace sv
