// sv_topk.hpp -- a wave's running top-F list in registers (value
// descending, index ascending), shared by the fan-out and the PRESTO
// expansion.
//
// Each wave keeps its current top-F in registers, one entry per lane (lane
// i = i-th best), and streams its share of a range of 16-byte vectors in
// increasing index order.  The list starts as the top-F of the wave's first
// 64-vector window (F rounds of a wave-wide selection, each a DPP
// reduction).  After that a lane's vector is a candidate only if its largest
// value beats the wave's F-th best so far (values are seen in index order,
// so an equal value can never displace an earlier entry); a candidate lane
// flags its qualifying values, which are read with register lane reads and
// inserted one at a time with a lane shift.  Most vectors cost one max and
// one compare.
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

__device__ __forceinline__ bool top_better(float va, int32_t ia, float vb, int32_t ib) {
  return va > vb || (va == vb && ia < ib);
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

// (v, i) <- the better of itself and the pair DPP pattern CTRL brings in.
template <int CTRL, int ROWS>
__device__ __forceinline__ void best_step(float& v, int32_t& i) {
  const float ov = dpp_f<CTRL, ROWS>(v, v);
  const int32_t oi = dpp_i<CTRL, ROWS>(i, i);
  if (oi != kNoIdx && (i == kNoIdx || top_better(ov, oi, v, i))) {
    v = ov;
    i = oi;
  }
}

// The wave's best pair (value desc, index asc; kNoIdx never wins), in
// every lane: a reduction within rows of 16, then across rows, ending in
// lane 63.
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
  const bool here = top_better(v, i, lv, li) && lane < F;
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

// Merge n sorted-or-not entries (src[0..n), written by other blocks of the
// launch) into the wave's list (lv, li) of F entries: 64 device-scope loads
// at a time, one per lane, then the entries are taken from the lanes in
// turn; an entry that does not beat the current F-th best is skipped.
__device__ __forceinline__ void wave_merge_entries(const TopEntry* src, int n, int F, float& lv, int32_t& li,
                                                   int lane) {
  for (int e0 = 0; e0 < n; e0 += kWave) {
    TopEntry mine;
    mine.val = kNegInf;
    mine.idx = kNoIdx;
    if (e0 + lane < n) mine = get_entry(src + e0 + lane);
    const int cnt = n - e0 < kWave ? n - e0 : kWave;
    for (int i = 0; i < cnt; ++i) {
      const int32_t ti = __builtin_amdgcn_readlane(mine.idx, i);
      if (ti == kNoIdx) continue;
      const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.val), i));
      const float fv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), F - 1));
      const int32_t fi = __builtin_amdgcn_readlane(li, F - 1);
      if (fi != kNoIdx && !top_better(tv, ti, fv, fi)) continue;
      wave_insert(lv, li, tv, ti, F, lane);
    }
  }
}

// Scan vectors [v0, v1) of a value source into the wave's list (lv, li) of
// at most F entries (F <= 64).  Src provides
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

template <int NT, int E, class Src>
__device__ TopPair wave_list_scan(const Src src, int64_t v0, int64_t v1, int V, int F) {
  float lv = kNegInf;
  int32_t li = kNoIdx;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int count = 0;  // entries held (wave-uniform)
  float thr = kNegInf;
  if (F > 0) {
    // each wave walks its own 64-vector windows in increasing order, with
    // the loads of kWin windows in flight at once
    constexpr int kWin = 4;
    const int64_t stride = (int64_t)(NT / kWave) * kWave;
    const int64_t step = stride * kWin;
    int64_t base0 = v0 + (int64_t)wave * kWave;
    typename Src::Data d[kWin];
    if (base0 < v1) {
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t v = base0 + u * stride + lane;
        d[u] = src.load(v < v1 ? v : v1 - 1);  // unconditional (clamped) so the loads overlap
      }
    }
    for (; base0 < v1; base0 += step) {
      // software pipelined: the next kWin windows are in flight while these
      // are scanned (past the end the prefetch is clamped to the last vector)
      typename Src::Data nx[kWin];
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t v = base0 + step + u * stride + lane;
        nx[u] = src.load(v < v1 ? v : v1 - 1);
      }
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t base = base0 + u * stride;
        const int64_t v = base + lane;
        float x[E];
        float vm = kNegInf;
        const bool valid = v < v1;
        if (valid) {
          src.values(d[u], v, x);
          vm = x[0];
#pragma unroll
          for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[e]);
        }
        if (count == 0) {
          // first window of this wave: take its top-F directly, F rounds of a
          // wave-wide (value desc, index asc) selection
          uint32_t taken = 0;
          for (int k = 0; k < F; ++k) {
            float bv = kNegInf;
            int32_t bi = kNoIdx;
            if (valid) {
#pragma unroll
              for (int e = 0; e < E; ++e) {
                const int64_t gi = v * E + e;
                if (!((taken >> e) & 1u) && gi < V && (!Src::kSkipNegInf || x[e] > kNegInf) &&
                    (bi == kNoIdx || x[e] > bv)) {
                  bv = x[e];
                  bi = (int32_t)gi;
                }
              }
            }
            float wv = bv;
            int32_t wi = bi;
            wave_best(wv, wi);
            if (wi == kNoIdx) break;  // the window has fewer than F elements
            if (lane == k) {
              lv = wv;
              li = wi;
            }
            if (bi == wi) taken |= 1u << (wi - (int32_t)(v * E));
            ++count;
          }
          if (count == F) thr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), F - 1));
          continue;
        }
        // later windows: a lane is a candidate only if its largest element
        // beats the F-th best so far; it then flags which of its elements do
        uint32_t mine = 0;
        if (valid && (count < F || vm > thr)) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if ((count < F || x[e] > thr) && v * E + e < V && (!Src::kSkipNegInf || x[e] > kNegInf))
              mine |= 1u << e;
        }
        uint64_t cm = __ballot(mine != 0);
        while (cm) {
          const int src = __builtin_ctzll(cm);
          cm &= cm - 1;
          uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
          while (bits) {
            const int e = __builtin_ctz(bits);
            bits &= bits - 1;
            // register read from one (uniform) lane: no LDS round trip
            float xe = 0.f;
#pragma unroll
            for (int q = 0; q < E; ++q)
              if (q == e) xe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[q]), src));
            if (count < F || xe > thr) {
              wave_insert(lv, li, xe, (int32_t)((base + src) * E + e), F, lane);
              if (count < F) ++count;
              thr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), F - 1));
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kWin; ++u) d[u] = nx[u];
    }
  }
  return TopPair{lv, li};
}

// The block's list of the F best values of [v0, v1) (F <= 64; every wave
// of the block calls it with the same arguments).  Block thread t owns the
// vectors v0 + t + k * NT.
//  Pass 1 streams the range once; each thread keeps only its best element
//  (value desc, then vector asc), about one max and one compare per vector.
//  The block's F best threads by that element are the only threads that can
//  own a top-F value: a value owned by any other thread is beaten by the F
//  selected threads' bests.  So
//  pass 2 re-reads just those threads' vectors (F times the range / NT
//  vectors, mostly still in L2), spread over the waves; each wave lists
//  the values of its share that reach the F-th selected best, inserting
//  each with a lane shift.
// Each wave returns its list (lane l = l-th best); the block's top F is the
// top F of the waves' lists.  (Keeping running top-F lists during the
// stream instead costs an insertion per new record, about F ln(n / F) per
// list, which dominated at F >= 4.)
template <int NT, int E, class Src>
__device__ TopPair block_topk_scan(const Src src, int64_t v0, int64_t v1, int V, int F) {
  constexpr int NW = NT / kWave;
  constexpr int kWin = 4;  // vectors in flight per thread
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  __shared__ float s_m[NT];
  __shared__ int32_t s_mv[NT];
  __shared__ int32_t s_sel[kWave];
  __shared__ int s_nsel;
  __shared__ float s_tf;
  float lv = kNegInf;
  int32_t li = kNoIdx;
  if (F <= 0) return TopPair{lv, li};
  // pass 1: this thread's best element, as (value, vector offset)
  float m = kNegInf;
  int32_t mv = kNoIdx;
  if (v0 < v1) {  // block-uniform
    typename Src::Data d[kWin];
    int64_t v = v0 + tid;
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int64_t a = v + (int64_t)u * NT;
      d[u] = src.load(a < v1 ? a : v1 - 1);  // clamped: every load is issued
    }
    for (; v < v1; v += (int64_t)kWin * NT) {
      typename Src::Data nx[kWin];
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t a = v + (int64_t)(kWin + u) * NT;
        nx[u] = src.load(a < v1 ? a : v1 - 1);
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
          if (has && (mv == kNoIdx || vm > m)) {
            m = vm;
            mv = (int32_t)(vu - v0);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kWin; ++u) d[u] = nx[u];
    }
  }
  s_m[tid] = m;
  s_mv[tid] = mv;
  lds_sync();
  // the F best threads (wave 0: F rounds of a wave-wide selection over the
  // NW entries each lane holds)
  if (wave == 0) {
    float em[NW];
    int32_t ev_i[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      em[w] = s_m[w * kWave + lane];
      ev_i[w] = s_mv[w * kWave + lane];
    }
    uint32_t taken = 0;
    int n = 0;
    float tf = kNegInf;
    for (; n < F; ++n) {
      float bv = kNegInf;
      int32_t bi = kNoIdx;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float ev = em[w];
        const int32_t ei = ev_i[w];
        if (!((taken >> w) & 1u) && ei != kNoIdx && (bi == kNoIdx || top_better(ev, ei, bv, bi))) {
          bv = ev;
          bi = ei;
        }
      }
      float wv = bv;
      int32_t wi = bi;
      wave_best(wv, wi);
      if (wi == kNoIdx) break;  // fewer than F threads hold an element
      const int owner = wi % NT;  // the thread whose vectors hold it
      if (lane == (owner & (kWave - 1))) taken |= 1u << (owner / kWave);
      if (lane == 0) s_sel[n] = owner;
      tf = wv;
    }
    if (lane == 0) {
      s_nsel = n;
      s_tf = n == F ? tf : kNegInf;  // fewer threads than F: every listable value qualifies
    }
  }
  lds_sync();
  // pass 2: the selected threads' vectors, kWin per thread at a time
  const int nsel = s_nsel;
  const float tf = s_tf;
  const int64_t span = v1 - v0;
  const int64_t nk = (span + NT - 1) / NT;  // vectors per thread at most
  const int64_t total = (int64_t)nsel * nk;
  int count = 0;
  for (int64_t base = 0; base < total; base += (int64_t)kWin * NT) {
    typename Src::Data d[kWin];
    int64_t rel[kWin];
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int64_t t = base + (int64_t)u * NT + tid;
      rel[u] = -1;
      if (t < total) {
        const int s = (int)(t / nk);
        const int64_t r = s_sel[s] + (t - (int64_t)s * nk) * NT;
        if (r < span) rel[u] = r;
      }
      d[u] = src.load(v0 + (rel[u] >= 0 ? rel[u] : 0));
    }
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      float x[E];
      uint32_t mine = 0;
      if (rel[u] >= 0) {
        const int64_t vv = v0 + rel[u];
        src.values(d[u], vv, x);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (x[e] >= tf && vv * E + e < V && (!Src::kSkipNegInf || x[e] > kNegInf)) mine |= 1u << e;
      }
      uint64_t cm = __ballot(mine != 0);
      while (cm) {
        const int sl = __builtin_ctzll(cm);
        cm &= cm - 1;
        uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)mine, sl);
        const int64_t vs = v0 + readlane_i64(rel[u], sl);
        while (bits) {
          const int e = __builtin_ctz(bits);
          bits &= bits - 1;
          float xe = 0.f;
#pragma unroll
          for (int q = 0; q < E; ++q)
            if (q == e) xe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[q]), sl));
          const int32_t ie = (int32_t)(vs * E + e);
          const float fv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), F - 1));
          const int32_t fi = __builtin_amdgcn_readlane(li, F - 1);
          if (count < F || top_better(xe, ie, fv, fi)) {
            wave_insert(lv, li, xe, ie, F, lane);
            if (count < F) ++count;
          }
        }
      }
    }
  }
  return TopPair{lv, li};
}

// Per-wave lists whose merge is the block's top F of [v0, v1).
template <int NT, int E, class Src>
__device__ TopPair wave_topk_scan(const Src src, int64_t v0, int64_t v1, int V, int F) {
  return block_topk_scan<NT, E>(src, v0, v1, V, F);
}

}  // namespace sv
