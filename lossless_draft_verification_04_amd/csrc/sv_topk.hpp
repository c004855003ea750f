// sv_topk.hpp -- a block's top-F values of a range of 16-byte vectors
// (value descending, index ascending), shared by the fan-out, the SpecBranch
// fork and the PRESTO expansion.
//
// Lists live in registers, one entry per lane (lane i = i-th best).  The scan
// (block_topk) takes two passes: every thread first keeps only its best
// vector; groups of threads bound the block's F-th best value from below;
// only the threads whose best reaches the bound are looked at again (from
// registers, mostly), their values at or above it are listed in LDS, and
// the list is ranked (by one wave, or by the block when it is long).
// Entries compare as one 64-bit key (top_key).  Lists from other blocks are
// merged by rounds of a wave-wide selection (wave_merge_entries).
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

// A value source for the scan below provides
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

// Order key of an entry (value descending, index ascending) as one unsigned
// 64-bit compare, larger = better: the value's bits map to unsigned integers
// in the value order (-0 keyed as +0, so equal values tie), and the index is
// complemented (a lower index keys higher; kNoIdx keys below every element
// index).  Key 0 is below every entry and stands for "none".
__device__ __forceinline__ uint64_t top_key(float v, int32_t i) {
  const uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(~(uint32_t)i);
}
__device__ __forceinline__ int32_t key_index(uint64_t k) { return (int32_t)~(uint32_t)k; }
__device__ __forceinline__ uint64_t readlane_u64(uint64_t k, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// k <- the larger of itself and the key DPP pattern CTRL brings in.
template <int CTRL, int ROWS>
__device__ __forceinline__ void key_max_step(uint64_t& k) {
  const int32_t lo = (int32_t)(uint32_t)k;
  const int32_t hi = (int32_t)(uint32_t)(k >> 32);
  const uint64_t o = ((uint64_t)(uint32_t)dpp_i<CTRL, ROWS>(hi, hi) << 32) | (uint32_t)dpp_i<CTRL, ROWS>(lo, lo);
  k = o > k ? o : k;
}
// Candidate entries a block collects for its final selection (LDS).
constexpr int kCand = 512;

// A listed candidate: the value's bits (low word) and its index (high word).
__device__ __forceinline__ uint64_t pack_cand(float v, int32_t i) {
  return ((uint64_t)(uint32_t)i << 32) | __float_as_uint(v);
}
__device__ __forceinline__ float cand_value(uint64_t c) { return __uint_as_float((uint32_t)c); }
__device__ __forceinline__ uint64_t cand_key(uint64_t c) { return top_key(cand_value(c), (int32_t)(c >> 32)); }

// The F best of n <= 64 candidates (cand in LDS) as the wave's list: lane l
// <- the l-th best, empty entries past the n-th.  Every candidate counts the
// candidates with a larger key (its rank) and moves to the lane of that rank.
__device__ __forceinline__ void wave_rank(const uint64_t* cand, int n, int F, int lane, float& lv, int32_t& li) {
  lv = kNegInf;
  li = kNoIdx;
  const uint64_t c = lane < n ? cand[lane] : 0ull;
  const uint64_t k = lane < n ? cand_key(c) : 0ull;
  int above = 0;
  for (int j = 0; j < n; ++j) above += readlane_u64(k, j) > k ? 1 : 0;
  const int rank = lane < n ? above : lane;
  // the ranks are a permutation of the lanes: a forward permute puts every
  // candidate in the lane of its rank
  const int to = rank * 4;
  const uint32_t klo = (uint32_t)__builtin_amdgcn_ds_permute(to, (int)(uint32_t)k);
  const uint32_t khi = (uint32_t)__builtin_amdgcn_ds_permute(to, (int)(uint32_t)(k >> 32));
  const float pv = __int_as_float(__builtin_amdgcn_ds_permute(to, (int)(uint32_t)c));
  if (lane < n && lane < F) {
    lv = pv;
    li = key_index(((uint64_t)khi << 32) | klo);
  }
}

// The F best of n <= kCand candidates (cand in LDS), by the whole block
// (every thread calls it): the thread holding candidate i counts the keys
// above its own over all n (LDS broadcast reads), and the candidates ranked
// below F land in out[rank].  Returns the F-th best key (0 when n < F).
template <int NT>
__device__ __forceinline__ uint64_t block_select(const uint64_t* cand, uint64_t* keys, uint64_t* out, int n, int F,
                                                 uint64_t* s_kth) {
  for (int i = threadIdx.x; i < n; i += NT) keys[i] = cand_key(cand[i]);
  if (threadIdx.x == 0) *s_kth = 0ull;
  lds_sync();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint64_t k = keys[i];
    int above = 0;
    for (int j = 0; j < n; ++j) above += keys[j] > k ? 1 : 0;
    if (above < F) out[above] = cand[i];
    if (above == F - 1) *s_kth = k;
  }
  lds_sync();
  return *s_kth;
}

// Flag the values of vector vs (vs < 0: none; d its data) whose keys reach
// tau and append them to the candidate list (every append is counted; past
// kCand only the count grows).  Branch-free per value: a value's key is its
// order bits (-0 as +0) over its complemented index.
template <int E, class Src>
__device__ __forceinline__ void flag_candidates(const Src& src, const typename Src::Data& d, int64_t vs, int V,
                                                uint64_t tau, uint64_t* cand, int* nc) {
  if (vs < 0) return;
  float x[E];
  src.values(d, vs, x);
  const int32_t i0 = (int32_t)(vs * E);
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t b = __float_as_uint(x[e] + 0.f);  // -0 + 0 = +0
    const uint32_t o = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
    const uint64_t key = ((uint64_t)o << 32) | (uint32_t)~(uint32_t)(i0 + e);
    const bool ok = (i0 + e < V) & (!Src::kSkipNegInf | (x[e] > kNegInf)) & (key >= tau);
    mine |= (uint32_t)ok << e;
  }
  if (!mine) return;
  const int pos = atomicAdd(nc, __builtin_popcount(mine));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = pos + __builtin_popcount(mine & ((1u << e) - 1u));
    if (((mine >> e) & 1u) & (p < kCand)) cand[p] = pack_cand(x[e], i0 + e);
  }
}

// The block's top F values of [v0, v1) (F <= 64; every thread of the block
// calls it with the same arguments): wave 0 returns the list (lane l = l-th
// best, value descending, index ascending), the other waves empty entries.
// Block thread t owns the vectors v0 + t + k * NT.
//  Pass 1 streams the range once; each thread keeps only its best vector by
//  largest element (value desc, then vector asc): one max and one compare
//  per vector.  Its "thread key" is the key of that value at the vector's
//  first element index, a bound from above on the key of every element the
//  thread owns.
//  Bound: the block's threads form groups (64 of them for F <= 8, more for
//  larger F); p is the largest value such that at least F groups hold a
//  thread whose best value reaches it, so F distinct elements reach p and
//  every top-F value is at least p (tau = the key of value p at the
//  lowest-keyed index).
//  Pass 2 looks again at the vectors of the threads whose key reaches tau
//  and lists every value whose key reaches tau in LDS.  When every thread
//  owns at most kWin vectors they are all still in registers; otherwise each
//  thread has kept its best vector's data and the largest value of its other
//  vectors, so memory is read again (all the thread's vectors, spread over
//  its wave) only for a thread whose other vectors can reach tau.  The F
//  best listed values are the block's top F (one wave ranks up to 64 of
//  them, the block more).  If more than kCand values are listed (many ties
//  at p), tau rises to the F-th best key among the kept ones (again a bound
//  from below on the top F), and pass 2 is repeated.
// MAY_HOLD = false drops the all-in-registers path (it keeps kWin vectors
// live across the selection).
template <int NT, int E, bool MAY_HOLD = true, class Src>
__device__ __forceinline__ TopPair block_topk(const Src src, int64_t v0, int64_t v1, int V, int F) {
  constexpr int kWin = 4;   // vectors in flight per thread
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  __shared__ uint64_t s_cand[kCand];
  __shared__ uint32_t s_gm[NT];
  __shared__ uint64_t s_key[kCand];
  __shared__ uint64_t s_sel[kWave];
  __shared__ uint64_t s_tau;
  __shared__ int s_nc;
  float lv = kNegInf;
  int32_t li = kNoIdx;
  if (F <= 0) return TopPair{lv, li};
  const int64_t span = v1 - v0;
  const int64_t nk = (span + NT - 1) / NT;  // vectors per thread at most
  const bool held = MAY_HOLD && nk <= kWin;  // block-uniform
  // pass 1: this thread's best vector by its largest element (value desc,
  // then vector offset asc): value bm, offset bo, data bd; and the largest
  // element of its other vectors, mdrop (NaN: none; fmaxf returns the other
  // operand of a NaN)
  float bm = kNegInf;
  int32_t bo = kNoIdx;
  typename Src::Data bd{};
  float mdrop = __builtin_nanf("");
  typename Src::Data d[kWin];
  if (span > 0) {  // block-uniform
    // loads past the range are not issued: a load left in flight at the end
    // of the stream would be waited for after it
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      const int64_t a = v0 + tid + (int64_t)u * NT;
      if (a < v1) d[u] = src.load(a);
    }
    for (int64_t v = v0 + tid; v < v1; v += (int64_t)kWin * NT) {
      typename Src::Data nx[kWin];
      if (!held) {
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
          const int64_t a = v + (int64_t)(kWin + u) * NT;
          if (a < v1) nx[u] = src.load(a);
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
            const int32_t o = (int32_t)(vu - v0);
            const bool t = (bo == kNoIdx) | top_better(vm, o, bm, bo);
            // the value that is not the best from here on
            if (!t | (bo != kNoIdx)) mdrop = fmaxf(mdrop, t ? bm : vm);
            bm = t ? vm : bm;
            bo = t ? o : bo;
            if (t) bd = d[u];
          }
        }
      }
      if (held) break;  // d stays for pass 2
#pragma unroll
      for (int u = 0; u < kWin; ++u) d[u] = nx[u];
    }
  }
  SV_STAMP(0, 2);  // (timeline builds) this thread's pass 1 is done
  SV_STAMP_LAST(0, 9);  // (timeline builds) the last wave's pass 1 is done
  // the upper bound of vector offset o's element keys at value m
  auto vec_key = [&](float m, int32_t o) { return top_key(m, (int32_t)((v0 + o) * E)); };
  const uint64_t tkey = bo == kNoIdx ? 0ull : vec_key(bm, bo);
  // the bound: the largest value p (in its key's upper 16 bits: exact for
  // bf16 values) such that at least F of the block's 64 H thread groups (GS
  // consecutive threads each) hold a thread whose best value is at least p.
  // F distinct elements reach p, so every top-F value is at least p:
  // tau = key(p, lowest-keyed index).  H grows with F (at least 8 groups per
  // listed value, up to one thread per group), so the bound stays close to
  // the F-th best value.  Wave 0 finds p from the groups' maxima, H per
  // lane, by a binary search on the bits.
  constexpr int kMaxH = NT / kWave;
  static_assert(kMaxH >= 1 && kMaxH <= 16 && kMaxH * kWave == NT, "whole waves, at most 16");
  int H = 1;
  while (H < kMaxH && 8 * F > kWave * H) H *= 2;  // block-uniform
  const int GS = NT / (kWave * H);
  {
    uint64_t k = tkey;
    if (GS >= 2) key_max_step<kRowShr + 1, 0xF>(k);
    if (GS >= 4) key_max_step<kRowShr + 2, 0xF>(k);
    if (GS >= 8) key_max_step<kRowShr + 4, 0xF>(k);
    if (GS >= 16) key_max_step<kRowShr + 8, 0xF>(k);
    if ((lane & (GS - 1)) == GS - 1) s_gm[tid / GS] = (uint32_t)(k >> 32);  // 0: the group holds nothing
  }
  if (tid == 0) s_nc = 0;
  lds_sync();
  SV_STAMP(0, 6);  // (timeline builds) the groups' maxima are known
  if (wave == 0) {
    uint32_t p = 0;
    if (H == 1) {  // one group per lane (F <= 8)
      const uint32_t gh = s_gm[lane];
#pragma unroll
      for (int bit = 31; bit >= 16; --bit) {
        const uint32_t c = p | (1u << bit);
        if (__builtin_popcountll(__ballot(gh >= c)) >= F) p = c;
      }
    } else {
      uint32_t gh[kMaxH];
#pragma unroll
      for (int h = 0; h < kMaxH; ++h) gh[h] = h < H ? s_gm[h * kWave + lane] : 0u;
      for (int bit = 31; bit >= 16; --bit) {
        const uint32_t c = p | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int h = 0; h < kMaxH; ++h) cnt += __builtin_popcountll(__ballot(gh[h] >= c));  // empty groups are 0
        if (cnt >= F) p = c;
      }
    }
    if (lane == 0) s_tau = (uint64_t)p << 32;  // the value p at the lowest key of any index
  }
  lds_sync();
  SV_STAMP(0, 7);  // (timeline builds) the bound is known
  uint64_t tau = s_tau;
  int nc;
  for (;;) {  // block-uniform; tau rises on every repetition
    const bool sel = tkey != 0ull && tkey >= tau;
    if (MAY_HOLD && held) {
      // from registers: the selected threads flag their own values
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t vu = v0 + tid + (int64_t)u * NT;
        flag_candidates<E>(src, d[u], sel && vu < v1 ? vu : -1, V, tau, s_cand, &s_nc);
      }
    } else {
      // only the best vector can reach tau unless another one can (its key
      // is at most that of its value at the thread's first element index):
      // the best from registers, else every vector from memory
      const bool full = sel && mdrop == mdrop && top_key(mdrop, (int32_t)((v0 + tid) * E)) >= tau;
      flag_candidates<E>(src, bd, sel && !full ? v0 + bo : -1, V, tau, s_cand, &s_nc);
      // every vector of the wave's threads that may hold a dropped value,
      // spread over the wave's lanes (one vector per lane at a time: rare)
      const uint64_t fm = __ballot(full);
      if (fm) {  // wave-uniform
        const int nkk = (int)nk;
        const int items = __builtin_popcountll(fm) * nkk;
        for (int base = 0; base < items; base += kWave) {
          const int t = base + lane;
          const int j = t < items ? t / nkk : -1;
          // the j-th such lane of the wave
          int sl = 0;
          uint64_t m = fm;
          for (int q = 0; m; ++q) {
            const int bl = __builtin_ctzll(m);
            m &= m - 1;
            sl = j == q ? bl : sl;
          }
          int64_t vs = -1;
          if (j >= 0) {
            const int64_t r = (int64_t)(wave * kWave + sl) + (int64_t)(t - j * nkk) * NT;
            if (r < span) vs = v0 + r;
          }
          typename Src::Data dd;
          if (vs >= 0) dd = src.load(vs);
          flag_candidates<E>(src, dd, vs, V, tau, s_cand, &s_nc);
        }
      }
    }
    SV_STAMP(0, 8);  // (timeline builds) thread 0's wave has listed its values
    SV_STAMP_LAST(0, 10);  // (timeline builds) the last wave has listed its values
    lds_sync();
    nc = s_nc;
    if (nc <= kCand) break;
    // too many listed: raise tau to the F-th best kept key (kCand > F keys
    // are kept, all at or above tau, so it rises)
    tau = block_select<NT>(s_cand, s_key, s_sel, kCand, F, &s_tau);
    if (tid == 0) s_nc = 0;
    lds_sync();
  }
  SV_STAMP(0, 3);  // (timeline builds) the candidates are listed
  if (nc <= kWave) {  // block-uniform
    if (wave == 0) wave_rank(s_cand, nc, F, lane, lv, li);
  } else {
    block_select<NT>(s_cand, s_key, s_sel, nc, F, &s_tau);
    if (wave == 0 && lane < F) {  // nc > 64 >= F: every lane below F has an entry
      lv = cand_value(s_sel[lane]);
      li = (int32_t)(s_sel[lane] >> 32);
    }
  }
  return TopPair{lv, li};
}

}  // namespace sv
