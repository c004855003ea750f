// sv_walk.hpp -- a sequence's draw split over G co-resident blocks.
//
// The final draw of every entry point is an inverse-CDF search in index order
// over one weight row (draft-then-verify page §1 step 5 and §2.1: the
// residual norm(max(0, p - q)) at the first rejection, or p_{gamma+1} when
// every draft is accepted; for trees the residual after the rejected
// siblings).  A row is split into G slices, one per block.  Each block holds
// its slice in registers (up to kSliceTiles tiles of NT 16-byte vectors per
// row; longer slices are re-read from memory on each use), sums its weights,
// and the blocks exchange the slice sums; the block whose slice holds u * S
// searches it.
//
// Exchange: two 64-bit slot words per (sequence, pass parity, block), zero
// when the exchange starts (the tree's first launch zeroes them; the chain
// kernel keeps its slots zero between calls).  After a pass each block stores its value(s)
// with the pass's tag in the low byte (a double with its 8 lowest mantissa
// bits replaced, or a float in the high half) and its first wave polls the G
// slots of the pass until every tag matches: one or two device-scope stores
// per block and no separate arrival counter.  Two pass parities keep a slow
// block's slot from being overwritten while it is still read.  The G blocks
// of a sequence must be resident together (the host sizes G so that the
// whole launch fits on an otherwise idle device); waits are bounded and a
// block that waits too long sets SV_DERR_TIMEOUT and stops waiting, leaving
// that sequence's outputs invalid (a kernel on another stream that holds
// compute units long enough can cause this).
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int kSliceTiles = 4;   // tiles per row a block holds in registers
constexpr int kMaxG = 64;        // blocks (slices) per sequence
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr uint64_t kTagMask = 0xffull;

// Exclusive prefix sums in thread order of N per-thread values (excl) and
// their block totals (out; waves in index order), with one block barrier
// pair for all N.
template <int NT, int N>
__device__ void block_scan_vec(const double* v, double* excl, double* out, int n = N) {
  __shared__ double red[NT / kWave][N];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  double inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) inc[i] = i < n ? wave_incl_scan(v[i]) : 0.0;  // n: entries in use (block-uniform)
  lds_sync();
  if (lane == kWave - 1)
#pragma unroll
    for (int i = 0; i < N; ++i) red[w][i] = inc[i];
  lds_sync();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double before = 0.0, total = 0.0;
#pragma unroll
    for (int k = 0; k < NT / kWave; ++k) {
      if (k < w) before += red[k][i];
      total += red[k][i];
    }
    excl[i] = before + (inc[i] - v[i]);
    out[i] = total;
  }
}

// One block's slice [v0, v1) of a row pair (rowQ null: a single row).
// HELD: the slice spans at most TILES tiles and is kept in registers;
// otherwise it is streamed from memory on each use (separate kernels, so the
// streaming code's registers do not add to the held ones).
template <int DT, int NT, bool HELD, int TILES = kSliceTiles>
struct Slice {
  static constexpr int E = Fmt<DT>::kPerVec;
  static constexpr int kT = HELD ? TILES : 1;
  u32x4 p[kT], q[kT];
  double own[kT];   // this thread's weight sum per tile (last prepare)
  double excl[kT];  // the weight of the tile's earlier threads (last prepare)
  double tot[kT];   // the block's weight sum per tile (last prepare)
  const void* rowP;
  const void* rowQ;
  int64_t v0, v1;
  static constexpr bool held = HELD;

  __device__ __forceinline__ void load(const void* rp, const void* rq, int64_t a, int64_t b) {
    rowP = rp;
    rowQ = rq;
    v0 = a;
    v1 = b > a ? b : a;
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      p[u] = u32x4{0u, 0u, 0u, 0u};
      q[u] = p[u];
    }
    if constexpr (!HELD) return;
    // every tile's loads are issued together, with no branch between them
    // (a branch per tile let the compiler wait for one tile before issuing
    // the next); positions past the slice load its last vector (index 0 for
    // an empty slice), which valid() then ignores
    const int64_t last = v1 > 0 ? v1 - 1 : 0;
    int64_t vc[kT];
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      const int64_t v = v0 + (int64_t)u * NT + threadIdx.x;
      vc[u] = v < v1 ? v : last;
    }
    if (rq) {
#pragma unroll
      for (int u = 0; u < kT; ++u) {
        p[u] = load_vec(rp, vc[u]);
        q[u] = load_vec(rq, vc[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kT; ++u) p[u] = load_vec(rp, vc[u]);
    }
  }

  __device__ __forceinline__ bool valid(int u, int64_t* vi) const {
    const int64_t v = v0 + (int64_t)u * NT + threadIdx.x;
    *vi = v;
    return v < v1;
  }

  // Weight sums of sp over the slice: per thread and per tile, with each
  // tile's exclusive prefix over the threads (kept for a later search with
  // the same sp, so that the search needs no scan), and the block total
  // (fixed order).
  // sp.rowQ must be null, or the row pair the slice holds.
  __device__ __forceinline__ double prepare(const DrawSpec& sp, int V) {
    if constexpr (!HELD) return range_weight_sum<DT, NT>(sp, V, v0, v1);
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      own[u] = 0.0;
      int64_t v;
      if (valid(u, &v)) {
        float w[E];
        draw_weights_from<DT>(sp, V, v, p[u], q[u], w);
#pragma unroll
        for (int e = 0; e < E; ++e) own[u] += (double)w[e];
      }
    }
    // tiles past the slice's end are empty in every thread: not scanned
    const int used = (int)((v1 - v0 + NT - 1) / NT);
    block_scan_vec<NT, kT>(own, excl, tot, used < kT ? used : kT);
    double total = 0.0;
#pragma unroll
    for (int u = 0; u < kT; ++u) total += tot[u];
    return total;
  }

  // The block's weight sum of sp over the slice, as prepare returns it but
  // without the per-tile prefixes a search needs (for passes whose sums are
  // only exchanged; a search needs a prepare with the same sp first).
  __device__ __forceinline__ double total(const DrawSpec& sp, int V) const {
    if constexpr (!HELD) return range_weight_sum<DT, NT>(sp, V, v0, v1);
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      int64_t v;
      if (valid(u, &v)) {
        float w[E];
        draw_weights_from<DT>(sp, V, v, p[u], q[u], w);
#pragma unroll
        for (int e = 0; e < E; ++e) s += (double)w[e];
      }
    }
    return block_sum<NT>(s);
  }

  // (max, sum 2^(z c - c max)) of row P over the slice.
  __device__ __forceinline__ Partial row_stats(float c, int V) const {
    if constexpr (!HELD) return range_stats<DT, NT, 4>(rowP, V, v0, v1, c);
    const float M = max_logit(c, V);
    double s = 0.0;
    if (M != kNegInf) {
      const float cm = c * M;
#pragma unroll
      for (int u = 0; u < kT; ++u) {
        int64_t v;
        if (valid(u, &v)) {
          float x[E];
          unpack<DT>(p[u], x);
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (v * E + e < V) acc += fast_exp2(__builtin_fmaf(x[e], c, -cm));
          s += (double)acc;
        }
      }
    }
    Partial r;
    r.m = M;
    r.pad = 0.f;
    r.s = block_sum<NT>(s);
    return r;
  }

  // Largest logit of row P over the slice (-inf if none).
  __device__ __forceinline__ float max_logit(float c, int V) const {
    if constexpr (!HELD) return range_stats<DT, NT, 4>(rowP, V, v0, v1, c).m;
    float m = kNegInf;
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      int64_t v;
      if (valid(u, &v)) {
        float x[E];
        unpack<DT>(p[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (v * E + e < V) m = fmaxf(m, x[e]);
      }
    }
    return block_fmax<NT>(m);
  }

  // Last element with positive weight in held tile u_sel (every tile if
  // negative) of this thread (-1 if none).
  __device__ __forceinline__ int64_t last_positive(const DrawSpec& sp, int V, int u_sel) const {
    int64_t last = -1;
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      int64_t v;
      if ((u_sel < 0 || u == u_sel) && valid(u, &v)) {
        float w[E];
        draw_weights_from<DT>(sp, V, v, p[u], q[u], w);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (w[e] > 0.f) last = v * E + e;
      }
    }
    return last;
  }

  // Inverse-CDF search over the slice in index order, with the sums of the
  // last prepare (same sp): the first element whose running weight exceeds
  // `target`; if rounding leaves the target beyond the slice's weight, the
  // last positive element (-1 if none).  The same index in every thread.
  __device__ __forceinline__ int64_t search(const DrawSpec& sp, int V, double target) const {
    if constexpr (!HELD) return block_search<DT, NT>(sp, V, v0, v1, target);
    double cum = 0.0, loc = 0.0;
    int pick = -1;
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      if (pick < 0 && cum + tot[u] > target) {
        pick = u;
        loc = target - cum;
      }
      cum += tot[u];
    }
    if (pick < 0) return block_max_i64<NT>(last_positive(sp, V, -1));
    // the picked tile (block-uniform); every tile index stays a constant so
    // the held vectors stay in registers
    int64_t result = -1;
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      if (u == pick) {
        const double t_local = loc - excl[u];
        int64_t found = INT64_MAX;
        int64_t v;
        if (valid(u, &v) && own[u] > 0.0 && t_local >= 0.0 && t_local < own[u]) {
          float w[E];
          draw_weights_from<DT>(sp, V, v, p[u], q[u], w);
          double run = 0.0;
          int64_t last = -1;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            run += (double)w[e];
            if (found == INT64_MAX && run > t_local) found = v * E + e;
            if (w[e] > 0.f) last = v * E + e;
          }
          if (found == INT64_MAX) found = last;
        }
        // the first qualifying thread holds the smallest index (rounding can
        // let neighbouring threads' ranges overlap)
        __shared__ int64_t s_found[NT / kWave];
        const uint64_t q = __ballot(found != INT64_MAX);
        const int64_t wf = q ? readlane_i64(found, __builtin_ctzll(q)) : INT64_MAX;
        lds_sync();
        if ((threadIdx.x & (kWave - 1)) == 0) s_found[threadIdx.x / kWave] = wf;
        lds_sync();
        int64_t r = s_found[0];
#pragma unroll
        for (int w = 1; w < NT / kWave; ++w) r = s_found[w] < r ? s_found[w] : r;
        // rounding left the target past every thread: the tile's last positive element
        result = r != INT64_MAX ? r : block_max_i64<NT>(last_positive(sp, V, u));
      }
    }
    return result;
  }
};

// Exchange state of one block.
struct Exchange {
  uint64_t* slots;  // [2 parities][G][kSlotPad words, 2 used] of this sequence, zero at the start
  int32_t* err;
  int G, g;
  int pass;        // exchanges so far
  bool late;       // a wait ran out: later exchanges do not wait (first wave only)
  bool withhold;   // test switch: this block never publishes
  uint32_t limit;  // polls before a wait gives up
};

// Each block's slot words sit kSlotPad words (64 B) apart, so no two blocks
// store to one 64-byte span: with 16-byte slots, 8 blocks' stores and every
// block's polls met in one cache line, which measured 0.25-0.5 us slower per
// exchange of 16-64 blocks.
constexpr int kSlotPad = 8;
constexpr int kSlotWords = 2 * kSlotPad;  // slot words per block of a launch (2 parities)

// Workspace header words read by the waits (word 0 is the error word):
// [1] the number of polls after which a wait gives up (0: kSpinLimit);
// [2] nonzero: the last block of sequence 0 never publishes, so that its
//     partners' waits run out -- a switch for tests of the bounded waits
//     (every kernel still exits).  knobs may be null (the defaults).
constexpr int kKnobSpin = 1;
constexpr int kKnobWithhold = 2;

__device__ __forceinline__ Exchange make_exchange(void* slots, int32_t* err, const uint32_t* knobs, int b, int G,
                                                  int g) {
  Exchange x;
  x.slots = static_cast<uint64_t*>(slots) + (int64_t)b * kSlotWords * G;
  x.err = err;
  x.G = G;
  x.g = g;
  x.pass = 0;
  x.late = false;
  const uint32_t spin = knobs ? knobs[kKnobSpin] : 0u;
  x.limit = spin ? spin : kSpinLimit;
  x.withhold = knobs && knobs[kKnobWithhold] != 0u && b == 0 && G > 1 && g == G - 1;
  return x;
}

__device__ __forceinline__ uint64_t pack_sum(double v) {
  return (uint64_t)__double_as_longlong(v > 0.0 ? v : 0.0) & ~kTagMask;
}
__device__ __forceinline__ double unpack_sum(uint64_t w) { return __longlong_as_double((long long)(w & ~kTagMask)); }
__device__ __forceinline__ uint64_t pack_max(float m) { return (uint64_t)__float_as_uint(m) << 32; }
__device__ __forceinline__ float unpack_max(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }

// Publish this block's payload(s) (low byte zero; NW = 1 or 2 words) for the
// current pass and wait for the G blocks' payloads of the pass, left
// (without tags) in s_w0[0..G) (and s_w1[0..G)).
template <int NW>
__device__ __forceinline__ void exchange_n(Exchange& x, uint64_t p0, uint64_t p1, uint64_t* s_w0, uint64_t* s_w1) {
  const uint64_t tag = (uint64_t)(x.pass % 254) + 1;
  lds_sync();  // every wave is done with the previous exchange's words
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    uint64_t* set = x.slots + (int64_t)(x.pass & 1) * kSlotPad * x.G;
    uint64_t w0 = p0, w1 = p1;
    bool ok = (l >= x.G) || (l == x.g);
    if (x.G > 1) {
      if (l == x.g && !x.withhold) {
        st_dev(set + kSlotPad * l, p0 | tag);
        if (NW == 2) st_dev(set + kSlotPad * l + 1, p1 | tag);
      }
      uint32_t spins = 0;
      for (;;) {
        if (!ok) {
          w0 = ld_dev(set + kSlotPad * l);
          if (NW == 2) w1 = ld_dev(set + kSlotPad * l + 1);
          ok = (w0 & kTagMask) == tag && (NW == 1 || (w1 & kTagMask) == tag);
        }
        if (__all(ok) || x.late) break;
        if (++spins > x.limit) {
          if (l == 0) set_error(x.err, SV_DERR_TIMEOUT);
          x.late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (l < x.G) {
      s_w0[l] = w0 & ~kTagMask;
      if (NW == 2) s_w1[l] = w1 & ~kTagMask;
    }
  }
  lds_sync();
  ++x.pass;
}

__device__ __forceinline__ void exchange(Exchange& x, uint64_t payload, uint64_t* s_words) {
  exchange_n<1>(x, payload, 0ull, s_words, nullptr);
}

// Slice values of the last exchange as every wave holds them: lane l < G
// has slice l's value v and the inclusive prefix inc over slices 0..l (the
// same in every wave, so every thread takes the same decisions).
struct SliceSums {
  double v, inc;
};

// Scan of the lanes' slice values; returns the total.
__device__ __forceinline__ double scan_slices(double v, int G, SliceSums* ss) {
  ss->v = v;
  ss->inc = wave_incl_scan(v);
  return readlane_d(ss->inc, G - 1);
}

// The slice holding `target` (0 <= target < total) and the offset into
// it; rounding past the end picks the end of the last slice with positive
// weight.
__device__ __forceinline__ void pick_slice(const SliceSums& ss, int G, double target, int* pick, double* loc) {
  const int l = threadIdx.x & (kWave - 1);
  const uint64_t over = __ballot(l < G && ss.inc > target);
  if (over) {
    const int p = __builtin_ctzll(over);
    *pick = p;
    *loc = target - (readlane_d(ss.inc, p) - readlane_d(ss.v, p));
  } else {
    const uint64_t pos = __ballot(l < G && ss.v > 0.0);
    const int p = pos ? 63 - __builtin_clzll(pos) : 0;
    *pick = p;
    *loc = readlane_d(ss.v, p);  // its end
  }
}

// Exchange slice sums: every thread gets the total, and ss the scan for a
// later pick_slice.
__device__ __forceinline__ double exchange_sum(Exchange& x, double mine, uint64_t* s_words, SliceSums* ss) {
  exchange(x, pack_sum(mine), s_words);
  const int l = threadIdx.x & (kWave - 1);
  return scan_slices(l < x.G ? unpack_sum(s_words[l]) : 0.0, x.G, ss);
}

// Exchange slice maxima: every thread gets the maximum.
__device__ __forceinline__ float exchange_max(Exchange& x, float mine, uint64_t* s_words) {
  exchange(x, pack_max(mine), s_words);
  const int l = threadIdx.x & (kWave - 1);
  float m = l < x.G ? unpack_max(s_words[l]) : kNegInf;
  return wave_fmax(m);
}

// Exchange slice statistics (max m_l, sum s_l of 2^(z c - c m_l)): every
// thread gets the row maximum M and the total of the slice weights
// s_l 2^(c m_l - c M), and ss their scan for a later pick_slice.
__device__ __forceinline__ double exchange_stats(Exchange& x, const Partial& mine, float c, uint64_t* s_w0,
                                                 uint64_t* s_w1, SliceSums* ss, float* M_out) {
  exchange_n<2>(x, pack_max(mine.m), pack_sum(mine.s), s_w0, s_w1);
  const int l = threadIdx.x & (kWave - 1);
  const float m = l < x.G ? unpack_max(s_w0[l]) : kNegInf;
  const float M = wave_fmax(m);
  *M_out = M;
  const double v =
      (l >= x.G || m == kNegInf || M == kNegInf) ? 0.0 : unpack_sum(s_w1[l]) * exp2_d((double)(c * m) - (double)(c * M));
  return scan_slices(v, x.G, ss);
}

// Zero n slot words, spread over the blocks of a launch that precedes the
// exchanges (one word per thread).
__device__ __forceinline__ void zero_slots(void* slots, int64_t n, int64_t block, int nt) {
  const int64_t i = block * nt + threadIdx.x;
  if (i < n) static_cast<uint64_t*>(slots)[i] = 0ull;
}

}  // namespace sv
