// sv_chain_small.hip -- chain verification for small calls: every row held.
//
// The step of sv_chain.hip (draft-then-verify page §1 steps 3-5 and §2.1:
// accept with min(1, p/q), residual norm(max(0, p - q)), bonus row
// p_{gamma+1}; in PM mode the point-mass reading of the SpecDiff-2 page's
// Core method), for calls small enough that each of a sequence's G blocks
// holds its slice of every row the step may touch in registers: target rows
// 1..gamma+1 (the bonus row included) and draft rows 1..gamma.  One launch
// then needs two rounds between blocks and reads no row twice:
//  1. each block loads its slice of every row and reduces it to a part
//     (max, sum 2^(z c - c max)) per row; the parts are exchanged;
//  2. every block merges the parts, gathers p and q at the drafted tokens,
//     decides (the same decisions in every block), weights its held slice of
//     the draw row(s) -- residual p_{n+1} - q_{n+1}, p_{n+1} without the
//     rejected token, or the bonus row under its merged statistics -- and the
//     slice sums are exchanged; the block whose slice holds u * S searches.
// Every wait is bounded.  The last block of a sequence to finish with the
// exchange slots clears them and its exit counter; both live in the
// workspace's counter region, so both are zero when the next call starts.
#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_walk.hpp"

namespace sv {

constexpr int kSNT = 256;
constexpr int kSmallW = 2 * kSmallRows;  // words a block publishes in the first round

// Row r of sequence b among the held rows: target rows j = 0..gamma (r = j),
// then draft rows j = 0..gamma-1 (r = gamma + 1 + j).
template <int DT>
__device__ __forceinline__ const void* small_row(const ChainParams& a, int b, int r) {
  const bool t = r <= a.gamma;  // a select, not a branch
  const char* base = static_cast<const char*>(t ? a.tgt : a.drf);
  const int64_t row = t ? (int64_t)b * (a.gamma + 1) + r : (int64_t)b * a.gamma + (r - a.gamma - 1);
  return base + row * (t ? a.tgt_sb : a.drf_sb);
}

// Slot words of sequence b: G x kSmallW words of the first round, then the
// second round's exchange (two parities x G x 2 words).
__device__ __forceinline__ uint64_t* small_slots(const ChainParams& a, int b) {
  return static_cast<uint64_t*>(a.slots) + (int64_t)b * a.G * (kSmallW + kSlotWords);
}

// A block is done with the sequence's slots: every read of them is behind
// it, and every store to them came from wave 0.  Thread 0 counts the exit
// once those stores are complete and keeps the old count; small_exit_end
// (wave 0, any time later) lets the last block of the sequence clear the
// slots and the counter for the next call.  Between the two the counting
// atomic is in flight, so its latency overlaps whatever the block does next.
__device__ __forceinline__ uint32_t small_exit_begin(const ChainParams& a, int b) {
  uint32_t old = 0;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    old = __hip_atomic_fetch_add(a.cnt + (int64_t)b * a.cstride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return old;
}
__device__ __forceinline__ void small_exit_end(const ChainParams& a, int b, uint32_t old) {
  if (threadIdx.x >= kWave) return;
  if ((uint32_t)__builtin_amdgcn_readlane((int)old, 0) != (uint32_t)a.G - 1u) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.cnt + (int64_t)b * a.cstride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t* w = small_slots(a, b);
  for (int i = threadIdx.x; i < a.G * (kSmallW + kSlotWords); i += kWave) st_dev(w + i, 0ull);
}

// Elements n.. of a held vector become -inf (the vector holds fewer than
// E logits of the slice).
template <int DT>
__device__ __forceinline__ u32x4 mask_from(u32x4 v, int n) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == SV_BF16) {
      if (2 * i >= n) v[i] = (v[i] & 0xffff0000u) | 0xff80u;
      if (2 * i + 1 >= n) v[i] = (v[i] & 0x0000ffffu) | 0xff800000u;
    } else {
      if (i >= n) v[i] = 0xff800000u;
    }
  }
  return v;
}

template <int DT, bool PM, int TILES>
__global__ __launch_bounds__(kSNT) void chain_small_kernel(ChainParams a) {
  constexpr int E = Fmt<DT>::kPerVec;
  constexpr int kW = kSNT / kWave;
  const int b = blockIdx.x / a.G;
  const int g = blockIdx.x - b * a.G;
  const int R = PM ? a.gamma + 1 : 2 * a.gamma + 1;  // rows held
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // B * nvec is small on this path: 32-bit vector indices and byte offsets
  const int nvec = (int)a.nvec;
  const int spv = (nvec + a.G - 1) / a.G;
  const int v0 = g * spv < nvec ? g * spv : nvec;
  const int v1 = v0 + spv < nvec ? v0 + spv : nvec;
  SV_STAMP_START(0);
  SV_STAMP_TAG(0, 3, b);
  uint64_t* words1 = small_slots(a, b);
  Exchange x = make_exchange(a.slots, a.err, a.knobs, b, a.G, g);
  x.slots = words1 + (int64_t)a.G * kSmallW;

  // (every wave, lane j) the drafted token of position j + 1
  int32_t xt = -1;
  if (lane < a.gamma) xt = a.tok[(int64_t)b * a.gamma + lane];
  // every tile of every held row at once, through buffer resources: rows
  // past R have an empty range and vectors past the row read zeros, without
  // a memory access or a branch
  u32x4 d[kSmallRows][TILES];
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) {
    const __amdgpu_buffer_rsrc_t rs = range_rsrc(small_row<DT>(a, b, r < R ? r : 0), r < R ? (uint32_t)nvec * 16u : 0u);
#pragma unroll
    for (int u = 0; u < TILES; ++u) d[r][u] = load_range(rs, (uint32_t)(v0 + u * kSNT + (int)threadIdx.x) * 16u);
  }
  // the uniforms depend on nothing loaded: computed while the loads fly
  double rr = 1.0;
  if (lane < a.gamma) rr = uniform24(a.seed, (uint32_t)(lane + 1), (uint32_t)b, 0, a.round, 0);
  const double us = uniform24(a.seed, 0, (uint32_t)b, 0, a.round, 1);
  // (every wave, lane j) the drafted token's logits in target and draft row
  // j: waiting for the token (the oldest load) leaves the tiles in flight
  float zp = 0.f, zq = 0.f;
  if (lane < a.gamma) {
    const int64_t xc = (xt >= 0 && xt < a.V) ? xt : 0;
    zp = load_elem<DT>(small_row<DT>(a, b, lane), xc);
    if (!PM) zq = load_elem<DT>(small_row<DT>(a, b, a.gamma + 1 + lane), xc);
  }
  // the slice's ragged end: vectors past the slice, and logits past V, become -inf
#pragma unroll
  for (int u = 0; u < TILES; ++u) {
    const int vi = v0 + u * kSNT + (int)threadIdx.x;
    const int nval = vi < v1 ? (a.V - vi * E < E ? a.V - vi * E : E) : 0;
    if (nval < E)
#pragma unroll
      for (int r = 0; r < kSmallRows; ++r) d[r][u] = mask_from<DT>(d[r][u], nval);
  }

  // each row's part over the block's slice: per thread (max, sum under it),
  // per wave (all rows' reductions side by side; the wave's 64 sums in fp32,
  // a 6-level tree), then over the waves in fp64
  float mt[kSmallRows], mw[kSmallRows], st[kSmallRows];
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) {
    float z[TILES * E];
#pragma unroll
    for (int u = 0; u < TILES; ++u) unpack<DT>(d[r][u], z + u * E);
    float m = z[0];
#pragma unroll
    for (int e = 1; e < TILES * E; ++e) m = fmaxf(m, z[e]);
    const float cm = m == kNegInf ? 0.f : a.c * m;
    float t[TILES * E];
#pragma unroll
    for (int e = 0; e < TILES * E; ++e) t[e] = fast_exp2(__builtin_fmaf(z[e], a.c, -cm));
#pragma unroll
    for (int w = TILES * E / 2; w > 0; w >>= 1)
#pragma unroll
      for (int e = 0; e < w; ++e) t[e] += t[e + w];
    mt[r] = r < R ? m : kNegInf;
    st[r] = r < R ? t[0] : 0.f;
    mw[r] = mt[r];
  }
  rows_fmax_all(mw);
  SV_STAMP(0, 1);
  float sw[kSmallRows];
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) sw[r] = mt[r] == kNegInf ? 0.f : st[r] * fast_exp2(a.c * mt[r] - a.c * mw[r]);
  rows_fsum_all(sw);
  __shared__ float s_wm[kW][kSmallRows];
  __shared__ float s_ws[kW][kSmallRows];
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < kSmallRows; ++r) {
      s_wm[wave][r] = mw[r];
      s_ws[wave][r] = sw[r];
    }
  lds_sync();
  SV_STAMP(0, 2);

  // the first round: thread r publishes row r's part as two tagged words
  const uint64_t tag1 = 1;
  if (threadIdx.x < (unsigned)R) {
    const int r = threadIdx.x;
    float M = s_wm[0][r];
#pragma unroll
    for (int w = 1; w < kW; ++w) M = fmaxf(M, s_wm[w][r]);
    double S = 0.0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float m = s_wm[w][r];
      if (m != kNegInf) S += (double)s_ws[w][r] * (double)fast_exp2(a.c * m - a.c * M);
    }
    if (!x.withhold) {
      st_dev(words1 + (int64_t)g * kSmallW + 2 * r, pack_max(M) | tag1);
      st_dev(words1 + (int64_t)g * kSmallW + 2 * r + 1, pack_sum(S) | tag1);
    }
  }
  SV_STAMP(0, 3);
  // the waves share the wait and the merge: wave w takes rows w, w + 4,
  // w + 8 (those below R); lane q < G polls block q's two words of each
  constexpr int kRW = (kSmallRows + kW - 1) / kW;
  uint64_t wm[kRW], ws[kRW];
#pragma unroll
  for (int k = 0; k < kRW; ++k) wm[k] = ws[k] = 0ull;
  bool have = lane >= a.G;
  bool late = false;
  {
    const uint64_t* mine = words1 + (int64_t)lane * kSmallW;
    uint32_t spins = 0;
    for (;;) {
      if (!have) {
#pragma unroll
        for (int k = 0; k < kRW; ++k) {
          const int r = wave + kW * k < R ? wave + kW * k : 0;
          wm[k] = ld_dev(mine + 2 * r);
          ws[k] = ld_dev(mine + 2 * r + 1);
        }
        bool all = true;
#pragma unroll
        for (int k = 0; k < kRW; ++k)
          all &= wave + kW * k >= R || ((wm[k] & kTagMask) == tag1 && (ws[k] & kTagMask) == tag1);
        have = all;
      }
      if (__all(have)) break;
      if (++spins > x.limit) {
        late = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // merged statistics of the wave's rows: one all-lane reduction per row
  __shared__ float s_cm[kSmallRows];
  __shared__ double s_S[kSmallRows];
  __shared__ int s_late[kW];
  {
    float mq[kRW], M[kRW];
    double sq[kRW];
#pragma unroll
    for (int k = 0; k < kRW; ++k) {
      mq[k] = (lane < a.G && wave + kW * k < R) ? unpack_max(wm[k]) : kNegInf;
      M[k] = mq[k];
    }
    rows_fmax_all(M);
#pragma unroll
    for (int k = 0; k < kRW; ++k)
      sq[k] = (mq[k] == kNegInf || M[k] == kNegInf) ? 0.0 : unpack_sum(ws[k]) * (double)fast_exp2(a.c * mq[k] - a.c * M[k]);
    rows_sum_all(sq);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kRW; ++k) {
        const int r = wave + kW * k;
        if (r < R) {
          s_cm[r] = M[k] == kNegInf ? 0.f : a.c * M[k];
          s_S[r] = M[k] == kNegInf ? 0.0 : sq[k];
        }
      }
      s_late[wave] = late;
      if (late) set_error(a.err, SV_DERR_TIMEOUT);
    }
  }
  lds_sync();
  SV_STAMP(0, 4);
  bool any_late = false;
#pragma unroll
  for (int w = 0; w < kW; ++w) any_late |= s_late[w] != 0;
  if (any_late) {
    small_exit_end(a, b, small_exit_begin(a, b));
    return;
  }

  // decisions (every wave, lane j: position j + 1), the same in every block
  double p = 0.0, q = PM ? 1.0 : 0.0;
  bool acc = false;
  if (lane < a.gamma) {
    const int j = lane;
    RowStat P, Q;
    P.pad = Q.pad = 0.f;
    P.cm = s_cm[j];
    P.S = s_S[j];
    Q.cm = PM ? 0.f : s_cm[a.gamma + 1 + j];
    Q.S = PM ? 1.0 : s_S[a.gamma + 1 + j];
    if (xt >= 0 && xt < a.V) {
      p = prob_of(zp, a.c, P);
      if (!PM) q = prob_of(zq, a.c, Q);
    } else if (g == 0 && wave == 0) {
      set_error(a.err, SV_DERR_TOKEN);
    }
    if (g == 0 && wave == 0 && (!(P.S > 0.0) || !(Q.S > 0.0))) set_error(a.err, SV_DERR_ROW);
    acc = rr < accept_ratio(p, q);
  }
  const uint64_t rejected = ~(uint64_t)__ballot(acc);
  int n = rejected ? __builtin_ctzll(rejected) : kWave;
  if (n > a.gamma) n = a.gamma;
  __shared__ int32_t s_ex;  // the rejected token (n < gamma), for the point-mass draw
  const int32_t xn = __builtin_amdgcn_readlane(xt, n < a.gamma ? n : 0);
  if (threadIdx.x == 0) s_ex = (n < a.gamma && xn >= 0 && xn < a.V) ? xn : -1;

  SV_STAMP(0, 5);
  // the draw: target row n (the bonus row when n = gamma), with draft row n
  // for a residual
  const int rP = n;
  const int rQ = a.gamma + 1 + n;
  const float cmP = s_cm[rP];
  const double SP = s_S[rP];
  const bool twin = !PM && n < a.gamma;  // draft row n is held (rQ < R)
  const float cmQ = twin ? s_cm[rQ] : 0.f;
  const double SQ = twin ? s_S[rQ] : 0.0;
  const bool rows_ok = SP > 0.0 && (PM || n == a.gamma || SQ > 0.0);
  const bool resid = !PM && n < a.gamma && rows_ok;
  const bool pm_resid = PM && n < a.gamma && SP > 0.0;
  Slice<DT, kSNT, true, TILES> sl;
  sl.rowP = small_row<DT>(a, b, rP);
  sl.rowQ = resid ? small_row<DT>(a, b, rQ) : nullptr;
  sl.v0 = v0;
  sl.v1 = v1 > v0 ? v1 : v0;
#pragma unroll
  for (int u = 0; u < TILES; ++u) {
    sl.p[u] = u32x4{0u, 0u, 0u, 0u};
    sl.q[u] = sl.p[u];
  }
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r)
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
      if (r == rP) sl.p[u] = d[r][u];
      if (!PM && r == rQ) sl.q[u] = d[r][u];
    }
  DrawSpec sp;
  sp.rowP = sl.rowP;
  sp.rowQ = nullptr;
  sp.c = a.c;
  sp.coef = 1.f;
  sp.ex = nullptr;
  sp.nex = 0;
  sp.cmP = cmP;
  sp.invSP = 1.f;
  sp.cmQ = 0.f;
  sp.invSQ = 1.f;
  __shared__ uint64_t s_words[kMaxG];
  SliceSums ss;
  double total;
  lds_sync();  // s_ex is set
  if (resid) {
    sp.rowQ = sl.rowQ;
    sp.invSP = (float)(1.0 / SP);
    sp.cmQ = cmQ;
    sp.invSQ = (float)(1.0 / SQ);
    total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    if (!(total > 0.0)) {
      // residual mass rounded to 0: draw from p_{n+1} itself
      sp.rowQ = nullptr;
      total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    }
  } else if (pm_resid) {
    // p_{n+1} without the rejected token, under the row's own shift
    sp.ex = &s_ex;
    sp.nex = s_ex >= 0 ? 1 : 0;
    total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    if (!(total > 0.0)) {
      sp.nex = 0;
      total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
    }
  } else {
    // bonus draw, or a row without mass: a plain draw under the row's shift
    if (g == 0 && threadIdx.x == 0 && !(SP > 0.0)) set_error(a.err, SV_DERR_ROW);
    total = exchange_sum(x, sl.prepare(sp, a.V), s_words, &ss);
  }
  SV_STAMP(0, 6);
  int pick;
  double loc;
  pick_slice(ss, x.G, us * total, &pick, &loc);
  const uint32_t exits = small_exit_begin(a, b);  // the slots are read no more
  // a block other than the searching one stores the per-position outputs
  if (g == (x.G > 1 && pick == 0 ? 1 : 0) && wave == 0) {
    if (lane < a.gamma) {
      const int64_t o = (int64_t)b * a.gamma + lane;
      if (a.out_p) a.out_p[o] = (float)p;
      if (!PM && a.out_q) a.out_q[o] = (float)q;
    }
    if (lane == 0) a.out_n[b] = n;
  }
  if (pick == g) {
    const int64_t t = sl.search(sp, a.V, loc);
    if (threadIdx.x == 0) a.out_tok[b] = (int32_t)t;
  }
  small_exit_end(a, b, exits);
  SV_STAMP(0, 7);
  SV_STAMP_FLUSH(0);
}

SV_TIMELINE_SETTER(timeline_set_chain_small)

template <int TILES>
static hipError_t launch_small_tiles(const ChainParams& p, sv_dtype dt, hipStream_t s) {
  const dim3 grid((unsigned)p.B * p.G), block(kSNT);
  if (dt == SV_BF16) {
    if (p.pm)
      chain_small_kernel<SV_BF16, true, TILES><<<grid, block, 0, s>>>(p);
    else
      chain_small_kernel<SV_BF16, false, TILES><<<grid, block, 0, s>>>(p);
  } else {
    if (p.pm)
      chain_small_kernel<SV_F32, true, TILES><<<grid, block, 0, s>>>(p);
    else
      chain_small_kernel<SV_F32, false, TILES><<<grid, block, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_chain_small(const ChainParams& p, sv_dtype dt, int tiles, hipStream_t s) {
  return tiles == 1 ? launch_small_tiles<1>(p, dt, s) : launch_small_tiles<kSmallTiles>(p, dt, s);
}

template <int TILES>
static const void* small_kernel_fn(sv_dtype dt, bool pm) {
  if (dt == SV_BF16)
    return pm ? reinterpret_cast<const void*>(&chain_small_kernel<SV_BF16, true, TILES>)
              : reinterpret_cast<const void*>(&chain_small_kernel<SV_BF16, false, TILES>);
  return pm ? reinterpret_cast<const void*>(&chain_small_kernel<SV_F32, true, TILES>)
            : reinterpret_cast<const void*>(&chain_small_kernel<SV_F32, false, TILES>);
}

// Blocks of the small-chain kernel the device holds at once.
int chain_small_capacity(sv_dtype dt, bool pm, int tiles) {
  static int cache[2][2][2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& c = cache[tiles == 1][dt == SV_BF16][pm][dev];
  if (c == 0)
    c = device_capacity(tiles == 1 ? small_kernel_fn<1>(dt, pm) : small_kernel_fn<kSmallTiles>(dt, pm), kSNT, dev);
  return c;
}

}  // namespace sv
