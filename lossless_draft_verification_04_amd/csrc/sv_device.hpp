// sv_device.hpp -- device-side building blocks of the gfx950 verification
// kernels: Philox uniforms, 16-byte row loads, wave/block reductions and
// scans, online row statistics and the block-wide inverse-CDF search.
//
// Internal to libspecverify; shares nothing with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// ---------------------------------------------------------------------------
// Timeline builds (-DSV_TIMELINE, libspecverify_timeline.so): thread 0 of a
// block keeps the 100 MHz wall clock (s_memrealtime) of each phase end in slot
// k of the block's 16-slot record, written at the block's end to record
// base + blockIdx.x of a buffer the host registers (sv_timeline_set).  Slot 15
// holds a tag: role | seq << 8 | XCD << 40.  In the normal build the stamps
// compile to nothing.
// ---------------------------------------------------------------------------
constexpr int kTimelineSlots = 16;
#ifdef SV_TIMELINE
static __device__ uint64_t* g_timeline;
static __device__ uint64_t g_timeline_records;  // records the buffer holds
// A block's stamps wait in LDS and go to memory once, at the block's end
// (SV_STAMP_FLUSH): a global store in the middle of a kernel would be waited
// for by the next wait on a load (this chip counts stores and loads together).
__device__ __forceinline__ uint64_t* timeline_lds() {
  __shared__ uint64_t s_tl[kTimelineSlots];
  return s_tl;
}
__device__ __forceinline__ void timeline_put(int k, uint64_t v) {
  if (threadIdx.x == 0) timeline_lds()[k] = v;
}
// Slot k <- the latest of the values the block's waves put there.
__device__ __forceinline__ void timeline_last(int k, uint64_t v) {
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned long long*>(&timeline_lds()[k]), (unsigned long long)v);
}
__device__ __forceinline__ void timeline_flush(uint64_t base) {
  const uint64_t r = base + blockIdx.x;
  if (threadIdx.x == 0 && g_timeline && r < g_timeline_records)
    for (int k = 0; k < kTimelineSlots; ++k) g_timeline[r * kTimelineSlots + k] = timeline_lds()[k];
}
__device__ __forceinline__ void timeline_clear() {
  if (threadIdx.x == 0)
    for (int k = 0; k < kTimelineSlots; ++k) timeline_lds()[k] = 0;
}
#define SV_STAMP_START(base) (::sv::timeline_clear(), ::sv::timeline_put(0, __builtin_amdgcn_s_memrealtime()))
#define SV_STAMP(base, k) ::sv::timeline_put((k), __builtin_amdgcn_s_memrealtime())
#define SV_STAMP_VAL(base, k, v) ::sv::timeline_put((k), (uint64_t)(v))
#define SV_STAMP_LAST(base, k) ::sv::timeline_last((k), __builtin_amdgcn_s_memrealtime())
#define SV_STAMP_TAG(base, role, seq)                                                               \
  ::sv::timeline_put(15, (uint64_t)(role) | ((uint64_t)(uint32_t)(seq) << 8) |                     \
                             ((uint64_t)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xf) << 40))
#define SV_STAMP_FLUSH(base) ::sv::timeline_flush(base)
// Registers the stamp buffer of this translation unit (host side).
#define SV_TIMELINE_SETTER(name)                                                                    \
  hipError_t name(void* p, uint64_t records) {                                                      \
    const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &p, sizeof(p));                  \
    return e != hipSuccess ? e : hipMemcpyToSymbol(HIP_SYMBOL(g_timeline_records), &records, sizeof(records)); \
  }
// Accumulated intervals of a repeated phase (two kinds), per block.
struct Lap {
  uint64_t t = 0, sum[2] = {0, 0};
  __device__ __forceinline__ void start() { t = __builtin_amdgcn_s_memrealtime(); }
  __device__ __forceinline__ void lap(int i) {
    const uint64_t u = __builtin_amdgcn_s_memrealtime();
    sum[i] += u - t;
    t = u;
  }
};
#else
#define SV_STAMP_START(base) ((void)0)
#define SV_STAMP(base, k) ((void)0)
#define SV_STAMP_VAL(base, k, v) ((void)0)
#define SV_STAMP_LAST(base, k) ((void)0)
#define SV_STAMP_TAG(base, role, seq) ((void)0)
#define SV_STAMP_FLUSH(base) ((void)0)
#define SV_TIMELINE_SETTER(name)
struct Lap {
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void lap(int) {}
};
#endif

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element formats: one 16-byte load holds 8 bf16 or 4 fp32 logits.
// bf16 -> fp32 is exact: the 16 bits are the high half of the fp32 pattern;
// in a little-endian 32-bit word the lower-indexed element is the low half.
// ---------------------------------------------------------------------------
template <int DT>
struct Fmt;
template <>
struct Fmt<SV_BF16> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
};
template <>
struct Fmt<SV_F32> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
};

template <int DT>
__device__ __forceinline__ void unpack(const u32x4 d, float* x) {
  if constexpr (DT == SV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(d[i] << 16);
      x[2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(d[i]);
  }
}

__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t stride_bytes) {
  return static_cast<const char*>(base) + row * stride_bytes;
}

// Streaming 16-byte load with the non-temporal hint: the rows are read once,
// and the hint lets the loads bypass cache allocation (on this chip it raises
// the achievable read rate from ~5.9 to ~6.8 TB/s).
__device__ __forceinline__ u32x4 load_vec(const void* row, int64_t vi) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + vi);
}

// One logit as fp32 (gather of a single token).
template <int DT>
__device__ __forceinline__ float load_elem(const void* row, int64_t i) {
  if constexpr (DT == SV_BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[i];
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return reinterpret_cast<const float*>(row)[i];
  }
}

// One logit's bits (a gather whose value is used much later: keeping the
// raw bits lets the conversion wait until the use) and their fp32 value.
template <int DT>
__device__ __forceinline__ uint32_t load_bits(const void* row, int64_t i) {
  if constexpr (DT == SV_BF16)
    return reinterpret_cast<const uint16_t*>(row)[i];
  else
    return reinterpret_cast<const uint32_t*>(row)[i];
}
template <int DT>
__device__ __forceinline__ float bits_value(uint32_t w) {
  if constexpr (DT == SV_BF16)
    return __uint_as_float(w << 16);
  else
    return __uint_as_float(w);
}

// 2^x on the hardware exp unit (no denormal fix-up; terms that small are
// below 2^-126 of the row maximum and do not matter to any sum here).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x for a double x <= 0 whose exact value is wanted to fp32 accuracy
// (rescaling one part's sum to another shift when parts merge): the
// fraction goes through the fp32 unit and the integer part is exact, so the
// relative error is that of one v_exp_f32 (about 1e-7) for any x, where an
// fp32 argument would lose digits of x itself.
__device__ __forceinline__ double exp2_d(double x) {
  const double n = floor(x);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(x - n)), (int)fmax(n, -2000.0));
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of
// (c0,c1,c2,c3) -> (hi(B c2)^c1^k0, lo(B c2), hi(A c0)^c3^k1, lo(A c0)),
// A = 0xD2511F53, B = 0xCD9E8D57, key bumped by (0x9E3779B9, 0xBB67AE85)
// between rounds.  Only the first output word is used.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo_a = 0xD2511F53u * c0, hi_a = __umulhi(0xD2511F53u, c0);
    const uint32_t lo_b = 0xCD9E8D57u * c2, hi_b = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
  }
  return c0;
}

// Verifier uniform on the 2^-24 grid: key = seed (low, high), counter =
// (idx, b, k, (round << 2) | tag).
__device__ __forceinline__ double uniform24(uint64_t seed, uint32_t idx, uint32_t b, uint32_t k, uint32_t round,
                                            uint32_t tag) {
  const uint32_t w = philox_word0(idx, b, k, (round << 2) | tag, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (double)(w >> 8) * (1.0 / 16777216.0);
}

// a = p(x) / q(x); q(x) = 0 accepts iff p(x) > 0.
__device__ __forceinline__ double accept_ratio(double p, double q) {
  if (q > 0.0) return p / q;
  return p > 0.0 ? __builtin_huge_val() : 0.0;
}

// ---------------------------------------------------------------------------
// Wave / block collectives (block of NT threads = NT/64 waves).
// ---------------------------------------------------------------------------

// Block barrier for data exchanged through LDS only: it waits for this
// wave's LDS operations but not for its global loads or stores, so loads
// issued ahead of it stay in flight (a plain __syncthreads also waits for
// every outstanding global access, stores and loads being counted
// together on this architecture).  Global memory shared between blocks is
// ordered explicitly where it is handed off.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}
// Lane movement by DPP (gfx9 encodings): row_shr:n shifts within 16-lane
// rows, row_bcast:15 / row_bcast:31 broadcast lane 15 of each row to the
// next row / lane 31 to rows 2 and 3.  Lanes without a source, and rows
// outside ROWS, read `fill`.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d(double v, double fill) {
  const uint64_t b = (uint64_t)__double_as_longlong(v), f = (uint64_t)__double_as_longlong(fill);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)f, (int)(uint32_t)b, CTRL, ROWS, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(f >> 32), (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sum over the wave's lanes in lane order: four row shifts
// and two row broadcasts, no LDS traffic.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_d<kDppRowShr1, 0xF>(v, 0.0);
  v += dpp_d<kDppRowShr2, 0xF>(v, 0.0);
  v += dpp_d<kDppRowShr4, 0xF>(v, 0.0);
  v += dpp_d<kDppRowShr8, 0xF>(v, 0.0);
  v += dpp_d<kDppRowBcast15, 0xA>(v, 0.0);
  v += dpp_d<kDppRowBcast31, 0xC>(v, 0.0);
  return v;
}

// Lane l's value (l wave-uniform).
__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ int64_t readlane_i64(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Reductions of N values per lane at once, each left in every lane, by DPP
// lane movement: two quad permutations (lane i with i^1, then with i^2),
// then the half-row and row mirrors, give every lane of a 16-lane row its
// row's total; the four row totals are then read as scalars and combined in
// a fixed order.  At each step the two lanes of a pair combine the same two
// operands, so all lanes end with the same bits, and the N reductions'
// steps interleave (no LDS traffic, no wait between steps of one value).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
template <int N>
__device__ __forceinline__ void rows_fmax_all(float (&v)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = fmaxf(v[r], dpp_f<kDppQuadXor1>(v[r]));
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = fmaxf(v[r], dpp_f<kDppQuadXor2>(v[r]));
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = fmaxf(v[r], dpp_f<kDppRowHalfMirror>(v[r]));
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = fmaxf(v[r], dpp_f<kDppRowMirror>(v[r]));
#pragma unroll
  for (int r = 0; r < N; ++r)
    v[r] = fmaxf(fmaxf(readlane_f(v[r], 0), readlane_f(v[r], 16)), fmaxf(readlane_f(v[r], 32), readlane_f(v[r], 48)));
}
template <int N>
__device__ __forceinline__ void rows_fsum_all(float (&v)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_f<kDppQuadXor1>(v[r]);
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_f<kDppQuadXor2>(v[r]);
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_f<kDppRowHalfMirror>(v[r]);
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_f<kDppRowMirror>(v[r]);
#pragma unroll
  for (int r = 0; r < N; ++r)
    v[r] = (readlane_f(v[r], 0) + readlane_f(v[r], 16)) + (readlane_f(v[r], 32) + readlane_f(v[r], 48));
}
template <int N>
__device__ __forceinline__ void rows_sum_all(double (&v)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_d<kDppQuadXor1, 0xF>(v[r], 0.0);
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_d<kDppQuadXor2, 0xF>(v[r], 0.0);
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_d<kDppRowHalfMirror, 0xF>(v[r], 0.0);
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] += dpp_d<kDppRowMirror, 0xF>(v[r], 0.0);
#pragma unroll
  for (int r = 0; r < N; ++r)
    v[r] = (readlane_d(v[r], 0) + readlane_d(v[r], 16)) + (readlane_d(v[r], 32) + readlane_d(v[r], 48));
}

// One value per lane: the wave's maximum / sum, in every lane.
__device__ __forceinline__ float wave_fmax(float v) {
  float a[1] = {v};
  rows_fmax_all(a);
  return a[0];
}
__device__ __forceinline__ double wave_sum(double v) {
  double a[1] = {v};
  rows_sum_all(a);
  return a[0];
}

template <int NT>
__device__ float block_fmax(float v) {
  __shared__ float red[NT / kWave];
  v = wave_fmax(v);
  const int w = threadIdx.x / kWave;
  lds_sync();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  lds_sync();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Sum in a fixed order (wave butterfly, then waves in index order):
// deterministic for a given launch shape.
template <int NT>
__device__ double block_sum(double v) {
  __shared__ double red[NT / kWave];
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  lds_sync();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  lds_sync();
  double r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r += red[i];
  return r;
}

template <int NT>
__device__ int64_t block_max_i64(int64_t v) {
  __shared__ int64_t red[NT / kWave];
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  lds_sync();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  lds_sync();
  int64_t r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = max(r, red[i]);
  return r;
}

template <int NT>
__device__ int64_t block_min_i64(int64_t v) {
  __shared__ int64_t red[NT / kWave];
  v = wave_min(v);
  const int w = threadIdx.x / kWave;
  lds_sync();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  lds_sync();
  int64_t r = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = min(r, red[i]);
  return r;
}

// Exclusive prefix sum over the block in thread order; returns the total.
template <int NT>
__device__ double block_exclusive_scan(double v, double* excl) {
  __shared__ double wtot[NT / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const double inc = wave_incl_scan(v);
  lds_sync();
  if (lane == kWave - 1) wtot[w] = inc;
  lds_sync();
  double before = 0.0, total = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    if (i < w) before += wtot[i];
    total += wtot[i];
  }
  *excl = before + (inc - v);
  return total;
}

// ---------------------------------------------------------------------------
// Row statistics.  For logits z and c = log2(e) / T, a row's temperature
// softmax is p(v) = 2^(z_v c - c M) / S with M = max z and
// S = sum_v 2^(z_v c - c M).  A partial over part of a row is (M, S) with
// S relative to the fp32 product cm = c * M; partials merge by rescaling
// with 2^(cm_a - cm_b).
// ---------------------------------------------------------------------------
struct Partial {
  float m;   // max raw logit of the part (-inf if none finite)
  float pad;
  double s;  // sum of 2^(z c - c m) over the part
};

struct RowStat {
  float cm;  // c * (row max), the shift used for every term
  float pad;
  double S;  // sum_v 2^(z_v c - cm); 0 if the row has no finite logit
};

// Buffer resource over `bytes` bytes at `base` (raw, untyped: the gfx9
// word-3 format).  A load at an offset past `bytes` returns zeros without a
// memory access, so a prefetch past the end of a range needs no clamp.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// One 16-byte non-temporal load at byte offset `off` of a range.
__device__ __forceinline__ u32x4 load_range(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}

// Fold U vectors of one row into this thread's running (m, s): m the
// largest logit so far, s the sum of 2^(z c - c m).  MASK: vectors whose
// index first + u * NT is past the range (nv) count as -inf.
template <int DT, int NT, int U, bool MASK>
__device__ __forceinline__ void fold_vectors(const u32x4 (&d)[U], int64_t first, int64_t nv, float c, float& m,
                                             float& s) {
  constexpr int E = Fmt<DT>::kPerVec;
  float x[U * E];
#pragma unroll
  for (int u = 0; u < U; ++u) unpack<DT>(d[u], x + u * E);
  if constexpr (MASK) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (first + (int64_t)u * NT >= nv)
#pragma unroll
        for (int e = 0; e < E; ++e) x[u * E + e] = kNegInf;
  }
  float gm = x[0];
#pragma unroll
  for (int e = 1; e < U * E; ++e) gm = fmaxf(gm, x[e]);
  if (gm > m) {
    s *= fast_exp2(c * m - c * gm);
    m = gm;
  }
  if (m != kNegInf) {
    const float cm = c * m;
    float t[U * E];
#pragma unroll
    for (int e = 0; e < U * E; ++e) t[e] = fast_exp2(__builtin_fmaf(x[e], c, -cm));
#pragma unroll
    for (int w = U * E / 2; w > 0; w >>= 1)
#pragma unroll
      for (int e = 0; e < w; ++e) t[e] += t[e + w];
    s += t[0];
  }
}

// Online (max, sum) over vectors [v0, v1) of one row by a block of NT
// threads; U vectors in flight per thread, the next U issued before the
// current ones are folded.  Every thread runs the same number of groups of
// U * NT vectors (the last one masked), so no thread ends with a serial
// tail of dependent loads; prefetches past the range read zeros from the
// buffer resource and are never folded.  Every thread returns the block's
// partial.  A thread with `gather` set also loads the bits of element gx of
// the row (clamped into [0, V)) into *gbits; the load is issued after the
// first vectors of the stream, so waiting for gx (loaded by the caller) does
// not hold back the stream, and nothing waits for the gathered bits before
// the caller uses them.
template <int DT, int NT, int U>
__device__ Partial range_stats(const void* row, int V, int64_t v0, int64_t v1, float c, bool gather = false,
                               int32_t gx = 0, uint32_t* gbits = nullptr) {
  constexpr int E = Fmt<DT>::kPerVec;
  constexpr int64_t kGroup = (int64_t)U * NT;
  const int tid = threadIdx.x;
  const int64_t nfull = V / E;
  const int64_t vf = v1 < nfull ? v1 : nfull;
  float m = kNegInf;
  float s = 0.f;
  bool gathered = !gather;
  if (vf > v0) {
    // full vectors [v0, vf): at most 2^24 / 4 vectors, so byte offsets fit 32 bits
    const int64_t nv = vf - v0;
    const __amdgpu_buffer_rsrc_t rs = range_rsrc(static_cast<const u32x4*>(row) + v0, (uint32_t)(nv * 16));
    const int64_t full = nv / kGroup;
    uint32_t off = (uint32_t)tid * 16u;
    u32x4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load_range(rs, off + (uint32_t)(u * NT * 16));
    if (!gathered) {
      *gbits = load_bits<DT>(row, gx >= 0 && gx < V ? gx : 0);
      gathered = true;
    }
    for (int64_t k = 0; k < full; ++k) {
      off += (uint32_t)(kGroup * 16);
      u32x4 nxt[U];
#pragma unroll
      for (int u = 0; u < U; ++u) nxt[u] = load_range(rs, off + (uint32_t)(u * NT * 16));
      fold_vectors<DT, NT, U, false>(cur, 0, nv, c, m, s);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
    if (full * kGroup < nv) fold_vectors<DT, NT, U, true>(cur, full * kGroup + tid, nv, c, m, s);
  }
  if (!gathered) *gbits = load_bits<DT>(row, gx >= 0 && gx < V ? gx : 0);
  if (v1 > nfull && tid == 0) {
    // the row's last vector, holding fewer than E logits (v1 = nfull + 1)
    float x[E];
    unpack<DT>(load_vec(row, nfull), x);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (nfull * E + e >= V) x[e] = kNegInf;
    float gm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) gm = fmaxf(gm, x[e]);
    if (gm > m) {
      s *= fast_exp2(c * m - c * gm);
      m = gm;
    }
    if (m != kNegInf) {
      const float cm = c * m;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc += fast_exp2(__builtin_fmaf(x[e], c, -cm));
      s += acc;
    }
  }
  const float M = block_fmax<NT>(m);
  const double mine = (m == kNegInf) ? 0.0 : (double)s * (double)fast_exp2(c * m - c * M);
  const double S = block_sum<NT>(mine);
  Partial p;
  p.m = M;
  p.pad = 0.f;
  p.s = S;
  return p;
}


// p(v) of one gathered logit under a row statistic (0 for an empty row).
__device__ __forceinline__ double prob_of(float z, float c, const RowStat& st) {
  if (!(st.S > 0.0)) return 0.0;
  return (double)exp2f(__builtin_fmaf(z, c, -st.cm)) / st.S;
}

// ---------------------------------------------------------------------------
// Weights of the final draw, one 16-byte vector at a time (elements past V
// get weight 0).
//   residual: w = max(0, p - coef * q), p and q normalised by their row
//             statistics (coef = 1 for a chain, c_i for a tree node);
//   plain:    w = 2^(z c - cm) (bonus draw / fallback, unnormalised).
// Either form may exclude a short list of token ids (weight 0): the
// point-mass rule's rejected tokens.
// ---------------------------------------------------------------------------
struct DrawSpec {
  const void* rowP;
  const void* rowQ;  // null for a plain draw
  float c;           // log2(e) / T
  float cmP, invSP;  // residual: p = 2^(zP c - cmP) * invSP; plain: shift cmP, invSP unused
  float cmQ, invSQ;
  float coef;
  const int32_t* ex;  // excluded token ids (LDS, same in every thread)
  int32_t nex;        // their count (0: none)
};

template <int DT>
__device__ __forceinline__ void draw_weights_from(const DrawSpec& sp, int V, int64_t vi, const u32x4 dp,
                                                  const u32x4 dq, float* w) {
  constexpr int E = Fmt<DT>::kPerVec;
  float zp[E];
  unpack<DT>(dp, zp);
  if (sp.rowQ) {
    float zq[E];
    unpack<DT>(dq, zq);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float pw = fast_exp2(__builtin_fmaf(zp[e], sp.c, -sp.cmP)) * sp.invSP;
      const float qw = fast_exp2(__builtin_fmaf(zq[e], sp.c, -sp.cmQ)) * sp.invSQ;
      w[e] = fmaxf(__builtin_fmaf(-sp.coef, qw, pw), 0.f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = fast_exp2(__builtin_fmaf(zp[e], sp.c, -sp.cmP));
  }
  if ((vi + 1) * E > V) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (vi * E + e >= V) w[e] = 0.f;
  }
  for (int i = 0; i < sp.nex; ++i) {
    const int64_t d = (int64_t)sp.ex[i] - vi * E;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (d == e) w[e] = 0.f;
  }
}

template <int DT>
__device__ __forceinline__ void draw_weights(const DrawSpec& sp, int V, int64_t vi, float* w) {
  const u32x4 dp = load_vec(sp.rowP, vi);
  const u32x4 dq = sp.rowQ ? load_vec(sp.rowQ, vi) : dp;
  draw_weights_from<DT>(sp, V, vi, dp, dq, w);
}

// Sum of draw weights over vectors [v0, v1) by a block (double accumulation),
// kDrawU vectors per row in flight per thread (clamped addresses, masked
// contributions, so the loads are unconditional and overlap).
constexpr int kDrawU = 4;

template <int DT, int NT>
__device__ double range_weight_sum(const DrawSpec& sp, int V, int64_t v0, int64_t v1) {
  constexpr int E = Fmt<DT>::kPerVec;
  double acc = 0.0;
  if (v1 <= v0) return block_sum<NT>(0.0);
  for (int64_t base = v0 + threadIdx.x; base < v1; base += (int64_t)kDrawU * NT) {
    u32x4 dp[kDrawU], dq[kDrawU];
#pragma unroll
    for (int u = 0; u < kDrawU; ++u) {
      const int64_t v = base + (int64_t)u * NT;
      const int64_t vc = v < v1 ? v : v1 - 1;
      dp[u] = load_vec(sp.rowP, vc);
      if (sp.rowQ) dq[u] = load_vec(sp.rowQ, vc);
    }
#pragma unroll
    for (int u = 0; u < kDrawU; ++u) {
      const int64_t v = base + (int64_t)u * NT;
      if (v < v1) {
        float w[E];
        draw_weights_from<DT>(sp, V, v, dp[u], dq[u], w);
        double own = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) own += (double)w[e];
        acc += own;
      }
    }
  }
  return block_sum<NT>(acc);
}

// Inverse-CDF search over vectors [v0, v1) in index order: the first element
// whose running weight exceeds `target`.  Tiles of NT vectors, kDrawU tiles'
// loads in flight at once; in each tile the block scans per-thread sums, and
// the thread whose interval holds the target walks its own elements.  If
// rounding leaves the target beyond the range's weight, the last positive
// element is returned.  All threads return the same index.
template <int DT, int NT>
__device__ int64_t block_search(const DrawSpec& sp, int V, int64_t v0, int64_t v1, double target) {
  constexpr int E = Fmt<DT>::kPerVec;
  double cum = 0.0;
  int64_t last_pos = -1;
  for (int64_t base0 = v0; base0 < v1; base0 += (int64_t)kDrawU * NT) {
    u32x4 dp[kDrawU], dq[kDrawU];
#pragma unroll
    for (int u = 0; u < kDrawU; ++u) {
      const int64_t v = base0 + (int64_t)u * NT + threadIdx.x;
      const int64_t vc = v < v1 ? v : v1 - 1;
      dp[u] = load_vec(sp.rowP, vc);
      if (sp.rowQ) dq[u] = load_vec(sp.rowQ, vc);
    }
    for (int u = 0; u < kDrawU; ++u) {
      const int64_t base = base0 + (int64_t)u * NT;
      if (base >= v1) break;  // block-uniform
      const int64_t v = base + threadIdx.x;
      float w[E];
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] = 0.f;
      if (v < v1) draw_weights_from<DT>(sp, V, v, dp[u], dq[u], w);
      double own = 0.0;
      int64_t my_last = -1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        own += (double)w[e];
        if (w[e] > 0.f) my_last = v * E + e;
      }
      double excl;
      const double total = block_exclusive_scan<NT>(own, &excl);
      const int64_t tile_last = block_max_i64<NT>(my_last);
      if (tile_last >= 0) last_pos = tile_last;
      if (cum + total > target) {
        const double t_local = target - cum - excl;
        int64_t found = INT64_MAX;
        if (own > 0.0 && t_local >= 0.0 && t_local < own) {
          double run = 0.0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            run += (double)w[e];
            if (found == INT64_MAX && run > t_local) found = v * E + e;
          }
          if (found == INT64_MAX) found = my_last;
        }
        const int64_t r = block_min_i64<NT>(found);
        return r != INT64_MAX ? r : tile_last;
      }
      cum += total;
    }
  }
  return last_pos;
}

// ---------------------------------------------------------------------------
// Hand-off between the blocks of one launch.  Parts written by one block and
// merged by another travel through device-scope (agent) atomic stores and
// loads only: on gfx950 those are performed at the device-coherent level
// (they write through / re-fetch past the per-XCD L2), so no agent-scope
// fence - which would write back or invalidate a whole L2 per block - is
// needed.  Each block waits for its own stores to complete before counting
// its arrival; the last block to arrive reads every part.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_partial(Partial* dst, const Partial& v) {
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
  st_dev(d, (uint64_t)__float_as_uint(v.m));
  st_dev(d + 1, (uint64_t)__double_as_longlong(v.s));
}
__device__ __forceinline__ Partial get_partial(const Partial* src) {
  const uint64_t* d = reinterpret_cast<const uint64_t*>(src);
  Partial v;
  v.m = __uint_as_float((uint32_t)ld_dev(d));
  v.pad = 0.f;
  v.s = __longlong_as_double((long long)ld_dev(d + 1));
  return v;
}

// Count one arrival on `counter` once this block's hand-off stores have
// completed; true in every thread of the block that arrived last (of
// `total`).  That block resets the counter to 0 itself.
template <int NT>
__device__ bool arrive_last(uint32_t* counter, uint32_t total) {
  __shared__ int last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete (device-visible)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = (old == total - 1);
  }
  __syncthreads();
  return last != 0;
}

// Merge the parts of one row (in part order) into the row statistic; parts
// are read with device-scope loads (written by other blocks of the launch).
__device__ inline RowStat merge_parts(const Partial* parts, int n, float c) {
  float M = kNegInf;
  for (int i = 0; i < n; ++i) M = fmaxf(M, get_partial(parts + i).m);
  RowStat r;
  r.pad = 0.f;
  if (M == kNegInf) {
    r.cm = 0.f;
    r.S = 0.0;
    return r;
  }
  r.cm = c * M;
  double S = 0.0;
  for (int i = 0; i < n; ++i) {
    const Partial pi = get_partial(parts + i);
    if (pi.m == kNegInf) continue;
    S += pi.s * exp2_d((double)(c * pi.m) - (double)r.cm);
  }
  r.S = S;
  return r;
}

__device__ __forceinline__ void set_error(int32_t* err, int32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
