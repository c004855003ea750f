// sv_fanout.hip -- top-F fan-out of draft rows on gfx950.
//
// SSD / Saguaro review §3: the speculation cache holds the top-F_k tokens of
// the draft logits at every lookahead position k.  Here: for each row r the
// F[r] largest logits, value descending, index ascending on ties.
//
// One launch: a block per (row part).  Each wave keeps its current top-F in
// registers, one entry per lane (lane i = i-th best), and streams its share of
// the part in increasing index order.  The list starts as the top-F of the
// wave's first 64-vector window (F rounds of a wave-wide selection, each a
// DPP reduction).  After
// that a lane's 16-byte vector is a candidate only if its largest element
// beats the wave's F-th best so far (elements are seen in index order, so an
// equal value can never displace an earlier entry); a candidate lane flags
// its qualifying elements, which are read with register lane reads and
// inserted one at a time with a lane shift.  Most vectors cost one max and
// one compare.  The block merges its waves'
// lists; the last block of a row merges the parts' lists and writes them.
#include "sv_device.hpp"
#include "sv_internal.h"

namespace sv {

constexpr int kFNT = 256;

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

template <int DT>
__global__ __launch_bounds__(kFNT) void fanout_kernel(FanoutParams a) {
  constexpr int E = Fmt<DT>::kPerVec;
  const int r = blockIdx.x / a.nch;
  const int ch = blockIdx.x - r * a.nch;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int F = a.F[r];
  if (F < 0 || F > a.F_max) {
    if (threadIdx.x == 0 && ch == 0) set_error(a.err, SV_DERR_FANOUT);
    F = F < 0 ? 0 : a.F_max;
  }
  const void* row = row_ptr(a.logits, r, a.sb);
  float lv = kNegInf;
  int32_t li = kNoIdx;
  int count = 0;  // entries held (wave-uniform)
  float thr = kNegInf;
  const int64_t v0 = (int64_t)ch * a.vpc;
  const int64_t v1 = v0 + a.vpc < a.nvec ? v0 + a.vpc : a.nvec;
  if (F > 0) {
    // each wave walks its own 64-vector windows in increasing order, with
    // the loads of kWin windows in flight at once
    constexpr int kWin = 4;
    const int64_t stride = (int64_t)(kFNT / kWave) * kWave;
    const int64_t step = stride * kWin;
    int64_t base0 = v0 + (int64_t)wave * kWave;
    u32x4 d[kWin];
    if (base0 < v1) {
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t v = base0 + u * stride + lane;
        d[u] = load_vec(row, v < v1 ? v : v1 - 1);  // unconditional (clamped) so the loads overlap
      }
    }
    for (; base0 < v1; base0 += step) {
      // software pipelined: the next kWin windows are in flight while these
      // are scanned (past the end the prefetch is clamped to the last vector)
      u32x4 nx[kWin];
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t v = base0 + step + u * stride + lane;
        nx[u] = load_vec(row, v < v1 ? v : v1 - 1);
      }
#pragma unroll
      for (int u = 0; u < kWin; ++u) {
        const int64_t base = base0 + u * stride;
        const int64_t v = base + lane;
        float x[E];
        float vm = kNegInf;
        const bool valid = v < v1;
        if (valid) {
          unpack<DT>(d[u], x);
          if ((v + 1) * E > a.V) {
#pragma unroll
            for (int e = 0; e < E; ++e)
              if (v * E + e >= a.V) x[e] = kNegInf;
          }
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
                if (!((taken >> e) & 1u) && gi < a.V && (bi == kNoIdx || x[e] > bv)) {
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
            if ((count < F || x[e] > thr) && v * E + e < a.V) mine |= 1u << e;
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
  // merge the block's waves into wave 0's list
  __shared__ TopEntry s_list[kFNT / kWave][SV_MAX_FANOUT];
  __syncthreads();
  if (lane < SV_MAX_FANOUT) {
    s_list[wave][lane].val = lv;
    s_list[wave][lane].idx = li;
  }
  __syncthreads();
  TopEntry* parts = static_cast<TopEntry*>(a.part) + (int64_t)r * a.nch * a.F_max;
  if (wave == 0 && F > 0) {
    // each list is sorted: stop at its first entry that does not beat the
    // current F-th best
    for (int w = 1; w < kFNT / kWave; ++w)
      for (int e = 0; e < F; ++e) {
        const TopEntry t = s_list[w][e];
        const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), F - 1));
        const int32_t ti = __builtin_amdgcn_readlane(li, F - 1);
        if (t.idx == kNoIdx || (ti != kNoIdx && !top_better(t.val, t.idx, tv, ti))) break;
        wave_insert(lv, li, t.val, t.idx, F, lane);
      }
  }
  if (wave == 0 && lane < a.F_max) put_entry(parts + (int64_t)ch * a.F_max + lane, lane < F ? lv : kNegInf,
                                             lane < F ? li : kNoIdx);
  if (!arrive_last<kFNT>(&a.cnt[r], (uint32_t)a.nch)) return;
  if (wave == 0) {
    float fv = kNegInf;
    int32_t fi = kNoIdx;
    for (int c = 0; c < a.nch; ++c)
      for (int e = 0; e < F; ++e) {
        const TopEntry t = get_entry(parts + (int64_t)c * a.F_max + e);
        const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fv), F - 1));
        const int32_t ti = __builtin_amdgcn_readlane(fi, F - 1);
        if (t.idx == kNoIdx || (ti != kNoIdx && !top_better(t.val, t.idx, tv, ti))) break;
        wave_insert(fv, fi, t.val, t.idx, F, lane);
      }
    if (lane < a.F_max) {
      const bool keep = lane < F && fi != kNoIdx;
      a.out_ids[(int64_t)r * a.F_max + lane] = keep ? fi : -1;
      if (a.out_vals) a.out_vals[(int64_t)r * a.F_max + lane] = keep ? fv : kNegInf;
    }
    if (lane == 0) __hip_atomic_store(&a.cnt[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_fanout(const FanoutParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16)
    fanout_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kFNT), 0, s>>>(p);
  else
    fanout_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kFNT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
