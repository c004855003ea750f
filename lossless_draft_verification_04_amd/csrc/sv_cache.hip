// sv_cache.hip -- speculation-cache hit test on gfx950.
//
// SSD / Saguaro review §3 (cache strategy): the speculator caches, for every
// lookahead position k = 0..K, the top-F_k tokens of the draft logits at k;
// a verification outcome (n, t) -- n drafts accepted, then token t -- is
// served from the cache iff t is among the tokens cached for position n (the
// hit event of Definition 11).  Under the fan-out's order (value descending,
// index ascending on equal values) that is rank(t) < F_n with
//   rank(t) = #{v : z_v > z_t, or z_v == z_t and v < t}
// over draft row n, so the test is one counting pass over one row per
// sequence, and the rank is also the smallest fan-out that would have hit
// minus one.
//
// One launch: a block per (sequence, row part) counts the elements of its
// part that precede t (16-byte loads, four in flight per thread) and adds
// the count to the sequence's 64-bit workspace word together with one
// arrival in the high half.  Every count rides in the same atomic word, so
// the block that arrives last reads the total from its own fetch-add, writes
// rank and hit, and clears the word.
#include "sv_device.hpp"
#include "sv_internal.h"

namespace sv {

constexpr int kCNT = 256;
constexpr int kCU = 4;

// Elements of one 16-byte vector (index v) that precede token t: a larger
// logit, or an equal one at a lower index.
template <int DT>
__device__ __forceinline__ uint32_t count_before(const u32x4 d, int64_t v, int V, float zt, int64_t t) {
  constexpr int E = Fmt<DT>::kPerVec;
  float x[E];
  unpack<DT>(d, x);
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t i = v * E + e;
    c += (uint32_t)((i < V) & ((x[e] > zt) | ((x[e] == zt) & (i < t))));  // no branches
  }
  return c;
}

template <int DT>
__global__ __launch_bounds__(kCNT) void cache_rank_kernel(CacheParams a) {
  const int64_t bid = blockIdx.x;
  const int b = (int)(bid / a.nch);
  const int ch = (int)(bid - (int64_t)b * a.nch);
  const int32_t n = a.n[b], t = a.t[b];
  const bool ok = n >= 0 && n <= a.K && t >= 0 && t < a.V;
  // the fan-out of position n (F is given exactly when out_hit is), loaded
  // now so the last block does not wait for it after its fetch-add
  const int32_t Fn = (ok && threadIdx.x == 0 && a.F != nullptr) ? a.F[n] : 0;
  uint32_t cnt = 0;
  if (ok) {
    const void* row = row_ptr(a.drf, (int64_t)b * (a.K + 1) + n, a.sb);
    const float zt = load_elem<DT>(row, t);
    const int64_t v0 = (int64_t)ch * a.vpc;
    const int64_t v1 = v0 + a.vpc < a.nvec ? v0 + a.vpc : a.nvec;
    for (int64_t base = v0 + threadIdx.x; base < v1; base += (int64_t)kCU * kCNT) {
      u32x4 d[kCU];
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        const int64_t v = base + (int64_t)u * kCNT;
        d[u] = load_vec(row, v < v1 ? v : v1 - 1);  // clamped: the loads are unconditional and overlap
      }
#pragma unroll
      for (int u = 0; u < kCU; ++u) {
        const int64_t v = base + (int64_t)u * kCNT;
        if (v < v1) cnt += count_before<DT>(d[u], v, a.V, zt, t);
      }
    }
  }
  const uint32_t total = (uint32_t)block_sum<kCNT>((double)cnt);  // exact: at most V < 2^24
  if (threadIdx.x == 0) {
    uint64_t* word = a.words + b;
    const uint64_t old =
        __hip_atomic_fetch_add(word, (1ull << 32) | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old >> 32) == (uint32_t)(a.nch - 1)) {
      const int32_t rank = (int32_t)((uint32_t)old + total);
      a.out_rank[b] = ok ? rank : -1;
      if (a.out_hit) a.out_hit[b] = ok && rank < Fn ? 1 : 0;
      if (!ok) set_error(a.err, SV_DERR_TOKEN);
      __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_cache(const CacheParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16)
    cache_rank_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kCNT), 0, s>>>(p);
  else
    cache_rank_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kCNT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
