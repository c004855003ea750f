// sv_greedy.hip -- greedy (temperature 0) verification on gfx950.
//
// Draft-then-verify page §2.2 and §4: at temperature 0, p and q are one-hot,
// so a draft token is accepted iff it equals the target row's argmax; the
// correction / bonus is the argmax of the first non-matching row (or of row
// gamma+1).  Ties go to the lowest index.
//
// One launch: a block per (row part) streams its part once (16-byte loads,
// compare only), keeps the first maximal vector per thread, resolves the
// lowest index inside it, and reduces over the block.  The last block of a
// sequence merges the parts (in index order) and compares ids.
#include "sv_device.hpp"
#include "sv_internal.h"

namespace sv {

constexpr int kGNT = 192;
constexpr int kGU = 4;

struct ArgPart {
  float val;
  int32_t idx;
};

__device__ __forceinline__ void put_arg(ArgPart* dst, const ArgPart& v) {
  st_dev(reinterpret_cast<uint64_t*>(dst), (uint64_t)__float_as_uint(v.val) | ((uint64_t)(uint32_t)v.idx << 32));
}
__device__ __forceinline__ ArgPart get_arg(const ArgPart* src) {
  const uint64_t w = ld_dev(reinterpret_cast<const uint64_t*>(src));
  ArgPart v;
  v.val = __uint_as_float((uint32_t)w);
  v.idx = (int32_t)(uint32_t)(w >> 32);
  return v;
}

// (value desc, index asc), without branches
__device__ __forceinline__ bool arg_better(float va, int64_t ia, float vb, int64_t ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

template <int DT>
__device__ __forceinline__ float vec_max(const float* x) {
  constexpr int E = Fmt<DT>::kPerVec;
  float m = x[0];
#pragma unroll
  for (int e = 1; e < E; ++e) m = fmaxf(m, x[e]);
  return m;
}

// Lowest index of the maximum over vectors [v0, v1) of one row; every thread
// returns the block's answer.  Each thread keeps the raw bits of its best
// vector, so the lowest index inside it is found without reading it again
// (a re-read bypasses the caches like the stream and costs a whole memory
// line per thread).
template <int DT, int NT, int U>
__device__ ArgPart range_argmax(const void* row, int V, int64_t v0, int64_t v1) {
  constexpr int E = Fmt<DT>::kPerVec;
  const int64_t nfull = V / E;
  const int64_t vf = v1 < nfull ? v1 : nfull;
  float bv = kNegInf;
  int64_t bvec = -1;
  u32x4 bd = u32x4{0u, 0u, 0u, 0u};
  int64_t v = v0 + threadIdx.x;
  for (; v + (int64_t)(U - 1) * NT < vf; v += (int64_t)U * NT) {
    u32x4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = load_vec(row, v + (int64_t)u * NT);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[E];
      unpack<DT>(d[u], x);
      const float m = vec_max<DT>(x);
      if (bvec < 0 || m > bv) {
        bv = m;
        bvec = v + (int64_t)u * NT;
        bd = d[u];
      }
    }
  }
  for (; v < v1; v += NT) {
    const u32x4 d = load_vec(row, v);
    float x[E];
    unpack<DT>(d, x);
    if ((v + 1) * E > V) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (v * E + e >= V) x[e] = kNegInf;
    }
    const float m = vec_max<DT>(x);
    if (bvec < 0 || m > bv) {
      bv = m;
      bvec = v;
      bd = d;
    }
  }
  int64_t bidx = INT64_MAX;
  if (bvec >= 0) {
    float x[E];
    unpack<DT>(bd, x);
    if ((bvec + 1) * E > V) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (bvec * E + e >= V) x[e] = kNegInf;
    }
#pragma unroll
    for (int e = E - 1; e >= 0; --e)
      if (x[e] == bv) bidx = bvec * E + e;
  }
  // block reduction on (value desc, index asc)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int64_t oi = __shfl_xor(bidx, o, kWave);
    if (arg_better(ov, oi, bv, bidx)) {
      bv = ov;
      bidx = oi;
    }
  }
  __shared__ float rv[NT / kWave];
  __shared__ int64_t ri[NT / kWave];
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    rv[threadIdx.x / kWave] = bv;
    ri[threadIdx.x / kWave] = bidx;
  }
  __syncthreads();
  float fv = rv[0];
  int64_t fi = ri[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w)
    if (arg_better(rv[w], ri[w], fv, fi)) {
      fv = rv[w];
      fi = ri[w];
    }
  ArgPart r;
  r.val = fv;
  r.idx = fi == INT64_MAX ? 0 : (int32_t)fi;
  return r;
}

template <int DT>
__global__ __launch_bounds__(kGNT) void greedy_kernel(GreedyParams a) {
  const int rows = a.gamma + 1;
  const int64_t per_seq = (int64_t)rows * a.nch;
  const int64_t bid = blockIdx.x;
  const int b = (int)(bid / per_seq);
  const int64_t rem = bid - (int64_t)b * per_seq;
  const int j = (int)(rem / a.nch);
  const int ch = (int)(rem - (int64_t)j * a.nch);
  const void* row = row_ptr(a.tgt, (int64_t)b * rows + j, a.tgt_sb);
  const int64_t v0 = (int64_t)ch * a.vpc;
  const int64_t v1 = v0 + a.vpc < a.nvec ? v0 + a.vpc : a.nvec;
  const ArgPart part = range_argmax<DT, kGNT, kGU>(row, a.V, v0, v1);
  ArgPart* parts = static_cast<ArgPart*>(a.part) + (int64_t)b * per_seq;
  if (threadIdx.x == 0) put_arg(parts + (int64_t)j * a.nch + ch, part);
  if (!arrive_last<kGNT>(&a.cnt[b], (uint32_t)per_seq)) return;

  __shared__ int32_t g[SV_MAX_GAMMA + 1], s_tok[SV_MAX_GAMMA];
  for (int jj = threadIdx.x; jj < rows; jj += kGNT) {
    // the drafted token is loaded with the row's parts (one round of loads)
    const int32_t x = jj < a.gamma ? a.tok[(int64_t)b * a.gamma + jj] : 0;
    const ArgPart* pr = parts + (int64_t)jj * a.nch;
    const ArgPart p0 = get_arg(pr);
    float bv = p0.val;
    int32_t bi = p0.idx;
    for (int c = 1; c < a.nch; ++c) {
      const ArgPart pc = get_arg(pr + c);
      if (pc.val > bv) {  // parts are in index order: strict > keeps the lowest index
        bv = pc.val;
        bi = pc.idx;
      }
    }
    g[jj] = bi;
    if (jj < a.gamma) {
      s_tok[jj] = x;
      if (x < 0 || x >= a.V) set_error(a.err, SV_DERR_TOKEN);
    }
    if (a.out_argmax) a.out_argmax[(int64_t)b * rows + jj] = bi;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // n = leading matches: a ballot of the mismatches (gamma <= 64)
    const int l = threadIdx.x;
    const uint64_t miss = __ballot(l < a.gamma && s_tok[l] != g[l]);
    int n = miss ? __builtin_ctzll(miss) : a.gamma;
    if (n > a.gamma) n = a.gamma;
    if (l == 0) {
      a.out_n[b] = n;
      a.out_tok[b] = g[n];
      __hip_atomic_store(&a.cnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_greedy(const GreedyParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16)
    greedy_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kGNT), 0, s>>>(p);
  else
    greedy_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kGNT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
