// sv_fanout.hip -- top-F fan-out of draft rows on gfx950.
//
// SSD / Saguaro review §3: the speculation cache holds the top-F_k tokens of
// the draft logits at every lookahead position k.  Here: for each row r the
// F[r] largest logits, value descending, index ascending on ties.
//
// One launch: a block per (row part).  The block finds its part's top F
// (sv_topk.hpp); a row in one part is written by its block, otherwise the
// last block of the row merges the parts' lists and writes them.
#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_topk.hpp"

namespace sv {

constexpr int kFNT = 512;

template <int DT>
__global__ __launch_bounds__(kFNT) void fanout_kernel(FanoutParams a) {
  constexpr int E = Fmt<DT>::kPerVec;
  const int r = blockIdx.x / a.nch;
  const int ch = blockIdx.x - r * a.nch;
  SV_STAMP_START(0);
  SV_STAMP_TAG(0, 6, r);
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
  const int64_t v0 = (int64_t)ch * a.vpc;
  const int64_t v1 = v0 + a.vpc < a.nvec ? v0 + a.vpc : a.nvec;
  if (F > 0) {
    const TopPair t = block_topk<kFNT, E>(RowValues<DT>{row, a.V}, v0, v1, a.V, F);
    lv = t.v;
    li = t.i;
  }
  SV_STAMP(0, 4);
  // wave 0 holds the part's list
  TopEntry* parts = static_cast<TopEntry*>(a.part) + (int64_t)r * a.nch * a.F_max;
  if (a.nch == 1) {  // the whole row: no parts to merge
    if (wave == 0 && lane < a.F_max) {
      const bool keep = lane < F && li != kNoIdx;
      a.out_ids[(int64_t)r * a.F_max + lane] = keep ? li : -1;
      if (a.out_vals) a.out_vals[(int64_t)r * a.F_max + lane] = keep ? lv : kNegInf;
    }
    SV_STAMP(0, 5);
    SV_STAMP_FLUSH(0);
    return;
  }
  if (wave == 0 && lane < a.F_max) put_entry(parts + (int64_t)ch * a.F_max + lane, lane < F ? lv : kNegInf,
                                             lane < F ? li : kNoIdx);
  if (!arrive_last<kFNT>(&a.cnt[r], (uint32_t)a.nch)) return;
  if (wave == 0) {
    float fv = kNegInf;
    int32_t fi = kNoIdx;
    if (F > 0) wave_merge_entries(parts, a.nch * a.F_max, F, fv, fi, lane);
    if (lane < a.F_max) {
      const bool keep = lane < F && fi != kNoIdx;
      a.out_ids[(int64_t)r * a.F_max + lane] = keep ? fi : -1;
      if (a.out_vals) a.out_vals[(int64_t)r * a.F_max + lane] = keep ? fv : kNegInf;
    }
    if (lane == 0) __hip_atomic_store(&a.cnt[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

SV_TIMELINE_SETTER(timeline_set_fanout)

hipError_t launch_fanout(const FanoutParams& p, sv_dtype dt, const Plan& plan, hipStream_t s) {
  if (dt == SV_BF16)
    fanout_kernel<SV_BF16><<<dim3((unsigned)plan.grid1), dim3(kFNT), 0, s>>>(p);
  else
    fanout_kernel<SV_F32><<<dim3((unsigned)plan.grid1), dim3(kFNT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
