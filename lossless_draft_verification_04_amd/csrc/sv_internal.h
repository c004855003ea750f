// sv_internal.h -- host-side launch parameters shared by the library's
// translation units (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// Fixed workspace header: error word, then a counter region that every op
// leaves zeroed on exit, then op-specific scratch.
constexpr size_t kWsHeader = 256;
constexpr size_t kWsCounters = 65536;  // uint32 counters
constexpr size_t kWsFixed = kWsHeader + kWsCounters * sizeof(uint32_t);

struct ChainParams {
  const void* tgt;
  const void* drf;
  int64_t tgt_sb, drf_sb;  // row strides in bytes
  const int32_t* tok;
  int32_t B, K, gamma, V;
  float c;  // log2(e) / T
  uint64_t seed;
  uint32_t round;
  int32_t* out_k;
  int32_t* out_n;
  int32_t* out_tok;
  int32_t* out_n_cand;
  float* out_p;
  float* out_q;
  int32_t* err;
  const uint32_t* knobs;  // workspace header (wait bound, test switch), or null
  uint32_t* cnt;   // counter region: arrivals of sequence b at [b * cstride], draw exits at [(B + b) * cstride]
  int32_t cstride;
  void* part1;     // stats parts, [B][rows][nch1]
  float* zg;       // target logits of the drafted tokens, [B][K][gamma]
  float* zq;       // draft logits of the drafted tokens, [B][K][gamma]
  void* slots;     // draw slot words, [B][G][kSlotWords], in the counter region (zero between calls)
  int32_t nch1;
  int32_t G;       // draw blocks per sequence
  int64_t grid1;   // statistics blocks (the draw blocks follow them)
  bool held;       // slices of at most kSliceTiles tiles, held in registers
  bool pm;         // point-mass acceptance: target rows only
  bool xcd;        // a sequence's statistics blocks share one XCD (B a multiple of 8)
  int64_t vpc1, nvec;
};

struct GreedyParams {
  const void* tgt;
  int64_t tgt_sb;
  const int32_t* tok;
  int32_t B, gamma, V;
  int32_t* out_n;
  int32_t* out_tok;
  int32_t* out_argmax;
  int32_t* err;
  uint32_t* cnt;
  void* part;
  int32_t nch;
  int64_t vpc, nvec;
};

struct TreeParams {
  const void* tgt;
  const void* drf;
  int64_t tgt_sb, drf_sb;
  const int32_t* tok;
  const int32_t* parent;
  int32_t B, N, max_depth, V;
  float c;
  uint64_t seed;
  uint32_t round;
  int32_t* out_len;
  int32_t* out_path;
  int32_t* out_tok;
  float* out_p;
  float* out_q;
  int32_t* err;
  const uint32_t* knobs;  // workspace header (wait bound, test switch), or null
  void* part;
  float* zc;       // each child's logits under its parent's rows, [2][B][N] (target, draft)
  void* slots;     // walk slot words, [B][G][kSlotWords], zeroed by the stats launch
  int64_t nzero;   // 64-bit words of `slots` the stats launch zeroes
  int32_t nch;
  int32_t G;       // walk blocks per sequence
  bool held;       // slices of at most kSliceTiles tiles, held in registers
  bool pm;         // point-mass acceptance: target rows only
  bool all_rows;   // stream every node's rows (leaves too), not only those with children
  int64_t vpc, nvec;
};

struct PrestoParams {
  const void* tgt;
  const void* drf;
  int64_t tgt_sb, drf_sb;
  const int32_t* tok;
  const int32_t* parent;
  int32_t B, N, V;
  float c;           // log2(e) / T
  const float* lam;  // lambda per depth, [D]
  int32_t D, k, b_top;
  float* out_s;
  float* out_S;
  int32_t* out_node;
  int32_t* out_tok;
  float* out_score;
  int32_t* err;
  void* part;        // row statistics parts, [B][N][2][nch1] (tree statistics launch)
  float* zc;         // each child's logits under its parent's rows, [2][B][N]
  void* lists;       // expansion part lists, [B][N][nch2][k]
  void* leaf_lists;  // each leaf's merged list, [B][N][k]
  uint32_t* leaf_cnt;  // arrivals per node, [B][N], zeroed by the statistics launch
  int32_t nch1, nch2;
  int64_t vpc2, nvec;
};

struct BranchParams {
  const void* drf;  // draft rows q_1..q_{gamma+1} per sequence
  int64_t sb;
  const int32_t* tok;
  const int32_t* cls;  // predictor class per sequence, or null (every class 1)
  int32_t B, gamma, V;
  float c;  // log2(e) / T
  double eps;
  int32_t k_max;
  int32_t* out_pos;
  float* out_qb;
  int32_t* out_k;
  int32_t* out_ids;
  int32_t* err;
  uint32_t* cnt;   // per-sequence arrival counters
  void* part;      // statistics parts, [B][gamma+1][nch1]
  float* zq;       // draft logits of the drafted tokens, [B][gamma] (NaN: token out of range)
  void* lists;     // fork part lists, [B][nch2][k_max]
  int32_t nch1, nch2;
  int64_t vpc1, vpc2, nvec;
};

struct FanoutParams {
  const void* logits;
  int64_t sb;
  int32_t R, V;
  const int32_t* F;
  int32_t F_max;
  int32_t* out_ids;
  float* out_vals;
  int32_t* err;
  uint32_t* cnt;
  void* part;
  int32_t nch;
  int64_t vpc, nvec;
};

struct CacheParams {
  const void* drf;
  int64_t sb;
  int32_t B, K, V;
  const int32_t* n;
  const int32_t* t;
  const int32_t* F;
  int32_t* out_rank;
  int32_t* out_hit;
  int32_t* err;
  uint64_t* words;  // one per sequence in the counter region: arrivals (high) | count (low)
  int32_t nch;
  int64_t vpc, nvec;
};

// Workspace plans (chunking + scratch sizes), computed identically by
// sv_workspace_size and the entry points.
struct Plan {
  int32_t nch1 = 1, nch2 = 1;
  int64_t vpc1 = 0, vpc2 = 0, nvec = 0;
  size_t off_part1 = 0, off_jobs = 0, off_part2 = 0, off_lists = 0;
  size_t bytes = 0;
  int64_t grid1 = 0, grid2 = 0;
};

hipError_t launch_chain(const ChainParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);
#ifdef SV_TIMELINE
// Stamp-buffer setters of the timeline build, one per translation unit.
hipError_t timeline_set_chain(void* p, uint64_t records);
hipError_t timeline_set_chain_small(void* p, uint64_t records);
hipError_t timeline_set_tree(void* p, uint64_t records);
hipError_t timeline_set_fanout(void* p, uint64_t records);
#endif
// Small calls (sv_chain_small.hip): each of G blocks per sequence holds its
// slice (1 or kSmallTiles tiles of 256 vectors) of every row the step may
// touch (at most kSmallRows rows: target 1..gamma+1, draft 1..gamma).
constexpr int kSmallTiles = 2;
constexpr int kSmallRows = 9;
hipError_t launch_chain_small(const ChainParams& p, sv_dtype dt, int tiles, hipStream_t s);
int chain_small_capacity(sv_dtype dt, bool pm, int tiles);
hipError_t launch_greedy(const GreedyParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);
hipError_t launch_tree(const TreeParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);
hipError_t launch_fanout(const FanoutParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);
hipError_t launch_cache(const CacheParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);
hipError_t launch_branch(const BranchParams& p, sv_dtype dt, const Plan& plan, hipStream_t s);
hipError_t launch_presto(const PrestoParams& p, const TreeParams& stats, sv_dtype dt, const Plan& plan,
                         hipStream_t s);
hipError_t launch_fill_zero(void* ws, size_t bytes, hipStream_t s);

// Blocks of one launch of the chain kernel or the walk kernel (held or
// streamed slices) the current device holds at once (0 if unknown).
int chain_capacity(sv_dtype dt, bool held, bool pm);
int tree_walk_capacity(sv_dtype dt, bool held, bool pm);

// Blocks of kernel fn (block of nt threads) device dev holds at once.
inline int device_capacity(const void* fn, int nt, int dev) {
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, nt, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return per_cu * cus;
}

}  // namespace sv
