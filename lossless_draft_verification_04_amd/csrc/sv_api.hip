// sv_api.hip -- the C ABI of libspecverify: host-side argument checks,
// workspace planning and kernel launches on the caller's stream.
//
// Every check below runs before any HIP call, so invalid arguments are
// rejected synchronously and nothing is enqueued.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "sv_device.hpp"
#include "sv_internal.h"
#include "sv_walk.hpp"

namespace sv {

namespace {

constexpr int kSmallPartVecs = 4096;  // largest part (vectors) the chain plan forms to keep parts per row direct
constexpr int64_t kSmallDrawVecs = 131072;  // B * vectors per row at or below which the chain draw uses full tiles
constexpr int kBlockVecs = 1024;   // smallest row part (vectors): 4 in flight per thread of a 256-thread block
constexpr int kMaxResident = 4096;  // bound on the blocks of a draw / walk launch (two slot words each)

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int x = std::atoi(v);
  return x > 0 ? x : dflt;
}

// Blocks the streaming passes aim for (the chip has 256 CUs; four blocks of
// 256 threads per CU with four 16-byte loads in flight per thread keep the
// HBM busy; fewer, longer parts also mean fewer parts to merge).
// Overridable for tuning sweeps with SV_STATS_BLOCKS.
int stats_blocks() {
  static const int v = env_int("SV_STATS_BLOCKS", 1024);
  return v;
}
// Upper bound on the draw / walk blocks per sequence (SV_DRAW_G overrides it
// for tuning sweeps, up to kMaxG).  Measured on MI355X: at 48-64 blocks per
// sequence the exchange costs more than the shorter slices save (point-mass
// chain call on the 32 x 16 x 152064 batch: 46.4 us at 48, 41.5-42.0 us at
// 24-32, 46.7 us at 16; the other paths change by under 2% from 24 to 64).
constexpr int kDefaultDrawG = 32;
int draw_g_limit() {
  static const int v = env_int("SV_DRAW_G", kDefaultDrawG);
  return v < kMaxG ? v : kMaxG;
}

int per_vec(sv_dtype dt) { return dt == SV_BF16 ? 8 : 4; }
int elem_bytes(sv_dtype dt) { return dt == SV_BF16 ? 2 : 4; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Split rows of nvec vectors into parts of at least min_vecs vectors so that
// rows * parts ~ target.
void split(int64_t rows, int64_t nvec, int target, int32_t* nch, int64_t* vpc, int64_t min_vecs = kBlockVecs) {
  int64_t n = rows > 0 ? (target + rows - 1) / rows : 1;
  const int64_t cap = nvec / min_vecs > 1 ? nvec / min_vecs : 1;
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  int64_t per = (nvec + n - 1) / n;
  if (per < 1) per = 1;
  *vpc = per;
  *nch = (int32_t)((nvec + per - 1) / per);
}

bool bad_dtype(sv_dtype dt) { return dt != SV_BF16 && dt != SV_F32; }

sv_status check_rows(const void* base, int64_t stride, int32_t V, sv_dtype dt) {
  if (!base) return SV_EINVAL;
  if (stride < V) return SV_EINVAL;
  if (reinterpret_cast<uintptr_t>(base) % 16 != 0) return SV_EALIGN;
  if ((stride * elem_bytes(dt)) % 16 != 0) return SV_EALIGN;
  return SV_OK;
}

bool bad_temperature(float T) { return !(T > 0.f) || !std::isfinite(T); }

// Largest G a B-sequence launch may use (B * G <= kMaxResident).
int32_t g_cap(int32_t B) {
  if (B <= 0) return 1;
  const int32_t g = kMaxResident / B;
  return g < 1 ? 1 : (g > kMaxG ? kMaxG : g);
}

// Blocks per sequence of a draw / walk launch: as many as let all B * G
// blocks be resident together (capacity = blocks the device holds at once),
// within the slot region, and at most one per vector.
int32_t choose_g(int32_t B, int64_t nvec, int capacity) {
  if (B <= 0 || capacity <= 0) return 1;
  int64_t g = capacity / B;
  if (g > g_cap(B)) g = g_cap(B);
  if (g > draw_g_limit()) g = draw_g_limit();
  if (g > nvec) g = nvec;
  return g < 1 ? 1 : (int32_t)g;
}

// G and the kernel variant: slices held in registers when they span at most
// kSliceTiles tiles of 256 vectors at the held kernel's G, else streamed.
void pick_slices(int32_t B, int64_t nvec, int cap_held, int cap_stream, int32_t* G, bool* held) {
  const int32_t g = choose_g(B, nvec, cap_held);
  if ((nvec + g - 1) / g <= (int64_t)kSliceTiles * 256) {
    *G = g;
    *held = true;
  } else {
    *G = choose_g(B, nvec, cap_stream);
    *held = false;
  }
}

// pm: point-mass acceptance (target rows only).
sv_status plan_chain(sv_dtype dt, int32_t B, int32_t K, int32_t gamma, int32_t V, bool pm, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (B < 0 || K < 1 || gamma < 1 || V < 1) return SV_EINVAL;
  if (B > SV_MAX_SEQ || K > SV_MAX_K || gamma > SV_MAX_GAMMA || V > SV_MAX_V) return SV_EUNSUPPORTED;
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  const int64_t rows = (int64_t)B * (K + (pm ? 0 : 1)) * gamma;
  split(rows, pl->nvec, stats_blocks(), &pl->nch1, &pl->vpc1);
  // few short rows: at most the parts a draw block merges straight from
  // registers (4 per row, 8 in point-mass mode), which saves the draw blocks
  // a staging round when each part stays small
  const int32_t direct = pm ? 8 : 4;
  if (pl->nch1 > direct && (pl->nvec + direct - 1) / direct <= kSmallPartVecs) {
    pl->vpc1 = (pl->nvec + direct - 1) / direct;
    pl->nch1 = (int32_t)((pl->nvec + pl->vpc1 - 1) / pl->vpc1);
  }
  pl->grid1 = rows * pl->nch1;
  if (pl->grid1 + (int64_t)B * kMaxG > INT32_MAX) return SV_EUNSUPPORTED;
  size_t off = kWsFixed;
  pl->off_part1 = off;
  off = align_up(off + (size_t)rows * pl->nch1 * sizeof(Partial), 256);
  pl->off_part2 = off;  // gathered logits of the drafted tokens (target, then draft)
  off = align_up(off + (size_t)2 * B * K * gamma * sizeof(float), 256);
  pl->bytes = off;
  return SV_OK;
}

sv_status plan_greedy(sv_dtype dt, int32_t B, int32_t gamma, int32_t V, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (B < 0 || gamma < 1 || V < 1) return SV_EINVAL;
  if (B > SV_MAX_SEQ || gamma > SV_MAX_GAMMA || V > SV_MAX_V) return SV_EUNSUPPORTED;
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  const int64_t rows = (int64_t)B * (gamma + 1);
  split(rows, pl->nvec, stats_blocks(), &pl->nch1, &pl->vpc1);
  pl->grid1 = rows * pl->nch1;
  if (pl->grid1 > INT32_MAX) return SV_EUNSUPPORTED;
  size_t off = kWsFixed;
  pl->off_part1 = off;
  off = align_up(off + (size_t)rows * pl->nch1 * 8, 256);
  pl->bytes = off;
  return SV_OK;
}

constexpr int kWalkMaxParts = 64; // stats parts per row the walk stages

sv_status plan_tree(sv_dtype dt, int32_t B, int32_t N, int32_t V, bool pm, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (B < 0 || N < 1 || V < 1) return SV_EINVAL;
  if (B > SV_MAX_SEQ || N > SV_MAX_N || V > SV_MAX_V) return SV_EUNSUPPORTED;
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  const int64_t rows = (int64_t)B * N * (pm ? 1 : 2);
  // only rows of nodes with children are streamed (about half of them in a
  // bushy tree), by the blocks at the front of the grid: aim the block count
  // at twice the usual target, so that about the usual number stream
  split(rows, pl->nvec, 2 * stats_blocks(), &pl->nch1, &pl->vpc1);
  if (pl->nch1 > kWalkMaxParts) {
    pl->vpc1 = (pl->nvec + kWalkMaxParts - 1) / kWalkMaxParts;
    pl->nch1 = (int32_t)((pl->nvec + pl->vpc1 - 1) / pl->vpc1);
  }
  pl->grid1 = rows * pl->nch1;
  if (pl->grid1 > INT32_MAX) return SV_EUNSUPPORTED;
  size_t off = kWsFixed;
  pl->off_part1 = off;
  off = align_up(off + (size_t)rows * pl->nch1 * sizeof(Partial), 256);
  pl->off_jobs = off;  // walk slot words
  off = align_up(off + (size_t)B * kSlotWords * g_cap(B) * sizeof(uint64_t), 256);
  pl->off_part2 = off;  // gathered child logits
  off = align_up(off + (size_t)2 * B * N * sizeof(float), 256);
  pl->bytes = off;
  return SV_OK;
}

sv_status plan_fanout(sv_dtype dt, int32_t R, int32_t V, int32_t F_max, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (R < 0 || V < 1 || F_max < 1) return SV_EINVAL;
  if (R > (int32_t)kWsCounters || V > SV_MAX_V || F_max > SV_MAX_FANOUT) return SV_EUNSUPPORTED;
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  // 512-thread blocks: half the usual block count
  split(R, pl->nvec, stats_blocks() / 2, &pl->nch1, &pl->vpc1);
  pl->grid1 = (int64_t)R * pl->nch1;
  if (pl->grid1 > INT32_MAX) return SV_EUNSUPPORTED;
  size_t off = kWsFixed;
  pl->off_part1 = off;
  off = align_up(off + (size_t)R * pl->nch1 * F_max * 8, 256);
  pl->bytes = off;
  return SV_OK;
}

// Cache hit test: one row per sequence, split so the launch has about the
// usual block count; the per-sequence words live in the counter region.
sv_status plan_cache(sv_dtype dt, int32_t B, int32_t K, int32_t V, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (B < 0 || K < 0 || V < 1) return SV_EINVAL;
  if (B > SV_MAX_SEQ || K > SV_MAX_GAMMA || V > SV_MAX_V) return SV_EUNSUPPORTED;
  static_assert((size_t)SV_MAX_SEQ * sizeof(uint64_t) <= kWsCounters * sizeof(uint32_t), "cache words");
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  split(B, pl->nvec, stats_blocks(), &pl->nch1, &pl->vpc1);
  pl->grid1 = (int64_t)B * pl->nch1;
  if (pl->grid1 > INT32_MAX) return SV_EUNSUPPORTED;
  pl->bytes = kWsFixed;
  return SV_OK;
}

// PRESTO scoring: statistics of every node's row pair (all rows stream), then
// the expansion over the same rows (only leaves work); k proposals per part.
sv_status plan_presto(sv_dtype dt, int32_t B, int32_t N, int32_t V, int32_t k, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (B < 0 || N < 1 || V < 1 || k < 1) return SV_EINVAL;
  if (B > SV_MAX_SEQ || N > SV_MAX_N || V > SV_MAX_V || k > SV_MAX_FANOUT) return SV_EUNSUPPORTED;
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  const int64_t rows = (int64_t)B * N * 2;
  split(rows, pl->nvec, stats_blocks(), &pl->nch1, &pl->vpc1);
  if (pl->nch1 > kWalkMaxParts) {  // the expansion stages a row's parts in LDS
    pl->vpc1 = (pl->nvec + kWalkMaxParts - 1) / kWalkMaxParts;
    pl->nch1 = (int32_t)((pl->nvec + pl->vpc1 - 1) / pl->vpc1);
  }
  // the proposal scan costs a few operations per token and only leaves
  // (about half the nodes) work: twice the usual block count, with at most
  // 1024 / k parts per row (a leaf's last part merges the parts' lists)
  split((int64_t)B * N, pl->nvec, 2 * stats_blocks(), &pl->nch2, &pl->vpc2);
  const int32_t max_parts = 1024 / k;
  if (pl->nch2 > max_parts) {
    pl->vpc2 = (pl->nvec + max_parts - 1) / max_parts;
    pl->nch2 = (int32_t)((pl->nvec + pl->vpc2 - 1) / pl->vpc2);
  }
  pl->grid1 = rows * pl->nch1;
  pl->grid2 = (int64_t)B * N * pl->nch2;
  if (pl->grid1 > INT32_MAX || pl->grid2 > INT32_MAX) return SV_EUNSUPPORTED;
  size_t off = kWsFixed;
  pl->off_part1 = off;
  off = align_up(off + (size_t)rows * pl->nch1 * sizeof(Partial), 256);
  pl->off_part2 = off;  // gathered child logits, then each leaf's merged list (8-byte entries)
  off = align_up(off + (size_t)2 * B * N * sizeof(float), 256);
  off = align_up(off + (size_t)B * N * k * 8, 256);
  pl->off_lists = off;  // expansion part lists (8-byte entries)
  off = align_up(off + (size_t)B * N * pl->nch2 * k * 8, 256);
  pl->off_jobs = off;   // per-node arrival counters, zeroed by the statistics launch
  off = align_up(off + (size_t)B * N * sizeof(uint32_t) + 8, 256);
  pl->bytes = off;
  return SV_OK;
}

// SpecBranch fork: statistics of the gamma + 1 draft rows of every sequence,
// then one row per sequence scanned by several blocks.
sv_status plan_branch(sv_dtype dt, int32_t B, int32_t gamma, int32_t V, int32_t k_max, Plan* pl) {
  if (bad_dtype(dt)) return SV_EDTYPE;
  if (B < 0 || gamma < 1 || V < 1 || k_max < 1) return SV_EINVAL;
  if (B > SV_MAX_SEQ || gamma > SV_MAX_GAMMA || V > SV_MAX_V || k_max > SV_MAX_FANOUT) return SV_EUNSUPPORTED;
  pl->nvec = (V + per_vec(dt) - 1) / per_vec(dt);
  const int64_t rows = (int64_t)B * (gamma + 1);
  split(rows, pl->nvec, stats_blocks(), &pl->nch1, &pl->vpc1);
  split(B, pl->nvec, stats_blocks(), &pl->nch2, &pl->vpc2);
  // fork parts of at most 4 vectors per thread keep their vectors in
  // registers for the top-k's second pass; take them when that at most
  // doubles the part count
  constexpr int64_t kForkHeldVecs = 4 * 256;
  if (pl->vpc2 > kForkHeldVecs && (pl->nvec + kForkHeldVecs - 1) / kForkHeldVecs <= 2 * (int64_t)pl->nch2) {
    pl->vpc2 = kForkHeldVecs;
    pl->nch2 = (int32_t)((pl->nvec + kForkHeldVecs - 1) / kForkHeldVecs);
  }
  pl->grid1 = rows * pl->nch1;
  pl->grid2 = (int64_t)B * pl->nch2;
  if (pl->grid1 > INT32_MAX || pl->grid2 > INT32_MAX) return SV_EUNSUPPORTED;
  size_t off = kWsFixed;
  pl->off_part1 = off;
  off = align_up(off + (size_t)rows * pl->nch1 * sizeof(Partial), 256);
  pl->off_part2 = off;  // gathered draft logits
  off = align_up(off + (size_t)B * gamma * sizeof(float), 256);
  pl->off_lists = off;  // fork part lists (8-byte entries)
  off = align_up(off + (size_t)B * pl->nch2 * k_max * 8, 256);
  pl->bytes = off;
  return SV_OK;
}

sv_status check_ws(const void* ws, size_t ws_bytes, const Plan& pl) {
  if (!ws || ws_bytes < pl.bytes) return SV_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return SV_EALIGN;
  return SV_OK;
}

float log2e_over(float T) { return (float)(1.4426950408889634 / (double)T); }

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

hipError_t launch_fill_zero(void* ws, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(static_cast<uint32_t*>(ws), n);
  return hipGetLastError();
}

}  // namespace sv

using namespace sv;

extern "C" {

int32_t sv_version(void) { return 1; }

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EDTYPE: return "unsupported dtype";
    case SV_EALIGN: return "logit rows or workspace not 16-byte aligned";
    case SV_EWORKSPACE: return "workspace missing or too small";
    case SV_EUNSUPPORTED: return "shape beyond this build's limits";
    case SV_EHIP: return "HIP launch or copy failed";
    default: return "unknown status";
  }
}

sv_status sv_workspace_size(sv_op op, sv_dtype dt, int32_t B, int32_t K, int32_t gamma_or_N, int32_t V,
                            int32_t F_max, size_t* bytes) {
  if (!bytes) return SV_EINVAL;
  Plan pl;
  sv_status st;
  switch (op) {
    case SV_OP_CHAIN: st = plan_chain(dt, B, 1, gamma_or_N, V, false, &pl); break;
    case SV_OP_MULTI: st = plan_chain(dt, B, K, gamma_or_N, V, false, &pl); break;
    case SV_OP_GREEDY: st = plan_greedy(dt, B, gamma_or_N, V, &pl); break;
    case SV_OP_TREE: st = plan_tree(dt, B, gamma_or_N, V, false, &pl); break;
    case SV_OP_CHAIN_PM: st = plan_chain(dt, B, 1, gamma_or_N, V, true, &pl); break;
    case SV_OP_TREE_PM: st = plan_tree(dt, B, gamma_or_N, V, true, &pl); break;
    case SV_OP_CACHE: st = plan_cache(dt, B, gamma_or_N, V, &pl); break;
    case SV_OP_PRESTO: st = plan_presto(dt, B, gamma_or_N, V, F_max, &pl); break;
    case SV_OP_BRANCH: st = plan_branch(dt, B, gamma_or_N, V, F_max, &pl); break;
    case SV_OP_FANOUT: st = plan_fanout(dt, B, V, F_max, &pl); break;
    default: return SV_EINVAL;
  }
  if (st != SV_OK) return st;
  *bytes = pl.bytes;
  return SV_OK;
}

sv_status sv_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < kWsFixed) return SV_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return SV_EALIGN;
  return launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_get_device_error(void* ws, int32_t* flags, void* stream) {
  if (!ws || !flags) return SV_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t h = 0;
  if (hipMemcpyAsync(&h, ws, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return SV_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SV_EHIP;
  *flags = h;
  if (h != 0 && launch_fill_zero(ws, 4, s) != hipSuccess) return SV_EHIP;
  return SV_OK;
}

static sv_status verify_chain_like(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride,
                                   int64_t drf_stride, const int32_t* tok, int32_t B, int32_t K, int32_t gamma,
                                   int32_t V, float T, uint64_t seed, uint32_t round, int32_t* out_k, int32_t* out_n,
                                   int32_t* out_tok, int32_t* out_n_cand, float* out_p, float* out_q, bool pm,
                                   void* ws, size_t ws_bytes, void* stream, int32_t* err = nullptr) {
  Plan pl;
  sv_status st = plan_chain(dt, B, K, gamma, V, pm, &pl);
  if (st != SV_OK) return st;
  if (bad_temperature(T) || round >= (1u << 30)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  if ((st = check_rows(tgt, tgt_stride, V, dt)) != SV_OK) return st;
  if (!pm && (st = check_rows(drf, drf_stride, V, dt)) != SV_OK) return st;
  if (!tok || !out_n || !out_tok) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  char* w = static_cast<char*>(ws);
  ChainParams p;
  p.tgt = tgt;
  p.drf = drf;
  p.tgt_sb = tgt_stride * elem_bytes(dt);
  p.drf_sb = drf_stride * elem_bytes(dt);
  p.tok = tok;
  p.B = B;
  p.K = K;
  p.gamma = gamma;
  p.V = V;
  p.c = log2e_over(T);
  p.seed = seed;
  p.round = round;
  p.out_k = out_k;
  p.out_n = out_n;
  p.out_tok = out_tok;
  p.out_n_cand = out_n_cand;
  p.out_p = out_p;
  p.out_q = out_q;
  p.err = err ? err : reinterpret_cast<int32_t*>(w);
  p.knobs = err ? nullptr : reinterpret_cast<const uint32_t*>(w);
  // counter region (zero between calls): arrivals and draw exits, B
  // counters each (64 bytes apart for small batches), then the exchange
  // slots, which the kernel also leaves zero
  p.cnt = reinterpret_cast<uint32_t*>(w + kWsHeader);
  p.cstride = B <= 512 ? 16 : 1;
  p.slots = w + kWsHeader + align_up((size_t)8 * B * p.cstride, 256);
  p.part1 = w + pl.off_part1;
  p.zg = reinterpret_cast<float*>(w + pl.off_part2);
  p.zq = p.zg + (int64_t)B * K * gamma;
  p.nch1 = pl.nch1;
  p.grid1 = pl.grid1;
  p.pm = pm;
  p.xcd = B % 8 == 0;
  // all B * G draw blocks fit on the device at once (once the statistics
  // blocks, which are placed first and never wait, have finished)
  pick_slices(B, pl.nvec, chain_capacity(dt, true, pm), chain_capacity(dt, false, pm), &p.G, &p.held);
  if ((int64_t)B * pl.nvec <= kSmallDrawVecs && p.held) {
    // little to draw from: blocks of kSliceTiles full tiles each, so that
    // fewer blocks take part in each exchange
    const int64_t g = (pl.nvec + (int64_t)kSliceTiles * 256 - 1) / ((int64_t)kSliceTiles * 256);
    if (g < p.G) p.G = g < 1 ? 1 : (int32_t)g;
  }
  if (p.G > 1 && align_up((size_t)8 * B * p.cstride, 256) + (size_t)kSlotWords * 8 * B * p.G >
                     kWsCounters * sizeof(uint32_t))
    return SV_EUNSUPPORTED;  // not reached: B * G <= 4096 and B <= 2048 whenever G > 1
  p.vpc1 = pl.vpc1;
  p.nvec = pl.nvec;
  // small calls: every row held by G blocks per sequence, two rounds between
  // blocks (sv_chain_small.hip), when the slots fit the counter region; one
  // tile of 256 vectors per block where the blocks fit (more blocks share the
  // loads and the exponentials: 12.5 against 12.8 us at B=1, gamma=4,
  // V=32000), else two
  const int64_t small_rows = pm ? gamma + 1 : 2 * (int64_t)gamma + 1;
  if (K == 1 && small_rows <= kSmallRows && (int64_t)B * pl.nvec <= kSmallDrawVecs) {
    const size_t cnt_bytes = align_up((size_t)8 * B * p.cstride, 256);
    for (int tiles = 1; tiles <= kSmallTiles; tiles *= 2) {
      const int64_t g = (pl.nvec + (int64_t)tiles * 256 - 1) / ((int64_t)tiles * 256);
      if (g <= kMaxG && (int64_t)B * g <= chain_small_capacity(dt, pm, tiles) &&
          cnt_bytes + (size_t)B * g * (2 * kSmallRows + kSlotWords) * 8 <= kWsCounters * sizeof(uint32_t)) {
        p.G = (int32_t)g;
        return launch_chain_small(p, dt, tiles, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
      }
    }
  }
  return launch_chain(p, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_verify_chain(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                          const int32_t* draft_tok, int32_t B, int32_t gamma, int32_t V, float T, uint64_t seed,
                          uint32_t round, int32_t* out_n, int32_t* out_tok, float* out_p, float* out_q, void* ws,
                          size_t ws_bytes, void* stream) {
  return verify_chain_like(tgt, drf, dt, tgt_stride, drf_stride, draft_tok, B, 1, gamma, V, T, seed, round, nullptr,
                           out_n, out_tok, nullptr, out_p, out_q, false, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free chain verification.  The scratch space is this file-scope
// device array: each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so the array is only ever reached through the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept per device.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of the array (null if the lookup fails).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

sv_status sv_verify_chain_noalloc(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride,
                                  int64_t drf_stride, const int32_t* draft_tok, int32_t B, int32_t gamma, int32_t V,
                                  float T, uint64_t seed, uint32_t round, int32_t* out_n, int32_t* out_tok,
                                  float* out_p, float* out_q, int32_t* out_err, void* stream) {
  // the shape's scratch need, checked before any HIP call
  Plan pl;
  sv_status st = plan_chain(dt, B, 1, gamma, V, false, &pl);
  if (st != SV_OK) return st;
  if (pl.bytes > kScratchBytes) return SV_EUNSUPPORTED;
  if (B == 0) return verify_chain_like(tgt, drf, dt, tgt_stride, drf_stride, draft_tok, B, 1, gamma, V, T, seed,
                                       round, nullptr, out_n, out_tok, nullptr, out_p, out_q, false, nullptr, 0,
                                       stream);
  void* ws = scratch_for_current_device();
  if (!ws) return SV_EHIP;
  // every part and gathered logit the kernel reads is written earlier in
  // the same call, and its arrival counters and exchange slots start at
  // zero (the array starts zeroed and every call leaves them zero), so the
  // previous call's contents need no clearing; device errors go to out_err,
  // or to the array's own error word, which is never read
  return verify_chain_like(tgt, drf, dt, tgt_stride, drf_stride, draft_tok, B, 1, gamma, V, T, seed, round, nullptr,
                           out_n, out_tok, nullptr, out_p, out_q, false, ws, kScratchBytes, stream, out_err);
}

sv_status sv_verify_chain_pm(const void* tgt, sv_dtype dt, int64_t tgt_stride, const int32_t* draft_tok, int32_t B,
                             int32_t gamma, int32_t V, float T, uint64_t seed, uint32_t round, int32_t* out_n,
                             int32_t* out_tok, float* out_p, void* ws, size_t ws_bytes, void* stream) {
  return verify_chain_like(tgt, nullptr, dt, tgt_stride, 0, draft_tok, B, 1, gamma, V, T, seed, round, nullptr, out_n,
                           out_tok, nullptr, out_p, nullptr, true, ws, ws_bytes, stream);
}

sv_status sv_verify_multi(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                          const int32_t* draft_tok, int32_t B, int32_t K, int32_t gamma, int32_t V, float T,
                          uint64_t seed, uint32_t round, int32_t* out_k, int32_t* out_n, int32_t* out_tok,
                          int32_t* out_n_cand, float* out_p, float* out_q, void* ws, size_t ws_bytes, void* stream) {
  if (!out_k) return SV_EINVAL;
  return verify_chain_like(tgt, drf, dt, tgt_stride, drf_stride, draft_tok, B, K, gamma, V, T, seed, round, out_k,
                           out_n, out_tok, out_n_cand, out_p, out_q, false, ws, ws_bytes, stream);
}

sv_status sv_verify_greedy(const void* tgt, sv_dtype dt, int64_t stride, const int32_t* draft_tok, int32_t B,
                           int32_t gamma, int32_t V, int32_t* out_n, int32_t* out_tok, int32_t* out_argmax, void* ws,
                           size_t ws_bytes, void* stream) {
  Plan pl;
  sv_status st = plan_greedy(dt, B, gamma, V, &pl);
  if (st != SV_OK) return st;
  if (B == 0) return SV_OK;
  if ((st = check_rows(tgt, stride, V, dt)) != SV_OK) return st;
  if (!draft_tok || !out_n || !out_tok) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  char* w = static_cast<char*>(ws);
  GreedyParams p;
  p.tgt = tgt;
  p.tgt_sb = stride * elem_bytes(dt);
  p.tok = draft_tok;
  p.B = B;
  p.gamma = gamma;
  p.V = V;
  p.out_n = out_n;
  p.out_tok = out_tok;
  p.out_argmax = out_argmax;
  p.err = reinterpret_cast<int32_t*>(w);
  p.cnt = reinterpret_cast<uint32_t*>(w + kWsHeader);
  p.part = w + pl.off_part1;
  p.nch = pl.nch1;
  p.vpc = pl.vpc1;
  p.nvec = pl.nvec;
  return launch_greedy(p, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

static sv_status verify_tree_like(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride,
                                  int64_t drf_stride, const int32_t* node_tok, const int32_t* parent, int32_t B,
                                  int32_t N, int32_t max_depth, int32_t V, float T, uint64_t seed, uint32_t round,
                                  int32_t* out_len, int32_t* out_path, int32_t* out_tok, float* out_p, float* out_q,
                                  bool pm, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  sv_status st = plan_tree(dt, B, N, V, pm, &pl);
  if (st != SV_OK) return st;
  if (max_depth < 1 || max_depth > SV_MAX_N) return SV_EINVAL;
  if (bad_temperature(T) || round >= (1u << 30)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  if ((st = check_rows(tgt, tgt_stride, V, dt)) != SV_OK) return st;
  if (!pm && (st = check_rows(drf, drf_stride, V, dt)) != SV_OK) return st;
  if (!node_tok || !parent || !out_len || !out_path || !out_tok) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  char* w = static_cast<char*>(ws);
  TreeParams p;
  p.tgt = tgt;
  p.drf = drf;
  p.tgt_sb = tgt_stride * elem_bytes(dt);
  p.drf_sb = drf_stride * elem_bytes(dt);
  p.tok = node_tok;
  p.parent = parent;
  p.B = B;
  p.N = N;
  p.max_depth = max_depth;
  p.V = V;
  p.c = log2e_over(T);
  p.seed = seed;
  p.round = round;
  p.out_len = out_len;
  p.out_path = out_path;
  p.out_tok = out_tok;
  p.out_p = out_p;
  p.out_q = out_q;
  p.err = reinterpret_cast<int32_t*>(w);
  p.knobs = reinterpret_cast<const uint32_t*>(w);
  p.slots = w + pl.off_jobs;
  p.zc = reinterpret_cast<float*>(w + pl.off_part2);
  p.part = w + pl.off_part1;
  p.nch = pl.nch1;
  p.pm = pm;
  p.all_rows = false;
  pick_slices(B, pl.nvec, tree_walk_capacity(dt, true, pm), tree_walk_capacity(dt, false, pm), &p.G, &p.held);
  p.nzero = (int64_t)B * kSlotWords * p.G;
  p.vpc = pl.vpc1;
  p.nvec = pl.nvec;
  return launch_tree(p, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_verify_tree(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                         const int32_t* node_tok, const int32_t* parent, int32_t B, int32_t N, int32_t max_depth,
                         int32_t V, float T, uint64_t seed, uint32_t round, int32_t* out_len, int32_t* out_path,
                         int32_t* out_tok, float* out_p, float* out_q, void* ws, size_t ws_bytes, void* stream) {
  return verify_tree_like(tgt, drf, dt, tgt_stride, drf_stride, node_tok, parent, B, N, max_depth, V, T, seed, round,
                          out_len, out_path, out_tok, out_p, out_q, false, ws, ws_bytes, stream);
}

sv_status sv_verify_tree_pm(const void* tgt, sv_dtype dt, int64_t tgt_stride, const int32_t* node_tok,
                            const int32_t* parent, int32_t B, int32_t N, int32_t max_depth, int32_t V, float T,
                            uint64_t seed, uint32_t round, int32_t* out_len, int32_t* out_path, int32_t* out_tok,
                            float* out_p, void* ws, size_t ws_bytes, void* stream) {
  return verify_tree_like(tgt, nullptr, dt, tgt_stride, 0, node_tok, parent, B, N, max_depth, V, T, seed, round,
                          out_len, out_path, out_tok, out_p, nullptr, true, ws, ws_bytes, stream);
}

sv_status sv_fanout_topk(const void* logits, sv_dtype dt, int64_t stride, int32_t R, int32_t V, const int32_t* F,
                         int32_t F_max, int32_t* out_ids, float* out_vals, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  sv_status st = plan_fanout(dt, R, V, F_max, &pl);
  if (st != SV_OK) return st;
  if (R == 0) return SV_OK;
  if ((st = check_rows(logits, stride, V, dt)) != SV_OK) return st;
  if (!F || !out_ids) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  char* w = static_cast<char*>(ws);
  FanoutParams p;
  p.logits = logits;
  p.sb = stride * elem_bytes(dt);
  p.R = R;
  p.V = V;
  p.F = F;
  p.F_max = F_max;
  p.out_ids = out_ids;
  p.out_vals = out_vals;
  p.err = reinterpret_cast<int32_t*>(w);
  p.cnt = reinterpret_cast<uint32_t*>(w + kWsHeader);
  p.part = w + pl.off_part1;
  p.nch = pl.nch1;
  p.vpc = pl.vpc1;
  p.nvec = pl.nvec;
  return launch_fanout(p, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_cache_hit_test(const void* drf, sv_dtype dt, int64_t stride, int32_t B, int32_t K, int32_t V,
                            const int32_t* n, const int32_t* t, const int32_t* F, int32_t* out_rank, int32_t* out_hit,
                            void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  sv_status st = plan_cache(dt, B, K, V, &pl);
  if (st != SV_OK) return st;
  if (B == 0) return SV_OK;
  if ((st = check_rows(drf, stride, V, dt)) != SV_OK) return st;
  if (!n || !t || !out_rank || (!F) != (!out_hit)) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  char* w = static_cast<char*>(ws);
  CacheParams p;
  p.drf = drf;
  p.sb = stride * elem_bytes(dt);
  p.B = B;
  p.K = K;
  p.V = V;
  p.n = n;
  p.t = t;
  p.F = F;
  p.out_rank = out_rank;
  p.out_hit = out_hit;
  p.err = reinterpret_cast<int32_t*>(w);
  p.words = reinterpret_cast<uint64_t*>(w + kWsHeader);
  p.nch = pl.nch1;
  p.vpc = pl.vpc1;
  p.nvec = pl.nvec;
  return launch_cache(p, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_presto_score(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                          const int32_t* node_tok, const int32_t* parent, int32_t B, int32_t N, int32_t V, float T,
                          const float* lambda, int32_t D, int32_t k, int32_t b_top, float* out_s, float* out_S,
                          int32_t* out_node, int32_t* out_tok, float* out_score, void* ws, size_t ws_bytes,
                          void* stream) {
  Plan pl;
  sv_status st = plan_presto(dt, B, N, V, k, &pl);
  if (st != SV_OK) return st;
  if (bad_temperature(T) || D < 1 || b_top < 1) return SV_EINVAL;
  if (b_top > SV_MAX_FANOUT) return SV_EUNSUPPORTED;
  if (B == 0) return SV_OK;
  if ((st = check_rows(tgt, tgt_stride, V, dt)) != SV_OK) return st;
  if ((st = check_rows(drf, drf_stride, V, dt)) != SV_OK) return st;
  if (!node_tok || !parent || !lambda || !out_node || !out_tok) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  char* w = static_cast<char*>(ws);
  TreeParams t;
  std::memset(&t, 0, sizeof t);
  t.tgt = tgt;
  t.drf = drf;
  t.tgt_sb = tgt_stride * elem_bytes(dt);
  t.drf_sb = drf_stride * elem_bytes(dt);
  t.tok = node_tok;
  t.parent = parent;
  t.B = B;
  t.N = N;
  t.max_depth = N;
  t.V = V;
  t.c = log2e_over(T);
  t.err = reinterpret_cast<int32_t*>(w);
  t.knobs = nullptr;
  t.part = w + pl.off_part1;
  t.zc = reinterpret_cast<float*>(w + pl.off_part2);
  t.slots = w + pl.off_jobs;  // the expansion's per-node arrival counters
  t.nzero = ((int64_t)B * N + 1) / 2;
  t.nch = pl.nch1;
  t.G = 0;
  t.held = true;
  t.pm = false;
  t.all_rows = true;
  t.vpc = pl.vpc1;
  t.nvec = pl.nvec;
  PrestoParams p;
  p.tgt = tgt;
  p.drf = drf;
  p.tgt_sb = t.tgt_sb;
  p.drf_sb = t.drf_sb;
  p.tok = node_tok;
  p.parent = parent;
  p.B = B;
  p.N = N;
  p.V = V;
  p.c = t.c;
  p.lam = lambda;
  p.D = D;
  p.k = k;
  p.b_top = b_top;
  p.out_s = out_s;
  p.out_S = out_S;
  p.out_node = out_node;
  p.out_tok = out_tok;
  p.out_score = out_score;
  p.err = t.err;
  p.part = t.part;
  p.zc = t.zc;
  p.lists = w + pl.off_lists;
  p.leaf_lists = w + pl.off_part2 + align_up((size_t)2 * B * N * sizeof(float), 256);
  p.leaf_cnt = reinterpret_cast<uint32_t*>(w + pl.off_jobs);
  p.nch1 = pl.nch1;
  p.nch2 = pl.nch2;
  p.vpc2 = pl.vpc2;
  p.nvec = pl.nvec;
  return launch_presto(p, t, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_branch_fork(const void* drf, sv_dtype dt, int64_t stride, const int32_t* draft_tok, const int32_t* cls,
                         int32_t B, int32_t gamma, int32_t V, float T, float eps, int32_t k_max, int32_t* out_pos,
                         float* out_qb, int32_t* out_k, int32_t* out_ids, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  sv_status st = plan_branch(dt, B, gamma, V, k_max, &pl);
  if (st != SV_OK) return st;
  if (bad_temperature(T) || !std::isfinite(eps)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  if ((st = check_rows(drf, stride, V, dt)) != SV_OK) return st;
  if (!draft_tok || !out_pos || !out_ids) return SV_EINVAL;
  if ((st = check_ws(ws, ws_bytes, pl)) != SV_OK) return st;
  if (B > (int32_t)kWsCounters) return SV_EUNSUPPORTED;
  char* w = static_cast<char*>(ws);
  BranchParams p;
  p.drf = drf;
  p.sb = stride * elem_bytes(dt);
  p.tok = draft_tok;
  p.cls = cls;
  p.B = B;
  p.gamma = gamma;
  p.V = V;
  p.c = log2e_over(T);
  p.eps = (double)eps;
  p.k_max = k_max;
  p.out_pos = out_pos;
  p.out_qb = out_qb;
  p.out_k = out_k;
  p.out_ids = out_ids;
  p.err = reinterpret_cast<int32_t*>(w);
  p.cnt = reinterpret_cast<uint32_t*>(w + kWsHeader);
  p.part = w + pl.off_part1;
  p.zq = reinterpret_cast<float*>(w + pl.off_part2);
  p.lists = w + pl.off_lists;
  p.nch1 = pl.nch1;
  p.nch2 = pl.nch2;
  p.vpc1 = pl.vpc1;
  p.vpc2 = pl.vpc2;
  p.nvec = pl.nvec;
  return launch_branch(p, dt, pl, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_EHIP;
}

int32_t sv_geometric_fanout(int32_t F0, double a_p, double r, int32_t K, int32_t capped_last, int32_t* F_out) {
  if (!F_out || F0 < 0 || K < 0 || !(a_p > 0.0) || !(a_p < 1.0) || !(r >= 0.0)) return -1;
  int32_t sum = 0;
  for (int32_t k = 0; k <= K; ++k) {
    double f = (double)F0 * std::pow(a_p, (double)k / (1.0 + r));
    if (k == K && capped_last) f *= std::pow(1.0 - a_p, -1.0 / (1.0 + r));
    F_out[k] = (int32_t)std::ceil(f);
    sum += F_out[k];
  }
  return sum;
}

}  // extern "C"

extern "C" sv_status sv_timeline_set(void* buf, uint64_t records) {
#ifdef SV_TIMELINE
  if (!buf) records = 0;
  if (sv::timeline_set_chain(buf, records) != hipSuccess || sv::timeline_set_chain_small(buf, records) != hipSuccess ||
      sv::timeline_set_tree(buf, records) != hipSuccess || sv::timeline_set_fanout(buf, records) != hipSuccess)
    return SV_EHIP;
  return SV_OK;
#else
  (void)buf;
  (void)records;
  return SV_EUNSUPPORTED;
#endif
}
