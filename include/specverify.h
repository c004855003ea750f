/*
 * specverify.h -- C ABI of the MI355X (gfx950) draft-verification library.
 *
 * One call runs the data-parallel acceptance step of lossless speculative
 * decoding on the GPU: temperature softmax of target and draft logit rows,
 * acceptance of each draft token with probability min(1, p(x)/q(x)) against a
 * counter-based uniform, the longest accepted prefix, and the correction token
 * drawn from norm(max(0, p - q)) at the first rejection, or the bonus token
 * drawn from the next target row when every draft is accepted.
 *
 * Definitions followed (page title, section):
 *   - llm-infra-atlas "01 · Draft-then-verify: lossless algorithm core":
 *     §1 (one round, Leviathan Algorithm 1), §2.1 (accept with
 *     min(1, p/q), residual norm(max(0, p - q))), §2.2 (greedy = argmax-id
 *     match), §4 (bonus row; filters applied to both p and q; pseudocode).
 *   - "SpecDiff-2: Scaling Diffusion Drafter Alignment for Faster Speculative
 *     Decoding", Core method (K candidates from shared position marginals,
 *     the verifier keeps the best one).
 *   - "PRESTO: prefix-aligned tree drafting for diffusion speculative
 *     decoding", §2.1 (token tree, accept sequentially from the root until a
 *     mismatch).
 *   - SpecDiff-2 page, Core method, greedy acceptance (the point-mass entry
 *     points: a drafted token is accepted with the verifier's probability of
 *     it, the residual resampled on a rejection, no drafter probabilities).
 *   - "Speculative Speculative Decoding (SSD) / Saguaro" review, §3 (fan-out:
 *     top-F_k tokens of the draft logits per lookahead position k) and
 *     Theorem 12 (geometric F_k).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory on these paths; scratch space is
 *    the caller's workspace `ws` of `ws_bytes` bytes (size from
 *    sv_workspace_size).  A new workspace must be zero-filled once
 *    (sv_workspace_init, or any zero fill); every call leaves it ready for
 *    the next call of any op and any shape.  Calls that share one workspace
 *    must not overlap in time (same stream, or ordered by events).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call is asynchronous: SV_OK means "validated and enqueued".
 *    Launch failures are reported as SV_EHIP; device-side input errors set
 *    bits in the workspace's error word (sv_get_device_error).
 *  - Logit rows: `dt` is SV_BF16 or SV_F32; row r of a logit tensor starts
 *    at base + r * stride elements; the base address and stride * element
 *    size must be multiples of 16 bytes (SV_EALIGN otherwise); stride >= V.
 *    -inf logits mean probability 0; NaN is outside the contract.
 *  - Temperature T > 0 and finite scales target AND draft logits (z / T).
 *  - Uniforms: Philox4x32-10 (Salmon et al., SC'11), key = (seed low 32
 *    bits, seed high 32 bits), counter = (idx, b, k, (round << 2) | tag);
 *    the first output word w gives U = (w >> 8) * 2^-24.  tag 0: acceptance
 *    uniform of chain position idx = j (1-based) of candidate k, or of tree
 *    node idx (k = 0); tag 1: the one sampling uniform of sequence b
 *    (idx = k = 0).  round must be < 2^30.  Same inputs, seed and round give
 *    bit-identical outputs.
 *  - Decisions: accept draft x at a position iff U < p(x)/q(x) (q(x) = 0
 *    with p(x) > 0 always accepts).  Draws: inverse CDF in index order, the
 *    smallest v whose cumulative weight exceeds U * (total weight).
 *  - Device-side preconditions (not checked on the host): token ids in
 *    [0, V); every row has a finite logit; tree parent arrays valid.  A
 *    violation never causes an out-of-bounds access: it sets a bit in the
 *    error word and the affected decision rejects.
 *  - Cross-block waits.  The chain entry points (chain, point-mass chain,
 *    multi, noalloc) run one launch whose draw blocks wait until every
 *    statistics block of their sequence has counted its arrival; they and
 *    the walk launch of the tree entry points split each sequence's final
 *    draw over G blocks that exchange partial sums and wait for each other.
 *    Small chain calls (K = 1, at most 9 rows per sequence to hold, B * V
 *    small) instead run G blocks per sequence that each hold a slice of
 *    every row: they exchange their row statistics, then their draw sums.
 *    G is chosen so that all draw (walk) blocks are resident at once on an
 *    otherwise idle device once the statistics blocks, which never wait,
 *    are done.  A kernel running concurrently on another stream can keep
 *    some of those blocks from starting; the waiting blocks then give up
 *    after a bounded number of polls, set SV_DERR_TIMEOUT, and that call's
 *    outputs are invalid.  The call still completes and leaves the
 *    workspace ready for the next one.
 *  - Workspace header: 32-bit word 0 is the device error word; word 1 bounds
 *    the polls of a cross-block wait (0: the default, 2^22) and word 2 is a
 *    test switch that stops the last block of sequence 0 from publishing
 *    (0: off).  Words 1 and 2 are zero in a zero-filled workspace and are
 *    only set by tests of the bounded waits.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sv_status;
enum {
  SV_OK = 0,
  SV_EINVAL = 1,       /* bad size, null pointer, T <= 0, stride < V, ... */
  SV_EDTYPE = 2,       /* dtype not SV_BF16 / SV_F32 */
  SV_EALIGN = 3,       /* logit base or row stride not 16-byte aligned */
  SV_EWORKSPACE = 4,   /* ws is NULL or ws_bytes below sv_workspace_size */
  SV_EUNSUPPORTED = 5, /* beyond this build's limits (see SV_MAX_*) */
  SV_EHIP = 6          /* a HIP launch or copy failed */
};

typedef int32_t sv_dtype;
enum { SV_F32 = 0, SV_BF16 = 1 };

typedef int32_t sv_op;
enum {
  SV_OP_CHAIN = 0,
  SV_OP_GREEDY = 1,
  SV_OP_MULTI = 2,
  SV_OP_TREE = 3,
  SV_OP_FANOUT = 4,
  SV_OP_CHAIN_PM = 5,
  SV_OP_TREE_PM = 6,
  SV_OP_CACHE = 7,
  SV_OP_PRESTO = 8,
  SV_OP_BRANCH = 9
};

/* Limits of this build. */
#define SV_MAX_GAMMA 64        /* draft positions per chain */
#define SV_MAX_K 64            /* candidates per sequence */
#define SV_MAX_N 1024          /* tree nodes per sequence (root included) */
#define SV_MAX_FANOUT 64       /* F_max of sv_fanout_topk */
#define SV_MAX_V (1 << 24)     /* vocabulary size */
#define SV_MAX_SEQ 32768       /* sequences per call (rows per call for fan-out: 65536) */

/* Device error-word bits (sv_get_device_error). */
#define SV_DERR_TOKEN 1        /* a token id outside [0, V) was seen */
#define SV_DERR_TREE 2         /* parent array invalid, or a path longer than max_depth */
#define SV_DERR_FANOUT 4       /* F[r] outside [0, F_max] */
#define SV_DERR_ROW 8          /* a needed row has no finite logit */
#define SV_DERR_TIMEOUT 16     /* a draw or tree-walk block waited too long for its partners (results invalid) */

int32_t sv_version(void);
const char* sv_status_string(sv_status s);

/*
 * Workspace bytes for one call of `op` with the given shape.  gamma_or_N is
 * gamma (chain, greedy, multi, chain_pm, branch), N (tree, tree_pm, presto)
 * or K (cache); B is the number of sequences (or R, the number of rows, for
 * fan-out); K is used by multi only; F_max by fan-out, as k by presto and as
 * k_max by branch.
 * Returns SV_EINVAL / SV_EUNSUPPORTED for shapes the corresponding call would
 * reject.
 */
sv_status sv_workspace_size(sv_op op, sv_dtype dt, int32_t B, int32_t K, int32_t gamma_or_N, int32_t V,
                            int32_t F_max, size_t* bytes);

/* Zero-fill a workspace on `stream` (a kernel, safe inside graph capture). */
sv_status sv_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Synchronise `stream`, read and clear the workspace's device error word. */
sv_status sv_get_device_error(void* ws, int32_t* flags, void* stream);

/*
 * Chain verification (draft-verification page §1 steps 3-5, §2.1, §4).
 *   tgt   [B, gamma+1, V] rows p_1..p_{gamma+1}; row (b, j) at b*(gamma+1)+j
 *   drf   [B, gamma, V]   rows q_1..q_gamma;     row (b, j) at b*gamma+j
 *   draft_tok [B, gamma] int32, x_j drawn by the drafter from q_j
 * Outputs (device):
 *   out_n   [B] number of accepted drafts n (0..gamma); emitted tokens are
 *           x_1..x_n followed by out_tok
 *   out_tok [B] correction drawn from max(0, p_{n+1} - q_{n+1}) (from
 *           p_{n+1} if that mass rounds to 0), or the bonus from p_{gamma+1}
 *   out_p, out_q [B, gamma] float, p_j(x_j) and q_j(x_j) for every j; may be
 *           NULL (both or either)
 * Reads each needed row once (rows 1..gamma of both tensors), then one row
 * pair (or the bonus row) per sequence.
 */
sv_status sv_verify_chain(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                          const int32_t* draft_tok, int32_t B, int32_t gamma, int32_t V, float T, uint64_t seed,
                          uint32_t round, int32_t* out_n, int32_t* out_tok, float* out_p, float* out_q, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Greedy verification at temperature 0 (draft-verification page §2.2, §4:
 * p and q are one-hot, so acceptance is an id comparison).
 *   tgt [B, gamma+1, V], draft_tok [B, gamma]
 *   g_j = the smallest index attaining the maximum of target row j (values
 *   compared as numbers, -0 == +0); out_n = number of leading j with
 *   x_j == g_j; out_tok = g_{n+1}; out_argmax [B, gamma+1] (may be NULL).
 */
sv_status sv_verify_greedy(const void* tgt, sv_dtype dt, int64_t stride, const int32_t* draft_tok, int32_t B,
                           int32_t gamma, int32_t V, int32_t* out_n, int32_t* out_tok, int32_t* out_argmax, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Multi-candidate self-selection (SpecDiff-2 page, Core method): K drafts per
 * sequence sampled from shared draft marginals, each verified as a chain
 * against its own target rows with its own acceptance uniforms (counter
 * k = candidate); the longest accepted streak is kept (lowest k on ties) and
 * its correction / bonus is drawn with the sequence's sampling uniform.
 * K = 1 gives exactly sv_verify_chain's outputs.
 *   tgt [B, K, gamma+1, V], row (b, k, j) at (b*K + k)*(gamma+1) + j
 *   drf [B, gamma, V] shared by the K candidates
 *   draft_tok [B, K, gamma]
 * Outputs: out_k [B] kept candidate, out_n [B], out_tok [B],
 *   out_n_cand [B, K] (may be NULL), out_p / out_q [B, K, gamma] (may be NULL).
 */
sv_status sv_verify_multi(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                          const int32_t* draft_tok, int32_t B, int32_t K, int32_t gamma, int32_t V, float T,
                          uint64_t seed, uint32_t round, int32_t* out_k, int32_t* out_n, int32_t* out_tok,
                          int32_t* out_n_cand, float* out_p, float* out_q, void* ws, size_t ws_bytes, void* stream);

/*
 * Tree verification (PRESTO page §2.1; draft-verification page §2.1 rule at
 * every child).  Node 0 is the root (its token is ignored); parent[i] < i for
 * i >= 1.  Node u's rows P_u (tgt) and Q_u (drf) are the target and draft
 * distributions of u's children.  From the root, children are tried in
 * increasing node index: child c is accepted iff U_c < p_cur(tok_c) /
 * q(tok_c); after a rejection the residual becomes
 * p_cur <- norm(max(0, p_cur - q)), i.e. (p - c_i q)^+ / D_i with
 * c_{i+1} = c_i + D_i and D_i its mass (one pass over the row pair).
 * An accepted child becomes the current node.  When every child is
 * rejected the correction is drawn from the last residual; a node without
 * children gives the bonus draw from its P row.
 *   tgt, drf [B, N, V], row (b, i) at b*N + i (leaf draft rows are not read)
 *   node_tok, parent [B, N] int32
 * Outputs: out_len [B] accepted path length (<= max_depth), out_path
 *   [B, max_depth] accepted node ids in order (-1 padded), out_tok [B];
 *   out_p / out_q [B, N] (may be NULL): p(tok_i), q(tok_i) of the base
 *   distributions for every child i that was tried (others untouched).
 */
sv_status sv_verify_tree(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                         const int32_t* node_tok, const int32_t* parent, int32_t B, int32_t N, int32_t max_depth,
                         int32_t V, float T, uint64_t seed, uint32_t round, int32_t* out_len, int32_t* out_path,
                         int32_t* out_tok, float* out_p, float* out_q, void* ws, size_t ws_bytes, void* stream);

/*
 * sv_verify_chain for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and outputs, with no workspace argument.
 * Its scratch space is a device array of SV_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; the call allocates and
 * frees nothing.  Shapes whose chain workspace (sv_workspace_size with
 * SV_OP_CHAIN) exceeds that size are rejected with SV_EUNSUPPORTED before
 * anything is enqueued.  Every call on one GPU uses that GPU's array: calls
 * that overlap in time on one GPU (other streams, other host threads) race
 * and must be ordered by the caller.  Device-side input errors are OR-ed into
 * *out_err (a device int32 the caller zeroes before the call; NULL: not
 * reported).  The array is looked up on the first call on each device (with
 * that device current); SV_EHIP if that lookup fails.
 */
#define SV_NOALLOC_SCRATCH_BYTES (8u << 20)
sv_status sv_verify_chain_noalloc(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride,
                                  int64_t drf_stride, const int32_t* draft_tok, int32_t B, int32_t gamma, int32_t V,
                                  float T, uint64_t seed, uint32_t round, int32_t* out_n, int32_t* out_tok,
                                  float* out_p, float* out_q, int32_t* out_err, void* stream);

/*
 * Point-mass ("greedy acceptance") chain verification: SpecDiff-2 page, Core
 * method, read as the draft-then-verify page's §2.1 step with the draft
 * distribution a point mass at the drafted token (q = delta_x).  Lossless for
 * any drafter, and no draft logits are read.
 *   tgt [B, gamma+1, V] rows p_1..p_{gamma+1} as in sv_verify_chain;
 *   draft_tok [B, gamma] int32 (any tokens in [0, V): sampled, argmax, ...)
 * Decision: accept x_j iff U_j < p_j(x_j) (U_j as for sv_verify_chain).
 * Outputs (device):
 *   out_n   [B] accepted drafts n (0..gamma)
 *   out_tok [B] correction drawn from p_{n+1} with x_{n+1} removed (from
 *           p_{n+1} itself if what is left rounds to 0), or the bonus from
 *           p_{gamma+1}
 *   out_p   [B, gamma] float p_j(x_j) for every j; may be NULL
 * Reads target rows 1..gamma once, then one row per sequence.  Workspace:
 * SV_OP_CHAIN_PM.
 */
sv_status sv_verify_chain_pm(const void* tgt, sv_dtype dt, int64_t tgt_stride, const int32_t* draft_tok, int32_t B,
                             int32_t gamma, int32_t V, float T, uint64_t seed, uint32_t round, int32_t* out_n,
                             int32_t* out_tok, float* out_p, void* ws, size_t ws_bytes, void* stream);

/*
 * Point-mass tree verification (PRESTO page §2.1, sequential acceptance from
 * the root, with the point-mass step of sv_verify_chain_pm at every child).
 * Tree layout, max_depth, uniforms and outputs as for sv_verify_tree, without
 * draft rows.  At a node the children are tried in increasing index against a
 * running residual w (initially p_node, mass D = 1): child i is accepted iff
 * U_i < w(x_i) / D; a rejection removes x_i from w (D -= w(x_i), w(x_i) = 0),
 * so a sibling repeating a rejected token is rejected.  When every child is
 * rejected the correction is drawn from w (from p_node if w rounds to 0);
 * a node without children (or at max_depth) gives the bonus draw from its
 * row.  Lossless for any sibling tokens, deterministic top-F ones included.
 *   out_p [B, N] float: p_parent(x_i) of every child tried (untouched
 *         otherwise); may be NULL
 * Reads the target rows of nodes with children once, then one row per
 * sequence.  Workspace: SV_OP_TREE_PM.
 */
sv_status sv_verify_tree_pm(const void* tgt, sv_dtype dt, int64_t tgt_stride, const int32_t* node_tok,
                            const int32_t* parent, int32_t B, int32_t N, int32_t max_depth, int32_t V, float T,
                            uint64_t seed, uint32_t round, int32_t* out_len, int32_t* out_path, int32_t* out_tok,
                            float* out_p, void* ws, size_t ws_bytes, void* stream);

/*
 * Top-F fan-out (SSD / Saguaro review §3): for each row r the F[r] largest
 * logits, ordered by value descending and index ascending on ties.
 *   logits [R, V]; F [R] device int32 with 0 <= F[r] <= F_max
 *   out_ids [R, F_max] (-1 padded); out_vals [R, F_max] float (may be NULL,
 *   -inf padded)
 */
sv_status sv_fanout_topk(const void* logits, sv_dtype dt, int64_t stride, int32_t R, int32_t V, const int32_t* F,
                         int32_t F_max, int32_t* out_ids, float* out_vals, void* ws, size_t ws_bytes, void* stream);

/*
 * Speculation-cache hit test (SSD / Saguaro review §3, cache strategy: the
 * cache holds the top-F_k draft tokens of every lookahead position k = 0..K;
 * an outcome (n, t) -- n drafts accepted, then token t -- is served iff t is
 * among the tokens cached for position n, the hit event of Definition 11).
 *   drf [B, K+1, V] draft logits per lookahead position; row (b, k) at
 *       b*(K+1) + k (0 <= K <= SV_MAX_GAMMA)
 *   n, t [B] device int32: the realised outcome (e.g. out_n / out_tok of a
 *       verification call)
 *   F [K+1] device int32 fan-out per position (e.g. sv_geometric_fanout), or
 *       NULL together with out_hit
 * Outputs (device):
 *   out_rank [B] the 0-based position of t in draft row (b, n) under the
 *            fan-out's order (value descending, index ascending on equal
 *            values): #{v : z_v > z_t, or z_v == z_t and v < t}; so t is
 *            cached iff out_rank < F[n], and out_rank + 1 is the smallest
 *            fan-out that would have cached it
 *   out_hit  [B] 1 iff out_rank[b] < F[n[b]], else 0 (may be NULL with F)
 * n outside [0, K] or t outside [0, V) sets SV_DERR_TOKEN and gives rank -1,
 * hit 0.  Reads one draft row per sequence.  Workspace: SV_OP_CACHE (the
 * fixed part only).
 */
sv_status sv_cache_hit_test(const void* drf, sv_dtype dt, int64_t stride, int32_t B, int32_t K, int32_t V,
                            const int32_t* n, const int32_t* t, const int32_t* F, int32_t* out_rank, int32_t* out_hit,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * PRESTO prefix-aligned scoring and one priority expansion step ("PRESTO:
 * prefix-aligned tree drafting for diffusion speculative decoding", §4.1
 * eq. 9-10, §4.2, §4.3 self-speculative form: the tree's target rows give
 * the acceptance probability exactly).  Tree layout as for sv_verify_tree:
 * node u's rows P_u (tgt) and Q_u (drf) are the distributions of u's
 * children; depth(0) = 0, depth(i) = depth(parent(i)) + 1; lambda of depth
 * d >= 1 is lambda[min(d, D) - 1] (device float array of D >= 1 values).
 * Token score of a token t under node u at child depth d (natural log):
 *   s_u(t) = log Q_u(t) + lambda_d * log min(1, P_u(t) / Q_u(t))
 * (-inf where Q_u(t) = 0, or where P_u(t) = 0 and lambda_d > 0; lambda_d = 0
 * gives log Q_u(t)), i.e. the log of the proxy q * rho^lambda of §4.4 up to
 * its normaliser.
 * Outputs (device):
 *   out_s [B, N] s_i = s_{parent(i)}(tok_i) for i >= 1, 0 for the root
 *   out_S [B, N] path score, the sum of s along the root-to-i path (eq. 10)
 *   (out_s / out_S may be NULL)
 *   out_node, out_tok [B, b_top], out_score [B, b_top] (may be NULL): one
 *     expansion step from the leaves (nodes without children): each leaf u
 *     proposes its k best tokens by s_u(t) (score descending, token
 *     ascending; -inf scores are not proposed), a proposal's priority is
 *     S_u + s_u(t), and the b_top best proposals of the sequence are listed
 *     by priority descending, then node ascending, then token ascending;
 *     padded with node -1, token -1, score -inf.
 * 1 <= k, b_top <= SV_MAX_FANOUT.  Reads every node's row pair twice at most
 * (statistics, then the leaves' rows for the proposals).  Device errors: a
 * token outside [0, V) (its s is -inf), an invalid parent array, a row
 * without a finite logit.  Workspace: SV_OP_PRESTO with gamma_or_N = N and
 * F_max = k.
 */
sv_status sv_presto_score(const void* tgt, const void* drf, sv_dtype dt, int64_t tgt_stride, int64_t drf_stride,
                          const int32_t* node_tok, const int32_t* parent, int32_t B, int32_t N, int32_t V, float T,
                          const float* lambda, int32_t D, int32_t k, int32_t b_top, float* out_s, float* out_S,
                          int32_t* out_node, int32_t* out_tok, float* out_score, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * SpecBranch branch resampling ("SpecBranch: Speculative Decoding via Hybrid
 * Drafting and Rollback-Aware Branch Parallelism" notes, key designs 2-3).
 * The hybrid predictor's class per sequence (a trained network's output,
 * passed in) places the branch point b on the window's positions 1..gamma+1:
 *   cls 0: b = 1 (the round's first token);
 *   cls 1: b = the first j with q_j(x_j) < eps (b = gamma + 1 if none);
 *   cls 2: b = gamma + 1 (the next round's first token);
 * then k = max(1, floor(k_max * (1 - q(x_b)))) branches are the k largest
 * logits of draft row b (value descending, index ascending).  At
 * b = gamma + 1 no token is drafted: x_b is the row's most likely token, so
 * q(x_b) = max_v q_{gamma+1}(v).  q = softmax(z / T).
 *   drf [B, gamma+1, V] draft rows q_1..q_{gamma+1}; row (b, j) at
 *       b*(gamma+1) + (j-1)
 *   draft_tok [B, gamma] x_1..x_gamma; cls [B] device int32 or NULL (every
 *       class 1; a class outside {0, 1, 2} sets SV_DERR_TOKEN and reads as 1)
 * Outputs (device): out_pos [B] b (1-based); out_qb [B] q(x_b) (may be NULL);
 *   out_k [B] (may be NULL); out_ids [B, k_max] the branches (-1 padded).
 * 1 <= k_max <= SV_MAX_FANOUT.  Reads the gamma + 1 draft rows once, then
 * the branch row.  Workspace: SV_OP_BRANCH with gamma_or_N = gamma and
 * F_max = k_max.
 */
sv_status sv_branch_fork(const void* drf, sv_dtype dt, int64_t stride, const int32_t* draft_tok, const int32_t* cls,
                         int32_t B, int32_t gamma, int32_t V, float T, float eps, int32_t k_max, int32_t* out_pos,
                         float* out_qb, int32_t* out_k, int32_t* out_ids, void* ws, size_t ws_bytes, void* stream);

/*
 * Measurement aid (not a step of the method): reads the 16-byte vectors at
 * `buf` (DEVICE, 16-byte aligned; `bytes` rounded down to a multiple of 16)
 * with the row statistics kernels' load pattern -- 16-byte non-temporal
 * loads, `unroll` (2, 4 or 8) in flight per thread and the next `unroll`
 * issued before the current ones are used, blocks of 256 threads -- so that
 * the HBM read rate a launch shape reaches on this device can be timed beside
 * those kernels.  `mode` 0: `blocks` blocks over contiguous ranges; 1: the
 * same ranges grouped so that each of the 8 XCDs streams one contiguous
 * eighth (`blocks` a multiple of 8); 2: `blocks` persistent blocks taking
 * chunks of `chunk_bytes` (a multiple of 16, at least 4096) from a
 * device-wide counter.  `sink` (DEVICE, 3 x uint32, zero before the first
 * call) holds a store sink and mode 2's counters, which the kernel returns to
 * zero as it exits; calls that share a sink must not overlap.  SV_EINVAL on
 * any other argument value.  Asynchronous on `stream`.
 */
sv_status sv_read_probe(const void* buf, size_t bytes, int32_t blocks, int32_t mode, int32_t unroll,
                        size_t chunk_bytes, void* sink, void* stream);

/*
 * Measurement aid (not a step of the method): per-block wall-clock timelines.
 * A library built with -DSV_TIMELINE (libspecverify_timeline.so, from
 * `python -m lossless_draft_verification_04_amd.build --timeline`) makes
 * thread 0 of every block of the chain, small-call chain, tree and fan-out kernels
 * store the 100 MHz wall clock (s_memrealtime) at the end of each phase into
 * `buf` (DEVICE, `records` x 16 uint64 words, zero-filled by the caller):
 * record r holds block r of a launch, word 15 a tag (role | sequence << 8 |
 * XCD << 40; roles 1/2 chain statistics/draw blocks, 3 small-call chain, 4/5
 * tree statistics/walk, 6 fan-out), and a tree call's walk launch writes records from
 * 16384 on.  Blocks past `records` store nothing.  NULL stops the recording.
 * A stamp is one store per phase per block, so a timeline build runs close to
 * the normal one, but it is for measurement only.  The normal build returns
 * SV_EUNSUPPORTED.  Synchronous (call it while no kernel of the library runs).
 */
sv_status sv_timeline_set(void* buf, uint64_t records);

/*
 * Host helper, SSD / Saguaro review Theorem 12: F_k = ceil(F0 * a_p^(k/(1+r)))
 * for k < K; F_K uses the capped term F0 * a_p^(K/(1+r)) * (1-a_p)^(-1/(1+r))
 * when capped_last != 0, the plain term otherwise.  Writes K+1 values to the
 * HOST array F_out and returns their sum (-1 on invalid arguments).
 */
int32_t sv_geometric_fanout(int32_t F0, double a_p, double r, int32_t K, int32_t capped_last, int32_t* F_out);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
