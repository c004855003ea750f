// sv_oracle.cpp -- plain, single-threaded, fp64 CPU oracle for the lossless
// draft-verification acceptance step.
//
// TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
// the tests, the smoke check and the CPU-baseline leg of the benchmark may load
// it.  It shares no source, header, table or helper with the HIP library; the
// two meet only in the seeded input bytes they are both handed.
//
// Sources (the pages this follows; all formulas are restated, not pasted):
//   [DV]  llm-infra-atlas, "01 · Draft-then-verify: lossless algorithm core":
//         §1 (one round of speculative decoding, Leviathan Algorithm 1),
//         §2.1 (single-step rejection sampling: accept with min(1, p/q), else
//         draw from norm(max(0, p - q))), §2.2 (greedy = argmax-id match),
//         §4 (bonus row, filters applied to both p and q, pseudocode of one
//         round).
//   [SD2] "SpecDiff-2: Scaling Diffusion Drafter Alignment ..." wiki summary,
//         "Core method": K candidates drawn from shared position-wise
//         marginals, the verifier keeps the best one; greedy acceptance (the
//         chosen token accepted by a Bernoulli of the verifier probability,
//         the residual resampled on rejection, no drafter probability).
//   [PR]  "PRESTO: prefix-aligned tree drafting ...", §2.1 (token tree,
//         sequential acceptance from the root until a mismatch).
//   [SSD] "Speculative Speculative Decoding (SSD) / Saguaro" review, §3
//         fan-out definition and Theorem 12 (geometric fan-out F_k).
//   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
//         Easy as 1, 2, 3", SC'11 (the counter-based generator both sides use
//         for the verifier's uniforms).
//
// Readings taken where the pages leave a step open are listed in the header
// comment of each function (accept on r < a; residual row n+1; inverse-CDF
// sampling in index order; sibling residual updates with the node's draft q
// held fixed; ties to the lowest index).
//
// Everything is computed in double: bf16 and fp32 inputs convert exactly.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>
#include <algorithm>

namespace {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kF64 = 2;

constexpr double kInf = std::numeric_limits<double>::infinity();

// ---------------------------------------------------------------------------
// Philox4x32-10 (SC'11).  One round maps counter (c0,c1,c2,c3) under key
// (k0,k1) to (hi(B*c2)^c1^k0, lo(B*c2), hi(A*c0)^c3^k1, lo(A*c0)) with the
// paper's multipliers A = 0xD2511F53, B = 0xCD9E8D57; between rounds the key
// is bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85).  Ten rounds.
// ---------------------------------------------------------------------------
void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t pa = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    const uint64_t pb = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    const uint32_t hi_a = (uint32_t)(pa >> 32), lo_a = (uint32_t)pa;
    const uint32_t hi_b = (uint32_t)(pb >> 32), lo_b = (uint32_t)pb;
    const uint32_t n0 = hi_b ^ c[1] ^ k0;
    const uint32_t n1 = lo_b;
    const uint32_t n2 = hi_a ^ c[3] ^ k1;
    const uint32_t n3 = lo_a;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

// The verifier's uniform for (idx, b, k, round, tag): key = the 64-bit seed
// split into (low word, high word); counter = (idx, b, k, (round << 2) | tag).
// tag 0 = acceptance uniform (idx = 1-based chain position, or the tree node
// being tested), tag 1 = the one sampling uniform per sequence (idx = k = 0).
// The first output word w maps to (w >> 8) * 2^-24, a 24-bit grid in [0, 1).
double draw_uniform(uint64_t seed, uint32_t idx, uint32_t b, uint32_t k, uint32_t round, uint32_t tag) {
  const uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  const uint32_t ctr[4] = {idx, b, k, (round << 2) | (tag & 3u)};
  uint32_t out[4];
  philox4x32_10(ctr, key, out);
  return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

double load_logit(const void* base, int dtype, int64_t i) {
  if (dtype == kF32) return (double)((const float*)base)[i];
  if (dtype == kF64) return ((const double*)base)[i];
  const uint16_t h = ((const uint16_t*)base)[i];
  const uint32_t bits = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return (double)f;
}

// Temperature softmax of one logit row, [DV] §1 ("any sampler reduces to
// standard sampling of an adjusted distribution") and §4 (the same adjustment
// is applied to p and to q).  p(v) = exp((z_v - M)/T) / sum_w exp((z_w - M)/T)
// with M the row maximum.  A -inf logit is probability 0.  Returns false for a
// row with no finite logit (outside the contract).
bool softmax_row(const void* base, int dtype, int64_t row_off, int V, double T, std::vector<double>& p) {
  p.assign((size_t)V, 0.0);
  double M = -kInf;
  for (int v = 0; v < V; ++v) M = std::max(M, load_logit(base, dtype, row_off + v));
  if (!(M > -kInf)) return false;
  double S = 0.0;
  for (int v = 0; v < V; ++v) {
    p[v] = std::exp((load_logit(base, dtype, row_off + v) - M) / T);
    S += p[v];
  }
  for (int v = 0; v < V; ++v) p[v] /= S;
  return true;
}

// Acceptance ratio a = p(x)/q(x) of [DV] §2.1.  q(x) = 0 with p(x) > 0 is an
// unconditional accept (a = +inf); p(x) = q(x) = 0 never accepts (a = 0).
double accept_ratio(double px, double qx) {
  if (qx > 0.0) return px / qx;
  return px > 0.0 ? kInf : 0.0;
}

// Inverse-CDF draw from unnormalised weights w (>= 0) in index order: the
// smallest v whose cumulative C(v) = sum_{v' <= v} w(v') exceeds u * S, with S
// the total.  The strict ">" never selects a zero-weight cell.  If rounding
// leaves no such v, the last v with w(v) > 0 is taken and the margin is 0.
// margin = distance of u to the nearer edge of the chosen cell, normalised.
int sample_inverse_cdf(const std::vector<double>& w, double u, double* margin) {
  double S = 0.0;
  for (double x : w) S += x;
  const double target = u * S;
  double C = 0.0;
  for (size_t v = 0; v < w.size(); ++v) {
    const double prev = C;
    C += w[v];
    if (C > target) {
      if (margin) *margin = std::min(u - prev / S, C / S - u);
      return (int)v;
    }
  }
  int last = -1;
  for (size_t v = 0; v < w.size(); ++v)
    if (w[v] > 0.0) last = (int)v;
  if (margin) *margin = 0.0;
  return last;
}

// ---------------------------------------------------------------------------
// One chain round for one sequence ([DV] §1 steps 3-5, §4 pseudocode).
//   P[j], j = 0..gamma  : target distributions p_1 .. p_{gamma+1}
//   Q[j], j = 0..gamma-1: draft distributions q_1 .. q_gamma
//   x[j]                : draft tokens x_1 .. x_gamma
//   r[j]                : acceptance uniforms r_1 .. r_gamma
//   u                   : the sampling uniform
// Readings: accept x_j iff r_j < a_j (the page rejects on r > a; the two
// differ only on the tie r = a, a null event for a continuous r, and "<" keeps
// p(x) = 0 never accepted on a discrete grid that contains 0).  At the first
// reject (n accepted, 0-based row n = the rejected position) the correction is
// drawn from max(0, p_{n+1} - q_{n+1}); if that mass is 0 (only by rounding)
// it is drawn from p_{n+1}.  With every draft accepted the bonus is drawn from
// p_{gamma+1}.  a_trace[j] receives a_j for every decision made (NaN after).
// ---------------------------------------------------------------------------
struct ChainResult {
  int n = 0;
  int t = -1;
  double mdec = kInf;  // smallest |r_j - a_j| over the decisions made
  double mcdf = kInf;  // CDF margin of the final draw
  int sample_rows = 0; // logit rows the final draw needs (2 residual, 1 bonus)
};

ChainResult chain_round(const std::vector<std::vector<double>>& P, const std::vector<std::vector<double>>& Q,
                        const int32_t* x, int gamma, const double* r, double u, double* out_p, double* out_q,
                        double* a_trace, std::vector<double>* w_out) {
  ChainResult res;
  for (int j = 0; j < gamma; ++j) {
    const double px = P[j][x[j]], qx = Q[j][x[j]];
    if (out_p) out_p[j] = px;
    if (out_q) out_q[j] = qx;
  }
  if (a_trace)
    for (int j = 0; j < gamma; ++j) a_trace[j] = std::nan("");
  int n = 0;
  for (int j = 0; j < gamma; ++j) {
    const double a = accept_ratio(P[j][x[j]], Q[j][x[j]]);
    if (a_trace) a_trace[j] = a;
    res.mdec = std::min(res.mdec, std::fabs(r[j] - a));
    if (!(r[j] < a)) break;
    ++n;
  }
  res.n = n;
  const size_t V = P[0].size();
  std::vector<double> w(V, 0.0);
  if (n < gamma) {
    double mass = 0.0;
    for (size_t v = 0; v < V; ++v) {
      w[v] = std::max(0.0, P[n][v] - Q[n][v]);
      mass += w[v];
    }
    if (!(mass > 0.0)) w = P[n];
    res.sample_rows = 2;
  } else {
    w = P[gamma];
    res.sample_rows = 1;
  }
  res.t = sample_inverse_cdf(w, u, &res.mcdf);
  if (w_out) *w_out = w;
  return res;
}

// Greedy (temperature 0) verification, [DV] §2.2: p and q are one-hot, so a
// draft is accepted iff it equals the target argmax.  g_j = the smallest
// index attaining the row maximum (compared as numbers, so -0 == +0).
int row_argmax(const void* base, int dtype, int64_t off, int V) {
  double best = -kInf;
  int arg = 0;
  for (int v = 0; v < V; ++v) {
    const double z = load_logit(base, dtype, off + v);
    if (z > best) {
      best = z;
      arg = v;
    }
  }
  return arg;
}

// ---------------------------------------------------------------------------
// Tree round for one sequence ([PR] §2.1: accept sequentially from the root
// until a mismatch; [DV] §2.1 rule at every child; [DV] §4: unchosen siblings
// are discarded).  Node u's rows P_u, Q_u are the target and draft
// distributions over u's children; children of u are the nodes i > u with
// parent[i] == u, tried in increasing index.  Reading for siblings: the single
// step rule is repeated at each sibling with the node's draft q held fixed and
// p replaced by the residual after every rejection, p <- norm(max(0, p - q)).
// The residual after i rejections is (p - c_i q)^+ / D_i with c_0 = 0, D_0 = 1,
// c_{i+1} = c_i + D_i, D_{i+1} = sum_v (p(v) - c_{i+1} q(v))^+ (induction on
// max(0, (p - c q)^+/D - q) = (p - (c + D) q)^+ / D).  When every child is
// rejected the correction is drawn from the last residual; a node without
// children (or the end of the tree) gives the bonus draw from P_u.  A
// residual mass of 0 (rounding only) leaves the residual unchanged.
// ---------------------------------------------------------------------------
struct TreeResult {
  std::vector<int> path;
  int t = -1;
  double mdec = kInf;
  double mcdf = kInf;
  int row_passes = 0;  // logit rows re-read after the main pass: 2 per
                       // residual evaluation (the pair P_u, Q_u), 1 for a
                       // bonus draw from P_u
  bool ok = true;
};

struct TreeInputs {
  const void* tgt;
  const void* drf;
  int dtype;
  int64_t tgt_stride, drf_stride;
  const int32_t* node_tok;  // [N] of this sequence
  const int32_t* parent;    // [N] of this sequence
  int64_t row0;             // row index of node 0 of this sequence
  int N, V, max_depth;
  double T;
};

TreeResult tree_round(const TreeInputs& in, const double* r /*[N], r[i] for child i*/, double u,
                      double* out_p /*[N] or null*/, double* out_q, double* a_trace /*[N] or null*/,
                      std::vector<double>* w_out) {
  TreeResult res;
  if (a_trace)
    for (int i = 0; i < in.N; ++i) a_trace[i] = std::nan("");
  std::vector<double> p, q, w;
  int node = 0;
  for (;;) {
    std::vector<int> kids;
    for (int i = node + 1; i < in.N; ++i)
      if (in.parent[i] == node) kids.push_back(i);
    if (!softmax_row(in.tgt, in.dtype, (in.row0 + node) * in.tgt_stride, in.V, in.T, p)) {
      res.ok = false;
      return res;
    }
    if (kids.empty() || (int)res.path.size() >= in.max_depth) {
      if (!kids.empty()) res.ok = false;  // depth beyond max_depth: outside the contract
      res.row_passes += 1;  // the bonus row
      res.t = sample_inverse_cdf(p, u, &res.mcdf);
      if (w_out) *w_out = p;
      return res;
    }
    if (!softmax_row(in.drf, in.dtype, (in.row0 + node) * in.drf_stride, in.V, in.T, q)) {
      res.ok = false;
      return res;
    }
    double c = 0.0, D = 1.0;
    int accepted = -1;
    for (int ch : kids) {
      const int tok = in.node_tok[ch];
      if (tok < 0 || tok >= in.V) {
        res.ok = false;
        return res;
      }
      if (out_p) out_p[ch] = p[tok];
      if (out_q) out_q[ch] = q[tok];
      const double pcur = std::max(0.0, p[tok] - c * q[tok]) / D;
      const double a = accept_ratio(pcur, q[tok]);
      if (a_trace) a_trace[ch] = a;
      res.mdec = std::min(res.mdec, std::fabs(r[ch] - a));
      if (r[ch] < a) {
        accepted = ch;
        break;
      }
      const double c_next = c + D;
      double G = 0.0;
      for (int v = 0; v < in.V; ++v) G += std::max(0.0, p[v] - c_next * q[v]);
      res.row_passes += 2;
      if (G > 0.0) {
        c = c_next;
        D = G;
      }
    }
    if (accepted >= 0) {
      res.path.push_back(accepted);
      node = accepted;
      continue;
    }
    // every child rejected: draw the correction from (p - c q)^+ (mass D);
    // the last residual evaluation and this draw share one pass.
    w.assign((size_t)in.V, 0.0);
    for (int v = 0; v < in.V; ++v) w[v] = std::max(0.0, p[v] - c * q[v]);
    res.t = sample_inverse_cdf(w, u, &res.mcdf);
    if (w_out) *w_out = w;
    return res;
  }
}

// ---------------------------------------------------------------------------
// Point-mass ("greedy") acceptance, [SD2] "Core method": the chosen draft
// token is accepted with a Bernoulli of the verifier's probability and the
// residual is resampled on a rejection; no drafter probability is used.
// Reading: this is [DV] §2.1's single step with the draft replaced by a point
// mass at the chosen token, q = delta_x.  The acceptance ratio is p(x)/1 and
// the residual max(0, p - delta_x) is p with x removed (mass 1 - p(x)); [DV]
// §2.1's invariance argument holds for any q, so every step returns the
// target law.  Chain: x_j is accepted iff r_j < p_j(x_j); at the first
// rejection (0-based row n) the correction is drawn from p_{n+1} with x_{n+1}
// removed (from p_{n+1} itself if that mass is 0, by rounding only); with
// every draft accepted the bonus is drawn from p_{gamma+1}.  Draft rows are
// not used.  sample_rows = 1 either way.
// ---------------------------------------------------------------------------
ChainResult chain_round_pm(const std::vector<std::vector<double>>& P, const int32_t* x, int gamma, const double* r,
                           double u, double* out_p, double* a_trace, std::vector<double>* w_out) {
  ChainResult res;
  for (int j = 0; j < gamma; ++j)
    if (out_p) out_p[j] = P[j][x[j]];
  if (a_trace)
    for (int j = 0; j < gamma; ++j) a_trace[j] = std::nan("");
  int n = 0;
  for (int j = 0; j < gamma; ++j) {
    const double a = accept_ratio(P[j][x[j]], 1.0);  // q = delta_x: a = p(x)
    if (a_trace) a_trace[j] = a;
    res.mdec = std::min(res.mdec, std::fabs(r[j] - a));
    const bool accept = r[j] < a;
    if (!accept) break;
    ++n;
  }
  res.n = n;
  std::vector<double> w;
  if (n < gamma) {
    w = P[n];
    w[x[n]] = 0.0;  // the rejected token leaves the residual
    double mass = 0.0;
    for (double v : w) mass += v;
    if (!(mass > 0.0)) w = P[n];
  } else {
    w = P[gamma];  // every draft accepted: the bonus row
  }
  res.sample_rows = 1;
  res.t = sample_inverse_cdf(w, u, &res.mcdf);
  if (w_out) *w_out = w;
  return res;
}

// ---------------------------------------------------------------------------
// Tree with point-mass siblings ([PR] §2.1 sequential acceptance from the
// root; the point-mass step above at every child).  At node u the children
// (increasing index) are tried against a running residual w that starts as
// P_u, with mass D = 1: child i is accepted iff r_i < w(x_i) / D; on a
// rejection x_i is removed (D <- D - w(x_i), then w(x_i) <- 0), so a repeated
// sibling token is rejected for sure and removes nothing.  An accepted child
// becomes the current node.  When every child is rejected the correction is
// drawn from w (from P_u if its mass is 0, by rounding only); a node without
// children, or at max_depth, gives the bonus draw from P_u.  Every step is
// exactly lossless whatever the sibling tokens, deterministic top-F ones
// included.  Draft rows are not used; row_passes = 1 (the final draw).
// ---------------------------------------------------------------------------
TreeResult tree_round_pm(const TreeInputs& in, const double* r, double u, double* out_p, double* a_trace,
                         std::vector<double>* w_out) {
  TreeResult res;
  if (a_trace)
    for (int i = 0; i < in.N; ++i) a_trace[i] = std::nan("");
  std::vector<double> p, w;
  int node = 0;
  for (;;) {
    std::vector<int> kids;
    for (int i = node + 1; i < in.N; ++i)
      if (in.parent[i] == node) kids.push_back(i);
    if (!softmax_row(in.tgt, in.dtype, (in.row0 + node) * in.tgt_stride, in.V, in.T, p)) {
      res.ok = false;
      return res;
    }
    res.row_passes = 1;
    if (kids.empty() || (int)res.path.size() >= in.max_depth) {
      if (!kids.empty()) res.ok = false;
      res.t = sample_inverse_cdf(p, u, &res.mcdf);
      if (w_out) *w_out = p;
      return res;
    }
    w = p;
    double D = 1.0;
    int accepted = -1;
    for (int ch : kids) {
      const int tok = in.node_tok[ch];
      if (tok < 0 || tok >= in.V) {
        res.ok = false;
        return res;
      }
      if (out_p) out_p[ch] = p[tok];
      const double a = D > 0.0 ? accept_ratio(w[tok] / D, 1.0) : 0.0;
      if (a_trace) a_trace[ch] = a;
      res.mdec = std::min(res.mdec, std::fabs(r[ch] - a));
      if (r[ch] < a) {
        accepted = ch;
        break;
      }
      D -= w[tok];
      w[tok] = 0.0;
    }
    if (accepted >= 0) {
      res.path.push_back(accepted);
      node = accepted;
      continue;
    }
    double mass = 0.0;
    for (double v : w) mass += v;
    if (!(mass > 0.0)) w = p;
    res.t = sample_inverse_cdf(w, u, &res.mcdf);
    if (w_out) *w_out = w;
    return res;
  }
}

// ---------------------------------------------------------------------------
// PRESTO prefix-aligned scoring ([PR] §4.1, eq. 9-10; §4.3 self-speculative
// form: the target's conditional rows are available, so the acceptance
// probability rho = min(1, p/q) is exact rather than predicted).  Token score
// s = log q(t) + lambda * log rho(t): the log of the KL-regularised proxy
// p* ~ q * rho^lambda up to its normaliser ([PR] §4.4).  lambda = 0 gives
// log q (its rho term is taken as 0 even where rho = 0).  A token with
// q(t) = 0, or with p(t) = 0 while lambda > 0, scores -inf.
// ---------------------------------------------------------------------------
double presto_token_score(double p, double q, double lambda) {
  if (!(q > 0.0)) return -kInf;
  const double logq = std::log(q);
  if (lambda == 0.0) return logq;
  if (!(p > 0.0)) return -kInf;
  const double rho = std::min(1.0, p / q);
  return logq + lambda * std::log(rho);
}

// lambda of a node at depth d >= 1: lam[min(d, D) - 1].
double presto_lambda(const float* lam, int D, int d) { return (double)lam[std::min(d, D) - 1]; }

struct PrestoCand {
  double score;
  int node, tok;
};

}  // namespace

// ===========================================================================
// C interface (ctypes).  Row layouts match the library's:
//   chain : target row (b, j) = b*(gamma+1) + j, draft row (b, j) = b*gamma + j
//   multi : target row (b, k, j) = (b*K + k)*(gamma+1) + j, draft (b, j) shared
//   tree  : target / draft row (b, i) = b*N + i
//   greedy: target row (b, j) = b*(gamma+1) + j
// Strides are in elements.  Return 0 on success, nonzero on invalid input.
// ===========================================================================
extern "C" {

void svo_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) { philox4x32_10(ctr, key, out); }

double svo_uniform(uint64_t seed, uint32_t idx, uint32_t b, uint32_t k, uint32_t round, uint32_t tag) {
  return draw_uniform(seed, idx, b, k, round, tag);
}

// One chain round with explicit uniforms (used by the exact-enumeration pins).
int svo_chain_core(const void* tgt, const void* drf, int dtype, int64_t tgt_stride, int64_t drf_stride,
                   const int32_t* tok, int gamma, int V, double T, const double* r, double u, int32_t* out_n,
                   int32_t* out_tok, double* out_p, double* out_q, double* a_trace, double* w_out /*[V] normalised*/,
                   double* out_mdec, double* out_mcdf) {
  if (gamma < 1 || V < 1 || !(T > 0.0)) return 1;
  std::vector<std::vector<double>> P(gamma + 1), Q(gamma);
  for (int j = 0; j <= gamma; ++j)
    if (!softmax_row(tgt, dtype, (int64_t)j * tgt_stride, V, T, P[j])) return 2;
  for (int j = 0; j < gamma; ++j)
    if (!softmax_row(drf, dtype, (int64_t)j * drf_stride, V, T, Q[j])) return 2;
  for (int j = 0; j < gamma; ++j)
    if (tok[j] < 0 || tok[j] >= V) return 3;
  std::vector<double> w;
  ChainResult res = chain_round(P, Q, tok, gamma, r, u, out_p, out_q, a_trace, &w);
  *out_n = res.n;
  *out_tok = res.t;
  if (w_out) {
    double S = 0.0;
    for (double x : w) S += x;
    for (int v = 0; v < V; ++v) w_out[v] = w[v] / S;
  }
  if (out_mdec) *out_mdec = res.mdec;
  if (out_mcdf) *out_mcdf = res.mcdf;
  return 0;
}

// Batched chain verification with Philox uniforms (the library's
// sv_verify_chain semantics).  out_p/out_q [B*gamma] may be null;
// out_mdec/out_mcdf [B] may be null; out_rows [B] = rows of the final draw.
int svo_verify_chain(const void* tgt, const void* drf, int dtype, int64_t tgt_stride, int64_t drf_stride,
                     const int32_t* tok, int B, int gamma, int V, double T, uint64_t seed, uint32_t round,
                     int32_t* out_n, int32_t* out_tok, double* out_p, double* out_q, double* out_mdec,
                     double* out_mcdf, int32_t* out_rows) {
  if (B < 0 || gamma < 1 || V < 1 || !(T > 0.0)) return 1;
  std::vector<std::vector<double>> P(gamma + 1), Q(gamma);
  std::vector<double> r(gamma);
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j <= gamma; ++j)
      if (!softmax_row(tgt, dtype, ((int64_t)b * (gamma + 1) + j) * tgt_stride, V, T, P[j])) return 2;
    for (int j = 0; j < gamma; ++j)
      if (!softmax_row(drf, dtype, ((int64_t)b * gamma + j) * drf_stride, V, T, Q[j])) return 2;
    const int32_t* x = tok + (int64_t)b * gamma;
    for (int j = 0; j < gamma; ++j)
      if (x[j] < 0 || x[j] >= V) return 3;
    for (int j = 0; j < gamma; ++j) r[j] = draw_uniform(seed, (uint32_t)(j + 1), (uint32_t)b, 0, round, 0);
    const double u = draw_uniform(seed, 0, (uint32_t)b, 0, round, 1);
    ChainResult res = chain_round(P, Q, x, gamma, r.data(), u, out_p ? out_p + (int64_t)b * gamma : nullptr,
                                  out_q ? out_q + (int64_t)b * gamma : nullptr, nullptr, nullptr);
    out_n[b] = res.n;
    out_tok[b] = res.t;
    if (out_mdec) out_mdec[b] = res.mdec;
    if (out_mcdf) out_mcdf[b] = res.mcdf;
    if (out_rows) out_rows[b] = res.sample_rows;
  }
  return 0;
}

// Greedy verification ([DV] §2.2, §4: temperature 0 is an id comparison).
// n = number of leading j with x_j == argmax_j; t = argmax_{n+1}.
int svo_verify_greedy(const void* tgt, int dtype, int64_t stride, const int32_t* tok, int B, int gamma, int V,
                      int32_t* out_n, int32_t* out_tok, int32_t* out_argmax /*[B*(gamma+1)] or null*/) {
  if (B < 0 || gamma < 1 || V < 1) return 1;
  std::vector<int> g(gamma + 1);
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j <= gamma; ++j) g[j] = row_argmax(tgt, dtype, ((int64_t)b * (gamma + 1) + j) * stride, V);
    int n = 0;
    while (n < gamma && tok[(int64_t)b * gamma + n] == g[n]) ++n;
    out_n[b] = n;
    out_tok[b] = g[n];
    if (out_argmax)
      for (int j = 0; j <= gamma; ++j) out_argmax[(int64_t)b * (gamma + 1) + j] = g[j];
  }
  return 0;
}

// Multi-candidate self-selection ([SD2] "Core method"): K drafts share the
// draft marginals q_1..q_gamma; candidate k is verified as a chain against its
// own target rows with its own acceptance uniforms (idx j, k); the candidate
// with the longest accepted streak is kept (lowest k on ties) and its
// correction / bonus is drawn with the sequence's single sampling uniform.
// K = 1 is exactly the chain.  r_in (optional, [B*K*gamma]) and u_in
// (optional, [B]) replace the Philox uniforms (enumeration pins).
int svo_verify_multi(const void* tgt, const void* drf, int dtype, int64_t tgt_stride, int64_t drf_stride,
                     const int32_t* tok /*[B*K*gamma]*/, int B, int K, int gamma, int V, double T, uint64_t seed,
                     uint32_t round, const double* r_in, const double* u_in, int32_t* out_k, int32_t* out_n,
                     int32_t* out_tok, int32_t* out_n_cand /*[B*K] or null*/, double* out_p /*[B*K*gamma]*/,
                     double* out_q, double* out_mdec, double* out_mcdf, int32_t* out_rows) {
  if (B < 0 || K < 1 || gamma < 1 || V < 1 || !(T > 0.0)) return 1;
  std::vector<std::vector<double>> Q(gamma);
  std::vector<std::vector<std::vector<double>>> P(K, std::vector<std::vector<double>>(gamma + 1));
  std::vector<double> r(gamma);
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < gamma; ++j)
      if (!softmax_row(drf, dtype, ((int64_t)b * gamma + j) * drf_stride, V, T, Q[j])) return 2;
    for (int k = 0; k < K; ++k)
      for (int j = 0; j <= gamma; ++j)
        if (!softmax_row(tgt, dtype, (((int64_t)b * K + k) * (gamma + 1) + j) * tgt_stride, V, T, P[k][j])) return 2;
    const double u = u_in ? u_in[b] : draw_uniform(seed, 0, (uint32_t)b, 0, round, 1);
    int best_k = 0, best_n = -1;
    double mdec = kInf;
    std::vector<ChainResult> results(K);
    for (int k = 0; k < K; ++k) {
      const int32_t* x = tok + ((int64_t)b * K + k) * gamma;
      for (int j = 0; j < gamma; ++j)
        if (x[j] < 0 || x[j] >= V) return 3;
      for (int j = 0; j < gamma; ++j)
        r[j] = r_in ? r_in[((int64_t)b * K + k) * gamma + j]
                    : draw_uniform(seed, (uint32_t)(j + 1), (uint32_t)b, (uint32_t)k, round, 0);
      const int64_t o = ((int64_t)b * K + k) * gamma;
      results[k] = chain_round(P[k], Q, x, gamma, r.data(), u, out_p ? out_p + o : nullptr,
                               out_q ? out_q + o : nullptr, nullptr, nullptr);
      mdec = std::min(mdec, results[k].mdec);
      if (out_n_cand) out_n_cand[(int64_t)b * K + k] = results[k].n;
      if (results[k].n > best_n) {
        best_n = results[k].n;
        best_k = k;
      }
    }
    // The kept candidate's draw: chain_round already drew it with the shared
    // u from that candidate's own rows.
    out_k[b] = best_k;
    out_n[b] = best_n;
    out_tok[b] = results[best_k].t;
    if (out_mdec) out_mdec[b] = mdec;
    if (out_mcdf) out_mcdf[b] = results[best_k].mcdf;
    if (out_rows) out_rows[b] = results[best_k].sample_rows;
  }
  return 0;
}

// Tree verification with Philox uniforms; r_in ([B*N], r for child i at
// [b*N + i]) and u_in ([B]) optionally replace them.  out_path [B*max_depth]
// (-1 padded), out_len [B], out_tok [B]; out_p/out_q [B*N] receive p(tok_i)
// and q(tok_i) of every child i tested (untouched otherwise); a_trace [B*N]
// receives the acceptance ratio of every child tested (NaN otherwise);
// w_out [B*V] the normalised weights of the final draw; out_passes [B] the
// logit rows re-read after the main pass (see TreeResult).
int svo_verify_tree(const void* tgt, const void* drf, int dtype, int64_t tgt_stride, int64_t drf_stride,
                    const int32_t* node_tok, const int32_t* parent, int B, int N, int max_depth, int V, double T,
                    uint64_t seed, uint32_t round, const double* r_in, const double* u_in, int32_t* out_len,
                    int32_t* out_path, int32_t* out_tok, double* out_p, double* out_q, double* a_trace,
                    double* w_out, double* out_mdec, double* out_mcdf, int32_t* out_passes) {
  if (B < 0 || N < 1 || max_depth < 1 || V < 1 || !(T > 0.0)) return 1;
  std::vector<double> r(N), w;
  for (int b = 0; b < B; ++b) {
    const int32_t* par = parent + (int64_t)b * N;
    for (int i = 1; i < N; ++i)
      if (par[i] < 0 || par[i] >= i) return 4;
    for (int i = 0; i < N; ++i)
      r[i] = r_in ? r_in[(int64_t)b * N + i] : draw_uniform(seed, (uint32_t)i, (uint32_t)b, 0, round, 0);
    const double u = u_in ? u_in[b] : draw_uniform(seed, 0, (uint32_t)b, 0, round, 1);
    TreeInputs in{tgt, drf, dtype, tgt_stride, drf_stride, node_tok + (int64_t)b * N, par, (int64_t)b * N,
                  N, V, max_depth, T};
    TreeResult res = tree_round(in, r.data(), u, out_p ? out_p + (int64_t)b * N : nullptr,
                                out_q ? out_q + (int64_t)b * N : nullptr, a_trace ? a_trace + (int64_t)b * N : nullptr,
                                w_out ? &w : nullptr);
    if (!res.ok) return 5;
    out_len[b] = (int32_t)res.path.size();
    for (int d = 0; d < max_depth; ++d)
      out_path[(int64_t)b * max_depth + d] = d < (int)res.path.size() ? res.path[d] : -1;
    out_tok[b] = res.t;
    if (w_out) {
      double S = 0.0;
      for (double x : w) S += x;
      for (int v = 0; v < V; ++v) w_out[(int64_t)b * V + v] = w[v] / S;
    }
    if (out_mdec) out_mdec[b] = res.mdec;
    if (out_mcdf) out_mcdf[b] = res.mcdf;
    if (out_passes) out_passes[b] = res.row_passes;
  }
  return 0;
}

// Point-mass chain verification (chain_round_pm): target rows only, laid out
// as for svo_verify_chain.  r_in ([B*gamma]) and u_in ([B]) optionally replace
// the Philox uniforms; a_trace [B*gamma] (NaN where no decision) and w_out
// [B*V] (normalised weights of the final draw) may be null.
int svo_verify_chain_pm(const void* tgt, int dtype, int64_t tgt_stride, const int32_t* tok, int B, int gamma, int V,
                        double T, uint64_t seed, uint32_t round, const double* r_in, const double* u_in,
                        int32_t* out_n, int32_t* out_tok, double* out_p, double* a_trace, double* w_out,
                        double* out_mdec, double* out_mcdf, int32_t* out_rows) {
  if (B < 0 || gamma < 1 || V < 1 || !(T > 0.0)) return 1;
  std::vector<std::vector<double>> P(gamma + 1);
  std::vector<double> r(gamma), w;
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j <= gamma; ++j)
      if (!softmax_row(tgt, dtype, ((int64_t)b * (gamma + 1) + j) * tgt_stride, V, T, P[j])) return 2;
    const int32_t* x = tok + (int64_t)b * gamma;
    for (int j = 0; j < gamma; ++j)
      if (x[j] < 0 || x[j] >= V) return 3;
    for (int j = 0; j < gamma; ++j) {
      const uint32_t pos = (uint32_t)j + 1u;  // 1-based position, as in svo_verify_chain
      r[j] = r_in ? r_in[(int64_t)b * gamma + j] : draw_uniform(seed, pos, (uint32_t)b, 0, round, 0);
    }
    const double u = u_in ? u_in[b] : draw_uniform(seed, 0, (uint32_t)b, 0, round, 1);
    ChainResult res = chain_round_pm(P, x, gamma, r.data(), u, out_p ? out_p + (int64_t)b * gamma : nullptr,
                                     a_trace ? a_trace + (int64_t)b * gamma : nullptr, w_out ? &w : nullptr);
    out_n[b] = res.n;
    out_tok[b] = res.t;
    if (w_out) {
      double S = 0.0;
      for (double v : w) S += v;
      for (int v = 0; v < V; ++v) w_out[(int64_t)b * V + v] = w[v] / S;
    }
    if (out_mdec) out_mdec[b] = res.mdec;
    if (out_mcdf) out_mcdf[b] = res.mcdf;
    if (out_rows) out_rows[b] = res.sample_rows;
  }
  return 0;
}

// Point-mass tree verification (tree_round_pm), same layout and optional
// arguments as svo_verify_tree, without draft rows.
int svo_verify_tree_pm(const void* tgt, int dtype, int64_t tgt_stride, const int32_t* node_tok, const int32_t* parent,
                       int B, int N, int max_depth, int V, double T, uint64_t seed, uint32_t round, const double* r_in,
                       const double* u_in, int32_t* out_len, int32_t* out_path, int32_t* out_tok, double* out_p,
                       double* a_trace, double* w_out, double* out_mdec, double* out_mcdf, int32_t* out_passes) {
  if (B < 0 || N < 1 || max_depth < 1 || V < 1 || !(T > 0.0)) return 1;
  std::vector<double> r(N), w;
  for (int b = 0; b < B; ++b) {
    const int32_t* par = parent + (int64_t)b * N;
    for (int i = 1; i < N; ++i)
      if (par[i] < 0 || par[i] >= i) return 4;
    for (int i = 0; i < N; ++i)
      r[i] = r_in ? r_in[(int64_t)b * N + i] : draw_uniform(seed, (uint32_t)i, (uint32_t)b, 0, round, 0);
    const double u = u_in ? u_in[b] : draw_uniform(seed, 0, (uint32_t)b, 0, round, 1);
    TreeInputs in{tgt, nullptr, dtype, tgt_stride, 0, node_tok + (int64_t)b * N, par, (int64_t)b * N,
                  N, V, max_depth, T};
    TreeResult res = tree_round_pm(in, r.data(), u, out_p ? out_p + (int64_t)b * N : nullptr,
                                   a_trace ? a_trace + (int64_t)b * N : nullptr, w_out ? &w : nullptr);
    if (!res.ok) return 5;
    out_len[b] = (int32_t)res.path.size();
    for (int d = 0; d < max_depth; ++d)
      out_path[(int64_t)b * max_depth + d] = d < (int)res.path.size() ? res.path[d] : -1;
    out_tok[b] = res.t;
    if (w_out) {
      double S = 0.0;
      for (double v : w) S += v;
      for (int v = 0; v < V; ++v) w_out[(int64_t)b * V + v] = w[v] / S;
    }
    if (out_mdec) out_mdec[b] = res.mdec;
    if (out_mcdf) out_mcdf[b] = res.mcdf;
    if (out_passes) out_passes[b] = res.row_passes;
  }
  return 0;
}

// Top-F fan-out ([SSD] §3: the speculation cache takes the top-F_k tokens of
// the draft logits at lookahead position k).  Per row r: the F[r] largest
// logits, ordered by value descending and index ascending on ties (a stable
// sort), padded with -1 up to F_max.
int svo_fanout_topk(const void* logits, int dtype, int64_t stride, int R, int V, const int32_t* F, int F_max,
                    int32_t* out_ids, float* out_vals /*[R*F_max] or null*/) {
  if (R < 0 || V < 1 || F_max < 1) return 1;
  std::vector<int> idx(V);
  std::vector<double> z(V);
  for (int r = 0; r < R; ++r) {
    if (F[r] < 0 || F[r] > F_max) return 2;
    for (int v = 0; v < V; ++v) {
      idx[v] = v;
      z[v] = load_logit(logits, dtype, (int64_t)r * stride + v);
    }
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return z[a] > z[b]; });
    for (int f = 0; f < F_max; ++f) {
      const bool keep = f < F[r] && f < V;
      out_ids[(int64_t)r * F_max + f] = keep ? idx[f] : -1;
      if (out_vals) out_vals[(int64_t)r * F_max + f] = keep ? (float)z[idx[f]] : -std::numeric_limits<float>::infinity();
    }
  }
  return 0;
}

// Speculation-cache hit test ([SSD] §3, cache strategy: for every lookahead
// position k = 0..K the cache holds the top-F_k tokens of the draft logits at
// k; a verification outcome (k', t*) is served from the cache iff t* is among
// the tokens cached for k' = the hit event of Definition 11).  Draft row
// (b, k) = b*(K+1) + k.  For sequence b with outcome (n[b], t[b]):
// out_rank[b] = the 0-based position of t[b] in draft row (b, n[b]) under the
// fan-out's order (value descending, index ascending on equal values), so the
// outcome is cached iff out_rank[b] < F[n[b]]; out_hit[b] is that test (F and
// out_hit may be null).  The row is sorted in full by that total order.
int svo_cache_hit_test(const void* drf, int dtype, int64_t stride, int B, int K, int V, const int32_t* n,
                       const int32_t* t, const int32_t* F, int32_t* out_rank, int32_t* out_hit) {
  if (B < 0 || K < 0 || V < 1) return 1;
  std::vector<int> order(V);
  std::vector<double> z(V);
  for (int b = 0; b < B; ++b) {
    if (n[b] < 0 || n[b] > K || t[b] < 0 || t[b] >= V) return 3;
    const int64_t row = (int64_t)b * (K + 1) + n[b];
    for (int v = 0; v < V; ++v) {
      order[v] = v;
      z[v] = load_logit(drf, dtype, row * stride + v);
    }
    std::sort(order.begin(), order.end(), [&](int a, int c) { return z[a] > z[c] || (z[a] == z[c] && a < c); });
    int pos = 0;
    while (order[pos] != t[b]) ++pos;
    out_rank[b] = pos;
    if (F && out_hit) out_hit[b] = pos < F[n[b]] ? 1 : 0;
  }
  return 0;
}

// PRESTO scoring and one priority expansion step ([PR] §4.1-4.2), tree layout
// as for svo_verify_tree (node u's rows are the target / draft distributions
// of u's children; depth(0) = 0, depth(i) = depth(parent(i)) + 1).
//   out_s [B*N]: s_i = presto_token_score(P_u(x_i), Q_u(x_i), lambda_{depth(i)})
//                for i >= 1, u = parent(i); 0 for the root.
//   out_S [B*N]: path score S_i = sum of s along the root-to-i path (eq. 10).
//   Expansion (Algorithm 1, one step from the frontier = the leaves, nodes
//   without children): every leaf u proposes its k best tokens t by
//   presto_token_score(P_u(t), Q_u(t), lambda_{depth(u)+1}) (score
//   descending, token ascending; -inf scores are not proposed); a proposal's
//   priority is S_u + its score; the b_top best proposals of the sequence
//   (priority descending, then node ascending, then token ascending) go to
//   out_node / out_tok / out_score [B*b_top], padded with -1 / -1 / -inf.
int svo_presto_score(const void* tgt, const void* drf, int dtype, int64_t tgt_stride, int64_t drf_stride,
                     const int32_t* node_tok, const int32_t* parent, int B, int N, int V, double T, const float* lam,
                     int D, int k, int b_top, double* out_s, double* out_S, int32_t* out_node, int32_t* out_tok,
                     double* out_score) {
  if (B < 0 || N < 1 || V < 1 || !(T > 0.0) || D < 1 || k < 0 || b_top < 0) return 1;
  std::vector<double> P, Q;
  std::vector<int> depth(N), nkids(N);
  for (int b = 0; b < B; ++b) {
    const int32_t* par = parent + (int64_t)b * N;
    const int32_t* tok = node_tok + (int64_t)b * N;
    double* s_b = out_s + (int64_t)b * N;
    double* S_b = out_S + (int64_t)b * N;
    std::fill(nkids.begin(), nkids.end(), 0);
    depth[0] = 0;
    for (int i = 1; i < N; ++i) {
      if (par[i] < 0 || par[i] >= i) return 4;
      if (tok[i] < 0 || tok[i] >= V) return 3;
      depth[i] = depth[par[i]] + 1;
      nkids[par[i]] += 1;
    }
    s_b[0] = 0.0;
    std::vector<PrestoCand> cands;
    for (int u = 0; u < N; ++u) {
      const int64_t row = (int64_t)b * N + u;
      if (!softmax_row(tgt, dtype, row * tgt_stride, V, T, P)) return 2;
      if (!softmax_row(drf, dtype, row * drf_stride, V, T, Q)) return 2;
      for (int i = u + 1; i < N; ++i)
        if (par[i] == u) s_b[i] = presto_token_score(P[tok[i]], Q[tok[i]], presto_lambda(lam, D, depth[i]));
      if (nkids[u] == 0) {
        const double lam_child = presto_lambda(lam, D, depth[u] + 1);
        std::vector<PrestoCand> mine;
        for (int t = 0; t < V; ++t) {
          const double sc = presto_token_score(P[t], Q[t], lam_child);
          if (sc > -kInf) mine.push_back({sc, u, t});
        }
        std::sort(mine.begin(), mine.end(), [](const PrestoCand& a, const PrestoCand& c) {
          return a.score > c.score || (a.score == c.score && a.tok < c.tok);
        });
        for (int j = 0; j < k && j < (int)mine.size(); ++j) cands.push_back(mine[j]);
      }
    }
    // path scores: parents precede children
    S_b[0] = 0.0;
    for (int i = 1; i < N; ++i) S_b[i] = S_b[par[i]] + s_b[i];
    for (PrestoCand& c : cands) c.score += S_b[c.node];
    std::sort(cands.begin(), cands.end(), [](const PrestoCand& a, const PrestoCand& c) {
      if (a.score != c.score) return a.score > c.score;
      if (a.node != c.node) return a.node < c.node;
      return a.tok < c.tok;
    });
    for (int j = 0; j < b_top; ++j) {
      const bool has = j < (int)cands.size();
      out_node[(int64_t)b * b_top + j] = has ? cands[j].node : -1;
      out_tok[(int64_t)b * b_top + j] = has ? cands[j].tok : -1;
      out_score[(int64_t)b * b_top + j] = has ? cands[j].score : -kInf;
    }
  }
  return 0;
}

// SpecBranch branch resampling ([SB] "Key designs" 2-3): the hybrid
// predictor's class s in {0, 1, 2} (an input: the predictor itself is a
// trained network) places the branch point b on the window's positions
// 1..gamma+1 -- s = 0: the round's first token (b = 1); s = 1: the first
// drafted token whose draft probability falls below eps (b = gamma + 1 when
// none does); s = 2: the next round's first token (b = gamma + 1).  Then
// k = max(1, floor(k_max * (1 - q(x_b)))) branches are forked with the top-k
// tokens of the draft distribution at b (value descending, index ascending).
// At b = gamma + 1 no token is drafted yet: x_b is taken as the draft's most
// likely token there (the first maximal index), so q(x_b) = max q_{gamma+1}.
// Draft rows q_1..q_{gamma+1} at (b, j) = b*(gamma+1) + (j-1); tokens
// x_1..x_gamma at b*gamma + (j-1); s may be null (every class 1).  Outputs:
// out_pos [B] the 1-based branch position, out_qb [B] q(x_b), out_k [B],
// out_ids [B*k_max] the branch tokens (-1 padded); out_margin [B] (may be
// null) the distance of the two decisions to their edges: min over the
// tested positions of |q_j(x_j) - eps|, and of k_max * (1 - q(x_b)) to the
// nearest integer.
int svo_branch_fork(const void* drf, int dtype, int64_t stride, const int32_t* tok, const int32_t* cls, int B,
                    int gamma, int V, double T, double eps, int k_max, int32_t* out_pos, double* out_qb,
                    int32_t* out_k, int32_t* out_ids, double* out_margin) {
  if (B < 0 || gamma < 1 || V < 1 || !(T > 0.0) || k_max < 1) return 1;
  std::vector<double> q;
  std::vector<int> order(V);
  for (int b = 0; b < B; ++b) {
    const int s = cls ? cls[b] : 1;
    if (s < 0 || s > 2) return 5;
    const int32_t* x = tok + (int64_t)b * gamma;
    for (int j = 0; j < gamma; ++j)
      if (x[j] < 0 || x[j] >= V) return 3;
    const int64_t row0 = (int64_t)b * (gamma + 1);
    double margin = kInf;
    int pos = gamma + 1;
    if (s == 0) {
      pos = 1;
    } else if (s == 1) {
      for (int j = 1; j <= gamma; ++j) {
        if (!softmax_row(drf, dtype, (row0 + j - 1) * stride, V, T, q)) return 2;
        const double qx = q[x[j - 1]];
        margin = std::min(margin, std::fabs(qx - eps));
        if (qx < eps) {
          pos = j;
          break;
        }
      }
    }
    if (!softmax_row(drf, dtype, (row0 + pos - 1) * stride, V, T, q)) return 2;
    double qb;
    if (pos <= gamma) {
      qb = q[x[pos - 1]];
    } else {
      int best = 0;
      for (int v = 1; v < V; ++v)
        if (q[v] > q[best]) best = v;
      qb = q[best];
    }
    const double kf = (double)k_max * (1.0 - qb);
    const int k = std::max(1, (int)std::floor(kf));
    margin = std::min(margin, std::fabs(kf - std::round(kf)));
    // top-k of the draft row at b: a stable sort of the logits, descending
    for (int v = 0; v < V; ++v) order[v] = v;
    std::vector<double> z(V);
    for (int v = 0; v < V; ++v) z[v] = load_logit(drf, dtype, (row0 + pos - 1) * stride + v);
    std::stable_sort(order.begin(), order.end(), [&](int a, int c) { return z[a] > z[c]; });
    out_pos[b] = pos;
    out_qb[b] = qb;
    out_k[b] = k;
    for (int i = 0; i < k_max; ++i) out_ids[(int64_t)b * k_max + i] = (i < k && i < V) ? order[i] : -1;
    if (out_margin) out_margin[b] = margin;
  }
  return 0;
}

// Geometric fan-out of [SSD] Theorem 12: F_k = F_0 * a_p^{k/(1+r)} for k < K
// and, when capped_last, F_K = F_0 * a_p^{K/(1+r)} * (1 - a_p)^{-1/(1+r)};
// rounded up to integers.  Writes K+1 values; returns their sum.
int svo_geometric_fanout(int F0, double a_p, double r, int K, int capped_last, int32_t* F_out) {
  int total = 0;
  for (int k = 0; k <= K; ++k) {
    double f = (double)F0 * std::pow(a_p, (double)k / (1.0 + r));
    if (k == K && capped_last) f *= std::pow(1.0 - a_p, -1.0 / (1.0 + r));
    F_out[k] = (int32_t)std::ceil(f);
    total += F_out[k];
  }
  return total;
}

}  // extern "C"
