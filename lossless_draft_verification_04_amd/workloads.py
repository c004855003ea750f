"""Seeded synthetic inputs for the five verification workloads.

This module builds logits, draft tokens and trees; it holds none of the
verification arithmetic (no softmax, no acceptance ratio, no residual, no
argmax-with-ties, no top-F selection of the method).  Both the HIP path and
the CPU oracle are handed the bytes it produces.

Recipes (shapes and value distributions of the pages' workloads):

* ``normal``  - target logits i.i.d. N(0, 3^2); draft = target + N(0, 1^2).
* ``zipf``    - a Zipf(s = 1.1) log-probability profile under a per-row
  random rank permutation, ``z_v = -1.1 ln rho(v) + g_v`` with
  ``rho(v) = (a v + c) mod V + 1`` (a coprime to V) and ``g`` Gumbel(0, 1)
  noise (``gumbel=False`` drops the noise, as in the tree recipe).
* draft rows = target rows + N(0, sigma_j^2), sigma_j rising linearly from
  0.5 at position 1 to 2.5 at position gamma.
* draft tokens are drawn from q_j = softmax(draft_j / T) with the Gumbel-max
  construction (argmax of draft_j / T + Gumbel noise) on the stored values,
  so no probability is ever formed here.
* greedy windows plant a unique row maximum at a random index g_j (its
  logit is raised 1.0 above the rest of the row); the draft equals g_j with
  probability 0.9 * 0.95^j, else is uniform over the other V - 1 ids.
* trees grow from the root by repeatedly picking a uniformly random node
  that can still take a child (depth < max_depth, fewer than F_depth
  children, F_d = ceil(F0 * a_p^(d/(1+r)))) and giving it the next-ranked
  token of its draft row; nodes are then renumbered in BFS order with
  children in rank order.

All randomness comes from ``torch.Generator`` objects seeded explicitly, on
the CPU, so the bytes are the same on every machine.  Rows are stored with a
padded stride (a multiple of 16 bytes) when V needs it; the returned tensors
are views of shape [..., V].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Full-size workloads: sizes of the pages' settings (vocabularies of the
# LLaMA-2 / Qwen2.5 / LLaMA-3.1 families, gamma and K of the SpecDiff-2
# drafters, a 64-node depth-8 tree with geometric fan-out F0 = 8, a_p = 0.7).
CHAIN_SMALL = dict(B=1, gamma=4, V=32000, T=1.0, dtype="f32")
CHAIN_BATCHED = dict(B=32, gamma=16, V=152064, T=0.8, dtype="bf16")
GREEDY_WINDOW = dict(B=64, gamma=32, V=151936, dtype="bf16")
MULTI_CAND = dict(B=16, K=8, gamma=16, V=128256, T=1.0, dtype="bf16")
TREE_FANOUT = dict(B=8, N=64, max_depth=8, V=128256, T=1.0, dtype="bf16", F0=8, a_p=0.7, r=1.0)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}
_ROW_BLOCK = 64  # rows generated per block (bounds temporaries)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def padded_stride(V: int, dtype: str) -> int:
    """Smallest row stride >= V whose byte size is a multiple of 16."""
    per = 16 // torch.empty((), dtype=_TORCH_DTYPE[dtype]).element_size()
    return ((V + per - 1) // per) * per


def _alloc_rows(shape_rows, V, dtype, pad=True):
    """Allocate [*shape_rows, Vs] and return (storage, view [..., V])."""
    Vs = padded_stride(V, dtype) if pad else V
    store = torch.zeros(*shape_rows, Vs, dtype=_TORCH_DTYPE[dtype])
    return store, store[..., :V]


def _gumbel(shape, gen):
    u = torch.rand(shape, generator=gen, dtype=torch.float32).clamp_(min=1e-30)
    return -torch.log(-torch.log(u))


def _coprime(V: int, gen) -> int:
    while True:
        a = int(torch.randint(1, max(V, 2), (1,), generator=gen))
        if math.gcd(a, V) == 1:
            return a


def zipf_rows(n_rows: int, V: int, gen, s: float = 1.1, gumbel: bool = True) -> torch.Tensor:
    """[n_rows, V] float32 rows of -s ln rho(v) (+ Gumbel noise), rho a random affine rank bijection."""
    out = torch.empty(n_rows, V, dtype=torch.float32)
    v = torch.arange(V, dtype=torch.int64)
    for r0 in range(0, n_rows, _ROW_BLOCK):
        r1 = min(n_rows, r0 + _ROW_BLOCK)
        a = torch.tensor([_coprime(V, gen) for _ in range(r0, r1)], dtype=torch.int64)
        c = torch.randint(0, V, (r1 - r0,), generator=gen, dtype=torch.int64)
        rank = (a[:, None] * v[None, :] + c[:, None]) % V + 1
        blk = rank.to(torch.float32).log_().mul_(-s)
        if gumbel:
            blk += _gumbel((r1 - r0, V), gen)
        out[r0:r1] = blk
    return out


def sigma_schedule(gamma: int, lo: float = 0.5, hi: float = 2.5) -> torch.Tensor:
    if gamma == 1:
        return torch.tensor([lo])
    j = torch.arange(gamma, dtype=torch.float32)
    return lo + (hi - lo) * j / (gamma - 1)


def gumbel_max_tokens(logits_rows: torch.Tensor, T: float, gen, draws: int = 1) -> torch.Tensor:
    """Draw `draws` tokens per row from softmax(row / T) by the Gumbel-max construction.

    logits_rows [R, V] (any float dtype; the stored values are used) -> int32 [R, draws].
    """
    R, V = logits_rows.shape
    out = torch.empty(R, draws, dtype=torch.int32)
    for r in range(R):
        zr = logits_rows[r].to(torch.float32) / T
        for d in range(draws):
            out[r, d] = int(torch.argmax(zr + _gumbel((V,), gen)))
    return out


@dataclass
class Workload:
    kind: str
    params: dict
    tensors: dict = field(default_factory=dict)  # CPU tensors (views with padded storage)

    def to(self, device):
        """Copy every tensor to `device`, keeping the padded row stride."""
        out = {}
        for k, t in self.tensors.items():
            if t.dim() >= 1 and t.is_floating_point():
                base = t
                # rebuild the padded storage on the device and view it
                Vs = base.stride(-2) if base.dim() >= 2 else base.shape[-1]
                shape = list(base.shape)
                store = torch.empty(*shape[:-1], Vs, dtype=base.dtype, device=device)
                view = store[..., :shape[-1]]
                view.copy_(base)
                out[k] = view
            else:
                out[k] = t.to(device)
        return out


# ---------------------------------------------------------------------------
def chain_normal(B=1, gamma=4, V=32000, T=1.0, dtype="f32", seed=1001) -> Workload:
    """Chain inputs with N(0, 3^2) target logits and N(0, 1) draft noise."""
    gen = _gen(seed)
    _, tgt = _alloc_rows((B, gamma + 1), V, dtype)
    _, drf = _alloc_rows((B, gamma), V, dtype)
    t32 = torch.randn(B, gamma + 1, V, generator=gen) * 3.0
    d32 = t32[:, :gamma] + torch.randn(B, gamma, V, generator=gen)
    tgt.copy_(t32)
    drf.copy_(d32)
    tok = gumbel_max_tokens(drf.reshape(B * gamma, V), T, gen).reshape(B, gamma)
    return Workload("chain", dict(B=B, gamma=gamma, V=V, T=T, dtype=dtype, seed=seed),
                    dict(tgt=tgt, drf=drf, tok=tok))


def chain_zipf(B=32, gamma=16, V=152064, T=0.8, dtype="bf16", seed=1002, sig_lo=0.5, sig_hi=2.5,
               lookahead_row=False) -> Workload:
    """Chain inputs with Gumbel-perturbed Zipf target rows and rising draft noise.

    lookahead_row: also draw the drafter's row for position gamma+1 (target row gamma+1 plus N(0, sig_hi^2)
    noise) as ``drf_next`` [B, V], after everything else, so the other tensors do not change."""
    gen = _gen(seed)
    _, tgt = _alloc_rows((B, gamma + 1), V, dtype)
    _, drf = _alloc_rows((B, gamma), V, dtype)
    sig = sigma_schedule(gamma, sig_lo, sig_hi)
    for b in range(B):
        t32 = zipf_rows(gamma + 1, V, gen)
        d32 = t32[:gamma] + torch.randn(gamma, V, generator=gen) * sig[:, None]
        tgt[b].copy_(t32)
        drf[b].copy_(d32)
    tok = gumbel_max_tokens(drf.reshape(B * gamma, V), T, gen).reshape(B, gamma)
    tensors = dict(tgt=tgt, drf=drf, tok=tok)
    if lookahead_row:
        _, nxt = _alloc_rows((B,), V, dtype)
        for b in range(B):
            nxt[b].copy_(tgt[b, gamma].to(torch.float32) + torch.randn(V, generator=gen) * sig_hi)
        tensors["drf_next"] = nxt
    return Workload("chain", dict(B=B, gamma=gamma, V=V, T=T, dtype=dtype, seed=seed), tensors)


def redraw_tokens(wl: Workload, T: float, seed: int) -> torch.Tensor:
    """Draft tokens of a chain workload drawn afresh from q_j at temperature T (Gumbel-max); T = 0 takes the
    draft rows' first maximal index (the greedy drafter)."""
    p = wl.params
    rows = wl.tensors["drf"].reshape(p["B"] * p["gamma"], p["V"])
    if T == 0:
        tok = torch.argmax(rows.to(torch.float32), dim=1).to(torch.int32)[:, None]
    else:
        tok = gumbel_max_tokens(rows, T, _gen(seed))
    return tok.reshape(p["B"], p["gamma"]).contiguous()


def lookahead_rows(wl: Workload) -> torch.Tensor:
    """The drafter's rows for lookahead positions k = 0..gamma as one [B, gamma+1, V] tensor (padded rows):
    draft rows q_1..q_gamma, then ``drf_next``."""
    p = wl.params
    B, gamma, V = p["B"], p["gamma"], p["V"]
    _, out = _alloc_rows((B, gamma + 1), V, p["dtype"])
    out[:, :gamma].copy_(wl.tensors["drf"])
    out[:, gamma].copy_(wl.tensors["drf_next"])
    return out


def greedy_zipf(B=64, gamma=32, V=151936, dtype="bf16", seed=1003, match0=0.9, decay=0.95,
                plant=True) -> Workload:
    """Greedy window: the draft matches the target row's argmax with probability match0 * decay^j.

    plant=True puts a unique maximum (+1.0 over the row's top) at a random index of every row.
    plant=False keeps the Zipf + Gumbel rows as stored, so that rounding to the storage dtype leaves
    ties at the row maximum in some rows; the draft's "match" token is then the first maximal index
    of the stored row (the generator's choice of draft tokens, not a verification result)."""
    gen = _gen(seed)
    _, tgt = _alloc_rows((B, gamma + 1), V, dtype)
    planted = torch.randint(0, V, (B, gamma + 1), generator=gen, dtype=torch.int64)
    for b in range(B):
        t32 = zipf_rows(gamma + 1, V, gen)
        if plant:
            top = t32.max(dim=1).values
            t32[torch.arange(gamma + 1), planted[b]] = top + 1.0
        tgt[b].copy_(t32)
        if not plant:
            planted[b] = torch.argmax(tgt[b].to(torch.float32), dim=1)
    j = torch.arange(1, gamma + 1, dtype=torch.float64)
    p_match = match0 * decay ** j
    hit = torch.rand(B, gamma, generator=gen, dtype=torch.float64) < p_match[None, :]
    other = torch.randint(0, max(V - 1, 1), (B, gamma), generator=gen, dtype=torch.int64)
    g = planted[:, :gamma]
    other = other + (other >= g).to(torch.int64)  # uniform over the V - 1 ids != g
    if V == 1:
        other = g.clone()
    tok = torch.where(hit, g, other).to(torch.int32)
    return Workload("greedy", dict(B=B, gamma=gamma, V=V, dtype=dtype, seed=seed, plant=plant),
                    dict(tgt=tgt, tok=tok, planted=planted.to(torch.int32)))


def multi_zipf(B=16, K=8, gamma=16, V=128256, T=1.0, dtype="bf16", seed=1004, tgt_sigma=0.5) -> Workload:
    """K candidates drawn from shared draft marginals; per-candidate target rows."""
    gen = _gen(seed)
    _, tgt = _alloc_rows((B, K, gamma + 1), V, dtype)
    _, drf = _alloc_rows((B, gamma), V, dtype)
    sig = sigma_schedule(gamma)
    for b in range(B):
        base = zipf_rows(gamma + 1, V, gen)
        drf[b].copy_(base[:gamma] + torch.randn(gamma, V, generator=gen) * sig[:, None])
        for k in range(K):
            t = base.clone()
            t[1:] += torch.randn(gamma, V, generator=gen) * tgt_sigma
            tgt[b, k].copy_(t)
    tok = gumbel_max_tokens(drf.reshape(B * gamma, V), T, gen, draws=K)  # [B*gamma, K]
    tok = tok.reshape(B, gamma, K).permute(0, 2, 1).contiguous()
    return Workload("multi", dict(B=B, K=K, gamma=gamma, V=V, T=T, dtype=dtype, seed=seed),
                    dict(tgt=tgt, drf=drf, tok=tok))


def fanout_schedule(F0: int, a_p: float, r: float, depth: int):
    """F_d = ceil(F0 * a_p^(d/(1+r))) for d < depth (the tree generator's branching limits)."""
    return [int(math.ceil(F0 * a_p ** (d / (1.0 + r)))) for d in range(depth)]


def grow_tree(N: int, max_depth: int, F: list, gen):
    """Random tree shape: returns (parent, rank_in_parent, depth) in creation order."""
    parent, rank, depth, nkids = [-1], [0], [0], [0]
    while len(parent) < N:
        cand = [u for u in range(len(parent)) if depth[u] < max_depth and nkids[u] < F[depth[u]]]
        if not cand:
            break
        u = cand[int(torch.randint(0, len(cand), (1,), generator=gen))]
        parent.append(u)
        rank.append(nkids[u])
        depth.append(depth[u] + 1)
        nkids[u] += 1
        nkids.append(0)
    return parent, rank, depth


def tree_zipf(B=8, N=64, max_depth=8, V=128256, T=1.0, dtype="bf16", seed=1005, F0=8, a_p=0.7, r=1.0,
              draft_sigma=1.0) -> Workload:
    """Token trees with Zipf node rows, N(0, 1) draft noise and top-ranked children."""
    gen = _gen(seed)
    F = fanout_schedule(F0, a_p, r, max_depth)
    _, tgt = _alloc_rows((B, N), V, dtype)
    _, drf = _alloc_rows((B, N), V, dtype)
    parent_all = torch.full((B, N), -1, dtype=torch.int32)
    tok_all = torch.zeros(B, N, dtype=torch.int32)
    depth_all = torch.zeros(B, N, dtype=torch.int32)
    for b in range(B):
        par_c, rank_c, dep_c = grow_tree(N, max_depth, F, gen)
        n = len(par_c)
        t32 = zipf_rows(n, V, gen, gumbel=False)
        d32 = t32 + torch.randn(n, V, generator=gen) * draft_sigma
        d_st = d32.to(_TORCH_DTYPE[dtype])
        # BFS renumbering, children in rank order
        kids = [[] for _ in range(n)]
        for i in range(1, n):
            kids[par_c[i]].append(i)
        for u in range(n):
            kids[u].sort(key=lambda i: rank_c[i])
        order, head = [0], 0
        while head < len(order):
            order.extend(kids[order[head]])
            head += 1
        new_id = {old: new for new, old in enumerate(order)}
        # child token = the rank-th largest stored draft logit of its parent's row
        ranked = {}
        for u in range(n):
            if kids[u]:
                ranked[u] = torch.topk(d_st[u].to(torch.float32), len(kids[u])).indices
        for new, old in enumerate(order):
            tgt[b, new].copy_(t32[old])
            drf[b, new].copy_(d_st[old])
            depth_all[b, new] = dep_c[old]
            if old == 0:
                continue
            parent_all[b, new] = new_id[par_c[old]]
            tok_all[b, new] = int(ranked[par_c[old]][rank_c[old]])
    return Workload("tree", dict(B=B, N=N, max_depth=max_depth, V=V, T=T, dtype=dtype, seed=seed, F=F),
                    dict(tgt=tgt, drf=drf, tok=tok_all, parent=parent_all, depth=depth_all))


def chain_shaped_tree(chain: Workload) -> Workload:
    """Re-express a chain workload as a path tree (node i = draft position i, root = prefix)."""
    p = chain.params
    B, gamma, V = p["B"], p["gamma"], p["V"]
    N = gamma + 1
    tgt_c, drf_c, tok_c = chain.tensors["tgt"], chain.tensors["drf"], chain.tensors["tok"]
    _, tgt = _alloc_rows((B, N), V, p["dtype"])
    _, drf = _alloc_rows((B, N), V, p["dtype"])
    tgt.copy_(tgt_c)
    drf[:, :gamma].copy_(drf_c)
    drf[:, gamma].copy_(drf_c[:, gamma - 1])  # never read (leaf)
    parent = torch.arange(-1, N - 1, dtype=torch.int32).repeat(B, 1)
    tok = torch.zeros(B, N, dtype=torch.int32)
    tok[:, 1:] = tok_c
    return Workload("tree", dict(B=B, N=N, max_depth=gamma, V=V, T=p["T"], dtype=p["dtype"], seed=p["seed"]),
                    dict(tgt=tgt, drf=drf, tok=tok, parent=parent))


def to_numpy_logits(t: torch.Tensor):
    """CPU logits view -> numpy array for the oracle (bf16 as raw uint16 bits), keeping strides."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
