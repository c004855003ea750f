"""Benchmark of the verification hot path on one MI355X.

One step = one sv_verify_chain call over the batched chain workload
(B=32 sequences, gamma=16 drafts, V=152064, bf16 logits, T=0.8): every
needed logit row streamed once, decisions, and the correction / bonus draw.
Inputs are resident in HBM before the timed region; distinct copies of the
inputs (>= 2 GB in total) are rotated so the 256 MB last-level cache cannot
serve a repeat.

One HIP graph holds one call per input copy, repeated over the copies up to
at least 32 calls, and the timed loop replays it (plus a tail graph) so that
exactly `steps` calls run; host launch cost is then not in the step time
(the eager rate is reported beside it).

Prints ONE JSON line.  `value` is verified draft positions per second (B *
gamma per call).  `roofline` reports the call's algorithmic bytes (rows
1..gamma of target and draft, plus the row pair of the correction or the
bonus row, per sequence) over its mean duration from HIP events recorded on
the launch stream, against the 8 TB/s HBM peak.  `cpu_baseline` times the
CPU oracle (single-threaded fp64) on the same workload.  `variants` holds the
same measurements for the other rows of the hot path (greedy window,
multi-candidate, tree, fan-out, the small fp32 chain, the point-mass chain
and tree, which read no draft rows, the speculation-cache hit test with
its hit rate against temperature for geometric and uniform fan-out, the
SpecBranch fork, and PRESTO scoring with one priority expansion step on the
tree workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from lossless_draft_verification_04_amd import specverify as svx  # noqa: E402
from lossless_draft_verification_04_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 2.2e9
USE_GRAPHS = True
PMC_RECORD = os.path.join(ROOT, "profiles", "chain_batched_pmc.json")
KERNEL_SOURCES = [os.path.join(ROOT, "lossless_draft_verification_04_amd", "csrc", f)
                  for f in ("sv_device.hpp", "sv_walk.hpp", "sv_internal.h", "sv_api.hip", "sv_chain.hip")] + \
                 [os.path.join(ROOT, "include", "specverify.h")]
METRIC = "verified draft positions/sec + achieved HBM GB/s (% of MI355X peak), 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def esize(dt):
    return 2 if dt == "bf16" else 4


def n_copies(bytes_per_copy):
    """Distinct input copies whose total exceeds the 256 MB last-level cache (at most 32)."""
    return min(32, max(2, int(np.ceil(ROTATE_BYTES / max(bytes_per_copy, 1)))))


def time_calls(fn, copies, steps, warmup):
    """Run fn(copy) `warmup` times untimed, then `steps` times timed, with one
    pair of HIP events on the launch stream around the timed calls.

    Returns (ms_per_step wall, event ms per call)."""
    for i in range(warmup):
        fn(copies[i % len(copies)])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(steps):
        fn(copies[i % len(copies)])
    b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, a.elapsed_time(b) / steps


def time_graphs(fn, copies, steps, warmup):
    """Capture one HIP graph holding one call per input copy, repeated over the
    copies until it holds at least 32 calls (and a tail graph for the
    remainder), replay them so that exactly `steps` calls run, and bracket
    every replay with HIP events on the launch stream.

    Returns (ms_per_step wall, mean event ms per call)."""
    if not USE_GRAPHS:
        return time_calls(fn, copies, steps, warmup)
    fn(copies[0])  # workspace and code objects exist before capture
    torch.cuda.synchronize()
    L = len(copies) * max(1, -(-32 // len(copies)))
    L = min(L, max(steps, 1))

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(copies[i % len(copies)])
        return g

    full = capture(L)
    plan = [(full, L)] * (steps // L)
    if steps % L:
        plan.append((capture(steps % L), steps % L))
    for _ in range(max(1, -(-warmup // L))):
        full.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in plan]
    t0 = time.perf_counter()
    for (g, _), (a, b) in zip(plan, ev):
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per_call = sum(a.elapsed_time(b) for a, b in ev) / steps
    return wall, per_call


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per call from the committed rocprofv3 counter record, if it was
    taken on the current kernel sources (null otherwise)."""
    try:
        with open(PMC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_call")


def roofline(alg_bytes, ms):
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                traffic=measured_traffic())


def copy_probe(mib, reps=5):
    """Device-to-device copies of a known size, for scaling the traffic counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {mib} MiB ({mib * (1 << 20)} bytes read and written each)")


# ------------------------------------------------------------------ chain
def chain_alg_bytes(p, n):
    row = p["V"] * esize(p["dtype"])
    B, g = p["B"], p["gamma"]
    resid = sum(2 if int(x) < g else 1 for x in n)
    return (2 * g * B + resid) * row


def bench_chain(wl, steps, warmup, seed=0):
    p = wl.params
    T = float(np.float32(p["T"]))
    per_copy = wl.tensors["tgt"].numel() * esize(p["dtype"]) * 2
    copies = [wl.to("cuda") for _ in range(n_copies(per_copy))]
    fn = lambda g: svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], T, seed=seed, round_=0, want_pq=False)
    out = fn(copies[0])
    torch.cuda.synchronize()
    n = out["n"].cpu().numpy()
    e_wall, _ = time_calls(fn, copies, steps, warmup)
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    pos = p["B"] * p["gamma"]
    alg = chain_alg_bytes(p, n)
    return dict(positions_per_call=pos, positions_per_s=pos / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_accepted=float(n.mean()), copies=len(copies), eager_ms_per_step=e_wall), out


def device_copy(wl, keys):
    """The named tensors of a workload on the GPU (padded row strides kept)."""
    return W.Workload(wl.kind, wl.params, {k: wl.tensors[k] for k in keys}).to("cuda")


def bench_chain_pm(wl, steps, warmup, seed=0):
    """Point-mass chain on the chain workload: target rows 1..gamma per sequence, then one row."""
    p = wl.params
    T = float(np.float32(p["T"]))
    per_copy = wl.tensors["tgt"].numel() * esize(p["dtype"])
    copies = [device_copy(wl, ("tgt", "tok")) for _ in range(n_copies(per_copy))]
    fn = lambda g: svx.sv_verify_chain_pm(g["tgt"], g["tok"], T, seed=seed, round_=0, want_p=False)
    out = fn(copies[0])
    torch.cuda.synchronize()
    n = out["n"].cpu().numpy()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    B, g = p["B"], p["gamma"]
    pos = B * g
    alg = (g * B + B) * p["V"] * esize(p["dtype"])
    return dict(positions_per_call=pos, positions_per_s=pos / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_accepted=float(n.mean()), copies=len(copies))


def bench_greedy(wl, steps, warmup):
    p = wl.params
    per_copy = wl.tensors["tgt"].numel() * esize(p["dtype"])
    copies = [wl.to("cuda") for _ in range(n_copies(per_copy))]
    fn = lambda g: svx.sv_verify_greedy(g["tgt"], g["tok"], want_argmax=False)
    out = fn(copies[0])
    torch.cuda.synchronize()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    pos = p["B"] * p["gamma"]
    alg = p["B"] * (p["gamma"] + 1) * p["V"] * esize(p["dtype"])
    return dict(positions_per_call=pos, positions_per_s=pos / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_accepted=float(out["n"].float().mean().item()), copies=len(copies), _out=out)


def bench_multi(wl, steps, warmup):
    p = wl.params
    T = float(np.float32(p["T"]))
    per_copy = (wl.tensors["tgt"].numel() + wl.tensors["drf"].numel()) * esize(p["dtype"])
    copies = [wl.to("cuda") for _ in range(n_copies(per_copy))]
    fn = lambda g: svx.sv_verify_multi(g["tgt"], g["drf"], g["tok"], T, want_pq=False)
    out = fn(copies[0])
    torch.cuda.synchronize()
    n = out["n"].cpu().numpy()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    B, K, g, V = p["B"], p["K"], p["gamma"], p["V"]
    row = V * esize(p["dtype"])
    alg = (B * K * g + B * g) * row + sum(2 if int(x) < g else 1 for x in n) * row
    pos = B * K * g
    return dict(positions_per_call=pos, positions_per_s=pos / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_accepted=float(n.mean()), copies=len(copies), _out=out)


def tree_alg_bytes(wl, out):
    """Minimum HBM bytes of one call: the target and draft rows of every node with children (the row
    statistics), plus the row pair of every node on the walked path where at least one child was
    rejected (the residual passes and the final draw need that node's whole row pair), plus the target
    row of the last node when the walk ends in a bonus draw.  Counted from one call's outputs: a
    child was tried iff its p(tok) was written."""
    p = wl.params
    parent = wl.tensors["parent"]
    B, N = parent.shape
    tried = ~torch.isnan(out["p"].cpu())
    length = out["len"].cpu()
    path = out["path"].cpu()
    rows = 0
    for b in range(B):
        par = parent[b].tolist()
        internal = set(x for x in par if x >= 0)
        rows += 2 * len(internal)
        walked = [0] + [int(path[b, d]) for d in range(int(length[b]))]
        for i, node in enumerate(walked):
            n_tried = sum(1 for c in range(1, N) if par[c] == node and bool(tried[b, c]))
            accepted = 1 if i + 1 < len(walked) else 0
            if n_tried - accepted > 0:
                rows += 2  # the node's row pair, read once for its residual passes
        last = walked[-1]
        if last not in internal or length[b] >= p["max_depth"]:
            rows += 1  # bonus draw from the last node's target row
    return rows * p["V"] * esize(p["dtype"])


def bench_tree(wl, steps, warmup):
    p = wl.params
    T = float(np.float32(p["T"]))
    per_copy = (wl.tensors["tgt"].numel() + wl.tensors["drf"].numel()) * esize(p["dtype"])
    copies = [wl.to("cuda") for _ in range(n_copies(per_copy))]
    g0 = copies[0]
    out = svx.sv_verify_tree(g0["tgt"], g0["drf"], g0["tok"], g0["parent"], p["max_depth"], T, want_pq=True)
    torch.cuda.synchronize()
    alg = tree_alg_bytes(wl, out)
    fn = lambda g: svx.sv_verify_tree(g["tgt"], g["drf"], g["tok"], g["parent"], p["max_depth"], T, want_pq=False)
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    pos = p["B"] * (p["N"] - 1)
    return dict(positions_per_call=pos, positions_per_s=pos / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_accepted=float(out["len"].float().mean().item()), copies=len(copies), _out=out)


def bench_tree_pm(wl, steps, warmup):
    """Point-mass tree: the target row of every node with children, then one row per sequence (the
    final node's row for the draw without the rejected tokens, or the bonus row)."""
    p = wl.params
    T = float(np.float32(p["T"]))
    per_copy = wl.tensors["tgt"].numel() * esize(p["dtype"])
    copies = [device_copy(wl, ("tgt", "tok", "parent")) for _ in range(n_copies(per_copy))]
    fn = lambda g: svx.sv_verify_tree_pm(g["tgt"], g["tok"], g["parent"], p["max_depth"], T, want_p=False)
    out = fn(copies[0])
    torch.cuda.synchronize()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    parent = wl.tensors["parent"]
    B, N = parent.shape
    internal = sum(len(set(x for x in parent[b].tolist() if x >= 0)) for b in range(B))
    alg = (internal + B) * p["V"] * esize(p["dtype"])
    pos = B * (N - 1)
    return dict(positions_per_call=pos, positions_per_s=pos / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_accepted=float(out["len"].float().mean().item()), copies=len(copies))


def uniform_fanout(total, K):
    """K+1 positions sharing `total` cache slots evenly (the first positions take the remainder)."""
    return [total // (K + 1) + (1 if k < total % (K + 1) else 0) for k in range(K + 1)]


def bench_cache(wl, steps, warmup, temps=(0.0, 0.5, 1.0), rounds=32, F0=8, r_exp=1.0):
    """Speculation-cache hit test on the chain workload with the drafter's lookahead row: the kernel's time on
    the realised outcomes of one verification call, and the hit rate against temperature for the geometric
    fan-out (Theorem 12 with the acceptance rate measured at that temperature, capped last term) and a uniform
    fan-out with the same number of cache slots."""
    p = wl.params
    B, K, V = p["B"], p["gamma"], p["V"]
    rows_cpu = W.lookahead_rows(wl)
    g = wl.to("cuda")
    store = torch.empty(B, K + 1, rows_cpu.stride(1), dtype=rows_cpu.dtype, device="cuda")
    rows = store[..., :V]
    rows.copy_(rows_cpu)
    table = {}
    for T in temps:
        tok = W.redraw_tokens(wl, T, seed=int(1000 * T) + 7).cuda()
        ns, ts = [], []
        for rnd in range(1 if T == 0 else rounds):
            if T == 0:
                out = svx.sv_verify_greedy(g["tgt"], tok, want_argmax=False)
            else:
                out = svx.sv_verify_chain(g["tgt"], g["drf"], tok, float(np.float32(T)), seed=11, round_=rnd,
                                          want_pq=False)
            ns.append(out["n"].clone())
            ts.append(out["tok"].clone())
        n, t = torch.cat(ns), torch.cat(ts)
        nn = n.double()
        # acceptance rate per position: accepted over tried (a rejection ends the window)
        a_p = float(nn.sum() / (nn.sum() + (n < K).double().sum()))
        a_p = min(max(a_p, 0.01), 0.99)
        F_geo = svx.sv_geometric_fanout(F0, a_p, r_exp, K, capped_last=True)
        F_uni = uniform_fanout(sum(F_geo), K)
        res = {}
        for name, F in (("geometric", F_geo), ("uniform", F_uni)):
            Fd = torch.tensor(F, dtype=torch.int32, device="cuda")
            hits = [svx.sv_cache_hit_test(rows, nr, tr, Fd)["hit"] for nr, tr in zip(ns, ts)]
            res[name] = round(float(torch.cat(hits).double().mean()), 4)
        table[str(T)] = dict(outcomes=int(n.numel()), a_p=round(a_p, 4), slots=sum(F_geo), F_geometric=F_geo,
                             F_uniform=F_uni, hit_geometric=res["geometric"], hit_uniform=res["uniform"],
                             mean_accepted=round(float(nn.mean()), 3))
    # kernel time on one call's outcomes (T of the workload), rows rotated over copies
    out = svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], float(np.float32(p["T"])), want_pq=False)
    F = torch.tensor(svx.sv_geometric_fanout(F0, 0.7, r_exp, K, capped_last=True), dtype=torch.int32, device="cuda")
    per_copy = B * V * esize(p["dtype"])  # one row per sequence is read
    copies = []
    for _ in range(n_copies(per_copy * (K + 1))):
        c = torch.empty_like(store)[..., :V]
        c.copy_(rows)
        copies.append(dict(rows=c, n=out["n"].clone(), t=out["tok"].clone(), F=F))
    fn = lambda c: svx.sv_cache_hit_test(c["rows"], c["n"], c["t"], c["F"])
    fn(copies[0])
    torch.cuda.synchronize()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    return dict(sequences_per_call=B, sequences_per_s=B / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=per_copy, copies=len(copies), hit_rate_vs_T=table)


def bench_branch(wl, steps, warmup, eps=0.3, k_max=8):
    """SpecBranch fork on the chain workload with the lookahead row: the gamma + 1 draft rows of every sequence
    read for their statistics, then the branch row once more for its top-k."""
    p = wl.params
    B, g, V = p["B"], p["gamma"], p["V"]
    T = float(np.float32(p["T"]))
    rows_cpu = W.lookahead_rows(wl)
    per_copy = rows_cpu.numel() * esize(p["dtype"])
    cls = torch.randint(0, 3, (B,), generator=torch.Generator().manual_seed(5), dtype=torch.int32).cuda()
    copies = []
    for _ in range(n_copies(per_copy)):
        store = torch.empty(B, g + 1, rows_cpu.stride(1), dtype=rows_cpu.dtype, device="cuda")
        r = store[..., :V]
        r.copy_(rows_cpu)
        copies.append(dict(rows=r, tok=wl.tensors["tok"].cuda()))
    fn = lambda c: svx.sv_branch_fork(c["rows"], c["tok"], T, eps, k_max, cls)
    out = fn(copies[0])
    torch.cuda.synchronize()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    alg = (g + 2) * B * V * esize(p["dtype"])
    return dict(sequences_per_call=B, sequences_per_s=B / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, mean_branch_pos=float(out["pos"].float().mean().item()),
                mean_branches=float(out["k"].float().mean().item()), eps=eps, k_max=k_max, copies=len(copies))


PRESTO_LAMBDA = [0.5, 1.0, 1.5, 2.0]


def bench_presto(wl, steps, warmup, k=8, b_top=32):
    """PRESTO scoring and one expansion step on the tree workload: every node's row pair is read for its
    statistics, and each leaf's row pair once more for its proposals."""
    p = wl.params
    T = float(np.float32(p["T"]))
    per_copy = (wl.tensors["tgt"].numel() + wl.tensors["drf"].numel()) * esize(p["dtype"])
    copies = [wl.to("cuda") for _ in range(n_copies(per_copy))]
    lam = torch.tensor(PRESTO_LAMBDA, dtype=torch.float32, device="cuda")
    fn = lambda g: svx.sv_presto_score(g["tgt"], g["drf"], g["tok"], g["parent"], T, lam, k, b_top)
    fn(copies[0])
    torch.cuda.synchronize()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    parent = wl.tensors["parent"]
    B, N = parent.shape
    leaves = sum(N - len(set(x for x in parent[b].tolist() if x >= 0)) for b in range(B))
    alg = (2 * B * N + 2 * leaves) * p["V"] * esize(p["dtype"])
    return dict(nodes_per_call=B * N, nodes_per_s=B * N / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, leaves=leaves, k=k, b_top=b_top, lam=PRESTO_LAMBDA, copies=len(copies))


def bench_fanout(wl, steps, warmup):
    p = wl.params
    B, N, V = wl.tensors["drf"].shape
    F = torch.tensor([W.fanout_schedule(8, 0.7, 1.0, 9)[d] for d in wl.tensors["depth"].reshape(-1).tolist()],
                     dtype=torch.int32)
    per_copy = wl.tensors["drf"].numel() * esize(p["dtype"])
    copies = []
    for _ in range(n_copies(per_copy)):
        g = wl.to("cuda")
        copies.append(dict(x=g["drf"].reshape(B * N, V), F=F.cuda()))
    fn = lambda g: svx.sv_fanout_topk(g["x"], g["F"], 8, want_vals=False)
    fn(copies[0])
    torch.cuda.synchronize()
    wall, ev_ms = time_graphs(fn, copies, steps, warmup)
    alg = B * N * V * esize(p["dtype"])
    return dict(rows_per_call=B * N, rows_per_s=B * N / (wall * 1e-3), ms_per_step=wall, call_ms=ev_ms,
                alg_bytes=alg, copies=len(copies))


def summarize(r):
    d = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items() if not k.startswith("_")}
    d["achieved_GBps"] = round(r["alg_bytes"] / (r["call_ms"] * 1e-3) / 1e9, 1)
    d["frac_of_peak"] = round(d["achieved_GBps"] / HBM_PEAK_GBS, 4)
    return d


# ------------------------------------------------------------------ acceptance statistics (outside the timed region)
def acceptance_by_position(n, gamma):
    """alpha_j, j = 1..gamma: the fraction of windows that reached position j (n >= j - 1) and accepted it
    (n >= j); the draft-then-verify page §2.2's per-position acceptance, realised."""
    n = np.asarray(n).reshape(-1)
    out = []
    for j in range(1, gamma + 1):
        reached = int((n >= j - 1).sum())
        out.append(round(float((n >= j).sum()) / reached, 4) if reached else None)
    return out


def overlap_by_position(T, pairs):
    """beta_j = sum_v min(p_j(v), q_j(v)) = 1 - TV(p_j, q_j) (draft-then-verify page §2.2), the acceptance rate
    of position j when the draft is drawn from q_j, from the stored logits in fp64.  pairs[j]: the (target row,
    draft row) CPU tensors of position j."""
    out = []
    for j, rows in enumerate(pairs):
        vals = []
        for zt, zd in rows:
            a = zt.to(torch.float64) / T
            b = zd.to(torch.float64) / T
            pa = torch.softmax(a, 0)
            pb = torch.softmax(b, 0)
            vals.append(float(torch.minimum(pa, pb).sum()))
        out.append(round(float(np.mean(vals)), 4))
    return out


def chain_rounds(wl, g, rounds, seed=0):
    """Accepted counts of `rounds` verification calls on one input copy (rounds 0.. : fresh uniforms)."""
    T = float(np.float32(wl.params["T"]))
    ns = [svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], T, seed=seed, round_=r, want_pq=False)["n"]
          for r in range(rounds)]
    return torch.stack(ns).cpu().numpy()


def multi_rounds(wl, g, rounds, seed=0):
    T = float(np.float32(wl.params["T"]))
    ns = [svx.sv_verify_multi(g["tgt"], g["drf"], g["tok"], T, seed=seed, round_=r, want_pq=False)["n_cand"]
          for r in range(rounds)]
    return torch.stack(ns).cpu().numpy()


STAT_KIND = {"chain_small_f32": "chain", "greedy_window": "greedy", "multi_candidate": "multi", "tree": "tree"}


def chain_stats(wl, rounds):
    """alpha_j over `rounds` rounds of fresh uniforms on the benchmarked inputs, the mean accepted length, and
    beta_j of the stored rows (draft-then-verify page §2.2; the SpecDiff-2 page's position-wise acceptance)."""
    p = wl.params
    g = wl.to("cuda")
    n = chain_rounds(wl, g, rounds)
    tgt, drf = wl.tensors["tgt"], wl.tensors["drf"]
    B, gamma = p["B"], p["gamma"]
    T = float(np.float32(p["T"]))
    beta = overlap_by_position(T, [[(tgt[b, j], drf[b, j]) for b in range(B)] for j in range(gamma)])
    out = dict(rounds=rounds, alpha_j=acceptance_by_position(n, gamma), mean_accepted=round(float(n.mean()), 3),
               beta_j=beta, beta_mean=round(float(np.mean(beta)), 4))
    del g
    return out


def small_chain_beta(instances=64):
    """beta of the small chain generator over `instances` seeds (one sequence each), per position and overall."""
    rows = [[] for _ in range(W.CHAIN_SMALL["gamma"])]
    for s in range(instances):
        w = W.chain_normal(**W.CHAIN_SMALL, seed=1000 + s)
        for j in range(W.CHAIN_SMALL["gamma"]):
            rows[j].append((w.tensors["tgt"][0, j], w.tensors["drf"][0, j]))
    beta = overlap_by_position(float(np.float32(W.CHAIN_SMALL["T"])), rows)
    return dict(instances=instances, beta_j=beta, beta_mean=round(float(np.mean(beta)), 4))


def greedy_stats(wl, rounds):
    """Greedy verification has no uniforms: alpha_j is the realised match rate at position j over the window's
    sequences, beside the generator's planted match probability 0.9 * 0.95^j."""
    g = wl.to("cuda")
    n = svx.sv_verify_greedy(g["tgt"], g["tok"], want_argmax=False)["n"].cpu().numpy()
    gamma = wl.params["gamma"]
    del g
    return dict(alpha_j=acceptance_by_position(n, gamma), mean_accepted=round(float(n.mean()), 3),
                planted_match_j=[round(0.9 * 0.95 ** j, 4) for j in range(1, gamma + 1)])


def multi_stats(wl, rounds):
    """alpha_j per candidate chain (all K candidates' accepted counts pooled) and of the kept candidate, over
    `rounds` rounds of fresh uniforms, and the kept candidate's mean accepted length."""
    g = wl.to("cuda")
    T = float(np.float32(wl.params["T"]))
    nc, kept = [], []
    for r in range(rounds):
        o = svx.sv_verify_multi(g["tgt"], g["drf"], g["tok"], T, seed=0, round_=r, want_pq=False)
        nc.append(o["n_cand"].cpu().numpy())
        kept.append(o["n"].cpu().numpy())
    nc, kept = np.stack(nc), np.stack(kept)
    gamma = wl.params["gamma"]
    del g
    return dict(rounds=rounds, alpha_j_per_candidate=acceptance_by_position(nc, gamma),
                alpha_j_kept=acceptance_by_position(kept, gamma), mean_accepted_per_candidate=round(float(nc.mean()), 3),
                mean_accepted_kept=round(float(kept.mean()), 3))


def tree_stats(wl, rounds):
    """Accepted depth over `rounds` rounds: the fraction of walks that reached depth d and went one deeper."""
    g = wl.to("cuda")
    p = wl.params
    T = float(np.float32(p["T"]))
    L = np.stack([svx.sv_verify_tree(g["tgt"], g["drf"], g["tok"], g["parent"], p["max_depth"], T, seed=0,
                                     round_=r, want_pq=False)["len"].cpu().numpy() for r in range(rounds)])
    del g
    return dict(rounds=rounds, alpha_d=acceptance_by_position(L, p["max_depth"]), mean_depth=round(float(L.mean()), 3))


# ------------------------------------------------------------------ CPU oracle
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def margin_counts(excepted, mismatch):
    """Near-margin sequences (a decision with |r - a| < 1e-6 or a draw within 1e-6 of a CDF edge in the
    oracle's fp64 arithmetic) and the GPU/oracle mismatches among them and outside them."""
    excepted = np.asarray(excepted, bool)
    mismatch = np.asarray(mismatch, bool)
    return dict(sequences=int(excepted.size), near_margin=int(excepted.sum()),
                mismatches_near_margin=int((mismatch & excepted).sum()),
                mismatches_outside=int((mismatch & ~excepted).sum()))


def oracle_parity(runs):
    """The oracle on the exact inputs each benchmarked call verified (copy 0, same seed and round), compared
    with the GPU outputs of that call."""
    import oracle
    res = {}
    for name, (kind, wl, out) in runs.items():
        p = wl.params
        t0 = time.perf_counter()
        if kind == "chain":
            ref = oracle.verify_chain(W.to_numpy_logits(wl.tensors["tgt"]), W.to_numpy_logits(wl.tensors["drf"]),
                                      wl.tensors["tok"].numpy(), float(np.float32(p["T"])), 0, 0, p["dtype"])
            n, t = out["n"].cpu().numpy(), out["tok"].cpu().numpy()
            r = margin_counts((ref["mdec"] < 1e-6) | (ref["mcdf"] < 1e-6), (n != ref["n"]) | (t != ref["t"]))
        elif kind == "multi":
            ref = oracle.verify_multi(W.to_numpy_logits(wl.tensors["tgt"]), W.to_numpy_logits(wl.tensors["drf"]),
                                      wl.tensors["tok"].numpy(), float(np.float32(p["T"])), 0, 0, p["dtype"])
            k, n, t = (out[x].cpu().numpy() for x in ("k", "n", "tok"))
            r = margin_counts((ref["mdec"] < 1e-6) | (ref["mcdf"] < 1e-6),
                              (k != ref["k"]) | (n != ref["n"]) | (t != ref["t"]))
        elif kind == "tree":
            ref = oracle.verify_tree(W.to_numpy_logits(wl.tensors["tgt"]), W.to_numpy_logits(wl.tensors["drf"]),
                                     wl.tensors["tok"].numpy(), wl.tensors["parent"].numpy(), p["max_depth"],
                                     float(np.float32(p["T"])), 0, 0, p["dtype"])
            L, path, t = out["len"].cpu().numpy(), out["path"].cpu().numpy(), out["tok"].cpu().numpy()
            r = margin_counts((ref["mdec"] < 1e-6) | (ref["mcdf"] < 1e-6),
                              (L != ref["len"]) | (t != ref["t"]) | (path != ref["path"]).any(1))
        else:  # greedy: no uniforms, so no margin; every output compared
            ref = oracle.verify_greedy(W.to_numpy_logits(wl.tensors["tgt"]), wl.tensors["tok"].numpy(), p["dtype"])
            n, t = out["n"].cpu().numpy(), out["tok"].cpu().numpy()
            r = margin_counts(np.zeros(len(n), bool), (n != ref["n"]) | (t != ref["t"]))
        r["oracle_s"] = round(time.perf_counter() - t0, 2)
        res[name] = r
        log(f"oracle parity {name}: {r}")
    return res


def cpu_baseline(wl, budget_s):
    import oracle
    p = wl.params
    T = float(np.float32(p["T"]))
    tgt, drf = W.to_numpy_logits(wl.tensors["tgt"]), W.to_numpy_logits(wl.tensors["drf"])
    tok = wl.tensors["tok"].numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.verify_chain(tgt, drf, tok, T, 0, 0, p["dtype"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    pos = reps * p["B"] * p["gamma"]
    return dict(value=round(pos / el, 1), unit="positions/s", cores=1, kind="oracle",
                sample=f"the full {p['B']}-sequence batch of the benchmarked workload, {reps} pass(es), {el:.1f} s, "
                       f"single-threaded fp64 C++",
                cpu_model=cpu_model(), nproc=os.cpu_count())


# ------------------------------------------------------------------ read probe
PROBE_SHAPES = [  # (label, blocks, mode, unroll, chunk bytes)
    ("ranges_1024_u4", 1024, 0, 4, 0), ("ranges_2048_u4", 2048, 0, 4, 0), ("ranges_4096_u4", 4096, 0, 4, 0),
    ("ranges_1024_u8", 1024, 0, 8, 0), ("ranges_2048_u2", 2048, 0, 2, 0),
    ("xcd_ranges_1024_u4", 1024, 1, 4, 0), ("xcd_ranges_2048_u4", 2048, 1, 4, 0),
    ("queue_1024_64K_u4", 1024, 2, 4, 1 << 16), ("queue_1024_128K_u4", 1024, 2, 4, 1 << 17),
    ("queue_2048_32K_u4", 2048, 2, 4, 1 << 15), ("queue_768_64K_u8", 768, 2, 8, 1 << 16),
]


def read_probe(sizes_mb=(311, 642), reps=30, shapes=None):
    """HBM read rate of sv_read_probe (the statistics kernels' load pattern) over buffers of the headline's row
    bytes and the greedy window's, for several launch shapes, rotating copies so that the last-level cache cannot
    serve repeats.  The statistics kernel's own shape is ranges_1024_u4."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = {}
    for mb in sizes_mb:
        nbytes = mb * 1000 * 1000 // 16 * 16
        copies = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_() for _ in
                  range(max(2, int(np.ceil(ROTATE_BYTES / nbytes))))]
        for label, blocks, mode, unroll, chunk in (shapes or PROBE_SHAPES):
            call = lambda i: svx.sv_read_probe(copies[i % len(copies)], sink, blocks, mode, unroll, chunk)
            for i in range(6):
                call(i)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(reps):
                call(i)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            gbs = nbytes / (us * 1e-6) / 1e9
            res[f"{mb}MB/{label}"] = dict(us=round(us, 2), GBps=round(gbs, 1), frac_of_peak=round(gbs / HBM_PEAK_GBS, 4))
            log(f"read probe {mb} MB {label}: {us:.2f} us, {gbs:.1f} GB/s")
        del copies
        torch.cuda.empty_cache()
    assert int(sink[1].item()) == 0 and int(sink[2].item()) == 0, "probe counters not returned to zero"
    best = {}
    for mb in sizes_mb:
        k = max((x for x in res if x.startswith(f"{mb}MB/")), key=lambda x: res[x]["GBps"])
        best[f"{mb}MB"] = dict(shape=k.split("/", 1)[1], **res[k])
    return dict(shapes=res, best=best)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-variants", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of CPU oracle work")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of graph replays (profiling runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0, help="also run copies of this size (counter calibration)")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel-source hash and exit")
    ap.add_argument("--read-probe", action="store_true",
                    help="run only the HBM read probe (311 MB and 642 MB buffers) and print its JSON line")
    ap.add_argument("--no-read-probe", action="store_true", help="leave the read probe out of the default run")
    ap.add_argument("--no-stats", action="store_true", help="skip the acceptance statistics and the oracle parity")
    ap.add_argument("--stat-rounds", type=int, default=32, help="verification rounds behind each alpha_j")
    args = ap.parse_args()
    if args.source_hash:
        print(kernel_source_hash())
        return
    global USE_GRAPHS
    USE_GRAPHS = not args.eager
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verification step shards by sequence with no exchange, "
              "and this build runs no multi-GPU configuration.", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)
    if args.read_probe:
        log("read probe: sv_read_probe over rotating buffers")
        print(json.dumps({"read_probe": read_probe(), "device": dev_name, "peak_GBps": HBM_PEAK_GBS}), flush=True)
        return

    log("generating the batched chain workload (B=32, gamma=16, V=152064, bf16)")
    wl = W.chain_zipf(**W.CHAIN_BATCHED)
    r, head_out = bench_chain(wl, args.steps, args.warmup)
    head = summarize(r)
    log(f"chain_batched: {head}")
    runs = {"chain_batched": ("chain", wl, head_out)}
    stats = {}
    if not args.no_stats:
        stats["chain_batched"] = chain_stats(wl, args.stat_rounds)
        log(f"chain_batched statistics: {stats['chain_batched']}")

    variants = {}
    if not args.no_variants:
        steps_v = max(10, args.steps // 2)
        warm_v = max(3, args.warmup // 2)
        for name, mk, fn in [
            ("chain_small_f32", lambda: W.chain_normal(**W.CHAIN_SMALL),
             lambda w: (lambda ro: {**ro[0], "_out": ro[1]})(bench_chain(w, steps_v, warm_v))),
            ("chain_pm_batched", lambda: wl, lambda w: bench_chain_pm(w, steps_v, warm_v)),
            ("greedy_window", lambda: W.greedy_zipf(**W.GREEDY_WINDOW), lambda w: bench_greedy(w, steps_v, warm_v)),
            ("multi_candidate", lambda: W.multi_zipf(**W.MULTI_CAND), lambda w: bench_multi(w, steps_v, warm_v)),
            ("tree", lambda: W.tree_zipf(**W.TREE_FANOUT), lambda w: bench_tree(w, steps_v, warm_v)),
        ]:
            log(f"generating {name}")
            w = mk()
            res = fn(w)
            variants[name] = summarize(res)
            log(f"{name}: {variants[name]}")
            if not args.no_stats and name in STAT_KIND:
                kind = STAT_KIND[name]
                runs[name] = (kind, w, res["_out"])
                stats[name] = {"chain": chain_stats, "greedy": greedy_stats, "multi": multi_stats,
                               "tree": tree_stats}[kind](w, args.stat_rounds)
                if name == "chain_small_f32":
                    stats[name]["generator"] = small_chain_beta()
                log(f"{name} statistics: {stats[name]}")
            if name == "chain_pm_batched":
                log("generating the lookahead row for the cache hit test")
                wc = W.chain_zipf(**W.CHAIN_BATCHED, lookahead_row=True)
                variants["cache_hit_test"] = summarize(bench_cache(wc, steps_v, warm_v))
                log(f"cache_hit_test: {variants['cache_hit_test']}")
                variants["branch_fork"] = summarize(bench_branch(wc, steps_v, warm_v))
                log(f"branch_fork: {variants['branch_fork']}")
                del wc
            if name == "tree":
                variants["tree_pm"] = summarize(bench_tree_pm(w, steps_v, warm_v))
                log(f"tree_pm: {variants['tree_pm']}")
                variants["fanout_tree_draft_rows"] = summarize(bench_fanout(w, steps_v, warm_v))
                log(f"fanout: {variants['fanout_tree_draft_rows']}")
                variants["presto_tree"] = summarize(bench_presto(w, steps_v, warm_v))
                log(f"presto: {variants['presto_tree']}")
            del w
            torch.cuda.empty_cache()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(wl, args.cpu_budget)
        cpu["cores"] = 1
        if not args.no_stats:
            log("the oracle on the benchmarked inputs (near-margin decisions and mismatches)")
            for name, rec in oracle_parity(runs).items():
                stats.setdefault(name, {})["oracle_parity"] = rec

    probe = None
    if not args.no_read_probe:
        log("read probe beside the headline (311 MB: the headline's streamed row bytes)")
        probe = read_probe(sizes_mb=(311,))

    rl = roofline(r["alg_bytes"], r["call_ms"])
    rl["kernel"] = ("sv_verify_chain call (one chain_kernel launch: statistics blocks, then draw blocks); duration = "
                    "HIP events around the graph replays on the launch stream / calls")
    rl["alg_bytes_per_call"] = int(r["alg_bytes"])
    line = {
        "metric": METRIC,
        "value": round(r["positions_per_s"], 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "chain_batched: B=32, gamma=16, V=152064, bf16 logits (fp32 arithmetic), T=0.8, "
                               "Zipf(1.1)+Gumbel target rows, draft noise sigma 0.5..2.5",
                   "B": 32, "gamma": 16, "V": 152064, "logits": "bf16", "device": dev_name,
                   "input_copies_rotated": r["copies"], "mean_accepted": round(r["mean_accepted"], 3),
                   "launch": ("one HIP graph holds >= 32 calls rotating over the input copies; the timed loop "
                              "replays it so that exactly `steps` calls run" if USE_GRAPHS else "eager calls"),
                   "eager_ms_per_step": round(r["eager_ms_per_step"], 5)},
        "roofline": rl,
        "cpu_baseline": cpu,
        "statistics": stats or None,
        "read_probe": probe,
        "variants": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
