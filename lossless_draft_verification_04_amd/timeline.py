"""Per-phase wall-clock timelines of the chain, small-call chain, tree and fan-out kernels (a measurement tool).

Uses the timeline build of the library, in which thread 0 of every block stores the 100 MHz wall clock at the
end of each phase (`sv_timeline_set` in include/specverify.h).  On a GPU:

    python -m lossless_draft_verification_04_amd.build --timeline
    python -m lossless_draft_verification_04_amd.timeline

Each workload runs warm-up calls, then one stamped eager call per repetition.  Times are microseconds from the
first stamped block's start; "max" is over the blocks of a sequence (the last one decides when it is done).
The stamps are one store per phase per block, so the timed calls run close to the normal build's, but the
numbers are for locating time, not for the benchmark line.
"""
from __future__ import annotations

import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
os.environ.setdefault("SV_LIBRARY", os.path.join(_HERE, "libspecverify_timeline.so"))

import numpy as np  # noqa: E402
import torch  # noqa: E402

from . import specverify as svx  # noqa: E402
from . import workloads as W  # noqa: E402

RECORDS = 32768          # records of 16 words; a tree call's walk launch starts at record 16384
WALK_BASE = 16384
TICK_US = 0.01           # s_memrealtime runs at 100 MHz


class Stamps:
    def __init__(self, dev):
        self.buf = torch.zeros(RECORDS * 16, dtype=torch.int64, device=dev)
        svx.sv_timeline_set(self.buf)

    def take(self, fn):
        self.buf.zero_()
        torch.cuda.synchronize()
        out = fn()
        torch.cuda.synchronize()
        st = self.buf.view(RECORDS, 16).cpu().numpy().astype(np.int64)
        tag = st[:, 15]
        return out, st, tag & 0xFF, (tag >> 8) & 0xFFFFFFFF, (tag >> 40) & 0xF


def _fmt(v):
    return "—" if v is None or not np.isfinite(v) else f"{v:6.2f}"


def chain(stamps, reps, multi=False):
    if multi:
        wl = W.multi_zipf(**W.MULTI_CAND)
        g = wl.to("cuda")
        T = float(np.float32(wl.params["T"]))
        fn = lambda: svx.sv_verify_multi(g["tgt"], g["drf"], g["tok"], T, want_pq=False)  # noqa: E731
        title = "## multi, B=16, K=8, gamma=16, V=128256 bf16"
    else:
        wl = W.chain_zipf(**W.CHAIN_BATCHED)
        g = wl.to("cuda")
        T = float(np.float32(wl.params["T"]))
        fn = lambda: svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], T, want_pq=False)  # noqa: E731
        title = "## chain, B=32, gamma=16, V=152064 bf16 (the headline batch)"
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    lines = [title, ""]
    for rep in range(reps):
        out, st, role, seq, xcd = stamps.take(fn)
        S, D = np.nonzero(role == 1)[0], np.nonzero(role == 2)[0]
        t0 = st[np.concatenate([S, D]), 0].min()
        u = lambda v: (v - t0) * TICK_US  # noqa: E731

        def mx(rows, c):
            v = st[rows, c]
            v = v[v > 0]
            return u(v.max()) if len(v) else None

        ends = [mx(S[xcd[S] == x], 1) for x in range(8)]
        lines.append(f"call {rep}: statistics blocks {len(S)}, draw blocks {len(D)}, last exit {_fmt(mx(D, 6))}")
        lines.append("statistics end, max per XCD: " + ", ".join(_fmt(e) for e in ends))
        lines.append("")
        lines.append("| seq | XCD | n | statistics end | draw start | parts seen | decided | prepared | exchanged | "
                     "searched | exit |")
        lines.append("|---|---|---|---|---|---|---|---|---|---|---|")
        n = out["n"].cpu().numpy()
        for b in range(wl.params["B"]):
            ms, md = S[seq[S] == b], D[seq[D] == b]
            lines.append(f"| {b} | {int(xcd[ms][0]) if len(ms) else -1} | {int(n[b])} | {_fmt(mx(ms, 1))} | "
                         f"{_fmt(mx(md, 0))} | {_fmt(mx(md, 1))} | {_fmt(mx(md, 2))} | {_fmt(mx(md, 3))} | "
                         f"{_fmt(mx(md, 4))} | {_fmt(mx(md, 5))} | {_fmt(mx(md, 6))} |")
        lines.append("")
    return lines


def small(stamps, reps):
    wl = W.chain_normal(**W.CHAIN_SMALL)
    g = wl.to("cuda")
    fn = lambda: svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0, want_pq=False)  # noqa: E731
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    names = ["start", "wave max", "block parts", "published", "parts merged", "decided", "draw exchanged", "end"]
    lines = ["## small-call chain, B=1, gamma=4, V=32000 fp32", "", "| call | blocks | " + " | ".join(names) + " |",
             "|---|---|" + "---|" * len(names)]
    for rep in range(reps):
        _, st, role, _, _ = stamps.take(fn)
        Bk = np.nonzero(role == 3)[0]
        t0 = st[Bk, 0].min()
        cols = []
        for c in range(len(names)):
            v = st[Bk, c]
            v = v[v > 0]
            cols.append(f"{np.median((v - t0) * TICK_US):.2f} / {((v.max() - t0) * TICK_US):.2f}" if len(v) else "—")
        lines.append(f"| {rep} | {len(Bk)} | " + " | ".join(cols) + " |")
    lines += ["", "(median / max over the blocks)", ""]
    return lines


def tree(stamps, reps):
    wl = W.tree_zipf(**W.TREE_FANOUT)
    g = wl.to("cuda")
    p = wl.params
    T = float(np.float32(p["T"]))
    fn = lambda: svx.sv_verify_tree(g["tgt"], g["drf"], g["tok"], g["parent"], p["max_depth"], T,  # noqa: E731
                                    want_pq=False)
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    lines = ["## tree, B=8, N=64, V=128256 bf16", ""]
    for rep in range(reps):
        out, st, role, seq, xcd = stamps.take(fn)
        S = np.nonzero(role == 4)[0]
        Wk = np.nonzero(role == 5)[0]
        t0 = np.concatenate([st[S, 0], st[Wk, 0]])
        t0 = t0[t0 > 0].min()
        u = lambda v: (v - t0) * TICK_US  # noqa: E731
        ends = [u(st[S[xcd[S] == x], 1].max()) if (xcd[S] == x).any() else None for x in range(8)]
        lines.append(f"call {rep}: statistics blocks streaming {len(S)} (last start {_fmt(u(st[S, 0].max()))}), "
                     f"walk blocks {len(Wk)}")
        lines.append("statistics end, max per XCD: " + ", ".join(_fmt(e) for e in ends))
        lines.append("")
        lines.append("| seq | walk start | staged | nodes entered (children known) | passes | summing (µs) | "
                     "exchanging (µs) | final draw start | searched | end | depth |")
        lines.append("|---|---|---|---|---|---|---|---|---|---|---|")
        for b in range(p["B"]):
            m = Wk[seq[Wk] == b]

            def last(c):
                v = st[m, c]
                v = v[v > 0]
                return u(v.max()) if len(v) else None
            nodes = ", ".join(_fmt(last(c)).strip() for c in range(7, 12) if last(c) is not None)
            lines.append(f"| {b} | {_fmt(u(st[m, 0].min()))} | {_fmt(u(st[m, 1].max()))} | {nodes} | "
                         f"{int(st[m, 4].max())} | {st[m, 2].max() * TICK_US:.2f} | {st[m, 3].max() * TICK_US:.2f} | "
                         f"{_fmt(last(12))} | {_fmt(last(13))} | {_fmt(u(st[m, 5].max()))} | {int(st[m, 6].max())} |")
        lines.append("")
    return lines


def fanout(stamps, reps):
    wl = W.tree_zipf(**W.TREE_FANOUT)
    B, N, V = wl.tensors["drf"].shape
    F = torch.tensor([W.fanout_schedule(8, 0.7, 1.0, 9)[d] for d in wl.tensors["depth"].reshape(-1).tolist()],
                     dtype=torch.int32, device="cuda")
    x = wl.to("cuda")["drf"].reshape(B * N, V)
    fn = lambda: svx.sv_fanout_topk(x, F, 8, want_vals=False)  # noqa: E731
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    names = ["start", "thread 0 pass 1", "group maxima", "bound", "wave 0 listed", "candidates listed", "selected",
             "written"]
    cols_of = [0, 2, 6, 7, 8, 3, 4, 5]
    lines = [f"## fan-out, {B * N} tree draft rows, V={V} bf16", "",
             "| call | blocks | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for rep in range(reps):
        _, st, role, _, _ = stamps.take(fn)
        Bk = np.nonzero(role == 6)[0]
        t0 = st[Bk, 0].min()
        cols = []
        for c in cols_of:
            v = st[Bk, c]
            v = v[v > 0]
            cols.append(f"{np.median((v - t0) * TICK_US):.2f} / {((v.max() - t0) * TICK_US):.2f}" if len(v) else "—")
        lines.append(f"| {rep} | {len(Bk)} | " + " | ".join(cols) + " |")
        med = lambda a, b: np.median((st[Bk, b] - st[Bk, a]) * TICK_US)  # noqa: E731
        lines.append("")
        lines.append(f"per block (medians): pass 1 of thread 0 to group maxima {med(2, 6):.2f} (last wave's pass 1 "
                     f"{med(2, 9):.2f}), to the bound {med(6, 7):.2f}, to wave 0 listed {med(7, 8):.2f} (last wave "
                     f"{med(7, 10):.2f}), to all listed {med(8, 3):.2f}, to selected {med(3, 4):.2f}, to written "
                     f"{med(4, 5):.2f}")
        lines.append("")
    lines += ["(median / max over the blocks)", ""]
    return lines


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    reps = int(argv[0]) if argv else 2
    if not torch.cuda.is_available():
        raise SystemExit("timeline: needs a GPU")
    stamps = Stamps(torch.device("cuda", 0))
    lines = ["# Kernel timelines (timeline build, wall-clock stamps per block)", ""]
    for part in (chain, lambda st, r: chain(st, r, multi=True), small, tree, fanout):
        lines += part(stamps, reps)
        print("\n".join(lines), flush=True)
        lines = []
    svx.sv_timeline_set(None)


if __name__ == "__main__":
    main()
