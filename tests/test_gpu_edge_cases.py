"""GPU parity at the method's degenerate inputs, against the CPU oracle.

Zero probability at a drafted token.  A top-k or nucleus filter acts on both
the target and the draft distribution (draft-then-verify page §4, sampling
standardisation), so a drafted token can carry p(x) = 0 (the target filtered
it out) or q(x) = 0 while p(x) > 0.  The acceptance ratio of §2.1,
min(1, p/q), then rejects for sure (p = 0) or accepts for sure (q = 0,
p > 0); the residual max(0, p - q) never lands on a token the target
filtered out.  Each case is built so that the accepted lengths follow from
the masks alone, and the GPU is compared with the oracle on the same bytes.

Ties at the row maximum in greedy verification (draft-then-verify page §2.2:
greedy acceptance is an argmax-id match; ties go to the lowest index) on the
full greedy window with nothing planted, and on rows split over many row
parts with ties planted across parts.
"""
import numpy as np
import pytest
import torch

from lossless_draft_verification_04_amd import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu

NEG = float("-inf")


def _mask_chain(wl, pattern):
    """pattern[b] = (accept_until, kind): drafts 1..accept_until have q(x) = 0 (sure accepts); position
    accept_until + 1, if inside the window, has p(x) = 0 ('p'), or p = q = 0 ('pq'); returns the expected n."""
    tgt, drf, tok = wl.tensors["tgt"], wl.tensors["drf"], wl.tensors["tok"]
    gamma = tok.shape[1]
    want = []
    for b, (upto, kind) in enumerate(pattern):
        for j in range(upto):
            drf[b, j, tok[b, j]] = NEG
        if upto < gamma:
            tgt[b, upto, tok[b, upto]] = NEG
            if kind == "pq":
                drf[b, upto, tok[b, upto]] = NEG
        want.append(upto)
    return np.array(want)


@pytest.mark.parametrize("dtype,V", [("bf16", 30011), ("f32", 4099)])
def test_chain_zero_probability_drafts(dtype, V):
    gamma, B = 8, 18
    wl = W.chain_zipf(B=B, gamma=gamma, V=V, T=0.9, dtype=dtype, seed=31)
    pattern = [(b % (gamma + 1), "pq" if b % 3 == 0 else "p") for b in range(B)]
    want = _mask_chain(wl, pattern)
    for seed, rnd in [(0, 0), (7, 3)]:
        out, ref = PT.chain(wl, seed, rnd)
        assert np.array_equal(ref["n"], want), "oracle: q(x)=0 must accept and p(x)=0 must reject"
        assert np.array_equal(out["n"].cpu().numpy(), want)
        # the correction never lands on a token the target filtered out
        t = out["tok"].cpu().numpy()
        for b in range(B):
            assert torch.isfinite(wl.tensors["tgt"][b, want[b], t[b]].float())
    PT.device_error_clear()


def test_chain_pm_zero_probability_drafts():
    # point-mass acceptance (U < p(x)): a filtered-out draft is rejected for sure
    gamma, B = 6, 14
    wl = W.chain_zipf(B=B, gamma=gamma, V=20011, T=1.0, seed=32)
    tgt, tok = wl.tensors["tgt"], wl.tensors["tok"]
    cut = [b % (gamma + 1) for b in range(B)]
    for b in range(B):
        if cut[b] < gamma:
            tgt[b, cut[b], tok[b, cut[b]]] = NEG
    for seed in (0, 9):
        out, ref = PT.chain_pm(wl, seed, 1)
        assert (ref["n"] <= np.array(cut)).all()
        t = out["tok"].cpu().numpy()
        n = out["n"].cpu().numpy()
        for b in range(B):
            assert torch.isfinite(tgt[b, n[b], t[b]].float())
    PT.device_error_clear()


def test_multi_zero_probability_drafts():
    B, K, gamma, V = 6, 4, 8, 20011
    wl = W.multi_zipf(B=B, K=K, gamma=gamma, V=V, T=1.0, seed=33)
    tgt, drf, tok = wl.tensors["tgt"], wl.tensors["drf"], wl.tensors["tok"]
    want = np.zeros((B, K), np.int64)
    for b in range(B):
        for k in range(K):
            cut = (b + 2 * k) % (gamma + 1)
            # the shared draft row keeps q > 0 at other candidates' tokens unless they coincide; target rows are
            # per candidate, so p(x) = 0 at the cut only affects this candidate
            if cut < gamma:
                tgt[b, k, cut, tok[b, k, cut]] = NEG
            want[b, k] = cut
    for b in range(B):
        for k in range(K):
            for j in range(want[b, k]):
                drf[b, j, tok[b, k, j]] = NEG  # q(x) = 0: a sure accept for every candidate drafting x here
    for seed in (0, 4):
        out, ref = PT.multi(wl, seed, 2)
        # sure accepts up to the cut, a sure reject at it
        assert np.array_equal(ref["n_cand"], want)
    PT.device_error_clear()


def test_tree_zero_probability_children():
    wl = W.tree_zipf(B=6, N=40, max_depth=6, V=20011, T=1.0, seed=34)
    tgt, drf, tok, par = (wl.tensors[k] for k in ("tgt", "drf", "tok", "parent"))
    B, N = par.shape
    g = torch.Generator().manual_seed(35)
    kinds = torch.randint(0, 3, (B, N), generator=g)
    for b in range(B):
        for i in range(1, N):
            u = int(par[b, i])
            x = int(tok[b, i])
            if kinds[b, i] == 1:
                tgt[b, u, x] = NEG  # p(x) = 0 under its parent: rejected at any residual step
            elif kinds[b, i] == 2:
                drf[b, u, x] = NEG  # q(x) = 0 with p(x) > 0: accepted whenever it is tried
    for seed, rnd in [(0, 0), (3, 5)]:
        out, ref = PT.tree(wl, seed, rnd)
        path = ref["path"]
        for b in range(B):
            for d in range(int(ref["len"][b])):
                assert kinds[b, path[b, d]] != 1  # a p(x) = 0 child is never on the accepted path
            # every tried child with q(x) = 0 was accepted, so it ends its node's trials
            tried = np.nonzero(~np.isnan(ref["p"][b]))[0]
            for i in tried:
                if kinds[b, i] == 2 and ref["p"][b, i] > 0:
                    assert i in set(path[b, :ref["len"][b]].tolist())
        t = out["tok"].cpu().numpy()
        L = out["len"].cpu().numpy()
        for b in range(B):
            last = 0 if L[b] == 0 else int(out["path"][b, L[b] - 1])
            assert torch.isfinite(tgt[b, last, t[b]].float())
    PT.device_error_clear()


def test_tree_pm_zero_probability_children():
    wl = W.tree_zipf(B=6, N=40, max_depth=6, V=20011, T=1.0, seed=36)
    tgt, tok, par = (wl.tensors[k] for k in ("tgt", "tok", "parent"))
    B, N = par.shape
    for b in range(B):
        for i in range(1, N, 2):
            tgt[b, int(par[b, i]), int(tok[b, i])] = NEG
    for seed in (0, 6):
        out, ref = PT.tree_pm(wl, seed, 1)
        for b in range(B):
            for d in range(int(ref["len"][b])):
                assert ref["path"][b, d] % 2 == 0
    PT.device_error_clear()


# ----------------------------------------------------------------- greedy ties at the maximum
def _tie_rows(tgt):
    x = tgt.float()
    mx = x.max(-1, keepdim=True).values
    return (x == mx).sum(-1)


def test_greedy_full_window_unplanted_ties():
    wl = W.greedy_zipf(**W.GREEDY_WINDOW, plant=False, seed=1013)
    cnt = _tie_rows(wl.tensors["tgt"])
    PT.say(f"  rows with a tie at the maximum: {int((cnt > 1).sum())} of {cnt.numel()}")
    assert int((cnt > 1).sum()) >= 5
    out, ref = PT.greedy(wl)
    # the lowest tied index is the argmax of every tied row
    x = wl.tensors["tgt"].float()
    am = out["argmax"].cpu()
    for b, j in torch.nonzero(cnt > 1).tolist():
        first = int(torch.nonzero(x[b, j] == x[b, j].max())[0])
        assert int(am[b, j]) == first


def test_greedy_ties_across_row_parts():
    # two sequences: every row is split over several row parts, and ties at the maximum are planted in
    # different parts (one before and one after the first maximal index)
    V = 151936
    wl = W.greedy_zipf(B=2, gamma=32, V=V, plant=False, seed=1014)
    tgt = wl.tensors["tgt"]
    g = torch.Generator().manual_seed(37)
    for b in range(2):
        for j in range(0, 33, 2):
            row = tgt[b, j]
            m = row.float().max()
            first = int(torch.nonzero(row.float() == m)[0])
            lo = int(torch.randint(0, max(first - 20000, 1), (1,), generator=g))
            hi = int(torch.randint(min(first + 20000, V - 1), V, (1,), generator=g))
            if j % 4 == 0 and first > 20000:
                row[lo] = row[first]  # a new first maximum, parts earlier
            row[hi] = row[first]
    # draft tokens re-pointed at the (new) first maxima where they matched before
    tok = wl.tensors["tok"]
    x = tgt.float()
    for b in range(2):
        for j in range(32):
            if int(tok[b, j]) == int(wl.tensors["planted"][b, j]):
                tok[b, j] = int(torch.nonzero(x[b, j] == x[b, j].max())[0])
    PT.greedy(wl)
