"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: exact
enumeration of its output distribution against the target's chain rule,
closed forms for acceptance statistics, reductions to library routines,
known-answer vectors and an independent Philox implementation.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import scipy.special

import oracle
from tests import enum_pins as E

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


# --------------------------------------------------------------------------
# Philox4x32-10 (SC'11): known-answer vectors and PyTorch's header engine
# --------------------------------------------------------------------------
def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox_kat.txt")) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            v = [int(x, 16) for x in ln.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, want in rows:
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_philox_matches_pytorch_engine(tmp_path):
    import torch.utils.cpp_extension as ce
    exe = str(tmp_path / "philox_ref")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I" + ce.include_paths()[0],
                    os.path.join(HERE, "philox_torch_ref.cpp"), "-o", exe], check=True)
    rng = np.random.default_rng(7)
    cases = rng.integers(0, 2 ** 32, size=(300, 6), dtype=np.uint64)
    cases[:20, :4] = rng.integers(0, 64, size=(20, 4))  # small counters like the verifier's
    text = "\n".join(" ".join(str(int(x)) for x in row) for row in cases) + "\n"
    res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    got = [list(map(int, ln.split())) for ln in res.stdout.strip().splitlines()]
    assert len(got) == len(cases)
    for row, ref in zip(cases, got):
        assert list(oracle.philox4x32_10(row[:4], row[4:6])) == ref


def test_uniform_grid_and_uniformity():
    # U = (w >> 8) * 2^-24 of the first Philox word of counter (idx, b, k, round<<2|tag)
    seed = 0x1234_5678_9ABC_DEF0
    w = oracle.philox4x32_10([3, 5, 7, (9 << 2) | 1], [seed & 0xFFFFFFFF, seed >> 32])[0]
    assert oracle.uniform(seed, 3, 5, 7, 9, 1) == (int(w) >> 8) / 2.0 ** 24
    us = np.array([oracle.uniform(0, j, b, 0, 0, 0) for j in range(1, 65) for b in range(400)])
    assert us.min() >= 0.0 and us.max() < 1.0
    counts, _ = np.histogram(us, bins=32, range=(0, 1))
    chi2 = ((counts - len(us) / 32) ** 2 / (len(us) / 32)).sum()
    assert chi2 < 70.0  # 31 dof: p ~ 1e-4 tail


# --------------------------------------------------------------------------
# Losslessness by exact enumeration (draft-verification page §2.1 proof):
# the sequence produced by repeated rounds has exactly the target's law.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("gamma,m,T,pz,qz,seed", [
    (1, 3, 1.0, 0.0, 0.0, 11),
    (2, 3, 1.0, 0.0, 0.0, 12),
    (2, 2, 0.6, 0.3, 0.3, 13),   # zeros in p (never accepted) and q (residual must supply them)
    (3, 2, 1.7, 0.0, 0.4, 14),
    (3, 1, 1.0, 0.5, 0.0, 15),
])
def test_chain_round_is_lossless(gamma, m, T, pz, qz, seed):
    tab = E.Tables(5, seed, p_zero=pz, q_zero=qz)
    d = E.chain_sequence_distribution(tab, gamma, m, T=T)
    assert E.max_marginal_error(tab, d, m) < 1e-12


@pytest.mark.parametrize("parent,m,seed,T", [
    ([-1, 0, 0], 2, 21, 1.0),            # two i.i.d. siblings under the root
    ([-1, 0, 0, 1], 2, 22, 1.0),         # siblings + depth 2
    ([-1, 0, 0, 0], 1, 23, 0.8),         # three siblings
    ([-1, 0, 1, 1, 0], 1, 24, 1.3),      # siblings at depth 2 under the first child
])
def test_tree_round_with_iid_siblings_is_lossless(parent, m, seed, T):
    tab = E.Tables(5, seed, q_zero=0.2)
    d = E.tree_sequence_distribution(tab, parent, m, T=T)
    assert E.max_marginal_error(tab, d, m) < 1e-12


def test_single_step_acceptance_law():
    """gamma = 1: P(accept) = sum min(p, q) (page §2.2) and the emitted token ~ p (page §2.1)."""
    tab = E.Tables(6, 31, q_zero=0.3)
    p, q = tab.p(()), tab.q(())
    acc = 0.0
    emitted = np.zeros(6)
    T = 1.0
    for x in range(6):
        if q[x] == 0:
            continue
        tgt = np.stack([E.logits_of(p, T), E.logits_of(tab.p((x,)), T)])
        drf = E.logits_of(q, T)[None]

        def run(r, u, tgt=tgt, drf=drf, x=x):
            o = oracle.chain_core(tgt, drf, np.array([x]), T, r, u)
            return ((x,) if o["n"] else ()) + (o["t"],), o["a"], o["w"]

        for e, pr in E.enumerate_cells(run, 1, 6).items():
            if len(e) == 2:
                acc += q[x] * pr
            emitted[e[0]] += q[x] * pr
    beta = np.minimum(p, q).sum()
    assert abs(acc - beta) < 1e-14
    assert abs(beta - (1 - 0.5 * np.abs(p - q).sum())) < 1e-14
    assert np.max(np.abs(emitted - p)) < 1e-14


# --------------------------------------------------------------------------
# Acceptance statistics with Philox uniforms (page §2.2, §2.3, §3; the
# truncated-geometric law on the SpecBranch page's motivation section)
# --------------------------------------------------------------------------
def _fixed_rows(V, gamma, seed, same=False):
    rng = np.random.default_rng(seed)
    P = [rng.dirichlet(np.full(V, 0.5)) for _ in range(gamma + 1)]
    Q = [rng.dirichlet(np.full(V, 0.5)) for _ in range(gamma)]
    if same:
        P = [P[0]] * (gamma + 1)
        Q = [Q[0]] * gamma
    return P, Q


def _run_fixed(P, Q, B, seed, T=1.0):
    gamma, V = len(Q), len(P[0])
    rng = np.random.default_rng(seed)
    tgt = np.broadcast_to(np.stack([E.logits_of(p, T) for p in P]), (B, gamma + 1, V)).copy()
    drf = np.broadcast_to(np.stack([E.logits_of(q, T) for q in Q]), (B, gamma, V)).copy()
    tok = np.stack([rng.choice(V, size=B, p=Q[j]) for j in range(gamma)], axis=1).astype(np.int32)
    o = oracle.verify_chain(tgt, drf, tok, T, seed=seed, round_=3, dtype="f64")
    return o, tok


def test_positionwise_acceptance_equals_overlap():
    V, gamma, B = 12, 4, 40000
    P, Q = _fixed_rows(V, gamma, 41)
    o, _ = _run_fixed(P, Q, B, 41)
    n = o["n"]
    assert n.min() >= 0 and n.max() <= gamma  # 1 <= emitted <= gamma + 1
    for j in range(gamma):
        reached = (n >= j).sum()
        acc = (n >= j + 1).sum()
        beta = np.minimum(P[j], Q[j]).sum()
        sd = math.sqrt(beta * (1 - beta) / reached)
        assert abs(acc / reached - beta) < 4 * sd + 1e-3


def test_expected_length_product_of_accepts():
    V, gamma, B = 10, 5, 40000
    P, Q = _fixed_rows(V, gamma, 42)
    o, _ = _run_fixed(P, Q, B, 42)
    beta = np.array([np.minimum(P[j], Q[j]).sum() for j in range(gamma)])
    cum = np.cumprod(beta)
    En = cum.sum()  # c1 + c1 c2 + ...
    n = o["n"].astype(float)
    assert abs(n.mean() - En) < 4 * n.std() / math.sqrt(B)
    probs = [(1 - beta[0])] + [cum[k - 1] * (1 - beta[k]) for k in range(1, gamma)] + [cum[-1]]
    for k, pk in enumerate(probs):
        frac = (o["n"] == k).mean()
        assert abs(frac - pk) < 4 * math.sqrt(pk * (1 - pk) / B) + 1e-3


def test_iid_alpha_closed_form_and_truncated_geometric():
    V, gamma, B = 8, 6, 40000
    P, Q = _fixed_rows(V, gamma, 43, same=True)
    alpha = np.minimum(P[0], Q[0]).sum()
    o, _ = _run_fixed(P, Q, B, 43)
    tokens = o["n"] + 1.0
    want = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(tokens.mean() - want) < 4 * tokens.std() / math.sqrt(B)
    for k in range(gamma + 1):
        pk = (1 - alpha) * alpha ** k if k < gamma else alpha ** gamma
        frac = (o["n"] == k).mean()
        assert abs(frac - pk) < 4 * math.sqrt(pk * (1 - pk) / B) + 1e-3


def test_softmax_with_temperature_matches_library():
    rng = np.random.default_rng(5)
    B, gamma, V = 3, 4, 257
    for T in (0.3, 0.8, 1.0, 2.5):
        tgt = rng.normal(0, 3, (B, gamma + 1, V))
        drf = tgt[:, :gamma] + rng.normal(0, 1, (B, gamma, V))
        tgt[0, 1, :100] = -np.inf  # masked logits are probability 0
        tok = rng.integers(0, V, (B, gamma)).astype(np.int32)
        o = oracle.verify_chain(tgt, drf, tok, T, 0, 0, "f64")
        p_ref = scipy.special.softmax(tgt[:, :gamma] / T, axis=-1)
        q_ref = scipy.special.softmax(drf / T, axis=-1)
        pg = np.take_along_axis(p_ref, tok[..., None], -1)[..., 0]
        qg = np.take_along_axis(q_ref, tok[..., None], -1)[..., 0]
        assert np.allclose(o["p"], pg, rtol=1e-12, atol=0)
        assert np.allclose(o["q"], qg, rtol=1e-12, atol=0)


def test_bf16_and_f32_inputs_convert_exactly():
    rng = np.random.default_rng(6)
    V, gamma = 64, 3
    f32 = rng.normal(0, 3, (1, gamma + 1, V)).astype(np.float32)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)  # truncation gives exact bf16 values
    as_f64 = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tok = rng.integers(0, V, (1, gamma)).astype(np.int32)
    a = oracle.verify_chain(bits, bits[:, :gamma].copy(), tok, 1.0, 9, 1, "bf16")
    b = oracle.verify_chain(as_f64, as_f64[:, :gamma].copy(), tok, 1.0, 9, 1, "f64")
    assert np.array_equal(a["p"], b["p"]) and a["t"][0] == b["t"][0] and a["n"][0] == b["n"][0]
    c = oracle.verify_chain(f32, f32[:, :gamma].copy(), tok, 1.0, 9, 1, "f32")
    d = oracle.verify_chain(f32.astype(np.float64), f32[:, :gamma].astype(np.float64), tok, 1.0, 9, 1, "f64")
    assert np.array_equal(c["p"], d["p"]) and c["t"][0] == d["t"][0]


# --------------------------------------------------------------------------
# Greedy (page §2.2, §4): the chain rule fed one-hot p and q is an id match
# --------------------------------------------------------------------------
def _onehot_logits(idx, V):
    z = np.full(V, -1e4)
    z[idx] = 0.0
    return z


def test_greedy_equals_chain_on_one_hot_rows():
    rng = np.random.default_rng(8)
    B, gamma, V = 40, 6, 50
    tgt = rng.normal(0, 2, (B, gamma + 1, V))
    g = tgt.argmax(-1)
    tok = np.where(rng.random((B, gamma)) < 0.7, g[:, :gamma], rng.integers(0, V, (B, gamma))).astype(np.int32)
    og = oracle.verify_greedy(tgt, tok, "f64")
    assert np.array_equal(og["argmax"], g)
    P1 = np.stack([[_onehot_logits(g[b, j], V) for j in range(gamma + 1)] for b in range(B)])
    Q1 = np.stack([[_onehot_logits(tok[b, j], V) for j in range(gamma)] for b in range(B)])
    for seed in (0, 1, 99):
        oc = oracle.verify_chain(P1, Q1, tok, 1.0, seed, 0, "f64")
        assert np.array_equal(oc["n"], og["n"]) and np.array_equal(oc["t"], og["t"])


def test_greedy_ties_lowest_index_and_signed_zero():
    V = 32
    rows = np.full((1, 3, V), -5.0)
    rows[0, 0, [7, 3, 20]] = 2.0           # ties -> 3
    rows[0, 1, 9] = -0.0
    rows[0, 1, 4] = 0.0                    # -0 == +0 -> 4
    rows[0, 2, :] = 1.0                    # all equal -> 0
    o = oracle.verify_greedy(rows, np.array([[3, 4]], np.int32), "f64")
    assert list(o["argmax"][0]) == [3, 4, 0] == [int(np.argmax(r)) for r in rows[0]]
    assert o["n"][0] == 2 and o["t"][0] == 0
    bits = np.full((2, 5, V), 0x3F80, np.uint16)  # bf16 1.0 everywhere
    bits[1, 2, 17] = 0x4000  # 2.0
    o = oracle.verify_greedy(bits, np.array([[0, 0, 0, 1], [0, 0, 17, 0]], np.int32), "bf16")
    assert list(o["n"]) == [3, 4] and list(o["t"]) == [0, 0]


# --------------------------------------------------------------------------
# Multi-candidate and tree reductions
# --------------------------------------------------------------------------
def test_multi_k1_is_chain_and_each_candidate_is_its_chain():
    """SpecDiff-2 page, Core method: the kept candidate is verified as a chain (draft-then-verify page §2.1),
    so for any K its n is that candidate's own chain n and the emitted token is the chain's draw on ITS rows
    (its target row n+1 against the shared draft row, or its bonus row) with the sequence's one sampling
    uniform."""
    rng = np.random.default_rng(9)
    B, K, gamma, V = 40, 4, 5, 40
    tgt = rng.normal(0, 2, (B, K, gamma + 1, V))
    drf = tgt[:, 0, :gamma] + rng.normal(0, 1, (B, gamma, V))
    # drafts drawn near the target's mode so that streaks differ between candidates
    tok = np.argmax(tgt[:, :, :gamma] + rng.gumbel(0, 1.5, (B, K, gamma, V)), axis=-1).astype(np.int32)
    om = oracle.verify_multi(tgt, drf, tok, 0.9, 77, 5, "f64")
    alone = []
    for k in range(K):
        # candidate k alone, with the acceptance uniforms drawn at counter k and the shared sampling uniform
        r = np.array([[oracle.uniform(77, j + 1, b, k, 5, 0) for j in range(gamma)] for b in range(B)])
        o1 = oracle.verify_multi(tgt[:, k:k + 1].copy(), drf, tok[:, k:k + 1].copy(), 0.9, 77, 5, "f64",
                                 r=r[:, None, :])
        assert np.array_equal(o1["n"], om["n_cand"][:, k])
        alone.append(o1)
    ks = om["k"]
    for b in range(B):
        o1 = alone[ks[b]]
        assert om["t"][b] == o1["t"][b] and om["mcdf"][b] == o1["mcdf"][b]
        assert om["rows"][b] == o1["rows"][b]
    # the draw is not a candidate-independent quantity here: a kept candidate other than the first and the
    # last occurs, and another candidate's draw would have given another token
    assert np.any((ks != 0) & (ks != K - 1))
    for other in (0, K - 1):
        assert np.any(np.array([alone[other]["t"][b] != om["t"][b] for b in range(B)]) & (ks != other))
    assert np.array_equal(om["n"], om["n_cand"].max(1))
    assert np.array_equal(om["k"], np.argmax(om["n_cand"], 1))  # lowest k among the longest
    o1 = oracle.verify_multi(tgt[:, :1].copy(), drf, tok[:, :1].copy(), 0.9, 77, 5, "f64")
    oc = oracle.verify_chain(tgt[:, 0].copy(), drf, tok[:, 0].copy(), 0.9, 77, 5, "f64")
    for key in ("n", "t", "mdec", "mcdf"):
        assert np.array_equal(o1[key], oc[key])
    assert np.array_equal(o1["p"][:, 0], oc["p"]) and np.array_equal(o1["q"][:, 0], oc["q"])


def test_chain_shaped_tree_is_chain():
    rng = np.random.default_rng(10)
    B, gamma, V = 30, 6, 60
    for T in (1.0, 0.7):
        tgt = rng.normal(0, 2, (B, gamma + 1, V))
        drf = tgt[:, :gamma] + rng.normal(0, 1.5, (B, gamma, V))
        tok = rng.integers(0, V, (B, gamma)).astype(np.int32)
        oc = oracle.verify_chain(tgt, drf, tok, T, 5, 2, "f64")
        N = gamma + 1
        tdrf = np.concatenate([drf, drf[:, -1:]], axis=1)
        node_tok = np.concatenate([np.zeros((B, 1), np.int32), tok], 1)
        parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
        ot = oracle.verify_tree(tgt, tdrf, node_tok, parent, gamma, T, 5, 2, "f64")
        assert np.array_equal(ot["len"], oc["n"]) and np.array_equal(ot["t"], oc["t"])
        assert np.array_equal(ot["mdec"], oc["mdec"]) and np.array_equal(ot["mcdf"], oc["mcdf"])
        for b in range(B):
            L = oc["n"][b]
            assert list(ot["path"][b][:L]) == list(range(1, L + 1))
            seen = min(L + 1, gamma)
            assert np.array_equal(ot["p"][b, 1:1 + seen], oc["p"][b, :seen])


def test_tree_residual_recursion_matches_repeated_residuals():
    """(p - c_i q)^+ / D_i equals norm(max(0, p_cur - q)) applied i times."""
    rng = np.random.default_rng(11)
    for _ in range(50):
        V = 30
        p = rng.dirichlet(np.full(V, 0.4))
        q = rng.dirichlet(np.full(V, 0.4))
        cur = p.copy()
        c, D = 0.0, 1.0
        for _i in range(6):
            nxt = np.maximum(0, cur - q)
            if nxt.sum() <= 0:
                break
            cur = nxt / nxt.sum()
            c = c + D
            D = np.maximum(0, p - c * q).sum()
            assert np.max(np.abs(np.maximum(0, p - c * q) / D - cur)) < 1e-12


# --------------------------------------------------------------------------
# Fan-out (SSD review §3 and Theorem 12)
# --------------------------------------------------------------------------
def test_geometric_fanout_closed_form():
    with open(os.path.join(GOLDEN, "geometric_fanout.txt")) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            lhs, rhs = ln.split(":")
            F0, a_p, r, K, cap = lhs.split()
            want = [int(x) for x in rhs.split()]
            got = oracle.geometric_fanout(int(F0), float(a_p), float(r), int(K), bool(int(cap)))
            assert list(got) == want


def test_fanout_is_stable_sort():
    rng = np.random.default_rng(12)
    R, V, Fmax = 40, 300, 8
    bits = rng.integers(0x3F00, 0x3F08, size=(R, V)).astype(np.uint16)  # bf16 with many ties
    bits[::3] = rng.integers(0, 0xFFFF, size=bits[::3].shape).astype(np.uint16) & 0x7F7F  # finite, mixed sign
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    F = rng.integers(0, Fmax + 1, R).astype(np.int32)
    ids, got_vals = oracle.fanout_topk(bits, F, Fmax, "bf16")
    for r in range(R):
        order = np.argsort(-vals[r].astype(np.float64), kind="stable")
        assert list(ids[r][:F[r]]) == list(order[:F[r]])
        assert (ids[r][F[r]:] == -1).all()
        assert np.array_equal(got_vals[r][:F[r]], vals[r][order[:F[r]]])


# ---------------------------------------------------------------- point-mass mode
# SpecDiff-2 page, Core method ("greedy acceptance": accept the chosen token
# with a Bernoulli of the verifier probability, resample the residual on a
# rejection, no drafter probability), read as the draft-then-verify page's
# §2.1 step with a point-mass draft q = delta_x.

def test_pm_chain_equals_chain_with_point_mass_drafts():
    """The point-mass chain is the standard chain fed one-hot draft rows at
    the drafted tokens: same decisions, same residual, same draws."""
    rng = np.random.default_rng(31)
    for V, gamma, T in ((7, 3, 1.0), (40, 6, 0.7), (300, 5, 1.4)):
        B = 40
        tgt = rng.normal(scale=2.0, size=(B, gamma + 1, V))
        tgt[rng.random(tgt.shape) < 0.2] = -np.inf
        tgt[..., 0] = 0.0  # every row keeps a finite logit
        tok = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
        drf = np.full((B, gamma, V), -np.inf)
        for b in range(B):
            for j in range(gamma):
                drf[b, j, tok[b, j]] = 0.0
        for seed, rnd in ((0, 0), (7, 3)):
            a = oracle.verify_chain_pm(tgt, tok, T, seed, rnd, "f64")
            c = oracle.verify_chain(tgt, drf, tok, T, seed, rnd, "f64")
            assert np.array_equal(a["n"], c["n"]) and np.array_equal(a["t"], c["t"])
            assert np.array_equal(a["p"], c["p"])
            assert (a["rows"] == 1).all()


@pytest.mark.parametrize("gamma,m,T,pz,seed,chooser", [
    (2, 3, 1.0, 0.0, 41, "p_argmin"),
    (3, 3, 0.7, 0.3, 42, "q_argmax"),
    (2, 4, 1.3, 0.2, 43, "hash"),
])
def test_pm_chain_round_is_lossless_for_any_drafter(gamma, m, T, pz, seed, chooser):
    """Exact enumeration: with deterministic drafts (even the least likely
    token under the target), the emitted sequence's law is the target chain
    rule."""
    tab = E.Tables(V=4, seed=seed, p_zero=pz)
    choose = {
        "p_argmin": lambda ctx: int(np.argmin(tab.p(ctx))),
        "q_argmax": lambda ctx: int(np.argmax(tab.q(ctx))),
        "hash": lambda ctx: (sum(ctx) * 7 + len(ctx) * 3 + 1) % tab.V,
    }[chooser]
    d = E.chain_pm_sequence_distribution(tab, gamma, m, choose, T)
    assert E.max_marginal_error(tab, d, m) < 1e-12


@pytest.mark.parametrize("parent,m,seed,T", [
    ([-1, 0, 0, 0], 2, 51, 1.0),
    ([-1, 0, 0, 1, 1], 2, 52, 0.8),
    ([-1, 0, 1, 0, 2], 3, 53, 1.2),
])
def test_pm_tree_with_top_f_siblings_is_lossless(parent, m, seed, T):
    """Exact enumeration with deterministic top-F siblings (the k-th child is
    the draft's k-th most likely token): the point-mass rule keeps the target
    law, while the standard sibling rule with q held fixed does not."""
    tab = E.Tables(V=4, seed=seed, p_zero=0.2)
    d = E.tree_pm_sequence_distribution(tab, parent, m, T=T, pm=True)
    assert E.max_marginal_error(tab, d, m) < 1e-12
    if len(parent) > 2:
        d_std = E.tree_pm_sequence_distribution(tab, parent, m, T=T, pm=False)
        assert E.max_marginal_error(tab, d_std, m) > 1e-3


def test_pm_chain_shaped_tree_is_pm_chain():
    """A tree that is a single path gives exactly the point-mass chain."""
    rng = np.random.default_rng(61)
    B, gamma, V, T = 12, 5, 50, 0.9
    tgt = rng.normal(scale=2.0, size=(B, gamma + 1, V))
    tok = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    node_tok = np.concatenate([np.zeros((B, 1), np.int32), tok], axis=1)
    parent = np.tile(np.arange(-1, gamma, dtype=np.int32), (B, 1))
    # the uniforms the chain uses for x_j (counter idx j) are the tree's for node j
    for seed, rnd in ((0, 0), (3, 2)):
        c = oracle.verify_chain_pm(tgt, tok, T, seed, rnd, "f64")
        t = oracle.verify_tree_pm(tgt, node_tok, parent, gamma, T, seed, rnd, "f64")
        assert np.array_equal(c["n"], t["len"]) and np.array_equal(c["t"], t["t"])
        for b in range(B):
            assert np.array_equal(c["p"][b, :c["n"][b] + (c["n"][b] < gamma)],
                                  t["p"][b, 1:1 + c["n"][b] + (c["n"][b] < gamma)])


def test_pm_repeated_sibling_token_is_rejected_and_removes_nothing():
    """A sibling whose token was already rejected has residual probability 0:
    it is rejected for sure, and the final draw never returns that token."""
    V, T = 6, 1.0
    tgt = np.log(np.array([[0.30, 0.25, 0.20, 0.15, 0.05, 0.05]]))[None].repeat(3, axis=1)
    node_tok = np.array([[0, 2, 2]], np.int32)
    parent = np.array([[-1, 0, 0]], np.int32)
    # reject the first sibling (r >= p = 0.2), then the repeat has ratio 0
    o = oracle.verify_tree_pm(tgt, node_tok, parent, 2, T, 0, 0, "f64", r=np.array([[0.0, 0.5, 0.0]]),
                              u=np.array([0.999]), want_w=True)
    assert o["len"][0] == 0 and o["a"][0, 2] == 0.0 and o["t"][0] != 2
    w = o["w"][0]
    assert w[2] == 0.0 and np.isclose(w.sum(), 1.0)
    assert np.allclose(w, np.array([0.30, 0.25, 0.0, 0.15, 0.05, 0.05]) / 0.8)


# ---------------------------------------------------------------- speculation-cache hit test
# SSD / Saguaro review §3 (cache strategy): the cache holds the top-F_k draft
# tokens of every lookahead position k; an outcome (n, t) is a hit iff t is
# among the tokens cached for position n.

def _tie_heavy_rows(rng, B, K1, V):
    bits = rng.integers(0x3F00, 0x3F06, size=(B, K1, V)).astype(np.uint16)  # bf16 with many ties
    bits[:, ::2] = rng.integers(0, 0xFFFF, size=bits[:, ::2].shape).astype(np.uint16) & 0x7F7F
    bits[rng.random(bits.shape) < 0.05] = 0x8000  # -0.0, equal to +0.0 as a number
    bits[rng.random(bits.shape) < 0.05] = 0x0000
    bits[rng.random(bits.shape) < 0.05] = 0xFF80  # -inf (masked token)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def test_cache_rank_is_position_in_numpy_stable_order():
    rng = np.random.default_rng(61)
    B, K, V = 50, 4, 257
    bits, vals = _tie_heavy_rows(rng, B, K + 1, V)
    n = rng.integers(0, K + 1, B).astype(np.int32)
    t = rng.integers(0, V, B).astype(np.int32)
    out = oracle.cache_hit_test(bits, n, t, None, "bf16")
    for b in range(B):
        order = np.argsort(-vals[b, n[b]].astype(np.float64), kind="stable")
        assert out["rank"][b] == int(np.nonzero(order == t[b])[0][0])
    assert out["hit"] is None


def test_cache_rank_brute_force_count():
    """rank = #{v : z_v > z_t, or z_v == z_t and v < t}, counted by hand (f32 and f64 rows)."""
    rng = np.random.default_rng(62)
    for dtype, npdt in (("f32", np.float32), ("f64", np.float64)):
        B, K, V = 12, 2, 23
        z = rng.integers(-3, 3, size=(B, K + 1, V)).astype(npdt)
        z[rng.random(z.shape) < 0.1] = -np.inf
        n = rng.integers(0, K + 1, B).astype(np.int32)
        t = rng.integers(0, V, B).astype(np.int32)
        out = oracle.cache_hit_test(z, n, t, None, dtype)
        for b in range(B):
            row, tb = z[b, n[b]], int(t[b])
            want = sum(1 for v in range(V) if row[v] > row[tb] or (row[v] == row[tb] and v < tb))
            assert out["rank"][b] == want


def test_cache_hit_is_membership_in_the_fanout_cache():
    """hit(n, t) == t among the top-F_n ids the fan-out caches for position n (F = 0, ties, F >= V)."""
    rng = np.random.default_rng(63)
    S, K, V = 6, 3, 40
    bits, _ = _tie_heavy_rows(rng, S, K + 1, V)
    F = np.array([0, 3, 17, 45], np.int32)
    ids, _ = oracle.fanout_topk(bits.reshape(S * (K + 1), V), np.tile(F, S), 64, "bf16")
    ids = ids.reshape(S, K + 1, 64)
    # every outcome (n, t) of every sequence: the batch repeats each sequence's rows
    seq, n, t = np.meshgrid(np.arange(S), np.arange(K + 1), np.arange(V), indexing="ij")
    seq, n, t = seq.ravel(), n.ravel().astype(np.int32), t.ravel().astype(np.int32)
    out = oracle.cache_hit_test(np.ascontiguousarray(bits[seq]), n, t, F, "bf16")
    for i in range(len(seq)):
        cached = set(ids[seq[i], n[i]][:F[n[i]]].tolist()) - {-1}
        assert bool(out["hit"][i]) == (int(t[i]) in cached)
    assert out["hit"].sum() == S * (0 + 3 + 17 + 40)


def test_cache_rank_uniform_over_random_tokens():
    """A row of distinct values ranks every token exactly once: over all t, the ranks are 0..V-1."""
    rng = np.random.default_rng(64)
    V = 97
    z = rng.permutation(V).astype(np.float32)[None, None, :]
    ranks = [oracle.cache_hit_test(z, np.array([0], np.int32), np.array([v], np.int32), None, "f32")["rank"][0]
             for v in range(V)]
    assert sorted(ranks) == list(range(V))
    assert all(ranks[v] == V - 1 - int(z[0, 0, v]) for v in range(V))


def test_cache_rejects_outcomes_outside_the_window():
    z = np.zeros((2, 3, 5), np.float32)
    for n, t in (([0, 3], [0, 0]), ([0, -1], [0, 0]), ([0, 0], [0, 5]), ([0, 0], [-1, 0])):
        with pytest.raises(oracle.OracleError):
            oracle.cache_hit_test(z, np.array(n, np.int32), np.array(t, np.int32), None, "f32")


# ---------------------------------------------------------------- PRESTO scoring
# PRESTO page §4.1 (token score s = log q + lambda log rho, rho = min(1, p/q);
# path score = sum of token scores, eq. 10), §4.2 (priority expansion), §4.4
# (the proxy p* ~ q rho^lambda minimises KL(p || q) - lambda E_p[log rho]).

def _presto_tree(rng, B, N, V, masked=0.0):
    tgt = rng.normal(scale=2.0, size=(B, N, V))
    drf = tgt + rng.normal(scale=1.0, size=(B, N, V))
    if masked:
        tgt[rng.random(tgt.shape) < masked] = -np.inf
        drf[rng.random(drf.shape) < masked] = -np.inf
        tgt[..., 0] = 0.0
        drf[..., 0] = 0.0
    parent = np.full((B, N), -1, np.int32)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            parent[b, i] = rng.integers(0, i)
            tok[b, i] = rng.integers(0, V)
    return tgt, drf, tok, parent


def _log_softmax_rows(z, T):
    with np.errstate(invalid="ignore"):
        return scipy.special.log_softmax(z / T, axis=-1)


def test_presto_scores_match_log_softmax_and_ancestor_sums():
    rng = np.random.default_rng(71)
    B, N, V, T = 5, 14, 30, 0.8
    tgt, drf, tok, parent = _presto_tree(rng, B, N, V, masked=0.15)
    lam = np.array([0.5, 1.0, 0.0, 2.0], np.float32)
    out = oracle.presto_score(tgt, drf, tok, parent, T, lam, 2, 3, "f64")
    lp, lq = _log_softmax_rows(tgt, T), _log_softmax_rows(drf, T)
    for b in range(B):
        depth = [0] * N
        for i in range(1, N):
            depth[i] = depth[parent[b, i]] + 1
        for i in range(1, N):
            u, x = parent[b, i], tok[b, i]
            la = float(lam[min(depth[i], len(lam)) - 1])
            a, c = lp[b, u, x], lq[b, u, x]
            if c == -np.inf or (la > 0 and a == -np.inf):
                want = -np.inf
            else:
                want = c + (la * min(0.0, a - c) if la > 0 else 0.0)
            got = out["s"][b, i]
            assert (got == want) if want == -np.inf else abs(got - want) < 1e-12
            # ancestor sum, walked by hand
            S, j = 0.0, i
            while j > 0:
                S += out["s"][b, j]
                j = parent[b, j]
            assert (out["S"][b, i] == S) if S == -np.inf else abs(out["S"][b, i] - S) < 1e-12
        assert out["s"][b, 0] == 0.0 and out["S"][b, 0] == 0.0


@pytest.mark.parametrize("lam_val", [0.3, 1.0, 2.5])
def test_presto_proxy_minimises_the_kl_objective(lam_val):
    """With the root as the only node, the expansion proposes every token with
    its score s(t); softmax(s) must be the minimiser of KL(p || q) - lambda
    E_p[log rho], whose minimum is -log sum_t q(t) rho(t)^lambda."""
    rng = np.random.default_rng(72)
    V, T = 40, 1.1
    tgt = rng.normal(scale=2.0, size=(1, 1, V))
    drf = tgt + rng.normal(scale=1.5, size=(1, 1, V))
    out = oracle.presto_score(tgt, drf, np.zeros((1, 1), np.int32), np.full((1, 1), -1, np.int32), T,
                              np.array([lam_val], np.float32), V, V, "f64")
    assert sorted(out["tok"][0].tolist()) == list(range(V))
    s = np.empty(V)
    s[out["tok"][0]] = out["score"][0]
    p = scipy.special.softmax(tgt[0, 0] / T)
    q = scipy.special.softmax(drf[0, 0] / T)
    log_rho = np.minimum(0.0, np.log(p) - np.log(q))
    pstar = scipy.special.softmax(s)

    def objective(r):
        return float(np.sum(r * (np.log(r) - np.log(q))) - lam_val * np.sum(r * log_rho))

    closed = -math.log(float(np.sum(q * np.exp(lam_val * log_rho))))
    assert abs(objective(pstar) - closed) < 1e-10
    for _ in range(20):
        r = pstar * np.exp(rng.normal(scale=0.05, size=V))
        r /= r.sum()
        assert objective(r) > objective(pstar)


def test_presto_lambda_zero_expands_the_draft_top_k():
    """lambda = 0: the proxy is q itself, so a leaf proposes the fan-out's top-k of its draft row."""
    rng = np.random.default_rng(73)
    V, k = 200, 9
    bits = rng.integers(0x3F00, 0x3F20, size=(1, 1, V)).astype(np.uint16)  # bf16 with ties
    tgt_bits = rng.integers(0x3F00, 0x4000, size=(1, 1, V)).astype(np.uint16)
    out = oracle.presto_score(tgt_bits, bits, np.zeros((1, 1), np.int32), np.full((1, 1), -1, np.int32), 0.7,
                              np.array([0.0], np.float32), k, k, "bf16")
    ids, _ = oracle.fanout_topk(bits.reshape(1, V), np.array([k], np.int32), k, "bf16")
    assert out["tok"][0].tolist() == ids[0].tolist()
    assert (out["node"][0] == 0).all()


def test_presto_expansion_brute_force():
    rng = np.random.default_rng(74)
    B, N, V, T, k, b_top = 4, 11, 17, 0.9, 3, 7
    tgt, drf, tok, parent = _presto_tree(rng, B, N, V, masked=0.2)
    lam = np.array([0.7, 1.3, 0.4], np.float32)
    out = oracle.presto_score(tgt, drf, tok, parent, T, lam, k, b_top, "f64")
    lp, lq = _log_softmax_rows(tgt, T), _log_softmax_rows(drf, T)
    for b in range(B):
        depth = [0] * N
        for i in range(1, N):
            depth[i] = depth[parent[b, i]] + 1
        leaves = [u for u in range(N) if not (parent[b] == u).any()]
        cands = []
        for u in leaves:
            la = float(lam[min(depth[u] + 1, len(lam)) - 1])
            mine = []
            for t in range(V):
                a, c = lp[b, u, t], lq[b, u, t]
                if c == -np.inf or a == -np.inf:
                    continue
                mine.append((c + la * min(0.0, a - c), t))
            mine.sort(key=lambda e: (-e[0], e[1]))
            cands += [(out["S"][b, u] + sc, u, t) for sc, t in mine[:k]]
        cands.sort(key=lambda e: (-e[0], e[1], e[2]))
        for j in range(b_top):
            if j < len(cands):
                assert (out["node"][b, j], out["tok"][b, j]) == (cands[j][1], cands[j][2])
                want = cands[j][0]
                assert out["score"][b, j] == want if want == -np.inf else abs(out["score"][b, j] - want) < 1e-12
            else:
                assert out["node"][b, j] == -1 and out["score"][b, j] == -np.inf


def test_presto_rejects_bad_trees():
    z = np.zeros((1, 3, 5))
    with pytest.raises(oracle.OracleError):
        oracle.presto_score(z, z, np.zeros((1, 3), np.int32), np.array([[-1, 0, 2]], np.int32), 1.0,
                            np.array([1.0], np.float32), 2, 2, "f64")
    with pytest.raises(oracle.OracleError):
        oracle.presto_score(z, z, np.array([[0, 0, 5]], np.int32), np.array([[-1, 0, 0]], np.int32), 1.0,
                            np.array([1.0], np.float32), 2, 2, "f64")


# ---------------------------------------------------------------- SpecBranch fork
# SpecBranch notes, key designs 2-3: branch point by the hybrid predictor's class
# (0: the round's first token; 1: the first drafted token with q(x) < eps; 2:
# the next round's first token), k = max(1, floor(k_max (1 - q(x_b)))) branches
# forked with the top-k of the draft distribution at the branch point.

def _branch_brute(z, tok, cls, T, eps, k_max):
    B, g1, V = z.shape
    gamma = g1 - 1
    q = scipy.special.softmax(z / T, axis=-1)
    out = []
    for b in range(B):
        s = 1 if cls is None else int(cls[b])
        pos = 1 if s == 0 else gamma + 1
        if s == 1:
            for j in range(1, gamma + 1):
                if q[b, j - 1, tok[b, j - 1]] < eps:
                    pos = j
                    break
        row = q[b, pos - 1]
        qb = row[tok[b, pos - 1]] if pos <= gamma else row[int(np.argmax(row))]
        k = max(1, int(math.floor(k_max * (1.0 - qb))))
        order = np.argsort(-z[b, pos - 1], kind="stable")
        out.append((pos, qb, k, [int(order[i]) if i < k and i < V else -1 for i in range(k_max)]))
    return out


def test_branch_fork_brute_force():
    rng = np.random.default_rng(91)
    B, gamma, V, T, k_max = 60, 5, 23, 0.9, 6
    z = rng.integers(-3, 4, size=(B, gamma + 1, V)).astype(np.float64) * 0.7  # ties
    z[rng.random(z.shape) < 0.1] = -np.inf
    z[..., 0] = 0.0
    q = scipy.special.softmax(z / T, axis=-1)
    tok = np.array([[rng.choice(V, p=q[b, j]) for j in range(gamma)] for b in range(B)], np.int32)
    cls = rng.integers(0, 3, B).astype(np.int32)
    for eps in (0.05, 0.2, 0.6):
        got = oracle.branch_fork(z, tok, cls, T, eps, k_max, "f64")
        for b, (pos, qb, k, ids) in enumerate(_branch_brute(z, tok, cls, T, eps, k_max)):
            assert got["pos"][b] == pos and got["k"][b] == k and abs(got["qb"][b] - qb) < 1e-12
            assert got["ids"][b].tolist() == ids
        assert set(got["pos"].tolist()) > {1}  # several branch points occur


def test_branch_fork_special_cases():
    rng = np.random.default_rng(92)
    B, gamma, V, T = 30, 4, 40, 1.0
    z = rng.normal(scale=2.0, size=(B, gamma + 1, V))
    tok = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    never = oracle.branch_fork(z, tok, None, T, 0.0, 8, "f64")  # q(x) < 0 never holds
    assert (never["pos"] == gamma + 1).all()
    always = oracle.branch_fork(z, tok, None, T, 1.5, 8, "f64")  # q(x) <= 1 < eps
    assert (always["pos"] == 1).all()
    first = oracle.branch_fork(z, tok, np.zeros(B, np.int32), T, 0.5, 8, "f64")
    last = oracle.branch_fork(z, tok, np.full(B, 2, np.int32), T, 0.5, 8, "f64")
    assert (first["pos"] == 1).all() and (last["pos"] == gamma + 1).all()
    one = oracle.branch_fork(z, tok, None, T, 0.3, 1, "f64")
    assert (one["k"] == 1).all()
    # more branches where the branch point is less confident, never outside [1, k_max]
    r = oracle.branch_fork(z, tok, None, T, 0.3, 16, "f64")
    order = np.argsort(r["qb"])
    assert (np.diff(r["k"][order]) <= 0).all() and r["k"].min() >= 1 and r["k"].max() <= 16
    # the branches are the fan-out's top-k of the branch row
    z32 = z.astype(np.float32)
    r32 = oracle.branch_fork(z32, tok, None, T, 0.3, 16, "f32")
    rows = np.stack([z32[b, r32["pos"][b] - 1] for b in range(B)])
    ids, _ = oracle.fanout_topk(rows, r32["k"], 16, "f32")
    assert np.array_equal(ids, r32["ids"])
