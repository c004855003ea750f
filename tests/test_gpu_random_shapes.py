"""A seeded sweep of shapes for every entry point through the C ABI
against the CPU oracle (margin rule in tests/parity.py): batch size, draft
length, vocabulary (ragged), logit dtype, temperature, candidates and tree
shape drawn at random, so that the launch plans vary together (row parts per
row, draw blocks per sequence, register-held or streamed slices, parts
merged in registers, from LDS or from memory).  Sizes are kept small enough
for the oracle to finish each case in well under a second."""
import numpy as np
import pytest
import torch

from lossless_draft_verification_04_amd import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu

CASES = 24
ELEMS = 3_000_000  # logits per case (rows x V), bounding the oracle's work


def _shape(rng, rows_per_seq):
    V = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 5000)), int(rng.integers(5000, 160000))]))
    B = int(max(1, min(int(rng.integers(1, 48)), ELEMS // max(1, rows_per_seq * V))))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    T = float(rng.choice([0.3, 0.7, 1.0, 1.6]))
    return B, V, dtype, T


@pytest.mark.parametrize("case", range(CASES))
def test_random_chain_and_point_mass_chain(case):
    rng = np.random.default_rng(1000 + case)
    gamma = int(rng.integers(1, 65))
    B, V, dtype, T = _shape(rng, 2 * gamma + 1)
    gen = W.chain_zipf if rng.random() < 0.5 else W.chain_normal
    kw = dict(B=B, gamma=gamma, V=V, T=T, dtype=dtype, seed=2000 + case)
    wl = gen(**kw)
    seed, rnd = int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 20))
    PT.chain(wl, seed, rnd)
    PT.chain_pm(wl, seed, rnd)
    PT.device_error_clear()


@pytest.mark.parametrize("case", range(CASES))
def test_random_multi(case):
    rng = np.random.default_rng(3000 + case)
    K = int(rng.integers(1, 13))
    gamma = int(rng.integers(1, 33))
    B, V, dtype, T = _shape(rng, (K + 1) * (gamma + 1))
    wl = W.multi_zipf(B=B, K=K, gamma=gamma, V=V, T=T, dtype=dtype, seed=4000 + case)
    PT.multi(wl, int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 20)))
    PT.device_error_clear()


@pytest.mark.parametrize("case", range(CASES))
def test_random_tree_and_point_mass_tree(case):
    rng = np.random.default_rng(5000 + case)
    N = int(rng.integers(1, 200))
    depth = int(rng.integers(1, 11))
    B, V, dtype, T = _shape(rng, 2 * N)
    F0 = min(int(rng.integers(1, 10)), V)  # children are distinct top-ranked tokens of their parent's row
    # at most the largest tree the fan-out schedule and depth allow (every node must be placed)
    F = W.fanout_schedule(F0, 0.7, 1.0, depth)
    level, most = 1, 1
    for d in range(depth):
        level *= F[d]
        most += level
    N = min(N, most)
    wl = W.tree_zipf(B=B, N=N, max_depth=depth, V=V, T=T, dtype=dtype, seed=6000 + case, F0=F0)
    assert int((wl.tensors["parent"][:, 1:] < 0).sum()) == 0
    seed, rnd = int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 20))
    PT.tree(wl, seed, rnd)
    PT.tree_pm(wl, seed, rnd)
    PT.device_error_clear()


def _rows(rng, shape, V, dtype, ties):
    """Padded CPU rows of Gaussian logits (or small integers, for heavy ties,
    with a few -inf and -0 entries)."""
    g = W._gen(int(rng.integers(0, 1 << 31)))
    Vs = W.padded_stride(V, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    store = torch.zeros(*shape, Vs, dtype=tdt)
    x = store[..., :V]
    if ties:
        x.copy_(torch.randint(-3, 4, (*shape, V), generator=g).to(tdt))
        x[torch.rand(*shape, V, generator=g) < 0.03] = float("-inf")
        x[torch.rand(*shape, V, generator=g) < 0.03] = -0.0
    else:
        x.copy_((torch.randn(*shape, V, generator=g) * 2.0).to(tdt))
    return x


@pytest.mark.parametrize("case", range(CASES))
def test_random_greedy(case):
    rng = np.random.default_rng(7000 + case)
    gamma = int(rng.integers(1, 65))
    B, V, dtype, _ = _shape(rng, gamma + 1)
    PT.greedy(W.greedy_zipf(B=B, gamma=gamma, V=max(V, 2), dtype=dtype, seed=8000 + case))


@pytest.mark.parametrize("case", range(CASES))
def test_random_fanout(case):
    rng = np.random.default_rng(9000 + case)
    R = int(rng.integers(1, 600))
    _, V, dtype, _ = _shape(rng, 1)
    R = max(1, min(R, ELEMS // V))
    F_max = int(rng.integers(1, 65))
    F = torch.as_tensor(rng.integers(0, F_max + 1, R), dtype=torch.int32)
    PT.fanout(_rows(rng, (R,), V, dtype, ties=rng.random() < 0.5), F, F_max)
    PT.device_error_clear()


@pytest.mark.parametrize("case", range(CASES))
def test_random_cache(case):
    rng = np.random.default_rng(10000 + case)
    K = int(rng.integers(0, 65))
    B, V, dtype, _ = _shape(rng, K + 1)
    rows = _rows(rng, (B, K + 1), V, dtype, ties=rng.random() < 0.5)
    n = torch.as_tensor(rng.integers(0, K + 1, B), dtype=torch.int32)
    t = torch.as_tensor(rng.integers(0, V, B), dtype=torch.int32)
    F = torch.as_tensor(rng.integers(0, 12, K + 1), dtype=torch.int32) if rng.random() < 0.7 else None
    PT.cache(rows, n, t, F)
    PT.device_error_clear()


@pytest.mark.parametrize("case", range(CASES))
def test_random_presto(case):
    rng = np.random.default_rng(11000 + case)
    N = int(rng.integers(1, 120))
    depth = int(rng.integers(1, 9))
    B, V, dtype, T = _shape(rng, 2 * N)
    V = max(V, 16)
    F0 = int(rng.integers(1, 9))
    F = W.fanout_schedule(F0, 0.7, 1.0, depth)
    level, most = 1, 1
    for d in range(depth):
        level *= F[d]
        most += level
    N = min(N, most)
    wl = W.tree_zipf(B=B, N=N, max_depth=depth, V=V, T=T, dtype=dtype, seed=12000 + case, F0=F0)
    lam = [float(x) for x in rng.choice([0.0, 0.25, 0.5, 1.0, 2.0], int(rng.integers(1, 6)))]
    PT.presto(wl, lam, int(rng.integers(1, 65)), int(rng.integers(1, 65)))
    PT.device_error_clear()


@pytest.mark.parametrize("case", range(CASES))
def test_random_branch(case):
    rng = np.random.default_rng(13000 + case)
    gamma = int(rng.integers(1, 65))
    B, V, dtype, T = _shape(rng, gamma + 1)
    wl = W.chain_zipf(B=B, gamma=gamma, V=V, T=T, dtype=dtype, seed=14000 + case, lookahead_row=True)
    cls = torch.as_tensor(rng.integers(0, 3, B), dtype=torch.int32) if rng.random() < 0.7 else None
    PT.branch(W.lookahead_rows(wl), wl.tensors["tok"], cls, T, float(rng.choice([0.05, 0.3, 0.7])),
              int(rng.integers(1, 65)))
    PT.device_error_clear()
