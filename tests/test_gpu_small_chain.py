"""GPU parity of the small-call chain path (every row held by the draw blocks) against the oracle.

Chain calls with K = 1, at most 9 held rows (target rows 1..gamma+1 and draft rows 1..gamma, so
gamma <= 4; point mass: gamma <= 8), rows of at most 64 x 512 vectors and B * V small run one launch
in which each of a sequence's blocks holds its slice of every row (draft-then-verify page §1 steps
3-5 and §2.1).  These shapes are chosen inside those bounds: ragged vocabularies, both dtypes, every
gamma, the bonus draw (all drafts accepted), zero probabilities at the drafted token, rows with
masked logits, the bounded wait, and graph replays.
"""
import numpy as np
import pytest
import torch

from lossless_draft_verification_04_amd import specverify as svx
from lossless_draft_verification_04_amd import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu
NEG = float("-inf")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
# one 256-vector tile per block while a sequence's blocks number at most 64, else two: f32 V=65536 is 64
# one-tile blocks, V=65537 33 two-tile blocks; bf16 V=262144 is 64 two-tile blocks
@pytest.mark.parametrize("gamma,V,B", [(1, 1, 1), (1, 7, 3), (2, 100, 4), (3, 5000, 2), (4, 32000, 1),
                                       (4, 65536, 1), (4, 65537, 1), (2, 262144, 1), (4, 9999, 8)])
def test_small_chain_matches_oracle(dtype, gamma, V, B):
    wl = W.chain_normal(B=B, gamma=gamma, V=V, T=1.0, dtype=dtype, seed=400 + gamma * 7 + V % 97 + B)
    for seed, rnd in [(0, 0), (3, 1), (11, 5)]:
        PT.chain(wl, seed, rnd)
    PT.device_error_clear()


@pytest.mark.parametrize("gamma", [1, 4, 8])
def test_small_chain_pm_matches_oracle(gamma):
    wl = W.chain_normal(B=3, gamma=gamma, V=20011, T=0.8, dtype="bf16", seed=450 + gamma)
    for seed, rnd in [(0, 0), (5, 2)]:
        PT.chain_pm(wl, seed, rnd)
    PT.device_error_clear()


def test_small_chain_config1_rounds():
    wl = W.chain_normal(**W.CHAIN_SMALL)
    for rnd in range(12):
        PT.chain(wl, 0, rnd)
        PT.chain_pm(wl, 0, rnd)
    PT.device_error_clear()


def test_small_chain_bonus_and_zero_probabilities():
    # sequences 0-1: every draft has q(x) = 0 < p(x), so all are accepted and the bonus row is drawn;
    # sequence 2: position 2 has p(x) = 0 (rejected there); sequence 3: masked rows around the tokens
    gamma, B, V = 4, 4, 30011
    wl = W.chain_zipf(B=B, gamma=gamma, V=V, T=0.9, dtype="bf16", seed=461)
    tgt, drf, tok = wl.tensors["tgt"], wl.tensors["drf"], wl.tensors["tok"]
    for b in (0, 1):
        for j in range(gamma):
            drf[b, j, tok[b, j]] = NEG
    drf[2, 0, tok[2, 0]] = NEG
    tgt[2, 1, tok[2, 1]] = NEG
    keep = torch.zeros(V, dtype=torch.bool)
    keep[torch.randperm(V, generator=torch.Generator().manual_seed(5))[:2000]] = True
    for j in range(gamma + 1):
        k = keep.clone()
        if j < gamma:
            k[tok[3, j]] = True
        tgt[3, j][~k] = NEG
        if j < gamma:
            drf[3, j][~k] = NEG
    for seed, rnd in [(0, 0), (2, 3)]:
        out, ref = PT.chain(wl, seed, rnd)
        n = out["n"].cpu().numpy()
        assert n[0] == gamma and n[1] == gamma and n[2] == 1
        t = out["tok"].cpu().numpy()
        for b in range(B):
            assert torch.isfinite(tgt[b, n[b], t[b]].float())
    PT.device_error_clear()


def _knobs(spin, withhold):
    ws = svx.Workspace.get(PT.DEV, 16 << 20)
    torch.cuda.synchronize()
    ws[4:12].view(torch.int32).copy_(torch.tensor([spin, withhold], dtype=torch.int32))
    torch.cuda.synchronize()


def test_small_chain_wait_runs_out_and_the_next_call_is_exact():
    wl = W.chain_normal(B=2, gamma=3, V=20000, T=1.0, dtype="f32", seed=462)
    g = wl.to(PT.DEV)
    assert svx.sv_get_device_error(PT.DEV) == 0
    try:
        _knobs(2000, 1)
        PT.say("  small chain with a withheld publish (sequence 0, last block), wait bound 2000 polls")
        svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0, seed=1)
        torch.cuda.synchronize()
        assert svx.sv_get_device_error(PT.DEV) & svx.DERR_TIMEOUT
    finally:
        _knobs(0, 0)
        svx.sv_get_device_error(PT.DEV)
    PT.chain(wl, 1, 0)
    PT.device_error_clear()


def test_small_chain_graph_replays():
    wl = W.chain_normal(B=2, gamma=4, V=32000, T=1.0, dtype="f32", seed=463)
    g = wl.to(PT.DEV)
    eager = svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0, seed=4, round_=2)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in eager.items() if v is not None}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0, seed=4, round_=2)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            out = svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0, seed=4, round_=2)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(4):
        for k in out:
            if out[k] is not None:
                out[k].fill_(-7 if out[k].dtype == torch.int32 else float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        # an eager call of another entry point on the same workspace between replays
        svx.sv_verify_chain_pm(g["tgt"], g["tok"], 1.0, seed=9)
        torch.cuda.synchronize()
        for k, v in want.items():
            assert torch.equal(out[k], v), k
    PT.device_error_clear()
