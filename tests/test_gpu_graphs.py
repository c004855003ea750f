"""Every entry point captured in a HIP graph and replayed several times, with
eager calls of other entry points and synchronisations between the replays:
each replay must reproduce the eager call's outputs bit for bit (the
workspace's counters, slots and flags must be left ready by every call, and no
captured step may depend on state a previous call left behind)."""
import pytest
import torch

from lossless_draft_verification_04_amd import specverify as svx
from lossless_draft_verification_04_amd import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    if a.dtype == torch.float32:  # bit patterns: NaN and -0 compare too
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _outputs(out):
    if isinstance(out, dict):
        return out
    return {str(i): t for i, t in enumerate(out)}


def _replay_matches_eager(call, between):
    eager = _outputs(call())
    torch.cuda.synchronize()
    eager = {k: (None if v is None else v.clone()) for k, v in eager.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = _outputs(call())
    for rep in range(REPLAYS):
        for v in cap.values():
            if v is not None:
                v.fill_(-7)  # a replay must rewrite every output
        graph.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert _same(cap[k], eager[k]), (rep, k)
        between()  # eager work on the same workspace between the replays
        torch.cuda.synchronize()
    assert svx.sv_get_device_error(PT.DEV) == 0


@pytest.fixture(scope="module")
def inputs():
    chain = W.chain_zipf(B=6, gamma=8, V=30011, T=0.8, seed=91, lookahead_row=True)
    tree = W.tree_zipf(B=3, N=24, max_depth=6, V=20011, T=1.0, seed=92)
    multi = W.multi_zipf(B=3, K=3, gamma=6, V=12007, T=1.0, seed=93)
    greedy = W.greedy_zipf(B=5, gamma=6, V=16001, seed=94)
    return dict(chain=chain, c=chain.to(PT.DEV), tree=tree, t=tree.to(PT.DEV), m=multi.to(PT.DEV),
                g=greedy.to(PT.DEV), rows=W.lookahead_rows(chain))


def _other(inp):
    g = inp["g"]
    return lambda: svx.sv_verify_greedy(g["tgt"], g["tok"])


def test_graph_chain_pm(inputs):
    c = inputs["c"]
    T = PT.f32(0.8)
    _replay_matches_eager(lambda: svx.sv_verify_chain_pm(c["tgt"], c["tok"], T, seed=3, round_=2), _other(inputs))


def test_graph_multi(inputs):
    m = inputs["m"]
    _replay_matches_eager(lambda: svx.sv_verify_multi(m["tgt"], m["drf"], m["tok"], 1.0, seed=4, round_=1),
                          _other(inputs))


def test_graph_greedy(inputs):
    g = inputs["g"]
    c = inputs["c"]
    T = PT.f32(0.8)
    _replay_matches_eager(lambda: svx.sv_verify_greedy(g["tgt"], g["tok"]),
                          lambda: svx.sv_verify_chain(c["tgt"], c["drf"], c["tok"], T, seed=1))


@pytest.mark.parametrize("pm", [False, True])
def test_graph_tree(inputs, pm):
    t = inputs["t"]
    md = inputs["tree"].params["max_depth"]
    if pm:
        call = lambda: svx.sv_verify_tree_pm(t["tgt"], t["tok"], t["parent"], md, 1.0, seed=5, round_=3)
    else:
        call = lambda: svx.sv_verify_tree(t["tgt"], t["drf"], t["tok"], t["parent"], md, 1.0, seed=5, round_=3)
    _replay_matches_eager(call, _other(inputs))


def test_graph_fanout(inputs):
    t = inputs["t"]
    B, N, V = t["drf"].shape
    x = t["drf"].reshape(B * N, V)
    F = torch.tensor([(3 * r) % 9 for r in range(B * N)], dtype=torch.int32, device=PT.DEV)
    _replay_matches_eager(lambda: svx.sv_fanout_topk(x, F, 8), _other(inputs))


def test_graph_cache(inputs):
    rows_cpu = inputs["rows"]
    B, K1, V = rows_cpu.shape
    rows = torch.empty(B, K1, rows_cpu.stride(1), dtype=rows_cpu.dtype, device=PT.DEV)[..., :V]
    rows.copy_(rows_cpu)
    gen = torch.Generator().manual_seed(11)
    n = torch.randint(0, K1, (B,), generator=gen, dtype=torch.int32).to(PT.DEV)
    tk = torch.randint(0, V, (B,), generator=gen, dtype=torch.int32).to(PT.DEV)
    F = torch.tensor([(5 * k + 2) % 7 for k in range(K1)], dtype=torch.int32, device=PT.DEV)
    _replay_matches_eager(lambda: svx.sv_cache_hit_test(rows, n, tk, F), _other(inputs))


def test_graph_presto(inputs):
    t = inputs["t"]
    lam = torch.tensor([0.5, 1.0, 1.5], dtype=torch.float32, device=PT.DEV)
    _replay_matches_eager(lambda: svx.sv_presto_score(t["tgt"], t["drf"], t["tok"], t["parent"], 1.0, lam, 5, 12),
                          _other(inputs))


def test_graph_branch(inputs):
    rows_cpu = inputs["rows"]
    B, g1, V = rows_cpu.shape
    rows = torch.empty(B, g1, rows_cpu.stride(1), dtype=rows_cpu.dtype, device=PT.DEV)[..., :V]
    rows.copy_(rows_cpu)
    tok = inputs["chain"].tensors["tok"].to(PT.DEV)
    cls = torch.tensor([b % 3 for b in range(B)], dtype=torch.int32, device=PT.DEV)
    T = PT.f32(0.8)
    _replay_matches_eager(lambda: svx.sv_branch_fork(rows, tok, T, 0.3, 6, cls), _other(inputs))
