"""Device-side error paths of the C ABI (the error word of specverify.h), on the GPU.

- SV_DERR_TIMEOUT: the chain draw and the tree walk split a sequence over G blocks that exchange values and
  wait for each other with a bounded wait.  The test lowers the bound through the workspace header and
  switches on the test switch that makes the last block of sequence 0 never publish: its partners' waits run
  out, the bit is set, and every kernel still exits (the call's stream synchronises).  With the switch off
  again, the next call on the same workspace matches the oracle: a timed-out call leaves nothing behind.
- SV_DERR_TREE: parent arrays that are not parent-first, and paths longer than max_depth.
- SV_DERR_ROW: a needed row with no finite logit (outside the contract; it must not fault and must reject).
- The binding's checked mode raises on a set error word.
No test makes the GPU fault or hang: every wait here is bounded and ends.
"""
import numpy as np
import pytest
import torch

from lossless_draft_verification_04_amd import specverify as svx
from lossless_draft_verification_04_amd import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu
DEV = PT.DEV
NEG = float("-inf")


def _knobs(spin, withhold):
    # header words 1 and 2 of the binding's workspace for this device (large enough that the calls below reuse it)
    ws = svx.Workspace.get(DEV, 16 << 20)
    torch.cuda.synchronize()
    ws[4:12].view(torch.int32).copy_(torch.tensor([spin, withhold], dtype=torch.int32))
    torch.cuda.synchronize()


@pytest.fixture
def knobs_reset():
    yield
    _knobs(0, 0)
    svx.sv_get_device_error(DEV)


def test_chain_draw_wait_runs_out_and_every_kernel_exits(knobs_reset):
    wl = W.chain_zipf(B=4, gamma=6, V=60000, T=0.9, seed=71)
    g = wl.to(DEV)
    assert svx.sv_get_device_error(DEV) == 0
    _knobs(2000, 1)
    PT.say("  chain with a withheld publish (sequence 0, last draw block), wait bound 2000 polls")
    svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 0.9, seed=1)
    torch.cuda.synchronize()  # returns: every block of both launches exited
    assert svx.sv_get_device_error(DEV) & svx.DERR_TIMEOUT
    _knobs(0, 0)
    PT.chain(wl, 1, 0)  # the same workspace, switch off: exact again
    PT.device_error_clear()


def test_tree_walk_wait_runs_out_and_every_kernel_exits(knobs_reset):
    wl = W.tree_zipf(B=3, N=24, max_depth=6, V=40000, T=1.0, seed=72)
    g = wl.to(DEV)
    assert svx.sv_get_device_error(DEV) == 0
    _knobs(2000, 1)
    PT.say("  tree with a withheld publish (sequence 0, last walk block), wait bound 2000 polls")
    svx.sv_verify_tree(g["tgt"], g["drf"], g["tok"], g["parent"], 6, 1.0, seed=2)
    torch.cuda.synchronize()
    assert svx.sv_get_device_error(DEV) & svx.DERR_TIMEOUT
    _knobs(0, 0)
    PT.tree(wl, 2, 0)
    PT.device_error_clear()


def _valid_tree_outputs(out, N, max_depth, V):
    L = out["len"].cpu().numpy()
    path = out["path"].cpu().numpy()
    t = out["tok"].cpu().numpy()
    assert ((L >= 0) & (L <= max_depth)).all()
    for b in range(len(L)):
        assert ((path[b, :L[b]] >= 1) & (path[b, :L[b]] < N)).all()
        assert (path[b, L[b]:] == -1).all()
        assert -1 <= t[b] < V


def test_invalid_parent_arrays_set_the_tree_bit():
    wl = W.tree_zipf(B=4, N=20, max_depth=6, V=5000, T=1.0, seed=73)
    par = wl.tensors["parent"]
    par[0, 5] = 5      # its own parent
    par[1, 3] = 17     # a later node as parent
    par[2, 7] = -4     # negative
    par[3, 9] = 400    # outside the tree
    g = wl.to(DEV)
    for fn in ("tree", "tree_pm"):
        if fn == "tree":
            out = svx.sv_verify_tree(g["tgt"], g["drf"], g["tok"], g["parent"], 6, 1.0)
        else:
            out = svx.sv_verify_tree_pm(g["tgt"], g["tok"], g["parent"], 6, 1.0)
        torch.cuda.synchronize()
        assert svx.sv_get_device_error(DEV) & svx.DERR_TREE, fn
        _valid_tree_outputs(out, 20, 6, 5000)


def test_paths_longer_than_max_depth_set_the_tree_bit():
    wl = W.chain_shaped_tree(W.chain_zipf(B=3, gamma=6, V=4000, T=1.0, seed=74))
    # the drafts are the target's argmax with a sure accept: every walk runs to the depth limit with a child left
    tgt, drf, tok, par = (wl.tensors[k] for k in ("tgt", "drf", "tok", "parent"))
    for b in range(3):
        for i in range(1, 7):
            drf[b, i - 1, tok[b, i]] = NEG  # q(x) = 0, p(x) > 0: accepted
    g = wl.to(DEV)
    out = svx.sv_verify_tree(g["tgt"], g["drf"], g["tok"], g["parent"], 3, 1.0)
    torch.cuda.synchronize()
    assert svx.sv_get_device_error(DEV) & svx.DERR_TREE
    assert (out["len"].cpu().numpy() == 3).all()
    _valid_tree_outputs(out, 7, 3, 4000)


def test_rows_without_a_finite_logit_set_the_row_bit_and_reject():
    wl = W.chain_zipf(B=3, gamma=5, V=8000, T=1.0, seed=75)
    tok = wl.tensors["tok"]
    for b in range(3):
        for j in range(5):
            wl.tensors["drf"][b, j, tok[b, j]] = NEG  # sure accepts up to the empty row
    wl.tensors["tgt"][1, 2].fill_(NEG)  # sequence 1: target row 3 has no finite logit
    g = wl.to(DEV)
    for pm in (False, True):
        if pm:
            out = svx.sv_verify_chain_pm(g["tgt"], g["tok"], 1.0)
        else:
            out = svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0)
        torch.cuda.synchronize()
        assert svx.sv_get_device_error(DEV) & svx.DERR_ROW
        n = out["n"].cpu().numpy()
        assert n[1] <= 2  # p(x) = 0 at position 3: rejected there at the latest
        if not pm:
            assert n[0] == 5 and n[2] == 5
        t = out["tok"].cpu().numpy()
        assert (t[[0, 2]] >= 0).all()


def test_checked_mode_raises_on_device_errors():
    wl = W.chain_zipf(B=2, gamma=3, V=3000, T=1.0, seed=76)
    wl.tensors["tok"][0, 1] = 3000
    g = wl.to(DEV)
    svx.set_checked(True)
    try:
        with pytest.raises(svx.DeviceError) as ei:
            svx.sv_verify_chain(g["tgt"], g["drf"], g["tok"], 1.0)
        assert ei.value.flags & svx.DERR_TOKEN
        wl2 = W.chain_zipf(B=2, gamma=3, V=3000, T=1.0, seed=77)
        g2 = wl2.to(DEV)
        svx.sv_verify_chain(g2["tgt"], g2["drf"], g2["tok"], 1.0)  # clean input: no raise
    finally:
        svx.set_checked(False)
    assert svx.sv_get_device_error(DEV) == 0
