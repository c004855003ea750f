"""CPU oracle for the draft-verification acceptance step (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never touches it.

The arithmetic lives in ``sv_oracle.cpp`` (plain single-threaded C++, fp64);
this module only builds that file with g++ and marshals numpy arrays into it.
Logit arrays are passed as numpy arrays: ``float32``, ``float64``, or
``uint16`` holding raw bfloat16 bit patterns (``dtype="bf16"``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.cpp")
_LIB = os.path.join(_HERE, "libsv_oracle.so")

_DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2}
_lib = None


def build(force: bool = True) -> str:
    """Compile sv_oracle.cpp into libsv_oracle.so (IEEE arithmetic, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, u32, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double
    L.svo_philox4x32_10.argtypes = [P, P, P]
    L.svo_philox4x32_10.restype = None
    L.svo_uniform.argtypes = [u64, u32, u32, u32, u32, u32]
    L.svo_uniform.restype = f64
    L.svo_chain_core.argtypes = [P, P, i32, i64, i64, P, i32, i32, f64, P, f64, P, P, P, P, P, P, P, P]
    L.svo_chain_core.restype = i32
    L.svo_verify_chain.argtypes = [P, P, i32, i64, i64, P, i32, i32, i32, f64, u64, u32, P, P, P, P, P, P, P]
    L.svo_verify_chain.restype = i32
    L.svo_verify_greedy.argtypes = [P, i32, i64, P, i32, i32, i32, P, P, P]
    L.svo_verify_greedy.restype = i32
    L.svo_verify_multi.argtypes = [P, P, i32, i64, i64, P, i32, i32, i32, i32, f64, u64, u32, P, P,
                                   P, P, P, P, P, P, P, P, P]
    L.svo_verify_multi.restype = i32
    L.svo_verify_tree.argtypes = [P, P, i32, i64, i64, P, P, i32, i32, i32, i32, f64, u64, u32, P, P,
                                  P, P, P, P, P, P, P, P, P, P]
    L.svo_verify_tree.restype = i32
    L.svo_verify_chain_pm.argtypes = [P, i32, i64, P, i32, i32, i32, f64, u64, u32, P, P, P, P, P, P, P, P, P,
                                      P]
    L.svo_verify_chain_pm.restype = i32
    L.svo_verify_tree_pm.argtypes = [P, i32, i64, P, P, i32, i32, i32, i32, f64, u64, u32, P, P, P, P, P, P, P, P,
                                     P, P, P]
    L.svo_verify_tree_pm.restype = i32
    L.svo_fanout_topk.argtypes = [P, i32, i64, i32, i32, P, i32, P, P]
    L.svo_fanout_topk.restype = i32
    L.svo_cache_hit_test.argtypes = [P, i32, i64, i32, i32, i32, P, P, P, P, P]
    L.svo_cache_hit_test.restype = i32
    L.svo_presto_score.argtypes = [P, P, i32, i64, i64, P, P, i32, i32, i32, f64, P, i32, i32, i32, P, P, P, P, P]
    L.svo_presto_score.restype = i32
    L.svo_branch_fork.argtypes = [P, i32, i64, P, P, i32, i32, i32, f64, f64, i32, P, P, P, P, P]
    L.svo_branch_fork.restype = i32
    L.svo_geometric_fanout.argtypes = [i32, f64, f64, i32, i32, P]
    L.svo_geometric_fanout.restype = i32
    return L


def lib():
    global _lib
    if _lib is None:
        # SV_ORACLE_LIB: another build of sv_oracle.cpp (the sanitizer test's ASan/UBSan build)
        other = os.environ.get("SV_ORACLE_LIB")
        if other:
            _lib = _load(other)
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _load(_LIB)
    return _lib


class use_library:
    """Context manager: route every oracle call through another build of
    sv_oracle.cpp (the mutant tests plant mistakes in a copy of the source)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(a: np.ndarray, dtype: str):
    code = _DTYPE_CODE[dtype]
    want = {0: np.float32, 1: np.uint16, 2: np.float64}[code]
    if a.dtype != want:
        raise TypeError(f"logits for dtype={dtype} must be {np.dtype(want).name}, got {a.dtype}")
    if a.strides[-1] != a.itemsize:
        raise ValueError("logit rows must be contiguous along the vocabulary axis")
    return a, code


def _row_stride(a: np.ndarray) -> int:
    """Row stride in elements; every leading axis must step by whole rows of that stride."""
    if a.ndim < 2:
        return a.shape[-1]
    rs = a.strides[-2] // a.itemsize
    step = a.strides[-2]
    for ax in range(a.ndim - 2, 0, -1):
        step *= a.shape[ax]
        if a.shape[ax - 1] > 1 and a.strides[ax - 1] != step:
            raise ValueError("logit rows must be evenly spaced (one row stride across all leading axes)")
    return rs


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: invalid input (code {rc})")


# ---------------------------------------------------------------------------
def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().svo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, idx, b, k, round_, tag):
    return lib().svo_uniform(seed, idx, b, k, round_, tag)


def chain_core(tgt, drf, tok, T, r, u, dtype="f64"):
    """One chain round of one sequence with explicit uniforms.

    tgt [gamma+1, V], drf [gamma, V]; returns dict(n, t, p, q, a, w, mdec, mcdf).
    """
    tgt, code = _logits(tgt, dtype)
    drf, _ = _logits(drf, dtype)
    gamma, V = drf.shape[0], drf.shape[1]
    tok = _i32(tok)
    r = np.ascontiguousarray(r, dtype=np.float64)
    n = np.zeros(1, np.int32)
    t = np.zeros(1, np.int32)
    p = np.zeros(gamma)
    q = np.zeros(gamma)
    a = np.zeros(gamma)
    w = np.zeros(V)
    md = np.zeros(1)
    mc = np.zeros(1)
    rc = lib().svo_chain_core(_ptr(tgt), _ptr(drf), code, _row_stride(tgt), _row_stride(drf), _ptr(tok), gamma, V,
                              float(T), _ptr(r), float(u), _ptr(n), _ptr(t), _ptr(p), _ptr(q), _ptr(a), _ptr(w),
                              _ptr(md), _ptr(mc))
    _check(rc, "chain_core")
    return dict(n=int(n[0]), t=int(t[0]), p=p, q=q, a=a, w=w, mdec=float(md[0]), mcdf=float(mc[0]))


def verify_chain(tgt, drf, tok, T, seed, round_, dtype):
    """Batched chain verification.  tgt [B, gamma+1, V], drf [B, gamma, V], tok [B, gamma]."""
    tgt, code = _logits(tgt, dtype)
    drf, _ = _logits(drf, dtype)
    B, gamma, V = drf.shape
    assert tgt.shape[:2] == (B, gamma + 1)
    tok = _i32(tok)
    out = dict(n=np.zeros(B, np.int32), t=np.zeros(B, np.int32), p=np.zeros((B, gamma)), q=np.zeros((B, gamma)),
               mdec=np.zeros(B), mcdf=np.zeros(B), rows=np.zeros(B, np.int32))
    rc = lib().svo_verify_chain(_ptr(tgt), _ptr(drf), code, _row_stride(tgt), _row_stride(drf), _ptr(tok), B, gamma,
                                V, float(T), int(seed), int(round_), _ptr(out["n"]), _ptr(out["t"]), _ptr(out["p"]),
                                _ptr(out["q"]), _ptr(out["mdec"]), _ptr(out["mcdf"]), _ptr(out["rows"]))
    _check(rc, "verify_chain")
    return out


def verify_greedy(tgt, tok, dtype):
    """tgt [B, gamma+1, V], tok [B, gamma] -> dict(n, t, argmax[B, gamma+1])."""
    tgt, code = _logits(tgt, dtype)
    B, g1, V = tgt.shape
    gamma = g1 - 1
    tok = _i32(tok)
    out = dict(n=np.zeros(B, np.int32), t=np.zeros(B, np.int32), argmax=np.zeros((B, g1), np.int32))
    rc = lib().svo_verify_greedy(_ptr(tgt), code, _row_stride(tgt), _ptr(tok), B, gamma, V, _ptr(out["n"]),
                                 _ptr(out["t"]), _ptr(out["argmax"]))
    _check(rc, "verify_greedy")
    return out


def verify_multi(tgt, drf, tok, T, seed, round_, dtype, r=None, u=None):
    """tgt [B, K, gamma+1, V], drf [B, gamma, V] (shared), tok [B, K, gamma]."""
    tgt, code = _logits(tgt, dtype)
    drf, _ = _logits(drf, dtype)
    B, K, g1, V = tgt.shape
    gamma = g1 - 1
    assert drf.shape == (B, gamma, V)
    tok = _i32(tok)
    rr = None if r is None else np.ascontiguousarray(r, dtype=np.float64)
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    out = dict(k=np.zeros(B, np.int32), n=np.zeros(B, np.int32), t=np.zeros(B, np.int32),
               n_cand=np.zeros((B, K), np.int32), p=np.zeros((B, K, gamma)), q=np.zeros((B, K, gamma)),
               mdec=np.zeros(B), mcdf=np.zeros(B), rows=np.zeros(B, np.int32))
    rc = lib().svo_verify_multi(_ptr(tgt), _ptr(drf), code, _row_stride(tgt), _row_stride(drf), _ptr(tok), B, K,
                                gamma, V, float(T), int(seed), int(round_), _ptr(rr), _ptr(uu), _ptr(out["k"]),
                                _ptr(out["n"]), _ptr(out["t"]), _ptr(out["n_cand"]), _ptr(out["p"]), _ptr(out["q"]),
                                _ptr(out["mdec"]), _ptr(out["mcdf"]), _ptr(out["rows"]))
    _check(rc, "verify_multi")
    return out


def verify_tree(tgt, drf, node_tok, parent, max_depth, T, seed, round_, dtype, r=None, u=None, want_w=False):
    """tgt/drf [B, N, V], node_tok/parent [B, N]."""
    tgt, code = _logits(tgt, dtype)
    drf, _ = _logits(drf, dtype)
    B, N, V = tgt.shape
    node_tok = _i32(node_tok)
    parent = _i32(parent)
    rr = None if r is None else np.ascontiguousarray(r, dtype=np.float64)
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    out = dict(len=np.zeros(B, np.int32), path=np.zeros((B, max_depth), np.int32), t=np.zeros(B, np.int32),
               p=np.full((B, N), np.nan), q=np.full((B, N), np.nan), a=np.zeros((B, N)),
               w=np.zeros((B, V)) if want_w else None, mdec=np.zeros(B), mcdf=np.zeros(B),
               passes=np.zeros(B, np.int32))
    rc = lib().svo_verify_tree(_ptr(tgt), _ptr(drf), code, _row_stride(tgt), _row_stride(drf), _ptr(node_tok),
                               _ptr(parent), B, N, int(max_depth), V, float(T), int(seed), int(round_), _ptr(rr),
                               _ptr(uu), _ptr(out["len"]), _ptr(out["path"]), _ptr(out["t"]), _ptr(out["p"]),
                               _ptr(out["q"]), _ptr(out["a"]), _ptr(out["w"]), _ptr(out["mdec"]), _ptr(out["mcdf"]),
                               _ptr(out["passes"]))
    _check(rc, "verify_tree")
    return out


def verify_chain_pm(tgt, tok, T, seed, round_, dtype, r=None, u=None, want_w=False):
    """Point-mass chain verification.  tgt [B, gamma+1, V], tok [B, gamma]; no draft rows."""
    tgt, code = _logits(tgt, dtype)
    B, g1, V = tgt.shape
    gamma = g1 - 1
    tok = _i32(tok)
    rr = None if r is None else np.ascontiguousarray(r, dtype=np.float64)
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    out = dict(n=np.zeros(B, np.int32), t=np.zeros(B, np.int32), p=np.zeros((B, gamma)), a=np.zeros((B, gamma)),
               w=np.zeros((B, V)) if want_w else None, mdec=np.zeros(B), mcdf=np.zeros(B),
               rows=np.zeros(B, np.int32))
    rc = lib().svo_verify_chain_pm(_ptr(tgt), code, _row_stride(tgt), _ptr(tok), B, gamma, V, float(T), int(seed),
                                   int(round_), _ptr(rr), _ptr(uu), _ptr(out["n"]), _ptr(out["t"]), _ptr(out["p"]),
                                   _ptr(out["a"]), _ptr(out["w"]), _ptr(out["mdec"]), _ptr(out["mcdf"]),
                                   _ptr(out["rows"]))
    _check(rc, "verify_chain_pm")
    return out


def verify_tree_pm(tgt, node_tok, parent, max_depth, T, seed, round_, dtype, r=None, u=None, want_w=False):
    """Point-mass tree verification.  tgt [B, N, V], node_tok/parent [B, N]; no draft rows."""
    tgt, code = _logits(tgt, dtype)
    B, N, V = tgt.shape
    node_tok = _i32(node_tok)
    parent = _i32(parent)
    rr = None if r is None else np.ascontiguousarray(r, dtype=np.float64)
    uu = None if u is None else np.ascontiguousarray(u, dtype=np.float64)
    out = dict(len=np.zeros(B, np.int32), path=np.zeros((B, max_depth), np.int32), t=np.zeros(B, np.int32),
               p=np.full((B, N), np.nan), a=np.zeros((B, N)), w=np.zeros((B, V)) if want_w else None,
               mdec=np.zeros(B), mcdf=np.zeros(B), passes=np.zeros(B, np.int32))
    rc = lib().svo_verify_tree_pm(_ptr(tgt), code, _row_stride(tgt), _ptr(node_tok), _ptr(parent), B, N,
                                  int(max_depth), V, float(T), int(seed), int(round_), _ptr(rr), _ptr(uu),
                                  _ptr(out["len"]), _ptr(out["path"]), _ptr(out["t"]), _ptr(out["p"]), _ptr(out["a"]),
                                  _ptr(out["w"]), _ptr(out["mdec"]), _ptr(out["mcdf"]), _ptr(out["passes"]))
    _check(rc, "verify_tree_pm")
    return out


def fanout_topk(logits, F, F_max, dtype):
    """logits [R, V], F [R] -> (ids [R, F_max] (-1 padded), vals [R, F_max])."""
    logits, code = _logits(logits, dtype)
    R, V = logits.shape
    F = _i32(F)
    ids = np.zeros((R, F_max), np.int32)
    vals = np.zeros((R, F_max), np.float32)
    rc = lib().svo_fanout_topk(_ptr(logits), code, _row_stride(logits), R, V, _ptr(F), int(F_max), _ptr(ids),
                               _ptr(vals))
    _check(rc, "fanout_topk")
    return ids, vals


def cache_hit_test(drf, n, t, F, dtype):
    """Speculation-cache hit test.  drf [B, K+1, V] draft rows per lookahead position, outcome (n, t) [B],
    F [K+1] or None -> dict(rank [B], hit [B] or None)."""
    drf, code = _logits(drf, dtype)
    B, K1, V = drf.shape
    n, t = _i32(n), _i32(t)
    Fa = None if F is None else _i32(F)
    out = dict(rank=np.zeros(B, np.int32), hit=None if F is None else np.zeros(B, np.int32))
    rc = lib().svo_cache_hit_test(_ptr(drf), code, _row_stride(drf), B, K1 - 1, V, _ptr(n), _ptr(t), _ptr(Fa),
                                  _ptr(out["rank"]), _ptr(out["hit"]))
    _check(rc, "cache_hit_test")
    return out


def presto_score(tgt, drf, node_tok, parent, T, lam, k, b_top, dtype):
    """PRESTO scoring and one expansion step.  tgt, drf [B, N, V]; node_tok, parent [B, N]; lam [D] (lambda of
    depth d at lam[min(d, D) - 1]) -> dict(s, S [B, N], node, tok, score [B, b_top])."""
    tgt, code = _logits(tgt, dtype)
    drf, code2 = _logits(drf, dtype)
    B, N, V = tgt.shape
    node_tok, parent = _i32(node_tok), _i32(parent)
    lam = np.ascontiguousarray(lam, dtype=np.float32)
    out = dict(s=np.zeros((B, N)), S=np.zeros((B, N)), node=np.zeros((B, b_top), np.int32),
               tok=np.zeros((B, b_top), np.int32), score=np.zeros((B, b_top)))
    rc = lib().svo_presto_score(_ptr(tgt), _ptr(drf), code, _row_stride(tgt), _row_stride(drf), _ptr(node_tok),
                                _ptr(parent), B, N, V, float(T), _ptr(lam), len(lam), int(k), int(b_top),
                                _ptr(out["s"]), _ptr(out["S"]), _ptr(out["node"]), _ptr(out["tok"]),
                                _ptr(out["score"]))
    _check(rc, "presto_score")
    return out


def branch_fork(drf, tok, cls, T, eps, k_max, dtype):
    """SpecBranch fork.  drf [B, gamma+1, V] draft rows q_1..q_{gamma+1}; tok [B, gamma]; cls [B] or None
    -> dict(pos, qb, k [B], ids [B, k_max], margin [B])."""
    drf, code = _logits(drf, dtype)
    B, g1, V = drf.shape
    tok = _i32(tok)
    cl = None if cls is None else _i32(cls)
    out = dict(pos=np.zeros(B, np.int32), qb=np.zeros(B), k=np.zeros(B, np.int32),
               ids=np.zeros((B, k_max), np.int32), margin=np.zeros(B))
    rc = lib().svo_branch_fork(_ptr(drf), code, _row_stride(drf), _ptr(tok), _ptr(cl), B, g1 - 1, V, float(T),
                               float(eps), int(k_max), _ptr(out["pos"]), _ptr(out["qb"]), _ptr(out["k"]),
                               _ptr(out["ids"]), _ptr(out["margin"]))
    _check(rc, "branch_fork")
    return out


def geometric_fanout(F0, a_p, r, K, capped_last=False):
    out = np.zeros(K + 1, np.int32)
    lib().svo_geometric_fanout(int(F0), float(a_p), float(r), int(K), int(bool(capped_last)), _ptr(out))
    return out
