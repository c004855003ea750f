"""Python binding of libspecverify (ctypes): argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks their
shapes and layouts, allocates the outputs, and calls the C entry point of the
same name on torch's current stream.  Every step of the computation runs in
the HIP kernels of libspecverify.so; if that library is not built, importing
this module fails.

Layout rules (the C ABI's): logit tensors are [..., V] with a unit stride
along V and evenly spaced rows whose start addresses are 16-byte aligned
(row stride * element size a multiple of 16).  dtype bfloat16 or float32.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SV_LIBRARY selects another build of the library (the timeline build), by path
_LIB_PATH = os.environ.get("SV_LIBRARY") or os.path.join(_HERE, "libspecverify.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; build it with `python -m lossless_draft_verification_04_amd.build` "
        "(hipcc, gfx950)")

_lib = ctypes.CDLL(_LIB_PATH)

SV_OK, SV_EINVAL, SV_EDTYPE, SV_EALIGN, SV_EWORKSPACE, SV_EUNSUPPORTED, SV_EHIP = range(7)
SV_F32, SV_BF16 = 0, 1
(SV_OP_CHAIN, SV_OP_GREEDY, SV_OP_MULTI, SV_OP_TREE, SV_OP_FANOUT, SV_OP_CHAIN_PM, SV_OP_TREE_PM,
 SV_OP_CACHE, SV_OP_PRESTO, SV_OP_BRANCH) = range(10)
DERR_TOKEN, DERR_TREE, DERR_FANOUT, DERR_ROW, DERR_TIMEOUT = 1, 2, 4, 8, 16

_P = ctypes.c_void_p
_i32, _i64, _u32, _u64, _f32, _f64, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64,
                                           ctypes.c_float, ctypes.c_double, ctypes.c_size_t)

_SIGS = {
    "sv_version": ([], _i32),
    "sv_status_string": ([_i32], ctypes.c_char_p),
    "sv_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "sv_workspace_init": ([_P, _sz, _P], _i32),
    "sv_get_device_error": ([_P, ctypes.POINTER(_i32), _P], _i32),
    "sv_verify_chain": ([_P, _P, _i32, _i64, _i64, _P, _i32, _i32, _i32, _f32, _u64, _u32, _P, _P, _P, _P, _P,
                         _sz, _P], _i32),
    "sv_verify_greedy": ([_P, _i32, _i64, _P, _i32, _i32, _i32, _P, _P, _P, _P, _sz, _P], _i32),
    "sv_verify_multi": ([_P, _P, _i32, _i64, _i64, _P, _i32, _i32, _i32, _i32, _f32, _u64, _u32, _P, _P, _P, _P,
                         _P, _P, _P, _sz, _P], _i32),
    "sv_verify_tree": ([_P, _P, _i32, _i64, _i64, _P, _P, _i32, _i32, _i32, _i32, _f32, _u64, _u32, _P, _P, _P,
                        _P, _P, _P, _sz, _P], _i32),
    "sv_verify_chain_noalloc": ([_P, _P, _i32, _i64, _i64, _P, _i32, _i32, _i32, _f32, _u64, _u32, _P, _P, _P, _P,
                                 _P, _P], _i32),
    "sv_verify_chain_pm": ([_P, _i32, _i64, _P, _i32, _i32, _i32, _f32, _u64, _u32, _P, _P, _P, _P, _sz, _P], _i32),
    "sv_verify_tree_pm": ([_P, _i32, _i64, _P, _P, _i32, _i32, _i32, _i32, _f32, _u64, _u32, _P, _P, _P, _P, _P,
                           _sz, _P], _i32),
    "sv_fanout_topk": ([_P, _i32, _i64, _i32, _i32, _P, _i32, _P, _P, _P, _sz, _P], _i32),
    "sv_cache_hit_test": ([_P, _i32, _i64, _i32, _i32, _i32, _P, _P, _P, _P, _P, _P, _sz, _P], _i32),
    "sv_presto_score": ([_P, _P, _i32, _i64, _i64, _P, _P, _i32, _i32, _i32, _f32, _P, _i32, _i32, _i32, _P, _P,
                         _P, _P, _P, _P, _sz, _P], _i32),
    "sv_branch_fork": ([_P, _i32, _i64, _P, _P, _i32, _i32, _i32, _f32, _f32, _i32, _P, _P, _P, _P, _P, _sz, _P],
                       _i32),
    "sv_geometric_fanout": ([_i32, _f64, _f64, _i32, _i32, ctypes.POINTER(_i32)], _i32),
    "sv_read_probe": ([_P, _sz, _i32, _i32, _i32, _sz, _P, _P], _i32),
    "sv_timeline_set": ([_P, ctypes.c_uint64], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


class SpecVerifyError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {_lib.sv_status_string(status).decode()} (status {status})")
        self.status = status


def _check(status, what):
    if status != SV_OK:
        raise SpecVerifyError(status, what)


class DeviceError(RuntimeError):
    """Device-side input error bits (DERR_*) reported by a call in checked mode."""

    def __init__(self, flags, what):
        names = [n for n, b in (("token", DERR_TOKEN), ("tree", DERR_TREE), ("fanout", DERR_FANOUT),
                                ("row", DERR_ROW), ("timeout", DERR_TIMEOUT)) if flags & b]
        super().__init__(f"{what}: device error word {flags} ({', '.join(names)}); outputs of the call are invalid")
        self.flags = flags


_CHECKED = False


def set_checked(on: bool = True) -> None:
    """Checked mode: after every call, synchronise its stream and raise DeviceError if the workspace's device
    error word is set (and clear it).  Off by default: a call is then asynchronous and the word is read only
    through sv_get_device_error."""
    global _CHECKED
    _CHECKED = bool(on)


def _checked(device, what, workspace=None):
    if not _CHECKED:
        return
    ws = workspace if workspace is not None else Workspace.get(device, 0)
    flags = _i32(0)
    _check(_lib.sv_get_device_error(_ptr(ws), ctypes.byref(flags), _stream(device)), "sv_get_device_error")
    if flags.value:
        raise DeviceError(flags.value, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise SpecVerifyError(SV_EDTYPE, f"logits dtype {t.dtype}")


def _row_stride(t: torch.Tensor, what: str) -> int:
    """Row stride (elements) of a [..., V] logit tensor with evenly spaced rows."""
    if t.stride(-1) != 1:
        raise SpecVerifyError(SV_EINVAL, f"{what}: vocabulary axis must have unit stride")
    if t.dim() < 2:
        return t.shape[-1]
    rs = t.stride(-2)
    step = rs
    for ax in range(t.dim() - 2, 0, -1):
        step *= t.shape[ax]
        if t.shape[ax - 1] > 1 and t.stride(ax - 1) != step:
            raise SpecVerifyError(SV_EINVAL, f"{what}: rows must be evenly spaced")
    return rs


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32_tensor(t: torch.Tensor, shape, what):
    if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise SpecVerifyError(SV_EINVAL, f"{what}: want contiguous int32 {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


class Workspace:
    """Per-device scratch for the kernels (zero-filled on creation, grown on demand)."""

    _lock = threading.Lock()
    _cache = {}

    @classmethod
    def get(cls, device, nbytes: int) -> torch.Tensor:
        dev = torch.device(device)
        key = dev.index if dev.index is not None else torch.cuda.current_device()
        with cls._lock:
            ws = cls._cache.get(key)
            if ws is None or ws.numel() < nbytes:
                ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
                if ws.data_ptr() % 256:
                    raise SpecVerifyError(SV_EALIGN, "workspace allocation not 256-byte aligned")
                cls._cache[key] = ws
            return ws


def workspace_size(op, dt, B, K, gamma_or_N, V, F_max=1) -> int:
    n = _sz(0)
    _check(_lib.sv_workspace_size(op, dt, B, K, gamma_or_N, V, F_max, ctypes.byref(n)), "sv_workspace_size")
    return n.value


def sv_get_device_error(device=None) -> int:
    """Synchronise and read (and clear) the device error word of this device's workspace."""
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    ws = Workspace.get(device, 0)
    flags = _i32(0)
    _check(_lib.sv_get_device_error(_ptr(ws), ctypes.byref(flags), _stream(device)), "sv_get_device_error")
    return flags.value


def sv_verify_chain(tgt, drf, tok, T, seed=0, round_=0, want_pq=True, workspace=None):
    """tgt [B, gamma+1, V], drf [B, gamma, V], tok [B, gamma] int32 -> dict(n, tok, p, q)."""
    B, g1, V = tgt.shape
    gamma = g1 - 1
    if tuple(drf.shape) != (B, gamma, V) or drf.dtype != tgt.dtype:
        raise SpecVerifyError(SV_EINVAL, f"drf shape {tuple(drf.shape)} / dtype does not match tgt")
    _i32_tensor(tok, (B, gamma), "tok")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(dev, workspace_size(SV_OP_CHAIN, dt, B, 1, gamma, V))
    out_n = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty(B, dtype=torch.int32, device=dev)
    p = torch.empty(B, gamma, dtype=torch.float32, device=dev) if want_pq else None
    q = torch.empty(B, gamma, dtype=torch.float32, device=dev) if want_pq else None
    _check(_lib.sv_verify_chain(_ptr(tgt), _ptr(drf), dt, _row_stride(tgt, "tgt"), _row_stride(drf, "drf"),
                                _ptr(tok), B, gamma, V, float(T), int(seed), int(round_), _ptr(out_n), _ptr(out_tok),
                                _ptr(p), _ptr(q), _ptr(ws), ws.numel(), _stream(dev)), "sv_verify_chain")
    _checked(dev, "sv_verify_chain", workspace)
    return dict(n=out_n, tok=out_tok, p=p, q=q)


NOALLOC_SCRATCH_BYTES = 8 << 20


def sv_verify_chain_noalloc(tgt, drf, tok, T, seed=0, round_=0, want_pq=True, out_err=None):
    """sv_verify_chain through the allocation-free entry point: the library's own per-GPU scratch array, no
    workspace.  out_err: optional zeroed device int32 tensor [1] that receives the device error bits."""
    B, g1, V = tgt.shape
    gamma = g1 - 1
    if tuple(drf.shape) != (B, gamma, V) or drf.dtype != tgt.dtype:
        raise SpecVerifyError(SV_EINVAL, f"drf shape {tuple(drf.shape)} / dtype does not match tgt")
    _i32_tensor(tok, (B, gamma), "tok")
    if out_err is not None:
        _i32_tensor(out_err, (1,), "out_err")
    dt = _dtype_code(tgt)
    dev = tgt.device
    out_n = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty(B, dtype=torch.int32, device=dev)
    p = torch.empty(B, gamma, dtype=torch.float32, device=dev) if want_pq else None
    q = torch.empty(B, gamma, dtype=torch.float32, device=dev) if want_pq else None
    _check(_lib.sv_verify_chain_noalloc(_ptr(tgt), _ptr(drf), dt, _row_stride(tgt, "tgt"), _row_stride(drf, "drf"),
                                        _ptr(tok), B, gamma, V, float(T), int(seed), int(round_), _ptr(out_n),
                                        _ptr(out_tok), _ptr(p), _ptr(q), _ptr(out_err), _stream(dev)),
           "sv_verify_chain_noalloc")
    return dict(n=out_n, tok=out_tok, p=p, q=q)


def sv_verify_chain_pm(tgt, tok, T, seed=0, round_=0, want_p=True, workspace=None):
    """Point-mass acceptance. tgt [B, gamma+1, V], tok [B, gamma] int32 -> dict(n, tok, p)."""
    B, g1, V = tgt.shape
    gamma = g1 - 1
    _i32_tensor(tok, (B, gamma), "tok")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(
        dev, workspace_size(SV_OP_CHAIN_PM, dt, B, 1, gamma, V))
    out_n = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty(B, dtype=torch.int32, device=dev)
    p = torch.empty(B, gamma, dtype=torch.float32, device=dev) if want_p else None
    _check(_lib.sv_verify_chain_pm(_ptr(tgt), dt, _row_stride(tgt, "tgt"), _ptr(tok), B, gamma, V, float(T),
                                   int(seed), int(round_), _ptr(out_n), _ptr(out_tok), _ptr(p), _ptr(ws),
                                   ws.numel(), _stream(dev)), "sv_verify_chain_pm")
    _checked(dev, "sv_verify_chain_pm", workspace)
    return dict(n=out_n, tok=out_tok, p=p)


def sv_verify_greedy(tgt, tok, want_argmax=True, workspace=None):
    """tgt [B, gamma+1, V], tok [B, gamma] -> dict(n, tok, argmax [B, gamma+1])."""
    B, g1, V = tgt.shape
    gamma = g1 - 1
    _i32_tensor(tok, (B, gamma), "tok")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(dev, workspace_size(SV_OP_GREEDY, dt, B, 1, gamma, V))
    out_n = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty(B, dtype=torch.int32, device=dev)
    am = torch.empty(B, g1, dtype=torch.int32, device=dev) if want_argmax else None
    _check(_lib.sv_verify_greedy(_ptr(tgt), dt, _row_stride(tgt, "tgt"), _ptr(tok), B, gamma, V, _ptr(out_n),
                                 _ptr(out_tok), _ptr(am), _ptr(ws), ws.numel(), _stream(dev)), "sv_verify_greedy")
    _checked(dev, "sv_verify_greedy", workspace)
    return dict(n=out_n, tok=out_tok, argmax=am)


def sv_verify_multi(tgt, drf, tok, T, seed=0, round_=0, want_pq=True, workspace=None):
    """tgt [B, K, gamma+1, V], drf [B, gamma, V], tok [B, K, gamma] -> dict(k, n, tok, n_cand, p, q)."""
    B, K, g1, V = tgt.shape
    gamma = g1 - 1
    if tuple(drf.shape) != (B, gamma, V) or drf.dtype != tgt.dtype:
        raise SpecVerifyError(SV_EINVAL, f"drf shape {tuple(drf.shape)} / dtype does not match tgt")
    _i32_tensor(tok, (B, K, gamma), "tok")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(dev, workspace_size(SV_OP_MULTI, dt, B, K, gamma, V))
    out = dict(k=torch.empty(B, dtype=torch.int32, device=dev), n=torch.empty(B, dtype=torch.int32, device=dev),
               tok=torch.empty(B, dtype=torch.int32, device=dev),
               n_cand=torch.empty(B, K, dtype=torch.int32, device=dev),
               p=torch.empty(B, K, gamma, dtype=torch.float32, device=dev) if want_pq else None,
               q=torch.empty(B, K, gamma, dtype=torch.float32, device=dev) if want_pq else None)
    _check(_lib.sv_verify_multi(_ptr(tgt), _ptr(drf), dt, _row_stride(tgt, "tgt"), _row_stride(drf, "drf"),
                                _ptr(tok), B, K, gamma, V, float(T), int(seed), int(round_), _ptr(out["k"]),
                                _ptr(out["n"]), _ptr(out["tok"]), _ptr(out["n_cand"]), _ptr(out["p"]),
                                _ptr(out["q"]), _ptr(ws), ws.numel(), _stream(dev)), "sv_verify_multi")
    _checked(dev, "sv_verify_multi", workspace)
    return out


def sv_verify_tree(tgt, drf, node_tok, parent, max_depth, T, seed=0, round_=0, want_pq=True, workspace=None):
    """tgt, drf [B, N, V]; node_tok, parent [B, N] -> dict(len, path [B, max_depth], tok, p, q)."""
    B, N, V = tgt.shape
    if tuple(drf.shape) != (B, N, V) or drf.dtype != tgt.dtype:
        raise SpecVerifyError(SV_EINVAL, f"drf shape {tuple(drf.shape)} / dtype does not match tgt")
    _i32_tensor(node_tok, (B, N), "node_tok")
    _i32_tensor(parent, (B, N), "parent")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(dev, workspace_size(SV_OP_TREE, dt, B, 1, N, V))
    out = dict(len=torch.empty(B, dtype=torch.int32, device=dev),
               path=torch.empty(B, max_depth, dtype=torch.int32, device=dev),
               tok=torch.empty(B, dtype=torch.int32, device=dev),
               p=torch.full((B, N), float("nan"), dtype=torch.float32, device=dev) if want_pq else None,
               q=torch.full((B, N), float("nan"), dtype=torch.float32, device=dev) if want_pq else None)
    _check(_lib.sv_verify_tree(_ptr(tgt), _ptr(drf), dt, _row_stride(tgt, "tgt"), _row_stride(drf, "drf"),
                               _ptr(node_tok), _ptr(parent), B, N, int(max_depth), V, float(T), int(seed),
                               int(round_), _ptr(out["len"]), _ptr(out["path"]), _ptr(out["tok"]), _ptr(out["p"]),
                               _ptr(out["q"]), _ptr(ws), ws.numel(), _stream(dev)), "sv_verify_tree")
    _checked(dev, "sv_verify_tree", workspace)
    return out


def sv_verify_tree_pm(tgt, node_tok, parent, max_depth, T, seed=0, round_=0, want_p=True, workspace=None):
    """Point-mass acceptance. tgt [B, N, V]; node_tok, parent [B, N] -> dict(len, path, tok, p)."""
    B, N, V = tgt.shape
    _i32_tensor(node_tok, (B, N), "node_tok")
    _i32_tensor(parent, (B, N), "parent")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(dev, workspace_size(SV_OP_TREE_PM, dt, B, 1, N, V))
    out = dict(len=torch.empty(B, dtype=torch.int32, device=dev),
               path=torch.empty(B, max_depth, dtype=torch.int32, device=dev),
               tok=torch.empty(B, dtype=torch.int32, device=dev),
               p=torch.full((B, N), float("nan"), dtype=torch.float32, device=dev) if want_p else None)
    _check(_lib.sv_verify_tree_pm(_ptr(tgt), dt, _row_stride(tgt, "tgt"), _ptr(node_tok), _ptr(parent), B, N,
                                  int(max_depth), V, float(T), int(seed), int(round_), _ptr(out["len"]),
                                  _ptr(out["path"]), _ptr(out["tok"]), _ptr(out["p"]), _ptr(ws), ws.numel(),
                                  _stream(dev)), "sv_verify_tree_pm")
    _checked(dev, "sv_verify_tree_pm", workspace)
    return out


def sv_fanout_topk(logits, F, F_max, want_vals=True, workspace=None):
    """logits [R, V], F [R] int32 (device) -> (ids [R, F_max], vals [R, F_max] or None)."""
    R, V = logits.shape
    _i32_tensor(F, (R,), "F")
    dt = _dtype_code(logits)
    dev = logits.device
    ws = workspace if workspace is not None else Workspace.get(
        dev, workspace_size(SV_OP_FANOUT, dt, R, 1, 1, V, F_max))
    ids = torch.empty(R, F_max, dtype=torch.int32, device=dev)
    vals = torch.empty(R, F_max, dtype=torch.float32, device=dev) if want_vals else None
    _check(_lib.sv_fanout_topk(_ptr(logits), dt, _row_stride(logits, "logits"), R, V, _ptr(F), int(F_max), _ptr(ids),
                               _ptr(vals), _ptr(ws), ws.numel(), _stream(dev)), "sv_fanout_topk")
    _checked(dev, "sv_fanout_topk", workspace)
    return ids, vals


def sv_cache_hit_test(drf, n, t, F=None, workspace=None):
    """drf [B, K+1, V]; outcome n, t [B] int32 (device); F [K+1] int32 (device) or None
    -> dict(rank [B], hit [B] or None)."""
    B, K1, V = drf.shape
    _i32_tensor(n, (B,), "n")
    _i32_tensor(t, (B,), "t")
    if F is not None:
        _i32_tensor(F, (K1,), "F")
    dt = _dtype_code(drf)
    dev = drf.device
    ws = workspace if workspace is not None else Workspace.get(dev, workspace_size(SV_OP_CACHE, dt, B, 1, K1 - 1, V))
    rank = torch.empty(B, dtype=torch.int32, device=dev)
    hit = torch.empty(B, dtype=torch.int32, device=dev) if F is not None else None
    _check(_lib.sv_cache_hit_test(_ptr(drf), dt, _row_stride(drf, "drf"), B, K1 - 1, V, _ptr(n), _ptr(t), _ptr(F),
                                  _ptr(rank), _ptr(hit), _ptr(ws), ws.numel(), _stream(dev)), "sv_cache_hit_test")
    _checked(dev, "sv_cache_hit_test", workspace)
    return dict(rank=rank, hit=hit)


def sv_presto_score(tgt, drf, node_tok, parent, T, lam, k, b_top, want_scores=True, workspace=None):
    """tgt, drf [B, N, V]; node_tok, parent [B, N] int32; lam [D] float32 (device)
    -> dict(s, S [B, N] float or None, node, tok [B, b_top] int32, score [B, b_top] float)."""
    B, N, V = tgt.shape
    if tuple(drf.shape) != (B, N, V) or drf.dtype != tgt.dtype:
        raise SpecVerifyError(SV_EINVAL, f"drf shape {tuple(drf.shape)} / dtype does not match tgt")
    _i32_tensor(node_tok, (B, N), "node_tok")
    _i32_tensor(parent, (B, N), "parent")
    if lam.dtype != torch.float32 or lam.dim() != 1 or not lam.is_contiguous():
        raise SpecVerifyError(SV_EINVAL, "lam: want a contiguous float32 vector")
    dt = _dtype_code(tgt)
    dev = tgt.device
    ws = workspace if workspace is not None else Workspace.get(
        dev, workspace_size(SV_OP_PRESTO, dt, B, 1, N, V, int(k)))
    f = lambda *shape: torch.empty(*shape, dtype=torch.float32, device=dev)
    out = dict(s=f(B, N) if want_scores else None, S=f(B, N) if want_scores else None,
               node=torch.empty(B, b_top, dtype=torch.int32, device=dev),
               tok=torch.empty(B, b_top, dtype=torch.int32, device=dev), score=f(B, b_top))
    _check(_lib.sv_presto_score(_ptr(tgt), _ptr(drf), dt, _row_stride(tgt, "tgt"), _row_stride(drf, "drf"),
                                _ptr(node_tok), _ptr(parent), B, N, V, float(T), _ptr(lam), lam.numel(), int(k),
                                int(b_top), _ptr(out["s"]), _ptr(out["S"]), _ptr(out["node"]), _ptr(out["tok"]),
                                _ptr(out["score"]), _ptr(ws), ws.numel(), _stream(dev)), "sv_presto_score")
    _checked(dev, "sv_presto_score", workspace)
    return out


def sv_branch_fork(drf, tok, T, eps, k_max, cls=None, workspace=None):
    """drf [B, gamma+1, V] draft rows q_1..q_{gamma+1}; tok [B, gamma]; cls [B] int32 or None
    -> dict(pos, qb, k [B], ids [B, k_max])."""
    B, g1, V = drf.shape
    gamma = g1 - 1
    _i32_tensor(tok, (B, gamma), "tok")
    if cls is not None:
        _i32_tensor(cls, (B,), "cls")
    dt = _dtype_code(drf)
    dev = drf.device
    ws = workspace if workspace is not None else Workspace.get(
        dev, workspace_size(SV_OP_BRANCH, dt, B, 1, gamma, V, int(k_max)))
    out = dict(pos=torch.empty(B, dtype=torch.int32, device=dev), qb=torch.empty(B, dtype=torch.float32, device=dev),
               k=torch.empty(B, dtype=torch.int32, device=dev),
               ids=torch.empty(B, k_max, dtype=torch.int32, device=dev))
    _check(_lib.sv_branch_fork(_ptr(drf), dt, _row_stride(drf, "drf"), _ptr(tok), _ptr(cls), B, gamma, V, float(T),
                               float(eps), int(k_max), _ptr(out["pos"]), _ptr(out["qb"]), _ptr(out["k"]),
                               _ptr(out["ids"]), _ptr(ws), ws.numel(), _stream(dev)), "sv_branch_fork")
    _checked(dev, "sv_branch_fork", workspace)
    return out


def sv_read_probe(buf: torch.Tensor, sink: torch.Tensor, blocks=1024, mode=0, unroll=4, chunk_bytes=1 << 16):
    """Read every 16-byte vector of buf in the statistics kernels' load pattern (a bandwidth probe).  sink: int32
    [>= 3] on the device, zero before the first call (mode 2's counters; the kernel leaves them at zero)."""
    assert sink.numel() >= 3 and sink.element_size() == 4 and sink.device == buf.device
    _check(_lib.sv_read_probe(_ptr(buf), buf.numel() * buf.element_size(), int(blocks), int(mode), int(unroll),
                              int(chunk_bytes), _ptr(sink), _stream(buf.device)), "sv_read_probe")


def sv_timeline_set(buf):
    """Register a device buffer (uint64 [records, 16], zero-filled) for the timeline build's per-block stamps,
    or None to stop.  Raises on a library built without timelines (SV_EUNSUPPORTED)."""
    if buf is None:
        _check(_lib.sv_timeline_set(None, 0), "sv_timeline_set")
        return
    assert buf.dtype == torch.int64 and buf.is_contiguous() and buf.numel() % 16 == 0
    torch.cuda.synchronize(buf.device)
    _check(_lib.sv_timeline_set(_ptr(buf), buf.numel() // 16), "sv_timeline_set")


def sv_geometric_fanout(F0, a_p, r, K, capped_last=False):
    out = (_i32 * (K + 1))()
    s = _lib.sv_geometric_fanout(int(F0), float(a_p), float(r), int(K), int(bool(capped_last)), out)
    if s < 0:
        raise SpecVerifyError(SV_EINVAL, "sv_geometric_fanout")
    return list(out)
