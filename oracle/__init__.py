"""fp64 CPU oracle for the Wall Attention forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The product path
(``channel_decay_softmax_amd``) never imports this package and the two share
no code.

``wall_oracle.c`` holds the arithmetic (the product form of the Wall Attention
blog's "Definition: Wall Attention" section, with the README's optional
arguments, and the README's decode cache and cached decode); this module only
builds it with gcc, loads it with ctypes and converts arrays.  Every function here takes and returns float64 numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wall_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

__all__ = ["build", "wall_attn_oracle", "wall_attn_bwd_oracle", "prefix_scan_oracle", "kv_cache_oracle",
           "decode_oracle", "num_threads"]


def build(force: bool = True) -> str:
    """Compile wall_oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
             "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    """Load one build of wall_oracle.c and declare its entry points."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.wall_oracle_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                    ctypes.c_double, I, P, I, P, I]
    lib.wall_oracle_fwd.restype = ctypes.c_int
    lib.wall_oracle_prefix_scan.argtypes = [P, P, I, I, I, P, I, ctypes.c_double]
    lib.wall_oracle_prefix_scan.restype = ctypes.c_int
    lib.wall_oracle_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                    ctypes.c_double, I, P, I]
    lib.wall_oracle_bwd.restype = ctypes.c_int
    lib.wall_oracle_kv_cache.argtypes = [P, P, P, P, I, I, I, I, I, I]
    lib.wall_oracle_kv_cache.restype = ctypes.c_int
    lib.wall_oracle_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_double]
    lib.wall_oracle_decode.restype = ctypes.c_int
    lib.wall_oracle_num_threads.argtypes = []
    lib.wall_oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(_LIB)
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all visible cores)."""
    return int(_load().wall_oracle_num_threads())


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor on the CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def wall_attn_oracle(q, k, v, g, scale: Optional[float] = None, g_scalar=None,
                     sink_bias=None, window_size: Optional[int] = None, cu_seqlens=None,
                     rows: Optional[Sequence[int]] = None):
    """Product-form Wall Attention forward in fp64.

    Shapes follow the README: q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V],
    g [B,T,HQ,K] (natural-log gate), g_scalar [B,T,HQ], sink_bias [HQ],
    cu_seqlens [N+1] (B == 1).  ``rows`` optionally restricts the work to a
    set of flat token ids ``b*T + t``; the other rows of ``o`` / ``lse`` are
    left as NaN.  Returns ``(o [B,T,HQ,V], lse [B,T,HQ])``.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    gs, sk = _f64(g_scalar), _f64(sink_bias)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    assert k.shape == (B, T, H, K) and v.shape == (B, T, H, V) and g.shape == (B, T, HQ, K)
    if gs is not None:
        assert gs.shape == (B, T, HQ)
    if sk is not None:
        assert sk.shape == (HQ,)
    if scale is None:
        scale = K ** -0.5
    cu = None
    nseq = 0
    if cu_seqlens is not None:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        nseq = cu.shape[0] - 1
    rw = None
    if rows is not None:
        rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.full((B, T, HQ, V), np.nan)
    lse = np.full((B, T, HQ), np.nan)
    rc = _load().wall_oracle_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gs), _ptr(sk), _ptr(o), _ptr(lse),
        B, T, HQ, H, K, V, float(scale), int(window_size or 0), _ptr(cu), nseq,
        _ptr(rw), 0 if rw is None else rw.shape[0])
    if rc != 0:
        raise ValueError(f"wall_oracle_fwd rejected its arguments (code {rc})")
    return o, lse


def wall_attn_bwd_oracle(q, k, v, g, do, scale: Optional[float] = None, g_scalar=None, sink_bias=None,
                         window_size: Optional[int] = None, cu_seqlens=None):
    """Gradients of the product-form forward in fp64 for an upstream gradient
    ``do`` [B,T,HQ,V] of o.  Returns ``(dq, dk, dv, dg, dg_scalar, dsink)``;
    the last two are None when g_scalar / sink_bias is."""
    q, k, v, g, do = _f64(q), _f64(k), _f64(v), _f64(g), _f64(do)
    gs, sk = _f64(g_scalar), _f64(sink_bias)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    assert k.shape == (B, T, H, K) and v.shape == (B, T, H, V) and g.shape == (B, T, HQ, K)
    assert do.shape == (B, T, HQ, V)
    if scale is None:
        scale = K ** -0.5
    cu = None
    nseq = 0
    if cu_seqlens is not None:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        nseq = cu.shape[0] - 1
    dq, dk, dv, dg = np.empty_like(q), np.empty_like(k), np.empty_like(v), np.empty_like(g)
    dgs = None if gs is None else np.empty_like(gs)
    dsk = None if sk is None else np.empty_like(sk)
    rc = _load().wall_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gs), _ptr(sk), _ptr(do), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dgs), _ptr(dsk), B, T, HQ, H, K, V,
                                 float(scale), int(window_size or 0), _ptr(cu), nseq)
    if rc != 0:
        raise ValueError(f"wall_oracle_bwd rejected its arguments (code {rc})")
    return dq, dk, dv, dg, dgs, dsk


def prefix_scan_oracle(x, cu_seqlens=None, scale: float = 1.0 / np.log(2.0)):
    """Per-sequence prefix sum along T times ``scale`` (fp64); x is [B, T, ...]."""
    x = _f64(x)
    B, T = x.shape[:2]
    C = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    cu = None
    nseq = 0
    if cu_seqlens is not None:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        nseq = cu.shape[0] - 1
    out = np.empty_like(x)
    rc = _load().wall_oracle_prefix_scan(_ptr(x), _ptr(out), B, T, C, _ptr(cu), nseq, float(scale))
    if rc != 0:
        raise ValueError(f"wall_oracle_prefix_scan rejected its arguments (code {rc})")
    return out


def kv_cache_oracle(k, P, chunk_size: int = 64):
    """The README's decode cache in fp64: ``k_tilde [B,T,HQ,K]`` (keys with the
    decay folded in against per-chunk anchors) and ``r_cache [B,ceil(T/C),HQ,K]``
    (the anchors: floor of P at each chunk's first row, moved to a later row's
    floored P whenever that row lies more than 64 log2 units below it).  k is
    [B,T,H,K], P the log2 prefix [B,T,HQ,K]."""
    k, P = _f64(k), _f64(P)
    B, T, H, K = k.shape
    HQ = P.shape[2]
    assert P.shape == (B, T, HQ, K)
    C = int(chunk_size)
    NC = (T + C - 1) // C
    kt = np.empty((B, T, HQ, K))
    r = np.empty((B, NC, HQ, K))
    rc = _load().wall_oracle_kv_cache(_ptr(k), _ptr(P), _ptr(kt), _ptr(r), B, T, HQ, H, K, C)
    if rc != 0:
        raise ValueError(f"wall_oracle_kv_cache rejected its arguments (code {rc})")
    return kt, r


def decode_oracle(q, v, p_curr, k_tilde, r_cache, chunk_size: int = 64, sink_bias=None,
                  scale: Optional[float] = None):
    """The README's cached decode in fp64: q and p_curr [B,1,HQ,K] (the current
    query and its log2 prefix), v [B,T,H,V], the cache of kv_cache_oracle.
    Returns ``(o [B,1,HQ,V], lse [B,1,HQ])``."""
    q, v, pc = _f64(q), _f64(v), _f64(p_curr)
    kt, r, sk = _f64(k_tilde), _f64(r_cache), _f64(sink_bias)
    B, _, HQ, K = q.shape
    T, H, V = v.shape[1], v.shape[2], v.shape[3]
    C = int(chunk_size)
    assert q.shape == (B, 1, HQ, K) and pc.shape == (B, 1, HQ, K)
    assert kt.shape == (B, T, HQ, K) and r.shape == (B, (T + C - 1) // C, HQ, K)
    if sk is not None:
        assert sk.shape == (HQ,)
    if scale is None:
        scale = K ** -0.5
    o = np.empty((B, 1, HQ, V))
    lse = np.empty((B, 1, HQ))
    rc = _load().wall_oracle_decode(_ptr(q), _ptr(v), _ptr(pc), _ptr(kt), _ptr(r), _ptr(sk), _ptr(o),
                                    _ptr(lse), B, T, HQ, H, K, V, C, float(scale))
    if rc != 0:
        raise ValueError(f"wall_oracle_decode rejected its arguments (code {rc})")
    return o, lse
