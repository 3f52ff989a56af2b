"""ctypes binding of libwall.so (declared in include/wall.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback of any kind -- if the library is missing or the tensors
are not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwall.so")

WALL_F32, WALL_BF16 = 0, 1
WALL_OK, WALL_ERR_INVALID_ARG, WALL_ERR_UNSUPPORTED, WALL_ERR_LAUNCH, WALL_ERR_SCRATCH = 0, 1, 2, 3, 4
# bytes of the fixed per-GPU scratch of wall_attn_decode_noalloc
WALL_DECODE_SCRATCH_BYTES = 4 << 20

#: every symbol include/wall.h declares
EXPORTS = (
    "wall_status_string", "wall_version",
    "wall_prefix_scan_workspace_size", "wall_prefix_scan", "wall_prefix_append", "wall_stream_append",
    "wall_attn_fwd_workspace_size", "wall_attn_fwd",
    "wall_attn_fwd_prepare", "wall_attn_fwd_prepare_gate", "wall_attn_fwd_run",
    "wall_attn_bwd_workspace_size", "wall_attn_bwd",
    "wall_kv_cache_build", "wall_attn_decode_workspace_size", "wall_attn_decode",
    "wall_attn_decode_noalloc",
)

_lib = None


class WallError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load libwall.so (built by ``python -m channel_decay_softmax_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m channel_decay_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        E = ctypes.c_int
        L.wall_status_string.argtypes = [E]
        L.wall_status_string.restype = ctypes.c_char_p
        L.wall_version.argtypes = []
        L.wall_version.restype = ctypes.c_int
        L.wall_prefix_scan_workspace_size.argtypes = [I, I, I]
        L.wall_prefix_scan_workspace_size.restype = S
        L.wall_prefix_scan.argtypes = [P, E, P, I, I, I, P, I, F, P, S, P]
        L.wall_prefix_append.argtypes = [P, E, I, P, I, P, I, I, I, I, F, P]
        L.wall_stream_append.argtypes = [P, E, P, E, P, P, P, I, I, I, I, I, I, I, I, F, P]
        L.wall_prefix_scan.restype = E
        L.wall_attn_fwd_workspace_size.argtypes = [E, I, I, I, I, I, I, I]
        L.wall_attn_fwd_workspace_size.restype = S
        L.wall_attn_fwd.argtypes = [P, P, P, E, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, I,
                                    P, S, P]
        L.wall_attn_fwd.restype = E
        L.wall_attn_fwd_prepare.argtypes = [P, P, P, E, P, I, I, I, I, I, I, F, P, I, P, S, P]
        L.wall_attn_fwd_prepare.restype = E
        L.wall_attn_fwd_prepare_gate.argtypes = [P, P, P, E, P, E, P, I, I, I, I, I, I, F, P, I, P, S, P]
        L.wall_attn_fwd_prepare_gate.restype = E
        L.wall_attn_fwd_run.argtypes = [P, P, P, E, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, I,
                                        P, S, P]
        L.wall_attn_fwd_run.restype = E
        L.wall_attn_bwd_workspace_size.argtypes = [I, I, I, I, I]
        L.wall_attn_bwd_workspace_size.restype = S
        L.wall_attn_bwd.argtypes = [P, P, P, E, P, P, P, P, P, P, P, P, P, P, P, E, P, I, I, I, I, I, I, F, I,
                                    P, I, I, P, S, P]
        L.wall_attn_bwd.restype = E
        L.wall_kv_cache_build.argtypes = [P, E, P, P, P, I, I, I, I, I, I, I, I, P]
        L.wall_kv_cache_build.restype = E
        L.wall_attn_decode_workspace_size.argtypes = [I, I, I, I]
        L.wall_attn_decode_workspace_size.restype = S
        L.wall_attn_decode.argtypes = [P, P, E, P, I, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, S, P]
        L.wall_attn_decode.restype = E
        L.wall_attn_decode_noalloc.argtypes = [P, P, E, P, I, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
        L.wall_attn_decode_noalloc.restype = E
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().wall_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != WALL_OK:
        raise WallError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return WALL_BF16
    if t.dtype == torch.float32:
        return WALL_F32
    raise TypeError(f"unsupported dtype {t.dtype}: Wall Attention takes bfloat16 or float32")


def _on_gpu(*ts: Optional[torch.Tensor]) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("Wall Attention runs on the GPU only: every tensor must be on a HIP device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dense(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not t.is_contiguous() or t.data_ptr() % 16:
        t = t.contiguous().clone() if t.is_contiguous() else t.contiguous()
    return t


def prefix_scan_workspace_size(B: int, T: int, C: int) -> int:
    return int(lib().wall_prefix_scan_workspace_size(B, T, C))


def attn_fwd_workspace_size(dtype: torch.dtype, B: int, T: int, HQ: int, H: int, K: int, V: int,
                            num_seqs: int = 0) -> int:
    d = WALL_BF16 if dtype == torch.bfloat16 else WALL_F32
    return int(lib().wall_attn_fwd_workspace_size(d, B, T, HQ, H, K, V, num_seqs))


def wall_prefix_scan(x: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                     scale: float = 1.0 / math.log(2.0), out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[b,t,...] = scale * sum of x[b,u,...] from the start of t's sequence to t (float32).

    x is [B, T, ...] bfloat16/float32; cu_seqlens (int32 [N+1], B == 1) packs sequences."""
    dev = _on_gpu(x, cu_seqlens, out, workspace)
    x = _dense(x)
    B, T = x.shape[0], x.shape[1]
    C = x.numel() // (B * T)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.shape != x.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of x's shape (wall_prefix_append "
                         "writes into row slices)")
    nbytes = prefix_scan_workspace_size(B, T, C)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    cu, nseq, _ = _varlen(cu_seqlens, B, T, None)
    _check(lib().wall_prefix_scan(_ptr(x), _dtype(x), _ptr(out), B, T, C, _ptr(cu), nseq,
                                  float(scale), _ptr(workspace), workspace.numel(), _stream(dev)),
           "wall_prefix_scan")
    return out


def _out(t: Optional[torch.Tensor], shape, dtype: torch.dtype, dev: torch.device, what: str) -> torch.Tensor:
    """A caller-provided output (checked: shape, dtype, dense) or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return t


def _rows(t: torch.Tensor, n: int, C: int, what: str) -> int:
    """Batch stride (elements) of a [B, n, ...] tensor whose rows of C values are
    contiguous and consecutive within a batch row."""
    if t.dim() < 2 or t.shape[1] != n or t.numel() != t.shape[0] * n * C:
        raise ValueError(f"{what}: expected [B, {n}, ...] with {C} values per row")
    inner = t[0, 0] if t.dim() > 2 else None
    if t.dim() > 2 and not inner.is_contiguous():
        raise ValueError(f"{what}: each row must be contiguous")
    if n > 1 and t.stride(1) != C:
        raise ValueError(f"{what}: rows must be consecutive")
    return t.stride(0) if t.shape[0] > 1 else n * C


def wall_prefix_append(x: torch.Tensor, prev: Optional[torch.Tensor] = None,
                       scale: float = 1.0 / math.log(2.0), out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[b,t] = prev[b] + scale * (x[b,0] + ... + x[b,t]) (float32): the log2 prefix
    of rows appended to a sequence whose last prefix row is ``prev`` (None starts
    one).  x is [B, n, ...]; prev [B, ...] (e.g. P[:, t0-1]) and out [B, n, ...]
    (e.g. P[:, t0:t0+n]) may be row slices of a larger prefix buffer."""
    dev = _on_gpu(x, prev, out)
    B, n = x.shape[0], x.shape[1]
    C = x.numel() // (B * n)
    x_bs = _rows(x, n, C, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.shape != x.shape:
        raise ValueError("out must be float32 with x's shape")
    out_bs = _rows(out, n, C, "out")
    prev_bs = 0
    if prev is not None:
        if prev.dtype != torch.float32 or prev.numel() != B * C or prev.shape[0] != B:
            raise ValueError("prev must be float32 [B, ...] with one row of x's width")
        if prev.dim() > 1 and not prev[0].is_contiguous():
            raise ValueError("prev: each row must be contiguous")
        prev_bs = prev.stride(0) if B > 1 else C
    _check(lib().wall_prefix_append(_ptr(x), _dtype(x), x_bs, _ptr(prev), prev_bs, _ptr(out), out_bs, B, n, C,
                                    float(scale), _stream(dev)), "wall_prefix_append")
    return out


def wall_stream_append(g: torch.Tensor, k: torch.Tensor, P: torch.Tensor, k_tilde: torch.Tensor,
                       r_cache: torch.Tensor, chunk_size: int = 64, t0: int = 0, t1: Optional[int] = None,
                       scale: float = 1.0 / math.log(2.0)) -> None:
    """One turn of the streaming loop for rows t0 .. t1-1: P of the new rows from
    row t0-1 (in place, as wall_prefix_append) and their cache rows and chunk
    anchors (as build_wall_kv_cache), in one pass.  g, P, k_tilde are
    [B, T_cap, HQ, K] buffers, k [B, T_cap, H, K], r_cache [B, ceil(T_cap/C), HQ, K]."""
    _on_gpu(g, k, P, k_tilde, r_cache)
    B, T_cap, H, K = k.shape
    HQ = g.shape[2]
    NC = -(-T_cap // int(chunk_size))
    for t, shape, what in ((g, (B, T_cap, HQ, K), "g"), (P, (B, T_cap, HQ, K), "P"),
                           (k_tilde, (B, T_cap, HQ, K), "k_tilde"), (r_cache, (B, NC, HQ, K), "r_cache")):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous tensor of shape {shape}")
    if not k.is_contiguous() or P.dtype != torch.float32 or r_cache.dtype != torch.float32:
        raise ValueError("k must be contiguous; P and r_cache are float32")
    if k_tilde.dtype != k.dtype:
        raise TypeError("k_tilde has k's dtype")
    t1 = T_cap if t1 is None else int(t1)
    _check(lib().wall_stream_append(_ptr(g), _dtype(g), _ptr(k), _dtype(k), _ptr(P), _ptr(k_tilde),
                                    _ptr(r_cache), B, T_cap, HQ, H, K, int(chunk_size), int(t0), t1,
                                    float(scale), _stream(g.device)), "wall_stream_append")


def wall_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor,
                  G: Optional[torch.Tensor] = None, sink_bias: Optional[torch.Tensor] = None,
                  scale: Optional[float] = None, window_size: Optional[int] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused causal forward from the log2 prefixes P (and G).  Returns (o, lse)."""
    dev = _on_gpu(q, k, v, P, G, sink_bias, cu_seqlens, out, lse, workspace)
    q, k, v, P, G = _dense(q), _dense(k), _dense(v), _dense(P), _dense(G)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if k.shape != (B, T, H, K) or v.shape != (B, T, H, V) or P.shape != (B, T, HQ, K):
        raise ValueError("shapes must be q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], P [B,T,HQ,K]")
    if not (q.dtype == k.dtype == v.dtype) or P.dtype != torch.float32:
        raise TypeError("q, k, v share one dtype; P is float32")
    if G is not None and (G.shape != (B, T, HQ) or G.dtype != torch.float32):
        raise ValueError("G must be float32 [B,T,HQ]")
    if sink_bias is not None:
        sink_bias = _dense(sink_bias.to(torch.float32))
        if sink_bias.shape != (HQ,):
            raise ValueError("sink_bias must be [HQ]")
    if scale is None:
        scale = K ** -0.5
    cu, nseq, max_seqlen = _varlen(cu_seqlens, B, T, max_seqlen)
    out = _out(out, (B, T, HQ, V), q.dtype, dev, "out")
    if lse is not None or return_lse:
        lse = _out(lse, (B, T, HQ), torch.float32, dev, "lse")
    nbytes = attn_fwd_workspace_size(q.dtype, B, T, HQ, H, K, V, nseq)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().wall_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q), _ptr(P), _ptr(G), _ptr(sink_bias), _ptr(out),
        _ptr(lse), B, T, HQ, H, K, V, float(scale), int(window_size or 0), _ptr(cu), nseq,
        int(max_seqlen or 0), _ptr(workspace), workspace.numel(), _stream(dev)), "wall_attn_fwd")
    return out, lse


def check_cu_seqlens(cu_seqlens: torch.Tensor, B: int, T: int) -> int:
    """Validate packed-sequence offsets on the host (one device-to-host copy).
    Returns the longest sequence length."""
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    cu = cu_seqlens.detach().to("cpu", torch.int64)
    if cu.ndim != 1 or cu.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with at least two entries")
    if int(cu[0]) != 0 or int(cu[-1]) != T or bool((cu[1:] < cu[:-1]).any()):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return int((cu[1:] - cu[:-1]).max())


def _varlen(cu_seqlens: Optional[torch.Tensor], B: int, T: int, max_seqlen: Optional[int]):
    """(cu as dense int32, number of sequences, max_seqlen) after the host checks:
    the C ABI trusts device-side offsets and max_seqlen, so they are checked here."""
    if cu_seqlens is None:
        return None, 0, max_seqlen
    longest = check_cu_seqlens(cu_seqlens, B, T)
    if max_seqlen is None:
        max_seqlen = longest
    elif not longest <= int(max_seqlen) <= T:
        raise ValueError(f"max_seqlen {max_seqlen} must lie between the longest sequence ({longest}) and T ({T})")
    cu = _dense(cu_seqlens.to(torch.int32))
    return cu, cu.numel() - 1, int(max_seqlen)


def wall_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, o: torch.Tensor,
                  lse: torch.Tensor, dout: torch.Tensor, G: Optional[torch.Tensor] = None,
                  sink_bias: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                  window_size: Optional[int] = None, cu_seqlens: Optional[torch.Tensor] = None,
                  max_seqlen: Optional[int] = None, g_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Gradients of wall_attn_fwd for the upstream gradient ``dout`` of o.
    Returns (dq, dk, dv, dg, dg_scalar, dsink); dg / dg_scalar are the gradients
    of the natural-log gates in ``g_dtype`` (default: q's dtype), dg_scalar is
    None without G and dsink (float32) None without sink_bias."""
    dev = _on_gpu(q, k, v, P, o, lse, dout, G, sink_bias, cu_seqlens, workspace)
    q, k, v, P, o, lse, dout, G = (_dense(t) for t in (q, k, v, P, o, lse, dout, G))
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if dout.shape != (B, T, HQ, V) or dout.dtype != q.dtype or o.shape != (B, T, HQ, V):
        raise ValueError("o and dout must be [B,T,HQ,V] in q's dtype")
    if sink_bias is not None:
        sink_bias = _dense(sink_bias.to(torch.float32))
    if scale is None:
        scale = K ** -0.5
    gd = q.dtype if g_dtype is None else g_dtype
    cu, nseq, max_seqlen = _varlen(cu_seqlens, B, T, max_seqlen)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((B, T, HQ, K), dtype=gd, device=dev)
    dgs = None if G is None else torch.empty((B, T, HQ), dtype=gd, device=dev)
    dsink = None if sink_bias is None else torch.empty((HQ,), dtype=torch.float32, device=dev)
    nbytes = int(lib().wall_attn_bwd_workspace_size(B, T, HQ, K, nseq))
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().wall_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q), _ptr(P), _ptr(G), _ptr(sink_bias), _ptr(o), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dgs), WALL_BF16 if gd == torch.bfloat16 else WALL_F32,
        _ptr(dsink), B, T, HQ, H, K, V, float(scale), int(window_size or 0), _ptr(cu), nseq,
        int(max_seqlen or 0), _ptr(workspace), workspace.numel(), _stream(dev)), "wall_attn_bwd")
    return dq, dk, dv, dg, dgs, dsink


def wall_attn_fwd_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                       G: Optional[torch.Tensor] = None, sink_bias: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None, window_size: Optional[int] = None,
                       cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None):
    """The forward from the natural-log gate g: wall_attn_fwd_prepare_gate (P and the
    prepared workspace in one call) then wall_attn_fwd_run.  Returns (o, lse, P)."""
    dev = _on_gpu(q, k, v, g, G, sink_bias, cu_seqlens)
    q, k, v, g, G = _dense(q), _dense(k), _dense(v), _dense(g), _dense(G)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    if k.shape != (B, T, H, K) or v.shape != (B, T, H, V) or g.shape != (B, T, HQ, K):
        raise ValueError("shapes must be q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], g [B,T,HQ,K]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v share one dtype")
    if G is not None and (G.shape != (B, T, HQ) or G.dtype != torch.float32):
        raise ValueError("G must be float32 [B,T,HQ]")
    if sink_bias is not None:
        sink_bias = _dense(sink_bias.to(torch.float32))
        if sink_bias.shape != (HQ,):
            raise ValueError("sink_bias must be [HQ]")
    if scale is None:
        scale = K ** -0.5
    cu, nseq, max_seqlen = _varlen(cu_seqlens, B, T, max_seqlen)
    P = torch.empty((B, T, HQ, K), dtype=torch.float32, device=dev)
    ws = torch.empty(attn_fwd_workspace_size(q.dtype, B, T, HQ, H, K, V, nseq), dtype=torch.uint8, device=dev)
    wall_attn_fwd_prepare_gate(q, k, v, g, P, ws, scale, cu)
    o = torch.empty((B, T, HQ, V), dtype=q.dtype, device=dev)
    lse = torch.empty((B, T, HQ), dtype=torch.float32, device=dev)
    wall_attn_fwd_run(q, k, v, P, ws, o, lse, G, sink_bias, scale, window_size, cu, max_seqlen)
    return o, lse, P


class _WallAttn(torch.autograd.Function):
    """wall_attn with its gradients (q, k, v, g, g_scalar, sink_bias)."""

    @staticmethod
    def forward(ctx, q, k, v, g, g_scalar, sink_bias, scale, window_size, cu_seqlens, max_seqlen):
        G = None if g_scalar is None else wall_prefix_scan(g_scalar, cu_seqlens)
        o, lse, P = wall_attn_fwd_gate(q, k, v, g, G, sink_bias, scale, window_size, cu_seqlens, max_seqlen)
        ctx.save_for_backward(q, k, v, P, G, sink_bias, o, lse, cu_seqlens)
        ctx.set_materialize_grads(False)  # an unused lse gets no gradient tensor
        ctx.opts = (scale, window_size, max_seqlen, g.dtype, g_scalar is not None, sink_bias is not None)
        return o, lse

    @staticmethod
    def backward(ctx, do, dlse):
        q, k, v, P, G, sink_bias, o, lse, cu_seqlens = ctx.saved_tensors
        scale, window_size, max_seqlen, gdt, has_gs, has_sink = ctx.opts
        if dlse is not None:
            raise NotImplementedError("wall_attn: a gradient through lse is not supported")
        if do is None:
            do = torch.zeros_like(o)
        dq, dk, dv, dg, dgs, dsink = wall_attn_bwd(q, k, v, P, o, lse, do.contiguous(), G, sink_bias, scale,
                                                   window_size, cu_seqlens, max_seqlen, g_dtype=gdt)
        return dq, dk, dv, dg, dgs, dsink, None, None, None, None


def wall_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              scale: Optional[float] = None, g_scalar: Optional[torch.Tensor] = None,
              sink_bias: Optional[torch.Tensor] = None, window_size: Optional[int] = None,
              cu_seqlens: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Wall Attention forward, with the README's signature (wall_attn usage,
    "Training / prefill"): q [B,T,HQ,K], k [B,T,H,K], v [B,T,H,V], g [B,T,HQ,K]
    natural-log decay (g = 0 is softmax attention), scale default K**-0.5;
    optional g_scalar [B,T,HQ], sink_bias [HQ], window_size, cu_seqlens (B == 1).
    Runs wall_prefix_scan (g -> P, g_scalar -> G) and wall_attn_fwd on the
    current stream; when an input requires grad, o.backward() runs
    wall_attn_bwd.  Returns o [B,T,HQ,V] (and lse [B,T,HQ] if asked)."""
    _on_gpu(q, k, v, g, g_scalar, sink_bias, cu_seqlens)
    B, T = q.shape[:2]
    max_seqlen = None
    if cu_seqlens is not None:
        max_seqlen = check_cu_seqlens(cu_seqlens, B, T)
    if scale is None:
        scale = q.shape[3] ** -0.5
    if sink_bias is not None and sink_bias.dtype != torch.float32:
        sink_bias = sink_bias.float()
    o, lse = _WallAttn.apply(q, k, v, g, g_scalar, sink_bias, scale, window_size, cu_seqlens, max_seqlen)
    return (o, lse) if return_lse else o


def wall_attn_fwd_prepare(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor,
                          workspace: torch.Tensor, scale: Optional[float] = None,
                          cu_seqlens: Optional[torch.Tensor] = None) -> None:
    """Stage 1 of wall_attn_fwd: build the anchored key and query tiles and the value
    tiles in ``workspace``.  All tensors must already be dense and on one device (no
    copies are made here)."""
    dev = _on_gpu(q, k, v, P, workspace, cu_seqlens)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _check(lib().wall_attn_fwd_prepare(_ptr(q), _ptr(k), _ptr(v), _dtype(k), _ptr(P), B, T, HQ, H, K, V,
                                       float(K ** -0.5 if scale is None else scale), _ptr(cu_seqlens), nseq,
                                       _ptr(workspace), workspace.numel(), _stream(dev)), "wall_attn_fwd_prepare")


def wall_attn_fwd_prepare_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                               P: torch.Tensor, workspace: torch.Tensor, scale: Optional[float] = None,
                               cu_seqlens: Optional[torch.Tensor] = None) -> None:
    """Stage 1 of the forward from the gate: writes P = cumsum(g) / ln 2 (float32,
    [B,T,HQ,K]) and prepares ``workspace`` from it (one combined pass for B
    sequences of T rows with T a multiple of 128 and bf16 inputs).  All tensors
    must already be dense and on one device (no copies are made here)."""
    dev = _on_gpu(q, k, v, g, P, workspace, cu_seqlens)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _check(lib().wall_attn_fwd_prepare_gate(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q), _ptr(g), _dtype(g), _ptr(P), B, T, HQ, H, K, V,
        float(K ** -0.5 if scale is None else scale), _ptr(cu_seqlens), nseq, _ptr(workspace), workspace.numel(),
        _stream(dev)), "wall_attn_fwd_prepare_gate")


def wall_attn_fwd_run(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor,
                      workspace: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                      G: Optional[torch.Tensor] = None, sink_bias: Optional[torch.Tensor] = None,
                      scale: Optional[float] = None, window_size: Optional[int] = None,
                      cu_seqlens: Optional[torch.Tensor] = None,
                      max_seqlen: Optional[int] = None) -> None:
    """Stage 2 of wall_attn_fwd: the fused kernel, reading the prepared ``workspace``
    and the raw k, v of the prepare call.  All tensors must already be dense and on
    one device (no copies are made here)."""
    dev = _on_gpu(q, k, v, P, workspace, out, lse, G, sink_bias, cu_seqlens)
    B, T, HQ, K = q.shape
    H, V = k.shape[2], v.shape[3]
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _check(lib().wall_attn_fwd_run(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q), _ptr(P), _ptr(G), _ptr(sink_bias), _ptr(out), _ptr(lse),
        B, T, HQ, H, K, V, float(K ** -0.5 if scale is None else scale), int(window_size or 0),
        _ptr(cu_seqlens), nseq, int(max_seqlen or 0), _ptr(workspace), workspace.numel(),
        _stream(dev)), "wall_attn_fwd_run")


# --------------------------------------------------------------------------- decode


def build_wall_kv_cache(k: torch.Tensor, P: torch.Tensor, chunk_size: int = 64,
                        k_tilde: Optional[torch.Tensor] = None, r_cache: Optional[torch.Tensor] = None,
                        t0: int = 0, t1: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The README's build_wall_kv_cache: k [B,T_cap,H,K] (bfloat16/float32) and the
    log2 prefix P [B,T_cap,HQ,K] -> k_tilde [B,T_cap,HQ,K] (decay folded in against
    per-chunk anchors) and r_cache [B,ceil(T_cap/chunk_size),HQ,K] float32.
    Rows t0 .. t1-1 are written (default all); pass the cache tensors to append."""
    dev = _on_gpu(k, P, k_tilde, r_cache)
    k, P = _dense(k), _dense(P)
    B, T, H, K = k.shape
    HQ = P.shape[2]
    if P.shape != (B, T, HQ, K) or P.dtype != torch.float32:
        raise ValueError("P must be float32 [B,T,HQ,K] matching k [B,T,H,K]")
    NC = -(-T // int(chunk_size))
    if k_tilde is None:
        k_tilde = torch.empty((B, T, HQ, K), dtype=k.dtype, device=dev)
    if r_cache is None:
        r_cache = torch.empty((B, NC, HQ, K), dtype=torch.float32, device=dev)
    if k_tilde.shape != (B, T, HQ, K) or r_cache.shape != (B, NC, HQ, K):
        raise ValueError("k_tilde must be [B,T,HQ,K] and r_cache [B,ceil(T/C),HQ,K]")
    if not (k_tilde.is_contiguous() and r_cache.is_contiguous()):
        raise ValueError("k_tilde and r_cache must be contiguous")
    if k_tilde.dtype != k.dtype or r_cache.dtype != torch.float32:
        raise TypeError("k_tilde has k's dtype and r_cache is float32")
    t1 = T if t1 is None else int(t1)
    _check(lib().wall_kv_cache_build(_ptr(k), _dtype(k), _ptr(P), _ptr(k_tilde), _ptr(r_cache), B, T,
                                      HQ, H, K, int(chunk_size), int(t0), t1, _stream(dev)),
           "wall_kv_cache_build")
    return k_tilde, r_cache


def decode_workspace_size(B: int, T: int, HQ: int, V: int) -> int:
    return int(lib().wall_attn_decode_workspace_size(B, T, HQ, V))


def wall_attn_decode(q: torch.Tensor, v: torch.Tensor, p_curr: torch.Tensor, k_tilde: torch.Tensor,
                     r_cache: torch.Tensor, sink_bias: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, cache_chunk_size: int = 64,
                     seq_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     no_alloc: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """The README's wall_attn_decode: q and p_curr [B,1,HQ,K] (the newest token and
    its log2 prefix), v [B,T_cap,H,V], the cache of build_wall_kv_cache; attends to
    cached rows 0 .. seq_len-1 (default T_cap).  p_curr may be a row of a larger
    prefix buffer (P[:, t:t+1]).  Returns (o [B,1,HQ,V], lse [B,1,HQ]).  With
    no_alloc (and out and lse given) the call allocates nothing: it goes through
    wall_attn_decode_noalloc, whose split partials live in the library's fixed
    per-GPU scratch."""
    dev = _on_gpu(q, v, p_curr, k_tilde, r_cache, sink_bias, out, lse, workspace)
    q, v = _dense(q), _dense(v)
    if not (p_curr.dim() == 4 and p_curr[0, 0].is_contiguous() and p_curr.stride(0) % 4 == 0):
        p_curr = _dense(p_curr)
    pc_bs = p_curr.stride(0) if p_curr.shape[0] > 1 else 0
    B, _, HQ, K = q.shape
    T_cap, H, V = v.shape[1], v.shape[2], v.shape[3]
    T = T_cap if seq_len is None else int(seq_len)
    if q.shape[1] != 1 or p_curr.shape != (B, 1, HQ, K) or p_curr.dtype != torch.float32:
        raise ValueError("q and p_curr must be [B,1,HQ,K] (p_curr float32)")
    if k_tilde.shape != (B, T_cap, HQ, K) or not k_tilde.is_contiguous() or not r_cache.is_contiguous():
        raise ValueError("k_tilde must be a contiguous [B,T_cap,HQ,K] cache")
    if not (q.dtype == v.dtype == k_tilde.dtype) or r_cache.dtype != torch.float32:
        raise TypeError("q, v and k_tilde share one dtype; r_cache is float32")
    if sink_bias is not None:
        sink_bias = _dense(sink_bias.to(torch.float32))
    if scale is None:
        scale = K ** -0.5
    out = _out(out, (B, 1, HQ, V), q.dtype, dev, "out")
    lse = _out(lse, (B, 1, HQ), torch.float32, dev, "lse")
    if no_alloc:
        if workspace is not None:
            raise ValueError("no_alloc takes no workspace")
        _check(lib().wall_attn_decode_noalloc(
            _ptr(q), _ptr(v), _dtype(q), _ptr(p_curr), pc_bs, _ptr(k_tilde), _ptr(r_cache), _ptr(sink_bias),
            _ptr(out), _ptr(lse), B, T, T_cap, HQ, H, K, V, int(cache_chunk_size), float(scale), _stream(dev)),
            "wall_attn_decode_noalloc")
        return out, lse
    if workspace is None:
        workspace = torch.empty(decode_workspace_size(B, T, HQ, V), dtype=torch.uint8, device=dev)
    _check(lib().wall_attn_decode(
        _ptr(q), _ptr(v), _dtype(q), _ptr(p_curr), pc_bs, _ptr(k_tilde), _ptr(r_cache), _ptr(sink_bias),
        _ptr(out), _ptr(lse), B, T, T_cap, HQ, H, K, V, int(cache_chunk_size), float(scale),
        _ptr(workspace), workspace.numel(), _stream(dev)), "wall_attn_decode")
    return out, lse
