"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/wall.h declares, and rejects invalid arguments before any HIP call
(so these calls never touch a device)."""

import ctypes
import os
import re

import pytest
import torch

import channel_decay_softmax_amd as wall
from channel_decay_softmax_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wall.h")

OK, INVALID, UNSUPPORTED = wall.WALL_OK, wall.WALL_ERR_INVALID_ARG, wall.WALL_ERR_UNSUPPORTED
FAKE = 1 << 20  # a non-null, 256-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wall_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    L = wall.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.wall_version() == 100
    assert wall.status_string(OK) == "WALL_OK"
    assert wall.status_string(INVALID) == "WALL_ERR_INVALID_ARG"
    assert wall.status_string(UNSUPPORTED) == "WALL_ERR_UNSUPPORTED"
    assert wall.status_string(wall.WALL_ERR_LAUNCH) == "WALL_ERR_LAUNCH"
    assert wall.status_string(99) == "WALL_ERR_UNKNOWN"


def P(x):
    return None if x is None else ctypes.c_void_p(x)


def scan(x=FAKE, dtype=B.WALL_BF16, out=FAKE * 2, b=1, t=64, c=8, cu=None, nseq=0, ws=FAKE * 3,
         wsb=None):
    L = wall.lib()
    if wsb is None:
        wsb = L.wall_prefix_scan_workspace_size(b, t, c)
    return L.wall_prefix_scan(P(x), dtype, P(out), b, t, c, P(cu), nseq, 1.4426950408889634,
                              P(ws), wsb, None)


def append(x=FAKE, dtype=B.WALL_BF16, xbs=None, prev=None, pbs=0, out=FAKE * 2, obs=None, b=2, n=3, c=8):
    xbs = n * c if xbs is None else xbs
    obs = n * c if obs is None else obs
    return wall.lib().wall_prefix_append(P(x), dtype, xbs, P(prev), pbs, P(out), obs, b, n, c,
                                         1.4426950408889634, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(out=None), dict(b=0), dict(n=0), dict(c=0), dict(xbs=23), dict(obs=23),
    dict(prev=FAKE * 3, pbs=7), dict(x=FAKE + 1), dict(dtype=B.WALL_F32, x=FAKE + 2),
    dict(out=FAKE * 2 + 2), dict(prev=FAKE * 3 + 2, pbs=8), dict(out=FAKE + 8),
])
def test_prefix_append_rejects_invalid_arguments(kw):
    assert append(**kw) == INVALID


def test_prefix_append_rejects_unsupported_dtype():
    assert append(dtype=7) == UNSUPPORTED


def stream(g=FAKE, gdt=B.WALL_BF16, k=FAKE, dtype=B.WALL_BF16, Pp=FAKE, kt=FAKE, r=FAKE, b=2, tcap=256, hq=4,
           h=2, kk=128, c=64, t0=10, t1=11):
    return wall.lib().wall_stream_append(P(g), gdt, P(k), dtype, P(Pp), P(kt), P(r), b, tcap, hq, h, kk, c, t0, t1,
                                         1.4426950408889634, None)


@pytest.mark.parametrize("kw", [
    dict(g=None), dict(k=None), dict(Pp=None), dict(kt=None), dict(r=None), dict(b=0), dict(tcap=0), dict(hq=0),
    dict(hq=6, h=4), dict(t0=-1), dict(t1=10), dict(t1=257), dict(g=FAKE + 2), dict(r=FAKE + 4),
])
def test_stream_append_rejects_invalid_arguments(kw):
    assert stream(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(kk=96), dict(c=32), dict(dtype=5), dict(gdt=3)])
def test_stream_append_rejects_unsupported_shapes(kw):
    assert stream(**kw) == UNSUPPORTED


def fwd(q=FAKE, k=FAKE, v=FAKE, dtype=B.WALL_BF16, Pp=FAKE, G=None, sink=None, o=FAKE, lse=None,
        b=1, t=256, hq=4, h=2, kk=128, vv=128, window=0, cu=None, nseq=0, maxlen=0, ws=FAKE,
        wsb=None):
    L = wall.lib()
    if wsb is None:
        wsb = L.wall_attn_fwd_workspace_size(dtype if dtype in (0, 1) else 1, b, t, hq, h, kk, vv,
                                             nseq)
    return L.wall_attn_fwd(P(q), P(k), P(v), dtype, P(Pp), P(G), P(sink), P(o), P(lse), b, t, hq,
                           h, kk, vv, 0.088, window, P(cu), nseq, maxlen, P(ws), wsb, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(out=None), dict(ws=None), dict(b=0), dict(t=0), dict(c=0),
    dict(cu=FAKE, nseq=2, b=2), dict(cu=FAKE, nseq=0), dict(x=FAKE + 8), dict(out=FAKE + 4),
    dict(ws=FAKE + 128), dict(wsb=16), dict(out=FAKE),
])
def test_prefix_scan_rejects_invalid_arguments(kw):
    assert scan(**kw) == INVALID


def test_prefix_scan_rejects_unsupported_dtype():
    assert scan(dtype=7) == UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(Pp=None), dict(o=None), dict(ws=None),
    dict(b=0), dict(t=0), dict(hq=0), dict(h=0), dict(hq=6, h=4),
    dict(cu=FAKE, nseq=2, b=2, maxlen=128), dict(cu=FAKE, nseq=0, maxlen=128),
    dict(cu=FAKE, nseq=2, maxlen=0), dict(cu=FAKE, nseq=2, maxlen=1000),
    dict(q=FAKE + 2), dict(G=FAKE + 4), dict(sink=FAKE + 8), dict(lse=FAKE + 12),
    dict(ws=FAKE + 16), dict(wsb=1024), dict(cu=FAKE + 2, nseq=2, maxlen=128),
])
def test_fwd_rejects_invalid_arguments(kw):
    assert fwd(**kw) == INVALID


def test_fwd_run_needs_the_raw_keys_and_values():
    L = wall.lib()
    wsb = L.wall_attn_fwd_workspace_size(1, 1, 256, 4, 2, 128, 128, 0)
    for k, v in ((None, FAKE), (FAKE, None), (FAKE + 2, FAKE), (FAKE, FAKE + 4)):
        assert L.wall_attn_fwd_run(P(FAKE), P(k), P(v), 1, P(FAKE), None, None, P(FAKE), None, 1, 256, 4, 2,
                                   128, 128, 0.088, 0, None, 0, 0, P(FAKE), wsb, None) == INVALID


@pytest.mark.parametrize("kw", [dict(kk=96), dict(vv=32), dict(kk=256), dict(dtype=5)])
def test_fwd_rejects_unsupported_shapes(kw):
    assert fwd(**kw) == UNSUPPORTED


def cache(k=FAKE, dtype=B.WALL_BF16, Pp=FAKE, kt=FAKE, r=FAKE, b=2, tcap=300, hq=4, h=2, kk=128, c=64,
          t0=0, t1=300):
    return wall.lib().wall_kv_cache_build(P(k), dtype, P(Pp), P(kt), P(r), b, tcap, hq, h, kk, c, t0, t1,
                                          None)


def decode(q=FAKE, v=FAKE, dtype=B.WALL_BF16, pc=FAKE, pcs=0, kt=FAKE, r=FAKE, sink=None, o=FAKE, lse=None,
           b=2, t=300, tcap=512, hq=4, h=2, kk=128, vv=128, c=64, ws=FAKE, wsb=None):
    L = wall.lib()
    if wsb is None:
        wsb = L.wall_attn_decode_workspace_size(b, t, hq, vv)
    return L.wall_attn_decode(P(q), P(v), dtype, P(pc), pcs, P(kt), P(r), P(sink), P(o), P(lse), b, t, tcap,
                              hq, h, kk, vv, c, 0.088, P(ws), wsb, None)


@pytest.mark.parametrize("kw", [
    dict(k=None), dict(Pp=None), dict(kt=None), dict(r=None), dict(b=0), dict(tcap=0), dict(hq=0),
    dict(h=0), dict(hq=6, h=4), dict(c=0), dict(t0=-1), dict(t0=300), dict(t0=10, t1=10),
    dict(t1=301), dict(k=FAKE + 2), dict(Pp=FAKE + 4), dict(kt=FAKE + 8), dict(r=FAKE + 12),
])
def test_kv_cache_rejects_invalid_arguments(kw):
    assert cache(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(kk=96), dict(c=32), dict(c=100), dict(dtype=5)])
def test_kv_cache_rejects_unsupported_shapes(kw):
    assert cache(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(v=None), dict(pc=None), dict(kt=None), dict(r=None), dict(o=None), dict(ws=None),
    dict(b=0), dict(t=0), dict(tcap=0), dict(hq=0), dict(h=0), dict(hq=6, h=4), dict(t=513),
    dict(b=8192, hq=16, h=4), dict(q=FAKE + 2), dict(sink=FAKE + 4), dict(lse=FAKE + 8),
    dict(ws=FAKE + 16), dict(wsb=64), dict(pcs=100), dict(pcs=514),
])
def test_decode_rejects_invalid_arguments(kw):
    assert decode(**kw) == INVALID


def gate_prep(q=FAKE, k=FAKE, v=FAKE, dtype=B.WALL_BF16, g=FAKE * 2, gdt=B.WALL_BF16, Pw=FAKE * 3, b=1, t=256,
              hq=4, h=2, kk=128, vv=128, cu=None, nseq=0, ws=FAKE * 4, wsb=None):
    L = wall.lib()
    if wsb is None:
        wsb = L.wall_attn_fwd_workspace_size(dtype if dtype in (0, 1) else 1, b, t, hq, h, kk, vv, nseq)
    return L.wall_attn_fwd_prepare_gate(P(q), P(k), P(v), dtype, P(g), gdt, P(Pw), b, t, hq, h, kk, vv, 0.088,
                                        P(cu), nseq, P(ws), wsb, None)


@pytest.mark.parametrize("kw", [dict(g=None), dict(Pw=None), dict(q=None), dict(Pw=FAKE * 2), dict(g=FAKE * 2 + 4),
                                dict(wsb=64), dict(hq=6, h=4), dict(b=2, cu=FAKE * 5, nseq=2)])
def test_prepare_gate_rejects_invalid_arguments(kw):
    assert gate_prep(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(gdt=5), dict(kk=96), dict(dtype=5)])
def test_prepare_gate_rejects_unsupported(kw):
    assert gate_prep(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(kk=96), dict(vv=32), dict(c=32), dict(c=0 + 96), dict(dtype=5)])
def test_decode_rejects_unsupported_shapes(kw):
    assert decode(**kw) == UNSUPPORTED


def decode_noalloc(q=FAKE, v=FAKE, dtype=B.WALL_BF16, pc=FAKE, pcs=0, kt=FAKE, r=FAKE, sink=None, o=FAKE,
                   lse=None, b=2, t=300, tcap=512, hq=4, h=2, kk=128, vv=128, c=64):
    return wall.lib().wall_attn_decode_noalloc(P(q), P(v), dtype, P(pc), pcs, P(kt), P(r), P(sink), P(o),
                                               P(lse), b, t, tcap, hq, h, kk, vv, c, 0.088, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(v=None), dict(pc=None), dict(kt=None), dict(r=None), dict(o=None),
    dict(b=0), dict(t=0), dict(tcap=0), dict(hq=0), dict(h=0), dict(hq=6, h=4), dict(t=513),
    dict(b=8192, hq=16, h=4), dict(q=FAKE + 2), dict(sink=FAKE + 4), dict(lse=FAKE + 8), dict(pcs=100),
])
def test_decode_noalloc_rejects_invalid_arguments(kw):
    assert decode_noalloc(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(kk=96), dict(vv=32), dict(c=32), dict(dtype=5)])
def test_decode_noalloc_rejects_unsupported_shapes(kw):
    assert decode_noalloc(**kw) == UNSUPPORTED


@pytest.mark.parametrize("b,hq,vv", [(512, 16, 128), (8192, 2, 64), (64, 128, 128)])
def test_decode_noalloc_rejects_what_outgrows_its_scratch(b, hq, vv):
    """A call whose split partials would not fit the fixed scratch is refused
    before any device work, with its own status."""
    L = wall.lib()
    assert L.wall_attn_decode_workspace_size(b, 64, hq, vv) > wall.WALL_DECODE_SCRATCH_BYTES
    assert decode_noalloc(b=b, t=64, tcap=64, hq=hq, h=1, vv=vv) == wall.WALL_ERR_SCRATCH
    assert wall.status_string(wall.WALL_ERR_SCRATCH) == "WALL_ERR_SCRATCH"


def test_decode_noalloc_scratch_covers_the_decode_workload():
    """The decode workload (16 sequences, 16 query heads, V = 128) fits at any
    cache length."""
    L = wall.lib()
    for t in (1, 64, 8192, 1 << 20):
        assert L.wall_attn_decode_workspace_size(16, t, 16, 128) <= wall.WALL_DECODE_SCRATCH_BYTES


def bwd(q=FAKE, k=FAKE, v=FAKE, dtype=B.WALL_BF16, Pp=FAKE, G=None, sink=None, o=FAKE, lse=FAKE, do=FAKE,
        dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dgs=None, gdt=B.WALL_BF16, dsink=None, b=1, t=256, hq=4, h=2,
        kk=128, vv=128, window=0, cu=None, nseq=0, maxlen=0, ws=FAKE, wsb=None):
    L = wall.lib()
    if wsb is None:
        wsb = L.wall_attn_bwd_workspace_size(b, t, hq, kk, nseq)
    return L.wall_attn_bwd(P(q), P(k), P(v), dtype, P(Pp), P(G), P(sink), P(o), P(lse), P(do), P(dq), P(dk),
                           P(dv), P(dg), P(dgs), gdt, P(dsink), b, t, hq, h, kk, vv, 0.088, window, P(cu), nseq,
                           maxlen, P(ws), wsb, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(Pp=None), dict(o=None), dict(lse=None), dict(do=None),
    dict(dq=None), dict(dk=None), dict(dv=None), dict(dg=None), dict(ws=None), dict(G=FAKE),
    dict(sink=FAKE), dict(b=0), dict(t=0), dict(hq=6, h=4), dict(cu=FAKE, nseq=2, b=2, maxlen=128),
    dict(cu=FAKE, nseq=2, maxlen=0), dict(q=FAKE + 2), dict(dg=FAKE + 4), dict(ws=FAKE + 16), dict(wsb=1024),
])
def test_bwd_rejects_invalid_arguments(kw):
    assert bwd(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(kk=96), dict(vv=32), dict(dtype=5), dict(gdt=3),
                                # 64 heads x 2^19 sequences x ceil(2^19 / 128) blocks: past a 32-bit grid
                                dict(t=1 << 20, hq=64, h=64, cu=FAKE, nseq=1 << 19, maxlen=1 << 19)])
def test_bwd_rejects_unsupported_shapes(kw):
    assert bwd(**kw) == UNSUPPORTED


def test_workspace_sizes():
    L = wall.lib()
    assert L.wall_prefix_scan_workspace_size(0, 10, 10) == 0
    a = L.wall_prefix_scan_workspace_size(1, 8192, 2048)
    assert a >= 2 * 64 * 2048 * 4 and a % 256 == 0
    assert L.wall_attn_fwd_workspace_size(7, 1, 10, 1, 1, 64, 64, 0) == 0
    b16 = L.wall_attn_fwd_workspace_size(1, 1, 8192, 16, 4, 128, 128, 0)
    f32 = L.wall_attn_fwd_workspace_size(0, 1, 8192, 16, 4, 128, 128, 0)
    # bf16: key cache per query head + value tiles per kv head, 65 tiles bound;
    # float32 reads the raw tensors and keeps the sequence table and, for
    # wall_attn_fwd_prepare_gate, a prefix-scan workspace
    assert b16 >= 65 * 128 * (16 * 128 + 4 * 128) * 2
    assert a <= f32 <= a + 256
    assert L.wall_attn_fwd_workspace_size(1, 1, 1000, 2, 1, 64, 64, 9) > \
        L.wall_attn_fwd_workspace_size(1, 1, 1000, 2, 1, 64, 64, 1)


def test_python_wrappers_refuse_cpu_tensors():
    x = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU only"):
        wall.wall_prefix_scan(x)
    with pytest.raises(ValueError, match="GPU only"):
        wall.wall_prefix_append(x)
    with pytest.raises(ValueError, match="GPU only"):
        wall.wall_attn(x, x[:, :, :1], x[:, :, :1], x)


def test_cu_seqlens_host_checks():
    T = 10
    assert wall.check_cu_seqlens(torch.tensor([0, 3, 3, 10], dtype=torch.int32), 1, T) == 7
    for bad in ([1, 10], [0, 5, 4, 10], [0, 9], [0]):
        with pytest.raises(ValueError):
            wall.check_cu_seqlens(torch.tensor(bad, dtype=torch.int32), 1, T)
    with pytest.raises(ValueError):
        wall.check_cu_seqlens(torch.tensor([0, 10], dtype=torch.int32), 2, T)


_DEBUG_CALL = """
import channel_decay_softmax_amd as wall
from channel_decay_softmax_amd import _binding as B
L = wall.lib()
F = 1 << 20
P = lambda x: None if x is None else __import__('ctypes').c_void_p(x)
wsb = L.wall_attn_fwd_workspace_size(B.WALL_BF16, 1, 256, 6, 4, 128, 128, 0)
rc = L.wall_attn_fwd(P(F), P(F), P(F), B.WALL_BF16, P(F), None, None, P(F), None, 1, 256, 6, 4, 128, 128,
                     0.088, 0, None, 0, 0, P(F), wsb, None)
print('status', rc)
"""


@pytest.mark.parametrize("debug", ["1", None])
def test_wall_debug_reports_refused_calls(debug):
    """With WALL_DEBUG set, a refused call (here HQ % H != 0) names the check
    that failed on stderr; without it the library prints nothing."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("WALL_DEBUG", None)
    if debug:
        env["WALL_DEBUG"] = debug
    r = subprocess.run([sys.executable, "-c", _DEBUG_CALL], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert f"status {INVALID}" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("wall:")]
    if debug:
        assert any("refused the call: WALL_ERR_INVALID_ARG (wall_api.cpp:" in l for l in lines), r.stderr
    else:
        assert not lines, r.stderr
