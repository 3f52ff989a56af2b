"""wall_attn_decode_noalloc (the decode step that allocates nothing: its split
partials live in the library's fixed per-GPU scratch) against
wall_attn_decode with a workspace, through the C ABI, on the same inputs.
The two run the same kernels on the same split plan, so the outputs must
agree bit for bit.  Three calls in a row on one GPU, each smaller than the
one before: the scratch keeps the previous call's partials, which a later
call must never read."""

import pytest
import torch

import channel_decay_softmax_amd as wall
from wall_inputs import make_decode_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu] {msg}", flush=True)


CALLS = [
    dict(B=16, T=2000, HQ=16, H=4, K=128, V=128, C=64, dtype="bfloat16", sink=True),
    dict(B=2, T=300, HQ=4, H=2, K=64, V=64, C=64, dtype="bfloat16", sink=False),
    dict(B=1, T=129, HQ=2, H=1, K=128, V=64, C=128, dtype="float32", sink=True),
]


def test_noalloc_decode_matches_the_workspace_decode():
    for c in CALLS:
        say(f"decode without allocation: {c}")
        inp = make_decode_inputs("decode_bf16", chunk_size=c["C"], B=c["B"], T=c["T"], HQ=c["HQ"], H=c["H"],
                                 K=c["K"], V=c["V"], dtype=c["dtype"], sink=c["sink"])
        d = inp.to(DEV)
        T = c["T"]
        P = wall.wall_prefix_scan(d.g)
        kt, r = wall.build_wall_kv_cache(d.k, P, c["C"])
        o_ref, l_ref = wall.wall_attn_decode(d.q, d.v, P[:, T - 1:T], kt, r, sink_bias=d.sink_bias,
                                             scale=inp.scale, cache_chunk_size=c["C"])
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        wall.wall_attn_decode(d.q, d.v, P[:, T - 1:T], kt, r, sink_bias=d.sink_bias, scale=inp.scale,
                              cache_chunk_size=c["C"], out=o, lse=lse, no_alloc=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "o differs from the workspace decode"
        assert torch.equal(lse, l_ref), "lse differs from the workspace decode"
