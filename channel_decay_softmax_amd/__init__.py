"""MI355X-native Wall Attention forward (prefill).

The compute lives in libwall.so (HIP kernels for gfx950 behind the C ABI of
include/wall.h); this package only marshals torch tensors into it.

    from channel_decay_softmax_amd import wall_attn
    o = wall_attn(q, k, v, g, scale=K ** -0.5)   # [B, T, HQ, V]
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    WALL_BF16,
    WALL_ERR_INVALID_ARG,
    WALL_DECODE_SCRATCH_BYTES,
    WALL_ERR_LAUNCH,
    WALL_ERR_SCRATCH,
    WALL_ERR_UNSUPPORTED,
    WALL_F32,
    WALL_OK,
    WallError,
    attn_fwd_workspace_size,
    build_wall_kv_cache,
    check_cu_seqlens,
    decode_workspace_size,
    lib,
    prefix_scan_workspace_size,
    status_string,
    wall_attn,
    wall_attn_bwd,
    wall_attn_decode,
    wall_attn_fwd,
    wall_attn_fwd_gate,
    wall_attn_fwd_prepare,
    wall_attn_fwd_prepare_gate,
    wall_attn_fwd_run,
    wall_prefix_scan,
    wall_prefix_append,
    wall_stream_append,
)

__all__ = ["wall_attn", "wall_attn_fwd", "wall_attn_bwd", "wall_prefix_scan", "build_wall_kv_cache", "wall_attn_decode",
           "WallError", "lib"]
