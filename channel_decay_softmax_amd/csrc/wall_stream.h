// wall_stream.h -- one turn of the append-as-you-go loop (internal launcher).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wall {

struct StreamArgs {
    const void *g;      // [B, Tcap, HQ, K] natural-log gate, rows t0 .. t1-1 read
    const void *k;      // [B, Tcap, H, K], rows t0 .. t1-1 read
    float *P;           // [B, Tcap, HQ, K] log2 prefix: row t0-1 read (when t0 > 0), rows t0 .. t1-1 written
    void *kt;           // [B, Tcap, HQ, K] cache rows t0 .. t1-1 written
    float *r;           // [B, ceil(Tcap / C), HQ, K] chunk anchors: read, or written when a chunk opens
    int64_t B, Tcap, HQ, H, K, C, t0, t1;
    float scale;        // 1 / ln 2 for the log2 prefix of a natural-log gate
};
hipError_t launch_stream_append(const StreamArgs &a, bool g_bf16, bool k_bf16, hipStream_t st);

}  // namespace wall
