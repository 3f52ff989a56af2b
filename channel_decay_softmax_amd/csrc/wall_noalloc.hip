// wall_noalloc.hip -- wall_attn_decode_noalloc: the decode step with its
// split partials in a fixed device array of this library instead of a
// caller's workspace, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side stand-in, so the device address is taken
// once per device with hipGetSymbolAddress (the device current at the time)
// and kept; the kernels receive that address as their partials buffer, as
// they receive the workspace in wall_attn_decode.  The split kernel writes
// every partial it owns before the merge kernel reads it, so nothing needs
// clearing between calls; calls that overlap on one GPU share the array and
// race.
#include <atomic>
#include <mutex>

#include "wall_common.h"
#include "wall_entry.h"

namespace {

static __device__ __align__(256) float scratch[WALL_DECODE_SCRATCH_BYTES / sizeof(float)];

constexpr int MAX_DEVICES = 64;
std::atomic<float *> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mu;

// The current device's copy of `scratch` (its address taken on first use).
wall_status_t current_scratch(float **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return WALL_ERR_LAUNCH;
    if (dev >= MAX_DEVICES) return WALL_ERR_UNSUPPORTED;
    float *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return WALL_ERR_LAUNCH;
            p = static_cast<float *>(addr);
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return WALL_OK;
}

}  // namespace

extern "C" wall_status_t wall_attn_decode_noalloc(const void *q, const void *v, wall_dtype_t dtype,
                                                  const float *p_curr, int64_t p_curr_batch_stride,
                                                  const void *k_tilde, const float *r_cache, const float *sink_bias,
                                                  void *o, float *lse, int64_t B, int64_t T, int64_t T_cap,
                                                  int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size,
                                                  float scale, hipStream_t stream) {
    const wall_status_t st = wall::decode_check(q, v, dtype, p_curr, p_curr_batch_stride, k_tilde, r_cache,
                                                sink_bias, o, lse, B, T, T_cap, HQ, H, K, V, chunk_size);
    if (st != WALL_OK) return st;
    if (wall::decode_layout(B, T, HQ, V).total > WALL_DECODE_SCRATCH_BYTES) return WALL_ERR_SCRATCH;
    float *part = nullptr;
    const wall_status_t sp = current_scratch(&part);
    if (sp != WALL_OK) return sp;
    return wall::decode_launch(q, v, dtype, p_curr, p_curr_batch_stride, k_tilde, r_cache, sink_bias, o, lse, B, T,
                               T_cap, HQ, H, K, V, chunk_size, scale, part, stream);
}
