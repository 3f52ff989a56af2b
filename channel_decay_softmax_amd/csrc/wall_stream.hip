// wall_stream.hip -- one turn of the append-as-you-go decode loop in one pass
// (the README's streaming decode): for new rows t0 .. t1-1 of each sequence,
// the log2 prefix P from the previous row's (as wall_prefix_append computes
// it) and the cache rows and chunk anchors (as wall_kv_cache_build computes
// them, wall_cache.h), with the same float32 operations in the same order,
// so the results are those of the two separate calls bit for bit.
#include "wall_cache.h"
#include "wall_common.h"
#include "wall_stream.h"

namespace wall {
namespace {

template <typename T>
__device__ inline f32x8 load8(const T *p);
template <>
__device__ inline f32x8 load8<__bf16>(const __bf16 *p) {
    return __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p), f32x8);
}
template <>
__device__ inline f32x8 load8<float>(const float *p) {
    return *reinterpret_cast<const f32x8 *>(p);
}

// One thread per (sequence, query head, 8 channels); the new rows in order:
// first their prefix, then their cache rows chunk by chunk.
template <typename Tg, typename T, int K>
__global__ __launch_bounds__(256) void stream_append_kernel(StreamArgs a) {
    constexpr int CPR = K / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.B * a.HQ * CPR) return;
    const int c8 = (int)(idx % CPR);
    const int64_t hq = (idx / CPR) % a.HQ, b = idx / (CPR * a.HQ);
    const int64_t h = hq / (a.HQ / a.H);
    const int64_t NC = cdiv(a.Tcap, a.C);
    const int64_t rowP = a.HQ * K, rowK = a.H * K;
    const int64_t base = (b * a.Tcap * a.HQ + hq) * K + c8 * 8;       // [b, 0, hq, ch] in P, g, kt
    const int64_t kbase = (b * a.Tcap * a.H + h) * K + c8 * 8;        // [b, 0, h, ch] in k
    f32x8 prev = 0.f;
    if (a.t0 > 0) prev = *reinterpret_cast<const f32x8 *>(a.P + base + (a.t0 - 1) * rowP);
    f32x8 s = 0.f;
    for (int64_t t = a.t0; t < a.t1; ++t) {
        const f32x8 g8 = load8<Tg>(static_cast<const Tg *>(a.g) + base + t * rowP);
        f32x8 P;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s[e] += g8[e];
            P[e] = prev[e] + a.scale * s[e];
        }
        *reinterpret_cast<f32x8 *>(a.P + base + t * rowP) = P;
    }
    for (int64_t ja = a.t0; ja < a.t1;) {
        const int64_t c = ja / a.C, j0 = c * a.C, jb = j0 + a.C < a.t1 ? j0 + a.C : a.t1;
        cache_chunk<T>(static_cast<const T *>(a.k) + kbase, a.P + base, static_cast<T *>(a.kt) + base,
                       a.r + ((b * NC + c) * a.HQ + hq) * K + c8 * 8, rowP, rowK, j0, ja, jb);
        ja = jb;
    }
}

template <typename Tg, typename T>
hipError_t run(const StreamArgs &a, hipStream_t st) {
    const unsigned grid = (unsigned)cdiv(a.B * a.HQ * (a.K / 8), 256);
    if (a.K == 64)
        hipLaunchKernelGGL((stream_append_kernel<Tg, T, 64>), dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((stream_append_kernel<Tg, T, 128>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_append(const StreamArgs &a, bool g_bf16, bool k_bf16, hipStream_t st) {
    if (g_bf16) return k_bf16 ? run<__bf16, __bf16>(a, st) : run<__bf16, float>(a, st);
    return k_bf16 ? run<float, __bf16>(a, st) : run<float, float>(a, st);
}

}  // namespace wall
