// wall_prep.hip -- per-call preparation for the fused forward.
//
// 1. seg_table: one SegInfo per sequence (start row, length, index of its
//    first 128-row tile in the tiled workspace).  Tiles never straddle two
//    sequences, so a tile's rows always share one prefix P.
// 2. key cache: per (tile, query head) the anchors R[n] = floor(P[a][n]) at the
//    tile's middle row a, the carry record that moves a query from this
//    tile's anchors to the previous tile's, and the decay-rescaled keys
//        k~[j][n] = k[j][n] * exp2(R[n] - P[j][n]),
//    zero-padded to 128 rows.  This is the blog's per-tile anchor split
//    ("Fast training and inference", per-tile anchors:
//    exp2(P_i - P_j) = exp2(P_i - R) * exp2(R - P_j)) applied on the key
//    side once per (tile, head) instead of once per (query tile, key tile);
//    it is the same fold the README's decode cache performs with
//    k_tilde[j] = k[j] * exp2(R_c - P[j]).
// 3. value tiles: v copied per (tile, kv head), transposed to [V][128] for
//    the bf16 MFMA kernel (its PV operand reads keys contiguously) and kept
//    as [128][V] for the float32 kernel; zero-padded.
#include "wall_common.h"

namespace wall {
namespace {

__global__ __launch_bounds__(256) void seg_table_kernel(SegInfo *seg, const int32_t *cu, int nseg,
                                                        int T) {
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int per = (nseg + 255) / 256;
    const int s0 = tid * per, s1 = min(nseg, s0 + per);
    int local = 0;
    for (int s = s0; s < s1; ++s) {
        const int len = cu ? cu[s + 1] - cu[s] : T;
        local += (len + TILE - 1) / TILE;
    }
    part[tid] = local;
    __syncthreads();
    if (tid == 0) {  // exclusive scan of 256 partial tile counts
        int run = 0;
        for (int i = 0; i < 256; ++i) {
            const int x = part[i];
            part[i] = run;
            run += x;
        }
    }
    __syncthreads();
    int base = part[tid];
    for (int s = s0; s < s1; ++s) {
        const int start = cu ? cu[s] : s * T;
        const int len = cu ? cu[s + 1] - cu[s] : T;
        seg[s] = SegInfo{start, len, base, 0};
        base += (len + TILE - 1) / TILE;
    }
}

// The sequence whose tiles hold tile id `tile` (last s with tile_base <= tile).
__device__ inline int find_seg(const SegInfo *seg, int nseg, int tile) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg[mid].tile_base <= tile) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
    static __device__ inline f32x8 load(const __bf16 *p) {
        return __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p), f32x8);
    }
    static __device__ inline void store(__bf16 *p, f32x8 v) {
        *reinterpret_cast<bf16x8 *>(p) = __builtin_convertvector(v, bf16x8);
    }
};
template <>
struct Vec8<float> {
    static __device__ inline f32x8 load(const float *p) { return *reinterpret_cast<const f32x8 *>(p); }
    static __device__ inline void store(float *p, f32x8 v) { *reinterpret_cast<f32x8 *>(p) = v; }
};

template <typename T, int K>
__global__ __launch_bounds__(256) void key_cache_kernel(PrepArgs a) {
    constexpr int CPR = K / 8;          // 8-channel chunks per row
    constexpr int RPP = 256 / CPR;      // rows per pass
    const int tile = blockIdx.x, hq = blockIdx.y;
    const int s = find_seg(a.seg, (int)a.nseg, tile);
    const SegInfo sg = a.seg[s];
    const int c = tile - sg.tile_base;
    if (c < 0 || c * TILE >= sg.len) return;  // beyond the last used tile
    const int h = hq / (int)(a.HQ / a.H);
    const int c8 = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    const int arow = min(c * TILE + ANCHOR_ROW, sg.len - 1);
    const float *Pa = a.P + ((int64_t)(sg.start + arow) * a.HQ + hq) * K + c8 * 8;
    f32x8 R;
    for (int e = 0; e < 8; ++e) R[e] = floorf(Pa[e]);
    if (r0 == 0) {
        float *ap = a.anchor + ((int64_t)tile * a.HQ + hq) * K + c8 * 8;
        *reinterpret_cast<f32x8 *>(ap) = R;
        // carry record: the shift from this tile's anchors to the previous tile's
        bool up = false;
        uint32_t *rec = a.rec + ((int64_t)tile * a.HQ + hq) * REC_WORDS;
        for (int e = 0; e < 8; e += 2) {
            uint32_t w = 0;
            if (c > 0) {
                const int prow = (c - 1) * TILE + ANCHOR_ROW;  // anchor row of tile c-1 (< len)
                const float *Pp = a.P + ((int64_t)(sg.start + prow) * a.HQ + hq) * K + c8 * 8;
                const float d0 = floorf(Pp[e]) - R[e], d1 = floorf(Pp[e + 1]) - R[e + 1];
                up = up || d0 < 0.f || d1 < 0.f;
                const uint32_t s0 = (uint32_t)fminf(fmaxf(d0, 0.f), 255.f) * 128u;
                const uint32_t s1 = (uint32_t)fminf(fmaxf(d1, 0.f), 255.f) * 128u;
                w = s0 | (s1 << 16);
            }
            rec[(c8 * 8 + e) / 2] = w;
        }
        const bool any_up = __any(up);  // the r0 == 0 threads are lanes 0..K/8-1 of wave 0
        if (threadIdx.x == 0) rec[REC_GROW] = any_up ? 1u : 0u;
    }
    const T *kin = static_cast<const T *>(a.k);
    T *kout = static_cast<T *>(a.kt) + ((int64_t)tile * a.HQ + hq) * TILE * K;
    for (int r = r0; r < TILE; r += RPP) {
        const int j = c * TILE + r;
        f32x8 out = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (j < sg.len) {
            const int64_t tok = sg.start + j;
            const f32x8 kv = Vec8<T>::load(kin + (tok * a.H + h) * K + c8 * 8);
            const f32x8 pv = *reinterpret_cast<const f32x8 *>(a.P + (tok * a.HQ + hq) * K + c8 * 8);
            for (int e = 0; e < 8; ++e)
                out[e] = kv[e] * exp2f(fminf(fmaxf(R[e] - pv[e], EXP2_LO), EXP2_HI));
        }
        Vec8<T>::store(kout + r * K + c8 * 8, out);
    }
}

// Value tile of (tile, kv head): transposed [V][TILE] (TRANSPOSE) or [TILE][V].
template <typename T, int V, bool TRANSPOSE>
__global__ __launch_bounds__(256) void value_tile_kernel(PrepArgs a) {
    constexpr int CPR = V / 8;
    constexpr int RPP = 256 / CPR;
    constexpr int PITCH = V + 1;  // odd float pitch: conflict-free column reads
    __shared__ float sv[TILE * PITCH];
    const int tile = blockIdx.x, h = blockIdx.y;
    const int s = find_seg(a.seg, (int)a.nseg, tile);
    const SegInfo sg = a.seg[s];
    const int c = tile - sg.tile_base;
    if (c < 0 || c * TILE >= sg.len) return;
    const T *vin = static_cast<const T *>(a.v);
    T *vout = static_cast<T *>(a.vt) + ((int64_t)tile * a.H + h) * V * TILE;
    const int c8 = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    for (int r = r0; r < TILE; r += RPP) {
        const int j = c * TILE + r;
        f32x8 x = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (j < sg.len) x = Vec8<T>::load(vin + ((int64_t)(sg.start + j) * a.H + h) * V + c8 * 8);
        if (TRANSPOSE) {
            for (int e = 0; e < 8; ++e) sv[r * PITCH + c8 * 8 + e] = x[e];
        } else {
            Vec8<T>::store(vout + r * V + c8 * 8, x);
        }
    }
    if (!TRANSPOSE) return;
    __syncthreads();
    // write [V][TILE]: 16 threads cover one value row of 128 keys, 8 keys each
    const int k8 = threadIdx.x % (TILE / 8), d0 = threadIdx.x / (TILE / 8);
    for (int d = d0; d < V; d += 256 / (TILE / 8)) {
        f32x8 x;
        for (int e = 0; e < 8; ++e) x[e] = sv[(k8 * 8 + e) * PITCH + d];
        Vec8<T>::store(vout + d * TILE + k8 * 8, x);
    }
}

template <typename T, int K, int V, bool TRANSPOSE>
hipError_t run_prep(const PrepArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((key_cache_kernel<T, K>), dim3((unsigned)a.tiles, (unsigned)a.HQ),
                       dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((value_tile_kernel<T, V, TRANSPOSE>), dim3((unsigned)a.tiles, (unsigned)a.H),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, bool TRANSPOSE>
hipError_t dispatch_prep(const PrepArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_prep<T, 64, 64, TRANSPOSE>(a, st);
    if (a.K == 64 && a.V == 128) return run_prep<T, 64, 128, TRANSPOSE>(a, st);
    if (a.K == 128 && a.V == 64) return run_prep<T, 128, 64, TRANSPOSE>(a, st);
    return run_prep<T, 128, 128, TRANSPOSE>(a, st);
}

}  // namespace

hipError_t launch_seg_table(SegInfo *seg, const int32_t *cu, int64_t nseg, int64_t B, int64_t T,
                            hipStream_t st) {
    (void)B;
    hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(256), 0, st, seg, cu, (int)nseg, (int)T);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st) {
    return bf16 ? dispatch_prep<__bf16, true>(a, st) : dispatch_prep<float, false>(a, st);
}

}  // namespace wall
