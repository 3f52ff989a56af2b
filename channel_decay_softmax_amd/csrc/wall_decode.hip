// wall_decode.hip -- the decode path of the wall-attention-release README
// ("Decode (cached generation)"): a cache of decay-folded keys built once
// (and appended to as tokens arrive), then one query per head per step.
//
// Cache, per chunk c of C rows, query head hq and channel n (wall_cache.h):
//     k_tilde[j][n]  = k[j][n] * exp2(R[c][n] - P[j][n]),   c = j / C,
// with the anchor R[c][n] the floored prefix of the chunk's first row, moved
// to a later row's floored prefix whenever that row lies more than 64 log2
// units below it (the chunk's earlier rows lowered by the exact power of
// two), so every cached factor stays at most 2^64.
// Decode, query q at the row whose prefix is p (at or after every cached row):
//     logit_j = scale * sum_n q_n * exp2(p_n - R[j/C][n]) * k_tilde[j][n]
// which is the forward's logit (the blog's factored form, "Definition: Wall
// Attention") with the anchor cancelling; the query factor is at most 2.  The
// inner loop carries no gate arithmetic beyond one exp2 per channel per chunk.
//
// The decode is split over the keys (split-KV): each block takes S keys of
// up to four query heads of one kv head, one wave per head, 32 keys per round:
//   - q~ of the round's chunk (one exp2 per channel), each lane keeping the 8
//     channels it multiplies, in the cache's element type;
//   - a group of K/8 lanes reads one k_tilde row (whole rows per load), bf16
//     pairs through the packed dot product, summed over the group;
//   - the online softmax over the round, in log2 units;
//   - a group of V/8 lanes reads one value row and accumulates p * v in fp32.
//     The waves of a block read the same value rows (one kv head), so all but
//     the first read of each row hit the CU's L1.
// Small rounds keep each wave near 128 registers, so four waves share a SIMD:
// occupancy, rather than loads issued further ahead, is what covers the
// latency of HBM here.
// A second kernel merges the splits with the sink.  The kernels are bound
// by HBM: each step reads the cached keys of every query head, the values of
// every kv head and the anchors once.
#include "wall_cache.h"
#include "wall_common.h"

#include <type_traits>

namespace wall {
namespace {

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
    using Raw = bf16x8;
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

// ---------------------------------------------------------------- cache
// Thread = 8 channels of one (b, chunk, hq) among the chunks that rows t0..t1-1
// touch: its rows of the range in order (wall_cache.h).
template <typename T, int K>
__global__ __launch_bounds__(256) void kv_cache_kernel(CacheArgs a) {
    constexpr int CPR = K / 8;
    const int64_t c_first = a.t0 / a.C, nch = (a.t1 - 1) / a.C - c_first + 1;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.B * nch * a.HQ * CPR) return;
    const int c8 = (int)(idx % CPR);
    int64_t r = idx / CPR;
    const int64_t hq = r % a.HQ;
    r /= a.HQ;
    const int64_t c = c_first + r % nch, b = r / nch;
    const int64_t h = hq / (a.HQ / a.H);
    const int64_t j0 = c * a.C, ja = j0 > a.t0 ? j0 : a.t0, jb = j0 + a.C < a.t1 ? j0 + a.C : a.t1;
    const int64_t NC = cdiv(a.Tcap, a.C);
    cache_chunk<T>(static_cast<const T *>(a.k) + (b * a.Tcap * a.H + h) * K + c8 * 8,
                   a.P + (b * a.Tcap * a.HQ + hq) * K + c8 * 8,
                   static_cast<T *>(a.kt) + (b * a.Tcap * a.HQ + hq) * K + c8 * 8,
                   a.r + ((b * NC + c) * a.HQ + hq) * K + c8 * 8, a.HQ * K, a.H * K, j0, ja, jb);
}

// ---------------------------------------------------------------- decode
// Dot product of 8 channels of a cached key with the lane's 8 channels of q~.
__device__ inline float dot8(const bf16x8 &kk, const bf16x8 &qq) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{kk[e], kk[e + 1]}, bf16x2{qq[e], qq[e + 1]}, acc, false);
    return acc;
}
__device__ inline float dot8(const f32x8 &kk, const f32x8 &qq) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(kk[e], qq[e], acc);
    return acc;
}
template <typename T>
using Vec = typename std::conditional<std::is_same<T, __bf16>::value, bf16x8, f32x8>::type;

// x summed over aligned groups of W lanes (W = 8 or 16), every lane of a
// group receiving the group's sum: quad swaps, then half-row and row mirrors.
template <int CTRL>
__device__ inline float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int W>
__device__ inline float group_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (W == 16) x += dpp<0x140>(x);  // row_mirror
    return x;
}

// One round = RK keys.  QK: a group of K/8 lanes reads one key row (16 bytes
// a lane, whole rows per load), each lane against its own 8 channels of q~
// (registers), then the group's sum; 64/(K/8) keys per load.  PV: a group
// of V/8 lanes reads one value row the same way and accumulates p * v for
// its 8 channels; the groups are summed at the end.  With K == V the two
// mappings coincide and p stays in registers, else it goes through LDS.
// Wave w of the block is query head blockIdx.y * nwg + w (flattened with b).
template <typename T, int K, int V>
__global__ __launch_bounds__(256) void decode_split(DecodeArgs a) {
    constexpr int RK = 32;  // keys per round
    constexpr int GK = K / 8, NKQ = 64 / GK, NQ = RK / NKQ;  // QK: lanes per key, keys per load, loads
    constexpr int GV = V / 8, NKV = 64 / GV, NVL = RK / NKV;  // PV: the same for values
    __shared__ float ps[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int split = blockIdx.x, bh = blockIdx.y * a.nwg + w;
    const int64_t b = bh / a.HQ, hq = bh % a.HQ, h = hq / (a.HQ / a.H);
    const int s0 = split * a.S, s1 = min(a.T, s0 + a.S);
    const int gq = lane / GK, cq = lane % GK;
    const int gv = lane / GV, cv = lane % GV;
    const int64_t NC = cdiv(a.Tcap, a.C);
    const T *kt = static_cast<const T *>(a.kt) + (b * a.Tcap * a.HQ + hq) * K + cq * 8;
    const T *vb = static_cast<const T *>(a.v) + (b * a.Tcap * a.H + h) * V + cv * 8;
    const int64_t kstride = a.HQ * K, vstride = a.H * V;

    float m = -__builtin_inff(), l = 0.f;
    f32x8 o8 = {};
    // q and its prefix, once; the anchors of each round's chunk one round ahead
    const f32x8 qv = Vec8<T>::load(static_cast<const T *>(a.q) + bh * K + cq * 8);
    const f32x8 pv = *reinterpret_cast<const f32x8 *>(a.pc + b * a.pc_bs + hq * K + cq * 8);
    const float *rb = a.r + (b * NC * a.HQ + hq) * K + cq * 8;
    const int64_t rstride = a.HQ * K;
    f32x8 rv = *reinterpret_cast<const f32x8 *>(rb + (s0 / a.C) * rstride);
    for (int j0 = s0; j0 < s1; j0 += RK) {
        // the round's key and value rows, all in flight
        Vec<T> kk[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int j = j0 + NKQ * i + gq;
            // the cached keys of each query head are read once per call: loaded
            // past the caches, which keep the value rows the block's four query
            // heads share
            if (j < s1) kk[i] = __builtin_nontemporal_load(reinterpret_cast<const Vec<T> *>(kt + (int64_t)j * kstride));
            else kk[i] = Vec<T>{};
        }
        Vec<T> vv[NVL];
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int j = j0 + NKV * i + gv;
            if (j < s1) vv[i] = *reinterpret_cast<const Vec<T> *>(vb + (int64_t)j * vstride);
            else vv[i] = Vec<T>{};
        }
        // the lane's 8 channels of q~ = q * scale*log2e * exp2(p - R_c) for the
        // round's chunk (C is a multiple of 64: one chunk per round), in the cache dtype
        Vec<T> q8;
        {
            f32x8 qt;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qt[e] = qv[e] * a.qscale * exp2f(fminf(fmaxf(pv[e] - rv[e], EXP2_LO), EXP2_HI));
            if constexpr (std::is_same<T, __bf16>::value) q8 = __builtin_convertvector(qt, bf16x8);
            else q8 = qt;
        }
        if (j0 + RK < s1) rv = *reinterpret_cast<const f32x8 *>(rb + ((j0 + RK) / a.C) * rstride);
        float sc[NQ];
        float mt = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            sc[i] = group_sum<GK>(dot8(kk[i], q8));
            sc[i] = j0 + NKQ * i + gq < s1 ? sc[i] : -__builtin_inff();
            mt = fmaxf(mt, sc[i]);
        }
        // the round's max over the NKQ groups (each lane of a group holds the same values)
#pragma unroll
        for (int off = GK; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
        const float mn = fmaxf(m, mt);  // finite: key j0 is visible
        const float al = exp2f(m - mn);
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            sc[i] = exp2f(sc[i] - mn);
            ls += sc[i];
        }
#pragma unroll
        for (int off = GK; off < 64; off <<= 1) ls += __shfl_xor(ls, off);
        l = l * al + ls;
        o8 *= al;
        m = mn;
        if constexpr (GK != GV) {
            if (cq < NQ) ps[w][NKQ * cq + gq] = sc[cq];  // lane (gq, cq) holds key NKQ*cq + gq once
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const float p = GK == GV ? sc[i] : ps[w][NKV * i + gv];
            f32x8 x;
            if constexpr (std::is_same<T, __bf16>::value) x = __builtin_convertvector(vv[i], f32x8);
            else x = vv[i];
            o8 += p * x;
        }
        if constexpr (GK != GV) __syncthreads();  // p is rewritten next round
    }
    // the NKV key groups of each channel block
#pragma unroll
    for (int off = GV; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] += __shfl_xor(o8[e], off);
    float *pp = a.part + ((int64_t)split * a.B * a.HQ + bh) * (V + 2);
    if (gv == 0) {
        reinterpret_cast<f32x4 *>(pp + cv * 8)[0] = f32x4{o8[0], o8[1], o8[2], o8[3]};
        reinterpret_cast<f32x4 *>(pp + cv * 8)[1] = f32x4{o8[4], o8[5], o8[6], o8[7]};
    }
    if (lane == 0) {
        pp[V] = m;
        pp[V + 1] = l;
    }
}

// Merge of the splits of one (b, hq), thread = value channel.  The sink is
// one more logit (natural log, value 0) in the normaliser.
template <typename T, int V>
__global__ __launch_bounds__(V) void decode_merge(DecodeArgs a) {
    const int bh = blockIdx.x, d = threadIdx.x;
    const int64_t stride = (int64_t)a.B * a.HQ * (V + 2);
    const float *pp = a.part + (int64_t)bh * (V + 2);
    float M = -__builtin_inff();
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pp[s * stride + V]);
    const float sk = a.sink ? a.sink[bh % a.HQ] * LOG2E : -__builtin_inff();
    M = fmaxf(M, sk);
    float L = 0.f, od = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
        const float w = exp2f(pp[s * stride + V] - M);
        L += pp[s * stride + V + 1] * w;
        od += pp[s * stride + d] * w;
    }
    if (a.sink) L += exp2f(sk - M);
    static_cast<T *>(a.o)[(int64_t)bh * V + d] = (T)(od / L);
    if (d == 0 && a.lse) a.lse[bh] = LN2 * (M + log2f(L));
}

template <typename T, int K>
hipError_t run_cache(const CacheArgs &a, hipStream_t st) {
    const int64_t n = a.B * ((a.t1 - 1) / a.C - a.t0 / a.C + 1) * a.HQ * (K / 8);
    hipLaunchKernelGGL((kv_cache_kernel<T, K>), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, int K, int V>
hipError_t run_decode(const DecodeArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((decode_split<T, K, V>), dim3((unsigned)a.nsplit, (unsigned)(a.B * a.HQ / a.nwg)),
                       dim3(64 * a.nwg), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge<T, V>), dim3((unsigned)(a.B * a.HQ)), dim3(V), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_decode(const DecodeArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_decode<T, 64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_decode<T, 64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_decode<T, 128, 64>(a, st);
    return run_decode<T, 128, 128>(a, st);
}

}  // namespace

hipError_t launch_kv_cache(const CacheArgs &a, bool bf16, hipStream_t st) {
    if (bf16) return a.K == 64 ? run_cache<__bf16, 64>(a, st) : run_cache<__bf16, 128>(a, st);
    return a.K == 64 ? run_cache<float, 64>(a, st) : run_cache<float, 128>(a, st);
}

hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t st) {
    return bf16 ? dispatch_decode<__bf16>(a, st) : dispatch_decode<float>(a, st);
}

}  // namespace wall
