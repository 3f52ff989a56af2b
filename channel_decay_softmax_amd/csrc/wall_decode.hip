// wall_decode.hip -- the decode path of the wall-attention-release README
// ("Decode (cached generation)"): a cache of decay-folded keys built once
// (and appended to as tokens arrive), then one query per head per step.
//
// Cache, per chunk c of C rows, query head hq and channel n:
//     R[c][n]        = floor(P[c*C][n])                (anchor: the chunk's first row)
//     k_tilde[j][n]  = k[j][n] * exp2(R[c][n] - P[j][n]),   c = j / C
// Decode, query q at the row whose prefix is p:
//     logit_j = scale * sum_n q_n * exp2(p_n - R[j/C][n]) * k_tilde[j][n]
// which is the forward's logit (the blog's factored form, "Definition: Wall
// Attention") with the anchor cancelling; the inner loop carries no gate
// arithmetic beyond one exp2 per channel per chunk.
//
// The decode is split over the keys (split-KV): each block takes one (b, hq)
// and S keys, one wave, 64 keys per round:
//   - q~ of the round's chunk (K exps, once per chunk) goes to LDS in the
//     cache's element type;
//   - lane j takes key j of the round: its k_tilde row (K elements, 16-byte
//     loads) against q~ read from LDS by broadcast, bf16 pairs through the
//     packed dot product, in log2 units;
//   - the online softmax over the round (wave max / sum);
//   - p goes to LDS and the value rows are read row-contiguously (lane =
//     8 channels x one of 64/(V/8) key slots), accumulated in fp32.
// A second kernel merges the splits with the sink.  The kernels are bound
// by HBM: each step reads the cached keys of every query head, the values of
// every kv head and the anchors once.
#include "wall_common.h"

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

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// ---------------------------------------------------------------- cache
// Thread = 8 channels of one (b, row j, hq), rows t0 .. t1-1.  A chunk that
// opens inside the range takes its anchor from P (every thread of the chunk
// reads the first row's prefix; the first row's threads store it); a chunk
// opened by an earlier call reads the stored anchor.
template <typename T, int K>
__global__ __launch_bounds__(256) void kv_cache_kernel(CacheArgs a) {
    constexpr int CPR = K / 8;
    const int64_t nrows = a.t1 - a.t0;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.B * nrows * a.HQ * CPR) return;
    const int c8 = (int)(idx % CPR);
    int64_t r = idx / CPR;
    const int64_t hq = r % a.HQ;
    r /= a.HQ;
    const int64_t j = a.t0 + r % nrows, b = r / nrows;
    const int64_t h = hq / (a.HQ / a.H);
    const int64_t c = j / a.C, j0 = c * a.C;
    const int64_t NC = cdiv(a.Tcap, a.C);
    float *Rp = a.r + ((b * NC + c) * a.HQ + hq) * K + c8 * 8;
    f32x8 R;
    if (j0 >= a.t0) {
        const f32x8 Pa = *reinterpret_cast<const f32x8 *>(a.P + ((b * a.Tcap + j0) * a.HQ + hq) * K + c8 * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) R[e] = floorf(Pa[e]);
        if (j == j0) *reinterpret_cast<f32x8 *>(Rp) = R;
    } else {
        R = *reinterpret_cast<const f32x8 *>(Rp);
    }
    const f32x8 kv = Vec8<T>::load(static_cast<const T *>(a.k) + ((b * a.Tcap + j) * a.H + h) * K + c8 * 8);
    const f32x8 Pj = *reinterpret_cast<const f32x8 *>(a.P + ((b * a.Tcap + j) * a.HQ + hq) * K + c8 * 8);
    f32x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = kv[e] * exp2f(fminf(fmaxf(R[e] - Pj[e], EXP2_LO), EXP2_HI));
    Vec8<T>::store(static_cast<T *>(a.kt) + ((b * a.Tcap + j) * a.HQ + hq) * K + c8 * 8, out);
}

// ---------------------------------------------------------------- decode
// Dot product of 8 channels of a cached key with 8 channels of q~.
__device__ inline float dot8(const __bf16 *k, const __bf16 *q, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(k);
    const bf16x8 qq = *reinterpret_cast<const bf16x8 *>(q);
#pragma unroll
    for (int e = 0; e < 8; e += 2)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{kk[e], kk[e + 1]}, bf16x2{qq[e], qq[e + 1]}, acc, false);
    return acc;
}
__device__ inline float dot8(const float *k, const float *q, float acc) {
    const f32x8 kk = *reinterpret_cast<const f32x8 *>(k);
    const f32x8 qq = *reinterpret_cast<const f32x8 *>(q);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(kk[e], qq[e], acc);
    return acc;
}

template <typename T, int K, int V>
__global__ __launch_bounds__(64) void decode_split(DecodeArgs a) {
    __shared__ __attribute__((aligned(32))) T qs[K];
    __shared__ float ps[64];
    constexpr int CG = V / 8, KSL = 64 / CG;  // value loads: 8 channels x KSL keys
    const int lane = threadIdx.x;
    const int split = blockIdx.x, bh = blockIdx.y;
    const int64_t b = bh / a.HQ, hq = bh % a.HQ, h = hq / (a.HQ / a.H);
    const int s0 = split * a.S, s1 = min(a.T, s0 + a.S);
    const int cg = lane % CG, kg = lane / CG;
    const int64_t NC = cdiv(a.Tcap, a.C);
    const T *kt = static_cast<const T *>(a.kt) + (b * a.Tcap * a.HQ + hq) * K;
    const T *vb = static_cast<const T *>(a.v) + (b * a.Tcap * a.H + h) * V + cg * 8;
    const T *qg = static_cast<const T *>(a.q) + bh * K;
    const float *pg = a.pc + bh * K;

    float m = -__builtin_inff(), l = 0.f;
    f32x8 o8 = {};
    int64_t cprev = -1;
    for (int j0 = s0; j0 < s1; j0 += 64) {
        const int64_t c = j0 / a.C;  // C is a multiple of 64: one chunk per round
        if (c != cprev) {
            const float *R = a.r + ((b * NC + c) * a.HQ + hq) * K;
            for (int n = lane; n < K; n += 64)
                qs[n] = (T)((float)qg[n] * a.qscale * exp2f(fminf(fmaxf(pg[n] - R[n], EXP2_LO), EXP2_HI)));
            cprev = c;
            __syncthreads();
        }
        const int j = j0 + lane;
        float s = -__builtin_inff();
        if (j < s1) {
            const T *kr = kt + (int64_t)j * a.HQ * K;
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int n = 0; n < K; n += 16) {
                acc0 = dot8(kr + n, qs + n, acc0);
                acc1 = dot8(kr + n + 8, qs + n + 8, acc1);
            }
            s = acc0 + acc1;
        }
        // online softmax over the round (log2 units); at least key j0 is visible
        const float mn = fmaxf(m, wave_max(s));
        const float al = exp2f(m - mn);
        const float p = j < s1 ? exp2f(s - mn) : 0.f;
        l = l * al + wave_sum(p);
        o8 *= al;
        m = mn;
        ps[lane] = p;
        __syncthreads();
#pragma unroll 4
        for (int it = 0; it < 64 / KSL; ++it) {
            const int jj = it * KSL + kg;
            if (j0 + jj < s1) {
                const f32x8 vv = Vec8<T>::load(vb + (int64_t)(j0 + jj) * a.H * V);
                o8 += ps[jj] * vv;
            }
        }
        __syncthreads();  // q~ and p are rewritten next round
    }
    // the KSL key slots of each channel group
#pragma unroll
    for (int off = CG; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] += __shfl_xor(o8[e], off);
    float *pp = a.part + ((int64_t)split * a.B * a.HQ + bh) * (V + 2);
    if (kg == 0) {
        reinterpret_cast<f32x4 *>(pp + cg * 8)[0] = f32x4{o8[0], o8[1], o8[2], o8[3]};
        reinterpret_cast<f32x4 *>(pp + cg * 8)[1] = f32x4{o8[4], o8[5], o8[6], o8[7]};
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
    const int64_t n = a.B * (a.t1 - a.t0) * a.HQ * (K / 8);
    hipLaunchKernelGGL((kv_cache_kernel<T, K>), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, int K, int V>
hipError_t run_decode(const DecodeArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((decode_split<T, K, V>), dim3((unsigned)a.nsplit, (unsigned)(a.B * a.HQ)), dim3(64), 0, st,
                       a);
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
