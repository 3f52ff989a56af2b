// wall_scan.hip -- per-sequence prefix sum along T (the log2 prefix P of the
// Wall Attention blog's factored form, "Definition: Wall Attention", built
// in log2 units as the README's decode example does with a scaled cumsum).
//
// x is viewed as [rows, C] with rows = B*T.  Three kernels, float32 throughout:
//   A  chunk_sums : per 128-row chunk and channel, the sum since the chunk's
//                   last sequence start (or the whole chunk), plus a flag
//                   telling whether the chunk holds a start;
//   B  chunk_carry: a segmented exclusive scan of those sums over the chunks
//                   (a flag resets the running value), one thread per channel
//                   and chunk range;
//   C  finish     : each 32-row group loads its rows once into registers,
//                   sums them, takes the carry of its chunk plus the groups
//                   before it, and writes scale * prefix.
// Every thread moves 16 bytes per row (8 bf16 or 4 float32 channels when C
// allows, else one channel), coalesced along the channel axis.
#include "wall_common.h"

namespace wall {
namespace {

constexpr int ROWS_PER_GROUP = 32;              // rows per thread
constexpr int GROUPS = SCAN_CHUNK / ROWS_PER_GROUP;  // 4 row groups per chunk
constexpr int CV = 64;                          // channel vectors per block (one wave)
constexpr int CARRY_GROUPS = 16;                // chunk ranges per block in kernel B

template <int VEC>
using fvec = float __attribute__((ext_vector_type(VEC)));

// One row's VEC channels: the raw 16 bytes (or one element) and their float values.
template <typename Tin, int VEC>
struct Row;
template <>
struct Row<__bf16, 8> {
    using Raw = uint4;
    static __device__ inline Raw load(const __bf16 *p) { return *reinterpret_cast<const uint4 *>(p); }
    static __device__ inline fvec<8> val(Raw u) {
        return fvec<8>{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u),
                       __uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
                       __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)};
    }
};
template <>
struct Row<float, 4> {
    using Raw = f32x4;
    static __device__ inline Raw load(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
    static __device__ inline fvec<4> val(Raw u) { return u; }
};
template <>
struct Row<__bf16, 1> {
    using Raw = uint32_t;
    static __device__ inline Raw load(const __bf16 *p) { return *reinterpret_cast<const uint16_t *>(p); }
    static __device__ inline fvec<1> val(Raw u) { return fvec<1>{__uint_as_float(u << 16)}; }
};
template <>
struct Row<float, 1> {
    using Raw = float;
    static __device__ inline Raw load(const float *p) { return *p; }
    static __device__ inline fvec<1> val(Raw u) { return fvec<1>{u}; }
};
template <int VEC>
__device__ inline void store_row(__bf16 *p, fvec<VEC> v) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) p[e] = (__bf16)v[e];
}
template <int VEC>
__device__ inline void store_row(float *p, fvec<VEC> v) {
    if constexpr (VEC == 8) {
        reinterpret_cast<f32x4 *>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
        reinterpret_cast<f32x4 *>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
    } else if constexpr (VEC == 4) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
        *p = v[0];
    }
}
template <int VEC>
__device__ inline fvec<VEC> load_sum(const float *p) {
    fvec<VEC> v;
    if constexpr (VEC == 8) {
        const f32x4 a = reinterpret_cast<const f32x4 *>(p)[0], b = reinterpret_cast<const f32x4 *>(p)[1];
        v = fvec<8>{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else if constexpr (VEC == 4) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        v = fvec<4>{a[0], a[1], a[2], a[3]};
    } else {
        v = fvec<1>{*p};
    }
    return v;
}

// Bit i of word w is set when row row0 + 32*w + i starts a sequence.
__device__ inline void start_mask(uint32_t *smask, int64_t row0, int64_t rows, int T,
                                  const int32_t *cu, int nseq) {
    const int w = threadIdx.x;
    if (w >= GROUPS) return;
    const int64_t a = row0 + ROWS_PER_GROUP * w, b = a + ROWS_PER_GROUP;
    uint32_t m = 0;
    if (!cu) {
        int64_t first = (a + T - 1) / T * T;  // first multiple of T at or after a
        for (int64_t r = first; r < b && r < rows; r += T) m |= 1u << (r - a);
    } else {
        int lo = 0, hi = nseq;  // first s with cu[s] >= a
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (cu[mid] < a) lo = mid + 1; else hi = mid;
        }
        for (int s = lo; s < nseq && cu[s] < b; ++s)
            if (cu[s] < rows) m |= 1u << (cu[s] - a);
    }
    smask[w] = m;
}

template <typename Tin, int VEC>
__global__ __launch_bounds__(256) void scan_chunk_sums(const Tin *__restrict__ x,
                                                       float *__restrict__ csum,
                                                       int32_t *__restrict__ cflag, int64_t rows,
                                                       int64_t C, const int32_t *cu, int nseq,
                                                       int T) {
    using R = Row<Tin, VEC>;
    __shared__ uint32_t smask[GROUPS];
    __shared__ fvec<VEC> ssum[GROUPS][CV];
    __shared__ int sflag[GROUPS];
    const int chunk = blockIdx.x;
    const int64_t row0 = (int64_t)chunk * SCAN_CHUNK;
    start_mask(smask, row0, rows, T, cu, nseq);
    __syncthreads();
    const int rg = threadIdx.x / CV, cv = threadIdx.x % CV;
    const int64_t ch = ((int64_t)blockIdx.y * CV + cv) * VEC;
    const uint32_t mask = smask[rg];
    const int64_t r0 = row0 + ROWS_PER_GROUP * rg;
    fvec<VEC> s = {};
    if (ch < C) {
        if (r0 + ROWS_PER_GROUP <= rows) {
            typename R::Raw raw[ROWS_PER_GROUP];
#pragma unroll
            for (int i = 0; i < ROWS_PER_GROUP; ++i) raw[i] = R::load(x + (r0 + i) * C + ch);
#pragma unroll
            for (int i = 0; i < ROWS_PER_GROUP; ++i) {
                if ((mask >> i) & 1u) s = fvec<VEC>{};
                s += R::val(raw[i]);
            }
        } else {
            for (int i = 0; i < ROWS_PER_GROUP && r0 + i < rows; ++i) {
                if ((mask >> i) & 1u) s = fvec<VEC>{};
                s += R::val(R::load(x + (r0 + i) * C + ch));
            }
        }
    }
    ssum[rg][cv] = s;
    if (cv == 0) sflag[rg] = mask != 0;
    __syncthreads();
    if (rg == 0 && ch < C) {
        fvec<VEC> S = ssum[0][cv];
        int F = sflag[0];
        for (int g = 1; g < GROUPS; ++g) {
            S = sflag[g] ? ssum[g][cv] : S + ssum[g][cv];
            F |= sflag[g];
        }
        store_row<VEC>(csum + (int64_t)chunk * C + ch, S);
        if (blockIdx.y == 0 && cv == 0) cflag[chunk] = F;
    }
}

// Exclusive segmented scan of the chunk sums: carry[c] is the running sum
// (since the last sequence start) just before chunk c begins.  A block takes
// one wave of channels; its CARRY_GROUPS waves split the chunks.
template <int VEC>
__global__ __launch_bounds__(CV * CARRY_GROUPS) void scan_chunk_carry(const float *__restrict__ csum,
                                                                      const int32_t *__restrict__ cflag,
                                                                      float *__restrict__ carry,
                                                                      int64_t nchunk, int64_t C) {
    __shared__ fvec<VEC> gS[CARRY_GROUPS][CV];
    __shared__ int gF[CARRY_GROUPS];
    const int gi = threadIdx.x / CV, cv = threadIdx.x % CV;
    const int64_t ch = ((int64_t)blockIdx.x * CV + cv) * VEC;
    const int64_t per = (nchunk + CARRY_GROUPS - 1) / CARRY_GROUPS;
    const int64_t c0 = gi * per, c1 = c0 + per < nchunk ? c0 + per : nchunk;
    fvec<VEC> S = {};
    int F = 0;
    for (int64_t c = c0; c < c1; ++c) {
        const int f = cflag[c];
        if (ch < C) {
            const fvec<VEC> v = load_sum<VEC>(csum + c * C + ch);
            S = f ? v : S + v;
        }
        F |= f;
    }
    gS[gi][cv] = S;
    if (cv == 0) gF[gi] = F;
    __syncthreads();
    if (ch >= C) return;
    fvec<VEC> run = {};
    for (int g = 0; g < gi; ++g) run = gF[g] ? gS[g][cv] : run + gS[g][cv];
    for (int64_t c = c0; c < c1; ++c) {
        store_row<VEC>(carry + c * C + ch, run);
        const fvec<VEC> v = load_sum<VEC>(csum + c * C + ch);
        run = cflag[c] ? v : run + v;
    }
}

// EXCL: out = scale * the sum of the rows before r in its sequence (0 at a
// start) instead of up to and including r.  Tout: float32 or bf16 output.
template <typename Tin, int VEC, typename Tout, bool EXCL>
__global__ __launch_bounds__(256) void scan_finish(const Tin *__restrict__ x,
                                                   const float *__restrict__ carry,
                                                   Tout *__restrict__ out, int64_t rows, int64_t C,
                                                   const int32_t *cu, int nseq, int T, float scale) {
    using R = Row<Tin, VEC>;
    __shared__ uint32_t smask[GROUPS];
    __shared__ fvec<VEC> ssum[GROUPS][CV];
    __shared__ int sflag[GROUPS];
    const int chunk = blockIdx.x;
    const int64_t row0 = (int64_t)chunk * SCAN_CHUNK;
    start_mask(smask, row0, rows, T, cu, nseq);
    __syncthreads();
    const int rg = threadIdx.x / CV, cv = threadIdx.x % CV;
    const int64_t ch = ((int64_t)blockIdx.y * CV + cv) * VEC;
    const uint32_t mask = smask[rg];
    const int64_t r0 = row0 + ROWS_PER_GROUP * rg;
    const int nr = r0 + ROWS_PER_GROUP <= rows ? ROWS_PER_GROUP : (r0 < rows ? (int)(rows - r0) : 0);
    // the group's rows, read once and kept for the second pass
    typename R::Raw raw[ROWS_PER_GROUP];
    fvec<VEC> s = {};
    if (ch < C) {
#pragma unroll
        for (int i = 0; i < ROWS_PER_GROUP; ++i) raw[i] = i < nr ? R::load(x + (r0 + i) * C + ch) : typename R::Raw{};
#pragma unroll
        for (int i = 0; i < ROWS_PER_GROUP; ++i) {
            if ((mask >> i) & 1u) s = fvec<VEC>{};
            s += R::val(raw[i]);
        }
    }
    ssum[rg][cv] = s;
    if (cv == 0) sflag[rg] = mask != 0;
    __syncthreads();
    if (ch >= C) return;
    fvec<VEC> run = load_sum<VEC>(carry + (int64_t)chunk * C + ch);
    for (int g = 0; g < rg; ++g) run = sflag[g] ? ssum[g][cv] : run + ssum[g][cv];
#pragma unroll
    for (int i = 0; i < ROWS_PER_GROUP; ++i) {
        if ((mask >> i) & 1u) run = fvec<VEC>{};
        if (EXCL && i < nr) store_row<VEC>(out + (r0 + i) * C + ch, run * scale);
        run += R::val(raw[i]);
        if (!EXCL && i < nr) store_row<VEC>(out + (r0 + i) * C + ch, run * scale);
    }
}

template <typename Tin, int VEC, typename Tout = float, bool EXCL = false>
hipError_t run_scan(const Tin *x, Tout *out, int64_t B, int64_t T, int64_t C, const int32_t *cu,
                    int64_t nseq, float scale, void *ws, hipStream_t st) {
    const ScanLayout L = scan_layout(B, T, C);
    char *w = static_cast<char *>(ws);
    float *csum = reinterpret_cast<float *>(w + L.off_sum);
    float *carry = reinterpret_cast<float *>(w + L.off_carry);
    int32_t *cflag = reinterpret_cast<int32_t *>(w + L.off_flag);
    const int64_t rows = B * T;
    const dim3 grid((unsigned)L.nchunk, (unsigned)cdiv(C, (int64_t)CV * VEC));
    hipLaunchKernelGGL((scan_chunk_sums<Tin, VEC>), grid, dim3(256), 0, st, x, csum, cflag, rows, C,
                       cu, (int)nseq, (int)T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_chunk_carry<1>), dim3((unsigned)cdiv(C, (int64_t)CV)), dim3(CV * CARRY_GROUPS), 0,
                       st, csum, cflag, carry, L.nchunk, C);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_finish<Tin, VEC, Tout, EXCL>), grid, dim3(256), 0, st, x, carry, out, rows, C, cu,
                       (int)nseq, (int)T, scale);
    return hipGetLastError();
}

}  // namespace

namespace {

// ---------------------------------------------------------------- append
// Rows appended to a running prefix: one thread per (batch, channel), the n
// new rows in order, s += x_t, out_t = prev + scale * s.  Coalesced across
// channels; meant for the few rows of a decode step.
template <typename Tin>
__global__ __launch_bounds__(256) void prefix_append_kernel(const Tin *__restrict__ x, int64_t x_bs,
                                                            const float *__restrict__ prev, int64_t prev_bs,
                                                            float *__restrict__ out, int64_t out_bs,
                                                            int64_t B, int64_t n, int64_t C, float scale) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= B * C) return;
    const int64_t b = id / C, c = id % C;
    const float p = prev ? prev[b * prev_bs + c] : 0.f;
    const Tin *xr = x + b * x_bs + c;
    float *orow = out + b * out_bs + c;
    float s = 0.f;
    for (int64_t t = 0; t < n; ++t) {
        s += (float)xr[t * C];
        orow[t * C] = p + scale * s;
    }
}

}  // namespace

hipError_t launch_prefix_append(const void *x, bool x_bf16, int64_t x_bs, const float *prev, int64_t prev_bs,
                                float *out, int64_t out_bs, int64_t B, int64_t n, int64_t C, float scale,
                                hipStream_t st) {
    const dim3 grid((unsigned)cdiv(B * C, 256));
    if (x_bf16)
        hipLaunchKernelGGL(prefix_append_kernel<__bf16>, grid, dim3(256), 0, st, static_cast<const __bf16 *>(x),
                           x_bs, prev, prev_bs, out, out_bs, B, n, C, scale);
    else
        hipLaunchKernelGGL(prefix_append_kernel<float>, grid, dim3(256), 0, st, static_cast<const float *>(x),
                           x_bs, prev, prev_bs, out, out_bs, B, n, C, scale);
    return hipGetLastError();
}

hipError_t launch_scan_excl(const float *x, void *out, bool out_bf16, int64_t B, int64_t T, int64_t C,
                            const int32_t *cu, int64_t nseq, float scale, void *ws, hipStream_t st) {
    const bool vec = (C % 4) == 0;
    if (out_bf16) {
        __bf16 *o = static_cast<__bf16 *>(out);
        return vec ? run_scan<float, 4, __bf16, true>(x, o, B, T, C, cu, nseq, scale, ws, st)
                   : run_scan<float, 1, __bf16, true>(x, o, B, T, C, cu, nseq, scale, ws, st);
    }
    float *o = static_cast<float *>(out);
    return vec ? run_scan<float, 4, float, true>(x, o, B, T, C, cu, nseq, scale, ws, st)
               : run_scan<float, 1, float, true>(x, o, B, T, C, cu, nseq, scale, ws, st);
}

hipError_t launch_scan_chunk_sums(const void *x, bool x_bf16, int64_t B, int64_t T, int64_t C, void *ws,
                                  hipStream_t st) {
    const ScanLayout L = scan_layout(B, T, C);
    char *w = static_cast<char *>(ws);
    float *csum = reinterpret_cast<float *>(w + L.off_sum);
    int32_t *cflag = reinterpret_cast<int32_t *>(w + L.off_flag);
    const int64_t rows = B * T;
    if (x_bf16 && C % 8 == 0) {
        const dim3 grid((unsigned)L.nchunk, (unsigned)cdiv(C, (int64_t)CV * 8));
        hipLaunchKernelGGL((scan_chunk_sums<__bf16, 8>), grid, dim3(256), 0, st, static_cast<const __bf16 *>(x), csum,
                           cflag, rows, C, nullptr, 0, (int)T);
    } else if (!x_bf16 && C % 4 == 0) {
        const dim3 grid((unsigned)L.nchunk, (unsigned)cdiv(C, (int64_t)CV * 4));
        hipLaunchKernelGGL((scan_chunk_sums<float, 4>), grid, dim3(256), 0, st, static_cast<const float *>(x), csum,
                           cflag, rows, C, nullptr, 0, (int)T);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_scan(const void *x, bool x_bf16, float *out, int64_t B, int64_t T, int64_t C,
                       const int32_t *cu, int64_t nseq, float scale, void *ws, hipStream_t st) {
    const bool vec = (C % 4) == 0;
    if (x_bf16) {
        const __bf16 *xb = static_cast<const __bf16 *>(x);
        return (C % 8) == 0 ? run_scan<__bf16, 8>(xb, out, B, T, C, cu, nseq, scale, ws, st)
                            : run_scan<__bf16, 1>(xb, out, B, T, C, cu, nseq, scale, ws, st);
    }
    const float *xf = static_cast<const float *>(x);
    return vec ? run_scan<float, 4>(xf, out, B, T, C, cu, nseq, scale, ws, st)
               : run_scan<float, 1>(xf, out, B, T, C, cu, nseq, scale, ws, st);
}

}  // namespace wall
