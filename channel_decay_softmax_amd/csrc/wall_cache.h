// wall_cache.h -- the decode cache's rows and chunk anchors (device code shared
// by the cache build and the streaming append).
//
// The README's decode cache ("Decode (cached generation)") holds, per chunk
// of C rows, query head and channel, one anchor R and the keys
//     k_tilde[j] = k[j] * exp2(R - P[j]).
// R starts as floor(P) of the chunk's first row; when a later row t of the
// chunk has R - P[t] > CACHE_SPAN (its key factor would pass 2^CACHE_SPAN)
// the anchor moves to floor(P[t]) and the chunk's earlier rows are lowered by
// the exact power of two 2^(R_new - R_old).  Every cached key factor then
// stays at most 2^CACHE_SPAN, and a decode query (a row at or after every
// cached row) meets a query factor exp2(p - R) of at most 2, for any gate
// strength; a factor that underflows belongs to a term below
// 2^(CACHE_SPAN - 126) of the largest.
//
// Rows are written once at the anchor in force when they arrive and lowered
// on the bit pattern (exponent field minus the shift, 0 below the range), so
// lowering twice equals lowering once by the sum: a cache built in one call
// and the same rows appended in pieces hold the same bits.
#pragma once

#include "wall_common.h"

namespace wall {

constexpr float CACHE_SPAN = 64.0f;

template <typename T>
struct CacheIO;
template <>
struct CacheIO<__bf16> {
    using Raw = bf16x8;
    static __device__ inline f32x8 load(const __bf16 *p) {
        return __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(p), f32x8);
    }
    static __device__ inline Raw round(f32x8 v) { return __builtin_convertvector(v, bf16x8); }
    static __device__ inline Raw get(const __bf16 *p) { return *reinterpret_cast<const Raw *>(p); }
    static __device__ inline void put(__bf16 *p, Raw v) { *reinterpret_cast<Raw *>(p) = v; }
    // v * 2^-d for integer d >= 0: the exponent field lowered with a saturating
    // subtract on the magnitude
    static __device__ inline Raw lower(Raw v, f32x8 d) {
        typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
        u16x8 x = __builtin_bit_cast(u16x8, v), sh;
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[e] = (unsigned short)((uint32_t)fminf(fmaxf(d[e], 0.f), 255.f) << 7);
        const u16x8 sign = x & (unsigned short)0x8000;
        const u16x8 mag = __builtin_elementwise_sub_sat(x & (unsigned short)0x7fff, sh);
        return __builtin_bit_cast(Raw, sign | mag);
    }
};
template <>
struct CacheIO<float> {
    using Raw = f32x8;
    static __device__ inline f32x8 load(const float *p) { return *reinterpret_cast<const f32x8 *>(p); }
    static __device__ inline Raw round(f32x8 v) { return v; }
    static __device__ inline Raw get(const float *p) { return *reinterpret_cast<const Raw *>(p); }
    static __device__ inline void put(float *p, Raw v) { *reinterpret_cast<Raw *>(p) = v; }
    static __device__ inline Raw lower(Raw v, f32x8 d) {
        typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
        u32x8 x = __builtin_bit_cast(u32x8, v), sh;
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[e] = (uint32_t)fminf(fmaxf(d[e], 0.f), 255.f) << 23;
        const u32x8 sign = x & 0x80000000u;
        const u32x8 mag = __builtin_elementwise_sub_sat(x & 0x7fffffffu, sh);
        return __builtin_bit_cast(Raw, sign | mag);
    }
};

// The anchor after row t of a chunk whose anchor was R (row t not its first).
__device__ inline f32x8 cache_anchor_step(f32x8 R, f32x8 Pt) {
#pragma unroll
    for (int e = 0; e < 8; ++e) R[e] = R[e] - Pt[e] > CACHE_SPAN ? floorf(Pt[e]) : R[e];
    return R;
}

// Cache rows ja .. jb-1 (one chunk: ja / C == (jb - 1) / C) of batch row b,
// query head hq, channels 8*c8 .. +7: the chunk's anchor (read from r when the
// chunk opened before ja), the rows cached before ja lowered to the anchor
// after jb - 1, the new rows, and the anchor stored.  Pointers are at row 0
// of (b, hq) (kb: of (b, kv head)) and at channel 8*c8; rows rowP / rowK
// elements apart; Rp is the chunk's anchor slot.
template <typename T>
__device__ inline void cache_chunk(const T *kb, const float *Pb, T *ktb, float *Rp, int64_t rowP, int64_t rowK,
                                   int64_t j0, int64_t ja, int64_t jb) {
    using IO = CacheIO<T>;
    f32x8 R0 = {};
    if (ja > j0) R0 = *reinterpret_cast<const f32x8 *>(Rp);
    // the anchor after the new rows
    f32x8 Rf = R0;
    for (int64_t t = ja; t < jb; ++t) {
        const f32x8 Pt = *reinterpret_cast<const f32x8 *>(Pb + t * rowP);
        if (t == j0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) Rf[e] = floorf(Pt[e]);
        } else {
            Rf = cache_anchor_step(Rf, Pt);
        }
    }
    // rows cached by earlier calls, lowered to it
    if (ja > j0) {
        const f32x8 d = R0 - Rf;
        bool moved = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) moved = moved || d[e] > 0.f;
        if (moved)
            for (int64_t j = j0; j < ja; ++j) IO::put(ktb + j * rowP, IO::lower(IO::get(ktb + j * rowP), d));
    }
    // the new rows at the anchor in force when each arrives, lowered to Rf
    f32x8 Ra = R0;
    for (int64_t t = ja; t < jb; ++t) {
        const f32x8 Pt = *reinterpret_cast<const f32x8 *>(Pb + t * rowP);
        if (t == j0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) Ra[e] = floorf(Pt[e]);
        } else {
            Ra = cache_anchor_step(Ra, Pt);
        }
        const f32x8 kv = IO::load(kb + t * rowK);
        f32x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = kv[e] * exp2f(fminf(fmaxf(Ra[e] - Pt[e], EXP2_LO), EXP2_HI));
        IO::put(ktb + t * rowP, IO::lower(IO::round(x), Ra - Rf));
    }
    *reinterpret_cast<f32x8 *>(Rp) = Rf;
}

}  // namespace wall
