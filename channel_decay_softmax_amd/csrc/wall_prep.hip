// wall_prep.hip -- per-call preparation for the fused forward, one launch.
//
// Each block takes one 128-row tile of one sequence and either one query
// head (keys) or one kv head (values):
// 1. segments: the block finds the sequence its tile belongs to (one SegInfo
//    per sequence: start row, length, index of its first 128-row tile in the
//    tiled workspace; tiles never straddle two sequences, so a tile's rows
//    always share one prefix P); block (0, 0) also stores the table.
// 2. keys, per (tile, query head): the anchors R[n] = floor(P[a][n]) at the
//    tile's last row a, the carry record that moves a query from this tile's
//    anchors to the previous tile's, and the decay-rescaled keys
//        k~[j][n] = k[j][n] * exp2(R[n] - P[j][n]),
//    zero-padded to 128 rows.  This is the blog's per-tile anchor split
//    ("Fast training and inference", per-tile anchors:
//    exp2(P_i - P_j) = exp2(P_i - R) * exp2(R - P_j)) applied on the key
//    side once per (tile, head) instead of once per (query tile, key tile);
//    it is the same fold the README's decode cache performs with
//    k_tilde[j] = k[j] * exp2(R_c - P[j]).  The fused kernel reads these
//    keys only from queries after the tile, and the last row lies between
//    every such pair: for a prefix that falls, both factors are at most
//    about 1, so a factor that underflows belongs to a negligible term, at
//    any gate strength.  (Keys of a query's own tile are handled inside the
//    fused kernel from the raw keys.)
// 3. values, per (tile, kv head): v transposed to [V][128] for the bf16 MFMA
//    kernel (its PV operand reads keys contiguously, each thread transposing
//    an 8 x 8 block in registers); zero-padded.
// The float32 forward reads the raw tensors; for it only the sequence table
// is written (one block).
#include "wall_common.h"

namespace wall {
namespace {

// The sequence that holds tile `tile` (false past the last tile); block
// (0, 0) also stores the whole table.  Wave 0 scans the per-sequence tile
// counts 64 sequences at a time.
__device__ inline bool block_segment(const PrepArgs &a, int tile, bool write_table, SegInfo &out) {
    const int nseg = (int)a.nseg;
    if (!a.cu) {  // B sequences of T rows
        const int T = (int)a.T, tps = (T + TILE - 1) / TILE;
        if (write_table)
            for (int i = threadIdx.x; i < nseg; i += blockDim.x) a.seg[i] = SegInfo{i * T, T, i * tps, 0};
        const int s = tile / tps;
        out = SegInfo{s * T, T, s * tps, 0};
        return s < nseg;
    }
    __shared__ int found[4];
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        if (lane == 0) found[3] = 0;
        int run = 0;
        for (int g0 = 0; g0 < nseg; g0 += 64) {
            const int s = g0 + lane;
            const int start = s < nseg ? a.cu[s] : 0;
            const int len = s < nseg ? a.cu[s + 1] - start : 0;
            const int cnt = (len + TILE - 1) / TILE;
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off);
                if (lane >= off) incl += v;
            }
            const int base = run + incl - cnt;
            if (s < nseg) {
                if (write_table) a.seg[s] = SegInfo{start, len, base, 0};
                if (tile >= base && tile < base + cnt) {
                    found[0] = start;
                    found[1] = len;
                    found[2] = base;
                    found[3] = 1;
                }
            }
            run += __shfl(incl, 63);
        }
    }
    __syncthreads();
    out = SegInfo{found[0], found[1], found[2], 0};
    return found[3] != 0;
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

template <typename T, int K>
__device__ inline void key_tile(const PrepArgs &a, int tile, int hq, const SegInfo &sg) {
    constexpr int CPR = K / 8;          // 8-channel chunks per row
    constexpr int RPP = 256 / CPR;      // rows per pass
    constexpr int NPASS = TILE / RPP;
    const int c = tile - sg.tile_base;
    const int h = hq / (int)(a.HQ / a.H);
    const int c8 = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    const int arow = min(c * TILE + TILE - 1, sg.len - 1);
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
                const int prow = c * TILE - 1;  // anchor row of tile c-1: its last row
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
    // all of the thread's rows in flight before any is used
    f32x8 kv[NPASS], pv[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int j = c * TILE + r0 + p * RPP;
        kv[p] = f32x8{};
        pv[p] = f32x8{};
        if (j < sg.len) {
            const int64_t tok = sg.start + j;
            kv[p] = Vec8<T>::load(kin + (tok * a.H + h) * K + c8 * 8);
            pv[p] = *reinterpret_cast<const f32x8 *>(a.P + (tok * a.HQ + hq) * K + c8 * 8);
        }
    }
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        f32x8 out;
        for (int e = 0; e < 8; ++e) out[e] = kv[p][e] * exp2f(fminf(fmaxf(R[e] - pv[p][e], EXP2_LO), EXP2_HI));
        Vec8<T>::store(kout + (r0 + p * RPP) * K + c8 * 8, out);
    }
}

// Value tile of (tile, kv head), transposed [V][TILE].  Thread (kb, db)
// moves the 8 x 8 block of keys 8kb.. and values 8db..
template <typename T, int V>
__device__ inline void value_tile(const PrepArgs &a, int tile, int h, const SegInfo &sg) {
    constexpr int DB = V / 8, KB = TILE / 8;
    const int c = tile - sg.tile_base;
    const T *vin = static_cast<const T *>(a.v);
    T *vout = static_cast<T *>(a.vt) + ((int64_t)tile * a.H + h) * V * TILE;
    for (int t = threadIdx.x; t < DB * KB; t += blockDim.x) {
        const int db = t % DB, kb = t / DB;
        f32x8 x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = c * TILE + kb * 8 + i;
            x[i] = j < sg.len ? Vec8<T>::load(vin + ((int64_t)(sg.start + j) * a.H + h) * V + db * 8) : f32x8{};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f32x8 col;
#pragma unroll
            for (int i = 0; i < 8; ++i) col[i] = x[i][e];
            Vec8<T>::store(vout + (db * 8 + e) * TILE + kb * 8, col);
        }
    }
}

// Block id = tile * (HQ + H) + y; y < HQ: keys of query head y, else values
// of kv head y - HQ.  The heads of one tile are neighbours in launch order, so
// the query heads that share a kv head read its key rows from L2.
template <int K, int V>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    const int nh = (int)(a.HQ + a.H);
    const int tile = blockIdx.x / nh, y = blockIdx.x % nh;
    SegInfo sg;
    if (!block_segment(a, tile, tile == 0 && y == 0, sg)) return;  // beyond the last used tile
    if ((tile - sg.tile_base) * TILE >= sg.len) return;
    if (y < a.HQ)
        key_tile<__bf16, K>(a, tile, y, sg);
    else
        value_tile<__bf16, V>(a, tile, y - (int)a.HQ, sg);
}

// The sequence table alone (the float32 forward reads the raw tensors).
__global__ __launch_bounds__(256) void seg_table_kernel(PrepArgs a) {
    SegInfo sg;
    block_segment(a, 0, true, sg);
}

template <int K, int V>
hipError_t run_prep(const PrepArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((prep_kernel<K, V>), dim3((unsigned)((a.HQ + a.H) * a.tiles)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st) {
    if (!bf16) {
        hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if (a.K == 64 && a.V == 64) return run_prep<64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_prep<64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_prep<128, 64>(a, st);
    return run_prep<128, 128>(a, st);
}

}  // namespace wall
