// wall_fwd_bf16.hip -- fused causal Wall Attention forward, bf16 inputs, gfx950.
//
// Work decomposition.  A workgroup (4 waves) owns one (sequence, query head)
// and two 256-row query blocks, u and n-1-u, so every workgroup of a causal
// launch does the same number of tile pairs.  Wave w owns query rows
// 256u + 64w .. +63 as two 32-column MFMA n-blocks; its diagonal 128-row
// anchor tile is 2u + w/2.  Workgroup ids are remapped so each XCD receives a
// contiguous range of heads (their key caches then share that XCD's L2).
//
// Per key tile c (the block's last tile first, then older tiles down to the
// first tile the window reaches), with the tile's rescaled keys k~ and
// transposed values double-buffered in LDS by direct global->LDS loads (the
// next tile streams in while this one is computed):
//
//   q~  the wave's bf16 queries anchored at tile c, q * scale*log2e *
//       exp2(P_i - Rc).  Built from q and P at the wave's diagonal tile, then
//       carried from tile c+1 to tile c by lowering each bf16 exponent field
//       by the integer Rc - Rc+1 (>= 0 while the prefix does not grow) with a
//       saturating packed subtract: exact, and a value that would leave the
//       bf16 range becomes 0 and, the decay only growing further back, stays
//       negligible.  A tile where some channel's prefix grows rebuilds q~ from
//       q and P.  These are the per-tile anchors of the blog's "Fast training
//       and inference" section, with the key-side factor exp2(Rc - P_j)
//       already folded into k~;
//   S^T = k~ q~^T on v_mfma_f32_32x32x16_bf16 per 32-key sub-block, one query
//       column per lane, so all softmax state stays in-lane;
//   softmax online in the log2 domain, fp32; the running max is raised only
//       when a sub-block exceeds it by more than RESCALE (rare after the
//       diagonal tile); O is then rescaled in a branch of its own, after the
//       P formed with the old max has been accumulated;
//   O^T += v^T p^T on the same MFMA, p as bf16.
//
// Interior tiles are software-pipelined over their four 32-key sub-blocks:
// the exps of sub-block b share one basic block with the QK MFMAs of b-1 and
// the PV MFMAs of b+1, so a single wave keeps the matrix cores and the vector
// ALUs busy together.
// Diagonal and window-boundary tiles take a plain masked loop.
//
// The key rows fed to the S^T MFMA are permuted (bits 2 and 3 of the row
// index swapped) so each lane's output registers come out as runs of 8
// consecutive keys: exactly the k-slots the PV MFMA needs from that lane.
// LDS tiles are stored as 1 KB blocks padded to 1040 bytes, with the rows of
// a tile interleaved across blocks (row j in block j % NBLK): one wave's
// direct load fills exactly one block, the 16 rows an MFMA fragment read
// touches lie in 16 different blocks (distinct bank groups), and every
// fragment address is one per-lane base plus an immediate.
#include <float.h>

#include <type_traits>

#include "wall_common.h"

namespace wall {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_cvoid;

constexpr int NB = 1;          // 32-column MFMA n-blocks (query groups) per wave
constexpr int WQ = 32 * NB;    // query rows per wave
constexpr int BQ = 2 * TILE;   // query rows per block: two anchor tiles
constexpr int NW = BQ / WQ;    // waves per workgroup
constexpr int SB = 32;         // keys per sub-block (one MFMA m-tile)
constexpr int NSB = TILE / SB; // sub-blocks per tile
constexpr float RESCALE = 10.0f;  // log2 headroom before the running max is raised

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key row (within a 32-row block) that MFMA A-row m reads: bits 2 and 3 swapped.
__device__ inline int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Combine a value with the one held by lane ^ 32 (the other half of the wave
// holds the same query's other keys): after v_permlane32_swap each lane holds
// both halves' values, one in each result.
__device__ inline float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One tile as 1 KB blocks of whole rows (ROWB bytes each), row j stored in
// block j % NBLK at slot j / NBLK; blocks are BLK_PITCH bytes apart.
constexpr int BLK_PITCH = 1040;
template <int NROWS, int ROWB>
struct TileLayout {
    static constexpr int NBLK = NROWS * ROWB / 1024;
    static constexpr int BYTES = NBLK * BLK_PITCH;
    static __device__ inline int byte(int row) { return (row % NBLK) * BLK_PITCH + (row / NBLK) * ROWB; }
};

template <int K, int V>
struct Layouts {
    using KL = TileLayout<TILE, 2 * K>;  // rescaled keys, row = key
    using VL = TileLayout<V, 2 * TILE>;  // values transposed, row = value channel
};

// Small per-tile rows, double-buffered like the tiles.
template <int K>
struct TileRows {
    uint32_t dsh[2][K / 2];     // per buffer: 128*(Rc - Rc+1) per channel pair, as two u16
    int32_t grow[2];            // some channel has Rc < Rc+1 (its prefix grows over the tile)
    float gk[2][TILE];          // G (log2) of the tile's keys; 0 beyond the sequence
};

// One lane's accumulators and softmax state for its two query columns.
template <int V>
struct Acc {
    f32x16 O[NB][V / 32];
    float m[NB], l[NB];
};

template <int K>
using QOp = bf16x8[NB][K / 16];  // [n-block][k-step]: 8 channels 16*s8 + 8*hl + e of one query

// q~ at tile c straight from q and P: bf16(q * scale*log2e * exp2(P_i - Rc)).
template <int K>
__device__ inline void load_qop(const FwdArgs &a, const SegInfo &sg, int hq, int c, const int (&qrow)[NB],
                                int hl, QOp<K> &qop) {
    constexpr int KS = K / 16;
    const int64_t HQ = a.HQ;
    const __bf16 *qg = static_cast<const __bf16 *>(a.q);
    const float *Rc = a.anchor + ((int64_t)(sg.tile_base + c) * HQ + hq) * K;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const bool valid = qrow[nb] < sg.len;
        const int64_t tok = (int64_t)sg.start + (valid ? qrow[nb] : 0);
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8) {
            const int ch0 = 16 * s8 + 8 * hl;
            const bf16x8 qv = *reinterpret_cast<const bf16x8 *>(qg + (tok * HQ + hq) * K + ch0);
            const f32x8 pv8 = *reinterpret_cast<const f32x8 *>(a.P + (tok * HQ + hq) * K + ch0);
            const f32x8 rv = *reinterpret_cast<const f32x8 *>(Rc + ch0);
            f32x8 qh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xe = fminf(fmaxf(pv8[e] - rv[e], EXP2_LO), EXP2_HI);
                qh[e] = valid ? (float)qv[e] * a.qscale * exp2f(xe) : 0.f;
            }
            qop[nb][s8] = __builtin_convertvector(qh, bf16x8);
        }
    }
}

// Carry q~ from tile c+1's anchor to tile c's: lower each bf16 exponent field
// by 128*(Rc - Rc+1) with unsigned saturation on the magnitude, keeping the
// sign.  Exact while the result is a normal number; a value pushed out of
// range becomes 0 (or a bf16 denormal).
template <int K>
__device__ inline void shift_qop(const TileRows<K> &rows, int buf, int hl, QOp<K> &qop) {
    constexpr int KS = K / 16;
#pragma unroll
    for (int s8 = 0; s8 < KS; ++s8) {
        const uint4 d = *reinterpret_cast<const uint4 *>(&rows.dsh[buf][8 * s8 + 4 * hl]);
        const uint32_t dv[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint4 x4 = __builtin_bit_cast(uint4, qop[nb][s8]);
            const uint32_t xv[4] = {x4.x, x4.y, x4.z, x4.w};
            uint32_t out[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u16x2 mag = __builtin_bit_cast(u16x2, xv[e] & 0x7fff7fffu);
                const u16x2 r = __builtin_elementwise_sub_sat(mag, __builtin_bit_cast(u16x2, dv[e]));
                out[e] = (xv[e] & 0x80008000u) | __builtin_bit_cast(uint32_t, r);
            }
            qop[nb][s8] = __builtin_bit_cast(bf16x8, uint4{out[0], out[1], out[2], out[3]});
        }
    }
}

// Key fragments of sub-block b (A operands of the S^T MFMAs): lane (col, hl)
// reads key row 32b + perm(col), channels 16*s8 + 8*hl .. +7.
template <int K>
__device__ inline void load_kfrag(const char *kb, int b, int kbase, bf16x8 (&kf)[K / 16]) {
    using KL = typename Layouts<K, K>::KL;
    // key 32b + perm(col): same block as key perm(col), (32 / NBLK) * b slots further
    const char *base = kb + kbase + b * (SB / KL::NBLK) * (2 * K);
#pragma unroll
    for (int s8 = 0; s8 < K / 16; ++s8) kf[s8] = *reinterpret_cast<const bf16x8 *>(base + 32 * s8);
}

// S^T for one sub-block (32 keys) against the wave's n-blocks.
template <int K>
__device__ inline void qk(const bf16x8 (&kf)[K / 16], const QOp<K> &qop, f32x16 (&S)[NB]) {
#pragma unroll
    for (int s8 = 0; s8 < K / 16; ++s8)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            S[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s8], qop[nb][s8], s8 ? S[nb] : f32x16{}, 0, 0, 0);
}

// O^T += v^T p^T for sub-block b (two 16-key MFMA k-steps).
template <int K, int V>
__device__ inline void pv(const char *vb, int b, int vbase, const bf16x8 (&P)[NB][2], Acc<V> &acc) {
    constexpr int VT = V / 32;
    using VL = typename Layouts<K, V>::VL;
    const char *base = vb + vbase;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ks = 2 * b + t;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            // lane (col, hl): value row 32*vt + col, keys 16*ks + 8*hl .. +7
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                base + vt * (32 / VL::NBLK) * (2 * TILE) + 32 * ks);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc.O[nb][vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[nb][t], acc.O[nb][vt], 0, 0, 0);
        }
    }
}

// Online softmax of one sub-block, first half: masked scores into x and the
// running max.  The max is raised only when the sub-block exceeds it by more
// than RESCALE; then l is rescaled here and alpha (1 otherwise) is returned
// for O, which the caller rescales with rescale_o once every P formed with
// the old max has been accumulated.  MASKED applies causality, the window
// and the sequence end; HAS_G subtracts the keys' scalar-gate prefix (the
// query's own G_i is added back in the epilogue).
template <int K, int V, bool MASKED, bool HAS_G>
__device__ inline void softmax_max(const TileRows<K> &rows, int buf, int b, int hl,
                                   const f32x16 (&S)[NB], Acc<V> &acc, float (&x)[NB][16],
                                   float (&alpha)[NB], int key0, const int (&qrow)[NB], int len,
                                   int window) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kin = SB * b + 16 * (r / 8) + 8 * hl + (r % 8);  // key within the tile
            float y = S[nb][r];
            if (HAS_G) y -= rows.gk[buf][kin];
            if (MASKED) {
                const int key = key0 + kin;
                bool vis = key <= qrow[nb] && key < len;
                if (window > 0) vis = vis && (qrow[nb] - key < window);
                y = vis ? y : -INFINITY;
            }
            x[nb][r] = y;
            mx = fmaxf(mx, y);
        }
        const float mt = pair_max(mx);
        const float m_new = mt > acc.m[nb] + RESCALE ? mt : acc.m[nb];
        alpha[nb] = fast_exp2(acc.m[nb] - m_new);
        acc.l[nb] *= alpha[nb];
        acc.m[nb] = m_new;
    }
}

// O *= alpha when some lane raised its max (rare after the first tiles).
template <int V>
__device__ inline void rescale_o(Acc<V> &acc, const float (&alpha)[NB]) {
    bool any = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) any = any || alpha[nb] != 1.0f;
    if (__any(any)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int vt = 0; vt < V / 32; ++vt) acc.O[nb][vt] *= alpha[nb];
    }
}

// Second half: p = exp2(x - m) as bf16 (the PV operand) and the row sum of
// the rounded p, as the PV product sees it.
template <int V>
__device__ inline void softmax_exp(const float (&x)[NB][16], Acc<V> &acc, bf16x8 (&P)[NB][2]) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        float sum = acc.l[nb];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x8 pv8;
#pragma unroll
            for (int e = 0; e < 8; ++e) pv8[e] = fast_exp2(x[nb][8 * t + e] - acc.m[nb]);
            P[nb][t] = __builtin_convertvector(pv8, bf16x8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pr = {P[nb][t][2 * e], P[nb][t][2 * e + 1]};
                sum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum, false);
            }
        }
        acc.l[nb] = sum;
    }
}

// Direct global->LDS copy of one key tile (k~) and one value tile (v^T) into
// buffer `buf`: one wave instruction per 1 KB block, written lane-linearly;
// lane l fetches 16 bytes of the block's row l / (ROWB/16).
template <int K, int V>
__device__ inline void load_tile(char *kd, char *vd, const __bf16 *kt, const __bf16 *vt, int w,
                                 int lane) {
    using KL = typename Layouts<K, V>::KL;
    using VL = typename Layouts<K, V>::VL;
    constexpr int KCPR = K / 8, VCPR = TILE / 8;  // 16-byte chunks per row
    static_assert(KL::NBLK % NW == 0 && VL::NBLK % NW == 0, "blocks split evenly over waves");
#pragma unroll
    for (int i = 0; i < KL::NBLK / NW; ++i) {
        const int blk = i * NW + w;
        const int row = (lane / KCPR) * KL::NBLK + blk;
        const __bf16 *src = kt + row * K + (lane % KCPR) * 8;
        __builtin_amdgcn_global_load_lds((glb_cvoid *)src, (lds_void *)(kd + blk * BLK_PITCH),
                                         16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VL::NBLK / NW; ++i) {
        const int blk = i * NW + w;
        const int row = (lane / VCPR) * VL::NBLK + blk;
        const __bf16 *src = vt + row * TILE + (lane % VCPR) * 8;
        __builtin_amdgcn_global_load_lds((glb_cvoid *)src, (lds_void *)(vd + blk * BLK_PITCH),
                                         16, 0, 0);
    }
}

template <int K, int V, bool HAS_G>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    constexpr int KS = K / 16, VT = V / 32;
    using KL = typename Layouts<K, V>::KL;
    using VL = typename Layouts<K, V>::VL;
    // Each tile buffer is an LDS variable of its own: the compiler then knows
    // that reading one buffer does not depend on the direct loads still
    // filling the other, and does not wait for them.
    __shared__ __attribute__((aligned(16))) char k0[KL::BYTES];
    __shared__ __attribute__((aligned(16))) char k1[KL::BYTES];
    __shared__ __attribute__((aligned(16))) char v0[VL::BYTES];
    __shared__ __attribute__((aligned(16))) char v1[VL::BYTES];
    __shared__ TileRows<K> rows;

    const int nblocks_max = (a.max_tiles + 1) / 2;  // 256-row blocks of the longest sequence
    const int npairs = (nblocks_max + 1) / 2;
    const int nwork = a.nseg * npairs * a.HQ;
    int bid = blockIdx.x;
    // Workgroups are dispatched round robin over the 8 XCDs; give each XCD a
    // contiguous range of work ids so the tiles of one head share an L2.
    if (nwork % 8 == 0) bid = (bid % 8) * (nwork / 8) + bid / 8;
    const int hq = bid / (a.nseg * npairs);
    const int rem = bid % (a.nseg * npairs);
    const int s = rem / npairs, p = rem % npairs;
    const SegInfo sg = a.seg[s];
    const int ntiles = (sg.len + TILE - 1) / TILE;
    const int nblk = (sg.len + BQ - 1) / BQ;
    if (p >= (nblk + 1) / 2) return;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hl = lane >> 5;
    const int var = w / (NW / 2);  // which of the block's two anchor tiles is this wave's diagonal
    // per-lane byte offsets of the MFMA fragments in a tile buffer
    const int kbase = KL::byte(key_perm(col)) + 16 * hl;
    const int vbase = VL::byte(col) + 16 * hl;
    const int h = hq / (a.HQ / a.H);
    const __bf16 *qg = static_cast<const __bf16 *>(a.q);
    const __bf16 *ktg = static_cast<const __bf16 *>(a.kt);
    const __bf16 *vtg = static_cast<const __bf16 *>(a.vt);
    __bf16 *og = static_cast<__bf16 *>(a.o);
    const int64_t HQ = a.HQ;
    // threads 0..63 prepare a channel pair of each tile's shift row, threads 0..127 one key's G
    const int pv_j = tid;
    const bool pv_pair = tid < 64 && 2 * pv_j < K;

    for (int pass = 0; pass < 2; ++pass) {
        const int u = pass == 0 ? p : nblk - 1 - p;
        if (pass == 1 && u == p) break;
        const int qt_w = 2 * u + var;
        const int q0w = BQ * u + WQ * w;
        const bool wave_on = q0w < sg.len;
        int qrow[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) qrow[nb] = q0w + 32 * nb + col;
        const int c_hi = min(2 * u + 1, ntiles - 1);
        int c_lo = 0;
        if (a.window > 0) {
            const int kmin = BQ * u - a.window + 1;
            c_lo = kmin > 0 ? kmin / TILE : 0;
        }

        float g_i[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) g_i[nb] = 0.f;
        if (HAS_G && wave_on) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                if (qrow[nb] < sg.len) g_i[nb] = a.G[((int64_t)sg.start + qrow[nb]) * HQ + hq];
        }
        QOp<K> qop;

        Acc<V> acc;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) acc.O[nb][vt] = f32x16{};
            acc.m[nb] = -FLT_MAX;
            acc.l[nb] = 0.f;
        }

        // per-tile rows prepared by threads 0..127: the anchor pair of the tile being
        // prepared (rc) and of the tile after it (rp), and one key's G
        float rc0 = 0.f, rc1 = 0.f, rp0 = 0.f, rp1 = 0.f, gval = 0.f;
        auto fetch_rows = [&](int c) {
            if (pv_pair) {
                const float *R = a.anchor + ((int64_t)(sg.tile_base + c) * HQ + hq) * K;
                rc0 = R[2 * pv_j];
                rc1 = R[2 * pv_j + 1];
            }
            if (HAS_G && tid < TILE) {
                const int j = c * TILE + tid;
                gval = j < sg.len ? a.G[((int64_t)sg.start + j) * HQ + hq] : 0.f;
            }
        };
        auto write_rows = [&](int bb, bool first) {
            if (tid < 64) {
                bool up = false;
                if (pv_pair) {
                    const float d0 = first ? 0.f : rc0 - rp0, d1 = first ? 0.f : rc1 - rp1;  // Rc - Rc+1
                    up = d0 < 0.f || d1 < 0.f;
                    const uint32_t s0 = (uint32_t)fminf(fmaxf(d0, 0.f), 255.f) * 128u;
                    const uint32_t s1 = (uint32_t)fminf(fmaxf(d1, 0.f), 255.f) * 128u;
                    rows.dsh[bb][pv_j] = s0 | (s1 << 16);
                }
                const bool any_up = __any(up);
                if (tid == 0) rows.grow[bb] = any_up;
            }
            if (HAS_G && tid < TILE) rows.gk[bb][tid] = gval;
            rp0 = rc0;
            rp1 = rc1;
        };
        auto kt_tile = [&](int c) { return ktg + ((int64_t)(sg.tile_base + c) * HQ + hq) * TILE * K; };
        auto vt_tile = [&](int c) { return vtg + ((int64_t)(sg.tile_base + c) * a.H + h) * V * TILE; };

        // ---- prologue: tile c_hi into buffer 0
        __syncthreads();  // the previous block's last reads of both buffers are done
        fetch_rows(c_hi);
        load_tile<K, V>(k0, v0, kt_tile(c_hi), vt_tile(c_hi), w, lane);
        write_rows(0, true);
        if (c_hi - 1 >= c_lo) fetch_rows(c_hi - 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // One key tile c held in buffer PB (tile c_hi in buffer 0, then alternating);
        // the buffer is a compile-time choice so every LDS access names its variable.
        auto tile_step = [&](int c, auto pb_tag) {
            constexpr int PB = decltype(pb_tag)::value;
            const char *kb = PB ? k1 : k0;
            const char *vb = PB ? v1 : v0;
            if (c - 1 >= c_lo)
                load_tile<K, V>(PB ? k0 : k1, PB ? v0 : v1, kt_tile(c - 1), vt_tile(c - 1), w, lane);

            if (wave_on && c <= qt_w) {
                const bool diag = c == qt_w;
                const bool wtile = a.window > 0 && q0w + WQ - 1 - TILE * c >= a.window;
                const int key0 = TILE * c;
                if (diag || rows.grow[PB]) load_qop<K>(a, sg, hq, c, qrow, hl, qop);
                else shift_qop<K>(rows, PB, hl, qop);
                if (!diag && !wtile) {
                    // interior tile, software-pipelined over its four sub-blocks: the
                    // exps of sub-block b share a basic block with the QK MFMAs of b-1
                    // and the PV MFMAs of b+1, so one wave keeps both units busy
                    f32x16 S[NSB][NB];
                    bf16x8 P[NSB][NB][2];
                    bf16x8 kf[K / 16];
                    load_kfrag<K>(kb, NSB - 1, kbase, kf);
                    qk<K>(kf, qop, S[NSB - 1]);
                    load_kfrag<K>(kb, NSB - 2, kbase, kf);
#pragma unroll
                    for (int b = NSB - 1; b >= 0; --b) {
                        float x[NB][16], alpha[NB];
                        softmax_max<K, V, false, HAS_G>(rows, PB, b, hl, S[b], acc, x, alpha, key0,
                                                        qrow, sg.len, 0);
                        if (b > 0) qk<K>(kf, qop, S[b - 1]);
                        if (b > 1) load_kfrag<K>(kb, b - 2, kbase, kf);
                        if (b < NSB - 1) pv<K, V>(vb, b + 1, vbase, P[b + 1], acc);
                        softmax_exp<V>(x, acc, P[b]);
                        rescale_o<V>(acc, alpha);  // O = (O + P(b+1) V) * alpha
                    }
                    pv<K, V>(vb, 0, vbase, P[0], acc);
                } else {
                    // diagonal / window-boundary tile: masked, sub-blocks wholly in the
                    // future of all this wave's queries skipped
                    const int b_hi = diag ? min(3, (q0w + WQ - 1 - key0) / SB) : 3;
                    for (int b = b_hi; b >= 0; --b) {
                        f32x16 S[NB];
                        bf16x8 P[NB][2];
                        bf16x8 kf[K / 16];
                        load_kfrag<K>(kb, b, kbase, kf);
                        qk<K>(kf, qop, S);
                        float x[NB][16], alpha[NB];
                        softmax_max<K, V, true, HAS_G>(rows, PB, b, hl, S, acc, x, alpha, key0, qrow,
                                                       sg.len, a.window);
                        rescale_o<V>(acc, alpha);
                        softmax_exp<V>(x, acc, P);
                        pv<K, V>(vb, b, vbase, P, acc);
                    }
                }
            }

            __builtin_amdgcn_s_waitcnt(0);  // tile c-1 has landed in LDS, its rows in registers
            if (c - 1 >= c_lo) {
                write_rows(PB ^ 1, false);
                if (c - 2 >= c_lo) fetch_rows(c - 2);
            }
            __syncthreads();
        };
        for (int c = c_hi; c >= c_lo; c -= 2) {
            tile_step(c, std::integral_constant<int, 0>{});
            if (c - 1 >= c_lo) tile_step(c - 1, std::integral_constant<int, 1>{});
        }

        // ---- epilogue: sink, normalisation, o and lse
        if (wave_on) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float l_tot = pair_sum(acc.l[nb]);
                const float m_true = acc.m[nb] + g_i[nb];
                float m_fin = m_true, l_fin = l_tot;
                if (a.sink) {
                    const float sb = a.sink[hq] * LOG2E;
                    m_fin = fmaxf(m_true, sb);
                    l_fin = l_tot * exp2f(m_true - m_fin) + exp2f(sb - m_fin);
                }
                const float fac = exp2f(m_true - m_fin) / l_fin;
                if (qrow[nb] < sg.len) {
                    const int64_t tok = (int64_t)sg.start + qrow[nb];
                    __bf16 *orow = og + (tok * HQ + hq) * V;
#pragma unroll
                    for (int vt = 0; vt < VT; ++vt) {
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            f32x4 y;
#pragma unroll
                            for (int e = 0; e < 4; ++e) y[e] = acc.O[nb][vt][4 * r4 + e] * fac;
                            *reinterpret_cast<bf16x4 *>(orow + 32 * vt + 8 * r4 + 4 * hl) =
                                __builtin_convertvector(y, bf16x4);
                        }
                    }
                    if (a.lse && hl == 0) a.lse[tok * HQ + hq] = (m_fin + log2f(l_fin)) * LN2;
                }
            }
        }
    }
}

template <int K, int V>
hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
    const int nblocks_max = (a.max_tiles + 1) / 2;
    const int npairs = (nblocks_max + 1) / 2;
    const int64_t nwork = (int64_t)a.nseg * npairs * a.HQ;
    if (a.G)
        hipLaunchKernelGGL((fwd_bf16_kernel<K, V, true>), dim3((unsigned)nwork), dim3(NW * 64), 0, st, a);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<K, V, false>), dim3((unsigned)nwork), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_fwd<64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_fwd<64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_fwd<128, 64>(a, st);
    return run_fwd<128, 128>(a, st);
}

}  // namespace wall
