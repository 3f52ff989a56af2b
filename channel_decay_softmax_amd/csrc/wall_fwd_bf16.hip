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
//       diagonal tile) and that test follows the exps, so it does not split
//       the MFMA/VALU interleave;
//   O^T += v^T p^T on the same MFMA, p as bf16.
//
// Interior tiles overlap the two units across sub-blocks: the QK of sub-block
// b and then the PV of sub-block b+1 are issued before the softmax of b, so
// the matrix cores run that PV while the vector ALUs take the softmax.
// Diagonal and window-boundary tiles take a plain masked loop.
//
// The key rows fed to the S^T MFMA are permuted (bits 2 and 3 of the row
// index swapped) so each lane's output registers come out as runs of 8
// consecutive keys: exactly the k-slots the PV MFMA needs from that lane.
// LDS rows keep their 16-byte chunks XOR-swizzled by the row index, which
// makes every MFMA fragment read free of bank conflicts.
#include <float.h>

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

__device__ inline float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <int K, int V>
struct Smem {
    __bf16 k[2][TILE * K];      // rescaled keys, row = key, 16-byte chunks swizzled
    __bf16 v[2][V * TILE];      // values transposed, row = value channel, swizzled
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
template <int K, int V>
__device__ inline void shift_qop(const Smem<K, V> &sm, int buf, int hl, QOp<K> &qop) {
    constexpr int KS = K / 16;
#pragma unroll
    for (int s8 = 0; s8 < KS; ++s8) {
        const uint4 d = *reinterpret_cast<const uint4 *>(&sm.dsh[buf][8 * s8 + 4 * hl]);
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

// S^T for sub-block b (32 keys) against both n-blocks.
template <int K, int V>
__device__ inline void qk(const Smem<K, V> &sm, int buf, int b, int col, int hl, const QOp<K> &qop,
                          f32x16 (&S)[NB]) {
    constexpr int KS = K / 16, CPR = K / 8;
    const int row = SB * b + key_perm(col);
    const __bf16 *base = sm.k[buf] + row * K;
#pragma unroll
    for (int s8 = 0; s8 < KS; ++s8) {
        const int ch = (2 * s8 + hl) ^ (row % CPR);
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(base + ch * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            S[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[nb][s8], s8 ? S[nb] : f32x16{}, 0, 0, 0);
    }
}

// O^T += v^T p^T for sub-block b (two 16-key MFMA k-steps).
template <int K, int V>
__device__ inline void pv(const Smem<K, V> &sm, int buf, int b, int col, int hl,
                          const bf16x8 (&P)[NB][2], Acc<V> &acc) {
    constexpr int VT = V / 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ks = 2 * b + t;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const int row = 32 * vt + col;
            const int ch = (2 * ks + hl) ^ (row % 16);
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sm.v[buf] + row * TILE + ch * 8);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc.O[nb][vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[nb][t], acc.O[nb][vt], 0, 0, 0);
        }
    }
}

// Online softmax of one sub-block's scores into bf16 p, one n-block at a
// time.  MASKED applies causality, the window and the sequence end; HAS_G
// subtracts the keys' scalar-gate prefix (the query's own G_i is added back
// in the epilogue).
template <int K, int V, bool MASKED, bool HAS_G>
__device__ inline void softmax(const Smem<K, V> &sm, int buf, int b, int hl, const f32x16 (&S)[NB],
                               Acc<V> &acc, bf16x8 (&P)[NB][2], int key0, const int (&qrow)[NB],
                               int len, int window) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        float x[16], p[16];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kin = SB * b + 16 * (r / 8) + 8 * hl + (r % 8);  // key within the tile
            float y = S[nb][r];
            if (HAS_G) y -= sm.gk[buf][kin];
            if (MASKED) {
                const int key = key0 + kin;
                bool vis = key <= qrow[nb] && key < len;
                if (window > 0) vis = vis && (qrow[nb] - key < window);
                y = vis ? y : -INFINITY;
            }
            x[r] = y;
            mx = fmaxf(mx, y);
        }
        const float mt = fmaxf(mx, xor32(mx));
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(x[r] - acc.m[nb]);
        if (__any(mt > acc.m[nb] + RESCALE)) {  // rare after the first tiles: raise the max, redo
            const float m_new = fmaxf(acc.m[nb], mt);
            const float alpha = fast_exp2(acc.m[nb] - m_new);
#pragma unroll
            for (int vt = 0; vt < V / 32; ++vt) acc.O[nb][vt] *= alpha;
            acc.l[nb] *= alpha;
            acc.m[nb] = m_new;
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(x[r] - m_new);
        }
        float sum = acc.l[nb];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x8 pv8;
#pragma unroll
            for (int e = 0; e < 8; ++e) pv8[e] = p[8 * t + e];
            P[nb][t] = __builtin_convertvector(pv8, bf16x8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // row sum of the rounded p, as the PV product sees it
                const bf16x2 pr = {P[nb][t][2 * e], P[nb][t][2 * e + 1]};
                sum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, sum, false);
            }
        }
        acc.l[nb] = sum;
    }
}

// Direct global->LDS copy of one key tile (k~) and one value tile (v^T) into
// buffer `buf`.  Each wave instruction writes 1 KB of LDS lane-linearly; the
// source address of each lane realises the XOR chunk swizzle.
template <int K, int V>
__device__ inline void load_tile(Smem<K, V> &sm, int buf, const __bf16 *kt, const __bf16 *vt,
                                 int w, int lane) {
    constexpr int CPR = K / 8;
#pragma unroll
    for (int i = 0; i < K / (4 * NW); ++i) {
        const int x = (i * NW + w) * 64 + lane;
        const int row = x / CPR, pch = x % CPR;
        const __bf16 *src = kt + row * K + ((pch ^ (row % CPR)) * 8);
        __bf16 *dst = sm.k[buf] + (i * NW + w) * 512;
        __builtin_amdgcn_global_load_lds((glb_cvoid *)src, (lds_void *)dst, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V / (4 * NW); ++i) {
        const int x = (i * NW + w) * 64 + lane;
        const int row = x / 16, pch = x % 16;
        const __bf16 *src = vt + row * TILE + ((pch ^ (row % 16)) * 8);
        __bf16 *dst = sm.v[buf] + (i * NW + w) * 512;
        __builtin_amdgcn_global_load_lds((glb_cvoid *)src, (lds_void *)dst, 16, 0, 0);
    }
}

template <int K, int V, bool HAS_G>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    constexpr int KS = K / 16, VT = V / 32;
    __shared__ __attribute__((aligned(16))) Smem<K, V> sm;

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
                    sm.dsh[bb][pv_j] = s0 | (s1 << 16);
                }
                const bool any_up = __any(up);
                if (tid == 0) sm.grow[bb] = any_up;
            }
            if (HAS_G && tid < TILE) sm.gk[bb][tid] = gval;
            rp0 = rc0;
            rp1 = rc1;
        };
        auto kt_tile = [&](int c) { return ktg + ((int64_t)(sg.tile_base + c) * HQ + hq) * TILE * K; };
        auto vt_tile = [&](int c) { return vtg + ((int64_t)(sg.tile_base + c) * a.H + h) * V * TILE; };

        // ---- prologue: tile c_hi into buffer 0
        int buf = 0;
        __syncthreads();  // the previous block's last reads of both buffers are done
        fetch_rows(c_hi);
        load_tile<K, V>(sm, 0, kt_tile(c_hi), vt_tile(c_hi), w, lane);
        write_rows(0, true);
        if (c_hi - 1 >= c_lo) fetch_rows(c_hi - 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int c = c_hi; c >= c_lo; --c) {
            if (c - 1 >= c_lo) load_tile<K, V>(sm, buf ^ 1, kt_tile(c - 1), vt_tile(c - 1), w, lane);

            if (wave_on && c <= qt_w) {
                const bool diag = c == qt_w;
                const bool wtile = a.window > 0 && q0w + WQ - 1 - TILE * c >= a.window;
                const int key0 = TILE * c;
                if (diag || sm.grow[buf]) load_qop<K>(a, sg, hq, c, qrow, hl, qop);
                else shift_qop<K, V>(sm, buf, hl, qop);
                if (!diag && !wtile) {
                    // interior tile: per sub-block, QK(b) is issued, then PV(b+1) -- which
                    // does not depend on it -- so the matrix cores run PV(b+1) while the
                    // vector ALUs take the softmax of sub-block b
                    bf16x8 Pn[NB][2];
#pragma unroll
                    for (int b = NSB - 1; b >= 0; --b) {
                        f32x16 S[NB];
                        bf16x8 P[NB][2];
                        qk<K, V>(sm, buf, b, col, hl, qop, S);
                        if (b < NSB - 1) pv<K, V>(sm, buf, b + 1, col, hl, Pn, acc);
                        softmax<K, V, false, HAS_G>(sm, buf, b, hl, S, acc, P, key0, qrow, sg.len, 0);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            Pn[nb][0] = P[nb][0];
                            Pn[nb][1] = P[nb][1];
                        }
                    }
                    pv<K, V>(sm, buf, 0, col, hl, Pn, acc);
                } else {
                    // diagonal / window-boundary tile: masked, sub-blocks wholly in the
                    // future of all this wave's queries skipped
                    const int b_hi = diag ? min(3, (q0w + WQ - 1 - key0) / SB) : 3;
                    for (int b = b_hi; b >= 0; --b) {
                        f32x16 S[NB];
                        bf16x8 P[NB][2];
                        qk<K, V>(sm, buf, b, col, hl, qop, S);
                        softmax<K, V, true, HAS_G>(sm, buf, b, hl, S, acc, P, key0, qrow, sg.len,
                                                   a.window);
                        pv<K, V>(sm, buf, b, col, hl, P, acc);
                    }
                }
            }

            __builtin_amdgcn_s_waitcnt(0);  // tile c-1 has landed in LDS, its rows in registers
            if (c - 1 >= c_lo) {
                write_rows(buf ^ 1, false);
                if (c - 2 >= c_lo) fetch_rows(c - 2);
            }
            __syncthreads();
            buf ^= 1;
        }

        // ---- epilogue: sink, normalisation, o and lse
        if (wave_on) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float l_tot = acc.l[nb] + xor32(acc.l[nb]);
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
