// wall_bwd_mfma.hip -- backward of the causal Wall Attention forward for bf16
// inputs on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation).  Same gradients as the float32 kernels of wall_bwd.hip:
//     dS_ij = A_ij (do_i . v_j - D_i),  dv_j = sum_i A_ij do_i,
//     dq_i  = scale 2^(P_i - R) sum_j dS_ij k~_j,
//     dk_j  = ln2 2^(R - P_j) sum_i dS_ij q~_i            (per query head),
// with q~ = q scale log2e 2^(P - R) and k~ = k 2^(R - P) rounded to bf16, A and
// dS rounded to bf16 as MFMA operands, everything else in float32.
//
// Work decomposition.  A block owns one 128-row tile of one (query head,
// sequence): keys in the dk/dv kernel, queries in the dq kernel; its waves own
// 32 rows each (one MFMA block).  Every tile is anchored per channel at the
// floored prefix of its middle row (row 64, or the last row of a shorter
// tail), as the forward anchors its tiles, so both exp2 factors of a pair
// stay within 2^(+-change of P over 64 rows); bwd_anchor_kernel writes every
// row's q~ and k~ at its own tile's anchor once.  The other side streams
// through LDS 32 rows at a time, each tile both row-major (the MFMA's first
// operand) and transposed (the second operand of the product that contracts
// over the streamed rows), moved to the block's anchor by an exact power of
// two as it is staged; the next tile's global loads are issued before the
// current tile's products, and the tiles are double-buffered in LDS (one
// barrier per tile).  Staging lanes take consecutive rows of one 8-channel
// chunk, so the transposed copy is written as runs of consecutive bf16.  The
// block's own rows stay in registers as second operands.
//
// dk/dv (per key block, queries from the block's first key on; 8 waves):
//   dk waves  S = q~ k~^T, dP = do v^T (32 streamed queries x the wave's 32
//             keys), A and dS in-lane, dk += dS^T q~; A to LDS;
//   dv waves  stage the tiles; one tile behind, dv += A^T do.
// dq (per query block, keys up to the block's last query; 4 waves):
//   S^T = k~ q~^T, dP^T = v do^T (32 streamed keys x the wave's 32 queries);
//   dq += dS k~; the waves stage the tiles together.
// Both kernels run two waves per SIMD: no wave of the dk/dv kernel holds both
// accumulator sets, and two 4-wave dq blocks share a CU.
//
// The streamed rows of the first products are fed in the order that swaps
// bits 2 and 3 of the row index, so each lane's 16 accumulator registers hold
// two runs of 8 consecutive streamed rows: exactly the k-slots the lane
// supplies to the second product, with no data exchange between lanes.
//
// X.  The gate gradient is a suffix sum of X_t = q_t (.) dq_t - k_t (.) dk_t^(hq),
// whose terms cancel pair by pair: the pair (i, j) adds dS_ij q~_i k~_j to X_i
// and takes it from X_j.  The kernels therefore form both sides from the
// same bf16 q~ and k~ the products use, ln2 q~_i (.) sum_j dS_ij k~_j and
// ln2 k~_j (.) sum_i dS_ij q~_i (the anchors of the two kernels differ by
// integers, which moves q~ and k~ by exact powers of two), so the rounding of
// the operands cancels in the sums as the exact terms do.  Built from the
// unrounded q and k instead, each pair would leave a residue of the operand
// rounding (2^-9 relative), and over a long sequence these residues add up
// to several times the error of dq and dk themselves.
//
// A block handles a single query head, so dk and dv leave as float32 per
// query head partials, summed over the heads of a kv group by
// bwd_reduce_kernel.  The dk/dv kernel also subtracts k (.) dk^(hq) and the
// column sums of dS from the X and Y rows the dq kernel wrote (it runs after
// it on the same stream).
#include <float.h>

#include <type_traits>

#include "wall_common.h"

namespace wall {
namespace {

constexpr int BR = 128;      // rows per block
constexpr int BT = 32;       // streamed rows per tile
constexpr int NW = 4;        // waves per block
constexpr int NTH = NW * 64;
constexpr int TP = BT + 8;   // transposed tile row pitch (elements): 80 bytes

// exp2 of a clamped anchored exponent on v_exp_f32 itself: results below
// the float32 normal range may come back as 0, which only drops terms below
// 2^-126 of the largest.  Every anchored factor of this file goes through it,
// so the staged operands and the epilogue's recomputed ones agree bit for bit.
__device__ inline float clamp2(float e) { return __builtin_amdgcn_exp2f(fminf(fmaxf(e, EXP2_LO), EXP2_HI)); }
__device__ inline int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 lds8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Row-major tiles: 16-byte chunk c of row r sits at chunk c ^ 4 when bit 3
// of r is set (else at c), rows PITCH elements apart.  With a pitch of 4
// dwords modulo the 32 banks, the 8 rows one 8-lane phase of a first-operand
// read touches ({0..3, 8..11} + 16k + 4m, the bits-2-and-3 order) and the 8
// consecutive rows of a staging write then fall on 8 different 4-bank
// groups.
template <int PITCH>
__device__ inline int roff(int r, int chunk) { return r * PITCH + 8 * (chunk ^ (((r >> 3) & 1) << 2)); }
template <int PITCH>
constexpr int rows_size() { return BT * PITCH; }

__device__ inline f32x8 to_f32(uint4 raw) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, raw), f32x8);
}

// Block index -> (query head, sequence, row block).  The row block is the
// slowest index and runs from the heaviest end (most partner rows) down, so
// the longest blocks start first; consecutive ids are consecutive (head,
// sequence) pairs, which with HQ * nseg a multiple of 8 keeps each pair on one
// XCD.
struct BlockPos {
    int hq, seg, rb;
};
__device__ inline BlockPos block_pos(const BwdArgs &a, int nblk, bool heavy_first_low) {
    const int hs_n = a.HQ * a.nseg;
    const int rank = blockIdx.x / hs_n, hs = blockIdx.x % hs_n;
    BlockPos p;
    p.hq = hs % a.HQ;
    p.seg = hs / a.HQ;
    p.rb = heavy_first_low ? rank : nblk - 1 - rank;
    return p;
}

// ---------------------------------------------------------------- tile anchors, q~ and k~
// Per (128-row tile, query head): R = floor(P) at the tile's middle row, and
// every row's q~ = q scale log2e 2^(P - R) and k~ = k 2^(R - P) in bf16.  The
// dq and dk/dv kernels use their own tile's rows as they are and move a
// streamed tile to their block's anchor by the integer difference of the two
// anchors: an exact power of two, applied with v_ldexp_f32 instead of an
// exp2 per element.
template <int K>
__global__ __launch_bounds__(256) void bwd_anchor_kernel(BwdArgs a, int nblk) {
    __shared__ float sR[K];
    // one block per (tile of a sequence, query head), tiles fastest
    const int tile = blockIdx.x % nblk, hs = blockIdx.x / nblk, hq = hs % a.HQ;
    const SegInfo sg = a.seg[hs / a.HQ];
    const int r0 = tile * BR;
    if (r0 >= sg.len) return;
    const int n = min(BR, sg.len - r0), tid = threadIdx.x;
    const int64_t HQ = a.HQ, s0 = sg.start;
    const int h = hq / (a.HQ / a.H);
    if (tid < K) {
        const float R = floorf(a.P[(s0 + r0 + min(ANCHOR_ROW, n - 1)) * HQ * K + hq * K + tid]);
        sR[tid] = R;
        a.Rt[((int64_t)(sg.tile_base + tile) * HQ + hq) * K + tid] = R;
    }
    __syncthreads();
    const __bf16 *qg = static_cast<const __bf16 *>(a.q);
    const __bf16 *kg = static_cast<const __bf16 *>(a.k);
    __bf16 *qh = static_cast<__bf16 *>(a.qh);
    __bf16 *kh = static_cast<__bf16 *>(a.kh);
    for (int c = tid; c < n * (K / 8); c += 256) {
        const int r = c / (K / 8), ch = 8 * (c % (K / 8));
        const int64_t t = s0 + r0 + r, ix = (t * HQ + hq) * K + ch;
        const f32x8 qq = to_f32(*reinterpret_cast<const uint4 *>(qg + ix));
        const f32x8 kk = to_f32(*reinterpret_cast<const uint4 *>(kg + (t * a.H + h) * K + ch));
        const f32x4 *pp = reinterpret_cast<const f32x4 *>(a.P + ix);
        const f32x4 p0 = pp[0], p1 = pp[1];
        f32x8 xq, xk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pv = e < 4 ? p0[e] : p1[e - 4];
            xq[e] = qq[e] * a.qscale * clamp2(pv - sR[ch + e]);
            xk[e] = kk[e] * clamp2(sR[ch + e] - pv);
        }
        *reinterpret_cast<bf16x8 *>(qh + ix) = __builtin_convertvector(xq, bf16x8);
        *reinterpret_cast<bf16x8 *>(kh + ix) = __builtin_convertvector(xk, bf16x8);
    }
}

// 2^(to - from) applied to an anchored value: from, to are integer anchors
__device__ inline float shift_anchor(float x, float to, float from) {
    return ldexpf(x, (int)fminf(fmaxf(to - from, -1000.0f), 1000.0f));
}

// ---------------------------------------------------------------- dk, dv
// Eight waves in two roles over the same staged tiles: waves 0-3 own 32 keys
// each for dk (S, dP, A, dS, dk += dS^T q~, and the X and Y updates), waves
// 4-7 the same keys for dv (dv += A^T do).  A dk wave leaves its bf16 A in
// LDS in the lane order of the dv product's first operand, and the dv wave
// of the same keys consumes it one tile later (after the tile's barrier), so
// no barrier is added; do^T keeps three buffers for that lag.  The dv waves
// also stage every tile, so the dk waves' chain holds only their products and
// the softmax.  Each role holds one accumulator set, so both fit two waves
// per SIMD.
constexpr int NTH_KV = 2 * NTH;

template <int K, int V, bool HAS_G>
__global__ __launch_bounds__(NTH_KV) void bwd_dkdv_mfma(BwdArgs a, int nblk) {
    constexpr int RPK = K + 8, RPV = V + 8;
    constexpr int CK = BT * K / 8, CV = BT * V / 8;  // 8-element chunks per tile
    // the four dv waves stage the tiles (NTH threads)
    constexpr int UK = (CK + NTH - 1) / NTH, UV = (CV + NTH - 1) / NTH;
    // two buffers of each streamed tile: one read while the other is filled
    __shared__ __attribute__((aligned(16))) __bf16 sQ[2][rows_size<RPK>()];  // q~ rows
    __shared__ __attribute__((aligned(16))) __bf16 sQT[2][K * TP];           // q~ transposed
    __shared__ __attribute__((aligned(16))) __bf16 sO[2][rows_size<RPV>()];  // do rows
    __shared__ __attribute__((aligned(16))) __bf16 sOT[3][V * TP];           // do transposed
    __shared__ __attribute__((aligned(16))) __bf16 sP[2][NW][2][64 * 8];     // A from the dk waves
    __shared__ __attribute__((aligned(16))) float sL[2][BT];
    __shared__ __attribute__((aligned(16))) float sD[2][BT];
    __shared__ __attribute__((aligned(16))) float sGq[2][BT];
    __shared__ float sR[K];

    const BlockPos bp = block_pos(a, nblk, true);
    const SegInfo sg = a.seg[bp.seg];
    const int hq = bp.hq, j0 = bp.rb * BR;
    if (j0 >= sg.len) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
    const int64_t HQ = a.HQ;
    const int h = hq / (a.HQ / a.H);
    const int len = sg.len, jn = min(BR, len - j0);
    const int64_t s0 = sg.start;
    const __bf16 *vg = static_cast<const __bf16 *>(a.v);
    const __bf16 *dog = static_cast<const __bf16 *>(a.dout);

    if (tid < K) sR[tid] = floorf(a.P[(s0 + j0 + min(ANCHOR_ROW, jn - 1)) * HQ * K + hq * K + tid]);
    __syncthreads();

    const int qend = a.window > 0 ? min(len, j0 + jn - 1 + a.window) : len;

    const __bf16 *qhg = static_cast<const __bf16 *>(a.qh);
    const __bf16 *khg = static_cast<const __bf16 *>(a.kh);
    // prefetch registers for one tile: q~ at its own tile's anchor and that anchor
    uint4 qraw[UK], oraw[UV];
    f32x8 araw[UK];
    float il = 0.f, id = 0.f, ig = 0.f;
    const int sid = tid - NTH;  // staging thread index (dv waves)
    auto load_tile = [&](int q0) {
        // rows past the sequence load its last row (in bounds) and are zeroed when stored
        const float *rt = a.Rt + ((int64_t)(sg.tile_base + q0 / BR) * HQ + hq) * K;
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = sid + NTH * u, r = c % BT, ch = 8 * (c / BT), i = min(q0 + r, len - 1);
            if (CK % NTH == 0 || c < CK) {
                qraw[u] = *reinterpret_cast<const uint4 *>(qhg + ((s0 + i) * HQ + hq) * K + ch);
                const f32x4 *pp = reinterpret_cast<const f32x4 *>(rt + ch);
                const f32x4 p0 = pp[0], p1 = pp[1];
                araw[u] = f32x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            }
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int c = sid + NTH * u, r = c % BT, ch = 8 * (c / BT), i = min(q0 + r, len - 1);
            if (CV % NTH == 0 || c < CV)
                oraw[u] = *reinterpret_cast<const uint4 *>(dog + ((s0 + i) * HQ + hq) * V + ch);
        }
        if (sid < BT) {
            const int i = q0 + sid;
            il = id = ig = 0.f;
            if (i < len) {
                const int64_t t = (s0 + i) * HQ + hq;
                il = a.lse[t] * LOG2E;
                id = a.D[t];
                if (HAS_G) ig = a.G[t];
            }
        }
    };
    auto store_tile = [&](int buf, int q0, int tix) {
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = sid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            if (CK % NTH == 0 || c < CK) {
                const f32x8 qq = to_f32(qraw[u]);
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = shift_anchor(qq[e], araw[u][e], sR[ch + e]);
                if (q0 + r >= len) x = 0.f;
                const bf16x8 b = __builtin_convertvector(x, bf16x8);
                *reinterpret_cast<bf16x8 *>(&sQ[buf][roff<RPK>(r, ch / 8)]) = b;
#pragma unroll
                for (int e = 0; e < 8; ++e) sQT[buf][(ch + e) * TP + r] = b[e];
            }
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int c = sid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            if (CV % NTH == 0 || c < CV) {
                const uint4 z = {0, 0, 0, 0};
                const bf16x8 b = __builtin_bit_cast(bf16x8, q0 + r < len ? oraw[u] : z);
                *reinterpret_cast<bf16x8 *>(&sO[buf][roff<RPV>(r, ch / 8)]) = b;
#pragma unroll
                for (int e = 0; e < 8; ++e) sOT[tix % 3][(ch + e) * TP + r] = b[e];
            }
        }
        if (sid < BT) {
            sL[buf][sid] = il;
            sD[buf][sid] = id;
            sGq[buf][sid] = ig;
        }
    };

    // Tile it lives in buffer it & 1.  Iteration it computes on it, then
    // stores tile it+1 (loaded during iteration it-1) into the other buffer,
    // which every wave finished reading before the previous barrier; one
    // barrier per tile.
    const bool stager = w >= NW;
    if (stager) {
        load_tile(j0);
        store_tile(0, j0, 0);
    }
    __syncthreads();
    if (stager && j0 + BT < qend) load_tile(j0 + BT);

    // One role's whole walk over the query tiles; the two instantiations keep
    // their accumulators apart.  Every wave runs every tile: a tile with no
    // visible pair for its keys (at most the first three, or three past the
    // window) is masked to zero, and the accumulators stay on one straight
    // path through the loop.
    auto walk = [&](auto dk_role) {
        constexpr bool DK = decltype(dk_role)::value;
        constexpr int NA = DK ? K / 32 : V / 32;
        const int wr = w % NW;
        const int jw = j0 + 32 * wr, j = jw + l32;
        const bool jok = j < len;
        const int64_t tj = s0 + (jok ? j : 0);
        f32x16 acc[NA];
#pragma unroll
        for (int n = 0; n < NA; ++n) acc[n] = 0.f;
        // dv += A^T do for tile tix, A left in LDS by the dk wave of these keys
        auto dv_step = [&](int tix) {
            bf16x8 pb[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) pb[c] = lds8(&sP[tix & 1][wr][c][lane * 8]);
#pragma unroll
            for (int n = 0; n < NA; ++n)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[n] = mfma(pb[c], lds8(&sOT[tix % 3][(32 * n + l32) * TP + 16 * c + 8 * hl]), acc[n]);
        };
        float colsum = 0.f;
        int it = 0;
        if constexpr (DK) {
            // the wave's keys as second operands: k~ (its own tile's anchor is the
            // block's) and v rows of key j
            bf16x8 kop[K / 16], vop[V / 16];
#pragma unroll
            for (int s = 0; s < K / 16; ++s) {
                const int ch = 16 * s + 8 * hl;
                uint4 raw = {0, 0, 0, 0};
                if (jok) raw = *reinterpret_cast<const uint4 *>(khg + (tj * HQ + hq) * K + ch);
                kop[s] = __builtin_bit_cast(bf16x8, raw);
            }
#pragma unroll
            for (int s = 0; s < V / 16; ++s) {
                const int ch = 16 * s + 8 * hl;
                uint4 raw = {0, 0, 0, 0};
                if (jok) raw = *reinterpret_cast<const uint4 *>(vg + (tj * a.H + h) * V + ch);
                vop[s] = __builtin_bit_cast(bf16x8, raw);
            }
            const float gj = (HAS_G && jok) ? a.G[tj * HQ + hq] : 0.f;
            for (int q0 = j0; q0 < qend; q0 += BT, ++it) {
                const int cur = it & 1;
                const int qrow = swap23(l32);
                f32x16 S = 0.f, dP = 0.f;
#pragma unroll
                for (int s = 0; s < K / 16; ++s)
                    S = mfma(lds8(&sQ[cur][roff<RPK>(qrow, 2 * s + hl)]), kop[s], S);
#pragma unroll
                for (int s = 0; s < V / 16; ++s)
                    dP = mfma(lds8(&sO[cur][roff<RPV>(qrow, 2 * s + hl)]), vop[s], dP);
                // every pair of the tile visible: no mask
                const bool full = jw + 31 < len && q0 >= jw + 31 && q0 + BT <= len &&
                                  (a.window <= 0 || q0 + BT - 1 - jw < a.window);
                bf16x8 db[2];
                // two copies of the softmax step: without the mask for a full tile,
                // with it for the diagonal, the window edge and a sequence's end
                auto softmax = [&](auto masked) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int qi0 = 16 * c + 8 * hl;
                        // the 8 rows' values, read unconditionally ahead of their use
                        f32x4 L4[2], D4[2], G4[2];
#pragma unroll
                        for (int x = 0; x < 2; ++x) {
                            L4[x] = *reinterpret_cast<const f32x4 *>(&sL[cur][qi0 + 4 * x]);
                            D4[x] = *reinterpret_cast<const f32x4 *>(&sD[cur][qi0 + 4 * x]);
                            if (HAS_G) G4[x] = *reinterpret_cast<const f32x4 *>(&sGq[cur][qi0 + 4 * x]);
                        }
                        f32x8 p8, d8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float Gi = HAS_G ? G4[e / 4][e % 4] : 0.f;
                            float p = __builtin_amdgcn_exp2f(S[8 * c + e] + Gi - gj - L4[e / 4][e % 4]);
                            if constexpr (decltype(masked)::value) {
                                const int i = q0 + qi0 + e;
                                const bool vis = jok && i >= j && i < len && (a.window <= 0 || i - j < a.window);
                                p = vis ? p : 0.f;
                            }
                            const float ds = p * (dP[8 * c + e] - D4[e / 4][e % 4]);
                            colsum += ds;
                            p8[e] = p;
                            d8[e] = ds;
                        }
                        // A goes straight to LDS for the dv wave of these keys
                        *reinterpret_cast<bf16x8 *>(&sP[cur][wr][c][lane * 8]) = __builtin_convertvector(p8, bf16x8);
                        db[c] = __builtin_convertvector(d8, bf16x8);
                    }
                };
                if (full)
                    softmax(std::false_type{});
                else
                    softmax(std::true_type{});
#pragma unroll
                for (int n = 0; n < NA; ++n)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        acc[n] = mfma(db[c], lds8(&sQT[cur][(32 * n + l32) * TP + 16 * c + 8 * hl]), acc[n]);
                __syncthreads();
            }
        } else {
            // one tile behind the dk waves; these waves also stage every tile
            for (int q0 = j0; q0 < qend; q0 += BT, ++it) {
                if (it > 0) dv_step(it - 1);
                if (q0 + BT < qend) store_tile((it & 1) ^ 1, q0 + BT, it + 1);
                __syncthreads();
                if (q0 + 2 * BT < qend) load_tile(q0 + 2 * BT);
            }
            if (it > 0) dv_step(it - 1);
        }

        if (jw >= len) return;
        if constexpr (DK) {
            colsum += __shfl_xor(colsum, 32);
            if (hl == 0 && jok) a.Y[tj * HQ + hq] -= colsum;
        }
        // accumulator register r of lane (l32, hl): key jw + 8(r/4) + 4hl + r%4, channel 32n + l32
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int jr = jw + 8 * (r / 4) + 4 * hl + (r % 4);
            if (jr >= len) continue;
            const int64_t t = s0 + jr;
#pragma unroll
            for (int n = 0; n < NA; ++n) {
                const int ch = 32 * n + l32;
                if constexpr (DK) {
                    const int64_t ix = (t * HQ + hq) * K + ch;
                    a.dkp[ix] = LN2 * clamp2(sR[ch] - a.P[ix]) * acc[n][r];
                    // k (.) dk^(hq) from the bf16 k~ the dq products used (see the X note above)
                    a.X[ix] -= LN2 * (float)khg[ix] * acc[n][r];
                } else {
                    a.dvp[(t * HQ + hq) * V + ch] = acc[n][r];
                }
            }
        }
    };
    if (w < NW)
        walk(std::true_type{});
    else
        walk(std::false_type{});
}

// ---------------------------------------------------------------- dq
template <int K, int V, bool HAS_G>
__global__ __launch_bounds__(NTH, 2) void bwd_dq_mfma(BwdArgs a, int nblk) {
    constexpr int RPK = K + 8, RPV = V + 8;
    constexpr int CK = BT * K / 8, CV = BT * V / 8;
    constexpr int UK = CK / NTH, UV = CV / NTH;
    static_assert(CK % NTH == 0 && CV % NTH == 0, "tile chunks");
    __shared__ __attribute__((aligned(16))) __bf16 sK[2][rows_size<RPK>()];  // k~ rows
    __shared__ __attribute__((aligned(16))) __bf16 sKT[2][K * TP];           // k~ transposed
    __shared__ __attribute__((aligned(16))) __bf16 sV[2][rows_size<RPV>()];  // v rows
    __shared__ __attribute__((aligned(16))) float sGk[2][BT];
    __shared__ float sR[K];

    const BlockPos bp = block_pos(a, nblk, false);
    const SegInfo sg = a.seg[bp.seg];
    const int hq = bp.hq, i0 = bp.rb * BR;
    if (i0 >= sg.len) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
    const int64_t HQ = a.HQ;
    const int h = hq / (a.HQ / a.H);
    const int len = sg.len, in_ = min(BR, len - i0);
    const int64_t s0 = sg.start;
    const __bf16 *vg = static_cast<const __bf16 *>(a.v);
    const __bf16 *dog = static_cast<const __bf16 *>(a.dout);

    if (tid < K) sR[tid] = floorf(a.P[(s0 + i0 + min(ANCHOR_ROW, in_ - 1)) * HQ * K + hq * K + tid]);
    __syncthreads();

    // the wave's queries as second operands
    const int iw = i0 + 32 * w, i = iw + l32;
    const bool iok = i < len;
    const int64_t ti = s0 + (iok ? i : 0);
    const __bf16 *qhg = static_cast<const __bf16 *>(a.qh);
    const __bf16 *khg = static_cast<const __bf16 *>(a.kh);
    // the block is one tile: its rows' q~ are at the block's anchor already
    bf16x8 qop[K / 16], oop[V / 16];
#pragma unroll
    for (int s = 0; s < K / 16; ++s) {
        const int ch = 16 * s + 8 * hl;
        uint4 raw = {0, 0, 0, 0};
        if (iok) raw = *reinterpret_cast<const uint4 *>(qhg + (ti * HQ + hq) * K + ch);
        qop[s] = __builtin_bit_cast(bf16x8, raw);
    }
#pragma unroll
    for (int s = 0; s < V / 16; ++s) {
        const int ch = 16 * s + 8 * hl;
        uint4 raw = {0, 0, 0, 0};
        if (iok) raw = *reinterpret_cast<const uint4 *>(dog + (ti * HQ + hq) * V + ch);
        oop[s] = __builtin_bit_cast(bf16x8, raw);
    }
    const float lse2 = iok ? a.lse[ti * HQ + hq] * LOG2E : 0.f;
    const float Di = iok ? a.D[ti * HQ + hq] : 0.f;
    const float Gi = (HAS_G && iok) ? a.G[ti * HQ + hq] : 0.f;

    f32x16 dq[K / 32];
#pragma unroll
    for (int n = 0; n < K / 32; ++n) dq[n] = 0.f;
    float rowsum = 0.f;

    const int ilast = i0 + in_ - 1;
    const int klo = a.window > 0 ? max(0, i0 - a.window + 1) / BT * BT : 0;

    // prefetch registers for one tile: k~ at its own tile's anchor and that anchor
    uint4 kraw[UK], vraw[UV];
    f32x8 araw[UK];
    float kgv = 0.f;
    auto load_tile = [&](int k0) {
        // rows past the sequence load its last row (in bounds) and are zeroed when stored
        const float *rt = a.Rt + ((int64_t)(sg.tile_base + k0 / BR) * HQ + hq) * K;
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            const int64_t t = s0 + min(k0 + r, len - 1);
            kraw[u] = *reinterpret_cast<const uint4 *>(khg + (t * HQ + hq) * K + ch);
            const f32x4 *pp = reinterpret_cast<const f32x4 *>(rt + ch);
            const f32x4 p0 = pp[0], p1 = pp[1];
            araw[u] = f32x8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            vraw[u] = *reinterpret_cast<const uint4 *>(vg + ((s0 + min(k0 + r, len - 1)) * a.H + h) * V + ch);
        }
        if (HAS_G && tid < BT) {
            const int jj = k0 + tid;
            kgv = jj < len ? a.G[(s0 + jj) * HQ + hq] : 0.f;
        }
    };
    auto store_tile = [&](int buf, int k0) {
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            const f32x8 kk = to_f32(kraw[u]);
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = shift_anchor(kk[e], sR[ch + e], araw[u][e]);
            if (k0 + r >= len) x = 0.f;
            const bf16x8 b = __builtin_convertvector(x, bf16x8);
            *reinterpret_cast<bf16x8 *>(&sK[buf][roff<RPK>(r, ch / 8)]) = b;
#pragma unroll
            for (int e = 0; e < 8; ++e) sKT[buf][(ch + e) * TP + r] = b[e];
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            const uint4 z = {0, 0, 0, 0};
            *reinterpret_cast<uint4 *>(&sV[buf][roff<RPV>(r, ch / 8)]) = k0 + r < len ? vraw[u] : z;
        }
        if (HAS_G && tid < BT) sGk[buf][tid] = kgv;
    };

    // double-buffered as in the dk/dv kernel
    load_tile(klo);
    store_tile(0, klo);
    __syncthreads();
    if (klo + BT <= ilast) load_tile(klo + BT);
    for (int k0 = klo, it = 0; k0 <= ilast; k0 += BT, ++it) {
        const int cur = it & 1;
        // every wave runs every tile, as in the dk/dv kernel
        {
        f32x16 S = 0.f, dP = 0.f;
        const int krow = swap23(l32);
#pragma unroll
        for (int s = 0; s < K / 16; ++s) S = mfma(lds8(&sK[cur][roff<RPK>(krow, 2 * s + hl)]), qop[s], S);
#pragma unroll
        for (int s = 0; s < V / 16; ++s) dP = mfma(lds8(&sV[cur][roff<RPV>(krow, 2 * s + hl)]), oop[s], dP);

        // every pair of the tile visible: no mask
        const bool full = iw + 31 < len && k0 + BT - 1 <= iw &&
                          (a.window <= 0 || iw + 31 - k0 < a.window);
        bf16x8 db[2];
        auto softmax = [&](auto masked) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int kj0 = 16 * c + 8 * hl;
                f32x4 G4[2];
                if (HAS_G) {
#pragma unroll
                    for (int x = 0; x < 2; ++x) G4[x] = *reinterpret_cast<const f32x4 *>(&sGk[cur][kj0 + 4 * x]);
                }
                f32x8 d8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float Gj = HAS_G ? G4[e / 4][e % 4] : 0.f;
                    float p = __builtin_amdgcn_exp2f(S[8 * c + e] + Gi - Gj - lse2);
                    if constexpr (decltype(masked)::value) {
                        const int jj = k0 + kj0 + e;
                        const bool vis = iok && jj <= i && (a.window <= 0 || i - jj < a.window);
                        p = vis ? p : 0.f;
                    }
                    const float ds = p * (dP[8 * c + e] - Di);
                    rowsum += ds;
                    d8[e] = ds;
                }
                db[c] = __builtin_convertvector(d8, bf16x8);
            }
        };
        if (full)
            softmax(std::false_type{});
        else
            softmax(std::true_type{});
#pragma unroll
        for (int n = 0; n < K / 32; ++n)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dq[n] = mfma(db[c], lds8(&sKT[cur][(32 * n + l32) * TP + 16 * c + 8 * hl]), dq[n]);
        }
        if (k0 + BT <= ilast) store_tile(cur ^ 1, k0 + BT);
        __syncthreads();
        if (k0 + 2 * BT <= ilast) load_tile(k0 + 2 * BT);
    }

    if (iw >= len) return;
    rowsum += __shfl_xor(rowsum, 32);
    if (hl == 0 && iok) {
        a.Y[ti * HQ + hq] = rowsum;
        a.Z[ti * HQ + hq] = a.sink ? -exp2f(a.sink[hq] * LOG2E - lse2) * Di : 0.f;
    }
    __bf16 *dqg = static_cast<__bf16 *>(a.dq);
    // accumulator register r of lane (l32, hl): query iw + 8(r/4) + 4hl + r%4, channel 32n + l32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ir = iw + 8 * (r / 4) + 4 * hl + (r % 4);
        if (ir >= len) continue;
        const int64_t t = s0 + ir;
#pragma unroll
        for (int n = 0; n < K / 32; ++n) {
            const int ch = 32 * n + l32;
            const int64_t ix = (t * HQ + hq) * K + ch;
            dqg[ix] = (__bf16)(a.scale * clamp2(a.P[ix] - sR[ch]) * dq[n][r]);
            a.X[ix] = LN2 * (float)qhg[ix] * dq[n][r];
        }
    }
}

// ---------------------------------------------------------------- dk, dv: sum over the kv group
template <int K, int V>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a, int64_t nrow_h) {
    // one (row, kv head) per 32 lanes; K/32 and V/32 consecutive channels per
    // lane, read as one vector per query head of the group
    constexpr int KL = K / 32, VL = V / 32;
    const int64_t rh = (int64_t)blockIdx.x * 8 + threadIdx.x / 32;
    if (rh >= nrow_h) return;
    const int l = threadIdx.x % 32;
    const int64_t t = rh / a.H;
    const int h = (int)(rh % a.H), grp = a.HQ / a.H;
    float sk[KL] = {}, sv[VL] = {};
    for (int g = 0; g < grp; ++g) {
        const float *pk = a.dkp + (t * a.HQ + h * grp + g) * K + l * KL;
        const float *pv = a.dvp + (t * a.HQ + h * grp + g) * V + l * VL;
#pragma unroll
        for (int e = 0; e < KL; ++e) sk[e] += pk[e];
#pragma unroll
        for (int e = 0; e < VL; ++e) sv[e] += pv[e];
    }
    __bf16 *dkg = static_cast<__bf16 *>(a.dk) + rh * K + l * KL;
    __bf16 *dvg = static_cast<__bf16 *>(a.dv) + rh * V + l * VL;
#pragma unroll
    for (int e = 0; e < KL; ++e) dkg[e] = (__bf16)sk[e];
#pragma unroll
    for (int e = 0; e < VL; ++e) dvg[e] = (__bf16)sv[e];
}

template <int K, int V, bool HAS_G>
hipError_t run(const BwdArgs &a, hipStream_t st) {
    const int nblk = (int)cdiv(a.max_seqlen, BR);
    const unsigned nb = (unsigned)((int64_t)a.HQ * a.nseg * nblk);
    hipLaunchKernelGGL((bwd_anchor_kernel<K>), dim3(nb), dim3(256), 0, st, a, nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_mfma<K, V, HAS_G>), dim3(nb), dim3(NTH), 0, st, a, nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_mfma<K, V, HAS_G>), dim3(nb), dim3(NTH_KV), 0, st, a, nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nrow_h = (int64_t)a.rows * a.H;
    hipLaunchKernelGGL((bwd_reduce_kernel<K, V>), dim3((unsigned)cdiv(nrow_h, 8)), dim3(256), 0, st, a, nrow_h);
    return hipGetLastError();
}

template <int K, int V>
hipError_t run_g(const BwdArgs &a, hipStream_t st) {
    return a.G ? run<K, V, true>(a, st) : run<K, V, false>(a, st);
}

}  // namespace

hipError_t launch_bwd_mfma(const BwdArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_g<64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_g<64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_g<128, 64>(a, st);
    return run_g<128, 128>(a, st);
}

}  // namespace wall
