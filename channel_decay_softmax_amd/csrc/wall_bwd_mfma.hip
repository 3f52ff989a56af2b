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
// 32 rows each (one MFMA block, one anchor block).  The other side streams
// through LDS 32 rows at a time, each tile both row-major (the MFMA's first
// operand) and transposed (the second operand of the product that contracts
// over the streamed rows); the next tile's global loads are issued before the
// current tile's products, and the tiles are double-buffered in LDS (one
// barrier per tile).  Staging lanes take consecutive rows of one 8-channel
// chunk, so the transposed copy is written as runs of consecutive bf16.  The
// block's own rows stay in registers as second operands.
//
// Anchors (the anchor identity exp2(P_i - P_j) = exp2(P_i - R) exp2(R - P_j)
// of the Wall Attention blog, "Fast training and inference"), per query head
// and channel, with A_b = floor(P) of 32-row block b's last row:
//   * bwd_anchor_kernel writes A_b, each row's q~ at A_(b-1) of the block
//     before its own and k~ at its own block's A_b (both factors at most 2
//     for a falling prefix), and flags a block whose rows lie more than
//     BWD_SPREAD log2 units from A_b or A_(b-1);
//   * a pair whose rows lie in different 128-row tiles is read at a tile
//     boundary: floor(P) of the row before the query tile in the dq kernel,
//     A of the key tile's last block in the dk/dv kernel; both lie between
//     the two rows, so both factors stay at most 2;
//   * a pair inside one tile is read at A of the key's block (dq kernel) or
//     of the block before the query's (dk/dv kernel), again between the rows
//     unless the two rows share a block: then one factor is at most
//     2^(BWD_SPREAD + 1), and the pairs of a flagged block are left to the
//     pair-by-pair kernel of wall_bwd_diag.hip, which runs first;
//   * every move of q~ or k~ to another anchor is an exact power of two of the
//     stored bf16 value (a moved value that leaves the bf16 normal range may
//     round differently, below 2^-126), so each pair's product q~ k~ is the
//     same in both kernels; the accumulators move between anchors the same way, only ever
//     downwards (the dq kernel walks the key tiles upwards, the dk/dv kernel
//     the query tiles after its tile first, then its own tile from the last
//     block down).
// A term lost to an underflowing factor is below 2^(BWD_SPREAD + 1 - 126) of
// |dS q k| for the rows it belongs to.
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
// ln2 k~_j (.) sum_i dS_ij q~_i at the accumulators' final anchors (all
// anchors are integers, which moves q~ and k~ by exact powers of two), so the
// rounding of the operands cancels in the sums as the exact terms do.  Built
// from the unrounded q and k instead, each pair would leave a residue of the
// operand rounding (2^-9 relative), and over a long sequence these residues
// add up to several times the error of dq and dk themselves.
//
// A block handles a single query head, so dk and dv leave as float32 per
// query head partials, summed over the heads of a kv group by
// bwd_reduce_kernel.  The dk/dv kernel also subtracts k (.) dk^(hq) and the
// column sums of dS from the X and Y rows the dq kernel wrote (it runs after
// it on the same stream).  For the rows of a flagged block both kernels add
// the pair-by-pair kernel's parts (dqd, dkp, dvp, X, Y) instead of
// overwriting them.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "wall_common.h"

namespace wall {
namespace {

constexpr int BR = 128;      // rows per block
constexpr int BT = 32;       // streamed rows per tile
constexpr int NW = 4;        // waves per block
constexpr int NTH = NW * 64;
constexpr int TP = BT + 8;   // transposed tile row pitch (elements): 80 bytes
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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

// ---------------------------------------------------------------- block anchors, q~ and k~
// Per (128-row tile, query head): the anchors A_b of its four 32-row blocks,
// every row's q~ = q scale log2e 2^(P - A_(b-1)) and k~ = k 2^(A_b - P) in bf16,
// and the spread flags (sequence + 1 for a flagged block, else 0).  The dq and
// dk/dv kernels move these rows to other anchors by integer differences of
// anchors: exact powers of two, applied with v_ldexp_f32.
template <int K>
__global__ __launch_bounds__(256) void bwd_anchor_kernel(BwdArgs a, int nblk) {
    constexpr int NBK = BR / BWD_BLK;
    __shared__ float sA[NBK + 1][K];  // A_(first - 1), A_first .. A_(first + 3)
    __shared__ int sflag;
    __shared__ uint32_t sqm[NBK], skm[NBK];
    __shared__ uint32_t sC[2][NBK][4][K / 2];  // per wave the channels' largest |q~|, |k~| (u16 pairs)
    // one block per (tile of a sequence, query head), tiles fastest
    const int tile = blockIdx.x % nblk, hs = blockIdx.x / nblk, hq = hs % a.HQ, sidx = hs / a.HQ;
    const SegInfo sg = a.seg[sidx];
    const int r0 = tile * BR;
    if (r0 >= sg.len) return;
    const int n = min(BR, sg.len - r0), tid = threadIdx.x;
    const int64_t HQ = a.HQ, s0 = sg.start;
    const int h = hq / (a.HQ / a.H);
    const int64_t gb0 = (int64_t)(sg.tile_base + tile) * NBK;
    if (tid == 0) sflag = 0;
    if (tid < NBK) {
        sqm[tid] = 0u;
        skm[tid] = 0u;
    }
    if (tid < K) {
        const float *Pc = a.P + hq * K + tid;
        sA[0][tid] = r0 > 0 ? floorf(Pc[(s0 + r0 - 1) * HQ * K]) : 0.f;
#pragma unroll
        for (int b = 0; b < NBK; ++b) {
            if (BWD_BLK * b >= n) break;
            const float A = floorf(Pc[(s0 + r0 + min(BWD_BLK * b + BWD_BLK - 1, n - 1)) * HQ * K]);
            sA[b + 1][tid] = A;
            a.Ab[((gb0 + b) * HQ + hq) * K + tid] = A;
        }
    }
    __syncthreads();
    const __bf16 *qg = static_cast<const __bf16 *>(a.q);
    const __bf16 *kg = static_cast<const __bf16 *>(a.k);
    __bf16 *qh = static_cast<__bf16 *>(a.qh);
    __bf16 *kh = static_cast<__bf16 *>(a.kh);
    int spread = 0;
    uint32_t qm[NBK] = {}, km[NBK] = {};  // the largest stored |q~|, |k~| per block (bf16 magnitude bits)
    // per block the largest stored |q~|, |k~| of each of the thread's 8 channels
    // (the thread's channel chunk, tid % (K / 8), is the same at every row)
    u16x2 qc[NBK][4] = {}, kc[NBK][4] = {};
    for (int c = tid; c < n * (K / 8); c += 256) {
        const int r = c / (K / 8), ch = 8 * (c % (K / 8)), b = r / BWD_BLK;
        const int64_t t = s0 + r0 + r, ix = (t * HQ + hq) * K + ch;
        const f32x8 qq = to_f32(*reinterpret_cast<const uint4 *>(qg + ix));
        const f32x8 kk = to_f32(*reinterpret_cast<const uint4 *>(kg + (t * a.H + h) * K + ch));
        const f32x4 *pp = reinterpret_cast<const f32x4 *>(a.P + ix);
        const f32x4 p0 = pp[0], p1 = pp[1];
        f32x8 xq, xk;
        bool far = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pv = e < 4 ? p0[e] : p1[e - 4];
            const float Ap = sA[b][ch + e], Ao = sA[b + 1][ch + e];
            xq[e] = qq[e] * a.qscale * clamp2(pv - Ap);
            xk[e] = kk[e] * clamp2(Ao - pv);
            far = far || fabsf(pv - Ap) > BWD_SPREAD || fabsf(pv - Ao) > BWD_SPREAD;
        }
        if (far) spread |= 1 << b;
        const bf16x8 bq = __builtin_convertvector(xq, bf16x8), bk = __builtin_convertvector(xk, bf16x8);
        *reinterpret_cast<bf16x8 *>(qh + ix) = bq;
        *reinterpret_cast<bf16x8 *>(kh + ix) = bk;
        const uint4 uq = __builtin_bit_cast(uint4, bq), uk = __builtin_bit_cast(uint4, bk);
        const uint32_t wq[4] = {uq.x, uq.y, uq.z, uq.w}, wk[4] = {uk.x, uk.y, uk.z, uk.w};
        uint32_t mq = 0u, mk = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mq = max(mq, max(wq[e] & 0x7fffu, (wq[e] >> 16) & 0x7fffu));
            mk = max(mk, max(wk[e] & 0x7fffu, (wk[e] >> 16) & 0x7fffu));
        }
#pragma unroll
        for (int bb = 0; bb < NBK; ++bb) {
            qm[bb] = bb == b ? max(qm[bb], mq) : qm[bb];
            km[bb] = bb == b ? max(km[bb], mk) : km[bb];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u16x2 xq = __builtin_bit_cast(u16x2, wq[e] & 0x7fff7fffu);
                const u16x2 xk = __builtin_bit_cast(u16x2, wk[e] & 0x7fff7fffu);
                qc[bb][e] = bb == b ? __builtin_elementwise_max(qc[bb][e], xq) : qc[bb][e];
                kc[bb][e] = bb == b ? __builtin_elementwise_max(kc[bb][e], xk) : kc[bb][e];
            }
        }
    }
    // the channel maxima over the wave's lanes of the same chunk (lanes K/8 apart),
    // then lanes 0 .. K/8 - 1 leave the wave's maxima of chunk `lane` in LDS
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int off = K / 8; off < 64; off <<= 1) {
                qc[bb][e] = __builtin_elementwise_max(
                    qc[bb][e], __builtin_bit_cast(u16x2, __shfl_xor(__builtin_bit_cast(int, qc[bb][e]), off)));
                kc[bb][e] = __builtin_elementwise_max(
                    kc[bb][e], __builtin_bit_cast(u16x2, __shfl_xor(__builtin_bit_cast(int, kc[bb][e]), off)));
            }
            const int lane = tid & 63;
            if (lane < K / 8) {
                sC[0][bb][tid >> 6][4 * lane + e] = __builtin_bit_cast(uint32_t, qc[bb][e]);
                sC[1][bb][tid >> 6][4 * lane + e] = __builtin_bit_cast(uint32_t, kc[bb][e]);
            }
        }
    if (spread) atomicOr(&sflag, spread);
    // the wave's maxima, then one atomic per wave and block
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb) {
        uint32_t x = qm[bb], y = km[bb];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            x = max(x, (uint32_t)__shfl_xor((int)x, off));
            y = max(y, (uint32_t)__shfl_xor((int)y, off));
        }
        if ((tid & 63) == 0) {
            if (x) atomicMax(&sqm[bb], x << 16);  // as float32 bits
            if (y) atomicMax(&skm[bb], y << 16);
        }
    }
    __syncthreads();
    if (tid < NBK) {
        uint32_t *bm = a.bmax + ((gb0 + tid) * HQ + hq) * BWD_BM;
        bm[0] = BWD_BLK * tid < n ? sqm[tid] : 0u;
        bm[1] = BWD_BLK * tid < n ? skm[tid] : 0u;
    }
    // all four entries of the tile, also those of blocks past a short tail (0)
    if (tid < NBK) a.flag[(gb0 + tid) * HQ + hq] = (BWD_BLK * tid < n && ((sflag >> tid) & 1)) ? sidx + 1 : 0;
    // the channel maxima of each block over the four waves: cmax[block, hq, {q, k}, K]
    for (int x = tid; x < 2 * NBK * (K / 2); x += 256) {
        const int qk = x / (NBK * (K / 2)), bb = (x / (K / 2)) % NBK, pr = x % (K / 2);
        u16x2 m = {0, 0};
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, sC[qk][bb][ww][pr]));
        reinterpret_cast<uint32_t *>(a.cmax + ((gb0 + bb) * HQ + hq) * 2 * K + qk * K)[pr] = __builtin_bit_cast(uint32_t, m);
    }
}

// ---------------------------------------------------------------- far tiles
// A pair in different 128-row tiles is read at an anchor between its rows:
// the dq kernel moves each key's k~ down to the anchor before its query tile,
// the dk/dv kernel each query's q~ down to the anchor of its key tile's last
// block.  Channel n of a value stored at anchor A_b and moved to A_x is below
// the block's largest stored magnitude of that channel (recorded by the anchor
// pass) times 2^(A_x,n - A_b,n), so a pair's score S_ij = q~_i . k~_j is below
// the sum over the channels of the two sides' bounds.  Without a scalar gate
// or a window the kernels leave out the pairs of a (query block, key tile) or
// (query tile, key block) whose bound is at most 2^(e - 26), with
// 2^e <= L_i = lse_i log2e for every query row of the pair: there S_ij lies
// below a quarter of half the float32 spacing of L_i, so S_ij - L_i rounds to
// -L_i and A_ij = 2^-L_i exactly, as the products would give it.  Such a pair
// adds bf16(2^-L_i) do_i to dv_j, which the dk/dv kernel takes from per-block
// suffix sums of those rows (the two small kernels below); its terms of dq_i,
// dk_j and X (each with the factor q~_i k~_j of a score below 2^(e - 26), i.e.
// at most |dS_ij| 2^(e - 26) in X) are dropped.  Pairs whose moved values all
// round to 0 in bf16 (from the block's largest magnitude over all channels,
// at most 2^-134 after the move) have every such term exactly 0 and are left
// out as well.  The dq kernel starts its walk at the first key block that has
// to be kept; the dk/dv kernel stops after the last query block that has to
// be kept.
//
// The exponent bound for a block of largest magnitude m (float bits), moved
// by gap: the moved values lie below 2^(this).
__device__ inline int moved_exponent(uint32_t mbits, float gap) {
    if (mbits == 0u) return -100000;
    int e;
    (void)frexpf(__uint_as_float(mbits), &e);  // m < 2^e
    return e + (int)fminf(fmaxf(gap, -100000.f), 100000.f);
}

// The far-pair test of one block against the other side's per-channel bounds
// M_n (in LDS): the moved values of the block's channels n are below
// c_n 2^(x_n - y_n), c_n its largest stored magnitude (bf16 bits in cm), x and y
// the anchors the move goes between, so every score of its pairs is below
// sum_n c_n 2^(x_n - y_n) M_n.  The pairs are left out when that bound is at
// most 2^(e - 26) (e >= -60 from the block's rows, see above; the sum is
// rounded and scaled by 1.001 against its float32 rounding) or when every moved
// value rounds to 0 (max_n (x_n - y_n) past -134 below the block's largest).
template <int K>
__device__ inline bool far_block_out(const uint16_t *cm, const float *x, const float *y, const float *M,
                                     uint32_t bmax_bits, int e) {
    float gap = -3.0e38f, bound = 0.f;
#pragma unroll 4
    for (int n = 0; n < K; n += 8) {
        const uint4 cw = *reinterpret_cast<const uint4 *>(cm + n);
        const uint32_t cv[4] = {cw.x, cw.y, cw.z, cw.w};
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(x + n), x1 = *reinterpret_cast<const f32x4 *>(x + n + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float d = (i < 4 ? x0[i] : x1[i - 4]) - y[n + i];
            gap = fmaxf(gap, d);
            const float c = __uint_as_float((i & 1 ? cv[i / 2] >> 16 : cv[i / 2] & 0xffffu) << 16);
            bound = fmaf(ldexpf(c, (int)fminf(fmaxf(d, -1000.f), 1000.f)), M[n + i], bound);
        }
    }
    if (moved_exponent(bmax_bits, gap) <= -134) return true;
    if (e < -60) return false;
    return bound * 1.001f <= ldexpf(1.f, e - 26);  // a NaN or inf bound keeps the block
}

// Per (32-row block, query head): the sum over its rows i < len of
// bf16(2^-L_i) do_i per value channel (the weights the dk/dv kernel's products
// give a pair of score 0), 64 threads per block, V/64 channels each.
template <int V>
__global__ __launch_bounds__(256) void bwd_wsum_kernel(BwdArgs a, int nblk) {
    constexpr int NBK = BR / BWD_BLK, CPT = V / 64;
    const int tile = blockIdx.x % nblk, hs = blockIdx.x / nblk, hq = hs % a.HQ, sidx = hs / a.HQ;
    const SegInfo sg = a.seg[sidx];
    const int r0 = tile * BR;
    if (r0 >= sg.len) return;
    const int b = threadIdx.x / 64, c0 = (threadIdx.x % 64) * CPT;
    const int64_t HQ = a.HQ;
    const int rb0 = r0 + BWD_BLK * b;
    float acc[CPT] = {};
    float lmin = FLT_MAX;  // the smallest L_i of the block's rows
    const __bf16 *dog = static_cast<const __bf16 *>(a.dout);
    // eight rows' loads in flight at a time (rows past the sequence weigh 0)
    for (int r8 = 0; r8 < BWD_BLK; r8 += 8) {
        float p[8], x[8][CPT];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const bool in = rb0 + r8 + r < sg.len;
            // a row past the sequence reads its last row (in bounds) with weight 0
            const int64_t t = sg.start + min(rb0 + r8 + r, sg.len - 1);
            const float L = a.lse[t * HQ + hq] * LOG2E;
            p[r] = in ? (float)(__bf16)__builtin_amdgcn_exp2f(-L) : 0.f;
            lmin = in ? fminf(lmin, L) : lmin;
#pragma unroll
            for (int e = 0; e < CPT; ++e) x[r][e] = (float)dog[(t * HQ + hq) * V + c0 + e];
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int e = 0; e < CPT; ++e) acc[e] += p[r] * x[r][e];
    }
    const int64_t gb = (int64_t)(sg.tile_base + tile) * NBK + b;
#pragma unroll
    for (int e = 0; e < CPT; ++e) a.wsum[(gb * HQ + hq) * V + c0 + e] = acc[e];
    // e with 2^e <= L_i for every row of the block (the far-tile rule above);
    // none for a block with some L_i <= 0 (or none in the sequence: no pairs)
    if (threadIdx.x % 64 == 0) {
        int e = BWD_NO_EXP;
        if (lmin > 0.f && lmin < FLT_MAX) {
            (void)frexpf(lmin, &e);  // 2^(e-1) <= lmin < 2^e
            e -= 1;
        }
        a.bmax[(gb * HQ + hq) * BWD_BM + 2] = (uint32_t)e;
    }
}

// Per (sequence, query head): the block sums above turned, in place, into the
// sums from each block to the sequence's end.  1024 threads: V channels times
// 1024 / V segments of the sequence's blocks; each segment sums its blocks,
// then walks them from its end down starting from the sum of the later
// segments (two reads of each block sum, the second from L2).
template <int V>
__global__ __launch_bounds__(1024) void bwd_wsuffix_kernel(BwdArgs a) {
    constexpr int NBK = BR / BWD_BLK, NS = 1024 / V;
    __shared__ float part[NS][V];
    const int sidx = blockIdx.x / a.HQ, hq = blockIdx.x % a.HQ;
    const int c = threadIdx.x % V, sgi = threadIdx.x / V;
    const SegInfo sg = a.seg[sidx];
    const int nb = (sg.len + BWD_BLK - 1) / BWD_BLK, per = (nb + NS - 1) / NS;
    const int b0 = min(nb, sgi * per), b1 = min(nb, b0 + per);
    const int64_t stride = (int64_t)a.HQ * V;
    float *w = a.wsum + ((int64_t)sg.tile_base * NBK * a.HQ + hq) * V + c;
    float s = 0.f;
#pragma unroll 8
    for (int b = b0; b < b1; ++b) s += w[(int64_t)b * stride];
    part[sgi][c] = s;
    __syncthreads();
    float acc = 0.f;
    for (int t = NS - 1; t > sgi; --t) acc += part[t][c];
    int b = b1 - 1;
    for (; b >= b0 + 7; b -= 8) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = w[(int64_t)(b - i) * stride];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc += x[i];
            w[(int64_t)(b - i) * stride] = acc;
        }
    }
    for (; b >= b0; --b) {
        acc += w[(int64_t)b * stride];
        w[(int64_t)b * stride] = acc;
    }
}

// x * 2^d per element for integer-valued d: an exact power of two of a bf16
// value, rounded back to bf16 (exact unless it leaves the normal range)
__device__ inline bf16x8 scale8(bf16x8 x, f32x8 d) {
    const f32x8 f = __builtin_convertvector(x, f32x8);
    f32x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = ldexpf(f[e], (int)fminf(fmaxf(d[e], -1000.0f), 1000.0f));
    return __builtin_convertvector(y, bf16x8);
}
__device__ inline f32x8 lds_f8(const float *p) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 2^(to - from) applied to an anchored value: from, to are integer anchors
__device__ inline float shift_anchor(float x, float to, float from) {
    return ldexpf(x, (int)fminf(fmaxf(to - from, -1000.0f), 1000.0f));
}

// ---------------------------------------------------------------- moves of staged tiles
// Every row of a tile staged by the off-tile walks moves by the same
// per-channel power of two 2^-dec_n, dec_n = from_n - to_n for two integer
// anchors.  A table of these moves is formed once per tile, two tiles ahead of
// its use, by one wave (channels 2l and 2l+1 in lane l): per channel pair the
// bf16 exponent-field decrements (min(dec, 255) << 7 in two u16) and the
// decrements themselves (two int16), and per tile whether every decrement is
// >= 0.  A staged bf16 value then moves by a saturating 16-bit subtract on its
// magnitude when they all are (the same bits as ldexp for a result in the
// normal range; 0, or a value below 2^-126, otherwise), else by ldexp.
constexpr int DEC_SLOTS = 4;  // tables in flight: formed at tile t - 3, read at t - 1
struct alignas(16) DecTab {
    uint32_t w[DEC_SLOTS][64];  // exponent-field decrements, K/2 <= 64 channel pairs
    uint32_t s[DEC_SLOTS][64];  // signed decrements
    int fast[DEC_SLOTS];        // every decrement of the tile >= 0
};
// Lane l of the forming wave (l < K/2 holds channels 2l, 2l+1 of `to` and `from`).
template <int K>
__device__ inline void dec_form(DecTab &t, int slot, int lane, f32x2 to, f32x2 from) {
    bool neg = false;
    if (lane < K / 2) {
        const int d0 = (int)fminf(fmaxf(from[0] - to[0], -1000.f), 1000.f);
        const int d1 = (int)fminf(fmaxf(from[1] - to[1], -1000.f), 1000.f);
        neg = d0 < 0 || d1 < 0;
        t.w[slot][lane] = ((uint32_t)min(max(d0, 0), 255) << 7) | ((uint32_t)min(max(d1, 0), 255) << 23);
        t.s[slot][lane] = ((uint32_t)d0 & 0xffffu) | ((uint32_t)d1 << 16);
    }
    const uint64_t any = __ballot(neg);
    if (lane == 0) t.fast[slot] = any == 0ull;
}
// Eight staged bf16 (raw bits) of channels ch .. ch + 7 moved by table `slot`.
__device__ inline bf16x8 dec_apply(const DecTab &t, int slot, bool fast, int ch, uint4 raw) {
    const uint32_t xv[4] = {raw.x, raw.y, raw.z, raw.w};
    if (fast) {
        const uint4 dw = *reinterpret_cast<const uint4 *>(&t.w[slot][ch / 2]);
        const uint32_t dv[4] = {dw.x, dw.y, dw.z, dw.w};
        uint32_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const u16x2 mag = __builtin_bit_cast(u16x2, xv[e] & 0x7fff7fffu);
            const u16x2 r = __builtin_elementwise_sub_sat(mag, __builtin_bit_cast(u16x2, dv[e]));
            out[e] = (xv[e] & 0x80008000u) | __builtin_bit_cast(uint32_t, r);
        }
        return __builtin_bit_cast(bf16x8, uint4{out[0], out[1], out[2], out[3]});
    }
    const uint4 sw = *reinterpret_cast<const uint4 *>(&t.s[slot][ch / 2]);
    const uint32_t sv[4] = {sw.x, sw.y, sw.z, sw.w};
    f32x8 x = to_f32(raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = ldexpf(x[e], -(int)(short)(sv[e / 2] >> (16 * (e % 2))));
    return __builtin_convertvector(x, bf16x8);
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
    constexpr int NBK = BR / BWD_BLK;
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
    // anchors: sA[0] = A of the block before the tile, sA[1 + b] = A of its block b
    __shared__ __attribute__((aligned(16))) float sA[NBK + 1][K];
    __shared__ int sFl[NBK];
    // per buffer: 1 + the index of the staged query tile when some of its moved
    // q~ is not 0 (a tile whose staged q~ is all 0 is left to the dead-tile path)
    __shared__ int sLive[2];
    __shared__ int sLast;  // the last query tile past the key tile that has to be kept
    __shared__ float sKM[K];  // per channel the bound of the key tile's k~ moved to A_K
    __shared__ DecTab sDec;  // the moves of staged q~ to A_K (tiles after the key tile)

    const BlockPos bp = block_pos(a, nblk, true);
    const SegInfo sg = a.seg[bp.seg];
    const int hq = bp.hq, j0 = bp.rb * BR;
    if (j0 >= sg.len) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
    const int64_t HQ = a.HQ;
    const int h = hq / (a.HQ / a.H);
    const int len = sg.len, jn = min(BR, len - j0);
    const int64_t s0 = sg.start;
    const int64_t gb0 = (int64_t)(sg.tile_base + bp.rb) * NBK;
    const __bf16 *vg = static_cast<const __bf16 *>(a.v);
    const __bf16 *dog = static_cast<const __bf16 *>(a.dout);

    if (tid < K) {
        sA[0][tid] = j0 > 0 ? a.Ab[((gb0 - 1) * HQ + hq) * K + tid] : 0.f;
#pragma unroll
        for (int b = 0; b < NBK; ++b)
            if (BWD_BLK * b < jn) sA[b + 1][tid] = a.Ab[((gb0 + b) * HQ + hq) * K + tid];
    }
    if (tid < NBK) sFl[tid] = BWD_BLK * tid < jn ? a.flag[(gb0 + tid) * HQ + hq] : 0;
    if (tid < 2) sLive[tid] = -1;
    __syncthreads();

    const int qend = a.window > 0 ? min(len, j0 + jn - 1 + a.window) : len;
    // Query tiles in the order the dk accumulators need: those after the key
    // tile (read at A of its last block, sA[NBK]), then the tile's own blocks
    // from the last down (own block bq read at the stored anchor of its q~).
    int n_off = qend > j0 + BR ? (qend - j0 - BR + BT - 1) / BT : 0;
    // The walk stops after the last query tile that has to be kept (see "far
    // tiles"); the rows after it, to the end of the sequence, reach dv through
    // the suffix sums of bf16(2^-L_i) do_i.
    int wcut = -1;  // the first sequence block left to the suffix sums
    if (!HAS_G && a.window <= 0 && n_off > 0) {
        if (tid == 0) sLast = -1;
        // per channel the bound of the tile's k~ moved to A_K: the largest over
        // its blocks b of the stored |k~| times 2^(A_K - A_b)
        if (tid < K) {
            float m = 0.f;
            for (int b = 0; b < NBK; ++b) {
                if (BWD_BLK * b >= jn) break;
                const float c = __uint_as_float((uint32_t)a.cmax[((gb0 + b) * HQ + hq) * 2 * K + K + tid] << 16);
                m = fmaxf(m, ldexpf(c, (int)fminf(fmaxf(sA[NBK][tid] - sA[b + 1][tid], -1000.f), 1000.f)));
            }
            sKM[tid] = m;
        }
        __syncthreads();
        for (int t = tid; t < n_off; t += NTH_KV) {
            const int b = (j0 + BR + BT * t) / BWD_BLK;  // the tile's block (BT rows)
            const int64_t gb = (int64_t)sg.tile_base * NBK + b;
            const uint32_t *bm = a.bmax + (gb * HQ + hq) * BWD_BM;
            // the block's q~, stored at A_(b-1), moved to A_K
            if (!far_block_out<K>(a.cmax + (gb * HQ + hq) * 2 * K, a.Ab + ((gb - 1) * HQ + hq) * K, sA[NBK], sKM,
                                  bm[0], (int)bm[2]))
                atomicMax(&sLast, t);
        }
        __syncthreads();
        const int keep = sLast + 1;
        if (keep < n_off) {
            wcut = (j0 + BR + BT * keep) / BWD_BLK;
            n_off = keep;
        }
    }
    const int n_dg = (min(qend, j0 + jn) - j0 + BT - 1) / BT;
    const int ntl = n_off + n_dg;
    auto tile_q0 = [&](int it) { return it < n_off ? j0 + BR + BT * it : j0 + BT * (ntl - 1 - it); };

    const __bf16 *qhg = static_cast<const __bf16 *>(a.qh);
    const __bf16 *khg = static_cast<const __bf16 *>(a.kh);
    // prefetch registers for one tile: q~ at its stored anchor and that anchor
    uint4 qraw[UK], oraw[UV];
    float il = 0.f, id = 0.f, ig = 0.f;
    const int sid = tid - NTH;  // staging thread index (dv waves)
    auto load_tile = [&](int it) {
        const int q0 = tile_q0(it);
        // rows past the sequence load its last row (in bounds) and are zeroed when stored
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = sid + NTH * u, r = c % BT, ch = 8 * (c / BT), i = min(q0 + r, len - 1);
            if (CK % NTH == 0 || c < CK) qraw[u] = *reinterpret_cast<const uint4 *>(qhg + ((s0 + i) * HQ + hq) * K + ch);
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
    auto store_tile = [&](int buf, int it, int tix) {
        const int q0 = tile_q0(it);
        uint32_t nz = 0u;
        // a tile after the key tile: q~ moved from A_(b-1) of its rows to A_K
        const int slot = it & (DEC_SLOTS - 1);
        const bool fast = it < n_off && sDec.fast[slot];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = sid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            if (CK % NTH == 0 || c < CK) {
                bf16x8 b = it < n_off ? dec_apply(sDec, slot, fast, ch, qraw[u]) : __builtin_bit_cast(bf16x8, qraw[u]);
                if (q0 + r >= len) b = __builtin_bit_cast(bf16x8, uint4{0u, 0u, 0u, 0u});
                *reinterpret_cast<bf16x8 *>(&sQ[buf][roff<RPK>(r, ch / 8)]) = b;
#pragma unroll
                for (int e = 0; e < 8; ++e) sQT[buf][(ch + e) * TP + r] = b[e];
                const uint4 ub = __builtin_bit_cast(uint4, b);
                nz |= ub.x | ub.y | ub.z | ub.w;
            }
        }
        if ((nz & 0x7fff7fffu) != 0u || it >= n_off) sLive[buf] = it + 1;
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
    // The move tables of the tiles after the key tile: the first dv wave forms
    // table t during iteration t - 3 (the first three before the walk) from
    // the anchors A_(b-1) of tile t's rows, loaded one iteration before.
    const bool former = w == NW;
    auto tab_anchor = [&](int t) {  // A_(b-1) of tile t's rows, channels 2 lane and 2 lane + 1
        const float *ab = a.Ab + ((gb0 + tile_q0(t) / BWD_BLK - bp.rb * NBK - 1) * HQ + hq) * K + 2 * lane;
        return *reinterpret_cast<const f32x2 *>(ab);
    };
    auto tab_form = [&](int t, f32x2 to) {
        const f32x2 from = lane < K / 2 ? *reinterpret_cast<const f32x2 *>(&sA[NBK][2 * lane]) : f32x2{0.f, 0.f};
        dec_form<K>(sDec, t & (DEC_SLOTS - 1), lane, to, from);
    };
    f32x2 an = {0.f, 0.f};
    if (former) {
        for (int t = 0; t < min(3, n_off); ++t) tab_form(t, lane < K / 2 ? tab_anchor(t) : f32x2{0.f, 0.f});
        if (3 < n_off && lane < K / 2) an = tab_anchor(3);
    }
    __syncthreads();
    const bool stager = w >= NW;
    if (stager) {
        load_tile(0);
        store_tile(0, 0, 0);
    }
    __syncthreads();
    if (stager && 1 < ntl) load_tile(1);

    // One role's whole walk over the query tiles; the two instantiations keep
    // their accumulators apart.  Every wave runs every tile after the key
    // tile (a tile with no visible pair for its keys, at most three past the
    // window, is masked to zero) and, of its own tile, the blocks at or after
    // its keys' block, except that block itself when it is flagged.
    auto walk = [&](auto dk_role) {
        constexpr bool DK = decltype(dk_role)::value;
        constexpr int NA = DK ? K / 32 : V / 32;
        const int wr = w % NW;
        const int jw = j0 + 32 * wr, j = jw + l32;
        const bool jok = j < len;
        const int64_t tj = s0 + (jok ? j : 0);
        const bool flagged = sFl[wr] != 0;
        // the own-tile block of tile it (or -1), and whether this wave computes it
        auto own_block = [&](int it) { return it < n_off ? -1 : ntl - 1 - it; };
        auto active = [&](int it) {
            const int bq = own_block(it);
            return bq < 0 || bq > wr || (bq == wr && !flagged);
        };
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
        // anchor index (into sA) of the dk accumulators, -1 before the first tile
        int fa = -1;
        if constexpr (DK) {
            // the wave's keys as second operands: k~ at its block's anchor (moved to
            // the anchor of each tile) and v rows of key j
            auto load_k = [&](bf16x8 *kv) {
#pragma unroll
                for (int s = 0; s < K / 16; ++s) {
                    const int ch = 16 * s + 8 * hl;
                    uint4 raw = {0, 0, 0, 0};
                    if (jok) raw = *reinterpret_cast<const uint4 *>(khg + (tj * HQ + hq) * K + ch);
                    kv[s] = __builtin_bit_cast(bf16x8, raw);
                }
            };
            bf16x8 vop[V / 16];
#pragma unroll
            for (int s = 0; s < V / 16; ++s) {
                const int ch = 16 * s + 8 * hl;
                uint4 raw = {0, 0, 0, 0};
                if (jok) raw = *reinterpret_cast<const uint4 *>(vg + (tj * a.H + h) * V + ch);
                vop[s] = __builtin_bit_cast(bf16x8, raw);
            }
            // 8 channels at channel block s times 2^(sA[p] - sA[m])
            auto move = [&](bf16x8 v8, int s, int p, int m) {
                const int ch = 16 * s + 8 * hl;
                return scale8(v8, lds_f8(&sA[p][ch]) - lds_f8(&sA[m][ch]));
            };
            // the accumulators at anchor sA[x]: acc(x) = acc(fa) 2^(sA[fa] - sA[x])
            // (at most 1 for a falling prefix: x only rises)
            auto acc_to = [&](int x) {
                if (fa >= 0) {
#pragma unroll
                    for (int n = 0; n < NA; ++n) {
                        const int d = (int)fminf(fmaxf(sA[fa][32 * n + l32] - sA[x][32 * n + l32], -1000.f), 1000.f);
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[n][r] = ldexpf(acc[n][r], d);
                    }
                }
                fa = x;
            };
            const float gj = (HAS_G && jok) ? a.G[tj * HQ + hq] : 0.f;
            // one query tile: S, dP, A, dS and dk += dS^T q~; S from the wave's k~
            // operands kget and the staged q~ rows passed through qget
            // FULL: the tile may skip the masks when every pair is visible (the
            // own tile's few blocks always take the masked copy: one copy less code)
            auto tile = [&](int it, auto kget, auto qget, auto FULL) {
                const int cur = it & 1;
                const int q0 = tile_q0(it);
                const int qrow = swap23(l32);
                f32x16 S = 0.f, dP = 0.f;
#pragma unroll
                for (int s = 0; s < K / 16; ++s)
                    S = mfma(qget(lds8(&sQ[cur][roff<RPK>(qrow, 2 * s + hl)]), s), kget(s), S);
#pragma unroll
                for (int s = 0; s < V / 16; ++s) dP = mfma(lds8(&sO[cur][roff<RPV>(qrow, 2 * s + hl)]), vop[s], dP);
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
                if (decltype(FULL)::value && full)
                    softmax(std::false_type{});
                else
                    softmax(std::true_type{});
#pragma unroll
                for (int n = 0; n < NA; ++n)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        acc[n] = mfma(db[c], lds8(&sQT[cur][(32 * n + l32) * TP + 16 * c + 8 * hl]), acc[n]);
            };
            auto dead_tile = [&](int it) {
                const int cur = it & 1, q0 = tile_q0(it);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int qi0 = 16 * c + 8 * hl;
                    f32x4 L4[2];
#pragma unroll
                    for (int x = 0; x < 2; ++x) L4[x] = *reinterpret_cast<const f32x4 *>(&sL[cur][qi0 + 4 * x]);
                    f32x8 p8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = q0 + qi0 + e;
                        const bool vis = jok && i < len && (a.window <= 0 || i - j < a.window);
                        p8[e] = vis ? __builtin_amdgcn_exp2f(-L4[e / 4][e % 4]) : 0.f;
                    }
                    *reinterpret_cast<bf16x8 *>(&sP[cur][wr][c][lane * 8]) = __builtin_convertvector(p8, bf16x8);
                }
            };
            // The query tiles after the key tile at sA[NBK], with k~ moved there
            // once; then the own tile's blocks bq: S at the stored k~'s anchor
            // sA[wr + 1], the staged q~ (at sA[bq]) moved there as it is read,
            // and dk += dS^T q~ at sA[bq].  Each loop holds one set of k~ registers.
            int it = 0;
            if (n_off > 0) {
                bf16x8 kop[K / 16];
                load_k(kop);
#pragma unroll
                for (int s = 0; s < K / 16; ++s) kop[s] = move(kop[s], s, NBK, wr + 1);
                acc_to(NBK);
                for (; it < n_off; ++it) {
                    // A tile whose moved q~ is 0 on every row and channel (far
                    // queries under strong decay): every score is exactly 0 and every
                    // product with q~ is 0, so dk gains nothing and A is bf16(2^-L_i)
                    // for each visible pair, written for the dv waves without the
                    // products (the probabilities the full step would give)
                    const bool live = HAS_G || __builtin_amdgcn_readfirstlane(sLive[it & 1]) == it + 1;
                    if (live)
                        tile(it, [&](int s) { return kop[s]; }, [&](bf16x8 x, int) { return x; }, std::true_type{});
                    else
                        dead_tile(it);
                    __syncthreads();
                }
            }
            {
                bf16x8 kst[K / 16];
                load_k(kst);
                for (; it < ntl; ++it) {
                    if (active(it)) {
                        const int x = own_block(it);
                        acc_to(x);
                        // q~ 2^(sA[x] - sA[wr + 1]): at most 1 for a later block
                        tile(it, [&](int s) { return kst[s]; },
                             [&](bf16x8 qv, int s) { return move(qv, s, x, wr + 1); }, std::false_type{});
                    }
                    __syncthreads();
                }
            }
        } else {
            // one tile behind the dk waves; these waves also stage every tile
            for (int it = 0; it < ntl; ++it) {
                if (it > 0 && active(it - 1)) dv_step(it - 1);
                if (it + 1 < ntl) store_tile((it & 1) ^ 1, it + 1, it + 1);
                __syncthreads();
                // the table before the tile's loads: its anchors, loaded before the
                // previous tile's, are in (store_tile waited for those)
                if (former && it + 3 < n_off) {
                    tab_form(it + 3, an);
                    if (it + 4 < n_off && lane < K / 2) an = tab_anchor(it + 4);
                }
                if (it + 2 < ntl) load_tile(it + 2);
            }
            if (ntl > 0 && active(ntl - 1)) dv_step(ntl - 1);
        }

        if (jw >= len) return;
        if constexpr (DK) {
            colsum += __shfl_xor(colsum, 32);
            if (hl == 0 && jok) a.Y[tj * HQ + hq] -= colsum;
        }
        // the dk accumulators' anchor (the key block's own with none)
        const int fx = fa >= 0 ? fa : wr + 1;
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
                    const float F = sA[fx][ch];
                    float dk = LN2 * clamp2(F - a.P[ix]) * acc[n][r];
                    if (flagged) dk += a.dkp[ix];
                    // the partials are read once, by the group sum: stored past the
                    // caches, which keep the rows the walks stream
                    __builtin_nontemporal_store(dk, &a.dkp[ix]);
                    // k (.) dk^(hq) from the bf16 k~ the dq products used (see the X note above)
                    a.X[ix] -= LN2 * shift_anchor((float)khg[ix], F, sA[wr + 1][ch]) * acc[n][r];
                } else {
                    const int64_t ix = (t * HQ + hq) * V + ch;
                    // the rows after the walk: the same bf16(2^-L_i) do_i for every key
                    const float far =
                        wcut >= 0 ? a.wsum[(((int64_t)sg.tile_base * NBK + wcut) * HQ + hq) * V + ch] : 0.f;
                    __builtin_nontemporal_store((flagged ? a.dvp[ix] + acc[n][r] : acc[n][r]) + far, &a.dvp[ix]);
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
    constexpr int NBK = BR / BWD_BLK;
    static_assert(CK % NTH == 0 && CV % NTH == 0, "tile chunks");
    __shared__ __attribute__((aligned(16))) __bf16 sK[2][rows_size<RPK>()];  // k~ rows
    __shared__ __attribute__((aligned(16))) __bf16 sKT[2][K * TP];           // k~ transposed
    __shared__ __attribute__((aligned(16))) __bf16 sV[2][rows_size<RPV>()];  // v rows
    __shared__ __attribute__((aligned(16))) float sGk[2][BT];
    // anchors: sA[0] = A of the block before the tile, sA[1 + b] = A of its block b
    __shared__ __attribute__((aligned(16))) float sA[NBK + 1][K];
    __shared__ int sFl[NBK];
    // per buffer: 1 + the first row of the staged key tile when some of its
    // moved k~ is not 0 (a tile staged as all 0 adds nothing and is skipped)
    __shared__ int sLive[2];
    __shared__ int sFirst;  // the first key block before the query tile that has to be kept
    __shared__ int sLe;        // e with 2^e <= L_i on the tile's rows
    __shared__ float sQM[K];  // per channel the bound of the tile's q~ moved to sA[0]
    __shared__ DecTab sDec;   // the moves of staged k~ to sA[0] (key tiles before the query tile)

    const BlockPos bp = block_pos(a, nblk, false);
    const SegInfo sg = a.seg[bp.seg];
    const int hq = bp.hq, i0 = bp.rb * BR;
    if (i0 >= sg.len) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hl = lane >> 5;
    const int64_t HQ = a.HQ;
    const int h = hq / (a.HQ / a.H);
    const int len = sg.len, in_ = min(BR, len - i0);
    const int64_t s0 = sg.start;
    const int64_t gb0 = (int64_t)(sg.tile_base + bp.rb) * NBK;
    const __bf16 *vg = static_cast<const __bf16 *>(a.v);
    const __bf16 *dog = static_cast<const __bf16 *>(a.dout);

    if (tid < K) {
        sA[0][tid] = i0 > 0 ? a.Ab[((gb0 - 1) * HQ + hq) * K + tid] : 0.f;
#pragma unroll
        for (int b = 0; b < NBK; ++b)
            if (BWD_BLK * b < in_) sA[b + 1][tid] = a.Ab[((gb0 + b) * HQ + hq) * K + tid];
    }
    if (tid < NBK) sFl[tid] = BWD_BLK * tid < in_ ? a.flag[(gb0 + tid) * HQ + hq] : 0;
    if (tid < 2) sLive[tid] = -1;
    __syncthreads();

    // the wave's queries as second operands
    const int iw = i0 + 32 * w, i = iw + l32;
    const bool iok = i < len;
    const int64_t ti = s0 + (iok ? i : 0);
    const bool flagged = sFl[w] != 0;
    const __bf16 *qhg = static_cast<const __bf16 *>(a.qh);
    const __bf16 *khg = static_cast<const __bf16 *>(a.kh);
    // q~ as stored (at sA[w], the anchor of the block before the wave's)
    auto load_q = [&](bf16x8 *qv) {
#pragma unroll
        for (int s = 0; s < K / 16; ++s) {
            const int ch = 16 * s + 8 * hl;
            uint4 raw = {0, 0, 0, 0};
            if (iok) raw = *reinterpret_cast<const uint4 *>(qhg + (ti * HQ + hq) * K + ch);
            qv[s] = __builtin_bit_cast(bf16x8, raw);
        }
    };
    bf16x8 oop[V / 16];
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
    // anchor index (into sA) of the accumulators, -1 before the first tile;
    // acc(x) = acc(fa) 2^(sA[x] - sA[fa]) (at most 1 for a falling prefix: x only falls)
    int fa = -1;
    auto acc_to = [&](int x) {
        if (fa >= 0) {
#pragma unroll
            for (int n = 0; n < K / 32; ++n) {
                const int d = (int)fminf(fmaxf(sA[x][32 * n + l32] - sA[fa][32 * n + l32], -1000.f), 1000.f);
#pragma unroll
                for (int r = 0; r < 16; ++r) dq[n][r] = ldexpf(dq[n][r], d);
            }
        }
        fa = x;
    };
    // 8 channels of q~ (or k~) at anchor sA[to] from anchor sA[from]: x 2^(sA[from] - sA[to])
    // for q~, x 2^(sA[to] - sA[from]) for k~
    auto lower_q = [&](bf16x8 x, int s, int from, int to) {
        const int ch = 16 * s + 8 * hl;
        return scale8(x, lds_f8(&sA[from][ch]) - lds_f8(&sA[to][ch]));
    };

    const int ilast = i0 + in_ - 1;
    int klo = a.window > 0 ? max(0, i0 - a.window + 1) / BT * BT : 0;
    // the walk starts at the first key block that has to be kept (see "far
    // tiles"); the blocks before it add nothing to dq or X beyond the dropped terms
    if (!HAS_G && a.window <= 0 && klo < i0) {
        if (tid == 0) {
            sFirst = i0 / BWD_BLK;
            sLe = INT_MAX;
        }
        // per channel the bound of the tile's q~ moved to sA[0]: the largest over
        // its blocks b (q~ stored at sA[b]) of the stored |q~| times 2^(sA[b] - sA[0])
        if (tid < K) {
            float m = 0.f;
            for (int b = 0; b < NBK; ++b) {
                if (BWD_BLK * b >= in_) break;
                const float c = __uint_as_float((uint32_t)a.cmax[((gb0 + b) * HQ + hq) * 2 * K + tid] << 16);
                m = fmaxf(m, ldexpf(c, (int)fminf(fmaxf(sA[b][tid] - sA[0][tid], -1000.f), 1000.f)));
            }
            sQM[tid] = m;
        }
        __syncthreads();
        // e with 2^e <= L_i for every row of the tile
        if (tid < NBK && BWD_BLK * tid < in_) atomicMin(&sLe, (int)a.bmax[((gb0 + tid) * HQ + hq) * BWD_BM + 2]);
        __syncthreads();
        const int le = sLe;
        const int nfar = (i0 - klo) / BWD_BLK;
        for (int t = tid; t < nfar; t += NTH) {
            const int b = klo / BWD_BLK + t;
            const int64_t gb = (int64_t)sg.tile_base * NBK + b;
            // the block's k~, stored at A_b, moved to A_Q = sA[0]
            if (!far_block_out<K>(a.cmax + (gb * HQ + hq) * 2 * K + K, sA[0], a.Ab + (gb * HQ + hq) * K, sQM,
                                  a.bmax[(gb * HQ + hq) * BWD_BM + 1], le))
                atomicMin(&sFirst, b);
        }
        __syncthreads();
        klo = sFirst * BWD_BLK;
    }

    // prefetch registers for one tile: k~ at its block's anchor and that anchor
    uint4 kraw[UK], vraw[UV];
    float kgv = 0.f;
    auto load_tile = [&](int k0) {
        // rows past the sequence load its last row (in bounds) and are zeroed when stored
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            const int64_t t = s0 + min(k0 + r, len - 1);
            kraw[u] = *reinterpret_cast<const uint4 *>(khg + (t * HQ + hq) * K + ch);
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
        uint32_t nz = 0u;
        // a tile before the query tile: k~ moved from the anchor of its block to sA[0]
        const int slot = ((k0 - klo) / BT) & (DEC_SLOTS - 1);
        const bool fast = k0 < i0 && sDec.fast[slot];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            bf16x8 b = k0 < i0 ? dec_apply(sDec, slot, fast, ch, kraw[u]) : __builtin_bit_cast(bf16x8, kraw[u]);
            if (k0 + r >= len) b = __builtin_bit_cast(bf16x8, uint4{0u, 0u, 0u, 0u});
            *reinterpret_cast<bf16x8 *>(&sK[buf][roff<RPK>(r, ch / 8)]) = b;
#pragma unroll
            for (int e = 0; e < 8; ++e) sKT[buf][(ch + e) * TP + r] = b[e];
            const uint4 ub = __builtin_bit_cast(uint4, b);
            nz |= ub.x | ub.y | ub.z | ub.w;
        }
        if ((nz & 0x7fff7fffu) != 0u || k0 >= i0) sLive[buf] = k0 + 1;
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int c = tid + NTH * u, r = c % BT, ch = 8 * (c / BT);
            // a row past the sequence stores zeros (selected per dword, in registers)
            const bool ok = k0 + r < len;
            uint4 vv = vraw[u];
            vv.x = ok ? vv.x : 0u;
            vv.y = ok ? vv.y : 0u;
            vv.z = ok ? vv.z : 0u;
            vv.w = ok ? vv.w : 0u;
            *reinterpret_cast<uint4 *>(&sV[buf][roff<RPV>(r, ch / 8)]) = vv;
        }
        if (HAS_G && tid < BT) sGk[buf][tid] = kgv;
    };

    // one key tile: S, dP, dS and dq += dS k~; S from the wave's q~ operands
    // qget and the staged k~ rows passed through kget
    // FULL: as in the dk/dv kernel
    auto tile = [&](int k0, int cur, auto qget, auto kget, auto FULL) {
        f32x16 S = 0.f, dP = 0.f;
        const int krow = swap23(l32);
#pragma unroll
        for (int s = 0; s < K / 16; ++s)
            S = mfma(kget(lds8(&sK[cur][roff<RPK>(krow, 2 * s + hl)]), s), qget(s), S);
#pragma unroll
        for (int s = 0; s < V / 16; ++s) dP = mfma(lds8(&sV[cur][roff<RPV>(krow, 2 * s + hl)]), oop[s], dP);

        // every pair of the tile visible: no mask
        const bool full = iw + 31 < len && k0 + BT - 1 <= iw && (a.window <= 0 || iw + 31 - k0 < a.window);
        bf16x8 db[2];
        auto softmax = [&](auto masked) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int kj0 = 16 * c + 8 * hl;
                f32x4 G4[2];
                if (HAS_G) {
#pragma unroll
                    for (int x2 = 0; x2 < 2; ++x2) G4[x2] = *reinterpret_cast<const f32x4 *>(&sGk[cur][kj0 + 4 * x2]);
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
        if (decltype(FULL)::value && full)
            softmax(std::false_type{});
        else
            softmax(std::true_type{});
#pragma unroll
        for (int n = 0; n < K / 32; ++n)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dq[n] = mfma(db[c], lds8(&sKT[cur][(32 * n + l32) * TP + 16 * c + 8 * hl]), dq[n]);
    };
    // The move tables of the key tiles before the query tile: wave 0 forms
    // table t during iteration t - 3 (the first three before the walk) from
    // the anchors of tile t's block, loaded one iteration before.
    const int nofft = (i0 - klo) / BT;
    auto tab_anchor = [&](int t) {  // A of tile t's key block, channels 2 lane and 2 lane + 1
        const float *ab = a.Ab + ((gb0 - bp.rb * NBK + (klo + BT * t) / BWD_BLK) * HQ + hq) * K + 2 * lane;
        return *reinterpret_cast<const f32x2 *>(ab);
    };
    auto tab_form = [&](int t, f32x2 from) {
        const f32x2 to = lane < K / 2 ? *reinterpret_cast<const f32x2 *>(&sA[0][2 * lane]) : f32x2{0.f, 0.f};
        dec_form<K>(sDec, t & (DEC_SLOTS - 1), lane, to, from);
    };
    f32x2 an = {0.f, 0.f};
    if (w == 0) {
        for (int t = 0; t < min(3, nofft); ++t) tab_form(t, lane < K / 2 ? tab_anchor(t) : f32x2{0.f, 0.f});
        if (3 < nofft && lane < K / 2) an = tab_anchor(3);
    }
    __syncthreads();
    auto advance = [&](int k0, int cur) {
        if (k0 + BT <= ilast) store_tile(cur ^ 1, k0 + BT);
        __syncthreads();
        // the table before the tile's loads (as in the dk/dv kernel)
        const int t3 = (k0 - klo) / BT + 3;
        if (w == 0 && t3 < nofft) {
            tab_form(t3, an);
            if (t3 + 1 < nofft && lane < K / 2) an = tab_anchor(t3 + 1);
        }
        if (k0 + 2 * BT <= ilast) load_tile(k0 + 2 * BT);
    };

    // double-buffered as in the dk/dv kernel.  The key tiles before the query
    // tile at sA[0], with q~ moved there once; then the tile's own blocks b
    // (for the waves at or after block b, the wave's own block only when it is
    // not flagged): S at the stored q~'s anchor sA[w], the staged k~ moved
    // there as it is read, and dq += dS k~ at the block's own anchor sA[1 + b].
    // Each loop holds one set of q~ registers.
    load_tile(klo);
    store_tile(0, klo);
    __syncthreads();
    if (klo + BT <= ilast) load_tile(klo + BT);
    int k0 = klo, it = 0;
    if (k0 < i0) {
        bf16x8 qop[K / 16];
        load_q(qop);
#pragma unroll
        for (int s = 0; s < K / 16; ++s) qop[s] = lower_q(qop[s], s, w, 0);
        acc_to(0);
        for (; k0 < i0; k0 += BT, ++it) {
            // a tile staged as all 0 (far keys under strong decay) adds exactly
            // nothing to dq and X; without a scalar gate nothing else reads it
            const bool live = HAS_G || __builtin_amdgcn_readfirstlane(sLive[it & 1]) == k0 + 1;
            if (live)
                tile(k0, it & 1, [&](int s) { return qop[s]; }, [&](bf16x8 x, int) { return x; }, std::true_type{});
            advance(k0, it & 1);
        }
    }
    {
        bf16x8 qst[K / 16];
        load_q(qst);
        for (; k0 <= ilast; k0 += BT, ++it) {
            const int b = (k0 - i0) / BT;
            if (b < w || (b == w && !flagged)) {
                const int x = b + 1;
                acc_to(x);
                // k~ 2^(sA[w] - sA[x]): at most 1 for an earlier block
                tile(k0, it & 1, [&](int s) { return qst[s]; },
                     [&](bf16x8 kv, int s) { return lower_q(kv, s, w, x); }, std::false_type{});
            }
            advance(k0, it & 1);
        }
    }

    if (iw >= len) return;
    rowsum += __shfl_xor(rowsum, 32);
    if (hl == 0 && iok) {
        a.Y[ti * HQ + hq] = flagged ? a.Y[ti * HQ + hq] + rowsum : rowsum;
        a.Z[ti * HQ + hq] = a.sink ? -exp2f(a.sink[hq] * LOG2E - lse2) * Di : 0.f;
    }
    // the accumulators' anchor (the stored q~'s with none)
    const int fx = fa >= 0 ? fa : w;
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
            const float F = sA[fx][ch];
            float dqv = a.scale * clamp2(a.P[ix] - F) * dq[n][r];
            float xv = LN2 * shift_anchor((float)qhg[ix], sA[w][ch], F) * dq[n][r];
            if (flagged) {
                dqv += a.dqd[ix];
                xv += a.X[ix];
            }
            __builtin_nontemporal_store((__bf16)dqv, &dqg[ix]);  // a result: not read again
            a.X[ix] = xv;
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
    for (int e = 0; e < KL; ++e) __builtin_nontemporal_store((__bf16)sk[e], &dkg[e]);  // results: not read again
#pragma unroll
    for (int e = 0; e < VL; ++e) __builtin_nontemporal_store((__bf16)sv[e], &dvg[e]);
}

template <int K, int V, bool HAS_G>
hipError_t run(const BwdArgs &a, hipStream_t st) {
    const int nblk = (int)cdiv(a.max_seqlen, BR);
    const unsigned nb = (unsigned)((int64_t)a.HQ * a.nseg * nblk);
    hipLaunchKernelGGL((bwd_anchor_kernel<K>), dim3(nb), dim3(256), 0, st, a, nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!HAS_G && a.window <= 0) {  // the dv sums of the rows the dk/dv walk may leave out
        hipLaunchKernelGGL((bwd_wsum_kernel<V>), dim3(nb), dim3(256), 0, st, a, nblk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_wsuffix_kernel<V>), dim3((unsigned)(a.nseg * a.HQ)), dim3(1024), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the pairs inside flagged blocks, before the kernels that add them
    e = launch_bwd_diag(a, true, false, st);
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
