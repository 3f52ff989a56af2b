// wall_prep.hip -- per-call preparation for the fused forward, one launch.
//
// Each block takes one 128-row tile of one sequence and either one query
// head (keys) or one kv head (values):
// 1. segments: the block finds the sequence its tile belongs to (one SegInfo
//    per sequence: start row, length, index of its first 128-row tile in the
//    tiled workspace; tiles never straddle two sequences, so a tile's rows
//    always share one prefix P); block (0, 0) also stores the table.
// 2. keys and queries, per (tile, query head): the anchors R[n] =
//    floor(P[a][n]) at the tile's last row a, the carry record that moves a
//    query from this tile's anchors to the previous tile's, and the
//    decay-rescaled keys
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
//    any gate strength.  For the fused kernel's diagonal phase (the keys of a
//    query's own tile) the same rows again, each 32-row block anchored at its
//    own last row A: k[j] * exp2(A - P[j]) and q[j] * scale*log2e *
//    exp2(P[j] - A), the carry records between those anchors, and per tile a
//    mask of the blocks whose rows lie more than DIAG_SPREAD from their anchor.
// 3. values, per (tile, kv head): v transposed to [V][128] for the bf16 MFMA
//    kernel (its PV operand reads keys contiguously, each thread transposing
//    an 8 x 8 block in registers); zero-padded; and the tile's float32 sum
//    of its value rows per channel.
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

// The records of (tile, query head) for channels 8*c8 .. +7 (anchors R of the
// tile, A of its 32-row blocks, Lp of the previous tile; `later`: the tile is
// not its sequence's first): the anchor table entry, the tile's carry record
// (the shift from R to Lp, a bf16 exponent decrement) and the diagonal records
// (each block's shift from Lp, block b+1's to block b's).  Returns bit 0 set
// when some channel's tile shift is negative (the prefix grows) and, from bit
// 8, the diagonal records that grow.
template <int K>
__device__ inline uint32_t write_records(const PrepArgs &a, int tile, int hq, int c8, bool later, f32x8 R,
                                         const f32x8 (&A)[TILE / DBLK], f32x8 Lp, uint32_t &dmin) {
    constexpr int NB = TILE / DBLK;
    const int64_t HQ = a.HQ;
    *reinterpret_cast<f32x8 *>(a.anchor + ((int64_t)tile * HQ + hq) * K + c8 * 8) = R;
    auto shift = [](float d) { return (uint32_t)fminf(fmaxf(d, 0.f), 255.f) * 128u; };
    bool up = false;
    dmin = later ? 255u : 0u;
    uint32_t dgrow = 0;
    uint32_t *rec = a.rec + ((int64_t)tile * HQ + hq) * REC_WORDS;
    uint32_t *drec = a.drec + ((int64_t)tile * HQ + hq) * DREC_N * (K / 2);
    for (int e = 0; e < 8; e += 2) {
        const int wd = (c8 * 8 + e) / 2;
        uint32_t w = 0;
        if (later) {
            const float d0 = Lp[e] - R[e], d1 = Lp[e + 1] - R[e + 1];
            up = up || d0 < 0.f || d1 < 0.f;
            w = shift(d0) | (shift(d1) << 16);
            dmin = min(dmin, min(shift(d0), shift(d1)) / 128u);
        }
        rec[wd] = w;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint32_t x = 0;
            if (later) {
                const float d0 = Lp[e] - A[b][e], d1 = Lp[e + 1] - A[b][e + 1];
                if (d0 < 0.f || d1 < 0.f) dgrow |= 1u << b;
                x = shift(d0) | (shift(d1) << 16);
            }
            drec[b * (K / 2) + wd] = x;
        }
#pragma unroll
        for (int b = 0; b + 1 < NB; ++b) {
            const float d0 = A[b][e] - A[b + 1][e], d1 = A[b][e + 1] - A[b + 1][e + 1];
            if (d0 < 0.f || d1 < 0.f) dgrow |= 1u << (NB + b);
            drec[(NB + b) * (K / 2) + wd] = shift(d0) | (shift(d1) << 16);
        }
    }
    return (up ? 1u : 0u) | (dgrow << 8);
}

template <int K>
__device__ inline void key_tile(const PrepArgs &a, int tile, int hq, const SegInfo &sg) {
    constexpr int CPR = K / 8;          // 8-channel chunks per row
    constexpr int RPP = 256 / CPR;      // rows per pass
    constexpr int NPASS = TILE / RPP;
    constexpr int NB = TILE / DBLK;     // 32-row blocks per tile
    __shared__ uint32_t sflag, sdmin, skmax;
    __shared__ uint32_t skc[K];  // per channel the largest |k| (float bits)
    const int c = tile - sg.tile_base;
    const int h = hq / (int)(a.HQ / a.H);
    const int c8 = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    const int64_t HQ = a.HQ;
    if (threadIdx.x == 0) {
        sflag = 0u;
        sdmin = 255u;
        skmax = 0u;
    }
    if (threadIdx.x < K) skc[threadIdx.x] = 0u;
    __syncthreads();
    // anchors: the tile's last row (keys read from later tiles) and each
    // 32-row block's last row (the fused kernel's diagonal phase)
    const int arow = min(c * TILE + TILE - 1, sg.len - 1);
    const float *Pa = a.P + ((int64_t)(sg.start + arow) * HQ + hq) * K + c8 * 8;
    f32x8 R, A[NB];
    for (int e = 0; e < 8; ++e) R[e] = floorf(Pa[e]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int brow = min(c * TILE + DBLK * b + DBLK - 1, sg.len - 1);
        const f32x8 pb = *reinterpret_cast<const f32x8 *>(a.P + ((int64_t)(sg.start + brow) * HQ + hq) * K + c8 * 8);
        for (int e = 0; e < 8; ++e) A[b][e] = floorf(pb[e]);
    }
    if (r0 == 0) {
        f32x8 Lp = R;  // the previous tile's anchors (none for a sequence's first tile)
        if (c > 0) {
            const float *Pp = a.P + ((int64_t)(sg.start + c * TILE - 1) * HQ + hq) * K + c8 * 8;
            for (int e = 0; e < 8; ++e) Lp[e] = floorf(Pp[e]);
        }
        uint32_t dmin;
        const uint32_t gr = write_records<K>(a, tile, hq, c8, c > 0, R, A, Lp, dmin);
        const bool any_up = __any(gr & 1u);  // the r0 == 0 threads are lanes 0..K/8-1 of wave 0
        if (threadIdx.x == 0) a.rec[((int64_t)tile * HQ + hq) * REC_WORDS + REC_GROW] = any_up ? 1u : 0u;
        if (gr >> 8) atomicOr(&sflag, gr & ~0xffu);
        atomicMin(&sdmin, dmin);
    }
    const __bf16 *qin = static_cast<const __bf16 *>(a.q);
    const __bf16 *kin = static_cast<const __bf16 *>(a.k);
    const int64_t o0 = ((int64_t)tile * HQ + hq) * TILE * K;
    __bf16 *kout = static_cast<__bf16 *>(a.kt) + o0;
    __bf16 *kdout = static_cast<__bf16 *>(a.kd) + o0;
    __bf16 *qdout = static_cast<__bf16 *>(a.qd) + o0;
    // the thread's rows in two batches, each batch's loads in flight before any is used
    constexpr int NH = NPASS / 2;
    uint32_t flags = 0;
    float kmax = 0.f;
    f32x8 kmc = {};  // per channel of the thread's chunk the largest |k| of its rows
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        f32x8 kv[NH], pv[NH], qv[NH];
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int j = c * TILE + r0 + (half * NH + i) * RPP;
            kv[i] = f32x8{};
            pv[i] = f32x8{};
            qv[i] = f32x8{};
            if (j < sg.len) {
                const int64_t tok = sg.start + j;
                kv[i] = Vec8<__bf16>::load(kin + (tok * a.H + h) * K + c8 * 8);
                qv[i] = Vec8<__bf16>::load(qin + (tok * HQ + hq) * K + c8 * 8);
                pv[i] = *reinterpret_cast<const f32x8 *>(a.P + (tok * HQ + hq) * K + c8 * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int row = r0 + (half * NH + i) * RPP, b = row / DBLK;
            const bool valid = c * TILE + row < sg.len;
            f32x8 kl, kb, qb;
            float dev = 0.f;
            for (int e = 0; e < 8; ++e) {
                kmax = fmaxf(kmax, fabsf(kv[i][e]));
                kmc[e] = fmaxf(kmc[e], fabsf(kv[i][e]));
                kl[e] = kv[i][e] * __builtin_amdgcn_exp2f(fminf(fmaxf(R[e] - pv[i][e], EXP2_LO), EXP2_HI));
                const float x = pv[i][e] - A[b][e];
                dev = fmaxf(dev, fabsf(x));
                kb[e] = kv[i][e] * __builtin_amdgcn_exp2f(fminf(fmaxf(-x, EXP2_LO), EXP2_HI));
                qb[e] = qv[i][e] * a.qscale * __builtin_amdgcn_exp2f(fminf(fmaxf(x, EXP2_LO), EXP2_HI));
            }
            if (valid && dev > DIAG_SPREAD) flags |= 1u << b;
            Vec8<__bf16>::store(kout + row * K + c8 * 8, kl);
            Vec8<__bf16>::store(kdout + row * K + c8 * 8, kb);
            Vec8<__bf16>::store(qdout + row * K + c8 * 8, qb);
        }
    }
    if (flags) atomicOr(&sflag, flags);
    atomicMax(&skmax, __float_as_uint(kmax));  // non-negative floats order as their bits
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicMax(&skc[c8 * 8 + e], __float_as_uint(kmc[e]));
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *rec = a.rec + ((int64_t)tile * HQ + hq) * REC_WORDS;
        rec[REC_DIAG] = sflag;
        rec[REC_DMIN] = sdmin;
        rec[REC_KMAX] = skmax;
    }
    if (threadIdx.x < K) a.kcm[((int64_t)tile * HQ + hq) * K + threadIdx.x] = __uint_as_float(skc[threadIdx.x]);
}

// Value tile of (tile, kv head), transposed [V][TILE].  Thread (kb, db)
// moves the 8 x 8 block of keys 8kb.. and values 8db..  The tile's float32 sum
// over its rows per value channel (rows past the sequence count 0) goes to
// vsum: the fused kernel reads it for keys that every query of a block sees
// with the same weight.  Called by every thread of a block.
template <typename T, int V>
__device__ inline void value_tile(const PrepArgs &a, int tile, int h, const SegInfo &sg) {
    constexpr int DB = V / 8, KB = TILE / 8;
    static_assert(DB * KB <= 256, "one 8 x 8 block per thread");
    __shared__ float colsum[KB][V];
    const int c = tile - sg.tile_base;
    const T *vin = static_cast<const T *>(a.v);
    T *vout = static_cast<T *>(a.vt) + ((int64_t)tile * a.H + h) * V * TILE;
    const int t = threadIdx.x;
    if (t < DB * KB) {
        const int db = t % DB, kb = t / DB;
        f32x8 x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = c * TILE + kb * 8 + i;
            x[i] = j < sg.len ? Vec8<T>::load(vin + ((int64_t)(sg.start + j) * a.H + h) * V + db * 8) : f32x8{};
        }
        f32x8 cs = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) cs += x[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) colsum[kb][db * 8 + e] = cs[e];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f32x8 col;
#pragma unroll
            for (int i = 0; i < 8; ++i) col[i] = x[i][e];
            Vec8<T>::store(vout + (db * 8 + e) * TILE + kb * 8, col);
        }
    }
    __syncthreads();
    if (t < V) {
        float s = colsum[0][t];
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) s += colsum[kb][t];
        a.vsum[((int64_t)tile * a.H + h) * V + t] = s;
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
        key_tile<K>(a, tile, y, sg);
    else
        value_tile<__bf16, V>(a, tile, y - (int)a.HQ, sg);
}

// ---------------------------------------------------------------- prefix and preparation in one pass
// B sequences of T rows with T a multiple of TILE, so the scan's 128-row
// chunks are the tiles.  Block (tile c, slice y) takes SP_CV vectors of 8
// channels of HQ*K (one or two whole query heads), thread (sub, cv) the 8 rows
// of subgroup sub (of 16) and channels 8*cv .. +7 of the slice.  Pass 1 sums
// each thread's rows of g; from the tile's carry and the subgroup sums every
// thread then knows the prefix E_b at the end of each 32-row block (the sums
// of its four subgroups added in order to E_(b-1), E_(-1) = the carry; E_3 =
// the next tile's carry when that tile is in the same sequence, so that the
// next tile's Lp is the floor of the P stored here).  The carry of tile c is
// the sum of the chunk sums of the sequence's tiles 0 .. c-1, taken as 16
// interleaved partial sums (tiles c' = p mod 16 in order), then the parts in
// order: every block that needs the carry of a tile forms it the same way,
// so tile c's block and tile c+1's agree on it bit for bit.  Pass 2 runs along the
// thread's rows from the prefix before its subgroup: P = pscale * the running
// sum, except P = pscale * E_b at a block's last row, so that the anchors
// A_b = floor(pscale * E_b) and R = A_3 are the floors of the P stored at
// their rows; it writes P and the tile's keys and queries as key_tile does.
// Value tiles and the sequence table as in prep_kernel.
constexpr int SP_SUB = 8;                 // rows per thread
constexpr int SP_NSUB = TILE / SP_SUB;    // subgroups per tile
constexpr int SP_CV = 256 / SP_NSUB;      // channel vectors per block
__device__ inline bf16x8 raw8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
template <int K>
__device__ inline void scan_key_slice(const PrepArgs &a, int tile, int y) {
    constexpr int NB = TILE / DBLK, SPB = DBLK / SP_SUB;  // blocks per tile, subgroups per block
    constexpr int HPS = (SP_CV * 8 + K - 1) / K;            // query heads per slice
    __shared__ f32x8 ssum[SP_NSUB][SP_CV];
    __shared__ f32x8 spart[2][SP_NSUB][SP_CV];  // partial carries of this tile and the next
    __shared__ uint32_t sflag[HPS], sgrow[HPS], sdmin[HPS], skmax[HPS];
    __shared__ uint32_t skc[SP_CV * 8];  // per channel of the slice the largest |k| (float bits)
    const int tid = threadIdx.x, sub = tid / SP_CV, cv = tid % SP_CV, rb = sub / SPB;
    const int64_t C = a.HQ * K, HQ = a.HQ;
    const int64_t ch = ((int64_t)y * SP_CV + cv) * 8;
    const bool on = ch < C;
    const int hq = (int)(ch / K), hl = cv / (K / 8), c8 = (int)((ch % K) / 8);
    const int h = hq / (int)(a.HQ / a.H);
    const int tps = (int)(a.T / TILE), c = tile % tps;  // tile within its sequence
    const int64_t row0 = (int64_t)tile * TILE + SP_SUB * sub;  // the thread's first flat row
    const __bf16 *gin = static_cast<const __bf16 *>(a.g);
    if (tid < HPS) {
        sflag[tid] = 0u;
        sgrow[tid] = 0u;
        sdmin[tid] = 255u;
        skmax[tid] = 0u;
    }
    if (tid < SP_CV * 8) skc[tid] = 0u;
    // pass 1: the sum of the thread's rows; meanwhile the partial carries:
    // thread sub sums the chunk sums of the sequence's tiles sub, sub + 16, ..
    // before this tile (pc) and before the next (pn), in tile order (the
    // loads four at a time, zeros past the end)
    f32x8 s = {}, pc = {};
    if (on) {
        bf16x8 x[SP_SUB];
#pragma unroll
        for (int i = 0; i < SP_SUB; ++i) x[i] = raw8(gin + (row0 + i) * C + ch);
        const float *cs = a.csum + (int64_t)(tile - c) * C + ch;  // the sequence's first chunk
        for (int cc0 = sub; cc0 < c; cc0 += 4 * SP_NSUB) {
            f32x8 t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cc = cc0 + j * SP_NSUB;
                t[j] = cc < c ? *reinterpret_cast<const f32x8 *>(cs + (int64_t)cc * C) : f32x8{};
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) pc += t[j];
        }
#pragma unroll
        for (int i = 0; i < SP_SUB; ++i) s += __builtin_convertvector(x[i], f32x8);
    }
    f32x8 pn = pc;
    if (on && c % SP_NSUB == sub) pn += *reinterpret_cast<const f32x8 *>(a.csum + (int64_t)tile * C + ch);
    spart[0][sub][cv] = pc;
    spart[1][sub][cv] = pn;
    ssum[sub][cv] = s;
    __syncthreads();
    bool spread = false;
    if (on) {
        // the running sum before the tile (0 at a sequence's first tile)
        f32x8 carry = spart[0][0][cv], nextc = spart[1][0][cv];
#pragma unroll
        for (int p = 1; p < SP_NSUB; ++p) {
            carry += spart[0][p][cv];
            nextc += spart[1][p][cv];
        }
        // the prefix at the end of each block and before the thread's subgroup
        f32x8 E[NB], A[NB], run = carry;
        f32x8 acc = carry;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int u = 0; u < SPB; ++u) {
                if (b * SPB + u == sub) run = acc;
                acc += ssum[b * SPB + u][cv];
            }
            E[b] = acc;
        }
        if (c + 1 < tps) E[NB - 1] = nextc;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) A[b][e] = floorf(a.pscale * E[b][e]);
        const f32x8 R = A[NB - 1];
        if (sub == 0) {
            f32x8 Lp = R;
            if (c > 0)
#pragma unroll
                for (int e = 0; e < 8; ++e) Lp[e] = floorf(a.pscale * carry[e]);
            uint32_t dmin;
            const uint32_t gr = write_records<K>(a, tile, hq, c8, c > 0, R, A, Lp, dmin);
            if (gr) atomicOr(&sgrow[hl], gr);
            atomicMin(&sdmin[hl], dmin);
        }
        // pass 2: P along the rows, then the keys and queries at the anchors
        // the thread's block's anchor and end prefix, by selects (a runtime index
        // into the arrays would keep all of them live through pass 2)
        f32x8 Ab = A[0], Eb = E[0];
#pragma unroll
        for (int b = 1; b < NB; ++b) {
            const bool mine = rb == b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Ab[e] = mine ? A[b][e] : Ab[e];
                Eb[e] = mine ? E[b][e] : Eb[e];
            }
        }
        const __bf16 *qin = static_cast<const __bf16 *>(a.q);
        const __bf16 *kin = static_cast<const __bf16 *>(a.k);
        const int64_t o0 = ((int64_t)tile * HQ + hq) * TILE * K + c8 * 8;
        __bf16 *kout = static_cast<__bf16 *>(a.kt) + o0;
        __bf16 *kdout = static_cast<__bf16 *>(a.kd) + o0;
        __bf16 *qdout = static_cast<__bf16 *>(a.qd) + o0;
        // the rows' loads in flight as raw bf16 before any is used
        bf16x8 x[SP_SUB], kr[SP_SUB], qr[SP_SUB];
#pragma unroll
        for (int i = 0; i < SP_SUB; ++i) {
            const int64_t r = row0 + i;
            x[i] = raw8(gin + r * C + ch);
            kr[i] = raw8(kin + (r * a.H + h) * K + c8 * 8);
            qr[i] = raw8(qin + r * C + ch);
        }
        float kmax = 0.f;  // the largest |k| of the thread's rows
        f32x8 kmc = {};    // and of each of its channels
        const bool ends_block = (sub + 1) % SPB == 0;  // the thread holds its block's last row
#pragma unroll
        for (int i = 0; i < SP_SUB; ++i) {
            const int row = SP_SUB * sub + i;
            const f32x8 kv = __builtin_convertvector(kr[i], f32x8), qv = __builtin_convertvector(qr[i], f32x8);
            run += __builtin_convertvector(x[i], f32x8);
            const bool last = ends_block && i == SP_SUB - 1;
            f32x8 pv, kl, kb, qb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kmax = fmaxf(kmax, fabsf(kv[e]));
                kmc[e] = fmaxf(kmc[e], fabsf(kv[e]));
                pv[e] = a.pscale * (last ? Eb[e] : run[e]);
                kl[e] = kv[e] * __builtin_amdgcn_exp2f(fminf(fmaxf(R[e] - pv[e], EXP2_LO), EXP2_HI));
                const float d = pv[e] - Ab[e];
                spread = spread || fabsf(d) > DIAG_SPREAD;
                kb[e] = kv[e] * __builtin_amdgcn_exp2f(fminf(fmaxf(-d, EXP2_LO), EXP2_HI));
                qb[e] = qv[e] * a.qscale * __builtin_amdgcn_exp2f(fminf(fmaxf(d, EXP2_LO), EXP2_HI));
            }
            // P is not read again by the forward: stored past the caches, which
            // keep the prepared tiles for the fused kernel
            float *pw = a.Pw + ((int64_t)tile * TILE + row) * C + ch;
            __builtin_nontemporal_store(f32x4{pv[0], pv[1], pv[2], pv[3]}, reinterpret_cast<f32x4 *>(pw));
            __builtin_nontemporal_store(f32x4{pv[4], pv[5], pv[6], pv[7]}, reinterpret_cast<f32x4 *>(pw) + 1);
            Vec8<__bf16>::store(kout + row * K, kl);
            Vec8<__bf16>::store(kdout + row * K, kb);
            Vec8<__bf16>::store(qdout + row * K, qb);
        }
        atomicMax(&skmax[hl], __float_as_uint(kmax));  // non-negative floats order as their bits
#pragma unroll
        for (int e = 0; e < 8; ++e) atomicMax(&skc[cv * 8 + e], __float_as_uint(kmc[e]));
    }
    if (spread) atomicOr(&sflag[hl], 1u << rb);
    __syncthreads();
    // [tile, HQ, K] flat over the HQ * K channels of the gate
    if (tid < SP_CV * 8 && (int64_t)y * SP_CV * 8 + tid < C)
        a.kcm[(int64_t)tile * C + (int64_t)y * SP_CV * 8 + tid] = __uint_as_float(skc[tid]);
    if (on && c8 == 0 && sub == 0) {
        uint32_t *rec = a.rec + ((int64_t)tile * HQ + hq) * REC_WORDS;
        rec[REC_GROW] = sgrow[hl] & 1u;
        rec[REC_DIAG] = sflag[hl] | (sgrow[hl] & ~0xffu);
        rec[REC_DMIN] = sdmin[hl];
        rec[REC_KMAX] = skmax[hl];
    }
}

// Block id = tile * (nslice + H) + y; y < nslice: keys of slice y, else the
// values of kv head y - nslice.
template <int K, int V>
__global__ __launch_bounds__(256) void scan_prep_kernel(PrepArgs a, int nslice) {
    const int nh = nslice + (int)a.H;
    const int tile = blockIdx.x / nh, y = blockIdx.x % nh;
    if (tile == 0 && y == 0) {
        const int T = (int)a.T, tps = T / TILE;
        for (int i = threadIdx.x; i < a.nseg; i += blockDim.x) a.seg[i] = SegInfo{i * T, T, i * tps, 0};
    }
    if (y < nslice) {
        scan_key_slice<K>(a, tile, y);
    } else {
        const int T = (int)a.T, tps = T / TILE, s = tile / tps;
        value_tile<__bf16, V>(a, tile, y - nslice, SegInfo{s * T, T, s * tps, 0});
    }
}

template <int K, int V>
hipError_t run_scan_prep(const PrepArgs &a, hipStream_t st) {
    const int nslice = (int)cdiv(a.HQ * K, (int64_t)SP_CV * 8);
    const int64_t tiles = a.nseg * (a.T / TILE);
    hipLaunchKernelGGL((scan_prep_kernel<K, V>), dim3((unsigned)(tiles * (nslice + a.H))), dim3(256), 0, st, a,
                       nslice);
    return hipGetLastError();
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

hipError_t launch_scan_prep(const PrepArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_scan_prep<64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_scan_prep<64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_scan_prep<128, 64>(a, st);
    return run_scan_prep<128, 128>(a, st);
}

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
