// wall_fwd_bf16.hip -- fused causal Wall Attention forward, bf16 inputs, gfx950.
//
// Work decomposition.  A workgroup (8 waves) owns one 256-row query block u
// of one (sequence, query head).  Blocks are dispatched farthest into their
// sequence first, so the hardware dispatcher hands the short blocks to the
// workgroups that finish early (the work of a block is not known in advance:
// see the closed form below).  Wave w owns the 32 query rows 256u + 32w ..
// +31 (one MFMA n-block); waves 0-3 sit in the block's first 128-row tile 2u,
// waves 4-7 in the second, 2u+1.  Workgroup ids are remapped so each XCD
// receives a contiguous range of heads (their key caches then share that
// XCD's L2).
//
// Anchors.  exp2(P_i - P_j) is split as exp2(P_i - R) * exp2(R - P_j) at
// integer per-channel anchors R (the per-tile anchors of the blog's "Fast
// training and inference" section), chosen so that no factor of a term that
// matters leaves the float range, at any gate strength:
//   * keys of the tiles before the wave's own tile are read from the
//     prepared key cache, anchored at each tile's last row.  That row lies
//     between the key and the query, so for a prefix that falls both factors
//     are at most about 1, and a factor that underflows belongs to a term
//     that is itself below 2^-125;
//   * keys of the wave's own tile (the diagonal phase, below) are read at the
//     anchors of 32-row blocks.
//
// Diagonal phase (after the pipeline, per wave over its own tile).  The
// preparation step stores every tile again with each 32-row block anchored at
// its own last row A_b: keys k * exp2(A_b - P) and queries q * scale*log2e *
// exp2(P - A_b).  The block's keys are staged into the tile's key buffer; a
// wave takes its own rows' q~ at its block's anchor, its own 32 x 32 block at
// that anchor, then each earlier block b at A_b (a row between those keys and
// its queries: exact at any gate strength), lowering q~'s exponents by
// A_b - A_{b+1} from block to block; an online softmax continues the
// pipeline's, and O^T += v^T p^T with the tile's values.  While every row of
// the wave's block lies within DIAG_SPREAD = 100 log2 units of A_b, every
// factor of its own pairs stays within 2^+-100 and a lost term is below 2^-26;
// beyond that (flagged by the preparation step) the wave forms its own 32 x 32
// block pair by pair in float32 without any anchor,
// scale * sum_n q_in k_jn exp2(P_in - P_jn), and reads the earlier blocks with
// q~ rebuilt at the row just before its own.  The same prepared q~, lowered
// to the previous tile's anchors, starts the pipeline.
//
// Pipeline (the tiles before the wave's own).  Per wave, keys are walked from
// tile 2u (2u - 1 when the block has a single tile) down to the first tile
// the window reaches, one 32-key sub-block (one MFMA m-tile) per step; a
// tile at or after a wave's own tile is masked whole for that wave:
//
//   q~  the wave's bf16 queries anchored at key tile c, q * scale*log2e *
//       exp2(P_i - Rc).  The prepared block-anchored q~ lowered to the tile
//       before the wave's own, then carried from tile c to tile c-1 by lowering each bf16
//       exponent field by the integer R[c-1] - R[c] (>= 0 while the prefix
//       does not grow) with a saturating packed subtract: exact, and a value
//       that would leave the bf16 range becomes 0 and, the decay only
//       growing further back, stays negligible.  A tile where some channel's
//       prefix grows rebuilds q~ from q and P.  The key-side factor
//       exp2(Rc - P_j) is already folded into k~;
//   S^T = k~ q~^T - m on v_mfma_f32_32x32x16_bf16: the accumulator starts at
//       -m (the running max), so scores come back already relative to it,
//       one query column per lane, all softmax state in-lane;
//   softmax online in the log2 domain, fp32, with a lazy running max: the
//       exps of a sub-block are taken against the current m, and only when
//       a query's sum of them exceeds PSUM_LIM (or the lane has not seen a
//       visible key yet) does a branch of its own raise m to the sub-block's
//       max, move the scores, owe O a rescale and redo the exps;
//   O^T += v^T p^T on the same MFMA, p as bf16.
//
// Channel steps that have died (K = 128).  A channel that forgets fast (the
// blog's fast-forgetting channel group) leaves q~ = 0 in bf16 once a tile
// or two of decay lies between the keys and the wave's queries, and the
// carries only lower exponents further back.  At each tile boundary a wave
// whose queries all have q~ = 0 on the upper half of the channel steps (a
// ballot over its registers) stops issuing those steps' score products and
// carries for the rest of the pass: the products it drops are exactly 0, so
// the result is unchanged bit for bit.  A pass with a tile where some
// channel's prefix grows (q~ is rebuilt there) never drops them.
//
// Keys in closed form.  Far enough back, every product q~ k~ of a query is
// too small to move the score away from -m: the accumulator starts at -m, and
// a sum of products below a quarter of m's float32 unit in the last place
// leaves it at -m exactly, so the score is -m, p = bf16(2^-m), for each such
// key, the value the products would have given.  The kernel bounds the sum by
// K * max|q~| * max|k|: max|q~| of each query exactly at the start of the
// pipeline, then lowered at each tile by the smallest shift of the tile's
// carry record (every channel's exponent falls at least that much), max|k|
// over the pass's key tiles from the preparation step.  With no window, no
// scalar gate and no growing prefix in the pass, each wave votes at every tile
// boundary; once all eight waves have voted so, the remaining tiles need only
// p times the sum of their value rows (the preparation step's per-tile sums)
// in O and p per key in l, and the pipeline ends there.  Under the strong
// decay of fast-forgetting channels this leaves most key tiles of a long
// sequence to the closed form.
//
// Software pipeline.  Step b of tile c runs the softmax of sub-block b, the QK
// products of the next sub-block (b-1, or sub-block 3 of tile c-1) and the PV
// products of the previous one (b+1, or sub-block 0 of tile c+1), as one
// instruction stream whose order is fixed at compile time (TilePlan) and
// pinned with scheduling barriers: every LDS operand read is issued NPF reads
// ahead of its MFMA, and the VALU work of the softmax sits between the
// MFMAs.  Both waves of a SIMD run such streams, so each fills the other's
// gaps on the matrix core and the vector ALU.
//
// Tiles stream into LDS by direct buffer->LDS loads, double-buffered, with
// two workgroup barriers per tile: the values of tile c must be in place
// before step 2 of tile c (barrier V), the keys of tile c-1 before the first
// products of tile c-1 start in step 0 of tile c (barrier K).  Each barrier
// waits for its own earlier load batch only and then issues the next batch
// into the buffer just released; each buffer is an LDS variable of its own
// so the compiler does not wait on the loads either.  A key buffer also
// carries the tile's carry record (from the preparation step) and its keys'
// scalar-gate prefix.
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
#include <limits.h>

#include <array>
#include <type_traits>
#include <utility>

#include "wall_common.h"

namespace wall {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int WQ = 32;          // query rows per wave (one MFMA n-block)
constexpr int BQ = 2 * TILE;    // query rows per block: two anchor tiles
constexpr int NW = BQ / WQ;     // waves per workgroup
constexpr int SB = 32;          // keys per sub-block (one MFMA m-tile)
constexpr int NSB = TILE / SB;  // sub-blocks per tile (pipeline steps per tile)
// a query's sum of the 32 p of one sub-block above this raises m (so every p
// stays at most 2^12 before it is rounded to bf16 and summed in fp32)
constexpr float PSUM_LIM = 4096.0f;


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// Key row (within a 32-row block) that MFMA A-row m reads: bits 2 and 3 swapped.
__device__ __forceinline__ int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Combine a value with the one held by lane ^ 32 (the other half of the wave
// holds the same query's other keys): after v_permlane32_swap each lane holds
// both halves' values, one in each result.
// Keep the computation of x where it is written: the result is marked as
// used there, so the compiler cannot sink it past the branches of later ops
// (which would undo the interleaving the tile plan lays out).
template <class T>
__device__ __forceinline__ void pin(T &x) {
    asm volatile("" : "+v"(x));
}

// Scores are never NaN, so the NaN-propagating maximum serves; unlike fmaxf
// it needs no quieting of its inputs.
__device__ __forceinline__ float max3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that leaves direct-to-LDS loads in flight: the wave's own
// LDS reads and writes complete first, vector memory is not waited for.  The
// scheduling fences keep the surrounding stream on its side of the barrier.
__device__ __forceinline__ void tile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One tile as 1 KB blocks of whole rows (ROWB bytes each), row j stored in
// block j % NBLK at slot j / NBLK; blocks are BLK_PITCH bytes apart.
constexpr int BLK_PITCH = 1040;
template <int NROWS, int ROWB>
struct TileLayout {
    static constexpr int NBLK = NROWS * ROWB / 1024;
    static constexpr int BYTES = NBLK * BLK_PITCH;
    static constexpr int ROW_BYTES = ROWB;
    static __device__ __forceinline__ int byte(int row) { return (row % NBLK) * BLK_PITCH + (row / NBLK) * ROWB; }
};

// A key buffer holds the tile's rescaled keys, then its carry record (1 KB),
// then the scalar-gate prefix G of its 128 keys (0 beyond the sequence).
template <int K, int V>
struct Layouts {
    using KL = TileLayout<TILE, 2 * K>;  // rescaled keys, row = key
    using VL = TileLayout<V, 2 * TILE>;  // values transposed, row = value channel
    static constexpr int REC_OFF = KL::BYTES;
    static constexpr int GK_OFF = REC_OFF + REC_WORDS * 4;
    static constexpr int KBUF = GK_OFF + TILE * 4;
};

template <int K>
using QOp = bf16x8[K / 16];  // [k-step]: 8 channels 16*s8 + 8*hl + e of one query

// q~ at tile c straight from q and P: bf16(q * scale*log2e * exp2(P_i - Rc)).
// LEAN fences the scheduler between channel groups so the loads of one group
// are in flight at a time (for use while the accumulators are live).
template <int K, bool LEAN>
__device__ __forceinline__ void load_qop(const FwdArgs &a, const SegInfo &sg, int hq, int c, int qrow, int hl,
                                QOp<K> &qop) {
    constexpr int KS = K / 16;
    const int64_t HQ = a.HQ;
    const __bf16 *qg = static_cast<const __bf16 *>(a.q);
    const float *Rc = a.anchor + ((int64_t)(sg.tile_base + c) * HQ + hq) * K;
    if (LEAN) asm volatile("" : "+v"(qrow));  // keep the address arithmetic here, not hoisted
    const bool valid = qrow < sg.len;
    const int64_t tok = (int64_t)sg.start + (valid ? qrow : 0);
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
        qop[s8] = __builtin_convertvector(qh, bf16x8);
        if (LEAN) __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------- loads
// Direct buffer->LDS copies.  Each lane fetches BYTES from base + voff (a
// buffer resource of nbytes over base, so fetches past its end read zeros)
// and the wave writes them lane-linearly at LDS address `dst`.  They are
// written as assembly so that the compiler does not track them: it cannot
// tell the LDS buffers of copies in flight apart once control flow merges,
// and would then wait for every copy before any LDS read.  Every read of
// copied data here follows an explicit wait for the copies and a barrier.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int BYTES>
__device__ __forceinline__ void dma(const void *dst, const void *base, uint32_t nbytes, uint32_t voff,
                                    uint32_t soff) {
    static_assert(BYTES == 16 || BYTES == 4, "copy width");
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    // base, stride 0, size in bytes, raw-buffer format word; the operands are
    // wave-uniform, and readfirstlane keeps them in scalar registers even where
    // the compiler holds such a value in a vector register
    auto sgpr = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
    const u32x4 rs = {sgpr((uint32_t)b), sgpr((uint32_t)(b >> 32) & 0xffffu), sgpr(nbytes), 0x00020000u};
    const uint32_t m0 = sgpr((uint32_t)(uintptr_t)(lds_void *)dst);
    soff = sgpr(soff);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
                     : "memory", "m0");
#endif
}

// One tile laid out as L: one wave instruction per 1 KB block, written
// lane-linearly; lane l fetches 16 bytes of the block's row l / (ROW_BYTES/16).
// The blocks are spread over the workgroup's waves.
template <class L>
__device__ __forceinline__ uint32_t tile_lane_offset(int lane) {
    constexpr int CPR = L::ROW_BYTES / 16;  // 16-byte chunks per row
    return (uint32_t)((lane / CPR) * L::NBLK * L::ROW_BYTES + (lane % CPR) * 16);
}
template <class L>
__device__ __forceinline__ void load_tile(char *dst, const void *src, uint32_t lane_off, int w) {
    static_assert(L::NBLK % NW == 0, "blocks split evenly over waves");
#pragma unroll
    for (int i = 0; i < L::NBLK / NW; ++i) {
        const int blk = i * NW + w;
        dma<16>(dst + blk * BLK_PITCH, src, L::NBLK * 1024, lane_off, blk * L::ROW_BYTES);
    }
}
// Wave w's eighth of a tile's 1 KB carry record (8 lanes of 16 bytes).
__device__ __forceinline__ void load_rec(char *dst, const uint32_t *rec, int w, int lane) {
    if (lane < 8) dma<16>(dst + 128 * w, rec, REC_WORDS * 4, (uint32_t)(128 * w + 16 * lane), 0);
}
// Wave w's 16 keys of a tile's G values, gathered 4 bytes per lane from g0 =
// G of the tile's first key; keys at or beyond `nkeys` read 0.  The whole
// offset is in the lane offset, which the bounds check covers.
__device__ __forceinline__ void load_gk(char *dst, const float *g0, int64_t HQ, int nkeys, int w, int lane) {
    const uint32_t nbytes = nkeys > 0 ? (uint32_t)((int64_t)(nkeys - 1) * HQ * 4 + 4) : 0u;
    if (lane < 16) dma<4>(dst + 64 * w, g0, nbytes, (uint32_t)((16 * w + lane) * HQ * 4), 0);
}

// ---------------------------------------------------------------- tile plan
// The instruction stream of one tile, fixed at compile time.  Per step b
// (3, 2, 1, 0): softmax stages SMA (masks, gate), SMD0..7 (exps, packing and
// row sums of two keys each), SME (the last pair, the raise test and its
// rare branch); PV products (index t*VT + vt) and QK products (index s8);
// CARRY of one channel step of q~ to the next tile (after its last use in
// step 1, before BARK in step 0); the barriers BARV (start of step 2) and
// BARK (in step 0, after the carries); RESC (an owed rescale of O) ends each
// step.
enum OpKind : int { O_PV, O_QK, O_CARRY, O_SMA, O_SMD, O_SME, O_BARV, O_BARK, O_RESC };
struct TOp {
    int kind, step, idx;
};
constexpr bool is_read(int kind) { return kind == O_PV || kind == O_QK || kind == O_CARRY; }

template <int K, int V>
struct TilePlan {
    static constexpr int VT = V / 32, KS = K / 16;
    static constexpr int NPV = 2 * VT, NQK = KS, NSMD = 8, NCAR = KS, NC1 = NCAR / 2;
    static constexpr int MAXOPS = NSB * (NPV + NQK + KS + 16) + 4;
    using OpArr = std::array<TOp, MAXOPS>;
    // vector instructions per op (the common path), used to spread them evenly
    // over the step's matrix products
    static constexpr int cost(int kind) {
        return kind == O_SMA ? 2 : kind == O_SMD ? 4 : kind == O_SME ? 8 : kind == O_CARRY ? 12 : 0;
    }

    // One step b: its matrix products in order (three value products first,
    // in step 0 all but two, then BARK; then score and value products
    // alternating), and after each product as many
    // vector ops as keep their running total in proportion.  The softmax ops
    // form a chain (SMA, SMB, SMC, SMD0..7, SME; at most one of the first
    // three per slot, and SMD0 not in SMC's slot); score products wait for
    // SMC.  Carries are one queue over steps 1 and 0: a carry waits for the
    // last score product (in step 1) of its channel step, and all precede
    // BARK; each of the two steps budgets half of them.
    static constexpr int build_step(OpArr &a, int n, int b, int &car) {
        TOp mf[NPV + NQK + 1]{};
        int nm = 0, nmfma = 0;
        {
            // A barrier publishes data the products right after it would read
            // at once: let two products that read older data follow it first.
            int pv = 0, qk = 0;
            if (b == 0) {  // the carries go between these value products, before BARK
                for (; pv < NPV - 2; ++pv) mf[nm++] = TOp{O_PV, b, pv};
                mf[nm++] = TOp{O_BARK, b, 0};
                mf[nm++] = TOp{O_PV, b, pv++};
                mf[nm++] = TOp{O_PV, b, pv++};
            } else if (b == 2) {  // the values of this tile arrive at BARV
                mf[nm++] = TOp{O_QK, b, qk++};
                mf[nm++] = TOp{O_BARV, b, 0};
                mf[nm++] = TOp{O_QK, b, qk++};
                mf[nm++] = TOp{O_QK, b, qk++};
            } else {
                mf[nm++] = TOp{O_PV, b, pv++};
            }
            while (pv < NPV || qk < NQK) {
                if (qk < NQK) mf[nm++] = TOp{O_QK, b, qk++};
                if (pv < NPV) mf[nm++] = TOp{O_PV, b, pv++};
            }
        }
        nmfma = NPV + NQK;
        TOp chain[1 + NSMD]{};
        int nc = 0;
        chain[nc++] = TOp{O_SMA, b, 0};
        for (int k = 0; k < NSMD; ++k) chain[nc++] = TOp{O_SMD, b, k};
        const int c_hi = b <= 1 ? NCAR : 0;  // carries allowed in this step
        int ch_total = 0;
        for (int i = 0; i < nc; ++i) ch_total += cost(chain[i].kind);
        // the carries' budget and the products they are spread over
        const int car_total = b == 1 ? NC1 * cost(O_CARRY) : b == 0 ? (NCAR - car) * cost(O_CARRY) : 0;
        const int car_slots = b == 0 ? NPV - 2 : nmfma;
        int ci = 0, ch_placed = 0, car_placed = 0, done = 0, sma_slot = -1;
        bool qk_done[KS]{};
        for (int e = 0; e < nm; ++e) {
            const TOp m = mf[e];
            if (m.kind == O_BARK) {
                while (car < c_hi) a[n++] = TOp{O_CARRY, b, car++};
                a[n++] = m;
                continue;
            }
            if (m.kind == O_BARV) {
                a[n++] = m;
                continue;
            }
            a[n++] = m;
            ++done;
            if (m.kind == O_QK) qk_done[m.idx] = true;
            if (ci == 0) {  // SMA right after the first product (it reads what the last step's products wrote)
                a[n++] = chain[ci++];
                ch_placed += cost(O_SMA);
                sma_slot = done;
            }
            const int ch_t = ch_total * done / nmfma;
            const int car_t = car_total * (done < car_slots ? done : car_slots) / car_slots;
            for (;;) {
                const bool car_ok = car < c_hi && (b == 0 || qk_done[car]);
                const bool ch_ok = ci < nc && !(ci == 1 && sma_slot == done);
                if (car_ok && car_placed + cost(O_CARRY) / 2 <= car_t) {
                    a[n++] = TOp{O_CARRY, b, car++};
                    car_placed += cost(O_CARRY);
                } else if (ch_ok && ch_placed + cost(chain[ci].kind) / 2 <= ch_t) {
                    ch_placed += cost(chain[ci].kind);
                    a[n++] = chain[ci++];
                } else {
                    break;
                }
            }
        }
        if (b == 0)
            while (car < c_hi) a[n++] = TOp{O_CARRY, b, car++};
        while (ci < nc) a[n++] = chain[ci++];
        // after every product of the step: SME may move m, and with it the
        // scores the step's products just wrote
        a[n++] = TOp{O_SME, b, 0};
        a[n++] = TOp{O_RESC, b, 0};
        return n;
    }
    static constexpr int build(OpArr &a) {
        int n = 0, car = 0;
        for (int b = NSB - 1; b >= 0; --b) n = build_step(a, n, b, car);
        return n;
    }
    static constexpr OpArr make_ops() {
        OpArr a{};
        build(a);
        return a;
    }
    static constexpr int make_n() {
        OpArr a{};
        return build(a);
    }
    static constexpr OpArr OPS = make_ops();
    static constexpr int N = make_n();

    static constexpr int make_nr() {
        int r = 0;
        for (int i = 0; i < N; ++i) r += is_read(OPS[i].kind) ? 1 : 0;
        return r;
    }
    static constexpr int NR = make_nr();  // LDS operand reads per tile
    // Reads kept in flight: the largest of 7..4 that divides NR, so a read has
    // the same ring slot in every tile.
    static constexpr int NPF = (K == 128 && NR % 4 == 0) ? 4 : NR % 7 == 0 ? 7 : NR % 6 == 0 ? 6 : NR % 5 == 0 ? 5 : 4;
    static_assert(NR % NPF == 0, "reads per tile must fill whole rings");

    static constexpr int pos_of(int kind) {
        for (int i = 0; i < N; ++i)
            if (OPS[i].kind == kind) return i;
        return -1;
    }
    static constexpr int POS_BARV = pos_of(O_BARV), POS_BARK = pos_of(O_BARK);

    using ReadArr = std::array<int, MAXOPS>;
    static constexpr ReadArr make_cons() {  // position of the op consuming read r
        ReadArr c{};
        int k = 0;
        for (int i = 0; i < N; ++i)
            if (is_read(OPS[i].kind)) c[k++] = i;
        return c;
    }
    static constexpr ReadArr CONS = make_cons();
    static constexpr int consumer(int r) { return CONS[r % NR] + (r / NR) * N; }  // r >= NR: next tile
    static constexpr TOp read_op(int r) { return OPS[CONS[r % NR]]; }
    static constexpr ReadArr make_read_of() {  // read index consumed by the op at a position, else -1
        ReadArr ro{};
        int k = 0;
        for (int i = 0; i < MAXOPS; ++i) ro[i] = -1;
        for (int i = 0; i < N; ++i)
            if (is_read(OPS[i].kind)) ro[i] = k++;
        return ro;
    }
    static constexpr ReadArr READ_OF = make_read_of();
    // The position after which read r (NPF <= r < NR + NPF) is issued: once
    // its ring slot is free (read r - NPF consumed) and the data it reads is
    // in place (after the barrier that publishes it, for the values and keys
    // that arrive during this tile).
    static constexpr int guard(int r) {
        const TOp o = read_op(r);
        if (r < NR) {
            if (o.kind == O_PV && o.step <= 2) return POS_BARV;  // this tile's values
            if (o.kind == O_QK && o.step == 0) return POS_BARK;  // the next tile's keys
            return -1;
        }
        return o.kind == O_QK ? POS_BARK : -1;  // next tile's first reads: its keys
    }
    static constexpr int issue_pos(int r) {
        const int nat = consumer(r - NPF);
        const int g = guard(r);
        return nat > g ? nat : g;
    }
    static constexpr bool check() {
        for (int r = 0; r < NPF; ++r)
            if (read_op(r).step != NSB - 1) return false;  // the prefetched reads belong to step 3
        for (int r = NPF; r < NR + NPF; ++r)
            if (!(issue_pos(r) < consumer(r) && issue_pos(r) < N)) return false;
        return true;
    }
    static_assert(check(), "every read is issued before its use and within the tile");
};

// ---------------------------------------------------------------- per-wave pipeline
template <int K, int V, bool HAS_G>
struct Wave {
    using LY = Layouts<K, V>;
    using KL = typename LY::KL;
    using VL = typename LY::VL;
    using Plan = TilePlan<K, V>;
    static constexpr int VT = V / 32, KS = K / 16, NPF = Plan::NPF;
    // K = 128: a wave whose queries' q~ is 0 on the upper half of the channel
    // steps skips those steps' score products and carries
    static constexpr bool HAS_HALF = K == 128;

    // per-lane constants
    int kbase, vbase, hl, qrow;
    // accumulators and softmax state for the lane's query column: m is the
    // running max (log2 units) the scores are taken relative to; negm holds -m
    // in all 16 accumulator slots and starts every QK product.  Until a lane
    // has seen a visible key m is 0 and any score raises it (lim < 0).
    f32x16 O[VT];
    f32x16 negm;
    float m, l;
    float alpha;  // rescale O still owes for the current step (1 if none)
    float lim;    // a step's sum of p above this raises m: -1 until the first visible key, then PSUM_LIM
    QOp<K> qop;
    f32x16 S[2];           // S[b & 1]: scores of the sub-block softmaxed in step b
    uint32_t Pw[2][2][4];  // Pw[b & 1][t]: packed bf16 p of that sub-block, keys 16t + 8hl + e
    bf16x8 ring[NPF];      // LDS operand reads in flight
    float ex[2][2];        // exps of the last two key pairs, packed one op later
    bool half;             // q~ is 0 on the upper half of the channel steps (wave-uniform)
    float part[2];         // partial row sums of the current step

    // buffers: keys of this tile and the next (older) one, values of this tile
    // and of the previous (newer) one
    const char *kcur, *knext, *vcur, *vprev;

    // per-tile facts (wave-uniform)
    int key_tile0;   // first key of the current tile (sequence-relative)
    int mask_bits;   // bit B: step B's scores need window masks (all bits: a dead tile)
    bool dead;       // the tile is the wave's own tile or later: every key masked
    const char *recp;  // the tile's carry record, or zeros (no carry) for this wave
    bool carry_on_grow;  // ... by rebuilding it there (some channel's prefix grows)
    int window, len, q0w;

    __device__ static __forceinline__ bf16x8 as_bf16(const uint32_t (&w)[4]) {
        return __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
    }

    // ---- operand address of read r of plan PL (NEXT: a read of the next tile's step 3)
    template <int R>
    __device__ __forceinline__ const bf16x8 *src() const {
        constexpr bool NEXT = R >= Plan::NR;
        constexpr TOp o = Plan::read_op(R);
        if constexpr (o.kind == O_PV) {
            constexpr int vt = o.idx % VT, t = o.idx / VT;
            constexpr int sub = o.step == NSB - 1 ? 0 : o.step + 1;  // the previous sub-block
            constexpr int off = vt * (32 / VL::NBLK) * (2 * TILE) + 32 * (2 * sub + t);
            const char *vb = o.step == NSB - 1 ? (NEXT ? vcur : vprev) : vcur;
            return reinterpret_cast<const bf16x8 *>(vb + vbase + off);
        } else if constexpr (o.kind == O_QK) {
            constexpr int sub = o.step == 0 ? NSB - 1 : o.step - 1;  // the next sub-block
            constexpr int off = sub * (SB / KL::NBLK) * (2 * K) + 32 * o.idx;
            const char *kb = (o.step == 0 || NEXT) ? knext : kcur;
            return reinterpret_cast<const bf16x8 *>(kb + kbase + off);
        } else {
            // carry record words 8*s8 + 4*hl .. +3 of the current tile
            return reinterpret_cast<const bf16x8 *>(recp + 32 * o.idx + 16 * hl);
        }
    }
    template <int R>
    __device__ __forceinline__ void read() {
        ring[R % NPF] = *src<R>();
    }
    template <int... Rs>
    __device__ __forceinline__ void read_first(std::integer_sequence<int, Rs...>) {
        (read<Rs>(), ...);
    }
    // every query of the wave has q~ = 0 (either sign) on the upper half of the
    // channel steps (wave-uniform)
    __device__ __forceinline__ bool upper_dead() const {
        uint32_t acc = 0u;
#pragma unroll
        for (int s8 = KS / 2; s8 < KS; ++s8) {
            const uint4 x = __builtin_bit_cast(uint4, qop[s8]);
            acc |= x.x | x.y | x.z | x.w;
        }
        return __builtin_amdgcn_ballot_w64((acc & 0x7fff7fffu) != 0u) == 0u;
    }

    // ---- softmax stages of step B on S[B & 1]
    template <int B>
    __device__ __forceinline__ void sma() {
        f32x16 &s = S[B & 1];
        if (mask_bits & (1 << B)) {
            // visible keys of this lane's query, as offsets from its first key in
            // the sub-block: at most khi (none on a dead tile), at least klo (window)
            const int kb0 = key_tile0 + SB * B + 8 * hl;
            const int khi = dead ? -1 : min(qrow, len - 1) - kb0;
            if (window > 0) {
                const int klo = qrow - window + 1 - kb0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 16 * (r / 8) + (r % 8);
                    s[r] = (off <= khi && off >= klo) ? s[r] : -__builtin_inff();
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 16 * (r / 8) + (r % 8);
                    s[r] = off <= khi ? s[r] : -__builtin_inff();
                }
            }
        }
        if (HAS_G) {
            const float *gk = reinterpret_cast<const float *>(kcur + LY::GK_OFF) + SB * B + 8 * hl;
            const f32x8 g0 = *reinterpret_cast<const f32x8 *>(gk);
            const f32x8 g1 = *reinterpret_cast<const f32x8 *>(gk + 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s[e] -= g0[e];
                s[8 + e] -= g1[e];
            }
        }
    }
    // SMD KK: the exps of key pair KK.  The pair before it is rounded and
    // packed, and the one before that summed, in the same op, so that no op
    // waits for a result of its own.
    template <int B, int KK>
    __device__ __forceinline__ void smd() {
        const f32x16 &s = S[B & 1];
        if constexpr (KK > 0) pack<B, KK - 1>();
        if constexpr (KK > 1) rowsum<B, KK - 2>();
        ex[KK & 1][0] = fast_exp2(s[2 * KK]);
        ex[KK & 1][1] = fast_exp2(s[2 * KK + 1]);
        pin(ex[KK & 1][0]);
        pin(ex[KK & 1][1]);
    }
    template <int B, int KK>
    __device__ __forceinline__ void pack() {
        const bf16x2 p = {(__bf16)ex[KK & 1][0], (__bf16)ex[KK & 1][1]};
        Pw[B & 1][KK / 4][KK % 4] = __builtin_bit_cast(uint32_t, p);
        pin(Pw[B & 1][KK / 4][KK % 4]);
    }
    // row sum of the rounded p, two independent chains
    template <int B, int KK>
    __device__ __forceinline__ void rowsum() {
        const bf16x2 p = __builtin_bit_cast(bf16x2, Pw[B & 1][KK / 4][KK % 4]);
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        part[KK & 1] = __builtin_amdgcn_fdot2_f32_bf16(p, one, KK < 2 ? 0.f : part[KK & 1], false);
        pin(part[KK & 1]);
    }
    template <int B, int... KKs>
    __device__ __forceinline__ void redo(std::integer_sequence<int, KKs...>) {
        (smd<B, KKs>(), ...);
        pack<B, 7>();
        rowsum<B, 6>();
        rowsum<B, 7>();
    }
    // The step's last pair, then the raise test on the lane's sum of p.  The
    // branch (first visible keys, or p grown past PSUM_LIM) raises m to the
    // step's max, moves this step's scores and the next sub-block's (already
    // started from the old -m), owes O the factor, and redoes the exps.
    template <int B>
    __device__ __forceinline__ void sme() {
        pack<B, 7>();
        rowsum<B, 6>();
        rowsum<B, 7>();
        float ps = part[0] + part[1];
        const float pq = pair_sum(ps);  // the query's sum over the sub-block's 32 keys
        if (__any(pq > lim)) {
            f32x16 &s = S[B & 1];
            const float a = max3(max3(s[0], s[1], s[2]), max3(s[3], s[4], s[5]), max3(s[6], s[7], s[8]));
            const float b = max3(max3(s[9], s[10], s[11]), max3(s[12], s[13], s[14]), s[15]);
            const float mt = pair_max(__builtin_elementwise_maximum(a, b));
            const bool raise = lim < 0.f ? mt > -FLT_MAX : pq > lim;
            if (__any(raise)) {
                const float delta = raise ? mt : 0.f;
                const float al = fast_exp2(-delta);
                m += delta;
                l *= al;
                alpha *= al;
                lim = raise ? PSUM_LIM : lim;
                negm -= delta;
                s -= delta;
                S[(B + 1) & 1] -= delta;
                redo<B>(std::make_integer_sequence<int, Plan::NSMD>{});
                ps = part[0] + part[1];
            }
        }
        l += ps;
        pin(l);
    }
    __device__ __forceinline__ void resc() {
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) O[vt] *= alpha;
            alpha = 1.f;
        }
    }
};

// ---------------------------------------------------------------- the kernel
template <int K, int V, bool HAS_G>
struct Kernel {
    using W = Wave<K, V, HAS_G>;
    using LY = Layouts<K, V>;
    using KL = typename LY::KL;
    using VL = typename LY::VL;
    using Plan = TilePlan<K, V>;
    static constexpr int VT = V / 32, KS = K / 16, NPF = Plan::NPF, NR = Plan::NR, N = Plan::N;
    // buffer loads per wave per tile: the tile's blocks, then a slice of the
    // carry record (and of G) for the keys
    static constexpr int KLOADS = KL::NBLK / NW + 1 + (HAS_G ? 1 : 0), VLOADS = VL::NBLK / NW;

    const FwdArgs &a;
    W wv;
    char *k0, *k1, *v0, *v1;
    SegInfo sg;
    int hq, h, w, lane, qt_w, c_lo;
    uint32_t klane, vlane;
    bool wave_on;
    const char *zrec = nullptr;  // zeros in LDS: the shifts of no carry

    // per-tile facts of tile c whose keys (and carry record) are in kcur
    __device__ __forceinline__ void tile_facts(int c, const char *kcur) {
        wv.key_tile0 = TILE * c;
        // the wave's own tile (its keys were read in the diagonal phase) masks
        // every step; a window masks the steps whose first key is at or below lim
        const bool dead = c >= qt_w;
        int mb = dead ? (1 << NSB) - 1 : 0;
        if (!dead && wv.window > 0) {
            const int lim = wv.q0w + WQ - 1 - wv.window - TILE * c;
            if (lim >= 0) mb |= (2 << min(lim / SB, NSB - 1)) - 1;
        }
        wv.mask_bits = mb;
        wv.dead = dead;
        const bool grow = reinterpret_cast<const uint32_t *>(kcur + LY::REC_OFF)[REC_GROW] != 0u;
        // q~ sits at tile c's anchors only for a tile before the wave's own
        const bool go_on = wave_on && c < qt_w && c - 1 >= c_lo;
        // Without a carry the shifts are read from zeros.  A tile where some
        // channel's prefix grows rebuilds q~ at BARK, after all carries.
        wv.recp = go_on ? kcur + LY::REC_OFF : zrec;
        wv.carry_on_grow = go_on && grow;
    }

    __device__ __forceinline__ const __bf16 *kt_tile(int c) const {
        return static_cast<const __bf16 *>(a.kt) + ((int64_t)(sg.tile_base + c) * a.HQ + hq) * TILE * K;
    }
    __device__ __forceinline__ const __bf16 *vt_tile(int c) const {
        return static_cast<const __bf16 *>(a.vt) + ((int64_t)(sg.tile_base + c) * a.H + h) * V * TILE;
    }
    // keys of tile c (its carry record and G first) into key buffer kd
    __device__ __forceinline__ void issue_k(char *kd, int c) const {
        load_tile<KL>(kd, kt_tile(c), klane, w);
        load_rec(kd + LY::REC_OFF, a.rec + ((int64_t)(sg.tile_base + c) * a.HQ + hq) * REC_WORDS, w, lane);
        if (HAS_G)
            load_gk(kd + LY::GK_OFF, a.G + ((int64_t)sg.start + (int64_t)c * TILE) * a.HQ + hq, a.HQ,
                    sg.len - c * TILE, w, lane);
    }
    __device__ __forceinline__ void issue_v(char *vd, int c) const { load_tile<VL>(vd, vt_tile(c), vlane, w); }

    // ---- one op of the plan at position P for tile c held in buffers of parity PB
    // DEAD: a tile wholly after the wave's queries.  Its p are all 0, so only
    // the barriers and the score products of the next tile (step 0) remain.
    template <int PB, int P, bool DEAD>
    __device__ __forceinline__ void op(int c) {
        constexpr TOp o = Plan::OPS[P];
        constexpr int B = o.step;
        if constexpr (DEAD && o.kind != O_BARV && o.kind != O_BARK && !(o.kind == O_QK && o.step == 0)) {
            return;
        } else if constexpr (o.kind == O_PV) {
            constexpr int vt = o.idx % VT, t = o.idx / VT;
            const bf16x8 x = wv.ring[Plan::READ_OF[P] % NPF];
            wv.O[vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, W::as_bf16(wv.Pw[(B + 1) & 1][t]), wv.O[vt], 0,
                                                               0, 0);
        } else if constexpr (o.kind == O_QK) {
            const bf16x8 x = wv.ring[Plan::READ_OF[P] % NPF];
            f32x16 &sn = wv.S[(B + 1) & 1];
            if (W::HAS_HALF && o.idx >= KS / 2 && wv.half) return;
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, wv.qop[o.idx], o.idx == 0 ? wv.negm : sn, 0, 0, 0);
        } else if constexpr (o.kind == O_CARRY) {
            if (W::HAS_HALF && o.idx >= KS / 2 && wv.half) return;
            const bf16x8 x = wv.ring[Plan::READ_OF[P] % NPF];
            // lower each bf16 exponent field by the shift, saturating on the
            // magnitude (the four words interleaved: no op waits on the one before)
            const uint4 d = __builtin_bit_cast(uint4, x);
            const uint32_t dv[4] = {d.x, d.y, d.z, d.w};
            const uint4 x4 = __builtin_bit_cast(uint4, wv.qop[o.idx]);
            const uint32_t xv[4] = {x4.x, x4.y, x4.z, x4.w};
            u16x2 mag[4], r[4];
            uint32_t out[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) mag[e] = __builtin_bit_cast(u16x2, xv[e] & 0x7fff7fffu);
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = __builtin_elementwise_sub_sat(mag[e], __builtin_bit_cast(u16x2, dv[e]));
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (xv[e] & 0x80008000u) | __builtin_bit_cast(uint32_t, r[e]);
            wv.qop[o.idx] = __builtin_bit_cast(bf16x8, uint4{out[0], out[1], out[2], out[3]});
            pin(wv.qop[o.idx]);
        } else if constexpr (o.kind == O_SMA) {
            wv.template sma<B>();

        } else if constexpr (o.kind == O_SMD) {
            wv.template smd<B, o.idx>();
        } else if constexpr (o.kind == O_SME) {
            wv.template sme<B>();
        } else if constexpr (o.kind == O_RESC) {
            wv.resc();
        } else if constexpr (o.kind == O_BARV) {
            // the values of tile c are in place once the key batch issued after them
            // is the only one left in flight
            // (every tile issues the same loads, past the last one those of tile
            // c_lo again into a buffer no longer read, so that the counts are fixed)
            wait_vm<KLOADS>();
            tile_barrier();
            issue_v(PB ? v0 : v1, max(c - 1, c_lo));
        } else if constexpr (o.kind == O_BARK) {
            wait_vm<VLOADS>();
            tile_barrier();
            if (wv.carry_on_grow) {
                // some channel's prefix grows into tile c-1: rebuild q~ there instead
                // (before the key loads are issued, so that waiting for these
                // global loads never waits for them)
                load_qop<K, true>(a, sg, hq, c - 1, wv.qrow, wv.hl, wv.qop);
            }
            issue_k(PB ? k1 : k0, max(c - 2, c_lo));
        }
    }
    // ---- the diagonal phase: keys of the wave's own tile up to its last query
    //
    // The preparation step stored every row of the tile again with each 32-row
    // block anchored at its own last row: the keys (staged into the tile's key
    // buffer) and the queries (times scale*log2e).  A wave reads its own rows'
    // q~ at its block's anchor, its own block's keys at the same anchor, and
    // each earlier block's keys at that block's anchor, between them and the
    // wave's queries, carrying q~ from block to block.
    __device__ __forceinline__ const __bf16 *kd_tile(int c) const {
        return static_cast<const __bf16 *>(a.kd) + ((int64_t)(sg.tile_base + c) * a.HQ + hq) * TILE * K;
    }
    __device__ __forceinline__ const uint32_t *drec_tile(int c) const {
        return a.drec + ((int64_t)(sg.tile_base + c) * a.HQ + hq) * DREC_N * (K / 2);
    }
    __device__ __forceinline__ uint32_t diag_flags(int c) const {
        return a.rec[((int64_t)(sg.tile_base + c) * a.HQ + hq) * REC_WORDS + REC_DIAG];
    }
    // the prepared q~ of the lane's query (tile c), at its block's anchor
    __device__ __forceinline__ void load_qd(int c, QOp<K> &qd) const {
        const __bf16 *src = static_cast<const __bf16 *>(a.qd) +
                            (((int64_t)(sg.tile_base + c) * a.HQ + hq) * TILE + (wv.qrow - TILE * c)) * K;
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8) qd[s8] = *reinterpret_cast<const bf16x8 *>(src + 16 * s8 + 8 * wv.hl);
    }
    // q~ of the lane's query at the anchors floor(P[Pa row]) from q and P (0 for
    // a row past the sequence).  A rare path: one channel step in flight at a
    // time, so that it adds no register pressure.
    __device__ void diag_q(const float *Pa, QOp<K> &qo) const {
        const bool qv = wv.qrow < sg.len;
        const int64_t tok = (int64_t)sg.start + (qv ? wv.qrow : 0);
        const __bf16 *qg = static_cast<const __bf16 *>(a.q) + (tok * a.HQ + hq) * K;
        const float *pg = a.P + (tok * a.HQ + hq) * K;
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8) {
            const int ch0 = 16 * s8 + 8 * wv.hl;
            const f32x8 qv8 = __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(qg + ch0), f32x8);
            const f32x8 pv8 = *reinterpret_cast<const f32x8 *>(pg + ch0);
            const f32x8 rv = *reinterpret_cast<const f32x8 *>(Pa + ch0);
            f32x8 qh;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qh[e] = qv ? qv8[e] * a.qscale * exp2f(fminf(fmaxf(pv8[e] - floorf(rv[e]), EXP2_LO), EXP2_HI)) : 0.f;
            qo[s8] = __builtin_convertvector(qh, bf16x8);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // q~ lowered by a carry record (the u16 exponent decrements of the lane's
    // channels, as the pipeline's tile records): exact, or 0 below the bf16 range.
    __device__ __forceinline__ void carry_rec(QOp<K> &qd, const uint32_t *rec) const {
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8) {
            const uint4 d = *reinterpret_cast<const uint4 *>(rec + 8 * s8 + 4 * wv.hl);
            const uint32_t dv[4] = {d.x, d.y, d.z, d.w};
            const uint4 x4 = __builtin_bit_cast(uint4, qd[s8]);
            const uint32_t xv[4] = {x4.x, x4.y, x4.z, x4.w};
            uint32_t out[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u16x2 mag = __builtin_bit_cast(u16x2, xv[e] & 0x7fff7fffu);
                const u16x2 rr = __builtin_elementwise_sub_sat(mag, __builtin_bit_cast(u16x2, dv[e]));
                out[e] = (xv[e] & 0x80008000u) | __builtin_bit_cast(uint32_t, rr);
            }
            qd[s8] = __builtin_bit_cast(bf16x8, uint4{out[0], out[1], out[2], out[3]});
        }
    }
    // S^T of the keys of 32-row block b of the tile in kd against q~ (LDS
    // reads in the pipeline's operand order).
    __device__ __forceinline__ f32x16 diag_scores(const char *kd, int b, const QOp<K> &qd) const {
        const char *kb = kd + wv.kbase + b * (SB / KL::NBLK) * (2 * K);
        f32x16 S = {};
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8)
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kb + 32 * s8), qd[s8], S, 0,
                                                        0, 0);
        return S;
    }
    // The 32 x 32 block of the wave's own rows (keys from kb = the wave's first
    // row), pair by pair in float32: scale*log2e * sum_n q_in k_jn exp2(P_in - P_jn).
    // One key at a time, so that few registers are live (a rare path).
    __device__ f32x16 exact_scores(int kb) const {
        const int qrow = wv.qrow;
        const bool qv = qrow < sg.len;
        const int64_t qtok = (int64_t)sg.start + (qv ? qrow : 0);
        const __bf16 *qg = static_cast<const __bf16 *>(a.q) + (qtok * a.HQ + hq) * K;
        const float *pq = a.P + (qtok * a.HQ + hq) * K;
        const int kb0 = kb + 8 * wv.hl;
        f32x16 S = {};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = kb0 + 16 * (r / 8) + (r % 8);
            float acc = 0.f;
            if (qv && j <= qrow) {
                const int64_t jt = (int64_t)sg.start + j;
                const __bf16 *kg = static_cast<const __bf16 *>(a.k) + (jt * a.H + h) * K;
                const float *pk = a.P + (jt * a.HQ + hq) * K;
#pragma unroll 1
                for (int c8 = 0; c8 < K / 8; ++c8) {
                    const f32x8 qq = __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(qg + 8 * c8), f32x8);
                    const f32x8 pi = *reinterpret_cast<const f32x8 *>(pq + 8 * c8);
                    const f32x8 kk = __builtin_convertvector(*reinterpret_cast<const bf16x8 *>(kg + 8 * c8), f32x8);
                    const f32x8 pj = *reinterpret_cast<const f32x8 *>(pk + 8 * c8);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc = fmaf(qq[e] * kk[e], exp2f(fminf(fmaxf(pi[e] - pj[e], EXP2_LO), EXP2_HI)), acc);
                }
            }
            S[r] = acc * a.qscale;
        }
        return S;
    }
    // Masks, the online softmax of the 32 keys of block b (scores not relative
    // to m) and O^T += v^T p^T with the values of the tile in vd; G of the
    // tile's keys in kd.
    __device__ __forceinline__ void diag_block(f32x16 S, int kt0, int b, const char *kd, const char *vd) {
        const int qrow = wv.qrow, len = sg.len;
        const bool qv = qrow < len;
        const int kb0 = kt0 + SB * b + 8 * wv.hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = kb0 + 16 * (r / 8) + (r % 8);
            bool vis = qv && j <= qrow;
            if (a.window > 0) vis = vis && qrow - j < a.window;
            float x = S[r];
            if (HAS_G) x -= reinterpret_cast<const float *>(kd + LY::GK_OFF)[j - kt0];
            S[r] = vis ? x : -__builtin_inff();
        }
        const float m1 = max3(max3(S[0], S[1], S[2]), max3(S[3], S[4], S[5]), max3(S[6], S[7], S[8]));
        const float m2 = max3(max3(S[9], S[10], S[11]), max3(S[12], S[13], S[14]), S[15]);
        const float mn = fmaxf(wv.m, pair_max(__builtin_elementwise_maximum(m1, m2)));
        const float al = fast_exp2(wv.m - mn);
        uint32_t pw[2][4];
        float ps = 0.f;
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pp = {(__bf16)fast_exp2(S[8 * t + 2 * e] - mn), (__bf16)fast_exp2(S[8 * t + 2 * e + 1] - mn)};
                pw[t][e] = __builtin_bit_cast(uint32_t, pp);
                ps = __builtin_amdgcn_fdot2_f32_bf16(pp, one, ps, false);
            }
        wv.l = wv.l * al + ps;
        wv.m = mn;
        const char *vb = vd + wv.vbase;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            wv.O[vt] *= al;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 x =
                    *reinterpret_cast<const bf16x8 *>(vb + vt * (32 / VL::NBLK) * (2 * TILE) + 32 * (2 * b + t));
                wv.O[vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, W::as_bf16(pw[t]), wv.O[vt], 0, 0, 0);
            }
        }
    }
    // The walk of the wave (queries q0w.., tile qt, the tile's block-anchored
    // keys in kd and its values in vd, flags the tile's REC_DIAG word, qd the
    // wave's prepared q~) over its own tile, continuing the online softmax of
    // the pipeline (a lane that has seen no visible key yet restarts its max).
    __device__ void diag_walk(int qt, int q0w, uint32_t flags, const char *kd, const char *vd, QOp<K> &qd) {
        constexpr int NB = TILE / DBLK;
        const int wq = (q0w - TILE * qt) / WQ;  // the wave's 32-row block within its tile
        const int kt0 = TILE * qt;
        const bool flagged = (flags >> wq) & 1u;
        const uint32_t *drec = drec_tile(qt);
        // the lowest 32-key block any query of the wave sees
        int b_lo = 0;
        if (a.window > 0) {
            const int kmin = q0w - a.window + 1;
            if (kmin > kt0) b_lo = (kmin - kt0) / SB;
        }
        if (wv.lim < 0.f) wv.m = -FLT_MAX;
        if (!flagged) {
            diag_block(diag_scores(kd, wq, qd), kt0, wq, kd, vd);
        } else {
            // some row of the wave lies more than DIAG_SPREAD from its anchor: its
            // own block pair by pair, and q~ for the earlier blocks at the anchor
            // of the row just before the wave (block wq - 1's)
            diag_block(exact_scores(q0w), kt0, wq, kd, vd);
            if (wq > b_lo) diag_q(a.P + ((int64_t)(sg.start + q0w - 1) * a.HQ + hq) * K, qd);
        }
        // block b < wq is read with q~ at block b's anchor (its last row, between
        // its keys and the wave's queries); `cur` is the block whose anchor q~ is at
        int cur = flagged ? wq - 1 : wq;
        for (int b = wq - 1; b >= b_lo; --b) {
            if (b != cur) {
                if ((flags >> (8 + NB + b)) & 1u)
                    diag_q(a.P + ((int64_t)(sg.start + kt0 + SB * b + SB - 1) * a.HQ + hq) * K, qd);
                else
                    carry_rec(qd, drec + (NB + b) * (K / 2));
                cur = b;
            }
            diag_block(diag_scores(kd, b, qd), kt0, b, kd, vd);
        }
    }

    // reads issued after the op at position P
    template <int P, int R>
    __device__ __forceinline__ void maybe_read() {
        if constexpr (Plan::issue_pos(R) == P) wv.template read<R>();
    }
    template <int P, int... Rs>
    __device__ __forceinline__ void reads_after(std::integer_sequence<int, Rs...>) {
        (maybe_read<P, Rs + NPF>(), ...);
    }
    template <int PB, int P, bool DEAD>
    __device__ __forceinline__ void step(int c) {
        __builtin_amdgcn_sched_barrier(0);
        op<PB, P, DEAD>(c);
        reads_after<P>(std::make_integer_sequence<int, NR>{});
    }
    template <int PB, bool DEAD, int... Ps>
    __device__ __forceinline__ void run_tile_ops(int c, std::integer_sequence<int, Ps...>) {
        (step<PB, Ps, DEAD>(c), ...);
        __builtin_amdgcn_sched_barrier(0);
    }
    template <int PB>
    __device__ __forceinline__ void run_tile(int c) {
        run_tile_ops<PB, false>(c, std::make_integer_sequence<int, N>{});
    }
};

template <int K, int V, bool HAS_G>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    using KR = Kernel<K, V, HAS_G>;
    using W = Wave<K, V, HAS_G>;
    using LY = Layouts<K, V>;
    using KL = typename LY::KL;
    using VL = typename LY::VL;
    using Plan = TilePlan<K, V>;
    constexpr int VT = V / 32, KS = K / 16, NPF = Plan::NPF;
    // Each tile buffer is an LDS variable of its own: the compiler then knows
    // that reading one buffer does not depend on the direct loads still
    // filling another, and does not wait for them.
    __shared__ __attribute__((aligned(16))) char k0[LY::KBUF];
    __shared__ __attribute__((aligned(16))) char k1[LY::KBUF];
    __shared__ __attribute__((aligned(16))) char v0[VL::BYTES];
    __shared__ __attribute__((aligned(16))) char v1[VL::BYTES];
    __shared__ __attribute__((aligned(16))) char zrec[32 * KS];
    // the waves' votes of the last two tiles (all queries' q~ zero), and the
    // closed form's partial value sums
    constexpr int NPART = NW * 64 / V;
    __shared__ __attribute__((aligned(16))) uint32_t zvote[2][NW];
    __shared__ __attribute__((aligned(16))) uint32_t skm[K];  // per channel the largest |k| of the pass's tiles
    __shared__ __attribute__((aligned(16))) float zred[NPART][V];

    // One 256-row query block per workgroup.  The blocks farthest into their
    // sequence (the most key tiles) go first, so that workgroups that finish
    // early take the short ones.  Workgroups are dispatched round robin over
    // the 8 XCDs: XCD x takes a contiguous eighth of the (query head,
    // sequence) pairs, whose keys then share its L2.
    const int nblocks_max = (a.max_tiles + 1) / 2;  // 256-row blocks of the longest sequence
    const int nhs = a.nseg * a.HQ;
    const int bid = blockIdx.x;
    int rank, hs;
    if (nhs % 8 == 0) {
        const int per = nhs / 8, j = bid / 8;
        rank = j / per;
        hs = (bid % 8) * per + j % per;
    } else {
        rank = bid / nhs;
        hs = bid % nhs;
    }
    const int hq = hs / a.nseg, s = hs % a.nseg;
    const SegInfo sg = a.seg[s];
    const int ntiles = (sg.len + TILE - 1) / TILE;
    const int nblk = (sg.len + BQ - 1) / BQ;
    const int u = nblocks_max - 1 - rank;
    if (u >= nblk) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers and branches
    const int col = lane & 31, hl = lane >> 5;
    const int64_t HQ = a.HQ;

    // Values are multiplied by p = 0 before their first use in a block: give the
    // second value buffer finite contents once.
    for (int i = tid; i < VL::BYTES / 16; i += NW * 64) reinterpret_cast<uint4 *>(v1)[i] = uint4{0, 0, 0, 0};
    if (tid < 2 * KS) reinterpret_cast<uint4 *>(zrec)[tid] = uint4{0, 0, 0, 0};
    if (tid < K) skm[tid] = 0u;

    KR kr{a, {}, k0, k1, v0, v1, sg, hq, hq / (a.HQ / a.H), w, lane, 0, 0,
          tile_lane_offset<KL>(lane), tile_lane_offset<VL>(lane), false};
    W &wv = kr.wv;
    kr.zrec = zrec;
    wv.kbase = KL::byte(key_perm(col)) + 16 * hl;
    wv.vbase = VL::byte(col) + 16 * hl;
    wv.hl = hl;

    {
        const int qt_w = 2 * u + w / (NW / 2);
        const int q0w = BQ * u + WQ * w;
        const bool wave_on = q0w < sg.len;
        const int qrow = q0w + col;
        // the pipeline's tiles: from the block's first tile (2u; its keys are the
        // second tile's earlier keys) or, when the block has a single tile, the
        // one before it, down to the first tile the window reaches
        const int c_hi = 2 * u + 1 < ntiles ? 2 * u : 2 * u - 1;
        int c_lo = 0;
        if (a.window > 0) {
            const int kmin = BQ * u - a.window + 1;
            c_lo = kmin > 0 ? kmin / TILE : 0;
        }
        const bool run_pipe = c_hi >= c_lo;  // uniform over the workgroup
        int zc = c_lo - 1;  // last tile of the closed form (none: c_lo - 1)
        kr.qt_w = qt_w;
        kr.c_lo = c_lo;
        wv.qrow = qrow;
        wv.window = a.window;
        wv.len = sg.len;
        wv.q0w = q0w;

        float g_i = 0.f;
        if (HAS_G && wave_on && qrow < sg.len) g_i = a.G[((int64_t)sg.start + qrow) * HQ + hq];

        // ---- the pipeline's prologue: q~ at the anchors of the tile before the
        // wave's own; tile c_hi into buffers 0, the keys of tile c_hi - 1 into key
        // buffer 1
        __syncthreads();  // the previous block's last reads of every buffer are done
        if (run_pipe) kr.issue_k(k0, c_hi);
        if (wave_on && qt_w > 0 && run_pipe) {
            // the prepared q~ moved from the wave's block anchor to the previous
            // tile's (an exact exponent decrement); from q and P when the block
            // needs its pair-by-pair path or some channel's prefix grows
            const int wq = (q0w - TILE * qt_w) / WQ;
            const uint32_t fl = kr.diag_flags(qt_w);
            if (((fl >> wq) | (fl >> (8 + wq))) & 1u) {
                load_qop<K, false>(a, sg, hq, qt_w - 1, qrow, hl, wv.qop);
            } else {
                kr.load_qd(qt_w, wv.qop);
                kr.carry_rec(wv.qop, kr.drec_tile(qt_w) + wq * (K / 2));
            }
        } else {
#pragma unroll
            for (int s8 = 0; s8 < KS; ++s8) wv.qop[s8] = bf16x8{};
        }
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) wv.O[vt] = f32x16{};
        wv.negm = f32x16{};
        wv.m = 0.f;
        wv.half = false;
        wv.l = 0.f;
        wv.alpha = 1.f;
        wv.lim = wave_on ? -1.f : __builtin_inff();  // a wave with no rows never raises
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) wv.Pw[0][t][e] = 0u;
        // the pass's key tiles: whether some channel's prefix grows over one
        // of them (uniform over the workgroup), and per channel the largest |k|
        // of their keys (in LDS after the barrier below)
        bool grow = false;
        for (int c0 = c_lo; run_pipe && c0 <= c_hi; c0 += 64) {
            const int ct = c0 + lane;
            if (ct <= c_hi) grow = grow || a.rec[((int64_t)(sg.tile_base + ct) * HQ + hq) * REC_WORDS + REC_GROW] != 0u;
        }
        grow = __builtin_amdgcn_ballot_w64(grow) != 0u;
        if (!HAS_G && a.window <= 0 && run_pipe) {
            constexpr int TPC = NW * 64 / K;  // threads per channel
            float km = 0.f;
            for (int ct = c_lo + tid / K; ct <= c_hi; ct += TPC)
                km = fmaxf(km, a.kcm[((int64_t)(sg.tile_base + ct) * HQ + hq) * K + tid % K]);
            atomicMax(&skm[tid % K], __float_as_uint(km));  // non-negative floats order as their bits
        }
        // The keys of tile c_hi, q~ and the records are in; the values of tile
        // c_hi and the keys of tile c_hi - 1 stay in flight into the pipeline,
        // whose first barriers wait for them.
        __builtin_amdgcn_s_waitcnt(0);
        if (run_pipe) {
            kr.issue_v(v0, c_hi);
            kr.issue_k(k1, max(c_hi - 1, c_lo));
        }
        tile_barrier();

        if (run_pipe) {
            // the scores of the first sub-block (3 of tile c_hi), S[1]
            {
                const char *kb = k0 + wv.kbase + (NSB - 1) * (SB / KL::NBLK) * (2 * K);
#pragma unroll
                for (int s8 = 0; s8 < KS; ++s8) {
                    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(kb + 32 * s8);
                    wv.S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, wv.qop[s8], s8 ? wv.S[1] : wv.negm, 0, 0, 0);
                }
            }

            kr.wave_on = wave_on;
            // prefetch the first reads of tile c_hi (parity 0)
            wv.kcur = k0;
            wv.knext = k1;
            wv.vcur = v0;
            wv.vprev = v1;
            wv.read_first(std::make_integer_sequence<int, NPF>{});

            // A wave whose queries' q~ is 0 on the upper half of the channel
            // steps at a tile's anchors stays so at every earlier tile's (the
            // carries only lower exponents), unless some tile's prefix grows
            // and q~ is rebuilt: without such a tile in the pass, the wave runs
            // the half plan from the first tile where it finds that half dead.
            const bool half_ok = W::HAS_HALF && (!grow || !wave_on);
            // Keys whose scores come out as exactly -m (see the header): without a
            // window or a scalar gate, and with no tile of the pass where the prefix
            // grows, every wave votes at each tile whether every product of its
            // queries with every key left is too small to move -m in float32, and
            // no lane would raise its max on such keys.  qb bounds the sum over the
            // channels of the lane's query's |q~| at the current tile's anchors
            // times the channel's largest |k| over the pass (every |k~| is at most
            // |k| for a prefix that falls): exact q~ at the start, then lowered by
            // the smallest shift of each carry.
            // Once all eight waves have voted so at tile c + 1, the tiles c .. c_lo
            // are summed in closed form and the pipeline ends.
            const bool zero_ok = !HAS_G && a.window <= 0 && !grow;
            float qb = 0.f;
            if (zero_ok) {
                // the lane's channels 16 s8 + 8 hl + e, then the other half's
                float qs = 0.f;
#pragma unroll
                for (int s8 = 0; s8 < KS; ++s8) {
                    const f32x4 m0 = *reinterpret_cast<const f32x4 *>(&skm[16 * s8 + 8 * hl]);
                    const f32x4 m1 = *reinterpret_cast<const f32x4 *>(&skm[16 * s8 + 8 * hl + 4]);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        qs = fmaf(fabsf((float)wv.qop[s8][e]), e < 4 ? m0[e] : m1[e - 4], qs);
                }
                qb = pair_sum(qs);
            }
            auto zero_vote = [&](int c, const char *kc) {
                const float p0 = (float)(__bf16)fast_exp2(-wv.m);
                // a quarter of m's float32 unit in the last place
                const float thr = __uint_as_float(__float_as_uint(wv.m) & 0x7f800000u) * 0x1p-25f;
                const bool ok = wv.m >= 0.f && wv.lim >= 0.f && 32.f * p0 <= wv.lim && qb <= thr;
                const bool dead = !wave_on || __builtin_amdgcn_ballot_w64(!ok) == 0u;
                zvote[c & 1][w] = dead ? 1u : 0u;  // every lane stores the same word
                // q~ after this tile's carries (a wave carries on the tiles before its own, down to c_lo + 1)
                if (wave_on && c < qt_w && c - 1 >= c_lo)
                    qb = __builtin_amdgcn_ldexpf(qb, -(int)reinterpret_cast<const uint32_t *>(kc + LY::REC_OFF)[REC_DMIN]);
            };
            auto zero_all = [&](int c) {  // every wave voted at tile c + 1
                const uint4 x = reinterpret_cast<const uint4 *>(zvote[(c + 1) & 1])[0];
                const uint4 y = reinterpret_cast<const uint4 *>(zvote[(c + 1) & 1])[1];
                return __builtin_amdgcn_readfirstlane(x.x & x.y & x.z & x.w & y.x & y.y & y.z & y.w) != 0u;
            };
            int c = c_hi;
            for (;;) {
                wv.kcur = k0; wv.knext = k1; wv.vcur = v0; wv.vprev = v1;
                if (zero_ok) {
                    if (c < c_hi && zero_all(c)) { zc = c; break; }
                    zero_vote(c, k0);
                }
                kr.tile_facts(c, k0);
                if (W::HAS_HALF && half_ok && !wv.half) wv.half = wv.upper_dead();
                kr.template run_tile<0>(c);
                if (--c < c_lo) break;
                wv.kcur = k1; wv.knext = k0; wv.vcur = v1; wv.vprev = v0;
                if (zero_ok) {
                    if (zero_all(c)) { zc = c; break; }
                    zero_vote(c, k1);
                }
                kr.tile_facts(c, k1);
                if (W::HAS_HALF && half_ok && !wv.half) wv.half = wv.upper_dead();
                kr.template run_tile<1>(c);
                if (--c < c_lo) break;
            }
            // the loads issued past the last tile land before the buffers are reused
            wait_vm<0>();
            // the last sub-block's PV products (sub-block 0 of tile zc + 1, p in
            // Pw[0]): values in the buffer of that tile's parity
            {
                const char *vb = ((c_hi - zc - 1) & 1 ? v1 : v0) + wv.vbase;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int vt = 0; vt < VT; ++vt) {
                        const bf16x8 x =
                            *reinterpret_cast<const bf16x8 *>(vb + vt * (32 / VL::NBLK) * (2 * TILE) + 32 * t);
                        wv.O[vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, W::as_bf16(wv.Pw[0][t]), wv.O[vt], 0, 0, 0);
                    }
            }
        }

        // ---- the diagonal phase: the block's two tiles, waves 0-3 in tile 2u
        // (key buffer k0, values v0), waves 4-7 in tile 2u+1 (k1, v1)
        __syncthreads();  // every wave is past the pipeline's buffers
        const bool second = 2 * u + 1 < ntiles;
        char *kd = w < NW / 2 ? k0 : k1;
        char *vd = w < NW / 2 ? v0 : v1;
        load_tile<KL>(k0, kr.kd_tile(2 * u), kr.klane, w);
        kr.issue_v(v0, 2 * u);
        if (second) {
            load_tile<KL>(k1, kr.kd_tile(2 * u + 1), kr.klane, w);
            kr.issue_v(v1, 2 * u + 1);
        }
        if (HAS_G) {
            const int r0 = BQ * u;
            load_gk(k0 + LY::GK_OFF, a.G + ((int64_t)sg.start + r0) * HQ + hq, HQ, sg.len - r0, w, lane);
            if (second)
                load_gk(k1 + LY::GK_OFF, a.G + ((int64_t)sg.start + r0 + TILE) * HQ + hq, HQ, sg.len - r0 - TILE, w,
                        lane);
        }
        uint32_t dflags = 0u;
        if (wave_on) {
            kr.load_qd(qt_w, wv.qop);
            dflags = kr.diag_flags(qt_w);
        }
        // ---- the keys of tiles c_lo .. zc in closed form: every logit is 0, so
        // each key's p is bf16(2^-m) (the value the products would have given)
        // and O gains p times the keys' value sums, l p per key (each lane holds
        // half of a query's sum).  The per-tile sums of the preparation step,
        // summed in NPART interleaved parts.
        zc = __builtin_amdgcn_readfirstlane(zc);
        if (zc >= c_lo) {  // uniform over the workgroup
            const int ch = tid % V, part = tid / V;
            const float *vs = a.vsum + ((int64_t)sg.tile_base * a.H + kr.h) * V + ch;
            float acc = 0.f;
            for (int c0 = c_lo; c0 <= zc; c0 += 16 * NPART) {  // a uniform trip count
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c2 = c0 + part + i * NPART;
                    x[i] = c2 <= zc ? vs[(int64_t)c2 * a.H * V] : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) acc += x[i];
            }
            zred[part][ch] = acc;
        }

        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // the closed form's sums (in place since the barrier above)
        if (zc >= c_lo && wave_on) {
            const float p0 = (float)(__bf16)fast_exp2(-wv.m);
#pragma unroll
            for (int vt = 0; vt < VT; ++vt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int ch0 = 32 * vt + 8 * r4 + 4 * hl;
                    f32x4 sv = *reinterpret_cast<const f32x4 *>(&zred[0][ch0]);
#pragma unroll
                    for (int pt = 1; pt < NPART; ++pt) sv += *reinterpret_cast<const f32x4 *>(&zred[pt][ch0]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) wv.O[vt][4 * r4 + e] = fmaf(p0, sv[e], wv.O[vt][4 * r4 + e]);
                }
            wv.l = fmaf(p0, (float)(64 * (zc - c_lo + 1)), wv.l);
        }
        if (wave_on) kr.diag_walk(qt_w, q0w, dflags, kd, vd, wv.qop);

        // ---- epilogue: sink, normalisation, o and lse.  Every wave is past its
        // last LDS read (and every copy has landed) before o is staged in the
        // tile buffers.
        __syncthreads();
        if (wave_on) {
            const float l_tot = pair_sum(wv.l);
            const float m_true = wv.m + g_i;
            float m_fin = m_true, l_fin = l_tot;
            if (a.sink) {
                const float sb = a.sink[hq] * LOG2E;
                m_fin = fmaxf(m_true, sb);
                l_fin = l_tot * exp2f(m_true - m_fin) + exp2f(sb - m_fin);
            }
            const float fac = exp2f(m_true - m_fin) / l_fin;
            // o through LDS (the wave's own rows, OPITCH bytes apart so that the
            // 32 rows' writes spread over the banks, in one of the tile
            // buffers) so that each global store writes whole rows
            constexpr int OPITCH = 2 * V + 16;
            static_assert(2 * WQ * OPITCH <= LY::KBUF && 2 * WQ * OPITCH <= VL::BYTES, "staging fits");
            char *ob = ((w >> 1) == 0 ? k0 : (w >> 1) == 1 ? k1 : (w >> 1) == 2 ? v0 : v1) + (w & 1) * (WQ * OPITCH);
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = wv.O[vt][4 * r4 + e] * fac;
                    *reinterpret_cast<bf16x4 *>(ob + col * OPITCH + 2 * (32 * vt + 8 * r4 + 4 * hl)) =
                        __builtin_convertvector(y, bf16x4);
                }
            }
            constexpr int CPR = V * 2 / 16;  // 16-byte chunks per row
#pragma unroll
            for (int i = 0; i < WQ * CPR / 64; ++i) {
                const int r = (64 * i + lane) / CPR, ch = (64 * i + lane) % CPR;
                const uint4 x = *reinterpret_cast<const uint4 *>(ob + r * OPITCH + 16 * ch);
                if (q0w + r < sg.len) {
                    const int64_t tok = (int64_t)sg.start + q0w + r;
                    // o is not read again: stored past the caches, which keep the tiles
                    // the other workgroups still stream
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x),
                                                reinterpret_cast<u32x4 *>(static_cast<char *>(a.o) + ((tok * HQ + hq) * V) * 2 + 16 * ch));
                }
            }
            if (qrow < sg.len && a.lse && hl == 0)
                a.lse[((int64_t)sg.start + qrow) * HQ + hq] = (m_fin + log2f(l_fin)) * LN2;
        }
    }
}

template <int K, int V>
hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
    const int nblocks_max = (a.max_tiles + 1) / 2;
    const int64_t nwork = (int64_t)a.nseg * nblocks_max * a.HQ;
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
