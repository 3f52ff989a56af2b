// wall_common.h -- types, tile geometry and workspace layout shared by the
// HIP sources of the Wall Attention forward library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wall {

// ----------------------------------------------------------------- vector types
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// ----------------------------------------------------------------- geometry
// Rows of one key / query tile.  The forward anchors the keys of a tile per
// query head and per channel at the floored prefix of the tile's last row
// (for the queries of later tiles).
constexpr int TILE = 128;
// Rows per chunk of the two-level prefix scan.
constexpr int SCAN_CHUNK = 128;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Exponent clamp for exp2 of a real-valued anchored exponent: exp2 below
// -160 is exactly 0 in float32 (clamping any closer to -150 could round up to
// the smallest denormal), and 126 keeps every factor finite.
constexpr float EXP2_LO = -160.0f;
constexpr float EXP2_HI = 126.0f;

// One packed sequence (or one batch row).
struct SegInfo {
    int32_t start;      // first flat token row
    int32_t len;        // rows
    int32_t tile_base;  // index of the sequence's first tile in the tiled workspace
    int32_t pad;
};

inline __host__ __device__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline __host__ __device__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ----------------------------------------------------------------- workspace layouts
// Per (tile, query head) carry record, 1 KB: words 0..K/2-1 hold, per channel
// pair, 128*(R[t-1] - R[t]) clamped to [0, 255*128] as two u16 (the bf16
// exponent-field decrement that moves a query anchored at tile t to tile t-1;
// R[t] is the floored prefix of tile t's last row); word REC_GROW is 1 when
// some channel has R[t-1] < R[t] (a prefix that grows over the tile), else 0.
// All zero for a sequence's first tile.
constexpr int REC_WORDS = 256;
constexpr int REC_GROW = 128;
// Word REC_DIAG: bit b set when some row of the tile's 32-row block b lies more
// than DIAG_SPREAD log2 units from the block's anchor (its last row's floored
// prefix) on some channel: that block's own 32 x 32 pairs are then formed pair
// by pair.  Within it every factor of the block's own pairs stays inside
// 2^+-DIAG_SPREAD, and a term lost to an underflowing factor is below
// 2^(DIAG_SPREAD - 126).
constexpr int REC_DIAG = 129;
constexpr float DIAG_SPREAD = 100.0f;
// Word REC_DMIN: the smallest shift R[t-1] - R[t] over the tile's channels
// (clamped to [0, 255]; 0 for a sequence's first tile), so that a query's
// largest |q~| over its channels falls by at least 2^REC_DMIN from tile t to
// t-1.  Word REC_KMAX: the largest |k| of the tile's keys (float32 bits),
// which bounds every |k~| of the tile for a prefix that does not grow.
constexpr int REC_DMIN = 130;
constexpr int REC_KMAX = 131;
// Rows of one diagonal-phase block (one MFMA n-block of queries).
constexpr int DBLK = 32;
// Per (tile, query head) diagonal-phase carry records, DREC_N records of
// K/2 words in the tile record's format (u16 exponent decrements per channel,
// 128 * shift clamped to [0, 255*128]): record b (b < TILE/DBLK) moves a query
// from block b's anchor to the previous tile's anchor; record TILE/DBLK + b
// moves it from block b+1's anchor to block b's.  Bit 8 + r of the tile
// record's word REC_DIAG is set when some channel's shift of record r is
// negative (a prefix that grows; the kernel then rebuilds q~ from q and P).
constexpr int DREC_N = 2 * (TILE / DBLK);

// Scan workspace: chunk tail sums | exclusive chunk carries | chunk flags.
struct ScanLayout {
    int64_t nchunk;
    size_t off_sum, off_carry, off_flag, total;
};

inline ScanLayout scan_layout(int64_t B, int64_t T, int64_t C) {
    ScanLayout L;
    L.nchunk = cdiv(B * T, SCAN_CHUNK);
    size_t o = 0;
    L.off_sum = o;
    o = align_up(o + sizeof(float) * (size_t)(L.nchunk * C), 256);
    L.off_carry = o;
    o = align_up(o + sizeof(float) * (size_t)(L.nchunk * C), 256);
    L.off_flag = o;
    o = align_up(o + sizeof(int32_t) * (size_t)L.nchunk, 256);
    L.total = o;
    return L;
}

// Forward workspace: segment table | anchors | carry records | rescaled key
// tiles | transposed value tiles | block-anchored key and query tiles | the
// diagonal phase's carry records (all but the table for bf16 inputs only) |
// a scan workspace for the prefix of wall_attn_fwd_prepare_gate.
struct FwdLayout {
    int64_t nseg;        // sequences (num_seqs with packing, else B)
    int64_t tiles;       // upper bound on sum_s ceil(len_s / TILE)
    size_t off_seg, off_anchor, off_rec, off_kt, off_vt, off_kd, off_qd, off_drec, off_vsum, off_kcm, off_scan,
        total;
};

inline FwdLayout fwd_layout(int64_t esize, int64_t B, int64_t T, int64_t HQ, int64_t H,
                            int64_t K, int64_t V, int64_t num_seqs) {
    FwdLayout L;
    L.nseg = num_seqs > 0 ? num_seqs : B;
    // the float32 path reads the raw tensors: no tiles
    L.tiles = esize == 2 ? cdiv(B * T, TILE) + L.nseg : 0;
    size_t o = 0;
    L.off_seg = o;
    o = align_up(o + sizeof(SegInfo) * (size_t)L.nseg, 256);
    L.off_anchor = o;
    o = align_up(o + sizeof(float) * (size_t)(L.tiles * HQ * K), 256);
    L.off_rec = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)(L.tiles * HQ * REC_WORDS), 256);
    L.off_kt = o;
    o = align_up(o + (size_t)esize * (size_t)(L.tiles * HQ * TILE * K), 256);
    L.off_vt = o;
    o = align_up(o + (size_t)esize * (size_t)(L.tiles * H * V * TILE), 256);
    L.off_kd = o;
    o = align_up(o + (size_t)esize * (size_t)(L.tiles * HQ * TILE * K), 256);
    L.off_qd = o;
    o = align_up(o + (size_t)esize * (size_t)(L.tiles * HQ * TILE * K), 256);
    L.off_drec = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)(L.tiles * HQ * DREC_N * (K / 2)), 256);
    L.off_vsum = o;
    o = align_up(o + sizeof(float) * (size_t)(L.tiles * H * V), 256);
    L.off_kcm = o;
    o = align_up(o + sizeof(float) * (size_t)(L.tiles * HQ * K), 256);
    // the prefix scan of wall_attn_fwd_prepare_gate
    L.off_scan = o;
    o = align_up(o + scan_layout(B, T, HQ * K).total, 256);
    L.total = o;
    return L;
}

// ----------------------------------------------------------------- launchers (internal)
// Each returns hipSuccess or the launch error; arguments were validated by the C API.


hipError_t launch_scan(const void *x, bool x_bf16, float *out, int64_t B, int64_t T, int64_t C,
                       const int32_t *cu, int64_t nseq, float scale, void *ws, hipStream_t st);
// out[b, t] = prev[b] (or 0) + scale * (x[b, 0] + ... + x[b, t]) for t < n;
// batch strides in elements, rows of C contiguous.
hipError_t launch_prefix_append(const void *x, bool x_bf16, int64_t x_bs, const float *prev, int64_t prev_bs,
                                float *out, int64_t out_bs, int64_t B, int64_t n, int64_t C, float scale,
                                hipStream_t st);
// The exclusive form (scale * the sum of the earlier rows of the sequence) of
// a float32 input, written as float32 or bf16.
hipError_t launch_scan_excl(const float *x, void *out, bool out_bf16, int64_t B, int64_t T, int64_t C,
                            const int32_t *cu, int64_t nseq, float scale, void *ws, hipStream_t st);

struct PrepArgs {
    const void *q;     // [rows, HQ, K]
    const void *k;     // [rows, H, K]
    const void *v;     // [rows, H, V]
    const float *P;    // [rows, HQ, K]
    SegInfo *seg;      // [nseg], written here
    const int32_t *cu; // [nseg + 1] sequence starts, or null for B sequences of T rows
    float *anchor;     // [tiles, HQ, K] floored prefix of each tile's last row
    uint32_t *rec;     // [tiles, HQ, REC_WORDS]
    void *kt;          // [tiles, HQ, TILE, K] bf16, keys at the tile's anchor
    void *vt;          // [tiles, H, V, TILE] bf16
    void *kd;          // [tiles, HQ, TILE, K] bf16, keys at their 32-row block's anchor
    void *qd;          // [tiles, HQ, TILE, K] bf16, queries (times qscale) at their block's anchor
    uint32_t *drec;    // [tiles, HQ, DREC_N, K / 2] diagonal-phase carry records
    float qscale;      // scale * log2(e)
    int64_t nseg, tiles, HQ, H, K, V, T;
    // the prefix built here (launch_scan_prep): the bf16 gate g [rows, HQ, K],
    // P written [rows, HQ, K], the sums of g over each 128-row chunk of the
    // scan's first kernel [chunks, HQ*K], and the scale of the prefix
    const void *g;
    float *Pw;
    const float *csum;
    float pscale;
    float *vsum;       // [tiles, H, V] float32 sums of each value tile's rows (bf16 path)
    float *kcm;        // [tiles, HQ, K] per channel the largest |k| of the tile's keys (bf16 path)
};
// bf16: the sequence table, anchors, carry records, key and value tiles;
// float32: the sequence table only.
hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st);
// The same preparation with the prefix built in the same pass from a bf16 gate
// (B sequences of T rows, T a multiple of TILE, HQ*K a multiple of 8): P is
// written once, at the rows that end a 32-row block from the block sums (and
// at a tile's last row from the next tile's carry), so that each anchor is the
// floor of the P stored at its row.  Needs the chunk sums of
// launch_scan_chunk_sums first.
hipError_t launch_scan_prep(const PrepArgs &a, hipStream_t st);
// The scan's chunk sums alone (its first kernel), for B sequences of T rows,
// in a scan workspace of scan_layout(B, T, C).
hipError_t launch_scan_chunk_sums(const void *x, bool x_bf16, int64_t B, int64_t T, int64_t C, void *ws,
                                  hipStream_t st);

struct FwdArgs {
    const void *q;          // [rows, HQ, K]
    const void *k;          // [rows, H, K] raw keys (the query's own tile, float32 path)
    const void *v;          // [rows, H, V] raw values (float32 path)
    const float *P;         // [rows, HQ, K]
    const float *G;         // [rows, HQ] or null
    const float *sink;      // [HQ] or null
    const void *kt;         // [tiles, HQ, TILE, K] (bf16 path)
    const void *vt;         // [tiles, H, V, TILE] (bf16 path)
    const void *kd;         // [tiles, HQ, TILE, K] (bf16 path)
    const void *qd;         // [tiles, HQ, TILE, K] (bf16 path)
    const uint32_t *drec;   // [tiles, HQ, DREC_N, K / 2] (bf16 path)
    const float *anchor;    // [tiles, HQ, K] (bf16 path)
    const uint32_t *rec;    // [tiles, HQ, REC_WORDS]
    const SegInfo *seg;     // [nseg]
    void *o;                // [rows, HQ, V]
    float *lse;             // [rows, HQ] or null
    int32_t nseg, max_tiles, HQ, H, K, V;
    int32_t window;         // <= 0: none
    float qscale;           // scale * log2(e)
    const float *vsum;      // [tiles, H, V] float32 sums of each value tile's rows (bf16 path)
    const float *kcm;       // [tiles, HQ, K] per channel the largest |k| of the tile's keys (bf16 path)
};
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t st);

// ----------------------------------------------------------------- backward
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;  // [rows, HQ or H, K / V] in dtype
    const float *P, *G, *sink, *lse;   // P [rows, HQ, K]; G [rows, HQ] or null; sink [HQ] or null
    void *dq, *dk, *dv;                // in dtype
    float *dsink;                      // [HQ] or null
    float *D, *X, *Y, *Z;              // workspace: do.o; q.dq - k.dk per head; dS row - column sums; sink terms
    float *dkp, *dvp;                  // workspace: per query head dk [rows, HQ, K] and dv [rows, HQ, V]
    float *dqd;                        // workspace: dq of the pairs inside one 32-row block [rows, HQ, K]
    void *qh, *kh;                     // workspace (bf16 path): q~ and k~ [rows, HQ, K] bf16, see BWD_BLK
    float *Ab;                         // workspace (bf16 path): block anchors [blocks, HQ, K]
    int32_t *flag;                     // workspace (bf16 path): [blocks, HQ], sequence + 1 of a spread block, else 0
    uint32_t *bmax;                    // workspace (bf16 path): [blocks, HQ, BWD_BM], see BWD_BM
    uint16_t *cmax;                    // workspace (bf16 path): [blocks, HQ, 2, K] per channel the largest stored |q~|, |k~| (bf16 bits)
    float *wsum;                       // workspace (bf16 path): [blocks, HQ, V] sums of bf16(2^-L) do from a block on
    const SegInfo *seg;
    int32_t nseg, max_seqlen, rows, HQ, H, K, V, window;
    float scale, qscale;               // scale, scale * log2e
};
// The backward's anchor blocks: 32 rows, the block of row r of a sequence is
// 4 * tile_base + r / 32.  Block b's anchor A_b is the floored prefix of its
// last row (of the sequence's last row for a short tail block), A_(-1) = 0.
// q~ of a row is stored at the anchor of the block before its own, k~ at its
// own block's anchor, so either factor is at most 2 for a prefix that falls.
// A block is spread when some channel of one of its rows lies more than
// BWD_SPREAD log2 units from A_b or A_(b-1); pairs inside a spread block are
// formed pair by pair, every other pair through anchors.
constexpr int BWD_BLK = 32;
constexpr float BWD_SPREAD = 64.0f;
// Per (block, query head) record of the bf16 backward: the largest stored |q~|
// and |k~| of the block's rows (float bits), and e with 2^e <= L_i for every
// row of the block, L = lse log2e (int bits; BWD_NO_EXP when some L_i <= 0).
constexpr int BWD_BM = 4;
constexpr int BWD_NO_EXP = -100000;
hipError_t launch_bwd_seg(SegInfo *seg, const int32_t *cu, int64_t nseg, int64_t T, hipStream_t st);
hipError_t launch_bwd(const BwdArgs &a, bool bf16, hipStream_t st);
hipError_t launch_bwd_mfma(const BwdArgs &a, hipStream_t st);  // the dq, dk/dv and group-sum kernels, bf16
// pair-by-pair gradients of the pairs inside 32-row blocks: every block
// (flags null) or the spread ones
hipError_t launch_bwd_diag(const BwdArgs &a, bool bf16, bool all, hipStream_t st);
// Largest value channel count the backward takes (sizes the dv partials).
constexpr int64_t BWD_MAX_V = 128;

struct BwdLayout {
    size_t off_seg, off_D, off_X, off_Y, off_Z, off_part, off_dqd, off_qh, off_kh, off_rt, off_flag, off_bmax,
        off_cmax, off_wsum, off_scan, total;
};
inline BwdLayout bwd_layout(int64_t B, int64_t T, int64_t HQ, int64_t K, int64_t nseg) {
    BwdLayout L;
    const size_t rows = (size_t)(B * T);
    // anchor blocks: 4 per 128-row tile, a partial tile per sequence at most
    const size_t blocks = (size_t)(cdiv((int64_t)rows, TILE) + nseg) * (TILE / BWD_BLK);
    size_t o = 0;
    L.off_seg = o;
    o = align_up(o + sizeof(SegInfo) * (size_t)nseg, 256);
    L.off_D = o;
    o = align_up(o + sizeof(float) * rows * HQ, 256);
    L.off_X = o;
    o = align_up(o + sizeof(float) * rows * HQ * K, 256);
    L.off_Y = o;
    o = align_up(o + sizeof(float) * rows * HQ, 256);
    L.off_Z = o;
    o = align_up(o + sizeof(float) * rows * HQ, 256);
    L.off_part = o;
    o = align_up(o + sizeof(float) * rows * HQ * (K + BWD_MAX_V), 256);
    L.off_dqd = o;
    o = align_up(o + sizeof(float) * rows * HQ * K, 256);
    L.off_qh = o;
    o = align_up(o + 2 * rows * HQ * K, 256);
    L.off_kh = o;
    o = align_up(o + 2 * rows * HQ * K, 256);
    L.off_rt = o;
    o = align_up(o + sizeof(float) * blocks * HQ * K, 256);
    L.off_flag = o;
    o = align_up(o + sizeof(int32_t) * blocks * HQ, 256);
    L.off_bmax = o;
    o = align_up(o + sizeof(uint32_t) * blocks * HQ * BWD_BM, 256);
    L.off_cmax = o;
    o = align_up(o + sizeof(uint16_t) * blocks * HQ * 2 * K, 256);
    L.off_wsum = o;
    o = align_up(o + sizeof(float) * blocks * HQ * BWD_MAX_V, 256);
    L.off_scan = o;
    o = align_up(o + scan_layout(B, T, HQ * K).total, 256);
    L.total = o;
    return L;
}

// ----------------------------------------------------------------- decode
struct CacheArgs {
    const void *k;      // [B, Tcap, H, K]
    const float *P;     // [B, Tcap, HQ, K]
    void *kt;           // [B, Tcap, HQ, K]
    float *r;           // [B, ceil(Tcap / C), HQ, K]
    int64_t B, Tcap, HQ, H, K, C, t0, t1;  // rows t0 .. t1-1 are written
};
hipError_t launch_kv_cache(const CacheArgs &a, bool bf16, hipStream_t st);

struct DecodeArgs {
    const void *q;      // [B, HQ, K]
    const void *v;      // [B, Tcap, H, V]
    const float *pc;    // [B, HQ, K], batch rows pc_bs floats apart
    int64_t pc_bs;
    const void *kt;     // [B, Tcap, HQ, K]
    const float *r;     // [B, ceil(Tcap / C), HQ, K]
    const float *sink;  // [HQ] or null
    void *o;            // [B, HQ, V]
    float *lse;         // [B, HQ] or null
    float *part;        // [nsplit][B * HQ][V + 2]: o not normalised, m, l (log2 units)
    int32_t B, T, Tcap, HQ, H, K, V, C, nsplit, S;
    int32_t nwg;        // waves (query heads of one kv head) per block, divides HQ / H, <= 4
    float qscale;       // scale * log2(e)
};
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t st);

// Decode splits: about 2048 one-wave blocks when the keys allow, S keys each
// (a multiple of 64), every split non-empty.
struct DecodeLayout {
    int64_t nsplit, S;
    size_t total;
};
inline DecodeLayout decode_layout(int64_t B, int64_t T, int64_t HQ, int64_t V) {
    const int64_t rounds = cdiv(T, 64);
    int64_t want = cdiv(2048, B * HQ);
    if (want > rounds) want = rounds;
    if (want < 1) want = 1;
    DecodeLayout L;
    L.S = 64 * cdiv(rounds, want);
    L.nsplit = cdiv(T, L.S);
    L.total = align_up(sizeof(float) * (size_t)(L.nsplit * B * HQ * (V + 2)), 256);
    return L;
}

}  // namespace wall
