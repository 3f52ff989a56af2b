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
// Rows of one key / query tile.  Anchors are chosen per TILE rows, per query
// head and per channel, so this is also the anchor granularity.
constexpr int TILE = 128;
// Row of the tile whose floored prefix is the anchor: the middle row keeps
// both exp2 factors of every pair inside the tile within half the tile's
// prefix range.
constexpr int ANCHOR_ROW = 64;
// Rows per chunk of the two-level prefix scan.
constexpr int SCAN_CHUNK = 128;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Exponent clamp for exp2 of a real-valued anchored exponent: exp2 below
// -160 is exactly 0 in float32 (clamping any closer to -150 could round up to
// the smallest denormal), and 126 keeps every factor finite.
constexpr float EXP2_LO = -160.0f;
constexpr float EXP2_HI = 126.0f;

// Integer exponent that moves a value anchored at one tile to another tile's
// anchor (the difference of two integer anchors).  It is applied with ldexp
// to the anchored value itself, never materialised as a factor 2^d: such a
// factor is often below the float32 normal range (a fast channel's anchors
// are ~150 apart per tile) while the product it would form is a normal
// number, and a denormal factor is not reliably kept.  Capped at +127, which
// only a prefix that grows (gates above 1) by more than that can reach.
__device__ inline int anchor_shift(float d) { return (int)fminf(fmaxf(d, -1024.0f), 127.0f); }

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
// exponent-field decrement that moves a query anchored at tile t to tile t-1);
// word REC_GROW is 1 when some channel has R[t-1] < R[t] (a prefix that grows
// over the boundary), else 0.  All zero for a sequence's first tile.
constexpr int REC_WORDS = 256;
constexpr int REC_GROW = 128;

// Forward workspace: segment table | anchors | carry records | rescaled key
// tiles | transposed value tiles.
struct FwdLayout {
    int64_t nseg;        // sequences (num_seqs with packing, else B)
    int64_t tiles;       // upper bound on sum_s ceil(len_s / TILE)
    size_t off_seg, off_anchor, off_rec, off_kt, off_vt, total;
};

inline FwdLayout fwd_layout(int64_t esize, int64_t B, int64_t T, int64_t HQ, int64_t H,
                            int64_t K, int64_t V, int64_t num_seqs) {
    FwdLayout L;
    L.nseg = num_seqs > 0 ? num_seqs : B;
    L.tiles = cdiv(B * T, TILE) + L.nseg;
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
    L.total = o;
    return L;
}

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
    const void *k;     // [rows, H, K]
    const void *v;     // [rows, H, V]
    const float *P;    // [rows, HQ, K]
    SegInfo *seg;      // [nseg], written here
    const int32_t *cu; // [nseg + 1] sequence starts, or null for B sequences of T rows
    float *anchor;     // [tiles, HQ, K]
    uint32_t *rec;     // [tiles, HQ, REC_WORDS]
    void *kt;          // [tiles, HQ, TILE, K]
    void *vt;          // [tiles, H, V, TILE]
    int64_t nseg, tiles, HQ, H, K, V, T;
};
hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st);

struct FwdArgs {
    const void *q;          // [rows, HQ, K]
    const float *P;         // [rows, HQ, K]
    const float *G;         // [rows, HQ] or null
    const float *sink;      // [HQ] or null
    const void *kt;         // [tiles, HQ, TILE, K]
    const void *vt;         // [tiles, H, V, TILE]
    const float *anchor;    // [tiles, HQ, K]
    const uint32_t *rec;    // [tiles, HQ, REC_WORDS]
    const SegInfo *seg;     // [nseg]
    void *o;                // [rows, HQ, V]
    float *lse;             // [rows, HQ] or null
    int32_t nseg, max_tiles, HQ, H, K, V;
    int32_t window;         // <= 0: none
    float qscale;           // scale * log2(e)
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
    float *dkp, *dvp;                  // workspace: per query head dk [rows, HQ, K] and dv [rows, HQ, V] (bf16 path)
    void *qh, *kh;                     // workspace (bf16 path): q~ and k~ [rows, HQ, K] bf16 at their own tile's anchor
    float *Rt;                         // workspace (bf16 path): anchors [tiles, HQ, K], tile = seg.tile_base + row / 128
    const SegInfo *seg;
    int32_t nseg, max_seqlen, rows, HQ, H, K, V, window;
    float scale, qscale;               // scale, scale * log2(e)
};
hipError_t launch_bwd_seg(SegInfo *seg, const int32_t *cu, int64_t nseg, int64_t T, hipStream_t st);
hipError_t launch_bwd(const BwdArgs &a, bool bf16, hipStream_t st);
hipError_t launch_bwd_mfma(const BwdArgs &a, hipStream_t st);  // the dq, dk/dv and group-sum kernels, bf16
// Largest value channel count the backward takes (sizes the dv partials).
constexpr int64_t BWD_MAX_V = 128;

struct BwdLayout {
    size_t off_seg, off_D, off_X, off_Y, off_Z, off_part, off_qh, off_kh, off_rt, off_scan, total;
};
inline BwdLayout bwd_layout(int64_t B, int64_t T, int64_t HQ, int64_t K, int64_t nseg) {
    BwdLayout L;
    const size_t rows = (size_t)(B * T);
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
    L.off_qh = o;
    o = align_up(o + 2 * rows * HQ * K, 256);
    L.off_kh = o;
    o = align_up(o + 2 * rows * HQ * K, 256);
    L.off_rt = o;
    o = align_up(o + sizeof(float) * (size_t)(cdiv((int64_t)rows, TILE) + nseg) * HQ * K, 256);
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
