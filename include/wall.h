/*
 * wall.h -- C ABI of the MI355X (gfx950) Wall Attention forward library.
 *
 * Wall Attention (wall-attention-release README, introduction; Wall Attention
 * blog, "Definition: Wall Attention") is softmax attention whose QK inner
 * product carries a per-channel, per-timestep decay accumulated between the
 * two positions:
 *
 *   o_i = sum_{j<=i} softmax_j( scale * sum_n exp2(P_{i,n} - P_{j,n}) q_{i,n} k_{j,n}
 *                               + G_i - G_j ) v_j,
 *   P_t = (1/ln 2) * sum_{u<=t} g_u      (log2-unit prefix of the log gate g),
 *
 * g = 0 giving vanilla softmax attention.  The library exports the two steps
 * of the README's prefill path: the prefix scan (its decode example builds P
 * with a global cumsum scaled by 1/ln 2) and the fused causal forward.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a caller-owned, dense, row-major DEVICE pointer
 *     on the current HIP device, aligned to 16 bytes.  The library keeps no
 *     pointer after a call returns, allocates nothing, never synchronises and
 *     never aborts.
 *   - Debugging: with the environment variable WALL_DEBUG set to a value other
 *     than "0" (read once per process), a refused call prints its entry point,
 *     the failed check's line and the status to stderr, and each call that
 *     launches kernels synchronises the device before returning, so that a
 *     kernel fault is reported (as WALL_ERR_LAUNCH, with the HIP error on
 *     stderr) by the call that launched it.
 *   - Work is enqueued on `stream` (0 = the legacy default stream) and runs
 *     asynchronously; outputs are valid once the stream reaches that point.
 *   - Token-major layouts: a token row is (b, t) with flat id b*T + t; with
 *     cu_seqlens (B == 1) the flat id is the packed position t.
 *   - Argument checks run before any HIP call, so an invalid call returns its
 *     status without touching the device.  Contents of device buffers (e.g.
 *     cu_seqlens) cannot be checked without a synchronisation and are the
 *     caller's responsibility; they are listed under each call.  The library
 *     trusts the device-side sequence offsets and the max_seqlen it is given:
 *     offsets that are not as documented, or a max_seqlen below the longest
 *     sequence, give wrong results or out-of-range accesses.  (The Python
 *     wrappers wall_prefix_scan, wall_attn_fwd, wall_attn_bwd and wall_attn
 *     check both on the host; the stage wrappers wall_attn_fwd_prepare and
 *     wall_attn_fwd_run do not.)
 *   - Two calls that share a workspace or an output buffer must be ordered on
 *     one stream; calls on different streams with separate buffers are
 *     independent.
 */
#ifndef WALL_H
#define WALL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized; in C++ they have int as their fixed underlying
 * type, so that any int value (e.g. an unsupported dtype, which the entry
 * points reject) is a valid value of the type. */
#ifdef __cplusplus
#define WALL_ENUM_INT : int
#else
#define WALL_ENUM_INT
#endif

typedef enum WALL_ENUM_INT {
    WALL_F32 = 0,  /* IEEE binary32 */
    WALL_BF16 = 1, /* bfloat16 (1-8-7) */
} wall_dtype_t;

typedef enum WALL_ENUM_INT {
    WALL_OK = 0,
    WALL_ERR_INVALID_ARG = 1, /* null required pointer, bad size, bad alignment, short workspace */
    WALL_ERR_UNSUPPORTED = 2, /* valid but not implemented: a head size or dtype with no kernel */
    WALL_ERR_LAUNCH = 3,      /* a kernel launch failed; hipGetLastError() is reported */
    WALL_ERR_SCRATCH = 4,     /* a no-allocation entry point would need more than its fixed scratch */
} wall_status_t;

/* Human-readable name of a status value (static storage, never NULL); any
 * int is accepted, "WALL_ERR_UNKNOWN" for one that names no status. */
const char *wall_status_string(int s);

/* Library version as 10000*major + 100*minor + patch. */
int wall_version(void);

/* ------------------------------------------------------------------ prefix scan
 *
 * out[r, c] = scale * sum_{u = s(r) .. r} x[u, c]
 *
 * over token rows r of x viewed as [B*T, C], where s(r) is the first row of
 * the sequence that holds r (row b*T for batch b, or cu_seqlens[k] with
 * packing).  With x = g [B,T,HQ,K] (C = HQ*K) and scale = 1/ln 2 this is the
 * per-channel log2 prefix P of the Wall Attention blog's factored form
 * ("Definition: Wall Attention": P_t = sum_{u<=t} log gate_u) in the units
 * of the README's decode example.  With x = g_scalar [B,T,HQ] (C = HQ) it
 * is the prefix G of the FoX-style scalar gate.
 *
 *   x            [B, T, C] in x_dtype (WALL_BF16 or WALL_F32)
 *   out          [B, T, C] float32; may not alias x
 *   cu_seqlens   NULL, or int32 [num_seqs + 1] on the device with B == 1,
 *                cu[0] = 0, non-decreasing, cu[num_seqs] = T (empty
 *                sequences allowed).  Caller-checked contents.
 *   workspace    device scratch of at least
 *                wall_prefix_scan_workspace_size(B, T, C) bytes, 256-byte
 *                aligned; its contents on entry are ignored.
 * Accumulation is float32 along T (two-level: 128-row chunks, then a
 * segmented scan of chunk sums), so |error| grows like eps32 * |out|.
 * Errors: INVALID_ARG for a null x/out/workspace, B, T or C < 1, cu_seqlens
 * with B != 1 or num_seqs < 1, misalignment, a short workspace;
 * UNSUPPORTED for another dtype; LAUNCH on a failed launch. */
size_t wall_prefix_scan_workspace_size(int64_t B, int64_t T, int64_t C);

wall_status_t wall_prefix_scan(const void *x, wall_dtype_t x_dtype, float *out,
                               int64_t B, int64_t T, int64_t C,
                               const int32_t *cu_seqlens, int64_t num_seqs,
                               float scale,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------ prefix append
 *
 * out[b, t, c] = prev[b, c] + scale * sum_{u = 0 .. t} x[b, u, c],  t < n
 *
 * The running prefix of an append-as-you-go sequence (the README's
 * streaming decode loop: P of each new token from the previous token's P,
 * the blog's "Fast training and inference" cache that a decoder extends one
 * token at a time).  prev = NULL starts a sequence (prev = 0).  Rows of C
 * values are contiguous; consecutive batch rows are *_batch_stride elements
 * apart, so x, prev and out may be row slices of larger [B, T_cap, C]
 * buffers (out at row t0 and prev at row t0-1 of the same P buffer).
 *
 *   x     [B, n, C] in x_dtype (WALL_BF16 or WALL_F32), row stride C
 *   prev  NULL or [B, C] float32
 *   out   [B, n, C] float32; must not overlap x (prev may lie in out's buffer)
 * Accumulation: float32, s = x_0 + ... + x_t in order, then prev + scale*s,
 * so a prefix built by appends matches wall_prefix_scan's up to float32
 * rounding of |P| (not bit for bit).
 * Errors: INVALID_ARG for a null x/out, B, n or C < 1, a batch stride
 * below n*C (below C for prev), misalignment, out overlapping x;
 * UNSUPPORTED for another dtype; LAUNCH on a failed launch. */
wall_status_t wall_prefix_append(const void *x, wall_dtype_t x_dtype, int64_t x_batch_stride,
                                 const float *prev, int64_t prev_batch_stride, float *out,
                                 int64_t out_batch_stride, int64_t B, int64_t n, int64_t C,
                                 float scale, hipStream_t stream);

/* ------------------------------------------------------------------ fused forward
 *
 * The causal Wall Attention forward of the README's `wall_attn` (usage
 * "Training / prefill"), forward half only, with its optional arguments:
 *
 *   logit_ij (log2 units) = scale*log2(e) * sum_n exp2(P_in - P_jn) q_in k_jn
 *                           + (G_i - G_j)
 *   visible(i, j) = j <= i, same sequence, and (window_size <= 0 or i-j < window_size)
 *   sink: one extra logit sink_bias[hq] (natural log) with a zero value
 *   o_i  = sum_j 2^(logit_ij - M_i) v_j / Z_i   (M_i the row max, sink included)
 *   lse_i = ln 2 * (M_i + log2 Z_i)              (natural log, sink included)
 *
 * GQA: HQ query heads share H key/value heads, HQ % H == 0, query head hq
 * reads key/value head hq / (HQ / H) (README features list).  The decay P and
 * the scalar prefix G are per QUERY head.
 *
 *   q          [B, T, HQ, K]  dtype
 *   k          [B, T, H,  K]  dtype
 *   v          [B, T, H,  V]  dtype
 *   P          [B, T, HQ, K]  float32, log2 prefix of g (wall_prefix_scan with
 *                             scale 1/ln 2 and the same cu_seqlens)
 *   G          NULL or [B, T, HQ] float32, log2 prefix of g_scalar
 *   sink_bias  NULL or [HQ] float32, natural-log logit of the sink
 *   o          [B, T, HQ, V]  dtype (written)
 *   lse        NULL or [B, T, HQ] float32 (written)
 *   scale      multiplies the decayed dot product (the README passes K**-0.5)
 *   window_size  <= 0: no window; else W keys including the query itself
 *   cu_seqlens NULL, or as for wall_prefix_scan (B == 1); max_seqlen must be
 *              >= the longest sequence (unused without cu_seqlens).
 *   workspace  device scratch of at least wall_attn_fwd_workspace_size(...)
 *              bytes, 256-byte aligned; contents on entry are ignored.  It
 *              holds the decay-rescaled key cache, the transposed values and
 *              the per-tile anchors of this call.
 * Numerics: exp2(P_i - P_j) is split at integer per-channel anchors R (the
 * blog's per-tile anchors, section "Fast training and inference") as
 * exp2(P_i - R) * exp2(R - P_j).  A key of a 128-row tile before its
 * query's tile is read at the floored prefix of its own tile's last row, a
 * row between the two, so for a prefix that falls (g <= 0) neither factor
 * exceeds 2 and a factor that underflows belongs to a term below 2^-125 of
 * the largest.  The keys of the query's own tile are read at anchors chosen
 * by the query's group of 32 rows: the floored prefix at the middle of its
 * rows; or, when some row of the group lies more than 100 log2 units from
 * it, the row just before the group for the earlier keys and no anchor at
 * all (the decay formed pair by pair in float32) for the keys among the
 * group's rows.  The result therefore keeps its accuracy for every g <= 0,
 * down to closed gates; for a prefix that grows (g > 0) while it grows by
 * less than about 100 log2 units within any 128 rows and every factor
 * exp2(P_i - P_j) stays below about 2^100.  bf16 inputs use bf16 MFMA
 * operands with float32 accumulation and a float32 online softmax; float32
 * inputs are computed in float32 throughout (one anchor for all keys
 * before a 64-row query block, pair-by-pair decay inside it).
 * Errors: INVALID_ARG for a null required pointer, a size < 1, HQ % H != 0,
 * cu_seqlens with B != 1 or num_seqs < 1 or max_seqlen < 1, misalignment, a
 * short workspace; UNSUPPORTED for K or V not in {64, 128} or another dtype;
 * LAUNCH on a failed launch. */
size_t wall_attn_fwd_workspace_size(wall_dtype_t dtype, int64_t B, int64_t T,
                                    int64_t HQ, int64_t H, int64_t K, int64_t V,
                                    int64_t num_seqs);

wall_status_t wall_attn_fwd(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                            const float *P, const float *G, const float *sink_bias,
                            void *o, float *lse,
                            int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                            float scale, int64_t window_size,
                            const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                            void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------ the forward in two stages
 *
 * wall_attn_fwd is exactly wall_attn_fwd_prepare followed by
 * wall_attn_fwd_run on the same stream and workspace.  The split lets a
 * caller time or reuse the stages:
 *
 * wall_attn_fwd_prepare folds the decay into the keys once per 128-row tile
 * and query head -- the prefill counterpart of the README's
 * build_wall_kv_cache (k_tilde[j] = k[j] * exp2(R_c - P[j]) with a per-chunk
 * anchor R_c) -- and, for each tile's own queries, into the keys and the
 * queries (times scale*log2(e)) of every 32-row block at that block's own
 * anchor; it stores, in `workspace`, the sequence table, the anchors, these
 * rescaled keys and queries and the value tiles.  Arguments mean what they
 * mean for wall_attn_fwd (no G, sink, window or max_seqlen here).
 *
 * wall_attn_fwd_run reads that workspace (unchanged since a prepare call
 * with the same q, k, v, P, scale, shapes and cu_seqlens, ordered before it
 * on the stream) together with q, k, v, P, G and sink_bias, and writes o and
 * lse.
 * k and v are the prepare call's raw keys and values: the keys of each
 * query's own tile (and, for float32 inputs, every key and value) are read
 * from them.  `workspace` is read only.
 * Errors are those of wall_attn_fwd for the arguments each stage takes. */
wall_status_t wall_attn_fwd_prepare(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                                    const float *P,
                                    int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                                    float scale, const int32_t *cu_seqlens, int64_t num_seqs,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* wall_attn_fwd_prepare_gate: the prefix scan and the preparation in one
 * call.  It writes P = cumsum(g) / ln 2 per sequence (what wall_prefix_scan
 * with scale 1/ln 2 writes) and prepares `workspace` as wall_attn_fwd_prepare
 * does with that P; wall_attn_fwd_run then takes that P.
 *
 *   g        [B, T, HQ, K] in g_dtype (WALL_BF16 or WALL_F32), natural-log gate
 *   P        [B, T, HQ, K] float32 (written; may not alias g)
 *   other arguments as for wall_attn_fwd_prepare (scale as for wall_attn_fwd)
 *
 * B sequences of T rows (no cu_seqlens) with T a multiple of 128, bf16 q, k,
 * v and g and HQ*K a multiple of 8 take one combined pass: the scan's chunk
 * sums and carries (two small kernels), then one kernel that forms P along
 * the rows, writes it, and builds the anchored tiles from it without reading
 * it back.  There, at the last row of each 32-row block P is formed from the
 * block sums (at a tile's last row from the next tile's carry), so every
 * anchor is the floor of the P stored at its row; P then differs from
 * wall_prefix_scan's in float32 rounding only.  Any other case runs the scan
 * and the preparation one after the other (P exactly wall_prefix_scan's).
 * Errors: those of wall_attn_fwd_prepare; INVALID_ARG for a null g or P, P
 * aliasing g or misaligned; UNSUPPORTED for another g_dtype. */
wall_status_t wall_attn_fwd_prepare_gate(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                                         const void *g, wall_dtype_t g_dtype, float *P,
                                         int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                                         float scale, const int32_t *cu_seqlens, int64_t num_seqs,
                                         void *workspace, size_t workspace_bytes,
                                         hipStream_t stream);

wall_status_t wall_attn_fwd_run(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                                const float *P, const float *G, const float *sink_bias,
                                void *o, float *lse,
                                int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                                float scale, int64_t window_size,
                                const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                                const void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ------------------------------------------------------------------ backward
 *
 * Gradients of wall_attn_fwd (the README's training path: "exact analytic
 * gradients" for q, k, v, the decay gate g and the scalar gate g_scalar,
 * and the sink).  With s_ij the natural-log logit of wall_attn_fwd,
 * A_ij = exp(s_ij - lse_i) and D_i = dout_i . o_i:
 *   dS_ij = A_ij (dout_i . v_j - D_i)
 *   dv_j  = sum_i A_ij dout_i                       (summed over the query heads of j's kv head)
 *   dq_in = scale sum_j dS_ij exp2(P_in - P_jn) k_jn
 *   dk_jn = scale sum_i dS_ij exp2(P_in - P_jn) q_in (summed likewise)
 *   dg_un = sum_{t >= u in u's sequence} (q_tn dq_tn - k_tn dk^(hq)_tn)
 *   dg_scalar_u = sum_{t >= u} (sum_j dS_tj - sum_i dS_it)
 *   dsink = -sum_i exp(sink - lse_i) D_i
 * (dk^(hq): the query head's own part of dk; the decay between j and i is
 * the product of the gates g_u, j < u <= i, of the blog's "Definition: Wall
 * Attention", so dg collects every pair that straddles u).
 *
 *   q, k, v, P, G, sink_bias, cu_seqlens, max_seqlen, scale, window_size
 *               as passed to wall_attn_fwd
 *   o, lse      that call's outputs (lse required)
 *   dout        [B, T, HQ, V] dtype, the gradient of o
 *   dq [B,T,HQ,K], dk [B,T,H,K], dv [B,T,H,V]  dtype (written)
 *   dg          [B, T, HQ, K] in g_dtype (written), the gradient of the
 *               natural-log gate g (not of P)
 *   dg_scalar   [B, T, HQ] in g_dtype (written; required when G is given)
 *   dsink       [HQ] float32 (written; required when sink_bias is given)
 *   workspace   device scratch of at least wall_attn_bwd_workspace_size(...)
 *               bytes, 256-byte aligned, contents on entry ignored
 * Numerics: every pair (i, j) of rows in different 32-row blocks uses the
 * anchor identity exp2(P_i - P_j) = exp2(P_i - R) exp2(R - P_j) at an integer
 * per-channel anchor R = floor(P) of a row between j and i (the last row of
 * a block at or after j's and before i's), so for a prefix that falls both
 * factors are at most 2 at any gate strength, and a factor that underflows
 * belongs to a term below 2^-125 of |dS q k|.  The pairs inside one 32-row
 * block use the block's own last-row anchor (one factor up to 2^65) when
 * every row of the block lies within 64 log2 units of it and of the
 * previous block's anchor, and are otherwise formed pair by pair in float32
 * with one exp2 per pair and channel.  bf16 inputs: the five products run on
 * bf16 matrix cores with float32 accumulation (q~, k~, the probabilities
 * and dS rounded to bf16; softmax, scaling and the gate sums in float32);
 * every move of q~, k~ or an accumulator between anchors is an exact power
 * of two, and the q-side and k-side terms of dg are formed from the same
 * rounded q~ and k~, so their rounding cancels in dg's sums.  bf16 inputs
 * without g_scalar or a window: pairs of rows in different 128-row tiles
 * whose score is bounded (from each block's per-channel largest stored
 * |q~|, |k~| and the anchor gaps) by 2^(e - 26), with 2^e <= lse_i log2e, are left out of
 * the products: their probability is exactly 2^(-lse_i log2e) in float32,
 * their dv terms come from per-block suffix sums of those weights times
 * do_i, and their dq, dk and dg terms (each carrying that score as a
 * factor) are dropped.  float32
 * inputs: every product in float32 on the vector ALUs, the pairs inside each
 * 32-row block always pair by pair.  Over one sequence the summands of dg
 * (and of dg_scalar) add up to zero, so the suffix sums are taken as minus
 * the exclusive prefix sums.  Deterministic (no atomics on the results).
 * Errors: INVALID_ARG for a null required pointer, G without dg_scalar, a
 * sink without dsink, a size < 1, HQ % H != 0, bad cu_seqlens arguments,
 * misalignment, a short workspace; UNSUPPORTED for K or V not in {64, 128},
 * another dtype, or HQ * sequences * ceil(longest sequence / 128) above
 * INT32_MAX (one block each); LAUNCH on a failed launch. */
size_t wall_attn_bwd_workspace_size(int64_t B, int64_t T, int64_t HQ, int64_t K, int64_t num_seqs);

wall_status_t wall_attn_bwd(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                            const float *P, const float *G, const float *sink_bias,
                            const void *o, const float *lse, const void *dout,
                            void *dq, void *dk, void *dv, void *dg, void *dg_scalar,
                            wall_dtype_t g_dtype, float *dsink,
                            int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                            float scale, int64_t window_size,
                            const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                            void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------ decode cache
 *
 * The README's build_wall_kv_cache (section "Decode (cached generation)"):
 * the decay folded into the keys against per-chunk anchors, so that a
 * decode step never re-accumulates the prefix.  For chunk c of chunk_size
 * rows, query head hq and channel n:
 *
 *   k_tilde[b, j, hq, n]  = k[b, j, hq / (HQ/H), n] * exp2(r_cache[b, j/chunk_size, hq, n] - P[b, j, hq, n])
 *
 * The README names one anchor per chunk without fixing its row.  Here the
 * anchor of a chunk is floor(P) of its first row until a later row t of the
 * chunk lies more than 64 log2 units below it (r - P[t] > 64, its key
 * factor would pass 2^64); the anchor then moves to floor(P[t]) and the rows
 * of the chunk cached before t are lowered by the exact power of two
 * 2^(new - old) (on the bit pattern: exponent lowered, 0 below the range).
 * Every cached factor stays at most 2^64 and a decode query's factor at most
 * 2, at any gate strength (down to closed gates); a row lowered out of range
 * carries a term below 2^-60 of the largest.  Only rows t0 .. t1-1 of every
 * sequence are written (and, when an anchor moves, the earlier rows of its
 * chunk lowered): a call with t0 = 0, t1 = T builds the cache of a prefill,
 * a call with t1 = t0 + 1 appends one token.  A chunk opened by an earlier
 * call (on the same stream, or otherwise completed) continues from its
 * stored anchor, so building in pieces gives the bits of one build.  The
 * exponent is clamped to [-160, 126].
 *
 *   k           [B, T_cap, H, K]  dtype; rows t0 .. t1-1 are read
 *   P           [B, T_cap, HQ, K] float32 log2 prefix (wall_prefix_scan of g
 *               with scale 1/ln 2); rows t0 .. t1-1 are read
 *   k_tilde     [B, T_cap, HQ, K] dtype (rows t0 .. t1-1 written; the rows of
 *               their chunks before t0 rewritten when an anchor moves)
 *   r_cache     [B, ceil(T_cap / chunk_size), HQ, K] float32 (anchors of the
 *               chunks that rows t0 .. t1-1 touch: read when the chunk opened
 *               before t0, written)
 *   T_cap       rows allocated per sequence in k, P, k_tilde (and v below)
 * All pointers are caller-owned device memory, 16-byte aligned.
 * Errors: INVALID_ARG for a null pointer, a size < 1, HQ % H != 0, not
 * 0 <= t0 < t1 <= T_cap, misalignment, sizes past 2^40 elements;
 * UNSUPPORTED for K not in {64, 128}, chunk_size not a positive multiple of
 * 64, or another dtype; LAUNCH on a failed launch. */
wall_status_t wall_kv_cache_build(const void *k, wall_dtype_t dtype, const float *P,
                                  void *k_tilde, float *r_cache,
                                  int64_t B, int64_t T_cap, int64_t HQ, int64_t H, int64_t K,
                                  int64_t chunk_size, int64_t t0, int64_t t1,
                                  hipStream_t stream);

/* ------------------------------------------------------------------ streaming append
 *
 * One turn of the README's append-as-you-go decode loop for new rows
 * t0 .. t1-1 of every sequence, in one pass: the log2 prefix of the new rows
 * from the previous row's, exactly as wall_prefix_append computes it
 * (prev = P[b, t0-1], or 0 when t0 = 0; s = g_t0 + ... + g_t in float32;
 * P[b, t] = prev + scale * s), then the cache rows and chunk anchors exactly
 * as wall_kv_cache_build computes them from that P.  The results equal those
 * two calls bit for bit; the saving is one launch and one pass over P.
 *
 *   g           [B, T_cap, HQ, K] in g_dtype (WALL_BF16 or WALL_F32), rows t0 .. t1-1 read
 *   k           [B, T_cap, H, K] in dtype, rows t0 .. t1-1 read
 *   P           [B, T_cap, HQ, K] float32: row t0-1 read (t0 > 0), rows t0 .. t1-1 written
 *   k_tilde     [B, T_cap, HQ, K] in dtype, rows t0 .. t1-1 written
 *   k_tilde, r_cache   as for wall_kv_cache_build (the chunk of t0 continues
 *               from its stored anchor; the anchors of every touched chunk
 *               are written)
 *   scale       1 / ln 2 for the natural-log gate of the README
 * Errors: INVALID_ARG for a null pointer, a size < 1, HQ % H != 0, t0 < 0,
 * t1 <= t0 or t1 > T_cap, misalignment; UNSUPPORTED for K not in {64, 128},
 * chunk_size not a positive multiple of 64, or another dtype; LAUNCH on a
 * failed launch. */
wall_status_t wall_stream_append(const void *g, wall_dtype_t g_dtype, const void *k, wall_dtype_t dtype,
                                 float *P, void *k_tilde, float *r_cache, int64_t B, int64_t T_cap,
                                 int64_t HQ, int64_t H, int64_t K, int64_t chunk_size, int64_t t0,
                                 int64_t t1, float scale, hipStream_t stream);

/* ------------------------------------------------------------------ decode
 *
 * The README's wall_attn_decode: one query per (b, hq) -- the newest token,
 * whose log2 prefix is p_curr -- against the cached keys j = 0 .. T-1 of
 * its sequence (the newest token included, so every key is visible):
 *
 *   logit_j (log2 units) = scale*log2(e) * sum_n q_n * exp2(p_curr_n - r_cache[j/C, n]) * k_tilde[j, n]
 *   o  = sum_j 2^(logit_j - M) v_j / Z,  lse = ln 2 * (M + log2 Z)
 *
 * with the sink as in wall_attn_fwd.  This is the forward's last row: the
 * anchors cancel (blog, "Definition: Wall Attention", factored form).
 *
 *   q           [B, HQ, K] dtype (the README's [B, 1, HQ, K])
 *   v           [B, T_cap, H, V] dtype, rows 0 .. T-1 read
 *   p_curr      [B, HQ, K] float32, P at the query's row; batch rows are
 *               p_curr_batch_stride floats apart (0: HQ*K, dense), so p_curr
 *               may be the newest row of a [B, T_cap, HQ, K] prefix buffer
 *               (stride T_cap*HQ*K); a nonzero stride is a multiple of 4,
 *               at least HQ*K
 *   k_tilde, r_cache   a cache built by wall_kv_cache_build with this
 *               chunk_size and T_cap, rows 0 .. T-1 complete and no later
 *               row built (a row after the query could have moved the last
 *               chunk's anchor past it; rows are appended, never rolled back)
 *   sink_bias   NULL or [HQ] float32
 *   o           [B, HQ, V] dtype (written); lse NULL or [B, HQ] float32 (written)
 *   workspace   device scratch of at least
 *               wall_attn_decode_workspace_size(B, T, HQ, V) bytes, 256-byte
 *               aligned, contents on entry ignored (split-KV partials)
 * Numerics: q~ = q * scale*log2(e) * exp2(p_curr - R) is rounded to the cache
 * dtype once per chunk (at most 2, since the query row is at or after every
 * cached row and the anchor is the floor of one of them); dot products and
 * the softmax are float32.
 * Errors: INVALID_ARG for a null required pointer, a size < 1, HQ % H != 0,
 * T > T_cap, B*HQ > 65535, a bad p_curr stride, misalignment, a short
 * workspace; UNSUPPORTED for K
 * or V not in {64, 128}, chunk_size not a positive multiple of 64, or another
 * dtype; LAUNCH on a failed launch. */
size_t wall_attn_decode_workspace_size(int64_t B, int64_t T, int64_t HQ, int64_t V);

wall_status_t wall_attn_decode(const void *q, const void *v, wall_dtype_t dtype,
                               const float *p_curr, int64_t p_curr_batch_stride,
                               const void *k_tilde, const float *r_cache,
                               const float *sink_bias, void *o, float *lse,
                               int64_t B, int64_t T, int64_t T_cap, int64_t HQ, int64_t H,
                               int64_t K, int64_t V, int64_t chunk_size, float scale,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------ decode without allocation
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode step as wall_attn_decode, same arguments without the workspace,
 * same kernels and results bit for bit.  The split partials live in a fixed
 * device array of the library, WALL_DECODE_SCRATCH_BYTES per GPU, that each
 * GPU the library runs on holds until the process ends; its address is
 * taken once per device (the device current at the call, which must own
 * `stream`).  Nothing is allocated and nothing needs clearing: every call
 * writes the partials it reads.  Calls that overlap on one GPU (other
 * streams, other threads) share that array and race: order them.
 * Errors: those of wall_attn_decode (other than the workspace's);
 * WALL_ERR_SCRATCH when wall_attn_decode_workspace_size(B, T, HQ, V) would
 * exceed WALL_DECODE_SCRATCH_BYTES (about B * HQ <= 6000 at V = 128);
 * UNSUPPORTED for a device index of 64 or more; LAUNCH when the array's
 * address cannot be taken or a launch fails. */
#define WALL_DECODE_SCRATCH_BYTES ((size_t)4 << 20)

wall_status_t wall_attn_decode_noalloc(const void *q, const void *v, wall_dtype_t dtype,
                                       const float *p_curr, int64_t p_curr_batch_stride,
                                       const void *k_tilde, const float *r_cache,
                                       const float *sink_bias, void *o, float *lse,
                                       int64_t B, int64_t T, int64_t T_cap, int64_t HQ, int64_t H,
                                       int64_t K, int64_t V, int64_t chunk_size, float scale,
                                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WALL_H */
