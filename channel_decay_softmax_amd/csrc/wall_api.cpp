// wall_api.cpp -- the extern "C" boundary of the Wall Attention library (forward and decode).
//
// Every argument check below runs before the first HIP call, so invalid
// calls return their status without touching the device (and can be tested
// on a machine without a GPU).  The entry points then enqueue kernels on the
// caller's stream and return; nothing is allocated or synchronised here.
//
// WALL_DEBUG (environment variable, read once per process): when set to a
// value other than "0", every refused call prints its entry point, the
// source line of the check it failed and the status to stderr, and every
// launch is followed by a device synchronisation, so that a kernel fault is
// reported by the call that launched it (the only place the library then
// synchronises).
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "wall.h"

#include "wall_common.h"
#include "wall_entry.h"
#include "wall_stream.h"

using namespace wall;

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool debug_on() {
    static const bool on = [] {
        const char *e = std::getenv("WALL_DEBUG");
        return e != nullptr && *e != '\0' && std::strcmp(e, "0") != 0;
    }();
    return on;
}

}  // namespace

namespace wall {

// A refused call: its status, reported under WALL_DEBUG with the function and
// line of the failed check.
wall_status_t fail(const char *fn, int line, wall_status_t s) {
    if (debug_on()) std::fprintf(stderr, "wall: %s refused the call: %s (wall_api.cpp:%d)\n", fn,
                                 wall_status_string(s), line);
    return s;
}

}  // namespace wall

namespace {

wall_status_t launched(hipError_t e) {
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess && debug_on()) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        if (debug_on()) std::fprintf(stderr, "wall: launch failed: %s\n", hipGetErrorString(e));
        return WALL_ERR_LAUNCH;
    }
    return WALL_OK;
}

int64_t esize_of(wall_dtype_t d) { return d == WALL_BF16 ? 2 : (d == WALL_F32 ? 4 : 0); }

}  // namespace

namespace wall {

wall_status_t decode_check(const void *q, const void *v, wall_dtype_t dtype, const float *p_curr,
                           int64_t p_curr_batch_stride, const void *k_tilde, const float *r_cache,
                           const float *sink_bias, const void *o, const float *lse, int64_t B, int64_t T,
                           int64_t T_cap, int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size) {
    if (!q || !v || !p_curr || !k_tilde || !r_cache || !o) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B < 1 || T < 1 || T_cap < 1 || HQ < 1 || H < 1 || K < 1 || V < 1 || chunk_size < 1)
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (HQ % H != 0 || T > T_cap || B * HQ > 65535) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (p_curr_batch_stride != 0 && (p_curr_batch_stride < HQ * K || p_curr_batch_stride % 4 != 0))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B * T_cap > INT32_MAX / 2 || B * T_cap * HQ * (K > V ? K : V) > ((int64_t)1 << 40))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (dtype != WALL_BF16 && dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if ((K != 64 && K != 128) || (V != 64 && V != 128) || chunk_size % 64 != 0) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    const void *ptrs[] = {q, v, p_curr, k_tilde, r_cache, sink_bias, o, lse};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return WALL_OK;
}

wall_status_t decode_launch(const void *q, const void *v, wall_dtype_t dtype, const float *p_curr,
                            int64_t p_curr_batch_stride, const void *k_tilde, const float *r_cache,
                            const float *sink_bias, void *o, float *lse, int64_t B, int64_t T, int64_t T_cap,
                            int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size, float scale,
                            float *part, hipStream_t stream) {
    const DecodeLayout L = decode_layout(B, T, HQ, V);
    DecodeArgs a{};
    a.q = q;
    a.v = v;
    a.pc = p_curr;
    a.pc_bs = p_curr_batch_stride ? p_curr_batch_stride : HQ * K;
    a.kt = k_tilde;
    a.r = r_cache;
    a.sink = sink_bias;
    a.o = o;
    a.lse = lse;
    a.part = part;
    a.B = (int32_t)B;
    a.T = (int32_t)T;
    a.Tcap = (int32_t)T_cap;
    a.HQ = (int32_t)HQ;
    a.H = (int32_t)H;
    a.K = (int32_t)K;
    a.V = (int32_t)V;
    a.C = (int32_t)chunk_size;
    a.nsplit = (int32_t)L.nsplit;
    a.S = (int32_t)L.S;
    // the query heads of one kv head share a block (the largest divisor of HQ/H up to 4)
    a.nwg = 1;
    for (int32_t d = 4; d >= 1; --d)
        if ((HQ / H) % d == 0) {
            a.nwg = d;
            break;
        }
    a.qscale = scale * LOG2E;
    return launched(launch_decode(a, dtype == WALL_BF16, stream));
}

}  // namespace wall

extern "C" {

const char *wall_status_string(int s) {
    switch (s) {
        case WALL_OK: return "WALL_OK";
        case WALL_ERR_INVALID_ARG: return "WALL_ERR_INVALID_ARG";
        case WALL_ERR_UNSUPPORTED: return "WALL_ERR_UNSUPPORTED";
        case WALL_ERR_LAUNCH: return "WALL_ERR_LAUNCH";
        case WALL_ERR_SCRATCH: return "WALL_ERR_SCRATCH";
    }
    return "WALL_ERR_UNKNOWN";
}

int wall_version(void) { return 100; }  // 0.1.0

size_t wall_prefix_scan_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 1 || T < 1 || C < 1) return 0;
    return scan_layout(B, T, C).total;
}

wall_status_t wall_prefix_scan(const void *x, wall_dtype_t x_dtype, float *out, int64_t B,
                               int64_t T, int64_t C, const int32_t *cu_seqlens, int64_t num_seqs,
                               float scale, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!x || !out || !workspace) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B < 1 || T < 1 || C < 1) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B * T > INT32_MAX || B * T * C > (int64_t)1 << 40) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (cu_seqlens && (B != 1 || num_seqs < 1 || num_seqs > T)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (x_dtype != WALL_BF16 && x_dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 256) ||
        (cu_seqlens && !aligned(cu_seqlens, 4)))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (workspace_bytes < scan_layout(B, T, C).total) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if ((const void *)out == x) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return launched(launch_scan(x, x_dtype == WALL_BF16, out, B, T, C,
                                cu_seqlens, cu_seqlens ? num_seqs : 0, scale, workspace, stream));
}

wall_status_t wall_prefix_append(const void *x, wall_dtype_t x_dtype, int64_t x_batch_stride,
                                 const float *prev, int64_t prev_batch_stride, float *out,
                                 int64_t out_batch_stride, int64_t B, int64_t n, int64_t C, float scale,
                                 hipStream_t stream) {
    if (!x || !out) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B < 1 || n < 1 || C < 1 || B * n * C > (int64_t)1 << 40) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (x_batch_stride < n * C || out_batch_stride < n * C || (prev && prev_batch_stride < C))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (x_dtype != WALL_BF16 && x_dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if (!aligned(x, x_dtype == WALL_BF16 ? 2 : 4) || !aligned(out, 4) || (prev && !aligned(prev, 4)))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    // out may not overlap x; it may start right after prev (a running buffer)
    const char *o0 = reinterpret_cast<const char *>(out);
    const char *o1 = o0 + sizeof(float) * ((B - 1) * out_batch_stride + n * C);
    const char *x0 = static_cast<const char *>(x);
    const char *x1 = x0 + esize_of(x_dtype) * ((B - 1) * x_batch_stride + n * C);
    if (o0 < x1 && x0 < o1) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return launched(launch_prefix_append(x, x_dtype == WALL_BF16, x_batch_stride, prev, prev_batch_stride, out,
                                         out_batch_stride, B, n, C, scale, stream));
}

size_t wall_attn_fwd_workspace_size(wall_dtype_t dtype, int64_t B, int64_t T, int64_t HQ,
                                    int64_t H, int64_t K, int64_t V, int64_t num_seqs) {
    const int64_t es = esize_of(dtype);
    if (!es || B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1) return 0;
    return fwd_layout(es, B, T, HQ, H, K, V, num_seqs).total;
}

namespace {

struct FwdShape {
    int64_t B, T, HQ, H, K, V, nseq, maxlen;
};

// Checks shared by the forward entry points; returns WALL_OK or the status to report.
wall_status_t check_fwd(wall_dtype_t dtype, const FwdShape &s, const int32_t *cu,
                        int64_t num_seqs, int64_t max_seqlen, const void *workspace,
                        size_t workspace_bytes) {
    if (!workspace) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (s.B < 1 || s.T < 1 || s.HQ < 1 || s.H < 1 || s.K < 1 || s.V < 1) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (s.HQ % s.H != 0) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (s.B * s.T > INT32_MAX / 2 || s.B * s.T * s.HQ * (s.K > s.V ? s.K : s.V) > ((int64_t)1 << 40))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (cu && (s.B != 1 || num_seqs < 1 || num_seqs > s.T || max_seqlen < 1 || max_seqlen > s.T))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (dtype != WALL_BF16 && dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if ((s.K != 64 && s.K != 128) || (s.V != 64 && s.V != 128)) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if (cu && !aligned(cu, 4)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (!aligned(workspace, 256)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const FwdLayout L = fwd_layout(esize_of(dtype), s.B, s.T, s.HQ, s.H, s.K, s.V, cu ? num_seqs : 0);
    if (workspace_bytes < L.total) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return WALL_OK;
}

wall_status_t enqueue_prepare(const void *q, const void *k, const void *v, wall_dtype_t dtype, const float *P,
                              float scale, const FwdShape &s, const int32_t *cu, void *workspace,
                              hipStream_t stream) {
    const FwdLayout L = fwd_layout(esize_of(dtype), s.B, s.T, s.HQ, s.H, s.K, s.V, s.nseq);
    char *ws = static_cast<char *>(workspace);
    SegInfo *seg = reinterpret_cast<SegInfo *>(ws + L.off_seg);
    PrepArgs pa{q, k, v, P, seg, cu, reinterpret_cast<float *>(ws + L.off_anchor),
                reinterpret_cast<uint32_t *>(ws + L.off_rec), ws + L.off_kt, ws + L.off_vt, ws + L.off_kd,
                ws + L.off_qd, reinterpret_cast<uint32_t *>(ws + L.off_drec), scale * LOG2E,
                L.nseg, L.tiles, s.HQ, s.H, s.K, s.V, s.T};
    pa.vsum = reinterpret_cast<float *>(ws + L.off_vsum);
    pa.kcm = reinterpret_cast<float *>(ws + L.off_kcm);
    return launched(launch_prep(pa, dtype == WALL_BF16, stream));
}

wall_status_t enqueue_run(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                          const float *P, const float *G, const float *sink_bias, void *o, float *lse,
                          const FwdShape &s, float scale, int64_t window_size, const void *workspace,
                          hipStream_t stream) {
    const FwdLayout L = fwd_layout(esize_of(dtype), s.B, s.T, s.HQ, s.H, s.K, s.V, s.nseq);
    const char *ws = static_cast<const char *>(workspace);
    FwdArgs fa{};
    fa.q = q;
    fa.k = k;
    fa.v = v;
    fa.P = P;
    fa.G = G;
    fa.sink = sink_bias;
    fa.kt = ws + L.off_kt;
    fa.vt = ws + L.off_vt;
    fa.kd = ws + L.off_kd;
    fa.qd = ws + L.off_qd;
    fa.drec = reinterpret_cast<const uint32_t *>(ws + L.off_drec);
    fa.anchor = reinterpret_cast<const float *>(ws + L.off_anchor);
    fa.rec = reinterpret_cast<const uint32_t *>(ws + L.off_rec);
    fa.vsum = reinterpret_cast<const float *>(ws + L.off_vsum);
    fa.kcm = reinterpret_cast<const float *>(ws + L.off_kcm);
    fa.seg = reinterpret_cast<const SegInfo *>(ws + L.off_seg);
    fa.o = o;
    fa.lse = lse;
    fa.nseg = (int32_t)L.nseg;
    fa.max_tiles = (int32_t)cdiv(s.maxlen, TILE);
    fa.HQ = (int32_t)s.HQ;
    fa.H = (int32_t)s.H;
    fa.K = (int32_t)s.K;
    fa.V = (int32_t)s.V;
    fa.window = window_size > 0 ? (int32_t)(window_size > s.T ? s.T : window_size) : 0;
    fa.qscale = scale * LOG2E;
    return launched(dtype == WALL_BF16 ? launch_fwd_bf16(fa, stream) : launch_fwd_f32(fa, stream));
}

}  // namespace

wall_status_t wall_attn_fwd_prepare(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                                    const float *P, int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                                    int64_t V, float scale, const int32_t *cu_seqlens, int64_t num_seqs,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !P) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const FwdShape s{B, T, HQ, H, K, V, cu_seqlens ? num_seqs : 0, T};
    // max_seqlen plays no part in the preparation: pass T to the shared checks
    const wall_status_t st = check_fwd(dtype, s, cu_seqlens, num_seqs, T, workspace, workspace_bytes);
    if (st != WALL_OK) return st;
    const void *ptrs[] = {q, k, v, P};
    for (const void *p : ptrs)
        if (!aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return enqueue_prepare(q, k, v, dtype, P, scale, s, cu_seqlens, workspace, stream);
}

wall_status_t wall_attn_fwd_prepare_gate(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                                         const void *g, wall_dtype_t g_dtype, float *P, int64_t B, int64_t T,
                                         int64_t HQ, int64_t H, int64_t K, int64_t V, float scale,
                                         const int32_t *cu_seqlens, int64_t num_seqs, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !g || !P) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const FwdShape s{B, T, HQ, H, K, V, cu_seqlens ? num_seqs : 0, T};
    const wall_status_t st = check_fwd(dtype, s, cu_seqlens, num_seqs, T, workspace, workspace_bytes);
    if (st != WALL_OK) return st;
    if (g_dtype != WALL_BF16 && g_dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    const void *ptrs[] = {q, k, v, g, P};
    for (const void *p : ptrs)
        if (!aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (static_cast<const void *>(P) == g) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const FwdLayout L = fwd_layout(esize_of(dtype), B, T, HQ, H, K, V, s.nseq);
    char *ws = static_cast<char *>(workspace);
    void *sws = ws + L.off_scan;
    const float pscale = 1.4426950408889634f;  // 1 / ln 2: P in log2 units
    // one pass for B sequences of T rows (T a multiple of the tile) with bf16 inputs
    if (!cu_seqlens && dtype == WALL_BF16 && g_dtype == WALL_BF16 && T % TILE == 0 && (HQ * K) % 8 == 0) {
        wall_status_t sc = launched(launch_scan_chunk_sums(g, true, B, T, HQ * K, sws, stream));
        if (sc != WALL_OK) return sc;
        const ScanLayout SL = scan_layout(B, T, HQ * K);
        PrepArgs pa{q, k, v, P, reinterpret_cast<SegInfo *>(ws + L.off_seg), nullptr,
                    reinterpret_cast<float *>(ws + L.off_anchor), reinterpret_cast<uint32_t *>(ws + L.off_rec),
                    ws + L.off_kt, ws + L.off_vt, ws + L.off_kd, ws + L.off_qd,
                    reinterpret_cast<uint32_t *>(ws + L.off_drec), scale * LOG2E, L.nseg, L.tiles, HQ, H, K, V, T};
        pa.g = g;
        pa.Pw = P;
        pa.vsum = reinterpret_cast<float *>(ws + L.off_vsum);
        pa.kcm = reinterpret_cast<float *>(ws + L.off_kcm);
        pa.csum = reinterpret_cast<const float *>(static_cast<const char *>(sws) + SL.off_sum);
        pa.pscale = pscale;
        return launched(launch_scan_prep(pa, stream));
    }
    // otherwise the scan, then the preparation
    wall_status_t sc = launched(launch_scan(g, g_dtype == WALL_BF16, P, B, T, HQ * K, cu_seqlens,
                                            cu_seqlens ? num_seqs : 0, pscale, sws, stream));
    if (sc != WALL_OK) return sc;
    return enqueue_prepare(q, k, v, dtype, P, scale, s, cu_seqlens, workspace, stream);
}

wall_status_t wall_attn_fwd_run(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                                const float *P, const float *G, const float *sink_bias, void *o, float *lse,
                                int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                                float scale, int64_t window_size, const int32_t *cu_seqlens,
                                int64_t num_seqs, int64_t max_seqlen, const void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !P || !o) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const FwdShape s{B, T, HQ, H, K, V, cu_seqlens ? num_seqs : 0, cu_seqlens ? max_seqlen : T};
    const wall_status_t st =
        check_fwd(dtype, s, cu_seqlens, num_seqs, max_seqlen, workspace, workspace_bytes);
    if (st != WALL_OK) return st;
    const void *ptrs[] = {q, k, v, P, o, G, sink_bias, lse};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return enqueue_run(q, k, v, dtype, P, G, sink_bias, o, lse, s, scale, window_size, workspace, stream);
}

wall_status_t wall_attn_fwd(const void *q, const void *k, const void *v, wall_dtype_t dtype,
                            const float *P, const float *G, const float *sink_bias, void *o,
                            float *lse, int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                            int64_t V, float scale, int64_t window_size,
                            const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !P || !o) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const FwdShape s{B, T, HQ, H, K, V, cu_seqlens ? num_seqs : 0, cu_seqlens ? max_seqlen : T};
    const wall_status_t st =
        check_fwd(dtype, s, cu_seqlens, num_seqs, max_seqlen, workspace, workspace_bytes);
    if (st != WALL_OK) return st;
    const void *ptrs[] = {q, k, v, P, o, G, sink_bias, lse};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const wall_status_t sp = enqueue_prepare(q, k, v, dtype, P, scale, s, cu_seqlens, workspace, stream);
    if (sp != WALL_OK) return sp;
    return enqueue_run(q, k, v, dtype, P, G, sink_bias, o, lse, s, scale, window_size, workspace, stream);
}

size_t wall_attn_bwd_workspace_size(int64_t B, int64_t T, int64_t HQ, int64_t K, int64_t num_seqs) {
    if (B < 1 || T < 1 || HQ < 1 || K < 1) return 0;
    return bwd_layout(B, T, HQ, K, num_seqs > 0 ? num_seqs : B).total;
}

wall_status_t wall_attn_bwd(const void *q, const void *k, const void *v, wall_dtype_t dtype, const float *P,
                            const float *G, const float *sink_bias, const void *o, const float *lse,
                            const void *dout, void *dq, void *dk, void *dv, void *dg, void *dg_scalar,
                            wall_dtype_t g_dtype, float *dsink, int64_t B, int64_t T, int64_t HQ, int64_t H,
                            int64_t K, int64_t V, float scale, int64_t window_size, const int32_t *cu_seqlens,
                            int64_t num_seqs, int64_t max_seqlen, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    if (!q || !k || !v || !P || !o || !lse || !dout || !dq || !dk || !dv || !dg || !workspace)
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (G && !dg_scalar) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (sink_bias && !dsink) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (HQ % H != 0) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B * T > INT32_MAX / 2 || B * T * HQ * (K > V ? K : V) > ((int64_t)1 << 40)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (cu_seqlens && (B != 1 || num_seqs < 1 || num_seqs > T || max_seqlen < 1 || max_seqlen > T))
        return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (dtype != WALL_BF16 && dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if (g_dtype != WALL_BF16 && g_dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if ((K != 64 && K != 128) || (V != 64 && V != 128)) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    const void *ptrs[] = {q, k, v, P, G, sink_bias, o, lse, dout, dq, dk, dv, dg, dg_scalar, dsink, cu_seqlens};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (!aligned(workspace, 256)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const int64_t nseg = cu_seqlens ? num_seqs : B;
    // the backward launches one block per (query head, sequence, 128-row block of the longest sequence)
    if (HQ * nseg * cdiv(cu_seqlens ? max_seqlen : T, TILE) > INT32_MAX) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    const BwdLayout L = bwd_layout(B, T, HQ, K, nseg);
    if (workspace_bytes < L.total) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    char *ws = static_cast<char *>(workspace);
    SegInfo *seg = reinterpret_cast<SegInfo *>(ws + L.off_seg);
    wall_status_t st = launched(launch_bwd_seg(seg, cu_seqlens, nseg, T, stream));
    if (st != WALL_OK) return st;
    BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.P = P;
    a.G = G;
    a.sink = sink_bias;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dsink = sink_bias ? dsink : nullptr;
    a.D = reinterpret_cast<float *>(ws + L.off_D);
    a.X = reinterpret_cast<float *>(ws + L.off_X);
    a.Y = reinterpret_cast<float *>(ws + L.off_Y);
    a.Z = reinterpret_cast<float *>(ws + L.off_Z);
    a.dkp = reinterpret_cast<float *>(ws + L.off_part);
    a.dvp = a.dkp + B * T * HQ * K;
    a.dqd = reinterpret_cast<float *>(ws + L.off_dqd);
    a.qh = ws + L.off_qh;
    a.kh = ws + L.off_kh;
    a.Ab = reinterpret_cast<float *>(ws + L.off_rt);
    a.flag = reinterpret_cast<int32_t *>(ws + L.off_flag);
    a.bmax = reinterpret_cast<uint32_t *>(ws + L.off_bmax);
    a.cmax = reinterpret_cast<uint16_t *>(ws + L.off_cmax);
    a.wsum = reinterpret_cast<float *>(ws + L.off_wsum);
    a.seg = seg;
    a.nseg = (int32_t)nseg;
    a.max_seqlen = (int32_t)(cu_seqlens ? max_seqlen : T);
    a.rows = (int32_t)(B * T);
    a.HQ = (int32_t)HQ;
    a.H = (int32_t)H;
    a.K = (int32_t)K;
    a.V = (int32_t)V;
    a.window = window_size > 0 ? (int32_t)(window_size > T ? T : window_size) : 0;
    a.scale = scale;
    a.qscale = scale * LOG2E;
    st = launched(launch_bwd(a, dtype == WALL_BF16, stream));
    if (st != WALL_OK) return st;
    // dg = -(exclusive prefix of X), dg_scalar = -(exclusive prefix of Y), per sequence
    void *sws = ws + L.off_scan;
    const int64_t ns = cu_seqlens ? num_seqs : 0;
    st = launched(launch_scan_excl(a.X, dg, g_dtype == WALL_BF16, B, T, HQ * K, cu_seqlens, ns, -1.0f, sws,
                                   stream));
    if (st != WALL_OK || !G) return st;
    return launched(launch_scan_excl(a.Y, dg_scalar, g_dtype == WALL_BF16, B, T, HQ, cu_seqlens, ns, -1.0f, sws,
                                     stream));
}

wall_status_t wall_kv_cache_build(const void *k, wall_dtype_t dtype, const float *P, void *k_tilde,
                                  float *r_cache, int64_t B, int64_t T_cap, int64_t HQ, int64_t H,
                                  int64_t K, int64_t chunk_size, int64_t t0, int64_t t1,
                                  hipStream_t stream) {
    if (!k || !P || !k_tilde || !r_cache) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B < 1 || T_cap < 1 || HQ < 1 || H < 1 || K < 1 || chunk_size < 1) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (HQ % H != 0) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (t0 < 0 || t1 <= t0 || t1 > T_cap) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B * T_cap > INT32_MAX / 2 || B * T_cap * HQ * K > ((int64_t)1 << 40)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (dtype != WALL_BF16 && dtype != WALL_F32) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if ((K != 64 && K != 128) || chunk_size % 64 != 0) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    const void *ptrs[] = {k, P, k_tilde, r_cache};
    for (const void *p : ptrs)
        if (!aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const CacheArgs a{k, P, k_tilde, r_cache, B, T_cap, HQ, H, K, chunk_size, t0, t1};
    return launched(launch_kv_cache(a, dtype == WALL_BF16, stream));
}

wall_status_t wall_stream_append(const void *g, wall_dtype_t g_dtype, const void *k, wall_dtype_t dtype,
                                 float *P, void *k_tilde, float *r_cache, int64_t B, int64_t T_cap,
                                 int64_t HQ, int64_t H, int64_t K, int64_t chunk_size, int64_t t0,
                                 int64_t t1, float scale, hipStream_t stream) {
    if (!g || !k || !P || !k_tilde || !r_cache) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B < 1 || T_cap < 1 || HQ < 1 || H < 1 || K < 1 || chunk_size < 1) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (HQ % H != 0) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (t0 < 0 || t1 <= t0 || t1 > T_cap) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (B * T_cap > INT32_MAX / 2 || B * T_cap * HQ * K > ((int64_t)1 << 40)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if ((dtype != WALL_BF16 && dtype != WALL_F32) || (g_dtype != WALL_BF16 && g_dtype != WALL_F32))
        return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    if ((K != 64 && K != 128) || chunk_size % 64 != 0) return fail(__func__, __LINE__, WALL_ERR_UNSUPPORTED);
    const void *ptrs[] = {g, k, P, k_tilde, r_cache};
    for (const void *p : ptrs)
        if (!aligned(p, 16)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const StreamArgs a{g, k, P, k_tilde, r_cache, B, T_cap, HQ, H, K, chunk_size, t0, t1, scale};
    return launched(launch_stream_append(a, g_dtype == WALL_BF16, dtype == WALL_BF16, stream));
}

size_t wall_attn_decode_workspace_size(int64_t B, int64_t T, int64_t HQ, int64_t V) {
    if (B < 1 || T < 1 || HQ < 1 || V < 1) return 0;
    return decode_layout(B, T, HQ, V).total;
}

wall_status_t wall_attn_decode(const void *q, const void *v, wall_dtype_t dtype, const float *p_curr,
                               int64_t p_curr_batch_stride, const void *k_tilde, const float *r_cache, const float *sink_bias,
                               void *o, float *lse, int64_t B, int64_t T, int64_t T_cap, int64_t HQ,
                               int64_t H, int64_t K, int64_t V, int64_t chunk_size, float scale,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!workspace) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    const wall_status_t st = wall::decode_check(q, v, dtype, p_curr, p_curr_batch_stride, k_tilde, r_cache,
                                                sink_bias, o, lse, B, T, T_cap, HQ, H, K, V, chunk_size);
    if (st != WALL_OK) return st;
    if (!aligned(workspace, 256)) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    if (workspace_bytes < wall::decode_layout(B, T, HQ, V).total) return fail(__func__, __LINE__, WALL_ERR_INVALID_ARG);
    return wall::decode_launch(q, v, dtype, p_curr, p_curr_batch_stride, k_tilde, r_cache, sink_bias, o, lse, B, T,
                               T_cap, HQ, H, K, V, chunk_size, scale, static_cast<float *>(workspace), stream);
}

}  // extern "C"
