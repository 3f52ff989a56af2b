// wall_bwd.hip -- backward of the causal Wall Attention forward (the README's
// "exact analytic gradients" for q, k, v, g and g_scalar, and the sink).
//
// With the natural-log logits s_ij = scale * sum_n q_in k_jn 2^(P_in - P_jn)
// + (Gs_i - Gs_j), A_ij = exp(s_ij - lse_i) and D_i = do_i . o_i:
//     dS_ij = A_ij (do_i . v_j - D_i)
//     dv_j  = sum_i A_ij do_i,   dq_in = scale sum_j dS_ij k_jn 2^(P_in - P_jn),
//     dk_jn = scale sum_i dS_ij q_in 2^(P_in - P_jn)       (summed over query heads)
//     dsink = -sum_i exp(sink - lse_i) D_i
// The decay 2^(P_i - P_j) depends on the gate g_u for j < u <= i, which gives
// (blog, "Definition: Wall Attention", product form; differentiated here)
//     dg_u = sum_{t >= u} X_t,   X_t = q_t (.) dq_t - k_t (.) dk_t^(hq)
// (dk^(hq): the query head's own part of dk), and dg_scalar_u = sum_{t >= u}
// Y_t with Y_t = sum_j dS_tj - sum_i dS_it.  Over one sequence X and Y sum to
// zero (adding a constant to a sequence's P, or its running g_scalar sum,
// changes no logit), so the suffix sums equal minus the exclusive prefix
// sums, which the prefix scan computes.
//
// bwd_pre_kernel and dsink_kernel serve both input dtypes; bf16 inputs take
// the matrix-core kernels of wall_bwd_mfma.hip for the rest.  For float32
// inputs the kernels below run everything in float32 on the vector ALUs:
//   bwd_pre_kernel   D_i
//   (wall_bwd_diag.hip) the pairs inside every 32-row block, pair by pair:
//                    dq, dk and dv parts, X and Y of those pairs
//   bwd_dq_kernel    one block per (query head, sequence, 64 query rows): keys
//                    staged 32 at a time in LDS; adds dq, q (.) dq, the row
//                    sums of dS and writes the sink terms
//   bwd_dkdv_kernel  one block per (kv head, sequence, 64 keys), looping over
//                    the kv head's query heads and over the visible queries 32
//                    at a time; writes dk, dv and subtracts k (.) dk^(hq) and
//                    the column sums of dS from X and Y (it runs after the dq
//                    kernel on the same stream)
//   dsink_kernel     the sink sums
// and the exclusive prefix scans of X and Y give dg and dg_scalar.
//
// Anchors (the anchor identity of the Wall Attention blog, "Fast training
// and inference"): every pair of rows in different 32-row blocks is read at
// R = floor(P) of a row between them -- the row before the query block (dq
// kernel) or the key block's last row (dk/dv kernel) for rows of other
// 64-row blocks, the last row of the first half for the pairs across the two
// halves -- so for a prefix that falls both factors 2^(P_i - R) and
// 2^(R - P_j) are at most 2 at any gate strength.  The accumulators move from
// one anchor to the next by exact powers of two.
#include <float.h>

#include <type_traits>

#include "wall_common.h"

namespace wall {
namespace {

constexpr int BB = 64;  // rows per block (queries in dq, keys in dk/dv)
constexpr int BS = 32;  // rows per LDS stage
constexpr int NT = 256;

template <typename T>
__device__ inline float ld(const T *p) { return (float)*p; }
template <typename T>
__device__ inline void st(T *p, float x) { *p = (T)x; }

__device__ inline float clamp2(float e) { return exp2f(fminf(fmaxf(e, EXP2_LO), EXP2_HI)); }

// ---------------------------------------------------------------- sequence table
// One block of 256: per sequence its start, length and the index of its
// first 128-row tile (an inclusive scan of the tile counts, 256 at a time).
__global__ void bwd_seg_kernel(SegInfo *seg, const int32_t *cu, int nseg, int T) {
    __shared__ int part[256];
    const int tid = threadIdx.x;
    int base = 0;
    for (int s0 = 0; s0 < nseg; s0 += 256) {
        const int s = s0 + tid;
        int start = 0, len = 0;
        if (s < nseg) {
            start = cu ? cu[s] : s * T;
            len = cu ? cu[s + 1] - cu[s] : T;
        }
        const int cnt = (len + TILE - 1) / TILE;
        part[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int v = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += v;
            __syncthreads();
        }
        if (s < nseg) seg[s] = SegInfo{start, len, base + part[tid] - cnt, 0};
        base += part[255];
        __syncthreads();
    }
}

// ---------------------------------------------------------------- D = do . o
template <typename T, int V>
__global__ __launch_bounds__(NT) void bwd_pre_kernel(BwdArgs a, int64_t nrows) {
    // one row (token, head) per 16 lanes: V/16 consecutive channels each, so
    // each lane's share is one or two 16-byte loads per operand
    constexpr int VL = V / 16;
    const int64_t r = (int64_t)blockIdx.x * (NT / 16) + threadIdx.x / 16;
    const int l = threadIdx.x % 16;
    float acc = 0.f;
    if (r < nrows) {
        const T *o = static_cast<const T *>(a.o) + r * V + l * VL;
        const T *d = static_cast<const T *>(a.dout) + r * V + l * VL;
        T ov[VL], dv[VL];
#pragma unroll
        for (int c = 0; c < VL; ++c) {
            ov[c] = o[c];
            dv[c] = d[c];
        }
#pragma unroll
        for (int c = 0; c < VL; ++c) acc = fmaf((float)ov[c], (float)dv[c], acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (r < nrows && l == 0) a.D[r] = acc;
}

// ---------------------------------------------------------------- dq
// One block per (query head, sequence, 64 query rows: halves h0 and h1).  The
// keys before the block are read against A0 = floor(P) of the row before it;
// then the keys of h0 against A1 = floor(P) of h0's last row for the queries
// of h1, with the h1 accumulators moved from A0 to A1 (an exact power of two,
// at most 1).  The pairs inside h0 and inside h1 come from the pair-by-pair
// kernel (dqd, X, Y), which runs first.
template <typename T, int K, int V>
__global__ __launch_bounds__(NT) void bwd_dq_kernel(BwdArgs a, int nblk) {
    constexpr int QP = K + 1, VP = V + 1, SP = BS + 1, KQ = K / 4;
    extern __shared__ float smem[];
    float *sQ = smem;                 // [BB][QP] q * scale*log2e * 2^(P - anchor)
    float *sDO = sQ + BB * QP;        // [BB][VP]
    float *sK = sDO + BB * VP;        // [BS][QP] k * 2^(anchor - P)
    float *sV = sK + BS * QP;         // [BS][VP]
    float *sDS = sV + BS * VP;        // [BB][SP]
    float *sG = sDS + BB * SP;        // [BS] -G_j (log2 units)
    float *sA0 = sG + BS;             // [K] A0
    float *sA1 = sA0 + K;             // [K] A1

    const int bid = blockIdx.x;
    const int hq = bid / (a.nseg * nblk);
    const int rem = bid % (a.nseg * nblk);
    const SegInfo sg = a.seg[rem / nblk];
    const int qb = rem % nblk;
    if (qb * BB >= sg.len) return;
    const int tid = threadIdx.x, qi = tid / 4, sub = tid % 4;
    const int64_t HQ = a.HQ;
    const int h = hq / (a.HQ / a.H);
    const int i0 = qb * BB;
    const bool has_h1 = i0 + BS < sg.len;
    const T *qg = static_cast<const T *>(a.q);
    const T *kg = static_cast<const T *>(a.k);
    const T *vg = static_cast<const T *>(a.v);
    const T *dog = static_cast<const T *>(a.dout);
    const float *Pg = a.P + hq * K;

    if (tid < K) {
        sA0[tid] = i0 > 0 ? floorf(Pg[((int64_t)sg.start + i0 - 1) * HQ * K + tid]) : 0.f;
        sA1[tid] = has_h1 ? floorf(Pg[((int64_t)sg.start + i0 + BS - 1) * HQ * K + tid]) : 0.f;
    }
    __syncthreads();
    // q of rows first .. BB-1 of the block at anchor R
    auto stage_q = [&](int first, const float *R) {
        for (int x = tid; x < (BB - first) * K; x += NT) {
            const int r = first + x / K, n = x % K, row = i0 + r;
            float val = 0.f;
            if (row < sg.len) {
                const int64_t t = (int64_t)sg.start + row;
                val = ld(qg + (t * HQ + hq) * K + n) * a.qscale * clamp2(Pg[t * HQ * K + n] - R[n]);
            }
            sQ[r * QP + n] = val;
        }
    };
    stage_q(0, sA0);
    for (int x = tid; x < BB * V; x += NT) {
        const int r = x / V, c = x % V, row = i0 + r;
        sDO[r * VP + c] = row < sg.len ? ld(dog + (((int64_t)sg.start + row) * HQ + hq) * V + c) : 0.f;
    }
    const int qrow = i0 + qi;
    const bool qvalid = qrow < sg.len;
    const int64_t qt = (int64_t)sg.start + (qvalid ? qrow : 0);
    const float lse2 = qvalid ? a.lse[qt * HQ + hq] * LOG2E : 0.f;
    const float Di = qvalid ? a.D[qt * HQ + hq] : 0.f;
    const float gi = (a.G && qvalid) ? a.G[qt * HQ + hq] : 0.f;

    float acc[KQ];
#pragma unroll
    for (int n = 0; n < KQ; ++n) acc[n] = 0.f;
    float grow = 0.f;
    int lo = 0;
    if (a.window > 0) lo = max(0, i0 - a.window + 1);
    // stages: the keys before the block, then (for h1) the keys of h0
    const int nst_off = i0 > lo / BS * BS ? (i0 - lo / BS * BS) / BS : 0;
    const int nst = nst_off + (has_h1 ? 1 : 0);
    for (int st_i = 0; st_i < nst; ++st_i) {
        const bool own = st_i == nst_off;
        const int key0 = own ? i0 : lo / BS * BS + BS * st_i;
        const float *R = own ? sA1 : sA0;
        __syncthreads();
        if (own) {
            stage_q(BS, sA1);
            if (qi >= BS) {
#pragma unroll
                for (int n = 0; n < KQ; ++n) {
                    const int ch = sub * KQ + n;
                    acc[n] *= exp2f(sA1[ch] - sA0[ch]);
                }
            }
        }
        for (int x = tid; x < BS * K; x += NT) {
            const int r = x / K, n = x % K, j = key0 + r;
            float val = 0.f;
            if (j < sg.len) {
                const int64_t t = (int64_t)sg.start + j;
                val = ld(kg + (t * a.H + h) * K + n) * clamp2(R[n] - Pg[t * HQ * K + n]);
            }
            sK[r * QP + n] = val;
        }
        for (int x = tid; x < BS * V; x += NT) {
            const int r = x / V, c = x % V, j = key0 + r;
            sV[r * VP + c] = j < sg.len ? ld(vg + (((int64_t)sg.start + j) * a.H + h) * V + c) : 0.f;
        }
        if (tid < BS) {
            const int j = key0 + tid;
            sG[tid] = (a.G && j < sg.len) ? -a.G[((int64_t)sg.start + j) * HQ + hq] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < BS / 4; ++kk) {
            const int kr = sub * (BS / 4) + kk, key = key0 + kr;
            bool vis = qvalid && key <= qrow && key < sg.len && (!own || qi >= BS);
            if (a.window > 0) vis = vis && qrow - key < a.window;
            float dS = 0.f;
            if (vis) {
                float dot = 0.f;
                for (int n = 0; n < K; ++n) dot = fmaf(sQ[qi * QP + n], sK[kr * QP + n], dot);
                const float A = exp2f(dot + gi + sG[kr] - lse2);
                float dp = 0.f;
                for (int c = 0; c < V; ++c) dp = fmaf(sDO[qi * VP + c], sV[kr * VP + c], dp);
                dS = A * (dp - Di);
            }
            sDS[qi * SP + kr] = dS;
            grow += dS;
        }
        __syncthreads();
        for (int kr = 0; kr < BS; ++kr) {
            const float dS = sDS[qi * SP + kr];
            const float *kr_ = sK + kr * QP + sub * KQ;
#pragma unroll
            for (int n = 0; n < KQ; ++n) acc[n] = fmaf(dS, kr_[n], acc[n]);
        }
    }
    grow += __shfl_xor(grow, 1, 64);
    grow += __shfl_xor(grow, 2, 64);
    if (!qvalid) return;
    const float *R = qi >= BS ? sA1 : sA0;
    T *dqg = static_cast<T *>(a.dq) + (qt * HQ + hq) * K + sub * KQ;
    const int64_t base = (qt * HQ + hq) * K + sub * KQ;
#pragma unroll
    for (int n = 0; n < KQ; ++n) {
        const int ch = sub * KQ + n;
        const float dq = a.scale * clamp2(a.P[base + n] - R[ch]) * acc[n];
        st(dqg + n, dq + a.dqd[base + n]);
        a.X[base + n] += ld(qg + base + n) * dq;
    }
    if (sub == 0) {
        a.Y[qt * HQ + hq] += grow;
        a.Z[qt * HQ + hq] = a.sink ? -exp2f(a.sink[hq] * LOG2E - lse2) * Di : 0.f;
    }
}

// ---------------------------------------------------------------- dk, dv
// One block per (kv head, sequence, 64 keys: halves k0 and k1), looping over
// the kv head's query heads.  The queries after the block are read against
// B = floor(P) of its last row; then the queries of k1 against A = floor(P) of
// k0's last row for the keys of k0, whose accumulators move from B to A (an
// exact power of two, at most 1).  The pairs inside k0 and inside k1 come from
// the pair-by-pair kernel, whose per query head dk and dv parts (dkp, dvp) are
// added here.
template <typename T, int K, int V>
__global__ __launch_bounds__(NT) void bwd_dkdv_kernel(BwdArgs a, int nblk) {
    constexpr int QP = K + 1, VP = V + 1, SP = BS + 1, KQ = K / 4, VQ = V / 4;
    extern __shared__ float smem[];
    float *sK = smem;                 // [BB][QP] k * 2^(anchor - P) for the current query head
    float *sV = sK + BB * QP;         // [BB][VP]
    float *sQ = sV + BB * VP;         // [BS][QP] q * scale*log2e * 2^(P - anchor)
    float *sDO = sQ + BS * QP;        // [BS][VP]
    float *sA = sDO + BS * VP;        // [BB][SP]
    float *sDS = sA + BB * SP;        // [BB][SP]
    float *sI = sDS + BB * SP;        // [BS][4]: lse2, D, G (log2), valid
    float *sB = sI + BS * 4;          // [K] B
    float *sAk = sB + K;              // [K] A

    const int bid = blockIdx.x;
    const int h = bid / (a.nseg * nblk);
    const int rem = bid % (a.nseg * nblk);
    const SegInfo sg = a.seg[rem / nblk];
    const int kb = rem % nblk;
    if (kb * BB >= sg.len) return;
    const int tid = threadIdx.x, kj = tid / 4, sub = tid % 4;
    const int64_t HQ = a.HQ;
    const int group = a.HQ / a.H;
    const int j0 = kb * BB;
    const int key = j0 + kj;
    const bool kvalid = key < sg.len;
    const int64_t kt = (int64_t)sg.start + (kvalid ? key : 0);
    const T *qg = static_cast<const T *>(a.q);
    const T *kg = static_cast<const T *>(a.k);
    const T *vg = static_cast<const T *>(a.v);
    const T *dog = static_cast<const T *>(a.dout);

    for (int x = tid; x < BB * V; x += NT) {
        const int r = x / V, c = x % V, j = j0 + r;
        sV[r * VP + c] = j < sg.len ? ld(vg + (((int64_t)sg.start + j) * a.H + h) * V + c) : 0.f;
    }
    float dv[VQ], dk[KQ];
#pragma unroll
    for (int c = 0; c < VQ; ++c) dv[c] = 0.f;
#pragma unroll
    for (int n = 0; n < KQ; ++n) dk[n] = 0.f;
    int ihi = sg.len - 1;
    if (a.window > 0) ihi = min(ihi, min(j0 + BB, sg.len) - 1 + a.window - 1);
    // stages: the queries after the block, then (keys of k0) the queries of k1
    const int nst_off = ihi >= j0 + BB ? (ihi - (j0 + BB)) / BS + 1 : 0;
    const bool has_k1 = ihi >= j0 + BS;
    const int nst = nst_off + (has_k1 ? 1 : 0);

    for (int hq = h * group; hq < (h + 1) * group; ++hq) {
        const float *Pg = a.P + hq * K;
        __syncthreads();
        if (tid < K) {
            sB[tid] = j0 + BB - 1 < sg.len ? floorf(Pg[((int64_t)sg.start + j0 + BB - 1) * HQ * K + tid]) : 0.f;
            sAk[tid] = j0 + BS - 1 < sg.len ? floorf(Pg[((int64_t)sg.start + j0 + BS - 1) * HQ * K + tid]) : 0.f;
        }
        __syncthreads();
        auto stage_k = [&](int rows, const float *R) {
            for (int x = tid; x < rows * K; x += NT) {
                const int r = x / K, n = x % K, j = j0 + r;
                float val = 0.f;
                if (j < sg.len) {
                    const int64_t t = (int64_t)sg.start + j;
                    val = ld(kg + (t * a.H + h) * K + n) * clamp2(R[n] - Pg[t * HQ * K + n]);
                }
                sK[r * QP + n] = val;
            }
        };
        stage_k(BB, sB);
        const float gj = (a.G && kvalid) ? a.G[kt * HQ + hq] : 0.f;
        float dkh[KQ];
#pragma unroll
        for (int n = 0; n < KQ; ++n) dkh[n] = 0.f;
        float gcol = 0.f;
        for (int st_i = 0; st_i < nst; ++st_i) {
            const bool own = st_i == nst_off;
            const int q0 = own ? j0 + BS : j0 + BB + BS * st_i;
            const float *R = own ? sAk : sB;
            __syncthreads();
            if (own) {
                stage_k(BS, sAk);
                if (kj < BS && nst_off > 0) {
#pragma unroll
                    for (int n = 0; n < KQ; ++n) {
                        const int ch = sub * KQ + n;
                        dkh[n] *= exp2f(sB[ch] - sAk[ch]);
                    }
                }
            }
            for (int x = tid; x < BS * K; x += NT) {
                const int r = x / K, n = x % K, i = q0 + r;
                float val = 0.f;
                if (i < sg.len) {
                    const int64_t t = (int64_t)sg.start + i;
                    val = ld(qg + (t * HQ + hq) * K + n) * a.qscale * clamp2(Pg[t * HQ * K + n] - R[n]);
                }
                sQ[r * QP + n] = val;
            }
            for (int x = tid; x < BS * V; x += NT) {
                const int r = x / V, c = x % V, i = q0 + r;
                sDO[r * VP + c] = i < sg.len ? ld(dog + (((int64_t)sg.start + i) * HQ + hq) * V + c) : 0.f;
            }
            if (tid < BS) {
                const int i = q0 + tid;
                const bool ok = i < sg.len;
                const int64_t t = (int64_t)sg.start + (ok ? i : 0);
                sI[tid * 4 + 0] = ok ? a.lse[t * HQ + hq] * LOG2E : 0.f;
                sI[tid * 4 + 1] = ok ? a.D[t * HQ + hq] : 0.f;
                sI[tid * 4 + 2] = (a.G && ok) ? a.G[t * HQ + hq] : 0.f;
                sI[tid * 4 + 3] = ok ? 1.f : 0.f;
            }
            __syncthreads();
            for (int ii = 0; ii < BS / 4; ++ii) {
                const int ir = sub * (BS / 4) + ii, i = q0 + ir;
                bool vis = kvalid && sI[ir * 4 + 3] != 0.f && key <= i && (!own || kj < BS);
                if (a.window > 0) vis = vis && i - key < a.window;
                float A = 0.f, dS = 0.f;
                if (vis) {
                    float dot = 0.f;
                    for (int n = 0; n < K; ++n) dot = fmaf(sQ[ir * QP + n], sK[kj * QP + n], dot);
                    A = exp2f(dot + sI[ir * 4 + 2] - gj - sI[ir * 4 + 0]);
                    float dp = 0.f;
                    for (int c = 0; c < V; ++c) dp = fmaf(sDO[ir * VP + c], sV[kj * VP + c], dp);
                    dS = A * (dp - sI[ir * 4 + 1]);
                }
                sA[kj * SP + ir] = A;
                sDS[kj * SP + ir] = dS;
                gcol += dS;
            }
            __syncthreads();
            for (int ir = 0; ir < BS; ++ir) {
                const float A = sA[kj * SP + ir], dS = sDS[kj * SP + ir];
                const float *dor = sDO + ir * VP + sub * VQ;
                const float *qr = sQ + ir * QP + sub * KQ;
#pragma unroll
                for (int c = 0; c < VQ; ++c) dv[c] = fmaf(A, dor[c], dv[c]);
#pragma unroll
                for (int n = 0; n < KQ; ++n) dkh[n] = fmaf(dS, qr[n], dkh[n]);
            }
        }
        gcol += __shfl_xor(gcol, 1, 64);
        gcol += __shfl_xor(gcol, 2, 64);
        if (kvalid) {
            // this query head's part of dk: scale * 2^(R - P_j) * sum_i dS q 2^(P_i - R);
            // sQ carries scale*log2e, so the factor left is ln 2
            const float *R = (kj < BS && has_k1) ? sAk : sB;
            const int64_t base = (kt * HQ + hq) * K + sub * KQ;
            float *X = a.X + base;
#pragma unroll
            for (int n = 0; n < KQ; ++n) {
                const int ch = sub * KQ + n;
                const float d = LN2 * clamp2(R[ch] - a.P[base + n]) * dkh[n];
                dk[n] += d + a.dkp[base + n];
                X[n] -= ld(kg + (kt * a.H + h) * K + ch) * d;
            }
            const float *dvd = a.dvp + (kt * HQ + hq) * V + sub * VQ;
#pragma unroll
            for (int c = 0; c < VQ; ++c) dv[c] += dvd[c];
            if (sub == 0) a.Y[kt * HQ + hq] -= gcol;
        }
    }
    if (!kvalid) return;
    T *dkg = static_cast<T *>(a.dk) + (kt * a.H + h) * K + sub * KQ;
    T *dvg = static_cast<T *>(a.dv) + (kt * a.H + h) * V + sub * VQ;
#pragma unroll
    for (int n = 0; n < KQ; ++n) st(dkg + n, dk[n]);
#pragma unroll
    for (int c = 0; c < VQ; ++c) st(dvg + c, dv[c]);
}

// ---------------------------------------------------------------- dsink
__global__ __launch_bounds__(NT) void dsink_kernel(const float *Z, float *dsink, int64_t rows, int HQ) {
    const int hq = blockIdx.x;
    float acc = 0.f;
    for (int64_t r = threadIdx.x; r < rows; r += NT) acc += Z[r * HQ + hq];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    __shared__ float part[NT / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.f;
        for (int w = 0; w < NT / 64; ++w) s += part[w];
        dsink[hq] = s;
    }
}

template <typename T, int K, int V>
hipError_t run_valu(const BwdArgs &a, hipStream_t st);

template <typename T, int K, int V>
hipError_t run_bwd(const BwdArgs &a, hipStream_t st) {
    const int64_t nrows = (int64_t)a.rows * a.HQ;
    hipLaunchKernelGGL((bwd_pre_kernel<T, V>), dim3((unsigned)cdiv(nrows, NT / 16)), dim3(NT), 0, st, a, nrows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (std::is_same<T, __bf16>::value) {
        e = launch_bwd_mfma(a, st);
    } else {
        e = run_valu<T, K, V>(a, st);
    }
    if (e != hipSuccess) return e;
    if (a.dsink) {
        hipLaunchKernelGGL(dsink_kernel, dim3((unsigned)a.HQ), dim3(NT), 0, st, a.Z, a.dsink, (int64_t)a.rows,
                           (int)a.HQ);
        e = hipGetLastError();
    }
    return e;
}

template <typename T, int K, int V>
hipError_t run_valu(const BwdArgs &a, hipStream_t st) {
    hipError_t e;
    const int nblk = (int)cdiv(a.max_seqlen, BB);
    constexpr size_t smem_q =
        sizeof(float) * (BB * (K + 1) + BB * (V + 1) + BS * (K + 1) + BS * (V + 1) + BB * (BS + 1) + BS + 2 * K);
    constexpr size_t smem_k = sizeof(float) * (BB * (K + 1) + BB * (V + 1) + BS * (K + 1) + BS * (V + 1) +
                                               2 * BB * (BS + 1) + BS * 4 + 2 * K);
    static_assert(smem_q <= 160 * 1024 && smem_k <= 160 * 1024, "LDS per workgroup");
    // the pairs inside 32-row blocks first: the kernels below add its parts
    e = launch_bwd_diag(a, std::is_same<T, __bf16>::value, true, st);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_dq_kernel<T, K, V>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_q);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_dkdv_kernel<T, K, V>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_k);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<T, K, V>), dim3((unsigned)((int64_t)a.HQ * a.nseg * nblk)), dim3(NT), smem_q,
                       st, a, nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, K, V>), dim3((unsigned)((int64_t)a.H * a.nseg * nblk)), dim3(NT), smem_k,
                       st, a, nblk);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_bwd(const BwdArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_bwd<T, 64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_bwd<T, 64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_bwd<T, 128, 64>(a, st);
    return run_bwd<T, 128, 128>(a, st);
}

}  // namespace

hipError_t launch_bwd_seg(SegInfo *seg, const int32_t *cu, int64_t nseg, int64_t T, hipStream_t st) {
    hipLaunchKernelGGL(bwd_seg_kernel, dim3(1), dim3(256), 0, st, seg, cu, (int)nseg, (int)T);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, bool bf16, hipStream_t st) {
    return bf16 ? dispatch_bwd<__bf16>(a, st) : dispatch_bwd<float>(a, st);
}

}  // namespace wall
