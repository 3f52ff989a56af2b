// wall_bwd_diag.hip -- gradients of the pairs that lie inside one 32-row
// block, formed pair by pair in float32 (the backward of the Wall Attention
// blog's "Definition: Wall Attention", differentiated as in wall_bwd.hip).
//
// For a query row i and key row j of the same block (j <= i):
//     s_ij  = scale * sum_n q_in k_jn 2^(P_in - P_jn) + G_i - G_j
//     A_ij  = exp(s_ij - lse_i),   dS_ij = A_ij (do_i . v_j - D_i)
//     dq_in = scale * sum_j dS_ij k_jn 2^(P_in - P_jn)
//     dk_jn = scale * sum_i dS_ij q_in 2^(P_in - P_jn)    (this query head's part)
//     dv_j  = sum_i A_ij do_i
// with every decay factor its own exp2 of the float32 prefix difference: no
// anchor, so the pairs stay exact however far the prefix falls inside the
// block.  The kernel writes, for the rows of the blocks it handles,
//     dqd = dq part,  dkp = dk part,  dvp = dv part   (float32, per query head)
//     X   = q (.) dq part - k (.) dk part,   Y = row sums - column sums of dS
// which the dq and dk/dv kernels that run after it add to their own sums.
//
// Float32 inputs take every block here (their dq and dk/dv kernels leave the
// pairs inside 32-row blocks to it); bf16 inputs only the blocks the anchor
// pass flagged as spread, found from the flag table 64 entries per workgroup.
#include <float.h>

#include <type_traits>

#include "wall_common.h"

namespace wall {
namespace {

constexpr int NB = BWD_BLK;  // rows per block
constexpr int NT = 256;
constexpr int FLAGS_PER_WG = 64;

__device__ inline float ex2(float e) { return exp2f(fminf(fmaxf(e, EXP2_LO), EXP2_HI)); }

template <typename T>
__device__ inline float ld(const T *p) { return (float)*p; }

template <typename T, int K, int V>
__device__ void diag_block(const BwdArgs &a, float *smem, int hq, const SegInfo &sg, int blk) {
    constexpr int KP = K + 1, VP = V + 1, SP = NB + 1;
    float *sQ = smem;            // [NB][KP] q
    float *sK = sQ + NB * KP;    // [NB][KP] k
    float *sP = sK + NB * KP;    // [NB][KP] P
    float *sV = sP + NB * KP;    // [NB][VP] v
    float *sO = sV + NB * VP;    // [NB][VP] do
    float *sA = sO + NB * VP;    // [NB][SP] A (query row, key row)
    float *sS = sA + NB * SP;    // [NB][SP] dS
    float *sL = sS + NB * SP;    // [NB] lse (log2 units)
    float *sD = sL + NB;         // [NB] D
    float *sG = sD + NB;         // [NB] G
    const int tid = threadIdx.x;
    const int64_t HQ = a.HQ, H = a.H, s0 = sg.start;
    const int h = hq / (a.HQ / a.H);
    const int r0 = blk * NB, n = min(NB, sg.len - r0);
    const T *qg = static_cast<const T *>(a.q);
    const T *kg = static_cast<const T *>(a.k);
    const T *vg = static_cast<const T *>(a.v);
    const T *dog = static_cast<const T *>(a.dout);

    __syncthreads();  // the previous block's reads are done
    for (int x = tid; x < NB * K; x += NT) {
        const int r = x / K, c = x % K;
        float qv = 0.f, kv = 0.f, pv = 0.f;
        if (r < n) {
            const int64_t t = s0 + r0 + r;
            qv = ld(qg + (t * HQ + hq) * K + c);
            kv = ld(kg + (t * H + h) * K + c);
            pv = a.P[(t * HQ + hq) * K + c];
        }
        sQ[r * KP + c] = qv;
        sK[r * KP + c] = kv;
        sP[r * KP + c] = pv;
    }
    for (int x = tid; x < NB * V; x += NT) {
        const int r = x / V, c = x % V;
        float vv = 0.f, ov = 0.f;
        if (r < n) {
            const int64_t t = s0 + r0 + r;
            vv = ld(vg + (t * H + h) * V + c);
            ov = ld(dog + (t * HQ + hq) * V + c);
        }
        sV[r * VP + c] = vv;
        sO[r * VP + c] = ov;
    }
    if (tid < NB) {
        const bool ok = tid < n;
        const int64_t t = (s0 + r0 + (ok ? tid : 0)) * HQ + hq;
        sL[tid] = ok ? a.lse[t] * LOG2E : 0.f;
        sD[tid] = ok ? a.D[t] : 0.f;
        sG[tid] = (a.G && ok) ? a.G[t] : 0.f;
    }
    __syncthreads();

    // pairs: query row i = tid / 8, key rows j = tid % 8 + 8u
    {
        const int i = tid >> 3;
#pragma unroll
        for (int u = 0; u < NB / 8; ++u) {
            const int j = (tid & 7) + 8 * u;
            bool vis = i < n && j <= i;
            if (a.window > 0) vis = vis && i - j < a.window;
            float p = 0.f, ds = 0.f;
            if (vis) {
                float s = 0.f;
                for (int c = 0; c < K; ++c)
                    s = fmaf(sQ[i * KP + c] * sK[j * KP + c], ex2(sP[i * KP + c] - sP[j * KP + c]), s);
                p = exp2f(s * a.qscale + sG[i] - sG[j] - sL[i]);
                float dp = 0.f;
                for (int c = 0; c < V; ++c) dp = fmaf(sO[i * VP + c], sV[j * VP + c], dp);
                ds = p * (dp - sD[i]);
            }
            sA[i * SP + j] = p;
            sS[i * SP + j] = ds;
        }
    }
    __syncthreads();

    // per row r = tid / 8 (as query and as key), channels tid % 8 + 8m
    const int r = tid >> 3, c0 = tid & 7;
    if (r >= n) return;
    const int64_t t = s0 + r0 + r;
    for (int c = c0; c < K; c += 8) {
        const float pr = sP[r * KP + c];
        float dq = 0.f, dk = 0.f;
        for (int j = 0; j <= r; ++j) dq = fmaf(sS[r * SP + j] * sK[j * KP + c], ex2(pr - sP[j * KP + c]), dq);
        for (int i = r; i < n; ++i) dk = fmaf(sS[i * SP + r] * sQ[i * KP + c], ex2(sP[i * KP + c] - pr), dk);
        dq *= a.scale;
        dk *= a.scale;
        const int64_t ix = (t * HQ + hq) * K + c;
        a.dqd[ix] = dq;
        a.dkp[ix] = dk;
        a.X[ix] = sQ[r * KP + c] * dq - sK[r * KP + c] * dk;
    }
    for (int c = c0; c < V; c += 8) {
        float dv = 0.f;
        for (int i = r; i < n; ++i) dv = fmaf(sA[i * SP + r], sO[i * VP + c], dv);
        a.dvp[(t * HQ + hq) * V + c] = dv;
    }
    if (c0 == 0) {
        float y = 0.f;
        for (int j = 0; j <= r; ++j) y += sS[r * SP + j];
        for (int i = r; i < n; ++i) y -= sS[i * SP + r];
        a.Y[t * HQ + hq] = y;
    }
}

template <int K, int V>
constexpr size_t diag_smem() {
    return sizeof(float) * (3 * NB * (K + 1) + 2 * NB * (V + 1) + 2 * NB * (NB + 1) + 3 * NB);
}

// every (query head, sequence, block): one workgroup each
template <typename T, int K, int V>
__global__ __launch_bounds__(NT) void bwd_diag_all(BwdArgs a, int nblk) {
    extern __shared__ float smem[];
    const int blk = blockIdx.x % nblk, hs = blockIdx.x / nblk;
    const int hq = hs % a.HQ;
    const SegInfo sg = a.seg[hs / a.HQ];
    if (blk * NB >= sg.len) return;
    diag_block<T, K, V>(a, smem, hq, sg, blk);
}

// the flagged (block, query head) entries among FLAGS_PER_WG of the table
template <typename T, int K, int V>
__global__ __launch_bounds__(NT) void bwd_diag_flagged(BwdArgs a) {
    extern __shared__ float smem[];
    __shared__ int list[FLAGS_PER_WG];
    __shared__ int cnt;
    const SegInfo last = a.seg[a.nseg - 1];
    const int64_t total = (int64_t)(last.tile_base + (last.len + TILE - 1) / TILE) * (TILE / NB) * a.HQ;
    const int64_t f0 = (int64_t)blockIdx.x * FLAGS_PER_WG;
    if (f0 >= total) return;
    const int tid = threadIdx.x;
    if (tid == 0) cnt = 0;
    __syncthreads();
    // an entry names its sequence (1-based); one that names none, or a block
    // outside that sequence, is skipped
    if (tid < FLAGS_PER_WG && f0 + tid < total) {
        const int64_t f = f0 + tid;
        const int fl = a.flag[f];
        if (fl > 0 && fl <= a.nseg) {
            const SegInfo sg = a.seg[fl - 1];
            const int64_t blk = f / a.HQ - (int64_t)sg.tile_base * (TILE / NB);
            if (blk >= 0 && blk * NB < sg.len) list[atomicAdd(&cnt, 1)] = tid;
        }
    }
    __syncthreads();
    const int m = cnt;
    for (int e = 0; e < m; ++e) {
        const int64_t f = f0 + list[e];
        const int hq = (int)(f % a.HQ);
        const SegInfo sg = a.seg[a.flag[f] - 1];
        diag_block<T, K, V>(a, smem, hq, sg, (int)(f / a.HQ - (int64_t)sg.tile_base * (TILE / NB)));
    }
}

template <typename T, int K, int V>
hipError_t run(const BwdArgs &a, bool all, hipStream_t st) {
    constexpr size_t smem = diag_smem<K, V>();
    static_assert(smem <= 160 * 1024, "LDS per workgroup");
    if (all) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_diag_all<T, K, V>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        const int nblk = (int)cdiv(a.max_seqlen, NB);
        hipLaunchKernelGGL((bwd_diag_all<T, K, V>), dim3((unsigned)((int64_t)a.HQ * a.nseg * nblk)), dim3(NT), smem,
                           st, a, nblk);
        return hipGetLastError();
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_diag_flagged<T, K, V>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    // entries of the flag table: bounded by its allocated size
    const int64_t entries = (cdiv((int64_t)a.rows, TILE) + a.nseg) * (TILE / NB) * a.HQ;
    hipLaunchKernelGGL((bwd_diag_flagged<T, K, V>), dim3((unsigned)cdiv(entries, FLAGS_PER_WG)), dim3(NT), smem, st,
                       a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const BwdArgs &a, bool all, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run<T, 64, 64>(a, all, st);
    if (a.K == 64 && a.V == 128) return run<T, 64, 128>(a, all, st);
    if (a.K == 128 && a.V == 64) return run<T, 128, 64>(a, all, st);
    return run<T, 128, 128>(a, all, st);
}

}  // namespace

hipError_t launch_bwd_diag(const BwdArgs &a, bool bf16, bool all, hipStream_t st) {
    return bf16 ? dispatch<__bf16>(a, all, st) : dispatch<float>(a, all, st);
}

}  // namespace wall
