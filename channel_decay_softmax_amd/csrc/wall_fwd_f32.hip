// wall_fwd_f32.hip -- fused causal Wall Attention forward for float32 inputs.
//
// Same method as the bf16 kernel (per-tile anchors, float32 online softmax in
// the log2 domain, causal / window / sequence tile skipping) with every
// operand kept in float32, so the only rounding is float32 arithmetic.  It
// runs on the vector ALUs: one workgroup owns 64 query rows of one query
// head; keys are staged 32 at a time in LDS.  Thread t handles query t/4 and
// either keys 8*(t%4)..+7 (scores) or value channels of quarter t%4 (PV).
#include <float.h>

#include "wall_common.h"

namespace wall {
namespace {

constexpr int BQ = 64;  // query rows per workgroup
constexpr int BK = 32;  // keys per LDS stage

template <int K, int V>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a, int qtiles) {
    constexpr int QP = K + 1, KPT = K + 1, PP = BK + 1;
    constexpr int VD = V / 4;  // value channels per thread
    extern __shared__ float smem[];
    float *sQh = smem;              // [BQ][QP] q^ (diagonal-anchored)
    float *sQ = sQh + BQ * QP;      // [BQ][QP] q~ for the current key tile
    float *sK = sQ + BQ * QP;       // [BK][KPT]
    float *sV = sK + BK * KPT;      // [BK][V]
    float *sP = sV + BK * V;        // [BQ][PP]
    int *sShift = reinterpret_cast<int *>(sP + BQ * PP);  // [K]
    float *sBias = reinterpret_cast<float *>(sShift + K);  // [BK]

    const int bid = blockIdx.x;
    const int hq = bid / (a.nseg * qtiles);
    const int rem = bid % (a.nseg * qtiles);
    const int s = rem / qtiles, qb = rem % qtiles;
    const SegInfo sg = a.seg[s];
    if (qb * BQ >= sg.len) return;
    const int tid = threadIdx.x;
    const int qi = tid / 4, sub = tid % 4;
    const int h = hq / (a.HQ / a.H);
    const float *qg = static_cast<const float *>(a.q);
    const float *ktg = static_cast<const float *>(a.kt);
    const float *vtg = static_cast<const float *>(a.vt);
    float *og = static_cast<float *>(a.o);

    const int qrow = qb * BQ + qi;
    const bool qvalid = qrow < sg.len;
    const int64_t qtok = (int64_t)sg.start + (qvalid ? qrow : 0);
    const int cd = (qb * BQ) / TILE;  // anchor tile holding this query block
    const float *Rd = a.anchor + ((int64_t)(sg.tile_base + cd) * a.HQ + hq) * K;

    for (int x = tid; x < BQ * K; x += 256) {
        const int r = x / K, n = x % K;
        const int row = qb * BQ + r;
        float val = 0.f;
        if (row < sg.len) {
            const int64_t tok = sg.start + row;
            const float e = fminf(fmaxf(a.P[(tok * a.HQ + hq) * K + n] - Rd[n], EXP2_LO), EXP2_HI);
            val = qg[(tok * a.HQ + hq) * K + n] * a.qscale * exp2f(e);
        }
        sQh[r * QP + n] = val;
    }
    const float g_i = (a.G && qvalid) ? a.G[qtok * a.HQ + hq] : 0.f;

    float m_run = -FLT_MAX, l_run = 0.f;
    float acc[VD];
    for (int d = 0; d < VD; ++d) acc[d] = 0.f;

    const int qlast = min(qb * BQ + BQ - 1, sg.len - 1);
    int c_lo = 0;
    if (a.window > 0) {
        const int kmin = qb * BQ - a.window + 1;
        c_lo = kmin > 0 ? kmin / TILE : 0;
    }
    for (int c = cd; c >= c_lo; --c) {
        __syncthreads();
        if (tid < K) {
            const float rc = a.anchor[((int64_t)(sg.tile_base + c) * a.HQ + hq) * K + tid];
            sShift[tid] = anchor_shift(Rd[tid] - rc);
        }
        __syncthreads();
        for (int x = tid; x < BQ * K; x += 256) {
            const int r = x / K, n = x % K;
            sQ[r * QP + n] = __builtin_ldexpf(sQh[r * QP + n], sShift[n]);
        }
        const float *ktile = ktg + ((int64_t)(sg.tile_base + c) * a.HQ + hq) * TILE * K;
        const float *vtile = vtg + ((int64_t)(sg.tile_base + c) * a.H + h) * TILE * V;
        for (int kb = TILE / BK - 1; kb >= 0; --kb) {
            const int key0 = c * TILE + kb * BK;
            if (key0 > qlast) continue;  // wholly in the future of every query here
            if (a.window > 0 && qb * BQ - (key0 + BK - 1) >= a.window) continue;  // wholly outside
            __syncthreads();
            for (int x = tid; x < BK * K; x += 256) sK[(x / K) * KPT + x % K] = ktile[kb * BK * K + x];
            for (int x = tid; x < BK * V; x += 256) sV[x] = vtile[kb * BK * V + x];
            if (tid < BK) {
                const int j = key0 + tid;
                sBias[tid] = (a.G && j < sg.len) ? -a.G[((int64_t)sg.start + j) * a.HQ + hq] : 0.f;
            }
            __syncthreads();
            float sc[8];
            float mloc = -INFINITY;
            for (int kk = 0; kk < 8; ++kk) {
                const int kr = sub * 8 + kk, key = key0 + kr;
                float dot = 0.f;
                for (int n = 0; n < K; ++n) dot = fmaf(sQ[qi * QP + n], sK[kr * KPT + n], dot);
                float x = dot + (a.G ? g_i + sBias[kr] : 0.f);
                bool vis = key <= qrow && key < sg.len;
                if (a.window > 0) vis = vis && (qrow - key < a.window);
                x = vis ? x : -INFINITY;
                sc[kk] = x;
                mloc = fmaxf(mloc, x);
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 1, 64));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 2, 64));
            const float m_new = fmaxf(m_run, mloc);
            const float alpha = exp2f(m_run - m_new);
            float lsum = 0.f;
            for (int kk = 0; kk < 8; ++kk) {
                const float pr = exp2f(sc[kk] - m_new);
                sP[qi * PP + sub * 8 + kk] = pr;
                lsum += pr;
            }
            lsum += __shfl_xor(lsum, 1, 64);
            lsum += __shfl_xor(lsum, 2, 64);
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            __syncthreads();
            for (int d = 0; d < VD; ++d) acc[d] *= alpha;
            for (int kr = 0; kr < BK; ++kr) {
                const float pr = sP[qi * PP + kr];
                const float *vr = sV + kr * V + sub * VD;
                for (int d = 0; d < VD; ++d) acc[d] = fmaf(pr, vr[d], acc[d]);
            }
        }
    }

    float m_fin = m_run, l_fin = l_run;
    if (a.sink) {
        const float sb = a.sink[hq] * LOG2E;
        m_fin = fmaxf(m_run, sb);
        l_fin = l_run * exp2f(m_run - m_fin) + exp2f(sb - m_fin);
    }
    const float fac = exp2f(m_run - m_fin) / l_fin;
    if (qvalid) {
        float *orow = og + (qtok * a.HQ + hq) * V + sub * VD;
        for (int d = 0; d < VD; ++d) orow[d] = acc[d] * fac;
        if (a.lse && sub == 0) a.lse[qtok * a.HQ + hq] = (m_fin + log2f(l_fin)) * LN2;
    }
}

template <int K, int V>
hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
    constexpr size_t smem =
        sizeof(float) * (2 * BQ * (K + 1) + BK * (K + 1) + BK * V + BQ * (BK + 1) + K + BK);
    const int qtiles = (a.max_tiles * TILE + BQ - 1) / BQ;
    const int64_t nblk = (int64_t)a.nseg * qtiles * a.HQ;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_f32_kernel<K, V>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_f32_kernel<K, V>), dim3((unsigned)nblk), dim3(256), smem, st, a, qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t st) {
    if (a.K == 64 && a.V == 64) return run_fwd<64, 64>(a, st);
    if (a.K == 64 && a.V == 128) return run_fwd<64, 128>(a, st);
    if (a.K == 128 && a.V == 64) return run_fwd<128, 64>(a, st);
    return run_fwd<128, 128>(a, st);
}

}  // namespace wall
