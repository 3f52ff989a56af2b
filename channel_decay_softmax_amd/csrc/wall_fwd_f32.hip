// wall_fwd_f32.hip -- fused causal Wall Attention forward for float32 inputs.
//
// Every operand stays float32, so the only rounding is float32 arithmetic;
// the kernel runs on the vector ALUs.  A workgroup owns 64 query rows of one
// query head; keys stream through LDS 32 at a time from the block's last row
// down to the first key the window reaches.  Thread t handles query t/4 and
// either keys 8*(t%4)..+7 of a stage (scores) or value channels of quarter t%4
// (PV); float32 online softmax in the log2 domain.
//
// Anchors (the per-tile anchor identity of the Wall Attention blog, "Fast
// training and inference": exp2(P_i - P_j) = exp2(P_i - A) * exp2(A - P_j)):
//   * every key before the block is read against one anchor, the floored
//     prefix of the row just before the block.  That row lies between every
//     such key and every query of the block, so for a prefix that falls
//     both factors are at most 2, and a factor that underflows belongs to a
//     term below 2^-125 of the largest, at any gate strength;
//   * the keys among the block's own 64 rows are formed pair by pair,
//     scale * sum_n q_in k_jn exp2(P_in - P_jn), with no anchor.
// The kernel reads the raw q, k, v and P; the preparation step only supplies
// the sequence table.
#include <float.h>

#include "wall_common.h"

namespace wall {
namespace {

constexpr int BQ = 64;  // query rows per workgroup
constexpr int BK = 32;  // keys per LDS stage

template <int K, int V>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a, int qtiles) {
    constexpr int QP = K + 1, KP = K + 1, PP = BK + 1;
    constexpr int VD = V / 4;  // value channels per thread
    extern __shared__ float smem[];
    float *sQa = smem;               // [BQ][QP] q scale log2e exp2(P_i - A)
    float *sQr = sQa + BQ * QP;      // [BQ][QP] q scale log2e
    float *sPq = sQr + BQ * QP;      // [BQ][QP] P_i
    float *sK = sPq + BQ * QP;       // [BK][KP] k exp2(A - P_j), or k (own rows)
    float *sPk = sK + BK * KP;       // [BK][KP] P_j (own rows)
    float *sV = sPk + BK * KP;       // [BK][V]
    float *sP = sV + BK * V;         // [BQ][PP]
    float *sBias = sP + BQ * PP;     // [BK] -G_j
    float *sA = sBias + BK;          // [K] anchor of the keys before the block

    const int bid = blockIdx.x;
    const int hq = bid / (a.nseg * qtiles);
    const int rem = bid % (a.nseg * qtiles);
    const int s = rem / qtiles, qb = rem % qtiles;
    const SegInfo sg = a.seg[s];
    const int q0 = qb * BQ;
    if (q0 >= sg.len) return;
    const int tid = threadIdx.x;
    const int qi = tid / 4, sub = tid % 4;
    const int64_t HQ = a.HQ, H = a.H;
    const int h = hq / (a.HQ / a.H);
    const float *qg = static_cast<const float *>(a.q);
    const float *kg = static_cast<const float *>(a.k);
    const float *vg = static_cast<const float *>(a.v);
    float *og = static_cast<float *>(a.o);
    const int64_t s0 = sg.start;

    const int qrow = q0 + qi;
    const bool qvalid = qrow < sg.len;
    const int64_t qtok = s0 + (qvalid ? qrow : 0);

    if (tid < K) sA[tid] = q0 > 0 ? floorf(a.P[((s0 + q0 - 1) * HQ + hq) * K + tid]) : 0.f;
    __syncthreads();
    for (int x = tid; x < BQ * K; x += 256) {
        const int r = x / K, n = x % K;
        const int row = q0 + r;
        float qa = 0.f, qr = 0.f, pq = 0.f;
        if (row < sg.len) {
            const int64_t ix = ((s0 + row) * HQ + hq) * K + n;
            pq = a.P[ix];
            qr = qg[ix] * a.qscale;
            qa = qr * exp2f(fminf(fmaxf(pq - sA[n], EXP2_LO), EXP2_HI));
        }
        sQa[r * QP + n] = qa;
        sQr[r * QP + n] = qr;
        sPq[r * QP + n] = pq;
    }
    const float g_i = (a.G && qvalid) ? a.G[qtok * HQ + hq] : 0.f;

    float m_run = -FLT_MAX, l_run = 0.f;
    float acc[VD];
    for (int d = 0; d < VD; ++d) acc[d] = 0.f;

    const int qlast = min(q0 + BQ - 1, sg.len - 1);
    int klo = 0;
    if (a.window > 0) klo = max(0, q0 - a.window + 1) / BK * BK;
    for (int key0 = qlast / BK * BK; key0 >= klo; key0 -= BK) {
        const bool own = key0 >= q0;  // the stage holds keys of the block's own rows
        __syncthreads();
        for (int x = tid; x < BK * K; x += 256) {
            const int r = x / K, n = x % K;
            const int j = key0 + r;
            float kv = 0.f, pj = 0.f;
            if (j < sg.len) {
                kv = kg[((s0 + j) * H + h) * K + n];
                pj = a.P[((s0 + j) * HQ + hq) * K + n];
            }
            if (own) {
                sK[r * KP + n] = kv;
                sPk[r * KP + n] = pj;
            } else {
                sK[r * KP + n] = kv * exp2f(fminf(fmaxf(sA[n] - pj, EXP2_LO), EXP2_HI));
            }
        }
        for (int x = tid; x < BK * V; x += 256) {
            const int r = x / V, d = x % V;
            const int j = key0 + r;
            sV[x] = j < sg.len ? vg[((s0 + j) * H + h) * V + d] : 0.f;
        }
        if (tid < BK) {
            const int j = key0 + tid;
            sBias[tid] = (a.G && j < sg.len) ? -a.G[(s0 + j) * HQ + hq] : 0.f;
        }
        __syncthreads();
        float sc[8];
        float mloc = -INFINITY;
        for (int kk = 0; kk < 8; ++kk) {
            const int kr = sub * 8 + kk, key = key0 + kr;
            bool vis = qvalid && key <= qrow;
            if (a.window > 0) vis = vis && (qrow - key < a.window);
            float x = -INFINITY;
            if (vis) {
                float dot = 0.f;
                if (own) {
                    for (int n = 0; n < K; ++n) {
                        const float f = exp2f(fminf(fmaxf(sPq[qi * QP + n] - sPk[kr * KP + n], EXP2_LO), EXP2_HI));
                        dot = fmaf(sQr[qi * QP + n] * sK[kr * KP + n], f, dot);
                    }
                } else {
                    for (int n = 0; n < K; ++n) dot = fmaf(sQa[qi * QP + n], sK[kr * KP + n], dot);
                }
                x = dot + (a.G ? g_i + sBias[kr] : 0.f);
            }
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

    float m_fin = m_run, l_fin = l_run;
    if (a.sink) {
        const float sb = a.sink[hq] * LOG2E;
        m_fin = fmaxf(m_run, sb);
        l_fin = l_run * exp2f(m_run - m_fin) + exp2f(sb - m_fin);
    }
    const float fac = exp2f(m_run - m_fin) / l_fin;
    if (qvalid) {
        float *orow = og + (qtok * HQ + hq) * V + sub * VD;
        for (int d = 0; d < VD; ++d) orow[d] = acc[d] * fac;
        if (a.lse && sub == 0) a.lse[qtok * HQ + hq] = (m_fin + log2f(l_fin)) * LN2;
    }
}

template <int K, int V>
hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
    constexpr size_t smem =
        sizeof(float) * (3 * BQ * (K + 1) + 2 * BK * (K + 1) + BK * V + BQ * (BK + 1) + BK + K);
    static_assert(smem <= 160 * 1024, "LDS per workgroup");
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
