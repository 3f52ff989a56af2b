// wall_fwd_bf16.hip -- fused causal Wall Attention forward, bf16 inputs, gfx950.
//
// One workgroup (4 waves) owns one (sequence, query head) and two 128-row
// query tiles, p and n-1-p, so every workgroup of a causal launch does the
// same number of tile pairs.  Each wave owns 32 query rows.  For every key
// tile c (from the diagonal tile down to the first tile the window reaches):
//
//   anchors   q~ = ldexp(q^, Rdiag - Rc), where q^ = q * scale*log2e *
//             exp2(P_i - Rdiag) was built once per query tile (float32) and
//             Rd, Rc are the integer per-channel anchors of the diagonal and
//             of tile c, so exp2(P_i - P_j) = exp2(P_i - Rc) * exp2(Rc - P_j)
//             with the second factor already folded into the cached k~
//             (blog "Fast training and inference": per-tile anchors);
//   S^T       = k~ q~^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16
//             channels from LDS, B = the wave's 32 queries), so each lane
//             holds one query column: 64 of the tile's 128 scores;
//   softmax   online, float32, log2 domain: row max over the lane's scores
//             and its partner lane (lane ^ 32), exp2, running sum;
//   O^T      += v^T p^T on the same MFMA (A = 32 value channels x 16 keys
//             from the transposed value tile in LDS, B = the lane's bf16 p).
//
// The key rows fed to the S^T MFMA are permuted (bits 2 and 3 of the row
// index swapped) so that the MFMA's output rows for one lane come out as 8
// consecutive keys per register group -- exactly the k-slots the PV MFMA
// needs from that lane; no shuffles are needed between the two products.
#include <float.h>

#include "wall_common.h"

namespace wall {
namespace {

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ inline float wave_pair_sum(float x) { return x + __shfl_xor(x, 32, 64); }

// Key row (within a 32-row block) that the MFMA A-row m reads: bits 2 and 3 swapped.
__device__ inline int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int K, int V>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(FwdArgs a) {
    constexpr int KP = K + 8;     // LDS pitch (elements) of a key row
    constexpr int TP = TILE + 8;  // LDS pitch of a transposed value row
    constexpr int KS = K / 16;    // MFMA k-steps over channels
    constexpr int VT = V / 32;    // 32-wide value blocks
    __shared__ __attribute__((aligned(16))) __bf16 sK[TILE * KP];
    __shared__ __attribute__((aligned(16))) __bf16 sV[V * TP];
    __shared__ __attribute__((aligned(16))) int sShift[K];
    __shared__ __attribute__((aligned(16))) float sBias[TILE];

    const int npairs = (a.max_tiles + 1) / 2;
    const int nblk = a.nseg * npairs * a.HQ;
    int bid = blockIdx.x;
    // Workgroups are dispatched round robin over the 8 XCDs; give each XCD a
    // contiguous range of work ids so the tiles of one head share an L2.
    if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
    const int hq = bid / (a.nseg * npairs);
    const int rem = bid % (a.nseg * npairs);
    const int s = rem / npairs, p = rem % npairs;
    const SegInfo sg = a.seg[s];
    const int nq = (sg.len + TILE - 1) / TILE;
    if (p >= (nq + 1) / 2) return;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hl = lane >> 5;
    const int h = hq / (a.HQ / a.H);
    const __bf16 *qg = static_cast<const __bf16 *>(a.q);
    const __bf16 *ktg = static_cast<const __bf16 *>(a.kt);
    const __bf16 *vtg = static_cast<const __bf16 *>(a.vt);
    __bf16 *og = static_cast<__bf16 *>(a.o);

    for (int pass = 0; pass < 2; ++pass) {
        const int qt = pass == 0 ? p : nq - 1 - p;
        if (pass == 1 && qt == p) break;
        const int qrow = qt * TILE + wave * 32 + col;  // sequence-local query row
        const bool qvalid = qrow < sg.len;
        const int64_t qtok = (int64_t)sg.start + (qvalid ? qrow : 0);
        const float *Rd = a.anchor + ((int64_t)(sg.tile_base + qt) * a.HQ + hq) * K;

        // q^ = q * scale*log2e * exp2(P_i - Rdiag) for the lane's channels 16*s8 + 8*hl + e
        float qh[KS][8];
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8) {
            const int ch0 = 16 * s8 + 8 * hl;
            const bf16x8 qv = *reinterpret_cast<const bf16x8 *>(qg + (qtok * a.HQ + hq) * K + ch0);
            const f32x8 pv = *reinterpret_cast<const f32x8 *>(a.P + (qtok * a.HQ + hq) * K + ch0);
            const f32x8 rv = *reinterpret_cast<const f32x8 *>(Rd + ch0);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = fminf(fmaxf(pv[e] - rv[e], EXP2_LO), EXP2_HI);
                qh[s8][e] = qvalid ? (float)qv[e] * a.qscale * exp2f(x) : 0.f;
            }
        }
        const float g_i = (a.G && qvalid) ? a.G[qtok * a.HQ + hq] : 0.f;
        const float rdiag_t = tid < K ? Rd[tid] : 0.f;

        float m_run = -FLT_MAX, l_run = 0.f;
        f32x16 O[VT];
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) O[vt] = f32x16{};

        int c_lo = 0;
        if (a.window > 0) {
            const int kmin = qt * TILE - a.window + 1;
            c_lo = kmin > 0 ? kmin / TILE : 0;
        }
        for (int c = qt; c >= c_lo; --c) {
            __syncthreads();  // previous tile's LDS reads are done
            const __bf16 *ktp = ktg + ((int64_t)(sg.tile_base + c) * a.HQ + hq) * TILE * K;
            for (int x = tid; x < TILE * K / 8; x += 256) {
                const int row = x / (K / 8), c8 = x % (K / 8);
                *reinterpret_cast<bf16x8 *>(&sK[row * KP + c8 * 8]) =
                    *reinterpret_cast<const bf16x8 *>(ktp + x * 8);
            }
            const __bf16 *vtp = vtg + ((int64_t)(sg.tile_base + c) * a.H + h) * V * TILE;
            for (int x = tid; x < V * TILE / 8; x += 256) {
                const int row = x / (TILE / 8), c8 = x % (TILE / 8);
                *reinterpret_cast<bf16x8 *>(&sV[row * TP + c8 * 8]) =
                    *reinterpret_cast<const bf16x8 *>(vtp + x * 8);
            }
            if (tid < K) {
                const float rc = a.anchor[((int64_t)(sg.tile_base + c) * a.HQ + hq) * K + tid];
                sShift[tid] = anchor_shift(rdiag_t - rc);
            }
            if (a.G) {
                for (int x = tid; x < TILE; x += 256) {
                    const int j = c * TILE + x;
                    sBias[x] = j < sg.len ? -a.G[((int64_t)sg.start + j) * a.HQ + hq] : 0.f;
                }
            }
            __syncthreads();

            // ---- S^T = k~ q~^T
            f32x16 S[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) S[mt] = f32x16{};
#pragma unroll
            for (int s8 = 0; s8 < KS; ++s8) {
                const int ch0 = 16 * s8 + 8 * hl;
                const int4 sh0 = *reinterpret_cast<const int4 *>(&sShift[ch0]);
                const int4 sh1 = *reinterpret_cast<const int4 *>(&sShift[ch0 + 4]);
                const int sh[8] = {sh0.x, sh0.y, sh0.z, sh0.w, sh1.x, sh1.y, sh1.z, sh1.w};
                f32x8 qs;
#pragma unroll
                for (int e = 0; e < 8; ++e) qs[e] = __builtin_ldexpf(qh[s8][e], sh[e]);
                const bf16x8 qop = __builtin_convertvector(qs, bf16x8);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int krow = 32 * mt + key_perm(col);
                    const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(&sK[krow * KP + ch0]);
                    S[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop, S[mt], 0, 0, 0);
                }
            }

            // ---- bias, masks, online softmax (log2 domain)
            const bool diag = c == qt;
            const bool wmask = a.window > 0 && TILE * (qt - c) + TILE - 1 >= a.window;
            float mloc = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kin = 32 * mt + 16 * (r / 8) + 8 * hl + (r % 8);  // key within tile
                    const int key = c * TILE + kin;
                    float x = S[mt][r];
                    if (a.G) x += g_i + sBias[kin];
                    bool vis = true;
                    if (diag) vis = key <= qrow && key < sg.len;
                    if (wmask) vis = vis && (qrow - key < a.window);
                    x = vis ? x : -INFINITY;
                    S[mt][r] = x;
                    mloc = fmaxf(mloc, x);
                }
            }
            mloc = wave_pair_max(mloc);
            const float m_new = fmaxf(m_run, mloc);
            const float alpha = fast_exp2(m_run - m_new);
            float lsum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = fast_exp2(S[mt][r] - m_new);
                    S[mt][r] = pr;
                    lsum += pr;
                }
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) O[vt] *= alpha;

            // ---- O^T += v^T p^T
#pragma unroll
            for (int ks = 0; ks < TILE / 16; ++ks) {
                f32x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = S[ks / 2][8 * (ks % 2) + e];
                const bf16x8 pop = __builtin_convertvector(pv, bf16x8);
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) {
                    const bf16x8 vop = *reinterpret_cast<const bf16x8 *>(
                        &sV[(32 * vt + col) * TP + 16 * ks + 8 * hl]);
                    O[vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, O[vt], 0, 0, 0);
                }
            }
        }

        // ---- epilogue: sink, normalisation, o and lse
        const float l_tot = wave_pair_sum(l_run);
        float m_fin = m_run, l_fin = l_tot;
        if (a.sink) {
            const float sb = a.sink[hq] * LOG2E;
            m_fin = fmaxf(m_run, sb);
            l_fin = l_tot * exp2f(m_run - m_fin) + exp2f(sb - m_fin);
        }
        const float fac = exp2f(m_run - m_fin) / l_fin;
        if (qvalid) {
            __bf16 *orow = og + (qtok * a.HQ + hq) * V;
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = O[vt][4 * r4 + e] * fac;
                    *reinterpret_cast<bf16x4 *>(orow + 32 * vt + 8 * r4 + 4 * hl) =
                        __builtin_convertvector(x, bf16x4);
                }
            }
            if (a.lse && hl == 0) a.lse[qtok * a.HQ + hq] = (m_fin + log2f(l_fin)) * LN2;
        }
    }
}

template <int K, int V>
hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
    const int npairs = (a.max_tiles + 1) / 2;
    const int64_t nblk = (int64_t)a.nseg * npairs * a.HQ;
    hipLaunchKernelGGL((fwd_bf16_kernel<K, V>), dim3((unsigned)nblk), dim3(256), 0, st, a);
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
