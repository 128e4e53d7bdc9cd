// gdr_fwd.hip -- the chunked forward output and the gate's in-chunk cumsum.
//
// FlashQLA backward explainer §一: the gate is carried as its in-chunk
// cumulative sum (restarting at every chunk and sequence start) and the
// forward state h[c] (entering chunk c) is what the chunked form runs on.
// With V_new = U − W h[c] (W, U from the WY-factor kernel) the chunk output is
//     o = scale · diag(γ) Q h[c] + Pm V_new,   Pm = scale · lower(Γ ⊙ Q Kᵀ)
// (the same decomposition the backward differentiates).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

// ---------------------------------------------------------------- gate cumsum
// One thread per (chunk, value head): the chunk's prefix sums of the raw gate
// in token order, each one fp32 addition after the previous, starting from the
// chunk's first value itself (so every element is the same sequence of fp32
// additions a serial in-chunk scan performs).  Grid x: the (chunk, head)
// pairs of the longest sequence; grid y: the sequences (strided past 65535).
__global__ void gate_cumsum_kernel(const float* __restrict__ g, float* __restrict__ gc, const int32_t* __restrict__ cu,
                                   int nseq, int T, int HV, int BT, int maxC) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)maxC * HV) return;
    const int c = (int)(idx / HV), hv = (int)(idx % HV);
    for (int n = blockIdx.y; n < nseq; n += gridDim.y) {
        const long bos = cu ? (long)cu[n] : (long)n * T, eos = cu ? (long)cu[n + 1] : bos + T;
        const long t0 = bos + (long)c * BT;
        if (t0 >= eos) continue;
        const int len = (int)(eos - t0 < BT ? eos - t0 : BT);
        const float* gp = g + t0 * HV + hv;
        float* op = gc + t0 * HV + hv;
        float acc = 0.f;
        for (int s0 = 0; s0 < len; s0 += 16) {   // sixteen loads in flight, then the serial additions
            float x[16];
#pragma unroll
            for (int u = 0; u < 16; u++) x[u] = gp[(long)min(s0 + u, len - 1) * HV];
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (s0 + u < len) {
                    acc = s0 + u == 0 ? x[u] : acc + x[u];
                    op[(long)(s0 + u) * HV] = acc;
                }
            }
        }
    }
}

hipError_t launch_gate_cumsum(const Problem& p, const float* g, float* gc, hipStream_t s) {
    const long pairs = (long)p.maxC * p.HV;
    if (pairs == 0 || p.N == 0) return hipSuccess;
    const unsigned gy = (unsigned)(p.N < 65535 ? p.N : 65535);
    hipLaunchKernelGGL(gate_cumsum_kernel, dim3((unsigned)((pairs + 255) / 256), gy), dim3(256), 0, s, g, gc, p.cu,
                       p.N, p.T, p.HV, p.BT, (int)p.maxC);
    return hipGetLastError();
}

// ---------------------------------------------------------------- output
template <class T, int N> using vec_t = T __attribute__((ext_vector_type(N)));

template <class S, int KD, int VD>
struct FwdCfg {
    static constexpr int C = 64, PAD = 16 / (int)sizeof(S);
    static constexpr int LK = KD + PAD, LV = VD + PAD, LA = 64 + PAD;
    static constexpr size_t oQ = 0;                                     // Q [64][LK]
    static constexpr size_t oK = oQ + (size_t)C * LK * sizeof(S);       // K [64][LK], later the o tile
    static constexpr size_t oW = oK + (size_t)C * LK * sizeof(S);       // W [64][LK]
    static constexpr size_t oH = oW + (size_t)C * LK * sizeof(S);       // h[c] as [V][LK]
    static constexpr size_t oVn = oH + (size_t)VD * LK * sizeof(S);     // U, then V_new [64][LV]
    static constexpr size_t oPm = oVn + (size_t)C * LV * sizeof(S);     // Pm [64][LA]
    static constexpr size_t oG = oPm + (size_t)C * LA * sizeof(S);      // G [64]
    static constexpr size_t smem = oG + C * 4;
    static_assert(smem <= 160 * 1024, "LDS budget");
};

// Persistent: workgroup b handles units (chunk, value head) b, b + grid, ...;
// 512 threads (8 waves, two per SIMD); wave w computes rows 32 (w & 1) .. +31
// and column block w >> 1 of every output.  Products run in row form (a lane
// holds four adjacent columns of one row of each tile), so Pm, V_new and o
// move through LDS as 8-byte row pieces.  The next unit's Q, K, W, U, h and
// gate are loaded into registers while the current unit is computed.  W, U,
// h and o are read or written once, with non-temporal accesses.
// E: input type; S: operand type of the workspace tiles and of the MFMAs (fp16
// for 16-bit inputs, fp32 for fp32).
template <class E, class S, int KD, int VD>
__global__ void __launch_bounds__(512) fwd_out_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                      const float* __restrict__ gcum, const ChunkInfo* __restrict__ info,
                                                      const S* __restrict__ Wg, const S* __restrict__ Ug,
                                                      const E* __restrict__ hT, E* __restrict__ o, int HK, int HV,
                                                      float scale, int nunits) {
    static_assert(sizeof(E) == sizeof(S), "input and operand types share a width");
    using Cf = FwdCfg<S, KD, VD>;
    constexpr int C = 64, NT = 512, LK = Cf::LK, LV = Cf::LV, LA = Cf::LA;
    constexpr int EPE = 16 / (int)sizeof(E);
    static_assert(C * LV * sizeof(E) <= C * LK * sizeof(S), "o tile fits in the K buffer");
    static_assert(C * KD / EPE % NT == 0 && C * VD / EPE % NT == 0 && KD * VD / EPE % NT == 0, "whole vectors");
    constexpr int NQ = C * KD / EPE / NT, NU = C * VD / EPE / NT, NH = KD * VD / EPE / NT;
    using VE = vec_t<E, EPE>;
    using VS = vec_t<S, EPE>;
    extern __shared__ __align__(16) unsigned char smem[];
    S* sQ = (S*)(smem + Cf::oQ);
    S* sK = (S*)(smem + Cf::oK);
    S* sW = (S*)(smem + Cf::oW);
    S* sH = (S*)(smem + Cf::oH);
    S* sVn = (S*)(smem + Cf::oVn);
    S* sPm = (S*)(smem + Cf::oPm);
    float* sG = (float*)(smem + Cf::oG);
    E* sO = (E*)(smem + Cf::oK);
    const int w = wave_id();
    const int m0 = 32 * (w & 1);

    VE rq[NQ], rk[NQ], rh[NH];
    VS rw[NQ], ru[NU];
    float rg = 0.f;
    // loads of unit u (rows past the chunk read its last row; zeroed when staged)
    auto issue = [&](int u, int Cu, long tu) {
        const int hvu = u % HV, hku = hvu / (HV / HK);
        const long unit = (long)(u / HV) * HV + hvu;
        if (threadIdx.x < C) rg = gcum[(tu + min((int)threadIdx.x, Cu - 1)) * HV + hvu];
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const int idx = threadIdx.x + NT * i, r = min(idx / (KD / EPE), Cu - 1), c = (idx % (KD / EPE)) * EPE;
            rq[i] = *(const VE*)(q + ((tu + r) * HK + hku) * KD + c);
            rk[i] = *(const VE*)(k + ((tu + r) * HK + hku) * KD + c);
            rw[i] = __builtin_nontemporal_load((const VS*)(Wg + unit * C * KD + (long)idx * EPE));
        }
#pragma unroll
        for (int i = 0; i < NU; i++)
            ru[i] = __builtin_nontemporal_load((const VS*)(Ug + unit * C * VD + (long)(threadIdx.x + NT * i) * EPE));
#pragma unroll
        for (int i = 0; i < NH; i++)
            rh[i] = __builtin_nontemporal_load((const VE*)(hT + unit * KD * VD + (long)(threadIdx.x + NT * i) * EPE));
    };

    int u = blockIdx.x;
    if (u >= nunits) return;
    int cur_len = info[u / HV].len;
    long cur_t0 = info[u / HV].t0;
    issue(u, cur_len, cur_t0);
    for (; u < nunits; u += gridDim.x) {
        const int hv = u % HV, Cn = cur_len;
        const long t0 = cur_t0;
        const int un = u + (int)gridDim.x;
        const int nxt_len = un < nunits ? info[un / HV].len : 1;
        const long nxt_t0 = un < nunits ? info[un / HV].t0 : 0;

        // ---- stage Q, K (rows past the chunk zero), W, U, h[c] (as [V][K] rows), G
        if (threadIdx.x < C) sG[threadIdx.x] = rg;
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const int idx = threadIdx.x + NT * i, r = idx / (KD / EPE), c = (idx % (KD / EPE)) * EPE;
            VS yq, yk;
#pragma unroll
            for (int e = 0; e < EPE; e++) {
                yq[e] = r < Cn ? (S)(float)rq[i][e] : (S)0.f;
                yk[e] = r < Cn ? (S)(float)rk[i][e] : (S)0.f;
            }
            *(VS*)(sQ + r * LK + c) = yq;
            *(VS*)(sK + r * LK + c) = yk;
            *(VS*)(sW + r * LK + c) = rw[i];
        }
#pragma unroll
        for (int i = 0; i < NU; i++) {
            const int idx = threadIdx.x + NT * i, r = idx / (VD / EPE), c = (idx % (VD / EPE)) * EPE;
            *(VS*)(sVn + r * LV + c) = ru[i];
        }
#pragma unroll
        for (int i = 0; i < NH; i++) {
            const int c = threadIdx.x + NT * i;
            if constexpr (sizeof(E) == 2) {
                // 16-byte piece c of the state block: column 16 cb + (c % 16) of the
                // key block sb, keys 32 sb + 4 g + {0..3} and 32 sb + 16 + 4 g + {0..3}
                // with g = (c % 64) / 16, cb = (c / 64) / (KD / 32), sb = (c / 64) % (KD / 32)
                const int ln = c & 63, sb = (c >> 6) % (KD / 32), cb = (c >> 6) / (KD / 32);
                const int row = 16 * cb + (ln & 15), key = 32 * sb + 4 * (ln >> 4);
                vec_t<S, 4> lo, hi;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    lo[e] = (S)(float)rh[i][e];
                    hi[e] = (S)(float)rh[i][4 + e];
                }
                *(vec_t<S, 4>*)(sH + row * LK + key) = lo;
                *(vec_t<S, 4>*)(sH + row * LK + key + 16) = hi;
            } else {   // fp32 states are stored [V][K]
                const int row = (c * 4) / KD, key = (c * 4) % KD;
                *(VS*)(sH + row * LK + key) = rh[i];
            }
        }
        lds_barrier();
        // ---- the next unit's loads fly during this unit's compute
        if (un < nunits) issue(un, nxt_len, nxt_t0);

        // ---- Pm = scale · lower(Γ ⊙ Q Kᵀ), Γ[r][c] = exp(G_r − G_c)   (wave w: a 32 x 16 block)
        {
            const int n0 = 16 * (w >> 1);
            f32x4 aqk[2][1];
            zero_acc(aqk);
            wgemm_rf<S, 2, 1, KD, false, false>(aqk, sQ, LK, sK, LK, m0, n0);
            const int c0 = rf_col(n0, 0);
            const f32x4 gc = *(const f32x4*)(sG + c0);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int r = rf_row(m0, i);
                const float gr = sG[r];
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; e++) x[e] = c0 + e <= r ? scale * __expf(gr - gc[e]) * aqk[i][0][e] : 0.f;
                st4<S>(sPm + r * LA + c0, x);
            }
        }
        // ---- W h and Q h   (wave w: 32 rows x VD/4 columns); V_new = U − W h in place
        constexpr int TN = VD / 64;
        const int n0 = (VD / 4) * (w >> 1);
        f32x4 qh[2][TN];
        {
            f32x4 wh[2][TN];
            zero_acc(wh);
            zero_acc(qh);
            wgemm_rf<S, 2, TN, KD, false, false>(wh, sW, LK, sH, LK, m0, n0);
            wgemm_rf<S, 2, TN, KD, false, false>(qh, sQ, LK, sH, LK, m0, n0);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {   // the lane's own elements of U
                    S* p = sVn + rf_row(m0, i) * LV + rf_col(n0, j);
                    st4<S>(p, ld4<S>(p) - wh[i][j]);
                }
        }
        lds_barrier();   // Pm and V_new complete; K is no longer read
        // ---- o = scale · diag(γ) Q h + Pm V_new
        f32x4 ov[2][TN];
        zero_acc(ov);
        wgemm_rf<S, 2, TN, 64, false, true>(ov, sPm, LA, sVn, LV, m0, n0);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r = rf_row(m0, i);
            const float gq = scale * __expf(sG[r]);
#pragma unroll
            for (int j = 0; j < TN; j++) st4<E>(sO + r * LV + rf_col(n0, j), ov[i][j] + gq * qh[i][j]);
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < NU; i++) {
            const int idx = threadIdx.x + NT * i, r = idx / (VD / EPE), c = (idx % (VD / EPE)) * EPE;
            if (r < Cn)
                __builtin_nontemporal_store(*(const VE*)(sO + r * LV + c), (VE*)(o + ((t0 + r) * HV + hv) * VD + c));
        }
        lds_barrier();   // the next unit is staged over this one's LDS
        cur_len = nxt_len;
        cur_t0 = nxt_t0;
    }
}

template <class E, class S, int KD, int VD>
static hipError_t fwd_out_go(const Problem& p, const FwdArgs& a, hipStream_t s) {
    using Cf = FwdCfg<S, KD, VD>;
    auto kern = fwd_out_kernel<E, S, KD, VD>;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem) != hipSuccess)
        return hipErrorInvalidConfiguration;
    const long nunits = p.NT * p.HV;
    if (nunits > INT32_MAX) return hipErrorInvalidValue;
    // one persistent workgroup per CU (the LDS carve-up allows one), 256 CUs
    const unsigned grid = (unsigned)(nunits < 256 ? nunits : 256);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512), Cf::smem, s, (const E*)a.q, (const E*)a.k, a.gcum, a.info,
                       (const S*)a.W, (const S*)a.U, (const E*)a.hT, (E*)a.o, p.HK, p.HV, p.scale, (int)nunits);
    return hipGetLastError();
}

hipError_t launch_fwd_out(const Problem& p, const FwdArgs& a, hipStream_t s) {
    if (p.K == 128 && p.V == 128) {
        if (p.dtype == 2) return fwd_out_go<bf16, f16, 128, 128>(p, a, s);
        if (p.dtype == 1) return fwd_out_go<f16, f16, 128, 128>(p, a, s);
        return hipErrorInvalidValue;
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 2) return fwd_out_go<bf16, f16, 64, 64>(p, a, s);
        if (p.dtype == 1) return fwd_out_go<f16, f16, 64, 64>(p, a, s);
        return fwd_out_go<float, float, 64, 64>(p, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
