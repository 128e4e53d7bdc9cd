// kda_bwd.hip -- the KDA (per-channel gate) WY backward stage.
//
// Page: "chunk_kda_bwd_wy_dqkg_fused 算子" (MindSpeed-Ops).  Its 实现原理
// section splits the work per (chunk, batch·head) and names the intermediates
// dq = do·hᵀ, dk = v_new·dhᵀ, dw = −dv·hᵀ, then the gate/β/A corrections; its
// 多阶段 kernel table adds the A·dw corrections of dk/dg/db, a masked dA_pre
// and dA = −A(dA_pre·A).  Read with A as the chunk's lower-triangular WY
// inverse (the page's A being its transpose), these are the exact gradients of
//   Φ = scale<dO,(Q⊙γ)h> + <dh,(K⊙γ_C/γ)ᵀV_new> + <dh,diag(γ_C)h>
//       + <dv, A(β⊙V) − A(β⊙γ⊙K)h>,        γ = e^g (per channel)
// with respect to q, k, v, β, g and the strictly-lower L of A = (I+L)^{-1}:
//   dq  = scale (dO hᵀ) ⊙ γ,   dks = (V_new dhᵀ) ⊙ γ_C/γ,   dw = −dv hᵀ
//   dv' = β ⊙ Aᵀ dv,   dk = dks + βγ ⊙ Aᵀdw
//   db  = rowsum(Aᵀdv ⊙ V) + rowsum(Aᵀdw ⊙ γ ⊙ K)
//   dg  = Q⊙dq − K⊙dks + βγ⊙K⊙Aᵀdw,  last row + colsum(K⊙dks) + γ_C⊙rowsum(h⊙dh)
//   dA  = −strictlower(Aᵀ dA_pre Aᵀ),  dA_pre = dv(β⊙V)ᵀ + dw(β⊙γ⊙K)ᵀ
// The page runs this as six Ascend kernels to avoid the BT x BT post-processing
// in one kernel; with 160 KB of LDS per CU it is one gfx950 kernel here.
// One workgroup (8 waves) per (chunk, head); operands in the input type
// (fp16 MFMA for fp16, fp32 MFMA for fp32) with fp32 accumulation.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <class E> constexpr int kpad() { return sizeof(E) == 2 ? 8 : 4; }

template <class E, int KD, int VD>
struct KdaCfg {
    static constexpr int C = 64;
    static constexpr int LK = KD + kpad<E>(), LV = VD + kpad<E>(), LA = 64 + kpad<E>();
    static constexpr int TN = KD / 64;       // [64][KD] outputs: 2 row tiles x TN col tiles per wave
    static constexpr size_t oH = 0;                                          // h  [KD][LV]  (later dh)
    static constexpr size_t oX = oH + (size_t)KD * LV * sizeof(E);           // dO [64][LV]  (later V_new)
    static constexpr size_t oDV = oX + (size_t)C * LV * sizeof(E);           // dv_in [64][LV]
    static constexpr size_t oA = oDV + (size_t)C * LV * sizeof(E);           // A [64][LA]
    static constexpr size_t oDW = oA + (size_t)C * LA * sizeof(E);           // dw [64][LK]
    static constexpr size_t oKb = oDW + (size_t)C * LK * sizeof(E);          // β γ K [64][LK]
    static constexpr size_t oVb = oKb + (size_t)C * LK * sizeof(E);          // β V [64][LV]
    static constexpr size_t oP = oVb + (size_t)C * LV * sizeof(E);           // dA_pre, then M1 [64][LA]
    static constexpr size_t oSm = oP + (size_t)C * LA * sizeof(E);
    static constexpr int NCS = 2 * KD > 256 ? 2 * KD : 256;   // column partials [2][KD], later db partials [4][64]
    static constexpr size_t smem = oSm + (size_t)(64 + KD + NCS) * 4;
};

__device__ __forceinline__ void kda_find_chunk(const int32_t* __restrict__ cu, int N, int T, int BT, int ci, int& t0,
                                               int& len) {
    if (!cu) {
        const int ncs = (T + BT - 1) / BT, b = ci / ncs, c = ci % ncs;
        t0 = b * T + c * BT;
        len = min(BT, T - c * BT);
        return;
    }
    int base = 0;
    for (int n = 0; n < N; n++) {
        const int l = cu[n + 1] - cu[n], nc = (l + BT - 1) / BT;
        if (ci < base + nc) {
            const int c = ci - base;
            t0 = cu[n] + c * BT;
            len = min(BT, l - c * BT);
            return;
        }
        base += nc;
    }
    t0 = 0;
    len = 0;
}

template <class T, int N> using kdv = T __attribute__((ext_vector_type(N)));

// Register staging of a [64][D] row tile of a token-major tensor (row stride
// rs elements): issue() loads 16-byte vectors (rows at or past Cn read row
// Cn-1, a valid row), store() writes them to LDS (row pitch LD) with those
// rows zeroed.  Splitting the two lets every load of a unit be in flight
// before the first wait.
template <class T, int D>
struct KRows {
    static constexpr int EPV = 16 / (int)sizeof(T), VPR = D / EPV, N = 64 * VPR / 512;
    static_assert(64 * VPR % 512 == 0, "whole vectors per thread");
    kdv<T, EPV> v[N];
    __device__ __forceinline__ static int row(int i) { return ((int)threadIdx.x + 512 * i) / VPR; }
    __device__ __forceinline__ static int col(int i) { return ((int)threadIdx.x + 512 * i) % VPR * EPV; }
    __device__ __forceinline__ void issue(const T* __restrict__ g, long rs, int Cn) {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = *(const kdv<T, EPV>*)(g + min(row(i), Cn - 1) * rs + col(i));
    }
    template <int LD>
    __device__ __forceinline__ void store(T* s, int Cn) const {
#pragma unroll
        for (int i = 0; i < N; i++) {
            kdv<T, EPV> y = v[i];
            if (row(i) >= Cn) y = kdv<T, EPV>{};
            *(kdv<T, EPV>*)(s + row(i) * LD + col(i)) = y;
        }
    }
};

template <class E, int KD, int VD, int LD>
struct KdaStateRegs {
    static constexpr int VPR = VD / 4, NS = KD * VPR / 512;
    static_assert(KD * VPR % 512 == 0, "whole vectors per thread");
    f32x4 v[NS];
    __device__ __forceinline__ void issue(const float* __restrict__ g) {
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int idx = threadIdx.x + 512 * i, r = idx / VPR, c = idx % VPR;
            v[i] = *(const f32x4*)(g + (long)r * VD + c * 4);
        }
    }
    __device__ __forceinline__ void store(E* s) const {
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int idx = threadIdx.x + 512 * i, r = idx / VPR, c = idx % VPR;
            kdv<E, 4> y;
#pragma unroll
            for (int e = 0; e < 4; e++) y[e] = (E)v[i][e];
            *(kdv<E, 4>*)(s + r * LD + c * 4) = y;
        }
    }
};

template <class E, int KD, int VD>
__global__ void __launch_bounds__(512) kda_kernel(KdaArgs a, const int32_t* __restrict__ cu, int N, int T, int H,
                                                  float scale) {
    using Cf = KdaCfg<E, KD, VD>;
    constexpr int C = 64, LK = Cf::LK, LV = Cf::LV, LA = Cf::LA, TN = Cf::TN;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sH = (E*)(smem + Cf::oH);
    E* sX = (E*)(smem + Cf::oX);
    E* sDV = (E*)(smem + Cf::oDV);
    E* sA = (E*)(smem + Cf::oA);
    E* sDW = (E*)(smem + Cf::oDW);
    E* sKb = (E*)(smem + Cf::oKb);
    E* sVb = (E*)(smem + Cf::oVb);
    E* sP = (E*)(smem + Cf::oP);
    float* sB = (float*)(smem + Cf::oSm);
    float* sHD = sB + 64;        // rowsum_V(h ⊙ dh), per key
    float* sCS = sHD + KD;       // [2][KD] column partials of K ⊙ dks

    const int ci = blockIdx.x, hh = blockIdx.y;
    int t0i, Cn;
    kda_find_chunk(cu, N, T, 64, ci, t0i, Cn);
    const long t0 = t0i;
    const int w = wave_id();
    const int m0 = 32 * (w & 1), n0k = (KD / 4) * (w >> 1), n0s = 16 * (w >> 1);
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* vn = (const E*)a.v_new;
    const E* dO = (const E*)a.dO;
    const E* dvi = (const E*)a.dv_in;
    const E* Ain = (const E*)a.A;
    const E* beta = (const E*)a.beta;
    const long unit = (long)ci * H + hh;
    const float* hg = a.h + unit * KD * VD;
    const float* dhg = a.dh + unit * KD * VD;
    auto gidx = [&](int r, int c) { return ((t0 + r) * H + hh) * (long)KD + c; };   // [.,H,KD] element

    // ---- every global load of the unit is issued first, in a pinned order
    //      (β; h, dO, dv_in, A; K with its gates, V; dh, V_new), then staged
    //      into LDS as the phases below need it
    constexpr int EPE = 16 / (int)sizeof(E), NKV = C * KD / EPE / 512;
    const E bb = beta[(t0 + min((int)threadIdx.x & (C - 1), Cn - 1)) * H + hh];
    __builtin_amdgcn_sched_barrier(0);
    KdaStateRegs<E, KD, VD, LV> hreg;   // h stays in registers for rowsum_V(h ⊙ dh)
    hreg.issue(hg);
    KRows<E, VD> rdo, rdv;
    rdo.issue(dO + (t0 * H + hh) * VD, (long)H * VD, Cn);
    rdv.issue(dvi + (t0 * H + hh) * VD, (long)H * VD, Cn);
    KRows<E, 64> ra;
    ra.issue(Ain + (t0 * H + hh) * 64, (long)H * 64, Cn);
    __builtin_amdgcn_sched_barrier(0);
    kdv<E, EPE> rkv[NKV];
    f32x4 rgv[NKV][EPE / 4];
#pragma unroll
    for (int i = 0; i < NKV; i++) {
        const int idx = threadIdx.x + 512 * i, r = idx / (KD / EPE), c = (idx % (KD / EPE)) * EPE, rc = min(r, Cn - 1);
        rkv[i] = *(const kdv<E, EPE>*)(k + gidx(rc, c));
#pragma unroll
        for (int e4 = 0; e4 < EPE; e4 += 4) rgv[i][e4 / 4] = *(const f32x4*)(a.g + gidx(rc, c + e4));
    }
    KRows<E, VD> rv;
    rv.issue(v + (t0 * H + hh) * VD, (long)H * VD, Cn);
    __builtin_amdgcn_sched_barrier(0);
    KdaStateRegs<E, KD, VD, LV> dhreg;
    dhreg.issue(dhg);
    KRows<E, VD> rvn;
    rvn.issue(vn + (t0 * H + hh) * VD, (long)H * VD, Cn);
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage h, dO, dv_in, A (lower triangle), β
    if (threadIdx.x < C) sB[threadIdx.x] = (int)threadIdx.x < Cn ? (float)bb : 0.f;
    hreg.store(sH);
    rdo.template store<LV>(sX, Cn);
    rdv.template store<LV>(sDV, Cn);
#pragma unroll
    for (int i = 0; i < KRows<E, 64>::N; i++) {
        const int r = KRows<E, 64>::row(i), c = KRows<E, 64>::col(i);
        kdv<E, KRows<E, 64>::EPV> y;
#pragma unroll
        for (int e = 0; e < KRows<E, 64>::EPV; e++) y[e] = (r < Cn && c + e <= r) ? ra.v[i][e] : (E)0.f;
        *(kdv<E, KRows<E, 64>::EPV>*)(sA + r * LA + c) = y;
    }
    lds_barrier();
    {   // β γ K and β V
#pragma unroll
        for (int i = 0; i < NKV; i++) {
            const int idx = threadIdx.x + 512 * i, r = idx / (KD / EPE), c = (idx % (KD / EPE)) * EPE;
            kdv<E, EPE> y;
#pragma unroll
            for (int e4 = 0; e4 < EPE; e4 += 4)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    y[e4 + e] = (E)(r < Cn ? sB[r] * __expf(rgv[i][e4 / 4][e]) * (float)rkv[i][e4 + e] : 0.f);
            *(kdv<E, EPE>*)(sKb + r * LK + c) = y;
        }
#pragma unroll
        for (int i = 0; i < KRows<E, VD>::N; i++) {
            const int r = KRows<E, VD>::row(i), c = KRows<E, VD>::col(i);
            kdv<E, EPE> y;
#pragma unroll
            for (int e = 0; e < EPE; e++) y[e] = (E)(r < Cn ? sB[r] * (float)rv.v[i][e] : 0.f);
            *(kdv<E, EPE>*)(sVb + r * LV + c) = y;
        }
    }

    // ---- dq_acc = dO hᵀ,  dw = −dv hᵀ      (B = hᵀ: h stored [key][v] = [n][k])
    f32x4 dqa[2][TN], dwa[2][TN];
    zero_acc(dqa);
    zero_acc(dwa);
    wgemm_rf<E, 2, TN, VD, false, false>(dqa, sX, LV, sH, LV, m0, n0k);
    wgemm_rf<E, 2, TN, VD, false, false>(dwa, sDV, LV, sH, LV, m0, n0k);
    lds_barrier();
    // ---- swap in dh and V_new; dw -> LDS; rowsum_V(h ⊙ dh) in fp32 from the registers
    {
        dhreg.store(sH);
        constexpr int VPR = KdaStateRegs<E, KD, VD, LV>::VPR;   // lanes per key row (16 or 32)
#pragma unroll
        for (int i = 0; i < KdaStateRegs<E, KD, VD, LV>::NS; i++) {
            float x = 0.f;
#pragma unroll
            for (int e = 0; e < 4; e++) x += hreg.v[i][e] * dhreg.v[i][e];
#pragma unroll
            for (int off = 1; off < VPR; off <<= 1) x += __shfl_xor(x, off, 64);
            // all VPR lanes of the row hold the sum and write it
            sHD[(threadIdx.x + 512 * i) / VPR] = x;
        }
    }
    rvn.template store<LV>(sX, Cn);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) st4<E>(sDW + rf_row(m0, i) * LK + rf_col(n0k, j), -dwa[i][j]);
    lds_barrier();
    // ---- this lane's elements of g, k, q (key tiles) and v (value tiles), issued
    //      before the products that precede their use (rows past the chunk read
    //      its last row and are not used).  Row form: a lane's elements of a tile
    //      are four adjacent columns of one row (one 16-byte or 8-byte load).
    constexpr int TNV = VD / 64;
    const int n0v = (VD / 4) * (w >> 1);
    f32x4 pg[2][TN], pk[2][TN], pq[2][TN], pv[2][TNV], pgl[TN];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int rc = min(rf_row(m0, i), Cn - 1);
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const long o = gidx(rc, rf_col(n0k, j));
            pg[i][j] = *(const f32x4*)(a.g + o);
            pk[i][j] = ld4<E>(k + o);
            pq[i][j] = ld4<E>(q + o);
        }
#pragma unroll
        for (int j = 0; j < TNV; j++) pv[i][j] = ld4<E>(v + ((t0 + rc) * H + hh) * VD + rf_col(n0v, j));
    }
#pragma unroll
    for (int j = 0; j < TN; j++) pgl[j] = *(const f32x4*)(a.g + gidx(Cn - 1, rf_col(n0k, j)));
    // ---- dks_acc = V_new dhᵀ ; AdW = Aᵀ dw ; AdV = Aᵀ dv (V-tiles)
    f32x4 dka[2][TN], adw[2][TN];
    zero_acc(dka);
    zero_acc(adw);
    wgemm_rf<E, 2, TN, VD, false, false>(dka, sX, LV, sH, LV, m0, n0k);
    wgemm_rf<E, 2, TN, 64, true, true>(adw, sA, LA, sDW, LK, m0, n0k);
    // dv_out = β Aᵀ dv, db part 1 = rowsum(Aᵀdv ⊙ V)
    float dbr[2] = {0.f, 0.f};
    {
        f32x4 adv[2][TNV];
        zero_acc(adv);
        wgemm_rf<E, 2, TNV, 64, true, true>(adv, sA, LA, sDV, LV, m0, n0v);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rf_row(m0, i);
            if (rr < Cn) {
#pragma unroll
                for (int j = 0; j < TNV; j++) {
                    st4<E>((E*)a.dv_out + ((t0 + rr) * H + hh) * VD + rf_col(n0v, j), sB[rr] * adv[i][j]);
#pragma unroll
                    for (int e = 0; e < 4; e++) dbr[i] += adv[i][j][e] * pv[i][j][e];
                }
            }
        }
    }
    // ---- per-element outputs dq, dk and dg (last-row terms after the column sums)
    float csum[TN][4];
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) csum[j][e] = 0.f;
    f32x4 dgl[2][TN];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int rr = rf_row(m0, i);
#pragma unroll
        for (int j = 0; j < TN; j++) {
            dgl[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rr < Cn) {
                const long o = gidx(rr, rf_col(n0k, j));
                f32x4 dqv, dkv;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float gg = pg[i][j][e], gm = __expf(gg);
                    const float kk = pk[i][j][e], qq = pq[i][j][e];
                    dqv[e] = scale * dqa[i][j][e] * gm;
                    const float dks = dka[i][j][e] * __expf(pgl[j][e] - gg);
                    const float bgw = sB[rr] * gm * adw[i][j][e];
                    dkv[e] = dks + bgw;
                    dgl[i][j][e] = qq * dqv[e] - kk * dks + kk * bgw;
                    csum[j][e] += kk * dks;
                    dbr[i] += adw[i][j][e] * gm * kk;
                }
                *(f32x4*)(a.dq + o) = dqv;
                *(f32x4*)(a.dk + o) = dkv;
            }
        }
    }
    // column sums over this wave's 32 rows (the 16 lanes of a row group hold 16
    // rows of the same four columns) -> sCS[row half][key]
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float x = csum[j][e];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
            sCS[(w & 1) * KD + rf_col(n0k, j) + e] = x;   // every lane of the group holds the sum (no branch)
        }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int rr = rf_row(m0, i);
        if (rr < Cn) {
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int c0 = rf_col(n0k, j);
                f32x4 x = dgl[i][j];
                if (rr == Cn - 1)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        x[e] += sCS[c0 + e] + sCS[KD + c0 + e] + __expf(pg[i][j][e]) * sHD[c0 + e];
                *(f32x4*)(a.dg + gidx(rr, c0)) = x;
            }
        }
    }
    // ---- dA_pre = dv (βV)ᵀ + dw (βγK)ᵀ -> LDS (B operands stored [s][.] = [n][k])
    {
        f32x4 dap[2][1];
        zero_acc(dap);
        wgemm_rf<E, 2, 1, VD, false, false>(dap, sDV, LV, sVb, LV, m0, n0s);
        wgemm_rf<E, 2, 1, KD, false, false>(dap, sDW, LK, sKb, LK, m0, n0s);
#pragma unroll
        for (int i = 0; i < 2; i++) st4<E>(sP + rf_row(m0, i) * LA + rf_col(n0s, 0), dap[i][0]);
    }
    // db: reduce over the 4 row groups (lanes 16 apart hold the same row), then
    // over the 4 column blocks
    float* sDB = sCS;   // reuse [4][64] (column sums already consumed above)
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        float x = dbr[i];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        sDB[(w >> 1) * 64 + rf_row(m0, i)] = x;   // the four row groups hold the sum and write it
    }
    // ---- M1 = Aᵀ dA_pre
    f32x4 m1[2][1];
    zero_acc(m1);
    wgemm_rf<E, 2, 1, 64, true, true>(m1, sA, LA, sP, LA, m0, n0s);
    lds_barrier();
    if (threadIdx.x < Cn) {
        const int rr = threadIdx.x;
        a.db[(t0 + rr) * H + hh] = sDB[rr] + sDB[64 + rr] + sDB[128 + rr] + sDB[192 + rr];
    }
#pragma unroll
    for (int i = 0; i < 2; i++) st4<E>(sP + rf_row(m0, i) * LA + rf_col(n0s, 0), m1[i][0]);
    lds_barrier();
    // ---- dA = −strictlower(M1 Aᵀ)   (B = Aᵀ: A stored [s][j] = [n][k])
    {
        f32x4 da[2][1];
        zero_acc(da);
        wgemm_rf<E, 2, 1, 64, false, false>(da, sP, LA, sA, LA, m0, n0s);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rf_row(m0, i), c0 = rf_col(n0s, 0);
            if (rr < Cn) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; e++) x[e] = (c0 + e < rr) ? -da[i][0][e] : 0.f;
                *(f32x4*)(a.dA + ((t0 + rr) * H + hh) * 64 + c0) = x;
            }
        }
    }
}

template <class E, int KD, int VD>
static hipError_t kda_go(const Problem& p, const KdaArgs& a, hipStream_t s) {
    using Cf = KdaCfg<E, KD, VD>;
    auto kern = kda_kernel<E, KD, VD>;
    static_assert(Cf::smem <= 160 * 1024, "LDS budget");
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem) != hipSuccess)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.NT, p.HV), dim3(512), Cf::smem, s, a, p.cu, p.N, p.T, p.HV, p.scale);
    return hipGetLastError();
}

hipError_t launch_kda(const Problem& p, const KdaArgs& a, hipStream_t s) {
    if (p.K == 128 && p.V == 128) {
        if (p.dtype == 1) return kda_go<f16, 128, 128>(p, a, s);
        return hipErrorInvalidValue;
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 1) return kda_go<f16, 64, 64>(p, a, s);
        return kda_go<float, 64, 64>(p, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
