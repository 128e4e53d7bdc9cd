// kda_full.hip -- the full chunked backward of KDA (the gated delta rule with a
// per-channel gate), built around the WY stage of kda_bwd.hip.
//
// Page: "chunk_kda_bwd_wy_dqkg_fused 算子" (MindSpeed-Ops) -- 概述 places that
// operator inside the KDA chunk backward as its WY-representation gradient
// step; the other steps of that backward are the state recomputation, the
// per-channel dh scan and the intra-chunk attention / dL distribution written
// out here.
//
// Per chunk (C <= 64 rows), with G the in-chunk cumulative per-channel
// log-gate (C x K), γ = e^G, γ_C its last row, and h the state entering it:
//   Akk[r][s] = Σ_d k_r[d] k_s[d] e^{G_r[d] − G_s[d]},   L = strictlower(diag(β) Akk)
//   Aqk[r][s] = scale Σ_d q_r[d] k_s[d] e^{G_r[d] − G_s[d]}  (s <= r)
//   A = (I + L)^{-1},  W = A diag(β)(K ⊙ γ),  U = A diag(β) V,  K̃ = K ⊙ γ_C/γ
//   V_new = U − W h,   h' = diag(γ_C) h + K̃ᵀ V_new,   o = scale (Q ⊙ γ) h + Aqk V_new
// Backward (dh' the gradient of the state leaving the chunk):
//   dV_new = Aqkᵀ dO + K̃ dh'
//   dh     = diag(γ_C) dh' + scale (Q ⊙ γ)ᵀ dO − Wᵀ dV_new          (reverse scan)
//   WY stage (kda_bwd.hip): dq, dk, dv, dβ, dG partials and dL = dA
//   intra:  dAqk = lower(dO V_newᵀ)
//           dq += scale e^{G−m} ⊙ (dAqk (K ⊙ e^{m−G}))
//           dk += scale e^{m−G} ⊙ (dAqkᵀ (Q ⊙ e^{G−m}))
//                 + β ⊙ e^{G−m} ⊙ (dL (K ⊙ e^{m−G})) + e^{m−G} ⊙ (dLᵀ (β ⊙ K ⊙ e^{G−m}))
//           dG += Q ⊙ dq_intra − K ⊙ dk_qk + K ⊙ dk_row − K ⊙ dk_col
//           dβ += rowsum(K ⊙ e^{G−m} ⊙ (dL (K ⊙ e^{m−G})))
//   dg = in-chunk reverse cumsum of dG (per channel).
// m is the gate row in the middle of the chunk: e^{G_r − G_s} is formed as
// e^{G_r − m} e^{m − G_s}, each factor within e^{±(half the chunk's gate span)},
// so the gated products are plain fp32 MFMA contractions (the factors exceed
// the fp16 range).  Precondition: each channel's in-chunk gate span stays
// below about 170 (fp32 range of the factors).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"
#include "gdr_tri.hpp"

namespace gdr {

namespace {
template <class T, int N> using kvec = T __attribute__((ext_vector_type(N)));
template <class S> constexpr int kfpad() { return sizeof(S) == 2 ? 8 : 4; }

// fp32 slices of 32 channels: [64 rows][KSL + 4]
constexpr int KSL = 32, LSL = KSL + 4;
// value columns per state-scan workgroup
constexpr int KVS = 32;

// LDS carve-up of the KDA WY-factor kernel.
template <class S, int KD, int VD>
struct KPrepCfg {
    static constexpr int C = 64, LK = KD + kfpad<S>(), LV = VD + kfpad<S>(), LA = 64 + kfpad<S>(), LL = 68;
    static constexpr size_t oK = 0;                                        // K [64][LK] S (later W)
    static constexpr size_t oQ = oK + (size_t)C * LK * sizeof(S);          // Q [64][LK] S (later K ⊙ γ)
    static constexpr size_t oV = oQ + (size_t)C * LK * sizeof(S);          // V [64][LV] S (later U)
    static constexpr size_t oSl = oV + (size_t)C * LV * sizeof(S);         // 3 fp32 slices [64][LSL]
    static constexpr size_t oL = oSl + (size_t)3 * C * LSL * 4;            // L [64][LL] fp32
    static constexpr size_t oAf = oL + (size_t)C * LL * 4;                 // A [64][LL] fp32
    static constexpr size_t oAb = oAf + (size_t)C * LL * 4;                // A diag(β) [64][LA] S
    static constexpr size_t oT = oAb + (size_t)C * LA * sizeof(S);         // inverse scratch
    static constexpr size_t oB = oT + (size_t)4 * 2 * 16 * 17 * 4;        // β [64], m [KD]
    static constexpr size_t smem = oB + (size_t)(64 + KD) * 4;
    static_assert(smem <= 160 * 1024, "LDS budget");
};
}  // namespace

// ---------------------------------------------------------------- WY factors
// One workgroup per (chunk, head), the heads of a chunk on consecutive
// workgroups; 512 threads (8 waves: wave w owns rows 16 (w & 3) .. +15
// and column half w >> 2 of every product; the triangular inverse runs on
// waves 0..3).  Writes, per unit u = chunk * H + head:
// W, K̃, Qg = scale (Q ⊙ γ) as [u][64][KD], U as [u][64][VD], Aqk as
// [u][64][64] (operand type S), and A in the input type as [B*T, H, 64].
template <class E, class S, int KD, int VD>
__global__ void __launch_bounds__(512) kda_prep_kernel(KdaFullArgs a, int H, float scale) {
    using Cf = KPrepCfg<S, KD, VD>;
    constexpr int C = 64, NT = 512, LK = Cf::LK, LV = Cf::LV, LA = Cf::LA, LL = Cf::LL;
    constexpr int EPE = 16 / (int)sizeof(E);
    extern __shared__ __align__(16) unsigned char smem[];
    S* sK = (S*)(smem + Cf::oK);
    S* sQ = (S*)(smem + Cf::oQ);
    S* sV = (S*)(smem + Cf::oV);
    float* sKp = (float*)(smem + Cf::oSl);   // slices: K e^{G−m} (or Q e^{G−m}), K e^{m−G}
    float* sKm = sKp + C * LSL;
    float* sQp = sKm + C * LSL;
    float* sL = (float*)(smem + Cf::oL);
    float* sAf = (float*)(smem + Cf::oAf);
    S* sAb = (S*)(smem + Cf::oAb);
    float* sT = (float*)(smem + Cf::oT);
    float* sB = (float*)(smem + Cf::oB);
    float* sM = sB + 64;

    const int ci = (int)blockIdx.x / H, h = (int)blockIdx.x % H, w = wave_id();   // heads fastest
    const int m0 = 16 * (w & 3), hc = w >> 2;   // row group, column half
    const int Cn = a.info[ci].len;
    const long t0 = a.info[ci].t0;
    const long unit = (long)ci * H + h;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const float* G = a.gcum;
    const int ref = (Cn - 1) / 2;

    // ---- every load of the staging phase, then slice 0's G rows, in this order
    constexpr int NKV = C * KD / EPE / NT, NVV = C * VD / EPE / NT;   // K / Q and V vectors per thread
    static_assert(C * KD / EPE % NT == 0 && C * VD / EPE % NT == 0 && C * KSL / 4 == NT, "whole vectors per thread");
    const float bb = (float)((const E*)a.beta)[(t0 + min((int)threadIdx.x & (C - 1), Cn - 1)) * H + h];
    const float mm = G[((t0 + ref) * H + h) * KD + min((int)threadIdx.x, KD - 1)];
    __builtin_amdgcn_sched_barrier(0);
    kvec<E, EPE> xk[NKV], xq[NKV], xv[NVV];
#pragma unroll
    for (int i = 0; i < NKV; i++) {
        const int idx = threadIdx.x + NT * i, r = idx / (KD / EPE), c = idx % (KD / EPE) * EPE;
        const long o = ((t0 + min(r, Cn - 1)) * H + h) * KD + c;
        xk[i] = __builtin_nontemporal_load((const kvec<E, EPE>*)(k + o));
        xq[i] = __builtin_nontemporal_load((const kvec<E, EPE>*)(q + o));
    }
#pragma unroll
    for (int i = 0; i < NVV; i++) {
        const int idx = threadIdx.x + NT * i, r = idx / (VD / EPE), c = idx % (VD / EPE) * EPE;
        xv[i] = __builtin_nontemporal_load((const kvec<E, EPE>*)(v + ((t0 + min(r, Cn - 1)) * H + h) * VD + c));
    }
    // One slice vector per thread: row sr, channels sdd .. +3 of the slice;
    // G of that row and of the chunk's last row.
    const int sr = threadIdx.x / (KSL / 4), sdd = threadIdx.x % (KSL / 4) * 4;
    const long so = ((t0 + min(sr, Cn - 1)) * H + h) * KD + sdd, co = ((t0 + Cn - 1) * H + h) * KD + sdd;
    f32x4 xg = *(const f32x4*)(G + so), xc = *(const f32x4*)(G + co);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NKV; i++) {
        const int idx = threadIdx.x + NT * i, r = idx / (KD / EPE), c = idx % (KD / EPE) * EPE;
        kvec<S, EPE> yk, yq;
#pragma unroll
        for (int e = 0; e < EPE; e++) {
            yk[e] = r < Cn ? (S)(float)xk[i][e] : (S)0.f;
            yq[e] = r < Cn ? (S)(float)xq[i][e] : (S)0.f;
        }
        *(kvec<S, EPE>*)(sK + r * LK + c) = yk;
        *(kvec<S, EPE>*)(sQ + r * LK + c) = yq;
    }
#pragma unroll
    for (int i = 0; i < NVV; i++) {
        const int idx = threadIdx.x + NT * i, r = idx / (VD / EPE), c = idx % (VD / EPE) * EPE;
        kvec<S, EPE> yv;
#pragma unroll
        for (int e = 0; e < EPE; e++) yv[e] = r < Cn ? (S)(float)xv[i][e] : (S)0.f;
        *(kvec<S, EPE>*)(sV + r * LV + c) = yv;
    }
    if (threadIdx.x < C) sB[threadIdx.x] = (int)threadIdx.x < Cn ? bb : 0.f;
    if (threadIdx.x < KD) sM[threadIdx.x] = mm;
    lds_barrier();

    // ---- per 32-channel slice: the fp32 operands K e^{G−m}, K e^{m−G}, Q e^{G−m}
    //      of Akk and Aqk; K̃ = K ⊙ e^{G_C − G} and Qg = scale Q ⊙ e^G (straight
    //      to memory); K ⊙ γ over Q's buffer (each thread rewrites only the Q
    //      elements it has just read).  Akk, Aqk accumulate in fp32 MFMA
    //      (wave w: rows m0, columns 32 hc .. +31).
    f32x4 akk[1][2], aqk[1][2];
    zero_acc(akk);
    zero_acc(aqk);
    S* KTo = (S*)a.KT + unit * C * KD + sr * KD + sdd;
    S* QGo = (S*)a.QG + unit * C * KD + sr * KD + sdd;
#pragma unroll 1
    for (int s0 = 0; s0 < KD; s0 += KSL) {
        {
            const int d = s0 + sdd;
            const f32x4 m = *(const f32x4*)(sM + d);
            const kvec<S, 4> kv = *(const kvec<S, 4>*)(sK + sr * LK + d), qv = *(const kvec<S, 4>*)(sQ + sr * LK + d);
            f32x4 kp, km, qp;
            kvec<S, 4> kt, qg, kg;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float ep = __expf(xg[e] - m[e]), em = __expf(m[e] - xg[e]), eg = __expf(xg[e]);
                kp[e] = (float)kv[e] * ep;
                km[e] = (float)kv[e] * em;
                qp[e] = (float)qv[e] * ep;
                kt[e] = (S)((float)kv[e] * __expf(xc[e] - xg[e]));
                qg[e] = (S)(scale * (float)qv[e] * eg);
                kg[e] = (S)((float)kv[e] * eg);
            }
            *(f32x4*)(sKp + sr * LSL + sdd) = kp;
            *(f32x4*)(sKm + sr * LSL + sdd) = km;
            *(f32x4*)(sQp + sr * LSL + sdd) = qp;
            *(kvec<S, 4>*)(sQ + sr * LK + d) = kg;
            *(kvec<S, 4>*)(KTo + s0) = kt;
            *(kvec<S, 4>*)(QGo + s0) = qg;
        }
        if (s0 + KSL < KD) {   // the next slice's G rows, in flight during the products
            xg = *(const f32x4*)(G + so + s0 + KSL);
            xc = *(const f32x4*)(G + co + s0 + KSL);
        }
        lds_barrier();
        wgemm<float, 1, 2, KSL, false, false>(akk, sKp, LSL, sKm, LSL, m0, 32 * hc);
        wgemm<float, 1, 2, KSL, false, false>(aqk, sQp, LSL, sKm, LSL, m0, 32 * hc);
        lds_barrier();
    }
    // ---- L = strictlower(diag(β) Akk) -> LDS;  Aqk (scaled, lower incl. diagonal) -> memory
    {
        S* Ao = (S*)a.Aqk + unit * C * C;
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = acc_row(m0, 0, e), c = acc_col(32 * hc, j);
                sL[r * LL + c] = c < r ? sB[r] * akk[0][j][e] : 0.f;
                Ao[r * C + c] = (S)(c <= r ? scale * aqk[0][j][e] : 0.f);
            }
    }
    lds_barrier();
    tri_inverse64<LL, NT>(sL, sAf, sT);

    // ---- A diag(β) as an MFMA operand; A itself to memory (input type, [B*T, H, 64])
    for (int idx = threadIdx.x; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        const float x = sAf[r * LL + c];
        sAb[r * LA + c] = (S)(x * sB[c]);
        if (r < Cn) ((E*)a.A)[((t0 + r) * H + h) * C + c] = (E)x;
    }
    lds_barrier();
    // ---- W = A diag(β) (K ⊙ γ),  U = A diag(β) V   (wave w: rows m0, column half hc)
    {
        f32x4 aw[1][KD / 32], au[1][VD / 32];
        zero_acc(aw);
        zero_acc(au);
        wgemm<S, 1, KD / 32, 64, false, true>(aw, sAb, LA, sQ, LK, m0, (KD / 2) * hc);
        wgemm<S, 1, VD / 32, 64, false, true>(au, sAb, LA, sV, LV, m0, (VD / 2) * hc);
        lds_barrier();   // K and V are overwritten below
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = acc_row(m0, 0, e);
#pragma unroll
            for (int j = 0; j < KD / 32; j++) sK[r * LK + acc_col((KD / 2) * hc, j)] = (S)aw[0][j][e];
#pragma unroll
            for (int j = 0; j < VD / 32; j++) sV[r * LV + acc_col((VD / 2) * hc, j)] = (S)au[0][j][e];
        }
    }
    lds_barrier();
    {
        constexpr int EPS = 16 / (int)sizeof(S);
        S* Wo = (S*)a.W + unit * C * KD;
        S* Uo = (S*)a.U + unit * C * VD;
        for (int idx = threadIdx.x; idx < C * KD / EPS; idx += NT) {
            const int r = idx / (KD / EPS), c = (idx % (KD / EPS)) * EPS;
            *(kvec<S, EPS>*)(Wo + r * KD + c) = *(const kvec<S, EPS>*)(sK + r * LK + c);
        }
        for (int idx = threadIdx.x; idx < C * VD / EPS; idx += NT) {
            const int r = idx / (VD / EPS), c = (idx % (VD / EPS)) * EPS;
            *(kvec<S, EPS>*)(Uo + r * VD + c) = *(const kvec<S, EPS>*)(sV + r * LV + c);
        }
    }
}

// ---------------------------------------------------------------- state scans
// One workgroup (4 waves) per (sequence, head, KVS-column value slice,
// direction); both directions run in one launch (the reverse scan needs
// nothing the forward one writes).  The K x KVS fp32 state slice lives in MFMA
// accumulators (wave w: state rows (KD/4) w ..), a 16-bit copy of it in LDS is
// the operand of the per-chunk products.
//   forward:  stores h[c] (fp32 [NT,H,K,V]) and V_new (input type)
//   reverse:  stores dh[c] (fp32, gradient of the state leaving chunk c),
//             dV_new (input type) and dh0
template <class S, int KD>
struct KScanCfg {
    static constexpr int C = 64, LK = KD + kfpad<S>(), LS = KVS + kfpad<S>(), LA = 64 + kfpad<S>();
    static constexpr size_t oW = 0;                                     // W [64][LK]
    static constexpr size_t oKT = oW + (size_t)C * LK * sizeof(S);      // K̃ [64][LK]
    static constexpr size_t oQG = oKT + (size_t)C * LK * sizeof(S);     // Qg [64][LK] (reverse)
    static constexpr size_t oX = oQG + (size_t)C * LK * sizeof(S);      // U or dO slice [64][LS]
    static constexpr size_t oH = oX + (size_t)C * LS * sizeof(S);       // state copy [KD][LS]
    static constexpr size_t oVn = oH + (size_t)KD * LS * sizeof(S);     // V_new / dV_new slice [64][LS]
    static constexpr size_t oAq = oVn + (size_t)C * LS * sizeof(S);     // Aqk [64][LA] (reverse)
    static constexpr size_t oGC = oAq + (size_t)C * LA * sizeof(S);     // γ_C [KD] fp32
    static constexpr size_t smem = oGC + (size_t)KD * 4;
    static_assert(smem <= 160 * 1024, "LDS budget");
};

template <class E, class S, int KD, int VD, bool REV>
__device__ __forceinline__ void kda_scan_body(const KdaFullArgs& a, int H, int nseq, int job) {
    using Cf = KScanCfg<S, KD>;
    constexpr int C = 64, NT = 256, LK = Cf::LK, LS = Cf::LS, LA = Cf::LA;
    constexpr int TMH = KD / 64;   // 16-row tiles of state rows per wave
    constexpr int NJ = KVS / 16;   // 16-column tiles of the value slice
    constexpr int EPS = 16 / (int)sizeof(S);
    extern __shared__ __align__(16) unsigned char smem[];
    S* sW = (S*)(smem + Cf::oW);
    S* sKT = (S*)(smem + Cf::oKT);
    S* sQG = (S*)(smem + Cf::oQG);
    S* sX = (S*)(smem + Cf::oX);
    S* sH = (S*)(smem + Cf::oH);
    S* sVn = (S*)(smem + Cf::oVn);
    S* sAq = (S*)(smem + Cf::oAq);
    float* sGC = (float*)(smem + Cf::oGC);

    const int nvs = VD / KVS;
    const int vs = job % nvs, h = (job / nvs) % H, n = job / nvs / H;
    if (n >= nseq) return;
    const int w = wave_id();
    const int m0 = (KD / 4) * w;      // this wave's state rows
    const int vc0 = KVS * vs;         // this workgroup's value columns
    const int c_first = a.seq_chunk0[n], c_end = a.seq_chunk0[n + 1];
    const size_t KV = (size_t)KD * VD;

    // state slice: rows m0 + 16 i + 4 g + e, columns 16 j + r
    f32x4 st[TMH][NJ];
    {
        const float* init = REV ? a.dht : a.h0;
#pragma unroll
        for (int i = 0; i < TMH; i++)
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    st[i][j][e] = init ? init[((size_t)n * H + h) * KV + (size_t)acc_row(m0, i, e) * VD + vc0 +
                                              acc_col(0, j)]
                                       : 0.f;
    }
    const int nch = c_end - c_first;
    // operand registers of one chunk: the next chunk's are loaded while the
    // current one is computed
    constexpr int EPE = 16 / (int)sizeof(E);
    static_assert(EPE == EPS, "input and operand types share a width");
    static_assert(C * KD / EPS % NT == 0 && C * KVS / EPS % NT == 0 && C * C / EPS % NT == 0, "whole vectors");
    constexpr int NKW = C * KD / EPS / NT, NXS = C * KVS / EPS / NT, NAQ = C * C / EPS / NT;
    kvec<S, EPS> rW[NKW], rKT[NKW], rQG[REV ? NKW : 1], rU[REV ? 1 : NXS], rAq[REV ? NAQ : 1];
    kvec<E, EPE> rO[REV ? NXS : 1];
    float rgc = 0.f;
    auto chunk_at = [&](int it) { return REV ? c_end - 1 - it : c_first + it; };
    auto issue = [&](int it) {
        const int ci = chunk_at(it);
        const int Cn = a.info[ci].len;
        const long t0 = a.info[ci].t0;
        const long unit = (long)ci * H + h;
#pragma unroll
        for (int i = 0; i < NKW; i++) {
            const long o = unit * C * KD + (long)(threadIdx.x + NT * i) * EPS;
            rW[i] = *(const kvec<S, EPS>*)((const S*)a.W + o);
            rKT[i] = *(const kvec<S, EPS>*)((const S*)a.KT + o);
            if constexpr (REV) rQG[i] = *(const kvec<S, EPS>*)((const S*)a.QG + o);
        }
#pragma unroll
        for (int i = 0; i < NXS; i++) {
            const int idx = threadIdx.x + NT * i, r = idx / (KVS / EPS), c = (idx % (KVS / EPS)) * EPS;
            if constexpr (REV)   // dO slice; rows past the chunk read its last row (zeroed when staged)
                rO[i] = *(const kvec<E, EPE>*)((const E*)a.dO + ((t0 + min(r, Cn - 1)) * H + h) * VD + vc0 + c);
            else
                rU[i] = *(const kvec<S, EPS>*)((const S*)a.U + (unit * C + r) * VD + vc0 + c);
        }
        if constexpr (REV) {
#pragma unroll
            for (int i = 0; i < NAQ; i++)
                rAq[i] = *(const kvec<S, EPS>*)((const S*)a.Aqk + unit * C * C + (long)(threadIdx.x + NT * i) * EPS);
        }
        if (threadIdx.x < KD) rgc = a.gcum[((t0 + Cn - 1) * H + h) * KD + threadIdx.x];
    };
    if (nch > 0) issue(0);
    for (int it = 0; it < nch; it++) {
        const int ci = chunk_at(it);
        const int Cn = a.info[ci].len;
        const long t0 = a.info[ci].t0;
        const long unit = (long)ci * H + h;
        // ---- stage this chunk's operands (from the registers) and the state copy
#pragma unroll
        for (int i = 0; i < NKW; i++) {
            const int idx = threadIdx.x + NT * i, r = idx / (KD / EPS), c = (idx % (KD / EPS)) * EPS;
            *(kvec<S, EPS>*)(sW + r * LK + c) = rW[i];
            *(kvec<S, EPS>*)(sKT + r * LK + c) = rKT[i];
            if constexpr (REV) *(kvec<S, EPS>*)(sQG + r * LK + c) = rQG[i];
        }
#pragma unroll
        for (int i = 0; i < NXS; i++) {
            const int idx = threadIdx.x + NT * i, r = idx / (KVS / EPS), c = (idx % (KVS / EPS)) * EPS;
            kvec<S, EPS> x;
            if constexpr (REV) {
#pragma unroll
                for (int e = 0; e < EPS; e++) x[e] = r < Cn ? (S)(float)rO[i][e] : (S)0.f;
            } else {
                x = rU[i];
            }
            *(kvec<S, EPS>*)(sX + r * LS + c) = x;
        }
        if constexpr (REV) {
#pragma unroll
            for (int i = 0; i < NAQ; i++) {
                const int idx = threadIdx.x + NT * i, r = idx / (C / EPS), c = (idx % (C / EPS)) * EPS;
                *(kvec<S, EPS>*)(sAq + r * LA + c) = rAq[i];
            }
        }
        if (threadIdx.x < KD) sGC[threadIdx.x] = __expf(rgc);
        // state copy as [KD][KVS] and the fp32 state of this chunk boundary to memory
        {
            float* so = (REV ? a.dhs : a.hs) + unit * KV;
#pragma unroll
            for (int i = 0; i < TMH; i++)
#pragma unroll
                for (int j = 0; j < NJ; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int r = acc_row(m0, i, e), c = acc_col(0, j);
                        sH[r * LS + c] = (S)st[i][j][e];
                        so[(size_t)r * VD + vc0 + c] = st[i][j][e];
                    }
        }
        lds_barrier();
        if (it + 1 < nch) issue(it + 1);   // the next chunk's loads fly during this one's products
        // ---- V_new = U − W h   or   dV_new = Aqkᵀ dO + K̃ dh      (wave w: rows 16w, KVS columns)
        {
            f32x4 x[1][NJ];
            zero_acc(x);
            if (REV) {
                wgemm<S, 1, NJ, 64, true, true>(x, sAq, LA, sX, LS, 16 * w, 0);
                wgemm<S, 1, NJ, KD, false, true>(x, sKT, LK, sH, LS, 16 * w, 0);
            } else {
                wgemm<S, 1, NJ, KD, false, true>(x, sW, LK, sH, LS, 16 * w, 0);
            }
            E* out = (E*)(REV ? a.dvn : a.vn);
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = acc_row(16 * w, 0, e), c = acc_col(0, j);
                    const float y = REV ? x[0][j][e] : (float)sX[r * LS + c] - x[0][j][e];
                    const float yv = r < Cn ? y : 0.f;
                    sVn[r * LS + c] = (S)yv;
                    if (r < Cn) out[((t0 + r) * H + h) * VD + vc0 + c] = (E)yv;
                }
        }
        lds_barrier();
        // ---- h ← diag(γ_C) h + K̃ᵀ V_new    or    dh ← diag(γ_C) dh + Qgᵀ dO − Wᵀ dV_new
#pragma unroll
        for (int i = 0; i < TMH; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float gc = sGC[acc_row(m0, i, e)];
#pragma unroll
                for (int j = 0; j < NJ; j++) st[i][j][e] *= gc;
            }
        if (REV) {
            wgemm<S, TMH, NJ, 64, true, true>(st, sQG, LK, sX, LS, m0, 0);
            f32x4 t[TMH][NJ];
            zero_acc(t);
            wgemm<S, TMH, NJ, 64, true, true>(t, sW, LK, sVn, LS, m0, 0);
#pragma unroll
            for (int i = 0; i < TMH; i++)
#pragma unroll
                for (int j = 0; j < NJ; j++) st[i][j] -= t[i][j];
        } else {
            wgemm<S, TMH, NJ, 64, true, true>(st, sKT, LK, sVn, LS, m0, 0);
        }
        lds_barrier();   // the next chunk is staged over this one's LDS
    }
    if (REV && a.dh0) {
#pragma unroll
        for (int i = 0; i < TMH; i++)
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    a.dh0[((size_t)n * H + h) * KV + (size_t)acc_row(m0, i, e) * VD + vc0 + acc_col(0, j)] =
                        st[i][j][e];
    }
}

// blocks [0, jobs): forward scans; [jobs, 2 jobs): reverse scans.  Workgroups
// are dispatched round-robin over the 8 XCDs, so when jobs is a multiple of 8
// block b runs job (b % 8) jobs/8 + b/8: the value slices of one head then share
// an XCD and its L2, and read that head's W, K̃, Qg and Aqk from HBM once.
template <class E, class S, int KD, int VD>
__global__ void __launch_bounds__(256) kda_scan_kernel(KdaFullArgs a, int H, int nseq, int jobs) {
    const bool rev = (int)blockIdx.x >= jobs;
    int b = (int)blockIdx.x - (rev ? jobs : 0);
    if (jobs % 8 == 0) b = b % 8 * (jobs / 8) + b / 8;
    if (!rev) kda_scan_body<E, S, KD, VD, false>(a, H, nseq, b);
    else kda_scan_body<E, S, KD, VD, true>(a, H, nseq, b);
}

// ---------------------------------------------------------------- intra-chunk part
// One workgroup per (chunk, head), the heads of a chunk on consecutive
// workgroups; 512 threads.  Adds the Aqk and dL terms to the WY stage's
// partials and writes dq, dk (input type), dg (reverse-cumsummed), dβ.
// 71 KB of LDS; at K = V = 128 with 16-bit staging also at most 128 VGPRs, so
// two workgroups share a CU and one's barriers and loads overlap the other's
// products (the K = V = 64 instances need more registers and run one per CU).
template <class S, int VD>
struct KIntraCfg {
    static constexpr int C = 64, LV = VD + kfpad<S>(), LF = 68;
    static constexpr int WPE = sizeof(S) == 2 && VD == 128 ? 4 : 2;    // waves per SIMD
    static constexpr size_t szIO = (size_t)2 * C * LV * sizeof(S), szSl = (size_t)4 * C * LSL * 4;
    static constexpr size_t oDO = 0;                                   // dO [64][LV] S
    static constexpr size_t oVn = oDO + (size_t)C * LV * sizeof(S);    // V_new [64][LV] S
    static constexpr size_t oPA = 0;                                   // 4 fp32 slices [64][LSL], over dO and V_new
    static constexpr size_t oDAq = szIO > szSl ? szIO : szSl;          // dAqk [64][LF] fp32
    static constexpr size_t oDL = oDAq + (size_t)C * LF * 4;           // dL [64][LF] fp32
    static constexpr size_t oB = oDL + (size_t)C * LF * 4;             // β [64], dβ row sums [2][64]
    static constexpr size_t oBT = oB + (size_t)3 * 64 * 4;             // dG totals of 16-row blocks [4][KSL]
    static constexpr size_t smem = oBT + (size_t)4 * KSL * 4;
    static_assert(2 * smem <= 160 * 1024, "two workgroups per CU");
};

// 512 threads: wave w owns rows 16 (w & 3) .. +15 and half w >> 2 of the
// columns of every product.  Every global load is issued one step ahead: the
// next slice's q, k and G rows and the next slice's per-element operands are
// in flight during this slice's products.
template <class E, class S, int KD, int VD>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(KIntraCfg<S, VD>::WPE, KIntraCfg<S, VD>::WPE)))
kda_intra_kernel(KdaFullArgs a, int H, float scale) {
    using Cf = KIntraCfg<S, VD>;
    constexpr int C = 64, LV = Cf::LV, LF = Cf::LF;
    constexpr int EPE = 16 / (int)sizeof(E);
    constexpr int NIO = C * VD / EPE / 512, NDA = C * C / 4 / 512;   // dO / V_new and dL vectors per thread
    static_assert(C * VD / EPE % 512 == 0 && C * KSL / 4 == 512, "whole vectors per thread");
    extern __shared__ __align__(16) unsigned char smem[];
    S* sDO = (S*)(smem + Cf::oDO);
    S* sVn = (S*)(smem + Cf::oVn);
    float* sKm = (float*)(smem + Cf::oPA);   // K e^{m−G}
    float* sQp = sKm + C * LSL;              // Q e^{G−m}
    float* sKb = sQp + C * LSL;              // β K e^{G−m}
    float* sEp = sKb + C * LSL;              // e^{G−m}
    float* sDAq = (float*)(smem + Cf::oDAq);
    float* sDL = (float*)(smem + Cf::oDL);
    float* sB = (float*)(smem + Cf::oB);
    float* sRB = sB + 64;
    float* sBT = (float*)(smem + Cf::oBT);

    const int ci = (int)blockIdx.x / H, h = (int)blockIdx.x % H, w = wave_id(), l = lane_id();   // heads fastest
    const int m0 = 16 * (w & 3), hc = w >> 2;   // row group, column half
    const int Cn = a.info[ci].len;
    const long t0 = a.info[ci].t0;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const float* G = a.gcum;
    const int ref = (Cn - 1) / 2;

    // One slice vector per thread: row sr, channels sdd .. +3 of the slice.
    const int sr = threadIdx.x / (KSL / 4), sdd = threadIdx.x % (KSL / 4) * 4;
    const long so = ((t0 + min(sr, Cn - 1)) * H + h) * KD + sdd, mo = ((t0 + ref) * H + h) * KD + sdd;
    f32x4 xm, xg;
    kvec<E, 4> xk, xq;
    auto slice_issue = [&](int s0) {
        xm = *(const f32x4*)(G + mo + s0);
        xg = *(const f32x4*)(G + so + s0);
        xk = *(const kvec<E, 4>*)(k + so + s0);
        xq = *(const kvec<E, 4>*)(q + so + s0);
    };
    auto slice_store = [&]() {
        f32x4 km, qp, kb, epv;
        const float bt = sB[sr];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float ep = sr < Cn ? __expf(xg[e] - xm[e]) : 0.f, em = sr < Cn ? __expf(xm[e] - xg[e]) : 0.f;
            km[e] = (float)xk[e] * em;
            qp[e] = (float)xq[e] * ep;
            kb[e] = bt * (float)xk[e] * ep;
            epv[e] = ep;
        }
        *(f32x4*)(sKm + sr * LSL + sdd) = km;
        *(f32x4*)(sQp + sr * LSL + sdd) = qp;
        *(f32x4*)(sKb + sr * LSL + sdd) = kb;
        *(f32x4*)(sEp + sr * LSL + sdd) = epv;
    };
    // This lane's elements of q, k and the stage partials: rows m0 + 4 g + e,
    // channel 16 hc + (l & 15) of the slice.
    float pk[4], pq[4], pdq[4], pdk[4], pdg[4];
    auto elem_offset = [&](int e, int s0) {
        const int r = acc_row(m0, 0, e);
        return ((t0 + min(r, Cn - 1)) * H + h) * KD + s0 + acc_col(16 * hc, 0);
    };
    auto elem_issue = [&](int s0) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const long o = elem_offset(e, s0);
            pk[e] = (float)k[o];
            pq[e] = (float)q[o];
            pdq[e] = a.dqs[o];
            pdk[e] = a.dks[o];
            pdg[e] = a.dgs[o];
        }
    };

    // ---- every load of the first phase, then slice 0's, in this order
    const float bb = (float)((const E*)a.beta)[(t0 + min((int)threadIdx.x & (C - 1), Cn - 1)) * H + h];
    __builtin_amdgcn_sched_barrier(0);
    kvec<E, EPE> xo[NIO], xv[NIO];
#pragma unroll
    for (int i = 0; i < NIO; i++) {
        const int idx = threadIdx.x + 512 * i, r = idx / (VD / EPE), c = idx % (VD / EPE) * EPE;
        const long o = ((t0 + min(r, Cn - 1)) * H + h) * VD + c;
        xo[i] = __builtin_nontemporal_load((const kvec<E, EPE>*)((const E*)a.dO + o));
        xv[i] = __builtin_nontemporal_load((const kvec<E, EPE>*)((const E*)a.vn + o));
    }
    f32x4 xa[NDA];
#pragma unroll
    for (int i = 0; i < NDA; i++) {
        const int idx = threadIdx.x + 512 * i, r = idx / (C / 4), c = idx % (C / 4) * 4;
        xa[i] = __builtin_nontemporal_load((const f32x4*)(a.dA + ((t0 + min(r, Cn - 1)) * H + h) * C + c));
    }
    slice_issue(0);
    elem_issue(0);
    __builtin_amdgcn_sched_barrier(0);
    if (threadIdx.x < C) sB[threadIdx.x] = (int)threadIdx.x < Cn ? bb : 0.f;
#pragma unroll
    for (int i = 0; i < NIO; i++) {
        const int idx = threadIdx.x + 512 * i, r = idx / (VD / EPE), c = idx % (VD / EPE) * EPE;
        kvec<S, EPE> yo, yv;
#pragma unroll
        for (int e = 0; e < EPE; e++) {
            yo[e] = r < Cn ? (S)(float)xo[i][e] : (S)0.f;
            yv[e] = r < Cn ? (S)(float)xv[i][e] : (S)0.f;
        }
        *(kvec<S, EPE>*)(sDO + r * LV + c) = yo;
        *(kvec<S, EPE>*)(sVn + r * LV + c) = yv;
    }
#pragma unroll
    for (int i = 0; i < NDA; i++) {
        const int idx = threadIdx.x + 512 * i, r = idx / (C / 4), c = idx % (C / 4) * 4;
        *(f32x4*)(sDL + r * LF + c) = r < Cn ? xa[i] : zero4();
    }
    lds_barrier();
    // ---- dAqk = lower(dO V_newᵀ)    (wave w: rows m0, columns 32 hc .. +31)
    {
        f32x4 x[1][2];
        zero_acc(x);
        wgemm<S, 1, 2, VD, false, false>(x, sDO, LV, sVn, LV, m0, 32 * hc);
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = acc_row(m0, 0, e), c = acc_col(32 * hc, j);
                sDAq[r * LF + c] = c <= r ? x[0][j][e] : 0.f;
            }
    }
    lds_barrier();   // dO and V_new are no longer read: the slices take their place
    slice_store();
    lds_barrier();

    float rbeta[4] = {0.f, 0.f, 0.f, 0.f};   // Σ_d K e^{G−m} ⊙ (dL K e^{m−G}) for rows m0 + 4g + e (this half)
    const int g4 = l >> 4, dd = acc_col(16 * hc, 0);
#pragma unroll 1
    for (int s0 = 0; s0 < KD; s0 += KSL) {
        const int sn = s0 + KSL;   // the next slice
        if (sn < KD) slice_issue(sn);
        // wave w: rows m0, channels 16 hc .. +15 of the slice
        // p1 = dAqk · K e^{m−G}, p2 = dAqkᵀ · Q e^{G−m}, p3 = dL · K e^{m−G},
        // p4 = dLᵀ · β K e^{G−m}: one pass over the 64 rows of the chunk, p1 and
        // p3 sharing their K e^{m−G} operand
        f32x4 p1 = zero4(), p2 = zero4(), p3 = zero4(), p4 = zero4();
#pragma unroll 4
        for (int k0 = 0; k0 < C; k0 += Mma<float>::KS) {
            const float bkm = ld_trans<float>(sKm, LSL, 16 * hc, k0);
            const float bqp = ld_trans<float>(sQp, LSL, 16 * hc, k0);
            const float bkb = ld_trans<float>(sKb, LSL, 16 * hc, k0);
            p1 = Mma<float>::run(ld_direct<float>(sDAq, LF, m0, k0), bkm, p1);
            p3 = Mma<float>::run(ld_direct<float>(sDL, LF, m0, k0), bkm, p3);
            p2 = Mma<float>::run(ld_trans<float>(sDAq, LF, m0, k0), bqp, p2);
            p4 = Mma<float>::run(ld_trans<float>(sDL, LF, m0, k0), bkb, p4);
        }
        float dgt[4];   // this slice's dG term (stage partial included) for rows m0 + 4g + e
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = acc_row(m0, 0, e);
            const float ep = sEp[r * LSL + dd];
            const float em = ep > 0.f ? 1.f / ep : 0.f;
            const long o = elem_offset(e, s0);
            const float kv = pk[e], qv = pq[e];
            const float dqi = scale * ep * p1[e];
            const float dkq = scale * em * p2[e];
            const float dkr = sB[r] * ep * p3[e];
            const float dkc = em * p4[e];
            rbeta[e] += kv * ep * p3[e];
            const float dG = qv * dqi - kv * dkq + kv * dkr - kv * dkc;
            if (r < Cn) {
                ((E*)a.dq)[o] = (E)(pdq[e] + dqi);
                ((E*)a.dk)[o] = (E)(pdk[e] + dkq + dkr + dkc);
            }
            dgt[e] = r < Cn ? pdg[e] + dG : 0.f;
        }
        if (sn < KD) elem_issue(sn);
        // in-chunk reverse cumsum of dG per channel: within the lane's 4 rows,
        // across the 4 lane groups of the wave, then across the 16-row blocks
        const float t = dgt[0] + dgt[1] + dgt[2] + dgt[3];
        const float t1 = __shfl(t, l + 16, 64), t2 = __shfl(t, l + 32, 64), t3 = __shfl(t, l + 48, 64);
        const float later = (g4 < 3 ? t1 : 0.f) + (g4 < 2 ? t2 : 0.f) + (g4 < 1 ? t3 : 0.f);
        if (g4 == 0) sBT[(w & 3) * KSL + dd] = t + later;
        lds_barrier();
        float acc = later;
        for (int b = (w & 3) + 1; b < 4; b++) acc += sBT[b * KSL + dd];
#pragma unroll
        for (int e = 3; e >= 0; e--) {
            acc += dgt[e];
            if (acc_row(m0, 0, e) < Cn) a.dg[elem_offset(e, s0)] = acc;
        }
        if (sn < KD) slice_store();   // every wave is past this slice's products
        lds_barrier();
    }
    // ---- dβ = dβ_stage + row sums (over the 16 lanes of each row group)
#pragma unroll
    for (int e = 0; e < 4; e++) {
        float x = rbeta[e];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        sRB[64 * hc + m0 + 4 * (lane_id() >> 4) + e] = x;   // every lane of the group holds the sum
    }
    lds_barrier();
    if (threadIdx.x < Cn) {
        const int r = threadIdx.x;
        a.dbeta[(t0 + r) * H + h] = a.dbs[(t0 + r) * H + h] + (sRB[r] + sRB[64 + r]);
    }
}

// ---------------------------------------------------------------- launchers
// With no chunks at all (T = 0) only the scans run: their zero-chunk jobs pass
// dht (or zero) through to dh0.
template <class E, class S, int KD, int VD>
static hipError_t kda_full_go(const Problem& p, const KdaFullArgs& a, hipStream_t s, hipEvent_t* ev) {
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
    if (p.NT * p.HV > INT32_MAX) return hipErrorInvalidValue;   // one workgroup per (chunk, head), heads fastest
    hipError_t e;
    if (p.NT > 0) {
        auto kern = kda_prep_kernel<E, S, KD, VD>;
        const int sm = (int)KPrepCfg<S, KD, VD>::smem;
        if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, sm)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)(p.NT * p.HV)), dim3(512), sm, s, a, p.HV, p.scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = mark(1)) != hipSuccess) return e;
    {
        const int sm = (int)KScanCfg<S, KD>::smem;
        const int jobs = p.N * p.HV * (VD / KVS);
        auto kern = kda_scan_kernel<E, S, KD, VD>;
        if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, sm)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, dim3(2 * jobs), dim3(256), sm, s, a, p.HV, p.N, jobs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = mark(2)) != hipSuccess) return e;
    if (p.NT > 0) {
        KdaArgs k{};
        k.q = a.q; k.k = a.k; k.v = a.v; k.v_new = a.vn; k.g = a.gcum; k.beta = a.beta; k.A = a.A;
        k.h = a.hs; k.dO = a.dO; k.dh = a.dhs; k.dv_in = a.dvn; k.info = a.info;
        k.dq = a.dqs; k.dk = a.dks; k.dv_out = a.dv; k.db = a.dbs; k.dg = a.dgs; k.dA = a.dA;
        if ((e = launch_kda(p, k, s)) != hipSuccess) return e;
    }
    if ((e = mark(3)) != hipSuccess) return e;
    if (p.NT > 0) {
        auto kern = kda_intra_kernel<E, S, KD, VD>;
        const int sm = (int)KIntraCfg<S, VD>::smem;
        if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, sm)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)(p.NT * p.HV)), dim3(512), sm, s, a, p.HV, p.scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return mark(4);
}

hipError_t launch_kda_full(const Problem& p, const KdaFullArgs& a, hipStream_t s, hipEvent_t* ev) {
    if (p.K == 128 && p.V == 128) {
        if (p.dtype == 1) return kda_full_go<f16, f16, 128, 128>(p, a, s, ev);
        return hipErrorInvalidValue;
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 1) return kda_full_go<f16, f16, 64, 64>(p, a, s, ev);
        if (p.dtype == 0) return kda_full_go<float, float, 64, 64>(p, a, s, ev);
        return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
