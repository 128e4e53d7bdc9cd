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
// in one kernel; here it is one gfx950 kernel.  One workgroup of four waves per
// (chunk, head) (the heads of a chunk on consecutive workgroups), two
// workgroups per CU: the products that reduce over the
// value dimension (dO hᵀ, dv hᵀ, V_new dhᵀ, dv Vᵀ) accumulate over 32-column
// value slices, so only one slice of h, dh, dO, dv, V_new and V is staged at a
// time (about 51 KB of LDS at K = V = 128), and the next slice is loaded into
// registers while the current one is computed.  Operands in the input type
// (fp16 MFMA for fp16, fp32 MFMA for fp32) with fp32 accumulation; every
// product runs in row form (a lane holds four adjacent columns of one row of
// each 16 x 16 tile), so element-wise operands and outputs move as whole
// 8/16-byte row pieces.  The states, A and the element-wise g, k, q rows
// are read once, in whole cache lines, with non-temporal loads; the value
// slices (half a line of each row per slice) keep normal loads so the next
// slice finds the other half in the cache.  Chunk length BT = 64 or 16 (the two the page
// validates): a 16-row chunk runs in the same 64-row tile with the rows past
// it zero, and A and dA rows hold BT entries.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <class E> constexpr int kpad() { return sizeof(E) == 2 ? 8 : 4; }

template <class E, int KD, int VD>
struct KdaCfg {
    static constexpr int C = 64, VS = 32, NVS = VD / VS;
    static constexpr int LK = KD + kpad<E>(), LA = 64 + kpad<E>(), LS = VS + kpad<E>();
    static constexpr int TN = KD / 32;   // [64][KD] outputs: 2 row tiles x TN column tiles per wave (its column half)
    static constexpr size_t es = sizeof(E);
    static constexpr size_t szA = (size_t)C * LA * es, szH = (size_t)KD * LS * es, szS = (size_t)C * LS * es;
    static constexpr size_t oA = 0;             // A [64][LA] (lower triangle)
    static constexpr size_t oH = oA + szA;      // h slice [KD][LS] (key rows)
    static constexpr size_t odH = oH + szH;     // dh slice [KD][LS]
    static constexpr size_t oO = odH + szH;     // dO slice [64][LS]
    static constexpr size_t oDV = oO + szS;     // dv_in slice
    static constexpr size_t oN = oDV + szS;     // V_new slice
    static constexpr size_t oV = oN + szS;      // V slice
    static constexpr size_t oSm = oV + szS;     // floats: β [64], rowsum_V(h ⊙ dh) [KD], partials [NCS], last-row dg [KD]
    static constexpr int NCS = 2 * KD > 128 ? 2 * KD : 128;   // column partials [2][KD], later dβ partials [2][64]
    static constexpr size_t smem = oSm + (size_t)(64 + KD + NCS + KD) * 4;
    // after the value loop: dw [64][LK] over the h, dh slices; βγK [64][LK]
    // over the four row slices, then dA_pre and M1 [64][LA] over βγK
    static constexpr size_t oDW = oH, oKb = oO, oP = oO;
    static_assert((size_t)C * LK * es <= 2 * szH, "dw alias");
    static_assert((size_t)C * LK * es <= 4 * szS, "βγK alias");
    static_assert(szA <= 4 * szS, "dA_pre alias");
    static_assert(VD % VS == 0 && KD % 32 == 0, "tile shapes");
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
constexpr int KNT = 256;   // threads per workgroup

// A value fixed at this point of the program: the opaque step keeps the
// compiler from sinking the computation of a running partial sum to its
// final use (which would keep every slice's operands live until then).
__device__ __forceinline__ void kda_pin(float& x) { asm volatile("" : "+v"(x)); }

// The thread index behind an opaque step (as lane_o): per-thread offsets are
// rebuilt where they are used instead of being kept live across the unit.
__device__ __forceinline__ int kda_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & (KNT - 1);
}

// The unit's A rows in registers: a [64][64] tile of 16-byte vectors over the
// chunk's rows of BT (16 or 64) entries (rows at or past Cn read row Cn-1;
// columns past BT read the row's last vector), stored to LDS as the lower
// triangle (zero above the diagonal and in rows at or past Cn <= BT, which
// also clears every column past BT).
template <class E>
struct KdaARows {
    static constexpr int EPV = 16 / (int)sizeof(E), VPR = 64 / EPV, N = 64 * VPR / KNT;
    static_assert(64 * VPR % KNT == 0, "whole vectors per thread");
    kdv<E, EPV> v[N];
    __device__ __forceinline__ void issue(const E* __restrict__ g, int rs, int Cn, int BT) {
        const int t = kda_tid();
#pragma unroll
        for (int i = 0; i < N; i++) {
            const unsigned idx = t + KNT * i, r = min(idx / VPR, (unsigned)(Cn - 1));
            const unsigned c = min(idx % VPR * EPV, (unsigned)(BT - EPV));
            v[i] = __builtin_nontemporal_load((const kdv<E, EPV>*)at32(g, __umul24(r, (unsigned)rs) + c));
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(E* s, int Cn) const {
        const int t = kda_tid();
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int r = (t + KNT * i) / VPR, c = (t + KNT * i) % VPR * EPV;
            kdv<E, EPV> y;
#pragma unroll
            for (int e = 0; e < EPV; e++) y[e] = (r < Cn && c + e <= r) ? v[i][e] : (E)0.f;
            *(kdv<E, EPV>*)(s + r * LD + c) = y;
        }
    }
};

// One value slice (VS columns) of a unit in registers: h and dh [KD][VS] as
// fp32 16-byte pieces of key rows, and dO, dv_in, V_new, V [64][VS] as
// 16-byte pieces of token rows (rows at or past Cn read row Cn-1 and are
// zeroed when stored).  A thread covers the same key rows in every slice, so
// its partial rowsum_V(h ⊙ dh) accumulates across the slices in `hd`.
template <class E, int KD, int VD, int VS, int LS>
struct KdaSlice {
    static constexpr int SV = VS / 4, NS = KD * SV / KNT;             // h, dh vectors per thread
    static constexpr int EPV = 16 / (int)sizeof(E), RV = VS / EPV, NR = 64 * RV / KNT;   // token rows
    static_assert(KD * SV % KNT == 0 && 64 * RV % KNT == 0, "whole vectors per thread");
    f32x4 h[NS], dh[NS];
    kdv<E, EPV> o[NR], dv[NR], vn[NR], v[NR];
    __device__ __forceinline__ static int hrow(int t, int i) { return (t + KNT * i) / SV; }
    __device__ __forceinline__ static int hcol(int t, int i) { return (t + KNT * i) % SV * 4; }
    __device__ __forceinline__ static int trow(int t, int i) { return (t + KNT * i) / RV; }
    __device__ __forceinline__ static int tcol(int t, int i) { return (t + KNT * i) % RV * EPV; }
    // hg, dhg: the unit's [KD][VD] states; dO .. vv: [.,H,VD] tensors at the
    // unit's first row (row stride rs); all at the slice's first column
    __device__ __forceinline__ void issue(const float* __restrict__ hg, const float* __restrict__ dhg, const E* dO,
                                          const E* dvi, const E* vnw, const E* vv, int rs, int Cn) {
        const int t = kda_tid();
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const unsigned o_ = (unsigned)(hrow(t, i) * VD + hcol(t, i));
            h[i] = __builtin_nontemporal_load((const f32x4*)at32(hg, o_));
            dh[i] = __builtin_nontemporal_load((const f32x4*)at32(dhg, o_));
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const unsigned o_ = __umul24((unsigned)min(trow(t, i), Cn - 1), (unsigned)rs) + tcol(t, i);
            o[i] = *(const kdv<E, EPV>*)at32(dO, o_);
            dv[i] = *(const kdv<E, EPV>*)at32(dvi, o_);
            vn[i] = *(const kdv<E, EPV>*)at32(vnw, o_);
            v[i] = *(const kdv<E, EPV>*)at32(vv, o_);
        }
    }
    __device__ __forceinline__ void store(E* sH, E* sdH, E* sO, E* sDV, E* sN, E* sV, int Cn, float (&hd)[NS]) const {
        const int t = kda_tid();
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int o_ = hrow(t, i) * LS + hcol(t, i);
            st4<E>(sH + o_, h[i]);
            st4<E>(sdH + o_, dh[i]);
#pragma unroll
            for (int e = 0; e < 4; e++) hd[i] += h[i][e] * dh[i][e];
        }
#pragma unroll
        for (int i = 0; i < NR; i++) {
            const int r = trow(t, i), o_ = r * LS + tcol(t, i);
            const kdv<E, EPV> z{};
            *(kdv<E, EPV>*)(sO + o_) = r < Cn ? o[i] : z;
            *(kdv<E, EPV>*)(sDV + o_) = r < Cn ? dv[i] : z;
            *(kdv<E, EPV>*)(sN + o_) = r < Cn ? vn[i] : z;
            *(kdv<E, EPV>*)(sV + o_) = r < Cn ? v[i] : z;
        }
    }
};

// The lane's per-element operands of one column half of its [64][KD] tiles:
// the gate g, k and q at its rows (rows at or past Cn read row Cn-1) and the
// gate of the chunk's last row at its columns.
template <class E, int TH>
struct KdaElemOps {
    f32x4 g[2][TH], gl[TH];
    typename Vec4<E>::t k[2][TH], q[2][TH];
    __device__ __forceinline__ void issue(const float* g0, const E* k0p, const E* q0p, int rsk, int Cn, int m0,
                                          int n0) {
        const int l = lane_o(), rw = m0 + (l & 15), cg = 4 * (l >> 4);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const unsigned ro = __umul24((unsigned)min(rw + 16 * i, Cn - 1), (unsigned)rsk);
#pragma unroll
            for (int jj = 0; jj < TH; jj++) {
                const unsigned o = ro + n0 + 16 * jj + cg;
                g[i][jj] = __builtin_nontemporal_load((const f32x4*)at32(g0, o));
                k[i][jj] = __builtin_nontemporal_load((const typename Vec4<E>::t*)at32(k0p, o));
                q[i][jj] = __builtin_nontemporal_load((const typename Vec4<E>::t*)at32(q0p, o));
            }
        }
#pragma unroll
        for (int jj = 0; jj < TH; jj++)
            gl[jj] = *(const f32x4*)at32(g0, __umul24((unsigned)(Cn - 1), (unsigned)rsk) + n0 + 16 * jj + cg);
    }
};

// Row and column offsets of this lane's row-form accumulator elements, from a
// fresh lane index: element e of tile (i, j) of a wave block at (m0, n0) is
// row rw + 16 i, column n0 + 16 j + cg + e.
#define KDA_LANE_RC()                           \
    const int lq_ = lane_o();                   \
    const int rw = m0 + (lq_ & 15);             \
    const int cg = 4 * (lq_ >> 4)

template <class E, int KD, int VD>
__global__ void __launch_bounds__(KNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
kda_kernel(KdaArgs a, const int32_t* __restrict__ cu, int N, int T, int H, int BT, float scale) {
    using Cf = KdaCfg<E, KD, VD>;
    using M = Mma<E>;
    using frag = typename M::frag;
    constexpr int C = 64, VS = Cf::VS, NVS = Cf::NVS, LK = Cf::LK, LA = Cf::LA, LS = Cf::LS, TN = Cf::TN;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sA = (E*)(smem + Cf::oA);
    E* sH = (E*)(smem + Cf::oH);
    E* sdH = (E*)(smem + Cf::odH);
    E* sO = (E*)(smem + Cf::oO);
    E* sDV = (E*)(smem + Cf::oDV);
    E* sN = (E*)(smem + Cf::oN);
    E* sV = (E*)(smem + Cf::oV);
    E* sDW = (E*)(smem + Cf::oDW);
    E* sKb = (E*)(smem + Cf::oKb);
    E* sP = (E*)(smem + Cf::oP);
    float* sB = (float*)(smem + Cf::oSm);
    float* sHD = sB + 64;            // rowsum_V(h ⊙ dh), per key
    float* sCS = sHD + KD;           // [2][KD] column partials of K ⊙ dks, later [2][64] dβ partials
    float* sLast = sCS + Cf::NCS;    // dg of the chunk's last row before its column-sum terms

    const int ci = (int)blockIdx.x / H, hh = (int)blockIdx.x % H;   // heads fastest
    int t0i, Cn;
    kda_find_chunk(cu, N, T, BT, ci, t0i, Cn);   // chunks of BT <= 64 rows, each in a 64-row tile
    const long t0 = t0i;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int m0 = 32 * (w & 1);             // the wave's row half of every [64][.] result
    const int n0k = (KD / 2) * (w >> 1);     // its column half of [64][KD] results
    const int n0s = 32 * (w >> 1);           // of [64][64] results
    const int n0v = 16 * (w >> 1);           // of [64][VS] slice results
    const long unit = (long)ci * H + hh;
    const float* hg = a.h + unit * KD * VD;
    const float* dhg = a.dh + unit * KD * VD;
    const int rsv = H * VD, rsk = H * KD;    // token row strides of [.,H,V] and [.,H,K] tensors
    const long rowv = (t0 * H + hh) * VD, rowk = (t0 * H + hh) * KD;   // the unit's first row
    const E* dO0 = (const E*)a.dO + rowv;
    const E* dv0 = (const E*)a.dv_in + rowv;
    const E* vn0 = (const E*)a.v_new + rowv;
    const E* v0 = (const E*)a.v + rowv;
    const float* g0 = a.g + rowk;
    const E* k0p = (const E*)a.k + rowk;
    const E* q0p = (const E*)a.q + rowk;

    // ---- the unit's first loads, in a pinned order: β, A, the first slice
    const E bb = ((const E*)a.beta)[(t0 + min((int)threadIdx.x & (C - 1), Cn - 1)) * H + hh];
    __builtin_amdgcn_sched_barrier(0);
    KdaARows<E> ra;
    ra.issue((const E*)a.A + (t0 * H + hh) * BT, H * BT, Cn, BT);
    using Slice = KdaSlice<E, KD, VD, VS, LS>;
    Slice sl;
    sl.issue(hg, dhg, dO0, dv0, vn0, v0, rsv, Cn);
    __builtin_amdgcn_sched_barrier(0);

    f32x4 dqa[2][TN], dwa[2][TN], dka[2][TN], dap[2][2];
    zero_acc(dqa);
    zero_acc(dwa);
    zero_acc(dka);
    zero_acc(dap);
    float hd[Slice::NS];
#pragma unroll
    for (int i = 0; i < Slice::NS; i++) hd[i] = 0.f;
    float dbr[2] = {0.f, 0.f};   // dβ partials of the lane's rows rw, rw + 16
    constexpr int TH = TN / 2;
    KdaElemOps<E, TH> ops0, ops1;   // the element-wise phase's operands, per column half

    // ---- the value loop: dq_acc = dO hᵀ, dw = −dv hᵀ, dks_acc = V_new dhᵀ,
    //      dA_pre (V part) = dv Vᵀ (β on its columns after the loop), and per
    //      slice dv_out = β ⊙ Aᵀ dv with its dβ term rowsum(Aᵀ dv ⊙ V)
#pragma unroll
    for (int vs = 0; vs < NVS; vs++) {
        if (vs == 0) {
            if (threadIdx.x < C) sB[threadIdx.x] = (int)threadIdx.x < Cn ? (float)bb : 0.f;
            ra.template store<LA>(sA, Cn);
        }
        sl.store(sH, sdH, sO, sDV, sN, sV, Cn, hd);
#pragma unroll
        for (int i = 0; i < Slice::NS; i++) kda_pin(hd[i]);
        if (vs + 1 < NVS)   // the next slice, in flight during this one
            sl.issue(hg + (vs + 1) * VS, dhg + (vs + 1) * VS, dO0 + (vs + 1) * VS, dv0 + (vs + 1) * VS,
                     vn0 + (vs + 1) * VS, v0 + (vs + 1) * VS, rsv, Cn);
        else   // during the last slice: the first half's element-wise operands
            ops0.issue(g0, k0p, q0p, rsk, Cn, m0, n0k);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        {
            const int l = lane_o();
            const E* pO = frag_base<E, false>(sO, LS, m0, l);
            const E* pD = frag_base<E, false>(sDV, LS, m0, l);
            const E* pN = frag_base<E, false>(sN, LS, m0, l);
            const E* pH = frag_base<E, false>(sH, LS, n0k, l);
            const E* pdH = frag_base<E, false>(sdH, LS, n0k, l);
            const E* pV = frag_base<E, false>(sV, LS, n0s, l);
#pragma unroll
            for (int s = 0; s < VS / M::KS; s++) {
                const int k0 = s * M::KS;
                frag fo[2], fd[2];
                frags<E, 2, false>(fo, pO, LS, k0);
                frags<E, 2, false>(fd, pD, LS, k0);
                {
                    frag fh[TN];
                    frags<E, TN, false>(fh, pH, LS, k0);
                    mma_tiles<E>(dqa, fo, fh);
                    mma_tiles<E>(dwa, fd, fh);
                }
                __builtin_amdgcn_sched_barrier(0);
                {
                    frag fn[2], fdh[TN];
                    frags<E, 2, false>(fn, pN, LS, k0);
                    frags<E, TN, false>(fdh, pdH, LS, k0);
                    mma_tiles<E>(dka, fn, fdh);
                }
                __builtin_amdgcn_sched_barrier(0);
                {
                    frag fv[2];
                    frags<E, 2, false>(fv, pV, LS, k0);
                    mma_tiles<E>(dap, fd, fv);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        {
            f32x4 adv[2][1];
            zero_acc(adv);
            gemm4<E, 2, 1, 64, true, true>(adv, sA, LA, sDV, LS, m0, n0v);
            KDA_LANE_RC();
            E* dvb = (E*)a.dv_out + rowv + vs * VS;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int rr = rw + 16 * i, c0 = n0v + cg;
                const f32x4 vv = ld4<E>(sV + rr * LS + c0);
#pragma unroll
                for (int e = 0; e < 4; e++) dbr[i] += adv[i][0][e] * vv[e];
                if (rr < Cn)
                    *(typename Vec4<E>::t*)at32(dvb, __umul24((unsigned)rr, (unsigned)rsv) + c0) =
                        __builtin_convertvector(sB[rr] * adv[i][0], typename Vec4<E>::t);
            }
            kda_pin(dbr[0]);
            kda_pin(dbr[1]);
        }
        lds_barrier();   // the slice is read before the next one (or dw, βγK) overwrites it
    }

    // ---- dA_pre's V part takes β on its columns; rowsum_V(h ⊙ dh) per key
    //      (the SV threads of a key row are consecutive; all write the sum);
    //      dw -> LDS (over the h, dh slices)
    {
        KDA_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int j = 0; j < 2; j++) dap[i][j] *= *(const f32x4*)(sB + n0s + 16 * j + cg);
#pragma unroll
            for (int j = 0; j < TN; j++) st4<E>(sDW + (rw + 16 * i) * LK + n0k + 16 * j + cg, -dwa[i][j]);
        }
    }
    {
        const int t = kda_tid();
#pragma unroll
        for (int i = 0; i < Slice::NS; i++) {
            float x = hd[i];
#pragma unroll
            for (int off = 1; off < Slice::SV; off <<= 1) x += __shfl_xor(x, off, 64);
            sHD[Slice::hrow(t, i)] = x;
        }
    }
    // the last row's gate per key, for its column-sum terms
    const float glast = threadIdx.x < KD ? g0[(Cn - 1) * rsk + (int)threadIdx.x] : 0.f;
    lds_barrier();
    // ---- AdW = Aᵀ dw
    f32x4 adw[2][TN];
    zero_acc(adw);
    ops1.issue(g0, k0p, q0p, rsk, Cn, m0, n0k + 16 * TH);   // the second half's, in flight during AdW
    __builtin_amdgcn_sched_barrier(0);
    gemm4<E, 2, TN, 64, true, true>(adw, sA, LA, sDW, LK, m0, n0k);

    // ---- per-element outputs dq, dk, dg and βγK (-> LDS), in two column
    //      halves of the wave's tiles (the lane's g, k, q and last-row g
    //      loaded per half)
#pragma unroll
    for (int jh = 0; jh < 2; jh++) {
        __builtin_amdgcn_sched_barrier(0);
        KDA_LANE_RC();
        const KdaElemOps<E, TH>& op = jh == 0 ? ops0 : ops1;
        float csum[TH][4];
#pragma unroll
        for (int jj = 0; jj < TH; jj++)
#pragma unroll
            for (int e = 0; e < 4; e++) csum[jj][e] = 0.f;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rw + 16 * i;
            const float br = sB[rr];
#pragma unroll
            for (int jj = 0; jj < TH; jj++) {
                const int j = jh * TH + jj, c0 = n0k + 16 * j + cg;
                f32x4 dqv, dkv, dgv, kb;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float gg = op.g[i][jj][e], gm = __expf(gg);
                    const float kk = (float)op.k[i][jj][e], qq = (float)op.q[i][jj][e];
                    dqv[e] = scale * dqa[i][j][e] * gm;
                    const float dks = dka[i][j][e] * __expf(op.gl[jj][e] - gg);
                    const float bgw = br * gm * adw[i][j][e];
                    dkv[e] = dks + bgw;
                    dgv[e] = qq * dqv[e] - kk * dks + kk * bgw;
                    csum[jj][e] += kk * dks;
                    dbr[i] += adw[i][j][e] * gm * kk;
                    kb[e] = br * gm * kk;   // zero in rows at or past Cn (β is zero there)
                }
                st4<E>(sKb + rr * LK + c0, kb);
                if (rr < Cn) {
                    const unsigned o = __umul24((unsigned)rr, (unsigned)rsk) + c0;
                    *(f32x4*)at32(a.dq + rowk, o) = dqv;
                    *(f32x4*)at32(a.dk + rowk, o) = dkv;
                    if (rr == Cn - 1)
                        *(f32x4*)(sLast + c0) = dgv;
                    else
                        *(f32x4*)at32(a.dg + rowk, o) = dgv;
                }
            }
        }
        // column sums over the wave's 32 rows (the 16 lanes of a row group hold
        // 16 rows of the same four columns; every lane of the group writes the sum)
#pragma unroll
        for (int jj = 0; jj < TH; jj++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                float x = csum[jj][e];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
                sCS[(w & 1) * KD + n0k + 16 * (jh * TH + jj) + cg + e] = x;
            }
    }
    lds_barrier();
    // ---- dA_pre += dw (βγK)ᵀ; the last row's dg with its column-sum terms
    gemm4<E, 2, 2, KD, false, false>(dap, sDW, LK, sKb, LK, m0, n0s);
    if (threadIdx.x < KD) {
        const int c = threadIdx.x;
        a.dg[rowk + (long)(Cn - 1) * rsk + c] = sLast[c] + sCS[c] + sCS[KD + c] + __expf(glast) * sHD[c];
    }
    lds_barrier();
    // ---- dA_pre -> LDS (over βγK); dβ: over the 4 row groups, then the two column halves
    float* sDB = sCS;
    {
        KDA_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int j = 0; j < 2; j++) st4<E>(sP + (rw + 16 * i) * LA + n0s + 16 * j + cg, dap[i][j]);
            float x = dbr[i];
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            sDB[(w >> 1) * 64 + rw + 16 * i] = x;   // the four row groups hold the sum and write it
        }
    }
    lds_barrier();
    // ---- M1 = Aᵀ dA_pre
    f32x4 m1[2][2];
    zero_acc(m1);
    gemm4<E, 2, 2, 64, true, true>(m1, sA, LA, sP, LA, m0, n0s);
    if (threadIdx.x < Cn) {
        const int rr = threadIdx.x;
        a.db[(t0 + rr) * H + hh] = sDB[rr] + sDB[64 + rr];
    }
    lds_barrier();
    {
        KDA_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) st4<E>(sP + (rw + 16 * i) * LA + n0s + 16 * j + cg, m1[i][j]);
    }
    lds_barrier();
    // ---- dA = −strictlower(M1 Aᵀ)   (B = Aᵀ: A stored [s][j] = [n][k])
    {
        f32x4 da[2][2];
        zero_acc(da);
        gemm4<E, 2, 2, 64, false, false>(da, sP, LA, sA, LA, m0, n0s);
        KDA_LANE_RC();
        float* dAb = a.dA + (t0 * H + hh) * BT;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rw + 16 * i;
            if (rr < Cn) {
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int c0 = n0s + 16 * j + cg;   // a multiple of 4: inside the row when below BT
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; e++) x[e] = (c0 + e < rr) ? -da[i][j][e] : 0.f;
                    if (c0 < BT) *(f32x4*)at32(dAb, __umul24((unsigned)rr, (unsigned)(H * BT)) + c0) = x;
                }
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
    if (p.BT != 16 && p.BT != 64) return hipErrorInvalidValue;
    if (p.NT * p.HV > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)(p.NT * p.HV)), dim3(KNT), Cf::smem, s, a, p.cu, p.N, p.T, p.HV, p.BT,
                       p.scale);
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
