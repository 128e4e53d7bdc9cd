// gdr_grad.hip -- per-chunk gradients (K3) with the tail fused in.
//
// One workgroup (4 waves) per (chunk, key head); with G value heads per key
// head it takes the G heads of its group in turn and adds up the dq/dk group
// sums in a fixed order (the GQA reduction the FlashQLA backward explainer,
// §一 step ④, does in Python).
// Given h = h[c] (state entering the chunk) and dh = dh[c] (gradient of the
// state leaving it) from the scans, and recomputing the chunk's WY factors:
//   L = strictly-lower(diag(β)(K Kᵀ) ⊙ Γ),  A = (I+L)^{-1} (read from the prep kernel),
//   Pm = scale·lower(Γ ⊙ Q Kᵀ),  V_new = A·diag(β)(V − diag(γ) K h)
//   dV_new = Pmᵀ dO + diag(γ_C/γ) K dh
//   dPm = lower(dO V_newᵀ)                    T1 = dPm ⊙ Γ · scale
//   dq  = scale·diag(γ) dO hᵀ + T1 K
//   dW  = −dV_new hᵀ,   dv = diag(β) Aᵀ dV_new
//   dA  = dV_new (diag(β)V)ᵀ + dW (diag(βγ)K)ᵀ,   dL = −strictlower(Aᵀ dA Aᵀ)
//   E   = dL ⊙ Γ,  Eb = diag(β) E
//   dk  = T1ᵀ Q + diag(γ_C/γ) V_new dhᵀ + diag(βγ) Aᵀ dW + Eb K + Ebᵀ K
//   dβ  = rowsum(Aᵀ dV_new ⊙ V) + γ ⊙ rowsum(Aᵀ dW ⊙ K) + rowsum(dL ⊙ Γ ⊙ KKᵀ)
//   dG  = rowsum(Q ⊙ scale γ dO hᵀ) + rowsum(F) − colsum(F)          F  = dPm ⊙ Pm
//         − z + βγ ⊙ rowsum(Aᵀ dW ⊙ K) + rowsum(F2) − colsum(F2)      F2 = dL ⊙ L
//         with z = rowsum(K ⊙ diag(γ_C/γ) V_new dhᵀ);  the last row also
//         gains Σz + γ_C <dh, h>;
//   dg  = in-chunk reverse cumsum of dG  (same page, §一: the gate arrives as
//         its in-chunk cumsum and its gradient is reverse-cumsummed at the end).
// All contractions run on MFMA (16-bit operands for 16-bit inputs, fp32 for
// fp32 inputs) with fp32 accumulation; the state-dependent products are taken
// over V in 32-column slices.
//
// Layout for two workgroups per CU: the four waves form a 2 x 2 grid over
// every output (wave w owns rows 32*(w&1) .. +31 and the column half w>>1), so
// a wave's tile is 32 x 32 of a 64 x 64 result and 32 x 64 of a 64 x 128 one
// (six 1 KB fragment reads feed eight MFMAs); with 32-column value slices and
// the post-loop intermediates aliased onto dead slice buffers the workgroup
// needs under 80 KB of LDS at K = V = 128 (16-bit), so a CU runs two units at
// once and one unit's loads and barriers overlap the other's products.  The
// per-row reductions (dG, dβ) accumulate in registers and are reduced once,
// in a fixed order (deterministic, no atomics).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

// Row padding of the LDS tiles (elements): a 16-bit row pitch of D + 8 is 4
// dwords modulo the banks, fp32 D + 4.
template <class E> constexpr int gpad() { return sizeof(E) == 2 ? 8 : 4; }

constexpr int GNW = 4;            // waves per workgroup
constexpr int GNT = 64 * GNW;     // threads per workgroup

template <class E, int KD, int VD>
struct GradCfg {
    static constexpr int C = 64, VS = 32, NVS = VD / VS;
    static constexpr int LK = KD + gpad<E>(), LA = 64 + gpad<E>(), LS = VS + gpad<E>();
    static constexpr int TK = KD / 32;   // 16-column tiles per wave of a [64][KD] result (its column half)
    static constexpr size_t es = sizeof(E);
    // byte offsets.  The Q region holds the V slice, Z and V_new of the
    // current slice during the value loop (Q is reloaded after it).
    static constexpr size_t szK = (size_t)C * LK * es;
    static constexpr size_t szQ = (size_t)C * LK * es > (size_t)3 * C * LS * es ? (size_t)C * LK * es
                                                                                 : (size_t)3 * C * LS * es;
    static constexpr size_t szA = (size_t)C * LA * es;
    static constexpr size_t szH = (size_t)VS * LK * es;
    static constexpr size_t szS = (size_t)C * LS * es;
    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + szK;
    static constexpr size_t oA = oQ + szQ;
    static constexpr size_t oPm = oA + szA;
    static constexpr size_t oH = oPm + szA;
    static constexpr size_t odH = oH + szH;
    static constexpr size_t odO = odH + szH;
    static constexpr size_t odVn = odO + szS;
    static constexpr size_t oSm = odVn + szS;              // G, γ, β, e^{G_C−G}: 4 x 64 floats
    static constexpr size_t smem = oSm + 4 * 64 * 4;
    // slice buffers inside the Q region
    static constexpr size_t oV = oQ, oZ = oQ + szS, oVn = oQ + 2 * szS;
    // post-loop aliases: dW [64][LK] over H + dH, dA [64][LA] over dO + dV_new,
    // M1 over dW (after dW's last use), Eb over dA (after M1), the final
    // reductions over A (after its last use), dq staged in Q's region and dk in dW's
    static constexpr size_t odW = oH, odA = odO, oM1 = odW, oEb = odA, oRed = oA;
    static_assert((size_t)C * LK * es <= 2 * szH, "dW alias");
    static_assert(szA <= 2 * szS, "dA alias");
    static_assert(szA <= (size_t)C * LK * es, "M1 alias");
    static_assert(400 * 4 <= szA, "reduction alias");
    static_assert(VD % VS == 0 && KD % 32 == 0, "tile shapes");
};

// The thread index behind an opaque step (as lane_o).
__device__ __forceinline__ int tid_o() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t & (GNT - 1);
}

// Row and column offset of this lane's accumulator elements, from a fresh
// lane index (one per element-wise phase): element e of tile (i, j) of a
// wave block at (m0, n0) is row rw + 16 i, column n0 + 16 j + cg + e.
#define GRAD_LANE_RC()                          \
    const int lq_ = lane_o();                   \
    const int rw = m0 + (lq_ & 15);             \
    const int cg = 4 * (lq_ >> 4)

// Register staging of a [ROWS][D] row block (row stride rs elements): load()
// issues the 16-byte loads (rows at or past C read row C-1, a valid row),
// store() writes the block to LDS (row pitch LD) with rows past C zeroed.
// Splitting the two lets several blocks' loads be in flight together.
template <class E, int D, int LD, int ROWS = 64>
struct RowsReg {
    static constexpr int EPV = 16 / (int)sizeof(E), VPR = D / EPV, NV = ROWS * VPR, N = (NV + GNT - 1) / GNT;
    typename Vec16<E>::t v[N];
    int C;
    template <bool NT = false>
    __device__ __forceinline__ void load(const E* __restrict__ g, long rs, int Cn) {
        C = Cn;
        const int tid = tid_o();
        const unsigned urs = (unsigned)rs;   // row strides fit in 24 bits, offsets of a 64-row block in 32
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = tid + GNT * i;
            if (NV % GNT == 0 || idx < NV) {
                const unsigned r = min((unsigned)idx / VPR, (unsigned)(Cn - 1)), c = (unsigned)idx % VPR;
                const auto* p = (const typename Vec16<E>::t*)at32(g, __umul24(r, urs) + c * EPV);
                if constexpr (NT) v[i] = __builtin_nontemporal_load(p);
                else v[i] = *p;
            }
        }
    }
    __device__ __forceinline__ void store(E* s) const {
        const int tid = tid_o();
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = tid + GNT * i;
            if (NV % GNT == 0 || idx < NV) {
                const int r = (int)((unsigned)idx / VPR), c = (int)((unsigned)idx % VPR);
                typename Vec16<E>::t x = v[i];
                if (r >= C) x = typename Vec16<E>::t{};
                *(typename Vec16<E>::t*)(s + r * LD + c * EPV) = x;
            }
        }
    }
};

// Packed 16-bit pairs and their fp32-accumulated dot product.
template <class E> struct Pair;
template <> struct Pair<bf16> {
    typedef __bf16 t __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static float dot2(t a, t b, float c) { return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false); }
};
template <> struct Pair<f16> {
    typedef _Float16 t __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static float dot2(t a, t b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

// Register staging of NC value columns (vc0 .. vc0+NC-1, NC a multiple of 16)
// of one K x V state block, written to LDS as [NC columns][KD keys] (row pitch
// LD).  16-bit types read the workspace fragment order (one contiguous 16 B
// per thread, two 8 B LDS writes); fp32 reads the transposed [V][K] rows.
// The states are read once, so the loads are non-temporal (they leave the
// caches to the rows that are read again: Q, and the halves of the V and dO
// lines that the next value slice reads); so are the loads of A and K (read
// once per unit and key head) and, without GQA, Q's second read and the dq, dk
// stores.
template <class E, int KD, int LD, int NC>
struct StateReg {
    static constexpr bool FRAG = sizeof(E) == 2;
    static constexpr int N = NC * KD * (int)sizeof(E) / 16 / GNT;
    static_assert(N * 16 * GNT == NC * KD * (int)sizeof(E), "whole vectors per thread");
    typename Vec16<E>::t v[N];
    __device__ __forceinline__ void load(const E* __restrict__ blk, int vc0) {
        const E* src = blk + (long)vc0 * KD;   // NC columns: contiguous in both layouts
        const unsigned tid = tid_o();
#pragma unroll
        for (int i = 0; i < N; i++)
            v[i] = __builtin_nontemporal_load(
                (const typename Vec16<E>::t*)at32(src, (tid + GNT * i) * (16u / sizeof(E))));
    }
    // partial <this, o> over the elements this thread holds (same layout)
    __device__ __forceinline__ float dot(const StateReg& o) const {
        float acc = 0.f;
        if constexpr (sizeof(E) == 2) {   // packed pairs: one dot2 per two elements
            using p2 = typename Pair<E>::t;
#pragma unroll
            for (int i = 0; i < N; i++) {
                const p2* x = (const p2*)&v[i];
                const p2* y = (const p2*)&o.v[i];
#pragma unroll
                for (int e = 0; e < 4; e++) acc = Pair<E>::dot2(x[e], y[e], acc);
            }
        } else {
#pragma unroll
            for (int i = 0; i < N; i++)
#pragma unroll
                for (int e = 0; e < 4; e++) acc += v[i][e] * o.v[i][e];
        }
        return acc;
    }
    __device__ __forceinline__ void store(E* s) const {
        const int tid = tid_o();
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int c = tid + GNT * i;
            if constexpr (FRAG) {
                typedef short s4 __attribute__((ext_vector_type(4)));
                typedef short s8 __attribute__((ext_vector_type(8)));
                const unsigned ln = c & 63, sblk = ((unsigned)c >> 6) % (KD / 32), cb = ((unsigned)c >> 6) / (KD / 32);
                const int row = 16 * cb + (ln & 15), key = 32 * sblk + 4 * (ln >> 4);
                const s8 x = __builtin_bit_cast(s8, v[i]);
                *(s4*)(s + row * LD + key) = s4{x[0], x[1], x[2], x[3]};
                *(s4*)(s + row * LD + key + 16) = s4{x[4], x[5], x[6], x[7]};
            } else {
                const int row = (int)((unsigned)c / (KD / 4)), col = (int)((unsigned)c % (KD / 4)) * 4;
                *(typename Vec16<E>::t*)(s + row * LD + col) = v[i];
            }
        }
    }
};

// Coalesced store of a [64][D] LDS tile (row pitch LD) to rows < C of a global
// row block (row stride rs), 16 bytes per thread and instruction.
template <class E, int D, int LD, bool NT = false>
__device__ __forceinline__ void store_rows(E* __restrict__ g, long rs, const E* s, int C) {
    constexpr int EPV = 16 / (int)sizeof(E), VPR = D / EPV;
    const unsigned urs = (unsigned)rs;
#pragma unroll
    for (int it = 0; it < (64 * VPR + GNT - 1) / GNT; it++) {
        const unsigned idx = tid_o() + GNT * it;
        const unsigned r = idx / VPR, c = idx % VPR;
        if ((64 * VPR % GNT == 0 || idx < 64 * VPR) && (int)r < C)
        {
            const typename Vec16<E>::t x = *(const typename Vec16<E>::t*)(s + r * LD + c * EPV);
            auto* p = (typename Vec16<E>::t*)at32(g, __umul24(r, urs) + c * EPV);
            if constexpr (NT) __builtin_nontemporal_store(x, p);
            else *p = x;
        }
    }
}

// Sum over the 16 lanes that share a row group (lane bits 0..3), in every lane
// of the group: four DPP adds (swap neighbours, swap pairs, mirror within
// each half row, mirror the row), no LDS round trips.  Every lane of the
// wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float x) {
    x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]
    x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);   // row_half_mirror
    x = dpp_add<0x140>(x);   // row_mirror
    return x;
}
// Keeps a value in a register at this point: the arithmetic that produced it
// is not deferred to a later phase (where its operands would be kept live).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// Pins the per-lane partials after a phase that updated them (see pin).
__device__ __forceinline__ void pin_rows(float (&rg)[2], float (&rb)[2], float (&cs)[2][4], float& z) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        pin(rg[i]);
        pin(rb[i]);
#pragma unroll
        for (int e = 0; e < 4; e++) pin(cs[i][e]);
    }
    pin(z);
}

// sum over the 4 row groups (lane bits 4..5)
__device__ __forceinline__ float sum4g(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// One (chunk, value head) unit of the gradient: value head hv = hk·G + hi of
// key head hk, chunk ci, with blockIdx.x = ci·HK + hk: the workgroups of one
// chunk's heads are consecutive, so the launch walks the inputs (token rows
// of all heads) and the per-chunk states (unit-major) in address order.
template <class E, int KD, int VD, bool GRP>
__device__ __forceinline__ void grad_unit(const GradArgs& a, int HK, int HV, float scale, int hi) {
    using Cf = GradCfg<E, KD, VD>;
    constexpr int C = 64, VS = Cf::VS, NVS = Cf::NVS, LK = Cf::LK, LA = Cf::LA, LS = Cf::LS, TK = Cf::TK;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sK = (E*)(smem + Cf::oK);
    E* sQ = (E*)(smem + Cf::oQ);
    E* sA = (E*)(smem + Cf::oA);
    E* sPm = (E*)(smem + Cf::oPm);
    E* sH = (E*)(smem + Cf::oH);
    E* sdH = (E*)(smem + Cf::odH);
    E* sdO = (E*)(smem + Cf::odO);
    E* sdVn = (E*)(smem + Cf::odVn);
    E* sV = (E*)(smem + Cf::oV);     // V slice
    E* sZ = (E*)(smem + Cf::oZ);     // Z = diag(β)(V − diag(γ) K h) of the slice, then dv staging
    E* sVn = (E*)(smem + Cf::oVn);   // V_new = A Z of the slice
    E* sdW = (E*)(smem + Cf::odW);
    E* sdA = (E*)(smem + Cf::odA);
    E* sM1 = (E*)(smem + Cf::oM1);
    E* sEb = (E*)(smem + Cf::oEb);
    float* sG = (float*)(smem + Cf::oSm);
    float* sGam = sG + 64;
    float* sB = sGam + 64;
    float* sEg = sB + 64;   // e^{G_C − G_r}: the factor γ_C/γ
    float* sRed = (float*)(smem + Cf::oRed);   // row partials of dG, dβ [2][64] each, column partials [2][64], misc [8]

    int ci = (int)blockIdx.x / HK, hk = (int)blockIdx.x % HK;
    const int G = GRP ? HV / HK : 1;
    if constexpr (GRP) asm volatile("" : "+s"(ci), "+s"(hk));   // derived per unit, not kept live across units
    const ChunkInfo ch = a.info[ci];
    const int Cn = ch.len;
    const long t0 = ch.t0;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), l = lane_id();
    const int wr = w & 1, wc = w >> 1;
    const int m0 = 32 * wr;              // every output block of this wave starts at this row
    const int n0s = 32 * wc;             // column half of [64][64] results
    const int n0k = (KD / 2) * wc;       // column half of [64][KD] results
    const int n0v = 16 * wc;             // column half of [64][VS] slice results
    const int hv = GRP ? hk * G + hi : hk;
    const long unit = (long)ci * HV + hv;
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* dO = (const E*)a.dO;
    const E* hT = (const E*)a.hT + unit * VD * KD;
    const E* dhT = (const E*)a.dhT + unit * VD * KD;
    const E* beta = (const E*)a.beta;
    const long qrow = t0 * HK + hk, vrow = t0 * HV + hv;

    // Every load of the unit's start is issued before the first wait: the
    // gate and β (needed first), Q and K (the first product), then A and the
    // first value slice (in flight during Pm).  Every wave loads row
    // threadIdx.x % 64, unconditionally, so no wait sits at a branch join.
    const int rg = min(tid_o() & (C - 1), Cn - 1);
    const float gg = a.gcum[(t0 + rg) * HV + hv];
    const E bb = beta[(t0 + rg) * HV + hv];
    __builtin_amdgcn_sched_barrier(0);   // keep the issue order: the waits count on it
    RowsReg<E, KD, LK> rq, rk;
    rq.load(q + qrow * KD, (long)HK * KD, Cn);
    const bool need_k = !GRP || hi == 0;   // K's LDS region is not reused within a unit: later heads keep it
    if (need_k) rk.template load<true>(k + qrow * KD, (long)HK * KD, Cn);
    __builtin_amdgcn_sched_barrier(0);
    RowsReg<E, 64, LA> rA;
    StateReg<E, KD, LK, VS> rH, rdH;
    RowsReg<E, VS, LS> rdO, rV;
    rA.template load<true>((const E*)a.A + unit * C * C, C, C);
    rH.load(hT, 0);
    rdH.load(dhT, 0);
    rdO.load(dO + vrow * VD, (long)HV * VD, Cn);
    rV.load(v + vrow * VD, (long)HV * VD, Cn);
    if (GRP && hi > 0) lds_barrier();   // the previous head's last LDS reads (dq, dk rows, reductions)
    if (threadIdx.x < C) {
        const int r = threadIdx.x;
        sG[r] = gg;
        sGam[r] = __expf(gg);
        sB[r] = r < Cn ? (float)bb : 0.f;
    }
    rq.store(sQ);
    if (need_k) rk.store(sK);
    lds_barrier();
    const float gl = sG[C - 1], gC = sGam[C - 1];
    // dh[c] arrives scaled by dsc (a power of two); its products all pass
    // through the factor γ_C/γ, which takes 1/dsc along (and so does <dh, h>)
    const float idsc = a.dsc ? 1.f / a.dsc[(long)ch.seq * HV + hv] : 1.f;
    if (threadIdx.x < C) sEg[threadIdx.x] = idsc * __expf(gl - sG[threadIdx.x]);   // read after the next barrier

    // per-lane partial row sums (rows rw + 16i) and column sums (columns
    // n0s + 16j + cg + e of the [64][64] results)
    float rowG[2], rowB[2], colG[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        rowG[i] = rowB[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) colG[i][e] = 0.f;
    }
    float hdh = 0.f;   // partial <dh, h>

    // ---- Pm = scale · lower(Γ ⊙ Q Kᵀ)
    {
        f32x4 aqk[2][2];
        zero_acc(aqk);
        gemm4<E, 2, 2, KD, false, false>(aqk, sQ, LK, sK, LK, m0, n0s);
        GRAD_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rw + 16 * i;
            const float gr = sG[rr];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int c0 = n0s + 16 * j + cg;
                const f32x4 gc = *(const f32x4*)(sG + c0);
                f32x4 sv;
#pragma unroll
                for (int e = 0; e < 4; e++) sv[e] = (c0 + e <= rr) ? scale * __expf(gr - gc[e]) * aqk[i][j][e] : 0.f;
                st4<E>(sPm + rr * LA + c0, sv);
            }
        }
    }
    // ---- A = (I+L)^{-1} from the prep kernel
    rA.store(sA);

    // accumulators over the value slices.  dqi ends as dq and dks as dk;
    // dAz = dV_new Zᵀ is dA_pre (= dV_new (diag(β)V)ᵀ + dW (diag(βγ)K)ᵀ, since
    // Z = diag(β)(V − diag(γ) K h) and dW = −dV_new hᵀ).
    f32x4 dPm[2][2], dqi[2][TK], dWa[2][TK], dks[2][TK], dAz[2][2];
    zero_acc(dPm);
    zero_acc(dqi);
    zero_acc(dWa);
    zero_acc(dks);
    zero_acc(dAz);

    // the next slice (h, dh as rows v of [V][K]; dO, V) is loaded into
    // registers while the current one is computed
    // Pmᵀ's fragments (A operand of Pmᵀ dO) read once, in the first slice, and
    // kept: Pm does not change during the value loop
    typename Mma<E>::frag pmf[64 / Mma<E>::KS][2];
    StateReg<E, KD, LK, VS> nH, ndH;
    RowsReg<E, VS, LS> ndO, nV;
    RowsReg<E, KD, LK> nQ;
#pragma unroll
    for (int vs = 0; vs < NVS; vs++) {
        if (vs == 0) {
            rH.store(sH);
            rdH.store(sdH);
            hdh += rH.dot(rdH);   // <dh, h> over the slice, from the registers just stored
            rdO.store(sdO);
            lds_barrier();        // Pm has read Q: the slice buffers may take its region
            rV.store(sV);
        } else {
            nH.store(sH);
            ndH.store(sdH);
            hdh += nH.dot(ndH);
            ndO.store(sdO);
            nV.store(sV);
        }
        pin(hdh);
        if (vs + 1 < NVS) {
            nH.load(hT, (vs + 1) * VS);
            ndH.load(dhT, (vs + 1) * VS);
            ndO.load(dO + vrow * VD + (vs + 1) * VS, (long)HV * VD, Cn);
            nV.load(v + vrow * VD + (vs + 1) * VS, (long)HV * VD, Cn);
        }
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        // ---- K h and K dh (one read of K's fragments for both);
        //      Z = diag(β)(V − diag(γ) K h)
        f32x4 kdh[2][1];
        {
            f32x4 kh[2][1];
            zero_acc(kh);
            zero_acc(kdh);
            {
                const int l = lane_o();
                const E* pk = frag_base<E, false>(sK, LK, m0, l);
                const E* ph = frag_base<E, false>(sH, LK, n0v, l);
                const E* pd = frag_base<E, false>(sdH, LK, n0v, l);
#pragma unroll
                for (int s = 0; s < KD / Mma<E>::KS; s++) {
                    typename Mma<E>::frag fk[2], fh[1], fd[1];
                    frags<E, 2, false>(fk, pk, LK, s * Mma<E>::KS);
                    frags<E, 1, false>(fh, ph, LK, s * Mma<E>::KS);
                    frags<E, 1, false>(fd, pd, LK, s * Mma<E>::KS);
                    mma_tiles<E>(kh, fk, fh);
                    mma_tiles<E>(kdh, fk, fd);
                }
            }
            GRAD_LANE_RC();
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int rr = rw + 16 * i, c0 = n0v + cg;
                const f32x4 vv = ld4<E>(sV + rr * LS + c0);
                const float br = sB[rr], gr = sGam[rr];
                f32x4 sv;
#pragma unroll
                for (int e = 0; e < 4; e++) sv[e] = br * (vv[e] - gr * kh[i][0][e]);
                st4<E>(sZ + rr * LS + c0, sv);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (vs + 1 == NVS)   // Q (needed again after the loop; its LDS region holds the
            nQ.template load<!GRP>(q + qrow * KD, (long)HK * KD, Cn);   // slice buffers), in flight for the rest of the slice
        // ---- dV_new = Pmᵀ dO + diag(γ_C/γ) K dh
        {
            f32x4 pdo[2][1];
            zero_acc(pdo);
            {
                constexpr int KS = Mma<E>::KS;
                const int l = lane_o();
                if (vs == 0) {
                    const E* pa = frag_base<E, true>(sPm, LA, m0, l);
#pragma unroll
                    for (int s = 0; s < 64 / KS; s++) frags<E, 2, true>(pmf[s], pa, LA, s * KS);
                }
                const E* pb = frag_base<E, true>(sdO, LS, n0v, l);
#pragma unroll
                for (int s = 0; s < 64 / KS; s++) {
                    typename Mma<E>::frag fb[1];
                    frags<E, 1, true>(fb, pb, LS, s * KS);
                    mma_tiles<E>(pdo, pmf[s], fb);
                }
            }
            GRAD_LANE_RC();
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int rr = rw + 16 * i;
                st4<E>(sdVn + rr * LS + n0v + cg, pdo[i][0] + sEg[rr] * kdh[i][0]);
            }
        }
        lds_barrier();
        // ---- V_new = A Z
        {
            f32x4 vn[2][1];
            zero_acc(vn);
            gemm4<E, 2, 1, 64, false, true>(vn, sA, LA, sZ, LS, m0, n0v);
            GRAD_LANE_RC();
#pragma unroll
            for (int i = 0; i < 2; i++) st4<E>(sVn + (rw + 16 * i) * LS + n0v + cg, vn[i][0]);
        }
        lds_barrier();
        // ---- the state products and the V-separable outputs over the slice:
        //      dqi += dO hᵀ, dWa += dV_new hᵀ (one read of h), dPm += dO V_newᵀ,
        //      dAz += dV_new Zᵀ (the dO and dV_new fragments read once), dks +=
        //      V_new dhᵀ; scheduling fences keep each group's fragments out of
        //      the others' live ranges (the accumulators take half the registers)
        {
            using frag = typename Mma<E>::frag;
            constexpr int KS = Mma<E>::KS;
            const int l = lane_o();
            const E* pO = frag_base<E, false>(sdO, LS, m0, l);
            const E* pD = frag_base<E, false>(sdVn, LS, m0, l);
            const E* pN = frag_base<E, false>(sVn, LS, m0, l);
            const E* pHt = frag_base<E, true>(sH, LK, n0k, l);
            const E* pdHt = frag_base<E, true>(sdH, LK, n0k, l);
            const E* pNb = frag_base<E, false>(sVn, LS, n0s, l);
            const E* pZb = frag_base<E, false>(sZ, LS, n0s, l);
#pragma unroll
            for (int s = 0; s < VS / KS; s++) {
                frag fo[2], fd[2];
                frags<E, 2, false>(fo, pO, LS, s * KS);
                frags<E, 2, false>(fd, pD, LS, s * KS);
                {
                    frag fh[TK];
                    frags<E, TK, true>(fh, pHt, LK, s * KS);
                    mma_tiles<E>(dqi, fo, fh);
                    mma_tiles<E>(dWa, fd, fh);
                }
                __builtin_amdgcn_sched_barrier(0);
                {
                    frag fn[2], fz[2];
                    frags<E, 2, false>(fn, pNb, LS, s * KS);
                    frags<E, 2, false>(fz, pZb, LS, s * KS);
                    mma_tiles<E>(dPm, fo, fn);
                    mma_tiles<E>(dAz, fd, fz);
                }
                __builtin_amdgcn_sched_barrier(0);
                {
                    frag fa[2], fh[TK];
                    frags<E, 2, false>(fa, pN, LS, s * KS);
                    frags<E, TK, true>(fh, pdHt, LK, s * KS);
                    mma_tiles<E>(dks, fa, fh);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        {
            f32x4 adv[2][1];
            zero_acc(adv);
            gemm4<E, 2, 1, 64, true, true>(adv, sA, LA, sdVn, LS, m0, n0v);  // Aᵀ dV_new
            // dv = diag(β) Aᵀ dV_new, stored from the accumulators (four adjacent
            // columns of a row per lane: one 8-byte store); the row sums of
            // Aᵀ dV_new ⊙ V (dβ) accumulate in the lane's row partials
            GRAD_LANE_RC();
            E* dvb = (E*)a.dv + vrow * VD + vs * VS;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int rr = rw + 16 * i, c0 = n0v + cg;
                const f32x4 vv = ld4<E>(sV + rr * LS + c0);
#pragma unroll
                for (int e = 0; e < 4; e++) rowB[i] += adv[i][0][e] * vv[e];
                const f32x4 d = sB[rr] * adv[i][0];
                if (rr < Cn) *(typename Vec4<E>::t*)at32(dvb, __umul24((unsigned)rr, (unsigned)(HV * VD)) + (unsigned)c0) =
                    __builtin_convertvector(d, typename Vec4<E>::t);
            }
            pin(rowB[0]);
            pin(rowB[1]);
        }
        lds_barrier();   // the slice buffers are read before the next slice overwrites them
    }
    // ---- Q back into its region (it held the slice buffers)
    {
        nQ.store(sQ);
    }
    // ---- F = dPm ⊙ Pm -> dG; T1 = dPm ⊙ Γ · scale (over Pm, each wave its own block); dW -> LDS
    {
        GRAD_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rw + 16 * i;
            const float gr = sG[rr];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int c0 = n0s + 16 * j + cg;
                const f32x4 gc = *(const f32x4*)(sG + c0);
                const f32x4 pm = ld4<E>(sPm + rr * LA + c0);
                f32x4 sv;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const bool lo = c0 + e <= rr;
                    const float dp = lo ? dPm[i][j][e] : 0.f;
                    const float f = dp * pm[e];
                    rowG[i] += f;
                    colG[j][e] += f;
                    sv[e] = lo ? dp * scale * __expf(gr - gc[e]) : 0.f;
                }
                st4<E>(sPm + rr * LA + c0, sv);   // the lane's own elements, read just above
            }
        }
        pin_rows(rowG, rowB, colG, hdh);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < TK; j++) st4<E>(sdW + (rw + 16 * i) * LK + n0k + 16 * j + cg, -dWa[i][j]);
        // ---- dA_pre -> LDS
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) st4<E>(sdA + (rw + 16 * i) * LA + n0s + 16 * j + cg, dAz[i][j]);
    }
    lds_barrier();
    E* sT1 = sPm;

    // ---- dq = scale γ dO hᵀ + T1 K ;  dG += rowsum(Q ⊙ scale γ dO hᵀ)
    {
    GRAD_LANE_RC();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int rr = rw + 16 * i;
        const float sg = scale * sGam[rr];
#pragma unroll
        for (int j = 0; j < TK; j++) {
            const f32x4 qv = ld4<E>(sQ + rr * LK + n0k + 16 * j + cg);
            const f32x4 di = sg * dqi[i][j];
#pragma unroll
            for (int e = 0; e < 4; e++) rowG[i] += di[e] * qv[e];
            dqi[i][j] = di;
        }
    }
    }
    float zsum = 0.f;
    pin_rows(rowG, rowB, colG, zsum);
    gemm4<E, 2, TK, 64, false, true>(dqi, sT1, LA, sK, LK, m0, n0k);
    __builtin_amdgcn_sched_barrier(0);
    // ---- dk = diag(γ_C/γ) V_new dhᵀ (z terms) + diag(βγ) Aᵀ dW + T1ᵀ Q
    {
        f32x4 adw[2][TK];
        zero_acc(adw);
        gemm4<E, 2, TK, 64, true, true>(adw, sA, LA, sdW, LK, m0, n0k);
        GRAD_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rw + 16 * i;
            const float eg = sEg[rr], gr = sGam[rr], bg = sB[rr] * gr;
#pragma unroll
            for (int j = 0; j < TK; j++) {
                const f32x4 kv = ld4<E>(sK + rr * LK + n0k + 16 * j + cg);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float ds = eg * dks[i][j][e];
                    const float z = ds * kv[e];
                    const float aw = adw[i][j][e] * kv[e];
                    rowG[i] += bg * aw - z;
                    zsum += z;
                    rowB[i] += gr * aw;
                    dks[i][j][e] = ds + bg * adw[i][j][e];
                }
            }
        }
        pin_rows(rowG, rowB, colG, zsum);
    }
    __builtin_amdgcn_sched_barrier(0);
    gemm4<E, 2, TK, 64, true, true>(dks, sT1, LA, sQ, LK, m0, n0k);
    // ---- M1 = Aᵀ dA_pre (over dW, last read above: after the barrier)
    lds_barrier();
    {
        f32x4 m1[2][2];
        zero_acc(m1);
        gemm4<E, 2, 2, 64, true, true>(m1, sA, LA, sdA, LA, m0, n0s);
        GRAD_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) st4<E>(sM1 + (rw + 16 * i) * LA + n0s + 16 * j + cg, m1[i][j]);
    }
    lds_barrier();
    // ---- dL = −strictlower(M1 Aᵀ); dβ, dG (F2); Eb = diag(β) dL ⊙ Γ (over dA, last read above)
    {
        f32x4 dl[2][2], akk[2][2];
        zero_acc(dl);
        zero_acc(akk);
        gemm4<E, 2, 2, 64, false, false>(dl, sM1, LA, sA, LA, m0, n0s);
        gemm4<E, 2, 2, KD, false, false>(akk, sK, LK, sK, LK, m0, n0s);   // K Kᵀ (recomputed)
        GRAD_LANE_RC();
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int rr = rw + 16 * i;
            const float gr = sG[rr], br = sB[rr];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int c0 = n0s + 16 * j + cg;
                const f32x4 gc = *(const f32x4*)(sG + c0);
                f32x4 sv;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const bool lo = c0 + e < rr;
                    const float d = lo ? -dl[i][j][e] : 0.f;
                    const float ex = __expf(gr - gc[e]);
                    const float lg = lo ? ex * akk[i][j][e] : 0.f;   // Γ ⊙ KKᵀ
                    rowB[i] += d * lg;
                    const float f2 = d * br * lg;
                    rowG[i] += f2;
                    colG[j][e] += f2;
                    sv[e] = lo ? br * d * ex : 0.f;
                }
                st4<E>(sEb + rr * LA + c0, sv);
            }
        }
        pin_rows(rowG, rowB, colG, zsum);
    }
    // the previous head's dq, dk stores (every wave's) are ordered before the
    // loads of them below: release here, the barrier, acquire before the loads
    if (GRP && hi > 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    lds_barrier();
    // ---- dk += Eb K + Ebᵀ K
    gemm4<E, 2, TK, 64, false, true>(dks, sEb, LA, sK, LK, m0, n0k);
    gemm4<E, 2, TK, 64, true, true>(dks, sEb, LA, sK, LK, m0, n0k);

    // ---- GQA: the group's dq, dk summed over the earlier heads (rows in flight
    //      during the reductions, staged over Q's and dW's regions with them)
    const bool add_prev = GRP && hi > 0;
    RowsReg<E, KD, LK> pq, pk;
    if (add_prev) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        pq.load((const E*)a.dq + qrow * KD, (long)HK * KD, Cn);
        pk.load((const E*)a.dk + qrow * KD, (long)HK * KD, Cn);
    }
    // ---- reductions (fixed order), over A's region (last read by M1 Aᵀ):
    // rows over the 16 lanes of a group and the two column halves; columns
    // over the 4 row groups and the two row halves
    float* sRowG = sRed;
    float* sRowB = sRed + 128;
    float* sCol = sRed + 256;
    float* sMisc = sRed + 384;
    {
    GRAD_LANE_RC();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        // every row group holds the sum: all four write the same value (no branch)
        const float rgs = sum4g(rowG[i]);
        const float rbs = sum4g(rowB[i]);
        sRowG[wc * 64 + rw + 16 * i] = rgs;
        sRowB[wc * 64 + rw + 16 * i] = rbs;
    }
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) {   // all 16 lanes of the group hold the sum and write it (no branch)
            const float cs = sum16(colG[j][e]);
            sCol[wr * 64 + n0s + 16 * j + cg + e] = cs;
        }
    }
    {
        float hz = hdh, zz = zsum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            hz += __shfl_xor(hz, off, 64);
            zz += __shfl_xor(zz, off, 64);
        }
        sMisc[w] = hz;   // every lane holds the sum (no branch)
        sMisc[4 + w] = zz;
    }
    if (add_prev) {   // over Q (last read by T1ᵀ Q) and dW / M1 (last read by M1 Aᵀ)
        pq.store(sQ);
        pk.store(sdW);
    }
    lds_barrier();
    if (threadIdx.x < 64) {
        const int rr = threadIdx.x;
        float dG = sRowG[rr] + sRowG[64 + rr] - (sCol[rr] + sCol[64 + rr]);
        const float db = sRowB[rr] + sRowB[64 + rr];
        if (rr == C - 1) {
            float hd = 0.f, zs = 0.f;
            for (int i = 0; i < GNW; i++) { hd += sMisc[i]; zs += sMisc[4 + i]; }
            dG += zs + gC * idsc * hd;
        }
        if (rr < Cn) a.dbeta[(t0 + rr) * HV + hv] = db;
        // in-chunk reverse cumulative sum (suffix sums over the 64 rows,
        // one row per lane; padded rows carry the chunk-end terms)
        float x = dG;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(x, off, 64);
            x += rr + off < 64 ? y : 0.f;
        }
        if (rr < Cn) a.dg[(t0 + rr) * HV + hv] = x;
    }
    // ---- dq, dk through LDS for 16-byte stores: dq over Q's region (last read
    //      by T1ᵀ Q), dk over dW's (M1, last read by M1 Aᵀ)
    E* sdq = sQ;
    E* sdk = sdW;
    {
    GRAD_LANE_RC();
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < TK; j++) {
            // each element is read and written by the lane that owns it
            const int o = (rw + 16 * i) * LK + n0k + 16 * j + cg;
            const f32x4 zq = {0.f, 0.f, 0.f, 0.f};
            st4<E>(sdq + o, dqi[i][j] + (add_prev ? ld4<E>(sdq + o) : zq));
            st4<E>(sdk + o, dks[i][j] + (add_prev ? ld4<E>(sdk + o) : zq));
        }
    }
    lds_barrier();
    store_rows<E, KD, LK, !GRP>((E*)a.dq + qrow * KD, (long)HK * KD, sdq, Cn);
    store_rows<E, KD, LK, !GRP>((E*)a.dk + qrow * KD, (long)HK * KD, sdk, Cn);
}

// One workgroup per (chunk, key head), key heads fastest.  GRP (G = HV/HK > 1): the workgroup
// takes the G value heads hv = hk·G + hi of its key head one after the other
// and builds the group sums of dq and dk in the outputs themselves: the first
// head stores its dq, dk; every later one loads the rows stored so far (its
// own workgroup's, one unit earlier, so mostly from cache; coalesced, into the
// LDS staging tiles), adds its own in fp32 and stores the sum.  The order of
// the sum is fixed and the partial sums are rounded to the output type in
// between; no workspace is needed and every unit has the register footprint
// of a single head.
template <class E, int KD, int VD, bool GRP>
__global__ void __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
grad_kernel(GradArgs a, int HK, int HV, float scale) {
    if constexpr (!GRP) {
        grad_unit<E, KD, VD, false>(a, HK, HV, scale, 0);
    } else {
        const int G = HV / HK;
        for (int hi = 0; hi < G; hi++) grad_unit<E, KD, VD, true>(a, HK, HV, scale, hi);
    }
}

template <class E, int KD, int VD, bool GRP>
static hipError_t grad_go1(const Problem& p, const GradArgs& a, hipStream_t s) {
    using Cf = GradCfg<E, KD, VD>;
    static_assert(Cf::smem <= 160 * 1024, "LDS budget");
    auto kern = grad_kernel<E, KD, VD, GRP>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem);
    if (e != hipSuccess) return e;
    if (p.NT * p.HK > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)(p.NT * p.HK)), dim3(GNT), Cf::smem, s, a, p.HK, p.HV, p.scale);
    return hipGetLastError();
}

template <class E, int KD, int VD>
static hipError_t grad_go(const Problem& p, const GradArgs& a, hipStream_t s) {
    if (p.HV == p.HK) return grad_go1<E, KD, VD, false>(p, a, s);
    return grad_go1<E, KD, VD, true>(p, a, s);
}

hipError_t launch_grad(const Problem& p, const GradArgs& a, hipStream_t s) {
    if (p.K == 128 && p.V == 128) {
        if (p.dtype == 2) return grad_go<bf16, 128, 128>(p, a, s);
        if (p.dtype == 1) return grad_go<f16, 128, 128>(p, a, s);
        return hipErrorInvalidValue;   // fp32 at 128 exceeds the LDS budget
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 2) return grad_go<bf16, 64, 64>(p, a, s);
        if (p.dtype == 1) return grad_go<f16, 64, 64>(p, a, s);
        return grad_go<float, 64, 64>(p, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
