// gdr_grad.hip -- per-chunk gradients (K3) with the tail fused in.
//
// One workgroup (8 waves) per (chunk, key head) and launch; with G value heads
// per key head there are G launches, one per head of the group, that add up
// the dq/dk group sums in a fixed order (the GQA reduction the FlashQLA
// backward explainer, §一 step ④, does in Python).
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
// over V in 64-column slices so the LDS footprint stays under 150 KB.
// Every output tile of a wave uses rows 32*(w&1) .. +31, so the per-row
// reductions (dG, dβ) accumulate in registers and are reduced once, in a
// fixed order (deterministic, no atomics).
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

// Row padding of the LDS tiles.  16-bit tiles: 16 elements, so a row pitch of
// K + 16 or 64 + 16 elements is 8 dwords modulo the 32 banks and the four rows
// a transposing 64-bit fragment read touches fall in distinct banks (measured
// faster than a padding of 8 for both tile widths together, slower for either
// alone).
template <class E> constexpr int gpad() { return sizeof(E) == 2 ? 16 : 4; }

// Wave w owns rows 32*(w&1) .. +31 and the column block (w>>1) of every
// output; 8 waves (two per SIMD, so one wave's element-wise work overlaps the
// other's LDS and MFMA latency) measured faster than 4 at every workload.
// Cross-lane results (DPP and permute reductions) are written by every lane
// that holds them, never under a lane-dependent branch.
#ifndef GDR_GRAD_WAVES
#define GDR_GRAD_WAVES 8
#endif
constexpr int GNT = 64 * GDR_GRAD_WAVES;
constexpr int GNCB = GDR_GRAD_WAVES / 2;   // column blocks (waves w and w^1 share one)

template <class E, int KD, int VD>
struct GradCfg {
    static constexpr int C = 64, VH = 64, NVH = VD / VH;
    static constexpr int LK = KD + gpad<E>(), LA = 64 + gpad<E>(), LS = VH + gpad<E>(), LF = 68;
    static constexpr int TNK = KD / 16 / GNCB;   // 16-col tiles per wave for [64][KD] outputs
    static constexpr int TNS = 4 / GNCB;         // 16-col tiles per wave for [64][64] outputs
    // byte offsets.  The V slice lives in Q's buffer during the V loop (Q is
    // reloaded afterwards); after the loop the slice region holds dW, dA_pre,
    // M1 and Eb.
    static constexpr size_t oQ = 0;
    static constexpr size_t oK = oQ + (size_t)C * LK * sizeof(E);
    static constexpr size_t oA = oK + (size_t)C * LK * sizeof(E);
    static constexpr size_t oPm = oA + (size_t)C * LA * sizeof(E);
    static constexpr size_t oH = oPm + (size_t)C * LA * sizeof(E);
    static constexpr size_t odH = oH + (size_t)VH * LK * sizeof(E);
    static constexpr size_t odO = odH + (size_t)VH * LK * sizeof(E);
    static constexpr size_t oVn = odO + (size_t)C * LS * sizeof(E);
    static constexpr size_t odVn = oVn + (size_t)C * LS * sizeof(E);
    static constexpr size_t oSm = odVn + (size_t)C * LS * sizeof(E);
    // small arrays: G, β, γ, row partials 2x[4][64], col partials [2][64], misc [80]
    // dv slice [64][LS] staged for coalesced stores (16-bit types; fp32 stores directly)
    static constexpr bool DV_LDS = sizeof(E) == 2;
    static constexpr size_t oDv = oSm + (size_t)(3 * 64 + 8 * 64 + 2 * 64 + 80) * 4;
    // V_new of the slice gets its own [64][LS] buffer when it fits (else it
    // overwrites Z in place, one barrier later)
    static constexpr size_t oEnd = oDv + (DV_LDS ? (size_t)C * LS * sizeof(E) : 0);
    static constexpr bool VN2 = oEnd + (size_t)C * LS * sizeof(E) <= 160 * 1024;
    static constexpr size_t oVn2 = VN2 ? oEnd : oVn;
    static constexpr size_t smem = oEnd + (VN2 ? (size_t)C * LS * sizeof(E) : 0);
    static constexpr size_t oV = oQ;                                    // [64][LS] inside the V loop
    static constexpr size_t odW = oH;                                   // [64][LK]
    static constexpr size_t odA = odH;                                  // [64][LA]
    static constexpr size_t oM1 = odO;                                  // [64][LA]
    static constexpr size_t oEb = oVn;                                  // [64][LA]
    static_assert(LS <= LK && LA <= LK, "alias size");
    static_assert(LA == LS, "alias size");
};

template <class Ein, class E, int D, int LD>
__device__ __forceinline__ void g_load_rows(E* s, const Ein* __restrict__ g, long rs, int C, int rows = 64) {
    constexpr int EPV = 16 / sizeof(Ein);
    constexpr int VPR = D / EPV;
    for (int idx = threadIdx.x; idx < rows * VPR; idx += GNT) {
        const int r = idx / VPR, c = idx % VPR;
        typename Vec16<Ein>::t v;
        if (r < C) v = *(const typename Vec16<Ein>::t*)(g + r * rs + c * EPV);
        else v = typename Vec16<Ein>::t{};
        *(typename Vec16<E>::t*)(s + r * LD + c * EPV) = v;
    }
}

// 64 value columns (vc0 .. vc0+63) of one K x V state block from the workspace
// state layout into LDS as [64 columns][KD keys] (row pitch LD).  16-bit types
// read the fragment order (one contiguous 16 B per thread, two 8 B LDS
// writes); fp32 reads the transposed [V][K] rows.
template <class E, int KD, int LD>
__device__ __forceinline__ void g_load_state(E* s, const E* __restrict__ blk, int vc0) {
    if constexpr (sizeof(E) == 2) {
        typedef short s4 __attribute__((ext_vector_type(4)));
        typedef short s8 __attribute__((ext_vector_type(8)));
        const E* src = blk + (long)vc0 * KD;          // 64 columns = 4 contiguous [16 x KD] blocks
        for (int c = threadIdx.x; c < 64 * KD / 8; c += GNT) {
            const int ln = c & 63, sblk = (c >> 6) % (KD / 32), cb = (c >> 6) / (KD / 32);
            const int row = 16 * cb + (ln & 15), key = 32 * sblk + 4 * (ln >> 4);
            const s8 v = *(const s8*)(src + (long)c * 8);
            *(s4*)(s + row * LD + key) = s4{v[0], v[1], v[2], v[3]};
            *(s4*)(s + row * LD + key + 16) = s4{v[4], v[5], v[6], v[7]};
        }
    } else {
        g_load_rows<E, E, KD, LD>(s, blk + (long)vc0 * KD, KD, 64);
    }
}

// Register staging of a [ROWS][D] row block (row stride rs elements): load()
// issues the 16-byte loads (rows at or past C read row C-1, a valid row),
// store() writes the block to LDS (row pitch LD) with rows past C zeroed.
// Splitting the two lets several blocks' loads be in flight together.
template <class E, int D, int LD, int ROWS = 64>
struct RowsReg {
    static constexpr int EPV = 16 / (int)sizeof(E), VPR = D / EPV, NV = ROWS * VPR, N = (NV + GNT - 1) / GNT;
    typename Vec16<E>::t v[N];
    int C;
    __device__ __forceinline__ void load(const E* __restrict__ g, long rs, int Cn) {
        C = Cn;
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = threadIdx.x + GNT * i;
            if (NV % GNT == 0 || idx < NV) {
                const int r = min(idx / VPR, Cn - 1), c = idx % VPR;
                v[i] = *(const typename Vec16<E>::t*)(g + r * rs + c * EPV);
            }
        }
    }
    __device__ __forceinline__ void store(E* s) const {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int idx = threadIdx.x + GNT * i;
            if (NV % GNT == 0 || idx < NV) {
                const int r = idx / VPR, c = idx % VPR;
                typename Vec16<E>::t x = v[i];
                if (r >= C) x = typename Vec16<E>::t{};
                *(typename Vec16<E>::t*)(s + r * LD + c * EPV) = x;
            }
        }
    }
};

// Register staging of 64 value columns (vc0 .. vc0+63) of one K x V state
// block from the workspace state layout, written to LDS as [64 columns][KD]
// (see g_load_state).
template <class E, int KD, int LD>
struct StateReg {
    static constexpr bool FRAG = sizeof(E) == 2;
    static constexpr int N = 64 * KD * (int)sizeof(E) / 16 / GNT;
    typename Vec16<E>::t v[N];
    __device__ __forceinline__ void load(const E* __restrict__ blk, int vc0) {
        const E* src = blk + (long)vc0 * KD;   // 64 columns: contiguous in both layouts
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = *(const typename Vec16<E>::t*)(src + (long)(threadIdx.x + GNT * i) * (16 / sizeof(E)));
    }
    // partial <this, o> over the elements this thread holds (same layout)
    __device__ __forceinline__ float dot(const StateReg& o) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < N; i++)
#pragma unroll
            for (int e = 0; e < (int)(16 / sizeof(E)); e++) acc += (float)v[i][e] * (float)o.v[i][e];
        return acc;
    }
    __device__ __forceinline__ void store(E* s) const {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int c = threadIdx.x + GNT * i;
            if constexpr (FRAG) {
                typedef short s4 __attribute__((ext_vector_type(4)));
                typedef short s8 __attribute__((ext_vector_type(8)));
                const int ln = c & 63, sblk = (c >> 6) % (KD / 32), cb = (c >> 6) / (KD / 32);
                const int row = 16 * cb + (ln & 15), key = 32 * sblk + 4 * (ln >> 4);
                const s8 x = __builtin_bit_cast(s8, v[i]);
                *(s4*)(s + row * LD + key) = s4{x[0], x[1], x[2], x[3]};
                *(s4*)(s + row * LD + key + 16) = s4{x[4], x[5], x[6], x[7]};
            } else {
                const int row = c / (KD / 4), col = (c % (KD / 4)) * 4;
                *(typename Vec16<E>::t*)(s + row * LD + col) = v[i];
            }
        }
    }
};

// Coalesced store of a [64][D] LDS tile (row pitch LD) to rows < C of a global
// row block (row stride rs), 16 bytes per thread and instruction.
template <class E, int D, int LD>
__device__ __forceinline__ void store_rows(E* __restrict__ g, long rs, const E* s, int C) {
    constexpr int EPV = 16 / (int)sizeof(E), VPR = D / EPV;
    for (int idx = threadIdx.x; idx < 64 * VPR; idx += GNT) {
        const int r = idx / VPR, c = idx % VPR;
        if (r < C) *(typename Vec16<E>::t*)(g + r * rs + c * EPV) = *(const typename Vec16<E>::t*)(s + r * LD + c * EPV);
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

// sum over the 4 row groups (lane bits 4..5)
__device__ __forceinline__ float sum4g(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// One launch handles value head hv = hk * G + hi of every (chunk, key head).
// GRP (G > 1): the launches for hi = 0 .. G-1 run in order on one stream and
// carry the group sums of dq and dk in an fp32 workspace block per (chunk,
// key head) (fragment order, each element read back and rewritten only by the
// lane that owns it): the first launch writes its partials, later ones add
// theirs, and the last one stores the 16-bit sums.  The order of the sum is
// fixed, and every launch has the register footprint of a single head.
template <class E, int KD, int VD, bool GRP>
__global__ void __launch_bounds__(GNT) grad_kernel(GradArgs a, int HK, int HV, float scale, int hi) {
    using Cf = GradCfg<E, KD, VD>;
    constexpr int C = 64, TNK = Cf::TNK, TNS = Cf::TNS, LK = Cf::LK, LA = Cf::LA, LS = Cf::LS, LF = Cf::LF;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sQ = (E*)(smem + Cf::oQ);
    E* sK = (E*)(smem + Cf::oK);
    E* sA = (E*)(smem + Cf::oA);
    E* sPm = (E*)(smem + Cf::oPm);
    E* sH = (E*)(smem + Cf::oH);
    E* sdH = (E*)(smem + Cf::odH);
    E* sdO = (E*)(smem + Cf::odO);
    E* sV = (E*)(smem + Cf::oV);
    E* sVn = (E*)(smem + Cf::oVn);     // Z = diag(β)(V − diag(γ) K h) of the slice
    E* sVn2 = (E*)(smem + Cf::oVn2);   // V_new = A Z of the slice (own buffer when it fits)
    E* sdVn = (E*)(smem + Cf::odVn);
    E* sdW = (E*)(smem + Cf::odW);
    E* sdA = (E*)(smem + Cf::odA);
    E* sM1 = (E*)(smem + Cf::oM1);
    E* sEb = (E*)(smem + Cf::oEb);
    float* sG = (float*)(smem + Cf::oSm);
    float* sB = sG + 64;
    float* sGam = sB + 64;
    float* sRowG = sGam + 64;      // [2][64] row partials of dG per column block (4 x 64 reserved)
    float* sRowB = sRowG + 4 * 64; // [2][64] row partials of dβ
    float* sCol = sRowB + 4 * 64;  // [2][64] column partials of dG per row half
    float* sMisc = sCol + 2 * 64;  // [16 + 64]
    E* sDv = (E*)(smem + Cf::oDv);

    const int ci = blockIdx.x, hk = blockIdx.y, G = GRP ? HV / HK : 1;
    const ChunkInfo ch = a.info[ci];
    const int Cn = ch.len;
    const long t0 = ch.t0;
    const int w = wave_id(), l = lane_id(), r16 = l & 15, g4 = l >> 4;
    const int m0 = 32 * (w & 1);           // every output block of this wave starts at this row
    const int n0s = (64 / GNCB) * (w >> 1);   // column block for [64][64] outputs
    const int n0k = (KD / GNCB) * (w >> 1);   // column block for [64][KD] outputs
    const E* q = (const E*)a.q;
    const E* k = (const E*)a.k;
    const E* v = (const E*)a.v;
    const E* dO = (const E*)a.dO;
    const E* hT = (const E*)a.hT;
    const E* dhT = (const E*)a.dhT;
    const E* beta = (const E*)a.beta;

    f32x4 dq_tot[2][TNK], dk_tot[2][TNK];   // this head's dq, dk (then the group sums)

    {
        const int hv = GRP ? hk * G + hi : hk;
        const long unit = (long)ci * HV + hv;
        // Every load of the unit's start is issued before the first wait: the
        // gate and β (needed first), Q and K (the first product), then this
        // head's A and first value slice (in flight during Pm).  The waits
        // before the first LDS stores then cover only the first two groups.
        // (every wave loads row threadIdx.x % 64, unconditionally, so no wait
        // is placed at a branch join)
        const int rg = min((int)threadIdx.x & (C - 1), Cn - 1);
        const float gg = a.gcum[(t0 + rg) * HV + hv];
        const E bb = beta[(t0 + rg) * HV + hv];
        __builtin_amdgcn_sched_barrier(0);   // keep the issue order: the waits count on it
        RowsReg<E, KD, LK> rq, rk;
        rq.load(q + (t0 * HK + hk) * KD, (long)HK * KD, Cn);
        rk.load(k + (t0 * HK + hk) * KD, (long)HK * KD, Cn);
        __builtin_amdgcn_sched_barrier(0);
        RowsReg<E, 64, LA> rA;
        StateReg<E, KD, LK> rH, rdH;
        RowsReg<E, 64, LS> rdO, rV;
        rA.load((const E*)a.A + unit * C * C, C, C);
        rH.load(hT + unit * VD * KD, 0);
        rdH.load(dhT + unit * VD * KD, 0);
        rdO.load(dO + (t0 * HV + hv) * VD, (long)HV * VD, Cn);
        rV.load(v + (t0 * HV + hv) * VD, (long)HV * VD, Cn);
        if (threadIdx.x < C) {
            const int r = threadIdx.x;
            sG[r] = gg;
            sGam[r] = __expf(gg);
            sB[r] = r < Cn ? (float)bb : 0.f;
        }
        rq.store(sQ);
        rk.store(sK);
        lds_barrier();
        const float gl = sG[C - 1], gC = sGam[C - 1];

        // per-lane partial row sums (rows m0 + 16i + 4g4 + e) and column sums
        float rowG[2][4], rowB[2][4], colG[TNS];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) rowG[i][e] = rowB[i][e] = 0.f;
#pragma unroll
        for (int j = 0; j < TNS; j++) colG[j] = 0.f;
        float hdh = 0.f;   // partial <dh, h>

        // ---- S_qk -> Pm = scale · lower(Γ ⊙ Q Kᵀ)
        {
            f32x4 aqk[2][TNS];
            zero_acc(aqk);
            wgemm<E, 2, TNS, KD, false, false>(aqk, sQ, LK, sK, LK, m0, n0s);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNS; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int rr = acc_row(m0, i, e), cc = acc_col(n0s, j);
                    const float gm = (cc <= rr) ? __expf(sG[rr] - sG[cc]) : 0.f;
                    sPm[rr * LA + cc] = to_e<E>((cc <= rr) ? scale * gm * aqk[i][j][e] : 0.f);
                }
        }
        // ---- A = (I+L)^{-1} from the prep kernel, and the first slice
        rA.store(sA);
        rH.store(sH);
        rdH.store(sdH);
        hdh += rH.dot(rdH);   // <dh, h> over the first slice, from the registers just stored
        pin(hdh);
        rdO.store(sdO);
        lds_barrier();   // Pm has read Q: the V slice may take its buffer
        rV.store(sV);

        // persistent accumulators over the V slices
        f32x4 dPm[2][TNS], dqi[2][TNK], dWa[2][TNK], dks[2][TNK], dAp[2][TNS];
        zero_acc(dPm);
        zero_acc(dqi);
        zero_acc(dWa);
        zero_acc(dks);
        zero_acc(dAp);

        // the next value slice (h, dh as rows v of [V][K]; dO, V) is loaded into
        // registers while the current one is computed
        StateReg<E, KD, LK> nH, ndH;
        RowsReg<E, 64, LS> ndO, nV;
        RowsReg<E, KD, LK> nQ;   // Q returns to its buffer (which holds V during the loop)
#pragma unroll
        for (int vh = 0; vh < Cf::NVH; vh++) {
            if (vh > 0) {
                nH.store(sH);
                ndH.store(sdH);
                hdh += nH.dot(ndH);   // this slice's <dh, h>, before the registers take the next one
                pin(hdh);
                ndO.store(sdO);
                nV.store(sV);
            }
            if (vh + 1 < Cf::NVH) {
                nH.load(hT + unit * VD * KD, (vh + 1) * 64);
                ndH.load(dhT + unit * VD * KD, (vh + 1) * 64);
                ndO.load(dO + (t0 * HV + hv) * VD + (vh + 1) * 64, (long)HV * VD, Cn);
                nV.load(v + (t0 * HV + hv) * VD + (vh + 1) * 64, (long)HV * VD, Cn);
            } else {
                nQ.load(q + (t0 * HK + hk) * KD, (long)HK * KD, Cn);
            }
            lds_barrier();
            // ---- Kh, K dh, Pmᵀ dO  ->  Z = diag(β)(V − diag(γ) Kh),  dV_new
            {
                f32x4 kh[2][TNS], kdh[2][TNS], pdo[2][TNS];
                zero_acc(kh);
                zero_acc(kdh);
                zero_acc(pdo);
                wgemm<E, 2, TNS, KD, false, false>(kh, sK, LK, sH, LK, m0, n0s);
                wgemm<E, 2, TNS, KD, false, false>(kdh, sK, LK, sdH, LK, m0, n0s);
                wgemm<E, 2, TNS, 64, true, true>(pdo, sPm, LA, sdO, LS, m0, n0s);
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < TNS; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int rr = acc_row(m0, i, e), cc = acc_col(n0s, j);
                        const float z = sB[rr] * ((float)sV[rr * LS + cc] - sGam[rr] * kh[i][j][e]);
                        sVn[rr * LS + cc] = to_e<E>(z);
                        sdVn[rr * LS + cc] = to_e<E>(pdo[i][j][e] + __expf(gl - sG[rr]) * kdh[i][j][e]);
                    }
            }
            lds_barrier();
            // ---- V_new = A Z
            {
                f32x4 vn[2][TNS];
                zero_acc(vn);
                wgemm<E, 2, TNS, 64, false, true>(vn, sA, LA, sVn, LS, m0, n0s);
                if constexpr (!Cf::VN2) lds_barrier();   // V_new overwrites Z
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < TNS; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) sVn2[acc_row(m0, i, e) * LS + acc_col(n0s, j)] = to_e<E>(vn[i][j][e]);
            }
            lds_barrier();
            // ---- accumulate the state products and the V-separable outputs
            wgemm<E, 2, TNS, 64, false, false>(dPm, sdO, LS, sVn2, LS, m0, n0s);    // dO V_newᵀ
            wgemm<E, 2, TNK, 64, false, true>(dqi, sdO, LS, sH, LK, m0, n0k);    // dO hᵀ
            wgemm<E, 2, TNK, 64, false, true>(dWa, sdVn, LS, sH, LK, m0, n0k);   // dV_new hᵀ
            wgemm<E, 2, TNK, 64, false, true>(dks, sVn2, LS, sdH, LK, m0, n0k);  // V_new dhᵀ
            wgemm<E, 2, TNS, 64, false, false>(dAp, sdVn, LS, sV, LS, m0, n0s);     // dV_new Vᵀ
            {
                f32x4 adv[2][TNS];
                zero_acc(adv);
                wgemm<E, 2, TNS, 64, true, true>(adv, sA, LA, sdVn, LS, m0, n0s);    // Aᵀ dV_new
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < TNS; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int rr = acc_row(m0, i, e), cc = acc_col(n0s, j);
                        rowB[i][e] += adv[i][j][e] * (float)sV[rr * LS + cc];
                        if constexpr (Cf::DV_LDS) sDv[rr * LS + cc] = to_e<E>(sB[rr] * adv[i][j][e]);
                        else if (rr < Cn) ((E*)a.dv)[((t0 + rr) * HV + hv) * VD + vh * 64 + cc] = to_e<E>(sB[rr] * adv[i][j][e]);
                    }
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int e = 0; e < 4; e++) pin(rowB[i][e]);
            }
            lds_barrier();
            if constexpr (Cf::DV_LDS) store_rows<E, 64, LS>((E*)a.dv + (t0 * HV + hv) * VD + vh * 64, (long)HV * VD, sDv, Cn);
        }

        // ---- Q back into its buffer (it held the V slices)
        nQ.store(sQ);
        // ---- F = dPm ⊙ Pm -> dG; T1 = dPm ⊙ Γ · scale (over Pm); dW -> LDS
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < TNS; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int rr = acc_row(m0, i, e), cc = acc_col(n0s, j);
                const bool lo = cc <= rr;
                const float dp = lo ? dPm[i][j][e] : 0.f;
                const float f = dp * (float)sPm[rr * LA + cc];
                rowG[i][e] += f;
                colG[j] += f;
                sPm[rr * LA + cc] = to_e<E>(lo ? dp * scale * __expf(sG[rr] - sG[cc]) : 0.f);
            }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) pin(rowG[i][e]);
#pragma unroll
        for (int j = 0; j < TNS; j++) pin(colG[j]);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < TNK; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) sdW[acc_row(m0, i, e) * LK + acc_col(n0k, j)] = to_e<E>(-dWa[i][j][e]);
        lds_barrier();
        E* sT1 = sPm;

        // ---- dq = scale γ dO hᵀ + T1 K ;  dG += rowsum(Q ⊙ scale γ dO hᵀ)
        {
            f32x4 t1k[2][TNK];
            zero_acc(t1k);
            wgemm<E, 2, TNK, 64, false, true>(t1k, sT1, LA, sK, LK, m0, n0k);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNK; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int rr = acc_row(m0, i, e), cc = acc_col(n0k, j);
                        const float di = scale * sGam[rr] * dqi[i][j][e];
                        rowG[i][e] += di * (float)sQ[rr * LK + cc];
                        dq_tot[i][j][e] = di + t1k[i][j][e];
                    }
        }
        // ---- dk: T1ᵀ Q + diag(γ_C/γ) V_new dhᵀ (z terms) + diag(βγ) Aᵀ dW
        float zsum = 0.f;
        {
            f32x4 acc[2][TNK];
            zero_acc(acc);
            wgemm<E, 2, TNK, 64, true, true>(acc, sT1, LA, sQ, LK, m0, n0k);
            f32x4 adw[2][TNK];
            zero_acc(adw);
            wgemm<E, 2, TNK, 64, true, true>(adw, sA, LA, sdW, LK, m0, n0k);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNK; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int rr = acc_row(m0, i, e), cc = acc_col(n0k, j);
                        const float kv = (float)sK[rr * LK + cc];
                        const float ds = __expf(gl - sG[rr]) * dks[i][j][e];
                        const float z = ds * kv;
                        rowG[i][e] -= z;
                        zsum += z;
                        const float aw = adw[i][j][e] * kv;
                        rowB[i][e] += sGam[rr] * aw;
                        rowG[i][e] += sB[rr] * sGam[rr] * aw;
                        dk_tot[i][j][e] = acc[i][j][e] + ds + sB[rr] * sGam[rr] * adw[i][j][e];
                    }
        }
        // ---- dA_pre = dV_new (diag(β)V)ᵀ + dW (diag(βγ)K)ᵀ  -> LDS
        {
            f32x4 dwk[2][TNS];
            zero_acc(dwk);
            wgemm<E, 2, TNS, KD, false, false>(dwk, sdW, LK, sK, LK, m0, n0s);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNS; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int rr = acc_row(m0, i, e), cc = acc_col(n0s, j);
                    sdA[rr * LA + cc] = to_e<E>(sB[cc] * (dAp[i][j][e] + sGam[cc] * dwk[i][j][e]));
                }
        }
        lds_barrier();
        // ---- M1 = Aᵀ dA_pre
        {
            f32x4 m1[2][TNS];
            zero_acc(m1);
            wgemm<E, 2, TNS, 64, true, true>(m1, sA, LA, sdA, LA, m0, n0s);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNS; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) sM1[acc_row(m0, i, e) * LA + acc_col(n0s, j)] = to_e<E>(m1[i][j][e]);
        }
        lds_barrier();
        // ---- dL = −strictlower(M1 Aᵀ); dβ, dG (F2); Eb = diag(β) dL ⊙ Γ
        {
            f32x4 dl[2][TNS], akk[2][TNS];
            zero_acc(dl);
            zero_acc(akk);
            wgemm<E, 2, TNS, 64, false, false>(dl, sM1, LA, sA, LA, m0, n0s);
            wgemm<E, 2, TNS, KD, false, false>(akk, sK, LK, sK, LK, m0, n0s);   // K Kᵀ (recomputed)
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNS; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int rr = acc_row(m0, i, e), cc = acc_col(n0s, j);
                    const bool lo = cc < rr;
                    const float d = lo ? -dl[i][j][e] : 0.f;
                    const float lg = lo ? __expf(sG[rr] - sG[cc]) * akk[i][j][e] : 0.f;   // Γ ⊙ KKᵀ
                    rowB[i][e] += d * lg;
                    const float f2 = d * sB[rr] * lg;
                    rowG[i][e] += f2;
                    colG[j] += f2;
                    sEb[rr * LA + cc] = to_e<E>(lo ? sB[rr] * d * __expf(sG[rr] - sG[cc]) : 0.f);
                }
        }
        lds_barrier();
        // ---- dk += Eb K + Ebᵀ K
        {
            f32x4 acc[2][TNK];
            zero_acc(acc);
            wgemm<E, 2, TNK, 64, false, true>(acc, sEb, LA, sK, LK, m0, n0k);
            wgemm<E, 2, TNK, 64, true, true>(acc, sEb, LA, sK, LK, m0, n0k);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNK; j++) dk_tot[i][j] += acc[i][j];
        }

        // ---- reductions (fixed order): rows over the 16 lanes of a group and
        // the two column blocks; columns over the 4 row groups and 2 row halves
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float rg = sum16(rowG[i][e]);
                const float rb = sum16(rowB[i][e]);
                // every lane of the group holds the sum: all write the same value (no branch)
                const int rr = acc_row(m0, i, e);
                sRowG[(w >> 1) * 64 + rr] = rg;
                sRowB[(w >> 1) * 64 + rr] = rb;
            }
#pragma unroll
        for (int j = 0; j < TNS; j++) {   // all four row groups hold the sum and write it (no branch)
            const float cs = sum4g(colG[j]);
            sCol[(w & 1) * 64 + acc_col(n0s, j)] = cs;
        }
        {
            float hz = hdh, zz = zsum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                hz += __shfl_xor(hz, off, 64);
                zz += __shfl_xor(zz, off, 64);
            }
            sMisc[w] = hz;   // every lane holds the sum (no branch)
            sMisc[8 + w] = zz;
        }
        lds_barrier();
        if (threadIdx.x < 64) {
            const int rr = threadIdx.x;
            float dG = -(sCol[rr] + sCol[64 + rr]), db = 0.f;
#pragma unroll
            for (int cb = 0; cb < GNCB; cb++) {
                dG += sRowG[cb * 64 + rr];
                db += sRowB[cb * 64 + rr];
            }
            if (rr == C - 1) {
                float hd = 0.f, zs = 0.f;
                for (int i = 0; i < GNT / 64; i++) { hd += sMisc[i]; zs += sMisc[8 + i]; }
                dG += zs + gC * hd;
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
        if constexpr (GRP) {   // group sums through the workspace block of this (chunk, key head)
            float* st = a.gsum + ((long)ci * HK + hk) * 2 * 64 * KD;
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < TNK; j++) {
                    const int tl = (w * 2 + i) * TNK + j;
                    f32x4* pq = (f32x4*)(st + (tl * 64 + l) * 4);
                    f32x4* pk = (f32x4*)(st + 64 * KD + (tl * 64 + l) * 4);
                    if (hi > 0) {
                        dq_tot[i][j] += *pq;
                        dk_tot[i][j] += *pk;
                    }
                    if (hi + 1 < G) {
                        *pq = dq_tot[i][j];
                        *pk = dk_tot[i][j];
                    }
                }
            if (hi + 1 < G) return;   // uniform: only the last head of the group stores dq, dk
        }
    }
    // ---- the group sums dq, dk for this key head, through LDS (sH and sdH were last
    //      read before the dA_pre and M1 barriers above)
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < TNK; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int rr = acc_row(m0, i, e), cc = acc_col(n0k, j);
                sH[rr * LK + cc] = to_e<E>(dq_tot[i][j][e]);
                sdH[rr * LK + cc] = to_e<E>(dk_tot[i][j][e]);
            }
    lds_barrier();
    store_rows<E, KD, LK>((E*)a.dq + (t0 * HK + hk) * KD, (long)HK * KD, sH, Cn);
    store_rows<E, KD, LK>((E*)a.dk + (t0 * HK + hk) * KD, (long)HK * KD, sdH, Cn);
}

template <class E, int KD, int VD, bool GRP>
static hipError_t grad_go1(const Problem& p, const GradArgs& a, hipStream_t s) {
    using Cf = GradCfg<E, KD, VD>;
    static_assert(Cf::smem <= 160 * 1024, "LDS budget");
    auto kern = grad_kernel<E, KD, VD, GRP>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem);
    if (e != hipSuccess) return e;
    const int G = GRP ? p.HV / p.HK : 1;
    for (int hi = 0; hi < G; hi++) {
        hipLaunchKernelGGL(kern, dim3((unsigned)p.NT, p.HK), dim3(GNT), Cf::smem, s, a, p.HK, p.HV, p.scale, hi);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class E, int KD, int VD>
static hipError_t grad_go(const Problem& p, const GradArgs& a, hipStream_t s) {
    if (p.HV == p.HK) return grad_go1<E, KD, VD, false>(p, a, s);
    if (!a.gsum) return hipErrorInvalidValue;
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
