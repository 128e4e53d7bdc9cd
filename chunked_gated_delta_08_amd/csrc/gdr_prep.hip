// gdr_prep.hip -- chunk table and the per-chunk WY factors (K1a).
//
// For one chunk of C <= 64 rows and one value head, with the in-chunk
// cumulative log-gate G (γ_r = e^{G_r}, Γ_rs = e^{G_r - G_s}, s <= r):
//   L  = strictly-lower( diag(β) (K Kᵀ) ⊙ Γ ),   A = (I + L)^{-1}
//   W  = A diag(βγ) K,    U = A diag(β) V
//   Pm = scale · lower( Γ ⊙ Q Kᵀ )   (diagonal included)
//   R  = scale · diag(γ) Q − Pm W
// A itself is also written out (input type) for the gradient kernel, and
// K̃ = diag(γ_C/γ) K (scan operand type) for both scans.
// W and U drive the forward state scan (V_new = U − W h); R and W drive the
// reverse scan in the form dh ← γ_C dh + Rᵀ dO − Wᵀ (K̃ dh) given on the
// FlashQLA backward explainer page (§三, the dh kernel's three consumer groups:
// R = Q − Lower(P)·X with X = A·K, and Y = K·dh).
// Rows r >= C of a partial chunk are zero in K, Q, V, β; their gate is padded
// with G_{C-1}, so every padded row of W, U, R is exactly zero.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"
#include "gdr_tri.hpp"

namespace gdr {

__device__ __forceinline__ int last_le(const int32_t* __restrict__ a, int n, int x) {
    // largest i in [0, n) with a[i] <= x (a non-decreasing, a[0] <= x)
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// One workgroup: per-sequence chunk and segment counts (at least one segment
// per sequence, so that an empty sequence still gets its dh0), their exclusive
// prefix sums (seq_chunk0, seq_seg0, each with the total at [nseq]), then the
// chunk table and the segment table filled in parallel (binary search of
// each entry's sequence in the prefix arrays).  seg_order (if wanted): the
// segments ranked by descending chunk count, ties by index, so the scans can
// start the longest jobs first; each rank is a count over all segments (up to
// 1024 of them, held in LDS; beyond that, index order).
__global__ void __launch_bounds__(1024) chunk_table_kernel(const int32_t* __restrict__ cu, int N, int B, int T,
                                                           int BT, int L, ChunkInfo* __restrict__ info,
                                                           int32_t* __restrict__ seq_chunk0,
                                                           SegInfo* __restrict__ seg,
                                                           int32_t* __restrict__ seq_seg0,
                                                           int32_t* __restrict__ seg_order) {
    __shared__ int pc[1024], ps[1024], snc[1024];
    const int nseq = cu ? N : B;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (nseq + nt - 1) / nt;
    const int s0 = min(nseq, tid * per), s1 = min(nseq, s0 + per);
    int cc = 0, cs = 0;
    for (int n = s0; n < s1; n++) {
        const int len = cu ? (cu[n + 1] - cu[n]) : T;
        const int nc = (len + BT - 1) / BT;
        cc += nc;
        cs += nc > L ? (nc + L - 1) / L : 1;   // every sequence has a segment, empty ones too
    }
    pc[tid] = cc;
    ps[tid] = cs;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {   // inclusive scan (Hillis-Steele)
        const int a = tid >= off ? pc[tid - off] : 0, b = tid >= off ? ps[tid - off] : 0;
        __syncthreads();
        pc[tid] += a;
        ps[tid] += b;
        __syncthreads();
    }
    int bc = pc[tid] - cc, bs = ps[tid] - cs;
    for (int n = s0; n < s1; n++) {
        const int len = cu ? (cu[n + 1] - cu[n]) : T;
        const int nc = (len + BT - 1) / BT;
        seq_chunk0[n] = bc;
        seq_seg0[n] = bs;
        bc += nc;
        bs += nc > L ? (nc + L - 1) / L : 1;
    }
    if (tid == nt - 1) {
        seq_chunk0[nseq] = pc[nt - 1];
        seq_seg0[nseq] = ps[nt - 1];
    }
    __syncthreads();
    const int NT = pc[nt - 1], NS = ps[nt - 1];
    for (int c = tid; c < NT; c += nt) {
        const int n = last_le(seq_chunk0, nseq, c);
        const int lc = c - seq_chunk0[n];
        const int bos = cu ? cu[n] : n * T;
        const int len = cu ? (cu[n + 1] - cu[n]) : T;
        ChunkInfo ci;
        ci.seq = n;
        ci.t0 = bos + lc * BT;
        ci.len = min(BT, len - lc * BT);
        ci.pad = lc;
        info[c] = ci;
    }
    for (int j = tid; j < NS; j += nt) {
        const int n = last_le(seq_seg0, nseq, j);
        const int ls = j - seq_seg0[n];
        const int nc = seq_chunk0[n + 1] - seq_chunk0[n];
        SegInfo si;
        si.seq = n;
        si.lc0 = ls * L;
        si.c0 = seq_chunk0[n] + si.lc0;
        si.nc = min(L, nc - si.lc0);
        seg[j] = si;
        if (NS <= nt) snc[j] = si.nc;
    }
    if (!seg_order) return;
    if (NS > nt) {
        for (int j = tid; j < NS; j += nt) seg_order[j] = j;
        return;
    }
    __syncthreads();
    if (tid < NS) {
        const int c = snc[tid];
        int rank = 0;
        for (int i = 0; i < NS; i++) rank += snc[i] > c || (snc[i] == c && i < tid);
        seg_order[rank] = tid;
    }
}

hipError_t launch_chunk_table(const Problem& p, ChunkInfo* info, int32_t* seq_chunk0, SegInfo* seg,
                              int32_t* seq_seg0, int32_t* seg_order, hipStream_t s) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, s, p.cu, p.N, p.B, p.T, p.BT, p.L, info,
                       seq_chunk0, seg, seq_seg0, seg_order);
    return hipGetLastError();
}

// ---------------------------------------------------------------- helpers
// Copy a [64][D] LDS tile out to a dense row-major [64][D] block.  Every
// thread issues the same fixed number of 16-byte stores, so the compiler can
// count them and later waits on loads need not wait for these stores.
template <class E, int D, int LD, int NTHR>
__device__ __forceinline__ void store_tile_dense(E* __restrict__ g, const E* s) {
    constexpr int EPV = 16 / sizeof(E);
    constexpr int VPR = D / EPV;
    static_assert(64 * VPR % NTHR == 0, "whole vectors per thread");
#pragma unroll
    for (int it = 0; it < 64 * VPR / NTHR; it++) {
        const int idx = threadIdx.x + NTHR * it;
        const int r = idx / VPR, c = idx % VPR;
        typename Vec16<E>::t v;
#pragma unroll
        for (int e = 0; e < EPV; e++) v[e] = s[r * LD + c * EPV + e];
        *(typename Vec16<E>::t*)(g + (long)r * D + c * EPV) = v;
    }
}

template <class E> constexpr int pad_of() { return sizeof(E) == 2 ? 8 : 4; }

// ---------------------------------------------------------------- K1a
// LDS carve-up of the WY-factor kernel (byte offsets).  Regions are reused
// along the unit's phases: L becomes A in place (the inverse), then holds V
// (staged from registers once A is consumed) and U; the inverse's scratch and
// later W live over the two scaled copies of A.  16-bit at K = V = 128:
// 80,384 bytes, so two workgroups share a CU.
template <class E, class S, int KD, int VD>
struct PrepCfg {
    static constexpr int C = 64;
    static constexpr int LK = KD + pad_of<S>(), LV = VD + pad_of<S>(), LA = 64 + pad_of<S>(), LL = 68;
    static constexpr size_t szK = (size_t)C * LK * sizeof(S), szV = (size_t)C * LV * sizeof(S);
    static constexpr size_t szL = (size_t)C * LL * 4, szA = (size_t)C * LA * sizeof(S);
    static constexpr size_t oK = 0;                                    // K [64][LK] S (later R)
    static constexpr size_t oQ = oK + szK;                             // Q [64][LK] S
    static constexpr size_t oL = oQ + szK;                             // L -> A [64][LL] fp32, then V -> U [64][LV] S
    static constexpr size_t oPm = oL + (szL > szV ? szL : szV);        // Pm [64][LA] S
    static constexpr size_t oAw = oPm + szA;                           // A diag(βγ) [64][LA] S (inverse scratch before, W after)
    static constexpr size_t oAu = oAw + szA;                           // A diag(β) [64][LA] S
    static constexpr size_t oG = oAu + szA;                            // G, β [64] fp32
    static constexpr size_t smem = oG + (size_t)2 * C * 4;
    static_assert((size_t)4 * 2 * 16 * 17 * 4 <= 2 * szA, "inverse scratch over the scaled copies of A");
    static_assert(szK <= 2 * szA, "W over the scaled copies of A");
    static_assert(smem <= 160 * 1024, "LDS budget");
};

// Four waves per workgroup (the in-place inverse works on four 16-row block
// rows); 16-bit problems fit two workgroups per CU, so one workgroup's
// barrier-bound phases (the inverse) overlap the other's loads, products and
// stores.
template <class E> constexpr int prep_waves() { return 4; }

// Persistent: workgroup b handles units (chunk, value head) b, b + grid, ...
// Every 64-row product is tiled over the waves as two row halves x two
// column blocks.  The next unit's K, Q, gate and β are loaded into registers
// right after the current ones are staged in LDS, and its V right after the
// current V is staged (after the inverse), so those loads are in flight while
// the current unit is computed.  E: input type; S: scan operand type.
// A 16-byte load, non-temporal when NT (data read once by this launch).
template <bool NT, class T>
__device__ __forceinline__ T ld16(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// NTQK: q and k rows are read by one unit only (HK == HV), so their loads are
// non-temporal like those of v; under GQA the value heads of a group read the
// same rows one unit after another and the loads keep them in the caches.
template <class E, class S, int KD, int VD, bool WITH_R, bool NTQK>
__global__ void __launch_bounds__(64 * prep_waves<E>())
__attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 2 : 1, 2))) prep_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                   const E* __restrict__ v, const float* __restrict__ gcum,
                                                   const E* __restrict__ beta, const ChunkInfo* __restrict__ info,
                                                   int HK, int HV, float scale, S* __restrict__ Wg,
                                                   S* __restrict__ Ug, S* __restrict__ Rg, E* __restrict__ Ag,
                                                   S* __restrict__ KTg, int nunits) {
    static_assert(sizeof(E) == sizeof(S), "input and scan types share a width");
    using Cf = PrepCfg<E, S, KD, VD>;
    constexpr int C = 64, NTHR = 64 * prep_waves<E>(), NCB = prep_waves<E>() / 2;
    constexpr int LK = Cf::LK, LV = Cf::LV, LA = Cf::LA, LL = Cf::LL;
    constexpr int EPV = 16 / (int)sizeof(E);
    extern __shared__ __align__(16) unsigned char smem[];
    S* sK = (S*)(smem + Cf::oK);
    S* sQ = (S*)(smem + Cf::oQ);
    float* sL = (float*)(smem + Cf::oL);   // L, then A in place
    S* sV = (S*)(smem + Cf::oL);           // V, then U (after A is consumed)
    S* sAw = (S*)(smem + Cf::oAw);
    S* sAu = (S*)(smem + Cf::oAu);
    S* sW = (S*)(smem + Cf::oAw);          // W (after the W and U products)
    float* sT = (float*)(smem + Cf::oAw);  // the inverse's scratch
    S* sPm = (S*)(smem + Cf::oPm);
    float* sG = (float*)(smem + Cf::oG);
    float* sB = sG + C;

    const int w = wave_id();
    const int m0 = 32 * (w & 1);                // row half of every 64-row output
    static_assert(C * KD / EPV % NTHR == 0 && C * VD / EPV % NTHR == 0, "whole vectors per thread");
    constexpr int NKV = C * KD / EPV / NTHR, NVV = C * VD / EPV / NTHR;
    typename Vec16<E>::t rk[NKV], rv[NVV], rq[WITH_R ? NKV : 1];
    float rg = 0.f;
    E rb = E(0.f);   // raw β: converted and masked when staged (a conversion here would wait for the loads)
    // issue the loads of unit u (rows past the chunk read its last row; they
    // are zeroed when staged): gate, β, K, Q, then V separately
    auto issue_kq = [&](int u, int Cu, int tu) {
        const int hvu = u % HV, hku = hvu / (HV / HK);
        if (threadIdx.x < C) {   // first, so that waiting for them leaves the vectors in flight
            const int r = min((int)threadIdx.x, Cu - 1);
            rg = gcum[(tu + r) * HV + hvu];
            rb = beta[(tu + r) * HV + hvu];
        }
#pragma unroll
        for (int i = 0; i < NKV; i++) {
            const int idx = threadIdx.x + NTHR * i, r = min(idx / (KD / EPV), Cu - 1), cc = idx % (KD / EPV);
            rk[i] = ld16<NTQK>((const typename Vec16<E>::t*)(k + ((tu + r) * HK + hku) * KD + cc * EPV));
            if constexpr (WITH_R)
                rq[i] = ld16<NTQK>((const typename Vec16<E>::t*)(q + ((tu + r) * HK + hku) * KD + cc * EPV));
        }
    };
    auto issue_v = [&](int u, int Cu, int tu) {
        const int hvu = u % HV;
#pragma unroll
        for (int i = 0; i < NVV; i++) {
            const int idx = threadIdx.x + NTHR * i, r = min(idx / (VD / EPV), Cu - 1), cc = idx % (VD / EPV);
            rv[i] = ld16<true>((const typename Vec16<E>::t*)(v + ((tu + r) * HV + hvu) * VD + cc * EPV));
        }
    };
    auto to_s = [](const typename Vec16<E>::t& x, float f, bool keep) {
        typename Vec16<S>::t y;
#pragma unroll
        for (int e = 0; e < EPV; e++) y[e] = keep ? (S)(f * (float)x[e]) : (S)0.f;
        return y;
    };

    int u = blockIdx.x;
    if (u >= nunits) return;
    int cur_len = info[u / HV].len, cur_t0 = info[u / HV].t0;
    issue_kq(u, cur_len, cur_t0);
    issue_v(u, cur_len, cur_t0);
    for (; u < nunits; u += gridDim.x) {
    const int ci = u / HV, hv = u % HV;
    const int Cn = cur_len;
    const long t0 = cur_t0;
    const long unit = (long)ci * HV + hv;
    const int un = u + (int)gridDim.x;
    // read early: used for the prefetch below
    const int nxt_len = un < nunits ? info[un / HV].len : 1, nxt_t0 = un < nunits ? info[un / HV].t0 : 0;

    // ---- stage this unit
    if (threadIdx.x < C) {
        sG[threadIdx.x] = rg;
        sB[threadIdx.x] = (int)threadIdx.x < Cn ? (float)rb : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NKV; i++) {
        const int idx = threadIdx.x + NTHR * i, r = idx / (KD / EPV), c = idx % (KD / EPV);
        *(typename Vec16<S>::t*)(sK + r * LK + c * EPV) = to_s(rk[i], 1.f, r < Cn);
        if constexpr (WITH_R) *(typename Vec16<S>::t*)(sQ + r * LK + c * EPV) = to_s(rq[i], 1.f, r < Cn);
    }
    lds_barrier();

    // ---- K̃ = diag(γ_C/γ) K straight from the registers
    {
        const float gl = sG[C - 1];
        S* KTo = KTg + unit * C * KD;
#pragma unroll
        for (int i = 0; i < NKV; i++) {
            const int idx = threadIdx.x + NTHR * i, r = idx / (KD / EPV), c = idx % (KD / EPV);
            *(typename Vec16<S>::t*)(KTo + r * KD + c * EPV) = to_s(rk[i], __expf(gl - sG[r]), r < Cn);
        }
    }
    // ---- the next unit's K, Q, gate and β fly during this unit's compute
    if (un < nunits) issue_kq(un, nxt_len, nxt_t0);

    // ---- S_kk = K Kᵀ -> L ;  S_qk = Q Kᵀ -> Pm     (wave w: 32 rows x 64/NCB columns)
    {
        constexpr int TN = 4 / NCB;
        const int n0 = (64 / NCB) * (w >> 1);
        f32x4 akk[2][TN], aqk[2][TN];
        zero_acc(akk);
        wgemm_rf<S, 2, TN, KD, false, false>(akk, sK, LK, sK, LK, m0, n0);
        if (WITH_R) {
            zero_acc(aqk);
            wgemm_rf<S, 2, TN, KD, false, false>(aqk, sQ, LK, sK, LK, m0, n0);
        }
        // row form: four adjacent columns of one row per lane (16-byte L and
        // 8-byte Pm stores); branch-free: Γ_rc = exp(min(G_r − G_c, 0)), then
        // masked by a select
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r = rf_row(m0, i);
            const float gr = sG[r], br = sB[r];
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int c0 = rf_col(n0, j);
                const f32x4 gc = *(const f32x4*)(sG + c0);
                f32x4 lv, pv;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float gm = __expf(fminf(gr - gc[e], 0.f));
                    lv[e] = c0 + e < r ? br * gm * akk[i][j][e] : 0.f;
                    pv[e] = c0 + e <= r ? scale * gm * aqk[i][j][e] : 0.f;
                }
                *(f32x4*)(sL + r * LL + c0) = lv;
                if (WITH_R) st4<S>(sPm + r * LA + c0, pv);
            }
        }
    }
    lds_barrier();

    // ---- A = (I+L)^{-1}, in place
    float* sAf = sL;
    tri_inverse64_inplace<LL>(sL, sT);

    // ---- A diag(βγ), A diag(β) as MFMA operands (over the inverse's scratch);
    //      A itself to memory (input type)
    {
        E* Ao = Ag ? Ag + unit * C * C : nullptr;
        for (int idx = threadIdx.x; idx < C * C / EPV; idx += NTHR) {
            const int r = idx / (C / EPV), c0 = (idx % (C / EPV)) * EPV;
            typename Vec16<S>::t aw, au;
            typename Vec16<E>::t ao;
#pragma unroll
            for (int e = 0; e < EPV; e++) {
                const float x = sAf[r * LL + c0 + e], b = sB[c0 + e];
                aw[e] = (S)(x * b * __expf(sG[c0 + e]));
                au[e] = (S)(x * b);
                ao[e] = (E)x;
            }
            *(typename Vec16<S>::t*)(sAw + r * LA + c0) = aw;
            *(typename Vec16<S>::t*)(sAu + r * LA + c0) = au;
            if (Ao) *(typename Vec16<E>::t*)(Ao + r * C + c0) = ao;
        }
    }
    lds_barrier();   // A is read: V takes its region
#pragma unroll
    for (int i = 0; i < NVV; i++) {
        const int idx = threadIdx.x + NTHR * i, r = idx / (VD / EPV), c = idx % (VD / EPV);
        *(typename Vec16<S>::t*)(sV + r * LV + c * EPV) = to_s(rv[i], 1.f, r < Cn);
    }
    if (un < nunits) issue_v(un, nxt_len, nxt_t0);   // the next unit's V flies from here
    lds_barrier();

    // ---- W = A diag(βγ) K, U = A diag(β) V     (wave w: 32 rows, KD/NCB resp. VD/NCB columns)
    constexpr int TNK = KD / 16 / NCB, TNV = VD / 16 / NCB;
    const int n0k = (KD / NCB) * (w >> 1), n0v = (VD / NCB) * (w >> 1);
    // (one product's accumulators live at a time: U first, stored over V,
    // then W, stored over the copies of A)
    {
        f32x4 au[2][TNV];
        zero_acc(au);
        wgemm_rf<S, 2, TNV, 64, false, true>(au, sAu, LA, sV, LV, m0, n0v);
        lds_barrier();   // V is read: U takes its place
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < TNV; j++) st4<S>(sV + rf_row(m0, i) * LV + rf_col(n0v, j), au[i][j]);
    }
    {
        f32x4 aw[2][TNK];
        zero_acc(aw);
        wgemm_rf<S, 2, TNK, 64, false, true>(aw, sAw, LA, sK, LK, m0, n0k);
        lds_barrier();   // the copies of A are read: W takes their place
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < TNK; j++) st4<S>(sW + rf_row(m0, i) * LK + rf_col(n0k, j), aw[i][j]);
    }
    lds_barrier();

    if (WITH_R) {
        // ---- R = scale diag(γ) Q − Pm W
        f32x4 ar[2][TNK];
        zero_acc(ar);
        wgemm_rf<S, 2, TNK, 64, false, true>(ar, sPm, LA, sW, LK, m0, n0k);
        store_tile_dense<S, KD, LK, NTHR>(Wg + unit * C * KD, sW);
        store_tile_dense<S, VD, LV, NTHR>(Ug + unit * C * VD, sV);
        S* sR = sK;   // K is no longer read
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r = rf_row(m0, i);
            const float sgr = scale * __expf(sG[r]);
#pragma unroll
            for (int j = 0; j < TNK; j++) {
                const int c0 = rf_col(n0k, j);
                st4<S>(sR + r * LK + c0, sgr * ld4<S>(sQ + r * LK + c0) - ar[i][j]);
            }
        }
        lds_barrier();
        store_tile_dense<S, KD, LK, NTHR>(Rg + unit * C * KD, sR);
    } else {
        store_tile_dense<S, KD, LK, NTHR>(Wg + unit * C * KD, sW);
        store_tile_dense<S, VD, LV, NTHR>(Ug + unit * C * VD, sV);
    }
    lds_barrier();   // the next unit is staged over this one's LDS
    cur_len = nxt_len;
    cur_t0 = nxt_t0;
    }
}

template <class E, class S, int KD, int VD>
static size_t prep_smem() {
    return PrepCfg<E, S, KD, VD>::smem;
}

template <class E, class S, int KD, int VD>
static hipError_t prep_go(const Problem& p, const void* q, const void* k, const void* v, const float* gcum,
                          const void* beta, const ChunkInfo* info, void* W, void* U, void* R, void* A, void* KT,
                          hipStream_t s) {
    const size_t sm = prep_smem<E, S, KD, VD>();
    const long nunits = p.NT * p.HV;
    if (nunits > INT32_MAX) return hipErrorInvalidValue;
    // persistent workgroups: as many per CU as the LDS carve-up allows (two
    // for 16-bit problems, at most two: two waves per SIMD), 256 CUs
    const long per_cu = sm * 2 <= 160 * 1024 ? 2 : 1, nwg = 256 * per_cu;
    dim3 grid((unsigned)(nunits < nwg ? nunits : nwg));
    auto go = [&](auto kern, void* R_) {
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm) != hipSuccess)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kern, grid, dim3(64 * prep_waves<E>()), sm, s, (const E*)q, (const E*)k, (const E*)v, gcum,
                           (const E*)beta, info, p.HK, p.HV, p.scale, (S*)W, (S*)U, (S*)R_, (E*)A, (S*)KT, (int)nunits);
        return hipSuccess;
    };
    const bool own_qk = p.HK == p.HV;
    hipError_t e;
    if (q) e = own_qk ? go(prep_kernel<E, S, KD, VD, true, true>, R) : go(prep_kernel<E, S, KD, VD, true, false>, R);
    else
        e = own_qk ? go(prep_kernel<E, S, KD, VD, false, true>, nullptr)
                   : go(prep_kernel<E, S, KD, VD, false, false>, nullptr);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_prep(const Problem& p, const void* q, const void* k, const void* v, const float* gcum,
                       const void* beta, const ChunkInfo* info, void* W, void* U, void* R, void* A, void* KT,
                       hipStream_t s) {
    // dtype: 0 f32, 1 f16, 2 bf16; the scans use fp16 operands for 16-bit inputs
    if (p.K == 128 && p.V == 128) {
        if (p.dtype == 2) return prep_go<bf16, f16, 128, 128>(p, q, k, v, gcum, beta, info, W, U, R, A, KT, s);
        if (p.dtype == 1) return prep_go<f16, f16, 128, 128>(p, q, k, v, gcum, beta, info, W, U, R, A, KT, s);
        return hipErrorInvalidValue;   // fp32 is built at K = V = 64 only
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 2) return prep_go<bf16, f16, 64, 64>(p, q, k, v, gcum, beta, info, W, U, R, A, KT, s);
        if (p.dtype == 1) return prep_go<f16, f16, 64, 64>(p, q, k, v, gcum, beta, info, W, U, R, A, KT, s);
        return prep_go<float, float, 64, 64>(p, q, k, v, gcum, beta, info, W, U, R, A, KT, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
