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
// each entry's sequence in the prefix arrays).
__global__ void __launch_bounds__(1024) chunk_table_kernel(const int32_t* __restrict__ cu, int N, int B, int T,
                                                           int BT, int L, ChunkInfo* __restrict__ info,
                                                           int32_t* __restrict__ seq_chunk0,
                                                           SegInfo* __restrict__ seg,
                                                           int32_t* __restrict__ seq_seg0) {
    __shared__ int pc[1024], ps[1024];
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
    }
}

hipError_t launch_chunk_table(const Problem& p, ChunkInfo* info, int32_t* seq_chunk0, SegInfo* seg,
                              int32_t* seq_seg0, hipStream_t s) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, s, p.cu, p.N, p.B, p.T, p.BT, p.L, info,
                       seq_chunk0, seg, seq_seg0);
    return hipGetLastError();
}

// ---------------------------------------------------------------- helpers
// Cooperative copy of a [C][D] row block (row stride `rs` elements) into a
// zero-padded [64][LD] LDS tile, converting element type Ein -> Eout.
template <class Ein, class Eout, int D, int LD, int NTHR>
__device__ __forceinline__ void load_rows(Eout* s, const Ein* __restrict__ g, long rs, int C) {
    constexpr int EPV = 16 / sizeof(Ein);  // elements per 16-byte vector
    constexpr int VPR = D / EPV;
    for (int idx = threadIdx.x; idx < 64 * VPR; idx += NTHR) {
        const int r = idx / VPR, c = idx % VPR;
        typename Vec16<Ein>::t v;
        if (r < C) v = *(const typename Vec16<Ein>::t*)(g + r * rs + c * EPV);
        else v = typename Vec16<Ein>::t{};
#pragma unroll
        for (int e = 0; e < EPV; e++) s[r * LD + c * EPV + e] = (Eout)(float)v[e];
    }
}

// Copy a [64][D] LDS tile (rows < C) out to a dense row-major [64][D] block.
template <class E, int D, int LD, int NTHR>
__device__ __forceinline__ void store_tile_dense(E* __restrict__ g, const E* s) {
    constexpr int EPV = 16 / sizeof(E);
    constexpr int VPR = D / EPV;
    for (int idx = threadIdx.x; idx < 64 * VPR; idx += NTHR) {
        const int r = idx / VPR, c = idx % VPR;
        typename Vec16<E>::t v;
#pragma unroll
        for (int e = 0; e < EPV; e++) v[e] = s[r * LD + c * EPV + e];
        *(typename Vec16<E>::t*)(g + (long)r * D + c * EPV) = v;
    }
}

template <class E> constexpr int pad_of() { return sizeof(E) == 2 ? 8 : 4; }

// ---------------------------------------------------------------- K1a
// Grid (NT, HV), 256 threads.  E: input type; S: scan operand type.
template <class E, class S, int KD, int VD, bool WITH_R>
__global__ void __launch_bounds__(256) prep_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                   const E* __restrict__ v, const float* __restrict__ gcum,
                                                   const E* __restrict__ beta, const ChunkInfo* __restrict__ info,
                                                   int HK, int HV, float scale, S* __restrict__ Wg,
                                                   S* __restrict__ Ug, S* __restrict__ Rg, E* __restrict__ Ag,
                                                   S* __restrict__ KTg) {
    static_assert(sizeof(E) == sizeof(S), "input and scan types share a width");
    constexpr int C = 64, NTHR = 256;
    constexpr int LK = KD + pad_of<E>(), LV = VD + pad_of<E>(), LA = 64 + pad_of<E>(), LL = 68;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sK = (E*)smem;                       // K, later Kb = diag(βγ)K (type S)
    E* sV = sK + C * LK;                    // V, later Vb = diag(β)V (type S), later U
    E* sQ = sV + C * LV;                    // Q
    float* sL = (float*)(sQ + C * LK);      // L (fp32), later W (type S)
    constexpr int LW_BYTES = (C * LL * 4 > C * LK * (int)sizeof(S)) ? C * LL * 4 : C * LK * (int)sizeof(S);
    S* sA = (S*)((unsigned char*)sL + LW_BYTES);
    S* sPm = sA + C * LA;
    float* sG = (float*)(sPm + C * LA);
    float* sB = sG + C;
    S* sW = (S*)sL;

    const int ci = blockIdx.x, hv = blockIdx.y, hk = hv / (HV / HK);
    const ChunkInfo ch = info[ci];
    const int Cn = ch.len;
    const long t0 = ch.t0;
    const int w = wave_id(), l = lane_id();

    load_rows<E, E, KD, LK, NTHR>(sK, k + (t0 * HK + hk) * KD, (long)HK * KD, Cn);
    load_rows<E, E, VD, LV, NTHR>(sV, v + (t0 * HV + hv) * VD, (long)HV * VD, Cn);
    if (WITH_R) load_rows<E, E, KD, LK, NTHR>(sQ, q + (t0 * HK + hk) * KD, (long)HK * KD, Cn);
    if (threadIdx.x < C) {
        const int r = threadIdx.x;
        sG[r] = gcum[(t0 + min(r, Cn - 1)) * HV + hv];
        sB[r] = r < Cn ? (float)beta[(t0 + r) * HV + hv] : 0.f;
    }
    lds_barrier();

    // ---- S_kk = K Kᵀ -> L ;  S_qk = Q Kᵀ -> Pm     (wave w: 32x32 block)
    {
        const int m0 = 32 * (w & 1), n0 = 32 * (w >> 1);
        f32x4 akk[2][2], aqk[2][2];
        zero_acc(akk);
        wgemm<E, 2, 2, KD, false, false>(akk, sK, LK, sK, LK, m0, n0);
        if (WITH_R) {
            zero_acc(aqk);
            wgemm<E, 2, 2, KD, false, false>(aqk, sQ, LK, sK, LK, m0, n0);
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = acc_row(m0, i, e), c = acc_col(n0, j);
                    const float gm = (c <= r) ? __expf(sG[r] - sG[c]) : 0.f;
                    sL[r * LL + c] = (c < r) ? sB[r] * gm * akk[i][j][e] : 0.f;
                    if (WITH_R) sPm[r * LA + c] = to_e<S>((c <= r) ? scale * gm * aqk[i][j][e] : 0.f);
                }
    }
    lds_barrier();

    // ---- A = (I+L)^{-1} (wave 0, lane j owns column j); other waves scale K, V
    if (w == 0) {
        float a[C];
#pragma unroll
        for (int r = 0; r < C; r++) {
            float acc = (r == l) ? 1.f : 0.f;
            const float* Lr = sL + r * LL;
#pragma unroll
            for (int s = 0; s < r; s++) acc -= Lr[s] * a[s];
            a[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < C; r++) sA[r * LA + l] = to_e<S>(a[r]);
        if (Ag) {
            E* Ao = Ag + ((long)ci * HV + hv) * C * C;
#pragma unroll
            for (int r = 0; r < C; r++) Ao[r * C + l] = to_e<E>(a[r]);
        }
    } else {
        // Kb = diag(βγ) K written in place as type S; K̃ = diag(γ_C/γ) K to memory
        S* KTo = KTg + ((long)ci * HV + hv) * C * KD;
        for (int idx = threadIdx.x - 64; idx < C * KD; idx += NTHR - 64) {
            const int r = idx / KD, c = idx % KD;
            const float f = sB[r] * __expf(sG[r]);
            const float x = (float)sK[r * LK + c];
            KTo[r * KD + c] = to_e<S>(__expf(sG[C - 1] - sG[r]) * x);
            ((S*)sK)[r * LK + c] = to_e<S>(f * x);
        }
        for (int idx = threadIdx.x - 64; idx < C * VD; idx += NTHR - 64) {
            const int r = idx / VD, c = idx % VD;
            const float x = (float)sV[r * LV + c];
            ((S*)sV)[r * LV + c] = to_e<S>(sB[r] * x);
        }
    }
    lds_barrier();

    // ---- W = A Kb, U = A Vb      (wave w: all 64 rows, KD/4 resp. VD/4 columns)
    constexpr int TNK = KD / 64, TNV = VD / 64;
    f32x4 aw[4][TNK], au[4][TNV];
    zero_acc(aw);
    zero_acc(au);
    wgemm<S, 4, TNK, 64, false, true>(aw, sA, LA, (const S*)sK, LK, 0, w * (KD / 4));
    wgemm<S, 4, TNV, 64, false, true>(au, sA, LA, (const S*)sV, LV, 0, w * (VD / 4));
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = acc_row(0, i, e);
#pragma unroll
            for (int j = 0; j < TNK; j++) sW[r * LK + acc_col(w * (KD / 4), j)] = to_e<S>(aw[i][j][e]);
#pragma unroll
            for (int j = 0; j < TNV; j++) ((S*)sV)[r * LV + acc_col(w * (VD / 4), j)] = to_e<S>(au[i][j][e]);
        }
    lds_barrier();

    const long unit = (long)ci * HV + hv;
    if (WITH_R) {
        // ---- R = scale diag(γ) Q − Pm W
        f32x4 ar[4][TNK];
        zero_acc(ar);
        wgemm<S, 4, TNK, 64, false, true>(ar, sPm, LA, sW, LK, 0, w * (KD / 4));
        store_tile_dense<S, KD, LK, NTHR>(Wg + unit * C * KD, sW);
        store_tile_dense<S, VD, LV, NTHR>(Ug + unit * C * VD, (const S*)sV);
        lds_barrier();
        S* sR = (S*)sK;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = acc_row(0, i, e);
                const float gr = __expf(sG[r]);
#pragma unroll
                for (int j = 0; j < TNK; j++) {
                    const int c = acc_col(w * (KD / 4), j);
                    sR[r * LK + c] = to_e<S>(scale * gr * (float)sQ[r * LK + c] - ar[i][j][e]);
                }
            }
        lds_barrier();
        store_tile_dense<S, KD, LK, NTHR>(Rg + unit * C * KD, sR);
    } else {
        store_tile_dense<S, KD, LK, NTHR>(Wg + unit * C * KD, sW);
        store_tile_dense<S, VD, LV, NTHR>(Ug + unit * C * VD, (const S*)sV);
    }
}

template <class E, class S, int KD, int VD>
static size_t prep_smem() {
    constexpr int C = 64, LK = KD + pad_of<E>(), LV = VD + pad_of<E>(), LA = 64 + pad_of<E>(), LL = 68;
    constexpr int LW_BYTES = (C * LL * 4 > C * LK * (int)sizeof(S)) ? C * LL * 4 : C * LK * (int)sizeof(S);
    return (size_t)C * LK * sizeof(E) * 2 + (size_t)C * LV * sizeof(E) + LW_BYTES + 2 * (size_t)C * LA * sizeof(S) +
           2 * C * sizeof(float);
}

template <class E, class S, int KD, int VD>
static hipError_t prep_go(const Problem& p, const void* q, const void* k, const void* v, const float* gcum,
                          const void* beta, const ChunkInfo* info, void* W, void* U, void* R, void* A, void* KT,
                          hipStream_t s) {
    const size_t sm = prep_smem<E, S, KD, VD>();
    dim3 grid((unsigned)p.NT, p.HV);
    if (q) {
        auto kern = prep_kernel<E, S, KD, VD, true>;
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm) != hipSuccess)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kern, grid, dim3(256), sm, s, (const E*)q, (const E*)k, (const E*)v, gcum, (const E*)beta,
                           info, p.HK, p.HV, p.scale, (S*)W, (S*)U, (S*)R, (E*)A, (S*)KT);
    } else {
        auto kern = prep_kernel<E, S, KD, VD, false>;
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm) != hipSuccess)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kern, grid, dim3(256), sm, s, (const E*)q, (const E*)k, (const E*)v, gcum, (const E*)beta,
                           info, p.HK, p.HV, p.scale, (S*)W, (S*)U, (S*)nullptr, (E*)A, (S*)KT);
    }
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
