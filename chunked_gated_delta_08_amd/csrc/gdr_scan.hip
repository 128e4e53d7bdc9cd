// gdr_scan.hip -- the two sequential chunk scans (K1b forward states, K2 dh).
//
// Forward (state entering chunk c is h[c]; FlashQLA backward explainer §一
// step ②, "recompute h"):
//     V_new = U − W h[c],   h[c+1] = γ_C h[c] + K̃ᵀ V_new,   K̃ = diag(γ_C/γ) K
// Reverse (dh[c] is the gradient of the state leaving chunk c; same page §二
// "dS is walked back chunk by chunk" and §三's R-form of the recursion):
//     dh[c−1] = γ_C dh[c] + Rᵀ dO − Wᵀ (K̃ dh[c]),   dh0 = dh[−1]
// The K̃ row factor γ_C/γ_r is applied to V_new (resp. K dh) rather than to K.
//
// Parallel decomposition: every column of the K x V state evolves on its own
// (all updates multiply the state from the left), so a wave owns a K x 16
// column slice for the whole sequence, in fp32 accumulator registers.  A
// workgroup (4 waves) covers 64 columns; a grid row is (sequence, value head,
// 64-column group).  The state doubles as the MFMA B operand without any data
// movement: the accumulator holds rows {4g..4g+3} of every 16-row tile, so two
// tiles form one 32-deep k block in the permuted order
//     π(8g+i) = 32s + (i < 4 ? 4g + i : 16 + 4g + i − 4),
// and the A operand (W, K, or the transposed Kᵀ/Wᵀ) is read in the same order.
// Operand tiles are staged through LDS; the next-but-one chunk is prefetched
// into registers while the current one is computed.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <class E> constexpr int spad() { return sizeof(E) == 2 ? 8 : 4; }

template <class E, class S, int KD, int VD>
struct ScanCfg {
    static constexpr int C = 64;
    static constexpr int LK = KD + spad<S>();   // [64][KD] tiles
    static constexpr int LS = 64 + spad<S>();   // [64][64] column-group tiles
    static constexpr int NK = C * KD * (int)sizeof(S) / (16 * 256);  // 16-byte vectors per thread, [64][KD]
    static constexpr int NX = C * 64 * (int)sizeof(S) / (16 * 256);  // per thread, [64][64]
    static constexpr int KT = KD / 16;           // state tiles per wave
    static constexpr size_t smem = (size_t)3 * C * LK * sizeof(S) + (size_t)C * LS * sizeof(S) + C * sizeof(float);
};

// Register staging of one chunk's operand tiles (forward: K, W, U slice;
// reverse: K, W, R, dO slice).
template <class E, class S, int KD, int VD, bool REV>
struct Stage {
    using Cf = ScanCfg<E, S, KD, VD>;
    typename Vec16<E>::t k[Cf::NK];
    typename Vec16<S>::t w[Cf::NK];
    typename Vec16<S>::t r[REV ? Cf::NK : 1];
    typename Vec16<E>::t x[REV ? Cf::NX : 1];   // dO slice (reverse)
    typename Vec16<S>::t u[REV ? 1 : Cf::NX];   // U slice (forward)
    float g;
};

template <class E, class S, int KD, int VD, bool REV>
__device__ __forceinline__ void stage_issue(Stage<E, S, KD, VD, REV>& st, const E* __restrict__ k, const E* __restrict__ dO,
                                            const S* __restrict__ W, const S* __restrict__ U, const S* __restrict__ R,
                                            const float* __restrict__ gcum, const ChunkInfo& ch, long unit, int HK,
                                            int HV, int hk, int hv, int vg) {
    using Cf = ScanCfg<E, S, KD, VD>;
    constexpr int EPV = 16 / sizeof(S), VPR = KD / EPV, XPR = 64 / EPV;
    const long t0 = ch.t0;
    const int C = ch.len;
#pragma unroll
    for (int i = 0; i < Cf::NK; i++) {
        const int idx = threadIdx.x + 256 * i, row = idx / VPR, c = idx % VPR;
        if (row < C) st.k[i] = *(const typename Vec16<E>::t*)(k + ((t0 + row) * HK + hk) * KD + c * EPV);
        else st.k[i] = typename Vec16<E>::t{};
        st.w[i] = *(const typename Vec16<S>::t*)(W + (unit * Cf::C + row) * KD + c * EPV);
        if constexpr (REV) st.r[i] = *(const typename Vec16<S>::t*)(R + (unit * Cf::C + row) * KD + c * EPV);
    }
#pragma unroll
    for (int i = 0; i < Cf::NX; i++) {
        const int idx = threadIdx.x + 256 * i, row = idx / XPR, c = idx % XPR;
        if constexpr (REV) {
            if (row < C) st.x[i] = *(const typename Vec16<E>::t*)(dO + ((t0 + row) * HV + hv) * VD + vg * 64 + c * EPV);
            else st.x[i] = typename Vec16<E>::t{};
        } else {
            st.u[i] = *(const typename Vec16<S>::t*)(U + (unit * Cf::C + row) * VD + vg * 64 + c * EPV);
        }
    }
    if (threadIdx.x < Cf::C) st.g = gcum[(t0 + min((int)threadIdx.x, C - 1)) * HV + hv];
}

template <class E, class S, int KD, int VD, bool REV>
__device__ __forceinline__ void stage_commit(const Stage<E, S, KD, VD, REV>& st, S* sK, S* sW, S* sR, S* sX, float* sG) {
    using Cf = ScanCfg<E, S, KD, VD>;
    constexpr int EPV = 16 / sizeof(S), VPR = KD / EPV, XPR = 64 / EPV;
#pragma unroll
    for (int i = 0; i < Cf::NK; i++) {
        const int idx = threadIdx.x + 256 * i, row = idx / VPR, c = idx % VPR;
        typename Vec16<S>::t kv;
#pragma unroll
        for (int e = 0; e < EPV; e++) kv[e] = (S)(float)st.k[i][e];
        *(typename Vec16<S>::t*)(sK + row * Cf::LK + c * EPV) = kv;
        *(typename Vec16<S>::t*)(sW + row * Cf::LK + c * EPV) = st.w[i];
        if constexpr (REV) *(typename Vec16<S>::t*)(sR + row * Cf::LK + c * EPV) = st.r[i];
    }
#pragma unroll
    for (int i = 0; i < Cf::NX; i++) {
        const int idx = threadIdx.x + 256 * i, row = idx / XPR, c = idx % XPR;
        if constexpr (REV) {
            typename Vec16<S>::t xv;
#pragma unroll
            for (int e = 0; e < EPV; e++) xv[e] = (S)(float)st.x[i][e];
            *(typename Vec16<S>::t*)(sX + row * Cf::LS + c * EPV) = xv;
        } else {
            *(typename Vec16<S>::t*)(sX + row * Cf::LS + c * EPV) = st.u[i];
        }
    }
    if (threadIdx.x < Cf::C) sG[threadIdx.x] = st.g;
}

// X[i] += A[16i.., π keys] · B where B is the state (KT accumulator tiles,
// keys on rows) of this wave.  A is a [64][KD] row-major LDS tile.
template <class S, int KD, int LD>
__device__ __forceinline__ void rows_times_state(f32x4 (&X)[4], const S* sA, const f32x4 (&St)[KD / 16]) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
    if constexpr (sizeof(S) == 2) {
        using frag = typename Mma<S>::frag;
#pragma unroll
        for (int s = 0; s < KD / 32; s++) {
            frag b;
#pragma unroll
            for (int e = 0; e < 4; e++) { b[e] = (S)St[2 * s][e]; b[4 + e] = (S)St[2 * s + 1][e]; }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const S* p = sA + (16 * i + r) * LD + 32 * s + 4 * g;
                i16x4 lo = *(const i16x4*)p, hi = *(const i16x4*)(p + 16);
                i16x8 c = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                X[i] = Mma<S>::run(__builtin_bit_cast(frag, c), b, X[i]);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < KD / 16; t++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    X[i] = Mma<float>::run(sA[(16 * i + r) * LD + 16 * t + 4 * g + j], St[t][j], X[i]);
    }
}

// St[t] += (sA)ᵀ[16t.., π rows] · P where sA is a [64][KD] row-major LDS tile
// (so the A operand is its transpose) and P the 4 row tiles of a 64 x 16
// accumulator block (rows on the reduction index).
template <class S, int KD, int LD>
__device__ __forceinline__ void transT_times_rows(f32x4 (&St)[KD / 16], const S* sA, const f32x4 (&P)[4]) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
    if constexpr (sizeof(S) == 2) {
        using frag = typename Mma<S>::frag;
        frag b[2];
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int e = 0; e < 4; e++) { b[s][e] = (S)P[2 * s][e]; b[s][4 + e] = (S)P[2 * s + 1][e]; }
#pragma unroll
        for (int t = 0; t < KD / 16; t++)
#pragma unroll
            for (int s = 0; s < 2; s++) {
                i16x4 lo = ld_trans4<S>(sA, LD, 16 * t, 32 * s + 4 * g);
                i16x4 hi = ld_trans4<S>(sA, LD, 16 * t, 32 * s + 16 + 4 * g);
                i16x8 c = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                St[t] = Mma<S>::run(__builtin_bit_cast(frag, c), b[s], St[t]);
            }
    } else {
#pragma unroll
        for (int t = 0; t < KD / 16; t++)
#pragma unroll
            for (int tp = 0; tp < 4; tp++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    St[t] = Mma<float>::run(sA[(16 * tp + 4 * g + j) * LD + 16 * t + r], P[tp][j], St[t]);
    }
}

// Store a wave's K x 16 state slice: transposed [V][K] in type E (for the
// gradient kernel) and/or row-major [K][V] fp32.
template <class E, int KD, int VD>
__device__ __forceinline__ void store_state(const f32x4 (&St)[KD / 16], long unit, int col, E* hT, float* h32) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int t = 0; t < KD / 16; t++) {
        const int key = 16 * t + 4 * g;
        if (hT) {
            E* p = hT + (unit * VD + col) * KD + key;
            if constexpr (sizeof(E) == 2) {
                typedef E e4 __attribute__((ext_vector_type(4)));
                e4 v = {(E)St[t][0], (E)St[t][1], (E)St[t][2], (E)St[t][3]};
                *(e4*)p = v;
            } else {
                *(f32x4*)p = St[t];
            }
        }
        if (h32) {
#pragma unroll
            for (int e = 0; e < 4; e++) h32[(unit * KD + key + e) * VD + col] = St[t][e];
        }
    }
}

template <class E, class S, int KD, int VD, bool rev>
__device__ __forceinline__ void scan_body(const ScanArgs& a, int b, int HK, int HV, unsigned char* smem) {
    using Cf = ScanCfg<E, S, KD, VD>;
    constexpr int NVG = VD / 64, KT = KD / 16, C = 64;
    S* sK = (S*)smem;
    S* sW = sK + C * Cf::LK;
    S* sR = sW + C * Cf::LK;
    S* sX = sR + C * Cf::LK;
    float* sG = (float*)(sX + C * Cf::LS);

    const int vg = b % NVG, hv = (b / NVG) % HV, n = b / (NVG * HV);
    const int hk = hv / (HV / HK);
    const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
    const int col = vg * 64 + 16 * w + r;       // this lane's state column
    const int c0 = a.seq_chunk0[n], nc = a.seq_chunk0[n + 1] - c0;
    const E* k = (const E*)a.k;
    const E* dO = (const E*)a.dO;
    const S* W = (const S*)a.W;
    const S* U = (const S*)a.U;
    const S* R = (const S*)a.R;

    // state tiles: St[t][e] = state[16t + 4g + e][col]
    f32x4 St[KT];
    const float* init = rev ? a.dht : a.h0;
#pragma unroll
    for (int t = 0; t < KT; t++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            St[t][e] = init ? init[(((long)n * HV + hv) * KD + 16 * t + 4 * g + e) * VD + col] : 0.f;

    Stage<E, S, KD, VD, rev> s0, s1;
    auto chunk_of = [&](int i) { return rev ? c0 + nc - 1 - i : c0 + i; };
    auto issue = [&](Stage<E, S, KD, VD, rev>& st, int i) {
        const int ci = chunk_of(i);
        const ChunkInfo ch = a.info[ci];
        stage_issue<E, S, KD, VD, rev>(st, k, dO, W, U, R, a.gcum, ch, (long)ci * HV + hv, HK, HV, hk, hv, vg);
    };
    auto commit = [&](const Stage<E, S, KD, VD, rev>& st) { stage_commit<E, S, KD, VD, rev>(st, sK, sW, sR, sX, sG); };

    auto compute = [&](int i) {
        const int ci = chunk_of(i);
        const long unit = (long)ci * HV + hv;
        const float gl = sG[C - 1], gC = __expf(gl);
        f32x4 X[4];
#pragma unroll
        for (int m = 0; m < 4; m++) X[m] = zero4();
        if constexpr (!rev) {
            store_state<E, KD, VD>(St, unit, col, (E*)a.hT, a.h32);
            rows_times_state<S, KD, Cf::LK>(X, sW, St);                 // W h
            const ChunkInfo ch = a.info[ci];
#pragma unroll
            for (int m = 0; m < 4; m++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int row = 16 * m + 4 * g + e;
                    const float vn = (float)sX[row * Cf::LS + 16 * w + r] - X[m][e];   // V_new = U − W h
                    if (a.v_new && row < ch.len)
                        ((E*)a.v_new)[(((long)ch.t0 + row) * HV + hv) * VD + col] = (E)vn;
                    X[m][e] = vn * __expf(gl - sG[row]);
                }
#pragma unroll
            for (int t = 0; t < KT; t++) St[t] *= gC;
            transT_times_rows<S, KD, Cf::LK>(St, sK, X);               // + K̃ᵀ V_new
        } else {
            store_state<E, KD, VD>(St, unit, col, (E*)a.dhT, nullptr);
            rows_times_state<S, KD, Cf::LK>(X, sK, St);                 // K dh
#pragma unroll
            for (int m = 0; m < 4; m++)
#pragma unroll
                for (int e = 0; e < 4; e++) X[m][e] *= -__expf(gl - sG[16 * m + 4 * g + e]);   // −K̃ dh
#pragma unroll
            for (int t = 0; t < KT; t++) St[t] *= gC;
            // + Rᵀ dO
            if constexpr (sizeof(S) == 2) {
                using frag = typename Mma<S>::frag;
                frag bd[2];
#pragma unroll
                for (int s = 0; s < 2; s++) bd[s] = ld_trans<S>(sX, Cf::LS, 16 * w, 32 * s);
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int s = 0; s < 2; s++) St[t] = Mma<S>::run(ld_trans<S>(sR, Cf::LK, 16 * t, 32 * s), bd[s], St[t]);
            } else {
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int kb = 0; kb < 16; kb++)
                        St[t] = Mma<float>::run(sR[(4 * kb + g) * Cf::LK + 16 * t + r], sX[(4 * kb + g) * Cf::LS + 16 * w + r], St[t]);
            }
            transT_times_rows<S, KD, Cf::LK>(St, sW, X);               // − Wᵀ K̃ dh
        }
    };

    auto step = [&](int i, Stage<E, S, KD, VD, rev>& cur, Stage<E, S, KD, VD, rev>& nxt) {
        if (i + 2 < nc) issue(cur, i + 2);
        compute(i);
        __syncthreads();
        if (i + 1 < nc) commit(nxt);
        __syncthreads();
    };

    if (nc > 0) {
        issue(s0, 0);
        if (nc > 1) issue(s1, 1);
        commit(s0);
        __syncthreads();
        for (int i = 0; i < nc; i += 2) {
            step(i, s0, s1);
            if (i + 1 < nc) step(i + 1, s1, s0);
        }
    }

    // final state / dh0
    float* out = rev ? a.dh0 : a.ht;
    if (out) {
#pragma unroll
        for (int t = 0; t < KT; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) out[(((long)n * HV + hv) * KD + 16 * t + 4 * g + e) * VD + col] = St[t][e];
    }
}

template <class E, class S, int KD, int VD>
__global__ void __launch_bounds__(256) scan_kernel(ScanArgs a, int nfwd, int HK, int HV) {
    extern __shared__ __align__(16) unsigned char smem[];
    if ((int)blockIdx.x >= nfwd) scan_body<E, S, KD, VD, true>(a, (int)blockIdx.x - nfwd, HK, HV, smem);
    else scan_body<E, S, KD, VD, false>(a, (int)blockIdx.x, HK, HV, smem);
}

template <class E, class S, int KD, int VD>
static hipError_t scan_go(const Problem& p, const ScanArgs& a, hipStream_t s) {
    using Cf = ScanCfg<E, S, KD, VD>;
    const int nseq = p.cu ? p.N : p.B;
    const int per = nseq * p.HV * (VD / 64);
    const int nfwd = a.do_fwd ? per : 0, nrev = a.do_rev ? per : 0;
    if (nfwd + nrev == 0) return hipSuccess;
    auto kern = scan_kernel<E, S, KD, VD>;
    static_assert(Cf::smem <= 160 * 1024, "LDS budget");
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem) != hipSuccess)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3(nfwd + nrev), dim3(256), Cf::smem, s, a, nfwd, p.HK, p.HV);
    return hipGetLastError();
}

hipError_t launch_scans(const Problem& p, const ScanArgs& a, hipStream_t s) {
    if (p.K == 128 && p.V == 128) {
        if (p.dtype == 2) return scan_go<bf16, f16, 128, 128>(p, a, s);
        if (p.dtype == 1) return scan_go<f16, f16, 128, 128>(p, a, s);
        return scan_go<float, float, 128, 128>(p, a, s);
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 2) return scan_go<bf16, f16, 64, 64>(p, a, s);
        if (p.dtype == 1) return scan_go<f16, f16, 64, 64>(p, a, s);
        return scan_go<float, float, 64, 64>(p, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
