// gdr_scan.hip -- the two sequential chunk scans (K1b forward states, K2 dh).
//
// The per-chunk states go to the workspace transposed ([V][K] per chunk).
//
// Forward (state entering chunk c is h[c]; FlashQLA backward explainer §一
// step ②, "recompute h"):
//     V_new = U − W h[c],   h[c+1] = γ_C h[c] + K̃ᵀ V_new,   K̃ = diag(γ_C/γ) K
// Reverse (dh[c] is the gradient of the state leaving chunk c; same page §二
// "dS is walked back chunk by chunk" and §三's R-form of the recursion):
//     dh[c−1] = γ_C dh[c] + Rᵀ dO − Wᵀ (K̃ dh[c]),   dh0 = dh[−1]
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
// Operand tiles (W, U, R and K̃ = diag(γ_C/γ)K from the WY-factor kernel) are
// staged through LDS; the next-but-one chunk is prefetched into registers
// while the current one is computed.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <class E> constexpr int spad() { return sizeof(E) == 2 ? 8 : 4; }

template <class E, class S, int KD, int VD>
struct ScanCfg {
    static constexpr int C = 64;
    static constexpr int LK = KD + spad<S>();   // [64][KD] tiles
    static constexpr int LS = 64 + spad<S>();   // [64][64] column-group tiles
    static constexpr int EPV = 16 / (int)sizeof(S);
    static constexpr int NK = C * KD / (EPV * 256);   // 16-byte vectors per thread, [64][KD]
    static constexpr int NX = C * 64 / (EPV * 256);   // per thread, [64][64]
    static constexpr int KT = KD / 16;                // state tiles per wave
    // one LDS slot: K̃, W, R [64][LK] and the U / dO column slice [64][LS]
    static constexpr size_t slot_elems = (size_t)3 * C * LK + (size_t)C * LS;
    static constexpr size_t smem = 2 * slot_elems * sizeof(S);
};

// Register staging of one chunk's operand tiles (forward: K̃, W, U slice;
// reverse: K̃, W, R, dO slice) and the chunk's last cumulative gate.
template <class E, class S, int KD, int VD, bool REV>
struct Stage {
    using Cf = ScanCfg<E, S, KD, VD>;
    typename Vec16<S>::t k[Cf::NK];
    typename Vec16<S>::t w[Cf::NK];
    typename Vec16<S>::t r[REV ? Cf::NK : 1];
    typename Vec16<E>::t x[REV ? Cf::NX : 1];   // dO slice (reverse)
    typename Vec16<S>::t u[REV ? 1 : Cf::NX];   // U slice (forward)
    float gl;
    int cn;                                      // rows in the chunk (dO rows past it are zeroed at commit)
};

// X[i] += A[16i.., π keys] · B where B is the state (KT accumulator tiles,
// keys on rows) of this wave, times `sgn`.  A is a [64][KD] row-major LDS tile.
template <class S, int KD, int LD>
__device__ __forceinline__ void rows_times_state(f32x4 (&X)[4], const S* sA, const f32x4 (&St)[KD / 16], float sgn) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
    if constexpr (sizeof(S) == 2) {
        using frag = typename Mma<S>::frag;
#pragma unroll
        for (int s = 0; s < KD / 32; s++) {
            frag b;
#pragma unroll
            for (int e = 0; e < 4; e++) { b[e] = (S)(sgn * St[2 * s][e]); b[4 + e] = (S)(sgn * St[2 * s + 1][e]); }
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
                    X[i] = Mma<float>::run(sA[(16 * i + r) * LD + 16 * t + 4 * g + j], sgn * St[t][j], X[i]);
    }
}

// St[t] += (sA)ᵀ[16t.., π rows] · P · sgn where sA is a [64][KD] row-major LDS
// tile (so the A operand is its transpose) and P the 4 row tiles of a 64 x 16
// accumulator block (rows on the reduction index).
template <class S, int KD, int LD>
__device__ __forceinline__ void transT_times_rows(f32x4 (&St)[KD / 16], const S* sA, const f32x4 (&P)[4], float sgn) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
    if constexpr (sizeof(S) == 2) {
        using frag = typename Mma<S>::frag;
        frag b[2];
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int e = 0; e < 4; e++) { b[s][e] = (S)(sgn * P[2 * s][e]); b[s][4 + e] = (S)(sgn * P[2 * s + 1][e]); }
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
                    St[t] = Mma<float>::run(sA[(16 * tp + 4 * g + j) * LD + 16 * t + r], sgn * P[tp][j], St[t]);
    }
}

// Store a wave's K x 16 state slice: transposed [V][K] in type E (for the
// gradient kernel) and/or row-major [K][V] fp32.  All values are packed
// before the first store so that each store owns its data registers (a store
// whose data registers are reused right away stalls until the memory
// pipeline has read them).
template <class E, int KD, int VD, bool EST>
__device__ __forceinline__ void store_state(const f32x4 (&St)[KD / 16], long unit, int col, E* hT, float* h32) {
    const int g = lane_id() >> 4;
    if constexpr (EST) {
        E* p = hT + (unit * VD + col) * KD + 4 * g;
        if constexpr (sizeof(E) == 2) {
            typedef E e4 __attribute__((ext_vector_type(4)));
            e4 v[KD / 16];
#pragma unroll
            for (int t = 0; t < KD / 16; t++)
#pragma unroll
                for (int e = 0; e < 4; e++) v[t][e] = (E)St[t][e];
#pragma unroll
            for (int t = 0; t < KD / 16; t++) *(e4*)(p + 16 * t) = v[t];
        } else {
#pragma unroll
            for (int t = 0; t < KD / 16; t++) *(f32x4*)(p + 16 * t) = St[t];
        }
    }
    if (h32) {
#pragma unroll
        for (int t = 0; t < KD / 16; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) h32[(unit * KD + 16 * t + 4 * g + e) * VD + col] = St[t][e];
    }
}

template <class E, class S, int KD, int VD, bool rev, bool EST>
__device__ __forceinline__ void scan_body(const ScanArgs& a, int b, int HK, int HV, unsigned char* smem) {
    using Cf = ScanCfg<E, S, KD, VD>;
    using St_t = Stage<E, S, KD, VD, rev>;
    constexpr int NVG = VD / 64, KT = KD / 16, C = 64, EPV = Cf::EPV, LK = Cf::LK, LS = Cf::LS;
    constexpr int VPR = KD / EPV, XPR = 64 / EPV;
    S* slot[2] = {(S*)smem, (S*)smem + Cf::slot_elems};

    const int vg = b % NVG, hv = (b / NVG) % HV, n = b / (NVG * HV);
    const int hk = hv / (HV / HK);
    const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
    const int col = vg * 64 + 16 * w + r;       // this lane's state column
    const int c0 = a.seq_chunk0[n], nc = a.seq_chunk0[n + 1] - c0;
    const long bos = a.cu ? a.cu[n] : (long)n * a.T;            // first token of the sequence
    const int slen = a.cu ? a.cu[n + 1] - a.cu[n] : a.T;        // its length
    const E* dO = (const E*)a.dO;
    const S* W = (const S*)a.W;
    const S* U = (const S*)a.U;
    const S* R = (const S*)a.R;
    const S* KTl = (const S*)a.KT;
    (void)hk;

    // loop-invariant per-thread element offsets of the staged vectors
    int offK[Cf::NK], rowX[Cf::NX], offX[Cf::NX];
#pragma unroll
    for (int i = 0; i < Cf::NK; i++) {
        const int idx = threadIdx.x + 256 * i;
        offK[i] = (idx / VPR) * LK + (idx % VPR) * EPV;   // LDS offset; global = row*KD + c*EPV
    }
#pragma unroll
    for (int i = 0; i < Cf::NX; i++) {
        const int idx = threadIdx.x + 256 * i;
        rowX[i] = idx / XPR;
        offX[i] = (idx % XPR) * EPV;
    }

    // state tiles: St[t][e] = state[16t + 4g + e][col]
    f32x4 St[KT];
    const float* init = rev ? a.dht : a.h0;
#pragma unroll
    for (int t = 0; t < KT; t++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            St[t][e] = init ? init[(((long)n * HV + hv) * KD + 16 * t + 4 * g + e) * VD + col] : 0.f;

    auto chunk_of = [&](int i) { return rev ? c0 + nc - 1 - i : c0 + i; };
    auto local_of = [&](int i) { return rev ? nc - 1 - i : i; };   // chunk index within the sequence

    auto issue = [&](St_t& st, int i) {
        const int ci = chunk_of(i), lc = local_of(i);
        const long unit = (long)ci * HV + hv;
        const long t0 = bos + (long)lc * C;
        const int Cn = min(C, slen - lc * C);
        const S* Kb = KTl + unit * C * KD;
        const S* Wb = W + unit * C * KD;
        const S* Rb = R + unit * C * KD;
#pragma unroll
        for (int j = 0; j < Cf::NK; j++) {
            const int idx = threadIdx.x + 256 * j, go = (idx / VPR) * KD + (idx % VPR) * EPV;
            st.k[j] = *(const typename Vec16<S>::t*)(Kb + go);
            st.w[j] = *(const typename Vec16<S>::t*)(Wb + go);
            if constexpr (rev) st.r[j] = *(const typename Vec16<S>::t*)(Rb + go);
        }
#pragma unroll
        for (int j = 0; j < Cf::NX; j++) {
            if constexpr (rev) {
                // rows past the chunk end read a valid row; they are zeroed at
                // commit, where the data is needed anyway (a select here would
                // make the wave wait for the load it just issued)
                const int rowc = min(rowX[j], Cn - 1);
                st.x[j] = *(const typename Vec16<E>::t*)(dO + ((t0 + rowc) * HV + hv) * VD + vg * 64 + offX[j]);
            } else {
                st.u[j] = *(const typename Vec16<S>::t*)(U + (unit * C + rowX[j]) * VD + vg * 64 + offX[j]);
            }
        }
        st.gl = a.gcum[(t0 + Cn - 1) * HV + hv];
        st.cn = Cn;
    };
    auto commit = [&](const St_t& st, S* sl) {
        S* sK = sl;
        S* sW = sl + C * LK;
        S* sR = sl + 2 * C * LK;
        S* sX = sl + 3 * C * LK;
#pragma unroll
        for (int j = 0; j < Cf::NK; j++) {
            *(typename Vec16<S>::t*)(sK + offK[j]) = st.k[j];
            *(typename Vec16<S>::t*)(sW + offK[j]) = st.w[j];
            if constexpr (rev) *(typename Vec16<S>::t*)(sR + offK[j]) = st.r[j];
        }
#pragma unroll
        for (int j = 0; j < Cf::NX; j++) {
            typename Vec16<S>::t xv;
            if constexpr (rev) {
                const bool valid = rowX[j] < st.cn;
#pragma unroll
                for (int e = 0; e < EPV; e++) xv[e] = valid ? (S)(float)st.x[j][e] : (S)0.f;
            } else {
                xv = st.u[j];
            }
            *(typename Vec16<S>::t*)(sX + rowX[j] * LS + offX[j]) = xv;
        }
    };

    auto compute = [&](int i, const S* sl, float gl) {
        const S* sK = sl;
        const S* sW = sl + C * LK;
        const S* sR = sl + 2 * C * LK;
        const S* sX = sl + 3 * C * LK;
        const int ci = chunk_of(i);
        const long unit = (long)ci * HV + hv;
        const float gC = __expf(gl);
        f32x4 X[4];
        if constexpr (sizeof(S) == 2) {
            // All state-independent fragments of this chunk are read from LDS
            // first; the MFMA groups then only wait on their own operands.
            using frag = typename Mma<S>::frag;
            frag Ar[4][KD / 32];   // rows of W (fwd) or K̃ (rev), keys in π order
            frag At[KT][2];        // K̃ᵀ (fwd) or Wᵀ (rev), rows in π order
            frag Rt[rev ? KT : 1][2];
            frag Db[2];
            const S* sRow = rev ? sK : sW;
            const S* sTr = rev ? sW : sK;
#pragma unroll
            for (int sidx = 0; sidx < KD / 32; sidx++)
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const S* p = sRow + (16 * m + r) * LK + 32 * sidx + 4 * g;
                    i16x4 lo = *(const i16x4*)p, hi = *(const i16x4*)(p + 16);
                    i16x8 c = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    Ar[m][sidx] = __builtin_bit_cast(frag, c);
                }
            if constexpr (!rev) {
#pragma unroll
                for (int m = 0; m < 4; m++) {   // U in accumulator layout: one transposing read per tile
                    i16x4 u = ld_trans4<S>(sX, LS, 16 * w, 16 * m + 4 * g);
                    S uu[4];
                    __builtin_memcpy(uu, &u, 8);
#pragma unroll
                    for (int e = 0; e < 4; e++) X[m][e] = (float)uu[e];
                }
            } else {
#pragma unroll
                for (int sidx = 0; sidx < 2; sidx++) Db[sidx] = ld_trans<S>(sX, LS, 16 * w, 32 * sidx);
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int sidx = 0; sidx < 2; sidx++) Rt[t][sidx] = ld_trans<S>(sR, LK, 16 * t, 32 * sidx);
            }
#pragma unroll
            for (int t = 0; t < KT; t++)
#pragma unroll
                for (int sidx = 0; sidx < 2; sidx++) {
                    i16x4 lo = ld_trans4<S>(sTr, LK, 16 * t, 32 * sidx + 4 * g);
                    i16x4 hi = ld_trans4<S>(sTr, LK, 16 * t, 32 * sidx + 16 + 4 * g);
                    i16x8 c = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    At[t][sidx] = __builtin_bit_cast(frag, c);
                }
            // state store (before the update) and B fragments of the state
            store_state<E, KD, VD, EST>(St, unit, col, rev ? (E*)a.dhT : (E*)a.hT, rev ? nullptr : a.h32);
            const float sg = rev ? 1.f : -1.f;   // fwd: X = U − W h ; rev: X = K̃ dh
            frag Bs[KD / 32];
#pragma unroll
            for (int sidx = 0; sidx < KD / 32; sidx++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    Bs[sidx][e] = (S)(sg * St[2 * sidx][e]);
                    Bs[sidx][4 + e] = (S)(sg * St[2 * sidx + 1][e]);
                }
            if constexpr (rev) {
#pragma unroll
                for (int m = 0; m < 4; m++) X[m] = zero4();
            }
#pragma unroll
            for (int sidx = 0; sidx < KD / 32; sidx++)
#pragma unroll
                for (int m = 0; m < 4; m++) X[m] = Mma<S>::run(Ar[m][sidx], Bs[sidx], X[m]);
#pragma unroll
            for (int t = 0; t < KT; t++) St[t] *= gC;
            if constexpr (rev) {
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int sidx = 0; sidx < 2; sidx++) St[t] = Mma<S>::run(Rt[t][sidx], Db[sidx], St[t]);   // + Rᵀ dO
            } else if (a.v_new) {
                const int lc = local_of(i), clen = min(C, slen - lc * C);
                const long ct0 = bos + (long)lc * C;
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int row = 16 * m + 4 * g + e;
                        if (row < clen) ((E*)a.v_new)[((ct0 + row) * HV + hv) * VD + col] = (E)X[m][e];
                    }
            }
            const float sp = rev ? -1.f : 1.f;   // fwd: + K̃ᵀ V_new ; rev: − Wᵀ (K̃ dh)
            frag Bp[2];
#pragma unroll
            for (int sidx = 0; sidx < 2; sidx++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    Bp[sidx][e] = (S)(sp * X[2 * sidx][e]);
                    Bp[sidx][4 + e] = (S)(sp * X[2 * sidx + 1][e]);
                }
#pragma unroll
            for (int t = 0; t < KT; t++)
#pragma unroll
                for (int sidx = 0; sidx < 2; sidx++) St[t] = Mma<S>::run(At[t][sidx], Bp[sidx], St[t]);
        } else {
            // fp32 operands (16x16x4 MFMA): small sizes only, plain order
            if constexpr (!rev) {
                store_state<E, KD, VD, EST>(St, unit, col, (E*)a.hT, a.h32);
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int e = 0; e < 4; e++) X[m][e] = (float)sX[(16 * m + 4 * g + e) * LS + 16 * w + r];
                rows_times_state<S, KD, LK>(X, sW, St, -1.f);
                if (a.v_new) {
                    const int lc = local_of(i), clen = min(C, slen - lc * C);
                    const long ct0 = bos + (long)lc * C;
#pragma unroll
                    for (int m = 0; m < 4; m++)
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int row = 16 * m + 4 * g + e;
                            if (row < clen) ((E*)a.v_new)[((ct0 + row) * HV + hv) * VD + col] = (E)X[m][e];
                        }
                }
#pragma unroll
                for (int t = 0; t < KT; t++) St[t] *= gC;
                transT_times_rows<S, KD, LK>(St, sK, X, 1.f);
            } else {
                store_state<E, KD, VD, EST>(St, unit, col, (E*)a.dhT, nullptr);
#pragma unroll
                for (int m = 0; m < 4; m++) X[m] = zero4();
                rows_times_state<S, KD, LK>(X, sK, St, 1.f);
#pragma unroll
                for (int t = 0; t < KT; t++) St[t] *= gC;
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int kb = 0; kb < 16; kb++)
                        St[t] = Mma<float>::run(sR[(4 * kb + g) * LK + 16 * t + r], sX[(4 * kb + g) * LS + 16 * w + r], St[t]);
                transT_times_rows<S, KD, LK>(St, sW, X, -1.f);
            }
        }
    };

    // Two register stages and two LDS slots, one barrier per chunk: the loads
    // for chunk i+2 are issued before computing chunk i and written to LDS
    // after computing chunk i+1.  Indices are clamped at the sequence end so
    // the loop body is straight-line code.
    St_t s0, s1;
    float glv0 = 0.f, glv1 = 0.f;
    auto step = [&](int i, St_t& cur, St_t& nxt, float& gl_cur, float& gl_nxt, S* sl_cur, S* sl_nxt) {
        issue(cur, min(i + 2, nc - 1));
        compute(i, sl_cur, gl_cur);
        commit(nxt, sl_nxt);
        gl_nxt = nxt.gl;
        lds_barrier();
    };
    if (nc > 0) {
        issue(s0, 0);
        issue(s1, min(1, nc - 1));
        commit(s0, slot[0]);
        glv0 = s0.gl;
        lds_barrier();
        // The first chunk is peeled so that the loop is entered with the same
        // outstanding loads/stores as on its back edge (the compiler's wait
        // counts at the commits then allow two chunks of loads in flight).
        step(0, s0, s1, glv0, glv1, slot[0], slot[1]);
        for (int i = 1; i < nc; i += 2) {
            step(i, s1, s0, glv1, glv0, slot[1], slot[0]);
            if (i + 1 < nc) step(i + 1, s0, s1, glv0, glv1, slot[0], slot[1]);
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

// EST: the transposed states (hT for the forward scan, dhT for the reverse
// one) are stored in type E.  It is a template parameter so the store is not
// behind a runtime branch: the compiler's wait counts are then exact.
template <class E, class S, int KD, int VD, bool EST>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
scan_kernel(ScanArgs a, int nfwd, int HK, int HV) {
    extern __shared__ __align__(16) unsigned char smem[];
    if ((int)blockIdx.x >= nfwd) scan_body<E, S, KD, VD, true, EST>(a, (int)blockIdx.x - nfwd, HK, HV, smem);
    else scan_body<E, S, KD, VD, false, EST>(a, (int)blockIdx.x, HK, HV, smem);
}

template <class E, class S, int KD, int VD>
static hipError_t scan_go(const Problem& p, const ScanArgs& a, hipStream_t s) {
    using Cf = ScanCfg<E, S, KD, VD>;
    const int nseq = p.cu ? p.N : p.B;
    const int per = nseq * p.HV * (VD / 64);
    const int nfwd = a.do_fwd ? per : 0, nrev = a.do_rev ? per : 0;
    if (nfwd + nrev == 0) return hipSuccess;
    // either every launched scan stores its E-typed states or none does
    const bool est_f = !a.do_fwd || a.hT, est_r = !a.do_rev || a.dhT;
    const bool none_f = !a.do_fwd || !a.hT, none_r = !a.do_rev || !a.dhT;
    if (!(est_f && est_r) && !(none_f && none_r)) return hipErrorInvalidValue;
    auto kern = (est_f && est_r) ? scan_kernel<E, S, KD, VD, true> : scan_kernel<E, S, KD, VD, false>;
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
        return hipErrorInvalidValue;   // fp32 is built at K = V = 64 only
    }
    if (p.K == 64 && p.V == 64) {
        if (p.dtype == 2) return scan_go<bf16, f16, 64, 64>(p, a, s);
        if (p.dtype == 1) return scan_go<f16, f16, 64, 64>(p, a, s);
        return scan_go<float, float, 64, 64>(p, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
