// gdr_scan.hip -- the two sequential chunk scans (K1b forward states, K2 dh).
//
// The per-chunk states go to the workspace in the accumulators' fragment order
// (16-bit types) or transposed, [V][K] per chunk (fp32).
//
// Forward (state entering chunk c is h[c]; FlashQLA backward explainer §一
// step ②, where h is recomputed):
//     V_new = U − W h[c],   h[c+1] = γ_C h[c] + K̃ᵀ V_new,   K̃ = diag(γ_C/γ) K
// Reverse (dh[c] is the gradient of the state leaving chunk c; same page §二,
// where dS goes back one chunk at a time, and §三's R-form of the recursion):
//     dh[c−1] = γ_C dh[c] + Rᵀ dO − Wᵀ (K̃ dh[c]),   dh0 = dh[−1]
//
// Parallel decomposition: every column of the K x V state evolves on its own
// (all updates multiply the state from the left), so a wave owns a K x V/4
// column slice (V/64 blocks of 16 columns) for the whole sequence, in fp32
// accumulator registers.  A workgroup (4 waves) covers all V columns of one
// job, a run of chunks (a whole sequence or one of its segments) of one value
// head and direction, so each operand tile is read from HBM once per
// direction and pass, and every fragment read from LDS feeds V/64 MFMAs.
// The state doubles as the MFMA B operand without any data
// movement: the accumulator holds rows {4g..4g+3} of every 16-row tile, so two
// tiles form one 32-deep k block in the permuted order
//     π(8g+i) = 32s + (i < 4 ? 4g + i : 16 + 4g + i − 4),
// and the A operand (W, K, or the transposed Kᵀ/Wᵀ) is read in the same order.
// Operand tiles (W, U, R and K̃ = diag(γ_C/γ)K from the WY-factor kernel) are
// staged through LDS; the next-but-one chunk is prefetched into registers
// while the current one is computed.  Every tile is read once per pass and
// every per-chunk state written once, far ahead of its reader, so the loads
// and the state stores are non-temporal: they stream past the caches instead
// of evicting lines that are still to be used.
#include "gdr_device.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <class E> constexpr int spad() { return sizeof(E) == 2 ? 8 : 4; }

template <class E, class S, int KD, int VD>
struct ScanCfg {
    static constexpr int C = 64;
    static constexpr int LK = KD + spad<S>();   // [64][KD] tiles
    static constexpr int LS = VD + spad<S>();   // [64][VD] tiles (U or dO)
    static constexpr int EPV = 16 / (int)sizeof(S);
    static constexpr int NK = C * KD / (EPV * 256);   // 16-byte vectors per thread, [64][KD]
    static constexpr int NX = C * VD / (EPV * 256);   // per thread, [64][VD]
    static constexpr int KT = KD / 16;                // state row tiles
    static constexpr int NB = VD / 64;                // 16-column blocks per wave
    static constexpr int CW = VD / 4;                 // state columns per wave
    // one LDS slot: K̃, W, R [64][LK] and U / dO [64][LS]
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
    typename Vec16<E>::t x[REV ? Cf::NX : 1];   // dO tile (reverse)
    typename Vec16<S>::t u[REV ? 1 : Cf::NX];   // U tile (forward)
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

// Store a wave's K x 16 state block (columns col - r .. col - r + 15): in type
// E in the workspace state layout (fragment order, 16 B per lane and 1 KB per
// wave instruction; fp32: transposed [V][K]) and/or row-major [K][V] fp32.
// All values are packed before the first store so that each store owns its
// data registers.
template <class E, int KD, int VD, bool EST>
__device__ __forceinline__ void store_state(const f32x4 (&St)[KD / 16], long unit, int col, E* hT, float* h32) {
    const int g = lane_id() >> 4;
    if constexpr (EST) {
        if constexpr (sizeof(E) == 2) {
            typedef E e8 __attribute__((ext_vector_type(8)));
            E* p = hT + unit * VD * KD + ((long)(col / 16) * (KD / 32) * 64 + lane_id()) * 8;
            e8 v[KD / 32];
#pragma unroll
            for (int s = 0; s < KD / 32; s++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    v[s][e] = (E)St[2 * s][e];
                    v[s][4 + e] = (E)St[2 * s + 1][e];
                }
#pragma unroll
            for (int s = 0; s < KD / 32; s++) __builtin_nontemporal_store(v[s], (e8*)(p + 512 * s));
        } else {
            E* p = hT + (unit * VD + col) * KD + 4 * g;
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

// Initial / final state forms of one scan job.
enum StateForm { ST_NONE = 0, ST_ZERO = 0, ST_NAT = 2, ST_FRAG = 3 };

// One scan job: a run of chunks of one sequence and value head.
struct ScanJob {
    int n, hv;          // sequence, value head
    int c0, nc, lc0;    // first chunk (global index), chunk count, first chunk's index in the sequence
    int init_form;      // ST_ZERO, ST_NAT ([K][V] fp32), ST_FRAG (fp32 fragment order)
    const float* init;  // K x V block of the initial state
    int out_form;       // ST_NONE, ST_NAT or ST_FRAG
    float* out;         // K x V block of the final state
    float* out2;        // merged forward job: K x K block of the transfer matrix, in the
                        // fragment order with the values in the 16-bit operand type S
                        // (four per lane and tile; its transpose in the same order after
                        // it, in the block's second half): it only enters MFMAs as an operand
    float sc = 1.f;     // reverse jobs: the state and dO run scaled by sc (a power of two);
    float isc = 1.f;    // the per-chunk states dh[c] are stored scaled (the gradient kernel
                        // folds 1/sc into its factors), dh0 is stored times isc = 1/sc
};

// Scale of the reverse scans of (sequence n, value head hv): 1 without scaling.
__device__ __forceinline__ void job_scale(const ScanArgs& a, ScanJob& jb, int HV) {
    const float s = a.dsc ? a.dsc[(long)jb.n * HV + jb.hv] : 1.f;
    jb.sc = s;
    jb.isc = 1.f / s;   // exact: s is a power of two
}

// rev: reverse (dh) recursion, else forward.  EST: per-chunk states stored in
// type E.  HP (forward,
// local scans only): every wave also carries the same columns of the transfer
// matrix P = Π (γ_C I − K̃ᵀ W) of the segment, as extra state blocks that
// start from the identity and take U = 0 -- the same recursion as h with the
// same W and K̃ fragments, so one workgroup yields both local results.
template <class E, class S, int KD, int VD, bool rev, bool EST, bool HP = false>
__device__ __forceinline__ void scan_body(const ScanArgs& a, const ScanJob& jb, int HV, unsigned char* smem) {
    using Cf = ScanCfg<E, S, KD, VD>;
    using St_t = Stage<E, S, KD, VD, rev>;
    constexpr int KT = KD / 16, C = 64, EPV = Cf::EPV, LK = Cf::LK, LS = Cf::LS, NB = Cf::NB, CW = Cf::CW;
    static_assert(!HP || (!rev && !EST && sizeof(S) == 2), "merged blocks: forward local scans, 16-bit");
    constexpr int NBT = HP ? 2 * NB : NB;   // state blocks per wave (blocks NB.. are the transfer matrix)
    constexpr int VPR = KD / EPV, XPR = VD / EPV;
    S* slot[2] = {(S*)smem, (S*)smem + Cf::slot_elems};

    const int hv = jb.hv, n = jb.n;
    const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
    const int col0 = CW * w + r;                // this lane's state column in block 0 (block nb: + 16 nb)
    const float sc = rev ? jb.sc : 1.f, isc = rev ? jb.isc : 1.f;   // scaled reverse state (1 forward)
    const int c0 = jb.c0, nc = jb.nc;
    const long bos = a.cu ? a.cu[n] : (long)n * a.T;            // first token of the sequence
    const int slen = a.cu ? a.cu[n + 1] - a.cu[n] : a.T;        // its length
    const E* dO = (const E*)a.dO;
    const S* W = (const S*)a.W;
    const S* U = (const S*)a.U;
    const S* R = (const S*)a.R;
    const S* KTl = (const S*)a.KT;

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

    // state tiles: St[nb][t][e] = state[16t + 4g + e][col0 + 16 (nb % NB)]
    f32x4 St[NBT][KT];
#pragma unroll
    for (int nb = 0; nb < NBT; nb++)
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int cb = CW * w / 16 + nb % NB;
            if (HP && nb >= NB) {   // transfer matrix: from the identity
#pragma unroll
                for (int e = 0; e < 4; e++) St[nb][t][e] = 16 * t + 4 * g + e == col0 + 16 * (nb % NB) ? 1.f : 0.f;
            } else if (jb.init_form == ST_FRAG) {
                St[nb][t] = *(const f32x4*)(jb.init + ((cb * KT + t) * 64 + l) * 4);
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int row = 16 * t + 4 * g + e, col = col0 + 16 * nb;
                    St[nb][t][e] = jb.init_form == ST_NAT ? sc * jb.init[row * VD + col]
                                 : 0.f;
                }
            }
        }

    auto chunk_of = [&](int i) { return rev ? c0 + nc - 1 - i : c0 + i; };
    auto local_of = [&](int i) { return jb.lc0 + (rev ? nc - 1 - i : i); };   // chunk index within the sequence

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
            st.k[j] = __builtin_nontemporal_load((const typename Vec16<S>::t*)(Kb + go));
            st.w[j] = __builtin_nontemporal_load((const typename Vec16<S>::t*)(Wb + go));
            if constexpr (rev) st.r[j] = __builtin_nontemporal_load((const typename Vec16<S>::t*)(Rb + go));
        }
#pragma unroll
        for (int j = 0; j < Cf::NX; j++) {
            if constexpr (rev) {
                // rows past the chunk end read a valid row; they are zeroed at
                // commit, where the data is needed anyway (a select here would
                // make the wave wait for the load it just issued)
                const int rowc = min(rowX[j], Cn - 1);
                st.x[j] = __builtin_nontemporal_load(
                    (const typename Vec16<E>::t*)(dO + ((t0 + rowc) * HV + hv) * VD + offX[j]));
            } else {
                st.u[j] = __builtin_nontemporal_load(
                    (const typename Vec16<S>::t*)(U + (unit * C + rowX[j]) * VD + offX[j]));
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
                for (int e = 0; e < EPV; e++) xv[e] = valid ? (S)(sc * (float)st.x[j][e]) : (S)0.f;
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
        f32x4 X[NBT][4];
        if constexpr (sizeof(S) == 2) {
            // All state-independent fragments of this chunk are read from LDS
            // first; the MFMA groups then only wait on their own operands.
            using frag = typename Mma<S>::frag;
            frag Ar[4][KD / 32];   // rows of W (fwd) or K̃ (rev), keys in π order
            frag At[KT][2];        // K̃ᵀ (fwd) or Wᵀ (rev), rows in π order
            frag Rt[rev ? KT : 1][2];
            frag Db[NB][2];
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
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int m = 0; m < 4; m++) {   // U in accumulator layout: one transposing read per tile
                        i16x4 u = ld_trans4<S>(sX, LS, CW * w + 16 * nb, 16 * m + 4 * g);
                        S uu[4];
                        __builtin_memcpy(uu, &u, 8);
#pragma unroll
                        for (int e = 0; e < 4; e++) X[nb][m][e] = HP ? -(float)uu[e] : (float)uu[e];
                    }
#pragma unroll
                for (int nb = NB; nb < NBT; nb++)
#pragma unroll
                    for (int m = 0; m < 4; m++) X[nb][m] = zero4();
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int sidx = 0; sidx < 2; sidx++) Db[nb][sidx] = ld_trans<S>(sX, LS, CW * w + 16 * nb, 32 * sidx);
            }
            // (merged blocks: read after the first product group instead, which
            // keeps the wider state within the register file)
            if constexpr (!HP) {
#pragma unroll
            for (int t = 0; t < KT; t++)
#pragma unroll
                for (int sidx = 0; sidx < 2; sidx++) {
                    i16x4 lo = ld_trans4<S>(sTr, LK, 16 * t, 32 * sidx + 4 * g);
                    i16x4 hi = ld_trans4<S>(sTr, LK, 16 * t, 32 * sidx + 16 + 4 * g);
                    i16x8 c = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    At[t][sidx] = __builtin_bit_cast(frag, c);
                }
            }
            // state store (before the update) and B fragments of the state
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
                store_state<E, KD, VD, EST>(St[nb], unit, col0 + 16 * nb, rev ? (E*)a.dhT : (E*)a.hT,
                                            rev ? nullptr : a.h32);
            // fwd: X = U − W h ; rev: X = K̃ dh (sign applied below);
            // merged blocks: X = W S − U, then S ← γ S − K̃ᵀ X (the same update)
            const float sg = (rev || HP) ? 1.f : -1.f;
            frag Bs[NBT][KD / 32];
#pragma unroll
            for (int nb = 0; nb < NBT; nb++)
#pragma unroll
                for (int sidx = 0; sidx < KD / 32; sidx++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        Bs[nb][sidx][e] = (S)(sg * St[nb][2 * sidx][e]);
                        Bs[nb][sidx][4 + e] = (S)(sg * St[nb][2 * sidx + 1][e]);
                    }
            if constexpr (rev) {
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int m = 0; m < 4; m++) X[nb][m] = zero4();
            }
#pragma unroll
            for (int sidx = 0; sidx < KD / 32; sidx++)
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int nb = 0; nb < NBT; nb++) X[nb][m] = Mma<S>::run(Ar[m][sidx], Bs[nb][sidx], X[nb][m]);
            if constexpr (HP) {
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int sidx = 0; sidx < 2; sidx++) {
                        i16x4 lo = ld_trans4<S>(sTr, LK, 16 * t, 32 * sidx + 4 * g);
                        i16x4 hi = ld_trans4<S>(sTr, LK, 16 * t, 32 * sidx + 16 + 4 * g);
                        i16x8 c = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        At[t][sidx] = __builtin_bit_cast(frag, c);
                    }
            }
#pragma unroll
            for (int nb = 0; nb < NBT; nb++)
#pragma unroll
                for (int t = 0; t < KT; t++) St[nb][t] *= gC;
            if constexpr (rev) {
                // Rᵀ fragments are read here, after the K̃ dh products are
                // issued, to keep them out of the live range of the others
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int sidx = 0; sidx < 2; sidx++) Rt[t][sidx] = ld_trans<S>(sR, LK, 16 * t, 32 * sidx);
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int sidx = 0; sidx < 2; sidx++)
#pragma unroll
                        for (int nb = 0; nb < NB; nb++)
                            St[nb][t] = Mma<S>::run(Rt[t][sidx], Db[nb][sidx], St[nb][t]);   // + Rᵀ dO
            } else if (a.v_new) {
                const int lc = local_of(i), clen = min(C, slen - lc * C);
                const long ct0 = bos + (long)lc * C;
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int m = 0; m < 4; m++)
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int row = 16 * m + 4 * g + e;
                            if (row < clen)
                                ((E*)a.v_new)[((ct0 + row) * HV + hv) * VD + col0 + 16 * nb] = (E)X[nb][m][e];
                        }
            }
            // fwd: + K̃ᵀ V_new ; rev: − Wᵀ (K̃ dh) ; merged blocks: − K̃ᵀ X
            const float sp = (rev || HP) ? -1.f : 1.f;
            frag Bp[NBT][2];
#pragma unroll
            for (int nb = 0; nb < NBT; nb++)
#pragma unroll
                for (int sidx = 0; sidx < 2; sidx++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        Bp[nb][sidx][e] = (S)(sp * X[nb][2 * sidx][e]);
                        Bp[nb][sidx][4 + e] = (S)(sp * X[nb][2 * sidx + 1][e]);
                    }
#pragma unroll
            for (int t = 0; t < KT; t++)
#pragma unroll
                for (int sidx = 0; sidx < 2; sidx++)
#pragma unroll
                    for (int nb = 0; nb < NBT; nb++) St[nb][t] = Mma<S>::run(At[t][sidx], Bp[nb][sidx], St[nb][t]);
        } else {
            // fp32 operands (16x16x4 MFMA): K = V = 64 only (one 16-column block per wave), plain order
            static_assert(NB == 1, "fp32 scan is built for V = 64");
            if constexpr (!rev) {
                store_state<E, KD, VD, EST>(St[0], unit, col0, (E*)a.hT, a.h32);
#pragma unroll
                for (int m = 0; m < 4; m++)
#pragma unroll
                    for (int e = 0; e < 4; e++) X[0][m][e] = (float)sX[(16 * m + 4 * g + e) * LS + 16 * w + r];
                rows_times_state<S, KD, LK>(X[0], sW, St[0], -1.f);
                if (a.v_new) {
                    const int lc = local_of(i), clen = min(C, slen - lc * C);
                    const long ct0 = bos + (long)lc * C;
#pragma unroll
                    for (int m = 0; m < 4; m++)
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int row = 16 * m + 4 * g + e;
                            if (row < clen) ((E*)a.v_new)[((ct0 + row) * HV + hv) * VD + col0] = (E)X[0][m][e];
                        }
                }
#pragma unroll
                for (int t = 0; t < KT; t++) St[0][t] *= gC;
                transT_times_rows<S, KD, LK>(St[0], sK, X[0], 1.f);
            } else {
                store_state<E, KD, VD, EST>(St[0], unit, col0, (E*)a.dhT, nullptr);
#pragma unroll
                for (int m = 0; m < 4; m++) X[0][m] = zero4();
                rows_times_state<S, KD, LK>(X[0], sK, St[0], 1.f);
#pragma unroll
                for (int t = 0; t < KT; t++) St[0][t] *= gC;
#pragma unroll
                for (int t = 0; t < KT; t++)
#pragma unroll
                    for (int kb = 0; kb < 16; kb++)
                        St[0][t] = Mma<float>::run(sR[(4 * kb + g) * LK + 16 * t + r], sX[(4 * kb + g) * LS + 16 * w + r],
                                                   St[0][t]);
                transT_times_rows<S, KD, LK>(St[0], sW, X[0], -1.f);
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

    // final state
    if constexpr (HP) {   // the transfer-matrix blocks
        typedef S s4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int nb = NB; nb < NBT; nb++)
#pragma unroll
            for (int t = 0; t < KT; t++) {
                s4 x;
#pragma unroll
                for (int e = 0; e < 4; e++) x[e] = (S)St[nb][t][e];
                const int cb = CW * w / 16 + nb - NB;
                *(s4*)((S*)jb.out2 + ((cb * KT + t) * 64 + l) * 4) = x;
                // P_sᵀ in the same order in the block's second half: element
                // P[16t + 4g + e][16cb + r] is Pᵀ's [16cb + r][16t + 4g + e]
                S* pt = (S*)jb.out2 + KD * KD + ((t * KT + cb) * 64 + 16 * (r >> 2) + 4 * g) * 4 + (r & 3);
#pragma unroll
                for (int e = 0; e < 4; e++) pt[4 * e] = x[e];
            }
    }
    if (jb.out_form == ST_FRAG) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int t = 0; t < KT; t++) *(f32x4*)(jb.out + (((CW * w / 16 + nb) * KT + t) * 64 + l) * 4) = St[nb][t];
    } else if (jb.out_form == ST_NAT) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int t = 0; t < KT; t++)
#pragma unroll
                for (int e = 0; e < 4; e++) jb.out[(16 * t + 4 * g + e) * VD + col0 + 16 * nb] = isc * St[nb][t][e];
    }
}

// Segment bookkeeping shared by the kernels below.
struct SegView {
    SegInfo si;
    int j, ls, S;   // segment index, its index within the sequence, segments in the sequence
    bool first, last;
};
__device__ __forceinline__ SegView seg_view(const ScanArgs& a, int j) {
    SegView v;
    v.si = a.seg[j];
    v.j = j;
    const int s0 = a.seq_seg0[v.si.seq];
    v.ls = j - s0;
    v.S = a.seq_seg0[v.si.seq + 1] - s0;
    v.first = v.ls == 0;
    v.last = v.ls == v.S - 1;
    return v;
}

// Workgroup x of a launch of (segment, value head, direction) jobs: the
// forward jobs first (nfwd of them, 0 or NS*HV), then the reverse ones; within
// a direction segment by segment, in the segment order when there is one (the
// longest segments first, so the sequences' unequal lengths even out over the
// CUs), all heads of a segment together.
__device__ __forceinline__ void job_of(const ScanArgs& a, int x, int nfwd, int HV, bool& rev, int& j, int& hv) {
    rev = x >= nfwd;
    const int b = rev ? x - nfwd : x;
    j = a.seg_order ? a.seg_order[b / HV] : b / HV;
    hv = b % HV;
}

// The scans proper (one job per (segment, value head, direction)): forward
// jobs and reverse jobs (nfwd and gridDim - nfwd of them), placed by job_of.  A job starts from h0 / dht
// at the sequence ends and from the combined boundary states otherwise; the
// first reverse segment writes dh0 and the last forward one ht.
// EST: the states are stored in type E.  It is a template parameter so the
// store is not behind a runtime branch: the compiler's wait counts are then
// exact.
template <class E, class S, int KD, int VD, bool EST>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
scan_kernel(ScanArgs a, int nfwd, int HV) {
    extern __shared__ __align__(16) unsigned char smem[];
    bool rev;
    int j, hvj;
    job_of(a, (int)blockIdx.x, nfwd, HV, rev, j, hvj);
    const SegView v = seg_view(a, j);
    const long KV = (long)KD * VD;
    ScanJob jb;
    jb.n = v.si.seq;
    jb.hv = hvj;
    jb.c0 = v.si.c0;
    jb.nc = v.si.nc;
    jb.lc0 = v.si.lc0;
    const long nblk = ((long)jb.n * HV + jb.hv) * KV, sblk = ((long)v.j * HV + jb.hv) * KV;
    if (rev) {
        const bool from_end = v.last;
        jb.init_form = from_end ? (a.dht ? ST_NAT : ST_ZERO) : ST_FRAG;
        jb.init = from_end ? (a.dht ? a.dht + nblk : nullptr) : a.dhin + sblk;
        jb.out_form = v.first && a.dh0 ? ST_NAT : ST_NONE;
        jb.out = a.dh0 ? a.dh0 + nblk : nullptr;
        job_scale(a, jb, HV);
        scan_body<E, S, KD, VD, true, EST>(a, jb, HV, smem);
    } else {
        jb.init_form = v.first ? (a.h0 ? ST_NAT : ST_ZERO) : ST_FRAG;
        jb.init = v.first ? (a.h0 ? a.h0 + nblk : nullptr) : a.hstart + sblk;
        jb.out_form = v.last && a.ht ? ST_NAT : ST_NONE;
        jb.out = a.ht ? a.ht + nblk : nullptr;
        scan_body<E, S, KD, VD, false, EST>(a, jb, HV, smem);
    }
}

// Local segment scans (16-bit operands only), NS*HV jobs per role, placed by
// job_of:
//   forward: from zero over the segment -> hloc (not needed
//       for a sequence's last segment), together with the transfer matrix
//       P = Π (γ_C I − K̃ᵀ W) of the segment, from I -> P (both read the same
//       W and K̃ tiles, so one workgroup computes both; only for sequences
//       with more than one segment);
//   reverse: from zero over the segment -> dhloc (not
//       for a sequence's first segment).
// The caller passes arguments with no per-chunk outputs (hT, dhT, h32, v_new).
template <class E, class S, int KD, int VD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
seg_kernel(ScanArgs a, int NS, int HV) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int per = NS * HV;
    bool rev;
    int j, hvj;
    job_of(a, (int)blockIdx.x, per, HV, rev, j, hvj);
    const SegView v = seg_view(a, j);
    const long KV = (long)KD * VD;
    ScanJob jb;
    jb.n = v.si.seq;
    jb.hv = hvj;
    jb.c0 = v.si.c0;
    jb.nc = v.si.nc;
    jb.lc0 = v.si.lc0;
    jb.init = nullptr;
    jb.init_form = ST_ZERO;
    jb.out2 = nullptr;
    const long sblk = ((long)v.j * HV + jb.hv) * KV;
    if (rev) {
        if (v.first || !a.do_rev) return;
        jb.out_form = ST_FRAG;
        jb.out = a.dhloc + sblk;
        job_scale(a, jb, HV);
        scan_body<E, S, KD, VD, true, false>(a, jb, HV, smem);
    } else {
        if (v.S == 1) return;
        const bool want_h = !v.last && a.do_fwd;
        jb.out_form = want_h ? ST_FRAG : ST_NONE;
        jb.out = want_h ? a.hloc + sblk : nullptr;
        jb.out2 = a.P + sblk;
        scan_body<E, S, KD, VD, false, false, true>(a, jb, HV, smem);
    }
}

// Sequential combine over the segments of one (sequence, value head):
//   forward  h_start[s+1] = P_s h_start[s] + hloc_s       (h_start[0] = h0)
//   reverse  dh_in[s-1]   = P_sᵀ dh_in[s] + dhloc_s       (dh_in[S-1] = dht)
// writing every boundary state except the two sequence ends (which the scans
// read from h0 / dht).  The state columns evolve independently: each
// (sequence, value head, direction) job is split over VD/16 workgroups of one
// 16-column block each, and wave w of a workgroup forms rows 32w .. 32w+31 of
// the new state X as Xᵀ = Stᵀ Mᵀ with M = P_s (forward) or P_sᵀ (reverse).
// The A operand Stᵀ is read from a [16][K] 16-bit copy of the state in LDS
// (double-buffered, one barrier per step).  The B operand Mᵀ comes straight
// from global memory: the local scans store P_s in the accumulator fragment
// order (a lane's four values are four consecutive rows of one column, half of
// a B fragment of P) and P_sᵀ in the same order in the block's second half, so
// every fragment is two 8-byte loads, issued two segments ahead.  hloc enters
// as the accumulators' initial value; X leaves in the scans' fragment order.
// Grid: forward jobs then reverse jobs, N*HV*VD/16 each; 2*KD threads.
template <class S, int KD, int VD>
__global__ void __launch_bounds__(2 * KD) combine_kernel(ScanArgs a, int nseq, int HV) {
    static_assert(KD == VD, "the transfer matrix multiplies the state from the left");
    static_assert(sizeof(S) == 2, "transfer matrices are 16-bit");
    constexpr int KT = KD / 16, NCB = VD / 16, NTH = 2 * KD, LKT = KD + 8, NKS = KD / 32;
    constexpr int NI = 16 * KD / NTH;   // initial-state elements per thread
    typedef S s4 __attribute__((ext_vector_type(4)));
    using frag = typename Mma<S>::frag;
    extern __shared__ __align__(16) unsigned char smem[];
    S* sT = (S*)smem;   // two [16][LKT] buffers of Stᵀ
    const int per = nseq * HV * NCB;
    const bool rev = (int)blockIdx.x >= per;
    const int b = rev ? (int)blockIdx.x - per : (int)blockIdx.x;
    const int cbw = b % NCB, hv = b / NCB % HV, n = b / NCB / HV;
    const int s0 = a.seq_seg0[n], S_n = a.seq_seg0[n + 1] - s0;
    if (S_n < 2 || (rev ? !a.do_rev : !a.do_fwd)) return;
    const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
    const long KV = (long)KD * VD;
    auto blk = [&](float* base, int j) { return base + ((long)j * HV + hv) * KV; };

    // the initial state's 16 columns -> Stᵀ (reverse: in the scaled space)
    {
        const float* init = rev ? a.dht : a.h0;
        const float isc0 = rev && a.dsc ? a.dsc[(long)n * HV + hv] : 1.f;
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const int idx = threadIdx.x + NTH * i, k = idx / 16, c = idx % 16;
            const float x = init ? isc0 * init[((long)n * HV + hv) * KV + (long)k * VD + 16 * cbw + c] : 0.f;
            sT[c * LKT + k] = (S)x;
        }
    }
    // step q uses segment j(q): forward j = s0 + q (q = 0 .. S_n-2), reverse j = s0 + S_n-1-q
    const int nsteps = S_n - 1;
    auto seg_of = [&](int q) { return rev ? s0 + S_n - 1 - q : s0 + q; };
    // this lane's elements of X (and of hloc, and of the output) in the scans'
    // fragment order: X[32w + 16nt + r][16cbw + 4g + e] at float offset
    // ((cbw KT + 2w + nt) 64 + 16 (r/4) + 4g + e) 4 + r % 4
    auto foff = [&](int nt, int e) { return ((cbw * KT + 2 * w + nt) * 64 + 16 * (r >> 2) + 4 * g + e) * 4 + (r & 3); };
    struct Stg {
        s4 m[NKS][2][2];   // B fragments of Mᵀ: k-step, n tile, half
        float h[2][4];     // hloc
    };
    auto prefetch = [&](Stg& x, int q) {
        const int j = seg_of(q);
        const S* M = (const S*)blk(a.P, j) + (rev ? 0 : KD * KD);
        const float* H = blk(rev ? a.dhloc : a.hloc, j);
#pragma unroll
        for (int sk = 0; sk < NKS; sk++)
#pragma unroll
            for (int nt = 0; nt < 2; nt++) {
                // rows 32 sk + 8 g + {0..7} of column 32 w + 16 nt + r of Mᵀ's
                // stored tile (column block 2w + nt, row block 2 sk + g/2)
                const S* p = M + (((2 * w + nt) * KT + 2 * sk + (g >> 1)) * 64 + 32 * (g & 1) + r) * 4;
                x.m[sk][nt][0] = *(const s4*)p;
                x.m[sk][nt][1] = *(const s4*)(p + 64);
            }
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
            for (int e = 0; e < 4; e++) x.h[nt][e] = H[foff(nt, e)];
    };
    auto step = [&](int q, const Stg& x) {
        const S* cur = sT + (q & 1) * 16 * LKT;
        S* nxt = sT + ((q + 1) & 1) * 16 * LKT;
        f32x4 C[2];
#pragma unroll
        for (int nt = 0; nt < 2; nt++) C[nt] = f32x4{x.h[nt][0], x.h[nt][1], x.h[nt][2], x.h[nt][3]};
#pragma unroll
        for (int sk = 0; sk < NKS; sk++) {
            const frag fa = *(const frag*)(cur + r * LKT + 32 * sk + 8 * g);
#pragma unroll
            for (int nt = 0; nt < 2; nt++) {
                const s4 lo = x.m[sk][nt][0], hi = x.m[sk][nt][1];
                frag fb;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    fb[e] = lo[e];
                    fb[4 + e] = hi[e];
                }
                C[nt] = Mma<S>::run(fa, fb, C[nt]);
            }
        }
        // C[nt][e] = X[32w + 16nt + r][16cbw + 4g + e]
        const int jd = rev ? seg_of(q) - 1 : seg_of(q) + 1;   // the segment whose boundary state this is
        float* out = blk(rev ? a.dhin : a.hstart, jd);
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                out[foff(nt, e)] = C[nt][e];
                nxt[(4 * g + e) * LKT + 32 * w + 16 * nt + r] = (S)C[nt][e];
            }
        lds_barrier();   // the next state is complete; this one is no longer read
    };
    Stg x0, x1;
    prefetch(x0, 0);
    if (nsteps > 1) prefetch(x1, 1);
    lds_barrier();   // the initial state
    for (int q = 0; q < nsteps; q += 2) {
        step(q, x0);
        if (q + 2 < nsteps) prefetch(x0, q + 2);
        if (q + 1 < nsteps) {
            step(q + 1, x1);
            if (q + 3 < nsteps) prefetch(x1, q + 3);
        }
    }
}

// Scale of the reverse scans (16-bit operands).  The dh recursion is linear in
// (dO, dht), so it runs on s·dO and s·dht with s a power of two per (sequence,
// value head) chosen so that max(|dO|, |dht|)·s lies in [1/2, 1): gradients of
// a loss averaged over many tokens (|dO| ~ 1e-6 .. 1e-8) would otherwise fall
// below fp16's normal range when dO and the state are narrowed to fp16 MFMA
// operands.  The per-chunk states and dh0 are stored times 1/s (exact).
// dmax_kernel: blocks [0, 4·NT) take max |dO| over a quarter (16 rows) of one
// chunk for every value head (the rows are contiguous across the heads: each
// thread takes 16-byte vectors of one head, V/8 threads share a head), blocks
// [4·NT, 4·NT + N·HV) max |dht| over one K x V block.  dO is read with
// non-temporal loads (the next kernels stream a gigabyte before the scans
// read it again).
template <class E, int VD>
__global__ void __launch_bounds__(256) dmax_kernel(ScanArgs a, int NT, int HV, int KV) {
    typedef E e8 __attribute__((ext_vector_type(8)));
    constexpr int VPH = VD / 8;                      // vectors per head and row (16 at V = 128)
    __shared__ float red[256];
    const int b = blockIdx.x;
    if (b < 4 * NT) {
        const ChunkInfo ch = a.info[b >> 2];
        const int r0 = 16 * (b & 3), r1 = min(r0 + 16, ch.len);   // rows of this quarter (may be none)
        const E* dO = (const E*)a.dO + (long)ch.t0 * HV * VD;
        const int vpr = HV * VPH;                    // vectors per token row
        for (int h0 = 0; h0 < vpr; h0 += 256) {      // heads handled by this pass
            const int vi = h0 + (int)threadIdx.x;
            float m = 0.f;
            if (vi < vpr && r0 < r1)
                for (int rb = r0; rb < r1; rb += 8) {   // eight rows in flight (repeated last row: same max)
                    e8 x[8];
#pragma unroll
                    for (int u = 0; u < 8; u++)
                        x[u] = __builtin_nontemporal_load((const e8*)(dO + ((long)min(rb + u, r1 - 1) * vpr + vi) * 8));
#pragma unroll
                    for (int u = 0; u < 8; u++)
#pragma unroll
                        for (int e = 0; e < 8; e++) m = fmaxf(m, fabsf((float)x[u][e]));
                }
            // the VPH threads of a head are consecutive: reduce within the group
#pragma unroll
            for (int off = 1; off < VPH; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
            if (vi < vpr && vi % VPH == 0) a.cmax[(long)b * HV + vi / VPH] = m;
        }
        return;
    }
    const int j = b - 4 * NT;
    float m = 0.f;
    if (a.dht) {   // eight 16-byte loads in flight per thread
        const float* x = a.dht + (long)j * KV;
        for (int i0 = 0; i0 < KV / 4; i0 += 8 * 256) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = *(const f32x4*)(x + 4 * min(i0 + u * 256 + (int)threadIdx.x, KV / 4 - 1));
#pragma unroll
            for (int u = 0; u < 8; u++)
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3]))));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) a.hmax[j] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One block per (sequence, value head): the maximum over the sequence's chunks
// and its dht block, and the power of two s = 2^-e with max = f·2^e, f in [1/2, 1)
// (s = 1 when the maximum is zero or not finite).
__global__ void __launch_bounds__(256) dscale_kernel(ScanArgs a, int HV) {
    __shared__ float red[4];
    const int j = blockIdx.x, n = j / HV, hv = j % HV;
    const int c0 = 4 * a.seq_chunk0[n], c1 = 4 * a.seq_chunk0[n + 1];   // chunk quarters of the sequence
    float m = 0.f;
    for (int c = c0 + (int)threadIdx.x; c < c1; c += 256) m = fmaxf(m, a.cmax[(long)c * HV + hv]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), a.hmax[j]);
        float s = 1.f;
        if (m > 0.f && isfinite(m)) {
            int e;
            frexpf(m, &e);
            s = ldexpf(1.f, -e);
        }
        a.dsc[j] = s;
    }
}

template <class E, class S, int KD, int VD>
static hipError_t scan_go(const Problem& p, const ScanArgs& a, hipStream_t s) {
    using Cf = ScanCfg<E, S, KD, VD>;
    const int nseq = p.cu ? p.N : p.B;
    const int per = p.NS * p.HV;
    const int nfwd = a.do_fwd ? per : 0, nrev = a.do_rev ? per : 0;
    if (nfwd + nrev == 0) return hipSuccess;
    // either every launched scan stores its E-typed states or none does
    const bool est_f = !a.do_fwd || a.hT, est_r = !a.do_rev || a.dhT;
    const bool none_f = !a.do_fwd || !a.hT, none_r = !a.do_rev || !a.dhT;
    if (!(est_f && est_r) && !(none_f && none_r)) return hipErrorInvalidValue;
    static_assert(Cf::smem <= 160 * 1024, "LDS budget");
    if (p.maxS > 1) {
        if constexpr (sizeof(S) == 2) {
            ScanArgs a1 = a;   // local scans write only their final states
            a1.hT = nullptr; a1.dhT = nullptr; a1.h32 = nullptr; a1.v_new = nullptr;
            auto k1 = seg_kernel<E, S, KD, VD>;
            if (hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem) !=
                hipSuccess)
                return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL(k1, dim3(2 * per), dim3(256), Cf::smem, s, a1, p.NS, p.HV);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            constexpr int csm = 2 * 16 * (KD + 8) * (int)sizeof(S);
            hipLaunchKernelGGL((combine_kernel<S, KD, VD>), dim3(2 * nseq * p.HV * (VD / 16)), dim3(2 * KD), csm, s, a,
                               nseq, p.HV);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        } else {
            return hipErrorInvalidValue;   // fp32 problems are planned without segments
        }
    }
    auto kern = (est_f && est_r) ? scan_kernel<E, S, KD, VD, true> : scan_kernel<E, S, KD, VD, false>;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::smem) != hipSuccess)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3(nfwd + nrev), dim3(256), Cf::smem, s, a, nfwd, p.HV);
    return hipGetLastError();
}

// The reverse scans' scales (16-bit problems with a.dsc set): max |dO| per
// quarter chunk and max |dht| per block, then one power of two per (sequence,
// value head).  They read only dO and dht, so the call may run them before
// the WY factors.
template <class E, int VD>
static hipError_t scale_go(const Problem& p, const ScanArgs& a, hipStream_t s, int KV) {
    const int nseq = p.cu ? p.N : p.B;
    static_assert(VD % 8 == 0 && 64 % (VD / 8) == 0, "a head's vectors stay inside one wave");
    hipLaunchKernelGGL((dmax_kernel<E, VD>), dim3((unsigned)(4 * p.NT + (int64_t)nseq * p.HV)), dim3(256), 0, s, a,
                       (int)p.NT, p.HV, KV);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dscale_kernel, dim3((unsigned)(nseq * p.HV)), dim3(256), 0, s, a, p.HV);
    return hipGetLastError();
}

hipError_t launch_scan_scales(const Problem& p, const ScanArgs& a, hipStream_t s) {
    if (!a.do_rev || !a.dsc || p.dtype == 0) return hipSuccess;
    if (p.V == 128) return p.dtype == 2 ? scale_go<bf16, 128>(p, a, s, p.K * 128) : scale_go<f16, 128>(p, a, s, p.K * 128);
    if (p.V == 64) return p.dtype == 2 ? scale_go<bf16, 64>(p, a, s, p.K * 64) : scale_go<f16, 64>(p, a, s, p.K * 64);
    return hipErrorInvalidValue;
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
