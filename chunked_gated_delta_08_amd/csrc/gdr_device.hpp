// gdr_device.hpp -- device-side building blocks for the gfx950 kernels.
//
// MFMA operand layouts (16x16 output tile, wave64; verified on gfx950):
//   16-bit (v_mfma_f32_16x16x32_{bf16,f16}): lane l = 16*g + r holds
//       A[r][8g+i], B[8g+i][r] for i = 0..7, and D[4g+j][r] for j = 0..3.
//   fp32   (v_mfma_f32_16x16x4_f32):        lane l holds A[r][g], B[g][r],
//       and the same D layout.
// Operands come from LDS in one of two orientations:
//   "direct": the matrix is stored with its reduction index k contiguous
//             (A as [m][k], B as [n][k]) -> one 16-byte read per fragment;
//   "trans":  the matrix is stored with k strided (A as [k][m], B as [k][n])
//             -> two ds_read_b64_tr_b16 transposing reads per fragment.
//   ds_read_b64_tr_b16: within each 16-lane group, lane r addresses 8 bytes at
//   row (k0 + r/4), column (mn0 + 4*(r%4)); lane i then receives
//   X[k0 + j][mn0 + i] for j = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_launch.hpp"

namespace gdr {

using bf16 = __bf16;
using f16 = _Float16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier for LDS exchange only: waits for this wave's LDS traffic
// and meets the other waves, without the release fence of __syncthreads()
// (which makes every barrier wait for all outstanding global loads and
// stores).  No kernel here exchanges data through global memory inside a
// workgroup.  The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

template <class E> __device__ __forceinline__ E to_e(float x) { return (E)x; }
template <class E> __device__ __forceinline__ float to_f(E x) { return (float)x; }

// --------------------------------------------------------------------------
// MFMA traits
template <class E> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int KS = 32;
    using frag = bf16x8;
    __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<f16> {
    static constexpr int KS = 32;
    using frag = f16x8;
    __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int KS = 4;
    using frag = float;
    __device__ __forceinline__ static f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// --------------------------------------------------------------------------
// Fragment loads from LDS (padded row-major tiles, leading dimension ld).
// Requirements (16-bit): ld % 8 == 0, k0 % 8 == 0 for direct; ld % 4 == 0,
// mn0 % 4 == 0 for trans.
template <class E>
__device__ __forceinline__ typename Mma<E>::frag ld_direct(const E* X, int ld, int mn0, int k0) {
    const int l = lane_id();
    if constexpr (sizeof(E) == 2) {
        return *(const typename Mma<E>::frag*)(X + (mn0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
    } else {
        return X[(mn0 + (l & 15)) * ld + k0 + (l >> 4)];
    }
}

template <class E>
__device__ __forceinline__ typename Mma<E>::frag ld_trans(const E* X, int ld, int mn0, int k0) {
    const int l = lane_id();
    const int r = l & 15, g = l >> 4;
    if constexpr (sizeof(E) == 2) {
        const E* p = X + (k0 + 8 * g + (r >> 2)) * ld + mn0 + 4 * (r & 3);
        i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
        i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 4 * ld));
        i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        return __builtin_bit_cast(typename Mma<E>::frag, c);
    } else {
        return X[(k0 + g) * ld + mn0 + r];
    }
}

// Transposing read of 4 consecutive k (rows k0 + 4*g_sel .. +3 chosen by the
// caller through `krow`) for column mn0 + r of a [k][mn] tile: the building
// block for fragments whose k order is permuted (see the scans).
template <class E>
__device__ __forceinline__ i16x4 ld_trans4(const E* X, int ld, int mn0, int krow) {
    const int r = lane_id() & 15;
    const E* p = X + (krow + (r >> 2)) * ld + mn0 + 4 * (r & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
}

// --------------------------------------------------------------------------
// Wave-level GEMM: acc[i][j] += A[m0+16i.., k] * B[k, n0+16j..] over k < KD.
// AT: A stored [k][m] (else [m][k]).  BT_: B stored [k][n] (else [n][k]).
// The fragments of k-step s+1 are read from LDS before the MFMAs of k-step s
// are issued (register double buffer), so LDS latency overlaps the MFMAs.
template <class E, int TM, int TN, int KD, bool AT, bool BT_>
__device__ __forceinline__ void wgemm(f32x4 (&acc)[TM][TN], const E* A, int lda, const E* B, int ldb, int m0,
                                      int n0) {
    using M = Mma<E>;
    constexpr int NS = KD / M::KS;
    typename M::frag a[2][TM], b[2][TN];
    auto load = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < TM; i++)
            a[buf][i] = AT ? ld_trans<E>(A, lda, m0 + 16 * i, k0) : ld_direct<E>(A, lda, m0 + 16 * i, k0);
#pragma unroll
        for (int j = 0; j < TN; j++)
            b[buf][j] = BT_ ? ld_trans<E>(B, ldb, n0 + 16 * j, k0) : ld_direct<E>(B, ldb, n0 + 16 * j, k0);
    };
    load(0, 0);
#pragma unroll
    for (int s = 0; s < NS; s++) {
        if (s + 1 < NS) load((s + 1) & 1, (s + 1) * M::KS);
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) acc[i][j] = M::run(a[s & 1][i], b[s & 1][j], acc[i][j]);
    }
}

template <int TM, int TN>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = zero4();
}

// Row-form wave GEMM: as wgemm, but the MFMA takes the B fragment first, so
// each tile comes out transposed in the lanes: lane 16g + r holds row r and
// columns 4g .. 4g+3 of tile (i, j) (four adjacent columns of one row), i.e.
// element e at row rf_row(m0, i), column rf_col(n0, j) + e.
template <class E, int TM, int TN, int KD, bool AT, bool BT_>
__device__ __forceinline__ void wgemm_rf(f32x4 (&acc)[TM][TN], const E* A, int lda, const E* B, int ldb, int m0,
                                         int n0) {
    using M = Mma<E>;
    constexpr int NS = KD / M::KS;
    typename M::frag a[2][TM], b[2][TN];
    auto load = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < TM; i++)
            a[buf][i] = AT ? ld_trans<E>(A, lda, m0 + 16 * i, k0) : ld_direct<E>(A, lda, m0 + 16 * i, k0);
#pragma unroll
        for (int j = 0; j < TN; j++)
            b[buf][j] = BT_ ? ld_trans<E>(B, ldb, n0 + 16 * j, k0) : ld_direct<E>(B, ldb, n0 + 16 * j, k0);
    };
    load(0, 0);
#pragma unroll
    for (int s = 0; s < NS; s++) {
        if (s + 1 < NS) load((s + 1) & 1, (s + 1) * M::KS);
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) acc[i][j] = M::run(b[s & 1][j], a[s & 1][i], acc[i][j]);
    }
}
__device__ __forceinline__ int rf_row(int m0, int i) { return m0 + 16 * i + (lane_id() & 15); }
__device__ __forceinline__ int rf_col(int n0, int j) { return n0 + 16 * j + 4 * (lane_id() >> 4); }

// Four adjacent elements (one row of a tile in row form) as fp32, and back.
template <class E> struct Vec4;
template <> struct Vec4<bf16> { typedef __bf16 t __attribute__((ext_vector_type(4))); };
template <> struct Vec4<f16> { typedef _Float16 t __attribute__((ext_vector_type(4))); };
template <> struct Vec4<float> { typedef float t __attribute__((ext_vector_type(4))); };
template <class E>
__device__ __forceinline__ f32x4 ld4(const E* p) {
    return __builtin_convertvector(*(const typename Vec4<E>::t*)p, f32x4);
}
template <class E>
__device__ __forceinline__ void st4(E* p, f32x4 x) {
    *(typename Vec4<E>::t*)p = __builtin_convertvector(x, typename Vec4<E>::t);
}

// Row / column of accumulator element e of tile (i, j) for this lane.
__device__ __forceinline__ int acc_row(int m0, int i, int e) { return m0 + 16 * i + 4 * (lane_id() >> 4) + e; }
__device__ __forceinline__ int acc_col(int n0, int j) { return n0 + 16 * j + (lane_id() & 15); }

// The lane index, recomputed where it is used: the compiler cannot share it
// (or the addresses derived from it) between phases, so lane-dependent LDS
// offsets are rebuilt per product (two VALU ops) instead of being kept live
// across the whole kernel in registers the accumulators need.
// (the masks after the opaque step restore the value range, so index
// arithmetic stays on 24-bit multiplies)
__device__ __forceinline__ int lane_o() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l & 63;
}
// Fragment helpers.  A lane's base pointer into an operand X at rows /
// columns mn0 (tr: X stored [k][mn], else [mn][k]); fragment n of the k-step
// at k0 is that base plus a constant offset (16-bit: direct rows mn0 + r,
// keys 8g..8g+7; transposed reads start at row k0 + 8g + r/4, column
// mn0 + 4(r%4), and at 4 rows further).
template <class E, bool TR>
__device__ __forceinline__ const E* frag_base(const E* X, int ld, int mn0, int l) {
    const int r = l & 15, g = l >> 4;
    if constexpr (sizeof(E) == 2)
        return TR ? X + (8 * g + (r >> 2)) * ld + mn0 + 4 * (r & 3) : X + (mn0 + r) * ld + 8 * g;
    else
        return TR ? X + g * ld + mn0 + r : X + (mn0 + r) * ld + g;
}
template <class E, int N, bool TR>
__device__ __forceinline__ void frags(typename Mma<E>::frag (&f)[N], const E* base, int ld, int k0) {
#pragma unroll
    for (int n = 0; n < N; n++) {
        if constexpr (sizeof(E) == 2) {
            if constexpr (!TR) {
                f[n] = *(const typename Mma<E>::frag*)(base + 16 * n * ld + k0);
            } else {
                const E* q = base + k0 * ld + 16 * n;
                i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, q));
                i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, q + 4 * ld));
                i16x8 c = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                f[n] = __builtin_bit_cast(typename Mma<E>::frag, c);
            }
        } else {
            f[n] = TR ? base[k0 * ld + 16 * n] : base[16 * n * ld + k0];
        }
    }
}
// acc[i][j] += A-tile i times B-tile j, run as (Bᵀ Aᵀ)ᵀ: the MFMA takes the B
// fragment as its first operand, so the tile comes out in row form: lane
// 16g + r holds row r and columns 4g .. 4g+3 of the tile (four adjacent
// columns of one row: whole 8-byte stores, and one row per lane).
template <class E, int TM, int TN>
__device__ __forceinline__ void mma_tiles(f32x4 (&acc)[TM][TN], const typename Mma<E>::frag (&fa)[TM],
                                          const typename Mma<E>::frag (&fb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = Mma<E>::run(fb[j], fa[i], acc[i][j]);
}

// Wave-level product acc[i][j] += A[m0+16i.., k] * B[k, n0+16j..] over k < KD
// (AT: A stored [k][m], else [m][k]; BT_: B stored [k][n], else [n][k]); one
// k-step of fragments in registers at a time (the other workgroup on the CU
// covers the LDS latency); lane offsets from a fresh lane index (see lane_o).
template <class E, int TM, int TN, int KD, bool AT, bool BT_>
__device__ __forceinline__ void gemm4(f32x4 (&acc)[TM][TN], const E* A, int lda, const E* B, int ldb, int m0, int n0) {
    using M = Mma<E>;
    const int l = lane_o();
    const E* pa = frag_base<E, AT>(A, lda, m0, l);
    const E* pb = frag_base<E, BT_>(B, ldb, n0, l);
#pragma unroll
    for (int s = 0; s < KD / M::KS; s++) {
        typename M::frag fa[TM], fb[TN];
        frags<E, TM, AT>(fa, pa, lda, s * M::KS);
        frags<E, TN, BT_>(fb, pb, ldb, s * M::KS);
        mma_tiles<E>(acc, fa, fb);
    }
}

// base + off elements, with the byte offset formed in 32 bits: a uniform base
// and a 32-bit per-lane offset map onto the scalar-base addressing of global
// loads and stores (no 64-bit address arithmetic per lane).
template <class T>
__device__ __forceinline__ T* at32(T* base, unsigned off) {
    return (T*)((char*)base + off * (unsigned)sizeof(T));
}
template <class T>
__device__ __forceinline__ const T* at32(const T* base, unsigned off) {
    return (const T*)((const char*)base + off * (unsigned)sizeof(T));
}

// Global <-> register helpers
template <class E> struct Vec16;  // 16-byte vector of E
template <> struct Vec16<bf16> { using t = bf16x8; static constexpr int n = 8; };
template <> struct Vec16<f16> { using t = f16x8; static constexpr int n = 8; };
template <> struct Vec16<float> { using t = f32x4; static constexpr int n = 4; };

}  // namespace gdr
