// gdr_tri.hpp -- the blocked fp32 inverse of a unit lower-triangular 64 x 64
// matrix (the WY factor A = (I + L)^{-1} of one chunk), shared by the GDN and
// KDA WY-factor kernels.
#pragma once
#include "gdr_device.hpp"

namespace gdr {

// acc += X · Y for 16 x 16 fp32 blocks held row-major in LDS (fp32 MFMA, exact
// products): lane (r, g) feeds X[r][4s+g] and Y[4s+g][r] and holds
// (X·Y)[4g+j][r] in acc[j].
__device__ __forceinline__ void mm16(f32x4& acc, const float* X, int ldx, const float* Y, int ldy) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
    for (int s = 0; s < 4; s++) acc = Mma<float>::run(X[r * ldx + 4 * s + g], Y[(4 * s + g) * ldy + r], acc);
}
__device__ __forceinline__ void put16(float* Z, int ldz, const f32x4& acc, float sgn) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
    for (int j = 0; j < 4; j++) Z[(4 * g + j) * ldz + r] = sgn * acc[j];
}

// A = (I + L)^{-1} for the strictly lower 64 x 64 L in sL (fp32, pitch LL),
// written to sAf (fp32, pitch LL) by waves 0..3 together (the others only help
// to zero the blocks above the diagonal).  With 16 x 16
// blocks, D_i = (I + L_ii)^{-1} and A_ij = −D_i Σ_{j<=k<i} L_ik A_kj:
//   step 1: wave w inverts D_w by forward substitution (one lane per column);
//   step 2: A_10 = −D_1 L_10 D_0 and A_32 = −D_3 L_32 D_2; meanwhile
//           Y01 = L_21 D_1 and Y11 = L_31 D_1;
//   step 3: with Y00 = L_20 D_0 + L_21 A_10 and Y10 = L_30 D_0 + L_31 A_10,
//           A_20 = −D_2 Y00, A_21 = −D_2 Y01, A_30 = −(A_32 Y00 + D_3 Y10),
//           A_31 = −(A_32 Y01 + D_3 Y11)   (one block per wave).
// The block products are fp32 MFMAs on LDS operands; sT holds two [16][17]
// scratch blocks per wave.
template <int LL, int NTHR>
__device__ __forceinline__ void tri_inverse64(const float* sL, float* sAf, float* sT) {
    const int w = wave_id(), l = lane_id();
    constexpr int LT = 17;
    float* t0 = sT + w * 2 * 16 * LT;
    float* t1 = t0 + 16 * LT;
    auto Lb = [&](int i, int j) { return sL + 16 * i * LL + 16 * j; };
    auto Ab = [&](int i, int j) { return sAf + 16 * i * LL + 16 * j; };
    // step 1 (+ zero the blocks above the diagonal)
    if (w < 4 && l < 16) {
        const float* L = Lb(w, w);
        float a[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            float acc = r == l ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; s++) acc -= L[r * LL + s] * a[s];
            a[r] = acc;
        }
        float* D = Ab(w, w);
#pragma unroll
        for (int r = 0; r < 16; r++) D[r * LL + l] = a[r];
    }
    for (int idx = threadIdx.x; idx < 6 * 256; idx += NTHR) {
        const int blk = idx >> 8, e = idx & 255;
        const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2), bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        Ab(bi, bj)[(e >> 4) * LL + (e & 15)] = 0.f;
    }
    lds_barrier();
    // step 2
    {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (w >= 4) {
        } else if (w < 2) {
            const int i = 2 * w + 1, j = 2 * w;            // (1,0) or (3,2)
            mm16(acc, Lb(i, j), LL, Ab(j, j), LL);
            put16(t0, LT, acc, 1.f);
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            mm16(acc, Ab(i, i), LL, t0, LT);
            put16(Ab(i, j), LL, acc, -1.f);
        } else {
            mm16(acc, Lb(w, 1), LL, Ab(1, 1), LL);         // Y01 = L_21 D_1 or Y11 = L_31 D_1
            put16(t0, LT, acc, 1.f);
        }
    }
    lds_barrier();
    // step 3: wave w -> block (2 + (w >> 1), w & 1).  LDS operations of one
    // wave execute in order, so a wave may rewrite its own scratch block right
    // after reading it.
    {
        const float* Y01 = sT + 2 * 2 * 16 * LT;   // wave 2's first block
        const float* Y11 = sT + 3 * 2 * 16 * LT;   // wave 3's first block
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (w == 0 || w == 2) {
            mm16(acc, Lb(2, 0), LL, Ab(0, 0), LL);   // Y00 = L_20 D_0 + L_21 A_10
            mm16(acc, Lb(2, 1), LL, Ab(1, 0), LL);
            put16(t1, LT, acc, 1.f);
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (w == 0) {
                mm16(x, Ab(2, 2), LL, t1, LT);       // A_20 = −D_2 Y00
                put16(Ab(2, 0), LL, x, -1.f);
            } else {
                mm16(x, Ab(3, 2), LL, t1, LT);       // A_32 Y00
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
                mm16(acc, Lb(3, 0), LL, Ab(0, 0), LL);   // Y10 = L_30 D_0 + L_31 A_10
                mm16(acc, Lb(3, 1), LL, Ab(1, 0), LL);
                put16(t1, LT, acc, 1.f);
                mm16(x, Ab(3, 3), LL, t1, LT);       // + D_3 Y10
                put16(Ab(3, 0), LL, x, -1.f);        // A_30
            }
        } else if (w == 1) {
            mm16(acc, Ab(2, 2), LL, Y01, LT);        // A_21 = −D_2 Y01
            put16(Ab(2, 1), LL, acc, -1.f);
        } else if (w == 3) {
            mm16(acc, Ab(3, 2), LL, Y01, LT);        // A_31 = −(A_32 Y01 + D_3 Y11)
            mm16(acc, Ab(3, 3), LL, Y11, LT);
            put16(Ab(3, 1), LL, acc, -1.f);
        }
    }
    lds_barrier();
}

// In-place variant for a workgroup of exactly four waves: sLA holds L on
// entry (strictly lower, zero on and above the diagonal, fp32, pitch LL) and
// A = (I + L)^{-1} on exit, with the same block recursion.  Each block of A
// is written over the block of L it replaces once no wave reads that L block
// any more: D_w over L_ww (step 1, wave w alone); A_10, A_32 over L_10, L_32
// (step 2, the only step reading them); Y00 = L_20 D_0 + L_21 A_10 and
// Y10 = L_30 D_0 + L_31 A_10 go to scratch (step 3a); after a barrier
// A_20 = −D_2 Y00, A_21 = −D_2 Y01, A_30 = −(A_32 Y00 + D_3 Y10) and
// A_31 = −(A_32 Y01 + D_3 Y11), one block per wave (step 3b).  sT holds two
// [16][17] scratch blocks per wave.
template <int LL>
__device__ __forceinline__ void tri_inverse64_inplace(float* sLA, float* sT) {
    const int w = wave_id(), l = lane_id();
    constexpr int LT = 17;
    float* t0 = sT + w * 2 * 16 * LT;
    float* t1 = t0 + 16 * LT;
    auto Bk = [&](int i, int j) { return sLA + 16 * i * LL + 16 * j; };
    // step 1: lane l < 16 of wave w forms column l of D_w by forward
    // substitution, then writes the whole column (zeros above the diagonal)
    if (l < 16) {
        const float* L = sLA + 16 * w * LL + 16 * w;
        float a[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            float acc = r == l ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; s++) acc -= L[r * LL + s] * a[s];
            a[r] = acc;
        }
        float* D = sLA + 16 * w * LL + 16 * w;
#pragma unroll
        for (int r = 0; r < 16; r++) D[r * LL + l] = a[r];
    }
    lds_barrier();
    // step 2
    {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (w < 2) {
            const int i = 2 * w + 1, j = 2 * w;            // (1,0) or (3,2)
            mm16(acc, Bk(i, j), LL, Bk(j, j), LL);
            put16(t0, LT, acc, 1.f);
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            mm16(acc, Bk(i, i), LL, t0, LT);
            put16(Bk(i, j), LL, acc, -1.f);
        } else {
            mm16(acc, Bk(w, 1), LL, Bk(1, 1), LL);         // Y01 = L_21 D_1 or Y11 = L_31 D_1
            put16(t0, LT, acc, 1.f);
        }
    }
    lds_barrier();
    // step 3a: Y00 (wave 0) and Y10 (wave 1)
    if (w < 2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mm16(acc, Bk(2 + w, 0), LL, Bk(0, 0), LL);
        mm16(acc, Bk(2 + w, 1), LL, Bk(1, 0), LL);
        put16(t1, LT, acc, 1.f);
    }
    lds_barrier();
    // step 3b: wave w -> block (i, j) = (2 + (w >> 1), w & 1):
    // A_2j = −D_2 Y0j, A_3j = −(A_32 Y0j + D_3 Y1j), with Y00 / Y10 in the
    // second blocks of waves 0 / 1 and Y01 / Y11 in the first blocks of
    // waves 2 / 3 (offsets into the scratch, so no pointer is selected)
    {
        const int i = 2 + (w >> 1), j = w & 1;
        const int o0 = j == 0 ? 16 * LT : 4 * 16 * LT;       // Y0j
        const int o1 = j == 0 ? 3 * 16 * LT : 6 * 16 * LT;   // Y1j
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mm16(acc, Bk(i, 2), LL, sT + o0, LT);
        if (i == 3) mm16(acc, Bk(3, 3), LL, sT + o1, LT);
        put16(Bk(i, j), LL, acc, -1.f);
    }
    lds_barrier();
}

}  // namespace gdr
