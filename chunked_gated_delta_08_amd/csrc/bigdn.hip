// bigdn.hip -- BiGDN chunkwise layer on gfx950: the frame-level bidirectional
// gated delta rule with its normaliser stream, forward and backward.
//
// Source: Sana `fused_gdn_chunkwise_bwd.py` (phase C̄, phase B̄, the
// combine of both directions, phase Ā for the key-value and normaliser
// streams, the output-divide VJP, the fused RoPE/ReLU kernels and the
// full-channel RMSNorm backward of `FusedBiGDNChunkwiseFunction`).
//
// Per (batch, head), frame f of S tokens:
//   Qu = relu(RMSNorm(q)), Ku = k_scale relu(RMSNorm(k)), Qr/Kr = rope(Qu/Ku)
//   P_f = Kr^T diag(b) Kr   A_f = Kr^T diag(b) V   Pz_f = Ku^T diag(b) Ku   Bz_f = Ku^T b
//   Mf[f] = g_f (I - P_f) Mf[f-1] + A_f        (inclusive forward scan)
//   Mr[f-1] = g_f (I - P_f) Mr[f] + A_f         (exclusive reverse scan, Mr[F-1] = 0)
//   z: the same scans with (Pz, Bz)
//   out = Qr (Mf + Mr) / (Qu . (zf + zr) + eps)
// P and Pz are symmetric, so (I - P)^T = I - P in the gradient scans.
//
// Kernels (one launch each):
//   rms_stats   per token: inverse RMS of q and k over all H*D channels
//   phase_a     per frame: P, A, Pz, Bz on bf16 MFMA (reduction over tokens)
//   scan        per (batch*head, direction): a frame scan M <- X + g (M - P M)
//               for the states (forward) or the state gradients (backward),
//               state in fp32 MFMA accumulators, z alongside on the VALU
//   phase_c     per frame: num = Qr Mc (+ divide: the forward's output), or the
//               divide VJP, dQr = dnum Mc^T, dMc = Qr^T dnum, the normaliser
//               terms, unrope and the ReLU mask: dQn
//   abar        per frame: dA, dP + dP^T, dg of both directions and streams,
//               then per token tile dKr, dV, dbeta; unrope, mask: dKn
//   rms_bwd     per token: the RMSNorm VJP (dq, dk in place) and norm-weight
//               partial sums; wsum adds the partials.
#include "bigdn_launch.hpp"
#include "gdr_device.hpp"

namespace bigdn {
using namespace gdr;

constexpr int ST = 64;  // tokens per tile

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
// Sum over aligned groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = a[i], v[4 + i] = b[i];
}

// Token-tile mapping for 512 threads: each thread owns 16-byte chunks (8
// channels) of token rows; the chunk column c is fixed per thread.
template <int D>
struct TileMap {
    static constexpr int CPR = D / 8;            // chunks per token row
    static constexpr int NPT = ST * CPR / 512;   // chunks per thread
    static constexpr int RSTEP = 512 / CPR;      // rows between a thread's chunks
    static constexpr int LD = D + 16;            // padded 16-bit LDS row: pitch = 8 dwords mod 32 banks, so
                                                 // transposing fragment reads of 4 rows do not conflict
};

// RMSNorm scale, ReLU, k_scale and RoPE of one 8-channel chunk.
// u = scl * relu(raw * r * w);  y[i] = u[i] cos[i] + u[i^1] sin[i]
__device__ __forceinline__ void transform8(const bf16x8& raw, float r, const float (&w)[8], float scl,
                                           const float (&cs)[8], const float (&sn)[8], float (&u)[8],
                                           float (&y)[8], unsigned& mask) {
    mask = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float n = (float)raw[i] * r * w[i];
        mask |= (n > 0.f ? 1u : 0u) << i;
        u[i] = fmaxf(n, 0.f) * scl;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = u[i] * cs[i] + u[i ^ 1] * sn[i];
}

// --------------------------------------------------------------------------
// Inverse RMS over all C channels of each token, for q and k.  One wave per
// token.
__global__ void __launch_bounds__(256) bigdn_stats_kernel(const bf16* __restrict__ qkv, float* __restrict__ rq,
                                                        float* __restrict__ rk, int ntok, int C, float norm_eps) {
    const int l = lane_id();
    const int tok = blockIdx.x * 4 + wave_id();
    if (tok >= ntok) return;
    const bf16* q = qkv + (size_t)tok * 3 * C;
    const bf16* k = q + C;
    float sq = 0.f, sk = 0.f;
    const int nv = C / 8;   // 16-byte vectors per row
    for (int c0 = 0; c0 < nv; c0 += 256) {
        // four vectors of q and of k per lane in flight before any arithmetic
        // (indices past the row repeat its last vector and are weighted 0)
        bf16x8 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int c8 = min(c0 + l + 64 * u, nv - 1);
            a[u] = __builtin_nontemporal_load((const bf16x8*)(q + 8 * c8));
            b[u] = __builtin_nontemporal_load((const bf16x8*)(k + 8 * c8));
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const float wgt = c0 + l + 64 * u < nv ? 1.f : 0.f;
            float xq = 0.f, xk = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                xq += (float)a[u][i] * (float)a[u][i];
                xk += (float)b[u][i] * (float)b[u][i];
            }
            sq += wgt * xq;
            sk += wgt * xk;
        }
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    if (l == 0) {
        rq[tok] = 1.f / sqrtf(sq / (float)C + norm_eps);
        rk[tok] = 1.f / sqrtf(sk / (float)C + norm_eps);
    }
}

// --------------------------------------------------------------------------
// Phase A: per frame, P = Kr^T diag(b) Kr, A = Kr^T diag(b) V,
// Pz = Ku^T diag(b) Ku (bf16 MFMA over token tiles, fp32 accumulate) and
// Bz = Ku^T b (fp32 VALU).  Grid: one workgroup per frame, 512 threads.
template <int D>
struct ACfg {
    static constexpr int LD = TileMap<D>::LD;
    static constexpr size_t tile = (size_t)ST * LD * 2;
    static constexpr size_t smem = 5 * tile;
};

template <int D>
__global__ void __launch_bounds__(512) bigdn_phase_a_kernel(const bf16* __restrict__ qkv, const float* __restrict__ beta,
                                                      const float* __restrict__ rk, const float* __restrict__ kw,
                                                      const float* __restrict__ cosT, const float* __restrict__ sinT,
                                                      bf16* __restrict__ Pout, float* __restrict__ Aout,
                                                      float* __restrict__ Pzout, float* __restrict__ Bzout, int F,
                                                      int S, int H, float kscale) {
    using TMp = TileMap<D>;
    constexpr int CPR = TMp::CPR, NPT = TMp::NPT, RSTEP = TMp::RSTEP, LD = TMp::LD;
    constexpr int TM = D / 64, TN = D / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    bf16* sKb = (bf16*)smem;
    bf16* sK = sKb + ST * LD;
    bf16* sV = sK + ST * LD;
    bf16* sUb = sV + ST * LD;
    bf16* sU = sUb + ST * LD;

    // frame-major order: the workgroups resident at a time share a few frames,
    // whose rope-table rows then stay in L2
    const int BH = (int)gridDim.x / F, f = (int)blockIdx.x / BH, bh = (int)blockIdx.x - f * BH;
    const int fr = bh * F + f, b = bh / H, h = bh - b * H;
    const int N = F * S, C = H * D;
    const int t = threadIdx.x, w = wave_id(), c = t % CPR, row0 = t / CPR;
    float wk[8];
    ld8(kw + h * D + 8 * c, wk);
    float bz[8];
#pragma unroll
    for (int i = 0; i < 8; i++) bz[i] = 0.f;

    bf16x8 rK[NPT], rV[NPT];
    float rcs[NPT][8], rsn[NPT][8], rb[NPT], rr[NPT];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            const int s = s0 + row0 + p * RSTEP;
            if (s < S) {
                const size_t tok = (size_t)b * N + (size_t)f * S + s;
                const bf16* base = qkv + (tok * 3 + 1) * C + h * D + 8 * c;
                rK[p] = *(const bf16x8*)base;
                rV[p] = *(const bf16x8*)(base + C);
                const size_t ro = ((size_t)f * S + s) * D + 8 * c;
                ld8(cosT + ro, rcs[p]);
                ld8(sinT + ro, rsn[p]);
                rb[p] = beta[(size_t)fr * S + s];
                rr[p] = rk[tok];
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    rK[p][i] = (bf16)0.f;
                    rV[p][i] = (bf16)0.f;
                    rcs[p][i] = 0.f;
                    rsn[p][i] = 0.f;
                }
                rb[p] = 0.f;
                rr[p] = 0.f;
            }
        }
    };

    const int m0 = (D / 4) * (w & 3), n0 = (D / 2) * (w >> 2);
    f32x4 aP[TM][TN], aA[TM][TN], aZ[TM][TN];
    zero_acc(aP);
    zero_acc(aA);
    zero_acc(aZ);
    const int ntile = (S + ST - 1) / ST;
    fetch(0);
    for (int it = 0; it < ntile; ++it) {
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            float u[8], y[8];
            unsigned m;
            transform8(rK[p], rr[p], wk, kscale, rcs[p], rsn[p], u, y, m);
            const float bb = rb[p];
            bf16x8 vkb, vk, vub, vu;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                vkb[i] = (bf16)(bb * y[i]);
                vk[i] = (bf16)y[i];
                vub[i] = (bf16)(bb * u[i]);
                vu[i] = (bf16)u[i];
                bz[i] += bb * u[i];
            }
            const int o = (row0 + p * RSTEP) * LD + 8 * c;
            *(bf16x8*)(sKb + o) = vkb;
            *(bf16x8*)(sK + o) = vk;
            *(bf16x8*)(sUb + o) = vub;
            *(bf16x8*)(sU + o) = vu;
            *(bf16x8*)(sV + o) = rV[p];
        }
        if (it + 1 < ntile) fetch((it + 1) * ST);
        lds_barrier();
        wgemm<bf16, TM, TN, ST, true, true>(aP, sKb, LD, sK, LD, m0, n0);
        wgemm<bf16, TM, TN, ST, true, true>(aA, sKb, LD, sV, LD, m0, n0);
        wgemm<bf16, TM, TN, ST, true, true>(aZ, sUb, LD, sU, LD, m0, n0);
        lds_barrier();
    }
    const size_t DD = (size_t)D * D, fo = (size_t)fr * DD;
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const size_t o = fo + (size_t)acc_row(m0, i, e) * D + acc_col(n0, j);
                Pout[o] = (bf16)aP[i][j][e];
                Aout[o] = aA[i][j][e];
                Pzout[o] = aZ[i][j][e];
            }
    // Bz: add the per-thread partials of the threads sharing chunk column c
    float* red = (float*)smem;  // [RSTEP][D]; the tiles are free after the last barrier
#pragma unroll
    for (int i = 0; i < 8; i++) red[row0 * D + 8 * c + i] = bz[i];
    lds_barrier();
    if (t < D) {
        float s = 0.f;
        for (int r = 0; r < RSTEP; r++) s += red[r * D + t];
        Bzout[(size_t)fr * D + t] = s;
    }
}

// --------------------------------------------------------------------------
// Frame scans.  Per (batch*head, direction) one workgroup of 512 threads runs
//   M <- X[u + xshift] + g_c (M - P_c M),   z <- Xz[u + xshift] + g_c (z - Pz_c z)
// over the frames in ascending (u = i, c = u) or descending (u = F-1-i,
// c = u+1) order; step 0 has no product term; X is absent (zero) beyond the
// last frame.  Each step's M (bf16) and z (fp32) are stored at frame u.
//   state recompute:  dir 0 ascending, X = A       -> Mf (inclusive)
//                     dir 1 descending, xshift 1   -> Mr (exclusive)
//   state gradients:  dir 0 descending, X = dMc    -> Tf
//                     dir 1 ascending,  X = dMc    -> Tr
// The state lives in fp32 MFMA accumulators; P and the bf16 copy of M are
// staged in LDS (P scaled by -g, so the product accumulates into M in place);
// the next step's P, X and Pz slices are loaded into registers while the
// current step computes.
struct ScanArgs {
    const bf16* P;
    const float* Pz;
    const float* decay;
    const float* X;
    const float* Xz;
    bf16* out[2];
    float* outz[2];
    int asc[2];
    int xshift[2];
    int F;
};

template <int D>
struct SCfg {
    static constexpr int LD = D + 16;
    static constexpr int NP = 512 / D;  // threads per z column
    static constexpr size_t mat = (size_t)D * LD * 2;
    static constexpr size_t smem = 2 * mat + (size_t)D * 4 + (size_t)NP * D * 4;
};

template <int D>
__global__ void __launch_bounds__(512) bigdn_scan_kernel(ScanArgs a) {
    using Cf = SCfg<D>;
    constexpr int LD = Cf::LD, NP = Cf::NP, EPP = D / NP;
    constexpr int TM = D / 64, TN = D / 32;
    constexpr int NCK = D * D / 8 / 512;  // 16-byte chunks of P per thread
    extern __shared__ __align__(16) unsigned char smem[];
    bf16* sP = (bf16*)smem;
    bf16* sM = sP + D * LD;
    float* sz = (float*)(sM + D * LD);
    float* szp = sz + D;  // [NP][D]

    const int dir = blockIdx.x & 1, bh = blockIdx.x >> 1, F = a.F;
    const bool asc = a.asc[dir] != 0;
    const int xs = a.xshift[dir];
    const int t = threadIdx.x, w = wave_id();
    const int m0 = (D / 4) * (w & 3), n0 = (D / 2) * (w >> 2);
    const size_t DD = (size_t)D * D, fr0 = (size_t)bh * F;
    const int zd = t % D, zpart = t / D;
    bf16* out = a.out[dir];
    float* outz = a.outz[dir];

    // registers of the next step
    bf16x8 nP[NCK];
    f32x4 nX[TM][TN];
    float nXz = 0.f, ng = 0.f;
    int nC = 0;
    bool nHasX = false;
    auto fetch = [&](int i) {
        const int u = asc ? i : F - 1 - i;
        const int cI = asc ? u : u + 1;
        const int xi = u + xs;
        nHasX = xi < F;
        if (nHasX) {
            const float* X = a.X + (fr0 + xi) * DD;
#pragma unroll
            for (int ii = 0; ii < TM; ii++)
#pragma unroll
                for (int j = 0; j < TN; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) nX[ii][j][e] = X[(size_t)acc_row(m0, ii, e) * D + acc_col(n0, j)];
            if (t < D) nXz = a.Xz[(fr0 + xi) * D + t];
        }
        if (i > 0) {
            const bf16* P = a.P + (fr0 + cI) * DD;
#pragma unroll
            for (int q = 0; q < NCK; q++) nP[q] = *(const bf16x8*)(P + 8 * (t + 512 * q));
            nC = cI;
            ng = a.decay[fr0 + cI];
        }
    };

    f32x4 M[TM][TN];
    int uprev = -1;
    fetch(0);
    for (int i = 0; i < F; ++i) {
        const int u = asc ? i : F - 1 - i;
        // this step's operands are in the prefetch registers; the next step's
        // are loaded once they have been consumed
        const float cXz = nXz, g = ng;
        const bool hasX = nHasX;
        if (i == 0) {
#pragma unroll
            for (int ii = 0; ii < TM; ii++)
#pragma unroll
                for (int j = 0; j < TN; j++) M[ii][j] = hasX ? nX[ii][j] : zero4();
            if (t < D) sz[t] = hasX ? cXz : 0.f;
            if (i + 1 < F) fetch(i + 1);
        } else {
            // -g P staged, so that the product accumulates into M in place
#pragma unroll
            for (int q = 0; q < NCK; q++) {
                const int idx = t + 512 * q, r = idx / (D / 8), c8 = idx % (D / 8);
                bf16x8 v;
#pragma unroll
                for (int e = 0; e < 8; e++) v[e] = (bf16)(-g * (float)nP[q][e]);
                *(bf16x8*)(sP + r * LD + 8 * c8) = v;
            }
#pragma unroll
            for (int ii = 0; ii < TM; ii++)
#pragma unroll
                for (int j = 0; j < TN; j++)
#pragma unroll
                    for (int e = 0; e < 4; e++) M[ii][j][e] = (hasX ? nX[ii][j][e] : 0.f) + g * M[ii][j][e];
            lds_barrier();  // sP, sM and sz of the previous step complete
            // store the previous step's M (bf16, from its LDS copy) with 16-byte writes
#pragma unroll
            for (int q = 0; q < NCK; q++) {
                const int idx = t + 512 * q, r = idx / (D / 8), c8 = idx % (D / 8);
                *(bf16x8*)(out + (fr0 + uprev) * DD + (size_t)r * D + 8 * c8) = *(const bf16x8*)(sM + r * LD + 8 * c8);
            }
            {   // z partial: Pz is symmetric, so column reads (coalesced over zd)
                const float* Pz = a.Pz + (fr0 + nC) * DD;
                float zs = 0.f;
#pragma unroll 8
                for (int e = 0; e < EPP; e++) zs += Pz[(size_t)(zpart * EPP + e) * D + zd] * sz[zpart * EPP + e];
                szp[zpart * D + zd] = zs;
            }
            wgemm<bf16, TM, TN, D, false, true>(M, sP, LD, sM, LD, m0, n0);  // M = X + g M - g P M_old
            if (i + 1 < F) fetch(i + 1);
            lds_barrier();  // every read of sP, sM, sz done; partials visible
            if (t < D) {
                float pz = 0.f;
#pragma unroll
                for (int p = 0; p < NP; p++) pz += szp[p * D + t];
                sz[t] = (hasX ? cXz : 0.f) + g * (sz[t] - pz);
            }
        }
        // bf16 copy of M for the next product and for the store
#pragma unroll
        for (int ii = 0; ii < TM; ii++)
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) sM[acc_row(m0, ii, e) * LD + acc_col(n0, j)] = (bf16)M[ii][j][e];
        if (t < D) outz[(fr0 + u) * D + t] = sz[t];
        uprev = u;
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NCK; q++) {
        const int idx = t + 512 * q, r = idx / (D / 8), c8 = idx % (D / 8);
        *(bf16x8*)(out + (fr0 + uprev) * DD + (size_t)r * D + 8 * c8) = *(const bf16x8*)(sM + r * LD + 8 * c8);
    }
}

// --------------------------------------------------------------------------
// Phase C (forward output, or the backward's phase C̄).  Per frame, 512
// threads.  Mc = Mf + Mr (bf16 in LDS), zc = zf + zr.  Per token tile:
//   den = Qu . zc, num = Qr Mc.
// Forward: out = num / (den + eps).
// Backward: dnum = dout / (den + eps), dden = -sum(dout num) / (den + eps)^2,
//   dQr = dnum Mc^T, dMc += Qr^T dnum, dzc += dden Qu,
//   dQn = mask * (unrope(dQr) + dden zc)  -> the q slot of dqkv (bf16),
// then dMc and dzc are stored per frame.
template <int D>
struct CCfg {
    static constexpr int LD = D + 16, LDF = D + 4;
    static constexpr int RSTEP = TileMap<D>::RSTEP;
    static constexpr size_t mat = (size_t)D * LD * 2;
    static constexpr size_t tile = (size_t)ST * LD * 2;
    static constexpr size_t oMc = 0, oQr = mat, oDn = oQr + tile, oDO = oDn + tile, oDQ = oDO + tile;
    static constexpr size_t oZ = oDQ + (size_t)ST * LDF * 4;
    static constexpr size_t oRed = oZ + (size_t)D * 4;      // [2][ST]
    static constexpr size_t oZr = oRed + (size_t)2 * ST * 4;  // [RSTEP][D]
    static constexpr size_t smem = oZr + (size_t)RSTEP * D * 4;
};

template <int D, bool BWD>
__global__ void __launch_bounds__(512) bigdn_phase_c_kernel(const bf16* __restrict__ qkv, const float* __restrict__ rq,
                                                      const float* __restrict__ qw, const float* __restrict__ cosT,
                                                      const float* __restrict__ sinT, const bf16* __restrict__ Mf,
                                                      const bf16* __restrict__ Mr, const float* __restrict__ zf,
                                                      const float* __restrict__ zr, const bf16* __restrict__ dout,
                                                      bf16* __restrict__ outp, float* __restrict__ dMc,
                                                      float* __restrict__ dzc, int F, int S, int H, float eps) {
    using Cf = CCfg<D>;
    using TMp = TileMap<D>;
    constexpr int CPR = TMp::CPR, NPT = TMp::NPT, RSTEP = TMp::RSTEP, LD = Cf::LD, LDF = Cf::LDF;
    constexpr int TN = D / 32;                    // 64 x D outputs: 16 x (D/2) per wave
    constexpr int TMd = D / 64, TNd = D / 32;     // D x D outputs
    extern __shared__ __align__(16) unsigned char smem[];
    bf16* sMc = (bf16*)(smem + Cf::oMc);
    bf16* sQr = (bf16*)(smem + Cf::oQr);
    bf16* sDn = (bf16*)(smem + Cf::oDn);
    bf16* sDO = (bf16*)(smem + Cf::oDO);
    float* sDQ = (float*)(smem + Cf::oDQ);
    float* sZ = (float*)(smem + Cf::oZ);
    float* sRed = (float*)(smem + Cf::oRed);
    float* sZr = (float*)(smem + Cf::oZr);

    // frame-major order: the workgroups resident at a time share a few frames,
    // whose rope-table rows then stay in L2
    const int BH = (int)gridDim.x / F, f = (int)blockIdx.x / BH, bh = (int)blockIdx.x - f * BH;
    const int fr = bh * F + f, b = bh / H, h = bh - b * H;
    const int N = F * S, C = H * D;
    const int t = threadIdx.x, w = wave_id(), c = t % CPR, row0 = t / CPR;
    const size_t DD = (size_t)D * D;
    for (int idx = t; idx < D * D / 8; idx += 512) {
        const int r = idx / (D / 8), c8 = idx % (D / 8);
        const bf16x8 x = *(const bf16x8*)(Mf + (size_t)fr * DD + (size_t)r * D + 8 * c8);
        const bf16x8 y = *(const bf16x8*)(Mr + (size_t)fr * DD + (size_t)r * D + 8 * c8);
        bf16x8 s;
#pragma unroll
        for (int i = 0; i < 8; i++) s[i] = (bf16)((float)x[i] + (float)y[i]);
        *(bf16x8*)(sMc + r * LD + 8 * c8) = s;
    }
    if (t < D) sZ[t] = zf[(size_t)fr * D + t] + zr[(size_t)fr * D + t];
    float wq[8], zc[8];
    ld8(qw + h * D + 8 * c, wq);
#pragma unroll
    for (int i = 0; i < 8; i++) zc[i] = zf[(size_t)fr * D + 8 * c + i] + zr[(size_t)fr * D + 8 * c + i];
    float dz[8];
#pragma unroll
    for (int i = 0; i < 8; i++) dz[i] = 0.f;

    const int m0 = 16 * (w & 3), n0 = (D / 2) * (w >> 2);
    const int m0d = (D / 4) * (w & 3), n0d = (D / 2) * (w >> 2);
    f32x4 accM[TMd][TNd];
    if constexpr (BWD) zero_acc(accM);

    // the next tile's q and dout chunks are loaded into registers while the
    // current tile is computed
    bf16x8 pQ[NPT], pD[NPT];
    float pR[NPT];
    auto fetch = [&](int s0n) {
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            const int s = s0n + row0 + p * RSTEP;
            if (s < S) {
                const size_t tok = (size_t)b * N + (size_t)f * S + s;
                pQ[p] = *(const bf16x8*)(qkv + tok * 3 * C + h * D + 8 * c);
                pR[p] = rq[tok];
                if constexpr (BWD) pD[p] = *(const bf16x8*)(dout + (tok * H + h) * D + 8 * c);
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    pQ[p][i] = (bf16)0.f;
                    if constexpr (BWD) pD[p][i] = (bf16)0.f;
                }
                pR[p] = 0.f;
            }
        }
    };
    const int ntile = (S + ST - 1) / ST;
    fetch(0);
    for (int it = 0; it < ntile; ++it) {
        const int s0 = it * ST;
        float u[NPT][8], cs[NPT][8], sn[NPT][8], inv[NPT];
        unsigned msk[NPT];
        bool ok[NPT];
        bf16x8 rD[NPT];
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            const int row = row0 + p * RSTEP, s = s0 + row;
            ok[p] = s < S;
            const bf16x8 raw = pQ[p];
            const float r = pR[p];
            if constexpr (BWD) rD[p] = pD[p];
            {   // rows past the frame read its last row (no branch around the loads)
                const size_t ro = ((size_t)f * S + min(s, S - 1)) * D + 8 * c;
                float tc[8], ts[8];
                ld8(cosT + ro, tc);
                ld8(sinT + ro, ts);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    cs[p][i] = ok[p] ? tc[i] : 0.f;
                    sn[p][i] = ok[p] ? ts[i] : 0.f;
                }
            }
            float y[8];
            transform8(raw, r, wq, 1.f, cs[p], sn[p], u[p], y, msk[p]);
            float dp = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) dp += u[p][i] * zc[i];
            const float den = group_sum<CPR>(dp);
            inv[p] = 1.f / (den + eps);
            bf16x8 vy;
#pragma unroll
            for (int i = 0; i < 8; i++) vy[i] = (bf16)y[i];
            *(bf16x8*)(sQr + row * LD + 8 * c) = vy;
            if constexpr (BWD) {
                bf16x8 vd;
#pragma unroll
                for (int i = 0; i < 8; i++) vd[i] = (bf16)((float)rD[p][i] * inv[p]);
                *(bf16x8*)(sDn + row * LD + 8 * c) = vd;
                *(bf16x8*)(sDO + row * LD + 8 * c) = rD[p];
            } else {
                if (c == 0) sRed[row] = inv[p];
            }
        }
        if (it + 1 < ntile) fetch((it + 1) * ST);
        lds_barrier();
        f32x4 accN[1][TN];
        zero_acc(accN);
        wgemm<bf16, 1, TN, D, false, true>(accN, sQr, LD, sMc, LD, m0, n0);
        if constexpr (!BWD) {
            bf16* sO = sDO;
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = acc_row(m0, 0, e);
                    sO[r * LD + acc_col(n0, j)] = (bf16)(accN[0][j][e] * sRed[r]);
                }
            lds_barrier();
#pragma unroll
            for (int p = 0; p < NPT; p++) {
                if (!ok[p]) continue;
                const int row = row0 + p * RSTEP;
                const size_t tok = (size_t)b * N + (size_t)f * S + s0 + row;
                *(bf16x8*)(outp + (tok * H + h) * D + 8 * c) = *(const bf16x8*)(sO + row * LD + 8 * c);
            }
            lds_barrier();
        } else {
            // dden partial sums: sum over columns of dout * num
            float dd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    dd[e] += (float)sDO[acc_row(m0, 0, e) * LD + acc_col(n0, j)] * accN[0][j][e];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                dd[e] = group_sum<16>(dd[e]);
                if ((lane_id() & 15) == 0) sRed[(w >> 2) * ST + acc_row(m0, 0, e)] = dd[e];
            }
            f32x4 accQ[1][TN];
            zero_acc(accQ);
            wgemm<bf16, 1, TN, D, false, false>(accQ, sDn, LD, sMc, LD, m0, n0);
            wgemm<bf16, TMd, TNd, ST, true, true>(accM, sQr, LD, sDn, LD, m0d, n0d);
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) sDQ[acc_row(m0, 0, e) * LDF + acc_col(n0, j)] = accQ[0][j][e];
            lds_barrier();
#pragma unroll
            for (int p = 0; p < NPT; p++) {
                if (!ok[p]) continue;
                const int row = row0 + p * RSTEP;
                const float dden = -(sRed[row] + sRed[ST + row]) * inv[p] * inv[p];
                float dq[8];
                ld8(sDQ + row * LDF + 8 * c, dq);
                bf16x8 o;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float v = dq[i] * cs[p][i] + dq[i ^ 1] * sn[p][i ^ 1] + dden * zc[i];
                    o[i] = (bf16)(((msk[p] >> i) & 1u) ? v : 0.f);
                    dz[i] += dden * u[p][i];
                }
                const size_t tok = (size_t)b * N + (size_t)f * S + s0 + row;
                *(bf16x8*)(outp + tok * 3 * C + h * D + 8 * c) = o;
            }
            lds_barrier();
        }
    }
    if constexpr (BWD) {
        const size_t fo = (size_t)fr * DD;
#pragma unroll
        for (int i = 0; i < TMd; i++)
#pragma unroll
            for (int j = 0; j < TNd; j++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    dMc[fo + (size_t)acc_row(m0d, i, e) * D + acc_col(n0d, j)] = accM[i][j][e];
#pragma unroll
        for (int i = 0; i < 8; i++) sZr[row0 * D + 8 * c + i] = dz[i];
        lds_barrier();
        if (t < D) {
            float s = 0.f;
            for (int r = 0; r < RSTEP; r++) s += sZr[r * D + t];
            dzc[(size_t)fr * D + t] = s;
        }
    }
}

// --------------------------------------------------------------------------
// Combine of both scan directions and phase Ā (key-value and normaliser
// streams).  Per frame f, 512 threads.
// Stage 1:  dA = Tf[f] + Tr[f-1]
//           dPs = dP + dP^T = -g (Tf Mp^T + Mp Tf^T + Tr Mr^T + Mr Tr^T)
//           dg = <Tf, Mp - P Mp> + <Tr, Mr - P Mr> + (the same for z)
//   with Mp = Mf[f-1], Mr = Mr[f], Tr = Tr[f-1] (absent at f = 0).
// Stage 2, per token tile:  acc1 = Kr dPs + V dA^T,  acc2 = Kr dA,
//   dKr = b acc1, dV = b acc2, dbeta = (rowsum(acc1 Kr) + rowsum(acc2 V)) / 2
//   + the normaliser terms, which are rank-4 in Ku:
//   Ku dPzs = -g [(Ku.tzf) zp + (Ku.zp) tzf + (Ku.tzr) zr + (Ku.zr) tzr],
//   dKu_z = b (Ku dPzs + dBz), dbeta_z = -g (a1 a2 + a3 a4) + Ku.dBz;
//   dKn = k_scale mask (unrope(dKr) + dKu_z) -> the k slot, dV -> the v slot.
template <int D>
struct BCfg {
    static constexpr int LD = D + 16;
    static constexpr int NP = 512 / D;
    static constexpr size_t mat = (size_t)D * LD * 2;
    static constexpr size_t tile = (size_t)ST * LD * 2;
    static constexpr size_t r0 = 2 * mat > 4 * tile ? 2 * mat : 4 * tile;
    static constexpr size_t oA0 = 0, oA1 = mat;                             // stage 1
    static constexpr size_t oK = 0, oV = tile, oDK = 2 * tile, oDV = 3 * tile;  // stage 2
    static constexpr size_t oP = r0;                                       // P, then dPs
    static constexpr size_t oDA = oP + mat;
    static constexpr size_t oVec = oDA + mat;                              // 5 x [D] fp32
    static constexpr size_t oZp = oVec + (size_t)5 * D * 4;                // 2 x [NP][D]
    static constexpr size_t oRed = oZp + (size_t)2 * NP * D * 4;           // [2][ST]
    static constexpr size_t oBeta = oRed + (size_t)2 * ST * 4;             // [ST]
    static constexpr size_t oG = oBeta + (size_t)ST * 4;                   // [8]
    static constexpr size_t smem = oG + 8 * 4;
};

template <int D>
__global__ void __launch_bounds__(512) bigdn_abar_kernel(const bf16* __restrict__ qkv, const float* __restrict__ beta,
                                                   const float* __restrict__ decay, const float* __restrict__ rk,
                                                   const float* __restrict__ kw, const float* __restrict__ cosT,
                                                   const float* __restrict__ sinT, const bf16* __restrict__ P,
                                                   const float* __restrict__ Pz, const bf16* __restrict__ Mf,
                                                   const bf16* __restrict__ Mr, const float* __restrict__ zf,
                                                   const float* __restrict__ zr, const bf16* __restrict__ Tf,
                                                   const bf16* __restrict__ Tr, const float* __restrict__ tzf,
                                                   const float* __restrict__ tzr, bf16* __restrict__ dqkv,
                                                   float* __restrict__ dbeta, float* __restrict__ ddecay, int F,
                                                   int S, int H, float kscale) {
    using Cf = BCfg<D>;
    using TMp = TileMap<D>;
    constexpr int CPR = TMp::CPR, NPT = TMp::NPT, RSTEP = TMp::RSTEP, LD = Cf::LD, NP = Cf::NP, EPP = D / NP;
    constexpr int TN = D / 32;
    constexpr int TMd = D / 64, TNd = D / 32;
    constexpr int NCK = D * D / 8 / 512;
    extern __shared__ __align__(16) unsigned char smem[];
    bf16* sA0 = (bf16*)(smem + Cf::oA0);
    bf16* sA1 = (bf16*)(smem + Cf::oA1);
    bf16* sK = (bf16*)(smem + Cf::oK);
    bf16* sV = (bf16*)(smem + Cf::oV);
    bf16* sDK = (bf16*)(smem + Cf::oDK);
    bf16* sDV = (bf16*)(smem + Cf::oDV);
    bf16* sP = (bf16*)(smem + Cf::oP);
    bf16* sDP = sP;
    bf16* sDA = (bf16*)(smem + Cf::oDA);
    float* sTzf = (float*)(smem + Cf::oVec);
    float* sZp = sTzf + D;
    float* sTzr = sZp + D;
    float* sZr = sTzr + D;
    float* sDBz = sZr + D;
    float* sPz1 = (float*)(smem + Cf::oZp);
    float* sPz2 = sPz1 + NP * D;
    float* sRed = (float*)(smem + Cf::oRed);
    float* sBeta = (float*)(smem + Cf::oBeta);
    float* sG = (float*)(smem + Cf::oG);

    // frame-major order: the workgroups resident at a time share a few frames,
    // whose rope-table rows then stay in L2
    const int BH = (int)gridDim.x / F, f = (int)blockIdx.x / BH, bh = (int)blockIdx.x - f * BH;
    const int fr = bh * F + f, b = bh / H, h = bh - b * H;
    const int N = F * S, C = H * D;
    const int t = threadIdx.x, w = wave_id(), c = t % CPR, row0 = t / CPR;
    const size_t DD = (size_t)D * D, fo = (size_t)fr * DD;
    const bool hasPrev = f > 0;
    const float g = decay[fr];

    // ---- stage 1
#pragma unroll
    for (int q = 0; q < NCK; q++) {
        const int idx = t + 512 * q, r = idx / (D / 8), c8 = idx % (D / 8);
        const size_t o = (size_t)r * D + 8 * c8;
        *(bf16x8*)(sA0 + r * LD + 8 * c8) = *(const bf16x8*)(Tf + fo + o);
        *(bf16x8*)(sP + r * LD + 8 * c8) = *(const bf16x8*)(P + fo + o);
        if (hasPrev) *(bf16x8*)(sA1 + r * LD + 8 * c8) = *(const bf16x8*)(Mf + fo - DD + o);
    }
    if (t < D) {
        sTzf[t] = tzf[(size_t)fr * D + t];
        sZp[t] = hasPrev ? zf[(size_t)(fr - 1) * D + t] : 0.f;
        sTzr[t] = hasPrev ? tzr[(size_t)(fr - 1) * D + t] : 0.f;
        sZr[t] = zr[(size_t)fr * D + t];
    }
    lds_barrier();
    const int m0d = (D / 4) * (w & 3), n0d = (D / 2) * (w >> 2);
    float dg = 0.f;
    // z products: Pz zp and Pz zr (Pz symmetric: column access)
    {
        const int zd = t % D, zpart = t / D;
        const float* pz = Pz + fo;
        float s1 = 0.f, s2 = 0.f;
#pragma unroll 8
        for (int e = 0; e < EPP; e++) {
            const int ee = zpart * EPP + e;
            const float x = pz[(size_t)ee * D + zd];
            s1 += x * sZp[ee];
            s2 += x * sZr[ee];
        }
        sPz1[zpart * D + zd] = s1;
        sPz2[zpart * D + zd] = s2;
    }
    // dg term <T, M - P M> of the pair (T, M) staged in sA0, sA1
    auto dg_term = [&]() {
        f32x4 accT[TMd][TNd];
        zero_acc(accT);
        wgemm<bf16, TMd, TNd, D, false, true>(accT, sP, LD, sA1, LD, m0d, n0d);
#pragma unroll
        for (int i = 0; i < TMd; i++)
#pragma unroll
            for (int j = 0; j < TNd; j++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int o = acc_row(m0d, i, e) * LD + acc_col(n0d, j);
                    dg += (float)sA0[o] * ((float)sA1[o] - accT[i][j][e]);
                }
    };
    f32x4 accS[TMd][TNd];
    zero_acc(accS);
    if (hasPrev) {
        dg_term();
        wgemm<bf16, TMd, TNd, D, false, false>(accS, sA0, LD, sA1, LD, m0d, n0d);  // Tf Mp^T
        wgemm<bf16, TMd, TNd, D, false, false>(accS, sA1, LD, sA0, LD, m0d, n0d);  // Mp Tf^T
    }
    lds_barrier();  // stage-1 reads of sA0/sA1 done; z partials visible
    // dA = Tf[f] + Tr[f-1]; each thread re-reads the Tf chunks it staged itself
#pragma unroll
    for (int q = 0; q < NCK; q++) {
        const int idx = t + 512 * q, r = idx / (D / 8), c8 = idx % (D / 8);
        const size_t o = (size_t)r * D + 8 * c8;
        const bf16x8 tf = *(const bf16x8*)(sA0 + r * LD + 8 * c8);
        if (hasPrev) {
            const bf16x8 tr = *(const bf16x8*)(Tr + fo - DD + o);
            *(bf16x8*)(sA0 + r * LD + 8 * c8) = tr;
            *(bf16x8*)(sA1 + r * LD + 8 * c8) = *(const bf16x8*)(Mr + fo + o);
            bf16x8 sm;
#pragma unroll
            for (int i = 0; i < 8; i++) sm[i] = (bf16)((float)tf[i] + (float)tr[i]);
            *(bf16x8*)(sDA + r * LD + 8 * c8) = sm;
        } else {
            *(bf16x8*)(sDA + r * LD + 8 * c8) = tf;
        }
    }
    if (t < D) {
        float p1 = 0.f, p2 = 0.f;
#pragma unroll
        for (int p = 0; p < NP; p++) p1 += sPz1[p * D + t], p2 += sPz2[p * D + t];
        dg += sTzf[t] * (sZp[t] - p1) + sTzr[t] * (sZr[t] - p2);
        sDBz[t] = sTzf[t] + sTzr[t];
    }
    lds_barrier();
    if (hasPrev) {
        dg_term();
        wgemm<bf16, TMd, TNd, D, false, false>(accS, sA0, LD, sA1, LD, m0d, n0d);  // Tr Mr^T
        wgemm<bf16, TMd, TNd, D, false, false>(accS, sA1, LD, sA0, LD, m0d, n0d);  // Mr Tr^T
    }
    dg = wave_sum(dg);
    if (lane_id() == 0) sG[w] = dg;
    lds_barrier();  // every read of sP, sA0, sA1 done
#pragma unroll
    for (int i = 0; i < TMd; i++)
#pragma unroll
        for (int j = 0; j < TNd; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) sDP[acc_row(m0d, i, e) * LD + acc_col(n0d, j)] = (bf16)(-g * accS[i][j][e]);
    if (t == 0) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) s += sG[i];
        ddecay[fr] = s;
    }
    // (stage 2 starts with its own barrier before the first product)

    // ---- stage 2
    float wk[8];
    ld8(kw + h * D + 8 * c, wk);
    const int m0 = 16 * (w & 3), n0 = (D / 2) * (w >> 2);
    const int ntile = (S + ST - 1) / ST;
    const float* vTzf = sTzf + 8 * c;
    const float* vZp = sZp + 8 * c;
    const float* vTzr = sTzr + 8 * c;
    const float* vZr = sZr + 8 * c;
    const float* vDBz = sDBz + 8 * c;
    bf16x8 pK[NPT], pV[NPT];
    float pR[NPT], pB[NPT];
    auto fetch = [&](int s0n) {
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            const int s = s0n + row0 + p * RSTEP;
            if (s < S) {
                const size_t tok = (size_t)b * N + (size_t)f * S + s;
                const bf16* base = qkv + (tok * 3 + 1) * C + h * D + 8 * c;
                pK[p] = *(const bf16x8*)base;
                pV[p] = *(const bf16x8*)(base + C);
                pR[p] = rk[tok];
                pB[p] = beta[(size_t)fr * S + s];
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    pK[p][i] = (bf16)0.f;
                    pV[p][i] = (bf16)0.f;
                }
                pR[p] = 0.f;
                pB[p] = 0.f;
            }
        }
    };
    fetch(0);
    for (int it = 0; it < ntile; ++it) {
        const int s0 = it * ST;
        // per row: the four Ku dot products of the rank-4 normaliser term and
        // dbeta_z; the channel terms are rebuilt after the products
        float az[NPT][4], dbz[NPT], bbr[NPT];
        unsigned msk[NPT];
        bool ok[NPT];
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            const int row = row0 + p * RSTEP, s = s0 + row;
            ok[p] = s < S;
            const bf16x8 raw = pK[p], rv = pV[p];
            const float r = pR[p], bb = pB[p];
            float cs[8], sn[8];
            {   // rows past the frame read its last row (no branch around the loads)
                const size_t ro = ((size_t)f * S + min(s, S - 1)) * D + 8 * c;
                float tc[8], ts[8];
                ld8(cosT + ro, tc);
                ld8(sinT + ro, ts);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    cs[i] = ok[p] ? tc[i] : 0.f;
                    sn[i] = ok[p] ? ts[i] : 0.f;
                }
            }
            float u[8], y[8];
            transform8(raw, r, wk, kscale, cs, sn, u, y, msk[p]);
            float a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f, a5 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                a1 += u[i] * vTzf[i];
                a2 += u[i] * vZp[i];
                a3 += u[i] * vTzr[i];
                a4 += u[i] * vZr[i];
                a5 += u[i] * vDBz[i];
            }
            az[p][0] = group_sum<CPR>(a1);
            az[p][1] = group_sum<CPR>(a2);
            az[p][2] = group_sum<CPR>(a3);
            az[p][3] = group_sum<CPR>(a4);
            a5 = group_sum<CPR>(a5);
            dbz[p] = -g * (az[p][0] * az[p][1] + az[p][2] * az[p][3]) + a5;
            bbr[p] = bb;
            bf16x8 vy;
#pragma unroll
            for (int i = 0; i < 8; i++) vy[i] = (bf16)y[i];
            *(bf16x8*)(sK + row * LD + 8 * c) = vy;
            *(bf16x8*)(sV + row * LD + 8 * c) = rv;
            if (c == 0) sBeta[row] = bb;
        }
        if (it + 1 < ntile) fetch((it + 1) * ST);
        lds_barrier();
        f32x4 acc1[1][TN], acc2[1][TN];
        zero_acc(acc1);
        zero_acc(acc2);
        wgemm<bf16, 1, TN, D, false, false>(acc1, sK, LD, sDP, LD, m0, n0);
        wgemm<bf16, 1, TN, D, false, false>(acc1, sV, LD, sDA, LD, m0, n0);
        wgemm<bf16, 1, TN, D, false, true>(acc2, sK, LD, sDA, LD, m0, n0);
        float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int o = acc_row(m0, 0, e) * LD + acc_col(n0, j);
                db[e] += acc1[0][j][e] * (float)sK[o] + acc2[0][j][e] * (float)sV[o];
            }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = acc_row(m0, 0, e);
            db[e] = group_sum<16>(db[e]);
            if ((lane_id() & 15) == 0) sRed[(w >> 2) * ST + r] = db[e];
            const float bb = sBeta[r];
#pragma unroll
            for (int j = 0; j < TN; j++) {
                sDK[r * LD + acc_col(n0, j)] = (bf16)(bb * acc1[0][j][e]);
                sDV[r * LD + acc_col(n0, j)] = (bf16)(bb * acc2[0][j][e]);
            }
        }
        lds_barrier();
#pragma unroll
        for (int p = 0; p < NPT; p++) {
            if (!ok[p]) continue;
            const int row = row0 + p * RSTEP;
            const size_t tok = (size_t)b * N + (size_t)f * S + s0 + row;
            float cs[8], sn[8];
            const size_t ro = ((size_t)f * S + s0 + row) * D + 8 * c;
            ld8(cosT + ro, cs);
            ld8(sinT + ro, sn);
            const bf16x8 dk = *(const bf16x8*)(sDK + row * LD + 8 * c);
            bf16x8 o;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float dkz = bbr[p] * (-g * (az[p][0] * vZp[i] + az[p][1] * vTzf[i] + az[p][2] * vZr[i] +
                                                  az[p][3] * vTzr[i]) + vDBz[i]);
                const float v = (float)dk[i] * cs[i] + (float)dk[i ^ 1] * sn[i ^ 1] + dkz;
                o[i] = (bf16)(((msk[p] >> i) & 1u) ? v * kscale : 0.f);
            }
            bf16* base = dqkv + (tok * 3 + 1) * C + h * D + 8 * c;
            *(bf16x8*)base = o;
            *(bf16x8*)(base + C) = *(const bf16x8*)(sDV + row * LD + 8 * c);
            if (c == 0) dbeta[(size_t)fr * S + s0 + row] = 0.5f * (sRed[row] + sRed[ST + row]) + dbz[p];
        }
        lds_barrier();
    }
}

// --------------------------------------------------------------------------
// RMSNorm VJP over all C channels of a token, in place on the q and k slots
// of dqkv (which hold dQn and dKn):  dx = r w dy - r^3/C x sum(w dy x);
// per-block partial sums of dy x r for the norm weights, accumulated in each
// wave's own LDS row (lane-private addresses, so no synchronisation until the
// end; in registers they would cost 8·NCH VGPRs per lane and a wave per SIMD).
// One wave per (token, slot).
template <int NCH>
__global__ void __launch_bounds__(256) bigdn_rms_bwd_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ dqkv,
                                                            const float* __restrict__ rq, const float* __restrict__ rk,
                                                            const float* __restrict__ qw, const float* __restrict__ kw,
                                                            float* __restrict__ wpart, int ntok, int C) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* red = (float*)smem;  // [4][C]
    const int l = lane_id(), w = wave_id(), nc8 = C / 8;
    // work unit u = 2 * token + slot (0: q, 1: k); the unit stride is a multiple
    // of 4, so each wave keeps one slot and accumulates one weight gradient
    const int sl = w & 1;
    const float* wt = sl ? kw : qw;
    const float* rr = sl ? rk : rq;
    float* acc = red + w * C;   // this wave's partials; lane l owns channels 8 (l + 64 ch) .. +7
#pragma unroll
    for (int ch = 0; ch < NCH; ch++) {
        const int c8 = l + 64 * ch;
        if (c8 < nc8) {
            *(f32x4*)(acc + 8 * c8) = f32x4{0.f, 0.f, 0.f, 0.f};
            *(f32x4*)(acc + 8 * c8 + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const long nunit = 2L * ntok, ustep = (long)gridDim.x * 4;
    // the next unit's rows are loaded before the current one is reduced
    bf16x8 nx[NCH], ng[NCH];
    auto fetch = [&](long u) {
        const long tok = u >> 1;
        const bf16* x = qkv + (size_t)tok * 3 * C + (size_t)sl * C;
        const bf16* dx = dqkv + (size_t)tok * 3 * C + (size_t)sl * C;
#pragma unroll
        for (int ch = 0; ch < NCH; ch++) {
            const int c8 = l + 64 * ch;
            if (c8 < nc8) {
                nx[ch] = __builtin_nontemporal_load((const bf16x8*)(x + 8 * c8));
                ng[ch] = __builtin_nontemporal_load((const bf16x8*)(dx + 8 * c8));
            }
        }
    };
    long u = (long)blockIdx.x * 4 + w;
    if (u < nunit) fetch(u);
    for (; u < nunit; u += ustep) {
        const long tok = u >> 1;
        bf16* dx = dqkv + (size_t)tok * 3 * C + (size_t)sl * C;
        bf16x8 xr[NCH], gr[NCH];
#pragma unroll
        for (int ch = 0; ch < NCH; ch++) xr[ch] = nx[ch], gr[ch] = ng[ch];
        if (u + ustep < nunit) fetch(u + ustep);
        const float r = rr[tok];
        float corr = 0.f;
#pragma unroll
        for (int ch = 0; ch < NCH; ch++) {
            const int c8 = l + 64 * ch;
            if (c8 < nc8) {
                float w8[8];
                ld8(wt + 8 * c8, w8);
#pragma unroll
                for (int i = 0; i < 8; i++) corr += w8[i] * (float)gr[ch][i] * (float)xr[ch][i];
            }
        }
        corr = wave_sum(corr);
        const float k3 = r * r * r / (float)C * corr;
#pragma unroll
        for (int ch = 0; ch < NCH; ch++) {
            const int c8 = l + 64 * ch;
            if (c8 < nc8) {
                float w8[8], a8[8];
                ld8(wt + 8 * c8, w8);
                ld8(acc + 8 * c8, a8);
                bf16x8 o;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float xa = (float)xr[ch][i], ga = (float)gr[ch][i];
                    o[i] = (bf16)(r * w8[i] * ga - k3 * xa);
                    a8[i] += ga * xa * r;
                }
                *(f32x4*)(acc + 8 * c8) = f32x4{a8[0], a8[1], a8[2], a8[3]};
                *(f32x4*)(acc + 8 * c8 + 4) = f32x4{a8[4], a8[5], a8[6], a8[7]};
                *(bf16x8*)(dx + 8 * c8) = o;
            }
        }
    }
    __syncthreads();
    // waves 0, 2 hold q partials, waves 1, 3 k partials
    for (int i = threadIdx.x; i < 2 * C; i += 256) {
        const int slot = i / C, c = i - slot * C;
        wpart[(size_t)blockIdx.x * 2 * C + i] = red[slot * C + c] + red[(2 + slot) * C + c];
    }
}

// Sum of the per-block norm-weight partials: 64 channels per workgroup, the
// partial rows split over four thread rows (loads unrolled eight deep), then
// added in a fixed order through LDS.
__global__ void __launch_bounds__(256) bigdn_wsum_kernel(const float* __restrict__ wpart, float* __restrict__ dqw,
                                                         float* __restrict__ dkw, int nblk, int C) {
    __shared__ float part[4][64];
    const int t = threadIdx.x, cl = t & 63, rg = t >> 6;
    const int i = blockIdx.x * 64 + cl;
    float s = 0.f;
    if (i < 2 * C) {
#pragma unroll 8
        for (int k = rg; k < nblk; k += 4) s += wpart[(size_t)k * 2 * C + i];
    }
    part[rg][cl] = s;
    __syncthreads();
    if (rg == 0 && i < 2 * C) {
        const float v = part[0][cl] + part[1][cl] + part[2][cl] + part[3][cl];
        if (i < C) dqw[i] = v;
        else dkw[i - C] = v;
    }
}

// --------------------------------------------------------------------------
// Host side
static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Persistent RMSNorm-VJP workgroups: three per CU (158 VGPRs per lane, 32 KB
// of LDS each) on 256 CUs, so the grid is resident in one round.
static int rms_blocks(const Dims& d) {
    const long ntok = (long)d.B * d.F * d.S;
    const long nb = (ntok + 3) / 4;
    return (int)(nb < 768 ? nb : 768);
}

size_t plan(const Dims& d, bool bwd, char* base, Ws* w) {
    const size_t ntok = (size_t)d.B * d.F * d.S, NF = (size_t)d.B * d.H * d.F, DD = (size_t)d.D * d.D;
    const size_t C = (size_t)d.H * d.D;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + o : nullptr;
        o += al(bytes);
        return p;
    };
    Ws x{};
    x.rq = (float*)take(ntok * 4);
    x.rk = (float*)take(ntok * 4);
    x.P = take(NF * DD * 2);
    x.A = (float*)take(NF * DD * 4);
    x.Pz = (float*)take(NF * DD * 4);
    x.Bz = (float*)take(NF * d.D * 4);
    x.Mf = take(NF * DD * 2);
    x.Mr = take(NF * DD * 2);
    x.zf = (float*)take(NF * d.D * 4);
    x.zr = (float*)take(NF * d.D * 4);
    if (bwd) {
        x.dMc = (float*)take(NF * DD * 4);
        x.dzc = (float*)take(NF * d.D * 4);
        x.Tf = take(NF * DD * 2);
        x.Tr = take(NF * DD * 2);
        x.tzf = (float*)take(NF * d.D * 4);
        x.tzr = (float*)take(NF * d.D * 4);
        x.nblk = rms_blocks(d);
        x.wpart = (float*)take((size_t)x.nblk * 2 * C * 4);
    }
    if (w) *w = x;
    return o;
}

template <class K>
static hipError_t set_smem(K kern, size_t bytes) {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int D>
static hipError_t run_phase_a(const Dims& d, const Inputs& in, const Ws& w, hipStream_t s) {
    auto k = bigdn_phase_a_kernel<D>;
    if (set_smem(k, ACfg<D>::smem) != hipSuccess) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k, dim3(d.B * d.H * d.F), dim3(512), ACfg<D>::smem, s, (const bf16*)in.qkv, in.beta, w.rk,
                       in.kw, in.cos, in.sin, (bf16*)w.P, w.A, w.Pz, w.Bz, d.F, d.S, d.H, d.k_scale);
    return hipGetLastError();
}

template <int D>
static hipError_t run_scan(const Dims& d, const ScanArgs& a, hipStream_t s) {
    auto k = bigdn_scan_kernel<D>;
    if (set_smem(k, SCfg<D>::smem) != hipSuccess) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k, dim3(2 * d.B * d.H), dim3(512), SCfg<D>::smem, s, a);
    return hipGetLastError();
}

template <int D, bool BWD>
static hipError_t run_phase_c(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s) {
    auto k = bigdn_phase_c_kernel<D, BWD>;
    if (set_smem(k, CCfg<D>::smem) != hipSuccess) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k, dim3(d.B * d.H * d.F), dim3(512), CCfg<D>::smem, s, (const bf16*)in.qkv, w.rq, in.qw,
                       in.cos, in.sin, (const bf16*)w.Mf, (const bf16*)w.Mr, w.zf, w.zr, (const bf16*)in.dout,
                       (bf16*)(BWD ? out.dqkv : out.out), w.dMc, w.dzc, d.F, d.S, d.H, d.eps);
    return hipGetLastError();
}

template <int D>
static hipError_t run_abar(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s) {
    auto k = bigdn_abar_kernel<D>;
    if (set_smem(k, BCfg<D>::smem) != hipSuccess) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k, dim3(d.B * d.H * d.F), dim3(512), BCfg<D>::smem, s, (const bf16*)in.qkv, in.beta, in.decay,
                       w.rk, in.kw, in.cos, in.sin, (const bf16*)w.P, w.Pz, (const bf16*)w.Mf, (const bf16*)w.Mr,
                       w.zf, w.zr, (const bf16*)w.Tf, (const bf16*)w.Tr, w.tzf, w.tzr, (bf16*)out.dqkv, out.dbeta,
                       out.ddecay, d.F, d.S, d.H, d.k_scale);
    return hipGetLastError();
}

template <int NCH>
static hipError_t run_rms_bwd(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s) {
    const int C = d.H * d.D, ntok = d.B * d.F * d.S;
    const size_t sm = (size_t)4 * C * 4;
    auto k = bigdn_rms_bwd_kernel<NCH>;
    if (set_smem(k, sm) != hipSuccess) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k, dim3(w.nblk), dim3(256), sm, s, (const bf16*)in.qkv, (bf16*)out.dqkv, w.rq, w.rk, in.qw,
                       in.kw, w.wpart, ntok, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bigdn_wsum_kernel, dim3((2 * C + 63) / 64), dim3(256), 0, s, w.wpart, out.dqw, out.dkw, w.nblk, C);
    return hipGetLastError();
}

static hipError_t mark(hipEvent_t* ev, int i, hipStream_t s) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; }

#define BIGDN_TRY(x)                         \
    do {                                     \
        hipError_t e_ = (x);                 \
        if (e_ != hipSuccess) return e_;     \
    } while (0)

// stats, phase A and the state scans (shared by both directions of the layer)
template <int D>
static hipError_t run_states(const Dims& d, const Inputs& in, const Ws& w, hipStream_t s, hipEvent_t* ev) {
    const int ntok = d.B * d.F * d.S, C = d.H * d.D;
    BIGDN_TRY(mark(ev, 0, s));
    hipLaunchKernelGGL(bigdn_stats_kernel, dim3((ntok + 3) / 4), dim3(256), 0, s, (const bf16*)in.qkv, w.rq, w.rk, ntok,
                       C, d.norm_eps);
    BIGDN_TRY(hipGetLastError());
    BIGDN_TRY(mark(ev, 1, s));
    BIGDN_TRY(run_phase_a<D>(d, in, w, s));
    BIGDN_TRY(mark(ev, 2, s));
    ScanArgs a{};
    a.P = (const bf16*)w.P;
    a.Pz = w.Pz;
    a.decay = in.decay;
    a.X = w.A;
    a.Xz = w.Bz;
    a.out[0] = (bf16*)w.Mf;
    a.out[1] = (bf16*)w.Mr;
    a.outz[0] = w.zf;
    a.outz[1] = w.zr;
    a.asc[0] = 1;
    a.asc[1] = 0;
    a.xshift[0] = 0;
    a.xshift[1] = 1;
    a.F = d.F;
    BIGDN_TRY(run_scan<D>(d, a, s));
    return mark(ev, 3, s);
}

template <int D>
static hipError_t fwd_go(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s,
                         hipEvent_t* ev) {
    BIGDN_TRY(run_states<D>(d, in, w, s, ev));
    BIGDN_TRY((run_phase_c<D, false>(d, in, out, w, s)));
    return mark(ev, 4, s);
}

template <int D>
static hipError_t bwd_go(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s,
                         hipEvent_t* ev) {
    BIGDN_TRY(run_states<D>(d, in, w, s, ev));
    BIGDN_TRY((run_phase_c<D, true>(d, in, out, w, s)));
    BIGDN_TRY(mark(ev, 4, s));
    ScanArgs a{};
    a.P = (const bf16*)w.P;
    a.Pz = w.Pz;
    a.decay = in.decay;
    a.X = w.dMc;
    a.Xz = w.dzc;
    a.out[0] = (bf16*)w.Tf;
    a.out[1] = (bf16*)w.Tr;
    a.outz[0] = w.tzf;
    a.outz[1] = w.tzr;
    a.asc[0] = 0;
    a.asc[1] = 1;
    a.xshift[0] = 0;
    a.xshift[1] = 0;
    a.F = d.F;
    BIGDN_TRY(run_scan<D>(d, a, s));
    BIGDN_TRY(mark(ev, 5, s));
    BIGDN_TRY(run_abar<D>(d, in, out, w, s));
    BIGDN_TRY(mark(ev, 6, s));
    const int nch = (d.H * d.D / 8 + 63) / 64;
    if (nch <= 1) BIGDN_TRY(run_rms_bwd<1>(d, in, out, w, s));
    else if (nch <= 2) BIGDN_TRY(run_rms_bwd<2>(d, in, out, w, s));
    else if (nch <= 4) BIGDN_TRY(run_rms_bwd<4>(d, in, out, w, s));
    else BIGDN_TRY(run_rms_bwd<8>(d, in, out, w, s));
    return mark(ev, 7, s);
}

hipError_t launch_bigdn_fwd(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s,
                            hipEvent_t* ev) {
    if (d.D == 128) return fwd_go<128>(d, in, out, w, s, ev);
    if (d.D == 64) return fwd_go<64>(d, in, out, w, s, ev);
    return hipErrorInvalidValue;
}

hipError_t launch_bigdn_bwd(const Dims& d, const Inputs& in, const Outputs& out, const Ws& w, hipStream_t s,
                            hipEvent_t* ev) {
    if (d.D == 128) return bwd_go<128>(d, in, out, w, s, ev);
    if (d.D == 64) return bwd_go<64>(d, in, out, w, s, ev);
    return hipErrorInvalidValue;
}

}  // namespace bigdn
