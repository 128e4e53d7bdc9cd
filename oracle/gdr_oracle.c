/*
 * gdr_oracle.c -- plain fp64 CPU oracle for the gated delta rule backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP path.
 *
 * Sources (pages, by title and section):
 *  [P1] "FlashQLA 反向传播全解：fused_gdr_bwd 与 dh 梯度 Kernel 的设计取舍"
 *       (FlashQLA backward explainer).  §一 gives the entry conventions: the
 *       gate arrives as an in-chunk cumulative sum and its gradient is reverse-
 *       cumsummed at the end; dh0 is accumulated and returned in fp32; dht is
 *       optional and means zero when absent.  §二 gives the six outputs
 *       dq/dk/dv/dg/db/dh0 and the reverse-in-chunk dS recursion; §三 gives the
 *       R-form of that recursion.  §四 gives the test protocol (fp64 reference,
 *       element-wise).
 *  [P2] "chunk_kda_bwd_wy_dqkg_fused 算子" (MindSpeed-Ops KDA WY backward
 *       stage).  "参数说明" fixes shapes/dtypes; "实现原理 / 分块计算" names the
 *       intermediates dq = do·hᵀ, dk = v_new·dhᵀ, dw = −dv·hᵀ; the "多阶段
 *       kernel" table names the A·dw corrections, the masked dA_pre and
 *       dA = −A(dA_pre·A).
 *
 * The method (gated delta rule; state S is K x V):
 *     S_t = a_t (I − b_t k_t k_tᵀ) S_{t−1} + b_t k_t v_tᵀ ,   a_t = exp(ĝ_t)
 *     o_t = scale · S_tᵀ q_t
 * and the backward is the gradient of
 *     L = Σ_t <dO_t, o_t> + <dht, S_T>
 * with respect to q, k, v, ĝ, b and the initial state h0.
 *
 * Functions here:
 *   orc_gdr_fwd_token   plain token recurrence (forward).          [pinned]
 *   orc_gdr_bwd_token   hand-derived reverse-time gradients (O-1). [pinned]
 *   orc_gdr_bwd_chunked chunked WY-form forward+backward (O-2), a second,
 *                       independent derivation used for self-checks and for
 *                       the per-chunk states h[c] / dh[c].          [pinned]
 *   orc_kda_wy_bwd      exact VJP of the KDA WY-stage functional (O-K). [pinned]
 *   orc_kda_fwd_token   KDA (per-channel gate) token recurrence, forward. [pinned]
 *   orc_kda_bwd_token   its hand-derived reverse-time gradients (O-KF).   [pinned]
 *   orc_gcum_to_graw    recovers the raw gate from its in-chunk cumsum.
 *   orc_gate_cumsum     the in-chunk cumulative sum itself, in fp64. [pinned]
 * "Pinned" = checked by tests/test_oracle_*.py against finite differences,
 * closed forms and invariants that do not reuse the code below.
 *
 * Layouts (row-major, token axis flattened over batch):
 *   q,k [NTOK,HK,K]   v,dO [NTOK,HV,V]   gate,beta [NTOK,HV]
 *   states h0/dht/dh0/ht [N,HV,K,V]       per-chunk states [NCHUNK,HV,K,V]
 * Sequences: if cu == NULL there are N == B sequences of T tokens each;
 * otherwise sequence n covers tokens [cu[n], cu[n+1]).  Value head hv uses
 * key head hv / (HV/HK).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int B, T, HK, HV, K, V, N;
    const int64_t *cu; /* host [N+1] or NULL */
    double scale;
} orc_problem;

static void seq_range(const orc_problem *p, int n, int64_t *bos, int64_t *len) {
    if (p->cu) { *bos = p->cu[n]; *len = p->cu[n + 1] - p->cu[n]; }
    else { *bos = (int64_t)n * p->T; *len = p->T; }
}

int orc_num_seqs(const orc_problem *p) { return p->cu ? p->N : p->B; }

/* number of chunks of sequence n and the global index of its first chunk */
static int64_t chunk_base(const orc_problem *p, int BT, int n) {
    int64_t base = 0;
    for (int j = 0; j < n; j++) {
        int64_t b, l; seq_range(p, j, &b, &l);
        base += (l + BT - 1) / BT;
    }
    return base;
}

int64_t orc_num_chunks(const orc_problem *p, int BT) {
    return chunk_base(p, BT, orc_num_seqs(p));
}

/* ------------------------------------------------------------------------ */
/* Raw gate from its in-chunk cumulative sum ([P1] §一: the gate input is the
 * in-chunk cumsum; chunks restart at every sequence start). */
void orc_gcum_to_graw(const orc_problem *p, int BT, const float *gcum, double *graw) {
    int NS = orc_num_seqs(p);
    for (int n = 0; n < NS; n++) {
        int64_t bos, len; seq_range(p, n, &bos, &len);
        for (int64_t t = 0; t < len; t++)
            for (int h = 0; h < p->HV; h++) {
                int64_t i = (bos + t) * p->HV + h;
                double prev = (t % BT == 0) ? 0.0 : (double)gcum[i - p->HV];
                graw[i] = (double)gcum[i] - prev;
            }
    }
}

/* The in-chunk cumulative sum of the raw gate ([P1] §一: the forward saves
 * the gate as this sum; chunks are BT tokens long and restart at every
 * sequence start):  out[t] = Σ_{s in t's chunk, s <= t} graw[s], in fp64. */
void orc_gate_cumsum(const orc_problem *p, int BT, const double *graw, double *out) {
    int NS = orc_num_seqs(p);
    for (int n = 0; n < NS; n++) {
        int64_t bos, len; seq_range(p, n, &bos, &len);
        for (int h = 0; h < p->HV; h++) {
            double acc = 0.0;
            for (int64_t t = 0; t < len; t++) {
                int64_t i = (bos + t) * p->HV + h;
                if (t % BT == 0) acc = 0.0;
                acc += graw[i];
                out[i] = acc;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* One token step of the recurrence, in place:
 *   S <- a (I − b k kᵀ) S + b k vᵀ          (S is K x V, row-major) */
static void token_step(double *S, int K, int V, const double *kk, const double *vv, double a, double b) {
    double *kS = (double *)malloc(sizeof(double) * V);
    for (int j = 0; j < V; j++) {
        double s = 0;
        for (int i = 0; i < K; i++) s += kk[i] * S[i * V + j];
        kS[j] = s;
    }
    for (int i = 0; i < K; i++)
        for (int j = 0; j < V; j++)
            S[i * V + j] = a * (S[i * V + j] - b * kk[i] * kS[j]) + b * kk[i] * vv[j];
    free(kS);
}

/* Forward token recurrence.  Outputs (each may be NULL):
 *   o   [NTOK,HV,V]        o_t = scale S_tᵀ q_t (post-update state)
 *   ht  [N,HV,K,V]         final state of every sequence
 *   hc  [NCHUNK,HV,K,V]    state entering each chunk of size BT            */
int orc_gdr_fwd_token(const orc_problem *p, int BT, const double *q, const double *k, const double *v,
                      const double *graw, const double *beta, const double *h0,
                      double *o, double *ht, double *hc) {
    const int K = p->K, V = p->V, HV = p->HV, HK = p->HK, G = HV / HK;
    const int NS = orc_num_seqs(p);
    if (HV % HK) return -1;
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int n = 0; n < NS; n++)
        for (int hv = 0; hv < HV; hv++) {
            int hk = hv / G;
            int64_t bos, len; seq_range(p, n, &bos, &len);
            int64_t cb = chunk_base(p, BT > 0 ? BT : 1, n);
            double *S = (double *)calloc((size_t)K * V, sizeof(double));
            if (h0) memcpy(S, h0 + ((size_t)n * HV + hv) * K * V, sizeof(double) * K * V);
            for (int64_t t = 0; t < len; t++) {
                int64_t tok = bos + t;
                if (hc && BT > 0 && t % BT == 0)
                    memcpy(hc + ((size_t)(cb + t / BT) * HV + hv) * K * V, S, sizeof(double) * K * V);
                const double *kk = k + ((size_t)tok * HK + hk) * K;
                const double *vv = v + ((size_t)tok * HV + hv) * V;
                double a = exp(graw[tok * HV + hv]), b = beta[tok * HV + hv];
                token_step(S, K, V, kk, vv, a, b);
                if (o) {
                    const double *qq = q + ((size_t)tok * HK + hk) * K;
                    double *oo = o + ((size_t)tok * HV + hv) * V;
                    for (int j = 0; j < V; j++) {
                        double s = 0;
                        for (int i = 0; i < K; i++) s += S[i * V + j] * qq[i];
                        oo[j] = p->scale * s;
                    }
                }
            }
            if (ht) memcpy(ht + ((size_t)n * HV + hv) * K * V, S, sizeof(double) * K * V);
            free(S);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O-1: reverse-time gradients of the token recurrence, derived by hand from
 * S_t = a_t P_t S_{t−1} + b_t k_t v_tᵀ with P_t = I − b_t k_t k_tᵀ:
 *   dS_t   += scale q_t dO_tᵀ                (o_t reads the post-update state)
 *   dq_t    = scale S_t dO_t
 *   dv_t    = b_t dS_tᵀ k_t
 *   dĝ_t    = a_t <dS_t, P_t S_{t−1}>
 *   db_t    = k_tᵀ dS_t v_t − a_t k_tᵀ dS_t S_{t−1}ᵀ k_t
 *   dk_t    = b_t dS_t v_t − a_t b_t (dS_t S_{t−1}ᵀ + S_{t−1} dS_tᵀ) k_t
 *   dS_{t−1} = a_t P_t dS_t
 * States are checkpointed every CKPT tokens and recomputed per segment.
 * dq/dk are summed over the value heads that share a key head (GQA).      */
#define CKPT 64
int orc_gdr_bwd_token(const orc_problem *p, const double *q, const double *k, const double *v,
                      const double *graw, const double *beta, const double *h0,
                      const double *dO, const double *dht,
                      double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0) {
    const int K = p->K, V = p->V, HV = p->HV, HK = p->HK, G = HV / HK;
    const int NS = orc_num_seqs(p);
    if (HV % HK) return -1;
    int64_t ntok = 0;
    for (int n = 0; n < NS; n++) { int64_t b, l; seq_range(p, n, &b, &l); if (b + l > ntok) ntok = b + l; }
    memset(dq, 0, sizeof(double) * ntok * HK * K);
    memset(dk, 0, sizeof(double) * ntok * HK * K);
    /* parallel over (sequence, key head); the value heads of a group run in
     * turn so the dq/dk group sums need no atomics */
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int n = 0; n < NS; n++)
        for (int hk = 0; hk < HK; hk++) {
            int64_t bos, len; seq_range(p, n, &bos, &len);
            size_t KV = (size_t)K * V;
            int64_t nck = (len + CKPT - 1) / CKPT;
            double *ck = (double *)malloc(sizeof(double) * KV * (nck > 0 ? nck : 1));
            double *seg = (double *)malloc(sizeof(double) * KV * (CKPT + 1));
            double *dS = (double *)malloc(sizeof(double) * KV);
            double *u = (double *)malloc(sizeof(double) * (K > V ? K : V) * 4);
            for (int hv = hk * G; hv < (hk + 1) * G; hv++) {
                /* forward pass: checkpoints of the state entering each segment */
                double *S = seg;
                if (h0) memcpy(S, h0 + ((size_t)n * HV + hv) * KV, sizeof(double) * KV);
                else memset(S, 0, sizeof(double) * KV);
                for (int64_t t = 0; t < len; t++) {
                    if (t % CKPT == 0) memcpy(ck + (t / CKPT) * KV, S, sizeof(double) * KV);
                    int64_t tok = bos + t;
                    token_step(S, K, V, k + ((size_t)tok * HK + hk) * K, v + ((size_t)tok * HV + hv) * V,
                               exp(graw[tok * HV + hv]), beta[tok * HV + hv]);
                }
                /* backward */
                if (dht) memcpy(dS, dht + ((size_t)n * HV + hv) * KV, sizeof(double) * KV);
                else memset(dS, 0, sizeof(double) * KV);
                for (int64_t sgi = nck - 1; sgi >= 0; sgi--) {
                    int64_t t0 = sgi * CKPT, t1 = t0 + CKPT < len ? t0 + CKPT : len;
                    /* seg[j] = state S_{t0+j} (state after j tokens of the segment) */
                    memcpy(seg, ck + sgi * KV, sizeof(double) * KV);
                    for (int64_t t = t0; t < t1; t++) {
                        int64_t tok = bos + t;
                        double *Sn = seg + (t - t0 + 1) * KV;
                        memcpy(Sn, seg + (t - t0) * KV, sizeof(double) * KV);
                        token_step(Sn, K, V, k + ((size_t)tok * HK + hk) * K, v + ((size_t)tok * HV + hv) * V,
                                   exp(graw[tok * HV + hv]), beta[tok * HV + hv]);
                    }
                    for (int64_t t = t1 - 1; t >= t0; t--) {
                        int64_t tok = bos + t;
                        const double *St = seg + (t - t0 + 1) * KV;  /* S_t   */
                        const double *Sp = seg + (t - t0) * KV;      /* S_{t-1} */
                        const double *qq = q + ((size_t)tok * HK + hk) * K;
                        const double *kk = k + ((size_t)tok * HK + hk) * K;
                        const double *vv = v + ((size_t)tok * HV + hv) * V;
                        const double *dd = dO + ((size_t)tok * HV + hv) * V;
                        double a = exp(graw[tok * HV + hv]), b = beta[tok * HV + hv];
                        /* dS_t += scale q dOᵀ */
                        for (int i = 0; i < K; i++)
                            for (int j = 0; j < V; j++) dS[i * V + j] += p->scale * qq[i] * dd[j];
                        /* dq_t = scale S_t dO_t */
                        double *dqq = dq + ((size_t)tok * HK + hk) * K;
                        for (int i = 0; i < K; i++) {
                            double s = 0;
                            for (int j = 0; j < V; j++) s += St[i * V + j] * dd[j];
                            dqq[i] += p->scale * s;
                        }
                        /* dSv = dS v (K), dSk = dSᵀ k (V), Spk = S_{t-1}ᵀ k (V),
                         * kdS... */
                        double *dSv = u, *dSk = u + K, *Spk = u + K + V;
                        for (int i = 0; i < K; i++) {
                            double s = 0;
                            for (int j = 0; j < V; j++) s += dS[i * V + j] * vv[j];
                            dSv[i] = s;
                        }
                        for (int j = 0; j < V; j++) {
                            double s1 = 0, s2 = 0;
                            for (int i = 0; i < K; i++) { s1 += dS[i * V + j] * kk[i]; s2 += Sp[i * V + j] * kk[i]; }
                            dSk[j] = s1; Spk[j] = s2;
                        }
                        /* dv_t = b dSᵀ k */
                        double *dvv = dv + ((size_t)tok * HV + hv) * V;
                        for (int j = 0; j < V; j++) dvv[j] = b * dSk[j];
                        /* <dS, P S_{t-1}> = <dS, S_{t-1}> − b (dSᵀk)·(S_{t-1}ᵀk) */
                        double dSS = 0, kdSv = 0, kdSSk = 0;
                        for (size_t e = 0; e < KV; e++) dSS += dS[e] * Sp[e];
                        for (int i = 0; i < K; i++) kdSv += kk[i] * dSv[i];
                        for (int j = 0; j < V; j++) kdSSk += dSk[j] * Spk[j];
                        dg[tok * HV + hv] = a * (dSS - b * kdSSk);
                        dbeta[tok * HV + hv] = kdSv - a * kdSSk;
                        /* dk = b dS v − a b (dS S_{t-1}ᵀ k + S_{t-1} dSᵀ k) */
                        double *dkk = dk + ((size_t)tok * HK + hk) * K;
                        for (int i = 0; i < K; i++) {
                            double s1 = 0, s2 = 0;
                            for (int j = 0; j < V; j++) { s1 += dS[i * V + j] * Spk[j]; s2 += Sp[i * V + j] * dSk[j]; }
                            dkk[i] += b * dSv[i] - a * b * (s1 + s2);
                        }
                        /* dS_{t-1} = a (I − b k kᵀ) dS */
                        for (int i = 0; i < K; i++)
                            for (int j = 0; j < V; j++)
                                dS[i * V + j] = a * (dS[i * V + j] - b * kk[i] * dSk[j]);
                    }
                }
                if (dh0) memcpy(dh0 + ((size_t)n * HV + hv) * KV, dS, sizeof(double) * KV);
            }
            free(ck); free(seg); free(dS); free(u);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Small dense helpers for the chunked derivation (naive loops). */
/* C[m x n] = op(A) op(B); ta/tb select the transpose of a row-major operand. */
static void mm(int m, int n, int kd, const double *A, int ta, const double *B, int tb, double *C) {
    for (int i = 0; i < m; i++)
        for (int j = 0; j < n; j++) {
            double s = 0;
            for (int l = 0; l < kd; l++) {
                double a = ta ? A[l * m + i] : A[i * kd + l];
                double b = tb ? B[j * kd + l] : B[l * n + j];
                s += a * b;
            }
            C[i * n + j] = s;
        }
}

/* O-2: chunked WY form.  For each chunk of C <= BT tokens with in-chunk
 * cumulative log-gate G (γ_r = e^{G_r}, Γ_rs = e^{G_r − G_s}):
 *   L  = strict lower part of diag(b) (K Kᵀ) ⊙ Γ;  A = (I + L)^{-1}
 *   W  = A diag(bγ) K;   U = A diag(b) V;   Vn = U − W h
 *   Pm = scale · lower(incl. diagonal) of Γ ⊙ Q Kᵀ
 *   O  = scale diag(γ) Q h + Pm Vn;   h' = γ_C h + K̃ᵀ Vn,  K̃ = diag(γ_C/γ) K
 * Backward of the same expressions (chain rule, term by term), given the
 * gradient dh of the state leaving the chunk:
 *   dVn = Pmᵀ dO + K̃ dh
 *   dPm = lower(dO Vnᵀ);  dW = −dVn hᵀ;  dU = dVn
 *   dA  = dU (diag(b)V)ᵀ + dW (diag(bγ)K)ᵀ;  dL = −strictlower(Aᵀ dA Aᵀ)
 *   dh_in = γ_C dh + scale Qᵀ diag(γ) dO − Wᵀ dVn
 * and every gate-dependent factor contributes to dG (chunk-local), which is
 * finally reverse-cumsummed inside the chunk into the raw-gate gradient.
 * Outputs hc/dhc (nullable): state entering chunk c, and the gradient of the
 * state leaving chunk c.                                                    */
int orc_gdr_bwd_chunked(const orc_problem *p, int BT, const double *q, const double *k, const double *v,
                        const double *graw, const double *beta, const double *h0,
                        const double *dO, const double *dht,
                        double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0,
                        double *hc, double *dhc) {
    const int K = p->K, V = p->V, HV = p->HV, HK = p->HK, G = HV / HK;
    const int NS = orc_num_seqs(p);
    const double sc = p->scale;
    if (HV % HK || BT <= 0) return -1;
    int64_t ntok = 0;
    for (int n = 0; n < NS; n++) { int64_t b, l; seq_range(p, n, &b, &l); if (b + l > ntok) ntok = b + l; }
    memset(dq, 0, sizeof(double) * ntok * HK * K);
    memset(dk, 0, sizeof(double) * ntok * HK * K);
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int n = 0; n < NS; n++)
        for (int hk = 0; hk < HK; hk++) {
            int64_t bos, len; seq_range(p, n, &bos, &len);
            int64_t nc = (len + BT - 1) / BT, cb = chunk_base(p, BT, n);
            size_t KV = (size_t)K * V;
            int C = BT;
            double *hs = (double *)malloc(sizeof(double) * KV * (nc + 1));
            double *Qm = malloc(sizeof(double) * C * K), *Km = malloc(sizeof(double) * C * K);
            double *Vm = malloc(sizeof(double) * C * V), *dOm = malloc(sizeof(double) * C * V);
            double *Gc = malloc(sizeof(double) * C), *bt = malloc(sizeof(double) * C);
            double *L = malloc(sizeof(double) * C * C), *A = malloc(sizeof(double) * C * C);
            double *Pm = malloc(sizeof(double) * C * C), *T1 = malloc(sizeof(double) * C * C);
            double *T2 = malloc(sizeof(double) * C * C), *dA = malloc(sizeof(double) * C * C);
            double *dL = malloc(sizeof(double) * C * C), *dPm = malloc(sizeof(double) * C * C);
            double *W = malloc(sizeof(double) * C * K), *U = malloc(sizeof(double) * C * V);
            double *Vn = malloc(sizeof(double) * C * V), *dVn = malloc(sizeof(double) * C * V);
            double *Kt = malloc(sizeof(double) * C * K), *X = malloc(sizeof(double) * C * (K > V ? K : V));
            double *dW = malloc(sizeof(double) * C * K), *dqc = malloc(sizeof(double) * C * K);
            double *dkc = malloc(sizeof(double) * C * K), *dG = malloc(sizeof(double) * C);
            double *dH = malloc(sizeof(double) * KV), *dHn = malloc(sizeof(double) * KV);
            double *KK = malloc(sizeof(double) * C * C), *QK = malloc(sizeof(double) * C * C);
            double *XX = malloc(sizeof(double) * KV);
            for (int hv = hk * G; hv < (hk + 1) * G; hv++) {
                /* ---- load chunk c into dense tiles; rows >= Cc are absent ---- */
#define LOAD_CHUNK(c, Cc)                                                                   \
                do {                                                                        \
                    int64_t t0 = bos + (int64_t)(c) * BT;                                   \
                    (Cc) = (int)((len - (int64_t)(c) * BT) < BT ? (len - (int64_t)(c) * BT) : BT); \
                    double acc = 0;                                                         \
                    for (int r = 0; r < (Cc); r++) {                                        \
                        int64_t tok = t0 + r;                                               \
                        memcpy(Qm + r * K, q + ((size_t)tok * HK + hk) * K, sizeof(double) * K); \
                        memcpy(Km + r * K, k + ((size_t)tok * HK + hk) * K, sizeof(double) * K); \
                        memcpy(Vm + r * V, v + ((size_t)tok * HV + hv) * V, sizeof(double) * V); \
                        memcpy(dOm + r * V, dO + ((size_t)tok * HV + hv) * V, sizeof(double) * V); \
                        acc += graw[tok * HV + hv]; Gc[r] = acc; bt[r] = beta[tok * HV + hv]; \
                    }                                                                       \
                } while (0)
                /* builds L, A, W, U, Pm, Kt for the loaded chunk */
#define PREP_CHUNK(Cc)                                                                      \
                do {                                                                        \
                    mm((Cc), (Cc), K, Km, 0, Km, 1, KK);                                    \
                    mm((Cc), (Cc), K, Qm, 0, Km, 1, QK);                                    \
                    for (int r = 0; r < (Cc); r++)                                          \
                        for (int s = 0; s < (Cc); s++) {                                    \
                            double Gm = exp(Gc[r] - Gc[s]);                                 \
                            L[r * (Cc) + s] = (s < r) ? bt[r] * KK[r * (Cc) + s] * Gm : 0.0; \
                            Pm[r * (Cc) + s] = (s <= r) ? sc * QK[r * (Cc) + s] * Gm : 0.0; \
                        }                                                                   \
                    /* A = (I+L)^{-1} by forward substitution, row by row */                \
                    for (int r = 0; r < (Cc); r++)                                          \
                        for (int s = 0; s < (Cc); s++) {                                    \
                            double a = (r == s) ? 1.0 : 0.0;                                \
                            for (int j = 0; j < r; j++) a -= L[r * (Cc) + j] * A[j * (Cc) + s]; \
                            A[r * (Cc) + s] = a;                                            \
                        }                                                                   \
                    for (int r = 0; r < (Cc); r++) {                                        \
                        double gr = exp(Gc[r]);                                             \
                        for (int i = 0; i < K; i++) X[r * K + i] = bt[r] * gr * Km[r * K + i]; \
                    }                                                                       \
                    mm((Cc), K, (Cc), A, 0, X, 0, W);                                       \
                    for (int r = 0; r < (Cc); r++)                                          \
                        for (int j = 0; j < V; j++) X[r * V + j] = bt[r] * Vm[r * V + j];   \
                    mm((Cc), V, (Cc), A, 0, X, 0, U);                                       \
                    for (int r = 0; r < (Cc); r++) {                                        \
                        double f = exp(Gc[(Cc) - 1] - Gc[r]);                               \
                        for (int i = 0; i < K; i++) Kt[r * K + i] = f * Km[r * K + i];      \
                    }                                                                       \
                } while (0)
                /* ---------------- forward over chunks: hs[c] ---------------- */
                if (h0) memcpy(hs, h0 + ((size_t)n * HV + hv) * KV, sizeof(double) * KV);
                else memset(hs, 0, sizeof(double) * KV);
                for (int64_t c = 0; c < nc; c++) {
                    int Cc; LOAD_CHUNK(c, Cc); PREP_CHUNK(Cc);
                    double *h = hs + c * KV, *hn = hs + (c + 1) * KV;
                    mm(Cc, V, K, W, 0, h, 0, X);
                    for (int e = 0; e < Cc * V; e++) Vn[e] = U[e] - X[e];
                    mm(K, V, Cc, Kt, 1, Vn, 0, hn);
                    double gC = exp(Gc[Cc - 1]);
                    for (size_t e = 0; e < KV; e++) hn[e] += gC * h[e];
                    if (hc) memcpy(hc + ((size_t)(cb + c) * HV + hv) * KV, h, sizeof(double) * KV);
                }
                /* ---------------- backward over chunks ---------------- */
                if (dht) memcpy(dH, dht + ((size_t)n * HV + hv) * KV, sizeof(double) * KV);
                else memset(dH, 0, sizeof(double) * KV);
                for (int64_t c = nc - 1; c >= 0; c--) {
                    int Cc; LOAD_CHUNK(c, Cc); PREP_CHUNK(Cc);
                    double *h = hs + c * KV;
                    if (dhc) memcpy(dhc + ((size_t)(cb + c) * HV + hv) * KV, dH, sizeof(double) * KV);
                    double gC = exp(Gc[Cc - 1]);
                    /* Vn */
                    mm(Cc, V, K, W, 0, h, 0, X);
                    for (int e = 0; e < Cc * V; e++) Vn[e] = U[e] - X[e];
                    /* dVn = Pmᵀ dO + K̃ dH */
                    mm(Cc, V, Cc, Pm, 1, dOm, 0, dVn);
                    mm(Cc, V, K, Kt, 0, dH, 0, X);
                    for (int e = 0; e < Cc * V; e++) dVn[e] += X[e];
                    /* dPm = lower(dO Vnᵀ) */
                    mm(Cc, Cc, V, dOm, 0, Vn, 1, dPm);
                    for (int r = 0; r < Cc; r++) for (int s = r + 1; s < Cc; s++) dPm[r * Cc + s] = 0;
                    for (int r = 0; r < Cc; r++) dG[r] = 0;
                    /* dq: scale diag(γ) dO hᵀ + (dPm ⊙ Γ scale) K; and dG from γ in O */
                    mm(Cc, K, V, dOm, 0, h, 1, dqc);
                    for (int r = 0; r < Cc; r++) {
                        double gr = exp(Gc[r]), s = 0;
                        for (int i = 0; i < K; i++) { dqc[r * K + i] *= sc * gr; s += Qm[r * K + i] * dqc[r * K + i]; }
                        dG[r] += s;
                    }
                    /* T1 = dPm ⊙ Γ scale (gradient of QKᵀ through Pm) */
                    for (int r = 0; r < Cc; r++)
                        for (int s = 0; s < Cc; s++) T1[r * Cc + s] = (s <= r) ? dPm[r * Cc + s] * sc * exp(Gc[r] - Gc[s]) : 0.0;
                    mm(Cc, K, Cc, T1, 0, Km, 0, X);
                    for (int e = 0; e < Cc * K; e++) dqc[e] += X[e];
                    /* dG from Γ in Pm: rowsum(F) − colsum(F), F = dPm ⊙ Pm */
                    for (int r = 0; r < Cc; r++)
                        for (int s = 0; s <= r; s++) { double f = dPm[r * Cc + s] * Pm[r * Cc + s]; dG[r] += f; dG[s] -= f; }
                    /* dk from Pm */
                    mm(Cc, K, Cc, T1, 1, Qm, 0, dkc);
                    /* dk from K̃: diag(γ_C/γ) Vn dHᵀ ; dG from K̃'s gate factor */
                    mm(Cc, K, V, Vn, 0, dH, 1, X);
                    {
                        double zs = 0;
                        for (int r = 0; r < Cc; r++) {
                            double f = exp(Gc[Cc - 1] - Gc[r]), z = 0;
                            for (int i = 0; i < K; i++) { double t = f * X[r * K + i]; dkc[r * K + i] += t; z += t * Km[r * K + i]; }
                            dG[r] -= z; zs += z;
                        }
                        dG[Cc - 1] += zs;
                    }
                    /* dG_C from γ_C h in h' */
                    { double s = 0; for (size_t e = 0; e < KV; e++) s += dH[e] * h[e]; dG[Cc - 1] += gC * s; }
                    /* dW = −dVn hᵀ ; dU = dVn */
                    mm(Cc, K, V, dVn, 0, h, 1, dW);
                    for (int e = 0; e < Cc * K; e++) dW[e] = -dW[e];
                    /* U = A diag(b) V: dv = diag(b) Aᵀ dVn, db += rowsum(Aᵀ dVn ⊙ V) */
                    mm(Cc, V, Cc, A, 1, dVn, 0, X);
                    double *dvo = X;
                    for (int r = 0; r < Cc; r++) {
                        double s = 0;
                        for (int j = 0; j < V; j++) s += dvo[r * V + j] * Vm[r * V + j];
                        dbeta[(bos + c * BT + r) * HV + hv] = s;
                        for (int j = 0; j < V; j++) dv[((size_t)(bos + c * BT + r) * HV + hv) * V + j] = bt[r] * dvo[r * V + j];
                    }
                    /* W = A diag(bγ) K: dk += diag(bγ) Aᵀ dW; db += γ rowsum(Aᵀ dW ⊙ K); dG += bγ rowsum(..) */
                    {
                        double *AdW = malloc(sizeof(double) * Cc * K);
                        mm(Cc, K, Cc, A, 1, dW, 0, AdW);
                        for (int r = 0; r < Cc; r++) {
                            double gr = exp(Gc[r]), s = 0;
                            for (int i = 0; i < K; i++) { s += AdW[r * K + i] * Km[r * K + i]; dkc[r * K + i] += bt[r] * gr * AdW[r * K + i]; }
                            dbeta[(bos + c * BT + r) * HV + hv] += gr * s;
                            dG[r] += bt[r] * gr * s;
                        }
                        free(AdW);
                    }
                    /* dA = dU (diag(b)V)ᵀ + dW (diag(bγ)K)ᵀ */
                    for (int r = 0; r < Cc; r++) for (int j = 0; j < V; j++) X[r * V + j] = bt[r] * Vm[r * V + j];
                    mm(Cc, Cc, V, dVn, 0, X, 1, dA);
                    for (int r = 0; r < Cc; r++) { double gr = exp(Gc[r]); for (int i = 0; i < K; i++) X[r * K + i] = bt[r] * gr * Km[r * K + i]; }
                    mm(Cc, Cc, K, dW, 0, X, 1, T2);
                    for (int e = 0; e < Cc * Cc; e++) dA[e] += T2[e];
                    /* dL = −strictlower(Aᵀ dA Aᵀ) */
                    mm(Cc, Cc, Cc, A, 1, dA, 0, T2);
                    mm(Cc, Cc, Cc, T2, 0, A, 1, dL);
                    for (int r = 0; r < Cc; r++) for (int s = 0; s < Cc; s++) dL[r * Cc + s] = (s < r) ? -dL[r * Cc + s] : 0.0;
                    /* L_rs = b_r Γ_rs (k_r·k_s): db, dk, dG */
                    for (int r = 0; r < Cc; r++)
                        for (int s = 0; s < r; s++) {
                            double Gm = exp(Gc[r] - Gc[s]);
                            double E = dL[r * Cc + s] * Gm;
                            dbeta[(bos + c * BT + r) * HV + hv] += E * KK[r * Cc + s];
                            for (int i = 0; i < K; i++) {
                                dkc[r * K + i] += bt[r] * E * Km[s * K + i];
                                dkc[s * K + i] += bt[r] * E * Km[r * K + i];
                            }
                            double f = dL[r * Cc + s] * L[r * Cc + s];
                            dG[r] += f; dG[s] -= f;
                        }
                    /* scatter dq, dk (group sums), dg = in-chunk reverse cumsum of dG */
                    {
                        double acc = 0;
                        for (int r = Cc - 1; r >= 0; r--) {
                            int64_t tok = bos + c * BT + r;
                            acc += dG[r];
                            dg[tok * HV + hv] = acc;
                            for (int i = 0; i < K; i++) {
                                dq[((size_t)tok * HK + hk) * K + i] += dqc[r * K + i];
                                dk[((size_t)tok * HK + hk) * K + i] += dkc[r * K + i];
                            }
                        }
                    }
                    /* dH_in = γ_C dH + scale Qᵀ diag(γ) dO − Wᵀ dVn */
                    for (int r = 0; r < Cc; r++) { double gr = exp(Gc[r]); for (int j = 0; j < V; j++) X[r * V + j] = sc * gr * dOm[r * V + j]; }
                    mm(K, V, Cc, Qm, 1, X, 0, dHn);
                    mm(K, V, Cc, W, 1, dVn, 0, XX);
                    for (size_t e = 0; e < KV; e++) dH[e] = gC * dH[e] + dHn[e] - XX[e];
                }
                if (dh0) memcpy(dh0 + ((size_t)n * HV + hv) * KV, dH, sizeof(double) * KV);
#undef LOAD_CHUNK
#undef PREP_CHUNK
            }
            free(hs); free(Qm); free(Km); free(Vm); free(dOm); free(Gc); free(bt); free(L); free(A);
            free(Pm); free(T1); free(T2); free(dA); free(dL); free(dPm); free(W); free(U); free(Vn);
            free(dVn); free(Kt); free(X); free(dW); free(dqc); free(dkc); free(dG); free(dH); free(dHn);
            free(KK); free(QK); free(XX);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O-K: KDA WY stage ([P2]).  Per chunk (C rows), per head, with the per-
 * channel gate g (used as given: an in-chunk cumulative log-gate, [C x K]),
 * γ = e^g, γ_C its last row, and V_new, dO, dh, dv_in, h taken as constants,
 * the outputs are the exact gradients of
 *   Φ = scale<dO, (Q⊙γ) h> + <dh, (K⊙γ_C/γ)ᵀ V_new> + <dh, diag(γ_C) h>
 *       + <dv_in, A(b⊙V) − A(b⊙γ⊙K) h>
 * with respect to q, k, v, b, g and the strictly-lower L that defines the
 * lower-triangular A = (I+L)^{-1}.  This reproduces [P2]'s named steps:
 * dq = do·hᵀ (gated, scaled), dk = v_new·dhᵀ (gated), dw = −dv·hᵀ, the Aᵀ·dw
 * corrections, dA_pre, and dA = −Aᵀ dA_pre Aᵀ restricted to L's support.
 * A is read as the lower triangle of the [.., BT] input row block (its upper
 * part is ignored).  dA is written only on the strictly-lower part; entries
 * on and above the diagonal are set to zero.                                */
int orc_kda_wy_bwd(const orc_problem *p, int BT, const double *q, const double *k, const double *v,
                   const double *vnew, const double *g, const double *beta, const double *Ain,
                   const double *hst, const double *dO, const double *dhst, const double *dvin,
                   double *dq, double *dk, double *dvout, double *db, double *dg, double *dA) {
    const int K = p->K, V = p->V, H = p->HV;
    const int NS = orc_num_seqs(p);
    const double sc = p->scale;
    if (p->HK != p->HV || BT <= 0) return -1;
    int64_t nchunks = orc_num_chunks(p, BT);
    (void)nchunks;
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int n = 0; n < NS; n++)
        for (int hh = 0; hh < H; hh++) {
            int64_t bos, len; seq_range(p, n, &bos, &len);
            int64_t nc = (len + BT - 1) / BT, cb = chunk_base(p, BT, n);
            size_t KV = (size_t)K * V;
            int XW = K > V ? K : V;
            if (BT > XW) XW = BT;
            double *A = malloc(sizeof(double) * BT * BT), *X = malloc(sizeof(double) * BT * XW);
            double *dw = malloc(sizeof(double) * BT * K), *AdW = malloc(sizeof(double) * BT * K);
            double *AdV = malloc(sizeof(double) * BT * V), *dks = malloc(sizeof(double) * BT * K);
            double *dAp = malloc(sizeof(double) * BT * BT), *T = malloc(sizeof(double) * BT * BT);
            for (int64_t c = 0; c < nc; c++) {
                int64_t t0 = bos + c * BT;
                int C = (int)((len - c * BT) < BT ? (len - c * BT) : BT);
                const double *h = hst + ((size_t)(cb + c) * H + hh) * KV;
                const double *dh = dhst + ((size_t)(cb + c) * H + hh) * KV;
#define QK_(r, i) q[((size_t)(t0 + (r)) * H + hh) * K + (i)]
#define KK_(r, i) k[((size_t)(t0 + (r)) * H + hh) * K + (i)]
#define VV_(r, j) v[((size_t)(t0 + (r)) * H + hh) * V + (j)]
#define VN_(r, j) vnew[((size_t)(t0 + (r)) * H + hh) * V + (j)]
#define DO_(r, j) dO[((size_t)(t0 + (r)) * H + hh) * V + (j)]
#define DV_(r, j) dvin[((size_t)(t0 + (r)) * H + hh) * V + (j)]
#define GG_(r, i) g[((size_t)(t0 + (r)) * H + hh) * K + (i)]
#define BB_(r) beta[(t0 + (r)) * H + hh]
                for (int r = 0; r < C; r++)
                    for (int s = 0; s < C; s++)
                        A[r * C + s] = (s <= r) ? Ain[((size_t)(t0 + r) * H + hh) * BT + s] : 0.0;
                /* dq = scale (dO hᵀ) ⊙ γ */
                for (int r = 0; r < C; r++)
                    for (int i = 0; i < K; i++) {
                        double s = 0;
                        for (int j = 0; j < V; j++) s += DO_(r, j) * h[i * V + j];
                        dq[((size_t)(t0 + r) * H + hh) * K + i] = sc * s * exp(GG_(r, i));
                    }
                /* dk_s = (Vn dhᵀ) ⊙ γ_C/γ ; dw = −dv_in hᵀ */
                for (int r = 0; r < C; r++)
                    for (int i = 0; i < K; i++) {
                        double s1 = 0, s2 = 0;
                        for (int j = 0; j < V; j++) { s1 += VN_(r, j) * dh[i * V + j]; s2 += DV_(r, j) * h[i * V + j]; }
                        dks[r * K + i] = s1 * exp(GG_(C - 1, i) - GG_(r, i));
                        dw[r * K + i] = -s2;
                    }
                /* AdW = Aᵀ dw, AdV = Aᵀ dv_in */
                for (int r = 0; r < C; r++) {
                    for (int i = 0; i < K; i++) { double s = 0; for (int m = 0; m < C; m++) s += A[m * C + r] * dw[m * K + i]; AdW[r * K + i] = s; }
                    for (int j = 0; j < V; j++) { double s = 0; for (int m = 0; m < C; m++) s += A[m * C + r] * DV_(m, j); AdV[r * V + j] = s; }
                }
                for (int r = 0; r < C; r++) {
                    int64_t tok = t0 + r;
                    double b = BB_(r), sb = 0;
                    for (int j = 0; j < V; j++) {
                        dvout[((size_t)tok * H + hh) * V + j] = b * AdV[r * V + j];
                        sb += AdV[r * V + j] * VV_(r, j);
                    }
                    for (int i = 0; i < K; i++) {
                        double gm = exp(GG_(r, i));
                        double w = AdW[r * K + i] * gm * KK_(r, i);
                        sb += w;
                        dk[((size_t)tok * H + hh) * K + i] = dks[r * K + i] + b * gm * AdW[r * K + i];
                        dg[((size_t)tok * H + hh) * K + i] = QK_(r, i) * dq[((size_t)tok * H + hh) * K + i]
                                                              - KK_(r, i) * dks[r * K + i] + b * w;
                    }
                    db[tok * H + hh] = sb;
                }
                /* last row: + colsum(K ⊙ dk_s) + γ_C ⊙ rowsum_V(h ⊙ dh) */
                for (int i = 0; i < K; i++) {
                    double s = 0, hd = 0;
                    for (int r = 0; r < C; r++) s += KK_(r, i) * dks[r * K + i];
                    for (int j = 0; j < V; j++) hd += h[i * V + j] * dh[i * V + j];
                    dg[((size_t)(t0 + C - 1) * H + hh) * K + i] += s + exp(GG_(C - 1, i)) * hd;
                }
                /* dA_pre = dv_in (b⊙V)ᵀ + dw (b⊙γ⊙K)ᵀ ; dA = −strictlower(Aᵀ lower(dA_pre) Aᵀ) */
                for (int r = 0; r < C; r++)
                    for (int s = 0; s < C; s++) {
                        double t = 0;
                        if (s <= r) {
                            for (int j = 0; j < V; j++) t += DV_(r, j) * BB_(s) * VV_(s, j);
                            for (int i = 0; i < K; i++) t += dw[r * K + i] * BB_(s) * exp(GG_(s, i)) * KK_(s, i);
                        }
                        dAp[r * C + s] = t;
                    }
                mm(C, C, C, A, 1, dAp, 0, T);
                mm(C, C, C, T, 0, A, 1, X);
                for (int r = 0; r < C; r++)
                    for (int s = 0; s < BT; s++)
                        dA[((size_t)(t0 + r) * H + hh) * BT + s] = (s < r) ? -X[r * C + s] : 0.0;
#undef QK_
#undef KK_
#undef VV_
#undef VN_
#undef DO_
#undef DV_
#undef GG_
#undef BB_
            }
            free(A); free(X); free(dw); free(AdW); free(AdV); free(dks); free(dAp); free(T);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* KDA: the gated delta rule with a per-channel gate ([P2] 概述: the operator
 * is one stage of the KDA chunk backward).  State S (K x V) per sequence and
 * head (HK == HV == H), gate a_t = exp(ĝ_t) in R^K applied before the delta
 * update:
 *   X = diag(a_t) S_{t−1},  u_t = v_t − Xᵀ k_t,  S_t = X + b_t k_t u_tᵀ
 *   (= (I − b_t k_t k_tᵀ) diag(a_t) S_{t−1} + b_t k_t v_tᵀ),
 *   o_t = scale S_tᵀ q_t.
 * Layouts: q, k, ĝ [NTOK,H,K]; v, dO [NTOK,H,V]; b [NTOK,H]; states [N,H,K,V]. */
static void kda_step(double *S, int K, int V, const double *kk, const double *vv, const double *ga, double b,
                     double *u) {
    for (int i = 0; i < K; i++) {
        const double a = exp(ga[i]);
        for (int j = 0; j < V; j++) S[i * V + j] *= a;
    }
    for (int j = 0; j < V; j++) {
        double s = 0;
        for (int i = 0; i < K; i++) s += S[i * V + j] * kk[i];
        u[j] = vv[j] - s;
    }
    for (int i = 0; i < K; i++)
        for (int j = 0; j < V; j++) S[i * V + j] += b * kk[i] * u[j];
}

int orc_kda_fwd_token(const orc_problem *p, const double *q, const double *k, const double *v, const double *graw,
                      const double *beta, const double *h0, double *o, double *ht) {
    const int K = p->K, V = p->V, H = p->HV;
    const int NS = orc_num_seqs(p);
    if (p->HK != p->HV) return -1;
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int n = 0; n < NS; n++)
        for (int h = 0; h < H; h++) {
            int64_t bos, len; seq_range(p, n, &bos, &len);
            double *S = (double *)calloc((size_t)K * V, sizeof(double));
            double *u = (double *)malloc(sizeof(double) * V);
            if (h0) memcpy(S, h0 + ((size_t)n * H + h) * K * V, sizeof(double) * K * V);
            for (int64_t t = 0; t < len; t++) {
                const int64_t tok = bos + t;
                kda_step(S, K, V, k + ((size_t)tok * H + h) * K, v + ((size_t)tok * H + h) * V,
                         graw + ((size_t)tok * H + h) * K, beta[tok * H + h], u);
                if (o) {
                    const double *qq = q + ((size_t)tok * H + h) * K;
                    double *oo = o + ((size_t)tok * H + h) * V;
                    for (int j = 0; j < V; j++) {
                        double s = 0;
                        for (int i = 0; i < K; i++) s += S[i * V + j] * qq[i];
                        oo[j] = p->scale * s;
                    }
                }
            }
            if (ht) memcpy(ht + ((size_t)n * H + h) * K * V, S, sizeof(double) * K * V);
            free(u);
            free(S);
        }
    return 0;
}

/* O-KF: reverse-time gradients of L = Σ_t <dO_t, o_t> + <dht, S_T> for the KDA
 * recurrence, derived by hand from the step above (X, u as there):
 *   dS_t += scale q_t dO_tᵀ,        dq_t = scale S_t dO_t
 *   du = b dS_tᵀ k,  dv_t = du,     db_t = kᵀ dS_t u
 *   dk_t = b dS_t u − X du,         dX = dS_t − k duᵀ
 *   dĝ_t = rowsum(dX ⊙ X),          dS_{t−1} = diag(a_t) dX
 * States are checkpointed every CKPT tokens and recomputed per segment.      */
int orc_kda_bwd_token(const orc_problem *p, const double *q, const double *k, const double *v, const double *graw,
                      const double *beta, const double *h0, const double *dO, const double *dht,
                      double *dq, double *dk, double *dv, double *dg, double *dbeta, double *dh0) {
    const int K = p->K, V = p->V, H = p->HV;
    const int NS = orc_num_seqs(p);
    if (p->HK != p->HV) return -1;
    #pragma omp parallel for schedule(dynamic) collapse(2)
    for (int n = 0; n < NS; n++)
        for (int h = 0; h < H; h++) {
            int64_t bos, len; seq_range(p, n, &bos, &len);
            const size_t KV = (size_t)K * V;
            const int64_t nck = (len + CKPT - 1) / CKPT;
            double *ck = (double *)malloc(sizeof(double) * KV * (nck > 0 ? nck : 1));
            double *seg = (double *)malloc(sizeof(double) * KV * (CKPT + 1));
            double *dS = (double *)malloc(sizeof(double) * KV);
            double *X = (double *)malloc(sizeof(double) * KV);
            double *u = (double *)malloc(sizeof(double) * V);
            double *du = (double *)malloc(sizeof(double) * V);
            double *w = (double *)malloc(sizeof(double) * V);
            double *S = seg;
            if (h0) memcpy(S, h0 + ((size_t)n * H + h) * KV, sizeof(double) * KV);
            else memset(S, 0, sizeof(double) * KV);
            for (int64_t t = 0; t < len; t++) {
                if (t % CKPT == 0) memcpy(ck + (t / CKPT) * KV, S, sizeof(double) * KV);
                const int64_t tok = bos + t;
                kda_step(S, K, V, k + ((size_t)tok * H + h) * K, v + ((size_t)tok * H + h) * V,
                         graw + ((size_t)tok * H + h) * K, beta[tok * H + h], w);
            }
            if (dht) memcpy(dS, dht + ((size_t)n * H + h) * KV, sizeof(double) * KV);
            else memset(dS, 0, sizeof(double) * KV);
            for (int64_t sgi = nck - 1; sgi >= 0; sgi--) {
                const int64_t t0 = sgi * CKPT, t1 = t0 + CKPT < len ? t0 + CKPT : len;
                memcpy(seg, ck + sgi * KV, sizeof(double) * KV);
                for (int64_t t = t0; t < t1; t++) {
                    const int64_t tok = bos + t;
                    double *Sn = seg + (t - t0 + 1) * KV;
                    memcpy(Sn, seg + (t - t0) * KV, sizeof(double) * KV);
                    kda_step(Sn, K, V, k + ((size_t)tok * H + h) * K, v + ((size_t)tok * H + h) * V,
                             graw + ((size_t)tok * H + h) * K, beta[tok * H + h], w);
                }
                for (int64_t t = t1 - 1; t >= t0; t--) {
                    const int64_t tok = bos + t;
                    const double *St = seg + (t - t0 + 1) * KV, *Sp = seg + (t - t0) * KV;
                    const double *qq = q + ((size_t)tok * H + h) * K, *kk = k + ((size_t)tok * H + h) * K;
                    const double *vv = v + ((size_t)tok * H + h) * V, *dd = dO + ((size_t)tok * H + h) * V;
                    const double *ga = graw + ((size_t)tok * H + h) * K;
                    const double b = beta[tok * H + h];
                    for (int i = 0; i < K; i++)
                        for (int j = 0; j < V; j++) dS[i * V + j] += p->scale * qq[i] * dd[j];
                    double *dqq = dq + ((size_t)tok * H + h) * K;
                    for (int i = 0; i < K; i++) {
                        double s = 0;
                        for (int j = 0; j < V; j++) s += St[i * V + j] * dd[j];
                        dqq[i] = p->scale * s;
                    }
                    /* X = diag(a) S_{t−1}, u = v − Xᵀk */
                    for (int i = 0; i < K; i++) {
                        const double a = exp(ga[i]);
                        for (int j = 0; j < V; j++) X[i * V + j] = a * Sp[i * V + j];
                    }
                    for (int j = 0; j < V; j++) {
                        double s = 0, s2 = 0;
                        for (int i = 0; i < K; i++) { s += X[i * V + j] * kk[i]; s2 += dS[i * V + j] * kk[i]; }
                        u[j] = vv[j] - s;
                        du[j] = b * s2;
                    }
                    double *dvv = dv + ((size_t)tok * H + h) * V;
                    for (int j = 0; j < V; j++) dvv[j] = du[j];
                    double db = 0;
                    double *dkk = dk + ((size_t)tok * H + h) * K;
                    for (int i = 0; i < K; i++) {
                        double su = 0, xd = 0;
                        for (int j = 0; j < V; j++) { su += dS[i * V + j] * u[j]; xd += X[i * V + j] * du[j]; }
                        db += kk[i] * su;
                        dkk[i] = b * su - xd;
                    }
                    dbeta[tok * H + h] = db;
                    double *dgg = dg + ((size_t)tok * H + h) * K;
                    for (int i = 0; i < K; i++) {
                        const double a = exp(ga[i]);
                        double s = 0;
                        for (int j = 0; j < V; j++) {
                            const double dx = dS[i * V + j] - kk[i] * du[j];
                            s += dx * X[i * V + j];
                            dS[i * V + j] = a * dx;
                        }
                        dgg[i] = s;
                    }
                }
            }
            if (dh0) memcpy(dh0 + ((size_t)n * H + h) * KV, dS, sizeof(double) * KV);
            free(w); free(du); free(u); free(X); free(dS); free(seg); free(ck);
        }
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
