/*
 * gdr.h -- C ABI of the MI355X (gfx950) gated-delta-rule library: the chunked
 * backward, and the chunked forward it differentiates.
 *
 * Method (gated delta rule, state S_t is K x V per sequence and value head):
 *     S_t = a_t (I - b_t k_t k_tᵀ) S_{t-1} + b_t k_t v_tᵀ ,  a_t = exp(ĝ_t)
 *     o_t = scale * S_tᵀ q_t
 * The backward returns the gradients of  L = Σ_t <dO_t, o_t> + <dht, S_T>.
 *
 * Page references (by title and section):
 *  [P1] "FlashQLA 反向传播全解：fused_gdr_bwd 与 dh 梯度 Kernel 的设计取舍"
 *       -- §一: entry point, the gate arrives as its in-chunk cumulative sum and
 *       the gate gradient is reverse-cumsummed at the end, dh0 accumulated and
 *       returned in fp32, dq/dk/dv stored in the 16-bit input type, dht optional
 *       (absent == zero); step ② recomputes the per-chunk states h; §二: one
 *       backward produces dq, dk, dv, dg, db, dh0 walking chunks last-to-first.
 *  [P2] "chunk_kda_bwd_wy_dqkg_fused 算子" -- 函数签名 / 参数说明: argument list,
 *       shapes and dtypes of the KDA WY backward stage; 实现原理: its intermediates.
 *
 * Conventions for every call:
 *  - Tensors are caller-owned, contiguous, row-major DEVICE pointers unless a
 *    parameter says "host".  The library keeps no pointer after a call returns
 *    and never allocates device memory; scratch comes from a caller-provided
 *    workspace whose size is given by gdr_workspace_size().
 *  - The token axis is flattened over the batch: a [B,T,H,D] tensor is passed as
 *    [B*T,H,D].  With varlen (cu_seqlens != NULL) B must be 1 and sequence n is
 *    tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *  - Value head hv reads key head hv / (HV/HK) (grouped-query layout).
 *  - Calls are asynchronous on the given stream (NULL = default stream); inputs
 *    must stay valid and outputs untouched until the stream reaches the call.
 *  - Return value: GDR_OK (0) or a negative gdr_status.  Validation happens on
 *    the host before anything is launched; on error nothing is launched and no
 *    output is written.  gdr_strerror() maps a status to a string.
 *  - Reentrant: no global mutable state (a per-device attribute cache only).
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDR_F32 = 0, GDR_F16 = 1, GDR_BF16 = 2 } gdr_dtype;

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID = -1,     /* bad shape, dtype, null required pointer, bad cu_seqlens */
    GDR_ERR_UNSUPPORTED = -2, /* valid but not built: K != V, K not in {64,128}, BT != 64 */
    GDR_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than gdr_workspace_size() */
    GDR_ERR_LAUNCH = -4,      /* a HIP error was reported at launch */
    GDR_ERR_SCRATCH = -5      /* gdr_chunk_bwd_noalloc: the problem needs more workspace than
                                 GDR_NOALLOC_SCRATCH_BYTES */
} gdr_status;

typedef struct gdr_problem {
    int B, T;      /* batch and tokens per sequence (dense); varlen: B = 1, T = total tokens */
    int HK, HV;    /* key/query heads and value heads; HV % HK == 0 */
    int K, V;      /* key and value head dims */
    int BT;        /* chunk size */
    int N;         /* number of sequences when varlen; ignored when cu_seqlens == NULL */
    const int32_t *cu_seqlens;      /* device [N+1] or NULL (dense) */
    const int32_t *cu_seqlens_host; /* host mirror of cu_seqlens [N+1]; required iff cu_seqlens != NULL.
                                       It must hold the same values; it is read during the call only. */
    float scale;   /* output scale; <= 0 selects 1/sqrt(K) */
    gdr_dtype dtype; /* type of q, k, v, beta, dO and of dq, dk, dv */
    int seg_chunks;  /* chunks per segment of the sequential state scans (16-bit types): each
                        sequence is cut into segments that are scanned in parallel and joined
                        exactly by their transfer matrices.  0 = chosen from the chunk counts and
                        the head count; < 0 = never segment.  fp32 problems are never segmented.
                        Results agree up to rounding for every value. */
} gdr_problem;

/* Human-readable text for a gdr_status (static storage). */
const char *gdr_strerror(int status);

/* Number of chunks NT = sum over sequences of ceil(len / BT); -1 if invalid. */
int64_t gdr_num_chunks(const gdr_problem *p);

/* Workspace bytes needed by gdr_fwd_states / gdr_chunk_fwd / gdr_chunk_bwd for this problem
 * (0 if the problem is invalid).  The same workspace may be reused by later
 * calls on the same stream. */
size_t gdr_workspace_size(const gdr_problem *p);

/*
 * gdr_fwd_states -- recompute the per-chunk forward states ([P1] §一 step ②).
 *   k [B*T,HK,K], v [B*T,HV,V], beta [B*T,HV]    dtype
 *   g_cum [B*T,HV] fp32    in-chunk cumulative log-gate (restarts every BT tokens
 *                          and at every sequence start)
 *   h0 [N,HV,K,V] fp32     initial states, NULL = zero
 * Outputs:
 *   h_out  [NT,HV,K,V] fp32   state ENTERING each chunk (chunk-major over sequences)
 *   v_new_out [B*T,HV,V] dtype or NULL   the chunk's corrected values U - W h
 *   ht_out [N,HV,K,V] fp32 or NULL       final state of each sequence
 * ws/ws_bytes: workspace (>= gdr_workspace_size(p)).
 */
int gdr_fwd_states(const gdr_problem *p, const void *k, const void *v, const float *g_cum, const void *beta,
                   const float *h0, float *h_out, void *v_new_out, float *ht_out,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * gdr_gate_cumsum -- the gate in the form the chunked forward saves for the
 * backward ([P1] §一: in-chunk cumulative sum of the raw log-gate).
 *   g     [B*T,HV] fp32   raw per-token log-gate ĝ_t
 *   g_cum [B*T,HV] fp32   output: Σ ĝ_s over the tokens s <= t of t's chunk
 *                         (chunks of BT tokens, restarting at every sequence start)
 * Each element is accumulated in fp32 in token order starting from the chunk's
 * first token, so the result is bit-identical to a serial fp32 in-chunk scan.
 * g and g_cum must not overlap.  No workspace; errors as for every call.
 */
int gdr_gate_cumsum(const gdr_problem *p, const float *g, float *g_cum, hipStream_t stream);

/*
 * gdr_chunk_fwd -- the chunked forward of the gated delta rule: outputs o_t and
 * the final states S_T of the recurrence above ([P1] §一: the forward whose
 * saved gate and states the backward consumes).
 * Inputs:
 *   q, k [B*T,HK,K]  v [B*T,HV,V]  beta [B*T,HV]   dtype
 *   g_cum [B*T,HV] fp32     in-chunk cumulative log-gate (gdr_gate_cumsum)
 *   h0 [N,HV,K,V] fp32      initial states, NULL = zero
 * Outputs:
 *   o [B*T,HV,V] dtype      written in full
 *   ht_out [N,HV,K,V] fp32 or NULL (skip)
 * ws/ws_bytes: workspace (>= gdr_workspace_size(p)); it holds the per-chunk
 * states afterwards but nothing in it is part of the contract.
 * Per chunk, with W, U from the WY factors and h[c] the state entering it:
 *   o = scale·diag(γ) Q h[c] + scale·lower(Γ ⊙ Q Kᵀ) (U − W h[c]).
 * Precision as for gdr_chunk_bwd (16-bit inputs: fp16 operands, fp32 accumulate;
 * the per-chunk states are held in the input type between the scan and the
 * output kernel).
 */
int gdr_chunk_fwd(const gdr_problem *p, const void *q, const void *k, const void *v, const float *g_cum,
                  const void *beta, const float *h0, void *o, float *ht_out, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/*
 * gdr_chunk_fwd_events -- gdr_chunk_fwd for measurement tools.  Identical
 * computation and arguments; `events` (NULL or 4 caller-created hipEvent_t)
 * are recorded on `stream` before the first launch and after each of the three
 * stages: [0] start, [1] after the chunk table and WY-factor kernel, [2] after
 * the forward state scan, [3] after the output kernel.
 */
int gdr_chunk_fwd_events(const gdr_problem *p, const void *q, const void *k, const void *v, const float *g_cum,
                         const void *beta, const float *h0, void *o, float *ht_out, void *ws, size_t ws_bytes,
                         hipStream_t stream, hipEvent_t *events);

/*
 * gdr_chunk_bwd -- the backward of the chunkwise gated delta rule ([P1] §一, §二).
 * Inputs:
 *   q, k [B*T,HK,K]  v, dO [B*T,HV,V]  beta [B*T,HV]   dtype
 *   g_cum [B*T,HV] fp32     in-chunk cumulative log-gate, as for gdr_fwd_states
 *   h0  [N,HV,K,V] fp32     initial states, NULL = zero
 *   dht [N,HV,K,V] fp32     gradient of the final states, NULL = zero (identical
 *                           to passing zeros)
 * Outputs (all written in full):
 *   dq, dk [B*T,HK,K] dtype   summed over the value heads of each key head
 *   dv [B*T,HV,V] dtype
 *   dg [B*T,HV] fp32          gradient w.r.t. the RAW per-token log-gate ĝ_t
 *                             (already reverse-cumsummed inside each chunk)
 *   dbeta [B*T,HV] fp32
 *   dh0 [N,HV,K,V] fp32 or NULL (skip)
 * ws/ws_bytes: workspace (>= gdr_workspace_size(p)).
 * Precision: matrix products run on MFMA with fp32 accumulation; fp32 inputs
 * use fp32 operands throughout.  16-bit inputs use 16-bit operands; the state
 * scans use fp16 operands:
 *  - the reverse (dh) scan runs on s·dO and s·dht with s a power of two per
 *    (sequence, value head) that maps max(|dO|, |dht|) into [1/2, 1), so the
 *    magnitude of dO and dht is free (tested at x1e-9 .. x256 of randn);
 *  - the forward scan narrows the WY factors W, U = A·diag(β)·V and the state
 *    to fp16, so v must stay within fp16 range, |v| below about 1e4 in
 *    practice (tested at 256·randn with a slow gate over T = 4096).
 */
int gdr_chunk_bwd(const gdr_problem *p, const void *q, const void *k, const void *v, const float *g_cum,
                  const void *beta, const float *h0, const void *dO, const float *dht,
                  void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * gdr_chunk_bwd_events -- gdr_chunk_bwd for measurement tools.  Identical
 * computation and arguments; `events` (NULL or 4 caller-created hipEvent_t)
 * are recorded on `stream` before the first launch and after each of the three
 * stages: [0] start, [1] after the chunk table, the dO scale pass (16-bit
 * problems) and the WY-factor kernel, [2] after the two chunk scans, [3] after
 * the gradient kernel.  hipEventElapsedTime on
 * consecutive pairs gives the per-stage GPU time of this call.
 */
int gdr_chunk_bwd_events(const gdr_problem *p, const void *q, const void *k, const void *v, const float *g_cum,
                         const void *beta, const float *h0, const void *dO, const float *dht,
                         void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                         void *ws, size_t ws_bytes, hipStream_t stream, hipEvent_t *events);

/*
 * kda_chunk_bwd -- the KDA (per-channel gate) WY backward stage ([P2] 函数签名,
 * 参数说明, 实现原理).  Requires HK == HV == H; dtype F16 or F32 (the page
 * validates fp16/fp32 only; F32 is built at K = V = 64, F16 at 64 and 128;
 * chunk length BT = 16 or 64, the two the page validates; anything else
 * returns GDR_ERR_UNSUPPORTED before any launch).  Per chunk of C <= BT rows, with γ = exp(g):
 * returns the gradients of
 *   scale<dO,(Q⊙γ)h> + <dh,(K⊙γ_C/γ)ᵀV_new> + <dh,diag(γ_C)h> + <dv,A(β⊙V) - A(β⊙γ⊙K)h>
 * with respect to q, k, v, beta, g and the strictly-lower L of A = (I+L)^{-1}.
 * Inputs:
 *   q, k [B*T,H,K]   v, v_new, dO, dv_in [B*T,H,V]   beta [B*T,H]   dtype
 *   g [B*T,H,K] fp32 (per-channel in-chunk log-gate, used as given)
 *   A [B*T,H,BT] dtype (row r of a chunk holds that chunk's lower-triangular
 *                       matrix row; entries above the diagonal are ignored)
 *   h, dh [NT,H,K,V] fp32 (state entering / gradient of state leaving each chunk)
 * Outputs: dq, dk, dg [B*T,H,K] fp32; dv_out [B*T,H,V] dtype; db [B*T,H] fp32;
 *   dA [B*T,H,BT] fp32 (strictly-lower part; zeros on and above the diagonal
 *   and in columns beyond a partial chunk's length).
 * No workspace.
 */
int kda_chunk_bwd(const gdr_problem *p, const void *q, const void *k, const void *v, const void *v_new,
                  const float *g, const void *beta, const void *A, const float *h, const void *dO,
                  const float *dh, const void *dv_in, float *dq, float *dk, void *dv_out, float *db,
                  float *dg, float *dA, hipStream_t stream);

/*
 * kda_chunk_bwd_full -- the whole chunked backward of KDA, the gated delta rule
 * with a per-channel gate ([P2] 概述: the operator above is the "WY
 * representation gradient" stage of this backward; the other steps -- state
 * recomputation, the per-channel dh scan, the intra-chunk attention and dL
 * distribution -- run around it here).  Recurrence, per sequence and head
 * (HK == HV == H), gate a_t = exp(ĝ_t) in R^K:
 *     S_t = (I - b_t k_t k_tᵀ) diag(a_t) S_{t-1} + b_t k_t v_tᵀ,   o_t = scale S_tᵀ q_t
 * Returns the gradients of L = Σ_t <dO_t, o_t> + <dht, S_T>.
 * Inputs:
 *   q, k [B*T,H,K]  v, dO [B*T,H,V]  beta [B*T,H]   dtype (F16; F32 at K = 64)
 *   g_cum [B*T,H,K] fp32   in-chunk cumulative per-channel log-gate (restarts
 *                          every BT tokens and at every sequence start;
 *                          gdr_gate_cumsum with HV = H*K computes it)
 *   h0, dht [N,H,K,V] fp32 or NULL (zero)
 * Outputs (written in full): dq, dk [B*T,H,K] and dv [B*T,H,V] in dtype;
 *   dg [B*T,H,K] fp32 (w.r.t. the RAW per-channel gate, reverse-cumsummed in
 *   each chunk); dbeta [B*T,H] fp32; dh0 [N,H,K,V] fp32 or NULL (skip).
 * ws/ws_bytes: workspace (>= kda_workspace_size(p)).
 * Errors: GDR_ERR_INVALID if HK != HV; GDR_ERR_UNSUPPORTED for bf16, BT != 64,
 * K != V, K not in {64, 128}, fp32 at K = 128.
 * Precision: gated intra-chunk products in fp32 (each factor e^{±(G − m)} with m
 * the chunk's middle gate row; each channel's in-chunk gate span must stay
 * below about 170), other products fp16 operands with fp32 accumulation.
 */
size_t kda_workspace_size(const gdr_problem *p);
int kda_chunk_bwd_full(const gdr_problem *p, const void *q, const void *k, const void *v, const float *g_cum,
                       const void *beta, const float *h0, const void *dO, const float *dht,
                       void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * kda_chunk_bwd_full_events -- kda_chunk_bwd_full for measurement tools; `events`
 * (NULL or 5 caller-created hipEvent_t) are recorded on `stream` at the start
 * and after the WY factors, the two state scans, the WY stage and the
 * intra-chunk kernel.
 */
int kda_chunk_bwd_full_events(const gdr_problem *p, const void *q, const void *k, const void *v,
                              const float *g_cum, const void *beta, const float *h0, const void *dO,
                              const float *dht, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                              float *dh0, void *ws, size_t ws_bytes, hipStream_t stream, hipEvent_t *events);

/*
 * gdr_chunk_bwd_noalloc -- gdr_chunk_bwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same inputs, outputs,
 * computation and status codes as gdr_chunk_bwd; the workspace is a fixed
 * device array of GDR_NOALLOC_SCRATCH_BYTES inside the library (one per GPU,
 * held until the process ends).  This call allocates nothing: it makes no
 * hipMalloc / hipFree and calls no allocating routine.
 * Limit: problems with gdr_workspace_size(p) > GDR_NOALLOC_SCRATCH_BYTES are
 * rejected with GDR_ERR_SCRATCH before anything is launched (at K = V = 128 and
 * a 16-bit dtype the workspace is about 136 KB per (chunk, value head), e.g.
 * T = 4096 with 16 value heads fits).
 * Concurrency: every call on one GPU uses that GPU's single array, so calls
 * that overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller; consecutive calls on one stream are safe.
 * No part of the array needs to start at zero: every call writes what it reads.
 * gdr_noalloc_init() resolves the array's address on the current device (the
 * first call on a device does it too); it returns GDR_ERR_LAUNCH if that fails.
 */
#define GDR_NOALLOC_SCRATCH_BYTES (128u << 20)
int gdr_noalloc_init(void);
int gdr_chunk_bwd_noalloc(const gdr_problem *p, const void *q, const void *k, const void *v, const float *g_cum,
                          const void *beta, const float *h0, const void *dO, const float *dht,
                          void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GDR_H_ */
