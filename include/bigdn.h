/*
 * bigdn.h -- C ABI of the BiGDN chunkwise layer (frame-level bidirectional
 * gated delta rule with a normaliser stream) on MI355X (gfx950): its forward
 * output and its backward.
 *
 * Source page: Sana `fused_gdn_chunkwise_bwd.py` (BiGDN chunkwise backward):
 * `FusedBiGDNChunkwiseFunction` forward/backward, phase C̄ (`_phase_c_bwd_kernel`),
 * phase B̄ (`_phase_b_bidi_bwd_pytorch`), `combine_bidi_dA_dP_dg`, phase Ā
 * (`_phase_a_kv_bwd_kernel`, `_phase_a_z_bwd_kernel`), `output_divide_bwd`,
 * `fused_rope_relu_fwd` / `fused_rope_unrope_bwd` and the RMSNorm backward.
 *
 * Layer, per batch row b and head h, with N = F*S tokens in F frames of S
 * tokens, C = H*D channels:
 *   Qn = q * r_q * w_q, r_q = (sum_C q^2 / C + norm_eps)^(-1/2) over ALL heads
 *   (the same for k); Qu = relu(Qn), Ku = k_scale * relu(Kn);
 *   Qr = rope(Qu), Kr = rope(Ku), rope(X) = X*cos + pairflip(X)*sin with
 *   pairflip swapping channels 2i and 2i+1;
 *   P_f = Kr^T diag(beta) Kr, A_f = Kr^T diag(beta) V, Pz_f = Ku^T diag(beta) Ku,
 *   Bz_f = Ku^T beta over the tokens of frame f;
 *   Mf[f] = g_f (I - P_f) Mf[f-1] + A_f (Mf[-1] = 0);
 *   Mr[F-1] = 0, Mr[f-1] = g_f (I - P_f) Mr[f] + A_f; the same for z with (Pz, Bz);
 *   out = Qr (Mf[f] + Mr[f]) / (Qu . (zf[f] + zr[f]) + eps)   (g = decay).
 * The backward returns the gradients of sum(dout * out) w.r.t. qkv, beta,
 * decay and both norm weights.  Precision: bf16 activations, bf16 MFMA
 * operands with fp32 accumulation, fp32 states (as on the page, phase C̄ and
 * phase Ā comments).
 *
 * Conventions: device pointers, contiguous row-major; asynchronous on
 * `stream`; validation on the host before any launch (on error nothing is
 * launched and no output is written); status codes of gdr.h.  The library
 * allocates nothing: scratch comes from the caller's workspace of at least
 * bigdn_workspace_size() bytes (256-byte aligned), which the call overwrites.
 */
#ifndef BIGDN_H_
#define BIGDN_H_

#include "gdr.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bigdn_problem {
    int B;            /* batch rows (>= 1) */
    int F, S;         /* frames per row and tokens per frame (>= 1 each); N = F*S */
    int H, D;         /* heads and head dimension; D in {64, 128}, H*D <= 4096 */
    float k_scale;    /* key scale applied after the ReLU */
    float norm_eps;   /* RMSNorm epsilon (>= 0) */
    float eps;        /* output-divide epsilon (> 0) */
} bigdn_problem;

/* Bytes of workspace bigdn_fwd (bwd = 0) or bigdn_bwd (bwd != 0) needs; 0 if
 * the problem is invalid or unsupported. */
size_t bigdn_workspace_size(const bigdn_problem *p, int bwd);

/*
 * bigdn_fwd -- the layer output (the page's `FusedBiGDNChunkwiseFunction.forward`).
 *   qkv     bf16 [B, N, 3, H, D]   q, k, v of each token (q and k un-normalised)
 *   beta    fp32 [B, H, F, S]      write strength per token
 *   decay   fp32 [B, H, F]         frame decay g
 *   q_norm_weight, k_norm_weight   fp32 [H*D]
 *   rope_cos, rope_sin             fp32 [N, D]  (position n = f*S + s)
 *   out     bf16 [B, N, H, D]      written
 * Returns GDR_ERR_INVALID for a bad size or NULL pointer, GDR_ERR_UNSUPPORTED
 * for D not in {64, 128} or H*D > 4096, GDR_ERR_WORKSPACE for a short
 * workspace, GDR_ERR_LAUNCH if HIP reports a launch error.
 */
int bigdn_fwd(const bigdn_problem *p, const void *qkv, const float *beta, const float *decay,
              const float *q_norm_weight, const float *k_norm_weight, const float *rope_cos, const float *rope_sin,
              void *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * bigdn_bwd -- the layer backward (the page's `FusedBiGDNChunkwiseFunction.backward`),
 * recomputing the norms, the per-frame sums and both frame scans from the inputs.
 *   inputs as bigdn_fwd, plus dout bf16 [B, N, H, D]
 *   dqkv          bf16 [B, N, 3, H, D]  gradient w.r.t. qkv (before the norm)
 *   dbeta         fp32 [B, H, F, S]
 *   ddecay        fp32 [B, H, F]
 *   dq_norm_weight, dk_norm_weight  fp32 [H*D]
 * Every output is overwritten (no accumulation).  Errors as bigdn_fwd.
 */
int bigdn_bwd(const bigdn_problem *p, const void *qkv, const float *beta, const float *decay,
              const float *q_norm_weight, const float *k_norm_weight, const float *rope_cos, const float *rope_sin,
              const void *dout, void *dqkv, float *dbeta, float *ddecay, float *dq_norm_weight,
              float *dk_norm_weight, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * bigdn_fwd_events / bigdn_bwd_events -- the same calls for measurement tools.
 * `events` (NULL or caller-created hipEvent_t) are recorded on `stream`:
 * [0] start, [1] after the norm statistics, [2] after the per-frame sums,
 * [3] after the state scans, [4] after the output / divide-VJP kernel; the
 * backward adds [5] after the gradient scans, [6] after the combine and
 * phase-Ā kernel, [7] after the RMSNorm backward (5 events forward, 8 backward).
 */
int bigdn_fwd_events(const bigdn_problem *p, const void *qkv, const float *beta, const float *decay,
                     const float *q_norm_weight, const float *k_norm_weight, const float *rope_cos,
                     const float *rope_sin, void *out, void *ws, size_t ws_bytes, hipStream_t stream,
                     hipEvent_t *events);
int bigdn_bwd_events(const bigdn_problem *p, const void *qkv, const float *beta, const float *decay,
                     const float *q_norm_weight, const float *k_norm_weight, const float *rope_cos,
                     const float *rope_sin, const void *dout, void *dqkv, float *dbeta, float *ddecay,
                     float *dq_norm_weight, float *dk_norm_weight, void *ws, size_t ws_bytes, hipStream_t stream,
                     hipEvent_t *events);

#ifdef __cplusplus
}
#endif

#endif /* BIGDN_H_ */
