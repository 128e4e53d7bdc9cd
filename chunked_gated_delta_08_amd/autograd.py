"""torch.autograd wrapper around the library's chunked forward and backward.

FlashQLA backward explainer §一: the chunked gated delta rule is exposed to
training code as one autograd function; its forward saves the gate as the
in-chunk cumulative sum and its backward consumes that saved form.  Here the
forward is gdr_gate_cumsum + gdr_chunk_fwd and the backward is gdr_chunk_bwd
(states recomputed, not stored).  Argument marshalling only: every arithmetic
step runs in the library's kernels.

Layouts follow the C ABI (token axis flattened over the batch):
  q, k [B*T, HK, K]   v [B*T, HV, V]   g (raw log-gate) [B*T, HV] fp32
  beta [B*T, HV]      initial_state [N, HV, K, V] fp32
"""
import torch

from . import binding


class ChunkGatedDeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, h0, scale, cu_seqlens, B, BT, seg_chunks):
        q, k, v, g, beta = (t.contiguous() for t in (q, k, v, g, beta))
        h0 = None if h0 is None else h0.contiguous()
        g_cum = binding.gdr_gate_cumsum(g, cu_seqlens=cu_seqlens, B=B, BT=BT)
        out = binding.gdr_chunk_fwd(q, k, v, g_cum, beta, h0=h0, cu_seqlens=cu_seqlens, B=B, scale=scale, BT=BT,
                                    seg_chunks=seg_chunks)
        ctx.save_for_backward(q, k, v, g_cum, beta, h0, cu_seqlens)
        ctx.cfg = (scale, B, BT, seg_chunks)
        return out["o"], out["ht"]

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, g_cum, beta, h0, cu_seqlens = ctx.saved_tensors
        scale, B, BT, seg_chunks = ctx.cfg
        r = binding.gdr_chunk_bwd(q, k, v, g_cum, beta, do.contiguous(), dht=None if dht is None else dht.contiguous(),
                                  h0=h0, cu_seqlens=cu_seqlens, B=B, scale=scale, BT=BT,
                                  want_dh0=h0 is not None and ctx.needs_input_grad[5], seg_chunks=seg_chunks)
        return r["dq"], r["dk"], r["dv"], r["dg"], r["dbeta"].to(beta.dtype), r["dh0"], None, None, None, None, None


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, B=1, BT=64,
                           seg_chunks=0):
    """o, final_state = chunked gated delta rule over the raw log-gate `g` (fp32).

    Differentiable in q, k, v, g, beta and initial_state.  cu_seqlens: int32 CUDA
    tensor [N+1] (varlen; then the batch is 1) or None.  The final state is fp32."""
    return ChunkGatedDeltaRule.apply(q, k, v, g, beta, initial_state, scale, cu_seqlens, B, BT, seg_chunks)
