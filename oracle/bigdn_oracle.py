"""fp64 CPU oracle of the BiGDN chunkwise layer (bidirectional, frame-level gated
delta rule) and its hand-derived backward.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline leg
of bench.py may import this module.  It shares no code with the HIP path and
never imports the library package.

Source: Sana `fused_gdn_chunkwise_bwd.py` (the BiGDN chunkwise backward page).
The page prints the backward phases only; the forward it differentiates is read
off them (phase Ā-KV / Ā-Z fix P, A, P_z, B_z; phase B̄ and
`combine_bidi_dA_dP_dg` fix both frame scans and the reverse scan's exclusive
start; phase C̄ and the output-divide VJP fix num, den and the output; the
rope/relu kernels and the RMSNorm backward fix the input transforms).

Layouts (the page's): qkv [B, N, 3, H, D] with N = F*S tokens, frame f holding
tokens f*S .. f*S+S-1; beta [B, H, F, S]; decay [B, H, F]; q/k norm weights
[H*D]; rope cos/sin [F*S, D]; out and dout [B, N, H, D].

Forward, per (b, h):
  r_q = (sum_c q^2 / C + norm_eps)^(-1/2) over all C = H*D channels of a token
  Qn = q r_q w_q;  Kn = k r_k w_k
  Qu = relu(Qn);   Ku = k_scale relu(Kn)          (normaliser stream operands)
  Qr = rope(Qu);   Kr = rope(Ku)                  (key-value stream operands)
  rope(X) = X cos + pairflip(X) sin,  pairflip swaps channels d and d^1
  per frame f:  P_f = Kr^T diag(beta) Kr,  A_f = Kr^T diag(beta) V,
                Pz_f = Ku^T diag(beta) Ku,  Bz_f = Ku^T beta
  forward scan (inclusive):  Mf[f] = g_f (I - P_f) Mf[f-1] + A_f,  Mf[-1] = 0
  reverse scan (exclusive):  Mr[F-1] = 0,  Mr[f-1] = g_f (I - P_f) Mr[f] + A_f
  the same two scans for the vector z with (Pz, Bz)
  num_t = Qr_t (Mf[f] + Mr[f]);  den_t = Qu_t . (zf[f] + zr[f])
  out_t = num_t / (den_t + eps)
"""
import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def pairflip(x):
    """Swap channels (2i, 2i+1) along the last axis (rope helpers on the page)."""
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 1::2]
    y[..., 1::2] = x[..., 0::2]
    return y


def rope(x, cos, sin):
    """x [..., N, D] with cos/sin [N, D]: x*cos + pairflip(x)*sin (`_apply_rope`)."""
    return x * cos + pairflip(x) * sin


def unrope(dy, cos, sin):
    """VJP of rope: dy*cos + pairflip(dy*sin) (`_unrope`)."""
    return dy * cos + pairflip(dy * sin)


def _bhfsd(x, F, S):
    """[B, N, H, D] -> [B, H, F, S, D]."""
    B, N, H, D = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, H, F, S, D)


def _bnhd(x):
    """[B, H, F, S, D] -> [B, N, H, D]."""
    B, H, F, S, D = x.shape
    return x.reshape(B, H, F * S, D).transpose(0, 2, 1, 3)


def _transforms(qkv, qw, kw, cos, sin, F, S, k_scale, norm_eps):
    """RMSNorm over all channels of a token, ReLU, k_scale and RoPE
    (`FusedBiGDNChunkwiseFunction.forward`, `fused_rope_relu_fwd`)."""
    qkv = _f64(qkv)
    B, N, _, H, D = qkv.shape
    C = H * D
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    rq = 1.0 / np.sqrt((q * q).sum(axis=(2, 3)) / C + norm_eps)      # [B, N]
    rk = 1.0 / np.sqrt((k * k).sum(axis=(2, 3)) / C + norm_eps)
    wq = _f64(qw).reshape(H, D)
    wk = _f64(kw).reshape(H, D)
    Qn = q * rq[:, :, None, None] * wq
    Kn = k * rk[:, :, None, None] * wk
    Qu = np.maximum(Qn, 0.0)
    Ku = np.maximum(Kn, 0.0) * k_scale
    cs, sn = _f64(cos), _f64(sin)
    Qr = rope(Qu.transpose(0, 2, 1, 3), cs, sn).transpose(0, 2, 1, 3)
    Kr = rope(Ku.transpose(0, 2, 1, 3), cs, sn).transpose(0, 2, 1, 3)
    return dict(q=q, k=k, v=v, rq=rq, rk=rk, wq=wq, wk=wk, Qn=Qn, Kn=Kn, Qu=Qu, Ku=Ku, Qr=Qr, Kr=Kr,
                C=C, B=B, N=N, H=H, D=D)


def phase_a(Kr, Ku, V, beta):
    """Per-frame sums (phase Ā's forward): all [B, H, F, ...]."""
    Kb = np.swapaxes(Kr * beta[..., None], -1, -2)
    P = Kb @ Kr
    A = Kb @ V
    Kub = np.swapaxes(Ku * beta[..., None], -1, -2)
    Pz = Kub @ Ku
    Bz = Kub.sum(axis=-1)
    return P, A, Pz, Bz


def frame_scans(P, A, g):
    """Inclusive forward and exclusive reverse frame scans (phase B̄'s forward).
    P [B,H,F,D,D], A [B,H,F,D,E] (E = D for the state, E = 1 for z), g [B,H,F].
    Returns Mf, Mr [B,H,F,D,E]."""
    B, H, F, D, _ = P.shape
    I = np.eye(D)
    Mf = np.zeros_like(A)
    Mr = np.zeros_like(A)
    prev = np.zeros_like(A[:, :, 0])
    for f in range(F):
        prev = g[:, :, f, None, None] * ((I - P[:, :, f]) @ prev) + A[:, :, f]
        Mf[:, :, f] = prev
    for f in range(F - 1, 0, -1):
        Mr[:, :, f - 1] = g[:, :, f, None, None] * ((I - P[:, :, f]) @ Mr[:, :, f]) + A[:, :, f]
    return Mf, Mr


def bigdn_fwd(qkv, beta, decay, qw, kw, cos, sin, F, S, k_scale=1.0, norm_eps=1e-5, eps=1e-6, keep=False):
    """Layer output [B, N, H, D] (and, with keep=True, the intermediates)."""
    t = _transforms(qkv, qw, kw, cos, sin, F, S, k_scale, norm_eps)
    beta = _f64(beta)
    g = _f64(decay)
    Qr, Qu, Kr, Ku, V = (_bhfsd(t[n], F, S) for n in ("Qr", "Qu", "Kr", "Ku", "v"))
    P, A, Pz, Bz = phase_a(Kr, Ku, V, beta)
    Mf, Mr = frame_scans(P, A, g)
    zf, zr = frame_scans(Pz, Bz[..., None], g)
    Mc = Mf + Mr
    zc = (zf + zr)[..., 0]
    num = Qr @ Mc
    den = (Qu @ zc[..., None])[..., 0]
    out = num / (den[..., None] + eps)
    if not keep:
        return _bnhd(out)
    it = dict(t=t, Qr=Qr, Qu=Qu, Kr=Kr, Ku=Ku, V=V, P=P, A=A, Pz=Pz, Bz=Bz, Mf=Mf, Mr=Mr, zf=zf[..., 0],
              zr=zr[..., 0], num=num, den=den)
    return _bnhd(out), it


def frame_scans_bwd(dMc, P, Mf, Mr, g):
    """Reverse-mode through `frame_scans` given the gradient dMc of Mf + Mr.

    Forward scan: its state gradient runs backwards in f,
        Tf[f] = dMc[f] + g_{f+1} (I - P_{f+1})^T Tf[f+1];
    reverse scan: forwards in f,
        Tr[0] = dMc[0],  Tr[f] = dMc[f] + g_f (I - P_f)^T Tr[f-1];
    (phase B̄).  Per-frame parameter gradients (`combine_bidi_dA_dP_dg`):
        dA_f = Tf[f] + Tr[f-1]
        dP_f = -g_f (Tf[f] Mf[f-1]^T + Tr[f-1] Mr[f]^T)
        dg_f = <Tf[f], (I - P_f) Mf[f-1]> + <Tr[f-1], (I - P_f) Mr[f]>
    with the f-1 terms absent at f = 0."""
    B, H, F, D, _ = P.shape
    I = np.eye(D)
    IPt = np.swapaxes(I - P, -1, -2)
    Tf = np.zeros_like(dMc)
    Tr = np.zeros_like(dMc)
    Tf[:, :, F - 1] = dMc[:, :, F - 1]
    for f in range(F - 2, -1, -1):
        Tf[:, :, f] = dMc[:, :, f] + g[:, :, f + 1, None, None] * (IPt[:, :, f + 1] @ Tf[:, :, f + 1])
    Tr[:, :, 0] = dMc[:, :, 0]
    for f in range(1, F):
        Tr[:, :, f] = dMc[:, :, f] + g[:, :, f, None, None] * (IPt[:, :, f] @ Tr[:, :, f - 1])
    dA = Tf.copy()
    dA[:, :, 1:] += Tr[:, :, :-1]
    Mprev = np.zeros_like(Mf)
    Mprev[:, :, 1:] = Mf[:, :, :-1]
    gg = g[..., None, None]
    dP = -gg * (Tf @ np.swapaxes(Mprev, -1, -2))
    dP[:, :, 1:] -= gg[:, :, 1:] * (Tr[:, :, :-1] @ np.swapaxes(Mr[:, :, 1:], -1, -2))
    dg = (Tf * ((I - P) @ Mprev)).sum(axis=(-2, -1))
    dg[:, :, 1:] += (Tr[:, :, :-1] * ((I - P[:, :, 1:]) @ Mr[:, :, 1:])).sum(axis=(-2, -1))
    return dA, dP, dg


def bigdn_bwd(qkv, beta, decay, qw, kw, cos, sin, dout, F, S, k_scale=1.0, norm_eps=1e-5, eps=1e-6):
    """Gradients of sum(dout * out): dict dqkv [B,N,3,H,D], dbeta [B,H,F,S],
    ddecay [B,H,F], dqw, dkw [H*D]  (`FusedBiGDNChunkwiseFunction.backward`)."""
    _, it = bigdn_fwd(qkv, beta, decay, qw, kw, cos, sin, F, S, k_scale, norm_eps, eps, keep=True)
    t = it["t"]
    beta = _f64(beta)
    g = _f64(decay)
    B, H, C, D = t["B"], t["H"], t["C"], t["D"]
    dO = _bhfsd(_f64(dout), F, S)
    num, den = it["num"], it["den"]
    Mc = it["Mf"] + it["Mr"]
    zc = it["zf"] + it["zr"]
    Qr, Qu, Kr, Ku, V = it["Qr"], it["Qu"], it["Kr"], it["Ku"], it["V"]

    # output divide VJP
    dnum = dO / (den[..., None] + eps)
    dden = -(dO * num).sum(axis=-1) / (den + eps) ** 2
    # phase C̄: num = Qr Mc, den = Qu . zc
    dQr = dnum @ np.swapaxes(Mc, -1, -2)
    dMc = np.swapaxes(Qr, -1, -2) @ dnum
    dQu = dden[..., None] * zc[:, :, :, None, :]
    dzc = (dden[..., None] * Qu).sum(axis=3)
    # phase B̄ + combine, both streams
    dA, dP, dg_kv = frame_scans_bwd(dMc, it["P"], it["Mf"], it["Mr"], g)
    dBz, dPz, dg_z = frame_scans_bwd(dzc[..., None], it["Pz"], it["zf"][..., None], it["zr"][..., None], g)
    dBz = dBz[..., 0]
    # phase Ā-KV: P = Kr^T diag(beta) Kr, A = Kr^T diag(beta) V
    b_ = beta[..., None]
    dPs = dP + np.swapaxes(dP, -1, -2)
    KdPs = Kr @ dPs
    KdA = Kr @ dA
    dKr = b_ * (KdPs + V @ np.swapaxes(dA, -1, -2))
    dV = b_ * KdA
    dbeta = 0.5 * (KdPs * Kr).sum(-1) + (KdA * V).sum(-1)
    # phase Ā-Z: Pz = Ku^T diag(beta) Ku, Bz = Ku^T beta
    dPzs = dPz + np.swapaxes(dPz, -1, -2)
    KudPz = Ku @ dPzs
    dKu = b_ * (KudPz + dBz[:, :, :, None, :])
    dbeta = dbeta + 0.5 * (KudPz * Ku).sum(-1) + (Ku * dBz[:, :, :, None, :]).sum(-1)
    # RoPE and ReLU VJPs (`fused_rope_unrope_bwd`)
    cs, sn = _f64(cos).reshape(F, S, D), _f64(sin).reshape(F, S, D)
    dQu = dQu + unrope(dQr, cs, sn)
    dKu = dKu + unrope(dKr, cs, sn)
    dQn = _bnhd(dQu) * (t["Qn"] > 0)
    dKn = _bnhd(dKu) * (t["Kn"] > 0) * k_scale
    # RMSNorm VJP over all C channels of a token

    def rms_bwd(dy, x, r, w):
        gw = dy * w
        corr = (gw * x).sum(axis=(2, 3), keepdims=True)
        rr = r[:, :, None, None]
        dx = rr * gw - rr ** 3 / C * x * corr
        dw = (dy * x * rr).sum(axis=(0, 1)).reshape(-1)
        return dx, dw

    dq, dqw = rms_bwd(dQn, t["q"], t["rq"], t["wq"])
    dk, dkw = rms_bwd(dKn, t["k"], t["rk"], t["wk"])
    dqkv = np.stack([dq, dk, _bnhd(dV)], axis=2)
    return dict(dqkv=dqkv, dbeta=dbeta, ddecay=dg_kv + dg_z, dqw=dqw, dkw=dkw)
