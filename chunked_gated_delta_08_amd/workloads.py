"""Seeded synthetic inputs for the gated delta rule backward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, and it imports neither the library binding nor the oracle,
so both sides can take their inputs from it.

Recipes (shapes and value distributions follow the pages' workloads):
  q, k      randn, then L2-normalised per (token, key head) in fp32, then cast
  v, dO     randn
  gate      ĝ = logsigmoid(randn) per (token, value head), fp32 ("gate_scale"
            multiplies it; 1/64 gives the slow gate used for cross-chunk
            coverage); the library receives its in-chunk cumulative sum
  beta      sigmoid(randn)
  dht       0.1 * randn, fp32 [N, HV, K, V] (or absent)
  h0        absent (zero) unless asked for
Every draw comes from numpy.random.default_rng(seed) (PCG64) in a fixed order.
"""
import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def varlen_lengths(total=65536, n=12, lo=512, hi=10923, seed=0):
    """n sequence lengths, each uniform in [lo, hi], summing to `total`:
    draw n-1 lengths, take the remainder as the last one, redraw until it is in range."""
    rng = np.random.default_rng(seed)
    while True:
        lens = rng.integers(lo, hi, size=n - 1, endpoint=True)
        last = total - int(lens.sum())
        if lo <= last <= hi:
            return [int(x) for x in lens] + [last]


def cu_from_lengths(lens):
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int64)


def _logsigmoid(x):
    return -np.logaddexp(0.0, -x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _chunk_starts(ntok, BT, cu):
    """Boolean mask over tokens: True where an in-chunk cumulative sum restarts."""
    start = np.zeros(ntok, dtype=bool)
    bounds = [0, ntok] if cu is None else list(cu)
    for a, b in zip(bounds[:-1], bounds[1:]):
        start[a:b:BT] = True
    return start


def in_chunk_cumsum(graw, BT, cu=None, B=1, T=None):
    """fp32 in-chunk cumulative sum of the raw gate (restarts every BT tokens and at
    every sequence start), accumulated sequentially in fp32 -- the form in which a
    forward pass saves the gate for the backward."""
    g = np.asarray(graw, dtype=np.float32)
    ntok = g.shape[0]
    if cu is None:
        T = ntok // B if T is None else T
        cu = np.arange(0, ntok + 1, T)
    start = _chunk_starts(ntok, BT, cu)
    out = np.empty_like(g)
    acc = np.zeros(g.shape[1:], dtype=np.float32)
    for t in range(ntok):
        acc = g[t].copy() if start[t] else (acc + g[t]).astype(np.float32)
        out[t] = acc
    return out


def _in_chunk_cumsum_fast(graw, BT, cu):
    """Same values as in_chunk_cumsum (sequential fp32 adds), vectorised across chunks."""
    g = np.asarray(graw, dtype=np.float32)
    ntok = g.shape[0]
    starts = np.flatnonzero(_chunk_starts(ntok, BT, cu))
    ends = np.append(starts[1:], ntok)
    out = np.empty_like(g)
    lens = ends - starts
    acc = np.zeros((len(starts),) + g.shape[1:], dtype=np.float32)
    for r in range(int(lens.max()) if len(lens) else 0):
        sel = lens > r
        idx = starts[sel] + r
        acc[sel] = g[idx] if r == 0 else (acc[sel] + g[idx]).astype(np.float32)
        out[idx] = acc[sel]
    return out


def gdr_inputs(B, T, HK, HV, K, V, BT=64, dtype="bf16", seed=0, lengths=None, dht=True, h0=False,
               gate_scale=1.0, zero_gate=False, beta_zero=False):
    """Inputs of one backward call, as CPU torch tensors, token axis flattened.

    Returns a dict with q, k [NTOK,HK,K]; v, dO [NTOK,HV,V]; beta [NTOK,HV] (all in
    `dtype`); graw, gcum [NTOK,HV] fp32; dht, h0 [N,HV,K,V] fp32 or None;
    cu (int64 numpy [N+1]) or None.  For varlen pass `lengths` (then B must be 1).
    """
    rng = np.random.default_rng(seed)
    dt = DTYPES[dtype]
    if lengths is not None:
        assert B == 1
        cu = cu_from_lengths(lengths)
        ntok, N = int(cu[-1]), len(lengths)
    else:
        cu, ntok, N = None, B * T, B

    def randn(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    q = randn(ntok, HK, K)
    k = randn(ntok, HK, K)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = randn(ntok, HV, V)
    graw = (_logsigmoid(randn(ntok, HV).astype(np.float64)) * gate_scale).astype(np.float32)
    if zero_gate:
        graw[:] = 0.0
    beta = _sigmoid(randn(ntok, HV).astype(np.float64)).astype(np.float32)
    if beta_zero:
        beta[:] = 0.0
    dO = randn(ntok, HV, V)
    dht_a = (0.1 * randn(N, HV, K, V)).astype(np.float32) if dht else None
    h0_a = randn(N, HV, K, V) if h0 else None
    cu_chunks = cu if cu is not None else np.arange(B + 1) * T   # sequence starts (dense: every T tokens)
    gcum = _in_chunk_cumsum_fast(graw, BT, cu_chunks)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt)  # noqa: E731
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    return {"q": t(q), "k": t(k), "v": t(v), "beta": t(beta), "dO": t(dO),
            "graw": f(graw), "gcum": f(gcum), "dht": f(dht_a), "h0": f(h0_a), "cu": cu,
            "B": B, "T": T if lengths is None else ntok, "HK": HK, "HV": HV, "K": K, "V": V, "BT": BT,
            "N": N, "ntok": ntok, "dtype": dtype}


def kda_inputs(B=1, T=2048, H=32, K=128, V=128, BT=64, dtype="f16", seed=0):
    """Inputs of the KDA WY backward stage: randn q,k,v,v_new,dO,dv; per-channel
    g = logsigmoid(randn) fp32; beta = sigmoid(randn); A = randn [.., BT] with its
    strict upper triangle (within each chunk row block) set to zero; h, dh randn fp32."""
    rng = np.random.default_rng(seed)
    dt = DTYPES[dtype]
    ntok = B * T
    NT = (T + BT - 1) // BT

    def randn(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    q, k, v, vn = randn(ntok, H, K), randn(ntok, H, K), randn(ntok, H, V), randn(ntok, H, V)
    g = _logsigmoid(randn(ntok, H, K).astype(np.float64)).astype(np.float32)
    beta = _sigmoid(randn(ntok, H).astype(np.float64)).astype(np.float32)
    A = randn(ntok, H, BT)
    r = (np.arange(ntok) % T) % BT
    A *= (np.arange(BT)[None, None, :] <= r[:, None, None]).astype(np.float32)
    h = randn(B * NT, H, K, V)
    dO, dh, dv = randn(ntok, H, V), randn(B * NT, H, K, V), randn(ntok, H, V)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt)  # noqa: E731
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    return {"q": t(q), "k": t(k), "v": t(v), "v_new": t(vn), "g": f(g), "beta": t(beta), "A": t(A),
            "h": f(h), "dO": t(dO), "dh": f(dh), "dv": t(dv),
            "B": B, "T": T, "H": H, "K": K, "V": V, "BT": BT, "NT": NT, "dtype": dtype}


def kda_full_inputs(B=1, T=2048, H=32, K=128, V=128, BT=64, dtype="f16", seed=0, lengths=None, h0=False,
                    dht=True, gate_scale=1.0):
    """Inputs of one full KDA backward (per-channel gate), as CPU torch tensors.

    q, k [NTOK,H,K] (L2-normalised), v, dO [NTOK,H,V], beta [NTOK,H] in `dtype`;
    graw = gate_scale * logsigmoid(randn) [NTOK,H,K] fp32 and its in-chunk
    cumsum gcum; dht = 0.1 randn, h0 randn [N,H,K,V] fp32 or None."""
    rng = np.random.default_rng(seed)
    dt = DTYPES[dtype]
    if lengths is not None:
        assert B == 1
        cu = cu_from_lengths(lengths)
        ntok, N = int(cu[-1]), len(lengths)
    else:
        cu, ntok, N = None, B * T, B

    def randn(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    q = randn(ntok, H, K)
    k = randn(ntok, H, K)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = randn(ntok, H, V)
    graw = (_logsigmoid(randn(ntok, H, K).astype(np.float64)) * gate_scale).astype(np.float32)
    beta = _sigmoid(randn(ntok, H).astype(np.float64)).astype(np.float32)
    dO = randn(ntok, H, V)
    dht_a = (0.1 * randn(N, H, K, V)).astype(np.float32) if dht else None
    h0_a = randn(N, H, K, V) if h0 else None
    cu_chunks = cu if cu is not None else np.arange(B + 1) * T   # sequence starts (dense: every T tokens)
    gcum = _in_chunk_cumsum_fast(graw, BT, cu_chunks)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt)  # noqa: E731
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    return {"q": t(q), "k": t(k), "v": t(v), "beta": t(beta), "dO": t(dO), "graw": f(graw), "gcum": f(gcum),
            "dht": f(dht_a), "h0": f(h0_a), "cu": cu, "B": B, "T": T if lengths is None else ntok, "H": H, "K": K,
            "V": V, "BT": BT, "N": N, "ntok": ntok, "dtype": dtype}


def rope_tables(N, D, base=10000.0):
    """Rotary tables [N, D] fp32 for positions 0..N-1: channel pair (2i, 2i+1)
    turns by the angle n * base^(-2i/D); cos repeats per pair and sin carries
    the sign pattern (-sin, +sin), so x*cos + pairflip(x)*sin is a rotation."""
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.repeat(np.cos(ang), 2, axis=1)
    sin = np.stack([-np.sin(ang), np.sin(ang)], axis=-1).reshape(N, D)
    return cos.astype(np.float32), sin.astype(np.float32)


def bigdn_inputs(B=8, F=11, S=1024, H=16, D=128, seed=0, k_scale=None):
    """Inputs of one BiGDN layer call (CPU torch tensors).

    qkv = randn bf16 [B, N, 3, H, D] (N = F*S); beta = sigmoid(randn) fp32
    [B, H, F, S]; decay = sigmoid(randn) fp32 [B, H, F]; q/k norm weights
    1 + 0.1 randn fp32 [H*D]; rope tables from rope_tables(N, D); dout = randn
    bf16 [B, N, H, D].  k_scale defaults to 2/sqrt(S*D), which keeps the
    spectral norm of the frame sums P well below 1 at these distributions."""
    rng = np.random.default_rng(seed)
    N = F * S

    def randn(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    qkv = randn(B, N, 3, H, D)
    beta = _sigmoid(randn(B, H, F, S).astype(np.float64)).astype(np.float32)
    decay = _sigmoid(randn(B, H, F).astype(np.float64)).astype(np.float32)
    qw = (1 + 0.1 * randn(H * D)).astype(np.float32)
    kw = (1 + 0.1 * randn(H * D)).astype(np.float32)
    dout = randn(B, N, H, D)
    cos, sin = rope_tables(N, D)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    return {"qkv": f(qkv).to(torch.bfloat16), "beta": f(beta), "decay": f(decay), "qw": f(qw), "kw": f(kw),
            "cos": f(cos), "sin": f(sin), "dout": f(dout).to(torch.bfloat16), "B": B, "F": F, "S": S, "H": H, "D": D,
            "k_scale": float(2.0 / np.sqrt(S * D)) if k_scale is None else float(k_scale)}
