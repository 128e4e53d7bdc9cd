"""Pins of the fp64 BiGDN oracle (oracle/bigdn_oracle.py) to facts that do not
come from the oracle itself.

* central finite differences of L = Σ<dout, out> for every input the backward
  differentiates (qkv, β, decay, both norm weights): pins the hand-derived
  backward, all phases, to the forward;
* one frame (F = 1): the output is non-causal linear attention over the frame,
  summed token pair by token pair;
* decay = 0: frame f reads exactly the tokens of frames f and f + 1 (inclusive
  forward scan, exclusive reverse scan);
* any F: the scans equal the explicit sum over source frames of transfer
  products (crossing frame u in either direction applies decay_u (I − P_u));
* RoPE with rotation tables is norm preserving and the identity at angle 0,
  and its VJP is its adjoint; the RMSNorm output has unit mean square up to
  norm_eps;
* linearity of every gradient in dout.
"""
import numpy as np
import pytest

from oracle import bigdn_oracle as BO


def _rot_tables(N, D, rng, zero=False):
    ang = np.zeros((N, D // 2)) if zero else rng.uniform(-np.pi, np.pi, (N, D // 2))
    cos = np.repeat(np.cos(ang), 2, axis=1)
    sin = np.stack([-np.sin(ang), np.sin(ang)], axis=-1).reshape(N, D)
    return cos, sin


def _case(rng, B=1, F=3, S=5, H=2, D=4, k_scale=0.5, decay=None):
    N = F * S
    qkv = rng.standard_normal((B, N, 3, H, D))
    beta = rng.uniform(0.1, 0.9, (B, H, F, S))
    dec = rng.uniform(0.3, 0.95, (B, H, F)) if decay is None else np.full((B, H, F), decay)
    qw = 1 + 0.2 * rng.standard_normal(H * D)
    kw = 1 + 0.2 * rng.standard_normal(H * D)
    cos, sin = _rot_tables(N, D, rng)
    dout = rng.standard_normal((B, N, H, D))
    return dict(qkv=qkv, beta=beta, decay=dec, qw=qw, kw=kw, cos=cos, sin=sin, F=F, S=S, k_scale=k_scale), dout


def _fwd(c, **over):
    a = dict(c)
    a.update(over)
    return BO.bigdn_fwd(a["qkv"], a["beta"], a["decay"], a["qw"], a["kw"], a["cos"], a["sin"], a["F"], a["S"],
                        k_scale=a["k_scale"])


@pytest.mark.parametrize("B,F,S,H,D", [(1, 3, 5, 2, 4), (2, 2, 3, 1, 6), (1, 1, 4, 2, 4)])
def test_bigdn_bwd_finite_differences(B, F, S, H, D):
    rng = np.random.default_rng(100 + F * 10 + S)
    c, dout = _case(rng, B, F, S, H, D)
    grads = BO.bigdn_bwd(c["qkv"], c["beta"], c["decay"], c["qw"], c["kw"], c["cos"], c["sin"], dout, F, S,
                         k_scale=c["k_scale"])
    h = 1e-6
    for name, gname in (("qkv", "dqkv"), ("beta", "dbeta"), ("decay", "ddecay"), ("qw", "dqw"), ("kw", "dkw")):
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = ((_fwd(c, **{name: xp}) - _fwd(c, **{name: xm})) * dout).sum() / (2 * h)
        g = grads[gname]
        assert g.shape == x.shape, name
        err = np.abs(g - fd).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 1e-6, (name, err)


def test_bigdn_one_frame_is_linear_attention():
    rng = np.random.default_rng(1)
    c, _ = _case(rng, B=1, F=1, S=6, H=2, D=4)
    out = _fwd(c)
    t = BO._transforms(c["qkv"], c["qw"], c["kw"], c["cos"], c["sin"], 1, 6, c["k_scale"], 1e-5)
    for h in range(2):
        for n in range(6):
            num = np.zeros(4)
            den = 0.0
            for m in range(6):
                b = c["beta"][0, h, 0, m]
                num += b * np.dot(t["Qr"][0, n, h], t["Kr"][0, m, h]) * t["v"][0, m, h]
                den += b * np.dot(t["Qu"][0, n, h], t["Ku"][0, m, h])
            np.testing.assert_allclose(out[0, n, h], num / (den + 1e-6), rtol=1e-12, atol=1e-14)


def test_bigdn_zero_decay_reads_own_and_next_frame():
    rng = np.random.default_rng(2)
    F, S = 4, 3
    c, _ = _case(rng, B=1, F=F, S=S, H=1, D=4, decay=0.0)
    out = _fwd(c)
    t = BO._transforms(c["qkv"], c["qw"], c["kw"], c["cos"], c["sin"], F, S, c["k_scale"], 1e-5)
    for n in range(F * S):
        f = n // S
        src = range(f * S, min(F, f + 2) * S)
        num = sum(c["beta"][0, 0, m // S, m % S] * np.dot(t["Qr"][0, n, 0], t["Kr"][0, m, 0]) * t["v"][0, m, 0]
                  for m in src)
        den = sum(c["beta"][0, 0, m // S, m % S] * np.dot(t["Qu"][0, n, 0], t["Ku"][0, m, 0]) for m in src)
        np.testing.assert_allclose(out[0, n, 0], num / (den + 1e-6), rtol=1e-12, atol=1e-14)


def test_bigdn_scans_equal_transfer_product_sum():
    rng = np.random.default_rng(3)
    F, S, D = 5, 3, 4
    c, _ = _case(rng, B=1, F=F, S=S, H=1, D=D, k_scale=0.7)
    out = _fwd(c)
    t = BO._transforms(c["qkv"], c["qw"], c["kw"], c["cos"], c["sin"], F, S, c["k_scale"], 1e-5)
    g = c["decay"][0, 0]
    beta = c["beta"][0, 0].reshape(-1)
    Kr, Ku, V = t["Kr"][0, :, 0], t["Ku"][0, :, 0], t["v"][0, :, 0]

    def frame_sum(X, Y, f):
        return sum(beta[m] * np.outer(X[m], Y[m]) for m in range(f * S, f * S + S))

    def crossing(f, Pm):   # the map applied when a state crosses frame f
        return g[f] * (np.eye(D) - Pm(f))

    def transfer(fr, src, Pm):   # from source frame src to reading frame fr
        T = np.eye(D)
        if src < fr:
            for u in range(src + 1, fr + 1):
                T = crossing(u, Pm) @ T
        elif src > fr:
            for u in range(src - 1, fr, -1):
                T = crossing(u, Pm) @ T
        return T

    P = lambda f: frame_sum(Kr, Kr, f)  # noqa: E731
    Pz = lambda f: frame_sum(Ku, Ku, f)  # noqa: E731
    for n in range(F * S):
        fr = n // S
        num = np.zeros(D)
        den = 0.0
        for src in range(F):
            num += t["Qr"][0, n, 0] @ transfer(fr, src, P) @ frame_sum(Kr, V, src)
            bz = sum(beta[m] * Ku[m] for m in range(src * S, src * S + S))
            den += t["Qu"][0, n, 0] @ transfer(fr, src, Pz) @ bz
        np.testing.assert_allclose(out[0, n, 0], num / (den + 1e-6), rtol=1e-11, atol=1e-13)


def test_rope_rotation_and_adjoint():
    rng = np.random.default_rng(4)
    N, D = 7, 8
    cos, sin = _rot_tables(N, D, rng)
    x = rng.standard_normal((N, D))
    y = rng.standard_normal((N, D))
    np.testing.assert_allclose(np.linalg.norm(BO.rope(x, cos, sin), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    c0, s0 = _rot_tables(N, D, rng, zero=True)
    np.testing.assert_array_equal(BO.rope(x, c0, s0), x)
    # the VJP is the adjoint: <rope(x), y> = <x, unrope(y)>
    np.testing.assert_allclose((BO.rope(x, cos, sin) * y).sum(), (x * BO.unrope(y, cos, sin)).sum(), rtol=1e-13)
    # a 90-degree turn of the pair (x0, x1) gives (-x1, x0)
    c9 = np.zeros((1, 2))
    s9 = np.array([[-1.0, 1.0]])
    np.testing.assert_array_equal(BO.rope(np.array([[2.0, 3.0]]), c9, s9), np.array([[-3.0, 2.0]]))


def test_rmsnorm_unit_mean_square():
    rng = np.random.default_rng(5)
    c, _ = _case(rng, B=2, F=2, S=3, H=3, D=4)
    eps = 1e-5
    t = BO._transforms(c["qkv"], c["qw"], c["kw"], c["cos"], c["sin"], 2, 3, c["k_scale"], eps)
    ms = ((t["Qn"] / t["wq"]) ** 2).mean(axis=(2, 3))
    np.testing.assert_allclose(ms, 1 - eps * t["rq"] ** 2, rtol=1e-12)


def test_bigdn_bwd_linear_in_dout():
    rng = np.random.default_rng(6)
    c, d1 = _case(rng, B=1, F=3, S=4, H=2, D=4)
    d2 = rng.standard_normal(d1.shape)
    args = (c["qkv"], c["beta"], c["decay"], c["qw"], c["kw"], c["cos"], c["sin"])
    g1 = BO.bigdn_bwd(*args, d1, 3, 4, k_scale=c["k_scale"])
    g2 = BO.bigdn_bwd(*args, d2, 3, 4, k_scale=c["k_scale"])
    g3 = BO.bigdn_bwd(*args, 2 * d1 - 3 * d2, 3, 4, k_scale=c["k_scale"])
    for n in g1:
        np.testing.assert_allclose(g3[n], 2 * g1[n] - 3 * g2[n], rtol=1e-9, atol=1e-12)
