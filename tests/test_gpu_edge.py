"""GPU edge cases of every entry point, through the C ABI, against the fp64
oracle: no tokens at all (T = 0: no chunks, the state gradients pass straight
through), a single token per sequence, and a batch of one-token chunks.
Tolerances as in the other parity tests."""
import numpy as np
import pytest
import torch

from chunked_gated_delta_08_amd import workloads as W

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_gated_delta_08_amd import binding
    return binding


@pytest.mark.parametrize("Bb,T", [(2, 0), (3, 1), (1, 65)])
def test_bwd_degenerate_lengths(B, oracle, Bb, T):
    _log(f"[edge] gdr_chunk_bwd B={Bb} T={T} bf16 K=V=64 h0, dht")
    inp = W.gdr_inputs(Bb, T, 1, 2, 64, 64, dtype="bf16", seed=11, h0=True, gate_scale=1 / 8)
    d = {k: inp[k].cuda() for k in ("q", "k", "v", "beta", "dO", "gcum", "dht", "h0")}
    out = B.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["gcum"], d["beta"], d["dO"], dht=d["dht"], h0=d["h0"], B=Bb)
    torch.cuda.synchronize()
    if T == 0:   # no tokens: dh0 is dht itself
        np.testing.assert_array_equal(out["dh0"].cpu().numpy(), inp["dht"].numpy())
        return
    p = oracle.Problem(Bb, T, 1, 2, 64, 64)
    f = lambda t: t.double().numpy()  # noqa: E731
    graw = oracle.gcum_to_graw(p, 64, inp["gcum"].numpy())
    ref = oracle.gdr_bwd_token(p, f(inp["q"]), f(inp["k"]), f(inp["v"]), graw, f(inp["beta"]), f(inp["h0"]),
                               f(inp["dO"]), f(inp["dht"]))
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        e = rel_l2(out[n].float().cpu().numpy(), ref[n])
        _log(f"  {n} rel-L2 {e:.2e}")
        assert e <= (1e-3 if n == "dh0" else 2e-2), (n, e)


@pytest.mark.parametrize("Bb,T", [(2, 0), (3, 1)])
def test_fwd_degenerate_lengths(B, oracle, Bb, T):
    _log(f"[edge] gdr_gate_cumsum + gdr_chunk_fwd B={Bb} T={T} bf16 K=V=128 h0")
    inp = W.gdr_inputs(Bb, T, 1, 1, 128, 128, dtype="bf16", seed=12, h0=True)
    g = B.gdr_gate_cumsum(inp["graw"].cuda(), B=Bb)
    out = B.gdr_chunk_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), g, inp["beta"].cuda(),
                          h0=inp["h0"].cuda(), B=Bb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g.cpu().numpy(), inp["gcum"].numpy())
    if T == 0:   # no tokens: the final state is h0
        np.testing.assert_array_equal(out["ht"].cpu().numpy(), inp["h0"].numpy())
        return
    p = oracle.Problem(Bb, T, 1, 1, 128, 128)
    f = lambda t: t.double().numpy()  # noqa: E731
    ref = oracle.gdr_fwd_token(p, 64, f(inp["q"]), f(inp["k"]), f(inp["v"]), inp["graw"].double().numpy(),
                               f(inp["beta"]), f(inp["h0"]))
    for n in ("o", "ht"):
        e = rel_l2(out[n].float().cpu().numpy(), ref[n])
        _log(f"  {n} rel-L2 {e:.2e}")
        assert e <= 2e-2, (n, e)


@pytest.mark.parametrize("Bb,T", [(2, 0), (3, 1), (1, 65)])
def test_kda_full_degenerate_lengths(B, oracle, Bb, T):
    _log(f"[edge] kda_chunk_bwd_full B={Bb} T={T} f16 K=V=64 h0, dht")
    inp = W.kda_full_inputs(Bb, T, 2, 64, 64, dtype="f16", seed=13, h0=True, gate_scale=1 / 8)
    d = {k: inp[k].cuda() for k in ("q", "k", "v", "beta", "dO", "gcum", "dht", "h0")}
    out = B.kda_chunk_bwd_full(d["q"], d["k"], d["v"], d["gcum"], d["beta"], d["dO"], dht=d["dht"], h0=d["h0"],
                               B=Bb)
    torch.cuda.synchronize()
    if T == 0:
        np.testing.assert_array_equal(out["dh0"].cpu().numpy(), inp["dht"].numpy())
        return
    n_ = inp["ntok"]
    pg = oracle.Problem(Bb, T, 2 * 64, 2 * 64, 1, 1)
    graw = oracle.gcum_to_graw(pg, 64, inp["gcum"].numpy().reshape(n_, 128)).reshape(n_, 2, 64)
    p = oracle.Problem(Bb, T, 2, 2, 64, 64)
    f = lambda t: t.double().numpy()  # noqa: E731
    ref = oracle.kda_bwd_token(p, f(inp["q"]), f(inp["k"]), f(inp["v"]), graw, f(inp["beta"]), f(inp["h0"]),
                               f(inp["dO"]), f(inp["dht"]))
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        e = rel_l2(out[n].float().cpu().numpy(), ref[n])
        _log(f"  {n} rel-L2 {e:.2e}")
        assert e <= (1e-3 if n == "dh0" else 2e-2), (n, e)
