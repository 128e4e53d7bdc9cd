"""GPU parity of the full chunked KDA backward (kda_chunk_bwd_full, per-channel
gate) through the C ABI against the fp64 oracle's token recurrence (O-KF).

Tolerances (relative L2 per output tensor): 2e-2 for fp16 inputs, 1e-4 for
fp32 inputs, dh0 1e-3.  The oracle sees the raw gate recovered from the same
fp32 in-chunk cumsum the library receives.
"""
import numpy as np
import pytest
import torch

from chunked_gated_delta_08_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 2e-2}
TOL_DH0 = 1e-3


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


def _gpu(B, inp):
    d = {n: (None if inp[n] is None else inp[n].cuda()) for n in ("q", "k", "v", "gcum", "beta", "dO", "dht", "h0")}
    cu = None if inp["cu"] is None else torch.tensor(inp["cu"], dtype=torch.int32, device="cuda")
    out = B.kda_chunk_bwd_full(d["q"], d["k"], d["v"], d["gcum"], d["beta"], d["dO"], dht=d["dht"], h0=d["h0"],
                               cu_seqlens=cu, B=inp["B"], BT=inp["BT"])
    torch.cuda.synchronize()
    return {n: v.float().cpu().numpy() for n, v in out.items()}


def _oracle(oracle, inp, heads=None):
    H, K, V = inp["H"], inp["K"], inp["V"]
    hs = list(range(H)) if heads is None else heads
    f = lambda n: None if inp[n] is None else inp[n].double().numpy()[:, hs]  # noqa: E731
    gc = inp["gcum"].numpy()[:, hs]
    n = inp["ntok"]
    pg = oracle.Problem(inp["B"], inp["T"], len(hs) * K, len(hs) * K, 1, 1, cu_seqlens=inp["cu"])
    graw = oracle.gcum_to_graw(pg, inp["BT"], gc.reshape(n, len(hs) * K)).reshape(n, len(hs), K)
    p = oracle.Problem(inp["B"], inp["T"], len(hs), len(hs), K, V, cu_seqlens=inp["cu"])
    h0 = None if inp["h0"] is None else inp["h0"].double().numpy()[:, hs]
    dht = None if inp["dht"] is None else inp["dht"].double().numpy()[:, hs]
    return oracle.kda_bwd_token(p, f("q"), f("k"), f("v"), graw, f("beta"), h0, f("dO"), dht)


def _compare(got, ref, dtype, heads=None, label=""):
    errs = {}
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        g = got[name] if heads is None else got[name][:, heads]
        errs[name] = rel_l2(g, ref[name])
    _log(f"  {label} rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        lim = min(TOL[dtype], TOL_DH0) if name == "dh0" else TOL[dtype]
        assert e <= lim, (label, name, e, lim)


CASES = {
    # name: (B, T, H, K, V, dtype, lengths, extra)
    "f16_ragged_k128": (1, 300, 2, 128, 128, "f16", None, {}),
    "f16_slow_gate_h0": (1, 320, 1, 128, 128, "f16", None, {"gate_scale": 1 / 32, "h0": True}),
    "f16_varlen_h0": (1, None, 2, 128, 128, "f16", [70, 5, 130, 0, 64, 1], {"gate_scale": 1 / 8, "h0": True}),
    "f16_k64_batch2": (2, 150, 2, 64, 64, "f16", None, {"gate_scale": 1 / 16}),
    "fp32_k64_h0": (1, 200, 2, 64, 64, "f32", None, {"gate_scale": 1 / 16, "h0": True}),
    "fp32_k64_fast_gate": (2, 130, 1, 64, 64, "f32", None, {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_kda_full_parity(B, oracle, name):
    Bb, T, H, K, V, dt, lens, extra = CASES[name]
    _log(f"[kda full] {name}: B={Bb} T={T} H={H} K={K} {dt} lens={lens} {extra}")
    inp = W.kda_full_inputs(Bb, T, H, K, V, dtype=dt, seed=9, lengths=lens, **extra)
    got = _gpu(B, inp)
    ref = _oracle(oracle, inp)
    _compare(got, ref, dt, label=name)


def test_kda_full_deterministic(B):
    _log("[kda full] two runs bit-identical")
    inp = W.kda_full_inputs(1, 400, 2, 128, 128, dtype="f16", seed=10, gate_scale=1 / 8)
    a, b = _gpu(B, inp), _gpu(B, inp)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


@pytest.mark.slow
def test_kda_full_T2048_h32_all_heads(B, oracle):
    _log("[kda full] B=1 T=2048 H=32 K=V=128 f16, every head")
    inp = W.kda_full_inputs(1, 2048, 32, 128, 128, dtype="f16", seed=0)
    got = _gpu(B, inp)
    for n, v in got.items():
        assert np.isfinite(v).all(), n
    ref = _oracle(oracle, inp)
    _compare(got, ref, "f16", label="T2048_h32")
