"""GPU test of gdr_chunk_bwd_noalloc (the entry point with no workspace
argument, for callers that cannot allocate): its outputs match gdr_chunk_bwd's
on the same inputs to the parity bar (rel-L2 2e-2 per output for 16-bit
inputs, 1e-3 for dh0), on two calls in a row with the second one smaller (the
fixed scratch array keeps the first call's contents), and a problem larger than
the array is rejected before anything is launched."""
import numpy as np
import pytest
import torch

from chunked_gated_delta_08_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL, TOL_DH0 = 2e-2, 1e-3


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


def _dev(inp):
    d = {k: (None if inp[k] is None else inp[k].cuda()) for k in ("q", "k", "v", "beta", "dO", "gcum", "dht", "h0")}
    d["cu"] = None if inp["cu"] is None else torch.tensor(inp["cu"], dtype=torch.int32, device="cuda")
    return d


def _both(B, inp):
    d = _dev(inp)
    args = (d["q"], d["k"], d["v"], d["gcum"], d["beta"], d["dO"])
    kw = dict(dht=d["dht"], h0=d["h0"], cu_seqlens=d["cu"], B=inp["B"])
    got = B.gdr_chunk_bwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    ref = B.gdr_chunk_bwd(*args, **kw)
    torch.cuda.synchronize()
    return ({k: v.float().cpu().numpy() for k, v in got.items()},
            {k: v.float().cpu().numpy() for k, v in ref.items()})


def _check(got, ref, label):
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        e = rel_l2(got[name], ref[name])
        same = np.array_equal(got[name], ref[name])
        _log(f"  {label} {name}: rel-L2 {e:.2e} vs gdr_chunk_bwd (bit-identical: {same})")
        assert np.isfinite(got[name]).all(), (label, name)
        assert e <= (TOL_DH0 if name == "dh0" else TOL), (label, name, e)


def test_noalloc_two_calls_second_smaller(B):
    _log("[noalloc] call 1: varlen GQA bf16, lengths [900, 64, 1, 700], HK=2 HV=4 K=V=128, h0 and dht")
    inp1 = W.gdr_inputs(1, None, 2, 4, 128, 128, dtype="bf16", seed=11, lengths=[900, 64, 1, 700],
                        gate_scale=1 / 16, h0=True)
    got, ref = _both(B, inp1)
    _check(got, ref, "call 1")
    _log("[noalloc] call 2 (smaller): dense bf16 B=1 T=300 HK=HV=2 K=V=128, dht")
    inp2 = W.gdr_inputs(1, 300, 2, 2, 128, 128, dtype="bf16", seed=12)
    got, ref = _both(B, inp2)
    _check(got, ref, "call 2")


def test_noalloc_rejects_oversized(B):
    from chunked_gated_delta_08_amd.binding import GdrError
    _log("[noalloc] T=32768 HK=HV=16 K=V=128 needs more than the fixed scratch: rejected")
    p, keep = B.make_problem(1, 32768, 16, 16, 128, 128, torch.bfloat16)
    assert B.workspace_size(p) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(32768, 16, 128, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(32768, 16, dtype=torch.float32, device="cuda")
    b = torch.zeros(32768, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(GdrError) as ei:
        B.gdr_chunk_bwd_noalloc(x, x, x, g, b, x)
    assert ei.value.code == -5
