"""CPU tests of the C-ABI boundary: the library loads without a GPU, exports
every symbol include/gdr.h declares, and host-side validation rejects bad
arguments with the documented status codes before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from chunked_gated_delta_08_amd import binding
    return binding


def test_header_symbols_exported(B):
    hdr = open(os.path.join(ROOT, "include", "gdr.h")).read()
    declared = set(re.findall(r"^(?:const char \*|int64_t |size_t |int )(\w+)\(", hdr, flags=re.M))
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(B.lib, name), name


def _prob(lib, **kw):
    d = dict(B=1, T=256, HK=2, HV=2, K=64, V=64, BT=64, dtype=lib.GDR_BF16)
    d.update(kw)
    return lib.Problem(d["B"], d["T"], d["HK"], d["HV"], d["K"], d["V"], d["BT"], 0, None, None, 0.0, d["dtype"],
                       d.get("seg_chunks", 0))


FAKE = ctypes.c_void_p(256)   # never dereferenced: validation fails first


def _bwd(B, p, ws_bytes=1 << 40, **null):
    args = {n: FAKE for n in ("q", "k", "v", "g", "beta", "h0", "dO", "dht", "dq", "dk", "dv", "dg", "db", "dh0")}
    args.update(null)
    return B.lib.gdr_chunk_bwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["g"], args["beta"], args["h0"],
                               args["dO"], args["dht"], args["dq"], args["dk"], args["dv"], args["dg"], args["db"],
                               args["dh0"], FAKE, ws_bytes, None)


def test_workspace_and_chunks(B):
    p = _prob(B, T=300)
    assert B.num_chunks(p) == 5
    assert B.workspace_size(p) > 0
    bad = _prob(B, HK=3, HV=4)
    assert B.num_chunks(bad) == -1 and B.workspace_size(bad) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(HK=2, HV=3), -1), (dict(B=0), -1), (dict(T=-1), -1), (dict(dtype=7), -1),
    (dict(BT=32), -2), (dict(K=64, V=128), -2), (dict(K=96, V=96), -2),
    (dict(K=128, V=128, dtype=0), -2),
])
def test_invalid_problem(B, kw, code):
    assert _bwd(B, _prob(B, **kw)) == code


def test_small_workspace(B):
    p = _prob(B)
    assert _bwd(B, p, ws_bytes=B.workspace_size(p) - 1) == -3


@pytest.mark.parametrize("missing", ["q", "k", "v", "g", "beta", "dO", "dq", "dk", "dv", "dg", "db"])
def test_null_required_pointer(B, missing):
    assert _bwd(B, _prob(B), **{missing: None}) == -1


def _varlen(B, cu, T, N=None):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    p = _prob(B, T=T)
    p.N = len(cu) - 1 if N is None else N
    p.cu_seqlens = 512            # a device pointer the host never reads
    p.cu_seqlens_host = ctypes.addressof(arr)
    return p, arr


def test_varlen_validation(B):
    p, keep = _varlen(B, [0, 70, 75, 200], 200)
    assert B.num_chunks(p) == 2 + 1 + 2
    for cu, T in (([1, 70, 200], 200), ([0, 80, 70, 200], 200), ([0, 70, 199], 200)):
        p, keep = _varlen(B, cu, T)
        assert _bwd(B, p) == -1, cu
    p, keep = _varlen(B, [0, 70, 200], 200)
    p.cu_seqlens_host = None
    assert _bwd(B, p) == -1
    p, keep = _varlen(B, [0, 70, 200], 200)
    p.B = 2
    assert _bwd(B, p) == -1


def test_kda_validation(B):
    f = [FAKE] * 17
    p = _prob(B, HK=2, HV=4, dtype=B.GDR_F16)
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f, None) == -1
    p = _prob(B, dtype=B.GDR_BF16)
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f, None) == -2
    p = _prob(B, dtype=B.GDR_F16, BT=16)
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f, None) == -2
    p = _prob(B, dtype=B.GDR_F16)
    f2 = list(f)
    f2[6] = None   # A
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f2, None) == -1


def test_strerror(B):
    for c in (0, -1, -2, -3, -4):
        assert B.lib.gdr_strerror(c)


def _fwd(B, p, ws_bytes=1 << 40, **null):
    args = {n: FAKE for n in ("q", "k", "v", "g", "beta", "h0", "o", "ht")}
    args.update(null)
    return B.lib.gdr_chunk_fwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["g"], args["beta"],
                               args["h0"], args["o"], args["ht"], FAKE, ws_bytes, None)


def test_fwd_validation(B):
    assert _fwd(B, _prob(B, HK=2, HV=3)) == -1
    assert _fwd(B, _prob(B, BT=32)) == -2
    assert _fwd(B, _prob(B, K=128, V=128, dtype=0)) == -2
    p = _prob(B)
    assert _fwd(B, p, ws_bytes=B.workspace_size(p) - 1) == -3
    for missing in ("q", "k", "v", "g", "beta", "o"):
        assert _fwd(B, p, **{missing: None}) == -1, missing


def test_gate_cumsum_validation(B):
    p = _prob(B)
    assert B.lib.gdr_gate_cumsum(ctypes.byref(p), None, FAKE, None) == -1
    assert B.lib.gdr_gate_cumsum(ctypes.byref(p), FAKE, None, None) == -1
    # overlapping input and output
    assert B.lib.gdr_gate_cumsum(ctypes.byref(p), ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 64), None) == -1
    assert B.lib.gdr_gate_cumsum(ctypes.byref(_prob(B, HK=2, HV=3)), FAKE, FAKE, None) == -1
    # nothing to do: no tokens
    assert B.lib.gdr_gate_cumsum(ctypes.byref(_prob(B, T=0)), None, None, None) == 0


def _kda_full(B, p, ws_bytes=1 << 40, **null):
    args = {n: FAKE for n in ("q", "k", "v", "g", "beta", "h0", "dO", "dht", "dq", "dk", "dv", "dg", "db", "dh0")}
    args.update(null)
    return B.lib.kda_chunk_bwd_full(ctypes.byref(p), args["q"], args["k"], args["v"], args["g"], args["beta"],
                                    args["h0"], args["dO"], args["dht"], args["dq"], args["dk"], args["dv"],
                                    args["dg"], args["db"], args["dh0"], FAKE, ws_bytes, None)


def test_kda_full_validation(B):
    f16 = dict(dtype=B.GDR_F16)
    assert _kda_full(B, _prob(B, HK=2, HV=4, **f16)) == -1          # one head count only
    assert _kda_full(B, _prob(B)) == -2                              # bf16 not built
    assert _kda_full(B, _prob(B, BT=32, **f16)) == -2
    assert _kda_full(B, _prob(B, K=128, V=128, dtype=0)) == -2       # fp32 only at K = 64
    assert _kda_full(B, _prob(B, K=64, V=128, **f16)) == -2
    p = _prob(B, **f16)
    need = B.lib.kda_workspace_size(ctypes.byref(p))
    assert need > 0 and B.lib.kda_workspace_size(ctypes.byref(_prob(B))) == 0
    assert _kda_full(B, p, ws_bytes=need - 1) == -3
    for missing in ("q", "k", "v", "g", "beta", "dO", "dq", "dk", "dv", "dg", "db"):
        assert _kda_full(B, p, **{missing: None}) == -1, missing
