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
    hdr = "".join(open(os.path.join(ROOT, "include", h)).read() for h in ("gdr.h", "bigdn.h"))
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
    p = _prob(B, dtype=B.GDR_F16, BT=32)   # chunk lengths 16 and 64 are built
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f, None) == -2
    p = _prob(B, dtype=B.GDR_F32, K=128, V=128)   # fp32 is built at K = V = 64 only
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f, None) == -2
    p = _prob(B, dtype=B.GDR_F16)
    f2 = list(f)
    f2[6] = None   # A
    assert B.lib.kda_chunk_bwd(ctypes.byref(p), *f2, None) == -1


def test_strerror(B):
    for c in (0, -1, -2, -3, -4, -5):
        assert B.lib.gdr_strerror(c)


def test_noalloc_host_checks(B):
    # rejected on the host before the scratch array is touched (no GPU needed)
    args = [FAKE] * 14 + [None]
    big = _prob(B, T=32768, HK=16, HV=16, K=128, V=128)
    assert B.workspace_size(big) > B.NOALLOC_SCRATCH_BYTES
    assert B.lib.gdr_chunk_bwd_noalloc(ctypes.byref(big), *args) == -5
    assert B.lib.gdr_chunk_bwd_noalloc(ctypes.byref(_prob(B, HK=2, HV=3)), *args) == -1
    assert B.lib.gdr_chunk_bwd_noalloc(ctypes.byref(_prob(B, BT=32)), *args) == -2


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


def test_workspace_covers_both_plans(B):
    # At T = 32768 with 16 value heads the forward and the backward calls cut the
    # state scans into segments of different lengths; one workspace of
    # gdr_workspace_size() serves both, and each call rejects anything smaller.
    p = _prob(B, T=32768, HK=16, HV=16, K=128, V=128)
    n = B.workspace_size(p)
    assert n > 0
    assert _bwd(B, p, ws_bytes=n - 1) == -3
    assert _fwd(B, p, ws_bytes=n - 1) == -3


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


# ---- BiGDN layer (include/bigdn.h)

def _bprob(lib, **kw):
    d = dict(B=2, F=3, S=100, H=2, D=64, k_scale=0.1, norm_eps=1e-5, eps=1e-6)
    d.update(kw)
    return lib.BigdnProblem(d["B"], d["F"], d["S"], d["H"], d["D"], d["k_scale"], d["norm_eps"], d["eps"])


def _bigdn_bwd(lib, p, ws_bytes=1 << 40, **null):
    names = ["qkv", "beta", "decay", "qw", "kw", "cos", "sin", "dout", "dqkv", "dbeta", "ddecay", "dqw", "dkw"]
    args = [None if n in null else FAKE for n in names]
    return lib.lib.bigdn_bwd(ctypes.byref(p), *args, FAKE, ws_bytes, None)


def _bigdn_fwd(lib, p, ws_bytes=1 << 40, **null):
    names = ["qkv", "beta", "decay", "qw", "kw", "cos", "sin", "out"]
    args = [None if n in null else FAKE for n in names]
    return lib.lib.bigdn_fwd(ctypes.byref(p), *args, FAKE, ws_bytes, None)


def test_bigdn_workspace_size(B):
    p = _bprob(B, B=8, F=11, S=1024, H=16, D=128)
    fwd, bwd = B.bigdn_workspace_size(p, False), B.bigdn_workspace_size(p, True)
    NF, DD = 8 * 16 * 11, 128 * 128
    # forward: rms stats, P (bf16), A, Pz (fp32), both states (bf16) and vectors
    assert fwd >= 2 * 8 * 11264 * 4 + NF * DD * (2 + 4 + 4 + 2 + 2)
    assert bwd > fwd
    assert B.bigdn_workspace_size(_bprob(B, D=96), True) == 0
    assert B.bigdn_workspace_size(_bprob(B, F=0), True) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(F=0), -1), (dict(S=0), -1), (dict(H=0), -1), (dict(eps=0.0), -1),
    (dict(norm_eps=-1.0), -1), (dict(k_scale=float("inf")), -1), (dict(D=96), -2), (dict(D=32), -2),
    (dict(H=33, D=128), -2)])
def test_bigdn_invalid_problem(B, kw, code):
    assert _bigdn_bwd(B, _bprob(B, **kw)) == code
    assert _bigdn_fwd(B, _bprob(B, **kw)) == code


def test_bigdn_workspace_and_pointers(B):
    p = _bprob(B)
    need = B.bigdn_workspace_size(p, True)
    assert _bigdn_bwd(B, p, ws_bytes=need - 1) == -3
    assert _bigdn_fwd(B, p, ws_bytes=B.bigdn_workspace_size(p, False) - 1) == -3
    for n in ("qkv", "beta", "decay", "qw", "kw", "cos", "sin", "dout", "dqkv", "dbeta", "ddecay", "dqw", "dkw"):
        assert _bigdn_bwd(B, p, **{n: True}) == -1, n
    for n in ("qkv", "beta", "decay", "qw", "kw", "cos", "sin", "out"):
        assert _bigdn_fwd(B, p, **{n: True}) == -1, n
