"""CPU tests of the Python binding's argument checks: wrong dtypes, shapes or
layouts raise before any pointer reaches the library (the kernels read every
16-bit input with the problem's element type and the states as fp32 blocks of
[N, HV, K, V], so a mismatch would otherwise be read as garbage or past the
end of a buffer)."""
import pytest
import torch


@pytest.fixture(scope="module")
def B():
    from chunked_gated_delta_08_amd import binding
    return binding


def _gdr(ntok=256, HK=2, HV=4, K=64, V=64, dt=torch.bfloat16, N=1):
    return dict(q=torch.zeros(ntok, HK, K, dtype=dt), k=torch.zeros(ntok, HK, K, dtype=dt),
                v=torch.zeros(ntok, HV, V, dtype=dt), g_cum=torch.zeros(ntok, HV),
                beta=torch.zeros(ntok, HV, dtype=dt), dO=torch.zeros(ntok, HV, V, dtype=dt),
                dht=torch.zeros(N, HV, K, V), h0=torch.zeros(N, HV, K, V))


def _call(lib, a, **kw):
    return lib.check_gdr_args(a["q"], a["k"], a["v"], a["g_cum"], a["beta"], a["dO"], a["dht"], a["h0"],
                            need_dO=True, cuda=False, **kw)


def test_gdr_args_accept_valid(B):
    assert _call(B, _gdr()) == (1, 2, 4, 64, 64)
    a = _gdr()
    a["dht"] = a["h0"] = None
    assert _call(B, a) == (1, 2, 4, 64, 64)
    a = _gdr(N=3)
    assert _call(B, a, cu_seqlens=torch.tensor([0, 100, 200, 256], dtype=torch.int32))[0] == 3


@pytest.mark.parametrize("name,bad,exc", [
    ("beta", torch.zeros(256, 4), TypeError),                            # fp32 beta with bf16 q/k/v
    ("q", torch.zeros(256, 2, 64, dtype=torch.float16), TypeError),      # mixed 16-bit types
    ("dO", torch.zeros(256, 4, 64), TypeError),
    ("g_cum", torch.zeros(256, 4, dtype=torch.bfloat16), TypeError),     # the gate is fp32
    ("h0", torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16), TypeError),  # bf16 initial state
    ("dht", torch.zeros(1, 4, 64, 64, dtype=torch.float16), TypeError),
    ("beta", torch.zeros(256, 2, dtype=torch.bfloat16), ValueError),     # per key head instead of value head
    ("g_cum", torch.zeros(255, 4), ValueError),
    ("dO", torch.zeros(256, 4, 32, dtype=torch.bfloat16), ValueError),
    ("q", torch.zeros(256, 2, 32, dtype=torch.bfloat16), ValueError),
    ("h0", torch.zeros(2, 4, 64, 64), ValueError),                       # N mismatch
    ("dht", torch.zeros(1, 4, 64, 32), ValueError),
    ("dht", torch.zeros(1, 4, 64, 64).transpose(2, 3), ValueError),      # not contiguous
    ("v", torch.zeros(256, 4, 64, dtype=torch.bfloat16)[:, :, :].transpose(0, 1), ValueError),
])
def test_gdr_args_reject(B, name, bad, exc):
    a = _gdr()
    a[name] = bad
    with pytest.raises(exc):
        _call(B, a)


def test_gdr_args_reject_heads_and_lengths(B):
    a = _gdr(HK=3, HV=4)
    with pytest.raises(ValueError):
        _call(B, a)
    with pytest.raises(ValueError):
        _call(B, _gdr(), B=3)                                            # 256 tokens not a multiple of 3
    with pytest.raises(TypeError):
        _call(B, _gdr(), cu_seqlens=torch.tensor([0, 256], dtype=torch.int64))
    with pytest.raises(ValueError):
        B.check_gdr_args(None, *[_gdr()[n] for n in ("k", "v", "g_cum", "beta")], cuda=False)   # q required
    with pytest.raises(ValueError):
        _call(B, dict(_gdr(), dO=None))                                  # dO required for the backward


def test_gpu_tensor_required(B):
    a = _gdr()
    with pytest.raises(ValueError):
        B.check_gdr_args(a["q"], a["k"], a["v"], a["g_cum"], a["beta"], a["dO"], need_dO=True)


def _kda(ntok=128, H=2, K=64, V=64, dt=torch.float16, NT=2):
    z = lambda *s, d=dt: torch.zeros(*s, dtype=d)  # noqa: E731
    return dict(q=z(ntok, H, K), k=z(ntok, H, K), v=z(ntok, H, V), v_new=z(ntok, H, V),
                g=z(ntok, H, K, d=torch.float32), beta=z(ntok, H), A=z(ntok, H, 64),
                h=z(NT, H, K, V, d=torch.float32), dO=z(ntok, H, V), dh=z(NT, H, K, V, d=torch.float32),
                dv=z(ntok, H, V))


@pytest.mark.parametrize("name,bad,exc", [
    ("A", torch.zeros(128, 2, 64), TypeError),
    ("A", torch.zeros(128, 2, 32, dtype=torch.float16), ValueError),
    ("g", torch.zeros(128, 2, 64, dtype=torch.float16), TypeError),
    ("h", torch.zeros(2, 2, 64, 64, dtype=torch.float16), TypeError),
    ("dh", torch.zeros(3, 2, 64, 64), ValueError),
    ("beta", torch.zeros(128, 2), TypeError),
    ("dv", torch.zeros(128, 2, 32, dtype=torch.float16), ValueError),
])
def test_kda_stage_args(B, name, bad, exc):
    names = ("q", "k", "v", "v_new", "g", "beta", "A", "h", "dO", "dh", "dv")
    a = _kda()
    B.check_kda_stage_args(*[a[n] for n in names], NT=2, cuda=False)
    a[name] = bad
    with pytest.raises(exc):
        B.check_kda_stage_args(*[a[n] for n in names], NT=2, cuda=False)


def test_kda_full_args(B):
    z = torch.zeros
    ok = dict(q=z(128, 2, 64, dtype=torch.float16), k=z(128, 2, 64, dtype=torch.float16),
              v=z(128, 2, 64, dtype=torch.float16), g_cum=z(128, 2, 64), beta=z(128, 2, dtype=torch.float16),
              dO=z(128, 2, 64, dtype=torch.float16))
    assert B.check_kda_full_args(**ok, cuda=False) == 1
    for name, bad, exc in (("g_cum", z(128, 2), ValueError), ("beta", z(128, 2), TypeError),
                           ("dO", z(128, 2, 64), TypeError)):
        with pytest.raises(exc):
            B.check_kda_full_args(**dict(ok, **{name: bad}), cuda=False)
    with pytest.raises(ValueError):
        B.check_kda_full_args(**ok, h0=z(2, 2, 64, 64), cuda=False)
