"""ctypes binding of the fp64 CPU oracle (oracle/gdr_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline leg
of bench.py may import this module.  It never imports the library package and
the library never imports it.

Every function takes numpy arrays (any float dtype; they are converted to fp64
exactly) with the token axis flattened over the batch:
    q, k  [NTOK, HK, K]     v, dO  [NTOK, HV, V]     graw, beta  [NTOK, HV]
    states [N, HV, K, V]    per-chunk states [NCHUNK, HV, K, V]
`graw` is the RAW log-gate ĝ_t (use gcum_to_graw to recover it from the
in-chunk cumulative sum the library receives).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("HK", ctypes.c_int), ("HV", ctypes.c_int),
                ("K", ctypes.c_int), ("V", ctypes.c_int), ("N", ctypes.c_int),
                ("cu", ctypes.POINTER(ctypes.c_int64)), ("scale", ctypes.c_double)]


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b  # noqa: F401  (package-relative when imported as oracle.oracle)
            _b.build()
        _LIB = ctypes.CDLL(path)
        _LIB.orc_num_chunks.restype = ctypes.c_int64
        _LIB.orc_num_threads.restype = ctypes.c_int
    return _LIB


class Problem:
    """Problem sizes.  cu_seqlens (host int array [N+1]) selects varlen; then B must be 1."""

    def __init__(self, B, T, HK, HV, K, V, cu_seqlens=None, scale=None):
        self.B, self.T, self.HK, self.HV, self.K, self.V = int(B), int(T), int(HK), int(HV), int(K), int(V)
        self.cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        self.N = self.B if self.cu is None else len(self.cu) - 1
        self.scale = float(K) ** -0.5 if scale is None else float(scale)
        self.ntok = self.B * self.T if self.cu is None else int(self.cu[-1])

    def _c(self):
        p = _Problem(self.B, self.T, self.HK, self.HV, self.K, self.V, self.N, None, self.scale)
        if self.cu is not None:
            p.cu = self.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        return p

    def num_chunks(self, BT):
        return int(_lib().orc_num_chunks(ctypes.byref(self._c()), int(BT)))


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor on CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads():
    return int(_lib().orc_num_threads())


def gcum_to_graw(prob, BT, gcum):
    """Raw gate from the fp32 in-chunk cumulative sum (difference taken in fp64)."""
    g = np.ascontiguousarray(np.asarray(gcum, dtype=np.float32))
    out = np.zeros(g.shape, dtype=np.float64)
    _lib().orc_gcum_to_graw(ctypes.byref(prob._c()), int(BT), g.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                            _ptr(out))
    return out


def gate_cumsum(prob, BT, graw):
    """fp64 in-chunk cumulative sum of the raw gate (restarts every BT tokens and
    at every sequence start)."""
    g = _f64(graw)
    out = np.zeros(g.shape, dtype=np.float64)
    _lib().orc_gate_cumsum(ctypes.byref(prob._c()), int(BT), _ptr(g), _ptr(out))
    return out


def gdr_fwd_token(prob, BT, q, k, v, graw, beta, h0=None, want_o=True, want_hc=False):
    q, k, v, graw, beta, h0 = map(_f64, (q, k, v, graw, beta, h0))
    o = np.zeros((prob.ntok, prob.HV, prob.V)) if want_o else None
    ht = np.zeros((prob.N, prob.HV, prob.K, prob.V))
    hc = np.zeros((prob.num_chunks(BT), prob.HV, prob.K, prob.V)) if want_hc else None
    rc = _lib().orc_gdr_fwd_token(ctypes.byref(prob._c()), int(BT), _ptr(q), _ptr(k), _ptr(v), _ptr(graw),
                                  _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _ptr(hc))
    assert rc == 0
    return {"o": o, "ht": ht, "hc": hc}


def _grad_bufs(prob):
    return {"dq": np.zeros((prob.ntok, prob.HK, prob.K)), "dk": np.zeros((prob.ntok, prob.HK, prob.K)),
            "dv": np.zeros((prob.ntok, prob.HV, prob.V)), "dg": np.zeros((prob.ntok, prob.HV)),
            "dbeta": np.zeros((prob.ntok, prob.HV)), "dh0": np.zeros((prob.N, prob.HV, prob.K, prob.V))}


def gdr_bwd_token(prob, q, k, v, graw, beta, h0, dO, dht):
    """O-1: gradients of sum<dO,o> + <dht,S_T> by reverse-time token recurrence."""
    q, k, v, graw, beta, h0, dO, dht = map(_f64, (q, k, v, graw, beta, h0, dO, dht))
    o = _grad_bufs(prob)
    rc = _lib().orc_gdr_bwd_token(ctypes.byref(prob._c()), _ptr(q), _ptr(k), _ptr(v), _ptr(graw), _ptr(beta),
                                  _ptr(h0), _ptr(dO), _ptr(dht), _ptr(o["dq"]), _ptr(o["dk"]), _ptr(o["dv"]),
                                  _ptr(o["dg"]), _ptr(o["dbeta"]), _ptr(o["dh0"]))
    assert rc == 0
    return o


def gdr_bwd_chunked(prob, BT, q, k, v, graw, beta, h0, dO, dht):
    """O-2: chunked WY-form gradients; also returns per-chunk states hc / dhc."""
    q, k, v, graw, beta, h0, dO, dht = map(_f64, (q, k, v, graw, beta, h0, dO, dht))
    o = _grad_bufs(prob)
    nc = prob.num_chunks(BT)
    o["hc"] = np.zeros((nc, prob.HV, prob.K, prob.V))
    o["dhc"] = np.zeros((nc, prob.HV, prob.K, prob.V))
    rc = _lib().orc_gdr_bwd_chunked(ctypes.byref(prob._c()), int(BT), _ptr(q), _ptr(k), _ptr(v), _ptr(graw),
                                    _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dht), _ptr(o["dq"]), _ptr(o["dk"]),
                                    _ptr(o["dv"]), _ptr(o["dg"]), _ptr(o["dbeta"]), _ptr(o["dh0"]),
                                    _ptr(o["hc"]), _ptr(o["dhc"]))
    assert rc == 0
    return o


def kda_wy_bwd(prob, BT, q, k, v, v_new, g, beta, A, h, dO, dh, dv):
    """O-K: the KDA WY backward stage (HK == HV == H).  Returns dq, dk, dv, db, dg, dA."""
    q, k, v, v_new, g, beta, A, h, dO, dh, dv = map(_f64, (q, k, v, v_new, g, beta, A, h, dO, dh, dv))
    H, K, V, n = prob.HV, prob.K, prob.V, prob.ntok
    o = {"dq": np.zeros((n, H, K)), "dk": np.zeros((n, H, K)), "dv": np.zeros((n, H, V)),
         "db": np.zeros((n, H)), "dg": np.zeros((n, H, K)), "dA": np.zeros((n, H, BT))}
    rc = _lib().orc_kda_wy_bwd(ctypes.byref(prob._c()), int(BT), _ptr(q), _ptr(k), _ptr(v), _ptr(v_new),
                               _ptr(g), _ptr(beta), _ptr(A), _ptr(h), _ptr(dO), _ptr(dh), _ptr(dv),
                               _ptr(o["dq"]), _ptr(o["dk"]), _ptr(o["dv"]), _ptr(o["db"]), _ptr(o["dg"]),
                               _ptr(o["dA"]))
    assert rc == 0
    return o


def kda_fwd_token(prob, q, k, v, graw, beta, h0=None):
    """KDA (per-channel gate) token recurrence: o [NTOK,H,V], ht [N,H,K,V].
    graw is the raw per-channel log-gate [NTOK,H,K]; HK == HV == H."""
    q, k, v, graw, beta, h0 = map(_f64, (q, k, v, graw, beta, h0))
    o = np.zeros((prob.ntok, prob.HV, prob.V))
    ht = np.zeros((prob.N, prob.HV, prob.K, prob.V))
    rc = _lib().orc_kda_fwd_token(ctypes.byref(prob._c()), _ptr(q), _ptr(k), _ptr(v), _ptr(graw), _ptr(beta),
                                  _ptr(h0), _ptr(o), _ptr(ht))
    assert rc == 0
    return {"o": o, "ht": ht}


def kda_bwd_token(prob, q, k, v, graw, beta, h0, dO, dht):
    """O-KF: gradients of sum<dO,o> + <dht,S_T> for the KDA recurrence.
    Returns dq, dk, dg [NTOK,H,K]; dv [NTOK,H,V]; dbeta [NTOK,H]; dh0 [N,H,K,V]."""
    q, k, v, graw, beta, h0, dO, dht = map(_f64, (q, k, v, graw, beta, h0, dO, dht))
    n, H, K, V = prob.ntok, prob.HV, prob.K, prob.V
    o = {"dq": np.zeros((n, H, K)), "dk": np.zeros((n, H, K)), "dv": np.zeros((n, H, V)),
         "dg": np.zeros((n, H, K)), "dbeta": np.zeros((n, H)), "dh0": np.zeros((prob.N, H, K, V))}
    rc = _lib().orc_kda_bwd_token(ctypes.byref(prob._c()), _ptr(q), _ptr(k), _ptr(v), _ptr(graw), _ptr(beta),
                                  _ptr(h0), _ptr(dO), _ptr(dht), _ptr(o["dq"]), _ptr(o["dk"]), _ptr(o["dv"]),
                                  _ptr(o["dg"]), _ptr(o["dbeta"]), _ptr(o["dh0"]))
    assert rc == 0
    return o
