#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule chunked backward on one MI355X.

One step = one gdr_chunk_bwd call (chunk table + WY factors, the forward state
scan and the reverse dh scan, the per-chunk gradient kernel with the dg
reverse cumsum and GQA sums) over one batch of synthetic inputs already
resident in HBM.  Default workload: B=1, T=32768, 16 key / 16 value heads,
K=V=128, BT=64, bf16 inputs with fp32 gate, dht present.

With --path bigdn a step is one bigdn_bwd call: the BiGDN chunkwise layer
backward (frame-level bidirectional gated delta rule with its normaliser
stream, RoPE/ReLU and full-channel RMSNorm, recomputing the per-frame sums and
both frame scans) at B=8, F=11 frames of S=1024 tokens, H=16, D=128, bf16.

With --path fwd a step is instead the chunked forward: gdr_gate_cumsum on the
raw gate, then gdr_chunk_fwd (chunk table + WY factors, the forward state
scan, the output kernel), on the same inputs.  With --path kda a step is one
kda_chunk_bwd_full call (the full KDA backward, per-channel gate) at B=1,
T=2048, H=32, K=V=128, BT=64, fp16, dht present.

With --path kda_stage a step is one kda_chunk_bwd call (the KDA WY backward
stage alone) at B=1, T=2048, H=32, K=V=128, BT=64, fp16.

Timing protocol (every path): W untimed warm-up calls, then K timed calls;
before every call a 512 MiB scratch buffer is overwritten on the same stream
(outside the timed region) so that no input is served from the 256 MB
Infinity Cache; each call is bracketed by HIP events recorded by the library
on its launch stream, and ms_per_step is the median over the K calls (p10 and
p90 beside it).  The default bwd run also times the 32-head workload and the
12-sequence varlen GQA workload the same way and reports them in `also`.

Prints one JSON line: the headline metric (effective TFLOP/s under the FLOP
model below, with ms per call), a roofline entry for the dominant kernel
(timed with HIP events recorded by the library between its stages during the
timed steps), and the fp64 CPU oracle timed on a bounded sample.

FLOP model per (chunk of C rows, value head), dense tiles, recompute not
counted:  F(C) = 16 C K V + 18 C^2 K + 10 C^2 V + 13/3 C^3  (32.59 MFLOP at
C=64, K=V=128).  Forward: K Kᵀ, W = A(βγK), Q Kᵀ (2 C^2 K each), U = A(βV) and
Pm V_new (2 C^2 V each), W h, K̃ᵀ V_new and Q h (2 C K V each), the triangular
inverse (C^3 / 3):  F_fwd(C) = 6 C K V + 6 C^2 K + 4 C^2 V + C^3 / 3
(11.62 MFLOP at C=64, K=V=128).
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "dense_t32k_h16": dict(B=1, T=32768, HK=16, HV=16, K=128, V=128, lengths=None,
               name="gdn_bwd_T32768_hk16_hv16_K128_V128_BT64_bf16"),
    "dense_t32k_h32": dict(B=1, T=32768, HK=32, HV=32, K=128, V=128, lengths=None,
               name="gdn_bwd_T32768_hk32_hv32_K128_V128_BT64_bf16"),
    "varlen12_hk16_hv32": dict(B=1, T=None, HK=16, HV=32, K=128, V=128, lengths="varlen12",
               name="gdn_bwd_varlen12_65536tok_hk16_hv32_K128_V128_BT64_bf16"),
}


def flop_model(C, K, V):
    return 16 * C * K * V + 18 * C * C * K + 10 * C * C * V + 13.0 / 3.0 * C ** 3


def flop_model_fwd(C, K, V):
    return 6 * C * K * V + 6 * C * C * K + 4 * C * C * V + C ** 3 / 3.0


# Matrix-core work each chunk-parallel backward kernel executes per (chunk, value
# head), full 64-row tiles (C = 64): the products the kernel issues, recompute
# included -- not the algorithmic model above.
#   WY prep: K Kᵀ, Q Kᵀ, W = A·diag(βγ)K, Pm·W (2C²K each), U = A·diag(β)V
#            (2C²V), the blocked triangular inverse (C³/3)
#   gradient: K h, K dh, dO hᵀ, dV_new hᵀ, V_new dhᵀ (2CKV each); Q Kᵀ, T1 K,
#             T1ᵀ Q, Aᵀ dW, K Kᵀ (2C²K each), Eb K + Ebᵀ K (4C²K);
#             Pmᵀ dO, A Z, dO V_newᵀ, dV_new Zᵀ, Aᵀ dV_new (2C²V each);
#             Aᵀ dA_pre, M1 Aᵀ (2C³ each)
def mfma_work_prep(K, V, C=64):
    return 8 * C * C * K + 2 * C * C * V + C ** 3 / 3.0


def mfma_work_grad(K, V, C=64):
    return 10 * C * K * V + 14 * C * C * K + 10 * C * C * V + 4 * C ** 3


def kernel_bytes_kda(H, K, V, chunks, es=2):
    """Algorithmic bytes of each stage of the full KDA backward (inputs read
    once, outputs written once)."""
    ntok, nunits = sum(chunks), len(chunks) * H
    tk, tv = ntok * H * K, ntok * H * V          # elements of [NTOK,H,K] / [NTOK,H,V]
    st, stv, state = 64 * K * es, 64 * V * es, K * V * 4
    tri = 64 * 64 * es
    # WY factors: q, k, v, per-channel gate, beta in; W, U, K~, Qg, Aqk and A out
    prep = 2 * tk * es + tv * es + tk * 4 + ntok * H * es + nunits * (3 * st + stv + 2 * tri)
    # scans: W, K~, U in, h (fp32) and V_new out; W, K~, Qg, Aqk, dO in, dh (fp32) and dV_new out
    scans = nunits * (2 * st + stv + state) + tv * es + nunits * (3 * st + tri + state) + 2 * tv * es
    # WY stage: q, k, v, V_new, dO, dV_new, gate, beta, A, h, dh in; dq, dk, dg, dA (fp32), dv, db out
    stage = (2 * tk + 4 * tv) * es + tk * 4 + ntok * H * es + nunits * tri + 2 * nunits * state + \
        3 * tk * 4 + tv * es + ntok * H * 4 + ntok * H * 64 * 4
    # intra: dO, V_new, dA, beta, gate, q, k, stage dq/dk/dg/db in; dq, dk, dg, dbeta out
    intra = 2 * tv * es + ntok * H * 64 * 4 + ntok * H * es + tk * 4 + 2 * tk * es + 3 * tk * 4 + ntok * H * 4 + \
        2 * tk * es + tk * 4 + ntok * H * 4
    return {"prep": prep, "scans": scans, "stage": stage, "intra": intra}


def chunk_lengths(lengths, T, B, BT):
    seqs = [T] * B if lengths is None else lengths
    out = []
    for L in seqs:
        out += [BT] * (L // BT) + ([L % BT] if L % BT else [])
    return out


def kernel_bytes(cfg, chunks, es=2):
    """Algorithmic bytes of each stage (inputs read once, outputs written once)."""
    HK, HV, K, V = cfg["HK"], cfg["HV"], cfg["K"], cfg["V"]
    ntok, nunits, nkunits = sum(chunks), len(chunks) * HV, len(chunks) * HK
    tok_k, tok_v = ntok * K * es, ntok * V * es
    st = 64 * K * es              # one [64, K] workspace tile
    state = K * V * es            # one K x V state in the workspace
    gb = ntok * HV * (4 + es)     # gate (fp32) and beta
    # prep: q, k, v, gate, beta in; W, U, R, K~ tiles and A out (the stage's time
    # also covers the max |dO| pass of 16-bit problems, whose read of dO is not counted)
    prep = HK * (2 * tok_k) + HV * tok_v + gb + nunits * (4 * st + 64 * 64 * es)
    # forward scan: W, K~, U in, h states out; reverse scan: W, K~, R, dO in, dh states out
    scans = nunits * (3 * st) + nunits * state + nunits * (3 * st) + HV * tok_v + nunits * state
    # grad: q, k, v, dO, h and dh states, A, gate, beta in; dq, dk, dv, dg, dbeta out
    grad = HK * 2 * tok_k + HV * 2 * tok_v + nunits * (2 * state + 64 * 64 * es) + gb + \
        HK * 2 * tok_k + HV * tok_v + ntok * HV * 8
    return {"prep": prep, "scans": scans, "grad": grad}


def kernel_bytes_fwd(cfg, chunks, es=2):
    """Algorithmic bytes of each forward stage (inputs read once, outputs written once)."""
    HK, HV, K, V = cfg["HK"], cfg["HV"], cfg["K"], cfg["V"]
    ntok, nunits = sum(chunks), len(chunks) * HV
    tok_k, tok_v = ntok * K * es, ntok * V * es
    st, state = 64 * K * es, K * V * es
    gate = ntok * HV * 8                       # raw gate in, cumulative gate out (fp32)
    # prep: k, v, gate, beta in; W, U, K~ tiles out
    prep = HK * tok_k + HV * tok_v + ntok * HV * (4 + es) + nunits * 3 * st
    # forward scan: W, K~, U in; h states out
    scans = nunits * (3 * st + state)
    # output: q, k, W, U, h states and gate in; o out
    out = HK * 2 * tok_k + nunits * (2 * st + state) + ntok * HV * 4 + HV * tok_v
    return {"gate": gate, "prep": prep, "scans": scans, "out": out}


def hip_events(n):
    hip = ctypes.CDLL("libamdhip64.so")
    evs = (ctypes.c_void_p * n)()
    for i in range(n):
        assert hip.hipEventCreate(ctypes.byref(evs, i * ctypes.sizeof(ctypes.c_void_p))) == 0
    return hip, evs


def elapsed_ms(hip, a, b):
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
    return ms.value


EVICT_BYTES = 512 << 20


class Evictor:
    """Overwrites a 512 MiB device buffer on the launch stream: run before each
    timed call, outside its events, so the call reads its inputs from HBM."""

    def __init__(self, torch):
        self.buf = torch.empty(EVICT_BYTES // 4, dtype=torch.int32, device="cuda")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i)


def timed_calls(torch, hip, evs, nev, call, steps, warmup, evict):
    """W warm-ups, then K calls each preceded by the eviction write; call(i)
    records events [nev*i, nev*i + nev) around its stages.  Returns per-call
    ms (first to last event), per-stage ms averaged over the calls, and the
    wall-clock ms per step of the timed loop (evictions included)."""
    for _ in range(warmup):
        evict()
        call(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evict()
        call(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per_call, stage = [], [0.0] * (nev - 1)
    for i in range(steps):
        e = [evs[nev * i + j] for j in range(nev)]
        per_call.append(elapsed_ms(hip, e[0], e[-1]))
        for j in range(nev - 1):
            stage[j] += elapsed_ms(hip, e[j], e[j + 1]) / steps
    return per_call, stage, wall


def call_stats(per_call):
    import numpy as np
    a = np.asarray(per_call)
    return {"median_ms": round(float(np.median(a)), 4), "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "mean_ms": round(float(a.mean()), 4),
            "calls": int(a.size)}


def host_info(threads):
    """Host cores available to this process, the CPU model, and the threads a
    CPU leg used."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": int(threads), "host_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(inp, cfg, chunks, min_seconds=10.0, path="bwd"):
    """The fp64 oracle, unchanged, on the same inputs: full passes over every
    sequence and head of the workload, repeated until at least `min_seconds`
    of CPU time have elapsed (a bounded sample of the timed work)."""
    from oracle import oracle as O
    B, T, HK, HV, K, V = cfg["B"], inp["T"], cfg["HK"], cfg["HV"], cfg["K"], cfg["V"]
    p = O.Problem(B if inp["cu"] is None else 1, T, HK, HV, K, V, cu_seqlens=inp["cu"])
    if path == "kda":   # per-channel gate: recover it channel by channel
        pg = O.Problem(B, T, HV * K, HV * K, 1, 1)
        graw = O.gcum_to_graw(pg, 64, inp["gcum"].numpy().reshape(-1, HV * K)).reshape(-1, HV, K)
    else:
        graw = O.gcum_to_graw(p, 64, inp["gcum"].numpy())
    f = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    args = (f(inp["q"]), f(inp["k"]), f(inp["v"]), graw, f(inp["beta"]), None, f(inp["dO"]), f(inp["dht"]))
    passes, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        if path == "fwd":
            O.gdr_fwd_token(p, 64, args[0], args[1], args[2], args[3], args[4], None)
        elif path == "kda":
            O.kda_bwd_token(p, *args)
        else:
            O.gdr_bwd_token(p, *args)
        dt += time.perf_counter() - t0
        passes += 1
    model = flop_model_fwd if path == "fwd" else flop_model
    flops = passes * sum(model(c, K, V) for c in chunks) * HV
    nseq = B if inp["cu"] is None else len(inp["cu"]) - 1
    threads = min(O.num_threads(), nseq * (HV if path in ("fwd", "kda") else HK))
    what = {"fwd": "token recurrence (forward), OpenMP over (sequence, value head)",
            "kda": "KDA token recurrence with the hand-derived backward, OpenMP over (sequence, head)"}.get(
        path, "token recurrence with the hand-derived backward, OpenMP over (sequence, key head)")
    res = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"{passes} full pass(es) over the workload ({dt:.1f} s): fp64 {what}",
           "seconds": round(dt, 2)}
    res.update(host_info(threads))
    return res


def _traffic(kernel_name, workload, profiling):
    """HBM bytes per launch from the committed counter summary, while the
    code of the kernel's sources (comments and layout left out) still hashes to
    the digest recorded there (else None)."""
    tfile = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}_{workload}.json")
    if not os.path.exists(tfile):
        return None
    with open(tfile) as fh:
        t = json.load(fh)
    if t.get("source_digest") != profiling.source_digest(profiling.KERNEL_SOURCES[kernel_name]):
        return None
    return t.get("bytes_per_launch")


def _roofline(stage, kb, names, workload, profiling):
    """Roofline entry of the slowest stage's kernel (HBM-bound)."""
    dom = max(stage, key=stage.get)
    achieved = kb[dom] / (stage[dom] * 1e-3) / 1e9
    kernel_name = names[dom]
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic(kernel_name, workload, profiling),
            "kernel": kernel_name, "kernel_ms": round(stage[dom], 4), "algorithmic_bytes": kb[dom],
            "stage_ms": {k: round(v, 4) for k, v in stage.items()}}


# Algorithmic matrix-core work of the gradient kernel per (chunk, value head):
# the backward's products (12CKV + 14C^2K + 8C^2V + 4C^3 in the FLOP model)
# minus the dh scan's 6CKV -- 18.87 MFLOP at C = 64, K = V = 128.
def flop_grad_algorithmic(C, K, V):
    return 6 * C * K * V + 14 * C * C * K + 8 * C * C * V + 4 * C ** 3


def run_gdn(args, torch, binding, workloads, wkey, fwd, evict):
    """Times gdr_chunk_bwd (or gate cumsum + gdr_chunk_fwd) on one workload.
    Returns inputs, chunk lengths, per-call statistics and per-stage ms."""
    cfg = dict(WORKLOADS[wkey])
    lengths = workloads.varlen_lengths() if cfg["lengths"] == "varlen12" else None
    inp = workloads.gdr_inputs(cfg["B"], cfg["T"], cfg["HK"], cfg["HV"], cfg["K"], cfg["V"], dtype="bf16", seed=0,
                               lengths=lengths, dht=True)
    dev = {k: inp[k].cuda() for k in ("q", "k", "v", "beta", "dO", "gcum", "graw", "dht")}
    cu = None if inp["cu"] is None else torch.tensor(inp["cu"], dtype=torch.int32, device="cuda")
    T = inp["T"]
    prob, keep = binding.make_problem(cfg["B"], T, cfg["HK"], cfg["HV"], cfg["K"], cfg["V"], torch.bfloat16, 64, cu)
    N = inp["N"]
    ws = torch.empty(binding.workspace_size(prob), dtype=torch.uint8, device="cuda")
    P = binding._ptr
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nev = 5 if fwd else 4
    hip, evs = hip_events(nev * args.steps)
    evsz = ctypes.sizeof(ctypes.c_void_p)
    if fwd:
        gprob, gkeep = binding.make_problem(cfg["B"], T, 1, cfg["HV"], 1, 1, torch.float32, 64, cu)
        gc = torch.empty_like(dev["graw"])
        out = {"o": torch.empty_like(dev["v"]),
               "ht": torch.empty((N, cfg["HV"], cfg["K"], cfg["V"]), dtype=torch.float32, device="cuda")}
        args_c = [ctypes.byref(prob), P(dev["q"]), P(dev["k"]), P(dev["v"]), P(gc), P(dev["beta"]), None,
                  P(out["o"]), P(out["ht"]), P(ws), ws.numel(), sp]
    else:
        out = {"dq": torch.empty_like(dev["q"]), "dk": torch.empty_like(dev["k"]), "dv": torch.empty_like(dev["v"]),
               "dg": torch.empty(dev["gcum"].shape, dtype=torch.float32, device="cuda"),
               "dbeta": torch.empty(dev["beta"].shape, dtype=torch.float32, device="cuda"),
               "dh0": torch.empty((N, cfg["HV"], cfg["K"], cfg["V"]), dtype=torch.float32, device="cuda")}
        args_c = [ctypes.byref(prob), P(dev["q"]), P(dev["k"]), P(dev["v"]), P(dev["gcum"]), P(dev["beta"]), None,
                  P(dev["dO"]), P(dev["dht"]), P(out["dq"]), P(out["dk"]), P(out["dv"]), P(out["dg"]),
                  P(out["dbeta"]), P(out["dh0"]), P(ws), ws.numel(), sp]

    def check(rc):
        if rc != 0:
            raise binding.GdrError(rc, binding.lib.gdr_strerror(rc).decode())

    def call(i=None):
        if fwd:
            if i is not None:
                assert hip.hipEventRecord(ctypes.c_void_p(evs[nev * i]), sp) == 0
            check(binding.lib.gdr_gate_cumsum(ctypes.byref(gprob), P(dev["graw"]), P(gc), sp))
            ev = None if i is None else ctypes.byref(evs, (nev * i + 1) * evsz)
            check(binding.lib.gdr_chunk_fwd_events(*args_c, ev))
        else:
            ev = None if i is None else ctypes.byref(evs, nev * i * evsz)
            check(binding.lib.gdr_chunk_bwd_events(*args_c, ev))

    per_call, st, wall = timed_calls(torch, hip, evs, nev, call, args.steps, args.warmup, evict)
    names = (["gate", "prep", "scans", "out"] if fwd else ["prep", "scans", "grad"])
    stage = dict(zip(names, st))
    chunks = chunk_lengths(lengths, cfg["T"], cfg["B"], 64)
    del keep, ws, out, dev
    return {"cfg": cfg, "inp": inp, "chunks": chunks, "stats": call_stats(per_call), "stage": stage,
            "wall_ms": wall, "T": T}


def gdn_summary(r, fwd):
    """Per-workload figures: median ms, effective TFLOP/s, stage times and each
    stage's algorithmic HBM rate (and matrix-core rates for the backward's
    chunk-parallel kernels)."""
    cfg, chunks, stage = r["cfg"], r["chunks"], r["stage"]
    model = flop_model_fwd if fwd else flop_model
    F = sum(model(c, cfg["K"], cfg["V"]) for c in chunks) * cfg["HV"]
    ms = r["stats"]["median_ms"]
    kb = kernel_bytes_fwd(cfg, chunks) if fwd else kernel_bytes(cfg, chunks)
    units = len(chunks) * cfg["HV"]
    stages = {}
    for k, t in stage.items():
        gbs = kb[k] / (t * 1e-3) / 1e9
        e = {"ms": round(t, 4), "algorithmic_bytes": kb[k], "hbm_gbs": round(gbs, 1),
             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if not fwd and k == "prep":
            tf = mfma_work_prep(cfg["K"], cfg["V"]) * units / (t * 1e-3) / 1e12
            e.update({"mfma_executed_tflops": round(tf, 1), "mfma_executed_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        if not fwd and k == "grad":
            fa = sum(flop_grad_algorithmic(c, cfg["K"], cfg["V"]) for c in chunks) * cfg["HV"]
            tf = fa / (t * 1e-3) / 1e12
            tx = mfma_work_grad(cfg["K"], cfg["V"]) * units / (t * 1e-3) / 1e12
            e.update({"algorithmic_flop": fa, "mfma_tflops": round(tf, 1),
                      "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                      "mfma_executed_tflops": round(tx, 1), "mfma_executed_frac": round(tx / MFMA_BF16_PEAK_TFLOPS, 4)})
        stages[k] = e
    return {"F": F, "tflops": F / (ms * 1e-3) / 1e12, "kb": kb, "stages": stages}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense_t32k_h16", choices=list(WORKLOADS))
    ap.add_argument("--path", default="bwd", choices=["bwd", "fwd", "kda", "kda_stage", "bigdn"],
                    help="bwd: the chunked backward (default); fwd: gate cumsum + chunked forward; "
                         "kda: the full KDA backward at B=1 T=2048 H=32 K=V=128 fp16; "
                         "kda_stage: the KDA WY backward stage alone on the same shape; "
                         "bigdn: the BiGDN layer backward at B=8 F=11 S=1024 H=16 D=128 bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="bwd: time only --workload")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only (the backward of one GPU's share); "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from chunked_gated_delta_08_amd import binding, profiling, workloads

    evict = Evictor(torch)
    if args.path == "kda":
        return bench_kda(args, torch, binding, profiling, workloads, evict)
    if args.path == "kda_stage":
        return bench_kda_stage(args, torch, binding, profiling, workloads, evict)
    if args.path == "bigdn":
        return bench_bigdn(args, torch, binding, profiling, workloads, evict)
    fwd = args.path == "fwd"
    r = run_gdn(args, torch, binding, workloads, args.workload, fwd, evict)
    sm = gdn_summary(r, fwd)
    cfg, stage, kb = r["cfg"], r["stage"], sm["kb"]
    if fwd:
        kn = {"gate": "gate_cumsum_kernel", "prep": "prep_kernel", "scans": "scan_kernel", "out": "fwd_out_kernel"}
        roof = _roofline(stage, kb, kn, "fwd_" + args.workload, profiling)
    else:
        # the gradient kernel against the dense bf16 MFMA peak on its algorithmic
        # FLOPs (the backward's target), with its HBM view and executed work beside it
        g = sm["stages"]["grad"]
        roof = {"bound": "mfma", "achieved": g["mfma_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": g["mfma_frac"], "traffic": _traffic("grad_kernel", args.workload, profiling),
                "kernel": "grad_kernel", "kernel_ms": g["ms"], "algorithmic_flop": g["algorithmic_flop"],
                "hbm": {"achieved": g["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": g["hbm_frac"],
                        "algorithmic_bytes": g["algorithmic_bytes"]},
                "executed": {"tflops": g["mfma_executed_tflops"], "frac": g["mfma_executed_frac"]},
                "stage_ms": {k: round(v, 4) for k, v in stage.items()}}
    roof["stages"] = sm["stages"]
    st = r["stats"]
    wname = cfg["name"].replace("gdn_bwd", "gdn_fwd") if fwd else cfg["name"]
    what = "fwd" if fwd else "bwd"
    res = {"metric": f"GDN chunked {what} ms/call + eff. TFLOP/s at T=32k, H=16/32, K=V=128, BT=64",
           "value": round(sm["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": st["median_ms"], "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
           "wall_ms_per_step_with_evict": round(r["wall_ms"], 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded randn / logsigmoid / sigmoid, as the pages' workloads)",
           "config": {"workload": wname, "B": cfg["B"], "T": r["T"], "HK": cfg["HK"], "HV": cfg["HV"],
                      "K": cfg["K"], "V": cfg["V"], "BT": 64, "global_batch": cfg["B"], "seq_len": r["T"],
                      "parallelism": "none", "flop_model_gflop": round(sm["F"] / 1e9, 2),
                      "timing": "median of per-call HIP events, 512 MiB cache-evicting write before each call"},
           "roofline": roof}
    if not fwd and not args.no_also:
        also = []
        for wk in WORKLOADS:
            if wk == args.workload:
                continue
            ro = run_gdn(args, torch, binding, workloads, wk, False, evict)
            so = gdn_summary(ro, False)
            g = so["stages"]["grad"]
            also.append({"workload": ro["cfg"]["name"], "ms_per_call": ro["stats"]["median_ms"],
                         "p10_ms": ro["stats"]["p10_ms"], "p90_ms": ro["stats"]["p90_ms"],
                         "tflops": round(so["tflops"], 2), "flop_model_gflop": round(so["F"] / 1e9, 2),
                         "stage_ms": {k: round(v, 4) for k, v in ro["stage"].items()},
                         "grad_mfma_frac": g["mfma_frac"], "grad_hbm_frac": g["hbm_frac"],
                         "scans_hbm_frac": so["stages"]["scans"]["hbm_frac"]})
            del ro
        res["also"] = also
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(r["inp"], cfg, r["chunks"], path=args.path)
    print(json.dumps(res), flush=True)


def bench_kda(args, torch, binding, profiling, workloads, evict):
    """One step = one kda_chunk_bwd_full call at B=1, T=2048, H=32, K=V=128, fp16."""
    B, T, H, K, V = 1, 2048, 32, 128, 128
    cfg = dict(B=B, T=T, HK=H, HV=H, K=K, V=V, name="kda_bwd_T2048_h32_K128_V128_BT64_f16")
    inp = workloads.kda_full_inputs(B, T, H, K, V, dtype="f16", seed=0)
    dev = {n: inp[n].cuda() for n in ("q", "k", "v", "beta", "dO", "gcum", "dht")}
    prob, keep = binding.make_problem(B, T, H, H, K, V, torch.float16, 64, None)
    ws = torch.empty(int(binding.lib.kda_workspace_size(ctypes.byref(prob))), dtype=torch.uint8, device="cuda")
    out = {"dq": torch.empty_like(dev["q"]), "dk": torch.empty_like(dev["k"]), "dv": torch.empty_like(dev["v"]),
           "dg": torch.empty(dev["gcum"].shape, dtype=torch.float32, device="cuda"),
           "dbeta": torch.empty(dev["beta"].shape, dtype=torch.float32, device="cuda"),
           "dh0": torch.empty((B, H, K, V), dtype=torch.float32, device="cuda")}
    P = binding._ptr
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args_c = [ctypes.byref(prob), P(dev["q"]), P(dev["k"]), P(dev["v"]), P(dev["gcum"]), P(dev["beta"]), None,
              P(dev["dO"]), P(dev["dht"]), P(out["dq"]), P(out["dk"]), P(out["dv"]), P(out["dg"]), P(out["dbeta"]),
              P(out["dh0"]), P(ws), ws.numel(), sp]
    nev = 5
    hip, evs = hip_events(nev * args.steps)
    evsz = ctypes.sizeof(ctypes.c_void_p)

    def call(i=None):
        ev = None if i is None else ctypes.byref(evs, nev * i * evsz)
        rc = binding.lib.kda_chunk_bwd_full_events(*args_c, ev)
        if rc != 0:
            raise binding.GdrError(rc, binding.lib.gdr_strerror(rc).decode())

    per_call, st, wall = timed_calls(torch, hip, evs, nev, call, args.steps, args.warmup, evict)
    stats = call_stats(per_call)
    ms_per_step = stats["median_ms"]
    stage = dict(zip(["prep", "scans", "stage", "intra"], st))
    chunks = chunk_lengths(None, T, B, 64)
    F = sum(flop_model(c, K, V) for c in chunks) * H
    kb = kernel_bytes_kda(H, K, V, chunks)
    kn = {"prep": "kda_prep_kernel", "scans": "kda_scan_kernel", "stage": "kda_kernel", "intra": "kda_intra_kernel"}
    roof = _roofline(stage, kb, kn, "kda_t2048_h32", profiling)
    res = {"metric": "KDA chunked bwd (full, per-channel gate) ms/call + eff. TFLOP/s at T=2048, H=32, K=V=128, BT=64",
           "value": round(F / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "p10_ms": stats["p10_ms"], "p90_ms": stats["p90_ms"],
           "wall_ms_per_step_with_evict": round(wall, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16",
           "data": "synthetic (seeded randn / logsigmoid / sigmoid, as the pages' workloads)",
           "config": {"workload": cfg["name"], "B": B, "T": T, "HK": H, "HV": H, "K": K, "V": V, "BT": 64,
                      "global_batch": B, "seq_len": T, "parallelism": "none", "flop_model_gflop": round(F / 1e9, 2),
                      "timing": "median of per-call HIP events, 512 MiB cache-evicting write before each call"},
           "roofline": roof}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, cfg, chunks, path="kda")
    del keep
    print(json.dumps(res), flush=True)


def flop_model_kda_stage(C, K, V):
    """Products of the KDA WY backward stage per (chunk, head): dq = dO hᵀ,
    dk_s = V_new dhᵀ, dw = -dv hᵀ (2CKV each); Aᵀ dv, Aᵀ dw (2C²V, 2C²K), dA_pre
    (2C²V + 2C²K); the two C³ products of dA."""
    return 6 * C * K * V + 4 * C * C * (K + V) + 4 * C ** 3


def bench_kda_stage(args, torch, binding, profiling, workloads, evict):
    """One step = one kda_chunk_bwd call (the WY stage alone) at B=1, T=2048,
    H=32, K=V=128, BT=64, fp16, on the page's example inputs."""
    B, T, H, K, V, BT = 1, 2048, 32, 128, 128, 64
    inp = workloads.kda_inputs(B=B, T=T, H=H, K=K, V=V, BT=BT, dtype="f16", seed=0)
    names = ("q", "k", "v", "v_new", "g", "beta", "A", "h", "dO", "dh", "dv")
    dev = {n: inp[n].cuda() for n in names}
    prob, keep = binding.make_problem(B, T, H, H, K, V, torch.float16, BT, None)
    ntok = B * T
    out = {"dq": torch.empty((ntok, H, K), dtype=torch.float32, device="cuda"),
           "dk": torch.empty((ntok, H, K), dtype=torch.float32, device="cuda"),
           "dv": torch.empty_like(dev["v"]),
           "db": torch.empty((ntok, H), dtype=torch.float32, device="cuda"),
           "dg": torch.empty((ntok, H, K), dtype=torch.float32, device="cuda"),
           "dA": torch.empty((ntok, H, BT), dtype=torch.float32, device="cuda")}
    P = binding._ptr
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args_c = [ctypes.byref(prob)] + [P(dev[n]) for n in names] + \
        [P(out[n]) for n in ("dq", "dk", "dv", "db", "dg", "dA")] + [sp]
    nev = 2
    hip, evs = hip_events(nev * args.steps)

    def call(i=None):
        if i is not None:
            assert hip.hipEventRecord(ctypes.c_void_p(evs[nev * i]), sp) == 0
        rc = binding.lib.kda_chunk_bwd(*args_c)
        if rc != 0:
            raise binding.GdrError(rc, binding.lib.gdr_strerror(rc).decode())
        if i is not None:
            assert hip.hipEventRecord(ctypes.c_void_p(evs[nev * i + 1]), sp) == 0

    per_call, st, wall = timed_calls(torch, hip, evs, nev, call, args.steps, args.warmup, evict)
    stats = call_stats(per_call)
    ms = stats["median_ms"]
    chunks = chunk_lengths(None, T, B, BT)
    F = sum(flop_model_kda_stage(c, K, V) for c in chunks) * H
    # algorithmic bytes: every input read once, every output written once
    nbytes = sum(dev[n].numel() * dev[n].element_size() for n in names) + \
        sum(t.numel() * t.element_size() for t in out.values())
    gbs = nbytes / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": _traffic("kda_kernel", "kda_stage_t2048_h32", profiling),
            "kernel": "kda_kernel", "kernel_ms": ms, "algorithmic_bytes": nbytes,
            "floor_us": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 1)}
    res = {"metric": "KDA WY bwd stage (kda_chunk_bwd) ms/call + eff. TFLOP/s at T=2048, H=32, K=V=128, BT=64",
           "value": round(F / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "p10_ms": stats["p10_ms"], "p90_ms": stats["p90_ms"],
           "wall_ms_per_step_with_evict": round(wall, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16",
           "data": "synthetic (seeded randn / logsigmoid / sigmoid; A lower-triangular randn), the page's example",
           "config": {"workload": "kda_wy_stage_T2048_h32_K128_V128_BT64_f16", "B": B, "T": T, "HK": H, "HV": H,
                      "K": K, "V": V, "BT": BT, "global_batch": B, "seq_len": T, "parallelism": "none",
                      "flop_model_gflop": round(F / 1e9, 3),
                      "timing": "median of per-call HIP events, 512 MiB cache-evicting write before each call"},
           "roofline": roof}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_kda_stage(inp, F)
    del keep
    print(json.dumps(res), flush=True)


def cpu_baseline_kda_stage(inp, flops):
    """The oracle's KDA stage VJP (O-K), unchanged, over every head of the
    workload, repeated until at least 10 s have elapsed."""
    from oracle import oracle as O
    f = lambda n: inp[n].double().numpy()  # noqa: E731
    p = O.Problem(inp["B"], inp["T"], inp["H"], inp["H"], inp["K"], inp["V"])
    args = [f(n) for n in ("q", "k", "v", "v_new", "g", "beta", "A", "h", "dO", "dh", "dv")]
    passes, dt = 0, 0.0
    while dt < 10.0:
        t0 = time.perf_counter()
        O.kda_wy_bwd(p, inp["BT"], *args)
        dt += time.perf_counter() - t0
        passes += 1
    res = {"value": round(passes * flops / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"{passes} full pass(es) over the workload ({dt:.1f} s): fp64 VJP of the stage functional, "
                     "OpenMP over (chunk, head)", "seconds": round(dt, 2)}
    res.update(host_info(O.num_threads()))
    return res


def flop_model_bigdn(B, F, S, H, D):
    """Products of the page's BiGDN backward per frame (forward recompute not
    counted): phase C-bar dQ = dO Mc^T and dMc = Q^T dO (2 x 2SD^2); phase A-bar
    K dP, K dP^T, V dA^T, K dA (4 x 2SD^2) and K dPz, K dPz^T (2 x 2SD^2); the
    combine's dM Mprev^T and (I - P) Mprev for both directions (4 x 2D^3) and
    the two gradient scans' (I - P)^T dM (2 x 2D^3):  16 S D^2 + 12 D^3."""
    return B * H * F * (16 * S * D * D + 12 * D ** 3)


def kernel_bytes_bigdn(B, F, S, H, D, nblk):
    """Algorithmic HBM bytes per launch of each BiGDN backward stage: tensors
    read once and written once per launch (bf16 activations; fp32 gates, norm
    weights and rope tables; per-frame D x D intermediates as the kernels store
    them: P, Mf, Mr, Tf, Tr in bf16, A, Pz, dMc in fp32)."""
    ntok, NF, C = B * F * S, B * H * F, H * D
    act = ntok * C * 2                 # one bf16 [B, N, H, D] tensor
    rope = 2 * F * S * D * 4
    DDb, DDf, vec = NF * D * D * 2, NF * D * D * 4, NF * D * 4
    beta = ntok * H * 4
    return {
        "stats": 2 * act + 2 * ntok * 4,
        "phase_a": 2 * act + beta + ntok * 4 + C * 4 + rope + DDb + 2 * DDf + vec,
        "scans": DDb + 2 * DDf + vec + 2 * DDb + 2 * vec + NF * 4,
        "phase_c": 2 * act + ntok * 4 + C * 4 + rope + 2 * DDb + 2 * vec + act + DDf + vec,
        "gscans": DDf + DDb + DDf + vec + 2 * DDb + 2 * vec + NF * 4,
        "abar": 2 * act + beta + ntok * 4 + C * 4 + rope + DDb + DDf + 2 * DDb + 2 * DDb + 4 * vec + NF * 4
                + 2 * act + beta + NF * 4,
        "rms_bwd": 4 * act + 2 * ntok * 4 + 2 * C * 4 + 2 * act + 2 * nblk * 2 * C * 4 + 2 * C * 4,
    }


def cpu_baseline_bigdn(inp, flops_row):
    """The fp64 oracle (forward recompute + hand-derived backward), unchanged,
    on batch row 0 of the workload, repeated until at least 10 s have elapsed."""
    from oracle import bigdn_oracle as BO
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = 1
    f = lambda n: inp[n].double().numpy()[:1] if n in ("qkv", "beta", "decay", "dout") else inp[n].double().numpy()  # noqa: E731,E501
    args = [f(n) for n in ("qkv", "beta", "decay", "qw", "kw", "cos", "sin")]
    passes, dt = 0, 0.0
    while dt < 10.0:
        t0 = time.perf_counter()
        BO.bigdn_bwd(*args, f("dout"), inp["F"], inp["S"], k_scale=inp["k_scale"])
        dt += time.perf_counter() - t0
        passes += 1
    res = {"value": round(passes * flops_row / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"{passes} pass(es) over batch row 0 of {inp['B']} ({dt:.1f} s): fp64 numpy forward recompute "
                     "+ hand-derived backward, BLAS threads for the per-frame products",
           "seconds": round(dt, 2)}
    res.update(host_info(cores))
    return res


def bench_bigdn(args, torch, binding, profiling, workloads, evict):
    """One step = one bigdn_bwd call at B=8, F=11, S=1024, H=16, D=128, bf16."""
    B, F, S, H, D = 8, 11, 1024, 16, 128
    inp = workloads.bigdn_inputs(B, F, S, H, D, seed=0)
    dev = {n: inp[n].cuda() for n in ("qkv", "beta", "decay", "qw", "kw", "cos", "sin", "dout")}
    prob = binding.bigdn_problem(dev["qkv"], F, S, inp["k_scale"])
    ws = torch.empty(binding.bigdn_workspace_size(prob, True), dtype=torch.uint8, device="cuda")
    out = {"dqkv": torch.empty_like(dev["qkv"]), "dbeta": torch.empty_like(dev["beta"]),
           "ddecay": torch.empty_like(dev["decay"]), "dqw": torch.empty_like(dev["qw"]),
           "dkw": torch.empty_like(dev["kw"])}
    P = binding._ptr
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args_c = [ctypes.byref(prob), P(dev["qkv"]), P(dev["beta"]), P(dev["decay"]), P(dev["qw"]), P(dev["kw"]),
              P(dev["cos"]), P(dev["sin"]), P(dev["dout"]), P(out["dqkv"]), P(out["dbeta"]), P(out["ddecay"]),
              P(out["dqw"]), P(out["dkw"]), P(ws), ws.numel(), sp]
    nev = 8
    hip, evs = hip_events(nev * args.steps)
    evsz = ctypes.sizeof(ctypes.c_void_p)

    def call(i=None):
        ev = None if i is None else ctypes.byref(evs, nev * i * evsz)
        rc = binding.lib.bigdn_bwd_events(*args_c, ev)
        if rc != 0:
            raise binding.GdrError(rc, binding.lib.gdr_strerror(rc).decode())

    per_call, st, wall = timed_calls(torch, hip, evs, nev, call, args.steps, args.warmup, evict)
    stats = call_stats(per_call)
    ms_per_step = stats["median_ms"]
    names = ["stats", "phase_a", "scans", "phase_c", "gscans", "abar", "rms_bwd"]
    stage = dict(zip(names, st))
    Fl = flop_model_bigdn(B, F, S, H, D)
    nblk = min(768, (B * F * S + 3) // 4)
    kb = kernel_bytes_bigdn(B, F, S, H, D, nblk)
    kn = {"stats": "bigdn_stats_kernel", "phase_a": "bigdn_phase_a_kernel", "scans": "bigdn_scan_kernel",
          "phase_c": "bigdn_phase_c_kernel", "gscans": "bigdn_scan_kernel", "abar": "bigdn_abar_kernel",
          "rms_bwd": "bigdn_rms_bwd_kernel"}
    roof = _roofline(stage, kb, kn, "bigdn_b8_f11_s1024_h16", profiling)
    roof["call_algorithmic_bytes"] = sum(kb.values())
    roof["call_hbm_frac"] = round(sum(kb.values()) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    res = {"metric": "BiGDN chunkwise bwd ms/call + eff. TFLOP/s at B=8, F=11, S=1024, H=16, D=128",
           "value": round(Fl / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "p10_ms": stats["p10_ms"], "p90_ms": stats["p90_ms"],
           "wall_ms_per_step_with_evict": round(wall, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded randn / sigmoid, rotary tables, as the page's layer inputs)",
           "config": {"workload": "bigdn_bwd_B8_F11_S1024_H16_D128_bf16", "B": B, "F": F, "S": S, "H": H, "D": D,
                      "k_scale": inp["k_scale"], "global_batch": B, "seq_len": F * S, "parallelism": "none",
                      "flop_model_gflop": round(Fl / 1e9, 2)},
           "roofline": roof}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_bigdn(inp, Fl / B)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
