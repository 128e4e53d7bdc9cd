"""Reproducible rocprofv3 summaries for the library's kernels.

Subcommands (run with ``python -m chunked_gated_delta_08_amd.profiling``):

  copy [--mib M]
      Runs a plain elementwise device copy of known size (reads M MiB, writes M
      MiB, fp32, ``torch.mul(src, 1, out=dst)``) a few times: the calibration
      kernel for the FETCH_SIZE / WRITE_SIZE counters.
  stats --csv <prefix>_kernel_stats.csv --out <txt> --cmd "<command>"
      Writes a short text table of per-kernel dispatch counts and durations.
  traffic --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV
          --copy-mib M --workload W --cmd "<command>" --outdir DIR
      Turns per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the library kernels
      into HBM bytes per launch, each counter scaled by the ratio between the
      copy kernel's known bytes and what the same counter reads for it, and
      writes traffic_<kernel>_<workload>.json (+ one .txt for all kernels).

A traffic file records a digest of the kernel's sources (their code, comments
and layout left out); readers ignore it once that code has changed.
"""
import argparse
import collections
import csv
import hashlib
import re
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_CS = "chunked_gated_delta_08_amd/csrc/"
_COMMON = [_CS + "gdr_device.hpp", _CS + "gdr_launch.hpp", "chunked_gated_delta_08_amd/build.py"]
KERNEL_SOURCES = {
    "chunk_table_kernel": [_CS + "gdr_prep.hip"] + _COMMON,
    "prep_kernel": [_CS + "gdr_prep.hip", _CS + "gdr_tri.hpp"] + _COMMON,
    "scan_kernel": [_CS + "gdr_scan.hip"] + _COMMON,
    "seg_kernel": [_CS + "gdr_scan.hip"] + _COMMON,
    "combine_kernel": [_CS + "gdr_scan.hip"] + _COMMON,
    "dmax_kernel": [_CS + "gdr_scan.hip"] + _COMMON,
    "dscale_kernel": [_CS + "gdr_scan.hip"] + _COMMON,
    "grad_kernel": [_CS + "gdr_grad.hip"] + _COMMON,
    "kda_kernel": [_CS + "kda_bwd.hip"] + _COMMON,
    "fwd_out_kernel": [_CS + "gdr_fwd.hip"] + _COMMON,
    "gate_cumsum_kernel": [_CS + "gdr_fwd.hip"] + _COMMON,
    "kda_prep_kernel": [_CS + "kda_full.hip", _CS + "gdr_tri.hpp"] + _COMMON,
    "kda_scan_kernel": [_CS + "kda_full.hip"] + _COMMON,
    "kda_intra_kernel": [_CS + "kda_full.hip"] + _COMMON,
}
_BIGDN = [_CS + "bigdn.hip", _CS + "bigdn_launch.hpp"] + _COMMON
for _k in ("bigdn_stats_kernel", "bigdn_phase_a_kernel", "bigdn_scan_kernel", "bigdn_phase_c_kernel",
           "bigdn_abar_kernel", "bigdn_rms_bwd_kernel", "bigdn_wsum_kernel"):
    KERNEL_SOURCES[_k] = _BIGDN


def _code_of(text):
    """The text of a source file without its comments and layout: whitespace
    is kept only where it separates two identifier characters, so a digest of
    it follows the code alone (line breaks and indentation do not count)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"(?<!:)//[^\n]*", " ", text)   # comment to end of line
    text = " ".join(text.split())
    return re.sub(r"(?<![A-Za-z0-9_]) | (?![A-Za-z0-9_])", "", text)


def source_digest(files):
    """Digest of the code (comments and layout left out) of the given files."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_of(fh.read()).encode("utf-8"))
    return h.hexdigest()[:16]


def short_name(full):
    """Library kernel name (``gdr::grad_kernel<...>`` or its mangled form ->
    ``grad_kernel``), else None.  The whole identifier must match
    (``prep_kernel`` is not ``kda_prep_kernel``)."""
    for k in KERNEL_SOURCES:
        if f"{len(k)}{k}" in full or re.search(r"::" + k + r"[(<]", full):
            return k
    return None


def _copy(args):
    import torch
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(f"copy: {args.reps} x {args.mib} MiB read + {args.mib} MiB written", flush=True)


def _stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics ({args.title})", "",
             "command:", "  " + args.cmd, "",
             f"{'kernel':<28} {'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'total %':>8}"]
    evict = False
    for r in rows:
        nm = short_name(r["Name"])
        if nm is None and "FillFunctor" in r["Name"]:
            nm, evict = "bench_evict_fill", True
        nm = nm or r["Name"][:28]
        lines.append(f"{nm:<28} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.1f} "
                     f"{float(r['MinNs']) / 1e3:>10.1f} {float(r['MaxNs']) / 1e3:>10.1f} "
                     f"{float(r['Percentage']):>8.2f}")
    if evict:
        lines += ["", "bench_evict_fill: bench.py's 512 MiB cache-evicting write before each call (outside the call)"]
    lines += ["", "full kernel names:"] + [f"  {r['Name']}" for r in rows if short_name(r["Name"])]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_kernel(path, counter):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _copy_kib(path, counter):
    vals = [v for k, vs in _per_kernel(path, counter).items() if "MulFunctor" in k for v in vs]
    return sorted(vals)[len(vals) // 2]   # median over the copy dispatches


def _traffic(args):
    copy_bytes = args.copy_mib * (1 << 20)
    f_fetch = copy_bytes / (_copy_kib(args.copy_fetch, "FETCH_SIZE") * 1024)
    f_write = copy_bytes / (_copy_kib(args.copy_write, "WRITE_SIZE") * 1024)
    fetch = _per_kernel(args.fetch, "FETCH_SIZE")
    write = _per_kernel(args.write, "WRITE_SIZE")
    lines = [f"# HBM traffic per launch, workload {args.workload}", "",
             "commands:", "  " + args.cmd, "",
             f"copy calibration ({args.copy_mib} MiB read + written): FETCH_SIZE scale {f_fetch:.4f}, "
             f"WRITE_SIZE scale {f_write:.4f}", "",
             f"{'kernel':<20} {'launches':>8} {'FETCH KiB':>12} {'WRITE KiB':>12} {'HBM MB/launch':>14}"]
    for full in sorted(fetch):
        k = short_name(full)
        if k is None or full not in write:
            continue
        fk = sum(fetch[full]) / len(fetch[full])
        wk = sum(write[full]) / len(write[full])
        bpl = fk * 1024 * f_fetch + wk * 1024 * f_write
        lines.append(f"{k:<20} {len(fetch[full]):>8} {fk:>12.0f} {wk:>12.0f} {bpl / 1e6:>14.2f}")
        rec = {"kernel": k, "workload": args.workload, "fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
               "fetch_scale": f_fetch, "write_scale": f_write, "bytes_per_launch": round(bpl),
               "sources": KERNEL_SOURCES[k], "source_digest": source_digest(KERNEL_SOURCES[k]),
               "command": args.cmd}
        with open(os.path.join(args.outdir, f"traffic_{k}_{args.workload}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    with open(os.path.join(args.outdir, f"traffic_{args.workload}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m chunked_gated_delta_08_amd.profiling")
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload", "--cmd", "--outdir"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args(argv)
    {"copy": _copy, "stats": _stats, "traffic": _traffic}[args.cmd_name](args)


if __name__ == "__main__":
    sys.exit(main())
