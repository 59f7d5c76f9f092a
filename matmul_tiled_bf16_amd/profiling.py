"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    # kernel time (one run):
    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- python bench.py ...
    # HBM traffic (two counter runs, each its own pass), and the same two
    # counters for a plain device copy of known size (the calibration):
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- python bench.py ...
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- python bench.py ...
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/cfetch -o run -- python bench.py --copy-calibration
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/cwrite -o run -- python bench.py --copy-calibration

    python -m matmul_tiled_bf16_amd.profiling stats OUT/trace [gemm|group|attention] > profiles/<kernel>_<workload>_stats.txt
    python -m matmul_tiled_bf16_amd.profiling traffic OUT <workload> > profiles/<workload>_traffic.txt

FETCH_SIZE / WRITE_SIZE are reported in KiB per dispatch; the copy kernel
moves a known number of bytes, and the ratio of that number to what the
counter reads for it scales the kernel's reading to bytes.  A traffic file
records a hash of the sources its kernel family (GEMM, grouped GEMM or
attention) is built from; bench.py reports traffic only while those sources still match.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30  # bytes read and written by one calibration copy

def _gemm_source(f: str) -> bool:
    """Sources of the GEMM kernels and their launcher: everything but the fused
    attention and the split-K driver (host code plus its reduction kernel)."""
    b = os.path.basename(f)
    return not b.startswith("attention") and b != "splitk.hip"


# kernel families: the kernels' name patterns and the sources they are built from
FAMILIES = {
    "gemm": (("tile_gemm_kernel", "pingpong_gemm_kernel", "panel_gemm_kernel", "skinny_gemm_kernel",
              "generic_gemm_kernel"),
             lambda f: _gemm_source(f)),
    "group": (("group_gemm_kernel",), lambda f: _gemm_source(f)),
    "attention": (("attn_fwd_kernel",),
                  lambda f: os.path.basename(f) in ("attention.hpp", "attention.hip", "tile_gemm.hpp",
                                                    "common.hpp")),
}


def family_of(workload: str) -> str:
    if workload.startswith("attn_fwd"):
        return "attention"
    if workload.startswith("grouped"):
        return "group"
    return "gemm"


def source_hash(family: str = "gemm") -> str:
    """Hash of the sources the family's kernels are built from."""
    keep = FAMILIES[family][1]
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if not keep(f):
            continue
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv(path_dir: str, suffix: str):
    files = glob.glob(os.path.join(path_dir, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {path_dir}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    return name if len(name) <= 110 else name[:107] + "..."


def stats(trace_dir: str, family: str = "gemm") -> str:
    rows = _csv(trace_dir, "kernel_stats.csv")
    out = [f"# rocprofv3 --kernel-trace --stats summary  ({family} source hash {source_hash(family)})",
           f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel"]
    for r in rows:
        avg = float(r["AverageNs"]) / 1e3
        mn = float(r["MinNs"]) / 1e3
        mx = float(r["MaxNs"]) / 1e3
        out.append(f"{int(r['Calls']):>6} {avg:>10.2f} {mn:>10.2f} {mx:>10.2f} {float(r['Percentage']):>8.2f}  "
                   f"{_short(r['Name'])}")
    return "\n".join(out)


def _per_dispatch(path_dir: str, counter: str, match) -> list:
    vals = defaultdict(float)
    for r in _csv(path_dir, "counter_collection.csv"):
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return list(vals.values())


def traffic(out_dir: str, workload: str) -> str:
    family = family_of(workload)
    is_ours = lambda n: any(p in n for p in FAMILIES[family][0])
    is_copy = lambda n: "copy" in n.lower() and not is_ours(n)
    f = _per_dispatch(os.path.join(out_dir, "fetch"), "FETCH_SIZE", is_ours)
    w = _per_dispatch(os.path.join(out_dir, "write"), "WRITE_SIZE", is_ours)
    cf = _per_dispatch(os.path.join(out_dir, "cfetch"), "FETCH_SIZE", is_copy)
    cw = _per_dispatch(os.path.join(out_dir, "cwrite"), "WRITE_SIZE", is_copy)
    mean = lambda v: sum(v) / len(v)
    # the copy reads and writes COPY_BYTES: factor = true bytes per counted KiB
    kf = COPY_BYTES / mean(cf)
    kw = COPY_BYTES / mean(cw)
    fetch = mean(f) * kf
    write = mean(w) * kw
    lines = [
        f"# HBM traffic per launch of the {family} kernel, workload {workload}",
        f"source_hash = {source_hash(family)}",
        f"dispatches_fetch = {len(f)}",
        f"dispatches_write = {len(w)}",
        f"fetch_kib_counter = {mean(f):.1f}",
        f"write_kib_counter = {mean(w):.1f}",
        f"copy_bytes = {COPY_BYTES}",
        f"copy_fetch_kib_counter = {mean(cf):.1f}",
        f"copy_write_kib_counter = {mean(cw):.1f}",
        f"fetch_factor_bytes_per_kib = {kf:.2f}",
        f"write_factor_bytes_per_kib = {kw:.2f}",
        f"fetch_bytes = {fetch:.0f}",
        f"write_bytes = {write:.0f}",
        f"traffic_bytes = {fetch + write:.0f}",
    ]
    return "\n".join(lines)


def read_traffic(workload: str):
    """Traffic recorded for `workload`, or None if missing or the kernels changed since."""
    path = os.path.join(os.path.dirname(HERE), "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(family_of(workload)):
        return None
    return float(kv["traffic_bytes"])


def main(argv):
    if argv[0] == "stats":
        print(stats(argv[1], argv[2] if len(argv) > 2 else "gemm"))
    elif argv[0] == "traffic":
        print(traffic(argv[1], argv[2]))
    elif argv[0] == "hash":
        print(source_hash(argv[1] if len(argv) > 1 else "gemm"))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
