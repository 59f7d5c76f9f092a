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

    # counters of the intact kernel (four passes, each its own run; PASSES below):
    rocprofv3 --pmc <PASSES[i]> --output-format csv -d OUT/pmc<i+1> -o run -- python bench.py ...
    python -m matmul_tiled_bf16_amd.profiling counters OUT <kernel-name-part> > profiles/<kernel>_<workload>_counters.txt

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
              "kslice_gemm_kernel", "generic_gemm_kernel"),
             lambda f: _gemm_source(f)),
    "group": (("group_gemm_kernel",), lambda f: _gemm_source(f)),
    "attention": (("attn_pp_kernel",),
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


def traffic_note(workload: str) -> str:
    """Where a bench record's `traffic` comes from (it is never measured in the timed run)."""
    if read_traffic(workload) is None:
        return f"null: profiles/{workload}_traffic.txt is missing or was taken on other kernel sources"
    return (f"profiles/{workload}_traffic.txt: FETCH_SIZE and WRITE_SIZE counter runs of the same kernel "
            "sources (source hash matched), scaled by a plain-copy calibration; not measured in this run")


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


# Counter passes for the utilisation summary: each fits one rocprofv3 pass
# (at most 8 SQ, 4 TCC and 2 GRBM counters).
PASSES = [
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_BUSY_CU_CYCLES SQ_WAVE_CYCLES SQ_WAVES GRBM_GUI_ACTIVE",
    "SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_LDS_CMD_FIFO_FULL "
    "SQ_LDS_ADDR_CONFLICT SQ_LDS_UNALIGNED_STALL GRBM_GUI_ACTIVE",
    "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
    "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_VMEM_RD "
    "SQ_INSTS_VMEM_WR SQ_WAVES",
    # the HBM/L2 -> LDS copy path: texture address (TA) and data (TD) units, L1 (TCP)
    "TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum TD_TD_BUSY_sum TD_TC_STALL_sum GRBM_GUI_ACTIVE",
    "TA_BUFFER_TOTAL_CYCLES_sum TA_DATA_STALLED_BY_TC_CYCLES_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum "
    "TCP_PENDING_STALL_CYCLES_sum TCP_TCR_TCP_STALL_CYCLES_sum GRBM_GUI_ACTIVE",
]
N_XCD = 8            # MI355X: GRBM_GUI_ACTIVE reads the sum over its 8 XCDs
N_SIMD = 256 * 4     # 256 CUs x 4 SIMDs
FLOP_PER_CU_CLK = 4096  # dense bf16/fp16 MFMA


def _dispatches(path_dir: str, match):
    """{dispatch: {counter: value, '_ns': duration, '_regs': (...)}} for matching kernels."""
    out = defaultdict(dict)
    for r in _csv(path_dir, "counter_collection.csv"):
        if not match(r["Kernel_Name"]):
            continue
        d = out[r["Dispatch_Id"]]
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        d["_name"] = r["Kernel_Name"]
        d["_regs"] = (r.get("VGPR_Count"), r.get("Accum_VGPR_Count"), r.get("SGPR_Count"), r.get("Scratch_Size"),
                      r.get("Workgroup_Size"), r.get("Grid_Size"))
    return out


def counters(out_dir: str, pattern: str) -> str:
    """Utilisation summary of the kernels whose name contains `pattern`, from the
    four PASSES runs under out_dir/pmc1 .. pmc4 (means over their dispatches)."""
    passes = [_dispatches(os.path.join(out_dir, f"pmc{i + 1}"), lambda n: pattern in n) for i in range(len(PASSES))]
    mean = lambda ds, key: sum(d[key] for d in ds.values()) / len(ds)
    v = defaultdict(lambda: float("nan"))
    for ds in passes:
        for key in next(iter(ds.values())):
            if not key.startswith("_") and key not in v:
                v[key] = mean(ds, key)
    p1 = passes[0]
    any_d = next(iter(p1.values()))
    ns = sum(mean(ds, "_ns") for ds in passes) / len(passes)
    cyc = v["GRBM_GUI_ACTIVE"] / N_XCD
    flops = 512.0 * (v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + v.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0))
    wave_cyc = 4.0 * v["SQ_WAVE_CYCLES"]  # quad-cycles
    hits, miss = v["TCC_HIT_sum"], v["TCC_MISS_sum"]
    vg, ag, sg, scratch, wg, grid = any_d["_regs"]
    fam = next((f for f, (pats, _) in FAMILIES.items() if any(q in any_d["_name"] for q in pats)), "gemm")
    lines = [
        f"# rocprofv3 counters of {_short(any_d['_name'])}",
        f"source_hash = {source_hash(fam)}  ({fam} sources)",
        f"dispatches per pass = {[len(ds) for ds in passes]}",
        f"duration_us (counter runs) = {ns / 1e3:.2f}",
        f"registers: vgpr = {vg}, agpr = {ag}, sgpr = {sg}, scratch_bytes = {scratch}, "
        f"workgroup = {wg}, grid_threads = {grid}",
        "",
        "## clock and matrix cores",
        f"GRBM_GUI_ACTIVE per XCD = {cyc:.0f} cycles  -> shader clock {cyc / ns:.3f} GHz during the kernel",
        f"SQ_INSTS_MFMA = {v['SQ_INSTS_MFMA']:.0f}",
        f"MFMA flops (MOPS x 512) = {flops:.4g}",
        f"SQ_VALU_MFMA_BUSY_CYCLES = {v['SQ_VALU_MFMA_BUSY_CYCLES']:.0f}",
        f"MFMA busy = busy / (cycles x {N_SIMD} SIMDs) = {100 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_SIMD):.1f} %",
        f"MFMA flops / (cycles x 256 CUs x {FLOP_PER_CU_CLK}) = {100 * flops / (cyc * 256 * FLOP_PER_CU_CLK):.1f} %"
        f"  (of the peak at the measured clock)",
        f"MFMA flops / duration = {flops / ns / 1e3:.1f} TFLOP/s",
        f"CU busy = SQ_BUSY_CU_CYCLES / (cycles x 256) = {100 * v['SQ_BUSY_CU_CYCLES'] / (cyc * 256):.1f} %",
        "",
        "## LDS",
        f"SQ_INSTS_LDS = {v['SQ_INSTS_LDS']:.0f}",
        f"SQ_LDS_BANK_CONFLICT = {v['SQ_LDS_BANK_CONFLICT']:.0f} cycles"
        f"  ({100 * v['SQ_LDS_BANK_CONFLICT'] / v['SQ_LDS_IDX_ACTIVE']:.2f} % of SQ_LDS_IDX_ACTIVE)",
        f"SQ_LDS_ADDR_CONFLICT = {v['SQ_LDS_ADDR_CONFLICT']:.0f}, SQ_LDS_UNALIGNED_STALL = {v['SQ_LDS_UNALIGNED_STALL']:.0f}",
        f"SQ_LDS_IDX_ACTIVE = {v['SQ_LDS_IDX_ACTIVE']:.0f}  ({100 * v['SQ_LDS_IDX_ACTIVE'] / (cyc * 256):.1f} % of CU cycles)",
        f"SQ_LDS_CMD_FIFO_FULL = {v['SQ_LDS_CMD_FIFO_FULL']:.0f}  ({100 * v['SQ_LDS_CMD_FIFO_FULL'] / (cyc * 256):.1f} % of CU cycles)",
        f"SQ_WAIT_INST_LDS = {v['SQ_WAIT_INST_LDS']:.0f} quad-cycles ({100 * 4 * v['SQ_WAIT_INST_LDS'] / wave_cyc:.1f} % of wave time)",
        "",
        "## L2",
        f"TCC_HIT_sum = {hits:.0f}, TCC_MISS_sum = {miss:.0f}, hit rate = {100 * hits / (hits + miss):.1f} %",
        "",
        "## waves (fractions of SQ_WAVE_CYCLES, quad-cycles)",
        f"SQ_WAVES = {v['SQ_WAVES']:.0f}",
        f"waiting on anything (SQ_WAIT_ANY) = {100 * 4 * v['SQ_WAIT_ANY'] / wave_cyc:.1f} %",
        f"waiting for an issue slot (SQ_WAIT_INST_ANY) = {100 * 4 * v['SQ_WAIT_INST_ANY'] / wave_cyc:.1f} %",
        f"issuing (SQ_ACTIVE_INST_ANY) = {100 * 4 * v['SQ_ACTIVE_INST_ANY'] / wave_cyc:.1f} %",
        f"instructions per wave: VALU (incl. MFMA) {v['SQ_INSTS_VALU'] / v['SQ_WAVES']:.0f}, "
        f"MFMA {v['SQ_INSTS_MFMA'] / v['SQ_WAVES']:.0f}, SALU {v['SQ_INSTS_SALU'] / v['SQ_WAVES']:.0f}, "
        f"LDS {v['SQ_INSTS_LDS'] / v['SQ_WAVES']:.0f}, VMEM read {v['SQ_INSTS_VMEM_RD'] / v['SQ_WAVES']:.0f}, "
        f"VMEM write {v['SQ_INSTS_VMEM_WR'] / v['SQ_WAVES']:.0f}",
        "",
        "## copy path (TA: address unit, TD: data unit, TCP: L1; one of each per CU)",
        f"TA busy = {100 * v['TA_TA_BUSY_sum'] / (cyc * 256):.1f} % of CU cycles, "
        f"address path stalled by the cache {100 * v['TA_ADDR_STALLED_BY_TC_CYCLES_sum'] / (cyc * 256):.1f} %, "
        f"data path stalled {100 * v['TA_DATA_STALLED_BY_TC_CYCLES_sum'] / (cyc * 256):.1f} %",
        f"TA buffer cycles = {100 * v['TA_BUFFER_TOTAL_CYCLES_sum'] / (cyc * 256):.1f} % of CU cycles",
        f"TD busy = {100 * v['TD_TD_BUSY_sum'] / (cyc * 256):.1f} %, TD waiting for cache data "
        f"{100 * v['TD_TC_STALL_sum'] / (cyc * 256):.1f} %",
        f"L1->L2 read latency = {v['TCP_TCC_READ_REQ_LATENCY_sum'] / v['TCP_TCC_READ_REQ_sum']:.0f} cycles per request "
        f"({v['TCP_TCC_READ_REQ_sum']:.0f} requests)",
        f"L1 stalled on pending L2 data = {100 * v['TCP_PENDING_STALL_CYCLES_sum'] / (cyc * 256):.1f} %, "
        f"L1 request path stalled = {100 * v['TCP_TCR_TCP_STALL_CYCLES_sum'] / (cyc * 256):.1f} %",
    ]
    return "\n".join(lines)


def main(argv):
    if argv[0] == "stats":
        print(stats(argv[1], argv[2] if len(argv) > 2 else "gemm"))
    elif argv[0] == "traffic":
        print(traffic(argv[1], argv[2]))
    elif argv[0] == "counters":
        print(counters(argv[1], argv[2]))
    elif argv[0] == "passes":
        for ps in PASSES:
            print(ps)
    elif argv[0] == "hash":
        print(source_hash(argv[1] if len(argv) > 1 else "gemm"))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
