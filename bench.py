#!/usr/bin/env python3
"""Benchmark of the tiled GEMM/BMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = plan + launch of the whole product for one set of synthetic inputs
already resident in HBM (gemm_plan on the host, then gemm_run / bmm_run).
Before the W untimed warmup steps, the same step runs back to back for
--settle seconds (0.3 by default; reported as "clock_settle"): after an idle
GPU the first ~100 launches of a large product run 4-19% slower than the
steady state while the clocks and the power controller settle.  Then exactly
K timed steps between two device synchronisations.  Prints one JSON line.

Workloads (seeded synthetic inputs from synth/):
  square_8192   8192^3, NN, bf16 in, bf16 out        (default; MFMA-bound)
  square_8192_nt / _tn / _tt   the same product under the other op() layouts
  skinny_16     M=16, N=K=8192, B stored N x K, bf16 out  (HBM-bound)
  attention_s   128 x (2048x2048x128) S = Q K^T, fp32 out (HBM-bound)
  attention_o   128 x (2048x128x2048) O = P V,   fp32 out (HBM-bound)
  attn_fwd      128 x fused softmax(Q K^T / sqrt(128)) V, 2048 x 2048, d = 128,
                fp32 out (the same two products fused; MFMA-bound)
  group_moe     32 ragged expert GEMMs (8192 tokens, K = N = 1024, NN, bf16 out)
                in one grouped launch; also times one launch per problem
  splitk_long   1024 x 1024 x 65536 NN, bf16 out, K split into parts (gemm_splitk_run);
                also times the same product as one plain launch
  ragged_1000   1000^3 NN, fp32 out (ragged_1000_nt / _tn / _tt: the other layouts)
  square_256    256^3 NN, fp32 out

The "roofline" object rates the dominant kernel against MI355X's published
peak (dense bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s); its duration is the mean of
per-launch HIP events on the launch stream.  "cpu_baseline" times the CPU
oracle on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bf16 GEMM/BMM TFLOP/s and % of MFMA peak (GB/s and % HBM for skinny M)"
PEAK_MFMA = 2.5e15
PEAK_HBM = 8.0e12


def problems(name):
    import synth
    if name == "square_8192":
        return synth.square_8192()
    if name in ("square_8192_nt", "square_8192_tn", "square_8192_tt"):
        return synth.square_8192(layout=name[-2:])
    if name == "skinny_16":
        return synth.skinny_16()
    if name == "attention_s":
        return synth.attention_bmm()[:1]
    if name == "attention_o":
        return synth.attention_bmm()[1:]
    if name == "ragged_1000":
        return synth.ragged_1000()[:1]
    if name in ("ragged_1000_nt", "ragged_1000_tn", "ragged_1000_tt"):
        return [q for q in synth.ragged_1000() if q.name == name]
    if name == "square_256":
        return synth.square_256()
    raise SystemExit(f"unknown workload {name}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square_8192")
    ap.add_argument("--rotate", type=int, default=0,
                    help="copies of the larger operand to cycle through (defeats the 256 MiB Infinity "
                         "Cache); default 4 for HBM-bound workloads, 1 otherwise")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile", type=int, default=None, help="override the planner's tile (same variant)")
    ap.add_argument("--no-persist", action="store_true", help="clear the plan's persistent-launch flags")
    ap.add_argument("--no-prefetch", action="store_true", help="clear the plan's prefetch flag")
    ap.add_argument("--no-rotate-k", action="store_true", help="clear the plan's rotated-K-walk flag")
    ap.add_argument("--prefetch", action="store_true", help="set the plan's persistent and prefetch flags")
    ap.add_argument("--stream-c", type=int, default=-1, help="force the plan's non-temporal C flag (0/1)")
    ap.add_argument("--group-tile", type=int, default=-1, help="force the grouped launch's tile (group_moe)")
    ap.add_argument("--alpha", type=float, default=1.0, help="epilogue: C = alpha*AB + beta*C + bias")
    ap.add_argument("--beta", type=float, default=0.0, help="epilogue: scale of C's prior contents")
    ap.add_argument("--bias", action="store_true", help="epilogue: add a per-column bias")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of back-to-back steps before the warmup, while the clocks settle")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration measurements added to the default run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (to calibrate FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the design notes describe how the product would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    import matmul_tiled_bf16_amd as tg
    from matmul_tiled_bf16_amd import profiling, roofline

    if args.copy_calibration:
        src = torch.empty(profiling.COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": profiling.COPY_BYTES, "copies": 4}))
        return

    if args.workload == "attn_fwd":
        return run_attention(args, torch, tg, profiling)
    if args.workload == "group_moe":
        return run_group(args, torch, tg, profiling)
    if args.workload == "splitk_long":
        return run_splitk(args, torch, tg, profiling)

    (p,) = problems(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tin = torch.bfloat16 if p.in_dtype == "bf16" else torch.float16
    tout = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[p.out_dtype]
    out_size = {"fp32": 4, "bf16": 2, "fp16": 2}[p.out_dtype]

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(tin).to(dev)

    flops = roofline.gemm_flops(p.m, p.n, p.k, p.batch)
    nbytes = roofline.gemm_bytes(p.m, p.n, p.k, 2, out_size, p.batch)
    epi = args.alpha != 1.0 or args.beta != 0.0 or args.bias
    if args.beta != 0.0:
        nbytes += out_size * p.m * p.n * p.batch  # C is read as well as written
    if args.bias:
        nbytes += out_size * p.n
    bound = roofline.bound(p.m, p.n, p.k, 2, out_size, p.batch, PEAK_MFMA, PEAK_HBM)
    rotate = args.rotate or (4 if bound == "hbm" else 1)

    # the copies cycle through the operand that dominates the bytes (P of
    # O = P V is 16x its V), so that no launch finds it in the Infinity Cache
    big_a = p.A.size > p.B.size
    As = [up(p.A)] + ([up(p.A).clone() for _ in range(rotate - 1)] if big_a else [])
    Bs = [up(p.B)] + ([up(p.B).clone() for _ in range(rotate - 1)] if not big_a else [])
    Cs = [torch.empty((p.batch, p.m, p.n) if p.batch > 1 else (p.m, p.n), dtype=tout, device=dev)
          for _ in range(min(rotate, 2))]
    stream = torch.cuda.current_stream()
    bias = torch.randn(p.n, device=dev).to(tout) if args.bias else None
    if args.beta != 0.0:
        for C in Cs:
            C.copy_(torch.randn(C.shape, device=dev).to(tout))

    def step(i):
        pl = tg.plan(p.m, p.n, p.k, trans_a=p.trans_a, trans_b=p.trans_b, in_dtype=tin, out_dtype=tout,
                     lda=p.lda, ldb=p.ldb, ldc=p.ldc, batch=p.batch)
        if args.tile is not None:
            pl = tg.plan_tile(pl, pl.variant, args.tile)
        if args.no_persist:
            pl.flags &= ~(tg.FLAG_PERSIST | tg.FLAG_PREFETCH)
        if args.no_prefetch:
            pl.flags &= ~tg.FLAG_PREFETCH
        if args.no_rotate_k:
            pl.flags &= ~tg.FLAG_ROTATE_K
        if args.prefetch:
            pl.flags |= tg.FLAG_PERSIST | tg.FLAG_PREFETCH
        if args.stream_c == 0:
            pl.flags &= ~tg.FLAG_STREAM_C
        elif args.stream_c == 1:
            pl.flags |= tg.FLAG_STREAM_C
        A = As[i % len(As)]
        B = Bs[i % len(Bs)]
        C = Cs[i % len(Cs)]
        if epi:
            if p.batch == 1:
                tg.gemm_run_ex(pl, A, B, C, alpha=args.alpha, beta=args.beta, bias=bias, stream=stream)
            else:
                tg.bmm_run_ex(pl, p.batch, p.stride_a, p.stride_b, p.stride_c, A, B, C, alpha=args.alpha,
                              beta=args.beta, bias=bias, stream=stream)
        elif p.batch == 1:
            tg.gemm_run(pl, A, B, C, stream)
        else:
            tg.bmm_run(pl, p.batch, p.stride_a, p.stride_b, p.stride_c, A, B, C, stream)
        return pl

    settled = settle(torch, step, args.settle)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pl = step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    assert torch.isfinite(Cs[0].float()).all().item(), "non-finite output"

    # Kernel durations, measured live with HIP events on the launch stream: the
    # same launches, queued while the stream is held by a GPU-side sleep, so
    # that host time between launches (plan, marshalling) cannot show up
    # between the events.
    warm = held_warm(settled, args.warmup)
    mean_ms, kms, queued_ahead = gated_kernel_ms(torch, stream, step, args.steps, warm)
    kernel_s = mean_ms / 1e3

    tflops = flops / (ms_per_step / 1e3) / 1e12
    gbps = nbytes / (ms_per_step / 1e3) / 1e9
    if bound == "mfma":
        value, unit = tflops, "TFLOP/s"
        achieved, peak, runit = flops / kernel_s / 1e12, PEAK_MFMA / 1e12, "TFLOP/s"
    else:
        value, unit = gbps, "GB/s"
        achieved, peak, runit = nbytes / kernel_s / 1e9, PEAK_HBM / 1e9, "GB/s"

    trans = ("T" if p.trans_a else "N") + ("T" if p.trans_b else "N")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settled,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.in_dtype == "bf16" else "fp16",
        "data": "synthetic",
        "config": {"workload": p.name, "m": p.m, "n": p.n, "k": p.k, "batch": p.batch, "op": trans,
                   "in_dtype": p.in_dtype, "out_dtype": p.out_dtype, "a_copies": len(As), "b_copies": len(Bs),
                   "variant": int(pl.variant), "tile_index": int(pl.tile), "plan_flags": int(pl.flags),
                   **({"epilogue": {"alpha": args.alpha, "beta": args.beta, "bias": bool(args.bias)}} if epi else {})},
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * flops / (ms_per_step / 1e3) / PEAK_MFMA, 2),
        "gbps": round(gbps, 1),
        "pct_hbm_peak": round(100 * nbytes / (ms_per_step / 1e3) / PEAK_HBM, 2),
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
                     "frac": round(achieved / peak, 4), "traffic": profiling.read_traffic(p.name),
                     "traffic_source": profiling.traffic_note(p.name),
                     "kernel_ms": round(kernel_s * 1e3, 5),
                     "kernel_ms_each_min": round(float(np.min(kms)), 5),
                     "kernel_ms_each_p90": round(float(np.percentile(kms, 90)), 5),
                     "launches_queued_ahead": bool(queued_ahead),
                     "launches_warm_before_events": held_warm(settled, args.warmup),
                     "algorithmic": {"flops": flops, "bytes": nbytes}},
    }
    line["clock"] = clock_during(torch, stream, step, kernel_s)
    if args.workload == "square_8192" and not args.no_configs and not epi and args.tile is None:
        line["configs"] = run_configs(torch, tg, profiling)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p, unit, args.cpu_seconds)
        line["cpu_baseline"].update(cpu_context())
    print(json.dumps(line), flush=True)


def clock_during(torch, stream, step, kernel_s, seconds=3.0):
    """Shader clock and board power while the GPU runs about `seconds` of
    back-to-back launches of the timed step (the timed region itself is too
    short to sample; this window runs the same launches right after it).

    The GPU metrics table (amdsmi_get_gpu_metrics_info) refreshes only a
    few times a second, so every poll inside the window is not a new reading:
    only refreshes first seen after the clock settled (0.3 s in) and before
    the GPU went idle count, one sample per distinct firmware timestamp.
    Reports the clock of the first XCD and the spread over the eight XCDs.
    None of it if amdsmi is unavailable."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:  # no amdsmi library or no access to the device
        return {"error": f"amdsmi unavailable: {type(e).__name__}"}
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        h = handles[0]
        try:
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for c in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(c)
                if int(bdf.split(":")[1], 16) == bus:
                    h = c
                    break
        except Exception:
            pass
        cap = amdsmi.amdsmi_get_power_cap_info(h).get("power_cap")
        polls, stop = [], threading.Event()
        t00 = time.perf_counter()

        def num(v):
            return float(v) if isinstance(v, (int, float)) else None

        def poll():
            while not stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    xcds = [num(c) for c in (m.get("current_gfxclks") or [])]
                    xcds = [c for c in xcds if c is not None and c < 65535]
                    polls.append((time.perf_counter() - t00, m.get("firmware_timestamp"), num(m.get("current_gfxclk")),
                                  xcds, num(m.get("current_socket_power"))))
                except Exception:
                    pass
                stop.wait(0.02)

        n = max(16, int(seconds / max(kernel_s, 1e-6)))
        th = threading.Thread(target=poll, daemon=True)
        torch.cuda.synchronize()
        th.start()
        time.sleep(0.05)
        t_start = time.perf_counter() - t00
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        t_end = time.perf_counter() - t00
        stop.set()
        th.join()
        seen, body = set(), []
        for t, stamp, clk, xcds, pw in polls:
            key = stamp if stamp is not None else (clk, tuple(xcds), pw)
            if key in seen:
                continue
            seen.add(key)
            if t_start + 0.3 <= t <= t_end - 0.02 and clk is not None and pw is not None:
                body.append((clk, xcds, pw))
        if not body:
            return {"error": "no metrics refresh inside the launch window", "polls": len(polls)}
        clk = sorted(c for c, _, _ in body)
        pw = sorted(w for _, _, w in body)
        xall = sorted(x for _, xs, _ in body for x in xs)
        med = lambda v: v[len(v) // 2]
        return {"sclk_mhz_median": med(clk), "sclk_mhz_min": clk[0], "sclk_mhz_max": clk[-1],
                "sclk_mhz_xcd_min": xall[0] if xall else None, "sclk_mhz_xcd_max": xall[-1] if xall else None,
                "power_w_median": med(pw), "power_w_max": pw[-1],
                "power_cap_w": (cap / 1e6 if cap and cap > 1e5 else cap), "refreshes": len(body),
                "window": f"{n} back-to-back launches after the timed region, {t_end - t_start:.2f} s"}
    except Exception as e:
        return {"error": f"{type(e).__name__}: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def run_configs(torch, tg, profiling):
    """Every other configuration of the workload set, each on its own seeded
    inputs: kernel time per launch (HIP events around back-to-back launches
    queued while the stream is held), rate, and the fraction of the peak of
    its binding roofline.  HBM-bound products cycle through copies of B (or of
    their large operand) so that each launch reads from HBM, not from the
    256 MiB Infinity Cache."""
    import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    sets = [("square_256", synth.square_256(), 200), ("ragged_1000", synth.ragged_1000(), 200),
            ("skinny_16", synth.skinny_16(), 200), ("attention_bmm", synth.attention_bmm(), 20)]
    for _, probs, steps in sets:
        for p in probs:
            tin = torch.bfloat16 if p.in_dtype == "bf16" else torch.float16
            tout = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[p.out_dtype]
            osz = 4 if p.out_dtype == "fp32" else 2
            up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(tin).to(dev)
            flops = roofline_flops(p)
            nbytes = p.batch * ((p.m * p.k + p.k * p.n) * 2 + p.m * p.n * osz)
            bound = "mfma" if flops / nbytes >= PEAK_MFMA / PEAK_HBM else "hbm"
            # the operand that dominates the bytes is rotated for HBM-bound products
            big_a = p.A.size > p.B.size
            # small products are measured hot (their operands stay in the caches, as they
            # would between back-to-back calls); large HBM-bound ones from HBM
            small = p.name.startswith(("square_256", "ragged_1000"))
            # (S = Q K^T too: its 2 GiB output is stored non-temporally, so a single
            # copy of its 64 MiB operands could stay in the Infinity Cache)
            copies = 4 if bound == "hbm" and not small else 1
            A0, B0 = up(p.A), up(p.B)
            As = [A0] + [A0.clone() for _ in range(copies - 1)] if big_a else [A0]
            Bs = [B0] + [B0.clone() for _ in range(copies - 1)] if not big_a else [B0]
            C = torch.empty((p.batch, p.m, p.n) if p.batch > 1 else (p.m, p.n), dtype=tout, device=dev)
            pl = tg.plan(p.m, p.n, p.k, trans_a=p.trans_a, trans_b=p.trans_b, in_dtype=tin, out_dtype=tout,
                         lda=p.lda, ldb=p.ldb, ldc=p.ldc, batch=p.batch)

            def step(i, pl=pl, As=As, Bs=Bs, C=C, p=p):
                A, B = As[i % len(As)], Bs[i % len(Bs)]
                if p.batch == 1:
                    tg.gemm_run(pl, A, B, C, stream)
                else:
                    tg.bmm_run(pl, p.batch, p.stride_a, p.stride_b, p.stride_c, A, B, C, stream)

            settled = settle(torch, step, 0.05)
            mean_ms, kms, ahead = gated_kernel_ms(torch, stream, step, steps, held_warm(settled, 5))
            assert torch.isfinite(C.float()).all().item(), f"{p.name}: non-finite output"
            s = mean_ms / 1e3
            rate = flops / s / 1e12 if bound == "mfma" else nbytes / s / 1e9
            peak = PEAK_MFMA / 1e12 if bound == "mfma" else PEAK_HBM / 1e9
            out[p.name] = {
                "m": p.m, "n": p.n, "k": p.k, "batch": p.batch,
                "op": ("T" if p.trans_a else "N") + ("T" if p.trans_b else "N"),
                "out_dtype": p.out_dtype, "kernel_us": round(mean_ms * 1e3, 2),
                "kernel_us_each_min": round(float(np.min(kms)) * 1e3, 2),
                "tflops": round(flops / s / 1e12, 2), "gbps": round(nbytes / s / 1e9, 1),
                "bound": bound, "frac": round(rate / peak, 4),
                "operand_copies": copies, "hot_cache": small, "launches": steps, "queued_ahead": bool(ahead),
                "tile_index": int(pl.tile), "variant": int(pl.variant),
                "traffic": profiling.read_traffic(p.name), "traffic_source": profiling.traffic_note(p.name),
                "algorithmic": {"flops": flops, "bytes": nbytes}}
            del As, Bs, C, A0, B0
            torch.cuda.empty_cache()
    return out


def roofline_flops(p):
    return 2 * p.m * p.n * p.k * p.batch


def cpu_context():
    """The host CPU model, and the oracle on the full 256^3 product on one
    thread (a child process, so that the thread count is its own)."""
    import subprocess
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    code = ("import time, synth, oracle\n"
            "(p,) = synth.square_256()\n"
            "oracle.gemm_problem(p)\n"
            "t0 = time.perf_counter(); oracle.gemm_problem(p); t = time.perf_counter() - t0\n"
            "print(2 * 256 ** 3 / t / 1e9)\n")
    single = None
    try:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=120)
        single = round(float(r.stdout.strip().splitlines()[-1]), 3)
    except Exception:
        pass
    return {"cpu_model": model, "single_thread_square_256_gflops": single}


def run_attention(args, torch, tg, profiling):
    """The fused attention forward pass: one step = one attention_fwd launch
    over all heads.  Flops are the two products' 4 * batch * n_q * n_k * d
    (the softmax's exponentials are not counted); algorithmic bytes are Q, K,
    V read once and O written once."""
    import synth
    p = synth.attention_fwd()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tout = {"fp32": torch.float32, "bf16": torch.bfloat16}[p.out_dtype]
    out_size = 4 if p.out_dtype == "fp32" else 2

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    Q, K, V = up(p.Q), up(p.K), up(p.V)
    Os = [torch.empty((p.batch, p.n_q, p.d), dtype=tout, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream()
    flops = p.flops
    nbytes = p.batch * (2 * p.n_q * p.d + 2 * 2 * p.n_k * p.d + out_size * p.n_q * p.d)
    d = p.d

    def step(i):
        O = Os[i % 2]
        tg.attention_fwd(tg.TG_BF16, tg.TG_FP32 if out_size == 4 else tg.TG_BF16, p.batch, p.n_q, p.n_k, d,
                         p.scale, Q, d, p.n_q * d, K, d, p.n_k * d, V, d, p.n_k * d, O, d, p.n_q * d, stream)

    settled = settle(torch, step, args.settle)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    assert torch.isfinite(Os[0].float()).all().item(), "non-finite output"
    mean_ms, kms, queued_ahead = gated_kernel_ms(torch, stream, step, args.steps, held_warm(settled, args.warmup))
    kernel_s = mean_ms / 1e3
    tflops = flops / (ms_per_step / 1e3) / 1e12
    achieved = flops / kernel_s / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settled,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "batch": p.batch, "n_q": p.n_q, "n_k": p.n_k, "head_dim": p.d,
                   "scale": p.scale, "in_dtype": "bf16", "out_dtype": p.out_dtype, "fused": True},
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * flops / (ms_per_step / 1e3) / PEAK_MFMA, 2),
        "gbps": round(nbytes / (ms_per_step / 1e3) / 1e9, 1),
        "pct_hbm_peak": round(100 * nbytes / (ms_per_step / 1e3) / PEAK_HBM, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_MFMA, 4),
                     "traffic": profiling.read_traffic(p.name),
                     "traffic_source": profiling.traffic_note(p.name),
                     "kernel_ms": round(kernel_s * 1e3, 5),
                     "kernel_ms_each_min": round(float(np.min(kms)), 5),
                     "kernel_ms_each_p90": round(float(np.percentile(kms, 90)), 5),
                     "launches_queued_ahead": bool(queued_ahead),
                     "launches_warm_before_events": held_warm(settled, args.warmup),
                     "algorithmic": {"flops": flops, "bytes": nbytes}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_attention(p, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def run_group(args, torch, tg, profiling):
    """Grouped launch: one step = one gemm_group_run over every expert's
    product.  Algorithmic bytes are the tokens and the weights read once and
    the outputs written once; the group is HBM-bound when their ratio to the
    flops is below MI355X's ridge.  The same products launched one by one
    (gemm_plan + gemm_run each) are timed the same way for comparison."""
    import ctypes
    import synth
    p = synth.grouped_moe()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    X, W = up(p.X), up(p.W)
    T = int(p.counts.sum())
    Ys = [torch.empty((T, p.n), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    off = p.offsets
    es = 2
    tables = []
    for Y in Ys:
        arr = (tg.GroupProblem * len(p.counts))()
        for e, c in enumerate(p.counts):
            arr[e] = tg.GroupProblem(int(c), p.n, p.k, p.k, p.n, p.n, X.data_ptr() + es * int(off[e]) * p.k,
                                     W[e].data_ptr(), Y.data_ptr() + es * int(off[e]) * p.n)
        tables.append(arr)
    L = tg.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    count = len(p.counts)

    def step(i):
        st = L.gemm_group_run(tg.TG_BF16, tg.TG_BF16, 0, 0, tables[i % 2], count, args.group_tile, sh)
        if st != tg.TG_OK:
            raise tg.TgError(st, "gemm_group_run")

    def step_separate(i):
        Y = Ys[i % 2]
        for e, c in enumerate(p.counts):
            if c == 0:
                continue
            pl = tg.plan(int(c), p.n, p.k, in_dtype=torch.bfloat16, out_dtype=torch.bfloat16)
            tg.gemm_run(pl, X[int(off[e]):int(off[e + 1])], W[e], Y[int(off[e]):int(off[e + 1])], stream)

    settled = settle(torch, step, args.settle)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    assert torch.isfinite(Ys[0].float()).all().item(), "non-finite output"
    mean_ms, kms, queued_ahead = gated_kernel_ms(torch, stream, step, args.steps, held_warm(settled, args.warmup))
    sep_ms, _, sep_ahead = gated_kernel_ms(torch, stream, step_separate, max(args.steps // 4, 3),
                                           held_warm(settle(torch, step_separate, 0.05), 2, cap=25))
    flops = p.flops
    nbytes = p.algorithmic_bytes(es)
    bound = "mfma" if flops / nbytes > PEAK_MFMA / PEAK_HBM else "hbm"
    kernel_s = mean_ms / 1e3
    if bound == "mfma":
        achieved, peak, runit = flops / kernel_s / 1e12, PEAK_MFMA / 1e12, "TFLOP/s"
    else:
        achieved, peak, runit = nbytes / kernel_s / 1e9, PEAK_HBM / 1e9, "GB/s"
    tflops = flops / (ms_per_step / 1e3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settled,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "problems": count, "tokens": T, "n": p.n, "k": p.k, "op": "NN",
                   "group_tile": args.group_tile,
                   "in_dtype": "bf16", "out_dtype": p.out_dtype, "empty_problems": int((p.counts == 0).sum()),
                   "max_m": int(p.counts.max()), "min_m": int(p.counts.min())},
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * flops / (ms_per_step / 1e3) / PEAK_MFMA, 2),
        "gbps": round(nbytes / (ms_per_step / 1e3) / 1e9, 1),
        "pct_hbm_peak": round(100 * nbytes / (ms_per_step / 1e3) / PEAK_HBM, 2),
        "separate_launches": {"kernel_ms": round(sep_ms, 5), "launches": int((p.counts > 0).sum()),
                              "queued_ahead": bool(sep_ahead),
                              "grouped_speedup": round(sep_ms / mean_ms, 3)},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
                     "frac": round(achieved / peak, 4), "traffic": profiling.read_traffic(p.name),
                     "traffic_source": profiling.traffic_note(p.name),
                     "kernel_ms": round(kernel_s * 1e3, 5),
                     "kernel_ms_each_min": round(float(np.min(kms)), 5),
                     "kernel_ms_each_p90": round(float(np.percentile(kms, 90)), 5),
                     "launches_queued_ahead": bool(queued_ahead),
                     "launches_warm_before_events": held_warm(settled, args.warmup),
                     "algorithmic": {"flops": flops, "bytes": nbytes}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_group(p, "TFLOP/s", args.cpu_seconds)
    print(json.dumps(line), flush=True)


def run_splitk(args, torch, tg, profiling):
    """Split-K: one step = one gemm_splitk_run (a grouped launch of the K parts
    into an fp32 workspace, then the reduction) at the suggested split count.
    The product is MFMA-bound (arithmetic intensity above the ridge), but its
    64 output tiles leave most of the 256 CUs idle as one plain launch, which
    is timed the same way for comparison.  The roofline's duration is the
    step's (both kernels)."""
    import synth
    (p,) = synth.long_k()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    A, B = up(p.A), up(p.B)
    Cs = [torch.empty((p.m, p.n), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    pl = tg.plan(p.m, p.n, p.k, in_dtype=torch.bfloat16, out_dtype=torch.bfloat16)
    splits = tg.splitk_choose(pl)
    need = tg.splitk_workspace_bytes(pl, splits)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        tg.gemm_splitk_run(pl, splits, ws, need, A, B, Cs[i % 2], stream)

    def step_plain(i):
        tg.gemm_run(pl, A, B, Cs[i % 2], stream)

    settled = settle(torch, step, args.settle)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    assert torch.isfinite(Cs[0].float()).all().item(), "non-finite output"
    mean_ms, kms, queued_ahead = gated_kernel_ms(torch, stream, step, args.steps, held_warm(settled, args.warmup))
    plain_ms, _, plain_ahead = gated_kernel_ms(torch, stream, step_plain, max(args.steps // 2, 3),
                                               held_warm(settle(torch, step_plain, 0.05), 2))
    flops = p.flops
    nbytes = 2 * (p.m * p.k + p.k * p.n) + 2 * p.m * p.n
    kernel_s = mean_ms / 1e3
    achieved = flops / kernel_s / 1e12
    tflops = flops / (ms_per_step / 1e3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settled,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "m": p.m, "n": p.n, "k": p.k, "op": "NN", "in_dtype": "bf16",
                   "out_dtype": "bf16", "splits": splits, "workspace_bytes": need},
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(100 * flops / (ms_per_step / 1e3) / PEAK_MFMA, 2),
        "gbps": round(nbytes / (ms_per_step / 1e3) / 1e9, 1),
        "pct_hbm_peak": round(100 * nbytes / (ms_per_step / 1e3) / PEAK_HBM, 2),
        "plain_launch": {"kernel_ms": round(plain_ms, 5), "tile_index": int(pl.tile),
                         "queued_ahead": bool(plain_ahead), "splitk_speedup": round(plain_ms / mean_ms, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved * 1e12 / PEAK_MFMA, 4), "traffic": None,
                     "kernel_ms": round(kernel_s * 1e3, 5),
                     "kernel_ms_each_min": round(float(np.min(kms)), 5),
                     "kernel_ms_each_p90": round(float(np.percentile(kms, 90)), 5),
                     "launches_queued_ahead": bool(queued_ahead),
                     "launches_warm_before_events": held_warm(settled, args.warmup),
                     "algorithmic": {"flops": flops, "bytes": nbytes}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p, "TFLOP/s", args.cpu_seconds)
    print(json.dumps(line), flush=True)


def cpu_baseline_group(p, unit, seconds):
    """Time the CPU oracle on seeded output elements spread over all experts."""
    import oracle
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    off = p.offsets
    T = int(off[-1])

    def run(count, seed):
        tri = synth.sample_indices(seed, 1, T, p.n, count=count, edges=())
        e_of = np.searchsorted(off, tri[:, 1], side="right") - 1
        t0 = time.perf_counter()
        for e in np.unique(e_of):
            sel = tri[e_of == e].copy()
            sel[:, 1] -= off[e]
            rows = p.X[int(off[e]):int(off[e + 1])]
            oracle.gemm(rows, p.W[e], m=int(p.counts[e]), n=p.n, k=p.k, idx=sel)
        return time.perf_counter() - t0, len(tri)

    count, dt = 4096, 0.0
    while True:
        dt, _ = run(count, 77)
        if dt >= 0.5 or count >= 50_000_000:
            break
        count = min(50_000_000, count * 8)
    count = int(max(256, min(50_000_000, count * seconds / max(dt, 1e-4))))
    t, got = run(count, 78)
    flops = 2.0 * p.k * got
    return {"value": round(flops / t / 1e12, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{got} seeded output elements spread over the experts (each a {p.k}-term fp64 dot "
                      f"product), {t:.1f} s on {threads} threads; all {T * p.n} would take "
                      f"{t * T * p.n / got:.0f} s"}


def cpu_baseline_attention(p, seconds):
    """Time the CPU oracle on seeded query rows of the attention workload."""
    import oracle
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    kw = dict(n_q=p.n_q, n_k=p.n_k, head_dim=p.d, scale=p.scale, batch=p.batch)
    count, dt = 8, 0.0
    while True:
        rows = synth.attention_rows(77, p.batch, p.n_q, count=count, edges=())
        t0 = time.perf_counter()
        oracle.attention(p.Q, p.K, p.V, rows=rows, **kw)
        dt = max(time.perf_counter() - t0, 1e-4)
        if dt >= 0.5 or count >= p.batch * p.n_q:
            break
        count = min(p.batch * p.n_q, count * 8)
    count = int(max(8, min(p.batch * p.n_q, count * seconds / dt)))
    rows = synth.attention_rows(78, p.batch, p.n_q, count=count, edges=())
    t0 = time.perf_counter()
    oracle.attention(p.Q, p.K, p.V, rows=rows, **kw)
    t = time.perf_counter() - t0
    flops = 4.0 * p.n_k * p.d * len(rows)
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} seeded query rows of the same workload (each {p.n_k} fp64 scores of "
                      f"{p.d} terms, softmax, and a {p.n_k}-term weighted sum per output), {t:.1f} s on "
                      f"{threads} threads; all {p.batch * p.n_q} rows would take "
                      f"{t * p.batch * p.n_q / len(rows):.0f} s"}


def settle(torch, step, seconds):
    """Run the step back to back for about `seconds` (in batches that double,
    one device synchronisation after each) and return what ran: after an
    idle GPU the first ~100 launches of a large product are 4-19% slower than
    the steady state (8192^3: ~860 us in launches 10-20 against ~766 from the
    100th; O = P V: ~277 against ~233), while the clocks and the power
    controller adjust.  The timed steps come after this and the warmup."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n, batch, el = 0, 1, 0.0
    while el < seconds:
        for _ in range(batch):
            step(n)
            n += 1
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        batch = min(2 * batch, 4096)
    return {"launches": n, "seconds": round(el, 4), "ms_per_launch": round(el * 1e3 / n, 5) if n else None}


def held_warm(settled, warmup, seconds=0.1, cap=1000):
    """Untimed steps queued ahead of the event-timed ones behind the GPU
    sleep (the sleep lets the clocks drop again): about `seconds` of them,
    at least the warmup count and 1, at most `cap` (the stream's queue holds
    a bounded number of launches; past it the host waits for the GPU and the
    queue no longer stays ahead)."""
    per = settled.get("ms_per_launch") if settled else None
    need = int(seconds * 1e3 / per) + 1 if per else 1
    return max(warmup, 1, min(need, cap))


def _held(torch, stream, enqueue):
    """Run enqueue() while the stream is held by a GPU-side sleep, so that the
    host finishes queueing before the GPU starts; retried with a longer sleep
    if the sleep ran out first.  Returns whether the queue stayed ahead."""
    woke = torch.cuda.Event()
    cycles = 20_000_000
    for _attempt in range(4):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(cycles)
        woke.record(stream)
        enqueue()
        ahead = not woke.query()
        torch.cuda.synchronize()
        if ahead:
            return True
        cycles *= 4
    return False


def gated_kernel_ms(torch, stream, step, n, warm):
    """Kernel durations with host overhead kept out of the GPU timeline.

    Returns (mean ms per launch from one event pair around n back-to-back
    launches, per-launch ms from an event pair around each launch, whether
    the queue stayed ahead of the GPU in both passes).  The first figure is
    the kernel's own time (plus the sub-microsecond launch-to-launch gap);
    per-launch event pairs add a few microseconds of their own to each
    launch, so they serve only for the spread (min, p90)."""
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def batch():
        for i in range(warm):  # clocks ramp back up after the sleep
            step(i)
        t0.record(stream)
        for i in range(n):
            step(i)
        t1.record(stream)

    ahead_b = _held(torch, stream, batch)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def each():
        for i in range(warm):
            step(i)
        for i in range(n):
            starts[i].record(stream)
            step(i)
            ends[i].record(stream)

    ahead_e = _held(torch, stream, each)
    return t0.elapsed_time(t1) / n, [s.elapsed_time(e) for s, e in zip(starts, ends)], ahead_b and ahead_e


def cpu_baseline(p, unit, seconds):
    """Time the CPU oracle on a seeded sample of output elements (~`seconds` of work)."""
    import oracle
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # size the sample from timed trial runs that grow until they take long
    # enough to be measured without thread start-up dominating
    count, dt = 4096, 0.0
    while True:
        calib = synth.sample_indices(77, p.batch, p.m, p.n, count=count, edges=())
        t0 = time.perf_counter()
        oracle.gemm_problem(p, idx=calib)
        dt = max(time.perf_counter() - t0, 1e-4)
        if dt >= 0.5 or count >= 50_000_000:
            break
        count = min(50_000_000, count * 8)
    count = int(max(256, min(50_000_000, count * seconds / dt)))
    idx = synth.sample_indices(78, p.batch, p.m, p.n, count=count, edges=())
    t0 = time.perf_counter()
    oracle.gemm_problem(p, idx=idx)
    t = time.perf_counter() - t0
    flops = 2.0 * p.k * len(idx)
    # the same work rate expressed in the workload's unit
    if unit == "TFLOP/s":
        v = flops / t / 1e12
    else:
        total_flops = 2.0 * p.m * p.n * p.k * p.batch
        total_bytes = p.batch * ((p.m * p.k + p.k * p.n) * 2 + p.m * p.n * (4 if p.out_dtype == "fp32" else 2))
        v = (flops / t) / total_flops * total_bytes / 1e9
    return {"value": round(v, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{len(idx)} seeded output elements of the same workload (each a {p.k}-term fp64 dot "
                      f"product), {t:.1f} s on {threads} threads; full problem would take "
                      f"{t * p.m * p.n * p.batch / len(idx):.0f} s"}


if __name__ == "__main__":
    main()
