"""Benchmark of the CubicQuant dequant-GEMM hot path on one MI355X.

Default workload (one "step"): the Kimi-K3-shaped routed-expert decode at M = 1,
W2 G512: the fused gate_up product (6144 x 7168) then the down product
(7168 x 3072), A16 (bf16 activations, fp32 out). Each step reads a different
copy of the two weights from a rotation pool larger than twice the Infinity
Cache plus L2, so every launch streams its weights from HBM.

Prints ONE JSON line: metric/value (whole-step HBM GB/s of algorithmic bytes),
roofline of the dominant kernel (gate_up launch; average duration from HIP
events on the launch stream around graph replays of gate_up launches), the
M = 4096 half of the metric (prefill_a16: TFLOP/s against the bf16 MFMA peak;
prefill_a8: TOP/s against the int8 peak), the 16-expert decode step of one layer
(decode_step_16x, HBM GB/s), and the oracle CPU baseline on a bounded sample.
`--extra` adds, as extra fields (each also reported on stderr as it finishes):
the small-M W4 products, nearest-level encoding, data-free group fitting, the
routed-expert products and the whole routed-expert MLP step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16/bf16 MFMA, published
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published


def algorithmic_bytes(N, K, bits, group, M, a8=False):
    w = N * K * bits // 8 + 8 * N * (K // group)
    x = M * K * (1 if a8 else 2) + (4 * M if a8 else 0)
    y = 4 * M * N
    return w + x + y


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=50, help="rotating weight copies (at least 50)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--extra", action="store_true", help="also time prefill and small-M products")
    ap.add_argument("--crossover", type=int, default=0, metavar="REPS",
                    help="only time A16 against A8 over M, widths and the two expert shapes")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 20 plain device copies of MIB MiB (HBM counter calibration)")
    ap.add_argument("--counter-run", choices=("gate_up", "down", "prefill_a16", "prefill_a8", "decode_step",
                                              "decode_step_a8", "skinny_w4_m64"), default=None,
                    help="only launch this product --steps times, eagerly (the GEMVs on rotating "
                         "copies; for rocprofv3 --pmc passes)")
    ap.add_argument("--leg", choices=("prefill", "decode_step", "moe", "smallm"), default=None,
                    help="only run one workload block (prefill A16/A8, the 16-expert decode step, the "
                         "routed-expert legs of --extra, or the small-batch legs) and print it; for "
                         "profiler runs")
    ap.add_argument("--floors", action="store_true",
                    help="only time the floor kernels (empty launch, load-only streams of the gate_up "
                         "codes, dependent-load chase) and print them")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="only write --traffic-json from rocprofv3 --pmc outputs under DIR "
                         "(pmc_<COUNTER>_<gate_up|down|copy>/*counter_collection.csv); no GPU")
    return ap.parse_args()


# Sources of the GEMV kernel the roofline line describes; the stored HBM traffic
# figure is only reported while their hash matches the one it was measured on.
# The hash covers the code only: comments and blank lines are left out.
GEMV_SOURCES = ("common.h", "decode.h", "gemv_core.h", "rows.h", "launch.h", "gemv.hip", "gemv_rows.hip")


def _code_only(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (ln.split("//", 1)[0].rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def gemv_source_hash():
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, "dequant_gemm_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(path):
    """HBM bytes per gate_up launch from the committed rocprofv3 counter runs,
    or None when absent or measured on other kernel sources."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("gemv_source_hash") != gemv_source_hash():
        return None
    return t.get("decode_gate_up_bytes_per_launch")


def _pmc_means(path, match):
    """Mean Counter_Value per dispatch of the kernels whose name contains `match`,
    from one rocprofv3 --pmc run (one counter) under `path`."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    vals = []
    for f in files:
        with open(f, newline="") as fh:
            vals += [float(r["Counter_Value"]) for r in csv.DictReader(fh) if match in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no dispatch of {match!r} under {path}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(src, out, copy_mib=256):
    """HBM bytes per gate_up / down launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the product kernel, each scaled by what the same counter reads
    for a plain device copy of copy_mib MiB (which reads and writes exactly
    that many bytes)."""
    nbytes = copy_mib * (1 << 20)
    cf, _ = _pmc_means(os.path.join(src, "pmc_FETCH_SIZE_copy"), "copyBuffer")
    cw, _ = _pmc_means(os.path.join(src, "pmc_WRITE_SIZE_copy"), "copyBuffer")
    ff, fw = nbytes / 1024.0 / cf, nbytes / 1024.0 / cw
    res = {"gemv_source_hash": gemv_source_hash(),
           "copy_calibration": {"bytes_read_and_written": nbytes, "FETCH_SIZE_KiB": cf,
                                "WRITE_SIZE_KiB": cw, "fetch_factor": round(ff, 6),
                                "write_factor": round(fw, 6)},
           "raw_KiB_per_dispatch": {}}
    n = None
    for k in ("gate_up", "down"):
        f, n = _pmc_means(os.path.join(src, f"pmc_FETCH_SIZE_{k}"), "k_gemv")
        w, _ = _pmc_means(os.path.join(src, f"pmc_WRITE_SIZE_{k}"), "k_gemv")
        res["raw_KiB_per_dispatch"][k] = {"FETCH_SIZE": f, "WRITE_SIZE": w}
        res[f"decode_{k}_bytes_per_launch"] = int(round((f * ff + w * fw) * 1024.0))
    res["dispatches_averaged"] = n
    res["commands"] = [
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_FETCH_SIZE_gate_up -o run -- "
        "python3 bench.py --counter-run gate_up --steps 60 --no-cpu-baseline",
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_WRITE_SIZE_gate_up -o run -- "
        "python3 bench.py --counter-run gate_up --steps 60 --no-cpu-baseline",
        "(the same two with --counter-run down, into pmc_*_down)",
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_FETCH_SIZE_copy -o run -- "
        "python3 bench.py --calibrate-copy 256",
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_WRITE_SIZE_copy -o run -- "
        "python3 bench.py --calibrate-copy 256",
        "python3 bench.py --write-traffic <dir>",
    ]
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps({"traffic_json": out, "gate_up": res["decode_gate_up_bytes_per_launch"],
                      "down": res["decode_down_bytes_per_launch"]}))


def calibrate_copy(mib):
    """A plain copy kernel of known size: each launch reads and writes exactly
    mib MiB, so FETCH_SIZE / WRITE_SIZE per dispatch give the counters' scale."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 20}), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds: float):
    """The oracle (numpy float64) on a sample of the decode workload: gate_up rows
    0..511 (all K), unpack + dequant + GEMV, repeated for ~seconds, with the BLAS
    allowed every core this process may run on. The unpack and dequant steps are
    numpy element-wise code on one thread; only the GEMV goes through BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    g = synth.make_generator(2)
    w = synth.make_weight(g, 512, 7168, 2, 512, "ternary", 0.015)
    x = synth.activations(g, 1, 7168)
    codes = w.codes.numpy()
    scales = w.scales.numpy()
    shapes = w.shapes.numpy().view(np.uint16)
    xb = x.view(__import__("torch").int16).numpy().view(np.uint16)
    packed = oracle.pack(codes, 2)
    nbytes = algorithmic_bytes(512, 7168, 2, 512, 1)
    reps = 0
    with threadpool_limits(limits=cores, user_api="blas"):
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        t0 = time.perf_counter()
        while True:
            c = oracle.unpack(packed, 512, 7168, 2)
            W = oracle.dequant(c, scales, shapes, 2, 512)
            oracle.gemm_a16(xb, W)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    vendor = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                       for i in blas) or "unknown"
    return {"value": round(reps * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu": _cpu_model(), "blas": vendor,
            "sample": f"decode gate_up rows 0..511 x K=7168 (W2 G512, M=1): unpack+dequant+GEMV, "
                      f"{reps} reps in {dt:.1f} s; BLAS on {cores} threads, unpack and dequant single-threaded numpy"}


def crossover(steps):
    """A16 against Dynamic A8 on the routed-expert shapes: gate_up 6144 x 7168 and
    down 7168 x 3072, 2-bit (G512), 5- and 8-bit (G128) codes, M in {1, 16, 64,
    256}. A8 is timed as the quantiser plus the product. Each product rotates
    over enough weight copies (at least 640 MB) that every launch reads its
    weight from HBM; graph replays, HIP events on the replay stream."""
    import torch

    import dequant_gemm_amd as cq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = []
    for name, N, K in (("gate_up", 6144, 7168), ("down", 7168, 3072)):
        for bits, group in ((2, 512), (5, 128), (8, 128)):
            g = synth.make_generator(7000 + 10 * bits + (N > K), dev)
            w = synth.make_weight(g, N, K, bits, group, "ternary" if bits == 2 else "uniform", 0.02, dev)
            base = cq.CubicWeight(cq.cubic_pack(w.codes, bits).reshape(-1), w.scales.contiguous(),
                                  w.shapes.contiguous(), N, K, bits, group)
            del w
            nb = algorithmic_bytes(N, K, bits, group, 0)
            copies = max(4, -(-640_000_000 // nb))
            pool = [base] + [cq.CubicWeight(base.codes.clone(), base.scales.clone(), base.shapes.clone(),
                                            N, K, bits, group) for _ in range(copies - 1)]
            for M in (1, 16, 64, 256):
                x = synth.activations(g, M, K, device=dev)
                y = torch.empty((M, N), dtype=torch.float32, device=dev)
                ws = torch.empty(max(1, cq.cubic_gemm_a16_workspace_bytes(M, K)), dtype=torch.uint8,
                                 device=dev)
                xq = torch.empty((M, K), dtype=torch.int8, device=dev)
                sx = torch.empty((M,), dtype=torch.float32, device=dev)
                t16 = _graph_time([(lambda c=c: cq.cubic_gemm_a16(x, c, out=y, workspace=ws)) for c in pool],
                                  steps, dev)
                tq = _graph_time([lambda: cq.act_quant_int8_per_token(x, xq, sx)] * 8, steps, dev)
                t8 = _graph_time([(lambda c=c: cq.cubic_gemm_a8(xq, sx, c, out=y)) for c in pool], steps, dev)
                rows.append({"shape": name, "bits": bits, "group": group, "M": M,
                             "a16_us": round(t16 * 1e3, 2), "a8_us": round((tq + t8) * 1e3, 2),
                             "a8_quant_us": round(tq * 1e3, 2), "a8_gemm_us": round(t8 * 1e3, 2),
                             "faster": "a16" if t16 <= tq + t8 else "a8", "copies": copies})
                print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
            del pool, base
            torch.cuda.empty_cache()
    print(json.dumps({"crossover": rows}), flush=True)


def _rotation_graphs(launch, R, c, dev):
    """HIP graphs G_0 .. G_{R/c - 1}: G_k replays steps k*c .. k*c + c - 1 of a
    rotation over R weight copies (`launch(i)` enqueues step i on copy i % R).
    Replaying them in order walks the whole pool, so every launch reads weights
    that no launch of the last R - 1 steps touched."""
    import torch
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        for i in range(R):
            launch(i)
    torch.cuda.synchronize()
    graphs = []
    for k in range(R // c):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for i in range(k * c, k * c + c):
                launch(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def _replay_ms(graphs, first, n, stream):
    """Time n graph replays (graphs[first], graphs[first + 1], ... cyclically)
    with HIP events on the replay stream; returns (ms, next index)."""
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    k = first
    for _ in range(n):
        graphs[k].replay()
        k = (k + 1) % len(graphs)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), k


def _chunk(steps, R):
    """Steps per graph: the largest c <= 10 that divides both the step count and R."""
    for c in range(10, 0, -1):
        if steps % c == 0 and R % c == 0:
            return c
    return 1


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only (one process, one device); "
                                   "--gpus must be 1"}))
        sys.exit(2)
    if args.write_traffic:
        write_traffic(args.write_traffic, args.traffic_json)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.crossover:
        crossover(args.crossover)
        return
    import torch

    import dequant_gemm_amd as cq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.floors:
        floors(dev)
        return
    if args.counter_run and args.counter_run not in ("gate_up", "down"):
        counter_run_other(cq, synth, dev, args.counter_run, args.steps)
        return
    if args.leg:
        stream = torch.cuda.current_stream(dev)
        if args.leg == "prefill":
            res = prefill_blocks(cq, synth, dev, stream)
        elif args.leg == "decode_step":
            res = {"decode_step_16x": decode_step_block(cq, synth, dev)}
        elif args.leg == "moe":
            res = moe_workloads(cq, synth, dev)
        else:
            res = smallm_workloads(cq, synth, dev)
        print(json.dumps({"leg": args.leg, **res}), flush=True)
        return
    (w_up, x_up), (w_dn, x_dn) = synth.decode_config(seed=2, device=dev)

    def to_cw(w):
        packed = cq.cubic_pack(w.codes, w.bits).reshape(-1)
        return cq.CubicWeight(packed, w.scales.contiguous(), w.shapes.contiguous(), w.N, w.K,
                              w.bits, w.group)

    base_up, base_dn = to_cw(w_up), to_cw(w_dn)
    del w_up.codes, w_dn.codes

    def clone(cw):
        return cq.CubicWeight(cw.codes.clone(), cw.scales.clone(), cw.shapes.clone(), cw.N, cw.K,
                              cw.bits, cw.group)

    R = max(50, args.copies)
    ups = [base_up] + [clone(base_up) for _ in range(R - 1)]
    dns = [base_dn] + [clone(base_dn) for _ in range(R - 1)]
    y_up = torch.empty((1, 6144), dtype=torch.float32, device=dev)
    y_dn = torch.empty((1, 7168), dtype=torch.float32, device=dev)
    if args.counter_run:
        pool, xx, yy = (ups, x_up, y_up) if args.counter_run == "gate_up" else (dns, x_dn, y_dn)
        for i in range(args.steps):
            cq.cubic_gemm_a16(xx, pool[i % R], out=yy)
        torch.cuda.synchronize()
        print(json.dumps({"counter_run": args.counter_run, "launches": args.steps}), flush=True)
        return
    bytes_up = algorithmic_bytes(6144, 7168, 2, 512, 1)
    bytes_dn = algorithmic_bytes(7168, 3072, 2, 512, 1)

    # One step = the gate_up product on copy i % R, then the down product on copy
    # (i + R / 2) % R. The launches are captured into HIP graphs of c steps that
    # together walk the whole pool (R copies, 880 MB at R = 50: over three times
    # the 256 MB Infinity Cache), so the timed region measures the GPU, not
    # Python's per-call cost, and every launch streams its weights from HBM
    # whatever the step count.
    def step(i):
        cq.cubic_gemm_a16(x_up, ups[i % R], out=y_up)
        cq.cubic_gemm_a16(x_dn, dns[(i + R // 2) % R], out=y_dn)

    def up_only(i):
        cq.cubic_gemm_a16(x_up, ups[i % R], out=y_up)

    c = _chunk(args.steps, R)
    g_step = _rotation_graphs(step, R, c, dev)
    g_up = _rotation_graphs(up_only, R, c, dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):                                    # W warmup steps, eager
        step(i)
    k_step = (-(-args.warmup // c)) % len(g_step)                   # the pool continues after them
    ms, _ = _replay_ms(g_step, k_step, args.steps // c, stream)     # exactly K steps
    ms_per_step = ms / args.steps
    _, k_up = _replay_ms(g_up, 0, len(g_up), stream)
    ms, _ = _replay_ms(g_up, k_up, 2 * len(g_up), stream)           # two passes over the pool
    up_avg_ms = ms / (2 * R)

    gbs = (bytes_up + bytes_dn) / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_up / (up_avg_ms * 1e-3) / 1e9
    traffic = stored_traffic(args.traffic_json)
    out = {
        "metric": "Cubic dequant-GEMM HBM GB/s (M=1 decode) and TFLOP/s (M=4096), % of roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "K3 routed-expert decode, W2 G512, M=1, A16: gate_up 6144x7168 + "
                               "down 7168x3072 per step", "rotating_weight_copies": R,
                   "steps_per_graph": c, "algorithmic_bytes_per_step": bytes_up + bytes_dn},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_gemv_rows<bf16, G=512, 2 staggered wave-loads a wave, 12-wave workgroups, x staged first> (gate_up 6144x7168, M=1)",
                     "avg_launch_us": round(up_avg_ms * 1e3, 3),
                     "timing": f"HIP events on the launch stream around graph replays of {2 * R} "
                               f"back-to-back gate_up launches over {R} rotating copies",
                     "algorithmic_bytes_per_launch": bytes_up},
    }
    del ups, dns, g_step, g_up
    torch.cuda.empty_cache()
    out.update(prefill_blocks(cq, synth, dev, stream))
    out["decode_step_16x"] = decode_step_block(cq, synth, dev)
    if args.extra:
        out["extra"] = extra_workloads(cq, synth, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def floors(dev):
    """Floors of one launch on this part, from the floor kernels of
    libcubic_floors.so, each timed as graph replays with HIP events:
    - empty kernels with the decode GEMV's grid (512 x 256) and with 1 x 64;
    - load-only streams over the codes of gate_up 6144 x 7168 W2 (11,010,048 bytes)
      on 50 rotating copies (551 MB, past the 256 MB last-level cache): the GEMV's
      access pattern (12-row workgroups, 16 rows x 64 bytes per wave load) and
      contiguous 1 KB wave loads on 512 and on 256 workgroups; the same for the
      16-expert decode step's 176 MB of codes in one launch (GEMV pattern, and
      contiguous with eight loads in flight per lane on 2688 and 768 workgroups);
    - one lane chasing a cyclic permutation of 2^27 uint32 (512 MB): the latency of
      a dependent load that misses every cache;
    - arrival probes over the gate_up codes: when a wave's first and last loads
      arrive with the old GEMV's pattern (16 rows x 64 bytes per wave load) and
      with whole rows per wave load."""
    import ctypes

    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "dequant_gemm_amd", "lib", "libcubic_floors.so"))
    vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint
    lib.floors_empty.argtypes = [u32, u32, vp, vp]
    lib.floors_rows.argtypes = [vp, i64, i64, vp, vp]
    lib.floors_contig.argtypes = [vp, u32, i64, vp, vp]
    lib.floors_contig8.argtypes = [vp, u32, i64, vp, vp]
    lib.floors_chase.argtypes = [vp, i64, vp, vp]
    for f in (lib.floors_empty, lib.floors_rows, lib.floors_contig, lib.floors_contig8, lib.floors_chase):
        f.restype = ctypes.c_int
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = torch.empty(8192 * 256, dtype=torch.int32, device=dev)
    op = ctypes.c_void_p(out.data_ptr())
    rows, row_bytes = 6144, 1792
    nbytes = rows * row_bytes
    bufs = [torch.full((nbytes,), i, dtype=torch.uint8, device=dev) for i in range(50)]

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"floor kernel launch failed ({rc})")

    res = {}
    res["empty_512x256_us"] = round(_graph_time([lambda: ok(lib.floors_empty(512, 256, op, st()))] * 50, 5, dev)
                                    * 1e3, 3)
    res["empty_1x64_us"] = round(_graph_time([lambda: ok(lib.floors_empty(1, 64, op, st()))] * 50, 5, dev) * 1e3, 3)
    for name, call in (
            ("stream_gemv_pattern_512wg", lambda b: ok(lib.floors_rows(b.data_ptr(), rows, row_bytes, op, st()))),
            ("stream_contig_512wg", lambda b: ok(lib.floors_contig(b.data_ptr(), 512, nbytes // 512, op, st()))),
            ("stream_contig_256wg", lambda b: ok(lib.floors_contig(b.data_ptr(), 256, nbytes // 256, op, st())))):
        ms = _graph_time([(lambda b=b: call(b)) for b in bufs], 5, dev)
        res[name + "_us"] = round(ms * 1e3, 3)
        res[name + "_GB/s"] = round(nbytes / ms / 1e6, 1)
    # When a wave's data arrives: each wave timestamps its start and the arrival
    # of its first and last load (100 MHz clock); per launch the medians over
    # waves, from the launch's earliest start; reported: the medians over 35
    # launches (after 5), each launch on the next copy.
    lib.floors_arrival.argtypes = [ctypes.c_int, vp, i64, vp, vp]
    lib.floors_arrival.restype = ctypes.c_int
    nw = 4 * ((rows + 11) // 12)
    stamps = torch.empty(3 * nw, dtype=torch.int64, device=dev)
    for kind, name in ((0, "arrival_gemv16_pattern"), (1, "arrival_whole_rows")):
        first, last, span = [], [], []
        for it in range(40):
            ok(lib.floors_arrival(kind, bufs[it % len(bufs)].data_ptr(), rows, ctypes.c_void_p(stamps.data_ptr()),
                                  st()))
            torch.cuda.synchronize(dev)
            if it < 5:
                continue
            t = stamps.view(nw, 3).cpu().numpy().astype(np.int64)
            t0 = t[:, 0].min()
            first.append(np.median(t[:, 1] - t0) * 0.01)
            last.append(np.median(t[:, 2] - t0) * 0.01)
            span.append((t[:, 2].max() - t0) * 0.01)
        res[name + "_first_us"] = round(float(np.median(first)), 3)
        res[name + "_last_us"] = round(float(np.median(last)), 3)
        res[name + "_span_us"] = round(float(np.median(span)), 3)
    del bufs
    # the 16-expert decode step's code bytes in one launch: 16 x 6144 rows of
    # 1792 bytes (176 MB), three rotating copies (528 MB)
    big_rows = 16 * rows
    big = big_rows * row_bytes
    bigs = [torch.full((big,), i, dtype=torch.uint8, device=dev) for i in range(3)]
    for name, call in (
            ("step16_gemv_pattern", lambda b: ok(lib.floors_rows(b.data_ptr(), big_rows, row_bytes, op, st()))),
            ("step16_contig8_2688wg", lambda b: ok(lib.floors_contig8(b.data_ptr(), 2688, big // 2688, op, st()))),
            ("step16_contig8_768wg", lambda b: ok(lib.floors_contig8(b.data_ptr(), 768, big // 768, op, st())))):
        ms = _graph_time([(lambda b=b: call(b)) for b in bigs], 5, dev)
        res[name + "_us"] = round(ms * 1e3, 3)
        res[name + "_GB/s"] = round(big / ms / 1e6, 1)
    res["step16_bytes"] = big
    del bigs
    n = 1 << 27
    perm = np.random.default_rng(11).permutation(n).astype(np.uint32)
    nxt = np.empty(n, dtype=np.uint32)
    nxt[perm] = np.roll(perm, -1)                      # one cycle through every index
    dn = torch.from_numpy(nxt.view(np.int32)).to(dev)
    del perm, nxt
    steps = 20000
    ok(lib.floors_chase(dn.data_ptr(), 1000, op, st()))
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    ok(lib.floors_chase(dn.data_ptr(), steps, op, st()))
    b.record()
    torch.cuda.synchronize()
    res["chase_ns_per_dependent_load"] = round(a.elapsed_time(b) * 1e6 / steps, 1)
    res["bytes_per_stream_launch"] = nbytes
    print(json.dumps({"floors": res}), flush=True)


def counter_run_other(cq, synth, dev, which, steps):
    """Eager launches of one product (no graphs), for counter passes: the M = 4096
    prefill products (W3 G256 6144 x 7168), the 16-expert decode step (A16 or A8,
    eight disjoint expert sets of 128 resident experts) or W4 G128 gate_up at 64 rows."""
    import torch
    if which in ("prefill_a16", "prefill_a8"):
        w, x = synth.prefill_config(seed=5, device=dev)
        cw = cq.CubicWeight(cq.cubic_pack(w.codes, 3).reshape(-1), w.scales, w.shapes, w.N, w.K, 3, 256)
        y = torch.empty((4096, 6144), dtype=torch.float32, device=dev)
        if which == "prefill_a16":
            ws = torch.empty(cq.cubic_gemm_a16_workspace_bytes(4096, 7168), dtype=torch.uint8, device=dev)
            run = lambda i: cq.cubic_gemm_a16(x, cw, out=y, workspace=ws)
        else:
            xq, sx = cq.act_quant_int8_per_token(x)
            run = lambda i: cq.cubic_gemm_a8(xq, sx, cw, out=y)
    elif which in ("decode_step", "decode_step_a8"):
        pool, x, ids, ws, y = _decode_step_setup(cq, synth, dev)
        if which == "decode_step":
            run = lambda i: cq.cubic_moe_grouped_gemm(x, ids[i % len(ids)], pool, 128, out=y, workspace=ws)
        else:
            xq, sx = cq.act_quant_int8_per_token(x)
            run = lambda i: cq.cubic_moe_grouped_gemm_a8(xq, sx, ids[i % len(ids)], pool, 128, out=y,
                                                         workspace=ws)
    else:
        (wu, xu), _ = synth.smallm_config(64, seed=3, device=dev)
        cw = cq.CubicWeight(cq.cubic_pack(wu.codes, 4).reshape(-1), wu.scales, wu.shapes, wu.N, wu.K, 4, 128)
        ws = torch.empty(max(1, cq.cubic_gemm_a16_workspace_bytes(64, wu.K)), dtype=torch.uint8, device=dev)
        y = torch.empty((64, wu.N), dtype=torch.float32, device=dev)
        run = lambda i: cq.cubic_gemm_a16(xu, cw, out=y, workspace=ws)
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run": which, "launches": steps}), flush=True)


def _decode_step_setup(cq, synth, dev):
    """128 resident gate_up experts 6144 x 7168 W2 G512, one token, eight disjoint
    top-16 sets of them, workspace and output."""
    import torch
    H, I, bits, group, E, topk = 7168, 3072, 2, 512, 128, 16
    N, cb = 2 * I, 2 * I * H * bits // 8
    codes = torch.empty(E * cb, dtype=torch.uint8, device=dev)
    scales = torch.empty((E, N, H // group), dtype=torch.float32, device=dev)
    shapes = torch.empty((E, N, H // group, 2), dtype=torch.int16, device=dev)
    for e in range(E):
        w = synth.moe_expert(e, seed=4, N=N, K=H, bits=bits, group=group, device=dev)
        cq.cubic_pack(w.codes, bits, out=codes[e * cb:(e + 1) * cb].view(N, H * bits // 8))
        scales[e] = w.scales
        shapes[e] = w.shapes
    pool = cq.CubicWeight(codes, scales.reshape(-1), shapes.reshape(-1), N, H, bits, group)
    x, _ = synth.moe_routing(seed=4, T=1, E=E, topk=topk, K=H, device=dev)
    perm = torch.randperm(E, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    ids = [perm[16 * k:16 * k + 16].view(1, topk).to(dev) for k in range(E // topk)]
    ws = torch.empty(cq.cubic_moe_workspace_bytes(1, topk, E), dtype=torch.uint8, device=dev)
    y = torch.empty((1, topk, N), dtype=torch.float32, device=dev)
    return pool, x, ids, ws, y


def prefill_blocks(cq, synth, dev, stream):
    """The M = 4096 half of the metric: W3 G256 weight 6144 x 7168, activations
    4096 x 7168 bf16 with 36 outlier columns. prefill_a16: one cubic_gemm_a16 call
    (activation preparation + k_prefill_a16). prefill_a8: act_quant_int8_per_token
    then cubic_gemm_a8 (k_prefill_a8), the roofline for the product kernel alone.
    MFMA-bound, so the weight is not rotated; graph replays, HIP events on the
    replay stream."""
    import torch
    res = {}
    w, x = synth.prefill_config(seed=5, device=dev)
    cw = cq.CubicWeight(cq.cubic_pack(w.codes, 3).reshape(-1), w.scales, w.shapes, w.N, w.K, 3, 256)
    del w.codes
    flops = 2.0 * 4096 * 6144 * 7168
    ws = torch.empty(cq.cubic_gemm_a16_workspace_bytes(4096, 7168), dtype=torch.uint8, device=dev)
    y = torch.empty((4096, 6144), dtype=torch.float32, device=dev)
    ms = _graph_time([lambda: cq.cubic_gemm_a16(x, cw, out=y, workspace=ws)] * 4, 5, dev)
    tf = flops / ms / 1e9
    res["prefill_a16"] = {
        "TFLOP/s": round(tf, 2), "ms": round(ms, 4),
        "workload": "W3 G256 6144x7168, M=4096 bf16, A16 (fp32 out)",
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_F16_PEAK_TFS, 4), "traffic": None,
                     "kernel": "cubic_gemm_a16 call: k_xprep + k_prefill_a16",
                     "avg_launch_us": round(ms * 1e3, 2),
                     "algorithmic_flops_per_launch": flops,
                     "timing": "HIP events around graph replays of 20 back-to-back calls"}}
    print(json.dumps({"prefill_a16": res["prefill_a16"]}), file=sys.stderr, flush=True)
    xq = torch.empty((4096, 7168), dtype=torch.int8, device=dev)
    sx = torch.empty((4096,), dtype=torch.float32, device=dev)
    ms_q = _graph_time([lambda: cq.act_quant_int8_per_token(x, xq, sx)] * 4, 5, dev)
    ms8 = _graph_time([lambda: cq.cubic_gemm_a8(xq, sx, cw, out=y)] * 4, 5, dev)
    t8 = flops / ms8 / 1e9
    res["prefill_a8"] = {
        "TOP/s": round(t8, 2), "gemm_ms": round(ms8, 4), "act_quant_ms": round(ms_q, 4),
        "TOP/s_with_act_quant": round(flops / (ms8 + ms_q) / 1e9, 2),
        "workload": "W3 G256 6144x7168, M=4096, Dynamic A8 (per-token int8)",
        "roofline": {"bound": "mfma", "achieved": round(t8, 2), "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(t8 / MFMA_I8_PEAK_TOPS, 4), "traffic": None,
                     "kernel": "k_prefill_a8", "avg_launch_us": round(ms8 * 1e3, 2),
                     "algorithmic_ops_per_launch": flops,
                     "timing": "HIP events around graph replays of 20 back-to-back launches"}}
    print(json.dumps({"prefill_a8": res["prefill_a8"]}), file=sys.stderr, flush=True)
    del x, xq, y, ws, cw
    torch.cuda.empty_cache()
    return res


def decode_step_block(cq, synth, dev):
    """The Kimi K3 decode step of one layer's routed experts: one token, top-16,
    as one grouped launch (routing + k_moe_stream) over gate_up 6144 x 7168 W2
    G512 experts. 128 experts are resident (1.5 GB); launch i takes the i-th of
    eight disjoint sets of 16, so consecutive launches share no expert and a set
    recurs only after 1.3 GB of other experts. Algorithmic bytes: 16 experts'
    codes and group parameters, the token row in, the 16 output rows out."""
    import torch
    H, bits, group, E, topk = 7168, 2, 512, 128, 16
    N = 6144
    pool, x, ids, ws, y = _decode_step_setup(cq, synth, dev)
    ms = _graph_time([(lambda i=i: cq.cubic_moe_grouped_gemm(x, i, pool, E, out=y, workspace=ws)) for i in ids],
                     5, dev)
    nb = topk * (N * H * bits // 8 + 8 * N * (H // group)) + H * 2 + topk * N * 4
    gbs = nb / ms / 1e6
    res = {"GB/s": round(gbs, 1), "us": round(ms * 1e3, 2), "bytes_per_launch": nb,
           "workload": "1 token x top-16 of 128 resident experts, gate_up 6144x7168 W2 G512, A16",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "cubic_moe_grouped_gemm call (one token: k_moe_stream<DecodeW2> reads the ids, no routing kernel)",
                        "avg_launch_us": round(ms * 1e3, 2),
                        "timing": "HIP events around graph replays of 40 launches over 8 disjoint "
                                  "expert sets"}}
    # the same step in the Dynamic A8 mode: the token's int8 row (quantised once,
    # outside the timed launches) against the same 16-expert sets
    xq, sx = cq.act_quant_int8_per_token(x)
    ms8 = _graph_time([(lambda i=i: cq.cubic_moe_grouped_gemm_a8(xq, sx, i, pool, E, out=y, workspace=ws))
                       for i in ids], 5, dev)
    nb8 = topk * (N * H * bits // 8 + 8 * N * (H // group)) + H + 4 + topk * N * 4
    g8 = nb8 / ms8 / 1e6
    res["a8"] = {"GB/s": round(g8, 1), "us": round(ms8 * 1e3, 2), "bytes_per_launch": nb8,
                 "kernel": "cubic_moe_grouped_gemm_a8 call (one token: k_moe_a8<2> reads the ids, no routing kernel)",
                 "frac_of_hbm_peak": round(g8 / HBM_PEAK_GBS, 4)}
    print(json.dumps({"decode_step_16x": res}), file=sys.stderr, flush=True)
    del pool
    torch.cuda.empty_cache()
    return res


def _graph_time(calls, reps, dev):
    """Average time of one pass over `calls` (a list of no-argument launchers),
    captured once into a HIP graph and replayed `reps` times; HIP events on the
    replay stream bracket the replays."""
    import torch
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps / len(calls)


def _leg(res, key, val):
    """Store one extra leg's result and report it on stderr as it finishes."""
    import sys
    res[key] = val
    print(json.dumps({key: val}), file=sys.stderr, flush=True)


def _report(res, key):
    """One extra leg done: its result on stderr, as progress."""
    import sys
    print(json.dumps({key: res[key]}), file=sys.stderr, flush=True)


def extra_workloads(cq, synth, dev, stream):
    """The other workloads, each timed as graph replays: small-batch W4 G128
    (M = 8, 64) over rotating weight copies, nearest-level encoding, group
    fitting, and the routed-expert products and MLP step (one token x 16
    experts; 64 tokens x 16 over 896 experts)."""
    res = smallm_workloads(cq, synth, dev)
    res.update(encode_workloads(cq, synth, dev))
    res.update(fit_workloads(cq, synth, dev))
    res.update(moe_workloads(cq, synth, dev))
    return res


def smallm_workloads(cq, synth, dev):
    """Small-batch W4 G128 products (M = 8, 64) over 16 rotating weight copies."""
    import torch
    res = {}
    copies = 16
    for M in (8, 64):
        (wu, xu), (wd, xd) = synth.smallm_config(M, seed=3, device=dev)
        for name, ww, xx in (("gate_up", wu, xu), ("down", wd, xd)):
            base = cq.CubicWeight(cq.cubic_pack(ww.codes, 4).reshape(-1), ww.scales, ww.shapes, ww.N,
                                  ww.K, 4, 128)
            pool = [base] + [cq.CubicWeight(base.codes.clone(), base.scales.clone(), base.shapes.clone(),
                                            base.N, base.K, 4, 128) for _ in range(copies - 1)]
            wsp = torch.empty(max(1, cq.cubic_gemm_a16_workspace_bytes(M, ww.K)), dtype=torch.uint8,
                              device=dev)
            yy = torch.empty((M, ww.N), dtype=torch.float32, device=dev)
            ms = _graph_time([(lambda c=c: cq.cubic_gemm_a16(xx, c, out=yy, workspace=wsp))
                              for c in pool], 4, dev)
            nb = algorithmic_bytes(ww.N, ww.K, 4, 128, M)
            res[f"smallm_w4_M{M}_{name}"] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                                              "frac_of_hbm_peak": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)}
            _report(res, f"smallm_w4_M{M}_{name}")
            del pool, base
        del wu, wd
        torch.cuda.empty_cache()
    return res


def encode_workloads(cq, synth, dev):
    """cubic_encode of fp32 gate_up 6144 x 7168 weights (W2 G512 and W4 G128):
    three rotating weight copies (528 MB), graph replays. Algorithmic bytes:
    4 per weight in, 1 per weight out, 8 per group of parameters."""
    import torch
    res = {}
    N, K = 6144, 7168
    for bits, group in ((2, 512), (4, 128)):
        g = synth.make_generator(9500 + bits, dev)
        w = synth.make_weight(g, N, K, bits, group, "ternary" if bits == 2 else "uniform", 0.02, dev)
        xs = [torch.randn((N, K), generator=g, device=dev) * 0.03 for _ in range(3)]
        out = torch.empty((N, K), dtype=torch.int8, device=dev)
        ms = _graph_time([(lambda x=x: cq.cubic_encode(x, w.scales, w.shapes, bits, group, out=out)) for x in xs],
                         5, dev)
        nb = N * K * 5 + 8 * N * (K // group)
        res[f"encode_w{bits}g{group}_gate_up"] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                                                   "frac_of_hbm_peak": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)}
        _report(res, f"encode_w{bits}g{group}_gate_up")
        del xs, w
        torch.cuda.empty_cache()
    return res


# fp32 VALU issue: 256 compute units x 4 SIMDs x 32 lanes per clock at 2.4 GHz =
# 78.6 T lane-instructions/s (the 157.3 TFLOP/s vector figure counts an fma as two)
VALU_PEAK_TINSTR = 256 * 4 * 32 * 2.4e9 / 1e12


def fit_workloads(cq, synth, dev):
    """cubic_fit (data-free group fitting, 8512 candidates per group): gate_up
    6144 x 7168 at W4 G128 (344,064 groups) and the 3 x 15,360-sample W4 G128
    reconstruction workload. VALU work per (weight, candidate) at W4: 12
    instructions (7 differences, 1 min and 3 three-way mins over |d|, 1 fma), the
    k_fit<4> inner loop (plus one move per four weights, not counted)."""
    import torch
    res = {}
    cands = 532 * 16
    g = synth.make_generator(9600, dev)
    w = torch.randn((6144, 7168), generator=g, device=dev) * 0.02
    ms = _graph_time([lambda: cq.cubic_fit(w, 4, 128)], 2, dev)
    instr = 6144 * 7168 * cands * 12
    res["fit_w4g128_gate_up"] = {"ms": round(ms, 3), "groups/s": round(6144 * 56 / ms * 1e3, 1),
                                 "valu_T_lane_instr/s": round(instr / ms / 1e9, 2),
                                 "frac_of_valu_issue_peak": round(instr / ms / 1e9 / VALU_PEAK_TINSTR, 4)}
    _report(res, "fit_w4g128_gate_up")
    gen = torch.Generator().manual_seed(9601)
    xs = [torch.rand(15360, generator=gen) * 2 - 1, torch.randn(15360, generator=gen),
          torch.distributions.Laplace(0.0, 1.0).sample((15360,))]
    ws = [x.to(torch.float32).reshape(-1, 128).to(dev) for x in xs]
    ms = _graph_time([(lambda x=x: cq.cubic_fit(x, 4, 128)) for x in ws], 5, dev)
    res["fit_w4g128_nrmse_15360x3"] = {"us_per_distribution": round(ms * 1e3, 2),
                                       "note": "120 groups per launch: fewer workgroups than compute units"}
    _report(res, "fit_w4g128_nrmse_15360x3")
    del w, ws
    torch.cuda.empty_cache()
    return res


def moe_workloads(cq, synth, dev):
    """Routed experts at the decode distributions, W2 G512: gate_up 6144 x 7168
    (the grouped product) and the whole MLP step (gate_up, SiLU * up in bf16,
    down 7168 x 3072, router-weighted sum). Decode step: one token routed to 16
    of 64 resident experts, four disjoint sets in turn (consecutive launches share
    no expert). Batch: 64 tokens x top-16
    over 896 experts (~600 touched). Algorithmic bytes: the touched experts'
    codes and group parameters plus activations in and outputs out; the step's
    intermediates ([P][2I] fp32, [P][I] bf16, [P][H] fp32 for P routed pairs)
    are not counted."""
    import torch
    res = {}
    H, I, bits, group = 7168, 3072, 2, 512

    def pool(E, seed, N, K):
        cb = N * K * bits // 8
        codes = torch.empty(E * cb, dtype=torch.uint8, device=dev)
        scales = torch.empty((E, N, K // group), dtype=torch.float32, device=dev)
        shapes = torch.empty((E, N, K // group, 2), dtype=torch.int16, device=dev)
        for e in range(E):
            w = synth.moe_expert(e, seed=seed, N=N, K=K, bits=bits, group=group, device=dev)
            cq.cubic_pack(w.codes, bits, out=codes[e * cb:(e + 1) * cb].view(N, K * bits // 8))
            scales[e] = w.scales
            shapes[e] = w.shapes
        return cq.CubicWeight(codes, scales.reshape(-1), shapes.reshape(-1), N, K, bits, group)

    def expert_bytes(N, K):
        return N * K * bits // 8 + 8 * N * (K // group)

    def row(ms, nb, **kw):
        r = {"us": round(ms * 1e3, 2)} if ms < 1 else {"ms": round(ms, 4)}
        r.update({"GB/s": round(nb / ms / 1e6, 1), "frac_of_hbm_peak": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)})
        r.update(kw)
        return r

    gu_b, dn_b = expert_bytes(2 * I, H), expert_bytes(H, I)
    E, topk = 64, 16
    gu, dn = pool(E, 4, 2 * I, H), pool(E, 6, H, I)
    x, _ = synth.moe_routing(seed=4, T=1, E=E, topk=topk, K=H, device=dev)
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(E, generator=g).to(torch.int32)          # 4 disjoint sets of 16
    ids = [perm[topk * k:topk * k + topk].view(1, topk).to(dev) for k in range(E // topk)]
    tw = torch.softmax(torch.rand((1, topk), generator=g), dim=1).to(dev)
    ws = torch.empty(cq.cubic_moe_workspace_bytes(1, topk, E), dtype=torch.uint8, device=dev)
    y = torch.empty((1, topk, 2 * I), dtype=torch.float32, device=dev)
    ms = _graph_time([(lambda i=i: cq.cubic_moe_grouped_gemm(x, i, gu, E, out=y, workspace=ws))
                      for i in ids], 5, dev)
    nb = topk * gu_b + H * 2 + topk * 2 * I * 4
    res["moe_decode_1tok_top16"] = row(ms, nb, bytes_per_launch=nb)
    _report(res, "moe_decode_1tok_top16")
    wsm = torch.empty(cq.cubic_moe_mlp_workspace_bytes(1, topk, E, H, I), dtype=torch.uint8, device=dev)
    ym = torch.empty((1, H), dtype=torch.float32, device=dev)
    ms = _graph_time([(lambda i=i: cq.cubic_moe_mlp(x, i, tw, gu, dn, E, out=ym, workspace=wsm))
                      for i in ids], 5, dev)
    nb = topk * (gu_b + dn_b) + H * 2 + H * 4
    res["moe_mlp_decode_1tok_top16"] = row(ms, nb, bytes_per_launch=nb)
    _report(res, "moe_mlp_decode_1tok_top16")
    xq, sx = cq.act_quant_int8_per_token(x)
    ms = _graph_time([(lambda i=i: cq.cubic_moe_grouped_gemm_a8(xq, sx, i, gu, E, out=y, workspace=ws))
                      for i in ids], 5, dev)
    nb = topk * gu_b + H + 4 + topk * 2 * I * 4
    res["moe_a8_decode_1tok_top16"] = row(ms, nb, bytes_per_launch=nb)
    _report(res, "moe_a8_decode_1tok_top16")
    wsa = torch.empty(cq.cubic_moe_mlp_a8_workspace_bytes(1, topk, E, H, I), dtype=torch.uint8, device=dev)
    ms = _graph_time([(lambda i=i: cq.cubic_moe_mlp_a8(x, i, tw, gu, dn, E, out=ym, workspace=wsa))
                      for i in ids], 5, dev)
    nb = topk * (gu_b + dn_b) + H * 2 + H * 4
    res["moe_mlp_a8_decode_1tok_top16"] = row(ms, nb, bytes_per_launch=nb)
    _report(res, "moe_mlp_a8_decode_1tok_top16")
    del gu, dn, ws, wsm, wsa, y
    torch.cuda.empty_cache()
    E, T = 896, 64
    gu, dn = pool(E, 4, 2 * I, H), pool(E, 6, H, I)
    x, tid = synth.moe_routing(seed=4, T=T, E=E, topk=topk, K=H, device=dev)
    tw = torch.softmax(torch.rand((T, topk), generator=torch.Generator().manual_seed(8)), dim=1).to(dev)
    touched = int(torch.unique(tid).numel())
    ws = torch.empty(cq.cubic_moe_workspace_bytes(T, topk, E), dtype=torch.uint8, device=dev)
    y = torch.empty((T, topk, 2 * I), dtype=torch.float32, device=dev)
    ms = _graph_time([lambda: cq.cubic_moe_grouped_gemm(x, tid, gu, E, out=y, workspace=ws)], 3, dev)
    nb = touched * gu_b + T * H * 2 + T * topk * 2 * I * 4
    res["moe_896x64tok_top16"] = row(ms, nb, touched_experts=touched)
    _report(res, "moe_896x64tok_top16")
    xq, sx = cq.act_quant_int8_per_token(x)
    ms = _graph_time([lambda: cq.cubic_moe_grouped_gemm_a8(xq, sx, tid, gu, E, out=y, workspace=ws)], 3, dev)
    nb = touched * gu_b + T * (H + 4) + T * topk * 2 * I * 4
    res["moe_a8_896x64tok_top16"] = row(ms, nb, touched_experts=touched)
    _report(res, "moe_a8_896x64tok_top16")
    del ws, y
    wsm = torch.empty(cq.cubic_moe_mlp_workspace_bytes(T, topk, E, H, I), dtype=torch.uint8, device=dev)
    ym = torch.empty((T, H), dtype=torch.float32, device=dev)
    ms = _graph_time([lambda: cq.cubic_moe_mlp(x, tid, tw, gu, dn, E, out=ym, workspace=wsm)], 3, dev)
    nb = touched * (gu_b + dn_b) + T * H * 2 + T * H * 4
    res["moe_mlp_896x64tok_top16"] = row(ms, nb, touched_experts=touched)
    _report(res, "moe_mlp_896x64tok_top16")
    del wsm
    wsa = torch.empty(cq.cubic_moe_mlp_a8_workspace_bytes(T, topk, E, H, I), dtype=torch.uint8, device=dev)
    ms = _graph_time([lambda: cq.cubic_moe_mlp_a8(x, tid, tw, gu, dn, E, out=ym, workspace=wsa)], 3, dev)
    res["moe_mlp_a8_896x64tok_top16"] = row(ms, nb, touched_experts=touched)
    _report(res, "moe_mlp_a8_896x64tok_top16")
    del gu, dn, wsa, ym
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
