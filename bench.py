"""Benchmark: TFLOP/s and fraction of the MFMA dense peak of C = A @ B on one MI355X.

One step is one product over the workload's synthetic operands (seeded, see
dense_gemm_07_amd/inputs.py), inputs already resident in HBM. The timed steps
call the library's normal gemm entry point with its built-in config choice;
--autotune first benchmarks the candidates and times the cached winner (a
one-time cost, reported separately). Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # MI355X dense: MFMA bf16/fp16, fp32
SPEC_SCLK_MHZ = 2400.0  # the shader clock the peaks above assume
HBM_GBPS = 8000.0
METRIC = "TFLOP/s and % of MFMA dense peak, 4096³ bf16 GEMM on 1 MI355X"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["dense_gemm_07_amd/csrc/dg_kernels.hpp", "dense_gemm_07_amd/csrc/dg_internal.hpp",
                  "dense_gemm_07_amd/csrc/mfma_units.hpp"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, cfg):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source and on the tile shape cfg runs; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    # The recorded kernel's tile: the first three integer template arguments
    # (gemm_simt names its two dtypes first, the MFMA kernels one).
    m = re.search(r"dg::\w+<(?:dg::\w+, )+(\d+), (\d+), (\d+)", (rec.get("kernels") or [""])[0])
    if not m or tuple(int(x) for x in m.groups()) != (cfg.block_m, cfg.block_n, cfg.block_k):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_median(csv_path, counter, kernel_substr=None):
    """Median value of one rocprofv3 counter over the dispatches of one kernel:
    the kernel whose name contains kernel_substr, or, if None, the kernel
    dispatched most often in the run."""
    import csv
    import statistics
    groups = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and (kernel_substr is None or kernel_substr in r["Kernel_Name"]):
            groups.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not groups:
        raise SystemExit(f"no {counter} samples for {kernel_substr!r} in {csv_path}")
    vals = [v for g in groups.values() for v in g] if kernel_substr else max(groups.values(), key=len)
    return statistics.median(vals), sorted(groups) if kernel_substr else [max(groups, key=lambda k: len(groups[k]))]


def record_traffic(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib, commands):
    """HBM bytes per GEMM launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a device copy of
    copy_mib MiB; written to profiles/traffic_<workload>.json with the hash of
    the kernel sources it was taken on."""
    fetch, kernels = _counter_median(fetch_csv, "FETCH_SIZE", "dg::gemm")
    write, _ = _counter_median(write_csv, "WRITE_SIZE", "dg::gemm")
    copy_kib = copy_mib * 1024.0
    cf, _ = _counter_median(copy_fetch_csv, "FETCH_SIZE")
    cw, _ = _counter_median(copy_write_csv, "WRITE_SIZE")
    fs, ws = copy_kib / cf, copy_kib / cw
    rec = {"workload": workload, "kernels": kernels, "kernel_source_hash": kernel_source_hash(),
           "fetch_size_kib_raw": fetch, "write_size_kib_raw": write,
           "copy_calibration_mib": copy_mib, "copy_fetch_size_kib_raw": cf, "copy_write_size_kib_raw": cw,
           "fetch_scale": fs, "write_scale": ws,
           "hbm_read_bytes_per_launch": round(fetch * fs * 1024), "hbm_write_bytes_per_launch": round(write * ws * 1024),
           "hbm_bytes_per_launch": round((fetch * fs + write * ws) * 1024), "commands": commands}
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def cpu_baseline(w, a_cpu, b_cpu, target_s=10.0):
    """The oracle, as it stands, on a row slice of the same product."""
    import oracle
    from dense_gemm_07_amd import inputs

    oracle.build()
    A = inputs.bits(a_cpu, w.in_dtype)
    B = inputs.bits(b_cpu, w.in_dtype)
    # Two probes separate the fixed cost (decoding B) from the per-row cost,
    # then the slice is sized to about target_s of wall time (at most all of C).
    probes = []
    for r in (min(w.M, 16), min(w.M, 64)):
        t0 = time.perf_counter()
        oracle.gemm(A[:r], B, w.in_dtype)
        probes.append((r, time.perf_counter() - t0))
    (r1, t1), (r2, t2) = probes
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-9)
    rows = int(min(w.M, max(r2, (target_s - max(t1 - per_row * r1, 0.0)) / per_row)))
    rows -= rows % 8 if rows > 8 else 0
    if rows > r2:
        t0 = time.perf_counter()
        oracle.gemm(A[:rows], B, w.in_dtype)
        dt = time.perf_counter() - t0
    else:
        rows, dt = r2, t2
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of C (A[{rows},{w.K}] @ B[{w.K},{w.N}], {w.in_dtype}), "
                      f"{dt:.2f} s wall, fp64 k-ascending sums"}


def warm_up(step, steps, settle_ms):
    """The untimed warm-up: `steps` steps, then more until `settle_ms` of wall time has passed since
    the first. When a load starts from idle, the board's power manager first lets the clock run high,
    then pulls it down past its sustained level for some 10 ms before settling (a kernel trace of
    back-to-back 4096^3 launches: 107 us, then 116-140 us, then a steady 105.7 us). A timed region
    inside that dip measures the transient, not the sustained rate. Returns the extra steps run."""
    import torch
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    extra, batch = 0, 4
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        extra += batch
        batch = min(2 * batch, 256)
    return extra


def sclk_file(dev_index):
    """The device's sysfs list of shader clock levels (the current one marked '*'), or None if unreadable."""
    import torch
    p = torch.cuda.get_device_properties(dev_index)
    try:
        bdf = "%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    except AttributeError:
        return None
    path = f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk"
    return path if os.access(path, os.R_OK) else None


def read_sclk_mhz(path):
    """The shader clock (MHz) on the marked line of pp_dpm_sclk, or None."""
    try:
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line.endswith("*"):
                    return float(line.split(":", 1)[1].rstrip("*").strip().lower().removesuffix("mhz"))
    except (OSError, ValueError, IndexError):
        return None
    return None


def clock_window(step, dev_index, seconds, achieved=None, peak=None):
    """Shader clock while `step` runs back to back for about `seconds` (after the timed region, so the
    throughput figure is unaffected). A thread reads pp_dpm_sclk every 5 ms; the steps are issued in
    batches with a synchronisation between them. With `achieved` and `peak` (a peak quoted at
    SPEC_SCLK_MHZ) it also gives the peak scaled to the median clock and achieved / that."""
    import threading

    import torch
    path = sclk_file(dev_index)
    if path is None or seconds <= 0:
        return None
    before = read_sclk_mhz(path)
    samples, running = [], threading.Event()
    running.set()

    def poll():
        while running.is_set():
            v = read_sclk_mhz(path)
            if v is not None:
                samples.append(v)
            time.sleep(0.005)
    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    batch = 8
    while time.perf_counter() - t0 < seconds:
        tb = time.perf_counter()
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        if time.perf_counter() - tb < 0.02:
            batch *= 2
    running.clear()
    th.join()
    after = read_sclk_mhz(path)
    if not samples:
        return None
    ss = sorted(samples)
    out = {"source": "pp_dpm_sclk", "before_mhz": before, "after_mhz": after,
           "during_mhz": {"median": ss[len(ss) // 2], "min": ss[0], "max": ss[-1], "samples": len(ss)},
           "window_s": round(time.perf_counter() - t0, 2), "spec_mhz": SPEC_SCLK_MHZ}
    if achieved is not None and peak is not None:
        adj = peak * ss[len(ss) // 2] / SPEC_SCLK_MHZ
        out["clock_adjusted_peak"] = round(adj, 1)
        out["frac_of_clock_adjusted_peak"] = round(achieved / adj, 4)
    return out


def bench_attention(args):
    """Attention forward: O = softmax(QK^T/sqrt(d) [causal]) V, [batch, heads, seq, head_dim] bf16."""
    import torch

    import dense_gemm_07_amd as dg

    B, H, S, D = max(1, args.batch), args.heads, args.seq, args.head_dim
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn((B, H, S, D), generator=gen).to(torch.bfloat16).to(dev) for _ in range(3))
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    step = lambda: dg.attention(q, k, v, out=o, causal=args.causal, stream=stream)
    settle_steps = warm_up(step, args.warmup, args.settle_ms)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # Useful work: two S x S x D products per (batch, head); a causal mask keeps
    # the S (S + 1) / 2 allowed (query, key) pairs.
    pairs = S * (S + 1) / 2 if args.causal else S * S
    flops = 4.0 * B * H * pairs * D
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    result = {
        "metric": f"attention forward TFLOP/s (bf16, seq {S}, head_dim {D}) on 1 MI355X",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"attention fwd b{B} h{H} s{S} d{D}{' causal' if args.causal else ''} bf16",
                   "batch": B, "heads": H, "seq": S, "head_dim": D, "causal": args.causal},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None},
        "settle": {"ms": args.settle_ms, "extra_warmup_steps": settle_steps},
    }
    result["sclk"] = clock_window(step, dev.index or 0, args.clock_seconds, tflops, peak)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="square_4096_bf16")
    ap.add_argument("--autotune", action="store_true", help="autotune first and time the winner")
    ap.add_argument("--no-autotune", action="store_true", help="(default) time the built-in config choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, run torch's device copy of a MIB-sized buffer --steps times "
                         "(reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="no GPU work: turn rocprofv3 counter CSVs into profiles/traffic_<workload>.json")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the calibration copy (with --record-traffic)")
    ap.add_argument("--commands", default="", help="commands that produced the CSVs (with --record-traffic)")
    ap.add_argument("--epilogue", default="none", choices=["none", "bias", "bias_relu", "bias_gelu", "residual"],
                    help="time dg_gemm_ex with a fused epilogue: fp32 bias per column (+ activation), or "
                         "C = A@B + R with a separate residual R of C's dtype")
    ap.add_argument("--batch", type=int, default=1, help="time a strided batch of this many products (dg_gemm_ex)")
    ap.add_argument("--split-k", action="store_true",
                    help="time dg_gemm_ex with a workspace (the library may split K)")
    ap.add_argument("--config", default="",
                    help="time an explicit kernel config BMxBNxBK:waves:stages:group_m:xcd_remap[:k_splits] "
                         "(ablations; k_splits > 1, or sk for stream-K, with --split-k)")
    ap.add_argument("--misalign-a", action="store_true",
                    help="view A one element past a 16-byte boundary (forces the register-staged kernel)")
    ap.add_argument("--rotate", type=int, default=1, metavar="SETS",
                    help="cycle the product through SETS copies of (A, B, C), so that more than the "
                         "256 MB Infinity Cache is touched between reuses (cold-cache numbers)")
    ap.add_argument("--attention", action="store_true",
                    help="time the attention forward kernel instead (--batch, --heads, --seq, --head-dim, --causal)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="keep warming up (beyond --warmup steps) until this much wall time has passed, "
                         "so the timed steps run at the board's settled clock (0: exactly --warmup steps)")
    ap.add_argument("--clock-seconds", type=float, default=0.5,
                    help="after the timed steps, run the same step this long while sampling the shader "
                         "clock (0: skip)")
    ap.add_argument("--heads", type=int, default=16)
    ap.add_argument("--seq", type=int, default=8192)
    ap.add_argument("--head-dim", type=int, default=64)
    ap.add_argument("--causal", action="store_true")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic, args.copy_mib, args.commands)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (a product shards "
              f"across GPUs without exchange, but the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch

    import dense_gemm_07_amd as dg
    from dense_gemm_07_amd import inputs
    from dense_gemm_07_amd.build import LIB, build

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": args.steps}), flush=True)
        return
    if not os.path.exists(LIB):
        build()
    if args.attention:
        bench_attention(args)
        return
    w = inputs.find(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb = max(1, args.batch)
    ex = args.epilogue != "none" or nb > 1 or args.split_k
    out_dt = inputs.TORCH_DTYPES[w.out_dtype]
    if nb > 1:
        a_cpu, b_cpu = inputs.make_batch(w, nb, seed=0)
        a, b = a_cpu.to(dev), b_cpu.to(dev)
        c = torch.empty((nb, w.M, w.N), dtype=out_dt, device=dev)
    else:
        a_cpu, b_cpu = inputs.make(w, seed=0)
        a = inputs.to_device_like(a_cpu, dev)
        b = inputs.to_device_like(b_cpu, dev)
        c = torch.empty((w.M, w.N), dtype=out_dt, device=dev)
        if args.misalign_a:
            buf = torch.empty(a.numel() + 1, dtype=a.dtype, device=dev)
            view = buf[1:].view(a.shape)
            view.copy_(a)
            a = view
    # Epilogue operands (seeded): an fp32 bias per column, or a residual of C's dtype.
    gen = torch.Generator().manual_seed(1)
    epi = {}
    extra_bytes = 0
    if args.epilogue.startswith("bias"):
        epi["bias"] = torch.randn((nb, w.N) if nb > 1 else (w.N,), generator=gen).to(dev)
        epi["activation"] = {"bias": None, "bias_relu": "relu", "bias_gelu": "gelu"}[args.epilogue]
        extra_bytes = 4 * w.N * nb
    elif args.epilogue == "residual":
        epi["residual"] = torch.randn(c.shape, generator=gen).to(out_dt).to(dev)
        epi["beta"] = 1.0
        extra_bytes = c.numel() * c.element_size()
    torch.cuda.synchronize()

    tune_s = 0.0
    if args.autotune and not args.no_autotune and not ex:
        t0 = time.perf_counter()
        cfg, _ = dg.autotune(a, b, out=c, repeats=10)
        tune_s = time.perf_counter() - t0
    explicit = None
    if args.config:
        shape, waves, stages, group_m, xcd, *more = args.config.split(":")
        bm, bn, bk = (int(x) for x in shape.split("x"))
        explicit = next((k for k in dg.candidates(dg._dtype_code(a.dtype), dg._dtype_code(c.dtype))
                         if (k.block_m, k.block_n, k.block_k, k.waves, k.stages) ==
                         (bm, bn, bk, int(waves), int(stages))), None)
        if explicit is None:
            raise SystemExit(f"no compiled kernel {args.config}")
        explicit.group_m, explicit.xcd_remap = int(group_m), int(xcd)
        explicit.k_splits = (dg.STREAM_K if more[0] == "sk" else int(more[0])) if more else 1
        if (explicit.k_splits > 1 or explicit.k_splits == dg.STREAM_K) and not args.split_k:
            raise SystemExit("a config with k_splits > 1 or sk needs --split-k (the workspace)")
    if explicit is not None:
        cfg = explicit
    elif ex:
        ws_bytes = dg.DEFAULT_WORKSPACE_BYTES if args.split_k else 0
        cfg, _ = dg.select_config_ex(w.M, w.N, w.K, a.stride()[-2:], b.stride()[-2:], c.stride()[-2:],
                                     dg._dtype_code(a.dtype), dg._dtype_code(c.dtype), batch=nb,
                                     workspace_bytes=ws_bytes, ptr_a=a.data_ptr(), ptr_b=b.data_ptr(),
                                     ptr_c=c.data_ptr(),
                                     batch_strides=(a.stride(0), b.stride(0), c.stride(0)) if nb > 1 else (0, 0, 0))
    else:
        cfg, _ = dg.select_config(a, b, c)
    print(f"# workload {w.name}: config {cfg} (autotune {tune_s:.2f} s)", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    # Operand sets the steps cycle through (--rotate: copies of A, B and C, so
    # that B is not in the Infinity Cache when a product reads it).
    if args.rotate > 1 and (nb > 1 or args.misalign_a):
        raise SystemExit("--rotate is for single products with aligned operands")
    sets = [(a, b, c)] + [(a.clone(), b.clone(), torch.empty_like(c)) for _ in range(args.rotate - 1)]
    turn = [0]

    def next_set():
        s = sets[turn[0]]
        turn[0] = (turn[0] + 1) % len(sets)
        return s

    if explicit is not None and not ex:
        def step():
            sa, sb, sc = next_set()
            dg.gemm_config(sa, sb, explicit, out=sc, stream=stream)
    elif ex:
        def step():
            sa, sb, sc = next_set()
            dg.gemm_ex(sa, sb, out=sc, stream=stream, workspace=True if args.split_k else None, config=explicit,
                       **epi)
    else:
        def step():
            sa, sb, sc = next_set()
            dg.gemm(sa, sb, out=sc, stream=stream)
    settle_steps = warm_up(step, args.warmup, args.settle_ms)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # Per-launch durations (median, min, p90) from an event pair around each
    # launch, in a second pass over the same number of steps, so the events do
    # not enter the throughput figure above.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    launch_us = {"median": round(per[len(per) // 2], 2), "min": round(per[0], 2),
                 "p90": round(per[min(len(per) - 1, int(0.9 * len(per)))], 2)}

    flops = w.flops * nb
    nbytes = w.compulsory_bytes() * nb + extra_bytes
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.in_dtype]
    traffic = measured_traffic(w.name, cfg) if not ex else None
    hbm_bound = flops / nbytes < peak * 1e12 / (HBM_GBPS * 1e9)
    if hbm_bound:  # below the ridge: algorithmic bytes over time against the HBM peak
        gbps = nbytes / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / HBM_GBPS, 4), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4), "traffic": traffic}
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": f"gemm {w.M}x{w.N}x{w.K} {w.in_dtype}->{w.out_dtype}",
                   "name": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "b_layout": "col-major" if w.b_colmajor else "row-major",
                   "kernel_config": cfg.as_dict(), "autotune_s": round(tune_s, 3)},
        "roofline": roofline,
        "launch_us": launch_us,
        "settle": {"ms": args.settle_ms, "extra_warmup_steps": settle_steps},
    }
    if args.rotate > 1:
        result["config"]["rotate_sets"] = args.rotate
        result["roofline"]["traffic"] = None
    if ex:
        result["config"].update({"epilogue": args.epilogue, "batch": nb, "split_k_allowed": args.split_k})
    if args.config or args.misalign_a:
        result["config"].update({"explicit_config": args.config, "misaligned_a": args.misalign_a})
        result["roofline"]["traffic"] = None  # the recorded counters belong to the default configuration
    # Observed shader clock (the board lowers it under its power cap); the clock-adjusted
    # fraction applies to the matrix-core roof only.
    mfma = roofline["bound"] == "mfma"
    result["sclk"] = clock_window(step, dev.index or 0, args.clock_seconds,
                                  tflops if mfma else None, peak if mfma else None)
    if not args.no_cpu_baseline and not ex and not args.config and not args.misalign_a:
        result["cpu_baseline"] = cpu_baseline(w, a_cpu, b_cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
