#!/usr/bin/env python3
"""Benchmark of the fused, chunked top-K KL loss (forward + backward) on one
MI355X.

One step = one kd_topk_kl_fwd_bwd call over the whole synthetic batch
(every slice: teacher softmax, logits GEMM with softmax statistics and
gather, teacher correction, dH and dW GEMMs, loss), inputs resident in HBM.
Prints one JSON line:
  value      tokens/s over the whole job (T * steps / wall time)
  roofline   the dominant kernel's achieved TFLOP/s (algorithmic flops per
             launch / mean launch time from HIP events recorded around its
             launches on the library's stream during the timed steps)
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s & TFLOP/s fused top-K KL fwd+bwd, T=32k V=201k; % bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0
GEMM_KERNELS = {2: "gemm_logits", 4: "gemm_dh", 6: "gemm_dw"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Kernels whose HBM traffic bench.py reports, the symbol text that names them
# in a rocprofv3 counter file, and the sources that determine their code.
_GEMM_SRC = ("kd_gemm_fast.hip", "kd_mfma_tile.h", "kd_device.h", "kd_internal.h")
_ROW_SRC = ("kd_rowops.hip", "kd_device.h", "kd_internal.h")
_TK_SRC = ("kd_teacher.hip", "kd_mfma_tile.h", "kd_select.h", "kd_device.h",
           "kd_internal.h")
TRAFFIC_KERNELS = {
    "loss": [("k_fast_logits(", "gemm_logits", _GEMM_SRC),
             ("k_fast_dh", "gemm_dh", _GEMM_SRC),
             ("k_fast_dw", "gemm_dw", _GEMM_SRC),
             ("k_fast_logits_redo(", "flagged_rows", _GEMM_SRC),
             ("k_transpose_h(", "transpose_h", _GEMM_SRC),
             ("k_lse_fix<", "lse_fix", _ROW_SRC),
             ("k_reduce_dh(", "reduce_dh", _ROW_SRC),
             ("k_prep_rows(", "prep_rows", _ROW_SRC)],
    "teacher_topk": [("k_tk_gemm<0>", "tk_sample", _TK_SRC),
                     ("k_tk_gemm<1>", "tk_filter", _TK_SRC),
                     ("k_tk_theta(", "tk_theta", _TK_SRC),
                     ("k_tk_select(", "tk_select", _TK_SRC),
                     ("k_tk_stream<", "tk_stream", _TK_SRC)],
}


def source_sha(files):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_kl_loss_amd", "csrc")
    for name in sorted(files):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, config_key):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs, or None when they were taken on another configuration or the
    kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            k = json.load(f)["kernels"][kernel]
    except (OSError, ValueError, KeyError):
        return None
    if k.get("config") != config_key or k.get("source_sha") != source_sha(k["sources"]):
        return None
    return k.get("bytes_per_launch")


def record_traffic(op, config_key, fetch_dir, write_dir, copy_bytes):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of the op's kernels from two
    rocprofv3 --pmc runs (csv output), scaled by what the same counter reads
    for the runtime's device-to-device copy of copy_bytes (a reference of
    known traffic), into profiles/traffic.json."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                              recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copy = [v for n, vs in vals.items() if "copyBuffer" in n for v in vs]
        if not copy:
            raise SystemExit(f"no copy-kernel dispatch in {d}: run with --copy-calibration")
        factor = copy_bytes / (max(copy) * 1024.0)
        for pat, name, srcs in TRAFFIC_KERNELS["teacher_topk" if op == "teacher_topk" else "loss"]:
            vs = [v for n, v_ in vals.items() if pat in n for v in v_]
            if not vs:
                continue
            k = out.setdefault(name, {"config": config_key, "sources": list(srcs),
                                      "source_sha": source_sha(srcs),
                                      "dispatches": len(vs)})
            kib = sum(vs) / len(vs)
            key = "fetch" if counter == "FETCH_SIZE" else "write"
            k[f"{key}_kib_raw"] = round(kib)
            k[f"{key}_factor"] = round(factor, 4)
            k[f"{key}_bytes_per_launch"] = int(kib * 1024 * factor)
    for k in out.values():
        k["bytes_per_launch"] = k.get("fetch_bytes_per_launch", 0) + \
            k.get("write_bytes_per_launch", 0)
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec.setdefault("kernels", {})
    rec["about"] = ("HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE and "
                    "WRITE_SIZE runs (one counter per run), each scaled so that "
                    "a device-to-device copy of known size reads and writes its "
                    "own size; written by bench.py --record-traffic")
    rec["kernels"].update(out)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    log(f"traffic of {sorted(out)} written to {TRAFFIC_FILE}")


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def peak_from_device(hip):
    """bf16 dense peak from the device's CU count and peak clock
    (4096 flop per clock per CU for bf16 MFMA on gfx950)."""
    cus = hip.device_attribute(hip.ATTR_MULTIPROCESSOR_COUNT)
    khz = hip.device_attribute(hip.ATTR_CLOCK_RATE_KHZ)
    return {"cus": cus, "clock_mhz": khz / 1e3,
            "bf16_tflops": round(cus * khz * 1e3 * 4096 / 1e12, 1)}


def cpu_baseline(x, target_s):
    """The oracle, as it stands, on the first R tokens of the workload."""
    import numpy as np
    from oracle import kd_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) \
            if threadpool_info() else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))

    def run(R):
        m = None if x.mask is None else x.mask[:R]
        t0 = time.perf_counter()
        orc.kd_topk_kl(x.H[:R], x.W, x.topk_idx[:R], x.topk_logit[:R], m,
                       x.tau, chunk=R)
        return time.perf_counter() - t0

    # the oracle has a fixed cost (upcasting W) plus a per-token cost
    t8 = run(8)
    t32 = run(32)
    per = max((t32 - t8) / 24, 1e-6)
    fixed = max(t8 - 8 * per, 0.0)
    R = int(max(32, min(x.T, 4096, (target_s - fixed) / per)))
    log(f"cpu baseline: oracle on {R} tokens (~{fixed + per * R:.0f} s)")
    dt = run(R)
    model, affinity = cpu_info()
    return {"value": R / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "affinity_cpus": affinity,
            "sample": f"first {R} of {x.T} tokens of {x.name} "
                      f"(full d={x.d}, V={x.V}, K={x.K}), fp64 NumPy, one "
                      f"chunk; {dt:.1f} s wall"}


def config_key(args):
    """The configuration a traffic record belongs to."""
    import synth
    spec = synth.WORKLOADS[args.workload]
    default = 4096 if args.op == "teacher_topk" else spec["chunk"]
    return f"{args.op} {args.workload} chunk {args.chunk or default}"


def bench_vendor_gemm(args):
    """Reference timing, outside the library: torch's bf16 matrix products
    (hipBLASLt on ROCm) on the three products of one slice of the workload,
    C = the slice size, with the operands in the layouts the loss's kernels
    read (H_c [C, d] and W [V, d] row-major, probabilities [C, V] row-major)
    and bf16 outputs, no epilogue.  Context for the loss's GEMM rates on the
    same chip and clock, not a result of the library."""
    import torch

    import synth
    spec = synth.WORKLOADS[args.workload]
    C, d, V = args.chunk or spec["chunk"], spec["d"], spec["V"]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    H = torch.randn(C, d, device=dev, generator=g).to(torch.bfloat16)
    W = (torch.randn(V, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    P = torch.rand(C, V, device=dev, generator=g).to(torch.bfloat16)
    flop = 2.0 * C * d * V
    products = (("logits", "H_c W^T -> [C, V]", lambda: torch.nn.functional.linear(H, W)),
                ("dH", "P W -> [C, d]", lambda: torch.mm(P, W)),
                ("dW", "P^T H_c -> [V, d]", lambda: torch.mm(P.t(), H)))
    out = {}
    for name, what, f in products:
        for _ in range(max(args.warmup, 1)):
            f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            f()
            ev[i + 1].record()
        torch.cuda.synchronize()
        ts = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        ms = ts[len(ts) // 2]
        out[name] = {"product": what, "ms_median": round(ms, 4), "ms_min": round(ts[0], 4),
                     "tflops": round(flop / ms / 1e9, 2),
                     "frac_of_bf16_peak": round(flop / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
        log(f"vendor {name}: {ms:.3f} ms, {flop / ms / 1e9:.1f} TFLOP/s")
    print(json.dumps({"reference": "vendor bf16 GEMM (torch.mm -> hipBLASLt), no epilogue",
                      "workload": args.workload, "C": C, "d": d, "V": V,
                      "flops_per_product": flop, "steps": args.steps, "products": out}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--op", choices=("loss", "fwd", "bwd", "teacher_topk",
                                     "entropy_filter", "reverse_kl", "jsd"),
                    default="loss",
                    help="loss: kd_topk_kl_fwd_bwd (default); fwd: "
                         "kd_topk_kl_fwd (loss only); bwd: kd_topk_kl_bwd "
                         "(gradients, logits recomputed); teacher_topk: "
                         "kd_teacher_topk, the teacher cache build; "
                         "entropy_filter: kd_entropy_filter (top 70%% of "
                         "tokens by teacher entropy); reverse_kl / jsd: "
                         "kd_topk_div_fwd_bwd, the divergence over the "
                         "top-K support")
    ap.add_argument("--workload", default="t32k")
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--sweep", default="1024,2048,4096,8192,16384,32768",
                    help="slice sizes timed after the main measurement (loss "
                         "op; a few steps each, reported as chunk_sweep, with "
                         "the workspace each needs); empty to skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE; csv output) of this "
                         "--op/--workload/--chunk made with --copy-calibration "
                         "BYTES, then exit (no GPU needed)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="reference only, not the loss: time the vendor "
                         "library's plain bf16 GEMMs (torch.mm -> hipBLASLt) "
                         "on the three products of one slice of --workload "
                         "(no epilogue), print one JSON line and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="before the timed region, copy BYTES device-to-device "
                         "3 times (a reference kernel of known traffic for "
                         "rocprofv3 counter runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU "
              f"path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    if args.record_traffic:
        if not args.copy_calibration:
            raise SystemExit("--record-traffic needs --copy-calibration BYTES")
        return record_traffic(args.op, config_key(args), *args.record_traffic,
                              args.copy_calibration)
    if args.vendor_gemm:
        return bench_vendor_gemm(args)
    if args.op == "teacher_topk":
        return bench_teacher(args)
    if args.op == "entropy_filter":
        return bench_filter(args)
    if args.op in ("reverse_kl", "jsd"):
        return bench_div(args)

    import numpy as np
    import torch

    import synth
    import top_kl_loss_amd as kd
    from top_kl_loss_amd import hip

    torch.cuda.init()
    lib = kd.load_library()
    log(f"generating workload {args.workload}")
    t0 = time.perf_counter()
    x = synth.workload(args.workload, teacher_device="cuda")
    chunk = args.chunk or x.chunk
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s: T={x.T} d={x.d} "
        f"V={x.V} K={x.K} {x.dtype} tau={x.tau} chunk={chunk}")
    dev = torch.device("cuda:0")
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        dt_code = kd.KD_BF16
    else:
        H = torch.from_numpy(x.H).to(dev)
        W = torch.from_numpy(x.W).to(dev)
        dt_code = kd.KD_F32
    idx = torch.from_numpy(x.topk_idx).to(dev)
    lg = torch.from_numpy(x.topk_logit).to(dev)
    mask = None if x.mask is None else torch.from_numpy(x.mask).to(dev)
    T, d, V, K = x.T, x.d, x.V, x.K
    # the forward alone has a workspace of its own (no probabilities or
    # gradient buffers)
    ws_size = kd.kd_topk_kl_fwd_workspace_size if args.op == "fwd" else \
        kd.kd_topk_kl_workspace_size
    ws_bytes = ws_size(T, d, V, K, chunk, dt_code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    rl = torch.empty(T, **f32)
    dH = torch.empty(T, d, **f32)
    dW = torch.empty(V, d, **f32)
    torch.cuda.synchronize()
    hip.set_device(0)
    stream = hip.Stream()

    mptr = None if mask is None else mask.data_ptr()
    lse = torch.empty(T, **f32)
    grad_loss = torch.ones(1, **f32)

    def step():
        if args.op == "fwd":
            st = lib.kd_topk_kl_fwd(
                H.data_ptr(), W.data_ptr(), dt_code, idx.data_ptr(), lg.data_ptr(),
                mptr, T, d, V, K, float(x.tau), chunk, loss.data_ptr(),
                rl.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws_bytes, stream.value)
        elif args.op == "bwd":
            st = lib.kd_topk_kl_bwd(
                H.data_ptr(), W.data_ptr(), dt_code, idx.data_ptr(), lg.data_ptr(),
                mptr, T, d, V, K, float(x.tau), chunk, 0, grad_loss.data_ptr(),
                dH.data_ptr(), dW.data_ptr(), ws.data_ptr(), ws_bytes, stream.value)
        else:
            st = lib.kd_topk_kl_fwd_bwd(
                H.data_ptr(), W.data_ptr(), dt_code, idx.data_ptr(), lg.data_ptr(),
                mptr, T, d, V, K, float(x.tau), chunk, 0, loss.data_ptr(),
                rl.data_ptr(), dH.data_ptr(), dW.data_ptr(), ws.data_ptr(),
                ws_bytes, stream.value)
        if st != 0:
            raise RuntimeError(kd.kd_status_string(st))

    n_chunks = (T + chunk - 1) // chunk
    launches_per_step = 3 + 8 * n_chunks

    def run_logged(mask_bits, n_steps, cap):
        """Run n_steps with the launch log on; returns [(kind, ms)]."""
        starts = [hip.Event() for _ in range(cap)]
        ends = [hip.Event() for _ in range(cap)]
        arr_s = (ctypes.c_void_p * cap)(*[e.value for e in starts])
        arr_e = (ctypes.c_void_p * cap)(*[e.value for e in ends])
        kinds = (ctypes.c_int32 * cap)()
        count = ctypes.c_int32(0)
        kd.kd_set_launch_log(mask_bits, arr_s, arr_e, kinds, cap,
                             ctypes.byref(count))
        try:
            for _ in range(n_steps):
                step()
            stream.synchronize()
        finally:
            kd.kd_set_launch_log(0, None, None, None, 0, None)
        return [(kinds[i], starts[i].elapsed_ms(ends[i]))
                for i in range(count.value)]

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 x {args.copy_calibration} bytes")

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step()
    stream.synchronize()

    # One logged step over every kernel: per-kernel time split and the
    # dominant kernel.
    per_kind = {}
    for kind, ms in run_logged(0x7FF, 1, launches_per_step):
        per_kind.setdefault(kind, []).append(ms)
    split = {kd.KERNEL_NAMES[k]: round(sum(v), 4) for k, v in sorted(per_kind.items())}
    dom = max(per_kind, key=lambda k: sum(per_kind[k]))
    log(f"per-kernel ms in one step: {split}; dominant {kd.KERNEL_NAMES[dom]}")

    # Timed region: K steps between full synchronisations of both runtimes;
    # the dominant kernel's launches are bracketed by events on the stream.
    cap = n_chunks * args.steps
    starts = [hip.Event() for _ in range(cap)]
    ends = [hip.Event() for _ in range(cap)]
    arr_s = (ctypes.c_void_p * cap)(*[e.value for e in starts])
    arr_e = (ctypes.c_void_p * cap)(*[e.value for e in ends])
    kinds = (ctypes.c_int32 * cap)()
    count = ctypes.c_int32(0)
    kd.kd_set_launch_log(1 << dom, arr_s, arr_e, kinds, cap, ctypes.byref(count))
    step_ev = [hip.Event() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    hip.synchronize()
    log(f"timing {args.steps} step(s)")
    t_start = time.perf_counter()
    for i in range(args.steps):
        step_ev[i].record(stream.value)
        step()
    step_ev[args.steps].record(stream.value)
    stream.synchronize()
    t_end = time.perf_counter()
    torch.cuda.synchronize()
    kd.kd_set_launch_log(0, None, None, None, 0, None)
    wall = t_end - t_start
    ms_step = wall * 1e3 / args.steps
    dom_ms = [starts[i].elapsed_ms(ends[i]) for i in range(count.value)]
    dom_avg = sum(dom_ms) / len(dom_ms)
    per_step = sorted(step_ev[i].elapsed_ms(step_ev[i + 1]) for i in range(args.steps))
    # device memory in use around one more call: the library allocates nothing
    hip.synchronize()
    free0, total = hip.mem_get_info()
    step()
    stream.synchronize()
    free1, _ = hip.mem_get_info()

    flops_step = (2.0 if args.op == "fwd" else 6.0) * T * d * V
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    tokens_s = T * args.steps / wall
    # Each of the three GEMMs does 2 T d V flops per step in all; per launch
    # that is the step's share per launch of the kernel (the dW GEMM runs
    # once per group of slices, and a ragged last slice is smaller).
    dom_per_step = len(dom_ms) / args.steps
    flops_launch = 2.0 * T * d * V / dom_per_step if dom in GEMM_KERNELS else None
    if flops_launch is not None:
        ach = flops_launch / (dom_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kd.KERNEL_NAMES[dom],
                "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_for(kd.KERNEL_NAMES[dom], config_key(args)),
                "launch_ms": round(dom_avg, 4), "launches": len(dom_ms),
                "flops_per_launch": flops_launch}
    else:
        roof = {"bound": "hbm", "kernel": kd.KERNEL_NAMES[dom], "achieved": None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": None,
                "traffic": None, "launch_ms": round(dom_avg, 4)}

    lval = float(loss.item()) if args.op != "bwd" else None
    metric = {"loss": METRIC,
              "fwd": METRIC.replace("fwd+bwd", "forward only (kd_topk_kl_fwd)"),
              "bwd": METRIC.replace("fwd+bwd", "backward with logits recomputed "
                                    "(kd_topk_kl_bwd)")}[args.op]
    out = {
        "metric": metric, "value": round(tokens_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": x.dtype,
        "data": "synthetic",
        "config": {"workload": x.name, "T": T, "d": d, "V": V, "K": K,
                   "tau": x.tau, "chunk": chunk,
                   "masked": 0 if x.mask is None else int(T - x.mask.sum()),
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
        "extra_hbm_bytes": ws_bytes,
        "dense_extra_hbm_bytes": 8 * T * V,
        "hbm": {"workspace_bytes": ws_bytes,
                "device_used_delta_during_call_bytes": int(free0 - free1),
                "device_total_bytes": int(total)},
        "step_ms": {"median": round(per_step[len(per_step) // 2], 3),
                    "min": round(per_step[0], 3)},
        "peak_from_device": peak_from_device(hip),
        "loss": lval,
        "kernel_ms_one_step": split,
        "roofline": roof,
    }
    if args.op == "loss" and args.sweep:
        out["chunk_sweep"] = chunk_sweep(
            lib, (H, W, idx, lg, mptr, dt_code), x, ws, stream,
            [int(c) for c in args.sweep.split(",")])
    if not args.no_cpu_baseline and args.op == "loss":
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def chunk_sweep(lib, inputs, x, ws, stream, chunks, steps=3):
    """kd_topk_kl_fwd_bwd at other slice sizes on the same inputs: per slice
    size, one warm-up call and `steps` timed calls (HIP events on the call's
    stream), the workspace it needs and the loss (equal for every size)."""
    import torch
    import top_kl_loss_amd as kd
    from top_kl_loss_amd import hip
    H, W, idx, lg, mptr, dt_code = inputs
    T, d, V, K = x.T, x.d, x.V, x.K
    f32 = dict(dtype=torch.float32, device=H.device)
    loss, dH, dW = torch.empty(1, **f32), torch.empty(T, d, **f32), torch.empty(V, d, **f32)
    res = []
    for c in chunks:
        need = kd.kd_topk_kl_workspace_size(T, d, V, K, c, dt_code)
        buf = ws if need <= ws.numel() else torch.empty(need, dtype=torch.uint8,
                                                        device=H.device)

        def call():
            st = lib.kd_topk_kl_fwd_bwd(
                H.data_ptr(), W.data_ptr(), dt_code, idx.data_ptr(), lg.data_ptr(),
                mptr, T, d, V, K, float(x.tau), c, 0, loss.data_ptr(), None,
                dH.data_ptr(), dW.data_ptr(), buf.data_ptr(), need, stream.value)
            if st != 0:
                raise RuntimeError(kd.kd_status_string(st))

        call()
        ev = [hip.Event() for _ in range(steps + 1)]
        for i in range(steps):
            ev[i].record(stream.value)
            call()
        ev[steps].record(stream.value)
        stream.synchronize()
        ms = sorted(ev[i].elapsed_ms(ev[i + 1]) for i in range(steps))
        med = ms[len(ms) // 2]
        res.append({"chunk": c, "ms_per_step": round(med, 3),
                    "tokens_per_s": round(T / (med * 1e-3), 1),
                    "tflops": round(6.0 * T * d * V / (med * 1e-3) / 1e12, 2),
                    "workspace_bytes": need, "loss": float(loss.item())})
        log(f"chunk {c}: {med:.2f} ms per step, workspace {need / 1e9:.2f} GB")
        del buf
    return res


TEACHER_METRIC = ("tokens/s & TFLOP/s teacher top-100 cache build (LM-head GEMM + "
                  "per-row top-K), T=32k V=201k; % bf16 MFMA peak")
TK_KINDS = {11: "tk_sample", 12: "tk_theta", 13: "tk_filter", 14: "tk_select",
            15: "tk_stream"}


def cpu_baseline_teacher(x, K, target_s):
    """The teacher-cache oracle, as it stands, on the first R rows."""
    from oracle import teacher_topk as tko
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) \
            if threadpool_info() else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))

    def run(R):
        t0 = time.perf_counter()
        tko.teacher_topk_cache(x.H[:R], x.W, K)
        return time.perf_counter() - t0

    t4 = run(4)
    t16 = run(16)
    per = max((t16 - t4) / 12, 1e-6)
    fixed = max(t4 - 4 * per, 0.0)
    R = int(max(16, min(x.T, 4096, (target_s - fixed) / per)))
    log(f"cpu baseline: teacher oracle on {R} rows (~{fixed + per * R:.0f} s)")
    dt = run(R)
    model, affinity = cpu_info()
    return {"value": R / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "affinity_cpus": affinity,
            "sample": f"first {R} of {x.T} rows of {x.name} (full d={x.d}, "
                      f"V={x.V}, K={K}), fp64 NumPy matmul + per-row "
                      f"lexsort; {dt:.1f} s wall"}


def bench_teacher(args):
    """One step = one kd_teacher_topk call over T = 32768 rows of a random
    bf16 teacher (d = 2880, V = 201088, K = 100): the cache the loss reads."""
    import numpy as np
    import torch

    import synth
    import top_kl_loss_amd as kd
    from top_kl_loss_amd import hip

    torch.cuda.init()
    lib = kd.load_library()
    spec = synth.WORKLOADS[args.workload]
    T, d, V, K = spec["T"], spec["d"], spec["V"], spec["K"]
    chunk = args.chunk or 4096
    log(f"generating teacher head for {args.workload}: T={T} d={d} V={V}")
    t0 = time.perf_counter()
    x = synth.teacher_head(f"{args.workload}_teacher", case=spec["case"], T=T,
                           d=d, V=V, dtype=synth.BF16)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; K={K} chunk={chunk}")
    dev = torch.device("cuda:0")
    H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    ws_bytes = kd.kd_teacher_topk_workspace_size(T, d, V, K, chunk, kd.KD_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ids = torch.empty(T, K, dtype=torch.int32, device=dev)
    vals = torch.empty(T, K, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    hip.set_device(0)
    stream = hip.Stream()

    def step():
        st = lib.kd_teacher_topk(H.data_ptr(), W.data_ptr(), kd.KD_BF16, T, d,
                                 V, K, chunk, ids.data_ptr(), vals.data_ptr(),
                                 ws.data_ptr(), ws_bytes, stream.value)
        if st != 0:
            raise RuntimeError(kd.kd_status_string(st))

    n_chunks = (T + chunk - 1) // chunk
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 x {args.copy_calibration} bytes")
    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step()
    stream.synchronize()

    def logged(mask_bits, n_steps, cap):
        starts = [hip.Event() for _ in range(cap)]
        ends = [hip.Event() for _ in range(cap)]
        arr_s = (ctypes.c_void_p * cap)(*[e.value for e in starts])
        arr_e = (ctypes.c_void_p * cap)(*[e.value for e in ends])
        kinds = (ctypes.c_int32 * cap)()
        count = ctypes.c_int32(0)
        kd.kd_set_launch_log(mask_bits, arr_s, arr_e, kinds, cap,
                             ctypes.byref(count))
        # the library reads arr_s / arr_e at every logged launch: the caller
        # keeps them alive until the log is removed
        return starts, ends, kinds, count, (arr_s, arr_e)

    # one logged step over every kernel: the time split and the dominant one
    s_, e_, k_, c_, keep = logged(0x1F << 11, 1, 5 * n_chunks)
    step()
    stream.synchronize()
    kd.kd_set_launch_log(0, None, None, None, 0, None)
    per_kind = {}
    for i in range(c_.value):
        per_kind.setdefault(k_[i], []).append(s_[i].elapsed_ms(e_[i]))
    split = {TK_KINDS[k]: round(sum(v), 4) for k, v in sorted(per_kind.items())}
    dom = max(per_kind, key=lambda k: sum(per_kind[k]))
    log(f"per-kernel ms in one step: {split}; dominant {TK_KINDS[dom]}")

    del keep
    starts, ends, kinds, count, keep = logged(1 << dom, args.steps,
                                              n_chunks * args.steps)
    torch.cuda.synchronize()
    hip.synchronize()
    log(f"timing {args.steps} step(s)")
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    stream.synchronize()
    t_end = time.perf_counter()
    kd.kd_set_launch_log(0, None, None, None, 0, None)
    del keep
    wall = t_end - t_start
    ms_step = wall * 1e3 / args.steps
    dom_ms = [starts[i].elapsed_ms(ends[i]) for i in range(count.value)]
    dom_avg = sum(dom_ms) / len(dom_ms)
    tflops = 2.0 * T * d * V / (ms_step * 1e-3) / 1e12

    # algorithmic work of the dominant kernel per launch
    nseg = (V + 255) // 256
    # the library's sampled-segment count: about K nseg / ns <= 4096
    # candidates expected per row, ns in [32, 128], at most nseg
    ns = min(max(-(-K * nseg // 4096), 32), 128, nseg)
    stride = 1 if ns == nseg else nseg // ns
    cols = {11: ns * 256, 13: (nseg - ns) * 256}.get(dom)
    if cols is not None:
        flops_launch = 2.0 * chunk * d * cols
        ach = flops_launch / (dom_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": TK_KINDS[dom], "achieved": round(ach, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_for(TK_KINDS[dom], config_key(args)),
                "launch_ms": round(dom_avg, 4), "launches": len(dom_ms),
                "flops_per_launch": flops_launch}
    else:
        roof = {"bound": "hbm", "kernel": TK_KINDS[dom], "achieved": None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": None,
                "traffic": None, "launch_ms": round(dom_avg, 4)}
    got = ids.cpu().numpy()
    assert np.all((got >= 0) & (got < V)), "ids out of range"
    out = {
        "metric": TEACHER_METRIC, "value": round(T * args.steps / wall, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": x.name, "T": T, "d": d, "V": V, "K": K,
                   "chunk": chunk, "sampled_segments": ns,
                   "sample_stride": stride, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
        "extra_hbm_bytes": ws_bytes,
        "dense_logits_bytes": 4 * T * V,
        "kernel_ms_one_step": split,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_teacher(x, K, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_filter(args):
    """One step = one kd_entropy_filter call (top-fraction mode, 70%) over
    the workload's teacher cache: T rows of K fp32 logits."""
    import numpy as np
    import torch

    import synth
    import top_kl_loss_amd as kd
    from top_kl_loss_amd import hip

    torch.cuda.init()
    lib = kd.load_library()
    x = synth.workload(args.workload, teacher_device="cuda")
    T, K = x.T, x.K
    dev = torch.device("cuda:0")
    lg = torch.from_numpy(x.topk_logit).to(dev)
    mask = None if x.mask is None else torch.from_numpy(x.mask).to(dev)
    ws_bytes = kd.kd_entropy_filter_workspace_size(T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(T, dtype=torch.uint8, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    hip.set_device(0)
    stream = hip.Stream()

    def step():
        st = lib.kd_entropy_filter(lg.data_ptr(),
                                   None if mask is None else mask.data_ptr(),
                                   T, K, float(x.tau), 1, 0.7, out.data_ptr(),
                                   ent.data_ptr(), ws.data_ptr(), ws_bytes,
                                   stream.value)
        if st != 0:
            raise RuntimeError(kd.kd_status_string(st))

    for _ in range(args.warmup):
        step()
    stream.synchronize()
    starts = [hip.Event() for _ in range(args.steps)]
    ends = [hip.Event() for _ in range(args.steps)]
    arr_s = (ctypes.c_void_p * args.steps)(*[e.value for e in starts])
    arr_e = (ctypes.c_void_p * args.steps)(*[e.value for e in ends])
    count = ctypes.c_int32(0)
    kd.kd_set_launch_log(1 << 17, arr_s, arr_e, None, args.steps, ctypes.byref(count))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    stream.synchronize()
    wall = time.perf_counter() - t0
    kd.kd_set_launch_log(0, None, None, None, 0, None)
    call_ms = [starts[i].elapsed_ms(ends[i]) for i in range(count.value)]
    avg = sum(call_ms) / len(call_ms)
    # algorithmic bytes: read the logits and the mask, write entropy and mask
    nbytes = T * K * 4 + 2 * T + 4 * T
    gbs = nbytes / (avg * 1e-3) / 1e9
    kept = int(out.sum().item())
    print(json.dumps({
        "metric": "tokens/s entropy token filter (top 70% by teacher entropy) "
                  "over the top-100 cache",
        "value": round(T * args.steps / wall, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": x.name, "T": T, "K": K, "tau": x.tau,
                   "mode": "top_fraction", "fraction": 0.7, "kept": kept},
        "roofline": {"bound": "hbm", "kernel": "entropy_filter (3 launches)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5),
                     "traffic": None, "launch_ms": round(avg, 4)},
    }), flush=True)


def cpu_baseline_div(x, kind, target_s):
    """The divergence oracle, as it stands, on the first R tokens."""
    from oracle import kd_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) \
            if threadpool_info() else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))

    def run(R):
        m = None if x.mask is None else x.mask[:R]
        t0 = time.perf_counter()
        orc.topk_divergence(x.H[:R], x.W, x.topk_idx[:R], x.topk_logit[:R], m,
                            x.tau, kind)
        return time.perf_counter() - t0

    t8 = run(8)
    t32 = run(32)
    per = max((t32 - t8) / 24, 1e-6)
    fixed = max(t8 - 8 * per, 0.0)
    R = int(max(32, min(x.T, 2048, (target_s - fixed) / per)))
    log(f"cpu baseline: divergence oracle on {R} tokens (~{fixed + per * R:.0f} s)")
    dt = run(R)
    model, affinity = cpu_info()
    return {"value": R / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "affinity_cpus": affinity,
            "sample": f"first {R} of {x.T} tokens of {x.name} (full d={x.d}, "
                      f"V={x.V}, K={x.K}), fp64 NumPy (dense logits); "
                      f"{dt:.1f} s wall"}


def bench_div(args):
    """One step = one kd_topk_div_fwd_bwd call (reverse KL or JSD over the
    top-K support: loss, dH and dW) over the workload's whole batch."""
    import numpy as np
    import torch

    import synth
    import top_kl_loss_amd as kd
    from top_kl_loss_amd import hip

    torch.cuda.init()
    lib = kd.load_library()
    x = synth.workload(args.workload, teacher_device="cuda")
    T, d, V, K = x.T, x.d, x.V, x.K
    dev = torch.device("cuda:0")
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        W = torch.from_numpy(x.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        dt_code, esize = kd.KD_BF16, 2
    else:
        H = torch.from_numpy(x.H).to(dev)
        W = torch.from_numpy(x.W).to(dev)
        dt_code, esize = kd.KD_F32, 4
    idx = torch.from_numpy(x.topk_idx).to(dev)
    lg = torch.from_numpy(x.topk_logit).to(dev)
    mask = None if x.mask is None else torch.from_numpy(x.mask).to(dev)
    ws_bytes = kd.kd_topk_div_workspace_size(T, d, V, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss, rl = torch.empty(1, **f32), torch.empty(T, **f32)
    dH, dW = torch.empty(T, d, **f32), torch.empty(V, d, **f32)
    code = kd.DIVERGENCES[args.op]
    torch.cuda.synchronize()
    stream = hip.Stream()

    def step():
        st = lib.kd_topk_div_fwd_bwd(
            code, H.data_ptr(), W.data_ptr(), dt_code, idx.data_ptr(), lg.data_ptr(),
            None if mask is None else mask.data_ptr(), T, d, V, K, float(x.tau), 0,
            loss.data_ptr(), rl.data_ptr(), dH.data_ptr(), dW.data_ptr(),
            ws.data_ptr(), ws_bytes, stream.value)
        if st != 0:
            raise RuntimeError(kd.kd_status_string(st))

    for _ in range(args.warmup):
        step()
    stream.synchronize()
    cap = args.steps
    starts = [hip.Event() for _ in range(cap)]
    ends = [hip.Event() for _ in range(cap)]
    arr_s = (ctypes.c_void_p * cap)(*[e.value for e in starts])
    arr_e = (ctypes.c_void_p * cap)(*[e.value for e in ends])
    count = ctypes.c_int32(0)
    kd.kd_set_launch_log(1 << 18, arr_s, arr_e, None, cap, ctypes.byref(count))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    stream.synchronize()
    wall = time.perf_counter() - t0
    kd.kd_set_launch_log(0, None, None, None, 0, None)
    call_ms = [starts[i].elapsed_ms(ends[i]) for i in range(count.value)]
    avg = sum(call_ms) / len(call_ms)
    # algorithmic bytes: H, W and the cache read once, dH and dW written once
    nbytes = (T + V) * d * esize + T * K * 8 + (T + V) * d * 4
    gathered = 3 * T * K * d * esize
    gbs = nbytes / (avg * 1e-3) / 1e9
    metric = (f"tokens/s {'reverse KL' if args.op == 'reverse_kl' else 'Jensen-Shannon'} "
              f"over the top-{K} support, fwd+bwd (kd_topk_div_fwd_bwd)")
    out = {
        "metric": metric, "value": round(T * args.steps / wall, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": x.dtype, "data": "synthetic",
        "config": {"workload": x.name, "T": T, "d": d, "V": V, "K": K, "tau": x.tau,
                   "masked": 0 if x.mask is None else int(T - x.mask.sum()),
                   "parallelism": "single GPU"},
        "loss": float(loss.item()),
        "extra_hbm_bytes": ws_bytes,
        "roofline": {"bound": "hbm", "kernel": "divergence (all kernels of the call)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "launch_ms": round(avg, 4), "algorithmic_bytes": nbytes,
                     "gathered_row_bytes": gathered},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_div(x, args.op, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
