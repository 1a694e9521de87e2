#!/usr/bin/env python3
"""Throughput of the fused W4A4 + rank-r linear layer on one MI355X.

A step is one call of the whole layer (quantization pass + residual
contraction with the rank-r epilogue) over one batch of synthetic,
seeded inputs already resident in HBM.  Successive steps rotate through
enough copies of the inputs and outputs (> 512 MB) that the 256 MB
Infinity Cache cannot serve them warm.

The timed steps run as a captured HIP graph (no host launch gaps between
kernels); the per-kernel durations come from graphs of back-to-back
launches of each stage, timed with events on their stream.

Prints one JSON line.  ``value`` is the effective TOPS of the whole call,
2*M*N*K*batch / time.  ``roofline`` covers the dominant kernel (the
contraction).  ``cpu_baseline`` times the CPU oracle on the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS of fused W4A4+rank-4 linear; % of int8 MFMA / HBM roofline"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, 2.5 PFLOP/s
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4 / fp6 MFMA, 10.1 PFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "tiled": os.path.join(ROOT, "w4a4_rank_assisted_amd", "csrc", "gemm_tiled.hip"),
    "skinny": os.path.join(ROOT, "w4a4_rank_assisted_amd", "csrc", "gemm_skinny.hip"),
}


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(M, K, N, r, batch, y_bytes, group=64):
    """Minimum bytes the whole layer must move (inputs once, output once)."""
    G = K // group
    x = M * K * 2 + K * 2 + batch * (K * r * 2)
    w = batch * (K * N // 2 + G * N * 2 + r * N * 2 + N * 2)
    y = batch * M * N * y_bytes
    return x + w + y


def contract_bytes(M, K, N, r, batch, y_bytes, group=64):
    """Minimum bytes of the contraction stage: int4 activation codes and
    their fp16 scales, U, the packed weights with their scales, L2, bias, Y."""
    G = K // group
    a = M * K // 2 + M * G * 2 + batch * M * r * 4
    w = batch * (K * N // 2 + G * N * 2 + r * N * 2 + N * 2)
    return a + w + batch * M * N * y_bytes


def traffic_key(layer: str, tokens, M: int, group: int) -> str:
    """Entry name of a layer in the traffic file."""
    key = layer if tokens is None else f"{layer}_M{M}"
    return key if group == 64 else f"{key}_g{group}"


def read_traffic(kernel: str, layer: str):
    """HBM bytes per launch measured by rocprofv3 counters, if they were
    taken on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(layer, {}).get(kernel)
    if not ent or ent.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return ent.get("bytes_per_launch")


def _sample_rows(M: int, n: int):
    """n rows spread evenly over [0, M), always including the first and last."""
    import numpy as np

    n = max(2, min(n, M))
    return np.unique(np.linspace(0, M - 1, n).round().astype(np.int32))


def cpu_baseline(layers, specs, seconds: float, rows_per_layer: int):
    """The CPU oracle, as it stands, on a bounded sample of the workload:
    the same evenly spaced rows of every layer (all output columns, every
    projection), repeated until `seconds` of wall time have accumulated.
    Rows are independent (the quantizer is per token), so the sample's rate
    is the oracle's rate on the whole workload."""
    import oracle

    o = oracle.Oracle()
    picks = [_sample_rows(sp.M, rows_per_layer) for sp in specs]
    reps, ops, t0 = 0, 0, time.perf_counter()
    while True:
        for lay, sp, rows in zip(layers, specs, picks):
            o.linear_batched(lay, rows=rows)
            ops += 2 * rows.size * sp.K * sp.N * sp.batch
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 20:
            break
    sample = "; ".join(f"{rows.size} of {sp.M} rows of {sp.name} ({sp.K}->{sp.N}, batch {sp.batch})"
                       for sp, rows in zip(specs, picks))
    out = {
        "value": round(ops / el / 1e12, 6),
        "unit": "TOPS",
        "cores": o.num_threads(),
        "kind": "oracle",
        "sample": (f"{sample}: quantize + brute-force int32 group sums + fp64 output, "
                   f"{reps} repetition(s), {el:.1f} s"),
    }
    return out


def cpu_single_thread_tiny(seconds: float = 2.0):
    """Seconds per call of the oracle on one thread for the tiny smoke layer
    (64 x 256 -> 256), the whole layer."""
    import oracle
    from synth import make_layer

    o = oracle.Oracle()
    lay = make_layer("tiny")
    threads = o.num_threads()
    o.set_num_threads(1)
    try:
        reps, t0 = 0, time.perf_counter()
        while True:
            o.linear_batched(lay)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        o.set_num_threads(threads)
    return {"layer": "tiny 64x256->256", "threads": 1, "s_per_call": round(el / reps, 6)}


# hipDeviceAttribute_t values (hip_runtime_api.h, ROCm 7): peak engine clock
# in kHz, LDS bytes per compute unit
_HIP_ATTR_CLOCK_KHZ = 5
_HIP_ATTR_LDS_PER_CU = 10002


def _hip_attributes(dev: int = 0):
    """Peak clock and LDS size from the HIP runtime already in the process
    (found through /proc/self/maps; None where it cannot be read)."""
    import ctypes

    path = None
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
    except OSError:
        pass
    if path is None:
        return None, None
    hip = ctypes.CDLL(path)
    vals = []
    for attr in (_HIP_ATTR_CLOCK_KHZ, _HIP_ATTR_LDS_PER_CU):
        v = ctypes.c_int(0)
        ok = hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) == 0
        vals.append(v.value if ok else None)
    return vals[0], vals[1]


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    clock_khz, lds = _hip_attributes(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1), "hip": torch.version.hip,
            "peak_clock_mhz": None if clock_khz is None else clock_khz / 1000.0,
            "lds_bytes_per_cu": lds}


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def summarize_profiles(args):
    """Summaries of rocprofv3 output directories (csv output format).

    A directory with a kernel-trace ``*_kernel_stats.csv`` gives per-kernel
    launch counts and average durations.  Directories with
    ``*_counter_collection.csv`` give per-dispatch counter averages; when
    both FETCH_SIZE and WRITE_SIZE appear (separate passes over the same
    command) together with the reference copy (``--copy-mb``), the
    contraction's HBM bytes per launch are scaled by what the counters read
    for the copy, whose true traffic is known (read + write of its size).
    With --write-traffic the result goes into profiles/traffic.json, keyed by
    layer and kernel, together with the hash of the kernel source it was
    measured on."""
    out = []
    counters = {}
    copy = {}
    meta = {}
    for d in args.summarize:
        ks = _find(d, "kernel_stats.csv")
        if ks:
            out.append(f"kernel stats ({d}):")
            out.append(f"  {'kernel':70s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}")
            for r in sorted(_csv_rows(ks), key=lambda r: -float(r["TotalDurationNs"])):
                out.append(f"  {r['Name'][:70]:70s} {int(r['Calls']):6d} "
                           f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                           f"{float(r['MaxNs']) / 1e3:10.2f}")
        cc = _find(d, "counter_collection.csv")
        if cc:
            per = {}
            for r in _csv_rows(cc):
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
                per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            byname = {}
            for (did, name), vals in sorted(per.items(), key=lambda kv: int(kv[0][0])):
                for c, v in vals.items():
                    byname.setdefault(name, {}).setdefault(c, []).append(v)
            out.append(f"counters ({d}), average per dispatch:")
            for name, cs in sorted(byname.items()):
                short = name[:70]
                txt = ", ".join(f"{c} {sum(v) / len(v):.6g} (n={len(v)})" for c, v in cs.items())
                out.append(f"  {short:70s} {txt}")
                for c, v in cs.items():
                    if "copyBuffer" in name:
                        # the reference copies are the last three copies of the run
                        copy[c] = sum(v[-3:]) / len(v[-3:])
                    elif "k_gemm" in name:
                        # skip the first launches (warm-up, graph upload)
                        vv = v[2:] if len(v) > 4 else v
                        counters.setdefault(name, {})[c] = sum(vv) / len(vv)
    text = "\n".join(out)
    print(text)
    if copy and counters:
        log = [l for l in out]
        res = {}
        for name, cs in counters.items():
            if "FETCH_SIZE" not in cs or "WRITE_SIZE" not in cs:
                continue
            kern = "skinny" if "skinny" in name else "tiled"
            res[kern] = cs
        if res and "FETCH_SIZE" in copy and "WRITE_SIZE" in copy and args.copy_mb > 0:
            nb = int(args.copy_mb * 1e6) // 16 * 16
            f_fac = (nb / 1024) / copy["FETCH_SIZE"]      # true KiB read per counted KiB
            w_fac = (nb / 1024) / copy["WRITE_SIZE"]
            layer = traffic_key(args.layer, args.tokens, args.tokens, args.group)
            print(f"copy calibration: {args.copy_mb} MB; FETCH_SIZE factor {f_fac:.4f}, "
                  f"WRITE_SIZE factor {w_fac:.4f}")
            if args.write_traffic:
                try:
                    with open(TRAFFIC_FILE) as f:
                        rec = json.load(f)
                except (OSError, ValueError):
                    rec = {}
                for kern, cs in res.items():
                    fetch = cs["FETCH_SIZE"] * 1024 * f_fac
                    write = cs["WRITE_SIZE"] * 1024 * w_fac
                    rec.setdefault(layer, {})[kern] = {
                        "bytes_per_launch": int(fetch + write),
                        "fetch_bytes": int(fetch), "write_bytes": int(write),
                        "fetch_kib_counted": round(cs["FETCH_SIZE"], 1),
                        "write_kib_counted": round(cs["WRITE_SIZE"], 1),
                        "copy_factor_fetch": round(f_fac, 4), "copy_factor_write": round(w_fac, 4),
                        "source_sha256_16": source_hash(KERNEL_SOURCES[kern]),
                    }
                    print(f"{layer} {kern}: {int(fetch + write)} bytes per launch "
                          f"(fetch {int(fetch)}, write {int(write)})")
                with open(TRAFFIC_FILE, "w") as f:
                    json.dump(rec, f, indent=1, sort_keys=True)
                    f.write("\n")
    return 0


PROBE_LIB = os.path.join(ROOT, "w4a4_rank_assisted_amd", "_lib", "libhsq_probe.so")
PROBE_MODES = {0: "mfma_only", 1: "mfma_plus_1_fma_per_element", 2: "mfma_plus_2_fma_per_element",
               3: "mfma_plus_2_fma_plus_lds_reads", 4: "wide_tile_mfma_plus_2_fma",
               5: "wide_tile_mfma_plus_2_fma_plus_lds_reads"}


def _probe_lib():
    """libhsq_probe (measurement kernels), loaded after torch so that it binds
    to torch's HIP runtime."""
    import ctypes

    import torch  # noqa: F401

    if not os.path.exists(PROBE_LIB):
        raise OSError(f"{PROBE_LIB} is missing; build it with w4a4_rank_assisted_amd.build.build()")
    lib = ctypes.CDLL(PROBE_LIB)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.hsq_probe_mfma.argtypes = [I, I, I, I, P, P]
    lib.hsq_probe_read.argtypes = [P, S, I, P, P]
    lib.hsq_probe_copy.argtypes = [P, S, I, P, P]
    for f in (lib.hsq_probe_mfma, lib.hsq_probe_read, lib.hsq_probe_copy):
        f.restype = I
    return lib


def _time_graph(torch, launch, reps: int):
    """Milliseconds per launch: `reps` launches captured in one HIP graph,
    replayed between events on the capture stream (after one untimed
    replay); the median of three timed replays."""
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        launch(cap)                          # eager warm-up
        with torch.cuda.graph(g, stream=cap):
            for i in range(reps):
                launch(cap, i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(cap):
            t0.record(cap)
            g.replay()
            t1.record(cap)
        torch.cuda.synchronize()
        ts.append(t0.elapsed_time(t1) / reps)
    return sorted(ts)[1]


def measure_peaks(torch, full: bool = False):
    """Measured ceilings of this GPU (libhsq_probe): the int8 MFMA rate with
    the tiled contraction's wave tile and occupancy (512 workgroups of 8
    waves, 4 waves per SIMD), alone and with the contraction's per-element
    rescale work (and, with `full`, its LDS reads, and more occupancies);
    HBM read and copy rates of 16-byte loads over 1 GiB and over 27 MB
    buffers rotated through 540 MB (the size of a 16-token layer's weight
    stream, past the 256 MB MALL)."""
    import ctypes

    lib = _probe_lib()
    dev = torch.device("cuda:0")
    blocks, waves, iters = 512, 8, 2000
    sink = torch.empty(1024 * 64 * 16, dtype=torch.int32, device=dev)
    res = {"int8_mfma_tops": {}, "hbm_gbs": {}}
    configs = [(0, blocks, waves), (2, blocks, waves)]
    if full:
        configs = ([(m, blocks, waves) for m in (0, 1, 2, 3)] + [(0, 256, 4), (0, 256, 8), (0, 512, 16)] +
                   [(4, 256, 8), (5, 256, 8), (4, 512, 8), (5, 512, 8)])
    for mode, nb, nw in configs:
        def launch(stream, i=0, mode=mode, nb=nb, nw=nw):
            assert lib.hsq_probe_mfma(mode, iters, nb, nw, ctypes.c_void_p(sink.data_ptr()),
                                      ctypes.c_void_p(stream.cuda_stream)) == 0
        ms = _time_graph(torch, launch, 5)
        ops = nb * nw * iters * (16 if mode >= 4 else 8) * 2 * 16 * 16 * 64
        key = PROBE_MODES[mode] + ("" if (nb, nw) == (blocks, waves) and mode < 4 else f"_{nb}x{nw}waves")
        res["int8_mfma_tops"][key] = round(ops / (ms * 1e-3) / 1e12, 1)
    sblocks = 256 * 8
    big = 1 << 30
    src = torch.empty(big, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty(big, dtype=torch.uint8, device=dev)
    for kind, fn in (("read", lib.hsq_probe_read), ("copy", lib.hsq_probe_copy)):
        out = sink if kind == "read" else dst

        def launch_big(stream, i=0, fn=fn, out=out):
            assert fn(ctypes.c_void_p(src.data_ptr()), big, sblocks, ctypes.c_void_p(out.data_ptr()),
                      ctypes.c_void_p(stream.cuda_stream)) == 0
        ms = _time_graph(torch, launch_big, 3)
        res["hbm_gbs"][f"{kind}_1GiB"] = round(big * (1 if kind == "read" else 2) / (ms * 1e-3) / 1e9, 1)
        small, nbuf = 27 * 1000 * 1000 // 16 * 16, 20

        def launch_small(stream, i=0, fn=fn, out=out):
            off = (i % nbuf) * small
            o = out.data_ptr() + (0 if kind == "read" else off)
            assert fn(ctypes.c_void_p(src.data_ptr() + off), small, sblocks, ctypes.c_void_p(o),
                      ctypes.c_void_p(stream.cuda_stream)) == 0
        ms = _time_graph(torch, launch_small, nbuf)
        res["hbm_gbs"][f"{kind}_27MB_rotated"] = round(small * (1 if kind == "read" else 2) / (ms * 1e-3) / 1e9, 1)
    del src, dst
    return res


def probe_main(args):
    """The measured ceilings of this GPU as one JSON line (bench.py --probe)."""
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; use --gpus 1", file=sys.stderr)
        return 2
    import torch

    res = measure_peaks(torch, full=True)
    mf = res["int8_mfma_tops"]
    out = {
        "metric": "measured ceilings of the MI355X for the W4A4 contraction",
        "int8_mfma_tops": mf,
        "int8_mfma_frac_of_spec": {k: round(v / PEAK_INT8_TOPS, 4) for k, v in mf.items()},
        "hbm_gbs": res["hbm_gbs"],
        "hbm_frac_of_spec": {k: round(v / PEAK_HBM_GBS, 4) for k, v in res["hbm_gbs"].items()},
        "notes": ("MFMA probe: 512 workgroups x 8 waves (4 waves per SIMD) unless named, each wave the "
                  "tiled contraction's 4 x 2 tiles of v_mfma_i32_16x16x64_i8 per step with register "
                  "operands; the rescale modes add 1 or 2 fp32 FMAs per MFMA result element on the previous "
                  "step's results, the lds mode also the step's LDS operand reads. HBM: 16-byte "
                  "non-temporal loads (and stores), 2048 workgroups of 256 threads."),
        "device": device_info(torch),
    }
    print(json.dumps(out), flush=True)
    return 0


def calib_cpu_baseline(lay, W, seconds: float):
    """The calibration oracle (NumPy fp64) on the same projection: H, the
    deflation and the closed-form L2, repeated until `seconds` have passed."""
    from oracle import calibration as cal

    L1 = cal.bf16_matrix(lay["L1"][0])
    reps, t0 = 0, time.perf_counter()
    while True:
        H = cal.hessian(lay["X"], lay["lam"])
        cal.deflate(H, L1)
        E = cal.residual_error(W, lay["qw"][0], lay["sw"][0], lay["group"])
        cal.closed_form_l2(H, L1, E)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 20:
            break
    M, K = lay["X"].shape
    N = W.shape[1]
    return {"value": round(el / reps * 1e3, 2), "unit": "ms per calibration step",
            "cores": os.cpu_count(), "kind": "oracle",
            "sample": (f"Hessian of {M} tokens x {K} channels, deflation, closed-form L2 of one "
                       f"{K}x{N} projection, NumPy float64 (threaded BLAS), {reps} repetition(s), "
                       f"{el:.1f} s")}


def calib_main(args):
    """One calibration step of one projection: H = Xh^T Xh over the layer's
    tokens, its deflation by span(L1), and the closed-form L2 from the
    projection's full weight and packed residual.  Each kernel's inputs
    rotate through copies larger than the 256 MB Infinity Cache where they
    are HBM-bound.  Prints one JSON line with a roofline per kernel."""
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; use --gpus 1", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import w4a4_rank_assisted_amd as hsq
    from synth import layer_spec, make_full_weight, make_layer

    dev = torch.device("cuda:0")
    name = WORKLOADS[args.layer][1][0] if args.layer in WORKLOADS else args.layer
    spec = layer_spec(name, args.tokens, args.group)
    lay = make_layer(name, args.tokens, args.group)
    W = make_full_weight(lay, 0)
    M, K, N, r = spec.M, spec.K, spec.N, spec.r

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    X, lam, L1 = d16(lay["X"]), d16(lay["lam"]), d16(lay["L1"][0])
    Wd, sw = d16(W), d16(lay["sw"][0])
    packed = hsq.pack_weights(torch.from_numpy(lay["qw"][0]).to(dev))[0]
    hbytes = K * K * 4
    nh = max(1, math.ceil(args.rotate_mb * 1e6 / (2 * hbytes)))
    Hs = [torch.empty((K, K), dtype=torch.float32, device=dev) for _ in range(nh)]
    Hp = [torch.empty((K, K), dtype=torch.float32, device=dev) for _ in range(nh)]
    wbytes = W.size * 2 + packed.numel()
    nw = max(1, math.ceil(args.rotate_mb * 1e6 / wbytes))
    Ws = [(Wd.clone(), packed.clone()) for _ in range(nw)]
    hws = torch.empty(max(16, hsq._load().hsq_hessian_workspace_bytes(M, K)), dtype=torch.uint8, device=dev)
    dws = torch.empty(hsq._load().hsq_deflate_workspace_bytes(K, r), dtype=torch.uint8, device=dev)
    lws = torch.empty(hsq._load().hsq_closed_form_l2_workspace_bytes(K, N, r), dtype=torch.uint8,
                      device=dev)
    HL1 = torch.empty((K, r), dtype=torch.float32, device=dev)
    Cinv = torch.empty((r, r), dtype=torch.float64, device=dev)
    L2 = torch.empty((r, N), dtype=torch.float32, device=dev)
    lib = hsq._load()

    def stream():
        return hsq._stream()

    def hess(i):
        H = Hs[i % nh]
        assert lib.hsq_hessian_accumulate(X.data_ptr(), M, K, lam.data_ptr(), H.data_ptr(), 0,
                                          hws.data_ptr(), hws.numel(), stream()) == 0

    def defl(i):
        assert lib.hsq_deflate_hessian(Hs[i % nh].data_ptr(), K, L1.data_ptr(), r, Hp[i % nh].data_ptr(),
                                       HL1.data_ptr(), Cinv.data_ptr(), dws.data_ptr(), dws.numel(),
                                       stream()) == 0

    def l2(i):
        w, pk = Ws[i % nw]
        assert lib.hsq_closed_form_l2(HL1.data_ptr(), Cinv.data_ptr(), K, N, r, args.group, w.data_ptr(),
                                      pk.data_ptr(), sw.data_ptr(), L2.data_ptr(), lws.data_ptr(),
                                      lws.numel(), stream()) == 0

    def step(i):
        hess(i)
        defl(i)
        l2(i)

    for i in range(max(args.warmup, nh)):
        step(i)
    torch.cuda.synchronize()
    steps = args.steps
    cap = torch.cuda.Stream()
    graphs = {}
    for name, fn in (("step", step), ("hessian", hess), ("deflate", defl), ("l2", l2)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    fn(args.warmup + i)
        graphs[name] = g
    torch.cuda.synchronize()
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()

    def timed(name):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(cap):
            t0.record(cap)
            graphs[name].replay()
            t1.record(cap)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms = {k: timed(k) for k in ("step", "hessian", "deflate", "l2")}
    # algorithmic work: the symmetric product needs M*K*(K+1) flops (one
    # triangle); the deflation reads H twice (H L1 must be complete before
    # any entry of Hperp) and writes Hperp; the L2 pass reads the bf16
    # weight, the packed codes and their scales once
    hflops = M * K * (K + 1)
    dbytes = 3 * hbytes + 2 * K * r * 2 + K * r * 4
    lbytes = K * N * 2 + K * N // 2 + (K // args.group) * N * 2 + K * r * 4 + r * N * 4
    roofs = {
        "hessian": {"bound": "mfma", "achieved": round(hflops / (ms["hessian"] * 1e-3) / 1e12, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "flops_per_launch": hflops},
        "deflate": {"bound": "hbm", "achieved": round(dbytes / (ms["deflate"] * 1e-3) / 1e9, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "bytes_per_launch": dbytes},
        "l2": {"bound": "hbm", "achieved": round(lbytes / (ms["l2"] * 1e-3) / 1e9, 1),
               "peak": PEAK_HBM_GBS, "unit": "GB/s", "bytes_per_launch": lbytes},
    }
    for k, v in roofs.items():
        v["frac"] = round(v["achieved"] / v["peak"], 4)
        v["ms"] = round(ms[k], 5)
        v["traffic"] = None
    dom = max(roofs, key=lambda k: ms[k])
    out = {
        "metric": "calibration step (Hessian + deflation + closed-form L2) per projection",
        "value": round(ms["step"], 5), "unit": "ms", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms["step"], 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 MFMA / fp32 / fp64",
        "data": "synthetic",
        "config": {"workload": f"{spec.name} calibration: {M} tokens, {K} -> {N}, rank {r}",
                   "M": M, "K": K, "N": N, "rank": r, "group": args.group,
                   "rotated_H": nh, "rotated_W": nw},
        "kernels": roofs,
        "roofline": dict(roofs[dom], kernel=dom),
        "device": device_info(torch),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = calib_cpu_baseline(lay, W, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def mx_main(args):
    """The MX-fp4 variant of one layer (one projection): one step = the whole
    hsq_mx_lowrank_linear call (quantization pass with 1/lambda and the rank
    branch, scaled-fp4 MFMA contraction with the epilogue).  The
    residual is the int4 layer's dequantized residual re-quantized to
    MX-fp4.  Inputs rotate past the Infinity Cache.  The roofline is that
    of the whole call against the fp4 MFMA peak (the quantization pass
    included)."""
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; use --gpus 1", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import w4a4_rank_assisted_amd as hsq
    from synth import layer_spec, make_layer

    dev = torch.device("cuda:0")
    name = WORKLOADS[args.layer][1][0] if args.layer in WORKLOADS else args.layer
    spec = layer_spec(name, args.tokens)
    lay = make_layer(name, args.tokens)
    M, K, N, r = spec.M, spec.K, spec.N, spec.r

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    swf = lay["sw"][0].view(np.float16).astype(np.float32)
    R = (lay["qw"][0].astype(np.float32) * np.repeat(swf, lay["group"], axis=0)).astype(np.float32)
    packed0 = hsq.mx_pack_weights(torch.from_numpy(R).to(dev))
    lam, L1, L2, bias = d16(lay["lam"]), d16(lay["L1"][0]), d16(lay["L2"][0]), d16(lay["bias"][0])
    X0 = d16(lay["X"])
    set_bytes = X0.numel() * 2 + packed0.numel() + M * N * 2
    nsets = max(1, math.ceil(args.rotate_mb * 1e6 / set_bytes))
    sets = [dict(X=X0.clone(), P=packed0.clone(), Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
            for _ in range(nsets)]
    ws = torch.empty(hsq._load().hsq_mx_workspace_bytes(M, K, r), dtype=torch.uint8, device=dev)

    def step(i):
        st = sets[i % nsets]
        hsq.mx_lowrank_linear(st["X"], lam, st["P"], L1, L2, bias, N=N, y_dtype="bf16", out=st["Y"],
                              workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(args.steps):
                step(args.warmup + i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cap):
        t0.record(cap)
        g.replay()
        t1.record(cap)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    ops = 2 * M * N * K
    ach = ops / (ms * 1e-3) / 1e12
    out = {
        "metric": "effective TOPS of the MX-fp4 W4A4+rank-4 linear (scaled fp4 MFMA)",
        "value": round(ach, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4 (e2m1, e8m0 block-32 scales)", "data": "synthetic",
        "config": {"workload": f"{spec.name}: {spec.description} (MX-fp4 residual)", "M": M, "K": K, "N": N,
                   "rank": r, "rotated_sets": nsets},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_FP4_TFLOPS, 4), "traffic": None,
                     "kernel": "whole call (quantization pass + scaled fp4 MFMA contraction)",
                     "ops_per_launch": ops},
        "device": device_info(torch),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def chain_main(args):
    """The FLUX.1 MLP as one fused call (up layer, GELU and the down layer's
    quantization in the up contraction's epilogue, then the down
    contraction) vs the two layers as separate calls (the up layer writing
    bf16 Y, the down layer quantizing it again; no activation pass, so a
    lower bound on the unfused time).  Inputs and outputs rotate past the
    Infinity Cache.  Prints one JSON line."""
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; use --gpus 1", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import w4a4_rank_assisted_amd as hsq
    from synth import make_layer

    dev = torch.device("cuda:0")
    up_l, dn_l = make_layer("flux_up"), make_layer("flux_down")
    M, K = up_l["X"].shape
    H, N = up_l["qw"].shape[2], dn_l["qw"].shape[2]
    r1, r2 = up_l["L1"].shape[2], dn_l["L1"].shape[2]

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def upload(lay):
        return dict(lam=d16(lay["lam"]), packed=hsq.pack_weights(torch.from_numpy(lay["qw"][0]).to(dev))[0],
                    sw=d16(lay["sw"][0]), L1=d16(lay["L1"][0]), L2=d16(lay["L2"][0]), bias=d16(lay["bias"][0]))

    up0, dn0 = upload(up_l), upload(dn_l)
    X0 = d16(up_l["X"])
    set_bytes = X0.numel() * 2 + up0["packed"].numel() + dn0["packed"].numel() + M * N * 2 + M * H * 2
    nsets = max(1, math.ceil(args.rotate_mb * 1e6 / set_bytes))
    sets = []
    for _ in range(nsets):
        up = dict(up0, packed=up0["packed"].clone())
        dn = dict(dn0, packed=dn0["packed"].clone())
        sets.append(dict(X=X0.clone(), up=up, dn=dn, Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                         Yh=torch.empty((1, M, H), dtype=torch.bfloat16, device=dev)))
    wsc = torch.empty(hsq.mlp_workspace_bytes(M, K, H, N, r1, r2), dtype=torch.uint8, device=dev)
    wsu = torch.empty(hsq.workspace_bytes(M, K, H, r1, 1), dtype=torch.uint8, device=dev)
    wsd = torch.empty(hsq.workspace_bytes(M, H, N, r2, 1), dtype=torch.uint8, device=dev)

    def fused(i):
        st = sets[i % nsets]
        hsq.w4a4_lowrank_mlp(st["X"], st["up"], st["dn"], H=H, N=N, act="gelu_tanh", y_dtype="bf16",
                             out=st["Y"], workspace=wsc)

    def separate(i):
        st = sets[i % nsets]
        u, d = st["up"], st["dn"]
        hsq.w4a4_lowrank_linear(st["X"], u["lam"], u["packed"], u["sw"][None], u["L1"][None], u["L2"][None],
                                u["bias"][None], N=H, y_dtype="bf16", out=st["Yh"], workspace=wsu)
        hsq.w4a4_lowrank_linear(st["Yh"][0], d["lam"], d["packed"], d["sw"][None], d["L1"][None],
                                d["L2"][None], d["bias"][None], N=N, y_dtype="bf16", out=st["Y"][None],
                                workspace=wsd)

    for i in range(args.warmup):
        fused(i)
        separate(i)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graphs = {}
    for name, fn in (("fused", fused), ("separate", separate)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(args.steps):
                    fn(args.warmup + i)
        graphs[name] = g
    torch.cuda.synchronize()
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()

    def timed(name):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(cap):
            t0.record(cap)
            graphs[name].replay()
            t1.record(cap)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    ms_f, ms_s = timed("fused"), timed("separate")
    ops = 2 * M * (K * H + H * N)
    ach = ops / (ms_f * 1e-3) / 1e12
    out = {
        "metric": "effective TOPS of the fused W4A4+rank-4 MLP chain (up, GELU, down)",
        "value": round(ach, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_f, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"FLUX.1 MLP: {M} tokens, {K} -> {H} (GELU) -> {N}, rank {r1}/{r2}",
                   "M": M, "K": K, "H": H, "N": N, "rotated_sets": nsets},
        "separate_ms_per_step": round(ms_s, 5),
        "speedup_vs_separate": round(ms_s / ms_f, 4),
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_INT8_TOPS, 4), "traffic": None,
                     "kernel": "whole chain (both contractions dominate)", "ops_per_launch": ops},
        "device": device_info(torch),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layer", default="flux_mlp",
                    help="flux_mlp (FLUX.1 MLP: flux_up then flux_down per step) | tiny | pixart_up | "
                         "sana_qkv | flux_up | flux_down | qwen3_up | qwen3_down")
    ap.add_argument("--tokens", type=int, default=None, help="M for the qwen3 layers (16/256/2048)")
    ap.add_argument("--group", type=int, default=64, choices=[64, 128],
                    help="quantization group width (the pages' Qwen3-8B runs use 128)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "tiled", "skinny"])
    ap.add_argument("--act-quant", default="sym", choices=["sym", "asym"],
                    help="activation format: symmetric int4 (the layer's) or the asymmetric variant")
    ap.add_argument("--y-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--rotate-mb", type=float, default=640.0,
                    help="total bytes of rotated input/output copies (defeats the 256 MB MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-rows", type=int, default=192,
                    help="rows per layer in the CPU oracle's sample (evenly spaced, all columns)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=float, default=0.0,
                    help="after the timed region, run 3 device-to-device copies of this many MB "
                         "(the reference kernel for scaling rocprofv3 byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 output directories instead of running "
                         "(see summarize_profiles)")
    ap.add_argument("--write-traffic", action="store_true",
                    help="with --summarize: record the measured HBM bytes in profiles/traffic.json")
    ap.add_argument("--mx", action="store_true",
                    help="time the MX-fp4 variant of the layer (scaled fp4 MFMA) on --layer")
    ap.add_argument("--chain", action="store_true",
                    help="time the fused two-layer chain (FLUX.1 MLP: flux_up, GELU, flux_down) against "
                         "the two layers run one after the other")
    ap.add_argument("--probe", action="store_true",
                    help="measure this GPU's ceilings (int8 MFMA alone and with the rescale work, HBM "
                         "read and copy) with the kernels of libhsq_probe")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak probes of the default run")
    ap.add_argument("--calib", action="store_true",
                    help="time the calibration kernels (Hessian, deflation, closed-form L2) on the "
                         "layer instead of the inference path")
    args = ap.parse_args(argv)
    if args.summarize:
        return summarize_profiles(args)
    if args.probe:
        return probe_main(args)
    if args.calib:
        return calib_main(args)
    if args.chain:
        return chain_main(args)
    if args.mx:
        return mx_main(args)

    return linear_main(args)


# Workloads made of several layers, each on its own seeded input (layers of a
# block are checked and timed independently; the activation between them is
# not part of the method).  A step runs every layer once.
WORKLOADS = {
    "flux_mlp": ("FLUX.1 joint-token MLP, 4608 tokens (4096 image + 512 text): up-projection "
                 "3072 -> 12288, then down-projection 12288 -> 3072, each layer on its own seeded input",
                 ["flux_up", "flux_down"]),
}


def linear_main(args):
    """One step = the layer(s) of the workload, each as its quantization
    pass + residual contraction with the rank-r epilogue."""
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this layer's hot path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import w4a4_rank_assisted_amd as hsq
    from synth import layer_spec, make_layer

    dev = torch.device("cuda:0")
    if args.layer in WORKLOADS:
        wl_desc, names = WORKLOADS[args.layer]
        wl_name = args.layer
    else:
        names = [args.layer]
        wl_name, wl_desc = args.layer, None
    ydt = torch.bfloat16 if args.y_dtype == "bf16" else torch.float32
    y_bytes = 2 if args.y_dtype == "bf16" else 4

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    # per layer: the seeded tensors on the device, rotated copies of what a
    # step streams (X, packed W, sw, Y: more than the 256 MB MALL in total),
    # and the layer's workspace
    layers = []
    for name in names:
        spec = layer_spec(name, args.tokens, args.group)
        lay = make_layer(name, args.tokens, args.group)
        M, K, N, r, B = spec.M, spec.K, spec.N, spec.r, spec.batch
        X0, sw0 = d16(lay["X"]), d16(lay["sw"])
        packed0 = torch.cat([hsq.pack_weights(torch.from_numpy(lay["qw"][b]).to(dev))[0] for b in range(B)])
        set_bytes = X0.numel() * 2 + packed0.numel() + sw0.numel() * 2 + B * M * N * y_bytes
        nsets = max(1, math.ceil(args.rotate_mb * 1e6 / set_bytes))
        sets = [dict(X=X0.clone(), packed=packed0.clone(), sw=sw0.clone(),
                     Y=torch.empty((B, M, N), dtype=ydt, device=dev)) for _ in range(nsets)]
        del X0, sw0, packed0
        # the stage calls name their contraction kernel; the layer call takes
        # the library's own choice unless one is forced
        kernel = args.kernel
        if kernel == "auto":
            kernel = "skinny" if M <= 64 else "tiled"
        layers.append(dict(
            spec=spec, lay=lay, sets=sets, nsets=nsets, kernel=kernel, call_kernel=args.kernel,
            lam=d16(lay["lam"]), L1=d16(lay["L1"]) if r else None, L2=d16(lay["L2"]) if r else None,
            bias=d16(lay["bias"]),
            ws=torch.empty(hsq.workspace_bytes(M, K, N, r, B, args.group), dtype=torch.uint8, device=dev)))

    def quant(i):
        for L in layers:
            sp = L["spec"]
            hsq.quantize_stage(L["sets"][i % L["nsets"]]["X"], L["lam"], L["L1"], N=sp.N, batch=sp.batch,
                               workspace=L["ws"], group=args.group, act_quant=args.act_quant)

    def contract(i):
        for L in layers:
            sp, st = L["spec"], L["sets"][i % L["nsets"]]
            hsq.contract_stage(sp.M, sp.K, st["packed"], st["sw"], L["L2"], L["bias"], st["Y"], N=sp.N,
                               batch=sp.batch, r=sp.r, workspace=L["ws"], kernel=L["kernel"],
                               group=args.group)

    def step(i):
        # one call of the layer's entry point per layer (its quantization
        # pass and contraction on one stream)
        for L in layers:
            sp, st = L["spec"], L["sets"][i % L["nsets"]]
            hsq.w4a4_lowrank_linear(st["X"], L["lam"], st["packed"], st["sw"], L["L1"], L["L2"], L["bias"],
                                    N=sp.N, batch=sp.batch, y_dtype=args.y_dtype, out=st["Y"], workspace=L["ws"],
                                    kernel=L["call_kernel"], group=args.group, act_quant=args.act_quant)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed work is captured in HIP graphs and replayed, so the GPU runs
    # the kernels back to back without host launch gaps: one graph of the K
    # timed steps (rotating through the input sets), and, for the per-kernel
    # durations, one graph of K steps' quantization passes and one of K
    # steps' contractions.  Every graph is replayed once inside its own pair
    # of events on the capture stream (the stream its kernels run on).
    cap = torch.cuda.Stream()
    graphs = {}
    for name, fn in (("step", step), ("quantize", quant), ("contract", contract)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(args.steps):
                    fn(args.warmup + i)
        graphs[name] = g
    torch.cuda.synchronize()

    def timed(name):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(cap):
            t0.record(cap)
            graphs[name].replay()
            t1.record(cap)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    graphs["step"].replay()                  # untimed: first replay uploads the graph
    graphs["quantize"].replay()
    graphs["contract"].replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    total_ms = timed("step")
    wall = time.perf_counter() - wall0
    nl = len(layers)
    q_avg = timed("quantize") / (args.steps * nl)
    c_avg = timed("contract") / (args.steps * nl)
    ms_step = total_ms / args.steps

    # per-step spread: one-step graphs (one per input set), each replay
    # bracketed by events on the capture stream
    one = []
    for k in range(min(max(L["nsets"] for L in layers), args.steps)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                step(k)
        one.append(g)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    with torch.cuda.stream(cap):
        for i in range(args.steps):
            pairs[i][0].record(cap)
            one[i % len(one)].replay()
            pairs[i][1].record(cap)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in pairs]) * 1e3
    spread = {q: round(float(np.percentile(per_step, p)), 2)
              for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}

    if args.copy_mb > 0:
        nb = int(args.copy_mb * 1e6) // 16 * 16
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    specs = [L["spec"] for L in layers]
    ops = sum(sp.ops for sp in specs)
    value = ops / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel (the contraction, one launch per layer
    # and step): compute-bound at large M (int8 MFMA), HBM-bound when the
    # weights dominate (small M); achieved = algorithmic work per launch /
    # the average launch duration
    cbytes = sum(contract_bytes(sp.M, sp.K, sp.N, sp.r, sp.batch, y_bytes, args.group) for sp in specs)
    intensity = ops / cbytes
    ridge = PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    kernels = sorted(set(L["kernel"] for L in layers))
    kname = f"contract ({'/'.join(kernels)})" + (f", {nl} launches per step ({', '.join(names)})" if nl > 1 else "")
    # HBM bytes per launch from the counters (keyed by workload; for a
    # several-layer workload, the average over its launches)
    traffic = (read_traffic(kernels[0], traffic_key(args.layer, args.tokens, layers[0]["spec"].M, args.group))
               if len(kernels) == 1 else None)
    if intensity >= ridge:
        ach = ops / nl / (c_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_INT8_TOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_INT8_TOPS, 4), "traffic": traffic,
                "kernel": kname, "ops_per_launch": ops // nl,
                "note": "int8 MFMA operations (2 per multiply-accumulate) counted as FLOP"}
    else:
        ach = cbytes / nl / (c_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": kname, "bytes_per_launch": cbytes // nl}

    # the same launch against this GPU's measured ceilings (libhsq_probe):
    # the int8 MFMA probe's rate (MFMAs only, and with the exact two-FMA
    # rescale per element), or the HBM read rate of a 27 MB / 1 GiB stream
    if not args.no_peaks:
        peaks = measure_peaks(torch)
        roof["measured_peaks"] = peaks
        if roof["bound"] == "mfma":
            mp = peaks["int8_mfma_tops"]
            roof["frac_measured"] = round(roof["achieved"] / mp["mfma_only"], 4)
            roof["frac_of_rescale_ceiling"] = round(roof["achieved"] / mp["mfma_plus_2_fma_per_element"], 4)
        else:
            hb = peaks["hbm_gbs"]
            ref = hb["read_27MB_rotated"] if cbytes / nl < 64e6 else hb["read_1GiB"]
            roof["frac_measured"] = round(roof["achieved"] / ref, 4)

    sp0 = specs[0]
    cfg = {"workload": f"{wl_name}: {wl_desc or sp0.description}"}
    if nl == 1:
        cfg.update(M=sp0.M, K=sp0.K, N=sp0.N, rank=sp0.r, batch=sp0.batch)
    else:
        cfg["layers"] = [dict(name=sp.name, M=sp.M, K=sp.K, N=sp.N, rank=sp.r, batch=sp.batch) for sp in specs]
    cfg.update(group=args.group, y_dtype=args.y_dtype, contract_kernel="/".join(kernels),
               act_quant=args.act_quant, rotated_sets=[L["nsets"] for L in layers])
    abytes = sum(algorithmic_bytes(sp.M, sp.K, sp.N, sp.r, sp.batch, y_bytes, args.group) for sp in specs)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": cfg,
        "stages_ms": {"quantize": round(q_avg, 5), "contract": round(c_avg, 5),
                      "per": "launch (average over the workload's layers)",
                      "timing": "HIP graph replay, events on the capture stream"},
        "step_us": spread,
        "device": device_info(torch),
        "layer_hbm_frac": round(abytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
        "wall_s": round(wall, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.act_quant == "sym":
        out["cpu_baseline"] = cpu_baseline([L["lay"] for L in layers], specs, args.cpu_seconds,
                                           args.cpu_rows)
        out["cpu_single_thread"] = cpu_single_thread_tiny()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
