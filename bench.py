"""Benchmark: Bi-WKV forward (+ Q-Shift) throughput and HBM roofline on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--entry fused|biwkv|causal|gated|qshift|mix|backward|bidir]

One step = one pass of the whole hot path over one batch: the fused Q-Shift + Bi-WKV entry on the
high-resolution workload (B=4, 64x64 grid so T=4096, C=1024, bf16 k/v, fp32 accumulate and
output). Inputs are resident in HBM before timing; R copies of inputs and outputs are rotated so
each step's buffers were last touched more than 256 MB of traffic ago (the MALL size), i.e. every
step streams from HBM. Prints ONE JSON line.

Also:
    python bench.py --calibrate-copy      plain device copy of a known size (for counter scaling)
    python bench.py --summarize DIR       summarise rocprofv3 output (kernel stats / counters)
    python bench.py --record-counters KF KW CF CW
        turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench, the same two of
        --calibrate-copy) into profiles/hbm_counters_*.json: HBM bytes per launch, scaled so that
        the copy's counters read its known size, stamped with the hash of the kernel sources
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E peak
MALL_BYTES = 256 * 1024 * 1024
KERNEL_DIR = os.path.join(ROOT, "linear_complexity_vision_amd", "csrc")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters_biwkv_qshift_B4_T4096_C1024_bf16.json")
CALIBRATION_BYTES = 512 * 1024 * 1024
MIN_CPU_SECONDS = 3.0
COPY_KERNEL = "copy"  # substring of the device copy kernel's name in the counter output
KERNEL_NAMES = {"fused": "biwkv_row_kernel", "biwkv": "biwkv_row_kernel", "causal": "biwkv_row_kernel",
                "gated": "biwkv_row_kernel", "qshift": "qshift_kernel", "mix": "qshift_mix_kernel",
                "backward": "bwd_", "bidir": "biwkv_row_kernel"}
# entries made of several kernels: their counters are summed over every kernel of a call, and the
# calls are counted by a kernel that runs once per call
CALL_MARKER = {"backward": "bwd_reduce_kernel"}
N_MIX = 3  # mixing vectors of the mix entry (the R, K and V projection inputs)


def kernel_source_hash() -> str:
    """Hash of every kernel source file (the counters are only valid for the code they measured)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        h.update(name.encode())
        h.update(open(os.path.join(KERNEL_DIR, name), "rb").read())
    return h.hexdigest()[:16]


def alg_bytes(entry: str, B: int, H: int, W: int, C: int, kv_bytes: int, shift: int = 1, gamma: float = 0.25) -> int:
    """Algorithmic HBM bytes of one call: what the method must move.

    biwkv:  read k and v (kv_bytes each), write fp32 out, read w and u (causal: the same).
    gated:  as biwkv, plus one read of the gate input r (kv_bytes).
    fused:  as biwkv, but the Q-Shift zero-filled sources are never read.
    qshift: read the in-grid sources, write every output (fp32).
    mix:    read x once (its shifted reads are the same elements), write N_MIX fp32 outputs.
    backward: read k and v (kv_bytes each) and the fp32 upstream gradient, write fp32 dk and dv,
            read w and u, write dw and du.
    bidir:  as fused, for the sequence shift of a sparse input (H = 1, W = N): each shifted
            channel has `shift` zero-filled tokens per batch item.
    """
    T = H * W
    n = B * T * C
    g = [int(C * gamma * j) for j in (1, 2, 3, 4)]
    zero_per_b = shift * H * g[1] + shift * W * (g[3] - g[1])  # zero-filled outputs per batch item
    if entry in ("biwkv", "causal"):
        return 2 * kv_bytes * n + 4 * n + 8 * C
    if entry == "fused":
        return 2 * kv_bytes * (n - B * zero_per_b) + 4 * n + 8 * C
    if entry == "gated":
        return 3 * kv_bytes * n + 4 * n + 8 * C
    if entry == "qshift":
        return 4 * (n - B * zero_per_b) + 4 * n
    if entry == "mix":  # x read once (its shifted reads are the same elements), N_MIX outputs
        return 4 * n + 4 * N_MIX * n + 4 * N_MIX * C
    if entry == "backward":
        return 2 * kv_bytes * n + 4 * n + 8 * n + 16 * C
    if entry == "bidir":
        return 2 * kv_bytes * (n - B * shift * g[3]) + 4 * n + 8 * C
    raise ValueError(entry)


def _load_counters():
    """Counter-derived HBM bytes per launch, valid only for the kernel source they were taken on."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, entry: str) -> dict:
    """The float64 oracle (four-state RNN form, the method's own O(TC) algorithm) on host cores,
    over the whole workload; input conversion is outside the timed span."""
    import numpy as np

    import oracle

    k = wl.k.astype(np.float64)
    v = wl.v.astype(np.float64)
    w = wl.w.astype(np.float64)
    u = wl.u.astype(np.float64)
    threads = oracle.max_threads()
    oracle.biwkv_rnn(k[:, :64], v[:, :64], w, u, threads=threads)  # warm the library and threads
    if entry == "mix":
        mu = _mix_vectors(wl.C)
        t0 = time.perf_counter()
        oracle.qshift_mix(wl.k, mu, wl.H, wl.W, wl.shift, wl.gamma)
        dt = time.perf_counter() - t0
        elems = wl.B * wl.T * wl.C
        return {"value": elems / dt / 1e9, "unit": "Gtoken*ch/s", "cores": 1, "kind": "oracle",
                "seconds": dt, "cpu": _cpu_model(),
                "sample": f"whole workload ({wl.B}x{wl.T}x{wl.C}), {N_MIX} mixes; numpy float64 oracle"}
    if entry == "qshift":
        x32 = wl.k
        t0 = time.perf_counter()
        oracle.qshift(x32, wl.H, wl.W, wl.shift, wl.gamma)
        dt = time.perf_counter() - t0
        elems = wl.B * wl.T * wl.C
        return {"value": elems / dt / 1e9, "unit": "Gtoken*ch/s", "cores": 1, "kind": "oracle",
                "seconds": dt, "cpu": _cpu_model(),
                "sample": f"whole workload ({wl.B}x{wl.T}x{wl.C}); single-threaded oracle Q-Shift gather"}
    # the whole workload, repeated until at least MIN_CPU_SECONDS have passed
    reps = 0
    t0 = time.perf_counter()
    while True:
        if entry == "bidir":
            ks = oracle.qshift_bidir_f64(k, wl.shift, wl.gamma)
            vs = oracle.qshift_bidir_f64(v, wl.shift, wl.gamma)
            oracle.biwkv_rnn(ks, vs, w, u, threads=threads)
        elif entry == "fused":
            ks = oracle.qshift_f64(k, wl.H, wl.W, wl.shift, wl.gamma)
            vs = oracle.qshift_f64(v, wl.H, wl.W, wl.shift, wl.gamma)
            oracle.biwkv_rnn(ks, vs, w, u, threads=threads)
        elif entry == "causal":
            oracle.biwkv_causal_rnn(k, v, w, u, threads=threads)
        elif entry == "gated":
            oracle.biwkv_gated(k, v, _gate_input(wl).astype(np.float64), w, u, threads=threads)
        elif entry == "backward":
            oracle.biwkv_backward_rnn(k, v, w, u, _upstream_grad(wl).astype(np.float64), threads=threads)
        else:
            oracle.biwkv_rnn(k, v, w, u, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= MIN_CPU_SECONDS:
            break
    elems = wl.B * wl.T * wl.C
    return {"value": reps * elems / dt / 1e9, "unit": "Gtoken*ch/s", "cores": threads,
            "kind": "oracle", "seconds": dt, "repetitions": reps, "cpu": _cpu_model(),
            "sample": f"whole workload ({wl.B}x{wl.T}x{wl.C}) x{reps}; float64 "
                      + ("two-state causal RNN oracle" if entry == "causal" else
                         "linear-time gradient oracle (prefix and suffix sums)" if entry == "backward"
                         else "four-state RNN oracle")
                      + (" times the sigmoid gate" if entry == "gated" else "")
                      + (" after the oracle Q-Shift of k and v" if entry == "fused" else "")
                      + (" after the oracle bidirectional shift of k and v" if entry == "bidir" else "")}


def _gate_input(wl):
    """A seeded gate input r for the gated entry: N(0, 3^2) drawn in float64, rounded to the
    storage type of k (here bf16 values)."""
    import numpy as np

    import workloads
    g = np.random.Generator(np.random.PCG64(404))
    r = (g.standard_normal((wl.B, wl.T, wl.C)) * 3.0).astype(np.float32)
    return workloads.bf16_bits_to_f32(workloads.round_to_bf16_bits(r)) if wl.dtype == "bf16" else r


def _upstream_grad(wl):
    """A seeded upstream gradient dL/dy for the backward entry: N(0, 1), float32 [B, T, C]."""
    import numpy as np
    return np.random.Generator(np.random.PCG64(406)).standard_normal((wl.B, wl.T, wl.C)).astype(np.float32)


def _mix_vectors(C: int):
    """Seeded mixing vectors mu [N_MIX, C] in [0, 1) for the mix entry."""
    import numpy as np
    return np.random.Generator(np.random.PCG64(405)).uniform(0, 1, (N_MIX, C)).astype(np.float32)


def _rotation(bytes_per_set: int) -> int:
    return max(2, -(-2 * MALL_BYTES // bytes_per_set) + 1)


def run_bench(args) -> dict:
    import numpy as np
    import torch

    import linear_complexity_vision_amd as lib
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # the sparse-input entry runs on the masked-image workload of the same element count
    wl = workloads.make_mae(2) if args.entry == "bidir" else workloads.make(4)
    B, H, W, C = wl.B, wl.H, wl.W, wl.C
    T = H * W
    entry = args.entry
    ks, vs = wl.kv_storage()
    kb = torch.from_numpy(np.ascontiguousarray(ks)).view(torch.bfloat16).to(dev)
    vb = torch.from_numpy(np.ascontiguousarray(vs)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    u = torch.from_numpy(wl.u).to(dev)
    set_bytes = (kb.numel() + vb.numel()) * 2 + B * T * C * (16 if entry == "backward" else 4)
    R = _rotation(set_bytes)
    ks_ = [kb] + [kb.clone() for _ in range(R - 1)]
    vs_ = [vb] + [vb.clone() for _ in range(R - 1)]
    outs = [torch.empty((B, T, C), dtype=torch.float32, device=dev) for _ in range(R)]
    if entry in ("qshift", "mix"):
        xs = [torch.from_numpy(wl.k).to(dev).contiguous() for _ in range(R)]
    if entry == "mix":
        mu = torch.from_numpy(_mix_vectors(C)).to(dev)
        outs = [torch.empty((N_MIX, B, T, C), dtype=torch.float32, device=dev) for _ in range(R)]
    if entry == "backward":
        gs_ = [torch.from_numpy(_upstream_grad(wl)).to(dev) for _ in range(R)]
        dvs = [torch.empty((B, T, C), dtype=torch.float32, device=dev) for _ in range(R)]
        dws = [torch.empty((2, C), dtype=torch.float32, device=dev) for _ in range(R)]
    if entry == "gated":
        rb = torch.from_numpy(np.ascontiguousarray(workloads.round_to_bf16_bits(_gate_input(wl)))).view(
            torch.bfloat16).to(dev)
        rs_ = [rb] + [rb.clone() for _ in range(R - 1)]

    # One checked call per buffer set through the package, then the same C entry point called
    # with the already marshalled arguments (the timed loop measures the library, not Python).
    stream = torch.cuda.current_stream(dev)
    cl = lib.load_library()
    calls = []
    for r in range(R):
        if entry == "fused":
            lib.biwkv_qshift_forward(ks_[r], vs_[r], w, u, H, W, wl.shift, wl.gamma, out=outs[r])
            calls.append((cl.biwkv_qshift_forward,
                          (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                           outs[r].data_ptr(), B, H, W, C, wl.shift, wl.gamma, lib.BF16,
                           stream.cuda_stream)))
        elif entry == "bidir":
            lib.biwkv_qshift_bidir_forward(ks_[r], vs_[r], w, u, wl.shift, wl.gamma, out=outs[r])
            calls.append((cl.biwkv_qshift_bidir_forward,
                          (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                           outs[r].data_ptr(), B, T, C, wl.shift, wl.gamma, lib.BF16, stream.cuda_stream)))
        elif entry == "biwkv":
            lib.biwkv_forward(ks_[r], vs_[r], w, u, out=outs[r])
            calls.append((cl.biwkv_forward,
                          (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                           outs[r].data_ptr(), B, T, C, lib.BF16, stream.cuda_stream)))
        elif entry == "causal":
            lib.biwkv_causal_forward(ks_[r], vs_[r], w, u, out=outs[r])
            calls.append((cl.biwkv_causal_forward,
                          (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                           outs[r].data_ptr(), B, T, C, lib.BF16, stream.cuda_stream)))
        elif entry == "gated":
            lib.biwkv_gated_forward(ks_[r], vs_[r], rs_[r], w, u, out=outs[r])
            calls.append((cl.biwkv_gated_forward,
                          (ks_[r].data_ptr(), vs_[r].data_ptr(), rs_[r].data_ptr(), w.data_ptr(),
                           u.data_ptr(), outs[r].data_ptr(), B, T, C, lib.BF16, stream.cuda_stream)))
        elif entry == "backward":
            dk, dv, dw, du = lib.biwkv_backward(ks_[r], vs_[r], w, u, gs_[r])
            outs[r].copy_(dk)
            dvs[r].copy_(dv)
            dws[r][0].copy_(dw)
            dws[r][1].copy_(du)
            calls.append((cl.biwkv_backward,
                          (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                           gs_[r].data_ptr(), outs[r].data_ptr(), dvs[r].data_ptr(), dws[r][0].data_ptr(),
                           dws[r][1].data_ptr(), B, T, C, lib.BF16, stream.cuda_stream)))
        elif entry == "mix":
            lib.qshift_mix(xs[r], mu, H, W, wl.shift, wl.gamma, out=outs[r])
            calls.append((cl.qshift_mix, (xs[r].data_ptr(), mu.data_ptr(), outs[r].data_ptr(), B, H, W,
                                          C, N_MIX, wl.shift, wl.gamma, stream.cuda_stream)))
        else:
            lib.qshift(xs[r], H, W, wl.shift, wl.gamma, out=outs[r])
            calls.append((cl.qshift, (xs[r].data_ptr(), outs[r].data_ptr(), B, H, W, C, wl.shift,
                                      wl.gamma, stream.cuda_stream)))

    def step(i):
        fn, a = calls[i % R]
        rc = fn(*a)
        if rc != 0:
            raise lib.BiwkvError(rc, lib.status_string(rc))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert lib.stream_fault_flags(dev) == 0

    # HIP events on the launch stream bracket the timed region; the launches queue back to back
    # (host submission is faster than the kernel), so the event span / K is the average launch
    # duration including the short gaps between kernels.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert lib.stream_fault_flags(dev) == 0

    avg_ms = start.elapsed_time(end) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    elems = B * T * C
    kv_bytes = 4 if entry in ("qshift", "mix") else 2
    ab = alg_bytes(entry, B, H, W, C, kv_bytes, wl.shift, wl.gamma)
    achieved = ab / (avg_ms * 1e-3) / 1e9
    counters = _load_counters()
    traffic = None
    if counters is not None and entry in counters.get("entries", {}):
        traffic = counters["entries"][entry]["hbm_bytes_per_launch"]
    names = {"fused": "biwkv_qshift_forward", "biwkv": "biwkv_forward", "causal": "biwkv_causal_forward",
             "gated": "biwkv_gated_forward", "qshift": "qshift", "mix": "qshift_mix",
             "backward": "biwkv_backward", "bidir": "biwkv_qshift_bidir_forward"}
    return {
        "metric": ("Bi-WKV bwd" if entry == "backward" else "Bi-WKV fwd")
                  + " Gtoken*ch/s + achieved HBM GB/s (% peak) at "
                  + ("N=1024 visible tokens (sparse, MAE) C=1024" if entry == "bidir" else "T=4096 C=1024"),
        "value": elems * args.steps / wall / 1e9,
        "unit": "Gtoken*ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "entry": names[entry], "B": B, "T": T, "H": H, "W": W, "C": C,
                   "kv_storage": "bf16" if entry not in ("qshift", "mix") else "f32", "shift": wl.shift,
                   "gamma": wl.gamma, "buffer_sets_rotated": R},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "alg_bytes_per_launch": ab, "avg_launch_ms": avg_ms},
        "_wl": wl,
    }


def calibrate_copy(args) -> None:
    """A plain device copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE counters.

    The source is the oldest quarter of a buffer four times larger than the copy, written before
    the rest of it, so none of it is still held in the memory-side cache when the copy reads it."""
    import torch

    n = CALIBRATION_BYTES // 4
    big = torch.empty(4 * n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty(n, dtype=torch.float32, device="cuda:0")
    for _ in range(args.steps):
        for q in range(4):
            big[q * n:(q + 1) * n].fill_(1.0)
        dst.copy_(big[:n])  # one read and one write of CALIBRATION_BYTES
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": CALIBRATION_BYTES,
                      "bytes_written": CALIBRATION_BYTES, "launches": args.steps}))


def _counter_means(path: str, counter: str, kernel: str) -> float:
    """Mean per-dispatch value of `counter` over the largest-grid dispatches of kernels whose name
    contains `kernel` (smaller dispatches of the same kernel, e.g. set-up copies, are skipped)."""
    vals = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter or kernel not in row.get("Kernel_Name", ""):
                continue
            # one row per dispatch and counter (values of one dispatch's instances are summed)
            key = (f, row.get("Dispatch_Id", row.get("Correlation_Id")))
            grid = int(row.get("Grid_Size", "0"))
            v = vals.setdefault(key, [grid, 0.0])
            v[1] += float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} values for {kernel} under {path}")
    top = max(g for g, _ in vals.values())
    sel = [x for g, x in vals.values() if g == top]
    return sum(sel) / len(sel)


def _counter_per_call(path: str, counter: str, kernel: str, marker: str) -> float:
    """Sum of `counter` over every dispatch of kernels whose name contains `kernel`, divided by the
    number of dispatches of the once-per-call kernel `marker`: the value per call of an entry point
    that launches several kernels."""
    total, calls = 0.0, set()
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            name = row.get("Kernel_Name", "")
            if kernel in name:
                total += float(row["Counter_Value"])
            if marker in name:
                calls.add((f, row.get("Dispatch_Id", row.get("Correlation_Id"))))
    if not calls:
        raise SystemExit(f"no {counter} values for {marker} under {path}")
    return total / len(calls)


def record_counters(kf: str, kw: str, cf: str, cw: str, entry: str) -> None:
    """HBM traffic per launch of the bench kernel (per call, for entries of several kernels) from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what it reads for a device copy of
    CALIBRATION_BYTES."""
    if entry in CALL_MARKER:
        fetch = _counter_per_call(kf, "FETCH_SIZE", KERNEL_NAMES[entry], CALL_MARKER[entry])
        write = _counter_per_call(kw, "WRITE_SIZE", KERNEL_NAMES[entry], CALL_MARKER[entry])
    else:
        fetch = _counter_means(kf, "FETCH_SIZE", KERNEL_NAMES[entry])
        write = _counter_means(kw, "WRITE_SIZE", KERNEL_NAMES[entry])
    cal_fetch = _counter_means(cf, "FETCH_SIZE", COPY_KERNEL)
    cal_write = _counter_means(cw, "WRITE_SIZE", COPY_KERNEL)
    f_scale = CALIBRATION_BYTES / cal_fetch
    w_scale = CALIBRATION_BYTES / cal_write
    rec = {}
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        pass
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        rec = {"entries": {}}
    rec["kernel_source_sha256_16"] = kernel_source_hash()
    rec["calibration"] = {"bytes": CALIBRATION_BYTES, "fetch_kib": cal_fetch, "write_kib": cal_write,
                          "fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale}
    rec["entries"][entry] = {"fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
                             "hbm_bytes_per_launch": fetch * f_scale + write * w_scale}
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    json.dump(rec, open(COUNTERS_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec["entries"][entry]))


def summarize(path: str) -> None:
    """Summarise rocprofv3 CSV output under `path`: per-kernel durations or counter values."""
    stats = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    for f in stats:
        print(f"# kernel stats: {os.path.relpath(f, path)}")
        for row in csv.DictReader(open(f)):
            print(f"{row.get('Name', '?')[:90]:90s} calls={row.get('Calls')} "
                  f"avg_ns={float(row.get('AverageNs', 'nan')):.0f} min_ns={row.get('MinNs')} "
                  f"max_ns={row.get('MaxNs')} pct={row.get('Percentage')}")
    ctr = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    for f in ctr:
        print(f"# counters: {os.path.relpath(f, path)}")
        acc = {}
        for row in csv.DictReader(open(f)):
            key = (row.get("Kernel_Name", "?")[:90], row.get("Counter_Name"))
            acc.setdefault(key, []).append(float(row.get("Counter_Value", "nan")))
        for (kname, cname), vals in sorted(acc.items()):
            print(f"{kname:90s} {cname} dispatches={len(vals)} mean={sum(vals) / len(vals):.1f} "
                  f"min={min(vals):.1f} max={max(vals):.1f}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--entry", choices=["fused", "biwkv", "causal", "gated", "qshift", "mix", "backward", "bidir"],
                    default="fused")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--record-counters", nargs=4, metavar=("KF", "KW", "CF", "CW"))
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return 0
    if args.record_counters:
        record_counters(*args.record_counters, entry=args.entry)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the Bi-WKV path shards by batch, channel "
              "or token rows without changing the per-GPU kernel); run with --gpus 1", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(args)
        return 0
    res = run_bench(args)
    wl = res.pop("_wl")
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl, args.entry)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
