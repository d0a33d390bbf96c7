"""Benchmark: Bi-WKV forward (+ Q-Shift) throughput and HBM roofline on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5]
                    [--entry auto|fused|biwkv|causal|gated|qshift|mix|backward|bidir]

One step = one pass of the whole hot path over one batch: on the default workload (config 4: B=4,
64x64 grid so T=4096, C=1024, bf16 k/v, fp32 accumulate and output) the fused Q-Shift + Bi-WKV
entry. The same run also times the plain Bi-WKV forward (biwkv_forward) on the same inputs and
reports it under "gate_entry" with its own roofline. --config N runs workload N instead (its
fused entry on configs 2 and 4, biwkv_forward on 1, 3 and 5). Inputs are resident in HBM before
timing; R copies of inputs and outputs are rotated so each step's buffers were last touched more
than 2 x 256 MB (the memory-side cache) of traffic ago, i.e. every step streams from HBM. Prints
ONE JSON line.

Also reported: per-launch times (median, p10, p90 of event pairs around single launches), and a
measured memory ceiling for the same byte mix (libhbmceiling: k and v read, out written, nothing
else computed), with the kernel's fraction of it.

    python bench.py --calibrate-copy      plain device copy of a known size (for counter scaling)
    python bench.py --summarize DIR       summarise rocprofv3 output (kernel stats / counters)
    python bench.py --counters-table      the recorded HBM traffic of every entry against its algorithmic bytes
    python bench.py --summarize-sq D1 D2 D3   instruction mix, occupancy, LDS conflicts from three
                                          rocprofv3 --pmc passes of SQ counters
    python bench.py --record-counters KF KW CF CW [--config N --entry E]
        turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench, the same two of
        --calibrate-copy) into profiles/hbm_counters.json: HBM bytes per call, scaled so that the
        copy's counters read its known size, stamped with the hash of the kernel sources
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
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
CALIBRATION_BYTES = 512 * 1024 * 1024
MIN_CPU_SECONDS = 10.0
# entry timed by default per workload (the fused entry where the workload has Q-Shift), and the
# plain forward timed beside it
DEFAULT_ENTRY = {1: "biwkv", 2: "fused", 3: "biwkv", 4: "fused", 5: "biwkv"}
GATE_ENTRY = {2: "biwkv", 4: "biwkv"}
# entries whose byte mix is the forward's (k, v read once, fp32 out written): the memory ceiling
# applies to them
CEILING_ENTRIES = ("biwkv", "fused", "causal", "bidir")
# grid-stride streaming variants tried for the ceiling (blocks, unroll, policy: bit 0 non-temporal
# loads, bit 1 non-temporal stores, bit 2 8-byte pieces of k and v); the fastest is the ceiling
CEILING_VARIANTS = [(512, 1, 3), (2048, 1, 3), (8192, 2, 3), (8192, 4, 3), (1024, 1, 1), (4096, 2, 1),
                    (8192, 1, 7), (16384, 1, 7), (4096, 2, 7), (8192, 2, 7)]
COPY_KERNEL = "copy"  # substring of the device copy kernel's name in the counter output
KERNEL_NAMES = {"fused": "biwkv_row_kernel", "biwkv": "biwkv_row_kernel", "causal": "biwkv_row_kernel",
                "gated": "biwkv_row_kernel", "qshift": "qshift_kernel", "mix": "qshift_mix_kernel",
                "backward": "bwd_", "bidir": "biwkv_row_kernel"}
# entries made of several kernels: their counters are summed over every kernel of a call, and the
# calls are counted by a kernel that runs once per call (the backward's last kernel, the dw / du
# fold: bwd_reduce_kernel after the multi-launch form, bwd_one_reduce_kernel after one launch)
CALL_MARKER = {"backward": "reduce_kernel"}
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


def counter_key(config: int, entry: str) -> str:
    return f"config{config}:{entry}"


def _load_counters():
    """Counter-derived HBM bytes per call, valid only for the kernel source they were taken on."""
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


def _percentiles(xs):
    d = sorted(xs)
    pick = lambda q: d[min(len(d) - 1, int(q * (len(d) - 1) + 0.5))]
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9)}


def _time_calls(torch, stream, step, steps, warmup):
    """Warm-up, then the timed span of `steps` back-to-back calls (HIP events on the launch stream,
    a barrier and a device synchronisation on both sides), then `steps` more calls each between its
    own event pair. Returns (span seconds / call, wall seconds, per-call microseconds)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = start.elapsed_time(end) * 1e-3 / steps
    pairs = []
    for i in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(warmup + steps + i)
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) * 1e3 for a, b in pairs]
    return span, wall, per


def copy_ceiling(torch, stream, ks_, vs_, outs, n, kv_bytes, steps, warmup):
    """The memory ceiling of the forward's byte mix on this device: libhbmceiling's streaming
    kernels (k, v read, out = k + v written; nothing else) on the bench's own rotated buffers, the
    fastest of CEILING_VARIANTS. Returns (GB/s, microseconds per call, variant)."""
    import ctypes

    from linear_complexity_vision_amd import build

    lib = ctypes.CDLL(build.CEILING_LIB)
    f = lib.hbm_stream
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    R = len(outs)
    dt = 1 if kv_bytes == 2 else 0
    best = None
    for blocks, unroll, policy in CEILING_VARIANTS:
        def step(i, blocks=blocks, unroll=unroll, policy=policy):
            r = i % R
            rc = f(ks_[r].data_ptr(), vs_[r].data_ptr(), outs[r].data_ptr(), n, dt, 0, blocks, unroll, policy,
                   stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"hbm_stream failed ({rc})")
        span, _, _ = _time_calls(torch, stream, step, max(20, steps // 4), 5)
        if best is None or span < best[0]:
            best = (span, (blocks, unroll, policy))
    byts = 2 * kv_bytes * n + 4 * n
    return byts / best[0] / 1e9, best[0] * 1e6, {"blocks": best[1][0], "unroll": best[1][1], "policy": best[1][2],
                                                "bytes": byts}


def run_bench(args) -> dict:
    import numpy as np
    import torch

    import linear_complexity_vision_amd as lib
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    entry = DEFAULT_ENTRY[args.config] if args.entry == "auto" else args.entry
    # the sparse-input entry runs on the masked-image workload of the same element count
    wl = workloads.make_mae(2) if entry == "bidir" else workloads.make(args.config)
    B, H, W, C = wl.B, wl.H, wl.W, wl.C
    T = H * W
    n = B * T * C
    bf16 = wl.dtype == "bf16"
    kv_bytes = 2 if bf16 else 4
    ks, vs = wl.kv_storage()

    def dev_kv(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)

    kb, vb = dev_kv(ks), dev_kv(vs)
    w = torch.from_numpy(wl.w).to(dev)
    u = torch.from_numpy(wl.u).to(dev)
    set_bytes = (kb.numel() + vb.numel()) * kv_bytes + n * (16 if entry == "backward" else 4)
    R = _rotation(set_bytes)
    ks_ = [kb] + [kb.clone() for _ in range(R - 1)]
    vs_ = [vb] + [vb.clone() for _ in range(R - 1)]
    outs = [torch.empty((B, T, C), dtype=torch.float32, device=dev) for _ in range(R)]
    dt = lib.BF16 if bf16 else lib.F32
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
        r32 = _gate_input(wl)
        rb = dev_kv(workloads.round_to_bf16_bits(r32) if bf16 else r32)
        rs_ = [rb] + [rb.clone() for _ in range(R - 1)]

    # One checked call per buffer set through the package, then the same C entry point called
    # with the already marshalled arguments (the timed loop measures the library, not Python).
    stream = torch.cuda.current_stream(dev)
    cl = lib.load_library()

    def calls_for(e):
        calls = []
        for r in range(R):
            if e == "fused":
                lib.biwkv_qshift_forward(ks_[r], vs_[r], w, u, H, W, wl.shift, wl.gamma, out=outs[r])
                calls.append((cl.biwkv_qshift_forward,
                              (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                               outs[r].data_ptr(), B, H, W, C, wl.shift, wl.gamma, dt, stream.cuda_stream)))
            elif e == "bidir":
                lib.biwkv_qshift_bidir_forward(ks_[r], vs_[r], w, u, wl.shift, wl.gamma, out=outs[r])
                calls.append((cl.biwkv_qshift_bidir_forward,
                              (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                               outs[r].data_ptr(), B, T, C, wl.shift, wl.gamma, dt, stream.cuda_stream)))
            elif e == "biwkv":
                lib.biwkv_forward(ks_[r], vs_[r], w, u, out=outs[r])
                calls.append((cl.biwkv_forward,
                              (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                               outs[r].data_ptr(), B, T, C, dt, stream.cuda_stream)))
            elif e == "causal":
                lib.biwkv_causal_forward(ks_[r], vs_[r], w, u, out=outs[r])
                calls.append((cl.biwkv_causal_forward,
                              (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                               outs[r].data_ptr(), B, T, C, dt, stream.cuda_stream)))
            elif e == "gated":
                lib.biwkv_gated_forward(ks_[r], vs_[r], rs_[r], w, u, out=outs[r])
                calls.append((cl.biwkv_gated_forward,
                              (ks_[r].data_ptr(), vs_[r].data_ptr(), rs_[r].data_ptr(), w.data_ptr(),
                               u.data_ptr(), outs[r].data_ptr(), B, T, C, dt, stream.cuda_stream)))
            elif e == "backward":
                dk, dv, dw, du = lib.biwkv_backward(ks_[r], vs_[r], w, u, gs_[r])
                outs[r].copy_(dk)
                dvs[r].copy_(dv)
                dws[r][0].copy_(dw)
                dws[r][1].copy_(du)
                calls.append((cl.biwkv_backward,
                              (ks_[r].data_ptr(), vs_[r].data_ptr(), w.data_ptr(), u.data_ptr(),
                               gs_[r].data_ptr(), outs[r].data_ptr(), dvs[r].data_ptr(), dws[r][0].data_ptr(),
                               dws[r][1].data_ptr(), B, T, C, dt, stream.cuda_stream)))
            elif e == "mix":
                lib.qshift_mix(xs[r], mu, H, W, wl.shift, wl.gamma, out=outs[r])
                calls.append((cl.qshift_mix, (xs[r].data_ptr(), mu.data_ptr(), outs[r].data_ptr(), B, H, W,
                                              C, N_MIX, wl.shift, wl.gamma, stream.cuda_stream)))
            else:
                lib.qshift(xs[r], H, W, wl.shift, wl.gamma, out=outs[r])
                calls.append((cl.qshift, (xs[r].data_ptr(), outs[r].data_ptr(), B, H, W, C, wl.shift,
                                          wl.gamma, stream.cuda_stream)))
        return calls

    names = {"fused": "biwkv_qshift_forward", "biwkv": "biwkv_forward", "causal": "biwkv_causal_forward",
             "gated": "biwkv_gated_forward", "qshift": "qshift", "mix": "qshift_mix",
             "backward": "biwkv_backward", "bidir": "biwkv_qshift_bidir_forward"}
    counters = _load_counters()

    def measure(e):
        calls = calls_for(e)

        def step(i):
            fn, a = calls[i % R]
            rc = fn(*a)
            if rc != 0:
                raise lib.BiwkvError(rc, lib.status_string(rc))

        torch.cuda.synchronize()
        assert lib.stream_fault_flags(dev) == 0
        span, wall, per = _time_calls(torch, stream, step, args.steps, args.warmup)
        assert lib.stream_fault_flags(dev) == 0
        ab = alg_bytes(e, B, H, W, C, 4 if e in ("qshift", "mix") else kv_bytes, wl.shift, wl.gamma)
        achieved = ab / span / 1e9
        traffic = None
        if counters is not None:
            rec = counters.get("entries", {}).get(counter_key(args.config, e))
            traffic = rec["hbm_bytes_per_call"] if rec else None
        pct = _percentiles(per)
        return {"entry": names[e], "wall": wall, "span": span,
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "alg_bytes_per_launch": ab,
                             "avg_launch_ms": span * 1e3,
                             "launch_us": {k: round(v, 3) for k, v in pct.items()}}}

    main = measure(entry)
    gate = measure(GATE_ENTRY[args.config]) if entry == DEFAULT_ENTRY[args.config] and args.config in GATE_ENTRY \
        else None
    ceiling = None
    if entry in CEILING_ENTRIES and not args.no_ceiling:
        gbps, us, variant = copy_ceiling(torch, stream, ks_, vs_, outs, n, kv_bytes, args.steps, args.warmup)
        ceiling = {"gbps": gbps, "us": us, "variant": variant}
        for m in (main, gate):
            if m is not None:
                m["roofline"]["copy_ceiling_gbps"] = gbps
                m["roofline"]["frac_of_copy_ceiling"] = m["roofline"]["achieved"] / gbps

    metric_shape = ("N=1024 visible tokens (sparse, MAE) C=1024" if entry == "bidir" else f"T={T} C={C}")
    res = {
        "metric": ("Bi-WKV bwd" if entry == "backward" else "Bi-WKV fwd")
                  + " Gtoken*ch/s + achieved HBM GB/s (% peak) at " + metric_shape,
        "value": n * args.steps / main["wall"] / 1e9,
        "unit": "Gtoken*ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main["wall"] * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "entry": main["entry"], "B": B, "T": T, "H": H, "W": W, "C": C,
                   "kv_storage": "f32" if entry in ("qshift", "mix") else wl.dtype, "shift": wl.shift,
                   "gamma": wl.gamma, "buffer_sets_rotated": R},
        "roofline": main["roofline"],
        "_wl": wl,
        "_entry": entry,
    }
    if gate is not None:
        res["gate_entry"] = {"entry": gate["entry"], "value": n * args.steps / gate["wall"] / 1e9,
                             "unit": "Gtoken*ch/s", "roofline": gate["roofline"]}
    if ceiling is not None:
        res["copy_ceiling"] = ceiling
    return res


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


def _counter_rows(path: str, counter: str):
    """(kernel name, dispatch key, grid size, value) per dispatch of `counter` (values of one
    dispatch's instances summed)."""
    vals = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            key = (f, row.get("Dispatch_Id", row.get("Correlation_Id")))
            name = row.get("Kernel_Name", "")
            v = vals.setdefault(key, [name, int(row.get("Grid_Size", "0")), 0.0])
            v[2] += float(row["Counter_Value"])
    return [(name, key, grid, val) for key, (name, grid, val) in vals.items()]


def _counter_means(path: str, counter: str, kernel: str) -> float:
    """Mean per-dispatch value of `counter` over the largest-grid dispatches of kernels whose name
    contains `kernel` (smaller dispatches of the same kernel, e.g. set-up copies, are skipped)."""
    rows = [r for r in _counter_rows(path, counter) if kernel in r[0]]
    if not rows:
        raise SystemExit(f"no {counter} values for {kernel} under {path}")
    top = max(r[2] for r in rows)
    sel = [r[3] for r in rows if r[2] == top]
    return sum(sel) / len(sel)


# tile-kernel template flags (FUSED, CAUSAL, GATED) of each forward entry: a run of one entry also
# times the plain forward beside it, so the kernels are told apart by their flags
ROW_FLAGS = {"biwkv": (False, False, False), "fused": (True, False, False), "bidir": (True, False, False),
             "causal": (False, True, False), "gated": (False, False, True)}


def _row_flags(name: str):
    """(FUSED, CAUSAL, GATED) of a biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED,
    MODE> name, or None for any other kernel."""
    i = name.find("biwkv_row_kernel<")
    if i < 0:
        return None
    args = [a.strip() for a in name[i + len("biwkv_row_kernel<"):].split(">", 1)[0].split(",")]
    return args[4] == "true", args[6] == "true", args[7] == "true"


def kernel_of_entry(name: str, entry: str) -> bool:
    """Whether a kernel (by its demangled name) belongs to `entry`."""
    if entry in ROW_FLAGS:
        return _row_flags(name) == ROW_FLAGS[entry]
    return KERNEL_NAMES[entry] in name


def _counter_call_sum(path: str, counter: str, entry: str) -> float:
    """Per call of an entry made of one or more distinct kernels (same grid) that belong to
    `entry`: the sum over those kernels of each one's mean per dispatch, at the largest grid
    (a two-pass forward is a sums launch and an output launch)."""
    rows = [r for r in _counter_rows(path, counter) if kernel_of_entry(r[0], entry)]
    if not rows:
        raise SystemExit(f"no {counter} values for {entry} under {path}")
    top = max(r[2] for r in rows)
    by_name = {}
    for name, _, grid, val in rows:
        if grid == top:
            by_name.setdefault(name, []).append(val)
    return sum(sum(v) / len(v) for v in by_name.values())


def _counter_per_call(path: str, counter: str, kernel: str, marker: str) -> float:
    """Sum of `counter` over every dispatch of kernels whose name contains `kernel`, divided by the
    number of dispatches of the once-per-call kernel `marker`: the value per call of an entry point
    that launches several kernels."""
    rows = _counter_rows(path, counter)
    total = sum(val for name, _, _, val in rows if kernel in name)
    calls = sum(1 for name, _, _, _ in rows if marker in name)
    if not calls:
        raise SystemExit(f"no {counter} values for {marker} under {path}")
    return total / calls


def record_counters(kf: str, kw: str, cf: str, cw: str, config: int, entry: str) -> None:
    """HBM traffic per call of the entry on workload `config` from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what it reads for a device copy of CALIBRATION_BYTES."""
    if entry in CALL_MARKER:
        fetch = _counter_per_call(kf, "FETCH_SIZE", KERNEL_NAMES[entry], CALL_MARKER[entry])
        write = _counter_per_call(kw, "WRITE_SIZE", KERNEL_NAMES[entry], CALL_MARKER[entry])
    else:
        fetch = _counter_call_sum(kf, "FETCH_SIZE", entry)
        write = _counter_call_sum(kw, "WRITE_SIZE", entry)
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
    rec["entries"][counter_key(config, entry)] = {
        "fetch_kib_per_call": fetch, "write_kib_per_call": write,
        "hbm_bytes_per_call": fetch * f_scale + write * w_scale}
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    json.dump(rec, open(COUNTERS_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec["entries"][counter_key(config, entry)]))


def counters_table() -> None:
    """One line per recorded entry of profiles/hbm_counters.json: FETCH_SIZE and WRITE_SIZE per
    call, the scaled HBM bytes, the algorithmic bytes of the call and their ratio."""
    import workloads

    rec = json.load(open(COUNTERS_FILE))
    print(f"kernel sources sha256[:16]: {rec.get('kernel_source_sha256_16')}")
    cal = rec["calibration"]
    print(f"calibration: FETCH_SIZE {cal['fetch_kib']:.1f} KiB -> {cal['fetch_bytes_per_unit']:.2f} B per unit; "
          f"WRITE_SIZE {cal['write_kib']:.1f} KiB -> {cal['write_bytes_per_unit']:.2f} B per unit")
    for key, e in rec["entries"].items():
        config, entry = int(key.split(":")[0][len("config"):]), key.split(":")[1]
        wl = workloads.make_mae(2) if entry == "bidir" else workloads.make(config)
        kvb = 4 if entry in ("qshift", "mix") else (2 if wl.dtype == "bf16" else 4)
        ab = alg_bytes(entry, wl.B, wl.H, wl.W, wl.C, kvb, wl.shift, wl.gamma)
        shape = f"B{wl.B}_{'N' if entry == 'bidir' else 'T'}{wl.H * wl.W}_C{wl.C}_{'bf16' if kvb == 2 else 'f32'}"
        hbm = e["hbm_bytes_per_call"]
        print(f"config {config} {entry:9s} {shape:26s} FETCH {e['fetch_kib_per_call']:12.1f} KiB  WRITE "
              f"{e['write_kib_per_call']:12.1f} KiB  HBM {hbm / 1e6:9.2f} MB  algorithmic {ab / 1e6:9.2f} MB  "
              f"ratio {hbm / ab:.3f}")


def summarize_sq(d1: str, d2: str, d3: str) -> None:
    """Per-kernel instruction mix, occupancy and LDS conflicts from three rocprofv3 --pmc passes
    (d1: SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD
    SQ_INSTS_VMEM_WR SQ_INSTS_SMEM; d2: SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU; d3:
    SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE). Counters are summed over the shader engines of a
    dispatch and averaged over the dispatches of a kernel name. Per-wave counts = SQ_INSTS_* /
    SQ_WAVES; resident waves per SIMD = 4 SQ_WAVE_CYCLES / (SQ_BUSY_CYCLES x 8 CUs x 4 SIMDs);
    VALU-active share = 4 SQ_ACTIVE_INST_VALU / (SQ_BUSY_CYCLES x 32 SIMDs per SE)."""
    means: dict = {}
    for d in (d1, d2, d3):
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            acc: dict = {}
            for row in csv.DictReader(open(f)):
                key = (row.get("Kernel_Name", "?"), row.get("Counter_Name"))
                acc.setdefault(key, []).append(float(row.get("Counter_Value", "nan")))
            for (kname, cname), vals in acc.items():
                means.setdefault(kname, {})[cname] = sum(vals) / len(vals)
    for kname in sorted(means):
        m = means[kname]
        # the library's and the runtime's helper kernels (copies, fills, counter set-up) are skipped
        if "SQ_WAVES" not in m or m["SQ_WAVES"] <= 0 or any(x in kname for x in ("rocclr", "fill_", "init_counters")):
            continue
        w = m["SQ_WAVES"]
        print(kname.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0][:100])
        print(f"  waves {w:.0f}; per wave: VALU {m.get('SQ_INSTS_VALU', 0) / w:.0f} (transcendental "
              f"{m.get('SQ_INSTS_VALU_TRANS_F32', 0) / w:.0f}), SALU {m.get('SQ_INSTS_SALU', 0) / w:.0f}, "
              f"LDS {m.get('SQ_INSTS_LDS', 0) / w:.1f}, vector loads {m.get('SQ_INSTS_VMEM_RD', 0) / w:.1f}, "
              f"vector stores {m.get('SQ_INSTS_VMEM_WR', 0) / w:.1f}, scalar loads {m.get('SQ_INSTS_SMEM', 0) / w:.1f}")
        busy = m.get("SQ_BUSY_CYCLES", 0)
        if busy > 0:
            print(f"  busy {busy:.0f} cycles (summed over SEs); resident waves per SIMD "
                  f"{4 * m.get('SQ_WAVE_CYCLES', 0) / (busy * 8 * 4):.2f}; VALU-active share "
                  f"{4 * m.get('SQ_ACTIVE_INST_VALU', 0) / (busy * 32):.2f}; LDS bank-conflict cycles "
                  f"{m.get('SQ_LDS_BANK_CONFLICT', 0):.0f} of {m.get('SQ_LDS_IDX_ACTIVE', 0):.0f} LDS-active")


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
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, choices=[1, 2, 3, 4, 5], default=4)
    ap.add_argument("--entry", choices=["auto", "fused", "biwkv", "causal", "gated", "qshift", "mix", "backward",
                                        "bidir"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--two-pass", action="store_true",
                    help="every row through the two-pass form (BIWKV_OPT_TWO_PASS = 1), for comparison")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--summarize-sq", nargs=3, metavar=("D1", "D2", "D3"))
    ap.add_argument("--counters-table", action="store_true")
    ap.add_argument("--record-counters", nargs=4, metavar=("KF", "KW", "CF", "CW"))
    args = ap.parse_args()

    if args.counters_table:
        counters_table()
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return
    if args.summarize:
        summarize(args.summarize)
        return 0
    if args.record_counters:
        entry = DEFAULT_ENTRY[args.config] if args.entry == "auto" else args.entry
        record_counters(*args.record_counters, config=args.config, entry=entry)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the Bi-WKV path shards by batch, channel "
              "or token rows without changing the per-GPU kernel); run with --gpus 1", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(args)
        return 0
    if args.two_pass:
        import linear_complexity_vision_amd as lib
        lib.set_option(lib.OPT_TWO_PASS, 1)
    res = run_bench(args)
    if args.two_pass:
        res["config"]["two_pass"] = True
    wl = res.pop("_wl")
    entry = res.pop("_entry")
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl, entry)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
