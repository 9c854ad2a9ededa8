"""Benchmark of the S6 selective-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--step-size given|softplus] [--discretization zoh|euler] [--backward]
    python bench.py --microbench

A step is one selective_scan_fwd call over the whole workload (every row of the hot
path: discretisation, recurrence, readout, feed-through, gate, store) with its inputs
already resident in HBM.  The default workload is the long-context one the throughput
target is stated on: batch 4, L 16384, D 2560, N 16, bf16 I/O with fp32 state, SiLU gate.
Inputs are seeded synthetic data (s6_workloads), copied to the GPU once before timing.

Prints ONE JSON line: elements/s (batch*L*D*N per second) as `value`, the algorithmic HBM
bandwidth, the roofline of the scan kernel, and the CPU oracle timed on this host on a
bounded sample of the same workload.

Options measure the discretisation variants on the same workload: --step-size softplus
feeds the pre-activation (raw step sizes and a per-channel bias, s6_workloads.raw_step_sizes)
and lets the kernel apply softplus(raw + bias); --discretization euler uses the first-order
input coefficient.  The defaults are the plain ZOH scan with given step sizes.
--backward times selective_scan_bwd (all gradients, from a seeded dy) on the same workload
instead of the forward pass.

Timing: after the warm-up, the K timed calls run back to back between two device
synchronisations (ms_per_step, value) with HIP events around each call on its stream (the
kernel time the roofline uses: mean, median and minimum are reported).  Then K more calls are
timed the same way, each after 512 MiB written to a scratch buffer outside the events, which
evicts the L2 caches and the 256 MB Infinity Cache ("cold_cache").

--microbench instead prints the issue-rate and bandwidth probes of libselscan_microbench.so
(fp32 FMA and v_exp_f32 rates against wavefronts per SIMD, their overlap, streaming copy and
write bandwidth, and the shader clock the GPU held), the practical roofs of the scan, and the
arbitration probe (where 2.5 workgroups per compute unit are placed and how long their
wavefronts run, without and with the scan's issue-priority rotation).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import s6_workloads  # noqa: E402

METRIC = "scan elements/s (B*L*D*N per sec) + achieved HBM GB/s vs peak, 1 MI355X"
HBM_PEAK_GBS = 8000.0            # MI355X published HBM3E bandwidth
# fp32 vector ALU: 256 CU x 4 SIMD x 16 lanes x 2 flop (FMA) x 2.4 GHz = 78.6 TFLOP/s issuing
# one fp32 operation per lane per instruction.  The published 157.3 TFLOP/s counts packed fp32
# (two operations per lane per instruction), which this build disables for every kernel, so
# 78.6 is the ceiling the kernels can reach; the published figure is reported beside it.
VALU_PEAK_TFLOPS = 78.6
VALU_PUBLISHED_TFLOPS = 157.3
FLUSH_BYTES = 512 << 20          # written between cold-cache calls: more than L2 + 256 MB MALL
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_s6_amd", "csrc", f)
                  for f in ("scan_kernels.h", "scan_kernels.hip", "device_common.h")]
SSD_KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_s6_amd", "csrc", f)
                      for f in ("ssd_kernels.hip", "device_common.h")]
BWD_KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_s6_amd", "csrc", f)
                      for f in ("bwd_kernels.hip", "scan_kernels.h", "scan_kernels.hip", "device_common.h")]
BWD_TI_KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_s6_amd", "csrc", f)
                         for f in ("bwd_ti_kernels.hip", "bwd_kernels.hip", "scan_kernels.hip", "device_common.h")]
CONV_KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_s6_amd", "csrc", f)
                       for f in ("conv_kernels.hip", "device_common.h")]
COUNTERS = os.path.join(ROOT, "profiles", "scan_counters.json")

# Algorithmic ALU work, in FMA-slot units (one fp32 VALU instruction per lane = 1 slot = 2
# flop-equivalents).  The transcendentals (v_exp_f32, v_log_f32, v_rcp_f32) issue at half that
# rate on this GPU (bench.py --microbench: 7.7 against 15.6 lanes per clock per SIMD with eight
# wavefronts, and they overlap FMA issue only slightly), so each counts 2 slots:
#   per (b, l, d, n): delta*A (1) + exp (2) + (Abar-1)/A as one FMA (1) + B*u (1) + times (1)
#                     + state FMA (1) + readout FMA (1)                               = 8
#   per (b, l, d):    feed-through FMA (1); gate: -z*log2e (1) + exp (2) + 1+e (1) + rcp (2)
#                     + z*r (1) + y*silu (1)                                          = 1 + 8
#   time-invariant:   per (b, l, d, n): state FMA (1) + readout FMA (1)               = 2
#   first order (Euler), per (b, l, d, n): delta*A (1) + exp (2) + B*(delta u) (1) + state FMA (1)
#                     + readout FMA (1) = 6, plus delta*u (1) per (b, l, d)
#   softplus step size, per (b, l, d): + bias (1), |x|*log2e (1), exp (2), 1+e (1), log (2),
#                     t-1 (1), rcp (2), two products (2), max (1), add (1)            = 14
SLOTS_PER_ELEMENT = {"selective": 8, "time_invariant": 2, "euler": 6}
SLOTS_PER_TOKEN_D = 1
SLOTS_PER_TOKEN_GATE = 8
SLOTS_PER_TOKEN_EULER = 1
SLOTS_PER_TOKEN_SOFTPLUS = 14
#   backward, per (b, l, d, n): exp (2), c (1), h_t (2), readout (1), lambda (1), du (2),
#                     ddelta (3), dc/da (3), dA (3), dB (1), dC (1), carry (1)        = 21
#             per (b, l, d): gate and its derivative (about 12), Dskip terms (2)      = 14
SLOTS_BWD_PER_ELEMENT = 21
SLOTS_BWD_PER_TOKEN_D = 14
#   backward of fixed coefficients, per (b, l, d, n): h_t (2), lambda (1), readout (1), du (1),
#             sum lambda h_{t-1} (1), sum lambda u (1, dB's), dC (1), carry (1)         = 9
#             (dA and ddelta follow per (d, n) and chunk from the two sums: delta, B and
#             dc/da are fixed)
SLOTS_BWD_TI_PER_ELEMENT = 9


def algorithmic_bytes(inp: s6_workloads.Inputs, want_last: bool, bias: bool = False) -> int:
    """Bytes the method must move: u, delta, z read once and y written once per (b, l, d);
    B and C once; A, Dskip (and a step-size bias) once; last_state once.  No expanded (x N)
    state touches HBM."""
    b, L, D, N = inp.shape
    es = 2 if inp.io == "bf16" else 4
    tok = b * L * D
    total = tok * es * 2                                       # u read, y written
    total += (D if inp.ti else tok) * es                       # delta
    if inp.z is not None:
        total += tok * es
    total += 2 * (D * N if inp.ti else b * L * N) * es        # B, C
    total += D * N * 4                                          # A
    if inp.Dskip is not None:
        total += D * 4
    if bias:
        total += D * 4
    if want_last:
        total += b * D * N * 4
    return total


def backward_bytes(inp: s6_workloads.Inputs) -> int:
    """Bytes the backward pass must move: u, delta, z, dy read and du, ddelta, dz written per
    (b, l, d); B, C read and dB, dC written per (b, l, n); A, Dskip read and dA, dDskip written
    once.  Fixed coefficients: delta, ddelta per channel and B, C, dB, dC per (d, n)."""
    b, L, D, N = inp.shape
    es = 2 if inp.io == "bf16" else 4
    zt = 2 if inp.z is not None else 0
    if inp.ti:
        return b * L * D * es * (3 + zt) + 2 * D * es + 4 * D * N * es + 2 * (D * N + D) * 4
    return b * L * D * es * (4 + zt) + b * L * N * es * 4 + 2 * (D * N + D) * 4


def decode_bytes(inp: s6_workloads.Inputs, bias: bool = False) -> int:
    """One decode step: the running state [batch, D, N] fp32 read and written once; u,
    delta, z read and y written per (b, d); B, C per (b, n); A, Dskip once."""
    b, _, D, N = inp.shape
    es = 2 if inp.io == "bf16" else 4
    total = 2 * b * D * N * 4
    total += b * D * es * (3 + (1 if inp.z is not None else 0))
    total += 2 * b * N * es + D * N * 4 + (D * 4 if inp.Dskip is not None else 0) + (D * 4 if bias else 0)
    return total


def algorithmic_slots(inp: s6_workloads.Inputs, softplus: bool = False, euler: bool = False) -> int:
    b, L, D, N = inp.shape
    per_el = SLOTS_PER_ELEMENT["time_invariant" if inp.ti else "euler" if euler else "selective"]
    slots = per_el * b * L * D * N
    if euler and not inp.ti:
        slots += SLOTS_PER_TOKEN_EULER * b * L * D
    if softplus:
        slots += SLOTS_PER_TOKEN_SOFTPLUS * (D if inp.ti else b * L * D)
    if inp.Dskip is not None:
        slots += SLOTS_PER_TOKEN_D * b * L * D
    if inp.z is not None:
        slots += SLOTS_PER_TOKEN_GATE * b * L * D
    return slots


def kernel_source_hash(workload: str = "") -> str:
    """Hash of the sources of the kernels a workload runs (the scan kernels; for the
    scalar-decay workloads theirs; for a backward tag, "backward_<workload>", the backward's
    and the forward state pass's (fixed coefficients: their own backward's); for a tag ending
    in "+conv", the convolution mode's): the
    counters in the committed summary are valid only for the source they were taken on."""
    h = hashlib.sha256()
    srcs = (SSD_KERNEL_SOURCES if workload.startswith("ssd_")
            else BWD_TI_KERNEL_SOURCES if workload.startswith("backward_s4d_ti")
            else BWD_KERNEL_SOURCES if workload.startswith("backward_")
            else CONV_KERNEL_SOURCES if workload.endswith("+conv") else KERNEL_SOURCES)
    for path in srcs:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, per_launch_alg_bytes: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; otherwise None."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash(workload):
        return None
    return int(entry["hbm_bytes_per_launch"])


def host_cpu() -> dict:
    """This host's processor and the threads the oracle may use: the CPUs this process may
    run on, capped by OMP_NUM_THREADS where the environment sets the process's CPU share."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    nproc = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = nproc
    threads = allowed
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        threads = min(threads, int(share))
    return {"cpu_model": model, "nproc": nproc, "affinity": allowed, "omp_num_threads": share or None,
            "threads": threads}


def cpu_per_core(target_s: float = 1.5) -> dict:
    """The oracle's forward on one thread, elements/s, on the small and Mamba-130M widths
    workloads (the latter on a channel slice sized to about target_s)."""
    import oracle
    out = {}
    for name, D in (("small_f32", None), ("mamba130m_f32", 64)):
        inp = s6_workloads.generate(name, D=D)
        t0 = time.perf_counter()
        oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, nthreads=1)
        dt = time.perf_counter() - t0
        if D is not None and dt < target_s:                       # grow the slice once
            D = min(1536, max(64, int(64 * target_s / max(dt, 1e-3)) // 4 * 4))
            inp = s6_workloads.generate(name, D=D)
            t0 = time.perf_counter()
            oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, nthreads=1)
            dt = time.perf_counter() - t0
        b, L, Dq, N = inp.shape
        out[name] = {"value": b * L * Dq * N / dt, "unit": "elements/s",
                     "sample": "%d x %d x %d x %d, %.2f s" % (b, L, Dq, N, dt)}
    return out


def cpu_baseline(inp: s6_workloads.Inputs, target_s: float = 12.0, h0=None, bias=None, softplus=False,
                 euler=False, per_core: bool = False):
    """The oracle (fp64, as it stands) on a bounded sample of the workload's channels,
    timed on this host on every thread the process may use; scaled to elements/s.  ``h0``:
    initial state [batch, D, N]; ``bias``/``softplus``/``euler``: the step-size and
    discretisation options.  ``per_core`` adds one-thread figures on two other workloads."""
    import oracle
    host = host_cpu()
    cores = host["threads"]
    b, L, D, N = inp.shape
    oracle.build()
    nch = min(D, max(cores, 8))
    t_used = 0.0
    while True:
        ch = np.arange(nch)
        sub = s6_workloads.select_channels(inp, ch)
        t0 = time.perf_counter()
        oracle.fwd(sub.u, sub.delta, sub.A, sub.B, sub.C, sub.Dskip, sub.z, time_invariant=sub.ti,
                   h0=None if h0 is None else np.ascontiguousarray(h0[:, ch]), want_last=h0 is not None,
                   delta_bias=None if bias is None else np.ascontiguousarray(bias[ch]), delta_softplus=softplus,
                   euler=euler, nthreads=cores)
        t_used = time.perf_counter() - t0
        if t_used >= target_s * 0.5 or nch >= D:
            break
        nch = min(D, int(nch * max(2.0, target_s / max(t_used, 1e-3))))
    elements = b * L * nch * N
    out = {"value": elements / t_used, "unit": "elements/s", "cores": cores, "kind": "oracle",
           "sample": "%d of %d channels (all %d batch rows x %d tokens x %d states), fp64 recurrence, %.1f s wall"
                     % (nch, D, b, L, N, t_used), "host": host}
    if per_core:
        out["per_core"] = cpu_per_core()
    return out


MICROBENCH_LIB = os.path.join(ROOT, "selective_state_space_s6_amd", "libselscan_microbench.so")
SIMDS = 256 * 4                  # MI355X: 256 compute units of 4 SIMDs


def run_microbench():
    """The practical roofs, from libselscan_microbench.so (built with the scan's flags): fp32
    FMA, v_exp_f32 and DPP-operand multiply issue rates against wavefronts per SIMD (8
    independent chains per lane),
    exp2/FMA overlap, streaming copy and write bandwidth, and the shader clock held meanwhile
    (clock64 cycles against the constant-rate wall clock of the same wavefront)."""
    import ctypes
    import torch
    torch.cuda.init()                                # the library binds to the runtime torch loaded
    lib = ctypes.CDLL(MICROBENCH_LIB)
    lib.selscan_mb_compute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]
    lib.selscan_mb_bandwidth.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_float)]
    wall_khz = lib.selscan_mb_wall_clock_khz()
    chains_rounds = 8 * 8                            # operations per lane per loop iteration

    def compute(kind, waves_per_simd, iters):
        ms, cyc, tck = ctypes.c_float(), ctypes.c_uint64(), ctypes.c_uint64()
        rc = lib.selscan_mb_compute(kind, 256 * waves_per_simd, iters, ctypes.byref(ms), ctypes.byref(cyc),
                                    ctypes.byref(tck))
        if rc != 0:
            raise RuntimeError("microbench kind %d failed: %d (hip %d)" % (kind, rc, lib.selscan_mb_last_error()))
        mhz = cyc.value / (tck.value / (wall_khz * 1e3)) / 1e6 if tck.value and wall_khz else float("nan")
        lanes = 256 * waves_per_simd * 256 * iters * chains_rounds     # lane operations of one kind
        per_clk = lanes / (ms.value * 1e-3) / (mhz * 1e6) / SIMDS
        return {"waves_per_simd": waves_per_simd, "ms": round(ms.value, 4), "clock_mhz": round(mhz, 1),
                "lane_ops_per_s": lanes / (ms.value * 1e-3), "lanes_per_clk_per_simd": round(per_clk, 3)}

    out = {"fma": [compute(0, w, 4000) for w in (1, 2, 3, 4, 8)],
           "exp2": [compute(1, w, 1000) for w in (1, 2, 3, 4, 8)],
           "mul_dpp_row_broadcast": [compute(6, w, 2000) for w in (1, 2, 4, 8)]}
    # overlap: exp2 and r fma per exp2 (8 chains of each), 4 wavefronts per SIMD; compare the
    # time with the exp2 and fma runs of the same counts taken alone
    fma4 = next(r for r in out["fma"] if r["waves_per_simd"] == 4)
    exp4 = next(r for r in out["exp2"] if r["waves_per_simd"] == 4)
    t_fma_op = fma4["ms"] / (256 * 4 * 256 * 4000 * chains_rounds)
    t_exp_op = exp4["ms"] / (256 * 4 * 256 * 1000 * chains_rounds)
    mix = []
    for kind, ratio in ((2, 1), (3, 2), (4, 4), (5, 8)):
        r = compute(kind, 4, 1000)
        n = 256 * 4 * 256 * 1000 * chains_rounds
        r.update(ratio=ratio, ms_if_serial=round(n * (t_exp_op + ratio * t_fma_op), 4),
                 ms_if_overlapped=round(n * max(t_exp_op, ratio * t_fma_op), 4))
        mix.append(r)
    out["exp2_with_fma"] = mix
    bw = []
    for kind, name in ((0, "copy"), (1, "write")):
        nbytes = 1 << 30
        moved = nbytes * (2 if kind == 0 else 1)
        for blocks in (1024, 4096, 16384, 65536):       # workgroups of a grid-stride loop
            ms = ctypes.c_float()
            if lib.selscan_mb_bandwidth(kind, nbytes, blocks, 5, ctypes.byref(ms)) != 0:
                raise RuntimeError("bandwidth probe failed (hip %d)" % lib.selscan_mb_last_error())
            bw.append({"probe": name, "workgroups": blocks, "bytes": moved, "ms": round(ms.value, 4),
                       "gbs": round(moved / (ms.value * 1e-3) / 1e9, 1)})
    out["bandwidth"] = bw
    out["wall_clock_khz"] = wall_khz
    out["arbitration"] = arbitration_probe(lib)
    print(json.dumps({"microbench": out}), flush=True)


def arbitration_probe(lib) -> list:
    """The arbitration probe of libselscan_microbench.so: 2.5 workgroups of four wavefronts per
    compute unit (the long-context scan's grid shape), each repeating 64 FMAs and a barrier,
    with 40 KB of LDS per workgroup (at most four per compute unit), without and with the
    scan's issue-priority rotation.  Reports where the dispatcher put the workgroups (per
    compute unit, per SIMD) and the wavefronts' durations by how many share their SIMD."""
    import ctypes
    import collections
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = (5 * cus) // 2, 3000
    lib.selscan_mb_arbiter.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_float)]
    res = []
    for rotate in (0, 1):
        rec = (ctypes.c_uint64 * (blocks * 16))()
        ms = ctypes.c_float()
        if lib.selscan_mb_arbiter(rotate, blocks, iters, 40960, rec, ctypes.byref(ms)) != 0:
            raise RuntimeError("arbitration probe failed (hip %d)" % lib.selscan_mb_last_error())
        a = np.frombuffer(rec, dtype=np.uint64).reshape(blocks * 4, 4).astype(np.int64)
        t0, t1, hw, xcc = a[:, 0], a[:, 1], a[:, 2], a[:, 3] & 0xF
        # HW_ID: SIMD bits 5:4, compute unit 11:8, shader array 12, shader engine 15:13
        cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
        simd = cu * 4 + ((hw >> 4) & 3)
        wg_per_cu = collections.Counter(cu[0::4].tolist())
        waves_per_simd = collections.Counter(simd.tolist())
        dur = (t1 - t0) * 1e-2                                   # 100 MHz ticks -> us
        by = collections.defaultdict(list)
        for i in range(blocks * 4):
            by[waves_per_simd[int(simd[i])]].append(float(dur[i]))
        res.append({"rotate": rotate, "workgroups": blocks, "kernel_ms": round(ms.value, 4),
                    "span_us": round(float((t1.max() - t0.min()) * 1e-2), 1),
                    "starts_within_us": round(float((t0.max() - t0.min()) * 1e-2), 2),
                    "workgroups_per_cu": {str(k): v for k, v in sorted(collections.Counter(wg_per_cu.values()).items())},
                    "waves_per_simd": {str(k): v for k, v in sorted(collections.Counter(waves_per_simd.values()).items())},
                    "wave_us_by_waves_on_simd": {str(k): {"min": round(min(v), 1), "mean": round(float(np.mean(v)), 1),
                                                          "max": round(max(v), 1), "waves": len(v)}
                                                 for k, v in sorted(by.items())}})
    return res


def time_calls(step, stream, steps: int, warmup: int) -> dict:
    """Warm up, then time `steps` calls back to back (wall clock between device
    synchronisations, and HIP events around each call on `stream`), then `steps` more calls
    each after FLUSH_BYTES written to a scratch buffer outside the events."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    starts, ends = ev(), ev()
    torch.cuda.synchronize()                     # one GPU: the barrier is the device synchronisation
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm = [a.elapsed_time(e) for a, e in zip(starts, ends)]
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    cstarts, cends = ev(), ev()
    with torch.cuda.stream(stream):
        for i in range(steps):
            flush.fill_(float(i))
            cstarts[i].record(stream)
            step()
            cends[i].record(stream)
    torch.cuda.synchronize()
    cold = [a.elapsed_time(e) for a, e in zip(cstarts, cends)]
    del flush
    return {"wall": wall, "warm": warm, "cold": cold}


def timing_fields(tm: dict) -> dict:
    """kernel_ms (mean of the back-to-back calls: the roofline's time), its median and
    minimum, and the cold-cache statistics."""
    w, c = np.asarray(tm["warm"]), np.asarray(tm["cold"])
    return {"kernel_ms": float(w.mean()), "kernel_ms_median": float(np.median(w)), "kernel_ms_min": float(w.min()),
            "cold_cache": {"flush_bytes": FLUSH_BYTES, "calls": int(c.size), "ms_mean": float(c.mean()),
                           "ms_median": float(np.median(c)), "ms_min": float(c.min())}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="longctx_bf16",
                    choices=sorted(s6_workloads.WORKLOADS) + sorted(s6_workloads.SSD_WORKLOADS))
    ap.add_argument("--path", default="auto", choices=["auto", "single", "chunked", "conv"],
                    help="conv: the convolution mode (fixed coefficients only)")
    ap.add_argument("--ssd-path", default="auto", choices=["auto", "fused", "chunked", "segmented"],
                    help="scalar-decay workloads: automatic, on chip over the whole sequence (fused), chunk-parallel, or on chip over sequence segments")
    ap.add_argument("--step-size", default="given", choices=["given", "softplus"],
                    help="softplus: the kernel computes softplus(raw + bias) from a pre-activation")
    ap.add_argument("--discretization", default="zoh", choices=["zoh", "euler"])
    ap.add_argument("--backward", action="store_true", help="time the backward pass instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--microbench", action="store_true",
                    help="print the issue-rate and bandwidth probes (the practical roofs) instead")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the scan shards over batch/channels with no "
              "communication, or over the sequence with one exchange of per-segment state maps); --gpus %d is not "
              "supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    if args.microbench:
        return run_microbench()
    import torch
    import selective_state_space_s6_amd as ss

    if args.workload in s6_workloads.SSD_WORKLOADS:
        return bench_ssd(args)
    spec = s6_workloads.spec(args.workload)
    inp = s6_workloads.generate(args.workload)
    softplus = args.step_size == "softplus"
    euler = args.discretization == "euler"
    bias_np = None
    if softplus:
        raw, bias_np = s6_workloads.raw_step_sizes(inp)
        inp = dataclasses.replace(inp, delta=raw)
    opts = variant_options(args)
    if spec.get("decode"):
        return bench_decode(args, inp, bias_np, opts)
    if args.backward:
        return bench_backward(args, inp, bias_np, opts)
    want_last = bool(spec["last"])
    b, L, D, N = inp.shape
    E = b * L * D * N
    io = inp.io

    def dev(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        return t.to(torch.bfloat16) if io == "bf16" else t

    u, delta, B, C, z = dev(inp.u), dev(inp.delta), dev(inp.B), dev(inp.C), dev(inp.z)
    A = torch.from_numpy(inp.A).cuda()
    Ds = None if inp.Dskip is None else torch.from_numpy(inp.Dskip).cuda()
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    y = torch.empty_like(u)
    last = torch.empty((b, D, N), dtype=torch.float32, device="cuda") if want_last else None
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        ss.selective_scan_fwd(u, delta, A, B, C, Ds, z, y=y, last_state=last, path=args.path,
                              stream=stream.cuda_stream, delta_bias=bias, delta_softplus=softplus,
                              discretization=args.discretization)

    tm = time_calls(step, stream, args.steps, args.warmup)
    wall = tm["wall"]
    launch_ms = float(np.mean(tm["warm"]))

    if args.copy_calibration:
        copy_calibration()

    dims = ss.make_dims(u, delta, A, B, C, z, y, path=args.path, discretization=args.discretization,
                        delta_softplus=softplus)
    taken = ss.plan_path(dims)
    alg_bytes = algorithmic_bytes(inp, want_last, bias=softplus)
    slots = algorithmic_slots(inp, softplus=softplus, euler=euler)
    launch_s = launch_ms * 1e-3
    hbm_gbs = alg_bytes / launch_s / 1e9
    traffic = measured_traffic(args.workload + opts["suffix"] + ("+conv" if taken == "conv" else ""), alg_bytes)
    if taken == "conv":                                          # matrix products on the fp32 matrix cores
        roof = matrix_roofline(alg_bytes, conv_flops(inp), launch_s, traffic, MFMA_F32_PEAK_TFLOPS)
    else:
        roof = roofline(alg_bytes, slots, launch_s, traffic)    # the binding roof

    out = {
        "metric": METRIC,
        "value": E * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, s6_workloads: %s)" % args.workload,
        "config": {"workload": args.workload, "batch": b, "seq_len": L, "dim": D, "dstate": N, "io": io,
                   "state": "f32", "gate": inp.z is not None, "feedthrough": inp.Dskip is not None,
                   "last_state": want_last, "time_invariant": inp.ti, "path": taken,
                   "step_size": opts["step_size"], "discretization": args.discretization},
        **timing_fields(tm),
        "hbm_gbs": round(hbm_gbs, 1),
        "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": alg_bytes,
        "algorithmic_slots": slots,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, bias=bias_np, softplus=softplus, euler=euler, per_core=True)
    print(json.dumps(out), flush=True)


def variant_options(args) -> dict:
    """Names of the chosen options: the config entry and the key suffix of the committed
    counter summary ("" for the defaults)."""
    suffix = ("+softplus" if args.step_size == "softplus" else "") + ("+euler" if args.discretization == "euler" else "")
    return {"suffix": suffix,
            "step_size": "softplus(delta + bias[d]) in the kernel" if args.step_size == "softplus" else "given"}


def bench_backward(args, inp, bias_np, opts):
    """The backward pass (selective_scan_bwd: every gradient, states recomputed from
    checkpoints) over the whole workload, from a seeded output gradient."""
    import torch
    import selective_state_space_s6_amd as ss
    b, L, D, N = inp.shape
    io = inp.io

    def dev(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        return t.to(torch.bfloat16) if io == "bf16" else t

    u, delta, B, C, z = dev(inp.u), dev(inp.delta), dev(inp.B), dev(inp.C), dev(inp.z)
    A = torch.from_numpy(inp.A).cuda()
    Ds = None if inp.Dskip is None else torch.from_numpy(inp.Dskip).cuda()
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    softplus = bias_np is not None
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    dy = torch.randn(u.shape, generator=gen, device="cuda", dtype=torch.float32).to(u.dtype)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        ss.selective_scan_bwd(u, delta, A, B, C, Ds, z, dy=dy, delta_bias=bias, delta_softplus=softplus,
                              discretization=args.discretization, stream=stream)

    tm = time_calls(step, stream, args.steps, args.warmup)
    wall = tm["wall"]
    launch_ms = float(np.mean(tm["warm"]))
    if args.copy_calibration:
        copy_calibration()
    E = b * L * D * N
    alg = backward_bytes(inp)
    slots = (SLOTS_BWD_TI_PER_ELEMENT if inp.ti else SLOTS_BWD_PER_ELEMENT) * E + SLOTS_BWD_PER_TOKEN_D * b * L * D
    out = {
        "metric": METRIC,
        "value": E * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, s6_workloads: %s; dy standard normal)" % args.workload,
        "config": {"workload": args.workload, "batch": b, "seq_len": L, "dim": D, "dstate": N, "io": io,
                   "state": "f32", "gate": inp.z is not None, "feedthrough": inp.Dskip is not None,
                   "pass": "backward", "step_size": opts["step_size"], "discretization": args.discretization},
        **timing_fields(tm),
        "hbm_gbs": round(alg / (launch_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(alg / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": alg,
        "algorithmic_slots": slots,
        "roofline": roofline(alg, slots, launch_ms * 1e-3, measured_traffic("backward_" + args.workload + opts["suffix"], alg)),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(inp, bias_np, softplus, args.discretization == "euler")
    print(json.dumps(out), flush=True)


def cpu_baseline_backward(inp, bias, softplus, euler, target_s: float = 10.0):
    """The oracle's backward (fp64, single thread, as it stands) on the first batch row and a
    growing prefix of channels, timed on this host; scaled to elements/s."""
    import oracle
    oracle.build()
    b, L, D, N = inp.shape
    rng = np.random.default_rng(3)
    nch = 4
    while True:
        sub = s6_workloads.select_channels(inp, np.arange(nch))
        one = lambda a: None if a is None else a[:1]
        dy = rng.standard_normal((1, L, nch)).astype(np.float32)
        t0 = time.perf_counter()
        if inp.ti:                                    # delta, B, C per channel
            oracle.bwd(one(sub.u), sub.delta, sub.A, sub.B, sub.C, sub.Dskip, one(sub.z), dy=dy,
                       delta_bias=None if bias is None else bias[:nch], delta_softplus=softplus, euler=euler,
                       time_invariant=True)
        else:
            oracle.bwd(one(sub.u), one(sub.delta), sub.A, one(sub.B), one(sub.C), sub.Dskip, one(sub.z), dy=dy,
                       delta_bias=None if bias is None else bias[:nch], delta_softplus=softplus, euler=euler)
        t_used = time.perf_counter() - t0
        if t_used >= target_s * 0.5 or nch >= D:
            break
        nch = min(D, int(nch * max(2.0, target_s / max(t_used, 1e-3))))
    return {"value": L * nch * N / t_used, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": "batch row 0, %d of %d channels x %d tokens x %d states, fp64 backward, %.1f s wall"
                      % (nch, D, L, N, t_used)}


MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X published dense bf16 matrix peak
MFMA_F32_PEAK_TFLOPS = 157.3      # MI355X published dense fp32 matrix peak


def conv_flops(inp: s6_workloads.Inputs) -> float:
    """Algorithmic matrix work of the convolution mode: per (batch row, channel, 16-token block)
    the causal half of the 16 x 16 Toeplitz product of the lag kernel (136 multiply-adds), the
    block's end state from its tokens (16 N) and the readout of the carried state (16 N); 2 flops
    per multiply-add."""
    b, L, D, N = inp.shape
    blocks = (L + 15) // 16
    return 2.0 * b * D * blocks * (136 + 32 * N)


def matrix_roofline(alg_bytes: int, flops: float, seconds: float, traffic, peak: float):
    """The binding roof of a matrix-core kernel: its matrix work against `peak` or its bytes
    against HBM, whichever bounds the time more."""
    tflops = flops / seconds / 1e12
    if flops / (peak * 1e12) >= alg_bytes / (HBM_PEAK_GBS * 1e9):
        return {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": traffic}
    gbs = alg_bytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
SSD_CHUNK = 64


def ssd_flops(b, L, H, N, P=64, T=SSD_CHUNK) -> float:
    """Algorithmic matrix work of the chunked scalar-decay layer: per (batch row, head, chunk)
    the causal halves of C B^T (T(T+1)/2 x N) and of (mask o C B^T) X (T(T+1)/2 x P), the chunk
    state B^T diag(w) X (N x P x T) and the carried-state readout C H (T x N x P); 2 flops per
    multiply-add."""
    nch = (L + T - 1) // T
    per = T * (T + 1) / 2 * N * 2 + T * (T + 1) / 2 * P * 2 + N * P * T * 2 + T * N * P * 2
    return b * H * nch * per


def ssd_bytes(b, L, H, N, P=64) -> int:
    """Bytes the layer must move: x, z read and y written (bf16) per (b, l, h, p); delta per
    (b, l, h); B, C per (b, l, n); A, Dskip once."""
    return 3 * b * L * H * P * 2 + b * L * H * 2 + 2 * b * L * N * 2 + H * 4 + H * P * 4


def bench_ssd(args):
    """The scalar-decay (Mamba-2) layer, selective_scan_ssd_fwd, over the whole workload."""
    import torch
    import selective_state_space_s6_amd as ss
    inp = s6_workloads.generate_ssd(args.workload)
    b, L, H, P = inp.x.shape
    N = inp.B.shape[2]
    g = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    x, dl, B, C, z = g(inp.x), g(inp.delta), g(inp.B), g(inp.C), g(inp.z)
    A = torch.from_numpy(inp.A).cuda()
    Ds = torch.from_numpy(inp.Dskip).cuda()
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        ss.selective_scan_ssd_fwd(x, dl, A, B, C, Ds, z, y=y, discretization=args.discretization,
                                  path=args.ssd_path, stream=stream)

    tm = time_calls(step, stream, args.steps, args.warmup)
    wall = tm["wall"]
    launch_ms = float(np.mean(tm["warm"]))
    if args.copy_calibration:
        copy_calibration()
    E = b * L * H * P * N
    alg = ssd_bytes(b, L, H, N, P)
    fl = ssd_flops(b, L, H, N, P)
    sec = launch_ms * 1e-3
    t_hbm, t_mfma = alg / (HBM_PEAK_GBS * 1e9), fl / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": round(fl / sec / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(fl / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.workload, alg)}
    else:
        roof = {"bound": "hbm", "achieved": round(alg / sec / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(alg / sec / 1e9 / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload, alg)}
    out = {
        "metric": METRIC,
        "value": E * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, s6_workloads: %s)" % args.workload,
        "config": {"workload": args.workload, "batch": b, "seq_len": L, "heads": H, "headdim": P, "dstate": N,
                   "io": "bf16", "state": "f32", "gate": True, "feedthrough": True, "chunk": SSD_CHUNK,
                   "discretization": args.discretization, "layer": "scalar decay per head (Mamba-2 SSD)",
                   "path": args.ssd_path},
        **timing_fields(tm),
        "hbm_gbs": round(alg / sec / 1e9, 1),
        "hbm_frac": round(alg / sec / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_tflops": round(fl / sec / 1e12, 2),
        "algorithmic_bytes": alg,
        "algorithmic_flops": fl,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_ssd(inp)
    print(json.dumps(out), flush=True)


def cpu_baseline_ssd(inp, target_s: float = 10.0):
    """The oracle's recurrence with one decay per head (fp64, as it stands), on the first batch
    row and a growing number of heads, timed on this host; scaled to elements/s."""
    import oracle
    oracle.build()
    b, L, H, P = inp.x.shape
    N = inp.B.shape[2]
    cores = min(16, os.cpu_count() or 1)
    nh = 1
    while True:
        t0 = time.perf_counter()
        oracle.ssd_fwd(inp.x[:1, :, :nh], inp.delta[:1, :, :nh], inp.A[:nh], inp.B[:1], inp.C[:1],
                       inp.Dskip[:nh * P], inp.z[:1, :, :nh], want_last=False, nthreads=cores)
        t_used = time.perf_counter() - t0
        if t_used >= target_s * 0.5 or nh >= H:
            break
        nh = min(H, int(nh * max(2.0, target_s / max(t_used, 1e-3))))
    return {"value": L * nh * P * N / t_used, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "sample": "batch row 0, %d of %d heads x %d tokens x %d channels x %d states, fp64, %.1f s wall"
                      % (nh, H, L, P, N, t_used)}


def copy_calibration():
    """A plain 1 GiB device copy (3 times), for scaling HBM byte counters."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def roofline(alg_bytes: int, slots: int, seconds: float, traffic):
    """The binding roof (the larger of the two lower bounds on time) and the fraction of it.
    The ALU roof is the non-packed fp32 ceiling (VALU_PEAK_TFLOPS); the published, packed
    figure and the fraction of it are reported beside it."""
    hbm_gbs = alg_bytes / seconds / 1e9
    alu_tflops = 2.0 * slots / seconds / 1e12
    if 2.0 * slots / (VALU_PEAK_TFLOPS * 1e12) >= alg_bytes / (HBM_PEAK_GBS * 1e9):
        return {"bound": "alu", "achieved": round(alu_tflops, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(alu_tflops / VALU_PEAK_TFLOPS, 4), "traffic": traffic,
                "peak_basis": "fp32 VALU without packed fp32 (the build disables it): 256 CU x 4 SIMD x 16 lanes "
                              "x 2 flop x 2.4 GHz",
                "published_peak": VALU_PUBLISHED_TFLOPS,
                "frac_of_published": round(alu_tflops / VALU_PUBLISHED_TFLOPS, 4)}
    return {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


def bench_decode(args, inp, bias_np, opts):
    """One recurrent decode step per call (selective_scan_step) over the workload's batch:
    one token per batch row, the running state updated in place."""
    import torch
    import selective_state_space_s6_amd as ss
    b, _, D, N = inp.shape
    io = inp.io

    def dev(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x[:, 0], dtype=np.float32)).cuda()
        return t.to(torch.bfloat16) if io == "bf16" else t

    u, delta, B, C, z = dev(inp.u), dev(inp.delta), dev(inp.B), dev(inp.C), dev(inp.z)
    A = torch.from_numpy(inp.A).cuda()
    Ds = None if inp.Dskip is None else torch.from_numpy(inp.Dskip).cuda()
    h0 = s6_workloads.running_state(inp)
    state = torch.from_numpy(h0).cuda()
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    softplus = bias_np is not None
    y = torch.empty_like(u)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        ss.selective_scan_step(u, delta, A, B, C, Ds, z, y=y, state=state, stream=stream.cuda_stream,
                               delta_bias=bias, delta_softplus=softplus, discretization=args.discretization)

    tm = time_calls(step, stream, args.steps, args.warmup)
    wall = tm["wall"]
    launch_ms = float(np.mean(tm["warm"]))
    if args.copy_calibration:
        copy_calibration()
    E = b * D * N
    alg = decode_bytes(inp, bias=softplus)
    slots = algorithmic_slots(inp, softplus=softplus, euler=args.discretization == "euler")
    out = {
        "metric": METRIC,
        "value": E * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, s6_workloads: %s)" % args.workload,
        "config": {"workload": args.workload, "batch": b, "seq_len": 1, "dim": D, "dstate": N, "io": io,
                   "state": "f32", "gate": inp.z is not None, "feedthrough": inp.Dskip is not None,
                   "mode": "decode step (state in place)", "step_size": opts["step_size"],
                   "discretization": args.discretization},
        **timing_fields(tm),
        "hbm_gbs": round(alg / (launch_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(alg / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": alg,
        "algorithmic_slots": slots,
        "roofline": roofline(alg, slots, launch_ms * 1e-3, measured_traffic(args.workload + opts["suffix"], alg)),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, h0=h0, bias=bias_np, softplus=softplus,
                                           euler=args.discretization == "euler")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
