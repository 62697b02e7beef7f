#!/usr/bin/env python3
"""Selective-scan forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer]

A step is one call of ssm_scan_fwd (the whole forward: discretisation, scan, C
contraction, D skip, silu gate, final state) over one batch of seeded synthetic inputs
already resident in HBM. The default workload is a Mamba-1 layer's scan: batch 4, 2048
channels, 16 states, 2048 steps, bf16 storage, fp32 arithmetic.

Timing: a device-copy reference first, then the path itself untimed for about half a second
(--prewarm-seconds: the GPU's clocks rise over the first tenths of a second of sustained
load), W untimed warm-up calls, then exactly K calls back to back between two device
synchronisations, with one HIP event on the launch stream before the first call and one
after the last; the roofline's mean time per call is their interval over K. Isolated calls,
each between its own pair of events, are timed after the timed region. Calls rotate over
several independent input/output sets whose total size is well above the 256 MB Infinity
Cache, so every call reads HBM ("cold"). The value is the algorithmic bytes of K calls
divided by the wall time of the timed region. One JSON line is printed on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public specification
# ALU roofline. MI355X: 256 CUs x 4 SIMDs, 2.4 GHz; the fp32 vector peak of 157.3 TFLOP/s
# is 32 fp32 FMA lanes per SIMD per clock (a wave64 VALU instruction issues in 2 clocks);
# transcendentals (v_exp_f32) run at a quarter of that rate. The exact method needs, per
# (batch, channel, state, step) update: dt*A (mul), exp, (dt*u)*B (mul), h = dA*h + dBu
# (fma), y += C*h (fma): 4 VALU issue slots plus one exp = 4 more slots. Counting each
# slot as one FMA (2 flop), an update is 16 flop-equivalents against the 157.3 peak.
ALU_PEAK_TFLOPS = 157.3
FLOP_EQ_PER_UPDATE = 16
# The method's own arithmetic per update, as the roofline counts it: dt*A and (dt*u)*B (two
# mul), h = dA*h + dBu and y += C*h (two FMA, 4 flop): 6 flop, plus one exp. A transcendental
# retires at a quarter of the FMA rate, so the exp peak is 157.3e12 / 2 / 4 per second.
FLOPS_PER_UPDATE = 6
EXPS_PER_UPDATE = 1
EXP_PEAK_PER_S = ALU_PEAK_TFLOPS * 1e12 / 2 / 4
# The 157.3 TFLOP/s figure needs packed fp32 (v_pk_fma_f32: two fp32 FMAs per lane per
# instruction), which the library is compiled without. Without it a SIMD retires 16 fp32 FMA lanes per
# clock: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz = 78.6 TFLOP/s, a wave64 v_fma_f32
# every 4 clocks and a wave64 v_exp_f32 every 8 (bench.py --alu-probe measures both). The
# same update then costs 4 issue slots plus 2 for the exp: 12 flop-equivalents at 78.6.
ALU_PEAK_NO_PACKED_TFLOPS = 78.6
FLOP_EQ_PER_UPDATE_NO_PACKED = 12
# The backward's minimal work per update (the sequential adjoint): recompute the state
# (s*A, exp, (s*u)*B, fma: 6 slots), g = C dy + e (1), dC += dy h (1), dB += g s u (1),
# du += g s B (2), a h_prev (1), ds += g (A a h_prev + B u) (3), dA += g a h_prev s (2),
# e = a g (1): 18 issue slots = 36 flop-equivalents.
BWD_FLOP_EQ_PER_UPDATE = 36
INFINITY_CACHE_BYTES = 256 << 20
_CSRC = "selective_state_space_fwd_amd/csrc/"
_SHARED = [_CSRC + "device_math.h", _CSRC + "device_scan.h", _CSRC + "scan_launch.h"]
KERNEL_SOURCES = {"fwd": [_CSRC + "scan_kernels.hip", _CSRC + "scan_short.hip"] + _SHARED,
                  "bwd": [_CSRC + "scan_bwd.hip"] + _SHARED,
                  "ssd": [_CSRC + "ssd_kernels.hip"] + _SHARED}
# Dense bf16 MFMA peak of MI355X (AMD public specification, without sparsity).
MFMA_BF16_PEAK_TFLOPS = 2500.0
SHORT_MAX_SEQLEN = 32   # sequences up to this length take the short-sequence kernel


def kernel_hash(direction: str = "fwd") -> str:
    """sha256 (first 16 hex) of the sources of one direction's kernels: a committed traffic
    record counts only while it matches."""
    h = hashlib.sha256()
    for s in KERNEL_SOURCES[direction]:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, direction: str = "fwd"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel source; otherwise None."""
    prefix = {"fwd": "scan_fwd", "bwd": "scan_bwd", "ssd": "ssd_fwd"}[direction]
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash(direction):
        return None
    return rec.get("bytes_per_launch")


def to_device(x, torch, device):
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def cpu_baseline(w, inp, budget_s: float):
    """The oracle, untuned, on host cores over a bounded sample of the same workload:
    channels 0..k-1 of the leading batch rows, all seqlen steps."""
    import oracle
    from ssm_workloads import widen

    threads = oracle.default_threads()
    io = inp["io"]

    def sample(nb, nd):
        sl = lambda x: None if x is None else x[:nb, :nd]
        return (widen(sl(inp["u"]), io), widen(sl(inp["delta"]), io), inp["A"][:nd],
                widen(inp["B"][:nb], io), widen(inp["C"][:nb], io), inp["D"][:nd],
                widen(sl(inp["z"]), io), inp["delta_bias"][:nd], True,
                None if inp["h0"] is None else inp["h0"][:nb, :nd])

    def timed(nb, nd):
        args = sample(nb, nd)
        t0 = time.perf_counter()
        oracle.scan_ref(*args, nthreads=threads)
        return time.perf_counter() - t0

    timed(1, min(w.dim, threads))          # start the OpenMP thread pool outside any timing
    probe_d = min(w.dim, max(4 * threads, 64))
    t_probe = max(timed(1, probe_d), 1e-6)
    rows_wanted = int(budget_s / t_probe * probe_d)
    total_rows = w.batch * w.dim
    rows = max(probe_d, min(total_rows, rows_wanted))
    if rows >= w.dim:
        nb, nd = min(w.batch, rows // w.dim), w.dim
    else:
        nb, nd = 1, rows
    # when the whole workload is quicker than the budget, repeat it and take the mean
    reps = max(1, min(500, int(budget_s / max(timed(nb, nd), 1e-6)))) if rows == total_rows else 1
    secs = sum(timed(nb, nd) for _ in range(reps)) / reps
    sub = w.with_(batch=nb, dim=nd)
    # the same oracle on one thread, over the first channels of batch row 0 (about a second)
    one_d = max(1, min(w.dim, int(probe_d * 1.0 / max(t_probe * threads, 1e-6))))
    one_args = sample(1, one_d)
    t0 = time.perf_counter()
    oracle.scan_ref(*one_args, nthreads=1)
    one_secs = max(time.perf_counter() - t0, 1e-9)
    one_sub = w.with_(batch=1, dim=one_d)
    return {
        "value": round(sub.algorithmic_bytes() / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"float64 sequential oracle over batch rows 0..{nb - 1}, channels "
                   f"0..{nd - 1}, all {w.seqlen} steps ({nb * nd} of {total_rows} rows, "
                   f"{sub.algorithmic_bytes() / 1e6:.2f} MB algorithmic), mean of {reps} run(s) "
                   f"of {secs:.2f} s"),
        "seconds": round(secs, 3),
        "single_thread": {"value": round(one_sub.algorithmic_bytes() / one_secs / 1e9, 4),
                          "unit": "GB/s",
                          "sample": f"batch row 0, channels 0..{one_d - 1}, all {w.seqlen} steps",
                          "seconds": round(one_secs, 3)},
        "host": host_description(),
    }


def host_description():
    """CPU model and the number of cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def copy_reference(torch) -> dict:
    """Device copy of 512 MiB (torch's copy kernel; source and destination together exceed
    the Infinity Cache), median of 20 launches between HIP events after 10 untimed ones: the
    bandwidth a plain streaming kernel reaches on this GPU."""
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del src, dst
    return {"GBps": round(2 * n / (ms * 1e-3) / 1e9, 1), "bytes_read": n, "bytes_written": n,
            "kernel_us_median": round(ms * 1e3, 2)}


def copy_probe(torch, steps: int, warmup: int) -> int:
    """Plain copy of 1 GiB between two device buffers (torch's copy kernel): reads 1 GiB and
    writes 1 GiB per call."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n,
                      "kernel_us_median": round(float(np.median(ms)) * 1e3, 2),
                      "GBps_read_plus_write": round(2 * n / (float(np.median(ms)) * 1e-3) / 1e9, 1)}),
          flush=True)
    return 0


def alu_probe(torch, steps: int, warmup: int) -> int:
    """VALU issue rates under the library's compile flags: independent chains of wave64 v_fma_f32 and
    of wave64 v_exp_f32 (libssmprobe.so), at 16 waves per CU. Prints one JSON line."""
    import ctypes

    from selective_state_space_fwd_amd.build import PROBE_LIB_PATH

    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build first")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    lib.ssm_probe_alu.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.ssm_probe_alu.restype = ctypes.c_int
    lib.ssm_probe_ops_per_launch.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.ssm_probe_ops_per_launch.restype = ctypes.c_int64
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    blocks, iters = cus * 4, 200            # 4 workgroups of 4 waves: 16 waves per CU
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {"probe": "alu", "cus": cus, "waves_per_cu": 16,
           "note": "packed fp32 disabled at build time; lane-ops per second, and clocks per "
                   "wave64 instruction per SIMD at the 2.4 GHz peak clock"}
    lib.ssm_probe_fma_per_exp.argtypes = [ctypes.c_int]
    lib.ssm_probe_fma_per_exp.restype = ctypes.c_int
    secs = {}
    for kind, name in ((0, "v_fma_f32"), (1, "v_exp_f32"), (2, "mix_4fma_1exp"),
                       (3, "mix_2fma_1exp"), (4, "mix_1fma_1exp")):
        launch = lambda: lib.ssm_probe_alu(kind, blocks, iters, out.data_ptr(),
                                           stream.cuda_stream)
        for _ in range(warmup):
            if launch() != 0:
                raise RuntimeError("probe launch failed")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) * 1e-3 / steps
        secs[kind] = sec
        ops = lib.ssm_probe_ops_per_launch(blocks, iters)
        wave_instr_per_simd = ops / 64 / (cus * 4)
        if kind < 2:
            res[name] = {"lane_ops_per_s": round(ops / sec, 1),
                         "clk_per_wave_instr_at_2p4GHz": round(sec * 2.4e9 / wave_instr_per_simd,
                                                               3)}
        else:
            # ops FMA lane-operations plus ops / r exps: compare with the two streams run
            # one after the other (no overlap) and with the longer of the two alone.
            r = lib.ssm_probe_fma_per_exp(kind)
            serial = secs[0] + secs[1] / r
            res[name] = {"us_per_launch": round(sec * 1e6, 2),
                         "serial_model_us": round(serial * 1e6, 2),
                         "overlap_model_us": round(max(secs[0], secs[1] / r) * 1e6, 2),
                         "measured_over_serial": round(sec / serial, 4)}
    fma = res["v_fma_f32"]["lane_ops_per_s"]
    res["v_fma_f32"]["TFLOPs"] = round(2 * fma / 1e12, 2)
    print(json.dumps(res), flush=True)
    return 0


def forward_roofline(w, set_bytes: int, avg_ms: float, traffic, kernel: str) -> dict:
    """The forward's roofline on the metric's own basis: algorithmic bytes per launch over
    the mean launch time (HIP events on the launch stream), against the 8 TB/s HBM peak.

    Beside it, two compute views, labelled as such:
      * "alu": the method's arithmetic as counted per (b, d, n, t) update (dt*A, (dt*u)*B,
        the state FMA and the output FMA: 6 flop, plus one exp), against the 157.3 TFLOP/s
        fp32 vector peak and the exp rate that peak implies (a transcendental at a quarter
        of the FMA rate: 157.3e12 / 2 / 4 per second). On this count the HBM floor is the
        longer one, so the binding roof is HBM.
      * "alu_issue_no_packed": what the kernel can actually issue with packed fp32 disabled
        (4 wave64 VALU instructions at 4 clocks and one v_exp_f32 at 8 per update: 12
        flop-equivalents against 78.6 TFLOP/s), the floor the kernel is really measured
        against.
    """
    t = avg_ms * 1e-3
    achieved = set_bytes / t / 1e9
    t_hbm = set_bytes / (HBM_PEAK_GBS * 1e9)
    flops = FLOPS_PER_UPDATE * w.tuples
    exps = EXPS_PER_UPDATE * w.tuples
    t_flop = flops / (ALU_PEAK_TFLOPS * 1e12)
    t_exp = exps / EXP_PEAK_PER_S
    np_work = FLOP_EQ_PER_UPDATE_NO_PACKED * w.tuples
    np_achieved = np_work / t / 1e12
    return {
        "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
        "kernel_hash": kernel_hash(),
        "work": (f"{set_bytes} algorithmic bytes per launch (each input read once, each output "
                 f"written once) over the mean launch time {avg_ms * 1e3:.3f} us"),
        "floor_us": {"hbm": round(t_hbm * 1e6, 3), "alu_flops": round(t_flop * 1e6, 3),
                     "alu_exp": round(t_exp * 1e6, 3),
                     "alu_issue_no_packed": round(np_work / (ALU_PEAK_NO_PACKED_TFLOPS * 1e12)
                                                  * 1e6, 3)},
        "alu": {"flops_per_update": FLOPS_PER_UPDATE, "exps_per_update": EXPS_PER_UPDATE,
                "achieved": round(flops / t / 1e12, 3), "peak": ALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / t / 1e12 / ALU_PEAK_TFLOPS, 4),
                "exp_achieved_per_s": round(exps / t, 1), "exp_peak_per_s": EXP_PEAK_PER_S,
                "exp_frac": round(exps / t / EXP_PEAK_PER_S, 4)},
        "alu_issue_no_packed": {
            "achieved": round(np_achieved, 3), "peak": ALU_PEAK_NO_PACKED_TFLOPS,
            "unit": "TFLOP/s", "frac": round(np_achieved / ALU_PEAK_NO_PACKED_TFLOPS, 4),
            "work": (f"{FLOP_EQ_PER_UPDATE_NO_PACKED} flop-equivalents per update (4 wave64 "
                     "VALU instructions at 4 clocks + 1 v_exp_f32 at 8 clocks) x "
                     f"{w.tuples} updates per launch"),
            "basis": "the build disables packed fp32 (v_pk_fma_f32), which the 157.3 TFLOP/s "
                     "peak needs; this is the peak of the instructions the kernel can issue"},
    }


def prewarm(launch, seconds, torch) -> dict:
    """Runs the path untimed, in batches of 32 calls, until `seconds` of wall time have
    passed: the GPU's clocks rise over the first tenths of a second of sustained load (on the
    layer workload the first few hundred calls after start-up run up to 10% slower), and the
    metric is the throughput of a GPU under that load, not of its ramp."""
    calls = 0
    if seconds <= 0:
        return {"seconds": 0.0, "calls": 0}
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(32):
            launch(calls)
            calls += 1
        torch.cuda.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "calls": calls}


def timed_launches(launch, steps, warmup, stream, torch):
    """W untimed calls, then exactly K calls back to back between two synchronisations, with
    one HIP event on the launch stream before the first and one after the last (events
    between the calls would stop consecutive launches from overlapping their ends and add
    their own gaps: about 7 us per call on the layer workload). Then, outside the timed
    region, up to 50 more calls each between its own pair of events, for the duration of an
    isolated launch. Returns (wall seconds of the K calls, mean ms per call from the two
    events, per-call ms of the isolated launches)."""
    for i in range(warmup):
        launch(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = start.elapsed_time(end) / steps
    n_iso = min(steps, 50)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_iso)]
    for i in range(n_iso):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return wall, per_call_ms, np.array([a.elapsed_time(b) for a, b in ev])


def launch_stats(per_call_ms: float, iso_ms) -> dict:
    """Per-call times: the mean in the timed stream (its two events over K), and the
    median, p10 and p90 of isolated launches (each between its own pair of events)."""
    return {"mean_in_stream": round(per_call_ms * 1e3, 3),
            "isolated_median": round(float(np.median(iso_ms)) * 1e3, 3),
            "isolated_p10": round(float(np.percentile(iso_ms, 10)) * 1e3, 3),
            "isolated_p90": round(float(np.percentile(iso_ms, 90)) * 1e3, 3)}


def bench_bwd(args, w, inp, torch, ssm, dev) -> int:
    """The backward pass: ssm_scan_bwd on resident inputs, dout, dfinal and the saved
    states of a training forward (run once per buffer set, untimed)."""
    io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
    flags = (ssm.SSM_IO_BF16 if w.io == "bf16" else ssm.SSM_IO_F32) | ssm.SSM_DELTA_SOFTPLUS
    base = {k: to_device(inp[k], torch, dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                        "delta_bias", "h0")}
    set_bytes = w.bwd_algorithmic_bytes()
    nsets = args.sets or max(2, math.ceil(2 * INFINITY_CACHE_BYTES / set_bytes))
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 4242)
    sets = []
    for i in range(nsets):
        s = {k: (v if (i == 0 or v is None) else v.clone()) for k, v in base.items()}
        _, _, s["ckpt"] = ssm.scan_train(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"],
                                         z=s["z"], delta_bias=s["delta_bias"],
                                         delta_softplus=True, h0=s["h0"])
        s["dout"] = torch.randn(s["u"].shape, device=dev, generator=gen).to(io_t)
        s["dfinal"] = torch.randn((w.batch, w.dim, w.dstate), device=dev, generator=gen)
        f32 = dict(device=dev, dtype=torch.float32)
        s.update(du=torch.empty_like(s["u"]), ddelta=torch.empty_like(s["u"]),
                 dz=None if s["z"] is None else torch.empty_like(s["u"]),
                 dA=torch.empty((w.dim, w.dstate), **f32),
                 dB=torch.empty((w.batch, w.dstate, w.seqlen), **f32),
                 dC=torch.empty((w.batch, w.dstate, w.seqlen), **f32),
                 dD=torch.empty((w.dim,), **f32), dbias=torch.empty((w.dim,), **f32),
                 dh0=torch.empty((w.batch, w.dim, w.dstate), **f32))
        sets.append(s)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    # The calls run one after another on one stream, so they can share one workspace.
    ws_bytes = 0 if args.bwd_atomics else ssm.ssm_scan_bwd_workspace_bytes(
        w.batch, w.dim, w.dstate, w.seqlen, flags)
    ws = torch.empty((max(ws_bytes, 1),), device=dev, dtype=torch.uint8) if ws_bytes else None
    calls = [(ptr(s["u"]), ptr(s["delta"]), ptr(s["A"]), ptr(s["B"]), ptr(s["C"]), ptr(s["D"]),
              ptr(s["z"]), ptr(s["delta_bias"]), None, flags, ptr(s["ckpt"]), ptr(s["dout"]),
              ptr(s["dfinal"]), ptr(s["du"]), ptr(s["ddelta"]), ptr(s["dA"]), ptr(s["dB"]),
              ptr(s["dC"]), ptr(s["dD"]), ptr(s["dz"]), ptr(s["dbias"]), ptr(s["dh0"]),
              ptr(ws), ws_bytes, w.batch, w.dim, w.dstate, w.seqlen, sp) for s in sets]
    fn = ssm.lib().ssm_scan_bwd

    def launch(i):
        st = fn(*calls[i % nsets])
        if st != 0:
            raise ssm.SsmScanError(st)

    K = args.steps
    pre = prewarm(launch, args.prewarm_seconds, torch)
    wall, avg_ms, iso_ms = timed_launches(launch, K, args.warmup, stream, torch)
    achieved = set_bytes / (avg_ms * 1e-3) / 1e9
    alu_achieved = BWD_FLOP_EQ_PER_UPDATE * w.tuples / (avg_ms * 1e-3) / 1e12
    t_alu = BWD_FLOP_EQ_PER_UPDATE * w.tuples / (ALU_PEAK_TFLOPS * 1e12)
    t_hbm = set_bytes / (HBM_PEAK_GBS * 1e9)
    alu = {"achieved": round(alu_achieved, 3), "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(alu_achieved / ALU_PEAK_TFLOPS, 4),
           "work": (f"{BWD_FLOP_EQ_PER_UPDATE} flop-equivalents per (b,d,n,t) update (18 FMA "
                    f"issue slots of the sequential adjoint, exp at quarter rate) x {w.tuples}")}
    hbm = {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4),
           "work": f"{set_bytes} algorithmic bytes per launch"}
    main_, other = (("alu", alu), ("hbm", hbm)) if t_alu >= t_hbm else (("hbm", hbm), ("alu", alu))
    roofline = {"bound": main_[0], **main_[1],
                "traffic": None if args.bwd_atomics else load_traffic(args.workload, "bwd"),
                "kernel": ("scan_bwd_kernel (float atomics)" if args.bwd_atomics else
                           "scan_bwd_kernel + bwd_reduce_kernel (one call)"),
                "kernel_hash": kernel_hash("bwd"),
                "floor_us": {"alu": round(t_alu * 1e6, 3), "hbm": round(t_hbm * 1e6, 3)},
                other[0]: other[1]}
    value = set_bytes * K / wall / 1e9
    result = {
        "metric": f"scan backward GB/s (1 MI355X), {w.describe()}",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "prewarm": pre, "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64 inputs; dout, dfinal from a seeded torch generator)",
        "config": {"workload": w.describe(), "direction": "bwd", "batch": w.batch,
                   "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen, "io_dtype": w.io,
                   "gate": w.gate, "buffer_sets": nsets, "algorithmic_bytes": set_bytes,
                   "summed_gradients": ("float atomics" if args.bwd_atomics else
                                        f"workspace of {ws_bytes} bytes, fixed-order sums")},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tuples_per_s": round(w.tuples * K / wall, 1),
        "kernel_us": launch_stats(avg_ms, iso_ms),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_bwd(w, inp, args.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_bwd(w, inp, budget_s: float):
    """The backward oracle, untuned, on host cores over the leading channels of batch row 0
    (all steps), sized to about the time budget."""
    import oracle
    from ssm_workloads import widen

    threads = oracle.default_threads()
    io = inp["io"]
    rng = np.random.default_rng(w.seed + 4243)

    def timed(nd):
        sl = lambda x: None if x is None else x[:1, :nd]
        u = widen(sl(inp["u"]), io)
        args = (u, widen(sl(inp["delta"]), io), inp["A"][:nd], widen(inp["B"][:1], io),
                widen(inp["C"][:1], io), inp["D"][:nd], widen(sl(inp["z"]), io),
                inp["delta_bias"][:nd], True, None if inp["h0"] is None else inp["h0"][:1, :nd])
        dout = rng.standard_normal(u.shape)
        t0 = time.perf_counter()
        oracle.scan_bwd_ref(*args, dout=dout, dfinal=None, nthreads=threads)
        return time.perf_counter() - t0

    timed(min(w.dim, threads))
    probe = min(w.dim, max(4 * threads, 64))
    t_probe = max(timed(probe), 1e-6)
    nd = max(probe, min(w.dim, int(budget_s / t_probe * probe)))
    secs = timed(nd)
    sub = w.with_(batch=1, dim=nd)
    return {"value": round(sub.bwd_algorithmic_bytes() / secs / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": (f"float64 backward oracle over batch row 0, channels 0..{nd - 1}, all "
                       f"{w.seqlen} steps ({nd} of {w.batch * w.dim} rows), {secs:.2f} s"),
            "seconds": round(secs, 3)}


def ssd_mfma_flops(w) -> int:
    """Matrix-core flops one ssm_ssd_fwd call issues (16x16x32 bf16 products of 16384
    flops). A workgroup of 32 channels runs 2 x ns waves (ns = 4 state splits at 128 states,
    else 2). Per wave and 64-step block, up to 128 states (ssd_chunk_kernel, own = 4 / ns
    output tiles per wave): the carried-state product (own x dstate/32 k-blocks x 2 halves),
    the block-diagonal product in the separable form (own x 2 k-blocks x 2 halves; every
    block of the benchmark workloads takes that form) and the state update (2 tiles x 2
    k-blocks x 2 halves). At 256 states (ssd_fwd_kernel): the carried-state product over
    the wave's states for all 4 step tiles, the block matrix product (2 per output tile)
    and the state update. The prep kernel adds G (16 tiles x dstate/32 k-blocks per batch
    row and block)."""
    blocks = -(-w.seqlen // 64)
    ns = 4 if w.dstate == 128 else 2
    if w.dstate <= 128:
        own = 4 // ns
        per_wave = own * (w.dstate // 32) * 2 + own * 4 + 8
    else:
        nw = w.dstate // ns
        per_wave = 4 * (nw // 32) * 2 + 2 * (4 // ns) + (nw // 16) * 2 * 2
    waves = 2 * ns * w.batch * w.nheads * (-(-w.headdim // 32))
    prep = 16 * (w.dstate // 32) * w.batch
    return 16384 * blocks * (per_wave * waves + prep)


def bench_ssd(args, w, torch, ssm, dev) -> int:
    """The Mamba-2 (SSD) forward: one ssm_ssd_fwd call (prep and block-scan kernels) on
    resident inputs."""
    from ssm_workloads import make_ssd_inputs

    inp = make_ssd_inputs(w)
    flags = ssm.SSM_IO_BF16 | ssm.SSM_DELTA_SOFTPLUS | (ssm.SSM_INITIAL_STATE if w.initial_state else 0)
    base = {k: to_device(inp[k], torch, dev) for k in ("x", "dt", "B", "C", "z", "A", "D",
                                                        "dt_bias", "h0")}
    set_bytes = w.algorithmic_bytes()
    nsets = args.sets or max(2, math.ceil(2 * INFINITY_CACHE_BYTES / set_bytes))
    ws_bytes = ssm.ssm_ssd_workspace_bytes(w.batch, w.nheads, w.dstate, w.seqlen)
    sets = []
    for i in range(nsets):
        s = {k: (v if (i == 0 or v is None) else v.clone()) for k, v in base.items()}
        s["out"] = torch.empty_like(s["x"])
        s["fin"] = (s["h0"].clone() if s["h0"] is not None
                    else torch.empty((w.batch, w.dim, w.dstate), device=dev, dtype=torch.float32))
        s["ws"] = torch.empty((ws_bytes,), device=dev, dtype=torch.uint8)
        sets.append(s)
    stream = torch.cuda.current_stream(dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    calls = [(ptr(s["x"]), ptr(s["dt"]), ptr(s["A"]), ptr(s["B"]), ptr(s["C"]), ptr(s["D"]),
              ptr(s["z"]), ptr(s["dt_bias"]), None, flags, ptr(s["out"]), ptr(s["fin"]),
              ptr(s["ws"]), ws_bytes, w.batch, w.nheads, w.headdim, w.dstate, w.seqlen,
              stream.cuda_stream) for s in sets]
    fn = ssm.lib().ssm_ssd_fwd

    def launch(i):
        st = fn(*calls[i % nsets])
        if st != 0:
            raise ssm.SsmScanError(st)

    K = args.steps
    pre = prewarm(launch, args.prewarm_seconds, torch)
    wall, avg_ms, iso_ms = timed_launches(launch, K, args.warmup, stream, torch)
    achieved = set_bytes / (avg_ms * 1e-3) / 1e9
    flops = ssd_mfma_flops(w)
    t_hbm = set_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    mfma = {"achieved": round(flops / (avg_ms * 1e-3) / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(flops / (avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "work": f"{flops} bf16 MFMA flops issued per call"}
    hbm = {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4),
           "work": f"{set_bytes} algorithmic bytes per call"}
    main_, other = (("mfma", mfma), ("hbm", hbm)) if t_mfma >= t_hbm else (("hbm", hbm), ("mfma", mfma))
    roofline = {"bound": main_[0], **main_[1], "traffic": load_traffic(args.workload, "ssd"),
                "kernel": ("ssd_prep_kernel + ssd_chunk_kernel (one call)" if w.dstate <= 128
                           else "ssd_prep_kernel + ssd_fwd_kernel (one call)"),
                "kernel_hash": kernel_hash("ssd"),
                "floor_us": {"mfma": round(t_mfma * 1e6, 3), "hbm": round(t_hbm * 1e6, 3)},
                other[0]: other[1]}
    value = set_bytes * K / wall / 1e9
    result = {
        "metric": f"ssd GB/s & % HBM peak (1 MI355X), {w.describe()}",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "prewarm": pre, "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64 draws, Mamba-2 initialisation)",
        "config": {"workload": w.describe(), "batch": w.batch, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "seqlen": w.seqlen,
                   "io_dtype": w.io, "gate": w.gate, "dt_softplus": True,
                   "initial_state": w.initial_state, "buffer_sets": nsets,
                   "algorithmic_bytes": set_bytes},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kernel_us": launch_stats(avg_ms, iso_ms),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_ssd(w, inp, args.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_ssd(w, inp, budget_s: float):
    """The SSD oracle (float64 recurrence), untuned, on host cores: the whole workload,
    repeated to fill about the time budget."""
    import oracle
    from ssm_workloads import widen

    threads = oracle.default_threads()
    W = lambda k: widen(inp[k], "bf16")
    args = (W("x"), W("dt"), inp["A"], W("B"), W("C"), inp["D"],
            None if inp["z"] is None else W("z"), inp["dt_bias"], True, inp["h0"])
    t0 = time.perf_counter()
    oracle.ssd_ref(*args, nthreads=threads)
    one = time.perf_counter() - t0
    reps = max(1, min(50, int(budget_s / max(one, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.ssd_ref(*args, nthreads=threads)
    secs = (time.perf_counter() - t0) / reps
    return {"value": round(w.algorithmic_bytes() / secs / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": (f"float64 recurrence oracle over the whole workload, mean of {reps} "
                       f"run(s) of {secs:.2f} s"),
            "seconds": round(secs, 3)}


def bench_decode_loop(args, w, torch, ssm, dev) -> int:
    """T one-token forward calls per step, each reading and overwriting one fp32 state
    tensor (a decode loop over a layer's state cache), timed launched one by one from
    Python and as one replay of a captured HIP graph. The value is the graph's time per
    token."""
    from ssm_workloads import make_inputs

    T = args.decode_loop
    wl = w.with_(seqlen=T)
    inp = make_inputs(wl)
    tok = []
    for s in range(T):
        tok.append({k: to_device(np.ascontiguousarray(inp[k][..., s:s + 1]), torch, dev)
                    for k in ("u", "delta", "B", "C", "z")})
    par = {k: to_device(inp[k], torch, dev) for k in ("A", "D", "delta_bias", "h0")}
    state = par["h0"].clone()
    outs = [torch.empty_like(tok[s]["u"]) for s in range(T)]

    def loop():
        for s in range(T):
            g = tok[s]
            ssm.scan(g["u"], g["delta"], par["A"], g["B"], g["C"], D=par["D"], z=g["z"],
                     delta_bias=par["delta_bias"], delta_softplus=True, h0=state,
                     final_state=state, out=outs[s])

    def timed(step, K, W):
        for _ in range(W):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K

    K, W = args.steps, args.warmup
    eager = timed(loop, K, W)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        loop()
    replay = timed(graph.replay, K, W)
    tok_bytes = w.algorithmic_bytes()
    result = {
        "metric": f"decode loop time per token (1 MI355X), {w.describe()}, HIP graph replay",
        "value": round(replay / T * 1e6, 3),
        "unit": "us/token",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(replay * 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64 draws, shapes and distributions of the workload)",
        "config": {"workload": w.describe(), "tokens_per_step": T, "batch": w.batch,
                   "dim": w.dim, "dstate": w.dstate, "io_dtype": w.io,
                   "algorithmic_bytes_per_token": tok_bytes},
        "eager_us_per_token": round(eager / T * 1e6, 3),
        "graph_GBps": round(tok_bytes * T / replay / 1e9, 1),
        "tokens_per_s": round(w.batch * T / replay, 1),
        "note": "one state tensor is read and rewritten by every call (it stays in the caches "
                "across tokens); a step is T calls",
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-seconds", type=float, default=0.5,
                    help="untimed run of the path before the W warm-up calls (clock ramp); 0: none")
    ap.add_argument("--workload", default="layer")
    ap.add_argument("--sets", type=int, default=0,
                    help="input/output sets to rotate over (0: enough for 2x the Infinity Cache)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm (single set) timing")
    ap.add_argument("--direction", choices=("fwd", "bwd"), default="fwd",
                    help="fwd: the forward scan (the default, headline); bwd: the backward "
                         "pass from the forward's saved states")
    ap.add_argument("--bwd-atomics", action="store_true",
                    help="with --direction bwd: sum dA, dB, dC, dD and dbias with float atomics "
                         "(no workspace) instead of the reproducible workspace sums")
    ap.add_argument("--decode-loop", type=int, default=0, metavar="T",
                    help="with --workload decode: time a loop of T one-token calls that carry "
                         "the state in place, launched eagerly and as one captured HIP graph")
    ap.add_argument("--alu-probe", action="store_true",
                    help="measure the issue rates of wave64 v_fma_f32 and v_exp_f32 under this "
                         "build's flags (register-only probe kernels)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (HBM reference, and "
                         "the known-size kernel that scales the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): every "
              "(batch, channel) row of the scan is independent, so more GPUs would only "
              "split the batch with no exchange; no multi-GPU figure is measured.",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_probe:
        return copy_probe(torch, args.steps, args.warmup)
    if args.alu_probe:
        return alu_probe(torch, min(args.steps, 20), min(args.warmup, 3))

    import selective_state_space_fwd_amd as ssm
    from ssm_workloads import SSD_WORKLOADS, WORKLOADS, make_inputs

    if args.workload in SSD_WORKLOADS:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        return bench_ssd(args, SSD_WORKLOADS[args.workload], torch, ssm, dev)
    if args.workload not in WORKLOADS:
        print(f"unknown workload {args.workload}; choose from "
              f"{sorted(WORKLOADS) + sorted(SSD_WORKLOADS)}", file=sys.stderr)
        return 2
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode_loop:
        if w.seqlen != 1 or not w.initial_state:
            print("--decode-loop needs a one-step workload from a given state (decode)",
                  file=sys.stderr)
            return 2
        return bench_decode_loop(args, w, torch, ssm, dev)
    inp = make_inputs(w)
    if args.direction == "bwd":
        return bench_bwd(args, w, inp, torch, ssm, dev)
    io_flag = ssm.SSM_IO_BF16 if w.io == "bf16" else ssm.SSM_IO_F32
    flags = io_flag | ssm.SSM_DELTA_SOFTPLUS | (ssm.SSM_INITIAL_STATE if w.initial_state else 0)

    base = {k: to_device(inp[k], torch, dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                        "delta_bias", "h0")}
    set_bytes = w.algorithmic_bytes()
    nsets = args.sets or max(2, math.ceil(2 * INFINITY_CACHE_BYTES / set_bytes))
    sets = []
    for i in range(nsets):
        s = {k: (v if (i == 0 or v is None) else v.clone()) for k, v in base.items()}
        s["out"] = torch.empty_like(s["u"])
        s["fin"] = (s["h0"].clone() if s["h0"] is not None
                    else torch.empty((w.batch, w.dim, w.dstate), device=dev, dtype=torch.float32))
        sets.append(s)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    calls = [(ptr(s["u"]), ptr(s["delta"]), ptr(s["A"]), ptr(s["B"]), ptr(s["C"]), ptr(s["D"]),
              ptr(s["z"]), ptr(s["delta_bias"]), flags, ptr(s["out"]), ptr(s["fin"]),
              w.batch, w.dim, w.dstate, w.seqlen, sp) for s in sets]
    fn = ssm.lib().ssm_scan_fwd

    def launch(i):
        st = fn(*calls[i % nsets])
        if st != 0:
            raise ssm.SsmScanError(st)

    # The copy reference runs first: a few milliseconds of streaming that also take the GPU
    # out of its idle clock state before the warm-up calls (in a fresh process the first
    # ~60 calls otherwise run several microseconds slower each).
    copy = copy_reference(torch)
    K = args.steps
    pre = prewarm(launch, args.prewarm_seconds, torch)
    wall, avg_ms, iso_ms = timed_launches(launch, K, args.warmup, stream, torch)

    warm = None
    if not args.no_warm:
        wk = max(20, K // 2)
        evw = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(wk)]
        for i in range(wk):
            evw[i][0].record(stream)
            launch(0)
            evw[i][1].record(stream)
        torch.cuda.synchronize()
        wms = np.array([a.elapsed_time(b) for a, b in evw])
        warm = {"kernel_us_median": round(float(np.median(wms)) * 1e3, 3),
                "GBps": round(set_bytes / (float(np.median(wms)) * 1e-3) / 1e9, 1),
                "note": "one buffer set reused (reads may hit the Infinity Cache); not the metric"}

    value = set_bytes * K / wall / 1e9
    traffic = load_traffic(args.workload)
    kernel = "scan_short_kernel" if w.seqlen <= SHORT_MAX_SEQLEN else "scan_fwd_kernel"
    roofline = forward_roofline(w, set_bytes, avg_ms, traffic, kernel)

    result = {
        "metric": ("scan GB/s & % HBM peak (1 MI355X), b4 d2048 N16 L2048 bf16"
                   if args.workload == "layer" else
                   f"scan GB/s & % HBM peak (1 MI355X), {w.describe()}"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "prewarm": pre,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64 draws, shapes and distributions of the workload)",
        "config": {
            "workload": w.describe(),
            "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen,
            "io_dtype": w.io, "gate": w.gate, "delta_softplus": True,
            "initial_state": w.initial_state, "buffer_sets": nsets,
            "algorithmic_bytes": set_bytes,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "elements_per_s": round(w.elements * K / wall, 1),
        "tuples_per_s": round(w.tuples * K / wall, 1),
        "kernel_us": launch_stats(avg_ms, iso_ms),
        "per_launch_GBps": {"in_stream": round(set_bytes / (avg_ms * 1e-3) / 1e9, 2),
                            "isolated_median": round(
                                set_bytes / (float(np.median(iso_ms)) * 1e-3) / 1e9, 2),
                            "note": "algorithmic bytes over the mean time per call in the timed "
                                    "stream, and over the median of isolated calls"},
        "roofline": roofline,
        "warm": warm,
    }
    copy["pct_of_copy"] = round(100.0 * value / copy["GBps"], 2)
    copy["note"] = "value against a plain device copy measured in this run, before the metric"
    result["copy_reference"] = copy
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
