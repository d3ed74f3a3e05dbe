"""Benchmark: causal attention forward + backward on one MI355X.

One step = one pass of the whole path over one batch of the synthetic
long-context workload (B4, S2048, 16 heads of 64, bf16 in / fp32 accumulate):
xattn_fwd, then the backward as its two kernels (xattn_bwd_dq, xattn_bwd_dkdv,
which together are exactly xattn_bwd for that shape; for short bf16 sequences,
where xattn_bwd runs one kernel, xattn_bwd), all through the C ABI on torch's current
stream with inputs resident in HBM.  At least W untimed warmup steps (and at
least WARMUP_MIN_S seconds of them), then K timed steps between
synchronisations.  HIP events around the dk/dv kernel, the longest one
(timing-only events without a system-scope fence, so no cache flush separates
the kernels), give its average duration inside the timed region, and its
roofline is reported against MI355X's dense bf16 MFMA peak; the forward and dq
kernels are timed in loops of their own after the timed region.  The other
workloads (`secondary`) record no events inside their timed region, only at
its ends, and time every kernel in loops of its own.

Counted FLOPs (the FlashAttention-2 convention, causal half only):
    fwd 4*hd*nnz, bwd 10*hd*nnz per (batch, head), nnz = S(S+1)/2
Per-kernel algorithmic FLOPs per (batch, head): fwd 4*hd*nnz (Q.K^T, P.V),
dq kernel 6*hd*nnz (S, dP, dS.K), dk/dv kernel 8*hd*nnz (S, dP, P^T.dO, dS^T.Q),
the single backward kernel of short bf16 sequences the sum of the two (14*hd*nnz).

The CPU baseline times the fp64 oracle on a bounded sample of the same
workload (whole (batch, kv head) units) on the host's cores, rank 0, N = 1.

`next_rows` reports the step before attention, the per-head RMS QK-norm +
RoPE forward and backward, on the long-context workload's q input, against
MI355X's HBM bandwidth (algorithmic bytes: fwd reads x and writes out; bwd
reads x and the fp32 upstream gradient and writes the fp32 dx), and decode
attention (one new query per sequence and head against a K/V cache) on a
32768-position bf16 cache and on the long-context workload's last row, against
the same bandwidth (algorithmic bytes: the cached K and V once, q, o and lse),
a right-padded batch of 8 sequences with lengths 256..2048 through the
length-aware kernels, against the same batch run padded, and the composed path
(scores, softmax, products through S x S fp32 buffers) on the same workload as
the step, with the memory it needs.  None of them is part of the timed step.

Prints ONE JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s & % MFMA peak (B16 S256 H12 hd32; B4 S2048 hd64)"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}  # MI355X dense MFMA
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
HBM_GBS = 8000.0

KERNEL_FILES = {"fwd": "attn_fwd.hip", "dq": "attn_bwd_dq.hip", "dkdv": "attn_bwd_dkdv.hip",
                "bwd": "attn_bwd_short.hip"}
KERNEL_NAMES = {"fwd": "attn_fwd_kernel", "dq": "attn_bwd_dq_kernel", "dkdv": "attn_bwd_dkdv_kernel",
                "bwd": "attn_bwd_short_kernel"}

# HBM bytes per launch on the long-context workload from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (separate runs), scaled by the copy-kernel calibration (read x2.0,
# write x1.0), recorded with the sha256 of the kernel's sources at the time.
# Reported only while the sources still match.
MEASURED_TRAFFIC = {
    "dkdv": {"src": "be9299c1c75df814", "read": 83.21e6, "write": 67.23e6},
    "dq": {"src": "9bdfe6175be4adf4", "read": 95.51e6, "write": 34.60e6},
    "fwd": {"src": "1ac9b1478c3d988b", "read": 50.48e6, "write": 20.45e6},
}


def kernel_source_hash(kernel):
    """sha256 prefix of a kernel's sources and the device compile flags."""
    import hashlib

    from bwd_head_rms_amd import build
    csrc = os.path.join(ROOT, "bwd_head_rms_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_FILES[kernel], "attn_device.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    # compile flags without the include paths, which differ between checkouts
    flags = [f for f in build.COMMON + build.DEVICE_FLAGS if not os.path.isabs(f)]
    h.update(" ".join(flags).encode())
    extra = build.SOURCE_FLAGS.get(KERNEL_FILES[kernel], [])
    if extra:
        h.update((" " + " ".join(extra)).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    from bwd_head_rms_amd import inputs
    m = MEASURED_TRAFFIC.get(kernel)
    if workload != inputs.LONG_CONTEXT or not m or m["src"] != kernel_source_hash(kernel):
        return None
    return m["read"] + m["write"]


class TimingEvents:
    """HIP events used only for timing, created with hipEventDisableSystemFence
    through the HIP runtime that torch has loaded in this process.  An ordinary
    timing event performs a system-scope fence when it is recorded: a cache
    write-back and invalidation between the kernels it separates, so every
    kernel after one would start with a cold L2 and the step would run slower
    than back-to-back kernels do.  Elapsed times are read after a device
    synchronisation, which orders the host after the recorded work."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        import torch
        with open("/proc/self/maps") as fh:
            paths = sorted({line.split()[-1] for line in fh if "libamdhip64" in line})
        if not paths:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        if len(paths) > 1:  # use the copy torch runs on
            torch_lib = os.path.join(os.path.dirname(torch.__file__), "lib")
            paths = [p for p in paths if os.path.dirname(p) == torch_lib]
            if len(paths) != 1:
                raise RuntimeError("cannot tell which HIP runtime torch uses")
        self._ct = ctypes
        self._hip = ctypes.CDLL(paths[0])
        self._made = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def new(self):
        e = self._ct.c_void_p()
        self._check(self._hip.hipEventCreateWithFlags(self._ct.byref(e),
                                                      self._ct.c_uint(self.DISABLE_SYSTEM_FENCE)),
                    "hipEventCreateWithFlags")
        self._made.append(e)
        return e

    def record(self, e, stream_handle):
        self._check(self._hip.hipEventRecord(e, self._ct.c_void_p(stream_handle)), "hipEventRecord")

    def ms(self, a, b):
        f = self._ct.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(f), a, b), "hipEventElapsedTime")
        return f.value

    def close(self):
        for e in self._made:
            self._hip.hipEventDestroy(e)
        self._made = []


# Warm-up lasts at least this long whatever W is: the first milliseconds of
# work after idle run slower (measured on MI355X: the long-context step at
# 222-224 us after 5 warm-up steps, 202 us after 50).
WARMUP_MIN_S = 0.3


def warm_up(step, warmup):
    """Run `step` at least `warmup` times and for at least WARMUP_MIN_S seconds
    of GPU time; returns (steps run, seconds)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()  # keeps the host from running far ahead of the GPU
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def time_loop(fn, steps):
    """Milliseconds per call of `fn` over `steps` back-to-back calls on torch's
    current stream, between two timing events (after a synchronisation)."""
    import torch
    T = TimingEvents()
    sh = torch.cuda.current_stream().cuda_stream
    e0, e1 = T.new(), T.new()
    torch.cuda.synchronize()
    T.record(e0, sh)
    for _ in range(steps):
        fn()
    T.record(e1, sh)
    torch.cuda.synchronize()
    ms = T.ms(e0, e1) / steps
    T.close()
    return ms


def alg_bytes(w):
    """Algorithmic HBM bytes of one fwd+bwd step: every input read once and
    every output written once by each pass (fwd: q, k, v in, o and lse out;
    bwd: q, k, v, o, dO, lse in, fp32 dq, dk, dv out).  The per-row workspace
    is implementation overhead and not counted."""
    e = 2 if w.dtype == "bf16" else 4
    nq = w.B * w.H * w.S * w.hd
    nk = w.B * w.Hkv * w.S * w.hd
    rows = w.B * w.H * w.S
    fwd = e * (nq + 2 * nk) + e * nq + 4 * rows
    bwd = e * (3 * nq + 2 * nk) + 4 * rows + 4 * (nq + 2 * nk)
    return fwd + bwd


def step_roofline(w, ms_per_step):
    """The step against its own roofline: the time bound is the larger of the
    counted FLOPs at the dtype's dense MFMA peak and the algorithmic bytes at
    the HBM peak; frac = bound / measured time."""
    fl = counted_flops(w)["total"]
    by = alg_bytes(w)
    t_mfma = fl / (PEAK_TFLOPS[w.dtype] * 1e12)
    t_hbm = by / (PEAK_HBM_GBPS * 1e9)
    sec = ms_per_step / 1e3
    if t_mfma >= t_hbm:
        return {"bound": "mfma", "achieved": round(fl / sec / 1e12, 3), "peak": PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": round(t_mfma / sec, 5), "t_bound_us": round(t_mfma * 1e6, 2),
                "alg_bytes": by}
    return {"bound": "hbm", "achieved": round(by / sec / 1e9, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(t_hbm / sec, 5), "t_bound_us": round(t_hbm * 1e6, 2),
            "alg_bytes": by}


def counted_flops(w):
    nnz = w.S * (w.S + 1) / 2
    per = w.B * w.H * nnz * w.hd
    return {"fwd": 4 * per, "bwd": 10 * per, "total": 14 * per,
            "k_fwd": 4 * per, "k_dq": 6 * per, "k_dkdv": 8 * per}


def run_gpu(w, steps, warmup, kernel_events=True):
    import torch

    from bwd_head_rms_amd import _lib, inputs

    L = _lib.lib()
    dev = torch.device("cuda:0")
    arrs = inputs.generate_workload(w)
    t = {n: inputs.to_torch(a, w.dtype, dev) for n, a in arrs.items()}
    code = _lib.BF16 if w.dtype == "bf16" else _lib.F32
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty(t["q"].shape, **f32)
    dk = torch.empty(t["k"].shape, **f32)
    dv = torch.empty(t["k"].shape, **f32)
    ws_bytes = int(L.xattn_bwd_workspace_bytes(w.B, w.S, w.H, w.Hkv, w.hd, code))
    ws = torch.empty(ws_bytes // 4, **f32)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    dims = (w.B, w.S, w.H, w.Hkv, w.hd, w.scale, code)
    p = {n: x.data_ptr() for n, x in dict(q=t["q"], k=t["k"], v=t["v"], dO=t["dO"], o=o, lse=lse,
                                          dq=dq, dk=dk, dv=dv, ws=ws).items()}

    def fwd():
        _lib.check(L.xattn_fwd(p["q"], p["k"], p["v"], p["o"], p["lse"], *dims, sh))

    def bwd_dq():
        _lib.check(L.xattn_bwd_dq(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dO"], p["dq"],
                                  *dims, p["ws"], ws_bytes, sh))

    def bwd_dkdv():
        _lib.check(L.xattn_bwd_dkdv(p["q"], p["k"], p["v"], p["lse"], p["dO"], p["dk"], p["dv"],
                                    *dims, p["ws"], ws_bytes, sh))

    def bwd_single():
        _lib.check(L.xattn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dO"], p["dq"], p["dk"],
                               p["dv"], *dims, p["ws"], ws_bytes, sh))

    if int(L.xattn_bwd_kernel_count(w.B, w.S, w.H, w.Hkv, w.hd, code)) == 1:
        # short bf16 sequences: xattn_bwd is one kernel (dq, dk, dv together);
        # the events bracket it
        return _time_steps(steps, warmup, dev, fwd, [], bwd_single, "bwd", kernel_events)
    return _time_steps(steps, warmup, dev, fwd, [bwd_dq], bwd_dkdv, "dkdv", kernel_events,
                       extra={"dq": bwd_dq})


def _time_steps(steps, warmup, dev, fwd, before, timed, timed_name, kernel_events, extra=None):
    """Warm up, then time exactly `steps` steps (fwd, the `before` calls, then
    `timed`).  With kernel_events, two timing events bracket `timed` in every
    step (its duration inside the timed region, for the roofline); without,
    events mark only the region's start and end, and `timed` is timed in a
    loop of its own afterwards like the other kernels."""
    import numpy as np
    import torch

    sh = torch.cuda.current_stream(dev).cuda_stream

    def step():
        fwd()
        for f in before:
            f()
        timed()

    warm_steps, warm_s = warm_up(step, warmup)

    # Timed region: exactly `steps` steps.  Timing events sit at most around
    # the roofline's kernel: every event recorded between two kernels
    # lengthens the step by about a microsecond, which on the short workloads
    # is several percent of it.
    T = TimingEvents()
    e_start = T.new()
    ev = [[T.new() for _ in range(2)] for _ in range(steps)] if kernel_events else []
    e_end = T.new()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    T.record(e_start, sh)
    for i in range(steps):
        fwd()
        for f in before:
            f()
        if kernel_events:
            T.record(ev[i][0], sh)
        timed()
        if kernel_events:
            T.record(ev[i][1], sh)
    T.record(e_end, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = T.ms(e_start, e_end)
    timed_ms = (float(np.mean([T.ms(e[0], e[1]) for e in ev])) if kernel_events
                else time_loop(timed, steps))
    T.close()
    # the other kernels' durations, each timed over `steps` back-to-back
    # launches after the timed region (context, not part of the step's time)
    avg = {"fwd": time_loop(fwd, steps)}
    for name, f in (extra or {}).items():
        avg[name] = time_loop(f, steps)
    avg[timed_name] = timed_ms
    return {"ms_per_step": total_ms / steps, "wall_s": wall, "kernel_ms": avg,
            "warmup_steps": warm_steps, "warmup_s": round(warm_s, 3),
            "device": torch.cuda.get_device_name(dev)}


def run_secondary(w, steps, warmup):
    """One workload's fwd+bwd step, as the headline one is measured."""
    r = run_gpu(w, steps, warmup, kernel_events=False)
    sec = r["ms_per_step"] / 1e3
    tf = counted_flops(w)["total"] / sec / 1e12
    return {"workload": w.name, "dtype": w.dtype, "B": w.B, "S": w.S, "H": w.H, "Hkv": w.Hkv,
            "hd": w.hd, "ms_per_step": round(r["ms_per_step"], 5),
            "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in r["kernel_ms"].items()},
            "tflops": round(tf, 3), "pct_of_mfma_peak": round(100 * tf / PEAK_TFLOPS[w.dtype], 3),
            "tokens_per_s": round(w.B * w.S / sec, 1),
            "roofline": step_roofline(w, r["ms_per_step"])}


def norm_bytes(w):
    """Algorithmic HBM bytes of the QK-norm + RoPE step on the q input of `w`:
    fwd reads x and writes out (input dtype); bwd reads x (input dtype) and
    dout (fp32) and writes dx (fp32).  The weight, dw and the workspace are
    negligible and not counted."""
    n = w.B * w.S * w.H * w.hd
    e = 2 if w.dtype == "bf16" else 4
    return {"fwd": 2 * e * n, "bwd": (e + 8) * n}


def run_norm(w, steps, warmup):
    """Time xattn_qknorm_rope_fwd / _bwd on the q input of workload `w`:
    x [B, S, H, hd] in the workload dtype, dout fp32, inputs resident in HBM."""
    import numpy as np
    import torch

    from bwd_head_rms_amd import _lib, inputs

    L = _lib.lib()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(w.seed)
    x = inputs.to_torch(rng.standard_normal((w.B, w.S, w.H, w.hd)).astype(np.float32), w.dtype, dev)
    wt = torch.from_numpy((1.0 + 0.25 * rng.standard_normal(w.hd)).astype(np.float32)).to(dev)
    g = torch.from_numpy(rng.standard_normal((w.B, w.H, w.S, w.hd)).astype(np.float32)).to(dev)
    out = torch.empty((w.B, w.H, w.S, w.hd), dtype=x.dtype, device=dev)
    dx = torch.empty((w.B, w.S, w.H, w.hd), dtype=torch.float32, device=dev)
    dw = torch.empty((w.hd,), dtype=torch.float32, device=dev)
    wsb = int(L.xattn_qknorm_rope_bwd_workspace_bytes(w.B, w.S, w.H, w.hd))
    ws = torch.empty((max(1, wsb // 4),), dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream
    code = _lib.BF16 if w.dtype == "bf16" else _lib.F32
    dims = (w.B, w.S, w.H, w.hd, 1e-6, 10000.0, code)

    def fwd():
        _lib.check(L.xattn_qknorm_rope_fwd(x.data_ptr(), wt.data_ptr(), out.data_ptr(), *dims, sh))

    def bwd():
        _lib.check(L.xattn_qknorm_rope_bwd(x.data_ptr(), wt.data_ptr(), g.data_ptr(), dx.data_ptr(),
                                           dw.data_ptr(), *dims, ws.data_ptr(), wsb, sh))

    res = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        res[name] = time_loop(fn, steps)  # ms
    nb = norm_bytes(w)
    roof = {k: {"achieved": round(nb[k] / (res[k] / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(nb[k] / (res[k] / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
                "alg_bytes": nb[k]} for k in res}
    return {"workload": f"q input of {w.name}: x [{w.B},{w.S},{w.H},{w.hd}] {w.dtype}, dout fp32",
            "fwd_us": round(res["fwd"] * 1e3, 2), "bwd_us": round(res["bwd"] * 1e3, 2),
            "roofline": {"bound": "hbm", **roof}}


def host_cpu():
    """The host CPU: model name, physical cores and logical CPUs (from
    /proc/cpuinfo) and the CPUs this process may run on."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return {"cpu_model": model, "physical_cores": len(cores) or None,
            "logical_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(w, budget_units=None):
    """Time the fp64 oracle on whole (batch, kv head) units of the workload."""
    import numpy as np

    from bwd_head_rms_amd import inputs
    from oracle import default

    ref = default()
    threads = ref.max_threads()
    n_units = budget_units or max(1, min(w.B * w.Hkv, 2 * threads))
    arrs = inputs.generate_workload(w)
    b_needed = (n_units + w.Hkv - 1) // w.Hkv
    sub = {n: np.ascontiguousarray(a[:b_needed]) for n, a in arrs.items()}
    t0 = time.perf_counter()
    ref.run(sub["q"], sub["k"], sub["v"], sub["dO"], scale=w.scale, units=(0, n_units))
    dt = time.perf_counter() - t0
    nnz = w.S * (w.S + 1) / 2
    flops = 14 * nnz * w.hd * n_units * (w.H // w.Hkv)
    # the same oracle on one thread, one unit
    ref.set_threads(1)
    try:
        t1 = time.perf_counter()
        ref.run(sub["q"], sub["k"], sub["v"], sub["dO"], scale=w.scale, units=(0, 1))
        dt1 = time.perf_counter() - t1
    finally:
        ref.set_threads(0)
    flops1 = 14 * nnz * w.hd * (w.H // w.Hkv)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": dt, "threads_used": threads, **host_cpu(),
            "sample": f"{n_units} of {w.B * w.Hkv} (batch, kv head) units of {w.name} "
                      f"({n_units * (w.H // w.Hkv)} heads x S={w.S}, fwd+bwd, fp64)",
            "single_thread": {"value": flops1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "seconds": dt1, "sample": f"1 unit ({w.H // w.Hkv} heads x S={w.S})"}}


def calibrate_copy(nbytes, reps=5):
    """A plain elementwise copy (read nbytes, write nbytes) for scaling the HBM
    traffic counters: the same counters read on it give bytes per counter unit."""
    import torch
    n = nbytes // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "reps": reps}), flush=True)


def decode_bytes(wd):
    """Algorithmic HBM bytes of one decode step: K and V of every cached
    position once, q and o (input dtype), lse (fp32).  The chunk partials in the
    workspace are overhead and not counted."""
    e = 2 if wd.dtype == "bf16" else 4
    return 2 * wd.B * wd.Hkv * wd.T * wd.hd * e + 2 * wd.B * wd.H * wd.hd * e + 4 * wd.B * wd.H


def run_decode(wd, steps, warmup):
    """Time xattn_decode on decode workload `wd` (inputs resident in HBM):
    `steps` back-to-back calls between HIP events on the launch stream."""
    import torch

    from bwd_head_rms_amd import _lib, inputs

    L = _lib.lib()
    dev = torch.device("cuda:0")
    a = inputs.generate_decode(wd)
    t = {n: inputs.to_torch(x, wd.dtype, dev) for n, x in a.items()}
    del a
    o = torch.empty_like(t["q"])
    lse = torch.empty((wd.B, wd.H), dtype=torch.float32, device=dev)
    wsb = int(L.xattn_decode_workspace_bytes(wd.B, wd.T, wd.H, wd.Hkv, wd.hd))
    ws = torch.empty((max(1, wsb // 4),), dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream
    code = _lib.BF16 if wd.dtype == "bf16" else _lib.F32

    def call():
        _lib.check(L.xattn_decode(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), None,
                                  o.data_ptr(), lse.data_ptr(), wd.B, wd.T, wd.H, wd.Hkv, wd.hd,
                                  wd.scale, code, ws.data_ptr(), wsb, sh))

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = time_loop(call, steps)
    nb = decode_bytes(wd)
    gbs = nb / (ms / 1e3) / 1e9
    return {"workload": wd.name, "B": wd.B, "T": wd.T, "H": wd.H, "Hkv": wd.Hkv, "hd": wd.hd,
            "dtype": wd.dtype, "us": round(ms * 1e3, 2),
            "tokens_per_s": round(wd.B / (ms / 1e3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBPS, 4), "alg_bytes": nb}}


def run_ragged(rw, steps, warmup):
    """Time fwd + bwd of a right-padded batch with its lengths (xattn_fwd_ragged,
    xattn_bwd_ragged) and, for comparison, the plain kernels over the same
    padded batch.  TFLOP/s counts the causal work of the real rows only."""
    import numpy as np
    import torch

    from bwd_head_rms_amd import _lib, inputs

    L = _lib.lib()
    dev = torch.device("cuda:0")
    lens = rw.lens()
    a = inputs.generate(rw.B, rw.S, rw.H, rw.Hkv, rw.hd, rw.seed, shaped=True, dtype=rw.dtype)
    t = {n: inputs.to_torch(x, rw.dtype, dev) for n, x in a.items()}
    del a
    tl = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty_like(t["q"])
    lse = torch.empty((rw.B, rw.H, rw.S), dtype=torch.float32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty(t["q"].shape, **f32)
    dk = torch.empty(t["k"].shape, **f32)
    dv = torch.empty(t["k"].shape, **f32)
    code = _lib.BF16 if rw.dtype == "bf16" else _lib.F32
    wsb = int(L.xattn_bwd_workspace_bytes(rw.B, rw.S, rw.H, rw.Hkv, rw.hd, code))
    ws = torch.empty((wsb // 4,), **f32)
    sh = torch.cuda.current_stream(dev).cuda_stream
    dims = (rw.B, rw.S, rw.H, rw.Hkv, rw.hd, rw.scale, code)
    p = {n: x.data_ptr() for n, x in dict(q=t["q"], k=t["k"], v=t["v"], dO=t["dO"], o=o, lse=lse,
                                          dq=dq, dk=dk, dv=dv, ws=ws, lens=tl).items()}

    def ragged():
        _lib.check(L.xattn_fwd_ragged(p["q"], p["k"], p["v"], p["lens"], p["o"], p["lse"], *dims,
                                      sh))
        _lib.check(L.xattn_bwd_ragged(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dO"], p["lens"],
                                      p["dq"], p["dk"], p["dv"], *dims, p["ws"], wsb, sh))

    def padded():
        _lib.check(L.xattn_fwd(p["q"], p["k"], p["v"], p["o"], p["lse"], *dims, sh))
        _lib.check(L.xattn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dO"], p["dq"],
                               p["dk"], p["dv"], *dims, p["ws"], wsb, sh))

    ms = {}
    for name, fn in (("ragged", ragged), ("padded", padded)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ms[name] = time_loop(fn, steps)
    flops = sum(14.0 * rw.hd * rw.H * n * (n + 1) / 2 for n in lens)
    tf = flops / (ms["ragged"] / 1e3) / 1e12
    return {"workload": rw.name, "lens": lens, "ms_per_step": round(ms["ragged"], 5),
            "padded_ms_per_step": round(ms["padded"], 5),
            "speedup_vs_padded": round(ms["padded"] / ms["ragged"], 3),
            "tflops_real_rows": round(tf, 3),
            "pct_of_mfma_peak": round(100 * tf / PEAK_TFLOPS[rw.dtype], 3),
            "tokens_per_s": round(sum(lens) / (ms["ragged"] / 1e3), 1)}


def run_composed(w, steps, warmup):
    """Time the composed path (xattn_composed_fwd + _bwd: S x S fp32 buffers)
    on workload `w`, for comparison with the fused step.  Counted FLOPs as the
    headline (14*hd*nnz per (batch, head))."""
    import torch

    from bwd_head_rms_amd import _lib, inputs

    L = _lib.lib()
    dev = torch.device("cuda:0")
    arrs = inputs.generate_workload(w)
    t = {n: inputs.to_torch(a, w.dtype, dev) for n, a in arrs.items()}
    del arrs
    code = _lib.BF16 if w.dtype == "bf16" else _lib.F32
    nbuf = int(L.xattn_composed_buffer_bytes(w.B, w.S, w.H))
    f32 = dict(dtype=torch.float32, device=dev)
    p = torch.empty((nbuf // 4,), **f32)
    ds = torch.empty((nbuf // 4,), **f32)
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.B, w.H, w.S), **f32)
    dq = torch.empty(t["q"].shape, **f32)
    dk = torch.empty(t["k"].shape, **f32)
    dv = torch.empty(t["k"].shape, **f32)
    sh = torch.cuda.current_stream(dev).cuda_stream
    dims = (w.B, w.S, w.H, w.Hkv, w.hd, w.scale, code)

    def fwd():
        _lib.check(L.xattn_composed_fwd(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                        o.data_ptr(), lse.data_ptr(), p.data_ptr(), nbuf, *dims, sh))

    def bwd():
        _lib.check(L.xattn_composed_bwd(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                        p.data_ptr(), nbuf, t["dO"].data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), ds.data_ptr(), nbuf, *dims,
                                        sh))

    ms = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ms[name] = time_loop(fn, steps)
    tot = ms["fwd"] + ms["bwd"]
    tf = counted_flops(w)["total"] / (tot / 1e3) / 1e12
    return {"workload": w.name, "fwd_ms": round(ms["fwd"], 4), "bwd_ms": round(ms["bwd"], 4),
            "ms_per_step": round(tot, 4), "tflops": round(tf, 3),
            "pct_of_mfma_peak": round(100 * tf / PEAK_TFLOPS[w.dtype], 3),
            "s_by_s_buffers_bytes": 2 * nbuf,
            "fused_workspace_bytes": int(L.xattn_bwd_workspace_bytes(w.B, w.S, w.H, w.Hkv, w.hd,
                                                                     code))}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None, help="name from bwd_head_rms_amd.inputs.WORKLOADS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip QK-norm + RoPE, decode, ragged and composed ('next_rows')")
    ap.add_argument("--norm-only", action="store_true",
                    help="only time the QK-norm + RoPE step (for profiling its kernels)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time decode attention (for profiling its kernels)")
    ap.add_argument("--composed-only", action="store_true",
                    help="only time the composed path (for profiling its kernels)")
    ap.add_argument("--ragged-only", action="store_true",
                    help="only time the ragged batch and the same batch padded (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (for counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by batch or kv-head group with no exchange inside attention).",
              file=sys.stderr)
        sys.exit(2)

    from bwd_head_rms_amd import inputs
    w = inputs.WORKLOADS[args.workload or inputs.LONG_CONTEXT]
    if args.norm_only:
        print(json.dumps({"qknorm_rope": run_norm(w, args.steps, args.warmup)}), flush=True)
        return
    if args.composed_only:
        print(json.dumps({"composed": run_composed(w, args.steps, args.warmup)}), flush=True)
        return
    if args.decode_only:
        wd = inputs.DECODE_WORKLOADS[inputs.DECODE_BENCH]
        print(json.dumps({"decode": run_decode(wd, args.steps, args.warmup)}), flush=True)
        return
    if args.ragged_only:
        print(json.dumps({"ragged": run_ragged(inputs.RAGGED_BENCH, args.steps, args.warmup)}),
              flush=True)
        return
    fl = counted_flops(w)
    r = run_gpu(w, args.steps, args.warmup)
    sec = r["ms_per_step"] / 1e3
    tflops = fl["total"] / sec / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    km = r["kernel_ms"]
    kflops = {"fwd": fl["k_fwd"], "dq": fl["k_dq"], "dkdv": fl["k_dkdv"],
              "bwd": fl["k_dq"] + fl["k_dkdv"]}
    # the backward's longest kernel, timed by events inside the timed region:
    # dk/dv, or the single backward kernel of short bf16 sequences
    dom = "bwd" if "bwd" in km else "dkdv"
    bwd_ms = km["bwd"] if dom == "bwd" else km["dq"] + km["dkdv"]
    ach = kflops[dom] / (km[dom] / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "H": w.H, "Hkv": w.Hkv, "hd": w.hd,
                   "scale": w.scale, "causal": True, "parallelism": "none (1 GPU)"},
        "pct_of_mfma_peak": round(100 * tflops / peak, 3),
        "tokens_per_s": round(w.B * w.S / sec, 1),
        "fwd_tflops": round(fl["fwd"] / (km["fwd"] / 1e3) / 1e12, 3),
        "bwd_tflops": round(fl["bwd"] / (bwd_ms / 1e3) / 1e12, 3),
        "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in km.items()},
        "kernel_timing": f"{dom}: events around it in every timed step; the others: loops of K "
                         "launches each, after the timed region",
        "warmup_run": {"steps": r["warmup_steps"], "seconds": r["warmup_s"],
                       "min_seconds": WARMUP_MIN_S},
        "step_roofline": step_roofline(w, r["ms_per_step"]),
        "roofline": {"bound": "mfma", "kernel": KERNEL_NAMES[dom],
                     "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ach / peak, 5), "traffic": measured_traffic(dom, w.name),
                     "alg_flops_per_launch": kflops[dom]},
        "device": r["device"],
    }
    if not args.no_secondary and args.workload is None:
        # every other workload of the metric, each a full fwd+bwd step of its own
        out["secondary"] = [run_secondary(inputs.WORKLOADS[n], args.steps, args.warmup)
                            for n in inputs.WORKLOADS if n != w.name]
    if not args.no_next:
        out["next_rows"] = {
            "qknorm_rope": run_norm(w, args.steps, args.warmup),
            "decode": run_decode(inputs.DECODE_WORKLOADS[inputs.DECODE_BENCH], args.steps,
                                 args.warmup),
            "decode_long_context_last_row": run_decode(
                inputs.DECODE_WORKLOADS["decode_long_b4_t2048_h16_hd64_bf16"], args.steps,
                args.warmup),
            "ragged": run_ragged(inputs.RAGGED_BENCH, args.steps, args.warmup),
            "composed": run_composed(w, max(3, args.steps // 5), max(1, args.warmup // 5))}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
