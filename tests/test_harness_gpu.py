"""Harness checks on the GPU: the library allocates no device memory (every
entry point, after a first warm-up call that loads the kernels' code), and the
benchmark CLI prints one JSON line with the fields its contract names."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import gpu_helpers as Hh
from bwd_head_rms_amd import inputs

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_allocates_nothing():
    import torch
    from bwd_head_rms_amd import api
    B, S, H, Hkv, hd = 2, 300, 4, 2, 64
    a = inputs.generate(B, S, H, Hkv, hd, seed=3, dtype="bf16")
    t = Hh.to_dev(a, "bf16")
    f32 = dict(dtype=torch.float32, device="cuda")
    o, lse = torch.empty_like(t["q"]), torch.empty((B, H, S), **f32)
    dq, dk, dv = (torch.empty(x.shape, **f32) for x in (t["q"], t["k"], t["k"]))
    ws = torch.empty((api.workspace_bytes(B, S, H, Hkv, hd, 1) // 4,), **f32)
    lens = torch.tensor([S, 123], dtype=torch.int32, device="cuda")
    p = torch.empty((B, H, S, S), **f32)
    ds = torch.empty((B, H, S, S), **f32)
    x = torch.randn((B, S, H, hd), device="cuda").to(torch.bfloat16)
    w = torch.ones(hd, **f32)
    g = torch.randn((B, H, S, hd), **f32)
    nout = torch.empty((B, H, S, hd), dtype=torch.bfloat16, device="cuda")
    ndx, ndw = torch.empty((B, S, H, hd), **f32), torch.empty(hd, **f32)
    nws = torch.empty((max(1, api.qknorm_rope_workspace_bytes(B, S, H, hd) // 4),), **f32)
    qd = t["q"][:, :, -1].contiguous()
    od, ld = torch.empty_like(qd), torch.empty((B, H), **f32)
    dws = torch.empty((max(1, api.decode_workspace_bytes(B, S, H, Hkv, hd) // 4),), **f32)

    def every_entry_point():
        api.fwd(t["q"], t["k"], t["v"], o=o, lse=lse)
        api.bwd(t["q"], t["k"], t["v"], o, lse, t["dO"], dq=dq, dk=dk, dv=dv, workspace=ws)
        api.fwd(t["q"], t["k"], t["v"], o=o, lse=lse, lens=lens)
        api.bwd(t["q"], t["k"], t["v"], o, lse, t["dO"], dq=dq, dk=dk, dv=dv, workspace=ws, lens=lens)
        api.composed_fwd(t["q"], t["k"], t["v"], p=p)
        api.composed_bwd(t["q"], t["k"], t["v"], p, t["dO"], ds=ds)
        api.qknorm_rope_fwd(x, w, out=nout)
        api.qknorm_rope_bwd(x, w, g, dx=ndx, dw=ndw, workspace=nws)
        api.decode(qd, t["k"], t["v"], lens=lens, o=od, lse=ld, workspace=dws)
        torch.cuda.synchronize()

    # the first round loads every kernel's code and fills torch's cache with the
    # few outputs the bindings allocate (reused afterwards, so no new device memory)
    every_entry_point()
    free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    for _ in range(3):
        every_entry_point()
    free1, alloc1 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    Hh.log(f"  device free before {free0}, after {free1}; torch allocated {alloc0} -> {alloc1}")
    assert free1 == free0, "device memory changed across calls of the library"


def test_bench_cli_emits_contract_json():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--no-next"], capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip().startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
              "cpu_baseline"):
        assert k in d, f"missing {k}"
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    # warm-up: at least the W steps asked for, and at least its minimum duration
    wr = d["warmup_run"]
    assert wr["steps"] >= 1 and wr["seconds"] >= wr["min_seconds"] > 0
    assert d["config"]["workload"] == inputs.LONG_CONTEXT and d["dtype"] == "bf16"
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, f"roofline misses {k}"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["threads_used"] >= 1 and cb["logical_cpus"] >= 1 and "cpu_model" in cb
    # every other workload of the metric, each with its own roofline
    sec = {e["workload"]: e for e in d["secondary"]}
    assert set(sec) == set(inputs.WORKLOADS) - {inputs.LONG_CONTEXT}
    from bwd_head_rms_amd import _lib
    L = _lib.lib()
    for e in sec.values():
        # short bf16 sequences run the backward as one kernel
        single = L.xattn_bwd_kernel_count(e["B"], e["S"], e["H"], e["Hkv"], e["hd"],
                                          _lib.BF16 if e["dtype"] == "bf16" else _lib.F32) == 1
        want = {"fwd", "bwd"} if single else {"fwd", "dq", "dkdv"}
        assert e["ms_per_step"] > 0 and set(e["kernel_avg_us"]) == want
        assert e["roofline"]["bound"] in ("mfma", "hbm") and 0 < e["roofline"]["frac"] <= 1
    assert np.isfinite(d["value"]) and d["value"] > 0
    Hh.log(f"  bench JSON ok: value {d['value']} {d['unit']}")
