"""The benchmark CLI on the CPU: more than one GPU is refused with a message;
recorded HBM traffic is tied to the kernel sources and compile flags it was
measured with."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_per_source_flags_name_built_sources():
    from bwd_head_rms_amd import build
    assert set(build.SOURCE_FLAGS) <= set(build.SOURCES)


def test_traffic_record_follows_compile_flags(monkeypatch):
    """A change of a kernel's own compile flags changes its source hash, so the
    recorded traffic stops being reported until it is measured again; the other
    kernels' hashes are untouched."""
    import bench
    from bwd_head_rms_amd import build, inputs
    before = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_FILES}
    flags = dict(build.SOURCE_FLAGS)
    flags[bench.KERNEL_FILES["dq"]] = flags.get(bench.KERNEL_FILES["dq"], []) + ["-DXATTN_PROBE"]
    monkeypatch.setattr(build, "SOURCE_FLAGS", flags)
    after = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_FILES}
    assert after["dq"] != before["dq"]
    assert after["fwd"] == before["fwd"] and after["dkdv"] == before["dkdv"]
    if bench.MEASURED_TRAFFIC["dq"]["src"] == before["dq"]:
        monkeypatch.undo()
        assert bench.measured_traffic("dq", inputs.LONG_CONTEXT) is not None
        monkeypatch.setattr(build, "SOURCE_FLAGS", flags)
    assert bench.measured_traffic("dq", inputs.LONG_CONTEXT) is None


def test_algorithmic_counts_match_the_workload_table():
    """Counted FLOPs (14 hd nnz B H) and algorithmic bytes of each workload's
    step, as tabulated for the metric's configurations (MB = 1e6 bytes)."""
    import bench
    from bwd_head_rms_amd import inputs
    want = {  # name: (GFLOP counted, MB)
        "tiny_b1_s16_h2_hd16_f32": (6.09e-5, 0.025),
        "dim384_b16_s256_h12_hd32_f32": (2.830, 75.9),
        "dim384_b32_s256_h12_hd32_bf16": (5.659, 95.2),
        "gqa_b16_s1024_h8_kv2_hd64_f32": (60.19, 252.7),
        "gqa_b16_s1024_h8_kv2_hd64_bf16": (60.19, 152.0),
        "long_b4_s2048_h16_hd64_bf16": (120.32, 252.7),
    }
    for n, (gf, mb) in want.items():
        w = inputs.WORKLOADS[n]
        assert abs(bench.counted_flops(w)["total"] / 1e9 / gf - 1) < 2e-3, n
        assert abs(bench.alg_bytes(w) / 1e6 - mb) <= 0.05 + 1e-3 * mb, n
    # the long-context step: bound by the matrix cores, 47.8 us at the bf16 peak
    r = bench.step_roofline(inputs.WORKLOADS[inputs.LONG_CONTEXT], 0.2)
    assert r["bound"] == "mfma" and abs(r["t_bound_us"] - 47.81) < 0.05
    # the batch-32 dim384 bf16 step: bound by HBM, 11.9 us at 8 TB/s
    r = bench.step_roofline(inputs.WORKLOADS["dim384_b32_s256_h12_hd32_bf16"], 0.05)
    assert r["bound"] == "hbm" and abs(r["t_bound_us"] - 11.89) < 0.05
