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
