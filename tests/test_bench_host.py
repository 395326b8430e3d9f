"""Host-side pieces of bench.py (no GPU): the source hash that keys the
committed HBM counters to the kernels they were taken on."""
import os
import shutil

import bench


def _copy_tree(tmp_path):
    src = os.path.join(bench.ROOT, "fp8_scaled_quantization_scale_amd", "csrc")
    dst = tmp_path / "fp8_scaled_quantization_scale_amd" / "csrc"
    shutil.copytree(src, dst)
    return dst


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench._source_sha()
    gemm = csrc / "gemm.hip"
    text = gemm.read_text()
    # an edited comment, a new block comment and re-indented blank space: same hash
    gemm.write_text(text.replace("// gemm.hip --", "// gemm.hip (edited) --", 1) + "\n/* trailing note */\n\n")
    assert bench._source_sha() == base
    # a changed constant: a different hash
    gemm.write_text(text.replace("constexpr int kLag = 4;", "constexpr int kLag = 5;", 1))
    assert "constexpr int kLag = 4;" in text
    assert bench._source_sha() != base
    # the measurement kernels are not part of the hash
    gemm.write_text(text)
    probe = csrc / "probe.hip"
    probe.write_text(probe.read_text() + "\nstatic int unused_probe_constant = 1;\n")
    assert bench._source_sha() == base


def test_traffic_entry_needs_the_current_hash(tmp_path, monkeypatch):
    _copy_tree(tmp_path)
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench._source_sha()
    (prof / "traffic.json").write_text(
        '{"w": {"gemm_fprop": {"bytes_per_launch": 123, "source_sha": "%s"},'
        ' "gemm_dgrad": {"bytes_per_launch": 456, "source_sha": "0000000000000000"}}}' % sha)
    assert bench._traffic("w", "gemm_fprop") == 123
    assert bench._traffic("w", "gemm_dgrad") is None
    assert bench._traffic("other", "gemm_fprop") is None


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
