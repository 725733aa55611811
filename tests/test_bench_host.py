"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts the roofline uses, and the rule that counter-measured traffic is
reported only for the kernel sources it was measured on."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    n = 4096
    assert bench.algorithmic_bytes("bf16", n, n, n) == 2 * (n * n + n * n) + 2 * n * n
    assert bench.algorithmic_bytes("f32", n, n, n) == 4 * 3 * n * n
    # fp8: one byte per operand element, bf16 out, one fp32 scale per 64 x 64 block of A and B
    m = 8192
    blocks = (m // 64) * (m // 64)
    assert bench.algorithmic_bytes("fp8", m, m, m) == 2 * m * m + 2 * m * m + 4 * 2 * blocks
    # ragged: partial scale blocks count as whole ones
    assert bench.algorithmic_bytes("fp8", 65, 1, 1) == 65 + 1 + 2 * 65 + 4 * (2 * 1 + 1 * 1)


def test_tflops_is_two_mnk_over_time():
    assert abs(bench.tflops(4096, 4096, 4096, 1e-4) - 2 * 4096 ** 3 / 1e-4 / 1e12) < 1e-9


def _fake_tree(tmp_path, fetch, write, digest):
    csrc = tmp_path / "dense_gemm_13_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.HEADLINE_KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "dense_gemm_13_amd", "csrc", f), csrc / f)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_x.txt").write_text(
        f"# test\nkernel_source_digest: {digest}\nfetch_bytes_per_launch: {fetch}\n"
        f"write_bytes_per_launch: {write}\n")


def test_measured_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _fake_tree(tmp_path, 1000.0, 24.0, "0" * 16)
    assert bench.measured_traffic("x") is None            # taken on other sources
    digest = bench.kernel_source_digest()
    (tmp_path / "profiles" / "traffic_x.txt").unlink()
    shutil.rmtree(tmp_path / "profiles")
    shutil.rmtree(tmp_path / "dense_gemm_13_amd")
    _fake_tree(tmp_path, 1000.0, 24.0, digest)
    assert bench.measured_traffic("x") == 1024
    # any change to a headline source invalidates it
    src = tmp_path / "dense_gemm_13_amd" / "csrc" / bench.HEADLINE_KERNEL_SOURCES[0]
    src.write_text(src.read_text() + "\n// changed\n")
    assert bench.measured_traffic("x") is None
    assert bench.measured_traffic("missing") is None


def test_committed_traffic_summary_parses():
    """The committed headline summary has the fields bench.py reads."""
    path = os.path.join(ROOT, "profiles", "traffic_bf16_4096.txt")
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert len(kv["kernel_source_digest"]) == 16
    assert float(kv["fetch_bytes_per_launch"]) > 0 and float(kv["write_bytes_per_launch"]) > 0
