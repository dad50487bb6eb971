"""Host-side logic of bench.py (no GPU): the digest that ties the committed
traffic counters to the GEMM's code."""
import os
import shutil

import bench


def _copy_sources(tmp_path):
    paths = []
    for src in bench.GEMM_SOURCES:
        dst = tmp_path / os.path.basename(src)
        shutil.copy(src, dst)
        paths.append(str(dst))
    return paths


def test_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    paths = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "GEMM_SOURCES", paths)
    before = bench.gemm_code_digest()
    with open(paths[0], "a") as f:
        f.write("\n// a trailing comment\n/* and a\n   block comment */\n\n")
    text = open(paths[1]).read().replace("\n", "\n\n", 3)
    open(paths[1], "w").write(text)
    assert bench.gemm_code_digest() == before


def test_digest_changes_with_the_code(tmp_path, monkeypatch):
    paths = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "GEMM_SOURCES", paths)
    before = bench.gemm_code_digest()
    text = open(paths[0]).read()
    assert "kMinSkSteps" in open(paths[2]).read()
    open(paths[2], "a").write("\nconstexpr int kUnusedForTheTest = 1;\n")
    assert bench.gemm_code_digest() != before
    open(paths[0], "w").write(text.replace("kXcdRows", "kXcdRowz", 1))
    assert bench.gemm_code_digest() != before


def test_traffic_is_void_when_the_digest_differs(tmp_path, monkeypatch):
    paths = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "GEMM_SOURCES", paths)
    traffic = tmp_path / "traffic.txt"
    traffic.write_text(
        "gemm_code_sha256: %s\ncopy_bytes: 1024\ncopy_fetch_kib: 0.5\ncopy_write_kib: 1.0\n"
        "gateup_fetch_kib: 2.0\ngateup_write_kib: 3.0\n" % bench.gemm_code_digest())
    monkeypatch.setattr(bench, "traffic_file",
                        lambda w: str(traffic) if w == "dsv3_skew" else str(tmp_path / "none.txt"))
    # reads scaled by 1024 / (1024 * 0.5) = 2, writes by 1
    assert bench.measured_traffic("dsv3_skew") == 1024.0 * (2.0 * 2 + 3.0 * 1)
    assert bench.measured_traffic("qwen3") is None
    open(paths[0], "a").write("\nstatic int changed;\n")
    assert bench.measured_traffic("dsv3_skew") is None


def test_host_info_names_the_cpu_share():
    info = bench.host_info()
    assert 1 <= info["threads"] <= info["affinity_cpus"]
    assert info["cpu_model"] and info["blas"]


def test_more_than_one_gpu_is_refused():
    """The bench measures one GPU: --gpus N > 1 exits at once with a message
    (before torch is imported), so no multi-GPU figure is ever printed."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
