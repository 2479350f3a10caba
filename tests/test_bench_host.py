"""bench.py's host logic on the CPU: the kernel-code hash that keys the committed
traffic counters ignores comments and layout but not code, the counters scale by the
copy calibration, the issue-port figures come from the committed counters, and more
than one GPU is refused with a message."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _sha_of(bench, tmp_path, texts):
    files = []
    for i, t in enumerate(texts):
        f = tmp_path / f"src{i}.hip"
        f.write_text(t)
        files.append(str(f))
    old = bench.KERNEL_SOURCES
    bench.KERNEL_SOURCES = files
    try:
        return bench.kernel_code_sha()
    finally:
        bench.KERNEL_SOURCES = old


def test_code_hash_ignores_comments_and_layout(bench, tmp_path):
    a = "int f(int x) {\n  return x + 1; // one\n}\n/* block\n comment */\nconst char *s = \"// kept\";\n"
    b = "int f(int x)\n{\n    return x + 1;   // a different comment\n}\nconst char *s = \"// kept\";\n"
    c = "int f(int x) { return x + 2; }\nconst char *s = \"// kept\";\n"
    d = "int f(int x) { return x + 1; }\nconst char *s = \"// changed\";\n"
    ha, hb, hc, hd = (_sha_of(bench, tmp_path, [t]) for t in (a, b, c, d))
    assert ha == hb            # comments and whitespace only
    assert ha != hc            # code changed
    assert ha != hd            # a string literal is code, not a comment


def test_committed_traffic_file_parses_and_scales(bench):
    """The committed counter summary of the headline kernels (the whole 14B-shaped cache,
    25,165,824 blocks per launch) parses, and its scaled FETCH_SIZE + WRITE_SIZE sit
    within a few percent of the algorithmic 306 bytes per block."""
    rec = bench.read_summary(bench.TRAFFIC_FILE)
    assert int(rec["copy_bytes"]) == 268435456
    algorithmic = 25165824 * 306 / 1024
    for op in ("encode_turbo3", "decode_turbo3"):
        assert f"{op}.fetch_size_kib" in rec and f"{op}.write_size_kib" in rec
        # the same arithmetic as measured_traffic, independent of the hash check
        copy_kib = int(rec["copy_bytes"]) / 1024
        fetch = float(rec[f"{op}.fetch_size_kib"]) * copy_kib / float(rec["copy_fetch_size_kib"])
        write = float(rec[f"{op}.write_size_kib"]) * copy_kib / float(rec["copy_write_size_kib"])
        assert 0.99 < (fetch + write) / algorithmic < 1.05, op


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_issue_utilisation_from_the_committed_counters(bench, monkeypatch):
    """The decode-step q.K and attention carry their issue-port utilisation from the
    committed counter summaries: fractions in (0, 1), and None once the kernel code no
    longer has the hash the counters were taken with."""
    for which in ("qk", "attn"):
        rec = bench.read_summary(bench.ISSUE_FILES[which])
        monkeypatch.setattr(bench, "kernel_code_sha", lambda: rec["kernel_code_sha256_16"])
        u = bench.issue_utilisation(which)
        for k in ("valu_per_simd", "lds_per_cu", "mfma_per_simd"):
            assert 0.0 < u[k] < 1.0, (which, k, u)
        monkeypatch.setattr(bench, "kernel_code_sha", lambda: "0" * 16)
        assert bench.issue_utilisation(which) is None
