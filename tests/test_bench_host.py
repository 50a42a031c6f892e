"""Host-side checks of bench.py's bookkeeping (no GPU): which decode calls are timed,
how the committed counter summaries are read, and the algorithmic byte and flop counts."""
import os
import shutil

import pytest

import bench
from cross_model_shared_amd import workload as W


def test_timed_layers_sample_every_layer():
    layers = 36
    seen = set()
    for step in range(20):
        t = bench.timed_layers(step, layers)
        assert len(t) == bench.TIMED_LAYERS_PER_STEP
        assert all(0 <= x < layers for x in t)
        seen |= t
    assert seen == set(range(layers))
    assert bench.timed_layers(0, 2) == {0, 1}       # short counter runs time every call


def test_counter_summary_values_are_sane():
    """The committed summaries' figures, when they were taken on the current kernels (the bench
    reports null otherwise, until the counters are taken again)."""
    traffic, c = bench.measured_traffic(), bench.extend_counters()
    if traffic is None or c is None:
        pytest.skip("counter summaries predate the current kernel sources")
    assert 1.0 <= traffic / 2_794_965_412 < 1.05     # HBM bytes of a decode call vs algorithmic
    assert 0.0 < c["mfma_busy_frac"] <= 1.0
    flops = bench.extend_flops([8192] * 16, [512] * 16, 32, 128)
    assert 1.0 <= c["mfma_flop_executed"] / flops < 1.1   # the row-sum steps and masked diagonal halves


def test_stale_summary_reads_as_none(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, bench.PMC_SUMMARY)
    copy = tmp_path / "summary.md"
    shutil.copy(src, copy)
    text = copy.read_text().replace("kernel_source_sha256: `", "kernel_source_sha256: `0")
    copy.write_text(text)
    assert bench.summary_values(str(copy), bench.DECODE_SOURCES) is None
    assert bench.summary_values(str(tmp_path / "missing.md"), bench.DECODE_SOURCES) is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("int x = 1;  // one\n\n// note\nint y = 2;\n")
    b = tmp_path / "b.hip"
    b.write_text("int x = 1;  // changed comment\nint y = 2;\n")
    c = tmp_path / "c.hip"
    c.write_text("int x = 3;\nint y = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash(["a.hip"]) == bench.kernel_source_hash(["b.hip"])
    assert bench.kernel_source_hash(["a.hip"]) != bench.kernel_source_hash(["c.hip"])


def test_algorithmic_counts():
    wl = W.make_workload("qwen3_8b_n8")
    per_call = bench.decode_bytes(wl.lens, 64, 8, 32, 8, 128) + bench.append_bytes(64, 8, 128)
    assert per_call == 2_794_965_412
    assert bench.extend_flops([8192] * 16, [512] * 16, 32, 128) == 1_133_938_475_008
    # one token of one head: K and V rows read and written
    assert bench.append_bytes(1, 1, 128) == 128 * 2 * 2 * 2


@pytest.mark.parametrize("n", [2, 8])
def test_multi_gpu_request_is_refused(n):
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
