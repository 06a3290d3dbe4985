"""bench.py's host-side pieces: the one-GPU guard and the stored counter figures."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

W2 = "mixtral_r4_t4096_h4096_f14336_e8_top2"


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a configuration it did not run


def test_missing_summary_gives_none():
    assert bench.stored_figures("no_such_summary.md") is None
    assert bench.stored_traffic("no_such_workload", 64, True) is None
    assert bench.stored_mfma("no_such_workload", 64, False) is None


def test_stale_summary_gives_none(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "pmc_gemm1_w_tb64.md").write_text(
        "- gemm_source_sha256_16: `0000000000000000`\n- traffic_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "ffffffffffffffff")
    assert bench.stored_traffic("w", 64, False) is None
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0000000000000000")
    assert bench.stored_traffic("w", 64, False) == 123.0


@pytest.mark.parametrize("gathered", [False, True])
def test_committed_figures_are_physical(gathered):
    """When the committed summaries match the sources, their figures are in the
    range the hardware allows: MFMA busy a fraction, a clock at or below the
    2.4 GHz peak clock, traffic at least the compulsory bytes of the launch."""
    t = bench.stored_traffic(W2, 64, gathered)
    m = bench.stored_mfma(W2, 64, gathered)
    if t is None and m is None:
        pytest.skip("GEMM sources changed since the summaries were taken")
    if m is not None:
        busy, clk = m
        assert 0.05 < busy <= 1.0
        assert 0.5 < clk <= 2.45
    if t is not None:
        # padded rows 8448, valid 8219, H 4096, F 14336, both experts receive rows, W1 and W3
        a_rows = 8219 if gathered else 8448
        compulsory = 2 * (a_rows * 4096 + 2 * 2 * 14336 * 4096 + 8448 * 14336)
        assert t >= compulsory


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    for f in bench.GEMM_SOURCES:
        p = tmp_path / f
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text("int a = 1;  // one\n\n// a note\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.gemm_source_hash()
    (tmp_path / bench.GEMM_SOURCES[0]).write_text("int a = 1;  // the first\n// another note\nint b = 2;   \n")
    assert bench.gemm_source_hash() == h0
    (tmp_path / bench.GEMM_SOURCES[0]).write_text("int a = 1;\nint b = 3;\n")
    assert bench.gemm_source_hash() != h0
