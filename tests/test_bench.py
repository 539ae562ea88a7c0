"""CPU checks of bench.py's bookkeeping: the algorithmic byte and flop
figures its roofline divides by, the digest gate on recorded counter
figures, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gru_corrected_draft_amd import synth  # noqa: E402

S8 = synth.MODELS["qwen3-8b"]


def test_lmhead_figures_match_the_problem_size():
    # 2 flops per multiply-add over 15 positions x B requests x H x V:
    # 18.7 GFLOP at one request and 1195 GFLOP at 64 (Qwen3-8B shapes)
    assert bench.algorithmic(S8, 1, 0)["lm_flops"] == pytest.approx(18.67e9, rel=1e-3)
    assert bench.algorithmic(S8, 64, 0)["lm_flops"] == pytest.approx(1194.9e9, rel=1e-3)
    # lm_head read once (1244.7 MB in bf16) plus the hiddens and the fp32
    # base logits written once (9.1 MB at one request, 583.4 MB at 64)
    assert bench.algorithmic(S8, 1, 0)["lm_bytes"] == pytest.approx(1244.7e6 + 0.12e6 + 9.12e6, rel=1e-3)
    assert bench.algorithmic(S8, 64, 0)["lm_bytes"] == pytest.approx(1244.7e6 + 7.86e6 + 583.4e6, rel=1e-3)


def test_correction_bytes_by_mode():
    V, r = S8.vocab, S8.proj_dim
    # full vocabulary: fc2 (311.2 MB) and b2 once, one fp32 base row per request, u
    full = bench.algorithmic(S8, 8, 0)["correct_bytes"]
    assert full == V * r * 2 + V * 2 + 8 * V * 4 + 8 * r * 4
    # a pool of K rows per request: gathered rows, biases, compact base values, ids
    pool = bench.algorithmic(S8, 8, 2048)["correct_bytes"]
    assert pool == 8 * 2048 * (r * 2 + 2 + 4 + 4) + 8 * r * 4
    assert pool < full / 9
    # group unions: each union row once with its 16-byte record
    uni = bench.algorithmic(S8, 64, 2048, union_sizes=[50000, 51000])["correct_bytes"]
    assert uni == 101000 * (r * 2 + 16) + 64 * 2048 * 4 + 64 * r * 4


def test_step_bytes_are_the_stacked_rows_once():
    g, r = S8.gru_hidden, S8.proj_dim
    stacked, fc1 = (r + 3 * g) * g * 2, r * g * 2  # [fc1; W_hh] and fc1 alone, bf16
    # one correction step (2 proposals): the last step needs no W_hh rows;
    # a request's gate inputs and outputs add ~0.05 MB
    last = bench.algorithmic(S8, 1, 0, proposals=2)["step_bytes"]
    assert fc1 <= last < fc1 + 0.1e6
    # 14 steps: 13 with the stacked rows, the last without, averaged per launch
    step = bench.algorithmic(S8, 1, 0)["step_bytes"]
    assert step == pytest.approx((13 * stacked + fc1) / 14, abs=0.1e6)


def _profile(tmp_path, digest, body):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / "correct_8b_b1_k0_pmc.md").write_text(
        f"# counters\n\n{body}\nkernel_source_digest: {digest}\n")


def test_recorded_figures_need_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("correct", "8b_b1_k0", "abc") is None  # no file
    _profile(tmp_path, "abc", "hbm_bytes_per_launch: 312829056\nmfma_util: 0.2215\n")
    assert bench.read_traffic("correct", "8b_b1_k0", "abc") == 312829056.0
    assert bench.read_counter("correct", "8b_b1_k0", "abc", "mfma_util") == pytest.approx(0.2215)
    # taken on other sources: not reported
    assert bench.read_traffic("correct", "8b_b1_k0", "def") is None
    assert bench.read_counter("correct", "8b_b1_k0", "abc", "no_such_field") is None


def test_kernel_digest_covers_every_source(tmp_path, monkeypatch):
    d1 = bench.kernel_source_digest()
    assert len(d1) == 16 and d1 == bench.kernel_source_digest()
    csrc = tmp_path / "gru_corrected_draft_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d2 = bench.kernel_source_digest()
    (csrc / "b.h").write_text("y")
    d3 = bench.kernel_source_digest()
    assert d3 != d2 != d1
    # comments and blank lines do not count; code does, even one character
    (csrc / "b.h").write_text("// a note\ny  /* and another */\n\n")
    assert bench.kernel_source_digest() == d3
    (csrc / "b.h").write_text("y;")
    assert bench.kernel_source_digest() != d3


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_lower_bound_matches_the_byte_table():
    """The block's roofline time from the algorithmic bytes: 8B B = 1 K = 0
    about 0.72 ms (lm_head at HBM speed plus 14 fc2 passes and step
    products), B = 64 K = 0 about 1.19 ms (the LM-head MFMA-bound)."""
    import bench
    from gru_corrected_draft_amd import synth
    shape = synth.MODELS["qwen3-8b"]
    lb1 = bench.lower_bound_ms(bench.algorithmic(shape, 1, 0), shape, 1, 0, 15)
    lb64 = bench.lower_bound_ms(bench.algorithmic(shape, 64, 0), shape, 64, 0, 15)
    assert 0.70 < lb1 < 0.74, lb1
    assert 1.10 < lb64 < 1.25, lb64
    assert bench.MATRIX[0] == ("8b_b1", 0) and len(bench.MATRIX) == 7
