"""Host logic of bench.py (CPU): the single-GPU guard, the algorithmic FLOP
count of a slice, and the keying of the committed counter summaries on the
kernel code."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_flops_of_the_lite_slice():
    """116.77 GF of GEMMs and self-attention per block-step (14.01 TF over 4 x 30),
    0.25 GF of frame-local cross-attention per block-step (14.04 TF with it), and
    0.045 TF for the audio K/V, time MLP, patch embedding and head: 14.09 TF per
    batch-1 slice (0.587 TF per frame)."""
    total, hot = bench.flops_per_slice(synth.CONFIGS["slice"], 1, 4)
    assert abs(hot / 1e12 - 14.012) < 0.001
    assert abs(total / 1e12 - 14.09) < 0.005
    total3, _ = bench.flops_per_slice(synth.CONFIGS["slice"], 3, 4)
    assert abs(total3 / total - 3.0) < 1e-3          # every term scales with the batch except the time MLP


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {  // doubles\n  return 2 * x;\n}\n")
    b.write_text("// a new header comment\n\nint f(int x) {\n  return 2 * x;   \n}\n")
    c.write_text("int f(int x) {\n  return 3 * x;\n}\n")
    assert bench.kernel_code_hash(str(a)) == bench.kernel_code_hash(str(b))
    assert bench.kernel_code_hash(str(a)) != bench.kernel_code_hash(str(c))


def test_counter_summary_needs_the_current_code(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "k.json").write_text(json.dumps({"code_sha256": "abc", "hbm_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("abc", "k.json") == 123
    assert bench.traffic_from_profile("abd", "k.json") is None
    assert bench.traffic_from_profile("abc", "missing.json") is None


def test_committed_counter_summaries_match_the_kernel_code():
    """The committed FFN-down counter summaries were taken on the GEMM code in
    this tree (else bench.py reports traffic as null)."""
    h = bench.kernel_code_hash(os.path.join(ROOT, "audio_driven_talking_amd", "csrc", "gemm.hip"))
    for name in ("gemm_ffn2_slice_b1_counters.json", "gemm_mx_ffn2_slice_b1_counters.json"):
        d = json.load(open(os.path.join(ROOT, "profiles", name)))
        if d.get("code_sha256") != h:
            pytest.xfail(f"profiles/{name} predates the current gemm.hip code: re-take the counters")
        assert d["hbm_bytes_per_launch"] > d["algorithmic_bytes_per_launch"] > 0


def test_hot_class_flops_add_up():
    """The per-class FLOPs of the hot kernels add up to the slice's GEMM and
    attention FLOPs plus the cross-attention and the per-slice audio K/V; the
    hot fraction divides them by the summed class times."""
    cfg = synth.CONFIGS["slice"]
    per = bench.hot_flops_per_class(cfg, 1, 4)
    assert set(per) == set(bench.HOT_CLASSES)
    total, hot = bench.flops_per_slice(cfg, 1, 4)
    D, N, M = cfg.dim, cfg.tokens, cfg.tokens
    cross = 4 * 30 * 4 * M * cfg.audio_per_frame * D
    audio_kv = 30 * 2 * cfg.audio_tokens * D * 2 * D
    assert sum(per.values()) == hot + cross + audio_kv
    assert per["attn"] == 4 * 30 * 4 * N * N * D
    tf, frac = bench.hot_fraction({k: 1.0 for k in per}, per)   # 1 ms per class
    assert abs(tf - sum(per.values()) / (len(per) * 1e-3) / 1e12) < 1e-6
    assert abs(frac - tf / bench.PEAK_BF16_TFLOPS) < 1e-12


def test_vae_flops_of_the_slice_decoder():
    """Per convolution 2 x 27 C_in C_out per output position: conv_in 0.28,
    stage convolutions 9.06 + 18.12, 16.31 + 32.62, 30.81 + 61.61, conv_out
    44.84 GFLOP: 213.7 GFLOP per slice decode."""
    f = bench.vae_flops(synth.VAE_CONFIGS["slice"])
    assert abs(f / 1e9 - 213.65) < 0.05
