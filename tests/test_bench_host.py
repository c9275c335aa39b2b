"""CPU checks of bench.py's host logic: the FLOP accounting, the reading of the
committed HBM-traffic summaries, and the refusal of more than one GPU.  No
GPU is touched (the multi-GPU refusal returns before any device call)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("gattn_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_flop_accounting_is_the_pages_attention_term_on_causal_pairs():
    """12 hs per causal pair per (b, h) for forward + backward (the MFU
    estimate's 12 H hs T per token, restricted to j <= i), the backward twice
    the forward; at B12 H12 T1024 hs64 that is 58.04 GFLOP per layer."""
    b = _bench()
    B, H, T, hs = 12, 12, 1024, 64
    fwd, bwd = b.flops(B, H, T, hs)
    pairs = sum(i + 1 for i in range(T))  # j <= i, counted by brute force
    assert fwd == 4 * hs * pairs * B * H
    assert bwd == 2 * fwd
    assert fwd + bwd == 12 * hs * pairs * B * H
    assert round((fwd + bwd) / 1e9, 2) == 58.04
    # the FlashAttention-style count charges the backward 10 hs per pair
    assert b.flops(B, H, T, hs, bwd_per_pair=10)[1] == 10 * hs * pairs * B * H
    # T = 1: one pair per (b, h)
    assert b.flops(2, 3, 1, 8) == (4 * 8 * 6, 8 * 8 * 6)


def test_traffic_is_read_only_for_the_kernel_source_it_was_taken_on(tmp_path, monkeypatch):
    b = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = os.path.join(b.CSRC, "mfma16_bwd.hip")
    digest = b.source_digest(src)
    (prof / "dkdv_t_traffic.txt").write_text(
        f"kernel_source_sha256_16: {digest}\nhbm_bytes_per_launch: 140512522\n")
    (prof / "dq_t_traffic.txt").write_text(
        "kernel_source_sha256_16: 0123456789abcdef\nhbm_bytes_per_launch: 1\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.read_traffic("dkdv", "t") == 140512522.0
    assert b.read_traffic("dq", "t") is None  # taken on another source
    assert b.read_traffic("fwd", "t") is None  # no summary
    monkeypatch.setattr(b, "source_digest", lambda path: "ffffffffffffffff")
    assert b.read_traffic("dkdv", "t") is None  # the source changed since


def test_more_than_one_gpu_is_refused_with_a_message():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, env=env, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
