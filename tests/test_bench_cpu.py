"""Host logic of bench.py (no GPU).

- `--gpus N` with N != 1 exits with status 2 and a message, before anything touches a
  GPU, and prints no JSON line.
- The grouped GEMM's HBM traffic and per-pass trace figures are read from the summaries
  under profiles/ only while `gemm_mfma.hip` still has the SHA-256 recorded in them:
  a changed source, a missing summary or a summary without its machine-readable line
  gives None (the bench line then reports null, never a stale figure).
"""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module(root):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.ROOT = str(root)
    return mod


def _tree(tmp_path, source_text):
    src_dir = tmp_path / "token_dispatch_expert_router_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / "gemm_mfma.hip").write_text(source_text)
    (tmp_path / "profiles").mkdir()
    return hashlib.sha256(source_text.encode()).hexdigest()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_follows_the_kernel_source(tmp_path):
    sha = _tree(tmp_path, "// kernels\n")
    rec = {"kernel_source_sha256": sha, "traffic_bytes_per_step": 123, "algorithmic_bytes_per_step": 100}
    (tmp_path / "profiles" / "gemm_mfma_w1_hbm_traffic.md").write_text(
        "# summary\n\nmachine-readable: " + json.dumps(rec) + "\n")
    b = _bench_module(tmp_path)
    assert b.gemm_traffic("w1") == rec
    assert b.gemm_traffic("w2") is None  # no summary for this workload
    (tmp_path / "token_dispatch_expert_router_amd" / "csrc" / "gemm_mfma.hip").write_text(
        "// kernels, changed\n")
    assert b.gemm_traffic("w1") is None


def test_passes_follow_the_kernel_source(tmp_path):
    sha = _tree(tmp_path, "// kernels\n")
    passes = {"fwd gate/up": {"avg_us": 1.0, "calls": 22, "frac": 0.5}}
    rec = {"kernel_source_sha256": sha, "passes": passes}
    (tmp_path / "profiles" / "moe_layer_mixtral_8x22b_kernel_trace.md").write_text(
        "machine-readable: " + json.dumps(rec) + "\n")
    (tmp_path / "profiles" / "mixtral_g8t8_kernel_trace.md").write_text("# no record line\n")
    b = _bench_module(tmp_path)
    assert b.gemm_passes("mixtral_8x22b") == passes
    assert b.gemm_passes("mixtral_g8t8") is None
    (tmp_path / "token_dispatch_expert_router_amd" / "csrc" / "gemm_mfma.hip").write_text("// x\n")
    assert b.gemm_passes("mixtral_8x22b") is None
