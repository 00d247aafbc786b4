"""Host-side logic of bench.py that needs no GPU: the one-GPU rule, the counter record that gates
the roofline's `traffic` figure on the GEMM source it was taken on, and the shape of the CPU
baseline the bench line reports."""
import hashlib
import json
import os
import subprocess
import sys

import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run_bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_a_distributed_launch_is_refused_too():
    r = _run_bench(["--steps", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _tree(tmp_path, source, record):
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "fp8_delayed_scaling_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemm.hip").write_bytes(source)
    (tmp_path / "profiles" / "gemm_fp8_qkv_counters.json").write_text(json.dumps(record))


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    src = b"// a kernel source\n"
    rec = {"source_sha256": hashlib.sha256(src).hexdigest(), "traffic_bytes_per_launch": 3.0e9}
    _tree(tmp_path, src, rec)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic_record("gemm_fp8_qkv_counters.json", "gemm.hip") == 3.0e9
    # the kernel source changed after the counters were taken: no traffic figure
    (tmp_path / "fp8_delayed_scaling_amd" / "csrc" / "gemm.hip").write_bytes(src + b"// edited\n")
    assert bench._traffic_record("gemm_fp8_qkv_counters.json", "gemm.hip") is None


def test_traffic_record_missing_or_unreadable_gives_null(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic_record("gemm_fp8_qkv_counters.json", "gemm.hip") is None
    _tree(tmp_path, b"x", {})
    (tmp_path / "profiles" / "gemm_fp8_qkv_counters.json").write_text("{not json")
    assert bench._traffic_record("gemm_fp8_qkv_counters.json", "gemm.hip") is None


def test_cpu_baseline_reports_the_contract_fields(monkeypatch):
    """The oracle timed on a bounded sample: value / unit / cores / kind / sample present, the
    thread counts stated, the FLOP count matching the sample described (shapes shrunk here so the
    test takes a fraction of a second)."""
    M, N, K = 64, 48, 32
    monkeypatch.setattr(bench, "M", M)
    monkeypatch.setattr(bench, "N", N)
    monkeypatch.setattr(bench, "K", K)
    monkeypatch.setattr(bench, "HIST_L", 8)
    monkeypatch.setattr(bench, "CT_SHAPES", [(32, 48), (64, 80), (48, 16)])
    monkeypatch.setattr(bench, "PREP_SHAPE", (40, 24))
    x = S.normal_bf16(S.seed_for(90, 0), (M, K), 1.0)
    w = S.normal_bf16(S.seed_for(90, 1), (N, K), 0.02)
    b = S.normal_bf16(S.seed_for(90, 2), (N,), 0.1)
    dy = S.normal_bf16(S.seed_for(90, 3), (M, N), 0.01)
    cb = bench.cpu_baseline(x, w, b, dy)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["cores"] == bench._host_cores()
    assert cb["value"] > 0 and cb["seconds"] >= 0
    assert "16 of the 64 token rows" in cb["sample"] and f"3 x 2 x 16 x {N} x {K}" in cb["sample"]
    fam = cb["cast_family"]
    assert set(fam["cast_transpose_GBps"]) == {"32x48", "64x80", "48x16"}
    assert fam["backward_prep_40x24_GBps"]["GBps_1"] > 0 and fam["small_forward_128x256x256_us"] > 0


def test_threaded_oracle_driver_equals_the_oracle():
    """Row blocks on several host threads reassemble into exactly the oracle's own outputs."""
    import numpy as np

    import oracle
    x = S.outlier_bf16(S.seed_for(90, 5), (97, 40), 1.0)
    q, qt, a, si = oracle.cast_transpose(x, 0.5, 0)
    q2, qt2, a2, db2 = bench._oracle_ct(oracle, x, 0.5, 0, 6, with_dbias=True)
    assert np.array_equal(q, q2) and np.array_equal(qt, qt2) and np.float32(a) == np.float32(a2)
    assert np.allclose(db2, oracle.dbias(x), rtol=0, atol=1e-12)
    A, B = q[:, :32], q2[5:50, :32]
    r = oracle.gemm_bias(A, 0, 0.25, B, 0, 2.0, None)
    assert np.allclose(bench._oracle_gemm(oracle, A, 0, 0.25, B, 0, 2.0, None, 4), r, rtol=1e-15, atol=0)
