"""Host-side checks of bench.py's contract and of its flop and byte counts
(no GPU): the one-GPU refusal, the useful-flop convention, the count of
query-key pairs inside a mask against brute force, and that a stale HBM
counter record yields no traffic figure."""

import json
import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "ONE GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == ""  # no JSON line for a refused run


def test_useful_flops():
    c4 = dict(B=1, H=32, N=32768, d=128, causal=True)
    assert bench.fwd_flops(c4) == 4.0 * 32 * 32768 ** 2 * 128 / 2  # 8.796 TFLOP
    assert abs(bench.fwd_flops(c4) - 8.7961e12) < 1e8
    c5 = dict(B=4, H=16, N=4096, d=128, causal=True)
    assert bench.bwd_flops(c5) == 2.5 * bench.fwd_flops(c5)
    c2 = dict(B=4, H=16, N=2048, d=64, causal=False)
    assert bench.fwd_flops(c2) == 4.0 * 64 * 2048 ** 2 * 64


def test_algorithmic_bytes():
    c = dict(B=1, H=32, N=32768, d=128, causal=True)
    # Q, K, V read and O written in bf16, LSE written in fp32
    assert bench.fwd_algorithmic_bytes(c) == 4 * 32768 * 32 * 128 * 2 + 32 * 32768 * 4


def _pairs_brute(Nq, Nk, causal, window):
    n = 0
    for i in range(Nq):
        p = i + Nk - Nq
        for j in range(Nk):
            ok = True
            if causal and j > p:
                ok = False
            if window > 0 and abs(p - j) >= window:
                ok = False
            n += ok
    return n


def test_visible_pairs_against_brute_force():
    assert bench.visible_pairs(64, 64, True) == 64 * 65 // 2
    assert bench.visible_pairs(64, 64, False) == 64 * 64
    rng = np.random.default_rng(3)
    for _ in range(40):
        Nq, Nk = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        causal = bool(rng.integers(0, 2))
        window = int(rng.integers(0, 12))
        assert bench.visible_pairs(Nq, Nk, causal, window) == _pairs_brute(Nq, Nk, causal, window), (Nq, Nk, causal,
                                                                                                       window)


def test_stale_counter_record_gives_no_traffic(tmp_path, monkeypatch):
    rec = {"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123456789}
    f = tmp_path / "rec.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.read_traffic() == 123456789
    rec["kernel_source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.read_traffic() is None
