"""The benchmark's contract on the CPU: it refuses more than one GPU with a
message, its algorithmic byte counts are the ones the roofline figures use,
and a stored HBM-counter record applies only to the step-kernel sources it
was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_heavy_load_step_bytes():
    # 512 cached slots, G = 8, bf16: K and V 262,144 + the new token 1,024 +
    # q and the fp32 output 6,144 + scores read and written 4,104 + positions
    # 2,048 + the new position 4
    assert bench.per_unit_bytes(512, 8, 128, 2, "h2o") == 275_468
    assert bench.per_unit_bytes(512, 8, 128, 2, "h2o") * 4096 == 1_128_316_928
    # StreamingLLM keeps no scores
    assert bench.per_unit_bytes(512, 8, 128, 2, "streaming") == 275_468 - 4_104
    # E5M2 cache: one byte per cached element, bf16 activations
    assert bench.per_unit_bytes(512, 8, 128, 1, "h2o", act_b=2) == 275_468 - 131_072 - 256


@pytest.mark.parametrize("G", [1, 4, 8])
def test_kivi_bytes_per_token(G):
    # 192 bytes per quantized token (64 + 64 code bytes, a 32-token group's
    # two per-channel K grids spread over its tokens, four V grids per token),
    # 512 per residual token (bf16 K and V rows)
    base = bench.kivi_unit_bytes(1920, 100, G)
    assert bench.kivi_unit_bytes(1920 + 32, 100, G) - base == 32 * 192
    assert bench.kivi_unit_bytes(1920, 101, G) - base == 512


def test_traffic_record_applies_to_its_sources_only(monkeypatch):
    rec = bench.PROFILED_TRAFFIC[0]
    monkeypatch.setattr(bench, "sources_digest", lambda: rec["sources_digest"])
    got, src = bench.profiled_traffic(rec["workload"], rec["policy"], rec["kv_dtype"])
    want = (rec["fetch_kib"] * bench.FETCH_SCALE + rec["write_kib"] * bench.WRITE_SCALE) * 1024.0
    assert got == pytest.approx(want) and "stored record" in src
    monkeypatch.setattr(bench, "sources_digest", lambda: "0" * 16)
    got, src = bench.profiled_traffic(rec["workload"], rec["policy"], rec["kv_dtype"])
    assert got is None and "none" in src
