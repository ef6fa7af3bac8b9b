"""CPU checks of the benchmark's contract: the one-GPU refusal, the algorithmic
byte model its roofline divides by, and when the recorded HBM-counter traffic
applies."""

import hashlib
import importlib.util
import os
import subprocess
import sys

from weight_streaming_expert_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_algorithmic_bytes_of_the_decode_step():
    """The byte model written out from the shapes: MXFP4 rows of K elements
    take K/2 code bytes and K/32 scale bytes, the router is bf16, the head is
    one byte per weight plus an fp32 scale per row, and the logits are fp32."""
    H, I, E, V, L, k = 2560, 768, 512, 157184, 32, 8
    gate_up = 2 * I * (H // 2 + H // 32)
    down = H * (I // 2 + I // 32)
    expert = gate_up + down
    assert (gate_up, down, expert) == (2_088_960, 1_044_480, 3_133_440)
    layer = E * H * 2 + (k + 1) * expert
    assert layer == 30_822_400
    head = V * H + V * 4 + V * 4
    m = configs.DECODE_STEP.moe
    assert configs.moe_layer_bytes(m, k) == layer
    assert configs.head_bytes(V, H, 1, True) == head
    assert L * layer + head == 1_389_965_312
    # the verify pass reads the head once for its four rows
    assert configs.head_bytes(V, H, 4, True) - configs.head_bytes(V, H, 1, True) == 3 * V * 4


def test_traffic_record_applies_only_to_the_recorded_sources(tmp_path, monkeypatch):
    bench = _bench_module()
    digest = bench.step_source_digest()
    h = hashlib.sha256()
    for f in bench.STEP_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    assert digest == h.hexdigest()

    rec = tmp_path / "counters.md"
    rec.write_text(f"- `traffic_bytes_per_launch`: `123456789`\n- `sources_sha256`: `{digest}`\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.step_traffic_bytes() == 123456789

    rec.write_text("- `traffic_bytes_per_launch`: `123456789`\n- `sources_sha256`: `" + "0" * 64 + "`\n")
    assert bench.step_traffic_bytes() is None

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.step_traffic_bytes() is None
