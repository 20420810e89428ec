"""Pins the benchmark's pricing of decode as weight bytes streamed per token
against the one worked example the pages print (tests/golden/decode_traffic.txt:
Core AI card, decode table and the paragraph under it)."""
import os

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_traffic.txt")


def _golden():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 1
    return tuple(float(v) for v in rows[0])


def test_traffic_from_rate_and_bytes():
    tok, gb, traffic = _golden()
    ms = 1e3 / tok                             # ms per token at the printed rate
    assert round(bench.weight_gbs(gb * 1e9, ms)) == traffic


def test_rate_from_traffic_and_bytes():
    tok, gb, traffic = _golden()
    ms = gb * 1e9 / (traffic * 1e9) * 1e3      # one token streams gb at the printed traffic
    assert round(bench.tok_s(ms), 1) == tok


def test_batch_scales_tokens_not_bytes():
    assert bench.tok_s(2.0, 8) == 8 * bench.tok_s(2.0)
    assert bench.weight_gbs(18_029_690_880, 2.817) > 0.8 * bench.HBM_PEAK_GBS - 1   # 80% of 8 TB/s at 2.817 ms


def test_multi_gpu_refused():
    import subprocess, sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
