"""Host-side logic of bench.py, checked on the CPU: the algorithmic FLOP and byte counts
behind `value` and `roofline.achieved` (recounted here by brute force over the (query,
key) pairs and the rows a call moves), the rule that a counter-measured traffic figure is
reported only for the kernel source it was measured on, and the one-GPU guard.
"""
import hashlib
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("t,hq,d,hist", [(3, 2, 128, [5]), (7, 12, 128, [0, 4, 100]), (1, 1, 64, [0])])
def test_prefill_flops_counts_unmasked_pairs(t, hq, d, hist):
    pairs = 0
    for h0 in hist:
        for i in range(t):           # new token i sees keys 0 .. h0 + i
            for j in range(h0 + t):
                pairs += j <= h0 + i
    # QK^T and PV: 2 FLOPs per multiply-add, d multiply-adds each
    assert bench.prefill_flops(len(hist), t, hq, d, hist) == 2 * 2 * d * hq * pairs


def test_decode_bytes_counts_rows_moved():
    lens, hq, hkv, d = [3, 0, 17], 6, 2, 128
    row = d * 2  # one f16 row of a head
    want = 0
    for L in lens:
        want += L * hkv * 2 * row   # K and V cache rows read
        want += hkv * 2 * row       # the new k and v read
        want += hkv * 2 * row       # the appended K and V rows written
        want += hq * row * 2        # q read, out written
    assert bench.decode_bytes(lens, hq, hkv, d) == want


def test_traffic_only_for_the_measured_source(monkeypatch):
    csrc = os.path.join(ROOT, "kv_cache_causal_rope_amd", "csrc")
    src = tuple(hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()
                for f in ("prefill.hip", "device_common.h", "rope_device.h"))
    monkeypatch.setattr(bench, "TRAFFIC", {"prefill_attn:w": {"bytes": 123.0, "src": src}})
    assert bench.traffic("prefill_attn", "w") == 123.0
    assert bench.traffic("prefill_attn", "other") is None
    stale = (src[0][::-1],) + src[1:]
    monkeypatch.setattr(bench, "TRAFFIC", {"prefill_attn:w": {"bytes": 123.0, "src": stale}})
    assert bench.traffic("prefill_attn", "w") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
