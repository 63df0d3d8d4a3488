"""Host logic of bench.py (no GPU): the algorithmic byte accounting against
closed forms written out field by field, the ragged length draw, the counter
lookup and the refusal of more than one GPU."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kv_cache_bit_kivi_amd.inputs import WORKLOADS  # noqa: E402


def unit_bytes_by_field(T, D=128, G=32, R=128, kb=2, vb=2, e=2, gq=1):
    """Per (batch, kv head) unit, the bytes each phase moves, listed field by
    field: prefix pack of T tokens (the window keeps the last
    ((T - 1) mod R) + 1), flush of a full window, then the decode kernel and
    the merge on the state after the token's append."""
    r = (T - 1) % R + 1
    nq = T - r
    pack = {
        "read K and V": 2 * T * D * e,
        "key codes": nq * D * kb // 8,
        "value codes": nq * D * vb // 8,
        "key scale + zero (per block and channel)": (nq // G) * D * 2 * 2,
        "value scale + zero (per token and channel group)": nq * (D // G) * 2 * 2,
        "window written": 2 * r * D * e,
    }
    flush = {}
    if r == R:
        flush = {
            "window read": 2 * R * D * e,
            "key codes": R * D * kb // 8,
            "value codes": R * D * vb // 8,
            "key scale + zero": (R // G) * D * 4,
            "value scale + zero": R * (D // G) * 4,
        }
        nq, r = nq + R, 1
    else:
        r += 1
    decode = {
        "token read and written into the window": 2 * 2 * D * e,
        "key codes": nq * D * kb // 8,
        "value codes": nq * D * vb // 8,
        "key scale + zero": (nq // G) * D * 4,
        "value scale + zero": nq * (D // G) * 4,
        "window": 2 * r * D * e,
        "q": gq * D * e,
    }
    merge = {"out (fp32)": gq * D * 4}
    return sum(pack.values()), sum(flush.values()), sum(decode.values()), sum(merge.values())


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_algorithmic_bytes_closed_form(name):
    w = WORKLOADS[name]
    p, f, d, m = unit_bytes_by_field(w.tokens, w.head_dim, w.group_size, w.residual_length,
                                     w.k_bits, w.v_bits, 2, w.gq)
    U = w.batch * w.kv_heads
    assert bench.algorithmic_bytes(w) == {"pack": U * p, "flush": U * f, "decode": U * d, "merge": U * m}


def test_algorithmic_bytes_known_totals():
    # c1: 256 units; prefix 4096 tokens (3968 packed + 128 in the window)
    ab = bench.algorithmic_bytes(WORKLOADS["c1"])
    assert ab["pack"] == 256 * (2 * 4096 * 256 + 3968 * 64 + 124 * 512 + 3968 * 16 + 2 * 128 * 256)
    assert ab["pack"] == 651_165_696
    # the decode kernel after the flush reads 4096 packed tokens (96 B each at
    # 2/2 bits with G = 32) and one window token
    assert ab["decode"] + ab["merge"] == 256 * (1024 + 4096 * 96 + 512 + 256 + 512) == 101_253_120
    # c2, the default: 256 units at gq 4, 32768 packed tokens after the flush
    ab = bench.algorithmic_bytes(WORKLOADS["c2"])
    assert ab["decode"] == 256 * (1024 + 32768 * 96 + 512 + 4 * 256) == 805_961_728
    assert ab["flush"] == 256 * (128 * 512 + 128 * 96) == 19_922_944
    assert bench.step_bytes(ab) == ab["flush"] + ab["decode"] + 256 * 4 * 512


def test_ragged_bytes_are_per_sequence_sums():
    w = WORKLOADS["c1"]
    lens = bench.ragged_lengths(w)
    assert len(lens) == w.batch and all(w.tokens // 2 <= t <= w.tokens for t in lens)
    assert lens == bench.ragged_lengths(w)  # seeded
    tot = {"pack": 0, "flush": 0, "decode": 0, "merge": 0}
    for t in lens:
        p, f, d, m = unit_bytes_by_field(t)
        tot["pack"] += p
        tot["flush"] += f
        tot["decode"] += d
        tot["merge"] += m
    assert bench.algorithmic_bytes(w, lens) == {k: w.kv_heads * v for k, v in tot.items()}


def test_stats_of_durations():
    s = bench.stats([1e-6 * x for x in range(1, 101)])
    assert s["samples"] == 100 and s["us_mean"] == pytest.approx(50.5)
    assert s["us_median"] == pytest.approx(50.5) and s["us_p10"] == pytest.approx(10.9)


def test_traffic_lookup_checks_the_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    (tmp_path / "profiles").mkdir()
    good = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profiles" / "k_c1_counters.txt"
    prof.write_text(f"# counters\nhbm_bytes_per_launch: 12345\nkernel_source_sha256: {good}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("k", "c1", str(src)) == 12345.0
    src.write_text("kernel source, changed\n")
    assert bench.traffic_from_profile("k", "c1", str(src)) is None
    assert bench.traffic_from_profile("other", "c1", str(src)) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
