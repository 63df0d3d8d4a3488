"""Storage accounting of the oracle's packed format against the pages'
printed memory table (CPU only).  Fixture: tests/golden/llama3_8b_kv_cache_gb.txt
(page "KV-Cache Quantization: I Ran the Experiments", "Component 1" table and
"The memory math (verified)")."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "llama3_8b_kv_cache_gb.txt")
LAYERS, HEADS, D = 32, 8, 128


def _rows():
    rows, batch = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "batch":
            batch = tuple(float(x) for x in f[1:])
        else:
            rows.append(tuple(float(x) for x in f))
    return rows, batch


def _per_layer_bytes(oracle_mod, T, bits, R=128):
    c = oracle_mod.OracleCache(1, HEADS, D, T, bits, bits, 32, R)
    codes = (c.array("k_codes").size + c.array("v_codes").size) * 4
    meta = sum(c.array(n).size for n in ("k_scale", "k_zero", "v_scale", "v_zero")) * 2
    window_per_token = (c.array("k_resid").size + c.array("v_resid").size) * 2 / R
    return codes, meta, window_per_token


@pytest.mark.parametrize("row", range(4))
def test_code_bytes_match_printed_table(oracle_mod, row):
    rows, _ = _rows()
    T, fp16_gb, _, gb4, gb2 = rows[row]
    T = int(T)
    for bits, want in ((2, gb2), (4, gb4)):
        codes, meta, wpt = _per_layer_bytes(oracle_mod, T, bits)
        assert round(codes * LAYERS / 1e9, 2) == want
        # scale + zero-point: two fp16 values per group of 32 = 1 bit/element
        assert meta * 8 == 2 * HEADS * D * T
        # the full-precision window stores 16 bits per element
        assert round(wpt * T * LAYERS / 1e9, 2) == fp16_gb


def test_batch64_line(oracle_mod):
    _, (B, T, fp16_gb, gb4) = _rows()
    codes, _, wpt = _per_layer_bytes(oracle_mod, int(T), 4)
    assert abs(codes * LAYERS * B / 1e9 - gb4) < 1.0
    assert abs(wpt * T * LAYERS * B / 1e9 - fp16_gb) < 1.0
