"""Pins of the oracle's group quantizer and float conversions (CPU only).

Quantizer definition: page "KIVI: Asymmetric 2-Bit KV Cache Quantization
Guide", "Step 1" / "Step 2" (min/max scale, half-to-even rounding, clamp to
[0, qmax]), with the zero-point kept as the group minimum in floating point.
None of the pages prints a worked example, so the examples below are derived
by hand from that definition; each derivation is written next to it.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.exact_ref import quantize_group_exact, rn32

pytestmark = pytest.mark.filterwarnings("ignore")


def f16(vals):
    return np.asarray(vals, dtype=np.float16).astype(np.float32)


# ------------------------------------------------------------ conversions

def test_f16_to_f32_all_patterns(oracle_mod):
    # Every binary16 pattern: numpy's conversion is an independent library
    # routine; NaNs only need to stay NaN.
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle_mod.f16_to_f32(b) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_patterns(oracle_mod):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, 4000).astype(np.uint16)
    for b in bits:
        ref = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
        got = np.float32(oracle_mod.bf16_to_f32(b))
        if np.isnan(ref):
            assert np.isnan(got)
        else:
            assert got.view(np.uint32) == ref.view(np.uint32)


def test_f32_to_f16_rne_against_numpy(oracle_mod):
    rng = np.random.default_rng(2)
    # random magnitudes over the whole binary16 range, both signs, plus exact
    # midpoints between neighbouring binary16 values (the tie cases)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-26, 17, 20000))).astype(np.float32)
    grid = np.arange(0, 0x7bff, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0, 0x7bff, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = ((grid + nxt) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([65504, 65519.99, 65520, 1e-8, 6e-8, 0.0, -0.0])])
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle_mod.f32_to_f16(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------- hand-worked groups

def test_example_pattern_mod4(oracle_mod):
    # x_j = j mod 4: min 0, max 3, s = 3/3 = 1 exactly, so code_j = x_j,
    # S = fp16(1) = 0x3C00, Z = fp16(0) = 0x0000.
    x = f16(np.arange(32) % 4)
    codes, S, Z = oracle_mod.quantize_group(x, 2)
    assert codes.tolist() == (np.arange(32) % 4).tolist()
    assert (S, Z) == (0x3C00, 0x0000)


def test_example_ties_round_half_even(oracle_mod):
    # [0, 0.5, 1.5, 2.5, 3 x 28]: s = 1; quotients 0.5, 1.5, 2.5 are exact
    # ties and round to the even neighbours 0, 2, 2.  The dequantization error
    # at those three is exactly s/2.
    x = f16([0, 0.5, 1.5, 2.5] + [3] * 28)
    codes, S, Z = oracle_mod.quantize_group(x, 2)
    assert codes.tolist() == [0, 0, 2, 2] + [3] * 28
    err = [abs(float(x[j]) - oracle_mod.dequant(codes[j], S, Z)) for j in range(4)]
    assert err == [0.0, 0.5, 0.5, 0.5]


def test_example_constant_group_is_exact(oracle_mod):
    # Constant group: max - min = 0, so s = 0, every code is 0, S = +0 and
    # Z = the value (1.25 = 0x3D00); dequantization gives the value back.
    x = f16([1.25] * 32)
    codes, S, Z = oracle_mod.quantize_group(x, 2)
    assert codes.tolist() == [0] * 32
    assert (S, Z) == (0x0000, 0x3D00)
    assert oracle_mod.dequant(0, S, Z) == 1.25


def test_example_negative_range(oracle_mod):
    # [-1.5, -0.5, 0.5, 1.5] repeated: min -1.5, s = 3/3 = 1, codes j mod 4,
    # Z = fp16(-1.5) = 0xBE00.
    x = f16(np.array([-1.5, -0.5, 0.5, 1.5])[np.arange(32) % 4])
    codes, S, Z = oracle_mod.quantize_group(x, 2)
    assert codes.tolist() == (np.arange(32) % 4).tolist()
    assert (S, Z) == (0x3C00, 0xBE00)


def test_example_4bit_pattern(oracle_mod):
    # 4-bit: x_j = j mod 16, min 0, max 15, s = 15/15 = 1, codes = x_j.
    x = f16(np.arange(32) % 16)
    codes, S, Z = oracle_mod.quantize_group(x, 4)
    assert codes.tolist() == (np.arange(32) % 16).tolist()
    assert (S, Z) == (0x3C00, 0x0000)


def test_example_inexact_scale(oracle_mod):
    # [0, 1, 0 x 30], 2-bit: s = RN32(1/3) = 0x3EAAAAAB = 0.3333333432...;
    # the quotient 1/s = 2.99999991 rounds to 3.0 in binary32, code 3.
    # S = fp16(s) = 0x3555 = 0.333251953125, and 3*S = 0.999755859375, so the
    # error 2.44e-4 stays within s/2 + 3|s - S|.
    x = f16([0, 1] + [0] * 30)
    codes, S, Z = oracle_mod.quantize_group(x, 2)
    assert codes.tolist() == [0, 3] + [0] * 30
    assert (S, Z) == (0x3555, 0x0000)
    assert oracle_mod.dequant(3, S, Z) == 0.999755859375
    s = np.float32(1) / np.float32(3)
    assert s.view(np.uint32) == 0x3EAAAAAB


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("bits", [2, 4])
def test_min_max_codes_and_zero_point(oracle_mod, bits):
    # For s > 0: the minimum maps to code 0 and the maximum to qmax (the
    # quotient (max-min)/s is qmax up to one rounding), and Z is the fp16
    # value of the minimum; for fp16 inputs that is the minimum itself.
    rng = np.random.default_rng(3 + bits)
    qmax = (1 << bits) - 1
    for _ in range(500):
        x = f16(rng.standard_normal(32) * rng.uniform(0.01, 30))
        codes, S, Z = oracle_mod.quantize_group(x, bits)
        if x.max() == x.min():
            continue
        assert codes[np.argmin(x)] == 0
        assert codes[np.argmax(x)] == qmax
        assert oracle_mod.f16_to_f32(Z) == x.min() or (x.min() == 0 and Z == 0)
        assert codes.max() <= qmax


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_error_bound(oracle_mod, bits, dtype):
    # |x - (c*S + Z)| <= s/2 + qmax*|s - S| + |min - Z| (binary64, tiny slack
    # for the binary32 rounding of the quotient).  Ties reach s/2.
    rng = np.random.default_rng(11 + bits)
    qmax = (1 << bits) - 1
    for i in range(800):
        v = rng.standard_normal(32) * rng.uniform(1e-3, 40) + rng.uniform(-50, 50)
        if i % 7 == 0:
            v[rng.integers(0, 32)] *= 15  # outlier
        v = np.clip(v, -60000, 60000).astype(np.float32)
        if dtype == "f16":
            x = v.astype(np.float16).astype(np.float32)
        else:
            x = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)  # exact bf16 values
        codes, S, Z = oracle_mod.quantize_group(x, bits)
        mn, mx = float(x.min()), float(x.max())
        s = float(np.float32(np.float32(mx - mn) / np.float32(qmax)))
        Sv, Zv = oracle_mod.f16_to_f32(S), oracle_mod.f16_to_f32(Z)
        bound = s / 2 + qmax * abs(s - Sv) + abs(mn - Zv) + s * 2.0 ** -20
        for j in range(32):
            err = abs(float(x[j]) - oracle_mod.dequant(codes[j], S, Z))
            assert err <= bound, (i, j, err, bound)


# ------------------------------------------------ exact-rational reference

def _fr(v):
    return Fraction(float(v))


@pytest.mark.parametrize("bits", [2, 4])
def test_fp16_sweep_against_exact_rational(oracle_mod, bits):
    # For several (min, max) pairs, every binary16 value x in [min, max] (a
    # stride on the widest pairs) is quantized inside a group that also holds
    # min and max; codes must equal the exact-rational model.
    pairs = [(-1.0, 1.0), (0.1, 0.35), (-7.3, 2.9), (100.0, 113.5),
             (-0.001, 0.002), (-60.0, 40.0), (0.0, 1.0), (-3.0, -2.0)]
    allh = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    allh = np.unique(allh[np.isfinite(allh)])
    checked = 0
    for lo, hi in pairs:
        lo32, hi32 = f16([lo])[0], f16([hi])[0]
        xs = allh[(allh >= lo32) & (allh <= hi32)]
        if xs.size > 6000:
            xs = xs[:: xs.size // 6000 + 1]
        exact_mn, exact_mx = _fr(lo32), _fr(hi32)
        for start in range(0, xs.size, 30):
            chunk = xs[start:start + 30]
            group = np.concatenate([[lo32, hi32], chunk]).astype(np.float32)
            codes, _, _ = oracle_mod.quantize_group(group, bits)
            ref, _ = quantize_group_exact([exact_mn, exact_mx] + [_fr(v) for v in chunk], bits)
            assert codes.tolist() == ref, (lo, hi, start)
            checked += chunk.size
    assert checked > 20000


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_random_groups_against_exact_rational(oracle_mod, bits, dtype):
    rng = np.random.default_rng(100 + bits)
    for i in range(400):
        v = (rng.standard_normal(32) * rng.uniform(0.01, 20) + rng.uniform(-5, 5)).astype(np.float32)
        if dtype == "f16":
            x = v.astype(np.float16).astype(np.float32)
        else:
            x = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)
        codes, S, Z = oracle_mod.quantize_group(x, bits)
        ref, s = quantize_group_exact([_fr(t) for t in x], bits)
        assert codes.tolist() == ref, i
        # S is the binary16 rounding of the binary32 scale
        assert S == np.float32(float(s)).astype(np.float16).view(np.uint16)


def test_exact_model_matches_hardware_rounding_spotcheck():
    # Sanity of the test aid itself: rn32 agrees with numpy float32 rounding of
    # exactly representable binary64 quotients.
    rng = np.random.default_rng(7)
    for _ in range(2000):
        a, b = rng.standard_normal(2) * 10
        a32, b32 = np.float32(a), np.float32(b)
        assert rn32(_fr(a32) / _fr(b32)) == _fr(a32 / b32)
        assert rn32(_fr(a32) - _fr(b32)) == _fr(a32 - b32)


@pytest.mark.parametrize("bits", [2, 4])
def test_division_not_reciprocal_on_hard_cases(oracle_mod, bits):
    # The quantizer divides by s.  Multiplying by a rounded reciprocal instead
    # changes a code only when the quotient sits next to a half-integer, which
    # a sweep rarely hits, so the hard cases are searched for first (seeded
    # numpy search over fp16 triples) and then checked against the exact
    # model.  Each kept case is one where the reciprocal form gives another
    # code, so an oracle that used it would fail here.
    rng = np.random.default_rng(5 + bits)
    qmax = np.float32((1 << bits) - 1)
    n = 4_000_000
    a = (rng.standard_normal(n) * rng.uniform(0.1, 30, n)).astype(np.float16).astype(np.float32)
    b = (rng.standard_normal(n) * rng.uniform(0.1, 30, n)).astype(np.float16).astype(np.float32)
    mn, mx = np.minimum(a, b), np.maximum(a, b)
    u = rng.uniform(0, 1, n).astype(np.float32)
    x = np.clip((mn + (mx - mn) * u).astype(np.float16).astype(np.float32), mn, mx)
    with np.errstate(all="ignore"):
        s = ((mx - mn) / qmax).astype(np.float32)
        d = (x - mn).astype(np.float32)
        recip = np.rint((d * (np.float32(1) / s).astype(np.float32)).astype(np.float32))
        div = np.rint((d / s).astype(np.float32))
    idx = np.nonzero((s > 0) & (recip != div))[0][:60]
    assert idx.size >= 30
    for i in idx:
        group = np.array([mn[i], mx[i], x[i]], dtype=np.float32)
        codes, _, _ = oracle_mod.quantize_group(group, bits)
        ref, _ = quantize_group_exact([_fr(v) for v in group], bits)
        assert codes.tolist() == ref
        assert ref[2] != int(np.clip(recip[i], 0, qmax))
