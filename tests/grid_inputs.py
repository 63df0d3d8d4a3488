"""Grid-exact K/V inputs (test aid).

Every quantization group of these tensors holds values a + c*s with s a power
of two, c in 0..qmax, and both c = 0 and c = qmax present.  For such a group
the min/max quantizer recovers s, the codes c and the zero-point a exactly,
so dequantization reproduces the input bit for bit.  Attention over a cache
filled with them must therefore equal plain attention over the raw tensors.

Key groups run over G tokens of one channel, value groups over G channels of
one token (the axes of page "KIVI: Asymmetric 2-Bit KV Cache Quantization
Guide", "The Three Structural Innovations of KIVI").
"""
import numpy as np


def _groups(rng, n_groups, G, bits, extremes_in_first_half=False):
    qmax = (1 << bits) - 1
    codes = rng.integers(0, qmax + 1, size=(n_groups, G))
    span = G
    if extremes_in_first_half:
        # codes 0 and qmax only in the first G/2 slots; the second half draws
        # from 1..qmax-1 with both ends present, so a quantizer that grouped
        # G/2 elements would get a step of (qmax-2)/qmax of the true one there
        span = G // 2
        h = G // 2
        codes[:, h:] = rng.integers(1, qmax, size=(n_groups, G - h))
        codes[:, h] = 1
        codes[:, h + 1] = qmax - 1
    lo = rng.integers(0, span, size=n_groups)
    hi = (lo + 1 + rng.integers(0, span - 1, size=n_groups)) % span
    codes[np.arange(n_groups), lo] = 0
    codes[np.arange(n_groups), hi] = qmax
    step = np.exp2(rng.integers(-3, 1, size=(n_groups, 1))).astype(np.float64)
    base = rng.integers(-32, 32, size=(n_groups, 1)) / 8.0
    return base + codes * step


def grid_kv(B, H, T, D, G=32, k_bits=2, v_bits=2, seed=0, dtype=np.float16,
            extremes_in_first_half=False):
    """Returns K, V as float arrays [B][H][T][D] (values exact in fp16 and
    bf16) with T a multiple of G for the key grid; tokens past the last full
    block are still grid values, which is harmless.  With
    extremes_in_first_half the grid is exact only for groups of exactly G."""
    rng = np.random.default_rng(seed)
    Tb = (T + G - 1) // G
    # keys: group = (b, h, block, channel) over G tokens
    kg = _groups(rng, B * H * Tb * D, G, k_bits, extremes_in_first_half).reshape(B, H, Tb, D, G)
    K = kg.transpose(0, 1, 2, 4, 3).reshape(B, H, Tb * G, D)[:, :, :T]
    # values: group = (b, h, token, channel group) over G channels
    vg = _groups(rng, B * H * T * (D // G), G, v_bits, extremes_in_first_half).reshape(B, H, T, D)
    return K.astype(dtype), vg.astype(dtype)


def to_bits(a, dtype):
    """Raw 16-bit patterns of float values that are exact in `dtype`
    ("f16" or "bf16")."""
    a = np.asarray(a)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    f = a.astype(np.float32)
    assert np.all((f.view(np.uint32) & 0xFFFF) == 0), "value not exact in bf16"
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def from_bits(b, dtype):
    b = np.asarray(b, dtype=np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_fp64(q, K, V, scale, gq):
    """Textbook softmax(q K^T * scale) V in float64; q [B][Hq][D], K/V
    [B][H][T][D]; query head j uses kv head j // gq."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for j in range(Hq):
            h = j // gq
            s = (K[b, h] @ q[b, j]) * scale
            p = np.exp(s - s.max())
            out[b, j] = (p[:, None] * V[b, h]).sum(0) / p.sum()
    return out
