"""Attention over the whole input domain: keys with outlier channels near
2e4 in magnitude, queries up to |q| = 8 and value groups spanning +-30000
(fp16 and bf16 inputs; the stored scale and zero-point are fp16, so inputs
stay within +-65504).  The matrix-core decode scales its fp16 operands q*S and
p*S by powers of two chosen from the records' scale maxima; these cases need
that scaling (|q| * S far above 8188, value scales far above 1023).  Codes,
scales, zero-points, the per-record scale maxima and the window are compared
bit for bit; attention within 2e-3 of the binary64 oracle plus the binary32
rounding allowance of these inputs (printed with each case)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import bits16
from tests.attn_reference import attention, fp32_allowance
from tests.gpu_helpers import assert_cache_equal, assert_scale_max, gpu_arrays, oracle_arrays

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3


def _extreme_layer(B, H, Hq, T, seed):
    """K: N(0,1) plus per-channel offsets N(0,2), and 2..6 outlier channels
    per kv head at +-(2e4 + 4e3 z); V: N(0,1), with 1% of (token, channel
    group of 32) spanning +-30000 uniformly; q uniform in [-8, 8]."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, T, 128)) + rng.standard_normal((1, H, 1, 128)) * np.sqrt(2.0)
    for h in range(H):
        ch = rng.choice(128, size=int(rng.integers(2, 7)), replace=False)
        sign = rng.choice([-1.0, 1.0], size=ch.size)
        K[:, h, :, ch] = (sign[:, None, None] * (2e4 + 4e3 * rng.standard_normal((ch.size, B, T))))
    V = rng.standard_normal((B, H, T, 128))
    hit = rng.random((B, H, T, 4)) < 0.01
    for b, h, t, m in zip(*np.nonzero(hit)):
        V[b, h, t, 32 * m:32 * m + 32] = rng.uniform(-3e4, 3e4, 32)
    q = rng.uniform(-8.0, 8.0, (B, Hq, 128))
    clip = lambda a: np.clip(a, -65504.0, 65504.0).astype(np.float32)
    return clip(K), clip(V), clip(q)


CASES = [  # G, k_bits, v_bits, dtype, query heads per kv head
    (32, 2, 2, torch.float16, 4), (32, 2, 2, torch.float16, 1), (32, 2, 2, torch.bfloat16, 2),
    (32, 4, 4, torch.float16, 4), (32, 2, 4, torch.bfloat16, 4), (32, 4, 2, torch.float16, 8),
    (64, 2, 2, torch.float16, 4), (64, 4, 2, torch.bfloat16, 1), (64, 2, 4, torch.float16, 2),
    (64, 4, 4, torch.bfloat16, 8), (32, 2, 2, torch.float16, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"G{c[0]}_k{c[1]}v{c[2]}_{str(c[3])[6:]}_gq{c[4]}"
                                              for c in CASES])
def test_extreme_range_attention(case):
    G, kb, vb, dt, gq = case
    B, H, T = 2, 2, 700
    print(f"extreme range: G={G} k{kb}v{vb} {dt} gq={gq} B={B} H={H} T={T}+1", flush=True)
    K, V, q = _extreme_layer(B, H, H * gq, T + 1, seed=G + 10 * kb + vb + gq)
    k, v, qt = (torch.from_numpy(a).to(dt) for a in (K, V, q))
    cache = kivi.KiviCache(B, H, T + 1, k_bits=kb, v_bits=vb, group_size=G, residual_length=128,
                           dtype=dt, device=DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    cache.append(kd[:, :, :T].contiguous(), vd[:, :, :T].contiguous())
    ref = oracle.OracleCache(B, H, 128, T + 1, kb, vb, G, 128,
                             oracle.BF16 if dt == torch.bfloat16 else oracle.F16)
    ref.append(bits16(k), bits16(v))
    scale = 1.0 / np.sqrt(128)
    # the decode token flushes the full window inside the fused step
    out = cache.append_decode_attn(kd[:, :, T:].contiguous(), vd[:, :, T:].contiguous(), qt.to(DEV), scale)
    torch.cuda.synchronize()
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
    assert_cache_equal(gpu_arrays(cache), oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                       ref.num_blocks, G=G)
    assert_scale_max(cache, ref)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), "non-finite attention output"
    o_ref = ref.decode_attn(bits16(qt), scale)
    o64, lmax, spread, vsum = attention(ref, bits16(qt), scale, bf16=dt == torch.bfloat16)
    assert np.abs(o64 - o_ref).max() <= 1e-9 * np.abs(o_ref).max()
    allow = fp32_allowance(lmax, spread, vsum)
    err = np.abs(got - o_ref)
    i = np.unravel_index(np.argmax(err - allow), err.shape)
    print(f"  max |out| {np.abs(o_ref).max():.1f}, logit sums up to {lmax.max():.3e}: attention error "
          f"{err.max():.3e}; worst against its bound {err[i]:.3e} <= 2e-3 + {allow[i]:.3e}", flush=True)
    assert np.all(err <= TOL + allow), f"attention error {err[i]:.3e} at {i}"
