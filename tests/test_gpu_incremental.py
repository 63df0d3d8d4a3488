"""Decode after every single-token append: every fill state (n_quant, n_resid)
from one token through several window flushes, against the oracle advanced
the same way.  Covers the window-only start, every window length, the flush
transitions and the split planner at each size."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import bits16, make_layer, small
from tests.gpu_helpers import assert_cache_equal, gpu_arrays, oracle_arrays

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3

#        name          B  H  Hq  T    kb vb dtype           R
CASES = [("mha_r32",   2, 2, 2, 200, 2, 2, torch.float16, 32),
         ("gq4_r32",   1, 2, 8, 200, 2, 2, torch.float16, 32),
         ("gq2_4b",    1, 1, 2, 150, 4, 4, torch.bfloat16, 32),
         ("gq4_r128",  1, 1, 4, 300, 2, 4, torch.float16, 128)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_after_every_append(case):
    name, B, H, Hq, T, kb, vb, dt, R = case
    w = small(name, B, H, Hq, T, kb, vb, dt, residual_length=R)
    x = make_layer(w, seed=11, n_new=0)
    cache = kivi.KiviCache(B, H, T, k_bits=kb, v_bits=vb, residual_length=R, dtype=dt, device=DEV)
    ref = oracle.OracleCache(B, H, w.head_dim, T, kb, vb, w.group_size, R,
                             oracle.BF16 if dt == torch.bfloat16 else oracle.F16)
    kd, vd = x.k.to(DEV), x.v.to(DEV)
    kb16, vb16 = bits16(x.k), bits16(x.v)
    q = x.q.contiguous().to(DEV)
    qb = bits16(x.q)
    scale = 1.0 / np.sqrt(w.head_dim)
    worst = 0.0
    for t in range(T):
        cache.append(kd[:, :, t:t + 1].contiguous(), vd[:, :, t:t + 1].contiguous())
        ref.append(kb16[:, :, t:t + 1], vb16[:, :, t:t + 1])
        out = cache.decode_attn(q, scale).cpu().numpy().astype(np.float64)
        o_ref = ref.decode_attn(qb, scale)
        err = float(np.abs(out - o_ref).max())
        worst = max(worst, err)
        assert err <= TOL, f"{name}: token {t + 1} (n_quant {ref.n_quant}, n_resid {ref.n_resid}): {err:.3e}"
    torch.cuda.synchronize()
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
    assert_cache_equal(gpu_arrays(cache), oracle_arrays(ref), ref.n_quant, ref.n_resid,
                       ref.capacity, ref.num_blocks)
    print(f"{name}: worst attention error over {T} states {worst:.2e}", flush=True)
