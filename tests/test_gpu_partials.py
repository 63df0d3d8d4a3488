"""Where the attention error of the matrix-core decode comes from: with one
split over the packed tokens, the split's partial softmax state (m, l, o)
is compared with the same sums in binary64 over the oracle's dequantized
cache, and the window's partial likewise.  The scores enter the partial only
through m and the weights 2^(s_t - m), so the error of l (relative) and of
o / l separate the key side (logits) from the value side (weighted sums).
Printed per case; asserted against loose bounds."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import bits16, make_layer, small
from tests.attn_reference import dequantized

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

#        G   R   B  H  gq kb vb  dtype           T
CASES = [(64, 64, 1, 1, 4, 4, 2, torch.float16, 525),   # the shape of random configuration 104
         (64, 256, 1, 1, 2, 4, 2, torch.float16, 600),  # and of 45
         (32, 128, 2, 2, 4, 2, 2, torch.float16, 1000),
         (32, 128, 2, 2, 1, 2, 2, torch.bfloat16, 1000),
         (64, 128, 1, 2, 4, 4, 4, torch.float16, 800),
         (32, 128, 1, 2, 8, 2, 2, torch.float16, 900)]


@pytest.mark.parametrize("case", CASES, ids=[f"G{c[0]}_R{c[1]}_gq{c[4]}_k{c[5]}v{c[6]}" for c in CASES])
def test_split_partials(case):
    G, R, B, H, gq, kb, vb, dt, T = case
    w = dataclasses.replace(small("partials", B, H, H * gq, T, kb, vb, dt, residual_length=R), group_size=G)
    bf = dt == torch.bfloat16
    worst = {"l": 0.0, "o/l": 0.0, "win o/l": 0.0}
    for seed in range(6):
        x = make_layer(w, seed=100 + seed, n_new=0)
        cache = kivi.KiviCache(B, H, T, k_bits=kb, v_bits=vb, group_size=G, residual_length=R,
                               dtype=dt, device=DEV)
        cache.append(x.k.contiguous().to(DEV), x.v.contiguous().to(DEV))
        cache.set_splits(1)
        q = x.q
        scale = 1.0 / np.sqrt(128)
        cache.decode_attn(q.contiguous().to(DEV), scale)
        torch.cuda.synchronize()
        nq, nr = cache.n_quant, cache.n_resid
        Hq = H * gq
        n_split = (1 if nq > 0 else 0) + (1 if nr > 0 else 0)
        ws = cache.workspace(Hq)
        part = ws[:B * Hq * n_split * 130 * 4].view(torch.float32).view(B, Hq, n_split, 130).cpu().numpy()
        ref = oracle.OracleCache(B, H, 128, T, kb, vb, G, R, oracle.BF16 if bf else oracle.F16)
        ref.append(bits16(x.k), bits16(x.v))
        K, V = dequantized(ref, bf)
        qf = q.float().numpy().astype(np.float64)
        lam = scale / np.log(2.0)
        for b in range(B):
            for j in range(Hq):
                u = b * H + j // gq
                s = lam * (K[u] @ qf[b, j])
                for sp, (lo, hi) in enumerate([(0, nq), (nq, nq + nr)][:n_split] if nq > 0 else [(nq, nq + nr)]):
                    m_ref = s[lo:hi].max()
                    wt = np.exp2(s[lo:hi] - m_ref)
                    l_ref = wt.sum()
                    o_ref = wt @ V[u, lo:hi]
                    m, l, o = part[b, j, sp, 0], part[b, j, sp, 1], part[b, j, sp, 2:]
                    f = np.exp2(float(m) - m_ref)  # the partial's weights relative to binary64's
                    el = abs(l * f / l_ref - 1.0)
                    eo = np.abs(o / l - o_ref / l_ref).max()
                    key = "win o/l" if lo == nq else "o/l"
                    worst[key] = max(worst[key], eo)
                    if lo < nq:
                        worst["l"] = max(worst["l"], el)
    print(f"G={G} R={R} gq={gq} k{kb}v{vb} {dt}: packed split: relative error of l "
          f"{worst['l']:.2e}, of o/l {worst['o/l']:.2e}; window split o/l {worst['win o/l']:.2e}",
          flush=True)
    assert worst["l"] < 1e-3 and worst["o/l"] < 2e-3 and worst["win o/l"] < 1e-4
