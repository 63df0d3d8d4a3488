"""Group size G = 64 (the pages' group-size knob, page "KV-Cache Quantization:
I Ran the Experiments So You Don't Have To" and the config knobs of page
"KIVI: Asymmetric 2-Bit KV Cache Quantization Guide"): bulk and single-token
appends bit-exact against the oracle at G = 64, decode attention within
2e-3, and the same through sequences of different lengths, paged records and
the fused decode step, for 1, 2, 4 and 8 query heads per kv head.  A ratio
that is not built (16) must be rejected before anything is enqueued."""
import dataclasses

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
G = 64

#        name           B  H  Hq  T     kb vb dtype           R
CASES = [("mha",         2, 2, 2,  300,  2, 2, torch.float16,  128),
         ("gq4_4b_bf16", 1, 2, 8,  520,  4, 4, torch.bfloat16, 128),
         ("gq2_k2v4",    2, 1, 2,  1000, 2, 4, torch.float16,  64),
         ("gq4_k4v2",    1, 2, 8,  129,  4, 2, torch.float16,  64),
         ("T64",         1, 1, 4,  64,   2, 2, torch.float16,  64),
         ("T1",          1, 1, 1,  1,    2, 2, torch.float16,  64),
         ("r1024_flush", 1, 1, 4,  2048, 2, 2, torch.float16,  1024),
         ("r256_gq4",    2, 1, 4,  900,  2, 2, torch.bfloat16, 256),
         # 8 and 16 query heads per kv head: head groups reading 64-token
         # records as two 32-token streams
         ("gq8",         1, 2, 16, 700,  2, 2, torch.float16,  128),
         ("gq8_4b_bf16", 2, 1, 8,  300,  4, 4, torch.bfloat16, 64),
         ("gq8_k2v4",    1, 1, 8,  200,  2, 4, torch.float16,  64),
         ("gq16",        1, 1, 16, 333,  2, 2, torch.float16,  64)]


def _setup(case, extra=1):
    name, B, H, Hq, T, kb, vb, dt, R = case
    w = dataclasses.replace(small(name, B, H, Hq, T, kb, vb, dt, residual_length=R), group_size=G)
    x = make_layer(w, seed=8, n_new=extra)
    return w, x


def _caches(w, max_tokens):
    dtc = oracle.BF16 if w.dtype == torch.bfloat16 else oracle.F16
    gpu = kivi.KiviCache(w.batch, w.kv_heads, max_tokens, k_bits=w.k_bits, v_bits=w.v_bits,
                         group_size=G, residual_length=w.residual_length, dtype=w.dtype, device=DEV)
    ref = oracle.OracleCache(w.batch, w.kv_heads, w.head_dim, max_tokens, w.k_bits, w.v_bits, G,
                             w.residual_length, dtc)
    return gpu, ref


def _compare(gpu, ref):
    torch.cuda.synchronize()
    v = gpu.view()
    assert (v.n_quant, v.n_resid) == (ref.n_quant, ref.n_resid)
    assert_cache_equal(gpu_arrays(gpu), oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                       ref.num_blocks, G=G)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_group64_pack_decode(case):
    name, B, H, Hq, T, kb, vb, dt, R = case
    print(f"G=64 {name}: B={B} H={H} Hq={Hq} T={T} bits={kb}/{vb} R={R}", flush=True)
    w, x = _setup(case, extra=2 * R + 3)
    gpu, ref = _caches(w, T + 2 * R + 3)
    kb16, vb16 = bits16(x.k), bits16(x.v)
    gpu.append(x.k[:, :, :T].contiguous().to(DEV), x.v[:, :, :T].contiguous().to(DEV))
    ref.append(kb16[:, :, :T], vb16[:, :, :T])
    _compare(gpu, ref)
    scale = 1.0 / np.sqrt(128)
    q = x.q.contiguous().to(DEV)
    qb = bits16(x.q)
    worst = 0.0
    for t in range(T, T + 2 * R + 3):  # single-token appends through two window flushes
        gpu.append(x.k[:, :, t:t + 1].contiguous().to(DEV), x.v[:, :, t:t + 1].contiguous().to(DEV))
        ref.append(kb16[:, :, t:t + 1], vb16[:, :, t:t + 1])
        if t % 17 == 0 or t == T + 2 * R + 2:
            out = gpu.decode_attn(q, scale).cpu().numpy().astype(np.float64)
            err = float(np.abs(out - ref.decode_attn(qb, scale)).max())
            worst = max(worst, err)
            assert err <= TOL, f"{name}: after token {t}: {err:.3e}"
    _compare(gpu, ref)
    print(f"G=64 {name}: worst attention error {worst:.2e}", flush=True)


@pytest.mark.parametrize("Hq", [8, 16], ids=["gq4", "gq8"])
def test_group64_ragged_paged_fused(Hq):
    # sequences of different lengths, paged records and the fused step at G = 64
    B, H, R = 3, 2, 64
    lens = [0, 130, 257]
    steps = 70
    max_tokens = max(lens) + steps + 64
    w = dataclasses.replace(small("g64mix", B, H, Hq, max_tokens, 2, 2, torch.float16,
                                  residual_length=R), group_size=G)
    x = make_layer(w, seed=12, n_new=0)
    mk = lambda: kivi.KiviCache(B, H, max_tokens, group_size=G, residual_length=R, device=DEV)
    flat, paged = mk(), mk()
    nb = flat.view().num_blocks
    table = np.random.default_rng(3).permutation(B * nb).astype(np.int32).reshape(B, nb)
    table_d = torch.from_numpy(table).to(DEV)
    paged.set_page_table(table_d, B * nb)
    kd, vd = x.k.to(DEV), x.v.to(DEV)
    T0 = max(lens)
    for c in (flat, paged):
        c.append_varlen(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), lens)
    scale = 1.0 / np.sqrt(128)
    qs = torch.randn(steps, B, Hq, 128, generator=torch.Generator().manual_seed(5)).half()
    pos = list(lens)
    for t in range(steps):
        kn = torch.stack([kd[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        vn = torch.stack([vd[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        pos = [p + 1 for p in pos]
        q = qs[t].contiguous().to(DEV)
        o1 = flat.append_decode_attn(kn, vn, q, scale)
        o2 = paged.append_decode_attn(kn, vn, q, scale)
        assert torch.equal(o1, o2), f"step {t}: paged output differs"
    torch.cuda.synchronize()
    got = gpu_arrays(flat)
    nq, nr = flat.lengths()
    kb16, vb16 = bits16(x.k), bits16(x.v)
    for b in range(B):
        ref = oracle.OracleCache(1, H, 128, max_tokens, 2, 2, G, R, oracle.F16)
        ref.append(kb16[b:b + 1, :, :pos[b]], vb16[b:b + 1, :, :pos[b]])
        assert (ref.n_quant, ref.n_resid) == (nq[b], nr[b])
        mine = {k: a[b * H:(b + 1) * H] for k, a in got.items()}
        assert_cache_equal(mine, oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                           ref.num_blocks, G=G)
        o_ref = ref.decode_attn(bits16(qs[steps - 1][b:b + 1]), scale)
        err = float(np.abs(o1[b:b + 1].cpu().numpy().astype(np.float64) - o_ref).max())
        assert err <= TOL, f"sequence {b}: {err:.3e}"


def test_group64_unsupported_head_ratio():
    # 32 query heads per kv head are not built: rejected before anything is enqueued
    c = kivi.KiviCache(1, 1, 200, group_size=G, residual_length=128, device=DEV)
    k = torch.zeros(1, 1, 70, 128, dtype=torch.float16, device=DEV)
    c.append(k, k)
    q = torch.zeros(1, 32, 128, dtype=torch.float16, device=DEV)
    with pytest.raises(kivi.KiviError) as e:
        c.decode_attn(q, 0.1)
    assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
    with pytest.raises(kivi.KiviError) as e:
        c.append_decode_attn(k[:, :, :1].contiguous(), k[:, :, :1].contiguous(), q, 0.1)
    assert e.value.status == kivi.KIVI_ERR_UNSUPPORTED
    assert c.lengths() == ([0], [70])
