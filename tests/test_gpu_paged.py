"""Paged block records (kivi_cache_set_page_table): a cache whose blocks sit
in pages given by a permuted page table against the same cache in the
unit-major layout, fed identical inputs: every decode output bit-identical,
every packed block record byte-identical through the table, and the paged
cache against the oracle at the end.  Pools of batch x blocks pages and
smaller pools (sequences that never reach capacity) are covered, with
sequences of different lengths, the fused decode step and a reset sequence
refilled in its pages."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import bits16, make_layer, small

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3

#        name           B  H  Hq  kb vb dtype           R   prefill            steps full_pool
CASES = [("mha_full",    3, 2, 2,  2, 2, torch.float16,  32, [200, 64, 129],    60,  True),
         ("gq4_small",   4, 2, 8,  2, 4, torch.float16,  32, [300, 0, 31, 150],  40,  False),
         ("gq2_bf16_4b", 2, 1, 2,  4, 4, torch.bfloat16, 64, [130, 65],         70,  True),
         ("gq8_small",   2, 1, 8,  2, 2, torch.float16,  32, [100, 250],        20,  False)]


def records(cache):
    """The block region of the cache buffer as [records][block_bytes] bytes."""
    v = cache.view()
    n = cache.cfg.batch * cache.cfg.num_kv_heads * v.num_blocks
    return cache.buffer[: n * v.block_bytes].view(n, v.block_bytes)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_matches_unit_major(case):
    name, B, H, Hq, kb, vb, dt, R, lens, steps, full = case
    print(f"paged {name}: B={B} H={H} Hq={Hq} bits={kb}/{vb} R={R} prefill {lens} "
          f"{'full' if full else 'small'} pool", flush=True)
    max_tokens = 600
    w = small(name, B, H, Hq, max_tokens, kb, vb, dt, residual_length=R)
    x = make_layer(w, seed=4, n_new=0)
    mk = lambda: kivi.KiviCache(B, H, max_tokens, k_bits=kb, v_bits=vb, residual_length=R, dtype=dt,
                                device=DEV)
    flat, paged = mk(), mk()
    nb = flat.view().num_blocks
    # blocks each sequence will ever hold, and a random pool of pages for them
    need = [(l + steps + 2 * R) // 32 + 1 for l in lens]
    pool = B * nb if full else sum(need)
    assert pool <= B * nb
    perm = np.random.default_rng(len(name)).permutation(pool)
    table = np.zeros((B, nb), np.int32)
    k = 0
    for b in range(B):
        m = nb if full else need[b]
        table[b, :m] = perm[k:k + m]
        k += m
    table_d = torch.from_numpy(table).to(DEV)
    paged.set_page_table(table_d, pool)
    kd, vd = x.k.to(DEV), x.v.to(DEV)
    T0 = max(lens)
    for c in (flat, paged):
        c.append_varlen(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), lens)
    scale = 1.0 / np.sqrt(128)
    qs = torch.randn(steps, B, Hq, 128, generator=torch.Generator().manual_seed(2)).to(dt)
    pos = list(lens)

    def step(t):
        kn = torch.stack([kd[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        vn = torch.stack([vd[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        for b in range(B):
            pos[b] += 1
        q = qs[t].contiguous().to(DEV)
        o1 = flat.append_decode_attn(kn, vn, q, scale)
        o2 = paged.append_decode_attn(kn, vn, q, scale)
        assert torch.equal(o1, o2), f"{name}: step {t}: paged output differs"
        return o2

    for t in range(steps // 2):
        step(t)
    # sequence 1 finishes; a new request refills its pages
    for c in (flat, paged):
        c.reset_sequences([1])
    pos[1] = 0
    n1 = [0] * B
    n1[1] = 97
    for c in (flat, paged):
        c.append_varlen(kd[:, :, :97].contiguous(), vd[:, :, :97].contiguous(), n1)
    pos[1] = 97
    for t in range(steps // 2, steps):
        out = step(t)
    torch.cuda.synchronize()
    assert flat.lengths() == paged.lengths()
    nq, nr = paged.lengths()
    rf, rp = records(flat), records(paged)
    for b in range(B):
        for h in range(H):
            u = b * H + h
            for g in range(nq[b] // 32):
                a = rf[u * nb + g]
                p = rp[int(table[b, g]) * H + h]
                assert torch.equal(a, p), f"{name}: unit {u} block {g} (page {table[b, g]}) differs"
    # the paged cache against the oracle (last step's attention)
    dtc = oracle.BF16 if dt == torch.bfloat16 else oracle.F16
    kb16, vb16 = bits16(x.k), bits16(x.v)
    for b in range(B):
        ref = oracle.OracleCache(1, H, 128, max_tokens, kb, vb, 32, R, dtc)
        ref.append(kb16[b:b + 1, :, :pos[b]], vb16[b:b + 1, :, :pos[b]])  # (b = 1: the refill)
        assert (ref.n_quant, ref.n_resid) == (nq[b], nr[b])
        o_ref = ref.decode_attn(bits16(qs[steps - 1][b:b + 1]), scale)
        err = float(np.abs(out[b:b + 1].cpu().numpy().astype(np.float64) - o_ref).max())
        assert err <= TOL, f"{name}: sequence {b}: {err:.3e}"


def test_page_table_validation():
    c = kivi.KiviCache(2, 1, 100, residual_length=32, device=DEV)
    nb = c.view().num_blocks
    t = torch.zeros(2, nb, dtype=torch.int32, device=DEV)
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_set_page_table(c.handle, t.data_ptr(), nb - 1, 1)
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_set_page_table(c.handle, t.data_ptr(), nb, 2 * nb + 1)
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_cache_set_page_table(c.handle, t.data_ptr(), nb, 0)
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    c.set_page_table(t, 2 * nb)
    c.set_page_table(None, 0)
