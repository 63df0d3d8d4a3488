"""Seeded random configurations over the whole knob space at once: batch,
kv heads, query heads per kv head (1, 2, 4, 8), group size (32, 64), window
(a multiple of G up to 256), key and value bits, fp16 or bf16, unit-major or
paged records, equal or different prefill lengths, then single-token appends
through window flushes and fused decode steps.  Every sequence is compared
with an oracle cache of its own: packed arrays bit for bit, attention within
2e-3 at every 7th decode step and the last.  Combinations no hand-written case covers are
where a layout or sizing mistake would hide."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import bits16, make_layer, small
from tests.gpu_helpers import assert_cache_equal, gpu_arrays, oracle_arrays, paged_arrays

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.choice([32, 64]))
    R = int(G * rng.choice([1, 2, 4])) if G == 32 else int(rng.choice([64, 128, 256]))
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 3))
    gq = int(rng.choice([1, 2, 4, 8]))
    kb, vb = int(rng.choice([2, 4])), int(rng.choice([2, 4]))
    dt = torch.bfloat16 if rng.random() < 0.4 else torch.float16
    ragged = bool(rng.random() < 0.5)
    lens = [int(x) for x in rng.integers(0, 600, B)] if ragged else [int(rng.integers(1, 600))] * B
    steps = int(rng.integers(1, R + 40))
    paged = bool(rng.random() < 0.5)
    return dict(G=G, R=R, B=B, H=H, gq=gq, kb=kb, vb=vb, dt=dt, lens=lens, steps=steps,
                paged=paged)


@pytest.mark.parametrize("seed", range(128))
def test_random_configuration(seed):
    c = draw(seed)
    G, R, B, H, gq, kb, vb, dt = (c[k] for k in ("G", "R", "B", "H", "gq", "kb", "vb", "dt"))
    lens, steps = c["lens"], c["steps"]
    print(f"seed {seed}: {c}", flush=True)
    Hq = H * gq
    max_tokens = max(lens) + steps
    w = dataclasses.replace(small(f"rand{seed}", B, H, Hq, max_tokens, kb, vb, dt,
                                  residual_length=R), group_size=G)
    x = make_layer(w, seed=seed, n_new=0)
    cache = kivi.KiviCache(B, H, max_tokens, k_bits=kb, v_bits=vb, group_size=G,
                           residual_length=R, dtype=dt, device=DEV)
    nb = cache.view().num_blocks
    table = None
    if c["paged"]:
        table = np.random.default_rng(seed).permutation(B * nb).astype(np.int32).reshape(B, nb)
        cache.set_page_table(torch.from_numpy(table).to(DEV), B * nb)
    kd, vd = x.k.to(DEV), x.v.to(DEV)
    T0 = max(lens)
    if len(set(lens)) == 1:
        cache.append(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous())
    else:
        cache.append_varlen(kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), lens)
    scale = 1.0 / np.sqrt(128)
    dtc = oracle.BF16 if dt == torch.bfloat16 else oracle.F16
    kb16, vb16 = bits16(x.k), bits16(x.v)
    refs = []
    for b in range(B):
        ref = oracle.OracleCache(1, H, 128, max_tokens, kb, vb, G, R, dtc)
        ref.append(kb16[b:b + 1, :, :lens[b]], vb16[b:b + 1, :, :lens[b]])
        refs.append(ref)
    qgen = torch.Generator().manual_seed(seed)
    pos = list(lens)
    worst = 0.0
    for t in range(steps):
        kn = torch.stack([kd[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        vn = torch.stack([vd[b, :, pos[b]] for b in range(B)])[:, :, None].contiguous()
        for b in range(B):
            refs[b].append(kb16[b:b + 1, :, pos[b]:pos[b] + 1], vb16[b:b + 1, :, pos[b]:pos[b] + 1])
        pos = [p + 1 for p in pos]
        q = torch.randn(B, Hq, 128, generator=qgen).to(dt)
        out = cache.append_decode_attn(kn, vn, q.to(DEV), scale)
        if t % 7 == 0 or t == steps - 1:
            o = out.cpu().numpy().astype(np.float64)
            for b in range(B):
                err = float(np.abs(o[b:b + 1] - refs[b].decode_attn(bits16(q[b:b + 1]), scale)).max())
                worst = max(worst, err)
                assert err <= TOL, f"seed {seed}, step {t}, sequence {b}: {err:.3e}"
    torch.cuda.synchronize()
    got = gpu_arrays(cache) if not c["paged"] else paged_arrays(cache, table)
    nq, nr = cache.lengths()
    for b in range(B):
        ref = refs[b]
        assert (ref.n_quant, ref.n_resid) == (nq[b], nr[b])
        mine = {k: a[b * H:(b + 1) * H] for k, a in got.items()}
        assert_cache_equal(mine, oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                           ref.num_blocks, G=G)
    print(f"seed {seed}: worst attention error {worst:.2e}", flush=True)
