"""Parity at the full workload sizes, in the launch configuration the benchmark
times: bulk append of the prefix (one pack launch), then the decode step
kivi_append_decode_attn (the full window packed first, then token append and
split-K attention in one launch, then the merge) with the default split
planner.

Every (batch, kv head) unit of every layer is compared with the oracle, run
over the whole layer: packed arrays, per-record scale maxima and window bit
for bit, and the attention output of every query head within 2e-3.  The
workloads c1-c3, c2 with 8 query heads per kv head (the 64q/8kv shape of
70B-class models), and all 32 layers of c4, one layer's inputs at a time.
The cache beyond 4 GiB is compared on sampled units."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import WORKLOADS, bits16, make_layer
from tests.gpu_helpers import (assert_cache_equal, assert_scale_max, gpu_arrays, oracle_arrays,
                               paged_arrays, unit_oracle)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3

C2_GQ8 = dataclasses.replace(WORKLOADS["c2"], name="c2gq8", q_heads=64,
                             description="c2 with 64 query heads over 8 kv heads")


def _layer_parity(w, layer, name):
    """Whole-layer parity of one layer (seed = layer); returns (units, heads, worst error)."""
    T = w.tokens
    x = make_layer(w, seed=layer, device=DEV, n_new=1)
    cache = kivi.KiviCache(w.batch, w.kv_heads, T + 1, k_bits=w.k_bits, v_bits=w.v_bits,
                           group_size=w.group_size, residual_length=w.residual_length,
                           dtype=w.dtype, device=DEV)
    cache.append(x.k[:, :, :T].contiguous(), x.v[:, :, :T].contiguous())
    scale = 1.0 / np.sqrt(w.head_dim)
    out = cache.append_decode_attn(x.k[:, :, T:].contiguous(), x.v[:, :, T:].contiguous(),
                                   x.q.contiguous(), scale)
    torch.cuda.synchronize()
    assert (cache.n_quant, cache.n_resid) == (T, 1)  # every workload has T a multiple of R
    dt = oracle.BF16 if w.dtype == torch.bfloat16 else oracle.F16
    ref = oracle.OracleCache(w.batch, w.kv_heads, w.head_dim, T + 1, w.k_bits, w.v_bits, w.group_size,
                             w.residual_length, dt)
    ref.append(bits16(x.k), bits16(x.v))
    assert (ref.n_quant, ref.n_resid) == (T, 1)
    assert_cache_equal(gpu_arrays(cache), oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                       ref.num_blocks, G=w.group_size)
    assert_scale_max(cache, ref)
    o_ref = ref.decode_attn(bits16(x.q), scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - o_ref)
    U, Hq = w.batch * w.kv_heads, w.batch * w.q_heads
    print(f"workload {name} layer {layer}: {U} units bit-exact, {Hq} query heads, attention max abs "
          f"error {err.max():.2e}", flush=True)
    assert err.max() <= TOL, np.unravel_index(np.argmax(err), err.shape)
    return U, Hq, float(err.max())


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c2gq8"])
def test_fullsize_every_unit(name):
    w = C2_GQ8 if name == "c2gq8" else WORKLOADS[name]
    print(f"workload {name}: B={w.batch} H={w.kv_heads} Hq={w.q_heads} T={w.tokens} "
          f"bits={w.k_bits}/{w.v_bits} {w.dtype}", flush=True)
    units, heads, worst = _layer_parity(w, 0, name)
    print(f"workload {name}: compared {units} units and {heads} query heads of 1 layer "
          f"(worst {worst:.2e})", flush=True)


@pytest.mark.parametrize("first", [0, 8, 16, 24], ids=["layers0-7", "layers8-15", "layers16-23",
                                                     "layers24-31"])
def test_fullsize_c4_every_layer(first):
    # the 32 layers in four tests of eight (the oracle's binary64 attention
    # over 131072 tokens takes a few seconds per layer)
    w = WORKLOADS["c4"]
    print(f"workload c4: B={w.batch} H={w.kv_heads} Hq={w.q_heads} T={w.tokens}, layers {first}.."
          f"{first + 7} of {w.layers}", flush=True)
    units = heads = 0
    worst = 0.0
    for layer in range(first, first + 8):
        u, h, e = _layer_parity(w, layer, "c4")
        units, heads, worst = units + u, heads + h, max(worst, e)
    print(f"workload c4: compared {units} units and {heads} query heads over 8 layers "
          f"(worst {worst:.2e})", flush=True)


@pytest.mark.parametrize("paged", [False, True], ids=["unit_major", "paged"])
def test_cache_beyond_4gib_sampled_units(paged):
    # 1024 units of 32768 tokens at 4/4 bits: 160 B per token and unit, 5.4 GB
    # of records, so the last unit's records lie beyond 2^32 bytes (paged: a
    # seeded permutation of the records spreads every unit over the pool);
    # every record, window and partial offset must be formed in 64 bits
    w = dataclasses.replace(WORKLOADS["c2"], name="c2x4", kv_heads=32, q_heads=128, k_bits=4,
                            v_bits=4, description="c2 with 32 kv heads and 4-bit codes")
    assert w.batch * w.kv_heads * w.tokens * 160 > 1 << 32
    _sampled_parity(w, w.name + (" paged" if paged else ""), paged=paged)


def _sampled_parity(w, name, paged=False):
    T = w.tokens
    U = w.batch * w.kv_heads
    print(f"workload {name}: B={w.batch} H={w.kv_heads} Hq={w.q_heads} T={T} "
          f"bits={w.k_bits}/{w.v_bits} {w.dtype} (layer 0)", flush=True)
    x = make_layer(w, seed=0, device=DEV, n_new=1)
    cache = kivi.KiviCache(w.batch, w.kv_heads, T + 1, k_bits=w.k_bits, v_bits=w.v_bits,
                           group_size=w.group_size, residual_length=w.residual_length,
                           dtype=w.dtype, device=DEV)
    table = None
    if paged:
        nb = cache.view().num_blocks
        table = np.random.default_rng(7).permutation(w.batch * nb).astype(np.int32).reshape(w.batch, nb)
        cache.set_page_table(torch.from_numpy(table).to(DEV), w.batch * nb)
    cache.append(x.k[:, :, :T].contiguous(), x.v[:, :, :T].contiguous())
    cache.flush()
    scale = 1.0 / np.sqrt(w.head_dim)
    out = cache.append_decode_attn(x.k[:, :, T:].contiguous(), x.v[:, :, T:].contiguous(),
                                   x.q.contiguous(), scale)
    torch.cuda.synchronize()
    v = cache.view()
    assert (v.n_quant, v.n_resid) == (T, 1)  # every workload has T a multiple of R
    rng = np.random.default_rng(U)
    units = sorted({0, U - 1, *[int(u) for u in rng.integers(1, U - 1, 6)]})
    print(f"workload {name}: {len(units)} of {U} units sampled", flush=True)
    got = gpu_arrays(cache, units) if table is None else paged_arrays(cache, table, units)
    dt = oracle.BF16 if w.dtype == torch.bfloat16 else oracle.F16
    for i, u in enumerate(units):
        b, h = divmod(u, w.kv_heads)
        print(f"workload {name}: unit {u} (batch {b}, kv head {h})", flush=True)
        ref = unit_oracle(bits16(x.k[b, h]), bits16(x.v[b, h]), w, T + 1, dt)
        assert (ref.n_quant, ref.n_resid) == (v.n_quant, v.n_resid)
        mine = {k: a[i:i + 1] for k, a in got.items()}
        assert_cache_equal(mine, oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                           ref.num_blocks)
        heads = slice(h * w.gq, (h + 1) * w.gq)
        o_ref = ref.decode_attn(bits16(x.q[b:b + 1, heads]), scale)
        o_got = out[b:b + 1, heads].cpu().numpy().astype(np.float64)
        err = np.abs(o_got - o_ref).max()
        print(f"workload {name}: unit {u} attention max abs error {err:.2e}", flush=True)
        assert err <= TOL


def test_unit_beyond_2gib_of_records():
    """One (batch, kv head) unit whose block records span more than 2 GiB: 22.4M
    tokens at 2/2 bits, 3 KiB per 32-token record, so offsets inside the unit
    pass 2^31 bytes.  The decode over the unit-major records (stages loaded
    through buffer resources based at each step's first record) equals, bit for
    bit, the decode of the same records through an identity page table (global
    loads with 64-bit addresses); sampled records (the first, one in the middle
    and the last two, beyond 2 GiB) equal the oracle's packing of their own 32
    tokens, since quantization is local to a block.  (The oracle over all 22.4M
    tokens would take minutes.)"""
    from tests.gpu_helpers import natural_key_meta
    nblk = 700_416  # 700 416 x 3072 B > 2^31
    T, G, D, Hq = nblk * 32, 32, 128, 4
    print(f"unit beyond 2 GiB: T={T}, {nblk} records of 3072 B ({nblk * 3072 / 2**30:.2f} GiB)", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(11)
    k = (torch.randn(1, 1, T + 1, D, generator=gen, device=DEV) * 1.5).to(torch.float16)
    v = torch.randn(1, 1, T + 1, D, generator=gen, device=DEV).to(torch.float16)
    q = torch.randn(1, Hq, D, generator=gen, device=DEV).to(torch.float16)
    c = kivi.KiviCache(1, 1, T + 1, k_bits=2, v_bits=2, residual_length=128, dtype=torch.float16, device=DEV)
    c.append(k[:, :, :T].contiguous(), v[:, :, :T].contiguous())
    c.append(k[:, :, T:].contiguous(), v[:, :, T:].contiguous())
    assert c.lengths() == ([T], [1])
    scale = 1.0 / np.sqrt(D)
    o_unit = c.decode_attn(q, scale).clone()
    nb = c.view().num_blocks
    c.set_page_table(torch.arange(nb, dtype=torch.int32, device=DEV)[None].contiguous(), nb)
    o_paged = c.decode_attn(q, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o_unit).all()
    assert torch.equal(o_unit, o_paged), "unit-major and paged decodes of the same records differ"
    a = c.arrays()
    for g in (0, nblk // 2, nblk - 2, nblk - 1):
        ref = oracle.OracleCache(1, 1, D, G + 1, 2, 2, G, G, oracle.F16)
        ref.append(bits16(k[:, :, g * G:g * G + G + 1].cpu()), bits16(v[:, :, g * G:g * G + G + 1].cpu()))
        assert (ref.n_quant, ref.n_resid) == (G, 1)
        want = oracle_arrays(ref)
        got = {n: a[n][0, g].contiguous().cpu().numpy().reshape(1, -1) for n in
               ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")}
        got = {n: x.view(np.uint32) if "codes" in n else x.view(np.uint16) for n, x in got.items()}
        got["k_scale"], got["k_zero"] = natural_key_meta(got["k_scale"]), natural_key_meta(got["k_zero"])
        for n, x in got.items():
            w = want[n][:, :x.shape[1]]
            assert np.array_equal(x, w), f"record {g}: {n} differs from the oracle"
    print(f"unit beyond 2 GiB: decodes bit-identical, 4 sampled records match the oracle", flush=True)
