"""Helpers for the GPU parity tests: run the HIP library and the oracle on the
same seeded inputs and compare the valid regions of the packed layout."""
import numpy as np

import oracle
from kv_cache_bit_kivi_amd.inputs import bits16

ARRAYS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid")


def natural_key_meta(a):
    """A record's key scale or zero (uint16 [..., n*8], stored order) in
    channel order: stored position i of each 8 channels is channel
    kivi.KEY_META_ORDER[i]."""
    from kv_cache_bit_kivi_amd import kivi
    s = a.reshape(*a.shape[:-1], -1, 8)
    out = np.empty_like(s)
    out[..., list(kivi.KEY_META_ORDER)] = s
    return out.reshape(a.shape)


def gpu_arrays(cache, units=None):
    """Host copies of the GPU cache arrays, shaped per unit; optionally only
    the listed units (copied one by one to keep host memory small)."""
    import torch
    c = cache.cfg
    U = c.batch * c.num_kv_heads
    out = {}
    for name, t in cache.arrays().items():
        if units is not None:
            t = t[torch.as_tensor(units, device=t.device)]
        a = t.contiguous().view(t.shape[0], -1).cpu().numpy()
        out[name] = a.view(np.uint32) if ("codes" in name or name == "scale_max") else a.view(np.uint16)
        if name in ("k_scale", "k_zero"):
            out[name] = natural_key_meta(out[name])
    return out


def paged_arrays(cache, table, units=None):
    """Host copies of the packed fields per unit of a paged cache, gathering
    each unit's blocks through the page table (block g of sequence b, kv head
    h is record table[b][g] * H + h), plus the window arrays; optionally only
    the listed units."""
    import torch
    v, cfg = cache.view(), cache.cfg
    H, U, nb, bb = cfg.num_kv_heads, cfg.batch * cfg.num_kv_heads, v.num_blocks, v.block_bytes
    units = list(range(U)) if units is None else list(units)
    ob = v.blocks - cache.buffer.data_ptr()
    flat = cache.buffer[ob:ob + U * nb * bb].view(U * nb, bb)
    idx = torch.tensor([[int(table[u // H][g]) * H + u % H for g in range(nb)] for u in units],
                       device=flat.device)
    recs = flat[idx]  # [units][nb][block_bytes]
    G, D, n = cfg.group_size, cfg.head_dim, len(units)

    def field(off, nbytes, as_words):
        a = recs[:, :, off:off + nbytes].contiguous().view(n, -1).cpu().numpy()
        return a.view(np.uint32) if as_words else a.view(np.uint16)

    out = {
        "k_codes": field(v.off_k_codes, G * D * cfg.k_bits // 8, True),
        "k_scale": natural_key_meta(field(v.off_k_scale, 2 * D, False)),
        "k_zero": natural_key_meta(field(v.off_k_zero, 2 * D, False)),
        "v_codes": field(v.off_v_codes, G * D * cfg.v_bits // 8, True),
        "v_scale": field(v.off_v_scale, 2 * D, False),
        "v_zero": field(v.off_v_zero, 2 * D, False),
    }
    win = gpu_arrays(cache, units)
    out["k_resid"], out["v_resid"] = win["k_resid"], win["v_resid"]
    return out


def expected_scale_max(ref):
    """Per unit and packed block of the oracle cache: the largest key scale
    (low half) and value scale (high half) as fp16 bit patterns, uint32
    [U][n_quant / G].  Scales are >= 0, so the largest bit pattern is the
    largest value."""
    U, D, nb = ref.B * ref.H, ref.D, ref.num_blocks
    nblk = ref.n_quant // ref.G
    ks = ref.array("k_scale").reshape(U, nb, D)[:, :nblk].max(-1, initial=0).astype(np.uint32)
    vs = ref.array("v_scale").reshape(U, nb, D)[:, :nblk].max(-1, initial=0).astype(np.uint32)
    return ks | (vs << 16)


def assert_scale_max(cache, ref, units=None, table=None):
    """The GPU cache's per-record scale maxima equal the oracle's, for the
    packed blocks of the listed units (all by default; the oracle cache holds
    every unit of the GPU cache); paged caches give their table (record of
    unit u, block g: table[u // H][g] * H + u % H)."""
    import torch
    want = expected_scale_max(ref)
    H = cache.cfg.num_kv_heads
    flat = cache.arrays()["scale_max"].reshape(-1)
    units = range(want.shape[0]) if units is None else units
    nb = cache.view().num_blocks
    n = want.shape[1]
    if n == 0:
        return
    for u in units:
        if table is None:
            idx = torch.arange(u * nb, u * nb + n, device=flat.device)
        else:
            idx = torch.as_tensor([int(table[u // H][g]) * H + u % H for g in range(n)], device=flat.device)
        got = flat[idx].cpu().numpy().view(np.uint32)
        row = want[u]
        bad = np.nonzero(got != row)[0]
        assert bad.size == 0, (f"scale_max: {bad.size} mismatches, unit {u} block {bad[0]}: "
                               f"gpu {got[bad[0]]:#010x} oracle {row[bad[0]]:#010x}")


def oracle_arrays(ref):
    U = ref.B * ref.H
    return {n: a.reshape(U, -1) for n, a in ref.arrays().items()}


def valid_slices(n_quant, n_resid, cap, nb, D=128, G=32):
    """Selectors of the valid region of each per-unit flat array: packed
    tokens [0, n_quant) and window slots [0, n_resid)."""
    nblk = n_quant // G
    return {
        "k_codes": lambda a: a[:, : n_quant * (a.shape[1] // cap)],
        "k_scale": lambda a: a[:, : nblk * D],
        "k_zero": lambda a: a[:, : nblk * D],
        "v_codes": lambda a: a[:, : nblk * (a.shape[1] // nb)],
        "v_scale": lambda a: a[:, : nblk * D],
        "v_zero": lambda a: a[:, : nblk * D],
        "k_resid": lambda a: a[:, : n_resid * D],
        "v_resid": lambda a: a[:, : n_resid * D],
    }


def assert_cache_equal(got, want, n_quant, n_resid, cap, nb, G=32):
    sl = valid_slices(n_quant, n_resid, cap, nb, G=G)
    for name in ARRAYS:
        a, b = sl[name](got[name]), sl[name](want[name])
        assert a.shape == b.shape, (name, a.shape, b.shape)
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            u, i = bad[0]
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at unit {u} index {i}: "
                                 f"gpu {a[u, i]:#x} oracle {b[u, i]:#x}")


def oracle_for(x_k, x_v, w, max_tokens, n_tokens=None):
    """Oracle cache of a workload's layer over all units (small sizes)."""
    ref = oracle.OracleCache(w.batch, w.kv_heads, w.head_dim, max_tokens, w.k_bits, w.v_bits,
                             w.group_size, w.residual_length,
                             oracle.BF16 if "bfloat" in str(w.dtype) else oracle.F16)
    kb, vb = bits16(x_k), bits16(x_v)
    if n_tokens is not None:
        kb, vb = kb[:, :, :n_tokens], vb[:, :, :n_tokens]
    ref.append(kb, vb)
    return ref


def unit_oracle(k_unit, v_unit, w, max_tokens, dtype_code):
    """Oracle cache of one (batch, kv head) unit; k_unit/v_unit are host
    uint16 arrays [T][D]."""
    ref = oracle.OracleCache(1, 1, w.head_dim, max_tokens, w.k_bits, w.v_bits, w.group_size,
                             w.residual_length, dtype_code)
    ref.append(k_unit[None, None], v_unit[None, None])
    return ref
