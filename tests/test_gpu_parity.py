"""GPU parity of the HIP path against the CPU oracle on the same seeded
inputs: packed codes, metadata and window bit-exact; attention within 2e-3
max abs error (fp32 output).  Sizes span several blocks and ragged tails."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import bits16, make_layer, small
from tests.attn_reference import attention, fp32_allowance
from tests.gpu_helpers import assert_cache_equal, assert_scale_max, gpu_arrays, oracle_arrays, oracle_for

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3

#        name              B  H  Hq  T     kb vb dtype           R
CASES = [("c0",            1, 1, 1, 1024, 2, 2, torch.float16, 128),
         ("mha_ragged",    2, 3, 3, 300, 2, 2, torch.float16, 128),
         ("gqa4_bf16_4b",  2, 2, 8, 333, 4, 4, torch.bfloat16, 128),
         ("k2v4",          1, 2, 4, 257, 2, 4, torch.float16, 128),
         ("k4v2_r32",      2, 1, 8, 200, 4, 2, torch.float16, 32),
         ("gq8",           1, 2, 16, 700, 2, 2, torch.float16, 128),
         ("T1",            1, 1, 2, 1, 2, 2, torch.float16, 128),
         ("T32",           1, 1, 1, 32, 2, 2, torch.float16, 128),
         ("T128_fullwin",  1, 2, 2, 128, 2, 2, torch.float16, 128),
         ("T129",          1, 2, 2, 129, 2, 2, torch.bfloat16, 128),
         # 4 query heads per kv head: every head slot of a workgroup used
         ("gq4_f16",       2, 2, 8, 1000, 2, 2, torch.float16, 128),
         ("gq4_k2v4",      1, 2, 8, 700, 2, 4, torch.float16, 128),
         ("gq4_k4v2_r32",  1, 1, 4, 333, 4, 2, torch.float16, 32),
         ("gq4_window",    1, 2, 8, 100, 2, 2, torch.bfloat16, 128),
         ("gq4_T129",      2, 1, 4, 129, 2, 2, torch.float16, 128),
         ("gq4_long",      1, 1, 4, 4096, 2, 2, torch.float16, 128),
         # windows up to the largest accepted (R = 1024): window-only, a full
         # window that the decode token flushes, multi-head, 8 heads per kv head
         ("r1024_window",  1, 2, 8, 1000, 2, 2, torch.float16, 1024),
         ("r1024_flush",   1, 1, 2, 2048, 2, 2, torch.bfloat16, 1024),
         ("r256_mha_4b",   2, 2, 2, 700, 4, 4, torch.float16, 256),
         ("r1024_gq8",     1, 1, 8, 1500, 2, 2, torch.float16, 1024),
         # 8 query heads per kv head in one workgroup (the eight-head layout),
         # every bit pair, long caches
         ("gq8_k2v4_bf16", 1, 2, 16, 900, 2, 4, torch.bfloat16, 128),
         ("gq8_k4v2_long", 1, 1, 8, 3000, 4, 2, torch.float16, 128),
         ("gq8_4b_long",   2, 1, 8, 2500, 4, 4, torch.float16, 64),
         # 16 query heads per kv head: 2 head groups of 8 per split
         ("gq16",          2, 1, 16, 900, 2, 2, torch.float16, 128),
         ("gq16_bf16_4b",  1, 2, 32, 450, 4, 4, torch.bfloat16, 64)]
IDS = [c[0] for c in CASES]


def _setup(case, seed=0, extra=1):
    name, B, H, Hq, T, kb, vb, dt, R = case
    w = small(name, B, H, Hq, T, kb, vb, dt, residual_length=R)
    x = make_layer(w, seed=seed, n_new=extra)
    return w, x


def _gpu_cache(w, max_tokens):
    return kivi.KiviCache(w.batch, w.kv_heads, max_tokens, k_bits=w.k_bits, v_bits=w.v_bits,
                          residual_length=w.residual_length, dtype=w.dtype, device=DEV)


def _dev(t, lo, hi):
    return t[:, :, lo:hi].contiguous().to(DEV)


def _compare(cache, ref):
    torch.cuda.synchronize()
    v = cache.view()
    assert (v.n_quant, v.n_resid) == (ref.n_quant, ref.n_resid)
    assert_cache_equal(gpu_arrays(cache), oracle_arrays(ref), ref.n_quant, ref.n_resid,
                       ref.capacity, ref.num_blocks)
    assert_scale_max(cache, ref)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_prefix_pack_bitexact(case):
    w, x = _setup(case)
    T = w.tokens
    print(f"case {case[0]}: prefix append T={T}", flush=True)
    cache = _gpu_cache(w, T + 1)
    cache.append(_dev(x.k, 0, T), _dev(x.v, 0, T))
    _compare(cache, oracle_for(x.k, x.v, w, T + 1, n_tokens=T))


@pytest.mark.parametrize("case", CASES[:6], ids=IDS[:6])
def test_append_paths_bitexact(case):
    # token-by-token, ragged chunks and an explicit flush on the GPU all give
    # the oracle's bulk result
    w, x = _setup(case, seed=1, extra=0)
    T, R = w.tokens, w.residual_length
    ref = oracle_for(x.k, x.v, w, T, n_tokens=T)
    rng = np.random.default_rng(T)
    for mode in ("single", "chunks", "flush"):
        print(f"case {case[0]}: append mode {mode}", flush=True)
        cache = _gpu_cache(w, T)
        p = 0
        while p < T:
            if mode == "single":
                n = 1
            elif mode == "chunks":
                n = int(rng.integers(1, 2 * R + 40))
            else:
                n = R if p + R <= T else T - p
            n = min(n, T - p)
            cache.append(_dev(x.k, p, p + n), _dev(x.v, p, p + n))
            p += n
            if mode == "flush":
                cache.flush()
        if mode == "flush" and T % R == 0:
            # the final window was packed by the explicit flush; the oracle
            # packs it too when flushed
            ref_f = oracle_for(x.k, x.v, w, T, n_tokens=T)
            ref_f.flush()
            _compare(cache, ref_f)
        else:
            _compare(cache, ref)


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_decode_parity(case, out_dtype):
    # prefix + one decode token (which flushes a full window), then attention
    w, x = _setup(case, seed=2)
    T = w.tokens
    print(f"case {case[0]}: decode out {out_dtype}", flush=True)
    cache = _gpu_cache(w, T + 1)
    cache.append(_dev(x.k, 0, T), _dev(x.v, 0, T))
    cache.append(_dev(x.k, T, T + 1), _dev(x.v, T, T + 1))
    scale = 1.0 / np.sqrt(w.head_dim)
    out = cache.decode_attn(x.q.contiguous().to(DEV), scale, out_dtype=out_dtype)
    ref = oracle_for(x.k, x.v, w, T + 1)
    _compare(cache, ref)
    o_ref = ref.decode_attn(bits16(x.q), scale)
    got = out.float().cpu().numpy().astype(np.float64)
    tol = TOL if out_dtype == torch.float32 else TOL + np.abs(o_ref) * 2.0 ** -11
    err = np.abs(got - o_ref)
    assert np.all(err <= tol), f"max abs error {err.max():.3e}"


SPLIT_CASES = [c for c in CASES if c[0] in ("c0", "gqa4_bf16_4b", "gq8", "gq4_f16", "gq4_k4v2_r32",
                                             "gq4_long")]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_invariance_and_determinism(case):
    w, x = _setup(case, seed=3)
    T = w.tokens
    cache = _gpu_cache(w, T + 1)
    cache.append(_dev(x.k, 0, T + 1), _dev(x.v, 0, T + 1))
    q = x.q.contiguous().to(DEV)
    scale = 1.0 / np.sqrt(w.head_dim)
    n_items = cache.n_quant // 32 + (cache.n_resid + 31) // 32
    outs = {}
    for ns in (1, 2, 7, n_items, 0):
        print(f"case {case[0]}: n_split {ns}", flush=True)
        cache.set_splits(ns)
        outs[ns] = cache.decode_attn(q, scale).cpu().numpy()
    # q*S and p*S are rounded to fp16 hi + lo (2^-22 relative each) relative
    # to each split's own maximum, so changing the split count moves scores
    # by up to 2^-22 * sum_d |c q' S| (about 3e-5 on these inputs) and
    # outputs by that times max |v| (about 30).
    tol = 1e-4
    for ns, o in outs.items():
        d = np.max(np.abs(o - outs[1]))
        print(f"case {case[0]}: n_split {ns} vs 1: max abs diff {d:.2e}", flush=True)
        assert d < tol, (ns, d)
    again = cache.decode_attn(q, scale).cpu().numpy()
    assert np.array_equal(again, outs[0])


@pytest.mark.parametrize("kb,vb,dt", [(2, 2, torch.float16), (4, 4, torch.bfloat16)], ids=["2b_f16", "4b_bf16"])
def test_most_splits(kb, vb, dt):
    # The largest split count the kernels take: 32640 packed tokens (1020
    # streams) forced into 255 splits of one step each, plus the window's
    # partial = 256 partials per query head, all merged by one workgroup
    # (with 2 units the automatic plan is the same).  Against the oracle
    # (2e-3) and a 3-split plan (the split-invariance bound).
    w, x = _setup(("most_splits", 1, 2, 8, 32699, kb, vb, dt, 128), seed=6)
    T = w.tokens + 1
    cache = _gpu_cache(w, T)
    cache.append(_dev(x.k, 0, T), _dev(x.v, 0, T))
    assert (cache.n_quant, cache.n_resid) == (32640, 60)
    q = x.q.contiguous().to(DEV)
    scale = 1.0 / np.sqrt(w.head_dim)
    print(f"most splits {kb}/{vb} {dt}", flush=True)
    cache.set_splits(10 ** 6)
    most = cache.decode_attn(q, scale).cpu().numpy().astype(np.float64)
    cache.set_splits(3)
    few = cache.decode_attn(q, scale).cpu().numpy().astype(np.float64)
    ref = oracle_for(x.k, x.v, w, T)
    o_ref = ref.decode_attn(bits16(x.q), scale)
    print(f"most splits: vs oracle {np.max(np.abs(most - o_ref)):.2e}, vs 3 splits {np.max(np.abs(most - few)):.2e}",
          flush=True)
    assert np.max(np.abs(most - o_ref)) < TOL
    assert np.max(np.abs(most - few)) < 1e-4


def test_empty_and_errors_gpu():
    w, x = _setup(CASES[1])
    cache = _gpu_cache(w, 10)
    q = x.q.contiguous().to(DEV)
    with pytest.raises(kivi.KiviError) as e:
        cache.decode_attn(q, 0.1)
    assert e.value.status == kivi.KIVI_ERR_EMPTY
    cache.append(_dev(x.k, 0, 10), _dev(x.v, 0, 10))
    with pytest.raises(kivi.KiviError) as e:
        cache.append(_dev(x.k, 0, 1), _dev(x.v, 0, 1))
    assert e.value.status == kivi.KIVI_ERR_CAPACITY
    assert (cache.n_quant, cache.n_resid) == (0, 10)


def _hard_triples(bits, count, seed):
    # binary16 triples (min, max, x) where multiplying by a rounded reciprocal
    # gives another code than the division; the kernel's fast path must fall
    # back to the exact division on them
    rng = np.random.default_rng(seed)
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
    idx = np.nonzero((s > 0) & (recip != div))[0][:count]
    return mn[idx], mx[idx], x[idx]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("heads,blocks", [(1, 1), (72, 30)], ids=["one_round", "many_rounds"])
def test_quantizer_hard_cases_bitexact(bits, heads, blocks):
    # one launch of at most one round of workgroups repairs near ties by mask,
    # a bigger one by the careful pass: the same hard block, tiled over
    # `heads` kv heads and `blocks` blocks, reaches both
    mn, mx, xv = _hard_triples(bits, 128, 17 + bits)
    n = mn.size
    # keys: channel d of block 0 holds [mn, mx, x, x, ...] over its 32 tokens;
    # values: token t's channel group m holds [mn, mx, x, ...] over 32 channels
    T = 32
    K = np.empty((T, 128), np.float32)
    V = np.empty((T, 128), np.float32)
    for d in range(128):
        i = d % n
        K[:, d] = xv[i]
        K[0, d], K[1, d] = mn[i], mx[i]
    for t in range(T):
        for m in range(4):
            i = (t * 4 + m) % n
            V[t, m * 32:(m + 1) * 32] = xv[i]
            V[t, m * 32], V[t, m * 32 + 1] = mn[i], mx[i]
    k = torch.from_numpy(K.astype(np.float16))[None, None].repeat(1, heads, blocks, 1)
    v = torch.from_numpy(V.astype(np.float16))[None, None].repeat(1, heads, blocks, 1)
    kk = torch.cat([k, k[:, :, :1]], 2)  # one more token flushes the last block
    vv = torch.cat([v, v[:, :, :1]], 2)
    Tn = T * blocks + 1
    w = small("hard", 1, heads, heads, Tn, bits, bits, torch.float16, residual_length=32)
    cache = _gpu_cache(w, Tn)
    cache.append(kk.contiguous().to(DEV), vv.contiguous().to(DEV))
    ref = oracle.OracleCache(1, heads, 128, Tn, bits, bits, 32, 32)
    ref.append(bits16(kk), bits16(vv))
    assert ref.n_quant == 32 * blocks
    _compare(cache, ref)


@pytest.mark.parametrize("bits", [2, 4])
def test_tiny_scales_bf16_bitexact(bits):
    # bf16 groups whose scale falls below 2^-100 (spreads near 2^-120 and
    # subnormal inputs) next to ordinary groups: the kernel's reciprocal path
    # cannot serve them and the block must take the exact division
    rng = np.random.default_rng(5 + bits)
    T = 64
    K = rng.standard_normal((T, 128)).astype(np.float32)
    V = rng.standard_normal((T, 128)).astype(np.float32)
    base = np.float32(2.0 ** -118)
    K[:, 5] = base * (1 + rng.integers(0, 8, T) / 128)           # spread of a few bf16 ulps
    K[:, 9] = rng.integers(0, 6, T) * np.float32(2.0 ** -133)   # bf16 subnormals
    K[32:, 70] = -base * (1 + rng.integers(0, 4, 32) / 64)     # second block only
    V[3, 32:64] = base * (1 + rng.integers(0, 8, 32) / 128)
    V[40, 96:128] = rng.integers(0, 3, 32) * np.float32(2.0 ** -131)
    k = torch.from_numpy(K).to(torch.bfloat16)[None, None]
    v = torch.from_numpy(V).to(torch.bfloat16)[None, None]
    kk = torch.cat([k, k[:, :, :1]], 2)  # one more token flushes both blocks
    vv = torch.cat([v, v[:, :, :1]], 2)
    w = small("tiny", 1, 1, 1, T + 1, bits, bits, torch.bfloat16, residual_length=32)
    cache = _gpu_cache(w, T + 1)
    cache.append(kk.contiguous().to(DEV), vv.contiguous().to(DEV))
    ref = oracle.OracleCache(1, 1, 128, T + 1, bits, bits, 32, 32, oracle.BF16)
    ref.append(bits16(kk), bits16(vv))
    assert ref.n_quant == T
    _compare(cache, ref)


def test_binding_rejects_malformed_tensors():
    # the KiviCache convenience layer checks dtype, layout and shape before
    # calling the C ABI (which validates the arguments it can see)
    cache = kivi.KiviCache(2, 2, 64, device=DEV)
    good = torch.zeros(2, 2, 8, 128, dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        cache.append(good.to(torch.bfloat16), good)
    with pytest.raises(ValueError):
        cache.append(good.transpose(2, 3), good)
    with pytest.raises(ValueError):
        cache.append(good[:1].contiguous(), good[:1].contiguous())
    with pytest.raises(ValueError):
        cache.append_varlen(good, good, [8])
    cache.append(good, good)
    with pytest.raises(ValueError):
        cache.decode_attn(torch.zeros(2, 4, 64, dtype=torch.float16, device=DEV), 0.1)
    assert (cache.n_quant, cache.n_resid) == (0, 8)


def _attention_check(cache, ref, q, dt, what, extremes):
    # attention within 2e-3 of the binary64 oracle; inputs with extreme
    # ranges add the rounding allowance of a binary32 evaluation on them
    # (tests/attn_reference.py: no binary32 evaluation can promise 2e-3
    # there, tests/test_attention_conditioning.py)
    scale = 1.0 / np.sqrt(128)
    bf = dt == torch.bfloat16
    out = cache.decode_attn(q.to(DEV), scale).cpu().numpy().astype(np.float64)
    o_ref = ref.decode_attn(bits16(q), scale)
    o64, lmax, spread, vsum = attention(ref, bits16(q), scale, bf16=bf)
    assert np.abs(o64 - o_ref).max() <= 1e-9 * max(1.0, np.abs(o_ref).max())
    assert np.all(np.isfinite(out)), f"{what}: non-finite attention output"
    allow = fp32_allowance(lmax, spread, vsum) if extremes else np.zeros_like(spread)
    err = np.abs(out - o_ref)
    i = np.unravel_index(np.argmax(err - allow), err.shape)
    print(f"{what}: attention error {err.max():.3e} (worst against its bound: {err[i]:.3e} "
          f"<= 2e-3 + {allow[i]:.3e}; max |out| {np.abs(o_ref).max():.3e})", flush=True)
    assert np.all(err <= TOL + allow), f"{what}: attention error {err[i]:.3e} at {i}"
    return err


def _degenerate_layer(G, H, T, extremes, seed):
    # Ordinary data with degenerate groups planted in the first three blocks:
    # constant key channels and value groups (scale 0, zero-point = the value),
    # all-zero groups mixing +0 and -0 (zero-point +0), two-valued groups and,
    # with `extremes`, groups spanning -65280 .. 65280 (the widest span whose
    # ends both fp16 and bf16 hold).  Values are exact in fp16 and bf16.
    rng = np.random.default_rng(seed)
    big = 65280.0 if extremes else 5.0
    K = (rng.standard_normal((H, T, 128)) * 2).astype(np.float32)
    V = (rng.standard_normal((H, T, 128)) * 2).astype(np.float32)
    signed_zeros = lambda shape: np.where(rng.random(shape) < 0.5, 0.0, -0.0).astype(np.float32)
    consts = [0.0, 1.25, -2.0, 3.5, -0.0, 7.0, -big, big]
    for c in range(8):  # block 0: constant key channels 0..7
        K[:, :G, c] = consts[c]
    K[:, :G, 8:16] = signed_zeros((H, G, 8))
    K[:, :G, 16:24] = np.where(rng.random((H, G, 8)) < 0.5, -1.5, 2.25)
    K[:, :G, 24] = np.where(np.arange(G) % 2 == 0, -big, big)
    K[:, G:2 * G] = signed_zeros((H, G, 128))  # block 1: every key group zero
    K[:, 2 * G:3 * G, 100] = 0.5
    nv = 128 // G  # value groups per token
    for m in range(nv):  # token 0: every value group constant
        V[:, 0, m * G:(m + 1) * G] = consts[m + 1]
    V[:, 1] = signed_zeros((H, 128))
    V[:, 2, :G] = np.where(np.arange(G) % 2 == 0, -big, big)
    V[:, 2, G:2 * G] = np.where(rng.random((H, G)) < 0.5, -1.5, 2.25)
    V[:, G + 5] = big
    return torch.from_numpy(K)[None], torch.from_numpy(V)[None]


@pytest.mark.parametrize("extremes", [False, True], ids=["plain", "extremes"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("G", [32, 64])
def test_degenerate_groups_bitexact(G, dt, bits, extremes):
    # codes, scales, zero-points and window bit-exact on degenerate groups,
    # and attention against the oracle, the widest-span groups included
    H = 2
    T = 3 * G + 1
    print(f"degenerate G={G} {dt} bits={bits} extremes={extremes}", flush=True)
    K, V = _degenerate_layer(G, H, T, extremes, seed=G + bits)
    k, v = K.to(dt), V.to(dt)
    cache = kivi.KiviCache(1, H, T, k_bits=bits, v_bits=bits, group_size=G, residual_length=G,
                           dtype=dt, device=DEV)
    cache.append(k.contiguous().to(DEV), v.contiguous().to(DEV))
    ref = oracle.OracleCache(1, H, 128, T, bits, bits, G, G,
                             oracle.BF16 if dt == torch.bfloat16 else oracle.F16)
    ref.append(bits16(k), bits16(v))
    assert (ref.n_quant, ref.n_resid) == (3 * G, 1)
    torch.cuda.synchronize()
    assert (cache.n_quant, cache.n_resid) == (ref.n_quant, ref.n_resid)
    assert_cache_equal(gpu_arrays(cache), oracle_arrays(ref), ref.n_quant, ref.n_resid,
                       ref.capacity, ref.num_blocks, G=G)
    assert_scale_max(cache, ref)
    for gq in (1, 2, 4, 8):  # the matrix-core kernel (1, 2, 4) and the vector one (8)
        q = torch.randn(1, H * gq, 128, generator=torch.Generator().manual_seed(bits + gq)).to(dt)
        _attention_check(cache, ref, q, dt, f"degenerate G={G} {dt} bits={bits} extremes={extremes} gq={gq}",
                         extremes)
