"""Pins of the oracle's packed layout and residual-window state (CPU only).

Residual window: page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide",
item 3 of "The Three Structural Innovations of KIVI" and "Step 3"; page "KV
cache quantization with KIVI INT2 setup guide", defaults G = 32, R = 128.
The window is packed as a whole when it is full and another token arrives,
so it always holds between 1 and R tokens after an append.
"""
import numpy as np
import pytest

from tests.grid_inputs import grid_kv, to_bits


def _pattern_cache(oracle_mod, bits, mod):
    # D = G = R = 32; K[t][d] = V[t][d] = (t + d) mod `mod`; 33 tokens so the
    # first 32 are packed when the 33rd arrives.
    D = 32
    t = np.arange(33)[:, None]
    d = np.arange(D)[None, :]
    x = ((t + d) % mod).astype(np.float16)[None, None]
    c = oracle_mod.OracleCache(1, 1, D, 64, bits, bits, 32, 32)
    c.append(x.view(np.uint16), x.view(np.uint16))
    return c


def test_layout_2bit_hand_words(oracle_mod):
    # Per channel d the key group over tokens 0..31 holds (t + d) mod 4, so
    # min 0, max 3, s = 1 and code = value.  Word w of token t holds channels
    # 16w..16w+15; even channels go to the low half-word, odd to the high one
    # (2 bits each, increasing).  For token 0 the even channels carry
    # 0,2,0,2,.. -> 0x8888 and the odd ones 1,3,1,3,.. -> 0xDDDD, so the word
    # is 0xDDDD8888; tokens 1, 2, 3 shift the pattern to 0x2222DDDD,
    # 0x77772222 and 0x88887777.  Channels 16..31 repeat channels 0..15.
    c = _pattern_cache(oracle_mod, 2, 4)
    assert (c.n_quant, c.n_resid) == (32, 1)
    kc = c.array("k_codes").reshape(-1, 2)  # [token][word]
    expect = [0xDDDD8888, 0x2222DDDD, 0x77772222, 0x88887777]
    for t in range(32):
        assert kc[t].tolist() == [expect[t % 4]] * 2, t
    # Values: word w of (block 0, channel d) holds rows 16w..16w+15 with the
    # same order, stored word-major ([word][channel]); the value group of token t over channels gives codes
    # (t + d) mod 4 as well, so channel d shows the token-d word pattern.
    vc = c.array("v_codes").reshape(-1, 2, 32)[0]  # [word][channel]
    for d in range(32):
        assert vc[:, d].tolist() == [expect[d % 4]] * 2, d
    assert set(c.array("k_scale")[:32].tolist()) == {0x3C00}
    assert set(c.array("k_zero")[:32].tolist()) == {0}
    assert set(c.array("v_scale")[:32].tolist()) == {0x3C00}
    assert set(c.array("v_zero")[:32].tolist()) == {0}
    # the 33rd token sits in window slot 0
    slot0 = np.float16((32 + np.arange(32)) % 4).view(np.uint16)
    assert c.array("k_resid")[:32].tolist() == slot0.tolist()


def test_layout_4bit_hand_words(oracle_mod):
    # (t + d) mod 16 with 4-bit codes: 8 codes per word, nibbles; for token 0
    # word 0 (channels 0..7): even channels 0,2,4,6 -> 0x6420, odd 1,3,5,7 ->
    # 0x7531, word = 0x75316420; word 1 (channels 8..15) = 0xFDB9ECA8; words
    # 2 and 3 repeat them.
    c = _pattern_cache(oracle_mod, 4, 16)
    kc = c.array("k_codes").reshape(-1, 4)
    assert kc[0].tolist() == [0x75316420, 0xFDB9ECA8, 0x75316420, 0xFDB9ECA8]
    # token 8: codes (8 + d) mod 16 -> word 0 holds 8..15, word 1 holds 0..7
    assert kc[8].tolist() == [0xFDB9ECA8, 0x75316420, 0xFDB9ECA8, 0x75316420]
    vc = c.array("v_codes").reshape(-1, 4, 32)[0]  # [word][channel]
    assert vc[:, 0].tolist() == [0x75316420, 0xFDB9ECA8, 0x75316420, 0xFDB9ECA8]
    assert vc[:, 8].tolist() == [0xFDB9ECA8, 0x75316420, 0xFDB9ECA8, 0x75316420]


def test_layout_group64_hand_words(oracle_mod):
    # G = D = R = 64, 2-bit codes, 65 tokens.  Keys: K[t][d] = (t + d) mod 4,
    # times 3 for tokens 32..63; values: V[t][d] = (t + d) mod 4, times 3 for
    # channels 32..63.  Every group of 64 then spans 0..9, so s = 3 (0x4200)
    # and zero-point 0; a group of 32 would give s = 1 on the unscaled half.
    # Unscaled inputs 0,1,2,3 become codes 0,0,1,1 (thirds round to the
    # nearest integer); scaled ones 0,3,6,9 become 0,1,2,3.
    D, T = 64, 65
    t = np.arange(T)[:, None]
    d = np.arange(D)[None, :]
    base = (t + d) % 4
    K = (base * np.where((t >= 32) & (t < 64), 3, 1)).astype(np.float16)[None, None]
    V = (base * np.where(d >= 32, 3, 1)).astype(np.float16)[None, None]
    c = oracle_mod.OracleCache(1, 1, D, 128, 2, 2, 64, 64)
    c.append(K.view(np.uint16), V.view(np.uint16))
    assert (c.n_quant, c.n_resid) == (64, 1)
    # Codes 0,0,1,1 by (t + d) mod 4, packed as in the 32-group pin (even
    # channels in the low half-word, odd in the high, 2 bits each): token
    # t = 0 mod 4 -> even 0,1,0,1.. = 0x4444, odd 0x4444; t = 1 -> 0x4444
    # and 0x1111; t = 2 -> 0x1111 both; t = 3 -> 0x1111 and 0x4444.
    thirds = [0x44444444, 0x11114444, 0x11111111, 0x44441111]
    plain = [0xDDDD8888, 0x2222DDDD, 0x77772222, 0x88887777]
    kc = c.array("k_codes").reshape(-1, 4)  # [token][word], 16 channels a word
    for tok in range(64):
        want = thirds[tok % 4] if tok < 32 else plain[tok % 4]
        assert kc[tok].tolist() == [want] * 4, tok
    # value words: word w of channel d holds rows 16w..16w+15, [word][channel]
    vc = c.array("v_codes").reshape(-1, 4, D)[0]
    for ch in range(D):
        want = thirds[ch % 4] if ch < 32 else plain[ch % 4]
        assert vc[:, ch].tolist() == [want] * 4, ch
    assert set(c.array("k_scale")[:D].tolist()) == {0x4200}
    assert set(c.array("k_zero")[:D].tolist()) == {0}
    assert set(c.array("v_scale")[:64].tolist()) == {0x4200}
    assert set(c.array("v_zero")[:64].tolist()) == {0}
    assert c.array("k_resid")[:D].tolist() == K[0, 0, 64].view(np.uint16).tolist()


def _random_bits(rng, shape):
    x = (rng.standard_normal(shape) * 2 + rng.standard_normal(shape[-1])).astype(np.float16)
    return x.view(np.uint16)


@pytest.mark.parametrize("R", [32, 128])
def test_window_matches_list_model(oracle_mod, R):
    # A list model of the window: a full window is moved to the packed store
    # before the next token enters.  Counters and window contents must match
    # it after every chunk; the packed tokens must be the oldest ones.
    rng = np.random.default_rng(R)
    B, H, D, T = 2, 2, 64, 5 * R + 17
    K, V = grid_kv(B, H, T, D, seed=R)
    kb, vb = to_bits(K, "f16"), to_bits(V, "f16")
    c = oracle_mod.OracleCache(B, H, D, T, 2, 2, 32, R)
    window, packed = [], []
    pos = 0
    for n in [1, R - 1, 1, 1, 2 * R, 3, R + 7]:
        n = min(n, T - pos)
        c.append(kb[:, :, pos:pos + n], vb[:, :, pos:pos + n])
        for t in range(pos, pos + n):
            if len(window) == R:
                packed += window
                window = []
            window.append(t)
        pos += n
        assert (c.n_quant, c.n_resid) == (len(packed), len(window))
        assert c.n_quant % R == 0 and (n == 0 or 1 <= c.n_resid <= R)
        kres = c.array("k_resid").reshape(B, H, R, D)
        for i, t in enumerate(window):
            assert np.array_equal(kres[:, :, i], kb[:, :, t])
    # grid-exact inputs dequantize exactly, so the packed store must decode
    # to the oldest tokens, in order
    for u, t, d in [(0, 0, 0), (1, 17, 5), (2, 2 * R + 3, 40), (3, len(packed) - 1, 63)]:
        assert _key_hat(oracle_mod, c, u, t, d, D) == float(K.reshape(B * H, T, D)[u, t, d])


def _key_hat(oracle_mod, c, u, t, d, D):
    # decode one packed key element following the layout of the header:
    # token-major words of 16 channels, even codes low half, odd codes high
    kc = c.array("k_codes").reshape(-1, c.capacity, D // 16)
    ks = c.array("k_scale").reshape(-1, c.num_blocks, D)
    kz = c.array("k_zero").reshape(-1, c.num_blocks, D)
    w, i = int(kc[u, t, d // 16]), d % 16
    code = (w >> (2 * (i // 2) + 16 * (i % 2))) & 3
    return oracle_mod.dequant(code, ks[u, t // 32, d], kz[u, t // 32, d])


def test_flush_then_append_equals_bulk(oracle_mod):
    rng = np.random.default_rng(4)
    B, H, D, R = 1, 3, 64, 128
    kb = _random_bits(rng, (B, H, R + 1, D))
    vb = _random_bits(rng, (B, H, R + 1, D))
    a = oracle_mod.OracleCache(B, H, D, 300, 2, 2, 32, R)
    a.append(kb[:, :, :R], vb[:, :, :R])
    assert (a.n_quant, a.n_resid) == (0, R)
    a.flush()
    assert (a.n_quant, a.n_resid) == (R, 0)
    a.flush()  # not full: no-op
    assert (a.n_quant, a.n_resid) == (R, 0)
    a.append(kb[:, :, R:], vb[:, :, R:])
    b = oracle_mod.OracleCache(B, H, D, 300, 2, 2, 32, R)
    b.append(kb, vb)
    assert (b.n_quant, b.n_resid) == (R, 1)
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert np.array_equal(a.array(name), b.array(name)), name
    assert np.array_equal(a.array("k_resid").reshape(B, H, R, D)[:, :, 0],
                          b.array("k_resid").reshape(B, H, R, D)[:, :, 0])


@pytest.mark.parametrize("kbits,vbits,dtype", [(2, 2, 0), (4, 4, 1), (2, 4, 0)])
def test_path_independence(oracle_mod, kbits, vbits, dtype):
    # bulk append == token-by-token == arbitrary chunking, bit for bit
    rng = np.random.default_rng(kbits * 10 + vbits)
    B, H, D, T, R = 2, 2, 64, 333, 64
    kb = _random_bits(rng, (B, H, T, D))
    vb = _random_bits(rng, (B, H, T, D))
    if dtype == 1:  # bf16 patterns: take the top halves of fp32 values
        f = (rng.standard_normal((B, H, T, D)) * 3).astype(np.float32)
        kb = (f.view(np.uint32) >> 16).astype(np.uint16)
        vb = ((f * 0.5).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    caches = []
    for chunks in ([T], [1] * T, [5, 100, 1, 63, 64, 100]):
        c = oracle_mod.OracleCache(B, H, D, T, kbits, vbits, 32, R, dtype)
        p = 0
        for n in chunks:
            c.append(kb[:, :, p:p + n], vb[:, :, p:p + n])
            p += n
        assert p == T
        caches.append(c)
    ref = caches[0].arrays()
    assert (caches[0].n_quant, caches[0].n_resid) == (T - ((T - 1) % R + 1), (T - 1) % R + 1)
    for c in caches[1:]:
        assert (c.n_quant, c.n_resid) == (caches[0].n_quant, caches[0].n_resid)
        for name, arr in c.arrays().items():
            if name.endswith("resid"):
                r = c.n_resid
                arr = arr.reshape(B, H, R, D)[:, :, :r]
                want = ref[name].reshape(B, H, R, D)[:, :, :r]
            else:
                want = ref[name]
            assert np.array_equal(arr, want), name


def test_capacity_error_leaves_state(oracle_mod):
    rng = np.random.default_rng(9)
    c = oracle_mod.OracleCache(1, 1, 32, 40, 2, 2, 32, 32)
    kb = _random_bits(rng, (1, 1, 41, 32))
    c.append(kb[:, :, :30], kb[:, :, :30])
    with pytest.raises(OverflowError):
        c.append(kb[:, :, 30:41], kb[:, :, 30:41])
    assert (c.n_quant, c.n_resid) == (0, 30)
    c.append(kb[:, :, 30:40], kb[:, :, 30:40])
    assert (c.n_quant, c.n_resid) == (32, 8)


def test_grid_inputs_dequantize_exactly(oracle_mod):
    # Grid-exact data: every packed key decodes to its input.
    B, H, D, T, R = 1, 2, 64, 129, 64
    K, V = grid_kv(B, H, T, D, seed=3)
    c = oracle_mod.OracleCache(B, H, D, T, 2, 2, 32, R)
    c.append(to_bits(K, "f16"), to_bits(V, "f16"))
    assert c.n_quant == 128
    for u in range(B * H):
        for t in (0, 5, 31, 32, 77, 127):
            for d in (0, 1, 15, 16, 33, 63):
                assert _key_hat(oracle_mod, c, u, t, d, D) == float(K[0, u, t, d])
