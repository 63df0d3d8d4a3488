"""Binary64 attention quantities of an oracle cache, for tolerances.

Test infrastructure: unpacks the oracle's packed arrays (the canonical
layout of include/kivi.h) into dequantized keys and values, and evaluates
decode attention in binary64 together with the magnitudes that bound the
error of any binary32 evaluation of it:
  logit sums  L_t = lam * sum_d |q_d k^_td|     (lam = softmax_scale log2 e)
  spread      D_j = sum_t w_t |v^_tj - out_j|   (w: softmax weights)
  value sums  V_j = sum_t w_t |v^_tj|
A logit error e_t moves out_j by at most (2^(2 max e_t) - 1) D_j, and the
value sums bound the rounding of the weighted sum itself."""
import numpy as np


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _codes(words, bits, n):
    """Codes 0..n-1 of each word (split-half order), shape words.shape + (n,)."""
    i = np.arange(n)
    shift = bits * (i // 2) + 16 * (i % 2)
    return (words[..., None] >> shift) & ((1 << bits) - 1)


def dequantized(ref, bf16=False, magnitudes=False):
    """K^, V^ of every unit as float64 [U][T][D] (packed tokens, then the
    window), T = n_quant + n_resid.  With magnitudes=True also the sizes of
    the terms a folded evaluation sums for each key, c*S + |Z| for packed
    tokens and |k| for window tokens (same shape)."""
    U = ref.B * ref.H
    D, G, R = ref.D, ref.G, ref.R
    nq, nr, cap, nb = ref.n_quant, ref.n_resid, ref.capacity, ref.num_blocks
    kb, vb = ref.k_bits, ref.v_bits
    a = ref.arrays()
    kc = a["k_codes"].reshape(U, cap, D * kb // 32)
    kcodes = _codes(kc, kb, 32 // kb).reshape(U, cap, D)[:, :nq]
    ks = _f16(a["k_scale"]).reshape(U, nb, D)
    kz = _f16(a["k_zero"]).reshape(U, nb, D)
    blk = np.arange(nq) // G
    K = kcodes * ks[:, blk] + kz[:, blk]
    vc = a["v_codes"].reshape(U, nb, G * vb // 32, D)
    vcodes = _codes(vc, vb, 32 // vb)  # [U][nb][w][D][Pv]
    vcodes = vcodes.transpose(0, 1, 2, 4, 3).reshape(U, nb * G, D)[:, :nq]
    vs = _f16(a["v_scale"]).reshape(U, nb, D // G, G).transpose(0, 1, 3, 2).reshape(U, nb * G, D // G)[:, :nq]
    vz = _f16(a["v_zero"]).reshape(U, nb, D // G, G).transpose(0, 1, 3, 2).reshape(U, nb * G, D // G)[:, :nq]
    m = np.arange(D) // G
    V = vcodes * vs[:, :, m] + vz[:, :, m]
    conv = _bf16 if bf16 else _f16
    kr = conv(a["k_resid"]).reshape(U, R, D)[:, :nr]
    vr = conv(a["v_resid"]).reshape(U, R, D)[:, :nr]
    Kh, Vh = np.concatenate([K, kr], 1), np.concatenate([V, vr], 1)
    if not magnitudes:
        return Kh, Vh
    Km = np.concatenate([kcodes * ks[:, blk] + np.abs(kz[:, blk]), np.abs(kr)], 1)
    return Kh, Vh, Km


def attention(ref, q_bits, softmax_scale, bf16=False):
    """Binary64 attention of every query head and the error magnitudes:
    (out [B][Hq][D], L_max [B][Hq], D [B][Hq][D], V [B][Hq][D]).  L_max is
    the largest logit sum over the tokens, lam * sum_d |q_d| (c S + |Z|) for
    packed tokens (the magnitudes the folded products add up) and
    lam * sum_d |q_d k_d| for window tokens."""
    K, V, Km = dequantized(ref, bf16, magnitudes=True)
    conv = _bf16 if bf16 else _f16
    q = conv(q_bits)
    B, Hq, D = q.shape
    H = ref.H
    gq = Hq // H
    lam = softmax_scale / np.log(2.0)
    out = np.zeros((B, Hq, D))
    lmax = np.zeros((B, Hq))
    spread = np.zeros((B, Hq, D))
    vsum = np.zeros((B, Hq, D))
    for b in range(B):
        for j in range(Hq):
            u = b * H + j // gq
            s = lam * (K[u] @ q[b, j])
            w = np.exp2(s - s.max())
            w /= w.sum()
            o = w @ V[u]
            out[b, j] = o
            lmax[b, j] = lam * np.max(Km[u] @ np.abs(q[b, j]))
            spread[b, j] = w @ np.abs(V[u] - o)
            vsum[b, j] = w @ np.abs(V[u])
    return out, lmax, spread, vsum


KAPPA = 2.0 ** -16  # 256 units of binary32 rounding (u = 2^-24)


def fp32_allowance(lmax, spread, vsum):
    """Rounding allowance of a binary32 evaluation of decode attention, per
    output element: KAPPA times (L_max * D_j + V_j).

    A logit summed from terms whose magnitudes add up to L, with n roundings
    of binary32 partial sums, is off by at most about n u L, and a logit error
    e moves out_j by at most (2^(2e) - 1) D_j ~ 1.4 e D_j.  Each score of the
    matrix-core decode adds 8 x 32 = 256 products into one binary32
    accumulator (4 blocks of 32 channels, hi and lo operands) besides about
    20 roundings of the zero-point dot products, cross-lane sums and scaling,
    so KAPPA = 256 u is the deterministic bound of that accumulation; the
    errors measured on the GPU stay below 40% of it.  The V_j term covers the
    rounding of the weighted value sum and of out itself."""
    return KAPPA * (np.asarray(lmax)[..., None] * spread + vsum)


def fp32_attention(K, V, q, softmax_scale, H):
    """A plain binary32 evaluation of decode attention over dequantized K, V
    (float64 [U][T][D], rounded to binary32): sequential dot products over the
    channels, binary32 softmax and weighted sum.  q: float [B][Hq][D]."""
    K32, V32 = K.astype(np.float32), V.astype(np.float32)
    B, Hq, D = q.shape
    gq = Hq // H
    lam = np.float32(softmax_scale / np.log(2.0))
    out = np.zeros((B, Hq, D), np.float32)
    for b in range(B):
        for j in range(Hq):
            u = b * H + j // gq
            qq = np.asarray(q[b, j], np.float32)
            s = np.zeros(K32.shape[1], np.float32)
            for d in range(D):
                s = (s + qq[d] * K32[u, :, d]).astype(np.float32)
            s = (s * lam).astype(np.float32)
            w = np.exp2(s - s.max()).astype(np.float32)
            l, o = np.float32(0.0), np.zeros(D, np.float32)
            for t in range(w.size):
                l = np.float32(l + w[t])
                o = (o + w[t] * V32[u, t]).astype(np.float32)
            out[b, j] = o / l
    return out
