"""Sequences of different lengths in one batch: per-sequence appends
(kivi_append_varlen), single-token appends that flush each sequence's window
at its own time, resets of single sequences, and decode attention over
sequences of different lengths.  Every sequence is compared with an oracle
cache of its own (packed arrays bit for bit, attention within 2e-3); a
sequence without tokens must give zeros.

Sizes cross the group, window and launch-chunk boundaries (32 sequences per
pack launch, 64 per decode launch) and include empty sequences."""
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

#        name           B   H  Hq  kb vb dtype           R    prefill lengths                     steps
CASES = [("mha_mixed",   6,  2, 2,  2, 2, torch.float16,  128, [0, 1, 33, 128, 129, 300],          140),
         ("gq4_bf16_4b", 5,  2, 8,  4, 4, torch.bfloat16, 32,  [31, 32, 64, 95, 7],                40),
         ("gq8",         4,  1, 8,  2, 4, torch.float16,  128, [5, 260, 0, 128],                   20),
         ("k4v2_gq2",    3,  2, 4,  4, 2, torch.float16,  64,  [65, 0, 190],                       70),
         ("chunks",      70, 1, 4,  2, 2, torch.float16,  32,  [(7 * i) % 101 for i in range(70)], 3)]


class Harness:
    def __init__(self, case, seed=3):
        name, B, H, Hq, kb, vb, dt, R, lens, steps = case
        self.case = case
        self.B, self.H, self.Hq = B, H, Hq
        self.max_tokens = max(lens) + steps + 400
        w = small(name, B, H, Hq, self.max_tokens, kb, vb, dt, residual_length=R)
        self.w = w
        x = make_layer(w, seed=seed, n_new=0)
        self.k, self.v, self.q = x.k, x.v, x.q.contiguous()
        self.kb16, self.vb16, self.qb16 = bits16(x.k), bits16(x.v), bits16(x.q)
        self.cache = kivi.KiviCache(B, H, self.max_tokens, k_bits=kb, v_bits=vb, residual_length=R,
                                    dtype=dt, device=DEV)
        dtc = oracle.BF16 if dt == torch.bfloat16 else oracle.F16
        self.new_oracle = lambda: oracle.OracleCache(1, H, w.head_dim, self.max_tokens, kb, vb,
                                                     w.group_size, R, dtc)
        self.refs = [self.new_oracle() for _ in range(B)]
        self.used = [0] * B  # tokens of the input consumed per sequence
        self.qd = self.q.to(DEV)

    def append_varlen(self, lens):
        n_max = max(max(lens), 1)
        ks = torch.zeros(self.B, self.H, n_max, 128, dtype=self.k.dtype)
        vs = torch.zeros_like(ks)
        for b, n in enumerate(lens):
            if n:
                u = self.used[b]
                ks[b, :, :n] = self.k[b, :, u:u + n]
                vs[b, :, :n] = self.v[b, :, u:u + n]
                self.refs[b].append(self.kb16[b:b + 1, :, u:u + n], self.vb16[b:b + 1, :, u:u + n])
                self.used[b] += n
        self.cache.append_varlen(ks.to(DEV), vs.to(DEV), lens)

    def append_one(self):
        ks = torch.stack([self.k[b, :, self.used[b]] for b in range(self.B)])[:, :, None].contiguous()
        vs = torch.stack([self.v[b, :, self.used[b]] for b in range(self.B)])[:, :, None].contiguous()
        for b in range(self.B):
            u = self.used[b]
            self.refs[b].append(self.kb16[b:b + 1, :, u:u + 1], self.vb16[b:b + 1, :, u:u + 1])
            self.used[b] += 1
        self.cache.append(ks.to(DEV), vs.to(DEV))

    def reset(self, seqs):
        self.cache.reset_sequences(seqs)
        for b in seqs:
            self.refs[b] = self.new_oracle()

    def check_lengths(self):
        nq, nr = self.cache.lengths()
        want = [(r.n_quant, r.n_resid) for r in self.refs]
        assert list(zip(nq, nr)) == want, (list(zip(nq, nr)), want)

    def check_arrays(self):
        torch.cuda.synchronize()
        got = gpu_arrays(self.cache)
        H = self.H
        for b, ref in enumerate(self.refs):
            mine = {k: a[b * H:(b + 1) * H] for k, a in got.items()}
            assert_cache_equal(mine, oracle_arrays(ref), ref.n_quant, ref.n_resid, ref.capacity,
                               ref.num_blocks)

    def check_decode(self, tag):
        scale = 1.0 / np.sqrt(128)
        out = self.cache.decode_attn(self.qd, scale).cpu().numpy().astype(np.float64)
        gq = self.Hq // self.H
        worst = 0.0
        for b, ref in enumerate(self.refs):
            if ref.n_quant + ref.n_resid == 0:
                assert np.all(out[b] == 0.0), f"{tag}: empty sequence {b} must give zeros"
                continue
            o_ref = ref.decode_attn(self.qb16[b:b + 1], scale)
            err = float(np.abs(out[b:b + 1] - o_ref).max())
            worst = max(worst, err)
            assert err <= TOL, (f"{tag}: sequence {b} (n_quant {ref.n_quant}, n_resid {ref.n_resid}, "
                                f"gq {gq}): {err:.3e}")
        return worst


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_prefill_steps_reset(case):
    name, B, H, Hq, kb, vb, dt, R, lens, steps = case
    print(f"varlen {name}: B={B} H={H} Hq={Hq} bits={kb}/{vb} R={R} prefill {lens[:8]}...", flush=True)
    h = Harness(case)
    h.append_varlen(lens)
    h.check_lengths()
    h.check_arrays()
    worst = h.check_decode("after prefill")
    # single-token appends: each sequence's window fills and flushes at its own step
    for t in range(steps):
        h.append_one()
        h.check_lengths()
        worst = max(worst, h.check_decode(f"step {t}"))
    h.check_arrays()
    # a finished request's slot refilled, then a chunked append into every sequence
    h.reset([1])
    h.check_lengths()
    h.append_varlen([0] * B if B < 2 else [150 if b == 1 else 0 for b in range(B)])
    h.check_lengths()
    worst = max(worst, h.check_decode("after reset"))
    h.append_varlen([(37 * b + 5) % (R + 40) for b in range(B)])
    h.check_lengths()
    h.check_arrays()
    worst = max(worst, h.check_decode("after chunked append"))
    print(f"varlen {name}: worst attention error {worst:.2e}", flush=True)


def test_varlen_uniform_equals_append():
    # equal per-sequence counts take the uniform path: same state as kivi_append
    case = ("uniform", 3, 2, 4, 2, 2, torch.float16, 128, [200, 200, 200], 0)
    h = Harness(case)
    h.append_varlen([200, 200, 200])
    v = h.cache.view()
    assert (v.n_quant, v.n_resid) == (128, 72)
    h.check_lengths()
    h.check_arrays()
    h.check_decode("uniform")


def test_varlen_errors_leave_state():
    case = ("errors", 2, 1, 1, 2, 2, torch.float16, 32, [10, 20], 0)
    h = Harness(case)
    h.append_varlen([10, 20])
    k = torch.zeros(2, 1, 4, 128, dtype=torch.float16, device=DEV)
    with pytest.raises(kivi.KiviError) as e:
        h.cache.append_varlen(k, k, [5, 1])  # 5 > n_max
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    big = torch.zeros(2, 1, h.max_tokens, 128, dtype=torch.float16, device=DEV)
    with pytest.raises(kivi.KiviError) as e:
        h.cache.append_varlen(big, big, [0, h.max_tokens])
    assert e.value.status == kivi.KIVI_ERR_CAPACITY
    with pytest.raises(kivi.KiviError) as e:
        h.cache.reset_sequences([2])
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    h.check_lengths()
    h.check_arrays()
    # every sequence empty: decode has nothing to attend to
    h.reset([0, 1])
    with pytest.raises(kivi.KiviError) as e:
        h.cache.decode_attn(h.qd, 0.1)
    assert e.value.status == kivi.KIVI_ERR_EMPTY
