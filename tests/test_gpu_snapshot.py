"""A cache restored from a snapshot of its buffer (bytes copied back, the
lengths declared with kivi_cache_set_lengths) continues bit for bit like the
original: the decode step the benchmark repeats from a fixed state.  Also the
timing hook: events recorded around the decode kernel bracket a positive
time and leave the results unchanged."""
import numpy as np
import pytest
import torch

from kv_cache_bit_kivi_amd import kivi
from kv_cache_bit_kivi_amd.inputs import make_layer, small

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("gq,ragged", [(4, False), (1, True), (8, False)])
def test_restore_and_repeat_step(gq, ragged):
    B, H, T = 3, 2, 640
    w = small("snap", B, H, H * gq, T, 2, 2, torch.float16)
    x = make_layer(w, seed=gq, n_new=4, device=DEV)
    lens = [640, 500, 257] if ragged else [T] * B
    cache = kivi.KiviCache(B, H, T + 8, device=DEV)
    kp, vp = x.k[:, :, :T].contiguous(), x.v[:, :, :T].contiguous()
    if ragged:
        cache.append_varlen(kp, vp, lens)
    else:
        cache.append(kp, vp)
    nq, nr = cache.lengths()
    snap = cache.buffer.clone()
    scale = 1.0 / np.sqrt(128)
    outs = []
    for t in range(4):
        kn, vn = x.k[:, :, T + t:T + t + 1].contiguous(), x.v[:, :, T + t:T + t + 1].contiguous()
        outs.append(cache.append_decode_attn(kn, vn, x.q, scale).clone())
    after = cache.buffer.clone()
    lengths_after = cache.lengths()
    # restore the snapshot and repeat the same four steps
    cache.buffer.copy_(snap)
    cache.set_lengths(nq, nr)
    assert cache.lengths() == (nq, nr)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    kivi.kivi_set_timing_events(cache.handle, ev[0].cuda_event, ev[1].cuda_event)
    for t in range(4):
        kn, vn = x.k[:, :, T + t:T + t + 1].contiguous(), x.v[:, :, T + t:T + t + 1].contiguous()
        got = cache.append_decode_attn(kn, vn, x.q, scale)
        assert torch.equal(got, outs[t]), t
    kivi.kivi_set_timing_events(cache.handle, 0, 0)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0.0
    assert cache.lengths() == lengths_after
    assert torch.equal(cache.buffer, after)
    with pytest.raises(kivi.KiviError) as e:
        cache.set_lengths([100] * B, [1] * B)  # not a multiple of R
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    assert cache.lengths() == lengths_after


def test_stream_read_probe_runs():
    n = 64 << 20
    src = torch.ones(n, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(64 * 256, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    kivi.kivi_stream_read_probe(src.data_ptr(), n, sink.data_ptr(), sink.numel() * 4, 64, s)
    torch.cuda.synchronize()
    # XOR of 0x01010101 words: each thread read a whole number of 16-byte
    # pieces (4 words), so every thread's XOR is 0
    assert int(sink.abs().sum()) == 0
    with pytest.raises(kivi.KiviError):
        kivi.kivi_stream_read_probe(src.data_ptr(), n, sink.data_ptr(), 16, 64, s)
