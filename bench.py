"""Benchmark of the KIVI hot path on one MI355X.

One step = one decode step of every layer of the workload, from the state
the prefix leaves (n_quant = T - R packed tokens, n_resid = R window tokens):
  1. the full window is packed before the new token enters it (flush, one
     pack launch);
  2. the token is appended and split-K decode attention runs over the packed
     cache plus the window in the same launch (the decode kernel), then the
     cross-split merge (kivi_append_decode_attn: the flush, decode and merge
     launches);
  3. the lengths return to (T - R, R) on the host (kivi_cache_set_lengths).
     The new token is a copy of window slot 0's, so the flush packs the same
     window every step and the step's work and results repeat exactly.
The prefix pack (quantize + bit-pack T tokens per unit, the bulk prefill) is
timed on its own after the timed steps, as the "pack" phase.

Default workload: Llama-3-8B-shaped GQA layer, batch 32, 32 query / 8 kv
heads, T = 32768, 2-bit, G = 32, R = 128, fp16 (--workload c2).  `value` is
the step's algorithmic bytes (window read, codes + scale/zero written by the
flush, the token read and written, codes + scale/zero + window + q read by
the decode, out written by the merge) divided by the step time, in GB/s.
The roofline describes the decode kernel: its algorithmic bytes per launch
over its mean launch time, from HIP events recorded by the library right
around the kernel on the stream it runs on (kivi_set_timing_events).

Prints one JSON line.  Inputs are resident in HBM before timing starts.
"""
import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "fused 2-bit dequant decode-attn effective HBM GB/s + % peak; pack GB/s"


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence
    through the HIP runtime torch has loaded: a default event performs a
    system-scope fence when it is recorded (a write-back and invalidation of
    the caches), which delays the launches around each marker and lengthens
    the interval it measures."""
    _hip = None

    def __init__(self):
        if TimingEvent._hip is None:
            # the runtime torch has already loaded (found by its soname)
            hip = None
            for name in ("libamdhip64.so.7", "libamdhip64.so"):
                try:
                    hip = ctypes.CDLL(name)
                    break
                except OSError:
                    continue
            if hip is None:
                raise RuntimeError("HIP runtime library not found")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            TimingEvent._hip = hip
        self.handle = ctypes.c_void_p()
        if self._hip.hipEventCreateWithFlags(ctypes.byref(self.handle), 0x20000000) != 0:  # DisableSystemFence
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._hip.hipEventRecord(self.handle, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both completed)."""
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="c2", choices=["c0", "c1", "c2", "c3", "c4"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="untimed decode steps before the warm-up for this long (ms): from idle, the decode "
                        "runs up to a third slower for the first ~30 ms of sustained load")
    p.add_argument("--phase-every", type=int, default=2,
                   help="bracket the launches with HIP events on every N-th timed step")
    p.add_argument("--pack-iters", type=int, default=20, help="timed prefix packs (all layers each)")
    p.add_argument("--cold-iters", type=int, default=50,
                   help="decode-only launches with the last-level cache scrubbed before each")
    p.add_argument("--probe-iters", type=int, default=20, help="streaming-read probe launches")
    p.add_argument("--splits", type=int, default=0,
                   help="force this many token splits per sequence (0: the library's planner)")
    p.add_argument("--ragged", action="store_true",
                   help="sequences of different lengths: sequence b's prefix has T_b tokens, "
                        "drawn uniformly from [T/2, T] (seed 0)")
    p.add_argument("--q-heads", type=int, default=0,
                   help="query heads per sequence instead of the workload's (e.g. 64 on c2: the "
                        "64q/8kv shape of 70B-class models, 8 query heads per kv head)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 1 GiB device copy first (counter calibration "
                        "for profiler runs)")
    return p.parse_args()


# ------------------------------------------------------------ byte accounting

def algorithmic_bytes(w, lens=None):
    """Bytes the method must move per layer, per phase (whole batch), with
    every sequence's prefix T tokens long or sequence b's lens[b] long.
    Codes: bits/8 per element; scale + zero: 4 bytes per group of G.
      pack   : the prefix pack (read T tokens of K and V, write codes,
               scale/zero and the last r tokens into the window)
      flush  : a full window packed (read R tokens, write codes, scale/zero)
      decode : the decode kernel (the token read and written into the
               window; codes, scale/zero and window tokens read; q read)
      merge  : the merge kernel (out written, fp32; partials excluded)"""
    D, G, R = w.head_dim, w.group_size, w.residual_length
    e = 2  # fp16 / bf16
    codes = lambda n: n * D * (w.k_bits + w.v_bits) // 8
    meta = lambda n: (n // G) * D * 4 + n * (D // G) * 4
    tot = {"pack": 0, "flush": 0, "decode": 0, "merge": 0}
    for T in (lens if lens is not None else [w.tokens] * w.batch):
        r = (T - 1) % R + 1
        nq = T - r
        tot["pack"] += 2 * T * D * e + codes(nq) + meta(nq) + 2 * r * D * e
        if r == R:  # the full window is packed before the token enters
            tot["flush"] += 2 * R * D * e + codes(R) + meta(R)
            nq2, r2 = nq + R, 1
        else:
            nq2, r2 = nq, r + 1
        token = 2 * (2 * D * e)  # the appended token, read and written into the window
        tot["decode"] += token + codes(nq2) + meta(nq2) + 2 * r2 * D * e + w.gq * D * e
        tot["merge"] += w.gq * D * 4
    return {k: w.kv_heads * v for k, v in tot.items()}


def step_bytes(ab):
    """Bytes of one decode step (flush + decode + merge) of one layer."""
    return ab["flush"] + ab["decode"] + ab["merge"]


def ragged_lengths(w):
    """Prefix length of each sequence for --ragged: uniform in [T/2, T], seed 0."""
    import numpy as np
    return [int(x) for x in np.random.default_rng(0).integers(w.tokens // 2, w.tokens + 1, w.batch)]


def decode_kernel(w):
    """Name and source of the split-K decode kernel (every head ratio)."""
    return "decode_mfma", "kivi_decode_mfma.hip"


def traffic_from_profile(kernel, workload, kernel_src):
    """HBM bytes per launch of `kernel` on `workload` measured with rocprofv3
    counters (profiles/<kernel>_<workload>_counters.txt), if they were taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = open(kernel_src, "rb").read()
    if kv.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stats(samples_s):
    """mean, median, p10, p90 (microseconds) and count of durations in seconds."""
    import numpy as np
    a = np.asarray(samples_s) * 1e6
    return {"us_mean": float(a.mean()), "us_median": float(np.median(a)),
            "us_p10": float(np.percentile(a, 10)), "us_p90": float(np.percentile(a, 90)),
            "samples": int(a.size)}


# ---------------------------------------------------------------- GPU run

def run(args):
    import numpy as np
    import torch

    from kv_cache_bit_kivi_amd import kivi
    from kv_cache_bit_kivi_amd.inputs import WORKLOADS, make_layer

    w = WORKLOADS[args.workload]
    if args.q_heads:
        if args.q_heads % w.kv_heads:
            raise SystemExit(f"--q-heads {args.q_heads} is not a multiple of {w.kv_heads} kv heads")
        w = dataclasses.replace(w, name=f"{w.name}gq{args.q_heads // w.kv_heads}", q_heads=args.q_heads,
                                description=f"{w.description}, with {args.q_heads} query heads")
    dev = torch.device("cuda:0")
    T, R, B = w.tokens, w.residual_length, w.batch
    scale = 1.0 / np.sqrt(w.head_dim)
    lens = ragged_lengths(w) if args.ragged else [T] * B
    r0 = [(t - 1) % R + 1 for t in lens]  # window tokens of each prefix
    q0 = [t - r for t, r in zip(lens, r0)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    layers = []
    for layer in range(w.layers):
        x = make_layer(w, seed=layer, device=dev, n_new=0)
        cache = kivi.KiviCache(B, w.kv_heads, T + 1, k_bits=w.k_bits, v_bits=w.v_bits,
                               group_size=w.group_size, residual_length=w.residual_length,
                               dtype=w.dtype, device=dev)
        kp, vp = x.k.contiguous(), x.v.contiguous()
        if args.ragged:
            cache.append_varlen(kp, vp, lens)
        else:
            cache.append(kp, vp)
        # the decode token of sequence b: a copy of its window slot 0 (token
        # T_b - r_b), so that the flush packs the same window every step
        idx = torch.tensor(q0, device=dev)
        kn = kp[torch.arange(B, device=dev), :, idx].contiguous()  # [B][H][D]
        vn = vp[torch.arange(B, device=dev), :, idx].contiguous()
        L = dict(cache=cache, kp=kp, vp=vp, kn=kn, vn=vn, q=x.q.contiguous(),
                 out=torch.empty(B, w.q_heads, w.head_dim, dtype=torch.float32, device=dev))
        if args.splits:
            cache.set_splits(args.splits)
        ws = cache.workspace(w.q_heads)  # allocated before timing
        # the C-ABI calls of one step with their arguments resolved once (the
        # checks of the KiviCache convenience methods cost the host more than
        # a small step costs the GPU)
        L["lengths"] = ((ctypes.c_int32 * B)(*q0), (ctypes.c_int32 * B)(*r0))
        L["decode"] = (cache.handle, kn.data_ptr(), vn.data_ptr(), L["q"].data_ptr(), w.q_heads,
                       ctypes.c_float(scale), L["out"].data_ptr(), kivi.KIVI_F32, ws.data_ptr(),
                       ws.numel(), ctypes.c_void_p(sp))
        layers.append(L)
        del x
    # events of the marked steps: [0] before the call, [1] and [2] recorded by
    # the library right around the decode kernel, [3] after the call
    every = max(1, args.phase_every)
    marked = list(range(0, args.steps, every))[:256]
    events = {k: [[TimingEvent() for _ in range(4)] for _ in layers] for k in marked}
    for evs in events.values():
        for ev in evs:
            for e in ev:
                e.record(sp)
    torch.cuda.synchronize()
    lib = kivi.lib
    new_tok = [(ctypes.c_void_p(L["kn"].data_ptr()), ctypes.c_void_p(L["vn"].data_ptr())) for L in layers]
    null = ctypes.c_void_p(0)

    def step(evs=None):
        # one decode step of every layer
        for i, L in enumerate(layers):
            h = L["cache"].handle
            if lib.kivi_cache_set_lengths(h, *L["lengths"]) != kivi.KIVI_OK:
                raise kivi.KiviError(kivi.KIVI_ERR_INVALID_ARG, kivi.last_error_message())
            if evs is not None:
                ev = evs[i]
                lib.kivi_set_timing_events(h, ev[1].handle, ev[2].handle)
                ev[0].record(sp)
            a = L["decode"]
            st = lib.kivi_append_decode_attn(a[0], new_tok[i][0], new_tok[i][1], ctypes.c_void_p(a[3]), a[4],
                                             a[5], ctypes.c_void_p(a[6]), a[7], ctypes.c_void_p(a[8]), a[9],
                                             a[10])
            if st != kivi.KIVI_OK:
                raise kivi.KiviError(st, kivi.last_error_message())
            if evs is not None:
                ev[3].record(sp)
                lib.kivi_set_timing_events(h, null, null)

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Settle: from idle, MI355X runs the first ~30 ms of sustained load
    # slower (a kernel trace of the c2 decode: 155-171 us at the start, 208 us
    # after 3-7 ms, 163 us at 19 ms, 145-158 us from 40 ms on), so untimed
    # steps run until the clocks have settled, then the W warm-up steps and
    # the K timed ones.
    settle_steps, t_settle = 0, time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_settle:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        settle_steps += 5
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Each event record is a stream marker that the next launch waits for, so
    # the launches are bracketed on every `phase_every`-th timed step only (at
    # most 256 of them); the other steps run back to back as a serving loop
    # would.  `value` counts every timed step, marked or not.
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events.get(k))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    phase = {"flush": [], "decode": [], "merge": []}
    for evs in events.values():
        for ev in evs:
            phase["flush"].append(ev[0].elapsed_time(ev[1]) * 1e-3)
            phase["decode"].append(ev[1].elapsed_time(ev[2]) * 1e-3)
            phase["merge"].append(ev[2].elapsed_time(ev[3]) * 1e-3)

    # decode alone (the state after the step, kivi_decode_attn) with the
    # 256 MB last-level cache scrubbed before each launch pair
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    L0 = layers[0]
    c0 = L0["cache"]
    for _ in range(args.cold_iters):
        scrub.fill_(1)
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(sp)
        c0.decode_attn(L0["q"], scale, out=L0["out"])
        e1.record(sp)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e-3)

    # streaming-read probe: 4 GiB read once per launch
    probe = []
    nbytes = 4 << 30
    src = scrub.new_empty(nbytes)
    src.fill_(3)
    wgs = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
    for _ in range(args.probe_iters):
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(sp)
        kivi.kivi_stream_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), sink.numel() * 4, wgs, sp)
        e1.record(sp)
        torch.cuda.synchronize()
        probe.append(e0.elapsed_time(e1) * 1e-3)
    del src, sink, scrub

    # the prefix pack (bulk prefill), every layer per iteration
    pack = []
    for _ in range(args.pack_iters):
        for L in layers:
            e0, e1 = TimingEvent(), TimingEvent()
            c = L["cache"]
            c.reset()
            e0.record(sp)
            if args.ragged:
                c.append_varlen(L["kp"], L["vp"], lens)
            else:
                kivi.kivi_append(c.handle, L["kp"].data_ptr(), L["vp"].data_ptr(), T, sp)
            e1.record(sp)
            torch.cuda.synchronize()
            pack.append(e0.elapsed_time(e1) * 1e-3)
    return w, wall, phase, cold, probe, nbytes, pack, layers, (lens if args.ragged else None), settle_steps


def cpu_baseline(w, layers, lens=None):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    decode step (token append, which packs the full window first, then decode
    attention for every query head) on one batch row of the first layer at a
    time, cycling through the rows; each row's oracle cache is first filled
    with its prefix (untimed).  Stops after about ten seconds of timed oracle
    work or 40 s in all."""
    import numpy as np

    import oracle
    from kv_cache_bit_kivi_amd.inputs import bits16

    L = layers[0]
    dt = oracle.BF16 if "bfloat" in str(w.dtype) else oracle.F16
    done, t, nbytes, t_all = 0, 0.0, 0, time.perf_counter()
    while t < 10.0 and time.perf_counter() - t_all < 40.0:
        r = done % w.batch
        rows = slice(r, r + 1)
        T = w.tokens if lens is None else lens[r]
        ref = oracle.OracleCache(1, w.kv_heads, w.head_dim, w.tokens + 1, w.k_bits, w.v_bits,
                                 w.group_size, w.residual_length, dt)
        ref.append(bits16(L["kp"][rows, :, :T]), bits16(L["vp"][rows, :, :T]))
        kn, vn = bits16(L["kn"][rows, :, None]), bits16(L["vn"][rows, :, None])
        q = bits16(L["q"][rows])
        t0 = time.perf_counter()
        ref.append(kn, vn)
        ref.decode_attn(q, 1.0 / np.sqrt(w.head_dim))
        t += time.perf_counter() - t0
        done += 1
        nbytes += step_bytes(algorithmic_bytes(w, [T]))
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} batch rows (all {w.kv_heads} kv heads each, cycling through the "
                      f"{w.batch} rows of layer 0), one decode step each (the token append that "
                      f"packs the full window, then decode attention for every query head; the "
                      f"prefix pack that builds each row's cache is not timed); {t:.1f} s of "
                      f"oracle time; host CPU: {cpu_model()}, {os.cpu_count()} logical CPUs visible"}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the KIVI hot path "
              "shards by (batch, kv head) with no exchange, so N GPUs run N independent "
              "copies of this single-GPU measurement", file=sys.stderr)
        sys.exit(2)
    import numpy as np

    w, wall, phase, cold, probe, probe_bytes, pack, layers, lens, settle_steps = run(args)
    ab = algorithmic_bytes(w, lens)
    kname, ksrc = decode_kernel(w)
    phases = {}
    for k, desc in (("flush", "window flush (pack kernel), before the decode kernel"),
                    ("decode", f"{kname}: token append + split-K attention"),
                    ("merge", "decode_merge: cross-split merge, out written")):
        s = stats(phase[k])
        g = ab[k] / (s["us_mean"] * 1e-6) / 1e9
        phases[k] = dict(bytes=ab[k], **s, gbps=g, frac=g / PEAK_GBPS, launch=desc)
    s = stats(pack)
    phases["pack"] = dict(bytes=ab["pack"], **s, gbps=ab["pack"] / (s["us_median"] * 1e-6) / 1e9,
                          frac=ab["pack"] / (s["us_median"] * 1e-6) / 1e9 / PEAK_GBPS,
                          launch="prefix pack (prefill): quantize + bit-pack T tokens, copy the window")
    # decode alone reads no new token: the token's 4 D e bytes per unit less
    dec_bytes = ab["decode"] + ab["merge"] - 4 * w.head_dim * 2 * w.kv_heads * w.batch
    s = stats(cold)
    phases["decode_cold_llc"] = dict(bytes=dec_bytes, **s,
                                     gbps=dec_bytes / (s["us_median"] * 1e-6) / 1e9,
                                     frac=dec_bytes / (s["us_median"] * 1e-6) / 1e9 / PEAK_GBPS,
                                     launch="kivi_decode_attn alone (decode kernel + merge), "
                                            "last-level cache scrubbed before each")
    s = stats(probe)
    probe_gbps = probe_bytes / (s["us_median"] * 1e-6) / 1e9
    phases["stream_read_probe"] = dict(bytes=probe_bytes, **s, gbps=probe_gbps, frac=probe_gbps / PEAK_GBPS,
                                       launch="kivi_stream_read_probe: 4 GiB read once, 16-byte loads")
    # the roofline of the decode kernel: algorithmic bytes per launch over the
    # mean launch duration measured by the library's events in the timed steps
    dec = phases["decode"]
    achieved = dec["gbps"]
    dec["frac_of_stream_read"] = achieved / probe_gbps
    traffic = None if lens is not None else traffic_from_profile(
        kname, w.name, os.path.join(ROOT, "kv_cache_bit_kivi_amd", "csrc", ksrc))
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, layers, lens)
    per_step = step_bytes(ab) * w.layers
    res = {
        "metric": METRIC,
        "value": per_step / wall / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "arithmetic": "decode: f16 matrix-core operands (hi + lo halves of q*S and p*S, codes as exact f16) "
                      "with f32 accumulation and f32 softmax; pack: binary32 quantizer",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.batch,
                   "kv_heads": w.kv_heads, "q_heads": w.q_heads, "head_dim": w.head_dim,
                   "tokens": w.tokens, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "group_size": w.group_size, "residual_length": w.residual_length,
                   "kv_dtype": str(w.dtype).replace("torch.", ""), "layers": w.layers,
                   "step": "per layer: window flush + token append + split-K decode + merge, "
                           "from (T - R packed, R window)",
                   "lengths": ("every sequence T" if lens is None else
                               f"per sequence uniform in [T/2, T], seed 0 (mean {np.mean(lens):.0f})")},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": ab["decode"], "us_per_launch": dec["us_mean"],
                     "frac_of_stream_read": achieved / probe_gbps},
        "cpu_baseline": cpu,
        "phases": phases,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
