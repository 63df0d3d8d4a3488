"""Benchmark of the KIVI hot path on one MI355X.

One step = one pass of the whole hot path over one layer's synthetic batch:
  1. bulk append of the T-token prefix: quantize + bit-pack every full
     window straight from the input, copy the last R tokens to the window
     (one pack launch);
  2. the full window is packed before the decode token enters it (flush,
     one launch);
  3. the decode step: the token is appended and split-K decode attention
     runs over the packed cache plus the window in the same launch, then the
     cross-split merge (kivi_append_decode_attn, two launches).
The cache is reset (host counters only) at the start of each step.

Default workload: Llama-2-7B-shaped MHA layer, batch 8, 32 heads, T = 4096,
2-bit, G = 32, R = 128, fp16 (--workload c1).  `value` is the step's
algorithmic bytes (fp16 K/V read by the pack, codes + scale/zero + window
written and read back, q, out) divided by the step time, in GB/s.

Prints one JSON line.  Inputs are resident in HBM before timing starts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "fused 2-bit dequant decode-attn effective HBM GB/s + % peak; pack GB/s"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c1", choices=["c0", "c1", "c2", "c3", "c4"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--phase-every", type=int, default=4,
                   help="bracket the phases with HIP events on every N-th timed step")
    p.add_argument("--cold-iters", type=int, default=20,
                   help="decode-only iterations with the last-level cache scrubbed")
    p.add_argument("--ragged", action="store_true",
                   help="sequences of different lengths: sequence b's prefix has T_b tokens, "
                        "drawn uniformly from [T/2, T] (seed 0)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 1 GiB device copy first (counter calibration "
                        "for profiler runs)")
    return p.parse_args()


# ------------------------------------------------------------ byte accounting

def algorithmic_bytes(w, lens=None):
    """Bytes the method must move per step, per phase (whole batch), with
    every sequence's prefix T tokens long or sequence b's lens[b] long.
    Codes: bits/8 per element; scale + zero: 4 bytes per group of G."""
    D, G, R = w.head_dim, w.group_size, w.residual_length
    e = 2  # fp16 / bf16
    codes = lambda n: n * D * (w.k_bits + w.v_bits) // 8
    meta = lambda n: (n // G) * D * 4 + n * (D // G) * 4
    tot = {"pack": 0, "flush": 0, "decode": 0}
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
        tot["decode"] += (token + codes(nq2) + meta(nq2) + 2 * r2 * D * e + w.gq * D * e
                          + w.gq * D * 4)
    return {k: w.kv_heads * v for k, v in tot.items()}


def ragged_lengths(w):
    """Prefix length of each sequence for --ragged: uniform in [T/2, T], seed 0."""
    import numpy as np
    return [int(x) for x in np.random.default_rng(0).integers(w.tokens // 2, w.tokens + 1, w.batch)]


# the kernel each phase's roofline describes, and the source it is built from
PHASE_KERNEL = {
    "pack": ("pack_kernel", "kivi_pack.hip", "one launch: quantize + bit-pack the prefix, "
             "copy the last window"),
    "flush": ("pack_kernel", "kivi_pack.hip", "one launch: window flush"),
    "decode": ("decode split + merge", None, "two launches: token append + split-K attention, "
               "merge"),
}


def decode_source(w):
    return "kivi_decode_mfma.hip" if w.gq in (1, 2, 4) else "kivi_decode.hip"


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


# ---------------------------------------------------------------- GPU run

def run(args):
    import numpy as np
    import torch

    from kv_cache_bit_kivi_amd import kivi
    from kv_cache_bit_kivi_amd.inputs import WORKLOADS, make_layer

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    T = w.tokens
    scale = 1.0 / np.sqrt(w.head_dim)
    lens = ragged_lengths(w) if args.ragged else None
    layers = []
    for layer in range(w.layers):
        x = make_layer(w, seed=layer, device=dev, n_new=1)
        layers.append(dict(
            kp=x.k[:, :, :T].contiguous(), vp=x.v[:, :, :T].contiguous(),
            kn=x.k[:, :, T:].contiguous(), vn=x.v[:, :, T:].contiguous(), q=x.q,
            cache=kivi.KiviCache(w.batch, w.kv_heads, T + 1, k_bits=w.k_bits, v_bits=w.v_bits,
                                 group_size=w.group_size, residual_length=w.residual_length,
                                 dtype=w.dtype, device=dev),
            out=torch.empty(w.batch, w.q_heads, w.head_dim, dtype=torch.float32, device=dev)))
        del x
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    for L in layers:
        c = L["cache"]
        ws = c.workspace(w.q_heads)  # allocated before timing
        # the C-ABI calls of one step with their arguments resolved once: the
        # step then costs the host a few microseconds per call (the checks
        # of the KiviCache convenience methods take longer than a c1 step on
        # the GPU)
        L["append"] = (c.handle, L["kp"].data_ptr(), L["vp"].data_ptr(), T, sp)
        L["decode"] = (c.handle, L["kn"].data_ptr(), L["vn"].data_ptr(), L["q"].data_ptr(),
                       w.q_heads, float(scale), L["out"].data_ptr(), kivi.KIVI_F32,
                       ws.data_ptr(), ws.numel(), sp)
    torch.cuda.synchronize()

    def step(ev=None):
        # one pass of the hot path over every layer, phase by phase: the prefix
        # of every layer packed, then every layer's decode token appended, then
        # decode attention for every layer.  ev: four HIP events bracketing the
        # three phase groups, recorded on the stream every kernel is launched on.
        rec = (lambda n: ev[n].record(stream)) if ev is not None else (lambda n: None)
        rec(0)
        for L in layers:
            kivi.kivi_cache_reset(L["cache"].handle)
            if lens is None:
                kivi.kivi_append(*L["append"])
            else:  # sequence b takes the first lens[b] tokens of the prefix
                L["cache"].append_varlen(L["kp"], L["vp"], lens, stream=stream)
        rec(1)
        for L in layers:
            kivi.kivi_flush_residual(L["cache"].handle, sp)
        rec(2)
        for L in layers:
            kivi.kivi_append_decode_attn(*L["decode"])
        rec(3)

    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Each event record is a marker that the next launch waits for (about
    # 6.5 us between kernels, against no gap between two launches of one
    # call), so the phases are bracketed on every `phase_every`-th timed step
    # only; the other steps run as a serving loop would, without markers.
    # `value` counts every timed step, marked or not.
    marked = list(range(0, args.steps, max(1, args.phase_every)))
    events = {k: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for k in marked}
    # timed region: exactly `steps` steps between two synchronizations
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events.get(k))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps

    # per step, the average duration of one layer's launches of each phase
    phase = {"pack": [], "flush": [], "decode": []}
    n = len(layers)
    for ev in events.values():
        phase["pack"].append(ev[0].elapsed_time(ev[1]) * 1e-3 / n)
        phase["flush"].append(ev[1].elapsed_time(ev[2]) * 1e-3 / n)
        phase["decode"].append(ev[2].elapsed_time(ev[3]) * 1e-3 / n)

    # decode alone with the 256 MB last-level cache scrubbed before each call
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    L0 = layers[0]
    for _ in range(args.cold_iters):
        scrub.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L0["cache"].decode_attn(L0["q"], scale, out=L0["out"])
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e-3)
    del scrub
    return w, wall, phase, cold, layers, lens


def cpu_baseline(w, layers, lens=None):
    """The oracle, as it stands, on a bounded sample of the same workload: one
    step (prefix pack, decode-token append, decode attention for every query
    head) on one batch row of the first layer at a time (row b's prefix cut to
    lens[b] tokens when given), cycling through the rows until about ten
    seconds of CPU work are done."""
    import numpy as np

    import oracle
    from kv_cache_bit_kivi_amd.inputs import bits16

    L = layers[0]
    dt = oracle.BF16 if "bfloat" in str(w.dtype) else oracle.F16
    done, t, nbytes = 0, 0.0, 0
    while t < 10.0:
        r = done % w.batch
        rows = slice(r, r + 1)
        T = w.tokens if lens is None else lens[r]
        k, v = bits16(L["kp"][rows, :, :T]), bits16(L["vp"][rows, :, :T])
        kn, vn = bits16(L["kn"][rows]), bits16(L["vn"][rows])
        q = bits16(L["q"][rows])
        t0 = time.perf_counter()
        ref = oracle.OracleCache(1, w.kv_heads, w.head_dim, w.tokens + 1, w.k_bits,
                                 w.v_bits, w.group_size, w.residual_length, dt)
        ref.append(k, v)
        ref.append(kn, vn)
        ref.decode_attn(q, 1.0 / np.sqrt(w.head_dim))
        t += time.perf_counter() - t0
        done += 1
        nbytes += sum(algorithmic_bytes(w, [T]).values())
    b = nbytes
    return {"value": b / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} batch rows (all {w.kv_heads} kv heads each, cycling through the "
                      f"{w.batch} rows of layer 0), one step each (prefix pack, decode-token "
                      f"append, decode attention); {t:.1f} s of oracle time; host CPU: "
                      f"{cpu_model()}, {os.cpu_count()} logical CPUs visible"}


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

    w, wall, phase, cold, layers, lens = run(args)
    ab = algorithmic_bytes(w, lens)
    layers_n = w.layers
    step_bytes = sum(ab.values()) * layers_n
    # average launch-sequence duration per phase (HIP events in the timed steps)
    avg = {k: float(np.mean(v)) for k, v in phase.items()}
    med = {k: float(np.median(v)) for k, v in phase.items()}
    phases = {}
    for k in ("pack", "flush", "decode"):
        g = ab[k] / avg[k] / 1e9
        phases[k] = {"bytes": ab[k], "us_mean": avg[k] * 1e6, "us_median": med[k] * 1e6,
                     "us_p10": float(np.percentile(phase[k], 10)) * 1e6,
                     "us_p90": float(np.percentile(phase[k], 90)) * 1e6, "samples": len(phase[k]),
                     "gbps": g, "frac": g / PEAK_GBPS, "launches": PHASE_KERNEL[k][2]}
    cold_med = float(np.median(cold))
    phases["decode_cold_llc"] = {"bytes": ab["decode"], "us_median": cold_med * 1e6,
                                 "us_p10": float(np.percentile(cold, 10)) * 1e6,
                                 "us_p90": float(np.percentile(cold, 90)) * 1e6, "samples": len(cold),
                                 "gbps": ab["decode"] / cold_med / 1e9,
                                 "frac": ab["decode"] / cold_med / 1e9 / PEAK_GBPS}
    # roofline of the phase that takes the most time (pack and decode are one
    # dominant kernel each)
    dom = max(("pack", "decode"), key=lambda k: avg[k])
    kname, ksrc, _ = PHASE_KERNEL[dom]
    if dom == "decode":
        kname = "decode_mfma" if w.gq in (1, 2, 4) else "decode_split_valu"
        ksrc = decode_source(w)
    # (the committed counters describe the workload with every sequence T long)
    traffic = None if lens is not None else traffic_from_profile(
        kname, w.name, os.path.join(ROOT, "kv_cache_bit_kivi_amd", "csrc", ksrc))
    achieved = ab[dom] / avg[dom] / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, layers, lens)
    res = {
        "metric": METRIC,
        "value": step_bytes / wall / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.batch,
                   "kv_heads": w.kv_heads, "q_heads": w.q_heads, "head_dim": w.head_dim,
                   "tokens": w.tokens, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "group_size": w.group_size, "residual_length": w.residual_length,
                   "kv_dtype": str(w.dtype).replace("torch.", ""), "layers": w.layers,
                   "lengths": ("every sequence T" if lens is None else
                               f"per sequence uniform in [T/2, T], seed 0 (mean {np.mean(lens):.0f})")},
        "roofline": {"bound": "hbm", "kernel": f"{kname} ({dom})",
                     "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": ab[dom], "us_per_launch": avg[dom] * 1e6},
        "cpu_baseline": cpu,
        "phases": phases,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
