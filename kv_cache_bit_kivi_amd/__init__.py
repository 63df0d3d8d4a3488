"""KIVI hot path on AMD Instinct MI355X (gfx950): 2-/4-bit KV-cache
quantization (keys per channel, values per token, fp16/bf16 residual window)
fused with split-K decode attention, behind the C ABI of include/kivi.h.

`kv_cache_bit_kivi_amd.kivi` is the ctypes binding of libkivi.so; it raises at
import when the library has not been built.  `kv_cache_bit_kivi_amd.inputs`
draws the seeded synthetic workloads.
"""
