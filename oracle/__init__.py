"""Python binding of the plain CPU oracle of the KIVI hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
CPU-baseline leg of bench.py may import this module.  The product path never
imports it; the HIP library and this oracle share no code.

The arithmetic lives in kivi_oracle.c (plain C, binary32 quantizer with
correctly rounded IEEE operations, binary64 attention).  This module only
marshals numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F16, BF16 = 0, 1


class _OracleCache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("B", "H", "D", "T_max", "kb", "vb", "G", "R", "dtype",
                 "cap", "nb", "n_quant", "n_resid")] + [
        ("k_codes", ctypes.POINTER(ctypes.c_uint32)),
        ("k_scale", ctypes.POINTER(ctypes.c_uint16)),
        ("k_zero", ctypes.POINTER(ctypes.c_uint16)),
        ("v_codes", ctypes.POINTER(ctypes.c_uint32)),
        ("v_scale", ctypes.POINTER(ctypes.c_uint16)),
        ("v_zero", ctypes.POINTER(ctypes.c_uint16)),
        ("k_resid", ctypes.POINTER(ctypes.c_uint16)),
        ("v_resid", ctypes.POINTER(ctypes.c_uint16)),
    ]


def lib():
    """Loads liboracle.so (built by oracle/build.py), building it if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        u16, f32, i32 = ctypes.c_uint16, ctypes.c_float, ctypes.c_int
        vp = ctypes.c_void_p
        L.oracle_f16_to_f32.argtypes = [u16]
        L.oracle_f16_to_f32.restype = f32
        L.oracle_bf16_to_f32.argtypes = [u16]
        L.oracle_bf16_to_f32.restype = f32
        L.oracle_f32_to_f16.argtypes = [f32]
        L.oracle_f32_to_f16.restype = u16
        L.oracle_quantize_group.argtypes = [vp, i32, i32, vp, vp, vp]
        L.oracle_quantize_group.restype = None
        L.oracle_dequant.argtypes = [i32, u16, u16]
        L.oracle_dequant.restype = ctypes.c_double
        P = ctypes.POINTER(_OracleCache)
        L.oracle_cache_init.argtypes = [P] + [i32] * 9
        L.oracle_cache_init.restype = i32
        L.oracle_cache_free.argtypes = [P]
        L.oracle_cache_free.restype = None
        L.oracle_cache_len.argtypes = [P, i32]
        L.oracle_cache_len.restype = ctypes.c_size_t
        L.oracle_cache_append.argtypes = [P, vp, vp, i32]
        L.oracle_cache_append.restype = i32
        L.oracle_cache_flush.argtypes = [P]
        L.oracle_cache_flush.restype = None
        L.oracle_decode_attn.argtypes = [P, vp, i32, ctypes.c_double, vp]
        L.oracle_decode_attn.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def f16_to_f32(bits):
    return lib().oracle_f16_to_f32(int(bits))


def bf16_to_f32(bits):
    return lib().oracle_bf16_to_f32(int(bits))


def f32_to_f16(x):
    return lib().oracle_f32_to_f16(float(np.float32(x)))


def quantize_group(x, bits):
    """Quantizes one group of binary32 values -> (codes uint8, S bits, Z bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint16)
    z = np.zeros(1, dtype=np.uint16)
    lib().oracle_quantize_group(_ptr(x), x.size, bits, _ptr(codes), _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0])


def dequant(code, s_bits, z_bits):
    return lib().oracle_dequant(int(code), int(s_bits), int(z_bits))


def num_threads():
    return lib().oracle_num_threads()


_ARRAYS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero",
           "k_resid", "v_resid")


class OracleCache:
    """Host-side KIVI cache of one layer in the packed layout.

    Inputs are raw 16-bit patterns (np.uint16) of fp16 (dtype F16) or bf16
    (dtype BF16), shaped [B][H][n][D]."""

    def __init__(self, B, H, D, max_tokens, k_bits=2, v_bits=2, group_size=32,
                 residual_length=128, dtype=F16):
        self._c = _OracleCache()
        rc = lib().oracle_cache_init(ctypes.byref(self._c), B, H, D, max_tokens,
                                     k_bits, v_bits, group_size, residual_length,
                                     dtype)
        if rc != 0:
            raise ValueError("bad oracle cache config")
        self.B, self.H, self.D = B, H, D
        self.G, self.R = group_size, residual_length
        self.k_bits, self.v_bits, self.dtype = k_bits, v_bits, dtype

    def __del__(self):
        if getattr(self, "_c", None) is not None and _lib is not None:
            _lib.oracle_cache_free(ctypes.byref(self._c))
            self._c = None

    @property
    def n_quant(self):
        return self._c.n_quant

    @property
    def n_resid(self):
        return self._c.n_resid

    @property
    def capacity(self):
        return self._c.cap

    @property
    def num_blocks(self):
        return self._c.nb

    def array(self, name):
        """Copy of one packed-layout array, flat."""
        i = _ARRAYS.index(name)
        n = lib().oracle_cache_len(ctypes.byref(self._c), i)
        p = getattr(self._c, name)
        return np.ctypeslib.as_array(p, shape=(n,)).copy()

    def arrays(self):
        return {n: self.array(n) for n in _ARRAYS}

    def append(self, k_bits16, v_bits16):
        k = np.ascontiguousarray(k_bits16, dtype=np.uint16)
        v = np.ascontiguousarray(v_bits16, dtype=np.uint16)
        assert k.shape == v.shape and k.ndim == 4
        assert k.shape[0] == self.B and k.shape[1] == self.H and k.shape[3] == self.D
        rc = lib().oracle_cache_append(ctypes.byref(self._c), _ptr(k), _ptr(v), k.shape[2])
        if rc != 0:
            raise OverflowError("oracle cache capacity exceeded")

    def flush(self):
        lib().oracle_cache_flush(ctypes.byref(self._c))

    def decode_attn(self, q_bits16, softmax_scale):
        """q: raw 16-bit [B][Hq][D] -> out float64 [B][Hq][D]."""
        q = np.ascontiguousarray(q_bits16, dtype=np.uint16)
        assert q.ndim == 3 and q.shape[0] == self.B and q.shape[2] == self.D
        out = np.zeros(q.shape, dtype=np.float64)
        rc = lib().oracle_decode_attn(ctypes.byref(self._c), _ptr(q), q.shape[1],
                                      float(softmax_scale), _ptr(out))
        if rc != 0:
            raise ValueError("oracle decode: empty cache or bad head count")
        return out
