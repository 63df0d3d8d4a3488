"""ctypes binding of libkivi.so (include/kivi.h), same names as the C ABI.

This module only marshals arguments: every step of the KIVI hot path runs in
the HIP kernels of libkivi.so.  torch is used for device memory and streams
in the convenience class KiviCache.  There is no fallback: if libkivi.so is
missing or cannot be loaded, importing the binding raises.
"""
import ctypes
import os

# torch is imported before libkivi.so is loaded so that the process holds one
# HIP runtime: torch bundles its own libamdhip64 (same soname), and loading
# libkivi.so first would pull in a second copy from /opt/rocm.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkivi.so")

KIVI_OK = 0
KIVI_ERR_INVALID_ARG = 1
KIVI_ERR_UNSUPPORTED = 2
KIVI_ERR_CAPACITY = 3
KIVI_ERR_BUFFER_TOO_SMALL = 4
KIVI_ERR_EMPTY = 5
KIVI_ERR_HIP = 6

KIVI_F16, KIVI_BF16, KIVI_F32 = 0, 1, 2

EXPORTED = (
    "kivi_cache_bytes", "kivi_cache_create", "kivi_cache_destroy", "kivi_cache_reset",
    "kivi_append", "kivi_flush_residual", "kivi_decode_attn_workspace_bytes",
    "kivi_decode_attn", "kivi_set_decode_splits", "kivi_cache_get_view",
    "kivi_status_string", "kivi_last_error_message",
    "kivi_append_varlen", "kivi_cache_reset_sequences", "kivi_cache_get_lengths",
    "kivi_append_decode_attn", "kivi_cache_set_page_table", "kivi_cache_set_lengths",
    "kivi_set_timing_events", "kivi_stream_read_probe", "kivi_decode_attn_noalloc",
)



# Stored order of the key scale and zero of a block record inside each group
# of 8 channels: position i holds channel KEY_META_ORDER[i] (word w of the
# group holds channels w and w + 4; see include/kivi.h).
KEY_META_ORDER = (0, 4, 1, 5, 2, 6, 3, 7)


class kivi_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_kv_heads", "head_dim", "max_tokens", "k_bits", "v_bits",
        "group_size", "residual_length", "kv_dtype")]


class kivi_cache_view(ctypes.Structure):
    _fields_ = [
        ("n_quant", ctypes.c_int32), ("n_resid", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("block_bytes", ctypes.c_int32),
        ("off_k_codes", ctypes.c_int32), ("off_v_codes", ctypes.c_int32),
        ("off_k_scale", ctypes.c_int32), ("off_k_zero", ctypes.c_int32),
        ("off_v_scale", ctypes.c_int32), ("off_v_zero", ctypes.c_int32),
        ("blocks", ctypes.c_void_p),
        ("k_resid", ctypes.c_void_p), ("v_resid", ctypes.c_void_p),
        ("scale_max", ctypes.c_void_p),
    ]


class KiviError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(kivi_config)
    sig = {
        "kivi_cache_bytes": ([cfgp, ctypes.POINTER(sz)], i32),
        "kivi_cache_create": ([cfgp, vp, sz, ctypes.POINTER(vp)], i32),
        "kivi_cache_destroy": ([vp], i32),
        "kivi_cache_reset": ([vp], i32),
        "kivi_append": ([vp, vp, vp, i32, vp], i32),
        "kivi_flush_residual": ([vp, vp], i32),
        "kivi_append_varlen": ([vp, vp, vp, ctypes.POINTER(i32), i32, vp], i32),
        "kivi_cache_reset_sequences": ([vp, ctypes.POINTER(i32), i32], i32),
        "kivi_cache_get_lengths": ([vp, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "kivi_cache_set_page_table": ([vp, vp, i32, i32], i32),
        "kivi_decode_attn_workspace_bytes": ([vp, i32, ctypes.POINTER(sz)], i32),
        "kivi_decode_attn": ([vp, vp, i32, ctypes.c_float, vp, i32, vp, sz, vp], i32),
        "kivi_append_decode_attn": ([vp, vp, vp, vp, i32, ctypes.c_float, vp, i32, vp, sz, vp], i32),
        "kivi_decode_attn_noalloc": ([vp, vp, i32, ctypes.c_float, vp, i32, vp], i32),
        "kivi_set_decode_splits": ([vp, i32], i32),
        "kivi_cache_set_lengths": ([vp, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "kivi_set_timing_events": ([vp, vp, vp], i32),
        "kivi_stream_read_probe": ([vp, sz, vp, sz, i32, vp], i32),
        "kivi_cache_get_view": ([vp, ctypes.POINTER(kivi_cache_view)], i32),
        "kivi_status_string": ([i32], ctypes.c_char_p),
        "kivi_last_error_message": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def status_name(s):
    return lib.kivi_status_string(s).decode()


def last_error_message():
    return lib.kivi_last_error_message().decode()


def _check(status):
    if status != KIVI_OK:
        raise KiviError(status, last_error_message())


# ----------------------------------------------------------- raw C entry points

def kivi_cache_bytes(cfg):
    n = ctypes.c_size_t()
    _check(lib.kivi_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def kivi_cache_create(cfg, dev_ptr, dev_bytes):
    h = ctypes.c_void_p()
    _check(lib.kivi_cache_create(ctypes.byref(cfg), ctypes.c_void_p(dev_ptr), dev_bytes,
                                 ctypes.byref(h)))
    return h


def kivi_cache_destroy(h):
    _check(lib.kivi_cache_destroy(h))


def kivi_cache_reset(h):
    _check(lib.kivi_cache_reset(h))


def kivi_append(h, k_ptr, v_ptr, n_tokens, stream):
    _check(lib.kivi_append(h, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), n_tokens,
                           ctypes.c_void_p(stream)))


def kivi_flush_residual(h, stream):
    _check(lib.kivi_flush_residual(h, ctypes.c_void_p(stream)))


def _i32_array(values):
    values = [int(x) for x in values]
    return (ctypes.c_int32 * max(1, len(values)))(*values), len(values)


def kivi_append_varlen(h, k_ptr, v_ptr, n_tokens, n_max, stream):
    arr, _ = _i32_array(n_tokens)
    _check(lib.kivi_append_varlen(h, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), arr, n_max,
                                  ctypes.c_void_p(stream)))


def kivi_cache_reset_sequences(h, seqs):
    arr, n = _i32_array(seqs)
    _check(lib.kivi_cache_reset_sequences(h, arr, n))


def kivi_cache_set_page_table(h, table_ptr, page_stride, num_pages):
    _check(lib.kivi_cache_set_page_table(h, ctypes.c_void_p(table_ptr), page_stride, num_pages))


def kivi_cache_get_lengths(h, batch):
    nq = (ctypes.c_int32 * batch)()
    nr = (ctypes.c_int32 * batch)()
    _check(lib.kivi_cache_get_lengths(h, nq, nr))
    return list(nq), list(nr)


def kivi_decode_attn_workspace_bytes(h, num_q_heads):
    n = ctypes.c_size_t()
    _check(lib.kivi_decode_attn_workspace_bytes(h, num_q_heads, ctypes.byref(n)))
    return n.value


def kivi_decode_attn(h, q_ptr, num_q_heads, softmax_scale, out_ptr, out_dtype, ws_ptr,
                     ws_bytes, stream):
    _check(lib.kivi_decode_attn(h, ctypes.c_void_p(q_ptr), num_q_heads,
                                float(softmax_scale), ctypes.c_void_p(out_ptr), out_dtype,
                                ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.c_void_p(stream)))


def kivi_decode_attn_noalloc(h, q_ptr, num_q_heads, softmax_scale, out_ptr, out_dtype, stream):
    _check(lib.kivi_decode_attn_noalloc(h, ctypes.c_void_p(q_ptr), num_q_heads, float(softmax_scale),
                                        ctypes.c_void_p(out_ptr), out_dtype, ctypes.c_void_p(stream)))


def kivi_append_decode_attn(h, k_ptr, v_ptr, q_ptr, num_q_heads, softmax_scale, out_ptr,
                            out_dtype, ws_ptr, ws_bytes, stream):
    _check(lib.kivi_append_decode_attn(h, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                       ctypes.c_void_p(q_ptr), num_q_heads, float(softmax_scale),
                                       ctypes.c_void_p(out_ptr), out_dtype, ctypes.c_void_p(ws_ptr),
                                       ws_bytes, ctypes.c_void_p(stream)))


def kivi_set_decode_splits(h, n_split):
    _check(lib.kivi_set_decode_splits(h, n_split))


def kivi_cache_set_lengths(h, n_quant, n_resid):
    nq, _ = _i32_array(n_quant)
    nr, _ = _i32_array(n_resid)
    _check(lib.kivi_cache_set_lengths(h, nq, nr))


def kivi_set_timing_events(h, split_begin, split_end):
    _check(lib.kivi_set_timing_events(h, ctypes.c_void_p(split_begin), ctypes.c_void_p(split_end)))


def kivi_stream_read_probe(src_ptr, nbytes, sink_ptr, sink_bytes, workgroups, stream):
    _check(lib.kivi_stream_read_probe(ctypes.c_void_p(src_ptr), nbytes, ctypes.c_void_p(sink_ptr),
                                      sink_bytes, workgroups, ctypes.c_void_p(stream)))


def kivi_cache_get_view(h):
    v = kivi_cache_view()
    _check(lib.kivi_cache_get_view(h, ctypes.byref(v)))
    return v


# ------------------------------------------------------------ torch convenience

class KiviCache:
    """One layer's KIVI cache in a torch-allocated device buffer.

    Tensors passed in must be contiguous device tensors: k, v [B][H][n][D] in
    the cache's kv dtype, q [B][Hq][D].  Work is enqueued on the current torch
    stream unless a stream is given."""

    def __init__(self, batch, num_kv_heads, max_tokens, head_dim=128, k_bits=2, v_bits=2,
                 group_size=32, residual_length=128, dtype=None, device="cuda"):
        import torch
        self.torch = torch
        dtype = torch.float16 if dtype is None else dtype
        kv = {torch.float16: KIVI_F16, torch.bfloat16: KIVI_BF16}[dtype]
        self.cfg = kivi_config(batch, num_kv_heads, head_dim, max_tokens, k_bits, v_bits,
                               group_size, residual_length, kv)
        self.dtype = dtype
        self.nbytes = kivi_cache_bytes(self.cfg)
        self.buffer = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.handle = kivi_cache_create(self.cfg, self.buffer.data_ptr(), self.nbytes)
        self.device = self.buffer.device
        self._ws = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and lib is not None:
            lib.kivi_cache_destroy(h)
            self.handle = None

    def _stream(self, stream):
        return (self.torch.cuda.current_stream(self.device) if stream is None else stream).cuda_stream

    def _check_tensor(self, t, dtype, what):
        if not (t.is_contiguous() and t.dtype == dtype and t.device == self.device):
            raise ValueError(f"{what} must be a contiguous {dtype} tensor on {self.device} "
                             f"(got {t.dtype} on {t.device}, contiguous={t.is_contiguous()})")

    def _check_kv(self, t, n):
        c = self.cfg
        self._check_tensor(t, self.dtype, "k/v")
        if tuple(t.shape) != (c.batch, c.num_kv_heads, n, c.head_dim):
            raise ValueError(f"k/v shape {tuple(t.shape)} is not "
                             f"{(c.batch, c.num_kv_heads, n, c.head_dim)}")

    def _check_q(self, q):
        c = self.cfg
        self._check_tensor(q, self.dtype, "q")
        if q.dim() != 3 or q.shape[0] != c.batch or q.shape[2] != c.head_dim:
            raise ValueError(f"q shape {tuple(q.shape)} is not ({c.batch}, Hq, {c.head_dim})")

    def append(self, k, v, stream=None):
        n = k.shape[2]
        self._check_kv(k, n)
        self._check_kv(v, n)
        kivi_append(self.handle, k.data_ptr(), v.data_ptr(), n, self._stream(stream))

    def append_varlen(self, k, v, n_tokens, stream=None):
        """Sequence b appends its first n_tokens[b] tokens of k, v [B][H][n_max][D]."""
        n_max = k.shape[2]
        self._check_kv(k, n_max)
        self._check_kv(v, n_max)
        if len(n_tokens) != self.cfg.batch:
            raise ValueError(f"n_tokens has {len(n_tokens)} entries, batch is {self.cfg.batch}")
        kivi_append_varlen(self.handle, k.data_ptr(), v.data_ptr(), n_tokens, n_max,
                           self._stream(stream))

    def set_page_table(self, table, num_pages):
        """Paged block records: table is a device int32 tensor [B][page_stride]
        (kept alive here); None restores the unit-major layout."""
        if table is None:
            self._page_table = None
            kivi_cache_set_page_table(self.handle, 0, 0, 0)
            return
        t = self.torch
        self._check_tensor(table, t.int32, "table")
        if table.dim() != 2 or table.shape[0] != self.cfg.batch:
            raise ValueError(f"table shape {tuple(table.shape)} is not ({self.cfg.batch}, page_stride)")
        kivi_cache_set_page_table(self.handle, table.data_ptr(), table.shape[1], num_pages)
        self._page_table = table

    def record_index(self, u, g):
        """Index of the block record of unit u, block g in the block region."""
        H = self.cfg.num_kv_heads
        pt = getattr(self, "_page_table", None)
        if pt is None:
            return u * self.view().num_blocks + g
        b, h = divmod(u, H)
        return int(pt[b, g].item()) * H + h

    def reset_sequences(self, seqs):
        kivi_cache_reset_sequences(self.handle, seqs)

    def lengths(self):
        """(n_quant, n_resid) lists, one entry per sequence."""
        return kivi_cache_get_lengths(self.handle, self.cfg.batch)

    def set_lengths(self, n_quant, n_resid):
        """Declares per-sequence lengths of the buffer's contents (lists or
        ints for every sequence), e.g. after restoring a snapshot."""
        B = self.cfg.batch
        nq = [n_quant] * B if isinstance(n_quant, int) else list(n_quant)
        nr = [n_resid] * B if isinstance(n_resid, int) else list(n_resid)
        if len(nq) != B or len(nr) != B:
            raise ValueError(f"lengths need {B} entries")
        kivi_cache_set_lengths(self.handle, nq, nr)

    def flush(self, stream=None):
        kivi_flush_residual(self.handle, self._stream(stream))

    def reset(self):
        kivi_cache_reset(self.handle)

    def set_splits(self, n_split):
        kivi_set_decode_splits(self.handle, n_split)

    def workspace(self, num_q_heads):
        n = kivi_decode_attn_workspace_bytes(self.handle, num_q_heads)
        if self._ws is None or self._ws.numel() < n:
            self._ws = self.torch.empty(max(n, 4), dtype=self.torch.uint8, device=self.device)
        return self._ws

    def decode_attn(self, q, softmax_scale, out=None, out_dtype=None, stream=None):
        torch = self.torch
        c = self.cfg
        self._check_q(q)
        B, Hq, D = q.shape
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty(B, Hq, D, dtype=out_dtype, device=self.device)
        od = {torch.float16: KIVI_F16, torch.bfloat16: KIVI_BF16, torch.float32: KIVI_F32}[out.dtype]
        ws = self.workspace(Hq)
        kivi_decode_attn(self.handle, q.data_ptr(), Hq, softmax_scale, out.data_ptr(), od,
                         ws.data_ptr(), ws.numel(), self._stream(stream))
        return out

    def append_decode_attn(self, k_new, v_new, q, softmax_scale, out=None, out_dtype=None,
                           stream=None):
        """One decode step: append k_new, v_new [B][H][1][D] (one token per
        sequence), then decode attention including it."""
        torch = self.torch
        c = self.cfg
        self._check_kv(k_new, 1)
        self._check_kv(v_new, 1)
        self._check_q(q)
        B, Hq, D = q.shape
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty(B, Hq, D, dtype=out_dtype, device=self.device)
        od = {torch.float16: KIVI_F16, torch.bfloat16: KIVI_BF16, torch.float32: KIVI_F32}[out.dtype]
        ws = self.workspace(Hq)
        kivi_append_decode_attn(self.handle, k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), Hq,
                                softmax_scale, out.data_ptr(), od, ws.data_ptr(), ws.numel(),
                                self._stream(stream))
        return out

    def view(self):
        return kivi_cache_get_view(self.handle)

    @property
    def n_quant(self):
        return self.view().n_quant

    @property
    def n_resid(self):
        return self.view().n_resid

    def arrays(self):
        """Device tensors aliasing the cache fields, shaped [B*H][...] per unit.
        The packed fields are strided views into the block records: unit u,
        block g, field f lies at blocks + (u * NB + g) * block_bytes + off_f;
        "k_scale" and "k_zero" are in stored order (KEY_META_ORDER within each
        8 channels); "scale_max" holds one word per record index ([B*H][NB]
        unit-major)."""
        torch = self.torch
        v = self.view()
        c = self.cfg
        U = c.batch * c.num_kv_heads
        nb, D, G, R = v.num_blocks, c.head_dim, c.group_size, c.residual_length
        base = self.buffer.data_ptr()
        ob = v.blocks - base
        recs = self.buffer[ob:ob + U * nb * v.block_bytes].view(U, nb, v.block_bytes)

        def field(off, nbytes, dt):
            return recs[:, :, off:off + nbytes].view(dt)  # [U][nb][n]

        def sub(ptr, n, dt, esize):
            off = ptr - base
            return self.buffer[off:off + n * esize].view(dt).view(U, -1)

        return {
            "k_codes": field(v.off_k_codes, G * D * c.k_bits // 8, torch.int32),
            "k_scale": field(v.off_k_scale, 2 * D, torch.int16),
            "k_zero": field(v.off_k_zero, 2 * D, torch.int16),
            "v_codes": field(v.off_v_codes, G * D * c.v_bits // 8, torch.int32),
            "v_scale": field(v.off_v_scale, 2 * D, torch.int16),
            "v_zero": field(v.off_v_zero, 2 * D, torch.int16),
            "k_resid": sub(v.k_resid, U * R * D, torch.int16, 2),
            "v_resid": sub(v.v_resid, U * R * D, torch.int16, 2),
            # one word per block record, at the record's index
            "scale_max": sub(v.scale_max, U * nb, torch.int32, 4),
        }
