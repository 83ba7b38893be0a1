"""Python binding of libmoa: heterogeneous sliding-window attention on MI355X.

Argument marshalling only.  Every step of the path (span table, ring layout,
work lists, prefill, ring append, split-K decode, combine) runs in libmoa's
C++ host code and gfx950 HIP kernels; this module checks tensor shapes,
dtypes and devices, then passes raw pointers and the current HIP stream to
the C ABI declared in include/moa.h.  There is no fallback: if libmoa.so is
missing the import fails.

Example::

    plan = Plan(batch=1, n_q_heads=32, n_kv_heads=32, head_dim=128,
                n_prompt=8192, alpha=alpha, beta=beta, dtype="bf16")
    plan.prefill(q, k, v, o)                    # torch tensors on the GPU
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python heterogeneous_sliding_windows_amd/build.py` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

MOA_OK, MOA_EINVAL, MOA_EUNSUPPORTED, MOA_ENOMEM, MOA_EHIP, MOA_EWORKSPACE = 0, -1, -2, -3, -4, -5
MOA_F32, MOA_BF16 = 0, 1
MOA_PLAN_HOST_ONLY = 1
STATUS_NAMES = {0: "MOA_OK", -1: "MOA_EINVAL", -2: "MOA_EUNSUPPORTED", -3: "MOA_ENOMEM",
                -4: "MOA_EHIP", -5: "MOA_EWORKSPACE"}
DTYPES = {"f32": MOA_F32, "bf16": MOA_BF16}

# Every symbol include/moa.h declares.
EXPORTS = ("moa_spans", "moa_ring_offsets", "moa_plan_create", "moa_plan_create_ragged",
           "moa_plan_destroy", "moa_plan_tables", "moa_plan_seq_tables", "moa_cache_elems",
           "moa_decode_workspace_bytes", "moa_max_batch",
           "moa_plan_prefill_items", "moa_plan_decode_chunks", "moa_plan_decode_chunk",
           "moa_prefill", "moa_prefill_handoff", "moa_kv_append", "moa_decode",
           "moa_append_decode", "moa_append_decode_static", "moa_static_workspace_bytes",
           "moa_last_error", "moa_version")


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_prompt", ctypes.c_int64), ("alpha", ctypes.POINTER(ctypes.c_int64)),
                ("beta", ctypes.POINTER(ctypes.c_double)), ("dtype", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_sig = {
    "moa_spans": (ctypes.c_int, [_I64P, ctypes.POINTER(ctypes.c_double), ctypes.c_int32,
                                 ctypes.c_int64, _I32P]),
    "moa_ring_offsets": (ctypes.c_int, [_I32P, ctypes.c_int32, _I64P, _I64P]),
    "moa_plan_create": (ctypes.c_int, [ctypes.POINTER(_Problem), ctypes.c_uint32,
                                       ctypes.POINTER(_P)]),
    "moa_plan_create_ragged": (ctypes.c_int, [ctypes.POINTER(_Problem), _I64P, ctypes.c_uint32,
                                              ctypes.POINTER(_P)]),
    "moa_plan_destroy": (ctypes.c_int, [_P]),
    "moa_plan_tables": (ctypes.c_int, [_P, _I32P, _I64P, _I64P]),
    "moa_plan_seq_tables": (ctypes.c_int, [_P, _I32P, _I64P, _I64P]),
    "moa_cache_elems": (ctypes.c_int64, [_P]),
    "moa_decode_workspace_bytes": (ctypes.c_size_t, [_P]),
    "moa_max_batch": (ctypes.c_int64, [ctypes.POINTER(_Problem), ctypes.c_uint64]),
    "moa_plan_prefill_items": (ctypes.c_int64, [_P, _I32P]),
    "moa_plan_decode_chunks": (ctypes.c_int64, [_P, _I32P]),
    "moa_plan_decode_chunk": (ctypes.c_int32, [_P]),
    "moa_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "moa_prefill_handoff": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "moa_kv_append": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int64, ctypes.c_int64, _P]),
    "moa_decode": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]),
    "moa_append_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int64, _P, _P,
                                         ctypes.c_size_t, _P]),
    "moa_append_decode_static": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int64, _P, _P]),
    "moa_static_workspace_bytes": (ctypes.c_size_t, []),
    "moa_last_error": (ctypes.c_char_p, []),
    "moa_version": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(status):
    if status < 0:
        raise MoaError(status, last_error())
    return status


def last_error():
    return _lib.moa_last_error().decode()


def version():
    return _lib.moa_version().decode()


def _i64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return a, a.ctypes.data_as(_I64P)


def _f64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def spans(alpha, beta, n_prompt):
    """Span table (host-only; see moa_spans in include/moa.h)."""
    a, ap = _i64(alpha)
    b, bp = _f64(beta)
    if len(a) != len(b):
        raise ValueError("alpha and beta need one entry per KV head")
    out = np.zeros(len(a), dtype=np.int32)
    _check(_lib.moa_spans(ap, bp, len(a), int(n_prompt), out.ctypes.data_as(_I32P)))
    return out


def ring_offsets(span):
    """(offset[Hkv], slots_per_seq) of the ring pool (host-only)."""
    s = np.ascontiguousarray(np.asarray(span, dtype=np.int32))
    off = np.zeros(len(s), dtype=np.int64)
    tot = ctypes.c_int64(0)
    _check(_lib.moa_ring_offsets(s.ctypes.data_as(_I32P), len(s), off.ctypes.data_as(_I64P),
                                 ctypes.byref(tot)))
    return off, tot.value


def max_batch(n_q_heads, n_kv_heads, head_dim, n_prompt, alpha, beta, dtype, budget_bytes):
    """Largest batch whose K/V ring pools and decode workspace fit budget_bytes."""
    a, ap = _i64(alpha)
    b, bp = _f64(beta)
    pr = _Problem(1, int(n_q_heads), int(n_kv_heads), int(head_dim), int(n_prompt), ap, bp,
                  DTYPES[dtype])
    return _check(_lib.moa_max_batch(ctypes.byref(pr), int(budget_bytes)))


def static_workspace_bytes():
    """Size of the fixed scratch behind Plan.append_decode_static."""
    return int(_lib.moa_static_workspace_bytes())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """A problem (shapes + per-KV-head (alpha, beta) rules) with its tables.

    seq_len: optional per-sequence prompt lengths (a ragged batch, left
    padded to n_prompt = max(seq_len)); see moa_plan_create_ragged.
    Tables of every plan: seq_spans [B, Hkv], ring_offsets [B, Hkv] (first
    slot of each ring in the pools), seq_len [B].  A plan without per-sequence
    lengths also has spans [Hkv], offsets [Hkv] and slots_per_seq (None for a
    ragged plan).
    """

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, n_prompt, alpha, beta,
                 dtype="bf16", host_only=False, seq_len=None):
        self._h = None
        self.batch, self.n_q_heads, self.n_kv_heads = int(batch), int(n_q_heads), int(n_kv_heads)
        self.head_dim, self.n_prompt, self.dtype = int(head_dim), int(n_prompt), dtype
        self.host_only = bool(host_only)
        if dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
        self._alpha, ap = _i64(alpha)
        self._beta, bp = _f64(beta)
        if len(self._alpha) != self.n_kv_heads or len(self._beta) != self.n_kv_heads:
            raise ValueError("alpha and beta need n_kv_heads entries")
        pr = _Problem(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                      self.n_prompt, ap, bp, DTYPES[dtype])
        h = _P()
        flags = MOA_PLAN_HOST_ONLY if host_only else 0
        self.ragged = seq_len is not None
        if self.ragged:
            lens, lp = _i64(seq_len)
            if len(lens) != self.batch:
                raise ValueError("seq_len needs one entry per sequence")
            _check(_lib.moa_plan_create_ragged(ctypes.byref(pr), lp, flags, ctypes.byref(h)))
        else:
            _check(_lib.moa_plan_create(ctypes.byref(pr), flags, ctypes.byref(h)))
        self._h = h
        self.seq_spans = np.zeros((self.batch, self.n_kv_heads), dtype=np.int32)
        self.ring_offsets = np.zeros((self.batch, self.n_kv_heads), dtype=np.int64)
        self.seq_len = np.zeros(self.batch, dtype=np.int64)
        _check(_lib.moa_plan_seq_tables(h, self.seq_spans.ctypes.data_as(_I32P),
                                        self.ring_offsets.ctypes.data_as(_I64P),
                                        self.seq_len.ctypes.data_as(_I64P)))
        self.spans = self.offsets = self.slots_per_seq = None
        if not self.ragged:
            self.spans = np.zeros(self.n_kv_heads, dtype=np.int32)
            self.offsets = np.zeros(self.n_kv_heads, dtype=np.int64)
            tot = ctypes.c_int64(0)
            _check(_lib.moa_plan_tables(h, self.spans.ctypes.data_as(_I32P),
                                        self.offsets.ctypes.data_as(_I64P), ctypes.byref(tot)))
            self.slots_per_seq = tot.value
        self.cache_elems = _lib.moa_cache_elems(h)
        self.workspace_bytes = _lib.moa_decode_workspace_bytes(h)
        self.decode_chunk = _lib.moa_plan_decode_chunk(h)

    # -- inspection ---------------------------------------------------------
    def prefill_items(self):
        """[n, 6] int32 {b, h_q, q_tile, kt_lo, kt_hi, workgroup}, in workgroup order."""
        n = _check(_lib.moa_plan_prefill_items(self._h, None))
        out = np.zeros((n, 6), dtype=np.int32)
        _check(_lib.moa_plan_prefill_items(self._h, out.ctypes.data_as(_I32P)))
        return out

    def decode_chunks(self):
        """[n, 4] int32 {b, h_kv, first_slot, n_slots} of all sequences in launch order."""
        n = _check(_lib.moa_plan_decode_chunks(self._h, None))
        out = np.zeros((n, 4), dtype=np.int32)
        _check(_lib.moa_plan_decode_chunks(self._h, out.ctypes.data_as(_I32P)))
        return out

    # -- tensor checks --------------------------------------------------------
    def _torch_dtype(self):
        import torch
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    def _t(self, t, shape, name):
        import torch
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
        if t.dtype != self._torch_dtype():
            raise ValueError(f"{name} must be {self._torch_dtype()}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.data_ptr() % 16:
            raise ValueError(f"{name} must start at a 16-byte aligned address")
        return ctypes.c_void_p(t.data_ptr())

    def cache_shape(self):
        return (self.cache_elems,)

    # -- the hot path -----------------------------------------------------------
    def prefill(self, q, k, v, o, stream=None):
        B, Hq, Hk, N, D = self.batch, self.n_q_heads, self.n_kv_heads, self.n_prompt, self.head_dim
        args = (self._t(q, (B, Hq, N, D), "q"), self._t(k, (B, Hk, N, D), "k"),
                self._t(v, (B, Hk, N, D), "v"), self._t(o, (B, Hq, N, D), "o"))
        _check(_lib.moa_prefill(self._h, *args, _stream(stream)))
        return o

    def prefill_handoff(self, q, k, v, o, k_cache, v_cache, stream=None):
        """prefill() and kv_append(pos0=0) of the whole prompt in one launch."""
        B, Hq, Hk, N, D = self.batch, self.n_q_heads, self.n_kv_heads, self.n_prompt, self.head_dim
        args = (self._t(q, (B, Hq, N, D), "q"), self._t(k, (B, Hk, N, D), "k"),
                self._t(v, (B, Hk, N, D), "v"), self._t(o, (B, Hq, N, D), "o"),
                self._t(k_cache, self.cache_shape(), "k_cache"),
                self._t(v_cache, self.cache_shape(), "v_cache"))
        _check(_lib.moa_prefill_handoff(self._h, *args, _stream(stream)))
        return o

    def kv_append(self, k_cache, v_cache, k_new, v_new, pos0, stream=None):
        B, Hk, D = self.batch, self.n_kv_heads, self.head_dim
        if k_new.dim() != 4:
            raise ValueError("k_new must be [B, Hkv, n_new, D]")
        n_new = k_new.shape[2]
        args = (self._t(k_cache, self.cache_shape(), "k_cache"),
                self._t(v_cache, self.cache_shape(), "v_cache"),
                self._t(k_new, (B, Hk, n_new, D), "k_new"),
                self._t(v_new, (B, Hk, n_new, D), "v_new"))
        _check(_lib.moa_kv_append(self._h, *args, int(pos0), int(n_new), _stream(stream)))

    @staticmethod
    def _ws(workspace):
        import torch
        if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
                or not workspace.is_contiguous() or workspace.data_ptr() % 16:
            raise ValueError("workspace must be a contiguous, 16-byte aligned GPU tensor")
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()

    def decode(self, q, k_cache, v_cache, pos, o, workspace, stream=None):
        B, Hq, D = self.batch, self.n_q_heads, self.head_dim
        ws, ws_bytes = self._ws(workspace)
        args = (self._t(q, (B, Hq, D), "q"), self._t(k_cache, self.cache_shape(), "k_cache"),
                self._t(v_cache, self.cache_shape(), "v_cache"))
        _check(_lib.moa_decode(self._h, *args, int(pos), self._t(o, (B, Hq, D), "o"), ws,
                               ws_bytes, _stream(stream)))
        return o

    def append_decode(self, q, k_cache, v_cache, k_new, v_new, pos, o, workspace, stream=None):
        """kv_append(pos, one token) and decode(pos) in one launch (k_new, v_new [B, Hkv, D])."""
        B, Hq, Hk, D = self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim
        ws, ws_bytes = self._ws(workspace)
        args = (self._t(q, (B, Hq, D), "q"), self._t(k_cache, self.cache_shape(), "k_cache"),
                self._t(v_cache, self.cache_shape(), "v_cache"),
                self._t(k_new, (B, Hk, D), "k_new"), self._t(v_new, (B, Hk, D), "v_new"))
        _check(_lib.moa_append_decode(self._h, *args, int(pos), self._t(o, (B, Hq, D), "o"), ws,
                                      ws_bytes, _stream(stream)))
        return o

    def append_decode_static(self, q, k_cache, v_cache, k_new, v_new, pos, o, stream=None):
        """append_decode() with the library's fixed decode scratch instead of a workspace
        (moa_append_decode_static: allocates nothing; calls on one GPU share the scratch)."""
        B, Hq, Hk, D = self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim
        args = (self._t(q, (B, Hq, D), "q"), self._t(k_cache, self.cache_shape(), "k_cache"),
                self._t(v_cache, self.cache_shape(), "v_cache"),
                self._t(k_new, (B, Hk, D), "k_new"), self._t(v_new, (B, Hk, D), "v_new"))
        _check(_lib.moa_append_decode_static(self._h, *args, int(pos),
                                             self._t(o, (B, Hq, D), "o"), _stream(stream)))
        return o

    def new_cache(self):
        """(k_cache, v_cache) zero-filled ring pools on the current GPU."""
        import torch
        return (torch.zeros(self.cache_elems, dtype=self._torch_dtype(), device="cuda"),
                torch.zeros(self.cache_elems, dtype=self._torch_dtype(), device="cuda"))

    def new_workspace(self):
        """Decode workspace (scratch; no initial contents required)."""
        import torch
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device="cuda")

    def close(self):
        if self._h is not None:
            _lib.moa_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


from . import rules  # noqa: E402,F401  (per-layer rules files; needs Plan above)
