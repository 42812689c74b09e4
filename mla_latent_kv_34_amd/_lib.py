"""ctypes binding of libmla (include/mla.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and the current HIP stream are handed to the
C ABI, and a non-OK status becomes an exception.  Every step of the hot path
runs in the library's HIP kernels; there is no fallback.  PyTorch only
provides device memory and the stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
CHUNK_AUTO, CHUNK_EXPAND, CHUNK_ABSORB = range(3)  # mla_chunk_mode
MLA_BF16, MLA_F32 = 0, 1

EXPORTED = (
    "mla_cache_append", "mla_decode_workspace_size", "mla_decode", "mla_decode_step",
    "mla_decode_step_noalloc",
    "mla_decode_hidden_workspace_size", "mla_decode_hidden",
    "mla_decode_layer", "mla_merge_query_weights", "mla_decode_hidden_merged",
    "mla_merge_output_weights", "mla_decode_layer_merged",
    "mla_prefill_workspace_size", "mla_prefill", "mla_prefill_chunk_workspace_size",
    "mla_prefill_chunk", "mla_status_string", "mla_last_error",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class LibraryMissing(ImportError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
        ("d_latent", ctypes.c_int32), ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("reserved", ctypes.c_float), ("rope_base", ctypes.c_double),
    ]


class _Cache(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p), ("num_pages", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
    ]


@dataclass(frozen=True)
class Dims:
    """Sizes of one MLA layer as the library sees them."""
    n_heads: int
    d_nope: int
    d_rope: int
    d_latent: int
    page_size: int = 64
    dtype: torch.dtype = torch.bfloat16
    sm_scale: float = 0.0          # 0 -> 1/sqrt(d_nope + d_rope)
    rope_base: float = 10000.0

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope

    def _c(self) -> _Dims:
        if self.dtype == torch.bfloat16:
            dt = MLA_BF16
        elif self.dtype == torch.float32:
            dt = MLA_F32
        else:
            raise TypeError(f"unsupported dtype {self.dtype}")
        return _Dims(self.n_heads, self.d_nope, self.d_rope, self.d_latent, self.page_size, dt,
                     float(self.sm_scale), 0.0, float(self.rope_base))


_lib = None


def load() -> ctypes.CDLL:
    """Load libmla.so from the package directory (built by build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} is not built; run python -m mla_latent_kv_34_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.mla_cache_append.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P,
                                     ctypes.c_int32, P, P, P]
    lib.mla_cache_append.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, ctypes.c_int32]
    lib.mla_decode_workspace_size.restype = ctypes.c_size_t
    lib.mla_decode.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P, P, P, P, P,
                               P, P, ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_decode_step.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P, P, P,
                                    P, P, P, P, P, P, ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.mla_decode_step.restype = ctypes.c_int
    lib.mla_decode_step_noalloc.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P,
                                            P, P, P, P, P, P, P, ctypes.c_int32, P, P]
    lib.mla_decode_step_noalloc.restype = ctypes.c_int
    lib.mla_decode_hidden_workspace_size.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_int32]
    lib.mla_decode_hidden_workspace_size.restype = ctypes.c_size_t
    lib.mla_decode_hidden.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P,
                                      ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P,
                                      ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.mla_decode_hidden.restype = ctypes.c_int
    lib.mla_decode_layer.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P,
                                     ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P, P,
                                     ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.mla_decode_layer.restype = ctypes.c_int
    lib.mla_merge_query_weights.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, P, P, P, P]
    lib.mla_merge_query_weights.restype = ctypes.c_int
    lib.mla_decode_hidden_merged.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P,
                                             ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P, P, P,
                                             ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.mla_decode_hidden_merged.restype = ctypes.c_int
    lib.mla_merge_output_weights.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, P, P, P, P]
    lib.mla_merge_output_weights.restype = ctypes.c_int
    lib.mla_decode_layer_merged.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, P,
                                            ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P,
                                            ctypes.c_size_t, ctypes.c_int32, P, P]
    lib.mla_decode_layer_merged.restype = ctypes.c_int
    lib.mla_prefill_workspace_size.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, ctypes.c_int32]
    lib.mla_prefill_workspace_size.restype = ctypes.c_size_t
    lib.mla_prefill.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32, ctypes.c_int32,
                                P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P]
    lib.mla_prefill.restype = ctypes.c_int
    lib.mla_prefill_chunk_workspace_size.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_int32]
    lib.mla_prefill_chunk_workspace_size.restype = ctypes.c_size_t
    lib.mla_prefill_chunk.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + \
        [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_prefill_chunk.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != MLA_OK:
        lib = load()
        raise MlaError(status, f"{lib.mla_status_string(status).decode()}: {lib.mla_last_error().decode()}")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _cache(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor) -> _Cache:
    if pool.dim() != 3 or pool.shape[1] != dims.page_size or pool.shape[2] != dims.row:
        raise ValueError(f"pool must be [num_pages, {dims.page_size}, {dims.row}], got {tuple(pool.shape)}")
    _need(pool, "pool", dims.dtype)
    _need(page_table, "page_table", torch.int32, device=pool.device)
    if page_table.dim() != 2:
        raise ValueError("page_table must be [batch, max_pages]")
    return _Cache(pool.data_ptr(), pool.shape[0], page_table.shape[1], page_table.data_ptr())


class _Prepared:
    """A validated, packed C call; calling it re-issues the call on a stream."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep   # keeps the ctypes structs and tensors alive

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)))


class _Events:
    """The void*[2] array of hipEvent_t handles the C ABI takes (or NULL)."""

    def __init__(self, ev):
        self.arr = None
        self.ptr = None
        if ev is not None:
            self.arr = (ctypes.c_void_p * 2)(ev[0].cuda_event, ev[1].cuda_event)
            self.ptr = ctypes.cast(self.arr, ctypes.c_void_p)
            self.ev = ev


def _events(ev):
    return _Events(ev)


def cache_append(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, start_pos: torch.Tensor,
                 c_kv: torch.Tensor, k_rope: torch.Tensor, stream=None, prepare: bool = False):
    """Write n_new tokens per sequence at positions start_pos[b] + k (mla_cache_append).
    prepare=True returns a call(stream=None) that re-issues the same append."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    B, n_new = c_kv.shape[0], c_kv.shape[1]
    _need(c_kv, "c_kv", dims.dtype, (B, n_new, dims.d_latent), dev)
    _need(k_rope, "k_rope", dims.dtype, (B, n_new, dims.d_rope), dev)
    _need(start_pos, "start_pos", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    d = dims._c()
    call = _Prepared(lib.mla_cache_append,
                     [ctypes.byref(d), ctypes.byref(cache), B, _ptr(start_pos), n_new, _ptr(c_kv),
                      _ptr(k_rope)], keep=(d, cache, start_pos, c_kv, k_rope, page_table, pool))
    if prepare:
        return call
    call(stream)


def decode_workspace_size(dims: Dims, batch: int, n_workgroups: int = 0) -> int:
    d = dims._c()
    return int(load().mla_decode_workspace_size(ctypes.byref(d), batch, n_workgroups))


def decode(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
           q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           n_workgroups: int = 0, stream=None, timing_events=None, prepare: bool = False):
    """Weight-absorbed decode of one query per sequence (mla_decode); returns out.

    timing_events: optional pair of torch.cuda.Event recorded around the
    attention kernel.  prepare=True validates and packs the arguments once and
    returns (call, out) where call(stream=None) re-issues the same decode.
    """
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    B = q_nope.shape[0]
    H = dims.n_heads
    _need(q_nope, "q_nope", dims.dtype, (B, H, dims.d_nope), dev)
    _need(q_rope, "q_rope", dims.dtype, (B, H, dims.d_rope), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, H, dims.d_nope), dev)
    need = decode_workspace_size(dims, B, n_workgroups)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), _ptr(q_nope), _ptr(q_rope),
            _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace), wbytes, n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode, args, keep=(d, cache, seq_lens, q_nope, q_rope, w_uk, w_uv,
                                                  out, workspace, evs))
    if prepare:
        return call, out
    call(stream)
    return out


def decode_step(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                c_kv_new: torch.Tensor, k_rope_new: torch.Tensor, q_nope: torch.Tensor,
                q_rope: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                n_workgroups: int = 0, stream=None, timing_events=None, prepare: bool = False):
    """Append the newest token of every sequence (position seq_lens[b] - 1) and
    decode (mla_decode_step); returns out.  Arguments as for decode, plus
    c_kv_new [batch, d_latent] and k_rope_new [batch, d_rope]."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    B = q_nope.shape[0]
    H = dims.n_heads
    _need(c_kv_new, "c_kv_new", dims.dtype, (B, dims.d_latent), dev)
    _need(k_rope_new, "k_rope_new", dims.dtype, (B, dims.d_rope), dev)
    _need(q_nope, "q_nope", dims.dtype, (B, H, dims.d_nope), dev)
    _need(q_rope, "q_rope", dims.dtype, (B, H, dims.d_rope), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, H, dims.d_nope), dev)
    need = decode_workspace_size(dims, B, n_workgroups)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), _ptr(c_kv_new), _ptr(k_rope_new),
            _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace), wbytes,
            n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode_step, args, keep=(d, cache, seq_lens, c_kv_new, k_rope_new, q_nope,
                                                       q_rope, w_uk, w_uv, out, workspace, evs, pool,
                                                       page_table))
    if prepare:
        return call, out
    call(stream)
    return out


def decode_step_noalloc(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        c_kv_new: torch.Tensor, k_rope_new: torch.Tensor, q_nope: torch.Tensor,
                        q_rope: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                        out: torch.Tensor | None = None, n_workgroups: int = 0, stream=None,
                        timing_events=None, prepare: bool = False):
    """mla_decode_step_noalloc: decode_step with no workspace (the library's
    static scratch serves as one).  Arguments as for decode_step."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    B = q_nope.shape[0]
    H = dims.n_heads
    _need(c_kv_new, "c_kv_new", dims.dtype, (B, dims.d_latent), dev)
    _need(k_rope_new, "k_rope_new", dims.dtype, (B, dims.d_rope), dev)
    _need(q_nope, "q_nope", dims.dtype, (B, H, dims.d_nope), dev)
    _need(q_rope, "q_rope", dims.dtype, (B, H, dims.d_rope), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, H, dims.d_nope), dev)
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), _ptr(c_kv_new), _ptr(k_rope_new),
            _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(out), n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode_step_noalloc, args,
                     keep=(d, cache, seq_lens, c_kv_new, k_rope_new, q_nope, q_rope, w_uk, w_uv, out, evs,
                           pool, page_table))
    if prepare:
        return call, out
    call(stream)
    return out


def decode_hidden_workspace_size(dims: Dims, batch: int, d_model: int, d_q: int,
                                 n_workgroups: int = 0) -> int:
    d = dims._c()
    return int(load().mla_decode_hidden_workspace_size(ctypes.byref(d), batch, n_workgroups, d_model, d_q))


def decode_hidden(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                  h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor, w_dq: torch.Tensor,
                  w_uq: torch.Tensor, w_qr: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  n_workgroups: int = 0, stream=None, timing_events=None, prepare: bool = False):
    """Decode step from the newest hidden state of every sequence
    (mla_decode_hidden): h [batch, d_model]; w_dkv [d_latent, d_model],
    w_kr [d_rope, d_model], w_dq [d_q, d_model], w_uq [n_heads * d_nope, d_q],
    w_qr [n_heads * d_rope, d_q]; the rest as for decode_step.  Returns out."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    if h.dim() != 2:
        raise ValueError("h must be [batch, d_model]")
    B, d_model = h.shape
    d_q = w_dq.shape[0] if w_dq.dim() == 2 else -1
    H = dims.n_heads
    _need(h, "h", dims.dtype, (B, d_model), dev)
    _need(w_dkv, "w_dkv", dims.dtype, (dims.d_latent, d_model), dev)
    _need(w_kr, "w_kr", dims.dtype, (dims.d_rope, d_model), dev)
    _need(w_dq, "w_dq", dims.dtype, (d_q, d_model), dev)
    _need(w_uq, "w_uq", dims.dtype, (H * dims.d_nope, d_q), dev)
    _need(w_qr, "w_qr", dims.dtype, (H * dims.d_rope, d_q), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, H, dims.d_nope), dev)
    need = decode_hidden_workspace_size(dims, B, d_model, d_q, n_workgroups)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), d_model, d_q, _ptr(h),
            _ptr(w_dkv), _ptr(w_kr), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(w_uk), _ptr(w_uv),
            _ptr(out), _ptr(workspace), wbytes, n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode_hidden, args, keep=(d, cache, seq_lens, h, w_dkv, w_kr, w_dq, w_uq,
                                                         w_qr, w_uk, w_uv, out, workspace, evs, pool,
                                                         page_table))
    if prepare:
        return call, out
    call(stream)
    return out


def decode_layer(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                 h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor, w_dq: torch.Tensor,
                 w_uq: torch.Tensor, w_qr: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                 w_o: torch.Tensor, u: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 n_workgroups: int = 0, stream=None, timing_events=None, prepare: bool = False):
    """The attention layer of a decode step from the newest hidden states to
    the layer output (mla_decode_layer): decode_hidden, then u = W^O o with
    w_o [d_model, n_heads * d_nope].  Returns u [batch, d_model]; timing_events
    bracket the W^O projection."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    if h.dim() != 2:
        raise ValueError("h must be [batch, d_model]")
    B, d_model = h.shape
    d_q = w_dq.shape[0] if w_dq.dim() == 2 else -1
    H = dims.n_heads
    _need(h, "h", dims.dtype, (B, d_model), dev)
    _need(w_dkv, "w_dkv", dims.dtype, (dims.d_latent, d_model), dev)
    _need(w_kr, "w_kr", dims.dtype, (dims.d_rope, d_model), dev)
    _need(w_dq, "w_dq", dims.dtype, (d_q, d_model), dev)
    _need(w_uq, "w_uq", dims.dtype, (H * dims.d_nope, d_q), dev)
    _need(w_qr, "w_qr", dims.dtype, (H * dims.d_rope, d_q), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_o, "w_o", dims.dtype, (d_model, H * dims.d_nope), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if u is None:
        u = torch.empty((B, d_model), dtype=dims.dtype, device=dev)
    _need(u, "u", dims.dtype, (B, d_model), dev)
    need = decode_hidden_workspace_size(dims, B, d_model, d_q, n_workgroups)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), d_model, d_q, _ptr(h),
            _ptr(w_dkv), _ptr(w_kr), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(w_uk), _ptr(w_uv),
            _ptr(w_o), _ptr(u), _ptr(workspace), wbytes, n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode_layer, args, keep=(d, cache, seq_lens, h, w_dkv, w_kr, w_dq, w_uq,
                                                        w_qr, w_uk, w_uv, w_o, u, workspace, evs, pool,
                                                        page_table))
    if prepare:
        return call, u
    call(stream)
    return u


def merge_query_weights(dims: Dims, w_uq: torch.Tensor, w_uk: torch.Tensor,
                        w_uqk: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """W^UQK_i = W^UK_i^T W^UQ_i (mla_merge_query_weights): w_uq [n_heads *
    d_nope, d_q], w_uk [n_heads, d_nope, d_latent]; returns [n_heads,
    d_latent, d_q]."""
    lib = load()
    H = dims.n_heads
    if w_uq.dim() != 2:
        raise ValueError("w_uq must be [n_heads * d_nope, d_q]")
    d_q = w_uq.shape[1]
    dev = w_uq.device
    _need(w_uq, "w_uq", dims.dtype, (H * dims.d_nope, d_q), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    if w_uqk is None:
        w_uqk = torch.empty((H, dims.d_latent, d_q), dtype=dims.dtype, device=dev)
    _need(w_uqk, "w_uqk", dims.dtype, (H, dims.d_latent, d_q), dev)
    d = dims._c()
    _check(lib.mla_merge_query_weights(ctypes.byref(d), d_q, _ptr(w_uq), _ptr(w_uk), _ptr(w_uqk),
                                       _stream(stream)))
    return w_uqk


def decode_hidden_merged(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                         h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor, w_dq: torch.Tensor,
                         w_uqk: torch.Tensor, w_qr: torch.Tensor, w_uv: torch.Tensor,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         n_workgroups: int = 0, stream=None, timing_events=None, prepare: bool = False):
    """decode_hidden with the pre-merged query weight (mla_decode_hidden_merged):
    w_uqk [n_heads, d_latent, d_q] from merge_query_weights replaces w_uq and
    w_uk.  Returns out [batch, n_heads, d_nope]."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    if h.dim() != 2:
        raise ValueError("h must be [batch, d_model]")
    B, d_model = h.shape
    d_q = w_dq.shape[0] if w_dq.dim() == 2 else -1
    H = dims.n_heads
    _need(h, "h", dims.dtype, (B, d_model), dev)
    _need(w_dkv, "w_dkv", dims.dtype, (dims.d_latent, d_model), dev)
    _need(w_kr, "w_kr", dims.dtype, (dims.d_rope, d_model), dev)
    _need(w_dq, "w_dq", dims.dtype, (d_q, d_model), dev)
    _need(w_uqk, "w_uqk", dims.dtype, (H, dims.d_latent, d_q), dev)
    _need(w_qr, "w_qr", dims.dtype, (H * dims.d_rope, d_q), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, H, dims.d_nope), dev)
    need = decode_hidden_workspace_size(dims, B, d_model, d_q, n_workgroups)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), d_model, d_q, _ptr(h),
            _ptr(w_dkv), _ptr(w_kr), _ptr(w_dq), _ptr(w_uqk), _ptr(w_qr), _ptr(w_uv),
            _ptr(out), _ptr(workspace), wbytes, n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode_hidden_merged, args, keep=(d, cache, seq_lens, h, w_dkv, w_kr, w_dq,
                                                                w_uqk, w_qr, w_uv, out, workspace, evs,
                                                                pool, page_table))
    if prepare:
        return call, out
    call(stream)
    return out


def merge_output_weights(dims: Dims, w_o: torch.Tensor, w_uv: torch.Tensor,
                         w_ov: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """W^OV = [W^O_i W^UV_i]_i (mla_merge_output_weights): w_o [d_model,
    n_heads * d_nope], w_uv [n_heads, d_nope, d_latent]; returns [d_model,
    n_heads * d_latent]."""
    lib = load()
    H = dims.n_heads
    if w_o.dim() != 2:
        raise ValueError("w_o must be [d_model, n_heads * d_nope]")
    d_model = w_o.shape[0]
    dev = w_o.device
    _need(w_o, "w_o", dims.dtype, (d_model, H * dims.d_nope), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    if w_ov is None:
        w_ov = torch.empty((d_model, H * dims.d_latent), dtype=dims.dtype, device=dev)
    _need(w_ov, "w_ov", dims.dtype, (d_model, H * dims.d_latent), dev)
    d = dims._c()
    _check(lib.mla_merge_output_weights(ctypes.byref(d), d_model, _ptr(w_o), _ptr(w_uv), _ptr(w_ov),
                                        _stream(stream)))
    return w_ov


def decode_layer_merged(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor, w_dq: torch.Tensor,
                        w_uq: torch.Tensor, w_qr: torch.Tensor, w_uk: torch.Tensor, w_ov: torch.Tensor,
                        u: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        n_workgroups: int = 0, stream=None, timing_events=None, prepare: bool = False):
    """decode_layer with W^UV merged into W^O (mla_decode_layer_merged): w_ov
    [d_model, n_heads * d_latent] from merge_output_weights replaces w_uv and
    w_o.  Returns u [batch, d_model]; timing_events bracket the W^OV stage."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    if h.dim() != 2:
        raise ValueError("h must be [batch, d_model]")
    B, d_model = h.shape
    d_q = w_dq.shape[0] if w_dq.dim() == 2 else -1
    H = dims.n_heads
    _need(h, "h", dims.dtype, (B, d_model), dev)
    _need(w_dkv, "w_dkv", dims.dtype, (dims.d_latent, d_model), dev)
    _need(w_kr, "w_kr", dims.dtype, (dims.d_rope, d_model), dev)
    _need(w_dq, "w_dq", dims.dtype, (d_q, d_model), dev)
    _need(w_uq, "w_uq", dims.dtype, (H * dims.d_nope, d_q), dev)
    _need(w_qr, "w_qr", dims.dtype, (H * dims.d_rope, d_q), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_ov, "w_ov", dims.dtype, (d_model, H * dims.d_latent), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if u is None:
        u = torch.empty((B, d_model), dtype=dims.dtype, device=dev)
    _need(u, "u", dims.dtype, (B, d_model), dev)
    need = decode_hidden_workspace_size(dims, B, d_model, d_q, n_workgroups)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(seq_lens), d_model, d_q, _ptr(h),
            _ptr(w_dkv), _ptr(w_kr), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(w_uk), _ptr(w_ov),
            _ptr(u), _ptr(workspace), wbytes, n_workgroups]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_decode_layer_merged, args, keep=(d, cache, seq_lens, h, w_dkv, w_kr, w_dq,
                                                               w_uq, w_qr, w_uk, w_ov, u, workspace, evs,
                                                               pool, page_table))
    if prepare:
        return call, u
    call(stream)
    return u


def prefill_workspace_size(dims: Dims, batch: int, seq_len: int) -> int:
    d = dims._c()
    return int(load().mla_prefill_workspace_size(ctypes.byref(d), batch, seq_len))


def prefill(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, q_nope: torch.Tensor,
            q_rope: torch.Tensor, c_kv: torch.Tensor, k_rope: torch.Tensor, w_uk: torch.Tensor,
            w_uv: torch.Tensor, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, stream=None, timing_events=None,
            prepare: bool = False):
    """Un-absorbed causal prefill (mla_prefill); also writes the latent cache.
    timing_events and prepare as for decode()."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    B, T = q_nope.shape[0], q_nope.shape[1]
    H = dims.n_heads
    _need(q_nope, "q_nope", dims.dtype, (B, T, H, dims.d_nope), dev)
    _need(q_rope, "q_rope", dims.dtype, (B, T, H, dims.d_rope), dev)
    _need(c_kv, "c_kv", dims.dtype, (B, T, dims.d_latent), dev)
    _need(k_rope, "k_rope", dims.dtype, (B, T, dims.d_rope), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, T, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, T, H, dims.d_nope), dev)
    need = prefill_workspace_size(dims, B, T)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, T, _ptr(q_nope), _ptr(q_rope), _ptr(c_kv),
            _ptr(k_rope), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace), wbytes]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_prefill, args, keep=(d, cache, q_nope, q_rope, c_kv, k_rope, w_uk,
                                                   w_uv, out, workspace, evs))
    if prepare:
        return call, out
    call(stream)
    return out


def prefill_chunk_workspace_size(dims: Dims, batch: int, chunk_len: int, max_context: int,
                                 mode: int = CHUNK_AUTO) -> int:
    d = dims._c()
    return int(load().mla_prefill_chunk_workspace_size(ctypes.byref(d), batch, chunk_len, max_context,
                                                       int(mode)))


def prefill_chunk(dims: Dims, pool: torch.Tensor, page_table: torch.Tensor, start_pos: torch.Tensor,
                  q_nope: torch.Tensor, q_rope: torch.Tensor, c_kv: torch.Tensor, k_rope: torch.Tensor,
                  w_uk: torch.Tensor, w_uv: torch.Tensor, max_context: int, mode: int = 0,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
                  timing_events=None, prepare: bool = False):
    """Chunked prefill over an existing latent cache (mla_prefill_chunk): chunk
    row t of sequence b sits at position start_pos[b] + t and attends every
    position up to its own.  start_pos: int32 [batch] on the device;
    max_context bounds start_pos[b] + chunk_len.  Tensors as for prefill with
    seq_len = chunk_len; mode: CHUNK_AUTO, CHUNK_EXPAND or CHUNK_ABSORB
    (mla_chunk_mode); timing_events and prepare as for decode()."""
    lib = load()
    cache = _cache(dims, pool, page_table)
    dev = pool.device
    B, T = q_nope.shape[0], q_nope.shape[1]
    H = dims.n_heads
    _need(q_nope, "q_nope", dims.dtype, (B, T, H, dims.d_nope), dev)
    _need(q_rope, "q_rope", dims.dtype, (B, T, H, dims.d_rope), dev)
    _need(c_kv, "c_kv", dims.dtype, (B, T, dims.d_latent), dev)
    _need(k_rope, "k_rope", dims.dtype, (B, T, dims.d_rope), dev)
    _need(w_uk, "w_uk", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(w_uv, "w_uv", dims.dtype, (H, dims.d_nope, dims.d_latent), dev)
    _need(start_pos, "start_pos", torch.int32, (B,), dev)
    if page_table.shape[0] < B:
        raise ValueError("page_table has fewer rows than the batch")
    if out is None:
        out = torch.empty((B, T, H, dims.d_nope), dtype=dims.dtype, device=dev)
    _need(out, "out", dims.dtype, (B, T, H, dims.d_nope), dev)
    need = prefill_chunk_workspace_size(dims, B, T, max_context, mode)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = dims._c()
    args = [ctypes.byref(d), ctypes.byref(cache), B, _ptr(start_pos), T, int(max_context), int(mode), _ptr(q_nope),
            _ptr(q_rope), _ptr(c_kv), _ptr(k_rope), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace),
            wbytes]
    evs = _events(timing_events)
    args.append(evs.ptr)
    call = _Prepared(lib.mla_prefill_chunk, args, keep=(d, cache, start_pos, q_nope, q_rope, c_kv,
                                                         k_rope, w_uk, w_uv, out, workspace, evs, pool,
                                                         page_table))
    if prepare:
        return call, out
    call(stream)
    return out

