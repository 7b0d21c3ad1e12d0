"""TurboQuant KV-cache store and speculative verification attention on
AMD Instinct MI355X (gfx950).

This module is a thin ctypes binding of ``libtqkv.so`` (C ABI in
``include/tqkv.h``).  Every step of the computation runs in the library's HIP
kernels; Python only marshals arguments.  PyTorch provides device memory and
the current stream.  There is no fallback: if the library is missing or no
gfx950 device is current, calls raise.

Names mirror the C entry points::

    tqkv_slot_bytes(preset)                 tqkv_block_bytes(preset)
    tqkv_cache_bytes(preset, B, Hk, D, max_seq)
    tqkv_store(cache, K, V, seq_idx, pos)
    tqkv_verify_num_splits(cache, n_spec, Hq, num_splits)
    tqkv_verify_workspace_bytes(cache, n_spec, Hq, num_splits)
    tqkv_verify(cache, Q, seq_lens, n_spec, Hq, causal, ...)
    tqkv_verify_noalloc(cache, Q, seq_lens, n_spec, Hq, causal, ...)
    tqkv_store_verify(cache, K, V, Q, seq_lens, n_spec, Hq, causal, ...)
    tqkv_verify_varlen(cache, Q, cu_q, max_q, seq_lens, Hq, causal, ...)
    tqkv_paged_cache_bytes(preset, Hk, D, num_pages)
    tqkv_paged_store(paged, K, V, slot_mapping)
    tqkv_paged_verify_num_splits / tqkv_paged_verify_workspace_bytes /
    tqkv_paged_verify / tqkv_paged_verify_varlen / tqkv_paged_store_verify
        (paged, ...): the verify calls above on a paged cache
    tqkv_status_string(status)              tqkv_version()

``Cache`` owns a contiguous cache's device buffer and the descriptor the C
calls take; ``PagedCache`` owns a page pool and holds the block table of
the current batch.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "K8V4", "K3V4_NC", "K4V4_NC", "HEAD_DIM", "BLOCK_TOKENS", "MAX_QLEN", "TqkvError", "Cache", "PagedCache",
    "library_path", "tqkv_slot_bytes", "tqkv_block_bytes", "tqkv_cache_bytes", "tqkv_store",
    "tqkv_verify_num_splits", "tqkv_verify_workspace_bytes", "tqkv_verify", "tqkv_verify_noalloc",
    "tqkv_store_verify", "NOALLOC_SCRATCH_BYTES",
    "tqkv_verify_varlen", "tqkv_paged_cache_bytes", "tqkv_paged_store", "tqkv_paged_verify_num_splits",
    "tqkv_paged_verify_workspace_bytes", "tqkv_paged_verify", "tqkv_paged_verify_varlen",
    "tqkv_paged_store_verify", "tqkv_status_string", "tqkv_version",
]

K8V4 = 1
K3V4_NC = 2
K4V4_NC = 3
HEAD_DIM = 128
BLOCK_TOKENS = 16
MAX_QLEN = 128
NOALLOC_SCRATCH_BYTES = 8 << 20
Q_F32 = 0
Q_F16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libtqkv.so")


class TqkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (status %d)" % (where, tqkv_status_string(status), status))
        self.status = status


class _CacheDesc(ctypes.Structure):
    _fields_ = [("preset", ctypes.c_int32), ("B", ctypes.c_int32), ("Hk", ctypes.c_int32),
                ("D", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("base", ctypes.c_void_p)]


class _PagedDesc(ctypes.Structure):
    _fields_ = [("preset", ctypes.c_int32), ("Hk", ctypes.c_int32), ("D", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("base", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError("libtqkv.so not found at %s; build it with __graft_entry__.build()"
                          % library_path)
    L = ctypes.CDLL(library_path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    S = ctypes.c_size_t
    D = ctypes.POINTER(_CacheDesc)
    L.tqkv_slot_bytes.argtypes = [I]
    L.tqkv_slot_bytes.restype = S
    L.tqkv_block_bytes.argtypes = [I]
    L.tqkv_block_bytes.restype = S
    L.tqkv_cache_bytes.argtypes = [I, I, I, I, I]
    L.tqkv_cache_bytes.restype = S
    L.tqkv_store.argtypes = [D, P, P, P, P, I, P]
    L.tqkv_store.restype = I
    L.tqkv_verify_num_splits.argtypes = [D, I, I, I]
    L.tqkv_verify_num_splits.restype = I
    L.tqkv_verify_workspace_bytes.argtypes = [D, I, I, I, ctypes.POINTER(S)]
    L.tqkv_verify_workspace_bytes.restype = I
    L.tqkv_verify.argtypes = [D, P, I, P, I, I, I, I, ctypes.c_float, P, P, S, P]
    L.tqkv_verify.restype = I
    L.tqkv_verify_noalloc.argtypes = [D, P, I, P, I, I, I, I, ctypes.c_float, P, P]
    L.tqkv_verify_noalloc.restype = I
    L.tqkv_store_verify.argtypes = [D, P, P, P, I, P, I, I, I, I, ctypes.c_float, P, P, S, P]
    L.tqkv_store_verify.restype = I
    PD = ctypes.POINTER(_PagedDesc)
    F = ctypes.c_float
    L.tqkv_verify_varlen.argtypes = [D, P, I, P, I, P, I, I, I, F, P, P, S, P]
    L.tqkv_verify_varlen.restype = I
    L.tqkv_paged_cache_bytes.argtypes = [I, I, I, I]
    L.tqkv_paged_cache_bytes.restype = S
    L.tqkv_paged_store.argtypes = [PD, P, P, P, I, P]
    L.tqkv_paged_store.restype = I
    L.tqkv_paged_verify_num_splits.argtypes = [PD, I, I, I]
    L.tqkv_paged_verify_num_splits.restype = I
    L.tqkv_paged_verify_workspace_bytes.argtypes = [PD, I, I, I, ctypes.POINTER(S)]
    L.tqkv_paged_verify_workspace_bytes.restype = I
    L.tqkv_paged_verify.argtypes = [PD, P, I, P, I, I, I, I, F, P, P, S, P]
    L.tqkv_paged_verify.restype = I
    L.tqkv_paged_verify_varlen.argtypes = [PD, P, I, P, I, P, I, I, I, F, P, P, S, P]
    L.tqkv_paged_verify_varlen.restype = I
    L.tqkv_paged_store_verify.argtypes = [PD, P, P, P, I, P, I, I, I, I, F, P, P, S, P]
    L.tqkv_paged_store_verify.restype = I
    L.tqkv_status_string.argtypes = [I]
    L.tqkv_status_string.restype = ctypes.c_char_p
    L.tqkv_version.argtypes = []
    L.tqkv_version.restype = I
    _lib = L
    return L


def lib() -> ctypes.CDLL:
    """The loaded libtqkv.so (raises ImportError when it is not built)."""
    return _load()


# ---------------------------------------------------------------- sizes ---

def tqkv_slot_bytes(preset: int) -> int:
    return int(_load().tqkv_slot_bytes(preset))


def tqkv_block_bytes(preset: int) -> int:
    return int(_load().tqkv_block_bytes(preset))


def tqkv_cache_bytes(preset: int, B: int, Hk: int, D: int, max_seq: int) -> int:
    return int(_load().tqkv_cache_bytes(preset, B, Hk, D, max_seq))


def tqkv_paged_cache_bytes(preset: int, Hk: int, D: int, num_pages: int) -> int:
    return int(_load().tqkv_paged_cache_bytes(preset, Hk, D, num_pages))


def tqkv_status_string(status: int) -> str:
    return _load().tqkv_status_string(status).decode()


def tqkv_version() -> int:
    return int(_load().tqkv_version())


# ---------------------------------------------------------------- cache ---

class Cache:
    """A quantised KV cache in device memory (uint8 tensor) + its descriptor."""

    def __init__(self, preset: int, B: int, Hk: int, max_seq: int, device="cuda", buffer=None):
        nbytes = tqkv_cache_bytes(preset, B, Hk, HEAD_DIM, max_seq)
        if nbytes == 0:
            raise ValueError("invalid cache shape")
        if buffer is None:
            buffer = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        if buffer.dtype != torch.uint8 or buffer.numel() != nbytes or not buffer.is_contiguous():
            raise ValueError("cache buffer must be a contiguous uint8 tensor of %d bytes" % nbytes)
        self.preset, self.B, self.Hk, self.max_seq = preset, B, Hk, max_seq
        self.buffer = buffer
        self.desc = _CacheDesc(preset, B, Hk, HEAD_DIM, max_seq, buffer.data_ptr())

    @property
    def nbytes(self) -> int:
        return self.buffer.numel()


class PagedCache:
    """A page pool (uint8 tensor; page p holds head hk's 16-token block at
    byte (p * Hk + hk) * block bytes) + the block table of the current batch
    (int32 [B, max_pages] device tensor, set with ``set_block_table``)."""

    def __init__(self, preset: int, Hk: int, num_pages: int, device="cuda", buffer=None, block_table=None):
        nbytes = tqkv_paged_cache_bytes(preset, Hk, HEAD_DIM, num_pages)
        if nbytes == 0:
            raise ValueError("invalid pool shape")
        if buffer is None:
            buffer = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        if buffer.dtype != torch.uint8 or buffer.numel() != nbytes or not buffer.is_contiguous():
            raise ValueError("pool buffer must be a contiguous uint8 tensor of %d bytes" % nbytes)
        self.preset, self.Hk, self.num_pages = preset, Hk, num_pages
        self.buffer = buffer
        self.block_table = None
        self.B = 0
        self.desc = _PagedDesc(preset, Hk, HEAD_DIM, num_pages, buffer.data_ptr(), None, 0, 0)
        if block_table is not None:
            self.set_block_table(block_table)

    def set_block_table(self, block_table: torch.Tensor) -> None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor")
        if block_table.device != self.buffer.device:
            raise ValueError("block_table must be on the pool's device")
        self.block_table = block_table
        self.B = block_table.shape[0]
        self.desc.block_table = block_table.data_ptr()
        self.desc.B = block_table.shape[0]
        self.desc.max_pages = block_table.shape[1]

    @property
    def nbytes(self) -> int:
        return self.buffer.numel()


def _stream_ptr(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise TqkvError(status, where)


# ---------------------------------------------------------------- store ---

def tqkv_store(cache: Cache, K: torch.Tensor, V: torch.Tensor, seq_idx: torch.Tensor,
               pos: torch.Tensor, stream=None) -> None:
    """Quantise K, V (fp16 [T, Hk, 128], device) into ``cache`` at
    (seq_idx[t], pos[t]) (int32 [T], device); enqueued on ``stream``."""
    T = K.shape[0]
    if K.dtype != torch.float16 or V.dtype != torch.float16:
        raise TypeError("K and V must be float16")
    if K.shape != (T, cache.Hk, HEAD_DIM) or V.shape != K.shape:
        raise ValueError("K and V must have shape [T, Hk, 128]")
    if seq_idx.dtype != torch.int32 or pos.dtype != torch.int32:
        raise TypeError("seq_idx and pos must be int32")
    if seq_idx.shape != (T,) or pos.shape != (T,):
        raise ValueError("seq_idx and pos must have shape [T]")
    for x in (K, V, seq_idx, pos):
        if not x.is_contiguous() or x.device != cache.buffer.device:
            raise ValueError("tensors must be contiguous and on the cache's device")
    st = _load().tqkv_store(ctypes.byref(cache.desc), K.data_ptr(), V.data_ptr(), seq_idx.data_ptr(),
                            pos.data_ptr(), T, _stream_ptr(K, stream))
    _check(st, "tqkv_store")


# --------------------------------------------------------------- verify ---

def tqkv_verify_num_splits(cache: Cache, n_spec: int, Hq: int, num_splits: int = 0) -> int:
    return int(_load().tqkv_verify_num_splits(ctypes.byref(cache.desc), n_spec, Hq, num_splits))


def tqkv_verify_workspace_bytes(cache: Cache, n_spec: int, Hq: int, num_splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    st = _load().tqkv_verify_workspace_bytes(ctypes.byref(cache.desc), n_spec, Hq, num_splits,
                                             ctypes.byref(n))
    _check(st, "tqkv_verify_workspace_bytes")
    return int(n.value)


def _ws_bytes(cache, n_spec, Hq, num_splits):
    if isinstance(cache, PagedCache):
        return tqkv_paged_verify_workspace_bytes(cache, n_spec, Hq, num_splits)
    return tqkv_verify_workspace_bytes(cache, n_spec, Hq, num_splits)


def _verify_prep(cache, Q, seq_lens, n_spec, Hq, num_splits, out, workspace, cu_q=None, ws_needed=True):
    """Argument checks and defaults shared by the verify calls (dense Q
    [n_spec, B, Hq, 128], or ragged Q [cu_q[B], Hq, 128] when cu_q is given;
    ws_needed False: the call takes no workspace)."""
    if Q.dtype == torch.float32:
        qd = Q_F32
    elif Q.dtype == torch.float16:
        qd = Q_F16
    else:
        raise TypeError("Q must be float32 or float16")
    if isinstance(cache, PagedCache) and cache.block_table is None:
        raise ValueError("the paged cache has no block table")
    if cu_q is None:
        if Q.shape != (n_spec, cache.B, Hq, HEAD_DIM) or not Q.is_contiguous():
            raise ValueError("Q must be a contiguous [n_spec, B, Hq, 128] tensor")
    else:
        if cu_q.dtype != torch.int32 or cu_q.shape != (cache.B + 1,) or not cu_q.is_contiguous():
            raise ValueError("cu_q must be a contiguous int32 [B + 1] tensor")
        if Q.dim() != 3 or Q.shape[1:] != (Hq, HEAD_DIM) or not Q.is_contiguous():
            raise ValueError("Q must be a contiguous [rows, Hq, 128] tensor")
        if cu_q.device != Q.device:
            raise ValueError("cu_q must be on Q's device")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (cache.B,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    dev = cache.buffer.device
    if out is None:
        out = torch.empty(Q.shape, dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.shape != Q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like Q")
    # every buffer the kernels touch lives on the cache's device (a pointer
    # of another device, or of host memory, would be read by the kernels)
    for name, x in (("Q", Q), ("seq_lens", seq_lens), ("out", out), ("cu_q", cu_q), ("workspace", workspace)):
        if x is not None and x.device != dev:
            raise ValueError("%s must be on the cache's device (%s), not %s" % (name, dev, x.device))
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if ws_needed is False:
        return qd, out, None, 0
    need = _ws_bytes(cache, n_spec, Hq, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() if workspace is not None else 0
    return qd, out, ws_ptr, ws_len


def tqkv_verify(cache: Cache, Q: torch.Tensor, seq_lens: torch.Tensor, n_spec: int, Hq: int,
                causal: bool, num_splits: int = 0, sm_scale: float = 0.0,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """Verification attention; returns ``out`` (fp32 [n_spec, B, Hq, 128])."""
    if isinstance(cache, PagedCache):
        return tqkv_paged_verify(cache, Q, seq_lens, n_spec, Hq, causal, num_splits, sm_scale, out, workspace,
                                 stream)
    qd, out, ws_ptr, ws_len = _verify_prep(cache, Q, seq_lens, n_spec, Hq, num_splits, out, workspace)
    st = _load().tqkv_verify(ctypes.byref(cache.desc), Q.data_ptr(), qd, seq_lens.data_ptr(), n_spec,
                             Hq, int(bool(causal)), num_splits, float(sm_scale), out.data_ptr(),
                             ws_ptr, ws_len, _stream_ptr(Q, stream))
    _check(st, "tqkv_verify")
    return out


def tqkv_verify_noalloc(cache: Cache, Q: torch.Tensor, seq_lens: torch.Tensor, n_spec: int, Hq: int,
                        causal: bool, num_splits: int = 0, sm_scale: float = 0.0,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """tqkv_verify with the library's own per-device scratch array as the
    workspace: nothing is allocated (``out`` is required).  Raises
    TqkvError(TQKV_ERR_WORKSPACE) when the shape needs more than
    NOALLOC_SCRATCH_BYTES; calls that overlap on one device race on the
    array (issue them on one stream)."""
    if not isinstance(cache, Cache):
        raise TypeError("tqkv_verify_noalloc takes a contiguous Cache")
    if out is None:
        raise ValueError("tqkv_verify_noalloc needs a caller-provided out tensor")
    qd, out, _, _ = _verify_prep(cache, Q, seq_lens, n_spec, Hq, num_splits, out, None, ws_needed=False)
    st = _load().tqkv_verify_noalloc(ctypes.byref(cache.desc), Q.data_ptr(), qd, seq_lens.data_ptr(), n_spec,
                                     Hq, int(bool(causal)), num_splits, float(sm_scale), out.data_ptr(),
                                     _stream_ptr(Q, stream))
    _check(st, "tqkv_verify_noalloc")
    return out


def tqkv_store_verify(cache: Cache, K: torch.Tensor, V: torch.Tensor, Q: torch.Tensor, seq_lens: torch.Tensor,
                      n_spec: int, Hq: int, causal: bool, num_splits: int = 0, sm_scale: float = 0.0,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Store the n_spec new tokens of every sequence (K, V fp16 [n_spec, B, Hk, 128];
    token n of sequence b goes to position seq_lens[b] - n_spec + n) and run the
    verification attention in one launch; returns ``out``."""
    shape = (n_spec, cache.B, cache.Hk, HEAD_DIM)
    if K.dtype != torch.float16 or V.dtype != torch.float16:
        raise TypeError("K and V must be float16")
    if K.shape != shape or V.shape != shape or not K.is_contiguous() or not V.is_contiguous():
        raise ValueError("K and V must be contiguous [n_spec, B, Hk, 128] tensors")
    if K.device != cache.buffer.device or V.device != cache.buffer.device:
        raise ValueError("K and V must be on the cache's device")
    qd, out, ws_ptr, ws_len = _verify_prep(cache, Q, seq_lens, n_spec, Hq, num_splits, out, workspace)
    fn, name = ((_load().tqkv_paged_store_verify, "tqkv_paged_store_verify") if isinstance(cache, PagedCache)
                else (_load().tqkv_store_verify, "tqkv_store_verify"))
    st = fn(ctypes.byref(cache.desc), K.data_ptr(), V.data_ptr(), Q.data_ptr(), qd,
            seq_lens.data_ptr(), n_spec, Hq, int(bool(causal)), num_splits,
            float(sm_scale), out.data_ptr(), ws_ptr, ws_len, _stream_ptr(Q, stream))
    _check(st, name)
    return out


def tqkv_verify_varlen(cache: Cache, Q: torch.Tensor, cu_q: torch.Tensor, max_q: int, seq_lens: torch.Tensor,
                       Hq: int, causal: bool, num_splits: int = 0, sm_scale: float = 0.0,
                       out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """Verification attention with q_b = cu_q[b+1] - cu_q[b] queries for
    sequence b (rows cu_q[b].. of Q [rows, Hq, 128]); returns ``out``."""
    qd, out, ws_ptr, ws_len = _verify_prep(cache, Q, seq_lens, max_q, Hq, num_splits, out, workspace, cu_q)
    fn, name = ((_load().tqkv_paged_verify_varlen, "tqkv_paged_verify_varlen") if isinstance(cache, PagedCache)
                else (_load().tqkv_verify_varlen, "tqkv_verify_varlen"))
    st = fn(ctypes.byref(cache.desc), Q.data_ptr(), qd, cu_q.data_ptr(), max_q, seq_lens.data_ptr(), Hq,
            int(bool(causal)), num_splits, float(sm_scale), out.data_ptr(), ws_ptr, ws_len, _stream_ptr(Q, stream))
    _check(st, name)
    return out


# ---------------------------------------------------------------- paged ---

def tqkv_paged_store(cache: PagedCache, K: torch.Tensor, V: torch.Tensor, slot_mapping: torch.Tensor,
                     stream=None) -> None:
    """Quantise K, V (fp16 [T, Hk, 128], device) into the pool at
    slot_mapping[t] = page * 16 + position (int32 [T]; negative = skip)."""
    T = K.shape[0]
    if K.dtype != torch.float16 or V.dtype != torch.float16:
        raise TypeError("K and V must be float16")
    if K.shape != (T, cache.Hk, HEAD_DIM) or V.shape != K.shape:
        raise ValueError("K and V must have shape [T, Hk, 128]")
    if slot_mapping.dtype != torch.int32 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be an int32 [T] tensor")
    for x in (K, V, slot_mapping):
        if not x.is_contiguous() or x.device != cache.buffer.device:
            raise ValueError("tensors must be contiguous and on the pool's device")
    st = _load().tqkv_paged_store(ctypes.byref(cache.desc), K.data_ptr(), V.data_ptr(), slot_mapping.data_ptr(),
                                  T, _stream_ptr(K, stream))
    _check(st, "tqkv_paged_store")


def tqkv_paged_verify_num_splits(cache: PagedCache, n_spec: int, Hq: int, num_splits: int = 0) -> int:
    return int(_load().tqkv_paged_verify_num_splits(ctypes.byref(cache.desc), n_spec, Hq, num_splits))


def tqkv_paged_verify_workspace_bytes(cache: PagedCache, n_spec: int, Hq: int, num_splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    st = _load().tqkv_paged_verify_workspace_bytes(ctypes.byref(cache.desc), n_spec, Hq, num_splits,
                                                   ctypes.byref(n))
    _check(st, "tqkv_paged_verify_workspace_bytes")
    return int(n.value)


def tqkv_paged_verify(cache: PagedCache, Q: torch.Tensor, seq_lens: torch.Tensor, n_spec: int, Hq: int,
                      causal: bool, num_splits: int = 0, sm_scale: float = 0.0,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """tqkv_verify on a paged cache (its current block table)."""
    qd, out, ws_ptr, ws_len = _verify_prep(cache, Q, seq_lens, n_spec, Hq, num_splits, out, workspace)
    st = _load().tqkv_paged_verify(ctypes.byref(cache.desc), Q.data_ptr(), qd, seq_lens.data_ptr(), n_spec,
                                   Hq, int(bool(causal)), num_splits, float(sm_scale), out.data_ptr(),
                                   ws_ptr, ws_len, _stream_ptr(Q, stream))
    _check(st, "tqkv_paged_verify")
    return out


def tqkv_paged_verify_varlen(cache: PagedCache, *args, **kw) -> torch.Tensor:
    """tqkv_verify_varlen on a paged cache."""
    if not isinstance(cache, PagedCache):
        raise TypeError("cache must be a PagedCache")
    return tqkv_verify_varlen(cache, *args, **kw)


def tqkv_paged_store_verify(cache: PagedCache, *args, **kw) -> torch.Tensor:
    """tqkv_store_verify on a paged cache."""
    if not isinstance(cache, PagedCache):
        raise TypeError("cache must be a PagedCache")
    return tqkv_store_verify(cache, *args, **kw)
