"""Zigzag context-parallel prefill attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libcpattn.so`` (declared in
``include/cpattn.h``).  This module only marshals arguments: it checks
dtypes, devices and shapes, passes raw pointers and the current HIP stream,
and raises ``CpError`` with the library's message on a non-zero status.  All
computation happens in the library (host metadata builder and HIP kernels);
there is no CPU fallback -- if the library is missing, every call raises.

PyTorch is used for device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "CpError", "Meta", "MetaBuffers", "meta_build", "allgather_meta_build", "allgather_packed_meta_build", "zigzag_rerange",
    "zigzag_rerange_kv", "kv_scatter", "prefill_attn", "load_library", "LIB_PATH",
    "GATHERED_TO_ORIG", "ORIG_TO_GATHERED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

CP_OK = 0
CP_ERR_INVALID_ARG = -1
CP_ERR_UNSUPPORTED = -2
CP_ERR_BUFFER_TOO_SMALL = -3
CP_ERR_OVERFLOW = -4
CP_ERR_HIP = -5
META_ZIGZAG = 1
META_ALLGATHER = 2
GATHERED_TO_ORIG = 0
ORIG_TO_GATHERED = 1

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class CMeta(ctypes.Structure):
    """Mirror of ``cp_meta_t``."""
    _fields_ = [
        ("version", _i32), ("kind", _i32), ("cp_size", _i32), ("cp_rank", _i32), ("bs", _i32),
        ("attn_group", _i32), ("total_seq_lens", _i64), ("max_rank_len", _i32),
        ("total_q_prev_tokens", _i32), ("total_q_next_tokens", _i32),
        ("max_seqlen_q_prev", _i32), ("max_seqlen_q_next", _i32), ("n_local_rows", _i32),
        ("n_chunks", _i32), ("max_chunk_rows", _i32), ("n_seg", _i32), ("n_work", _i32),
        ("max_kv_len", _i32), ("q_tile", _i32), ("kv_align", _i32), ("mean_item_tiles", _i32),
        ("blob_bytes", _i64),
        ("off_split_list", _i64), ("off_zigzag_index", _i64), ("off_cp_reverse_index", _i64),
        ("off_reverse_split_len", _i64), ("off_per_rank_actual_token", _i64),
        ("off_kv_len_prev", _i64), ("off_kv_len_next", _i64), ("off_q_prev", _i64),
        ("off_q_next", _i64), ("off_cu_seqlens_q_prev", _i64), ("off_cu_seqlens_q_next", _i64),
        ("off_prefix", _i64), ("off_extend", _i64), ("off_chunks", _i64), ("off_segs", _i64),
        ("off_work", _i64),
    ]


class CpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"cpattn error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcpattn.so (built by ``context_prefill_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m context_prefill_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.cp_meta_build.argtypes = [_i32, _i32, _i32, P(_i32), P(_i32), _i64, _i32, _vp, _i64, P(CMeta)]
    lib.cp_allgather_meta_build.argtypes = [_i32, _i32, _i32, _i32, _vp, _i64, P(CMeta)]
    lib.cp_allgather_packed_meta_build.argtypes = [_i32, P(_i32), _i32, _i32, _i32, _vp, _i64, P(CMeta)]
    lib.cp_zigzag_rerange.argtypes = [_vp, P(CMeta), _i32, _vp, _vp, _i64, _vp]
    lib.cp_zigzag_rerange_kv.argtypes = [_vp, P(CMeta), _i32, _vp, _vp, _vp, _vp, _i64, _vp]
    lib.cp_kv_scatter.argtypes = [_vp, P(CMeta), _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                  _vp, _vp, _vp]
    lib.cp_prefill_attn.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, ctypes.c_float, _vp,
                                    P(CMeta), _i32, _i32, _vp, _vp, _vp]
    lib.cp_prefill_attn_noalloc.argtypes = lib.cp_prefill_attn.argtypes
    for fn in ("cp_meta_build", "cp_allgather_meta_build", "cp_allgather_packed_meta_build",
               "cp_zigzag_rerange", "cp_zigzag_rerange_kv", "cp_kv_scatter", "cp_prefill_attn",
               "cp_prefill_attn_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.cp_last_error.restype = ctypes.c_char_p
    lib.cp_last_error.argtypes = []
    lib.cp_version.restype = ctypes.c_char_p
    lib.cp_version.argtypes = []
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != CP_OK:
        raise CpError(rc, load_library().cp_last_error().decode())


def _i32_array(xs: Optional[Sequence[int]]):
    if xs is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(xs, dtype=np.int64))
    if arr.size and (arr.min() < -2**31 or arr.max() >= 2**31):
        raise CpError(CP_ERR_OVERFLOW, "length does not fit int32")
    arr = arr.astype(np.int32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(_i32))


class Meta:
    """Metadata of one call: the ``cp_meta_t`` summary, the host blob and,
    after ``to_device``, its device copy."""

    _LISTS = {
        "split_list": ("off_split_list", lambda m: m.bs * 2 * m.cp_size),
        "zigzag_index": ("off_zigzag_index", lambda m: 2 * m.bs),
        "cp_reverse_index": ("off_cp_reverse_index", lambda m: m.bs * 2 * m.cp_size),
        "reverse_split_len": ("off_reverse_split_len", lambda m: m.bs * 2 * m.cp_size),
        "per_rank_actual_token": ("off_per_rank_actual_token", lambda m: m.cp_size),
        "kv_len_prev": ("off_kv_len_prev", lambda m: m.bs),
        "kv_len_next": ("off_kv_len_next", lambda m: m.bs),
        "q_prev": ("off_q_prev", lambda m: m.bs),
        "q_next": ("off_q_next", lambda m: m.bs),
        "cu_seqlens_q_prev": ("off_cu_seqlens_q_prev", lambda m: m.bs + 1),
        "cu_seqlens_q_next": ("off_cu_seqlens_q_next", lambda m: m.bs + 1),
        "prefix": ("off_prefix", lambda m: m.bs),
        "extend": ("off_extend", lambda m: m.bs),
    }

    def __init__(self, cmeta: CMeta, blob: np.ndarray):
        self.c = cmeta
        self.blob = blob
        self.d_blob = None
        self._pinned = None

    def __getattr__(self, name):
        if name in Meta._LISTS:
            if self.c.kind != META_ZIGZAG:
                return []
            off_name, n = Meta._LISTS[name]
            off, cnt = getattr(self.c, off_name), n(self.c)
            return self.blob[off:off + 4 * cnt].view(np.int32).tolist()
        c = self.__dict__.get("c")
        if c is not None and name in dict(CMeta._fields_):
            return getattr(c, name)
        raise AttributeError(name)

    def to_device(self, device=None, non_blocking: bool = True, buffers: "Optional[MetaBuffers]" = None):
        """Copy the blob to device memory on the current stream (one H2D copy).

        Without ``buffers`` a pinned staging tensor and a device tensor are
        allocated for this metadata.  With ``buffers`` (a ``MetaBuffers``
        reused across calls) nothing is allocated once the buffers are large
        enough: the device copy lives in ``buffers`` until its next upload."""
        if buffers is not None:
            self.d_blob = buffers.upload(self.blob)
            return self
        import torch
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        pinned = torch.empty(self.blob.size, dtype=torch.uint8, pin_memory=True)
        pinned.numpy()[:] = self.blob
        d = torch.empty(self.blob.size, dtype=torch.uint8, device=dev)
        d.copy_(pinned, non_blocking=non_blocking)
        self._pinned = pinned  # keep the staging buffer alive with the metadata
        self.d_blob = d
        return self


class MetaBuffers:
    """Caller-owned staging for metadata blobs, reused call after call (the
    preallocated page-pointer array of the "Zigzag cp #3" pull request,
    instead of tensors built per call).

    Holds two pinned host buffers, used in turn, and one device buffer.  An
    upload waits (on the host) only until the copy that last read the pinned
    buffer it is about to refill has finished, i.e. when the GPU is two
    uploads behind; it then enqueues one asynchronous copy on the current
    stream.  The device buffer is overwritten by the next upload, so one
    ``MetaBuffers`` serves one live metadata at a time, and all its uploads
    and the kernels reading them must go to one stream.  Buffers grow (the
    only allocation) when a blob is larger than any before."""

    def __init__(self, device=None, capacity: int = 1 << 16):
        import torch
        self._torch = torch
        if device is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = torch.device(device)
        self._pin = self.device.type == "cuda"
        self.capacity = 0
        self._host = [None, None]
        self._events = [None, None]
        self._dev = None
        self._turn = 0
        self.grow_count = 0
        self._ensure(int(capacity))

    def _ensure(self, nbytes: int) -> None:
        if nbytes <= self.capacity:
            return
        torch = self._torch
        cap = max(nbytes, 2 * self.capacity)
        if self._pin:
            torch.cuda.current_stream(self.device).synchronize()   # old buffers may still be read
        self._host = [torch.empty(cap, dtype=torch.uint8, pin_memory=self._pin) for _ in range(2)]
        self._events = [None, None]
        self._dev = torch.empty(cap, dtype=torch.uint8, device=self.device)
        self.capacity = cap
        self.grow_count += 1

    def upload(self, blob: np.ndarray):
        """Stage ``blob`` and enqueue its copy to the device buffer; returns
        the device view holding it."""
        torch = self._torch
        n = int(blob.size)
        self._ensure(n)
        i = self._turn
        self._turn ^= 1
        ev = self._events[i]
        if ev is not None:
            ev.synchronize()          # the copy that last read this staging buffer is done
        host = self._host[i]
        host.numpy()[:n] = blob
        d = self._dev[:n]
        d.copy_(host[:n], non_blocking=self._pin)
        if self._pin:
            if ev is None:
                ev = self._events[i] = torch.cuda.Event()
            ev.record()
        return d


def meta_build(cp_size: int, cp_rank: int, extend_lens: Sequence[int],
               seq_lens: Optional[Sequence[int]] = None, num_tokens: Optional[int] = None,
               attn_group: int = 0, device=None, buffers: Optional[MetaBuffers] = None) -> Meta:
    """``cp_meta_build``: host-only zigzag metadata; ``device`` (or reusable
    ``buffers``) also copies it H2D."""
    lib = load_library()
    ext, ext_p = _i32_array(extend_lens)
    seq, seq_p = _i32_array(seq_lens)
    if seq is not None and seq.size != ext.size:
        raise CpError(CP_ERR_INVALID_ARG, "seq_lens and extend_lens differ in length")
    n_tok = int(sum(int(x) for x in extend_lens)) if num_tokens is None else int(num_tokens)
    cm = CMeta()
    _check(lib.cp_meta_build(cp_size, cp_rank, int(ext.size), ext_p, seq_p, n_tok, attn_group,
                             None, 0, ctypes.byref(cm)))
    blob = np.zeros(cm.blob_bytes, dtype=np.uint8)
    _check(lib.cp_meta_build(cp_size, cp_rank, int(ext.size), ext_p, seq_p, n_tok, attn_group,
                             blob.ctypes.data, blob.size, ctypes.byref(cm)))
    m = Meta(cm, blob)
    if buffers is not None:
        return m.to_device(buffers=buffers)
    return m.to_device(device) if device is not None else m


def allgather_meta_build(q_total: int, q_real: int, kv_len: int, attn_group: int,
                         device=None, buffers: Optional[MetaBuffers] = None) -> Meta:
    """``cp_allgather_meta_build``: metadata of the non-causal AllGather-KV share."""
    lib = load_library()
    cm = CMeta()
    _check(lib.cp_allgather_meta_build(q_total, q_real, kv_len, attn_group, None, 0, ctypes.byref(cm)))
    blob = np.zeros(cm.blob_bytes, dtype=np.uint8)
    _check(lib.cp_allgather_meta_build(q_total, q_real, kv_len, attn_group, blob.ctypes.data,
                                       blob.size, ctypes.byref(cm)))
    m = Meta(cm, blob)
    if buffers is not None:
        return m.to_device(buffers=buffers)
    return m.to_device(device) if device is not None else m


def allgather_packed_meta_build(doc_cu, q_start: int, q_total: int, attn_group: int,
                                device=None, buffers: Optional[MetaBuffers] = None) -> Meta:
    """``cp_allgather_packed_meta_build``: metadata of the non-causal
    AllGather-KV share of a packed global sequence (document boundaries
    ``doc_cu``; local query rows are global rows [q_start, q_start+q_total))."""
    lib = load_library()
    cu = np.ascontiguousarray(np.asarray(doc_cu, dtype=np.int32))
    if cu.ndim != 1 or cu.size < 2:
        raise CpError(CP_ERR_INVALID_ARG, "doc_cu must be 1-D with n_docs+1 >= 2 entries")
    cup = cu.ctypes.data_as(ctypes.POINTER(_i32))
    cm = CMeta()
    _check(lib.cp_allgather_packed_meta_build(cu.size - 1, cup, q_start, q_total, attn_group,
                                              None, 0, ctypes.byref(cm)))
    blob = np.zeros(cm.blob_bytes, dtype=np.uint8)
    _check(lib.cp_allgather_packed_meta_build(cu.size - 1, cup, q_start, q_total, attn_group,
                                              blob.ctypes.data, blob.size, ctypes.byref(cm)))
    m = Meta(cm, blob)
    if buffers is not None:
        return m.to_device(buffers=buffers)
    return m.to_device(device) if device is not None else m


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_tensor(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise CpError(CP_ERR_INVALID_ARG, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise CpError(CP_ERR_INVALID_ARG, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise CpError(CP_ERR_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need_device(meta: Meta):
    if meta.d_blob is None:
        raise CpError(CP_ERR_INVALID_ARG, "metadata has no device copy; call meta.to_device()")
    return ctypes.c_void_p(meta.d_blob.data_ptr())


def zigzag_rerange(meta: Meta, src, dst, direction: int = GATHERED_TO_ORIG) -> None:
    """``cp_zigzag_rerange`` on the current stream (rows = dim 0, any trailing shape)."""
    lib = load_library()
    row_bytes = src.element_size() * (src.numel() // max(src.shape[0], 1))
    if dst.element_size() * (dst.numel() // max(dst.shape[0], 1)) != row_bytes or src.dtype != dst.dtype:
        raise CpError(CP_ERR_INVALID_ARG, "src and dst rows differ")
    n_g = meta.cp_size * meta.max_rank_len
    rows_src, rows_dst = (n_g, meta.total_seq_lens) if direction == GATHERED_TO_ORIG else \
        (meta.total_seq_lens, n_g)
    if src.shape[0] != rows_src or dst.shape[0] != rows_dst:
        raise CpError(CP_ERR_INVALID_ARG, f"rows: src {src.shape[0]} (want {rows_src}), "
                                          f"dst {dst.shape[0]} (want {rows_dst})")
    _check(lib.cp_zigzag_rerange(_need_device(meta), ctypes.byref(meta.c), direction,
                                 _dev_tensor(src, "src"), _dev_tensor(dst, "dst"), row_bytes, _stream()))


def _rerange_rows(meta: Meta, src, dst, direction: int) -> int:
    row_bytes = src.element_size() * (src.numel() // max(src.shape[0], 1))
    if dst.element_size() * (dst.numel() // max(dst.shape[0], 1)) != row_bytes or src.dtype != dst.dtype:
        raise CpError(CP_ERR_INVALID_ARG, "src and dst rows differ")
    n_g = meta.cp_size * meta.max_rank_len
    rows_src, rows_dst = (n_g, meta.total_seq_lens) if direction == GATHERED_TO_ORIG else \
        (meta.total_seq_lens, n_g)
    if src.shape[0] != rows_src or dst.shape[0] != rows_dst:
        raise CpError(CP_ERR_INVALID_ARG, f"rows: src {src.shape[0]} (want {rows_src}), "
                                          f"dst {dst.shape[0]} (want {rows_dst})")
    return row_bytes


def zigzag_rerange_kv(meta: Meta, k_src, k_dst, v_src, v_dst, direction: int = GATHERED_TO_ORIG) -> None:
    """``cp_zigzag_rerange_kv`` on the current stream: K and V in one launch."""
    lib = load_library()
    row_bytes = _rerange_rows(meta, k_src, k_dst, direction)
    if _rerange_rows(meta, v_src, v_dst, direction) != row_bytes:
        raise CpError(CP_ERR_INVALID_ARG, "K and V rows differ")
    _check(lib.cp_zigzag_rerange_kv(_need_device(meta), ctypes.byref(meta.c), direction,
                                    _dev_tensor(k_src, "k_src"), _dev_tensor(k_dst, "k_dst"),
                                    _dev_tensor(v_src, "v_src"), _dev_tensor(v_dst, "v_dst"),
                                    row_bytes, _stream()))


def kv_scatter(meta: Meta, k_gathered, v_gathered, k_pool, v_pool, page_size: int,
               kv_page_indptr, kv_page_indices) -> None:
    """``cp_kv_scatter`` on the current stream."""
    import torch
    lib = load_library()
    num_pages, ps, h_kv, d = k_pool.shape
    if ps != page_size or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise CpError(CP_ERR_INVALID_ARG, "pool shape does not match page_size / each other")
    n_g = meta.cp_size * meta.max_rank_len
    for name, t in (("k_gathered", k_gathered), ("v_gathered", v_gathered)):
        if tuple(t.shape) != (n_g, h_kv, d):
            raise CpError(CP_ERR_INVALID_ARG, f"{name} shape {tuple(t.shape)} != {(n_g, h_kv, d)}")
    if kv_page_indptr.numel() != meta.bs + 1:
        raise CpError(CP_ERR_INVALID_ARG, "kv_page_indptr must have bs+1 entries")
    bf = torch.bfloat16
    _check(lib.cp_kv_scatter(
        _need_device(meta), ctypes.byref(meta.c),
        _dev_tensor(k_gathered, "k_gathered", bf), _dev_tensor(v_gathered, "v_gathered", bf),
        _dev_tensor(k_pool, "k_pool", bf), _dev_tensor(v_pool, "v_pool", bf),
        num_pages, page_size, h_kv, d,
        _dev_tensor(kv_page_indptr, "kv_page_indptr", torch.int32),
        _dev_tensor(kv_page_indices, "kv_page_indices", torch.int32), _stream()))


def prefill_attn(q, k_pool, v_pool, out, meta: Meta, scale: float, page_size: int,
                 kv_page_indptr, kv_page_indices, noalloc: bool = False) -> None:
    """``cp_prefill_attn`` on the current stream.

    q, out: [n_local_rows, H_q, D] bf16; k_pool, v_pool: [num_pages,
    page_size, H_kv, D] bf16 (a contiguous [S, H_kv, D] tensor can be viewed
    as pages with the identity page table).  The launch uses job counters in
    the header of ``meta.d_blob`` and leaves them zero, so two attention
    launches with the same device blob must not run concurrently.  With
    ``noalloc`` it calls ``cp_prefill_attn_noalloc``: the counters live in the
    library's per-device array instead and the blob is only read."""
    import torch
    lib = load_library()
    n, h_q, d = q.shape
    num_pages, ps, h_kv, d2 = k_pool.shape
    if ps != page_size or d2 != d or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise CpError(CP_ERR_INVALID_ARG, "pool shape does not match q / page_size")
    if n != meta.n_local_rows or tuple(out.shape) != tuple(q.shape):
        raise CpError(CP_ERR_INVALID_ARG, f"q rows {n} != metadata rows {meta.n_local_rows}")
    if kv_page_indptr.numel() != meta.bs + 1:
        raise CpError(CP_ERR_INVALID_ARG, "kv_page_indptr must have bs+1 entries")
    bf = torch.bfloat16
    fn = lib.cp_prefill_attn_noalloc if noalloc else lib.cp_prefill_attn
    _check(fn(
        _dev_tensor(q, "q", bf), _dev_tensor(k_pool, "k_pool", bf), _dev_tensor(v_pool, "v_pool", bf),
        _dev_tensor(out, "out", bf), h_q, h_kv, d, float(scale), _need_device(meta),
        ctypes.byref(meta.c), num_pages, page_size,
        _dev_tensor(kv_page_indptr, "kv_page_indptr", torch.int32),
        _dev_tensor(kv_page_indices, "kv_page_indices", torch.int32), _stream()))
