"""Thin Python binding of ``libdsa.so``, the MI355X (gfx950) DeepSeek Sparse Attention hot path.

Argument marshalling only: torch tensors are passed to the C ABI (``include/dsa.h``) as raw
device pointers together with the current HIP stream; every step of the computation runs in
the library's HIP kernels.  There is no fallback: if the library is missing, importing the
functions raises.

Entry points mirror the C ABI: ``indexer_scores``, ``topk``, ``sparse_mqa``, ``dense_mqa``,
``forward``, ``cache_append``, ``indexer_kl``, ``workspace_size`` / ``workspace_min`` / ``topk_workspace_size``.  A batch is described by its query and key row offsets
(``cu_q``, ``cu_k``: B + 1 integers); see ``include/dsa.h`` for the layouts.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = ["DsaError", "Dims", "Batch", "lib", "library_path", "indexer_scores", "topk",
           "topk_workspace_size", "indexer_scores_counted", "topk_counted", "COUNT_BINS", "sparse_mqa", "dense_mqa", "forward", "forward_noalloc", "NOALLOC_SCRATCH_BYTES",
           "check_indices", "debug_flags", "IDX_OUT_OF_RANGE", "IDX_NOT_CAUSAL", "IDX_NOT_SORTED", "IDX_BAD_PAGE",
           "cache_append", "indexer_kl",
           "workspace_size", "workspace_min", "PROD_DIMS", "TINY_DIMS", "PAGE_SIZE", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsa.so")
_lib = None

STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
          4: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Dims(ctypes.Structure):
    _fields_ = [("n_idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("sm_scale", ctypes.c_float)]

    @classmethod
    def of(cls, d) -> "Dims":
        """From any object with the same attribute names (e.g. dsa_inputs.Dims)."""
        return cls(d.n_idx_heads, d.idx_dim, d.topk, d.n_heads, d.qk_dim, d.v_dim, d.sm_scale)


class _CBatch(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("cu_q_host", ctypes.c_void_p),
                ("cu_k_host", ctypes.c_void_p), ("cu_q_dev", ctypes.c_void_p),
                ("cu_k_dev", ctypes.c_void_p), ("page_table_dev", ctypes.c_void_p),
                ("pages_per_seq", ctypes.c_int32), ("pool_rows", ctypes.c_int64)]


PAGE_SIZE = 64  # positions per cache page (DSA_PAGE_SIZE)


class Batch:
    """Sequence offsets in host and device memory, kept alive together.

    page_table: optional int32 array [B, pages_per_seq] of page ids; the caches are then paged
    (position p of sequence b is cache row page_table[b, p // 64] * 64 + p % 64) in a pool of
    pool_rows rows (0: not given; the gathers then trust the page ids)."""

    def __init__(self, cu_q, cu_k, device="cuda", page_table=None, pool_rows=0):
        self.cu_q = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int32))
        self.cu_k = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int32))
        if self.cu_q.shape != self.cu_k.shape or self.cu_q.ndim != 1 or len(self.cu_q) < 2:
            raise ValueError("cu_q and cu_k must be 1-D with the same length >= 2")
        self.cu_q_dev = torch.from_numpy(self.cu_q).to(device)
        self.cu_k_dev = torch.from_numpy(self.cu_k).to(device)
        self.page_table_dev = None
        pps = 0
        if page_table is not None:
            pt = torch.as_tensor(page_table, dtype=torch.int32)
            if pt.ndim != 2 or pt.shape[0] != len(self.cu_q) - 1:
                raise ValueError("page_table must be [n_seqs, pages_per_seq]")
            self.page_table_dev = pt.contiguous().to(device)
            pps = int(pt.shape[1])
        self.c = _CBatch(len(self.cu_q) - 1, self.cu_q.ctypes.data, self.cu_k.ctypes.data,
                         self.cu_q_dev.data_ptr(), self.cu_k_dev.data_ptr(),
                         None if self.page_table_dev is None else self.page_table_dev.data_ptr(), pps,
                         int(pool_rows))

    @property
    def n_seqs(self) -> int:
        return len(self.cu_q) - 1

    @property
    def n_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def n_k(self) -> int:
        return int(self.cu_k[-1])

    @property
    def max_len_k(self) -> int:
        return int(np.diff(self.cu_k).max())


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded ``libdsa.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_long_lightning_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, S, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
        st = ctypes.c_int
        for name, args in {
            "dsa_workspace_size": [P, P, P],
            "dsa_workspace_min": [P, P, P],
            "dsa_indexer_scores": [P, P, P, P, P, P, P, P, I64, P],
            "dsa_topk": [P, P, P, I64, P, P, S, P],
            "dsa_topk_workspace_size": [P, P, P],
            "dsa_indexer_scores_counted": [P, P, P, P, P, P, P, P, I64, P, P],
            "dsa_topk_counted": [P, P, P, I64, P, P, P],
            "dsa_sparse_mqa": [P, P, P, P, P, P, P, P, S, P],
            "dsa_dense_mqa": [P, P, P, P, P, P, P, S, P],
            "dsa_forward": [P, P, P, P, P, P, P, P, P, P, P, P, P, S, P],
            "dsa_forward_noalloc": [P, P, P, P, P, P, P, P, P, P, P, P, P],
            "dsa_check_indices": [P, P, P, P, P],
            "dsa_debug_flags": [P, ctypes.c_int],
            "dsa_indexer_kl": [P, P, P, P, P, P, P, I64, P, P, P],
            "dsa_cache_append": [P, P, P, P, P, P, P, ctypes.c_int32, P, P, P, P, P, P],
        }.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = st
        L.dsa_status_string.argtypes = [st]
        L.dsa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise DsaError(status, where)


def _dims(dims) -> Dims:
    return dims if isinstance(dims, Dims) else Dims.of(dims)


def workspace_size(dims, batch: Batch) -> int:
    out = ctypes.c_size_t(0)
    d = _dims(dims)
    _check(lib().dsa_workspace_size(ctypes.byref(d), ctypes.byref(batch.c), ctypes.byref(out)),
           "dsa_workspace_size")
    return int(out.value)


def workspace_min(dims, batch: Batch) -> int:
    out = ctypes.c_size_t(0)
    d = _dims(dims)
    _check(lib().dsa_workspace_min(ctypes.byref(d), ctypes.byref(batch.c), ctypes.byref(out)),
           "dsa_workspace_min")
    return int(out.value)


def indexer_scores(dims, batch: Batch, q8, q_scale, w, k8, k_scale, scores, score_stride: int,
                   stream=None):
    d = _dims(dims)
    _check(lib().dsa_indexer_scores(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q8), _ptr(q_scale),
                                    _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(scores),
                                    int(score_stride), _stream(stream)), "dsa_indexer_scores")
    return scores


COUNT_BINS = 1024  # per-row score counts of the fused indexer -> top-k (DSA_COUNT_BINS)


def indexer_scores_counted(dims, batch: Batch, q8, q_scale, w, k8, k_scale, scores, score_stride: int,
                           counts, stream=None):
    """indexer_scores for a prefill batch, also filling counts [T, COUNT_BINS] (uint32 / int32)."""
    d = _dims(dims)
    _check(lib().dsa_indexer_scores_counted(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q8), _ptr(q_scale),
                                            _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(scores), int(score_stride),
                                            _ptr(counts), _stream(stream)), "dsa_indexer_scores_counted")
    return scores, counts


def topk_counted(dims, batch: Batch, scores, score_stride: int, counts, idx, stream=None):
    """topk starting from the counts of indexer_scores_counted (one read of each row)."""
    d = _dims(dims)
    _check(lib().dsa_topk_counted(ctypes.byref(d), ctypes.byref(batch.c), _ptr(scores), int(score_stride),
                                  _ptr(counts), _ptr(idx), _stream(stream)), "dsa_topk_counted")
    return idx


def topk_workspace_size(dims, batch: Batch) -> int:
    out = ctypes.c_size_t(0)
    d = _dims(dims)
    _check(lib().dsa_topk_workspace_size(ctypes.byref(d), ctypes.byref(batch.c), ctypes.byref(out)),
           "dsa_topk_workspace_size")
    return int(out.value)


def topk(dims, batch: Batch, scores, score_stride: int, idx, ws=None, stream=None):
    """ws: optional uint8 device tensor of at least topk_workspace_size bytes (rows are then
    split over several workgroups); None selects each row with one workgroup."""
    d = _dims(dims)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_topk(ctypes.byref(d), ctypes.byref(batch.c), _ptr(scores), int(score_stride),
                          _ptr(idx), _ptr(ws), ws_bytes, _stream(stream)), "dsa_topk")
    return idx


def sparse_mqa(dims, batch: Batch, q, kv, idx, out, lse=None, ws=None, stream=None):
    d = _dims(dims)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_sparse_mqa(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q), _ptr(kv),
                                _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                _stream(stream)), "dsa_sparse_mqa")
    return out


def dense_mqa(dims, batch: Batch, q, kv, out, lse=None, ws=None, stream=None):
    """Causal attention of every query row over all earlier positions of its sequence."""
    d = _dims(dims)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_dense_mqa(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q), _ptr(kv), _ptr(out),
                               _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)), "dsa_dense_mqa")
    return out


def forward(dims, batch: Batch, q8, q_scale, w, k8, k_scale, q, kv, out, lse=None, idx_out=None,
            ws=None, stream=None):
    d = _dims(dims)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_forward(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q8), _ptr(q_scale),
                             _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(q), _ptr(kv), _ptr(out),
                             _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)),
           "dsa_forward")
    return out


IDX_OUT_OF_RANGE, IDX_NOT_CAUSAL, IDX_NOT_SORTED, IDX_BAD_PAGE = 1, 2, 4, 8  # DSA_IDX_* row flags


def check_indices(dims, batch: Batch, idx, row_flags, stream=None):
    """Flags of each index row (DSA_IDX_* bits, 0 for a row dsa_topk could have written)."""
    d = _dims(dims)
    _check(lib().dsa_check_indices(ctypes.byref(d), ctypes.byref(batch.c), _ptr(idx), _ptr(row_flags),
                                   _stream(stream)), "dsa_check_indices")
    return row_flags


def debug_flags(clear: bool = True) -> int:
    """The current device's DSA_DEBUG_CHECKS flag word (waits for the device)."""
    out = ctypes.c_uint32(0)
    _check(lib().dsa_debug_flags(ctypes.byref(out), int(clear)), "dsa_debug_flags")
    return int(out.value)


NOALLOC_SCRATCH_BYTES = 64 << 20  # DSA_NOALLOC_SCRATCH_BYTES


def forward_noalloc(dims, batch: Batch, q8, q_scale, w, k8, k_scale, q, kv, out, lse=None, idx_out=None,
                    stream=None):
    """dsa_forward with the library's fixed per-device scratch array as its workspace."""
    d = _dims(dims)
    _check(lib().dsa_forward_noalloc(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q8), _ptr(q_scale),
                                     _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(q), _ptr(kv), _ptr(out),
                                     _ptr(lse), _ptr(idx_out), _stream(stream)),
           "dsa_forward_noalloc")
    return out


PROD_DIMS = Dims(64, 128, 2048, 128, 576, 512, 1.0 / np.sqrt(192.0))
TINY_DIMS = Dims(4, 32, 32, 8, 80, 64, 1.0 / np.sqrt(80.0))


def indexer_kl(dims, batch: Batch, q, kv, lse, idx, scores, score_stride: int, kl, kl_rev=None,
               stream=None):
    """KL(P || softmax(I)) (and the reverse when kl_rev is given) per query row, P the
    heads-summed attention over the row's slots (idx rows, or every earlier position when
    idx is None)."""
    d = _dims(dims)
    _check(lib().dsa_indexer_kl(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q), _ptr(kv), _ptr(lse),
                                _ptr(idx), _ptr(scores), int(score_stride), _ptr(kl), _ptr(kl_rev),
                                _stream(stream)), "dsa_indexer_kl")
    return kl


def cache_append(dims, batch: Batch, q_idx, k_idx, kv_new, rope_cos, rope_sin, q8, q_scale,
                 k8_cache, k_scale_cache, kv_cache=None, stream=None):
    """RoPE + FP8 codes of the new tokens' indexer query and key; the key codes, scale and
    (if kv_new is given) latent row are written at each new token's cache row."""
    d = _dims(dims)
    _check(lib().dsa_cache_append(ctypes.byref(d), ctypes.byref(batch.c), _ptr(q_idx), _ptr(k_idx),
                                  _ptr(kv_new), _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.shape[0]),
                                  _ptr(q8), _ptr(q_scale), _ptr(k8_cache), _ptr(k_scale_cache),
                                  _ptr(kv_cache), _stream(stream)), "dsa_cache_append")
    return q8, q_scale
