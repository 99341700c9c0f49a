"""Python binding of libdsa.so, the MI355X DeepSeek Sparse Attention hot path.

Thin ctypes marshalling over the C ABI in ``include/dsa.h``: each function checks the
torch tensors it is given (device, dtype, contiguity), passes raw device pointers and
the current HIP stream, and raises ``RuntimeError`` on a non-zero status.  All the
work runs in the HIP kernels of ``csrc/``; nothing here computes.

Build the library with ``python -m sparse_attention_08_amd.build`` (or
``__graft_entry__.build()``); importing this module without it fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
PAGE_SIZE = 64
MAX_TOPK = 2048
MFMA_PROBE_WAVES = 2048      # DSA_MFMA_PROBE_WAVES
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
          4: "DSA_ERR_HIP"}


class DsaRows(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32),
                ("row_seq", ctypes.c_void_p),
                ("row_len", ctypes.c_void_p),
                ("max_row_len", ctypes.c_int32),
                ("seq_start", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p),
                ("max_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libdsa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m sparse_attention_08_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    rows_p = ctypes.POINTER(DsaRows)
    lib.dsa_status_string.argtypes = [i32]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_mfma_rate_probe.argtypes = [i32, vp, vp]
    lib.dsa_mfma_rate_probe.restype = i32
    lib.dsa_abi_version.argtypes = []
    lib.dsa_abi_version.restype = i32
    for name in ("dsa_indexer_logits", "dsa_indexer_logits_paged"):
        f = getattr(lib, name)
        f.argtypes = [rows_p, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp]
        f.restype = i32
    for name in ("dsa_indexer_topk", "dsa_indexer_topk_paged"):
        f = getattr(lib, name)
        f.argtypes = [rows_p, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, i32, vp, vp, sz, vp]
        f.restype = i32
    lib.dsa_indexer_topk_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dsa_indexer_topk_workspace_size.restype = sz
    lib.dsa_topk_workspace_size.argtypes = [i32, i32, i32]
    lib.dsa_topk_workspace_size.restype = sz
    lib.dsa_topk.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.dsa_topk.restype = i32
    lib.dsa_sparse_mla_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dsa_sparse_mla_workspace_size.restype = sz
    for name in ("dsa_sparse_mla_decode", "dsa_sparse_mla_decode_paged", "dsa_sparse_mla_prefill",
                 "dsa_sparse_mla_prefill_paged"):
        f = getattr(lib, name)
        f.argtypes = [rows_p, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        f.restype = i32
    lib.dsa_sparse_attention_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.dsa_sparse_attention_decode_workspace_size.restype = sz
    for name in ("dsa_sparse_attention_decode", "dsa_sparse_attention_decode_paged"):
        f = getattr(lib, name)
        f.argtypes = [rows_p, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, i32, vp,
                      i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
        f.restype = i32
    lib.dsa_sparse_attention_decode_noalloc.argtypes = [
        rows_p, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, i32, vp,
        i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp]
    lib.dsa_sparse_attention_decode_noalloc.restype = i32
    lib.dsa_prep_cache_write.argtypes = [i32, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.dsa_prep_cache_write.restype = i32
    lib.dsa_prep_queries.argtypes = [i32, vp, vp, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.dsa_prep_queries.restype = i32
    lib.dsa_prep.argtypes = [i32, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                             vp, vp]
    lib.dsa_prep.restype = i32
    lib.dsa_prefill_dense_mode.argtypes = [i32, i32]
    lib.dsa_prefill_dense_mode.restype = i32
    lib.dsa_mha_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.dsa_mha_prefill_workspace_size.restype = sz
    for name in ("dsa_mha_prefill", "dsa_mha_prefill_paged"):
        f = getattr(lib, name)
        f.argtypes = [rows_p, i32, ctypes.c_float, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        f.restype = i32
    lib.dsa_sparse_attention_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.dsa_sparse_attention_prefill_workspace_size.restype = sz
    for name in ("dsa_sparse_attention_prefill", "dsa_sparse_attention_prefill_paged"):
        f = getattr(lib, name)
        f.argtypes = [rows_p, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, i32, vp, i32,
                      ctypes.c_float, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        f.restype = i32
    _lib = lib
    return lib


def mfma_rate_probe(iters: int, out=None):
    """Measurement aid: launch dsa_mfma_rate_probe (2048 waves x iters x 8 bf16 MFMAs of
    16x16x32) on the current stream; returns the [2048] output it writes (time it with events)."""
    lib = load_library()
    if out is None:
        out = torch.empty(MFMA_PROBE_WAVES, dtype=torch.float32, device="cuda")
    _dev(out, "out", (torch.float32,))
    _shape(out, "out", (MFMA_PROBE_WAVES,))
    _check(lib.dsa_mfma_rate_probe(int(iters), _ptr(out), _stream()), "dsa_mfma_rate_probe")
    return out


def abi_version() -> int:
    return int(load_library().dsa_abi_version())


def status_string(status: int) -> str:
    return load_library().dsa_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"{what}: {status_string(status)}")


def _stream() -> Optional[int]:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtypes=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _shape(t: Optional[torch.Tensor], name: str, shape):
    """Checks t's shape against `shape` (None entries match any size); t None passes."""
    if t is None:
        return
    ok = t.dim() == len(shape) and all(e is None or int(d) == int(e) for d, e in zip(t.shape, shape))
    if not ok:
        want = "[" + ", ".join("*" if e is None else str(int(e)) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _rows_of(rows: "Rows", t: torch.Tensor, name: str):
    if int(t.shape[0]) != rows.num_rows:
        raise ValueError(f"{name} has {int(t.shape[0])} rows, the batch has {rows.num_rows}")


def _logits_shape(rows: "Rows", logits: torch.Tensor):
    if logits.dim() != 2:
        raise ValueError("logits must be [R, ld]")
    _rows_of(rows, logits, "logits")
    if int(logits.shape[1]) < rows.max_row_len:
        raise ValueError(f"logits rows hold {int(logits.shape[1])} scores, max_row_len is "
                         f"{rows.max_row_len}")


def _key_cache_shape(rows: "Rows", k: torch.Tensor, D: int, k_scale):
    """Key cache [N, D] (contiguous) or [P, 64, D] (paged), and its [N] / [P, 64] scales."""
    if rows.paged:
        _shape(k, "k", (None, rows.page_size, D))
        _shape(k_scale, "k_scale", (int(k.shape[0]), rows.page_size))
    else:
        _shape(k, "k", (None, D))
        _shape(k_scale, "k_scale", (int(k.shape[0]),))


def _latent_cache_shape(rows: "Rows", kv: torch.Tensor, Dqk: int):
    if rows.paged:
        _shape(kv, "kv", (None, rows.page_size, Dqk))
    else:
        _shape(kv, "kv", (None, Dqk))


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


class Rows:
    """A ragged batch of query rows (device arrays plus the host-side sizes).

    Row r belongs to sequence ``row_seq[r]`` and sees positions ``0 .. row_len[r]-1``.
    Give ``seq_start`` for a contiguous cache or ``page_table`` for a 64-token paged cache.
    """

    def __init__(self, row_seq: torch.Tensor, row_len: torch.Tensor, max_row_len: int, num_seqs: int,
                 seq_start: Optional[torch.Tensor] = None, page_table: Optional[torch.Tensor] = None,
                 page_size: int = PAGE_SIZE):
        self.row_seq = _dev(row_seq, "row_seq", (torch.int32,))
        self.row_len = _dev(row_len, "row_len", (torch.int32,))
        self.seq_start = None if seq_start is None else _dev(seq_start, "seq_start", (torch.int64,))
        self.page_table = None if page_table is None else _dev(page_table, "page_table", (torch.int32,))
        self.max_row_len = int(max_row_len)
        self.num_seqs = int(num_seqs)
        self.page_size = int(page_size)
        self.max_pages = 0 if self.page_table is None else int(self.page_table.shape[-1])

    @property
    def num_rows(self) -> int:
        return int(self.row_seq.shape[0])

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    def struct(self) -> DsaRows:
        return DsaRows(self.num_rows, self.num_seqs, _ptr(self.row_seq), _ptr(self.row_len),
                       self.max_row_len, _ptr(self.seq_start), _ptr(self.page_table), self.max_pages,
                       self.page_size if self.paged else 0)


# --------------------------------------------------------------------------- stage 1

def _indexer_shapes(rows: Rows, q, w, k, logits, q_scale, k_scale):
    if q.dim() != 3:
        raise ValueError("q must be [R, H, D]")
    _rows_of(rows, q, "q")
    R, H, D = (int(x) for x in q.shape)
    _shape(w, "w", (R, H))
    _shape(q_scale, "q_scale", (R, H))
    _logits_shape(rows, logits)
    _key_cache_shape(rows, k, D, k_scale)


def _indexer(paged: bool, rows: Rows, q, w, k, logits, q_scale=None, k_scale=None):
    lib = load_library()
    _dev(q, "q")
    _dev(k, "k")
    _dev(w, "w", (torch.float32,))
    _dev(logits, "logits", (torch.float32,))
    if q_scale is not None:
        _dev(q_scale, "q_scale", (torch.float32,))
    if k_scale is not None:
        _dev(k_scale, "k_scale", (torch.float32,))
    _indexer_shapes(rows, q, w, k, logits, q_scale, k_scale)
    st = rows.struct()
    fn = lib.dsa_indexer_logits_paged if paged else lib.dsa_indexer_logits
    s = fn(ctypes.byref(st), dtype_code(q), int(q.shape[1]), int(q.shape[2]), _ptr(q), _ptr(q_scale),
           _ptr(k), _ptr(k_scale), _ptr(w), _ptr(logits), int(logits.shape[-1]), _stream())
    _check(s, "dsa_indexer_logits_paged" if paged else "dsa_indexer_logits")
    return logits


def indexer_logits(rows: Rows, q, w, k, logits, q_scale=None, k_scale=None):
    """Lightning-indexer scores into ``logits`` [R, ld] (contiguous key cache)."""
    return _indexer(False, rows, q, w, k, logits, q_scale, k_scale)


def indexer_logits_paged(rows: Rows, q, w, k, logits, q_scale=None, k_scale=None):
    """Lightning-indexer scores into ``logits`` [R, ld] (64-token paged key cache)."""
    return _indexer(True, rows, q, w, k, logits, q_scale, k_scale)


# --------------------------------------------------------------------------- stage 2

def topk_workspace_size(num_rows: int, max_row_len: int, k: int) -> int:
    return int(load_library().dsa_topk_workspace_size(int(num_rows), int(max_row_len), int(k)))


def topk(logits, row_len, k: int, max_row_len: int, idx=None, ws=None):
    """Top-k positions per row (ascending, -1 padded) into ``idx`` [R, k] int32."""
    lib = load_library()
    _dev(logits, "logits", (torch.float32,))
    _dev(row_len, "row_len", (torch.int32,))
    if logits.dim() != 2:
        raise ValueError("logits must be [R, ld]")
    R = int(logits.shape[0])
    _shape(row_len, "row_len", (R,))
    if int(logits.shape[1]) < int(max_row_len):
        raise ValueError(f"logits rows hold {int(logits.shape[1])} scores, max_row_len is {max_row_len}")
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=logits.device)
    _dev(idx, "idx", (torch.int32,))
    _shape(idx, "idx", (R, k))
    need = topk_workspace_size(R, max_row_len, k)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device=logits.device)   # zero before first use
    s = lib.dsa_topk(_ptr(logits), int(logits.shape[-1]), _ptr(row_len), R, int(max_row_len), int(k),
                     _ptr(idx), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check(s, "dsa_topk")
    return idx


# --------------------------------------------------------------------------- stages 1 + 2

def indexer_topk_workspace_size(num_rows: int, max_row_len: int, dtype, k: int) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(torch.empty(0, dtype=dtype))
    return int(load_library().dsa_indexer_topk_workspace_size(int(num_rows), int(max_row_len), code,
                                                              int(k)))


def indexer_topk(rows: Rows, q, w, k, logits, topk_k: int, idx=None, q_scale=None, k_scale=None,
                 ws=None):
    """Indexer scores into ``logits`` and their top-k positions into ``idx`` in one call."""
    lib = load_library()
    _dev(q, "q")
    _dev(k, "k")
    _dev(w, "w", (torch.float32,))
    _dev(logits, "logits", (torch.float32,))
    if q_scale is not None:
        _dev(q_scale, "q_scale", (torch.float32,))
    if k_scale is not None:
        _dev(k_scale, "k_scale", (torch.float32,))
    _indexer_shapes(rows, q, w, k, logits, q_scale, k_scale)
    R = rows.num_rows
    if idx is None:
        idx = torch.empty((R, topk_k), dtype=torch.int32, device=logits.device)
    _dev(idx, "idx", (torch.int32,))
    _shape(idx, "idx", (R, topk_k))
    need = indexer_topk_workspace_size(R, rows.max_row_len, dtype_code(q), topk_k)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    st = rows.struct()
    fn = lib.dsa_indexer_topk_paged if rows.paged else lib.dsa_indexer_topk
    s = fn(ctypes.byref(st), dtype_code(q), int(q.shape[1]), int(q.shape[2]), _ptr(q), _ptr(q_scale),
           _ptr(k), _ptr(k_scale), _ptr(w), _ptr(logits), int(logits.shape[-1]), int(topk_k), _ptr(idx),
           _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check(s, "dsa_indexer_topk_paged" if rows.paged else "dsa_indexer_topk")
    return idx


# --------------------------------------------------------------------------- stage 3

def sparse_mla_workspace_size(num_rows: int, n_heads: int, d_v: int, k: int) -> int:
    return int(load_library().dsa_sparse_mla_workspace_size(int(num_rows), int(n_heads), int(d_v),
                                                             int(k)))


def _mla(name: str, rows: Rows, q, kv, idx, scale: float, d_v: int, out=None, lse=None, ws=None):
    lib = load_library()
    _dev(q, "q", (torch.float32, torch.bfloat16))
    _dev(kv, "kv", (q.dtype,))
    _dev(idx, "idx", (torch.int32,))
    if q.dim() != 3:
        raise ValueError("q must be [R, H, d_qk]")
    _rows_of(rows, q, "q")
    R, H, Dqk = (int(x) for x in q.shape)
    _latent_cache_shape(rows, kv, Dqk)
    if idx.dim() != 2:
        raise ValueError("idx must be [R, k]")
    _shape(idx, "idx", (R, None))
    k = int(idx.shape[-1])
    if out is None:
        out = torch.empty((R, H, d_v), dtype=q.dtype, device=q.device)
    _dev(out, "out", (q.dtype,))
    _shape(out, "out", (R, H, d_v))
    if lse is not None:
        _dev(lse, "lse", (torch.float32,))
        _shape(lse, "lse", (R, H))
    if not name.startswith("dsa_sparse_mla_prefill"):
        need = sparse_mla_workspace_size(R, H, d_v, k)
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    else:
        ws = None
    st = rows.struct()
    s = getattr(lib, name)(ctypes.byref(st), dtype_code(q), H, Dqk, int(d_v), float(scale), _ptr(q),
                           _ptr(kv), _ptr(idx), k, _ptr(out), _ptr(lse), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check(s, name)
    return out


def sparse_mla_decode(rows: Rows, q, kv, idx, scale: float, d_v: int, out=None, lse=None, ws=None):
    """Sparse MLA (MQA mode) over idx entries, contiguous latent cache; returns out [R,H,d_v]."""
    return _mla("dsa_sparse_mla_decode", rows, q, kv, idx, scale, d_v, out, lse, ws)


def sparse_mla_decode_paged(rows: Rows, q, kv, idx, scale: float, d_v: int, out=None, lse=None,
                            ws=None):
    """Sparse MLA (MQA mode) over idx entries, 64-token paged latent cache."""
    return _mla("dsa_sparse_mla_decode_paged", rows, q, kv, idx, scale, d_v, out, lse, ws)


def sparse_mla_prefill(rows: Rows, q, kv, idx, scale: float, d_v: int, out=None, lse=None):
    """Sparse MLA (MQA mode) for many query rows (prefill), contiguous latent cache."""
    return _mla("dsa_sparse_mla_prefill", rows, q, kv, idx, scale, d_v, out, lse, None)


def sparse_mla_prefill_paged(rows: Rows, q, kv, idx, scale: float, d_v: int, out=None, lse=None):
    """Sparse MLA (MQA mode) for many query rows (prefill or a chunk over a cached prefix),
    64-token paged latent cache."""
    return _mla("dsa_sparse_mla_prefill_paged", rows, q, kv, idx, scale, d_v, out, lse, None)


# --------------------------------------------------------------------------- stages 1 + 2 + 3

def sparse_attention_decode_workspace_size(num_rows: int, max_row_len: int, idx_dtype, topk: int,
                                           n_heads: int, d_v: int) -> int:
    code = idx_dtype if isinstance(idx_dtype, int) else dtype_code(torch.empty(0, dtype=idx_dtype))
    return int(load_library().dsa_sparse_attention_decode_workspace_size(
        int(num_rows), int(max_row_len), code, int(topk), int(n_heads), int(d_v)))


def sparse_attention_decode(rows: Rows, q_idx, w, k_idx, logits, topk: int, q, kv, scale: float,
                            d_v: int, idx=None, out=None, lse=None, q_scale=None, k_scale=None,
                            ws=None, noalloc: bool = False):
    """Indexer scores, their top-k and the sparse MLA over it, in one call (decode).

    Fills ``logits`` and ``idx`` as :func:`indexer_topk` and returns ``out`` as
    :func:`sparse_mla_decode` (``_paged`` for a paged ``rows``) would on that ``idx``.
    ``noalloc``: call dsa_sparse_attention_decode_noalloc (contiguous rows, no ``ws``), whose
    scratch is the library's static per-GPU array.
    """
    lib = load_library()
    if noalloc and (rows.paged or ws is not None):
        raise ValueError("noalloc takes contiguous rows and no workspace")
    for t, n in ((q_idx, "q_idx"), (k_idx, "k_idx"), (kv, "kv")):
        _dev(t, n)
    _dev(w, "w", (torch.float32,))
    _dev(logits, "logits", (torch.float32,))
    _dev(q, "q", (torch.float32, torch.bfloat16))
    if q_scale is not None:
        _dev(q_scale, "q_scale", (torch.float32,))
    if k_scale is not None:
        _dev(k_scale, "k_scale", (torch.float32,))
    if q_idx.dim() != 3 or q.dim() != 3:
        raise ValueError("q_idx must be [R, H_I, D_I] and q [R, H, d_qk]")
    _indexer_shapes(rows, q_idx, w, k_idx, logits, q_scale, k_scale)
    _rows_of(rows, q, "q")
    R, H, Dqk = (int(x) for x in q.shape)
    _latent_cache_shape(rows, kv, Dqk)
    if idx is None:
        idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
    _dev(idx, "idx", (torch.int32,))
    _shape(idx, "idx", (R, topk))
    if out is None:
        out = torch.empty((R, H, d_v), dtype=q.dtype, device=q.device)
    _dev(out, "out", (q.dtype,))
    _shape(out, "out", (R, H, d_v))
    if lse is not None:
        _dev(lse, "lse", (torch.float32,))
        _shape(lse, "lse", (R, H))
    st = rows.struct()
    if noalloc:
        s = lib.dsa_sparse_attention_decode_noalloc(
            ctypes.byref(st), dtype_code(q_idx), int(q_idx.shape[1]), int(q_idx.shape[2]),
            _ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), _ptr(logits),
            int(logits.shape[-1]), int(topk), _ptr(idx), dtype_code(q), H, Dqk, int(d_v),
            float(scale), _ptr(q), _ptr(kv), _ptr(out), _ptr(lse), _stream())
        _check(s, "dsa_sparse_attention_decode_noalloc")
        return out
    need = sparse_attention_decode_workspace_size(R, rows.max_row_len, dtype_code(q_idx), topk, H, d_v)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    name = "dsa_sparse_attention_decode_paged" if rows.paged else "dsa_sparse_attention_decode"
    s = getattr(lib, name)(
        ctypes.byref(st), dtype_code(q_idx), int(q_idx.shape[1]), int(q_idx.shape[2]), _ptr(q_idx),
        _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), _ptr(logits), int(logits.shape[-1]),
        int(topk), _ptr(idx), dtype_code(q), H, Dqk, int(d_v), float(scale), _ptr(q), _ptr(kv),
        _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check(s, name)
    return out


# --------------------------------------------------------------------------- input prep

def prep_cache_write(positions, cache_rows, cos_sin, k_idx_in, k_idx_cache, kv_in, kv_cache,
                     k_idx_scale=None):
    """RoPE + (fp8) quantisation + cache write for new tokens: indexer keys ``k_idx_in``
    [T, 128] bf16 into ``k_idx_cache`` (bf16, or fp8 e4m3 / uint8 with ``k_idx_scale``) and
    latent entries ``kv_in`` [T, 576] bf16 into ``kv_cache``, at the flat cache rows
    ``cache_rows`` [T] int64 (contiguous [N, ...] or paged [P, 64, ...] caches alike)."""
    lib = load_library()
    _dev(positions, "positions", (torch.int32,))
    _dev(cache_rows, "cache_rows", (torch.int64,))
    _dev(cos_sin, "cos_sin", (torch.float32,))
    _dev(k_idx_in, "k_idx_in", (torch.bfloat16,))
    _dev(kv_in, "kv_in", (torch.bfloat16,))
    _dev(k_idx_cache, "k_idx_cache", (torch.bfloat16, torch.float8_e4m3fn, torch.uint8))
    _dev(kv_cache, "kv_cache", (torch.bfloat16,))
    if k_idx_scale is not None:
        _dev(k_idx_scale, "k_idx_scale", (torch.float32,))
    T = int(positions.numel())
    if k_idx_in.numel() != T * 128 or kv_in.numel() != T * 576 or cache_rows.numel() != T:
        raise ValueError("k_idx_in must be [T, 128], kv_in [T, 576] and cache_rows [T]")
    n_rows = kv_cache.numel() // 576
    if k_idx_cache.numel() != n_rows * 128 or cos_sin.shape[-1] != 64:
        raise ValueError("k_idx_cache must hold as many 128-dim rows as kv_cache 576-dim rows, "
                         "and cos_sin must be [max_position, 64]")
    s = lib.dsa_prep_cache_write(T, _ptr(positions), _ptr(cache_rows), n_rows, _ptr(cos_sin),
                                 int(cos_sin.shape[0]), dtype_code(k_idx_cache), _ptr(k_idx_in),
                                 _ptr(k_idx_cache), _ptr(k_idx_scale), _ptr(kv_in), _ptr(kv_cache),
                                 _stream())
    _check(s, "dsa_prep_cache_write")


def prep_queries(positions, cos_sin, q_idx_in, q_idx, q, q_idx_scale=None):
    """RoPE + (fp8) quantisation of the query rows: indexer queries ``q_idx_in`` [R, 64, 128]
    bf16 into ``q_idx`` (bf16, or fp8 e4m3 / uint8 with ``q_idx_scale`` [R, 64]), and the MLA
    queries ``q`` [R, H, 576] bf16 rotated in place."""
    lib = load_library()
    _dev(positions, "positions", (torch.int32,))
    _dev(cos_sin, "cos_sin", (torch.float32,))
    _dev(q_idx_in, "q_idx_in", (torch.bfloat16,))
    _dev(q_idx, "q_idx", (torch.bfloat16, torch.float8_e4m3fn, torch.uint8))
    _dev(q, "q", (torch.bfloat16,))
    if q_idx_scale is not None:
        _dev(q_idx_scale, "q_idx_scale", (torch.float32,))
    R = int(positions.numel())
    if q_idx_in.numel() != R * 64 * 128 or q_idx.numel() != R * 64 * 128 or q.dim() != 3 \
            or q.shape[0] != R or q.shape[2] != 576 or cos_sin.shape[-1] != 64:
        raise ValueError("q_idx_in / q_idx must be [R, 64, 128], q [R, H, 576], cos_sin [P, 64]")
    s = lib.dsa_prep_queries(R, _ptr(positions), _ptr(cos_sin), int(cos_sin.shape[0]),
                             dtype_code(q_idx), _ptr(q_idx_in), _ptr(q_idx), _ptr(q_idx_scale),
                             int(q.shape[1]), _ptr(q), _stream())
    _check(s, "dsa_prep_queries")


def prep(positions, cache_rows, cos_sin, k_idx_in, k_idx_cache, kv_in, kv_cache, q_idx_in, q_idx,
         q, k_idx_scale=None, q_idx_scale=None):
    """:func:`prep_cache_write` and :func:`prep_queries` for new tokens that are also the query
    rows (decode, or a prefill chunk), in one launch."""
    lib = load_library()
    for t, n, d in ((positions, "positions", (torch.int32,)), (cache_rows, "cache_rows", (torch.int64,)),
                    (cos_sin, "cos_sin", (torch.float32,)), (k_idx_in, "k_idx_in", (torch.bfloat16,)),
                    (kv_in, "kv_in", (torch.bfloat16,)), (kv_cache, "kv_cache", (torch.bfloat16,)),
                    (q_idx_in, "q_idx_in", (torch.bfloat16,)), (q, "q", (torch.bfloat16,))):
        _dev(t, n, d)
    for t, n in ((k_idx_cache, "k_idx_cache"), (q_idx, "q_idx")):
        _dev(t, n, (torch.bfloat16, torch.float8_e4m3fn, torch.uint8))
    for t, n in ((k_idx_scale, "k_idx_scale"), (q_idx_scale, "q_idx_scale")):
        if t is not None:
            _dev(t, n, (torch.float32,))
    if dtype_code(k_idx_cache) != dtype_code(q_idx):
        raise ValueError("k_idx_cache and q_idx must have the same format")
    T = int(positions.numel())
    n_rows = kv_cache.numel() // 576
    if k_idx_in.numel() != T * 128 or kv_in.numel() != T * 576 or cache_rows.numel() != T \
            or q_idx_in.numel() != T * 64 * 128 or q_idx.numel() != T * 64 * 128 or q.dim() != 3 \
            or q.shape[0] != T or q.shape[2] != 576 or k_idx_cache.numel() != n_rows * 128 \
            or cos_sin.shape[-1] != 64:
        raise ValueError("shapes: k_idx_in [T,128], kv_in [T,576], cache_rows [T], q_idx_in / "
                         "q_idx [T,64,128], q [T,H,576], caches of equal rows, cos_sin [P,64]")
    s = lib.dsa_prep(T, _ptr(positions), _ptr(cache_rows), n_rows, _ptr(cos_sin),
                     int(cos_sin.shape[0]), dtype_code(k_idx_cache), _ptr(k_idx_in),
                     _ptr(k_idx_cache), _ptr(k_idx_scale), _ptr(kv_in), _ptr(kv_cache),
                     _ptr(q_idx_in), _ptr(q_idx), _ptr(q_idx_scale), int(q.shape[1]), _ptr(q),
                     _stream())
    _check(s, "dsa_prep")


# --------------------------------------------------------------------------- masked MHA mode

def prefill_dense_mode(max_row_len: int, topk: int) -> bool:
    """True when every row has at most ``topk`` positions: the dense MHA mode is then exactly
    DSA (the top-k selects everything)."""
    return bool(load_library().dsa_prefill_dense_mode(int(max_row_len), int(topk)))


def mha_prefill_workspace_size(num_seqs: int, n_heads: int, num_rows: int, max_row_len: int,
                               masked: bool) -> int:
    return int(load_library().dsa_mha_prefill_workspace_size(
        int(num_seqs), int(n_heads), int(num_rows), int(max_row_len), int(bool(masked))))


def mha_prefill(rows: Rows, q, kv, w_uk, w_uv, scale: float, idx=None, out=None, lse=None,
                ws=None):
    """Masked MHA mode: q [R, H, 192] bf16 against the latent cache ``kv`` decompressed through
    ``w_uk`` / ``w_uv`` [H, 128, 512]; over each row's top-k set ``idx`` [R, k] or, with
    idx None, over every position below its length.  Returns out [R, H, 128] bf16."""
    lib = load_library()
    _dev(q, "q", (torch.bfloat16,))
    _dev(kv, "kv", (torch.bfloat16,))
    _dev(w_uk, "w_uk", (torch.bfloat16,))
    _dev(w_uv, "w_uv", (torch.bfloat16,))
    if q.dim() != 3 or q.shape[2] != 192:
        raise ValueError("q must be [R, H, 192]")
    _rows_of(rows, q, "q")
    R, H = int(q.shape[0]), int(q.shape[1])
    _latent_cache_shape(rows, kv, 576)
    if w_uk.shape != (H, 128, 512) or w_uv.shape != (H, 128, 512) or kv.shape[-1] != 576:
        raise ValueError("w_uk / w_uv must be [H, 128, 512] and kv rows 576 wide")
    k = 0
    if idx is not None:
        _dev(idx, "idx", (torch.int32,))
        _shape(idx, "idx", (R, None))
        k = int(idx.shape[1])
    if out is None:
        out = torch.empty((R, H, 128), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,))
    _shape(out, "out", (R, H, 128))
    if lse is not None:
        _dev(lse, "lse", (torch.float32,))
        _shape(lse, "lse", (R, H))
    need = mha_prefill_workspace_size(rows.num_seqs, H, R, rows.max_row_len, idx is not None)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = rows.struct()
    name = "dsa_mha_prefill_paged" if rows.paged else "dsa_mha_prefill"
    s = getattr(lib, name)(ctypes.byref(st), H, float(scale), _ptr(q), _ptr(kv), _ptr(w_uk),
                           _ptr(w_uv), _ptr(idx), k, _ptr(out), _ptr(lse), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream())
    _check(s, name)
    return out


def sparse_attention_prefill_workspace_size(num_rows: int, num_seqs: int, max_row_len: int,
                                            idx_dtype, topk: int, n_heads: int,
                                            dense_threshold: int) -> int:
    code = idx_dtype if isinstance(idx_dtype, int) else dtype_code(torch.empty(0, dtype=idx_dtype))
    return int(load_library().dsa_sparse_attention_prefill_workspace_size(
        int(num_rows), int(num_seqs), int(max_row_len), code, int(topk), int(n_heads),
        int(dense_threshold)))


def sparse_attention_prefill(rows: Rows, q_idx, w, k_idx, logits, topk: int, q, kv, w_uk, w_uv,
                             scale: float, dense_threshold: int, idx=None, out=None, lse=None,
                             q_scale=None, k_scale=None, ws=None):
    """Prefill attention with the masked-MHA / MQA dispatch: q [R, H, 192] bf16 (nope | rope),
    the latent cache ``kv`` and ``w_uk`` / ``w_uv`` [H, 128, 512]; the indexer inputs as for
    :func:`indexer_topk`.  The masked MHA mode when ``rows.max_row_len <= dense_threshold``,
    else the MQA path (query absorbed through W_UK, sparse MLA, output through W_UV).
    Returns out [R, H, 128] bf16; ``logits`` / ``idx`` are written whenever the selection
    runs (always, except the dense MHA mode of rows no longer than ``topk``)."""
    lib = load_library()
    for t, n in ((q_idx, "q_idx"), (k_idx, "k_idx")):
        _dev(t, n)
    _dev(w, "w", (torch.float32,))
    _dev(logits, "logits", (torch.float32,))
    _dev(q, "q", (torch.bfloat16,))
    _dev(kv, "kv", (torch.bfloat16,))
    _dev(w_uk, "w_uk", (torch.bfloat16,))
    _dev(w_uv, "w_uv", (torch.bfloat16,))
    if q_scale is not None:
        _dev(q_scale, "q_scale", (torch.float32,))
    if k_scale is not None:
        _dev(k_scale, "k_scale", (torch.float32,))
    if q.dim() != 3 or q.shape[2] != 192 or q_idx.dim() != 3:
        raise ValueError("q must be [R, H, 192] and q_idx [R, H_I, D_I]")
    _indexer_shapes(rows, q_idx, w, k_idx, logits, q_scale, k_scale)
    _rows_of(rows, q, "q")
    R, H = int(q.shape[0]), int(q.shape[1])
    _latent_cache_shape(rows, kv, 576)
    if w_uk.shape != (H, 128, 512) or w_uv.shape != (H, 128, 512):
        raise ValueError("w_uk / w_uv must be [H, 128, 512]")
    if idx is None:
        idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
    _dev(idx, "idx", (torch.int32,))
    _shape(idx, "idx", (R, topk))
    if out is None:
        out = torch.empty((R, H, 128), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,))
    _shape(out, "out", (R, H, 128))
    if lse is not None:
        _dev(lse, "lse", (torch.float32,))
        _shape(lse, "lse", (R, H))
    need = sparse_attention_prefill_workspace_size(R, rows.num_seqs, rows.max_row_len,
                                                   dtype_code(q_idx), topk, H, dense_threshold)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = rows.struct()
    name = "dsa_sparse_attention_prefill_paged" if rows.paged else "dsa_sparse_attention_prefill"
    s = getattr(lib, name)(
        ctypes.byref(st), dtype_code(q_idx), int(q_idx.shape[1]), int(q_idx.shape[2]), _ptr(q_idx),
        _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), _ptr(logits), int(logits.shape[-1]),
        int(topk), _ptr(idx), H, float(scale), _ptr(q), _ptr(kv), _ptr(w_uk), _ptr(w_uv),
        _ptr(out), _ptr(lse), int(dense_threshold), _ptr(ws), ws.numel() * ws.element_size(),
        _stream())
    _check(s, name)
    return out
