"""fp64 CPU oracle for the DSA path (lightning indexer, top-k, sparse MLA in MQA mode).

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the GPU library never imports or links
this package, and this package never imports the GPU library.

The arithmetic lives in ``dsa_oracle.c`` (plain C, fp64, nested loops); this
module only marshals numpy arrays into it with ctypes.  Encoded inputs are
passed as their raw bits: bf16 as ``uint16``, OCP e4m3 as ``uint8``, fp32 as
``float32``.

Sources are cited by page title and section in ``dsa_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "dsa_oracle.c")

F32, BF16, E4M3 = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16, "fp8": E4M3, "e4m3": E4M3}


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
               "-pthread", "-o", _LIB_PATH, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB_PATH


class _Rows(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32),
                ("row_seq", ctypes.c_void_p),
                ("row_len", ctypes.c_void_p),
                ("seq_start", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p),
                ("max_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oref_bf16_to_f64.argtypes = [vp, vp, i64]
        lib.oref_e4m3_to_f64.argtypes = [vp, vp, i64]
        lib.oref_indexer.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                     ctypes.POINTER(_Rows), vp, i32, vp, i64, ctypes.c_int]
        lib.oref_topk_row.argtypes = [vp, i64, i32, vp]
        lib.oref_topk_rows.argtypes = [vp, i64, vp, i32, i32, vp, ctypes.c_int]
        lib.oref_topk_rows_f32.argtypes = [vp, i64, vp, i32, i32, vp, ctypes.c_int]
        lib.oref_sparse_mla.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, dbl,
                                        vp, vp, vp, i32, ctypes.POINTER(_Rows), vp, i32, vp, vp,
                                        ctypes.c_int]
        lib.oref_dense_mqa.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, dbl,
                                       vp, vp, ctypes.POINTER(_Rows), vp, i32, vp, vp, ctypes.c_int]
        lib.oref_cache_row.argtypes = [ctypes.POINTER(_Rows), i32, i64]
        lib.oref_cache_row.restype = i64
        lib.oref_bf16_codes.argtypes = [vp, vp, i64]
        lib.oref_e4m3_codes.argtypes = [vp, vp, i64]
        lib.oref_prep_keys.argtypes = [i32, vp, vp, i64, vp, i32, ctypes.c_int, vp, vp, vp, vp, vp]
        lib.oref_prep_queries.argtypes = [i32, vp, vp, i32, ctypes.c_int, i32, vp, vp, vp, i32, vp]
        lib.oref_mha_decompress.argtypes = [i32, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int]
        lib.oref_mha.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.POINTER(_Rows), vp, i32, dbl, vp,
                                 i32, vp, vp, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


class Rows:
    """Row description: query row r reads sequence row_seq[r], positions [0, row_len[r]).

    Exactly one of ``seq_start`` (contiguous cache) and ``page_table`` (paged cache) is given.
    """

    def __init__(self, row_seq, row_len, seq_start=None, page_table=None, page_size=64):
        self.row_seq = _c(row_seq, np.int32)
        self.row_len = _c(row_len, np.int32)
        self.seq_start = None if seq_start is None else _c(seq_start, np.int64)
        self.page_table = None if page_table is None else _c(page_table, np.int32)
        if (self.seq_start is None) == (self.page_table is None):
            raise ValueError("give exactly one of seq_start and page_table")
        self.page_size = int(page_size)
        self.max_pages = 0 if self.page_table is None else int(self.page_table.shape[-1])
        self.n_rows = int(self.row_seq.shape[0])

    def _struct(self):
        return _Rows(self.n_rows, _ptr(self.row_seq), _ptr(self.row_len), _ptr(self.seq_start),
                     _ptr(self.page_table), self.max_pages, self.page_size)

    def cache_row(self, b: int, s: int) -> int:
        st = self._struct()
        return int(_load().oref_cache_row(ctypes.byref(st), int(b), int(s)))


def _which(rows: Rows, which):
    if which is None:
        return np.arange(rows.n_rows, dtype=np.int32)
    return _c(which, np.int32)


def _enc(dtype: str):
    if dtype not in _DTYPES:
        raise ValueError(f"unknown dtype {dtype}")
    return _DTYPES[dtype]


def bf16_to_f64(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oref_bf16_to_f64(_ptr(bits), _ptr(out), bits.size)
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oref_e4m3_to_f64(_ptr(codes), _ptr(out), codes.size)
    return out


def _raw(a, dtype: str):
    return _c(a, {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "e4m3": np.uint8}[dtype])


def indexer(dtype: str, q, w, k, rows: Rows, q_scale=None, k_scale=None, which=None, ld=None,
            n_threads=None) -> np.ndarray:
    """I[r, s] = sum_j w[r,j] * relu(q[r,j,:] . k[row(s),:]) for s < row_len[r]; NaN elsewhere.

    q: [R, H, D]; w: [R, H] f32; k: [cache rows, D] (or [pages, page, D]); fp8 adds
    q_scale [R, H] and k_scale [cache rows] (or [pages, page]).
    """
    enc = _enc(dtype)
    q = _raw(q, dtype)
    k = _raw(k, dtype)
    w = _c(w, np.float32)
    H, D = int(q.shape[-2]), int(q.shape[-1])
    qs = None if q_scale is None else _c(q_scale, np.float32)
    ks = None if k_scale is None else _c(k_scale, np.float32)
    wh = _which(rows, which)
    if ld is None:
        ld = int(rows.row_len[wh].max()) if wh.size else 1
    out = np.full((wh.size, ld), np.nan, dtype=np.float64)
    st = rows._struct()
    rc = _load().oref_indexer(enc, H, D, _ptr(q), _ptr(qs), _ptr(w), _ptr(k), _ptr(ks),
                              ctypes.byref(st), _ptr(wh), wh.size, _ptr(out), ld,
                              n_threads or default_threads())
    if rc:
        raise ValueError("oref_indexer rejected its arguments")
    return out


def topk(scores, lens, k: int, n_threads=None) -> np.ndarray:
    """Top-k per row (score desc, position asc; -0 == +0), ascending positions, -1 padded.

    ``scores`` is [R, ld] float64 or float32 (float32 is widened exactly).
    """
    lens = _c(lens, np.int32)
    if scores.dtype == np.float32:
        x = _c(scores, np.float32)
        fn = _load().oref_topk_rows_f32
    else:
        x = _c(scores, np.float64)
        fn = _load().oref_topk_rows
    R = int(x.shape[0])
    out = np.empty((R, k), dtype=np.int32)
    rc = fn(_ptr(x), int(x.shape[1]), _ptr(lens), R, int(k), _ptr(out), n_threads or default_threads())
    if rc:
        raise ValueError("oref_topk rejected its arguments")
    return out


def sparse_mla(dtype: str, q, kv, idx, rows: Rows, scale: float, d_v: int, which=None,
               n_threads=None):
    """Sparse MQA attention over idx entries; returns (out [n,H,Dv] f64, lse [n,H] f64)."""
    enc = _enc(dtype)
    q = _raw(q, dtype)
    kv = _raw(kv, dtype)
    idx = _c(idx, np.int32)
    H, Dqk = int(q.shape[-2]), int(q.shape[-1])
    wh = _which(rows, which)
    out = np.empty((wh.size, H, d_v), dtype=np.float64)
    lse = np.empty((wh.size, H), dtype=np.float64)
    st = rows._struct()
    rc = _load().oref_sparse_mla(enc, H, Dqk, int(d_v), float(scale), _ptr(q), _ptr(kv), _ptr(idx),
                                 int(idx.shape[-1]), ctypes.byref(st), _ptr(wh), wh.size, _ptr(out),
                                 _ptr(lse), n_threads or default_threads())
    if rc:
        raise ValueError("oref_sparse_mla rejected its arguments")
    return out, lse


def dense_mqa(dtype: str, q, kv, rows: Rows, scale: float, d_v: int, which=None, n_threads=None):
    """Dense causal MQA attention over every position [0, row_len); returns (out, lse)."""
    enc = _enc(dtype)
    q = _raw(q, dtype)
    kv = _raw(kv, dtype)
    H, Dqk = int(q.shape[-2]), int(q.shape[-1])
    wh = _which(rows, which)
    out = np.empty((wh.size, H, d_v), dtype=np.float64)
    lse = np.empty((wh.size, H), dtype=np.float64)
    st = rows._struct()
    rc = _load().oref_dense_mqa(enc, H, Dqk, int(d_v), float(scale), _ptr(q), _ptr(kv),
                                ctypes.byref(st), _ptr(wh), wh.size, _ptr(out), _ptr(lse),
                                n_threads or default_threads())
    if rc:
        raise ValueError("oref_dense_mqa rejected its arguments")
    return out, lse


def max_abs_rel(x, ref) -> float:
    """Error metric: max_i |x_i - ref_i| / max_i |ref_i| over one output tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


# --------------------------------------------------------------------------- input prep

def bf16_codes(x) -> np.ndarray:
    """fp32 values -> bf16 codes (nearest, ties to the even code)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oref_bf16_codes(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_codes(x) -> np.ndarray:
    """fp32 values -> OCP E4M3FN codes (nearest finite, ties to the even code)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oref_e4m3_codes(_ptr(x), _ptr(out), x.size)
    return out


def prep_keys(idx_dtype: str, pos, rows_out, cos_sin, k_in, kv_in, k_cache, kv_cache,
              k_scale=None):
    """Key-side prep for new tokens, written into copies of k_cache / kv_cache (and k_scale);
    returns the updated copies.  k_in [T,128] and kv_in [T,576] are bf16 bits (uint16); the
    caches are [rows,128] (uint16 bf16 or uint8 e4m3) and [rows,576] uint16."""
    enc = _enc(idx_dtype)
    pos = _c(pos, np.int32)
    rows_out = _c(rows_out, np.int64)
    cos_sin = _c(cos_sin, np.float32)
    k_in = _c(k_in, np.uint16)
    kv_in = _c(kv_in, np.uint16)
    k_cache = np.array(k_cache, dtype=np.uint16 if enc == BF16 else np.uint8, copy=True, order="C")
    kv_cache = np.array(kv_cache, dtype=np.uint16, copy=True, order="C")
    ks = None if k_scale is None else np.array(k_scale, dtype=np.float32, copy=True, order="C")
    rc = _load().oref_prep_keys(pos.size, _ptr(pos), _ptr(rows_out), kv_cache.shape[0],
                                _ptr(cos_sin), cos_sin.shape[0], enc, _ptr(k_in), _ptr(k_cache),
                                _ptr(ks), _ptr(kv_in), _ptr(kv_cache))
    if rc:
        raise ValueError("oref_prep_keys rejected its arguments")
    return k_cache, kv_cache, ks


def prep_queries(idx_dtype: str, pos, cos_sin, qi_in, q):
    """Query-side prep: returns (qi_out, qi_scale or None, q rotated).  qi_in [R,H_I,128] and
    q [R,H,576] are bf16 bits (uint16)."""
    enc = _enc(idx_dtype)
    pos = _c(pos, np.int32)
    cos_sin = _c(cos_sin, np.float32)
    qi_in = _c(qi_in, np.uint16)
    q = np.array(q, dtype=np.uint16, copy=True, order="C")
    R, HI = int(qi_in.shape[0]), int(qi_in.shape[1])
    qi_out = np.zeros(qi_in.shape, dtype=np.uint16 if enc == BF16 else np.uint8)
    qs = np.zeros((R, HI), dtype=np.float32) if enc == E4M3 else None
    rc = _load().oref_prep_queries(R, _ptr(pos), _ptr(cos_sin), cos_sin.shape[0], enc, HI,
                                   _ptr(qi_in), _ptr(qi_out), _ptr(qs), int(q.shape[1]), _ptr(q))
    if rc:
        raise ValueError("oref_prep_queries rejected its arguments")
    return qi_out, qs, q


# --------------------------------------------------------------------------- masked MHA mode

def mha_decompress(kv, w_uk, w_uv, n_threads=None):
    """Per-head keys [rows, H, 192] and values [rows, H, 128] (fp64) of the latent cache rows
    kv [rows, 576] (bf16 bits) with W_UK, W_UV [H, 128, 512] (bf16 bits)."""
    kv = _c(kv, np.uint16).reshape(-1, 576)
    w_uk = _c(w_uk, np.uint16)
    w_uv = _c(w_uv, np.uint16)
    H = int(w_uk.shape[0])
    n = int(kv.shape[0])
    k = np.empty((n, H, 192), dtype=np.float64)
    v = np.empty((n, H, 128), dtype=np.float64)
    rc = _load().oref_mha_decompress(n, H, _ptr(kv), _ptr(w_uk), _ptr(w_uv), _ptr(k), _ptr(v),
                                     n_threads or default_threads())
    if rc:
        raise ValueError("oref_mha_decompress rejected its arguments")
    return k, v


def mha(q, k, v, rows: Rows, scale: float, idx=None, which=None, n_threads=None):
    """Masked MHA over decompressed keys / values: out [n_which, H, 128], lse [n_which, H].
    q [R, H, 192] bf16 bits; idx [R, topk] (a set per row) or None for dense causal."""
    q = _c(q, np.uint16)
    H = int(q.shape[1])
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    wh = _which(rows, which)
    idx_c = None if idx is None else _c(idx, np.int32)
    topk = 0 if idx_c is None else int(idx_c.shape[1])
    out = np.zeros((wh.size, H, 128), dtype=np.float64)
    lse = np.zeros((wh.size, H), dtype=np.float64)
    st = rows._struct()
    rc = _load().oref_mha(H, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st), _ptr(idx_c), topk,
                          float(scale), _ptr(wh), wh.size, _ptr(out), _ptr(lse),
                          n_threads or default_threads())
    if rc:
        raise ValueError("oref_mha rejected its arguments")
    return out, lse
