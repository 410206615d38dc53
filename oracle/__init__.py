"""fp64 CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
never calls the GPU library: the two share no code.

This module is argument marshalling (numpy arrays -> ctypes) around
``liboracle.so``, built from ``pkv_oracle.c`` by ``oracle/build.py``; every
definition and its citation lives in that C file.  bf16 arrays are passed as
their raw 16-bit patterns (numpy ``uint16``); fp32 arrays as ``float32``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
ERRORS = {
    0: "ok",
    1: "bad scalar argument",
    2: "needed block_table entry is -1 or out of the pool",
    3: "needed logical block index is past the table row",
    4: "negative cache_seqlens",
    5: "cu_seq_lens invalid",
    6: "length exceeds max_length",
}


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {code}: {ERRORS.get(code, '?')}")
        self.code = code


_lib = None


def lib():
    """Load liboracle.so, building it first only if it is not there."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.pkvo_decode.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, I, P, I]
        L.pkvo_decode.restype = I
        L.pkvo_varlen.argtypes = [I, P, P, P, P, P, I, I, I, I, I, I, I, I, D, P, I, P, I]
        L.pkvo_varlen.restype = I
        L.pkvo_cu_from_lengths.argtypes = [P, I, P]
        L.pkvo_cu_from_lengths.restype = None
        L.pkvo_request_index.argtypes = [P, I, I, P]
        L.pkvo_request_index.restype = I
        L.pkvo_locate.argtypes = [P, I, I, I, I, ctypes.c_int64, P]
        L.pkvo_locate.restype = I
        L.pkvo_partial.argtypes = [I, P, P, I, P, P, P]
        L.pkvo_partial.restype = None
        L.pkvo_merge2.argtypes = [D, D, P, D, D, P, I, P, P, P]
        L.pkvo_merge2.restype = None
        L.pkvo_finalize.argtypes = [D, P, I, P]
        L.pkvo_finalize.restype = None
        L.pkvo_cache_write.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I]
        L.pkvo_cache_write.restype = I
        L.pkvo_varlen_paged.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, D, P,
                                        I, P, I]
        L.pkvo_varlen_paged.restype = I
        L.pkvo_max_threads.argtypes = []
        L.pkvo_max_threads.restype = I
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a)
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def max_threads() -> int:
    return lib().pkvo_max_threads()


def decode(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None,
           scale=None, seqs=None, n_threads=0):
    """Paged decode attention in fp64.

    ``k_cache``/``v_cache`` ([num_blocks, bs, Hkv, D]) are updated IN PLACE by
    the append when ``k_new``/``v_new`` are given, so pass copies you own.
    Returns out [n_eval, Hq, D] float64 (n_eval = len(seqs) or batch).
    """
    dt = _dtype_code(q)
    for a in (k_cache, v_cache):
        if not (a.flags.c_contiguous and a.flags.writeable) or a.dtype != q.dtype:
            raise ValueError("k_cache/v_cache must be writable C-contiguous arrays of q's dtype")
    batch, _, Hq, D = q.shape
    num_blocks, bs, Hkv, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    bt = _c(block_table, np.int32)
    sl = _c(cache_seqlens, np.int32)
    q = _c(q)
    kn, vn = _c(k_new), _c(v_new)
    sq = _c(seqs, np.int32) if seqs is not None else None
    n_eval = len(sq) if sq is not None else batch
    out = np.zeros((n_eval, Hq, D), dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rc = lib().pkvo_decode(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(sl),
                           _ptr(kn), _ptr(vn), batch, Hq, Hkv, D, num_blocks, bs,
                           bt.shape[1], float(scale), _ptr(sq), n_eval, _ptr(out), int(n_threads))
    if rc:
        raise OracleError(rc)
    return out


def varlen(q, k, v, cu_seq_lens_q, cu_seq_lens_k, max_length_q, max_length_k,
           scale=None, rows=None, n_threads=0):
    """Packed variable-length attention (no mask) in fp64.

    q [1, total_q, Hq, D] or [total_q, Hq, D]; k, v likewise with Hkv.
    Returns out [n_eval, Hq, D] float64 (n_eval = len(rows) or total_q).
    """
    dt = _dtype_code(q)
    q3 = q.reshape(q.shape[-3:])
    k3 = k.reshape(k.shape[-3:])
    v3 = v.reshape(v.shape[-3:])
    total_q, Hq, D = q3.shape
    total_k, Hkv, _ = k3.shape
    cq = _c(cu_seq_lens_q, np.int32)
    ck = _c(cu_seq_lens_k, np.int32)
    batch = len(cq) - 1
    rr = _c(rows, np.int32) if rows is not None else None
    n_eval = len(rr) if rr is not None else total_q
    out = np.zeros((n_eval, Hq, D), dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    q3, k3, v3 = _c(q3), _c(k3), _c(v3)
    rc = lib().pkvo_varlen(dt, _ptr(q3), _ptr(k3), _ptr(v3), _ptr(cq), _ptr(ck),
                           int(max_length_q), int(max_length_k), batch, total_q, total_k,
                           Hq, Hkv, D, float(scale), _ptr(rr), n_eval, _ptr(out), int(n_threads))
    if rc:
        raise OracleError(rc)
    return out


def cache_write(k, v, cu_seq_lens, start, k_cache, v_cache, block_table):
    """Writes packed rows into the paged pools IN PLACE (pass copies you own).

    k, v [1, total, Hkv, D] or [total, Hkv, D]; row cu[b] + i of request b goes
    to token start[b] + i of sequence b.  Raises OracleError (pools untouched)
    when any row cannot be placed.
    """
    dt = _dtype_code(k)
    k3, v3 = _c(k.reshape(k.shape[-3:])), _c(v.reshape(v.shape[-3:]))
    for a in (k_cache, v_cache):
        if not (a.flags.c_contiguous and a.flags.writeable) or a.dtype != k.dtype:
            raise ValueError("k_cache/v_cache must be writable C-contiguous arrays of k's dtype")
    total, Hkv, D = k3.shape
    num_blocks, bs, Hkv2, D2 = k_cache.shape
    assert (Hkv2, D2) == (Hkv, D) and v_cache.shape == k_cache.shape
    cu = _c(cu_seq_lens, np.int32)
    st = _c(start, np.int32)
    bt = _c(block_table, np.int32)
    rc = lib().pkvo_cache_write(dt, _ptr(k3), _ptr(v3), _ptr(cu), _ptr(st), _ptr(k_cache),
                                _ptr(v_cache), _ptr(bt), len(cu) - 1, total, Hkv, D, num_blocks,
                                bs, bt.shape[1])
    if rc:
        raise OracleError(rc)


def varlen_paged(q, k_cache, v_cache, block_table, cu_seq_lens_q, seqlens_k, max_length_q,
                 max_length_k, scale=None, rows=None, n_threads=0):
    """Varlen attention (no mask) whose keys are the first seqlens_k[b] tokens
    of sequence b in the paged pools, in fp64.

    q [1, total_q, Hq, D] or [total_q, Hq, D].  Returns out [n_eval, Hq, D].
    """
    dt = _dtype_code(q)
    q3 = _c(q.reshape(q.shape[-3:]))
    total_q, Hq, D = q3.shape
    num_blocks, bs, Hkv, _ = k_cache.shape
    cq = _c(cu_seq_lens_q, np.int32)
    sk = _c(seqlens_k, np.int32)
    bt = _c(block_table, np.int32)
    kc, vc = _c(k_cache), _c(v_cache)
    rr = _c(rows, np.int32) if rows is not None else None
    n_eval = len(rr) if rr is not None else total_q
    out = np.zeros((n_eval, Hq, D), dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rc = lib().pkvo_varlen_paged(dt, _ptr(q3), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cq), _ptr(sk),
                                 int(max_length_q), int(max_length_k), len(cq) - 1, total_q, Hq,
                                 Hkv, D, num_blocks, bs, bt.shape[1], float(scale), _ptr(rr),
                                 n_eval, _ptr(out), int(n_threads))
    if rc:
        raise OracleError(rc)
    return out


def cu_from_lengths(lengths):
    l = _c(lengths, np.int32)
    cu = np.zeros(len(l) + 1, dtype=np.int32)
    lib().pkvo_cu_from_lengths(_ptr(l), len(l), _ptr(cu))
    return cu


def request_index(cu, total):
    cu = _c(cu, np.int32)
    req = np.full(max(total, 1), -1, dtype=np.int32)
    rc = lib().pkvo_request_index(_ptr(cu), len(cu) - 1, int(total), _ptr(req))
    if rc:
        raise OracleError(rc)
    return req[:total]


def locate(block_table, num_blocks, block_size, seq, t):
    """(logical block, offset, physical block) of logical token t of seq."""
    bt = _c(block_table, np.int32)
    w = np.zeros(3, dtype=np.int32)
    rc = lib().pkvo_locate(_ptr(bt), bt.shape[1], int(num_blocks), int(block_size), int(seq),
                           int(t), _ptr(w))
    if rc:
        raise OracleError(rc)
    return tuple(int(x) for x in w)


def partial(scores, values):
    """(m, l, acc) of a run of scores with value rows [n, d] (identity if n = 0)."""
    s = _c(np.asarray(scores, dtype=np.float64))
    v = np.asarray(values, dtype=np.float64)
    d = v.shape[-1] if v.ndim > 1 else (v.size // max(len(s), 1))
    v = _c(v.reshape(len(s), d))
    m, l = ctypes.c_double(), ctypes.c_double()
    acc = np.zeros(d, dtype=np.float64)
    lib().pkvo_partial(len(s), _ptr(s), _ptr(v), d, ctypes.byref(m), ctypes.byref(l), _ptr(acc))
    return m.value, l.value, acc


def merge2(p1, p2):
    m1, l1, a1 = p1
    m2, l2, a2 = p2
    a1 = _c(np.asarray(a1, dtype=np.float64))
    a2 = _c(np.asarray(a2, dtype=np.float64))
    m, l = ctypes.c_double(), ctypes.c_double()
    acc = np.zeros(len(a1), dtype=np.float64)
    lib().pkvo_merge2(float(m1), float(l1), _ptr(a1), float(m2), float(l2), _ptr(a2), len(a1),
                      ctypes.byref(m), ctypes.byref(l), _ptr(acc))
    return m.value, l.value, acc


def finalize(p):
    _, l, acc = p
    acc = _c(np.asarray(acc, dtype=np.float64))
    out = np.zeros(len(acc), dtype=np.float64)
    lib().pkvo_finalize(float(l), _ptr(acc), len(acc), _ptr(out))
    return out
