"""paged_kv_cache_296_amd -- paged attention on one AMD MI355X (gfx950).

Thin Python binding over ``libpkv.so`` (the C ABI declared in
``include/pkv.h``).  This module only marshals arguments: it checks tensor
placement, dtype and shape, allocates outputs and workspace with torch when
the caller does not pass them, and hands raw device pointers plus the current
HIP stream to the library.  Every step of the computation runs in the HIP
kernels; there is no CPU fallback.  If the library is not built, or no GPU is
visible, the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "PkvError", "decode", "decode_partials", "decode_merge", "varlen", "cache_write",
    "varlen_paged", "decode_workspace_bytes", "decode_partition_tokens", "check_decode_args",
    "check_varlen_args", "check_cache_write_args", "check_varlen_paged_args", "status_string",
    "abi_version", "lib_path", "ERR_BLOCK", "ERR_SPAN", "ERR_CU", "ERR_MAXLEN",
    "BlockManager", "OutOfBlocks", "copy_blocks", "decode_noalloc",
    "DECODE_NOALLOC_SCRATCH_BYTES", "stream_read", "stream_copy", "mfma_peak",
]

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ENOMEM = 0, 1, 2, 3, 4, 5
FP32, BF16 = 0, 1
ERR_BLOCK, ERR_SPAN, ERR_CU, ERR_MAXLEN = 1, 2, 4, 8

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libpkv.so")
_lib = None


class PkvError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})" if what else
                         status_string(status))


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is not built; run __graft_entry__.build() "
                              "(hipcc for gfx950) first")
        L = ctypes.CDLL(lib_path)
        P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.pkv_status_string.argtypes = [I]
        L.pkv_status_string.restype = ctypes.c_char_p
        L.pkv_abi_version.argtypes = []
        L.pkv_abi_version.restype = I
        L.pkv_check_decode_args.argtypes = [I] * 10
        L.pkv_check_decode_args.restype = I
        L.pkv_decode_partition_tokens.argtypes = [I] * 7
        L.pkv_decode_partition_tokens.restype = I
        L.pkv_decode_workspace_bytes.argtypes = [I] * 7
        L.pkv_decode_workspace_bytes.restype = SZ
        for name in ("pkv_decode", "pkv_decode_partials", "pkv_decode_merge"):
            fn = getattr(L, name)
            fn.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, SZ, P, P]
            fn.restype = I
        L.pkv_decode_noalloc.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P,
                                         P]
        L.pkv_decode_noalloc.restype = I
        L.pkv_check_varlen_args.argtypes = [I] * 9
        L.pkv_check_varlen_args.restype = I
        L.pkv_varlen.argtypes = [I, P, P, P, P, P, I, I, P, I, I, I, I, I, I, F, P, P]
        L.pkv_varlen.restype = I
        L.pkv_check_cache_write_args.argtypes = [I] * 8
        L.pkv_check_cache_write_args.restype = I
        L.pkv_cache_write.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P]
        L.pkv_cache_write.restype = I
        L.pkv_check_varlen_paged_args.argtypes = [I] * 11
        L.pkv_check_varlen_paged_args.restype = I
        L.pkv_varlen_paged.argtypes = [I, P, P, P, P, P, P, I, I, P, I, I, I, I, I, I, I, I, F,
                                       P, P]
        L.pkv_varlen_paged.restype = I
        I64, PP = ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p)
        L.pkv_bm_create.argtypes = [I, I, PP]
        L.pkv_bm_create.restype = I
        L.pkv_bm_destroy.argtypes = [P]
        L.pkv_bm_destroy.restype = None
        L.pkv_bm_num_free.argtypes = [P]
        L.pkv_bm_num_free.restype = I
        L.pkv_bm_ref_count.argtypes = [P, I]
        L.pkv_bm_ref_count.restype = I
        L.pkv_bm_allocate.argtypes = [P, I64, I]
        L.pkv_bm_allocate.restype = I
        L.pkv_bm_fork.argtypes = [P, I64, I64]
        L.pkv_bm_fork.restype = I
        L.pkv_bm_append.argtypes = [P, I64, I, P, P, P]
        L.pkv_bm_append.restype = I
        L.pkv_bm_release.argtypes = [P, I64]
        L.pkv_bm_release.restype = I
        L.pkv_bm_seq_len.argtypes = [P, I64]
        L.pkv_bm_seq_len.restype = I64
        L.pkv_bm_table.argtypes = [P, P, I, I, P, P]
        L.pkv_bm_table.restype = I
        L.pkv_copy_blocks.argtypes = [I, P, P, P, P, I, I, I, I, I, P, P]
        L.pkv_copy_blocks.restype = I
        L.pkv_stream_read.argtypes = [P, SZ, P, I, I, P]
        L.pkv_stream_read.restype = I
        L.pkv_stream_copy.argtypes = [P, P, SZ, I, P]
        L.pkv_stream_copy.restype = I
        L.pkv_mfma_peak.argtypes = [P, I, I, P]
        L.pkv_mfma_peak.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return _load().pkv_status_string(int(status)).decode()


def abi_version() -> int:
    return _load().pkv_abi_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"paged attention takes float32 or bfloat16 tensors, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU path)")


def _need_contig(**ts):
    for name, t in ts.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(stream, *args, **kw):
    """torch.empty on the stream the kernels will run on: the caching
    allocator then hands the block out again only to work ordered after them
    on that stream, even once the caller has dropped it."""
    if stream is None:
        return torch.empty(*args, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*args, **kw)


def check_decode_args(dtype, has_new, batch, num_heads, num_kv_heads, head_dim, num_blocks,
                      block_size, max_blocks_per_seq, partition_tokens=0) -> int:
    return _load().pkv_check_decode_args(int(dtype), int(has_new), batch, num_heads, num_kv_heads,
                                         head_dim, num_blocks, block_size, max_blocks_per_seq,
                                         partition_tokens)


def check_varlen_args(dtype, batch, total_q, total_k, num_heads, num_kv_heads, head_dim,
                      max_length_q, max_length_k) -> int:
    return _load().pkv_check_varlen_args(int(dtype), batch, total_q, total_k, num_heads,
                                         num_kv_heads, head_dim, max_length_q, max_length_k)


def decode_partition_tokens(batch, num_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, partition_tokens=0) -> int:
    return _load().pkv_decode_partition_tokens(batch, num_heads, num_kv_heads, head_dim,
                                               block_size, max_blocks_per_seq, partition_tokens)


def decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, partition_tokens=0) -> int:
    return _load().pkv_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim,
                                              block_size, max_blocks_per_seq, partition_tokens)


def decode(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None, *,
           softmax_scale=None, partition_tokens=0, out=None, workspace=None, err_flag=None,
           stream=None):
    """Paged decode attention; appends k_new/v_new in place when given.

    q [B, 1, Hq, D]; k_cache/v_cache [num_blocks, block_size, Hkv, D];
    block_table [B, max_blocks] int32; cache_seqlens [B] int32 (before the
    append, not modified); k_new/v_new [B, 1, Hkv, D] or None.  Returns out
    [B, 1, Hq, D] in q's dtype.
    """
    return _decode_call("pkv_decode", q, k_cache, v_cache, block_table, cache_seqlens, k_new,
                        v_new, softmax_scale, partition_tokens, out, workspace, err_flag,
                        stream)[0]


def decode_partials(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None, *,
                    softmax_scale=None, partition_tokens=0, out=None, workspace=None,
                    err_flag=None, stream=None):
    """First phase of decode (per-partition kernel and the append).  Returns
    (out, workspace); pass both to decode_merge with the same arguments."""
    return _decode_call("pkv_decode_partials", q, k_cache, v_cache, block_table, cache_seqlens,
                        k_new, v_new, softmax_scale, partition_tokens, out, workspace, err_flag,
                        stream)


def decode_merge(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None, *,
                 softmax_scale=None, partition_tokens=0, out=None, workspace=None, err_flag=None,
                 stream=None):
    """Second phase of decode: merge the partials in `workspace` into `out`."""
    if out is None:
        raise ValueError("decode_merge needs the out tensor decode_partials returned")
    return _decode_call("pkv_decode_merge", q, k_cache, v_cache, block_table, cache_seqlens, k_new,
                        v_new, softmax_scale, partition_tokens, out, workspace, err_flag,
                        stream)[0]


def _decode_call(fname, q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new,
                 softmax_scale, partition_tokens, out, workspace, err_flag, stream):
    lib = _load()
    _need_gpu(q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new, out, workspace,
              err_flag)
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                 cache_seqlens=cache_seqlens, k_new=k_new, v_new=v_new, out=out)
    dt = _dtype_code(q)
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [batch, 1, num_heads, head_dim]")
    B, _, Hq, D = q.shape
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or k_cache.shape[3] != D:
        raise ValueError("k_cache/v_cache must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    NB, bs, Hkv, _ = k_cache.shape
    for t in (k_cache, v_cache, k_new, v_new):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, caches and new K/V must share one dtype")
    if block_table.dtype != torch.int32 or cache_seqlens.dtype != torch.int32:
        raise TypeError("block_table and cache_seqlens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be [batch, max_blocks_per_seq], cache_seqlens [batch]")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new or neither")
    if k_new is not None and (tuple(k_new.shape) != (B, 1, Hkv, D) or k_new.shape != v_new.shape):
        raise ValueError("k_new/v_new must be [batch, 1, num_kv_heads, head_dim]")
    maxb = block_table.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rc = lib.pkv_check_decode_args(dt, int(k_new is not None), B, Hq, Hkv, D, NB, bs, maxb,
                                   int(partition_tokens))
    if rc:
        raise PkvError(rc, "pkv_decode arguments")
    if out is None:
        out = _empty(stream, q.shape, dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    need = lib.pkv_decode_workspace_bytes(B, Hq, Hkv, D, bs, maxb, int(partition_tokens))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        if fname == "pkv_decode_merge":
            raise ValueError("decode_merge needs the workspace decode_partials filled")
        workspace = _empty(stream, need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = getattr(lib, fname)(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                        _ptr(cache_seqlens), _ptr(k_new), _ptr(v_new), _ptr(out), B, Hq, Hkv, D,
                        NB, bs, maxb, float(softmax_scale), int(partition_tokens),
                        _ptr(workspace), wbytes, _ptr(err_flag), _stream(stream))
    if rc:
        raise PkvError(rc, fname)
    return out, workspace


DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None, *,
                   out, softmax_scale=None, partition_tokens=0, err_flag=None, stream=None):
    """pkv_decode_noalloc: decode with the library's static per-GPU scratch
    instead of a workspace, for callers that cannot allocate (graph capture).
    `out` is required; nothing is allocated.  Calls that overlap in time on
    one GPU share the scratch and race.  Returns out."""
    lib = _load()
    if out is None:
        raise ValueError("decode_noalloc allocates nothing: pass out")
    _need_gpu(q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new, out, err_flag)
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                 cache_seqlens=cache_seqlens, k_new=k_new, v_new=v_new, out=out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    if q.dim() != 4 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q [B, 1, Hq, D], caches [num_blocks, bs, Hkv, D], table [B, max_blocks]")
    B, _, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rc = lib.pkv_decode_noalloc(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_table), _ptr(cache_seqlens), _ptr(k_new), _ptr(v_new),
                                _ptr(out), B, Hq, Hkv, D, NB, bs, block_table.shape[1],
                                float(softmax_scale), int(partition_tokens), _ptr(err_flag),
                                _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_decode_noalloc")
    return out


def varlen(q, k, v, cu_seq_lens_q, cu_seq_lens_k, max_length_q, max_length_k, *,
           softmax_scale=None, out=None, err_flag=None, stream=None):
    """Attention over packed sequences, no mask.

    q [1, total_q, Hq, D]; k, v [1, total_k, Hkv, D]; cu_seq_lens_q/k
    [batch + 1] int32.  Returns out [1, total_q, Hq, D] in q's dtype.
    """
    lib = _load()
    _need_gpu(q, k, v, cu_seq_lens_q, cu_seq_lens_k, out, err_flag)
    _need_contig(q=q, k=k, v=v, cu_seq_lens_q=cu_seq_lens_q, cu_seq_lens_k=cu_seq_lens_k, out=out)
    dt = _dtype_code(q)
    if q.dim() != 4 or q.shape[0] != 1 or k.dim() != 4 or k.shape[0] != 1 or k.shape != v.shape:
        raise ValueError("q must be [1, total_q, Hq, D] and k, v [1, total_k, Hkv, D]")
    _, Tq, Hq, D = q.shape
    _, Tk, Hkv, D2 = k.shape
    if D2 != D or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share head_dim and dtype")
    if cu_seq_lens_q.dtype != torch.int32 or cu_seq_lens_k.dtype != torch.int32:
        raise TypeError("cu_seq_lens_q/k must be int32")
    if cu_seq_lens_q.dim() != 1 or cu_seq_lens_q.shape != cu_seq_lens_k.shape:
        raise ValueError("cu_seq_lens_q/k must both be [batch + 1]")
    B = cu_seq_lens_q.shape[0] - 1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rc = lib.pkv_check_varlen_args(dt, B, Tq, Tk, Hq, Hkv, D, int(max_length_q), int(max_length_k))
    if rc:
        raise PkvError(rc, "pkv_varlen arguments")
    if out is None:
        out = _empty(stream, q.shape, dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    rc = lib.pkv_varlen(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seq_lens_q), _ptr(cu_seq_lens_k),
                        int(max_length_q), int(max_length_k), _ptr(out), B, Tq, Tk, Hq, Hkv, D,
                        float(softmax_scale), _ptr(err_flag), _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_varlen")
    return out


def check_cache_write_args(dtype, batch, total, num_kv_heads, head_dim, num_blocks, block_size,
                           max_blocks_per_seq) -> int:
    """Host-only validation (no GPU needed); returns a status code."""
    return _load().pkv_check_cache_write_args(int(dtype), int(batch), int(total),
                                              int(num_kv_heads), int(head_dim), int(num_blocks),
                                              int(block_size), int(max_blocks_per_seq))


def check_varlen_paged_args(dtype, batch, total_q, num_heads, num_kv_heads, head_dim, num_blocks,
                            block_size, max_blocks_per_seq, max_length_q, max_length_k) -> int:
    """Host-only validation (no GPU needed); returns a status code."""
    return _load().pkv_check_varlen_paged_args(
        int(dtype), int(batch), int(total_q), int(num_heads), int(num_kv_heads), int(head_dim),
        int(num_blocks), int(block_size), int(max_blocks_per_seq), int(max_length_q),
        int(max_length_k))


def _cache_shape(k_cache, v_cache):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache/v_cache must both be [num_blocks, block_size, Hkv, D] of one dtype")
    return k_cache.shape


def cache_write(k, v, cu_seq_lens, start, k_cache, v_cache, block_table, *, err_flag=None,
                stream=None):
    """Writes packed rows into the paged cache in place.

    k, v [1, total, Hkv, D]; row cu_seq_lens[b] + i becomes token start[b] + i
    of sequence b (slot through block_table[b]).  Returns nothing; k_cache and
    v_cache are updated on the stream.
    """
    lib = _load()
    _need_gpu(k, v, cu_seq_lens, start, k_cache, v_cache, block_table, err_flag)
    _need_contig(k=k, v=v, cu_seq_lens=cu_seq_lens, start=start, k_cache=k_cache,
                 v_cache=v_cache, block_table=block_table)
    dt = _dtype_code(k)
    NB, bs, Hkv, D = _cache_shape(k_cache, v_cache)
    if k.dim() != 4 or k.shape[0] != 1 or k.shape != v.shape or tuple(k.shape[2:]) != (Hkv, D):
        raise ValueError("k, v must be [1, total, Hkv, D] matching the cache rows")
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype:
        raise ValueError("k, v and the caches must share a dtype")
    for name, t in (("cu_seq_lens", cu_seq_lens), ("start", start), ("block_table", block_table)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    B = start.shape[0]
    if cu_seq_lens.dim() != 1 or cu_seq_lens.shape[0] != B + 1 or block_table.dim() != 2 or \
            block_table.shape[0] != B:
        raise ValueError("cu_seq_lens must be [batch + 1], start [batch], block_table [batch, max_blocks]")
    total = k.shape[1]
    rc = lib.pkv_cache_write(dt, _ptr(k), _ptr(v), _ptr(cu_seq_lens), _ptr(start),
                             _ptr(k_cache), _ptr(v_cache), _ptr(block_table), B, total, Hkv, D,
                             NB, bs, block_table.shape[1], _ptr(err_flag), _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_cache_write")


def varlen_paged(q, k_cache, v_cache, block_table, cu_seq_lens_q, seqlens_k, max_length_q,
                 max_length_k, *, softmax_scale=None, out=None, err_flag=None, stream=None):
    """Varlen attention (no mask) with keys read through the block table.

    q [1, total_q, Hq, D]; caches [num_blocks, block_size, Hkv, D];
    block_table [batch, max_blocks] int32; cu_seq_lens_q [batch + 1] int32;
    seqlens_k [batch] int32 (keys of request b = its first seqlens_k[b]
    cached tokens).  Returns out [1, total_q, Hq, D] in q's dtype.
    """
    lib = _load()
    _need_gpu(q, k_cache, v_cache, block_table, cu_seq_lens_q, seqlens_k, out, err_flag)
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                 cu_seq_lens_q=cu_seq_lens_q, seqlens_k=seqlens_k, out=out)
    dt = _dtype_code(q)
    NB, bs, Hkv, D = _cache_shape(k_cache, v_cache)
    if q.dim() != 4 or q.shape[0] != 1 or q.shape[3] != D or k_cache.dtype != q.dtype:
        raise ValueError("q must be [1, total_q, Hq, D] with the caches' head_dim and dtype")
    for name, t in (("block_table", block_table), ("cu_seq_lens_q", cu_seq_lens_q),
                    ("seqlens_k", seqlens_k)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    B = seqlens_k.shape[0]
    if cu_seq_lens_q.dim() != 1 or cu_seq_lens_q.shape[0] != B + 1 or block_table.dim() != 2 or \
            block_table.shape[0] != B:
        raise ValueError("cu_seq_lens_q must be [batch + 1], seqlens_k [batch], block_table [batch, max_blocks]")
    _, Tq, Hq, _ = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rc = lib.pkv_check_varlen_paged_args(dt, B, Tq, Hq, Hkv, D, NB, bs, block_table.shape[1],
                                         int(max_length_q), int(max_length_k))
    if rc:
        raise PkvError(rc, "pkv_varlen_paged arguments")
    if out is None:
        out = _empty(stream, q.shape, dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    rc = lib.pkv_varlen_paged(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                              _ptr(cu_seq_lens_q), _ptr(seqlens_k), int(max_length_q),
                              int(max_length_k), _ptr(out), B, Tq, Hq, Hkv, D, NB, bs,
                              block_table.shape[1], float(softmax_scale), _ptr(err_flag),
                              _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_varlen_paged")
    return out


class OutOfBlocks(PkvError):
    """Not enough free blocks; the manager is unchanged."""


class BlockManager:
    """Host block manager of one paged pool (free list popped from its end,
    ref-counted sharing, copy-on-write decisions); native code in libpkv.

    Sequence ids are int keys.  ``append`` returns the copy-on-write pairs
    (src, dst) the caller must copy on the GPU (``copy_blocks``) before the
    new tokens are written.
    """

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _load()
        h = ctypes.c_void_p()
        rc = self._lib.pkv_bm_create(int(num_blocks), int(block_size), ctypes.byref(h))
        if rc:
            raise PkvError(rc, "pkv_bm_create")
        self._h = h
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    def _check(self, rc, what):
        if rc == ENOMEM:
            raise OutOfBlocks(rc, what)
        if rc:
            raise PkvError(rc, what)

    @property
    def num_free(self) -> int:
        return self._lib.pkv_bm_num_free(self._h)

    def ref_count(self, block: int) -> int:
        return self._lib.pkv_bm_ref_count(self._h, int(block))

    def allocate(self, seq: int, num_tokens: int) -> None:
        self._check(self._lib.pkv_bm_allocate(self._h, int(seq), int(num_tokens)), "allocate")

    def fork(self, parent: int, child: int) -> None:
        self._check(self._lib.pkv_bm_fork(self._h, int(parent), int(child)), "fork")

    def append(self, seq: int, num_tokens: int):
        """Grows seq; returns the list of copy-on-write (src, dst) pairs."""
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int()
        self._check(self._lib.pkv_bm_append(self._h, int(seq), int(num_tokens), ctypes.byref(src),
                                            ctypes.byref(dst), ctypes.byref(n)), "append")
        return [(src.value, dst.value)] if n.value else []

    def release(self, seq: int) -> None:
        self._check(self._lib.pkv_bm_release(self._h, int(seq)), "release")

    def seq_len(self, seq: int) -> int:
        return self._lib.pkv_bm_seq_len(self._h, int(seq))

    def table(self, seqs, max_blocks_per_seq: int):
        """(block_table [n, max_blocks_per_seq], seqlens [n]) as int32 CPU tensors."""
        ids = (ctypes.c_int64 * len(seqs))(*[int(x) for x in seqs])
        table = torch.empty((len(seqs), int(max_blocks_per_seq)), dtype=torch.int32)
        lens = torch.empty(len(seqs), dtype=torch.int32)
        self._check(self._lib.pkv_bm_table(self._h, ids, len(seqs), int(max_blocks_per_seq),
                                           ctypes.c_void_p(table.data_ptr()),
                                           ctypes.c_void_p(lens.data_ptr())), "table")
        return table, lens


def copy_blocks(k_cache, v_cache, src, dst, *, err_flag=None, stream=None):
    """Copies block src[i] onto block dst[i] in both pools (GPU, in place).
    src, dst: int32 GPU tensors of equal length."""
    lib = _load()
    _need_gpu(k_cache, v_cache, src, dst, err_flag)
    _need_contig(k_cache=k_cache, v_cache=v_cache, src=src, dst=dst)
    NB, bs, Hkv, D = _cache_shape(k_cache, v_cache)
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.shape != dst.shape or src.dim() != 1:
        raise ValueError("src and dst must be int32 vectors of one length")
    rc = lib.pkv_copy_blocks(_dtype_code(k_cache), _ptr(k_cache), _ptr(v_cache), _ptr(src),
                             _ptr(dst), src.shape[0], NB, bs, Hkv, D, _ptr(err_flag),
                             _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_copy_blocks")


def stream_read(buf, sink, workgroups=2048, nontemporal=True, stream=None):
    """Measurement aid: one plain streaming read of the device tensor `buf`
    (pkv_stream_read).  `sink` is a device tensor of at least workgroups *
    4096 bytes."""
    lib = _load()
    _need_gpu(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < workgroups * 4096 or not buf.is_contiguous():
        raise ValueError("sink too small or buf not contiguous")
    rc = lib.pkv_stream_read(_ptr(buf), nbytes, _ptr(sink), int(workgroups), int(bool(nontemporal)),
                             _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_stream_read")


def stream_copy(src, dst, workgroups=8192, stream=None):
    """Measurement aid: one plain device copy of `src` into `dst` (same
    byte size, contiguous, not overlapping; pkv_stream_copy)."""
    lib = _load()
    _need_gpu(src, dst)
    nbytes = src.numel() * src.element_size()
    if (dst.numel() * dst.element_size() != nbytes or not src.is_contiguous()
            or not dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous and of the same byte size")
    rc = lib.pkv_stream_copy(_ptr(src), _ptr(dst), nbytes, int(workgroups), _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_stream_copy")


def mfma_peak(sink, workgroups, iters, stream=None):
    """Measurement aid: a register-only loop of bf16 32x32x16 matrix-core
    products (pkv_mfma_peak); returns the flops of the call.  `sink` is a
    device tensor of at least workgroups * 1024 bytes."""
    lib = _load()
    _need_gpu(sink)
    if sink.numel() * sink.element_size() < workgroups * 1024:
        raise ValueError("sink too small")
    rc = lib.pkv_mfma_peak(_ptr(sink), int(workgroups), int(iters), _stream(stream))
    if rc:
        raise PkvError(rc, "pkv_mfma_peak")
    return int(workgroups) * 4 * int(iters) * 4 * 32768
