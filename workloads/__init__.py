"""Seeded synthetic inputs for paged attention, shared by the GPU path's tests,
the benchmark and the oracle checks.

This module draws numbers and lays them out; it holds none of the attention
arithmetic.  The same bytes it produces are handed to the GPU library and (via
a host copy) to the oracle.

Draw order for a case with seed s:
  1. lengths, then the physical-block permutation, from numpy PCG64(s);
  2. q, the K pool, the V pool, k_new, v_new, from a torch generator seeded
     with s on the target device, N(0, 1) in fp32 and rounded to bf16
     (round-to-nearest-even) for bf16 cases.
The GPU and CPU torch generators produce different streams; every comparison
therefore feeds both sides the bytes of ONE generation.

Block placement: the permutation of the pool is handed out in order, sequence
0 first, each sequence taking ceil(len / block_size) blocks; unused table
entries are -1.  The whole pool is filled with N(0, 1), so blocks that no
sequence owns hold finite garbage.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .blocks import BlockPool, OutOfBlocks  # noqa: F401  (re-export)

# The workloads the pages' decode and prefill batches are shaped like.
CONFIGS = {
    # HF "paged attention" page, decode example: 3 sequences with 30, 32, 70
    # cached tokens, block size 32, 4 table entries per sequence, the printed
    # table; fp32, 4 q heads = 4 kv heads, head_dim 64, new token appended.
    "tiny_decode_fp32": dict(
        kind="decode", seed=1, dtype="fp32", batch=3, num_heads=4, num_kv_heads=4, head_dim=64,
        block_size=32, lengths=[30, 32, 70], num_blocks=8, max_blocks_per_seq=4,
        table=[[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]], append=True,
        partition_tokens=0),
    # Decode batch, GQA 4: 64 sequences, 512..4096 cached tokens, 16-token
    # blocks drawn from a 20000-block pool.
    "decode_b64_gqa4": dict(
        kind="decode", seed=2, dtype="bf16", batch=64, num_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, lengths=("uniform", 512, 4096), num_blocks=20000,
        max_blocks_per_seq=256, append=False, partition_tokens=0),
    # Long-context decode, GQA 8: 256 sequences, log-uniform 1k..32k tokens,
    # pool = total blocks + 5 %, 512-token split-context partitions.
    "decode_b256_long": dict(
        kind="decode", seed=3, dtype="bf16", batch=256, num_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, lengths=("loguniform", 1024, 32768),
        num_blocks="total+5%", max_blocks_per_seq=2048, append=False, partition_tokens=512),
    # Varlen prefill: 16 sequences, q lengths 1..2048, keys = q length plus a
    # cached prefix of 0..2048, no mask.
    "varlen_prefill": dict(
        kind="varlen", seed=4, dtype="bf16", batch=16, num_heads=32, num_kv_heads=8,
        head_dim=128, q_lengths=("uniform", 1, 2048), prefix=("uniform", 0, 2048)),
    # Mixed continuous-batching step: 512 decode sequences (16..8192 tokens,
    # append with a fresh block from the free list at a block boundary) and 8
    # prefill sequences of 1024 tokens through the varlen path.
    "mixed_step": dict(
        kind="mixed", seed=5, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        decode=dict(batch=512, block_size=16, lengths=("uniform", 16, 8192),
                    num_blocks="total+5%", max_blocks_per_seq=513, append=True,
                    partition_tokens=512),
        prefill=dict(batch=8, q_lengths=("fixed", 1024), prefix=("fixed", 0))),
}


def draw_lengths(rng: np.random.Generator, spec, n: int) -> np.ndarray:
    """Sequence lengths: a list, ("fixed", v), ("uniform", lo, hi) integers
    inclusive, or ("loguniform", lo, hi) as floor(exp(U[ln lo, ln hi]))."""
    if isinstance(spec, (list, np.ndarray)):
        return np.asarray(spec, dtype=np.int64)
    kind = spec[0]
    if kind == "fixed":
        return np.full(n, spec[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=n, endpoint=True).astype(np.int64)
    if kind == "loguniform":
        u = rng.uniform(math.log(spec[1]), math.log(spec[2]), size=n)
        return np.minimum(np.floor(np.exp(u)).astype(np.int64), spec[2])
    raise ValueError(spec)


def _randn(shape, gen, device, dtype, chunk=1 << 27):
    """N(0,1) tensor of `shape`, drawn in fp32 chunk by chunk and rounded to
    `dtype` (bf16 rounding is round-to-nearest-even)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def _tdtype(name):
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclass
class DecodeCase:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    cache_seqlens: torch.Tensor
    k_new: torch.Tensor | None
    v_new: torch.Tensor | None
    softmax_scale: float
    partition_tokens: int
    lengths: np.ndarray           # cache_seqlens as numpy (before the append)
    free_list: list = field(default_factory=list)
    seed: int = 0

    @property
    def attended(self) -> np.ndarray:
        return self.lengths + (1 if self.k_new is not None else 0)


@dataclass
class VarlenCase:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seq_lens_q: torch.Tensor
    cu_seq_lens_k: torch.Tensor
    max_length_q: int
    max_length_k: int
    softmax_scale: float
    q_lengths: np.ndarray
    k_lengths: np.ndarray
    seed: int = 0


def make_decode(*, seed, dtype, batch, num_heads, num_kv_heads, head_dim, block_size, lengths,
                num_blocks, max_blocks_per_seq=None, append=False, partition_tokens=0,
                table=None, free_list_boundary_alloc=False, device="cpu", softmax_scale=None,
                placement="permuted", **_):
    """A paged decode batch.

    With ``append`` the table also holds the block that receives the new
    token.  With ``free_list_boundary_alloc`` (mixed step) the initial
    placement covers only the cached tokens; the unused rest of the
    permutation is a LIFO free list, and a sequence whose new token starts a
    block gets one block popped from it at table index len // block_size.
    """
    rng = np.random.default_rng(seed)
    L = draw_lengths(rng, lengths, batch)
    bs = block_size
    extra = 1 if append else 0
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(math.ceil((L.max() + extra) / bs)) if batch else 1)
    placed_len = L if free_list_boundary_alloc else L + extra
    need = np.ceil(placed_len / bs).astype(np.int64)
    if num_blocks == "total+5%":
        num_blocks = int(math.ceil(1.05 * int(need.sum())))
    free = []
    if table is not None:
        bt = np.asarray(table, dtype=np.int32)
    else:
        perm = rng.permutation(num_blocks).astype(np.int32)
        if placement == "contiguous":      # same draws, blocks handed out in order
            perm = np.arange(num_blocks, dtype=np.int32)
        if int(need.sum()) > num_blocks:
            raise ValueError("pool too small for the drawn lengths")
        bt = np.full((batch, max_blocks_per_seq), -1, dtype=np.int32)
        pos = 0
        for i in range(batch):
            n = int(need[i])
            bt[i, :n] = perm[pos:pos + n]
            pos += n
        free = list(perm[pos:])
        if free_list_boundary_alloc and append:
            pool = BlockPool(free)
            for i in range(batch):
                if L[i] % bs == 0:
                    bt[i, L[i] // bs] = pool.pop()
            free = pool.free
    tdt = _tdtype(dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _randn((batch, 1, num_heads, head_dim), gen, device, tdt)
    kc = _randn((num_blocks, bs, num_kv_heads, head_dim), gen, device, tdt)
    vc = _randn((num_blocks, bs, num_kv_heads, head_dim), gen, device, tdt)
    kn = vn = None
    if append:
        kn = _randn((batch, 1, num_kv_heads, head_dim), gen, device, tdt)
        vn = _randn((batch, 1, num_kv_heads, head_dim), gen, device, tdt)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return DecodeCase(q=q, k_cache=kc, v_cache=vc,
                      block_table=torch.from_numpy(bt).to(device),
                      cache_seqlens=torch.from_numpy(L.astype(np.int32)).to(device),
                      k_new=kn, v_new=vn, softmax_scale=softmax_scale,
                      partition_tokens=partition_tokens, lengths=L, free_list=free, seed=seed)


def make_varlen(*, seed, dtype, batch, num_heads, num_kv_heads, head_dim, q_lengths, prefix=None,
                k_lengths=None, device="cpu", softmax_scale=None, **_):
    """A packed varlen batch: len_k = len_q + prefix unless k_lengths is given."""
    rng = np.random.default_rng(seed)
    lq = draw_lengths(rng, q_lengths, batch)
    if k_lengths is not None:
        lk = draw_lengths(rng, k_lengths, batch)
    else:
        lk = lq + draw_lengths(rng, prefix, batch)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    tdt = _tdtype(dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _randn((1, int(cq[-1]), num_heads, head_dim), gen, device, tdt)
    k = _randn((1, int(ck[-1]), num_kv_heads, head_dim), gen, device, tdt)
    v = _randn((1, int(ck[-1]), num_kv_heads, head_dim), gen, device, tdt)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return VarlenCase(q=q, k=k, v=v, cu_seq_lens_q=torch.from_numpy(cq).to(device),
                      cu_seq_lens_k=torch.from_numpy(ck).to(device),
                      max_length_q=int(lq.max()) if batch else 0,
                      max_length_k=int(lk.max()) if batch else 0,
                      softmax_scale=softmax_scale, q_lengths=lq, k_lengths=lk, seed=seed)


@dataclass
class PagedPrefillCase:
    """A prefill step over a paged cache: request b has prefix[b] tokens
    cached already and q_lengths[b] new tokens whose K/V rows (packed) are to
    be written after them; its queries attend prefix + new keys."""
    q: torch.Tensor             # [1, total_new, Hq, D]
    k_new: torch.Tensor         # [1, total_new, Hkv, D] packed new rows
    v_new: torch.Tensor
    k_cache: torch.Tensor       # [num_blocks, block_size, Hkv, D] (prefix slots filled)
    v_cache: torch.Tensor
    block_table: torch.Tensor   # [batch, max_blocks] int32, covers prefix + new
    cu_seq_lens_q: torch.Tensor  # [batch + 1] int32 (also the new rows' cu)
    start: torch.Tensor         # [batch] int32 = prefix
    seqlens_k: torch.Tensor     # [batch] int32 = prefix + new
    max_length_q: int
    max_length_k: int
    softmax_scale: float
    q_lengths: np.ndarray
    prefix: np.ndarray
    seed: int = 0


def make_paged_prefill(*, seed, dtype, batch, num_heads, num_kv_heads, head_dim, q_lengths,
                       prefix, block_size=16, num_blocks="total+5%", device="cpu",
                       softmax_scale=None, **_):
    """Same lengths as make_varlen with the same seed (len_k = len_q +
    prefix), laid out in a paged pool: each sequence's prefix + new tokens get
    blocks from a seeded permutation of the pool; the pool (prefix included)
    is N(0,1)."""
    rng = np.random.default_rng(seed)
    lq = draw_lengths(rng, q_lengths, batch)
    pre = draw_lengths(rng, prefix, batch)
    tot = lq + pre
    bs = block_size
    need = np.ceil(tot / bs).astype(np.int64)
    if num_blocks == "total+5%":
        num_blocks = int(math.ceil(1.05 * int(need.sum()))) + 1
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = max(1, int(need.max()) if batch else 1)
    bt = np.full((batch, mb), -1, dtype=np.int32)
    pos = 0
    for i in range(batch):
        n = int(need[i])
        bt[i, :n] = perm[pos:pos + n]
        pos += n
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    tdt = _tdtype(dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _randn((1, int(cq[-1]), num_heads, head_dim), gen, device, tdt)
    kn = _randn((1, int(cq[-1]), num_kv_heads, head_dim), gen, device, tdt)
    vn = _randn((1, int(cq[-1]), num_kv_heads, head_dim), gen, device, tdt)
    kc = _randn((num_blocks, bs, num_kv_heads, head_dim), gen, device, tdt)
    vc = _randn((num_blocks, bs, num_kv_heads, head_dim), gen, device, tdt)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(device)
    return PagedPrefillCase(q=q, k_new=kn, v_new=vn, k_cache=kc, v_cache=vc, block_table=i32(bt),
                            cu_seq_lens_q=i32(cq), start=i32(pre), seqlens_k=i32(tot),
                            max_length_q=int(lq.max()) if batch else 0,
                            max_length_k=int(tot.max()) if batch else 0,
                            softmax_scale=softmax_scale, q_lengths=lq, prefix=pre, seed=seed)


def make_config(name: str, device="cpu", part=None, **overrides):
    """The named workload: a DecodeCase, a VarlenCase, or for the mixed step
    (decode, varlen) -- or just one of them with part="decode"/"prefill".
    `overrides` replace entries of a decode or varlen workload (e.g.
    placement="contiguous": the same draws with blocks handed out in order)."""
    c = dict(CONFIGS[name])
    kind = c.pop("kind")
    c.update(overrides)
    if kind == "decode":
        return make_decode(device=device, **c)
    if kind == "varlen":
        return make_varlen(device=device, **c)
    common = {k: c[k] for k in ("dtype", "num_heads", "num_kv_heads", "head_dim")}
    d = p = None
    if part in (None, "decode"):
        d = make_decode(device=device, seed=c["seed"], free_list_boundary_alloc=True, **common,
                        **c["decode"])
    if part in (None, "prefill"):
        p = make_varlen(device=device, seed=c["seed"] + 1000, **common, **c["prefill"])
    if part == "decode":
        return d
    if part == "prefill":
        return p
    return d, p


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy of a tensor's bytes: float32 stays float32, bf16 becomes
    its uint16 bit patterns (the oracle widens those exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_float(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)
