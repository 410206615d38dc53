"""Pins of the oracle's paged-prefill functions (cache write of packed rows,
varlen attention reading its keys through the block table).

CPU only.  The placement checks use the pages' worked examples (the
60-token table 7, 1, 12, 4 and the HF decode example's append slots); the
attention checks tie the paged varlen to the packed varlen -- itself pinned by
the HF varlen example and by a 50-digit brute force -- bit for bit, plus the
HF varlen example and the scalar-head example run through a paged pool.
"""
import numpy as np
import pytest

import oracle
from tests import bruteforce


def _bf16_bits(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if dtype == "fp32" else _bf16_bits(x)


def _place(pool, table_row, rows, bs, start=0):
    """Puts rows[i] at token start+i of a sequence by plain numpy indexing
    (independent of the oracle's cache write)."""
    for i, r in enumerate(rows):
        t = start + i
        pool[table_row[t // bs], t % bs] = r


# ------------------------------------------------------------- cache write

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_cache_write_sixty_token_placement(dtype, golden):
    g = golden("notes_60_token_example.json")
    rng = np.random.default_rng(21)
    bs, n = g["block_size"], g["length"]
    kc, vc = _draw(rng, (13, bs, 2, 4), dtype), _draw(rng, (13, bs, 2, 4), dtype)
    k0, v0 = kc.copy(), vc.copy()
    k, v = _draw(rng, (1, n, 2, 4), dtype), _draw(rng, (1, n, 2, 4), dtype)
    oracle.cache_write(k, v, [0, n], [0], kc, vc, np.array([g["block_table"]], np.int32))
    written = set()
    for lo, hi, phys in g["token_ranges_to_physical"]:
        for t in range(lo, hi + 1):
            assert np.array_equal(kc[phys, t - lo], k[0, t])
            assert np.array_equal(vc[phys, t - lo], v[0, t])
            written.add((phys, t - lo))
    for pb in range(13):
        for o in range(bs):
            if (pb, o) not in written:
                assert np.array_equal(kc[pb, o], k0[pb, o]) and np.array_equal(vc[pb, o], v0[pb, o])


def test_cache_write_decode_example_slots(golden):
    """One new row per sequence at start = cached length lands exactly where
    the HF decode example puts each new token."""
    g = golden("hf_decode_example.json")
    rng = np.random.default_rng(22)
    bs = g["block_size"]
    kc, vc = _draw(rng, (8, bs, 4, 8), "bf16"), _draw(rng, (8, bs, 4, 8), "bf16")
    k0 = kc.copy()
    k, v = _draw(rng, (1, 3, 4, 8), "bf16"), _draw(rng, (1, 3, 4, 8), "bf16")
    oracle.cache_write(k, v, [0, 1, 2, 3], g["cache_seqlens"], kc, vc,
                       np.array(g["block_table"], np.int32))
    changed = {tuple(x[:2]) for x in np.argwhere(kc != k0)}
    want = {(pb, g["cache_seqlens"][i] % bs) for i, pb in enumerate(g["new_token_physical_block"])}
    assert changed <= want
    for i, pb in enumerate(g["new_token_physical_block"]):
        o = g["cache_seqlens"][i] % bs
        assert np.array_equal(kc[pb, o], k[0, i]) and np.array_equal(vc[pb, o], v[0, i])


def test_cache_write_errors_leave_the_pool_untouched(golden):
    g = golden("hf_decode_example.json")
    bt = np.array(g["block_table"], np.int32)
    kc = np.zeros((8, 32, 1, 4), np.float32)
    k = np.ones((1, 3, 1, 4), np.float32)
    cases = [
        ([0, 1, 2, 3], [30, 32, 96], 2),   # sequence 2's token 96 needs table entry 3 = -1
        ([0, 1, 2, 3], [30, 32, 128], 3),  # token 128 is past the 4-entry row
        ([0, 1, 2, 3], [30, -1, 70], 4),   # negative start
        ([0, 2, 1, 3], [30, 32, 70], 5),   # decreasing cu
    ]
    for cu, start, code in cases:
        kk, vv = kc.copy(), kc.copy()
        with pytest.raises(oracle.OracleError) as e:
            oracle.cache_write(k, k, cu, start, kk, vv, bt)
        assert e.value.code == code
        assert np.array_equal(kk, kc) and np.array_equal(vv, kc)


# ------------------------------------------------- varlen over a paged pool

def _paged_copy(rng, k, v, cu_k, bs, extra_blocks=3, junk=False):
    """Scatter packed key rows into a randomly permuted pool; returns the
    pools, the block table and seqlens_k."""
    lens = np.diff(np.asarray(cu_k))
    nblk = [-(-int(L) // bs) for L in lens]
    mb = max(max(nblk), 1)
    pool_n = sum(nblk) + extra_blocks
    perm = rng.permutation(pool_n)
    table = np.full((len(lens), mb), -1, np.int32)
    shape = (pool_n, bs) + k.shape[-2:]
    kc = np.full(shape, np.nan, k.dtype) if (junk and k.dtype == np.float32) else np.zeros(shape, k.dtype)
    vc = kc.copy()
    used = 0
    for b, L in enumerate(lens):
        table[b, :nblk[b]] = perm[used:used + nblk[b]]
        used += nblk[b]
        _place(kc, table[b], k.reshape(k.shape[-3:])[cu_k[b]:cu_k[b + 1]], bs)
        _place(vc, table[b], v.reshape(v.shape[-3:])[cu_k[b]:cu_k[b + 1]], bs)
    return kc, vc, table, lens.astype(np.int32)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("bs", [4, 16])
def test_varlen_paged_equals_packed_bitwise(dtype, bs):
    rng = np.random.default_rng(23 + bs)
    lq = np.array([3, 0, 7, 1, 12], np.int32)
    lk = np.array([5, 4, 9, 0, 33], np.int32)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Hq, Hkv, D = 6, 2, 8
    q = _draw(rng, (1, cq[-1], Hq, D), dtype)
    k, v = _draw(rng, (1, ck[-1], Hkv, D), dtype), _draw(rng, (1, ck[-1], Hkv, D), dtype)
    kc, vc, table, sk = _paged_copy(rng, k, v, ck, bs, junk=True)
    paged = oracle.varlen_paged(q, kc, vc, table, cq, sk, lq.max(), lk.max())
    packed = oracle.varlen(q, k, v, cq, ck, lq.max(), lk.max())
    assert np.array_equal(paged, packed)


def test_varlen_paged_hf_example(golden):
    """The HF varlen example with its 8 key rows in a paged pool: request 0
    (no key) gives zeros, request 1 (one key) gives that value exactly,
    request 2 matches the decimal brute force."""
    g = golden("hf_varlen_example.json")
    rng = np.random.default_rng(24)
    Hq, Hkv, D = 4, 2, 8
    q = rng.standard_normal((1, g["total_q"], Hq, D)).astype(np.float32)
    k = rng.standard_normal((1, g["total_k"], Hkv, D)).astype(np.float32)
    v = rng.standard_normal((1, g["total_k"], Hkv, D)).astype(np.float32)
    kc, vc, table, sk = _paged_copy(rng, k, v, g["cu_seq_lens_k"], 4, junk=True)
    assert sk.tolist() == g["k_lengths"]
    out = oracle.varlen_paged(q, kc, vc, table, g["cu_seq_lens_q"], sk, g["max_length_q"],
                              g["max_length_k"])
    assert np.all(out[:10] == 0)
    for r in range(10, 13):
        for h in range(Hq):
            assert np.array_equal(out[r, h], v[0, 0, h // 2].astype(np.float64))
    want = bruteforce.varlen(q[0], k[0], v[0], g["cu_seq_lens_q"], g["cu_seq_lens_k"])
    np.testing.assert_allclose(out[13], want[13], rtol=1e-13, atol=1e-15)


def test_varlen_paged_scalar_head(golden):
    g = golden("scalar_head_example.json")
    bs, n = g["block_size"], g["length"]
    for placement in ([4, 1], [1, 0], [2, 4]):
        kc = np.full((5, bs, 1, 1), g["key"], np.float32)
        vc = np.full((5, bs, 1, 1), np.nan, np.float32)
        for t, val in enumerate(g["values"]):
            vc[placement[t // bs], t % bs, 0, 0] = val
        q = np.full((1, 2, 1, 1), g["query"], np.float32)   # two query rows, same request
        out = oracle.varlen_paged(q, kc, vc, np.array([placement], np.int32), [0, 2], [n], 2, n)
        assert out[0, 0, 0] == g["output"] and out[1, 0, 0] == g["output"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prefill_write_then_attend_equals_packed(dtype):
    """A prefill step over a cached prefix: the new rows are written after the
    prefix with the cache write, then the queries attend prefix + new through
    the table; the result equals packed varlen over the concatenated keys."""
    rng = np.random.default_rng(25)
    bs, Hq, Hkv, D = 8, 4, 2, 8
    prefix = np.array([0, 5, 16, 3], np.int32)
    new = np.array([6, 1, 9, 0], np.int32)
    tot = prefix + new
    B = len(prefix)
    nblk = [-(-int(t) // bs) for t in tot]
    pool_n = sum(nblk) + 2
    perm = rng.permutation(pool_n)
    table = np.full((B, max(nblk)), -1, np.int32)
    used = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[used:used + nblk[b]]
        used += nblk[b]
    kc = _draw(rng, (pool_n, bs, Hkv, D), dtype)
    vc = _draw(rng, (pool_n, bs, Hkv, D), dtype)
    k_full, v_full = [], []
    for b in range(B):   # the prefix already in the pool
        kp, vp = _draw(rng, (prefix[b], Hkv, D), dtype), _draw(rng, (prefix[b], Hkv, D), dtype)
        _place(kc, table[b], kp, bs)
        _place(vc, table[b], vp, bs)
        k_full.append(kp)
        v_full.append(vp)
    cn = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    kn, vn = _draw(rng, (1, cn[-1], Hkv, D), dtype), _draw(rng, (1, cn[-1], Hkv, D), dtype)
    oracle.cache_write(kn, vn, cn, prefix, kc, vc, table)
    q = _draw(rng, (1, cn[-1], Hq, D), dtype)
    paged = oracle.varlen_paged(q, kc, vc, table, cn, tot, new.max(), tot.max())
    kcat = np.concatenate([np.concatenate([k_full[b], kn[0, cn[b]:cn[b + 1]]]) for b in range(B)])
    vcat = np.concatenate([np.concatenate([v_full[b], vn[0, cn[b]:cn[b + 1]]]) for b in range(B)])
    ck = np.concatenate([[0], np.cumsum(tot)]).astype(np.int32)
    packed = oracle.varlen(q, kcat[None], vcat[None], cn, ck, new.max(), tot.max())
    assert np.array_equal(paged, packed)


def test_varlen_paged_errors():
    bt = np.array([[1, -1], [0, 2]], np.int32)
    kc = np.zeros((3, 4, 1, 4), np.float32)
    q = np.zeros((1, 3, 1, 4), np.float32)
    cases = [
        ([0, 1, 3], [5, 8], 8, 8, 2),     # sequence 0 needs entry 1 = -1
        ([0, 1, 3], [4, 9], 8, 9, 3),     # 9 keys need a third entry
        ([0, 1, 3], [-1, 8], 8, 8, 4),
        ([0, 1, 3], [4, 8], 8, 7, 6),     # 8 keys > max_length_k 7
        ([0, 2, 1], [4, 8], 8, 8, 5),
    ]
    for cu, sk, mq, mk, code in cases:
        with pytest.raises(oracle.OracleError) as e:
            oracle.varlen_paged(q, kc, kc, bt, cu, sk, mq, mk)
        assert e.value.code == code
