"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None compares the oracle with itself: each
checks a printed value from a worked example on the pages, a closed form, an
invariant the pages state, or a 50-digit brute force on tiny inputs.
"""
import math

import numpy as np
import pytest

import oracle
from tests import bruteforce


def _bf16_bits(x):
    """bf16 bit patterns of float32 values (round to nearest even)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return r


# ----------------------------------------------------------- index examples

def test_varlen_example_cumulative_lengths(golden):
    g = golden("hf_varlen_example.json")
    cq = oracle.cu_from_lengths(g["q_lengths"])
    ck = oracle.cu_from_lengths(g["k_lengths"])
    assert cq.tolist() == g["cu_seq_lens_q"]
    assert ck.tolist() == g["cu_seq_lens_k"]
    assert max(g["q_lengths"]) == g["max_length_q"] and max(g["k_lengths"]) == g["max_length_k"]
    assert cq[-1] == g["total_q"] and ck[-1] == g["total_k"]


def test_varlen_example_request_index(golden):
    g = golden("hf_varlen_example.json")
    assert oracle.request_index(g["cu_seq_lens_q"], g["total_q"]).tolist() == g["q_request_index"]
    assert oracle.request_index(g["cu_seq_lens_k"], g["total_k"]).tolist() == g["k_request_index"]


def test_request_index_rejects_bad_cu():
    with pytest.raises(oracle.OracleError):
        oracle.request_index([0, 5, 3], 3)      # decreasing
    with pytest.raises(oracle.OracleError):
        oracle.request_index([1, 5], 5)         # not starting at 0
    with pytest.raises(oracle.OracleError):
        oracle.request_index([0, 5], 6)         # wrong total


def test_decode_example_append_slots(golden):
    g = golden("hf_decode_example.json")
    bt = np.array(g["block_table"], dtype=np.int32)
    bs = g["block_size"]
    fits, phys = [], []
    for i, L in enumerate(g["cache_seqlens"]):
        j, o, pb = oracle.locate(bt, 8, bs, i, L)
        # the token at slot L fits in the block already holding cached tokens
        # iff it is not the first slot of a fresh logical block
        fits.append(o != 0)
        phys.append(pb)
        # the cached tokens live exactly in the listed blocks up to this one
        assert g["listed_cache_blocks"][i][: j + 1] == bt[i, : j + 1].tolist()
    assert fits == g["new_token_fits_in_current_block"]
    assert phys == g["new_token_physical_block"]
    assert [oracle.locate(bt, 8, bs, i, L)[:2] for i, L in enumerate(g["cache_seqlens"])] == \
        [(0, 30), (1, 0), (2, 6)]


def test_decode_example_unallocated_entry_is_an_error(golden):
    g = golden("hf_decode_example.json")
    bt = np.array(g["block_table"], dtype=np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.locate(bt, 8, g["block_size"], 0, 32)   # logical block 1 of sequence 0 is -1
    assert e.value.code == 2
    with pytest.raises(oracle.OracleError) as e:
        oracle.locate(bt, 8, g["block_size"], 2, 4 * 32)  # past the 4-entry row
    assert e.value.code == 3


def test_sixty_token_placement(golden):
    g = golden("notes_60_token_example.json")
    bt = np.array([g["block_table"]], dtype=np.int32)
    counts = {}
    for t in range(g["length"]):
        j, o, pb = oracle.locate(bt, 13, g["block_size"], 0, t)
        counts[j] = counts.get(j, 0) + 1
        for lo, hi, phys in g["token_ranges_to_physical"]:
            if lo <= t <= hi:
                assert pb == phys and o == t - lo
    assert [counts[j] for j in range(4)] == g["tokens_per_block"]


# ------------------------------------------------------- decode: the append

def _tiny_decode_case(rng, dtype, B=3, Hq=4, Hkv=4, D=8, bs=32, NB=8, table=None, lengths=None):
    table = np.array(table if table is not None else [[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]],
                     dtype=np.int32)
    lengths = np.array(lengths if lengths is not None else [30, 32, 70], dtype=np.int32)

    def draw(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return x if dtype == "fp32" else _bf16_bits(x)

    q = draw((B, 1, Hq, D))
    kc, vc = draw((NB, bs, Hkv, D)), draw((NB, bs, Hkv, D))
    kn, vn = draw((B, 1, Hkv, D)), draw((B, 1, Hkv, D))
    return q, kc, vc, table, lengths, kn, vn


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_example_append_is_the_only_write(dtype, golden):
    g = golden("hf_decode_example.json")
    rng = np.random.default_rng(11)
    q, kc, vc, bt, L, kn, vn = _tiny_decode_case(rng, dtype)
    k0, v0 = kc.copy(), vc.copy()
    oracle.decode(q, kc, vc, bt, L, kn, vn)
    changed_k = {tuple(x[:2]) for x in np.argwhere(kc != k0)}
    changed_v = {tuple(x[:2]) for x in np.argwhere(vc != v0)}
    want = {(pb, L[i] % g["block_size"]) for i, pb in enumerate(g["new_token_physical_block"])}
    assert changed_k <= want and changed_v <= want
    for i, pb in enumerate(g["new_token_physical_block"]):
        o = L[i] % g["block_size"]
        assert np.array_equal(kc[pb, o], kn[i, 0]) and np.array_equal(vc[pb, o], vn[i, 0])
    for untouched in (4, 7):   # blocks no sequence owns
        assert np.array_equal(kc[untouched], k0[untouched])


def test_decode_append_then_attend_counts_new_token():
    """With one cached token whose value is 0 and a new token of value 1 and
    equal scores, the output is 0.5: the new token is attended."""
    q = np.ones((1, 1, 1, 1), np.float32)
    kc = np.zeros((2, 4, 1, 1), np.float32)
    vc = np.zeros((2, 4, 1, 1), np.float32)
    out = oracle.decode(q, kc, vc, np.array([[1, -1]], np.int32), np.array([1], np.int32),
                        np.zeros((1, 1, 1, 1), np.float32), np.ones((1, 1, 1, 1), np.float32),
                        scale=1.0)
    assert out[0, 0, 0] == 0.5
    assert vc[1, 1, 0, 0] == 1.0


def test_decode_errors():
    q, kc, vc, bt, L, kn, vn = _tiny_decode_case(np.random.default_rng(0), "fp32")
    bad = bt.copy()
    bad[2, 2] = -1                       # sequence 2 needs its third block
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(q, kc.copy(), vc.copy(), bad, L)
    assert e.value.code == 2
    bad = bt.copy()
    bad[1, 1] = 8                        # outside an 8-block pool
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(q, kc.copy(), vc.copy(), bad, L, kn, vn)
    assert e.value.code == 2
    with pytest.raises(oracle.OracleError) as e:  # 128 cached + 1 does not fit 4 x 32
        oracle.decode(q, kc.copy(), vc.copy(), bt, np.array([30, 32, 128], np.int32), kn, vn)
    assert e.value.code == 3


# ------------------------------------------------- the scalar-head example

def test_scalar_head_example(golden):
    g = golden("scalar_head_example.json")
    bs, n = g["block_size"], g["length"]
    nblk = -(-n // bs)
    assert nblk == g["blocks_needed"] and nblk * bs == g["slots"]
    assert n - (nblk - 1) * bs == g["entries_in_second_block"]
    assert nblk * bs - n == g["free_slots_in_second_block"]
    q = np.full((1, 1, 1, 1), g["query"], np.float32)
    for placement in ([4, 1], [0, 1], [1, 0], [3, 2], [2, 4]):
        kc = np.full((5, bs, 1, 1), g["key"], np.float32)
        vc = np.full((5, bs, 1, 1), np.nan, np.float32)     # free slots hold junk
        for t, v in enumerate(g["values"]):
            vc[placement[t // bs], t % bs, 0, 0] = v
        out = oracle.decode(q, kc, vc, np.array([placement], np.int32), np.array([n], np.int32))
        assert out[0, 0, 0] == g["output"]
    # the same through the 4 -> 5 transition: 4 cached values, the 5th appended
    kc = np.zeros((5, bs, 1, 1), np.float32)
    vc = np.full((5, bs, 1, 1), np.nan, np.float32)
    for t in range(4):
        vc[4, t, 0, 0] = g["values"][t]
    out = oracle.decode(q, kc, vc, np.array([g["logical_to_physical"]], np.int32),
                        np.array([4], np.int32), np.zeros((1, 1, 1, 1), np.float32),
                        np.full((1, 1, 1, 1), g["values"][4], np.float32))
    assert out[0, 0, 0] == g["output"]


@pytest.mark.parametrize("n", [1, 2, 4, 7, 9, 16])
def test_scalar_head_mean_closed_form(n):
    """Equal weights give the mean of 1..n = (n + 1) / 2, exactly."""
    bs = 4
    nblk = -(-n // bs)
    perm = np.random.default_rng(n).permutation(nblk + 3)[:nblk]
    kc = np.zeros((nblk + 3, bs, 1, 1), np.float32)
    vc = np.zeros((nblk + 3, bs, 1, 1), np.float32)
    for t in range(n):
        vc[perm[t // bs], t % bs, 0, 0] = t + 1
    out = oracle.decode(np.ones((1, 1, 1, 1), np.float32), kc, vc, perm[None].astype(np.int32),
                        np.array([n], np.int32))
    assert out[0, 0, 0] == (n + 1) / 2


# ----------------------------------------------------------- closed forms

def test_single_key_gives_its_value():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 1, 2, 16)).astype(np.float32)
    kc = rng.standard_normal((1, 1, 2, 16)).astype(np.float32)
    vc = v.copy()
    q = rng.standard_normal((1, 1, 4, 16)).astype(np.float32)
    out = oracle.decode(q, kc, vc, np.array([[0]], np.int32), np.array([1], np.int32))
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, 0, h // 2].astype(np.float64))


def test_equal_scores_give_the_mean():
    rng = np.random.default_rng(4)
    vc = rng.standard_normal((3, 4, 1, 8)).astype(np.float32)
    kc = np.tile(rng.standard_normal((1, 1, 1, 8)).astype(np.float32), (3, 4, 1, 1))  # identical keys
    out = oracle.decode(rng.standard_normal((1, 1, 1, 8)).astype(np.float32), kc, vc,
                        np.array([[2, 0, 1]], np.int32), np.array([10], np.int32))
    rows = np.concatenate([vc[2], vc[0], vc[1][:2]]).astype(np.float64)[:, 0]
    want = np.array([math.fsum(rows[:, c]) / 10 for c in range(8)])
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)


def test_dominant_score_selects_its_value_and_needs_the_max_shift():
    """A score 800 above the rest: e^(-800) underflows to 0 in fp64, so the
    output is exactly that token's value.  Without subtracting the max,
    e^800 overflows and the result is not finite."""
    kc = np.zeros((2, 4, 1, 1), np.float32)
    kc[1, 2, 0, 0] = 800.0
    vc = np.arange(8, dtype=np.float32).reshape(2, 4, 1, 1) + 10
    out = oracle.decode(np.ones((1, 1, 1, 1), np.float32), kc, vc, np.array([[0, 1]], np.int32),
                        np.array([8], np.int32), scale=1.0)
    assert out[0, 0, 0] == vc[1, 2, 0, 0]


def test_output_within_value_bounds():
    rng = np.random.default_rng(5)
    q, kc, vc, bt, L, kn, vn = _tiny_decode_case(rng, "fp32", D=16)
    out = oracle.decode(q * 4, kc, vc, bt, L)
    for i in range(3):
        rows = np.concatenate([vc[pb] for pb in bt[i] if pb >= 0])[: L[i]]
        for h in range(4):
            assert np.all(out[i, h] <= rows[:, h].max(axis=0) + 1e-12)
            assert np.all(out[i, h] >= rows[:, h].min(axis=0) - 1e-12)


def test_zero_length_outputs_zeros():
    rng = np.random.default_rng(6)
    q, kc, vc, bt, L, kn, vn = _tiny_decode_case(rng, "fp32")
    out = oracle.decode(q, kc, vc, bt, np.array([0, 32, 0], np.int32))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)


# -------------------------------------------- paged equals contiguous

def _paged_from_contiguous(kv, bs, placement, NB):
    """Scatter a contiguous [n, Hkv, D] sequence into pool blocks."""
    pool = np.zeros((NB, bs) + kv.shape[1:], kv.dtype)
    for t in range(kv.shape[0]):
        pool[placement[t // bs], t % bs] = kv[t]
    return pool


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_paged_equals_contiguous_bitwise(dtype, golden):
    """The 60-token request on blocks 7, 1, 12, 4 and on random placements
    gives the same fp64 bits as the identity placement: only the addresses
    change, never the arithmetic."""
    g = golden("notes_60_token_example.json")
    rng = np.random.default_rng(7)
    n, bs, Hq, Hkv, D = g["length"], g["block_size"], 4, 2, 32
    mk = (lambda s: rng.standard_normal(s).astype(np.float32)) if dtype == "fp32" else \
        (lambda s: _bf16_bits(rng.standard_normal(s).astype(np.float32)))
    k, v, q = mk((n, Hkv, D)), mk((n, Hkv, D)), mk((1, 1, Hq, D))
    nblk = 4
    ident = [0, 1, 2, 3]
    base = oracle.decode(q, _paged_from_contiguous(k, bs, ident, 16),
                         _paged_from_contiguous(v, bs, ident, 16),
                         np.array([ident], np.int32), np.array([n], np.int32))
    for placement in [g["block_table"]] + [list(rng.permutation(16)[:nblk]) for _ in range(5)]:
        out = oracle.decode(q, _paged_from_contiguous(k, bs, placement, 16),
                            _paged_from_contiguous(v, bs, placement, 16),
                            np.array([placement], np.int32), np.array([n], np.int32))
        assert np.array_equal(out, base)
    # and it is the textbook dense softmax(q K^T / sqrt(D)) V
    wid = (lambda a: a.astype(np.float64)) if dtype == "fp32" else \
        (lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    K, V, Q = wid(k), wid(v), wid(q)
    for h in range(Hq):
        s = K[:, h // 2] @ Q[0, 0, h] / math.sqrt(D)
        w = np.exp(s - s.max())
        dense = (w / w.sum()) @ V[:, h // 2]
        np.testing.assert_allclose(base[0, h], dense, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- merges

def test_merge_law_matches_unsplit():
    rng = np.random.default_rng(8)
    for trial in range(20):
        n = int(rng.integers(1, 200))
        s = rng.standard_normal(n) * 3
        v = rng.standard_normal((n, 5))
        whole = oracle.finalize(oracle.partial(s, v))
        cuts = sorted(set(rng.integers(0, n + 1, size=int(rng.integers(1, 6))).tolist()) | {0, n})
        acc = oracle.partial([], np.zeros((0, 5)))
        for a, b in zip(cuts[:-1], cuts[1:]):
            acc = oracle.merge2(acc, oracle.partial(s[a:b], v[a:b]))
        np.testing.assert_allclose(oracle.finalize(acc), whole, rtol=1e-13, atol=1e-14)
        # and the textbook softmax
        w = np.exp(s - s.max())
        np.testing.assert_allclose(whole, (w / w.sum()) @ v, rtol=1e-13, atol=1e-14)


def test_merge_identity():
    ident = oracle.partial([], np.zeros((0, 3)))
    assert ident[0] == -math.inf and ident[1] == 0.0 and np.all(ident[2] == 0)
    m, l, a = oracle.merge2(ident, ident)
    assert m == -math.inf and l == 0.0 and np.all(a == 0)
    p = oracle.partial([0.5, -1.0], np.array([[1.0, 2, 3], [4, 5, 6]]))
    for left, right in ((ident, p), (p, ident)):
        m, l, a = oracle.merge2(left, right)
        assert m == p[0] and l == p[1] and np.array_equal(a, p[2])
    assert np.all(oracle.finalize(ident) == 0)


def test_merge_formula_two_parts_by_hand():
    """m = max(m1, m2), l = l1 e^(m1 - m) + l2 e^(m2 - m) with numbers."""
    m, l, a = oracle.merge2((1.0, 2.0, [2.0]), (3.0, 0.5, [1.0]))
    assert m == 3.0
    assert l == pytest.approx(2.0 * math.exp(-2.0) + 0.5, rel=1e-15)
    assert a[0] == pytest.approx(2.0 * math.exp(-2.0) + 1.0, rel=1e-15)


# ------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
def test_decode_matches_decimal_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    dtype = "fp32" if seed % 2 == 0 else "bf16"
    Hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 3))
    Hq, D, bs = Hkv * G, int(rng.integers(1, 5)), int(rng.integers(2, 5))
    B = int(rng.integers(1, 4))
    append = bool(seed % 3 != 2)
    L = rng.integers(0, 9, size=B)
    nb = [-(-(int(x) + append) // bs) for x in L]
    NB = sum(nb) + 2
    perm = rng.permutation(NB)
    mb = max(max(nb), 1)
    bt = np.full((B, mb), -1, np.int32)
    pos = 0
    for i in range(B):
        bt[i, :nb[i]] = perm[pos:pos + nb[i]]
        pos += nb[i]
    mk = (lambda s: rng.standard_normal(s).astype(np.float32)) if dtype == "fp32" else \
        (lambda s: _bf16_bits(rng.standard_normal(s).astype(np.float32)))
    q, kc, vc = mk((B, 1, Hq, D)), mk((NB, bs, Hkv, D)), mk((NB, bs, Hkv, D))
    kn, vn = (mk((B, 1, Hkv, D)), mk((B, 1, Hkv, D))) if append else (None, None)
    want, kw, vw = bruteforce.decode(q, kc, vc, bt, L, kn, vn)
    kc2, vc2 = kc.copy(), vc.copy()
    got = oracle.decode(q, kc2, vc2, bt, L.astype(np.int32), kn, vn)
    assert np.array_equal(kc2, kw) and np.array_equal(vc2, vw)
    scale = np.maximum(np.abs(want).max(axis=-1, keepdims=True), 1e-300)
    assert np.all(np.abs(got - want) / scale <= 1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_varlen_matches_decimal_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    dtype = "fp32" if seed % 2 == 0 else "bf16"
    B = int(rng.integers(1, 4))
    lq = rng.integers(0, 4, size=B)
    lk = rng.integers(0, 5, size=B)
    Hkv, G, D = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 5))
    Hq = Hkv * G
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    mk = (lambda s: rng.standard_normal(s).astype(np.float32)) if dtype == "fp32" else \
        (lambda s: _bf16_bits(rng.standard_normal(s).astype(np.float32)))
    q, k, v = mk((int(cq[-1]), Hq, D)), mk((int(ck[-1]), Hkv, D)), mk((int(ck[-1]), Hkv, D))
    want = bruteforce.varlen(q, k, v, cq, ck)
    got = oracle.varlen(q, k, v, cq, ck, int(lq.max()), int(lk.max()))
    scale = np.maximum(np.abs(want).max(axis=-1, keepdims=True), 1e-300)
    assert np.all(np.abs(got - want) / scale <= 1e-13)


# ------------------------------------------------ the varlen worked example

def test_varlen_example_values(golden):
    """On the printed example: request 0 has no key, so its 10 rows are 0;
    request 1 has one key, so its 3 rows equal that key's value exactly;
    request 2's row is checked against the decimal brute force."""
    g = golden("hf_varlen_example.json")
    rng = np.random.default_rng(9)
    Hq, Hkv, D = 4, 2, 8
    q = rng.standard_normal((1, g["total_q"], Hq, D)).astype(np.float32)
    k = rng.standard_normal((1, g["total_k"], Hkv, D)).astype(np.float32)
    v = rng.standard_normal((1, g["total_k"], Hkv, D)).astype(np.float32)
    out = oracle.varlen(q, k, v, g["cu_seq_lens_q"], g["cu_seq_lens_k"], g["max_length_q"],
                        g["max_length_k"])
    assert np.all(out[:10] == 0)
    for r in range(10, 13):
        for h in range(Hq):
            assert np.array_equal(out[r, h], v[0, 0, h // 2].astype(np.float64))
    want = bruteforce.varlen(q[0], k[0], v[0], g["cu_seq_lens_q"], g["cu_seq_lens_k"])
    np.testing.assert_allclose(out[13], want[13], rtol=1e-13, atol=1e-15)


def test_varlen_errors(golden):
    g = golden("hf_varlen_example.json")
    q = np.zeros((1, 14, 2, 4), np.float32)
    k = np.zeros((1, 8, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.varlen(q, k, k, g["cu_seq_lens_q"], g["cu_seq_lens_k"], 9, 7)   # 10 > max 9
    assert e.value.code == 6
    with pytest.raises(oracle.OracleError) as e:
        oracle.varlen(q, k, k, [0, 10, 9, 14], g["cu_seq_lens_k"], 10, 7)
    assert e.value.code == 5


def test_varlen_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    cq = np.array([0, 5, 9], np.int32)
    ck = np.array([0, 3, 11], np.int32)
    q = rng.standard_normal((9, 2, 4)).astype(np.float32)
    k = rng.standard_normal((11, 1, 4)).astype(np.float32)
    v = rng.standard_normal((11, 1, 4)).astype(np.float32)
    full = oracle.varlen(q, k, v, cq, ck, 5, 8)
    sub = oracle.varlen(q, k, v, cq, ck, 5, 8, rows=[8, 0, 4])
    assert np.array_equal(sub, full[[8, 0, 4]])
