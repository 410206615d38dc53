"""GPU parity of pkv_decode against the fp64 oracle, on the same seeded bytes.

Covers the pages' tiny example (fp32, append into the printed table), the
GQA-4 decode batch, the long-context GQA-8 batch and the mixed step's decode
half at their full sizes (every sequence against the oracle), and small cases spanning several tiles,
ragged tails, block sizes 16/32, head_dim 64/128, group sizes 1..32,
partition choices, lengths 0/1 and block boundaries.  Also bit-exact checks:
the append writes exactly the new rows, outputs do not depend on where the
blocks are, repeated calls agree, junk in unowned slots changes nothing, and
bad table entries raise the error flag without faults.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_296_amd as pkv
import workloads
from tests.parity import assert_close, gpu_to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return workloads.to_host_bits(t)


def run_case(case, dtype, seqs=None, check_pool=True, partition_tokens=None):
    """Run GPU decode on `case` and the oracle on a host copy; compare."""
    pt = case.partition_tokens if partition_tokens is None else partition_tokens
    kc0, vc0 = _bits(case.k_cache), _bits(case.v_cache)
    q = _bits(case.q)
    bt = case.block_table.cpu().numpy()
    sl = case.cache_seqlens.cpu().numpy()
    kn = _bits(case.k_new) if case.k_new is not None else None
    vn = _bits(case.v_new) if case.v_new is not None else None
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens,
                     case.k_new, case.v_new, softmax_scale=case.softmax_scale,
                     partition_tokens=pt, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the oracle appends into its own copy; without new rows it writes nothing
    kref, vref = (kc0.copy(), vc0.copy()) if kn is not None else (kc0, vc0)
    ref = oracle.decode(q, kref, vref, bt, sl, kn, vn, scale=case.softmax_scale, seqs=seqs)
    got = gpu_to_f64(out)[:, 0]
    if seqs is not None:
        got = got[seqs]
    rep = assert_close(got, ref, dtype, f"decode seed {case.seed}")
    if check_pool:
        assert np.array_equal(_bits(case.k_cache), kref), "K pool differs from the oracle's append"
        assert np.array_equal(_bits(case.v_cache), vref), "V pool differs from the oracle's append"
    return out, rep


def test_tiny_example_fp32():
    case = workloads.make_config("tiny_decode_fp32", device=DEV)
    kc0 = _bits(case.k_cache)
    out, rep = run_case(case, "fp32")
    # the three new rows land at (block, offset) (2, 30), (1, 0), (6, 6)
    kc1 = _bits(case.k_cache)
    changed = {tuple(x[:2]) for x in np.argwhere(kc1 != kc0)}
    assert changed == {(2, 30), (1, 0), (6, 6)}
    kn = _bits(case.k_new)
    assert np.array_equal(kc1[2, 30], kn[0, 0]) and np.array_equal(kc1[1, 0], kn[1, 0])
    assert np.array_equal(kc1[6, 6], kn[2, 0])


def test_decode_b64_gqa4_full():
    case = workloads.make_config("decode_b64_gqa4", device=DEV)
    run_case(case, "bf16", check_pool=False)


def test_decode_b256_long_full():
    """The long-context batch at full size (256 sequences, 1k..32k cached
    tokens, GQA 8, the persistent kernel with runs of 512-token partitions
    and the merge): every sequence and head against the oracle, and the
    pools unchanged (no append)."""
    case = workloads.make_config("decode_b256_long", device=DEV)
    _, rep = run_case(case, "bf16", check_pool=True)
    assert rep["rows"] == 256 * 64
    del case
    torch.cuda.empty_cache()


def test_mixed_step_decode_full():
    """The decode half of the mixed continuous-batching step at full size and
    in the launch the bench times (512 sequences, 16..8192 cached tokens, the
    new token appended in place with a fresh block from the free list at block
    boundaries, persistent kernel with runs): both pools bit for bit against
    the oracle's append (every appended row, nothing else touched), and every
    sequence's output against the oracle."""
    case = workloads.make_config("mixed_step", device=DEV, part="decode")
    assert (case.lengths % 16 == 0).any()
    _, rep = run_case(case, "bf16", check_pool=True)
    assert rep["rows"] == 512 * 32
    del case
    torch.cuda.empty_cache()


SMALL = []
for dtype in ("bf16", "fp32"):
    for D in (64, 128):
        for bs in (16, 32):
            SMALL.append(dict(dtype=dtype, head_dim=D, block_size=bs, num_heads=8, num_kv_heads=2))
SMALL_IDS = [f"{c['dtype']}-d{c['head_dim']}-bs{c['block_size']}" for c in SMALL]


@pytest.mark.parametrize("cfg", SMALL, ids=SMALL_IDS)
@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("pt", [0, 32, 64])
def test_small_grid(cfg, append, pt):
    # lengths hit 0, 1, block edges and several tiles; partitions of 2..4 blocks
    lengths = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200]
    seed = 1000 + SMALL.index(cfg) * 10 + int(append) * 3 + pt
    case = workloads.make_decode(seed=seed, batch=len(lengths), lengths=lengths,
                                 num_blocks=300, append=append, partition_tokens=pt,
                                 device=DEV, **cfg)
    run_case(case, cfg["dtype"])


@pytest.mark.parametrize("group", [1, 3, 4, 8, 16, 20, 32])
def test_group_sizes(group):
    case = workloads.make_decode(seed=2000 + group, dtype="bf16", batch=5,
                                 num_heads=2 * group, num_kv_heads=2, head_dim=128,
                                 block_size=16, lengths=("uniform", 1, 700), num_blocks=400,
                                 append=True, partition_tokens=0, device=DEV)
    run_case(case, "bf16")


@pytest.mark.parametrize("pt", [16, 48, 512, 4096])
def test_partition_sizes_long(pt):
    case = workloads.make_decode(seed=3000 + pt, dtype="bf16", batch=6, num_heads=16,
                                 num_kv_heads=2, head_dim=128, block_size=16,
                                 lengths=[1, 511, 512, 513, 3000, 4000], num_blocks=1200,
                                 max_blocks_per_seq=256, append=True, partition_tokens=pt,
                                 device=DEV)
    run_case(case, "bf16")


def test_append_crosses_block_with_free_list():
    """Mixed-step style: sequences whose new token starts a block get a
    block popped from the free list; the new rows land exactly there."""
    case = workloads.make_decode(seed=4000, dtype="bf16", batch=64, num_heads=32,
                                 num_kv_heads=8, head_dim=128, block_size=16,
                                 lengths=("uniform", 16, 400), num_blocks="total+5%",
                                 max_blocks_per_seq=30, append=True, partition_tokens=512,
                                 free_list_boundary_alloc=True, device=DEV)
    assert (case.lengths % 16 == 0).any()
    run_case(case, "bf16")


def test_placement_invariance_bitwise():
    """Same logical blocks, three different physical placements: bit-identical."""
    base = workloads.make_decode(seed=5000, dtype="bf16", batch=8, num_heads=16, num_kv_heads=4,
                                 head_dim=128, block_size=16, lengths=("uniform", 100, 900),
                                 num_blocks=600, append=False, partition_tokens=128, device=DEV)
    ref = pkv.decode(base.q, base.k_cache, base.v_cache, base.block_table, base.cache_seqlens,
                     partition_tokens=128)
    rng = np.random.default_rng(5)
    bt = base.block_table.cpu().numpy()
    for _ in range(3):
        perm = rng.permutation(600).astype(np.int32)      # physical block p -> perm[p]
        kc = torch.empty_like(base.k_cache)
        vc = torch.empty_like(base.v_cache)
        idx = torch.from_numpy(perm.astype(np.int64)).to(DEV)
        kc[idx] = base.k_cache
        vc[idx] = base.v_cache
        bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
        out = pkv.decode(base.q, kc, vc, torch.from_numpy(bt2).to(DEV), base.cache_seqlens,
                         partition_tokens=128)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # and repeated calls agree bitwise
    again = pkv.decode(base.q, base.k_cache, base.v_cache, base.block_table, base.cache_seqlens,
                       partition_tokens=128)
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))


def test_junk_outside_owned_slots_changes_nothing():
    case = workloads.make_decode(seed=6000, dtype="bf16", batch=10, num_heads=8, num_kv_heads=2,
                                 head_dim=128, block_size=16, lengths=("uniform", 1, 300),
                                 num_blocks=250, append=False, partition_tokens=64, device=DEV)
    ref = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens,
                     partition_tokens=64)
    bt = case.block_table.cpu().numpy()
    L = case.lengths
    owned = set(int(b) for b in bt.reshape(-1) if b >= 0)
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    nan = torch.tensor(float("nan"), dtype=kc.dtype, device=DEV)
    for p in range(250):
        if p not in owned:
            kc[p] = nan
            vc[p] = nan
    for i in range(len(L)):  # slots past each sequence's end in its last block
        last = (int(L[i]) - 1) // 16
        if L[i] % 16:
            kc[bt[i, last], L[i] % 16:] = nan
            vc[bt[i, last], L[i] % 16:] = nan
    out = pkv.decode(case.q, kc, vc, case.block_table, case.cache_seqlens, partition_tokens=64)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("pt", [0, 32])
def test_bad_table_entry_flags_and_nans(pt):
    case = workloads.make_decode(seed=7000, dtype="bf16", batch=4, num_heads=8, num_kv_heads=2,
                                 head_dim=128, block_size=16, lengths=[40, 70, 20, 90],
                                 num_blocks=40, append=True, partition_tokens=pt, device=DEV)
    bt = case.block_table.clone()
    bt[1, 2] = -1          # needed by sequence 1 (70 + 1 tokens -> 5 blocks)
    bt[3, 0] = 40          # outside the 40-block pool
    k_before = case.k_cache.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pkv.decode(case.q, case.k_cache, case.v_cache, bt, case.cache_seqlens, case.k_new,
                     case.v_new, partition_tokens=pt, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & pkv.ERR_BLOCK
    o = out.float().cpu()
    assert torch.isnan(o[1]).all() and torch.isnan(o[3]).all()
    assert torch.isfinite(o[0]).all() and torch.isfinite(o[2]).all()
    # the healthy sequences still match the oracle
    q = _bits(case.q)
    kref, vref = _bits(k_before), _bits(case.v_cache)
    good = case.block_table.cpu().numpy()
    ref = oracle.decode(q, kref, vref, good, case.cache_seqlens.cpu().numpy(), _bits(case.k_new),
                        _bits(case.v_new), seqs=[0, 2])
    assert_close(gpu_to_f64(out)[[0, 2], 0], ref, "bf16")


def test_length_beyond_table_flags():
    case = workloads.make_decode(seed=7100, dtype="bf16", batch=3, num_heads=8, num_kv_heads=2,
                                 head_dim=64, block_size=16, lengths=[10, 20, 30],
                                 num_blocks=20, max_blocks_per_seq=2, append=False, device=DEV)
    sl = torch.tensor([10, 33, -1], dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, sl, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & pkv.ERR_SPAN
    o = out.float().cpu()
    assert torch.isnan(o[1]).all() and torch.isnan(o[2]).all() and torch.isfinite(o[0]).all()


def test_scalar_head_example_on_gpu(golden):
    """The notes' scalar-head demo, embedded: head_dim 64 with the value in
    dimension 0 and zeros elsewhere (zero padding leaves the scores and the
    weights unchanged), keys 0, query e_0.  Five positions give 3 in any
    placement.  The kernel's blocks hold 16 positions, so the page's 4 -> 5
    block-crossing append is checked as the 16 -> 17 crossing, whose mean of
    1..17 is 9 by the same closed form (n + 1) / 2."""
    g = golden("scalar_head_example.json")
    bs = 16
    q = torch.zeros(1, 1, 1, 64, dtype=torch.float32, device=DEV)
    q[0, 0, 0, 0] = g["query"]
    kc = torch.zeros(6, bs, 1, 64, dtype=torch.float32, device=DEV)
    for placement in ([4, 1], [1, 4], [0, 5]):
        vc = torch.full((6, bs, 1, 64), float("nan"), dtype=torch.float32, device=DEV)
        vc[placement[0], :, :, :] = 0.0
        for t, v in enumerate(g["values"]):
            vc[placement[0], t, 0, 0] = v
        out = pkv.decode(q, kc, vc, torch.tensor([placement], dtype=torch.int32, device=DEV),
                         torch.tensor([len(g["values"])], dtype=torch.int32, device=DEV))
        assert abs(float(out[0, 0, 0, 0]) - g["output"]) <= 1e-6
        assert float(out[0, 0, 0, 1:].abs().max()) == 0.0
    for placement in ([4, 1], [2, 3]):
        vc = torch.zeros(6, bs, 1, 64, dtype=torch.float32, device=DEV)
        vc[placement[1]] = float("nan")          # the fresh block holds junk
        for t in range(16):
            vc[placement[0], t, 0, 0] = t + 1
        kn = torch.zeros(1, 1, 1, 64, dtype=torch.float32, device=DEV)
        vn = torch.zeros(1, 1, 1, 64, dtype=torch.float32, device=DEV)
        vn[0, 0, 0, 0] = 17.0
        out = pkv.decode(q, kc.clone(), vc, torch.tensor([placement], dtype=torch.int32, device=DEV),
                         torch.tensor([16], dtype=torch.int32, device=DEV), kn, vn)
        assert abs(float(out[0, 0, 0, 0]) - 9.0) <= 1e-6
        assert float(vc[placement[1], 0, 0, 0]) == 17.0


def test_empty_batch_and_zero_lengths():
    case = workloads.make_decode(seed=7200, dtype="bf16", batch=4, num_heads=8, num_kv_heads=8,
                                 head_dim=128, block_size=16, lengths=[0, 0, 0, 0],
                                 num_blocks=8, max_blocks_per_seq=4, append=False, device=DEV)
    out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens,
                     partition_tokens=16)
    assert torch.count_nonzero(out.float()) == 0
    q0 = case.q[:0]
    out0 = pkv.decode(q0, case.k_cache, case.v_cache, case.block_table[:0], case.cache_seqlens[:0])
    assert out0.shape[0] == 0


def test_two_phase_calls_equal_decode_bitwise():
    case = workloads.make_decode(seed=7300, dtype="bf16", batch=12, num_heads=32, num_kv_heads=8,
                                 head_dim=128, block_size=16, lengths=("uniform", 1, 2000),
                                 num_blocks=2000, append=True, partition_tokens=256, device=DEV)
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    ref = pkv.decode(case.q, kc, vc, case.block_table, case.cache_seqlens, case.k_new, case.v_new,
                     partition_tokens=256)
    out, ws = pkv.decode_partials(case.q, case.k_cache, case.v_cache, case.block_table,
                                  case.cache_seqlens, case.k_new, case.v_new, partition_tokens=256)
    out = pkv.decode_merge(case.q, case.k_cache, case.v_cache, case.block_table,
                           case.cache_seqlens, case.k_new, case.v_new, partition_tokens=256,
                           out=out, workspace=ws)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(kc.view(torch.int16), case.k_cache.view(torch.int16))


@pytest.mark.parametrize("pt", [16, 32])
def test_runs_of_partitions(pt):
    """Enough partitions that the work list streams several consecutive
    partitions per unit; tiny partitions put a boundary every tile or two,
    and lengths that are multiples of the partition make the new token open
    a partition of its own."""
    lengths = np.random.default_rng(pt).integers(1, 1500, size=64)
    lengths[:8] = [pt, 2 * pt, 3 * pt, 160, 320, 1024, 1008, 1]
    case = workloads.make_decode(seed=7400 + pt, dtype="bf16", batch=64, num_heads=16,
                                 num_kv_heads=8, head_dim=128, block_size=16,
                                 lengths=lengths.tolist(), num_blocks=8000, append=True,
                                 partition_tokens=pt, device=DEV)
    run_case(case, "bf16")


@pytest.mark.parametrize("D,bs", [(64, 16), (64, 32), (128, 32)])
def test_runs_of_partitions_other_shapes(D, bs):
    """The persistent kernel with runs of several partitions at the other
    head sizes and block sizes: bf16 K is loaded as whole head rows (8 rows
    of 128 B per load at head_dim 64, 4 of 256 B at 128) and re-laid into
    the operand layout in LDS, and a 32-token block holds two tiles."""
    lengths = np.random.default_rng(D + bs).integers(1, 1500, size=96)
    lengths[:6] = [32, 64, 96, 1024, 1023, 1]
    case = workloads.make_decode(seed=7500 + D + bs, dtype="bf16", batch=96, num_heads=16,
                                 num_kv_heads=8, head_dim=D, block_size=bs,
                                 lengths=lengths.tolist(), num_blocks=12000, append=True,
                                 partition_tokens=32, device=DEV)
    units = int(sum((int(L) + 1 + 31) // 32 for L in lengths)) * 8
    assert units > 2 * 3 * 1024  # beyond the direct grid's limit: the persistent kernel runs
    run_case(case, "bf16")


def test_work_list_past_the_cached_chunks():
    """4500 sequences: the plan kernel keeps the lengths of the first 4096
    (four chunks of 1024) in registers between its passes and reads the rest
    again; every sequence is compared with the oracle."""
    lengths = np.random.default_rng(4150).integers(0, 100, size=4500)
    lengths[[0, 4095, 4096, 4499]] = [0, 99, 1, 64]
    case = workloads.make_decode(seed=4150, dtype="bf16", batch=4500, num_heads=8,
                                 num_kv_heads=2, head_dim=128, block_size=16, lengths=lengths,
                                 num_blocks=40000, append=True, partition_tokens=16, device=DEV)
    run_case(case, "bf16")


@pytest.mark.parametrize("pt", [16, 48])
def test_large_batch_work_list(pt):
    """More than 1024 sequences through the persistent kernel: the work list
    is planned in chunks of 1024 sequences, runs of several partitions lead,
    and every sequence's last run is placed longest first across the whole
    batch.  Lengths include 0 (nothing cached, the new token only).  Repeated
    calls are bit-identical."""
    lengths = np.random.default_rng(4100 + pt).integers(0, 300, size=1500)
    lengths[:4] = [0, 1, pt, 299]
    case = workloads.make_decode(seed=4100 + pt, dtype="bf16", batch=1500, num_heads=8,
                                 num_kv_heads=2, head_dim=128, block_size=16, lengths=lengths,
                                 num_blocks=20000, append=True, partition_tokens=pt, device=DEV)
    out, _ = run_case(case, "bf16")
    # units within a length bucket are placed in arbitrary order and taken by
    # whichever wave is free, but each unit's arithmetic and the merge order
    # are fixed: repeated calls (the append rewrites the same rows) agree
    # bit for bit
    for _ in range(2):
        again = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table,
                           case.cache_seqlens, case.k_new, case.v_new,
                           softmax_scale=case.softmax_scale, partition_tokens=pt)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))
