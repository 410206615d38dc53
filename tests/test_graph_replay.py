"""The entry points captured in a HIP graph and replayed (GPU).

Every host-side choice the library makes (partition length, grid, direct or
persistent decode, workspace layout) depends on shapes only; the work list,
the run length and the ticket counter are set on the device by the plan
kernel, and no entry point records a memset or an allocation.  So a graph
captured once must give, on every replay, the bits an eager call gives on
the inputs the buffers hold at replay time.  Each graph is replayed several
times with eager work and synchronisations between the replays (the output
is poisoned before each replay), every replay is compared with the eager
call bit for bit, and then the inputs are changed in place (other lengths,
other queries, requests in another order) and the replay is compared with a
fresh eager call on them.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_296_amd as pkv
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 3


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


def _capture(fn):
    """fn() once eagerly on a side stream (one-time host lookups happen
    outside the capture), then captured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_matches(g, out, expect):
    for r in range(REPLAYS):
        out.fill_(float("nan"))          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, expect), f"replay {r}"


def _decode_case(batch, hi, seed, append):
    return workloads.make_decode(seed=seed, dtype="bf16", batch=batch, num_heads=32,
                                 num_kv_heads=8, head_dim=128, block_size=16,
                                 lengths=("uniform", 1, hi), num_blocks="total+5%",
                                 max_blocks_per_seq=(hi + 16) // 16 + 1, append=append,
                                 free_list_boundary_alloc=append, device=DEV)


def _decode_eager(case, noalloc=False):
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens,
            case.k_new, case.v_new)
    out = torch.empty_like(case.q)
    if noalloc:
        return pkv.decode_noalloc(*args, out=out, softmax_scale=case.softmax_scale)
    return pkv.decode(*args, softmax_scale=case.softmax_scale, out=out)


@pytest.mark.parametrize("batch,hi,noalloc", [
    (4, 300, False),      # few units: the direct grid
    (96, 3000, False),    # the persistent kernel with runs
    (96, 3000, True),     # the same through the library's static scratch
])
def test_decode_graph(batch, hi, noalloc):
    case = _decode_case(batch, hi, 7300 + batch, append=False)
    expect = _decode_eager(case, noalloc)
    B, _, Hq, D = case.q.shape
    NB, bs, Hkv, _ = case.k_cache.shape
    out = torch.empty_like(case.q)
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens)
    if noalloc:
        g = _capture(lambda: pkv.decode_noalloc(*args, out=out, softmax_scale=case.softmax_scale))
    else:
        ws = torch.empty(pkv.decode_workspace_bytes(B, Hq, Hkv, D, bs, case.block_table.shape[1]),
                         dtype=torch.uint8, device=DEV)
        g = _capture(lambda: pkv.decode(*args, softmax_scale=case.softmax_scale, out=out,
                                        workspace=ws))
    _replay_matches(g, out, expect)

    # new lengths (each at most the old one, so the table still covers them;
    # some zero) and new queries, written in place: the plan kernel in the
    # graph reads them
    rng = np.random.default_rng(batch)
    new_len = (case.lengths * rng.uniform(0, 1, batch)).astype(np.int32)
    new_len[0] = 0
    case.cache_seqlens.copy_(torch.from_numpy(new_len))
    case.q.copy_(torch.randn(case.q.shape, device=DEV).to(case.q.dtype))
    expect2 = _decode_eager(case, noalloc)
    assert not _same(expect2, expect)
    _replay_matches(g, out, expect2)


def test_decode_append_graph():
    # the append writes the same rows on every replay; pools and output must
    # equal one eager call's
    case = _decode_case(64, 2000, 7400, append=True)
    k0, v0 = case.k_cache.clone(), case.v_cache.clone()
    expect = _decode_eager(case)
    ke, ve = case.k_cache.clone(), case.v_cache.clone()
    case.k_cache.copy_(k0)
    case.v_cache.copy_(v0)
    out = torch.empty_like(case.q)
    g = _capture(lambda: pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table,
                                    case.cache_seqlens, case.k_new, case.v_new,
                                    softmax_scale=case.softmax_scale, out=out))
    _replay_matches(g, out, expect)
    assert _same(case.k_cache, ke) and _same(case.v_cache, ve)


def _reverse_cu(cu):
    lens = (cu[1:] - cu[:-1]).flip(0)
    return torch.cat([cu[:1], torch.cumsum(lens, 0).to(torch.int32)])


def test_varlen_graph():
    case = workloads.make_varlen(seed=7500, dtype="bf16", batch=12, num_heads=32, num_kv_heads=8,
                                 head_dim=128, q_lengths=("uniform", 1, 700),
                                 prefix=("uniform", 0, 900), device=DEV)
    call = lambda o: pkv.varlen(case.q, case.k, case.v, case.cu_seq_lens_q, case.cu_seq_lens_k,
                                case.max_length_q, case.max_length_k,
                                softmax_scale=case.softmax_scale, out=o)
    expect = call(torch.empty_like(case.q))
    out = torch.empty_like(case.q)
    g = _capture(lambda: call(out))
    _replay_matches(g, out, expect)
    # the requests in reverse order (same totals and maxima), in place: the
    # item list the kernel builds on the device follows them
    case.cu_seq_lens_q.copy_(_reverse_cu(case.cu_seq_lens_q))
    case.cu_seq_lens_k.copy_(_reverse_cu(case.cu_seq_lens_k))
    expect2 = call(torch.empty_like(case.q))
    assert not _same(expect2, expect)
    _replay_matches(g, out, expect2)


def test_paged_prefill_graph():
    pc = workloads.make_paged_prefill(seed=7600, dtype="bf16", batch=10, num_heads=32,
                                      num_kv_heads=8, head_dim=128,
                                      q_lengths=("uniform", 1, 600), prefix=("uniform", 0, 800),
                                      device=DEV)
    k0, v0 = pc.k_cache.clone(), pc.v_cache.clone()

    def step(o):
        pkv.cache_write(pc.k_new, pc.v_new, pc.cu_seq_lens_q, pc.start, pc.k_cache, pc.v_cache,
                        pc.block_table)
        pkv.varlen_paged(pc.q, pc.k_cache, pc.v_cache, pc.block_table, pc.cu_seq_lens_q,
                         pc.seqlens_k, pc.max_length_q, pc.max_length_k,
                         softmax_scale=pc.softmax_scale, out=o)
        return o

    expect = step(torch.empty_like(pc.q))
    ke, ve = pc.k_cache.clone(), pc.v_cache.clone()
    pc.k_cache.copy_(k0)
    pc.v_cache.copy_(v0)
    out = torch.empty_like(pc.q)
    g = _capture(lambda: step(out))
    _replay_matches(g, out, expect)
    assert _same(pc.k_cache, ke) and _same(pc.v_cache, ve)
