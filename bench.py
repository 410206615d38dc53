#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--placement permuted|contiguous]

A step is one pass of paged decode over the batch of the chosen workload
(default: the long-context batch -- 256 sequences, 64 q / 8 kv heads,
head_dim 128, 16-token blocks, log-uniform 1k..32k cached tokens, 512-token
split-context partitions): the plan kernel, the per-partition kernel
(block-table gather, QK^T, online softmax, P.V) and the (m, l) merge.  Inputs
are resident in HBM before timing starts.  W untimed steps, then exactly K
timed steps; before each timed step the 256 MB last-level cache is flushed
(a 1 GiB buffer is read, outside the timed interval), and each step is timed
by HIP events recorded on the launch stream around it.  `value` is KV
bytes read per second (algorithmic: every cached K and V element of each kv
head counted once) over the mean cold step time.

The same JSON line carries
  roofline        the per-partition kernel against the 8 TB/s HBM peak, its
                  duration taken from HIP events around each launch in the
                  timed region, and against the measured streaming-read
                  ceiling (`stream_peak`);
  stream_peak     pkv_stream_read over 8 GiB, with and without the
                  non-temporal hint: the practical HBM read ceiling;
  mfma_peak       pkv_mfma_peak, a register-only loop of the bf16 matrix-core
                  product the prefill tiles use: the practical MFMA ceiling
                  at the clock the part holds under that load;
  cpu_baseline    the fp64 oracle timed on the host on a bounded sample of the
                  same workload (about --cpu-seconds of work);
  warm            the same K steps back to back without flushing (wall clock);
  write_flush     the same K steps with the cache flushed by overwriting the
                  buffer instead of reading it (the step then also pays for
                  writing back the dirty lines that leaves);
  s1_placement    the paged batches with contiguous blocks vs randomly
                  permuted blocks (the pages' paged-vs-contiguous comparison);
  gqa4_decode     the 64-sequence GQA-4 batch, cold;
  prefill         the 16-sequence varlen prefill batch: algorithmic TFLOP/s
                  against the 2.5 PFLOP/s dense bf16 MFMA peak, cold, with
                  its own oracle baseline;
  paged_prefill   the same batch as a paged step: cache write of the new rows,
                  then varlen attention through the block table;
  mixed_step      the continuous-batching step: 512 decode sequences with the
                  in-place append, then 8 x 1024 prefill tokens, on one stream.
Only one GPU is supported: --gpus above 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-decode KV read GB/s (% of HBM peak) + queries/s; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30
FLUSH_WORKGROUPS = 2048
COLD = ("HIP events around each step on the launch stream; the last-level cache flushed "
        "(1 GiB read with the default cache policy) before each step, outside the timed "
        "interval")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kv_bytes(case):
    """Algorithmic KV bytes of one decode pass: sum_i L'_i * 2 * Hkv * D * elt."""
    _, _, Hkv, D = case.k_cache.shape
    elt = case.k_cache.element_size()
    return int(case.attended.sum()) * 2 * Hkv * D * elt


# the per-partition kernel each decode workload runs: the persistent kernel,
# or the direct grid for few units (up to two grid slots per resident wave)
DECODE_KERNEL = {"tiny_decode_fp32": "decode_direct_kernel"}


def varlen_flops(case):
    """Algorithmic flops: sum_b 4 * D * Hq * len_q * len_k (QK^T and P.V)."""
    _, _, Hq, D = case.q.shape
    return int(sum(4 * D * Hq * int(a) * int(b) for a, b in zip(case.q_lengths, case.k_lengths)))


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_296_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_file, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(kernel_file):
        return None
    return t.get("hbm_bytes_per_launch")


class Flusher:
    """Reads a buffer four times the size of the last-level cache with the
    default (allocating) cache policy, outside any timed interval, so that
    the next timed call finds none of its data cached.  A read and not a
    write: overwriting the buffer instead leaves the cache full of dirty
    lines, and the next call then pays for writing them back (measured:
    the 16-request cache write 31.0 -> 36.3 us, the long-context decode
    step 1462 -> 1500 us; with the read, the decode step equals steps run
    back to back, whose 9.4 GB cannot stay cached)."""

    def __init__(self, torch, dev):
        import paged_kv_cache_296_amd as pkv
        self.pkv = pkv
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.sink = torch.empty(FLUSH_WORKGROUPS * 4096, dtype=torch.uint8, device=dev)

    def __call__(self):
        self.pkv.stream_read(self.buf, self.sink, FLUSH_WORKGROUPS, False)


class OverwriteFlusher:
    """The other way to flush: overwrite the 1 GiB buffer.  Reported beside
    the headline only: it leaves the cache full of dirty lines that the
    timed call then writes back."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i & 0xFF)


def time_decode(pkv, torch, case, steps, warmup, flush=None):
    """Warmup, then `steps` timed decode steps, each one `decode` call (plan,
    per-partition kernel, merge) between two HIP events, as a caller runs it;
    then the same steps again as the two phase calls with an event between
    them, for the per-kernel split only (an event between the kernels costs
    a few microseconds of its own, so it stays out of the step time).  With
    `flush`, the cache is flushed before each step; without, the steps run
    back to back and the wall clock of the whole-call loop is taken too.
    Returns dict(step_ms, part_ms, merge_ms, wall_ms, out)."""
    out = torch.empty_like(case.q)
    B, _, Hq, D = case.q.shape
    NB, bs, Hkv, _ = case.k_cache.shape
    need = pkv.decode_workspace_bytes(B, Hq, Hkv, D, bs, case.block_table.shape[1],
                                      case.partition_tokens)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=case.q.device)
    kw = dict(softmax_scale=case.softmax_scale, partition_tokens=case.partition_tokens, out=out,
              workspace=ws)
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens,
            case.k_new, case.v_new)

    def whole():
        pkv.decode(*args, **kw)

    def split(ev):
        pkv.decode_partials(*args, **kw)
        ev.record()
        pkv.decode_merge(*args, **kw)

    def run(timed_step, nev):
        for _ in range(warmup):
            if flush is not None:
                flush()
            whole()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush is not None:
                flush()
            evs[i][0].record()
            timed_step(evs[i])
            evs[i][-1].record()
        torch.cuda.synchronize()
        return evs, (time.perf_counter() - t0) * 1e3 / steps

    evw, wall_ms = run(lambda ev: whole(), 2)
    evs, _ = run(lambda ev: split(ev[1]), 3)
    return {"step_ms": sum(e[0].elapsed_time(e[1]) for e in evw) / steps,
            "part_ms": sum(e[0].elapsed_time(e[1]) for e in evs) / steps,
            "merge_ms": sum(e[1].elapsed_time(e[2]) for e in evs) / steps,
            "wall_ms": None if flush is not None else wall_ms, "out": out}


def time_call(torch, fn, steps, warmup, flush=None):
    """Mean HIP-event time (ms) of fn() on the current stream, the cache
    flushed before every call when `flush` is given."""
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush()
        evs[i][0].record()
        fn()
        evs[i][1].record()
    torch.cuda.synchronize()
    return sum(e[0].elapsed_time(e[1]) for e in evs) / steps


def varlen_call(pkv, case, out):
    return lambda: pkv.varlen(case.q, case.k, case.v, case.cu_seq_lens_q, case.cu_seq_lens_k,
                              case.max_length_q, case.max_length_k,
                              softmax_scale=case.softmax_scale, out=out)


def stream_peak(pkv, torch, dev, steps=5):
    """pkv_stream_read over 8 GiB (32x the last-level cache; 1 MB per wave),
    with and without the non-temporal hint: GB/s of the mean call."""
    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wgs = 2048
    sink = torch.empty(wgs * 4096, dtype=torch.uint8, device=dev)
    res = {"bytes": nbytes, "workgroups": wgs}
    for name, nt in (("nontemporal", True), ("default", False)):
        ms = time_call(torch, lambda: pkv.stream_read(buf, sink, wgs, nt), steps, 2)
        res[f"{name}_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    res["frac_of_spec"] = round(res["nontemporal_gbs"] / HBM_PEAK_GBS, 4)
    del buf, sink
    torch.cuda.empty_cache()
    return res


def mfma_peak(pkv, torch, dev, steps=5):
    """pkv_mfma_peak: a register-only loop of the bf16 32x32x16 matrix-core
    product the prefill tiles use, 2 and 4 workgroups (2 and 4 waves per
    SIMD) per compute unit, about 2 ms per call: TFLOP/s of the mean call,
    the better of the two."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"instruction": "v_mfma_f32_32x32x16_bf16", "compute_units": cus}
    best = 0.0
    for per_cu in (2, 4):
        wgs = per_cu * cus
        iters = 32768 // per_cu
        sink = torch.empty(wgs * 1024, dtype=torch.uint8, device=dev)
        fl = [0]

        def run():
            fl[0] = pkv.mfma_peak(sink, wgs, iters)
        ms = time_call(torch, run, steps, 8)  # the clock ramps up over the first ~15 ms
        tf = fl[0] / (ms * 1e-3) / 1e12
        res[f"tflops_{per_cu}_per_cu"] = round(tf, 1)
        best = max(best, tf)
    res["tflops"] = round(best, 1)
    res["frac_of_spec"] = round(best / MFMA_BF16_PEAK_TFLOPS, 4)
    return res


def cpu_baseline(torch, case, seconds):
    """The fp64 oracle on the host over a bounded, seeded sample of the
    workload's sequences (all heads), until about `seconds` of work."""
    import numpy as np

    import oracle
    import workloads

    rng = np.random.default_rng(12345)
    order = rng.permutation(len(case.lengths))
    bt_all = case.block_table.cpu().numpy()
    _, bs, Hkv, D = case.k_cache.shape
    elt = case.k_cache.element_size()
    spent, done_bytes, seqs, tokens = 0.0, 0, 0, 0
    for i in order:
        i = int(i)
        n = int(case.lengths[i]) + (1 if case.k_new is not None else 0)
        nb = -(-n // bs)
        blocks = bt_all[i, :nb]
        idx = torch.from_numpy(blocks.astype(np.int64)).to(case.k_cache.device)
        kc = workloads.to_host_bits(case.k_cache.index_select(0, idx)).copy()
        vc = workloads.to_host_bits(case.v_cache.index_select(0, idx)).copy()
        bt = np.arange(nb, dtype=np.int32)[None]
        q = workloads.to_host_bits(case.q[i:i + 1])
        kn = workloads.to_host_bits(case.k_new[i:i + 1]) if case.k_new is not None else None
        vn = workloads.to_host_bits(case.v_new[i:i + 1]) if case.v_new is not None else None
        sl = np.array([case.lengths[i]], dtype=np.int32)
        t0 = time.perf_counter()
        oracle.decode(q, kc, vc, bt, sl, kn, vn, scale=case.softmax_scale)
        spent += time.perf_counter() - t0
        done_bytes += n * 2 * Hkv * D * elt
        seqs += 1
        tokens += n
        if spent >= seconds:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"{seqs} seeded-random sequences ({tokens} cached tokens, all "
                      f"{case.q.shape[2]} q heads) of the same workload, fp64 C oracle, "
                      "OpenMP over (sequence, head)"}


def cpu_baseline_varlen(case, seconds):
    """The fp64 varlen oracle on the host over seeded batches of 16 random
    query rows (all heads) of the prefill batch, until about `seconds`."""
    import numpy as np

    import oracle
    import workloads

    h = workloads.to_host_bits
    q, k, v = h(case.q), h(case.k), h(case.v)
    cq, ck = case.cu_seq_lens_q.cpu().numpy(), case.cu_seq_lens_k.cpu().numpy()
    row_req = np.searchsorted(cq, np.arange(q.shape[1]), side="right") - 1
    _, _, Hq, D = case.q.shape
    rng = np.random.default_rng(54321)
    spent, flops, nrows = 0.0, 0, 0
    while spent < seconds:
        rows = np.sort(rng.choice(q.shape[1], 16, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.varlen(q, k, v, cq, ck, case.max_length_q, case.max_length_k,
                      scale=case.softmax_scale, rows=rows)
        spent += time.perf_counter() - t0
        lk = (ck[row_req[rows] + 1] - ck[row_req[rows]]).astype(np.int64)
        flops += int((4 * D * Hq * lk).sum())
        nrows += len(rows)
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"{nrows} seeded-random query rows (all {Hq} q heads, each against all its "
                      "request's keys) of the same batch, fp64 C oracle, OpenMP over (row, head)"}


def decode_result(args_workload, case, t, K, W, pkv, torch):
    B, _, Hq, D = case.q.shape
    NB, bs, Hkv, _ = case.k_cache.shape
    kvb = kv_bytes(case)
    gbs = kvb / (t["step_ms"] * 1e-3) / 1e9
    ach = kvb / (t["part_ms"] * 1e-3) / 1e9
    eff_pt = pkv.decode_partition_tokens(B, Hq, Hkv, D, bs, case.block_table.shape[1],
                                         case.partition_tokens)
    dt = {torch.bfloat16: "bf16", torch.float32: "f32"}[case.q.dtype]
    return {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(t["step_ms"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": args_workload, "batch": B, "num_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": bs, "partition_tokens": eff_pt,
                   "append": case.k_new is not None, "placement": getattr(case, "placement", None),
                   "cached_tokens": int(case.lengths.sum()), "kv_bytes_per_step": kvb},
        "timing": COLD,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "queries_per_s": round(B / (t["step_ms"] * 1e-3), 1),
        "kernels_ms": {"plan_and_partial": round(t["part_ms"], 4),
                       "merge": round(t["merge_ms"], 4)},
        "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL.get(args_workload, "decode_partial_kernel"),
                     "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("decode.hip", args_workload)},
    }


def s1_leg(pkv, torch, workloads, name, base_case, steps, warmup, flush, dev):
    """The same decode batch with its blocks handed out in order (contiguous)
    against the randomly permuted placement; ratio > 1 means the permuted
    (paged) placement is slower."""
    contig = workloads.make_config(name, device=dev, placement="contiguous")
    tc = time_decode(pkv, torch, contig, steps, warmup, flush)
    del contig
    torch.cuda.empty_cache()
    tp = time_decode(pkv, torch, base_case, steps, warmup, flush)
    return {"permuted_ms": round(tp["step_ms"], 4), "contiguous_ms": round(tc["step_ms"], 4),
            "ratio_permuted_over_contiguous": round(tp["step_ms"] / tc["step_ms"], 4)}


def make_prefill_case(workloads, name, dev):
    """varlen_prefill: the 16-request batch; varlen_uniform: 16 requests of
    2048 query rows and 4096 keys each (the kernel's steady state, for
    counters)."""
    if name == "varlen_uniform":
        return workloads.make_varlen(seed=1, dtype="bf16", batch=16, num_heads=32, num_kv_heads=8,
                                     head_dim=128, q_lengths=("fixed", 2048),
                                     k_lengths=("fixed", 4096), device=dev)
    return workloads.make_config(name, device=dev)


def prefill_leg(pkv, torch, workloads, steps, warmup, flush, dev, cpu_seconds,
                name="varlen_prefill"):
    case = make_prefill_case(workloads, name, dev)
    out = torch.empty_like(case.q)
    fl = varlen_flops(case)
    ms = time_call(torch, varlen_call(pkv, case, out), steps, max(warmup, 10), flush)
    res = {"workload": name, "flops_per_step": fl, "ms_per_step": round(ms, 4),
           "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
           "frac_of_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "timing": COLD}
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_varlen(case, cpu_seconds)
    return res


def paged_prefill_leg(pkv, torch, workloads, steps, warmup, flush, dev):
    """The prefill batch as a paged step: the new rows are written into their
    cache slots (pkv_cache_write), then the queries attend prefix + new keys
    straight from the paged pool (pkv_varlen_paged)."""
    c = dict(workloads.CONFIGS["varlen_prefill"])
    c.pop("kind")
    pc = workloads.make_paged_prefill(device=dev, **c)
    total, Hkv, D = pc.k_new.shape[1:]
    row_bytes = Hkv * D * pc.k_new.element_size()
    write_bytes = 4 * total * row_bytes         # K and V rows, read once and written once
    fl = int(sum(4 * D * pc.q.shape[2] * int(a) * int(b)
                 for a, b in zip(pc.q_lengths, pc.q_lengths + pc.prefix)))
    out = torch.empty_like(pc.q)

    def write():
        pkv.cache_write(pc.k_new, pc.v_new, pc.cu_seq_lens_q, pc.start, pc.k_cache, pc.v_cache,
                        pc.block_table)

    def attend():
        pkv.varlen_paged(pc.q, pc.k_cache, pc.v_cache, pc.block_table, pc.cu_seq_lens_q,
                         pc.seqlens_k, pc.max_length_q, pc.max_length_k,
                         softmax_scale=pc.softmax_scale, out=out)

    # references: a plain device copy of the same rows (torch), and the
    # library's plain copy kernel over the same byte count (pkv_stream_copy,
    # one buffer holding K and V), same flush
    kd, vd = torch.empty_like(pc.k_new), torch.empty_like(pc.v_new)
    ck = time_call(torch, lambda: (kd.copy_(pc.k_new), vd.copy_(pc.v_new)), steps, warmup, flush)
    del kd, vd
    src = torch.empty(write_bytes // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sc = time_call(torch, lambda: pkv.stream_copy(src, dst), steps, warmup, flush)
    del src, dst
    wk = time_call(torch, write, steps, warmup, flush)
    ak = time_call(torch, attend, steps, max(warmup, 10), flush)
    sk = time_call(torch, lambda: (write(), attend()), steps, warmup, flush)
    return {"workload": "paged_prefill (varlen_prefill lengths, 16-token blocks, permuted pool)",
            "cache_write_ms": round(wk, 4), "cache_write_bytes": write_bytes,
            "cache_write_gbs": round(write_bytes / (wk * 1e-3) / 1e9, 1),
            "cache_write_frac_of_hbm_peak": round(write_bytes / (wk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "same_bytes_torch_copy_ms": round(ck, 4),
            "same_bytes_torch_copy_gbs": round(write_bytes / (ck * 1e-3) / 1e9, 1),
            "same_bytes_stream_copy_ms": round(sc, 4),
            "same_bytes_stream_copy_gbs": round(write_bytes / (sc * 1e-3) / 1e9, 1),
            "cache_write_frac_of_stream_copy": round(sc / wk, 4),
            "varlen_paged_ms": round(ak, 4), "flops": fl,
            "varlen_paged_tflops": round(fl / (ak * 1e-3) / 1e12, 2),
            "varlen_paged_frac_of_mfma_peak": round(fl / (ak * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "step_ms": round(sk, 4), "timing": COLD}


def mixed_leg(pkv, torch, workloads, steps, warmup, flush, dev):
    """The continuous-batching step: decode (append + attend) then the
    prefill, back to back on one stream, cold."""
    dcase, vcase = workloads.make_config("mixed_step", device=dev)
    dk = kv_bytes(dcase)
    vf = varlen_flops(vcase)
    td = time_decode(pkv, torch, dcase, steps, warmup, flush)
    out_v = torch.empty_like(vcase.q)
    vk = time_call(torch, varlen_call(pkv, vcase, out_v), steps, max(warmup, 10), flush)
    out_d = torch.empty_like(dcase.q)

    def whole():
        pkv.decode(dcase.q, dcase.k_cache, dcase.v_cache, dcase.block_table, dcase.cache_seqlens,
                   dcase.k_new, dcase.v_new, softmax_scale=dcase.softmax_scale,
                   partition_tokens=dcase.partition_tokens, out=out_d)
        varlen_call(pkv, vcase, out_v)()

    step_ms = time_call(torch, whole, steps, warmup, flush)
    ideal_ms = dk / (HBM_PEAK_GBS * 1e9) * 1e3 + vf / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    return {"workload": "mixed_step", "ms_per_step": round(step_ms, 4),
            "decode_kv_bytes": dk, "decode_ms": round(td["step_ms"], 4),
            "decode_gbs": round(dk / (td["step_ms"] * 1e-3) / 1e9, 2),
            "decode_partial_frac_of_hbm_peak": round(dk / (td["part_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_queries_per_s": round(dcase.q.shape[0] / (td["step_ms"] * 1e-3), 1),
            "prefill_flops": vf, "prefill_ms": round(vk, 4),
            "prefill_tflops": round(vf / (vk * 1e-3) / 1e12, 2),
            "roofline_ms": round(ideal_ms, 4),
            "frac_of_summed_roofline": round(ideal_ms / step_ms, 4), "timing": COLD}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b256_long",
                    choices=["decode_b256_long", "decode_b64_gqa4", "tiny_decode_fp32", "mixed_step",
                             "varlen_prefill", "varlen_uniform", "paged_prefill", "copy_1gib",
                             "stream_read", "mfma_peak"])
    ap.add_argument("--placement", default="permuted", choices=["permuted", "contiguous"],
                    help="block placement of a decode workload (contiguous: same draws, blocks in order)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip every leg after the headline")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_296_amd as pkv
    import workloads

    dev = "cuda"
    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup

    if args.workload == "copy_1gib":
        # plain copy of a known size: the calibration for HBM byte counters
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(W + K):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"workload": "copy_1gib", "bytes_read_per_launch": 1 << 30,
                          "bytes_written_per_launch": 1 << 30}))
        return

    if args.workload == "stream_read":
        print(json.dumps({"workload": "stream_read", **stream_peak(pkv, torch, dev, K)}))
        return

    if args.workload == "mfma_peak":
        print(json.dumps({"workload": "mfma_peak", **mfma_peak(pkv, torch, dev, K)}))
        return

    flush = Flusher(torch, dev)

    if args.workload in ("varlen_prefill", "varlen_uniform"):
        r = prefill_leg(pkv, torch, workloads, K, W, flush, dev,
                        0 if args.no_cpu_baseline else min(args.cpu_seconds, 10.0), args.workload)
        mp = mfma_peak(pkv, torch, dev)
        print(json.dumps({
            "metric": METRIC, "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
            "warmup": max(W, 10), "ms_per_step": r["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": args.workload, "batch": 16, "num_heads": 32,
                       "num_kv_heads": 8, "head_dim": 128, "flops_per_step": r["flops_per_step"]},
            "timing": COLD,
            "roofline": {"bound": "mfma", "kernel": "varlen_persistent_kernel",
                         "achieved": r["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": r["frac_of_mfma_peak"], "traffic": None,
                         "frac_of_measured_mfma": round(r["tflops"] / mp["tflops"], 4)},
            "mfma_peak": mp,
            "cpu_baseline": r.get("cpu_baseline")}))
        return

    if args.workload == "paged_prefill":
        print(json.dumps(paged_prefill_leg(pkv, torch, workloads, K, W, flush, dev)))
        return

    log("generating", args.workload, args.placement)
    if args.workload == "mixed_step":
        case = workloads.make_config("mixed_step", device=dev, part="decode",
                                     placement=args.placement)
    else:
        case = workloads.make_config(args.workload, device=dev, placement=args.placement)
    case.placement = args.placement
    torch.cuda.synchronize()
    log(f"timing {K} cold steps after {W} warmup; KV bytes/step {kv_bytes(case) / 1e9:.3f} GB")
    t = time_decode(pkv, torch, case, K, W, flush)
    res = decode_result(args.workload, case, t, K, W, pkv, torch)
    log(f"decode {res['value']:.1f} GB/s cold, partial kernel {res['roofline']['achieved']:.1f} GB/s "
        f"({t['part_ms']:.3f} ms)")
    warm = time_decode(pkv, torch, case, K, W, None)
    kvb = kv_bytes(case)
    res["warm"] = {"ms_per_step": round(warm["wall_ms"], 4),
                   "gbs": round(kvb / (warm["wall_ms"] * 1e-3) / 1e9, 2),
                   "partial_kernel_ms": round(warm["part_ms"], 4),
                   "timing": "the same steps back to back, wall clock, no flush"}

    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        res["cpu_baseline"] = cpu_baseline(torch, case, args.cpu_seconds)
        log("cpu baseline", res["cpu_baseline"]["value"], "GB/s on", res["cpu_baseline"]["cores"], "threads")
    else:
        res["cpu_baseline"] = None

    if not args.no_extra:
        log("the same steps with the cache flushed by overwriting 1 GiB")
        ow = OverwriteFlusher(torch, dev)
        tw = time_decode(pkv, torch, case, K, W, ow)
        res["write_flush"] = {"ms_per_step": round(tw["step_ms"], 4),
                              "gbs": round(kvb / (tw["step_ms"] * 1e-3) / 1e9, 2),
                              "partial_kernel_ms": round(tw["part_ms"], 4),
                              "timing": "as the headline, but the cache flushed by overwriting "
                                        "the 1 GiB buffer: the step also writes back the dirty "
                                        "lines that leaves"}
        del ow
        torch.cuda.empty_cache()

    if not args.no_extra and args.workload == "decode_b256_long" and args.placement == "permuted":
        n, w = max(K // 2, 5), max(W // 2, 2)
        log("stream-read ceiling")
        res["stream_peak"] = stream_peak(pkv, torch, dev)
        res["roofline"]["frac_of_measured_stream"] = round(
            res["roofline"]["achieved"] / res["stream_peak"]["nontemporal_gbs"], 4)
        log("stream", res["stream_peak"])
        log("S1 placement: long-context batch")
        s1 = {"decode_b256_long": s1_leg(pkv, torch, workloads, "decode_b256_long", case, n, w,
                                         flush, dev)}
        del case
        torch.cuda.empty_cache()
        log("GQA-4 batch")
        g4 = workloads.make_config("decode_b64_gqa4", device=dev)
        tg = time_decode(pkv, torch, g4, K, W, flush)
        g4b = kv_bytes(g4)
        res["gqa4_decode"] = {"workload": "decode_b64_gqa4", "ms_per_step": round(tg["step_ms"], 4),
                              "gbs": round(g4b / (tg["step_ms"] * 1e-3) / 1e9, 2),
                              "hbm_frac": round(g4b / (tg["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "kernel": DECODE_KERNEL.get("decode_b64_gqa4", "decode_partial_kernel"),
                              "kernel_ms": round(tg["part_ms"], 4),
                              "kernel_frac_of_hbm_peak": round(g4b / (tg["part_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "timing": COLD}
        log("gqa4", res["gqa4_decode"])
        s1["decode_b64_gqa4"] = s1_leg(pkv, torch, workloads, "decode_b64_gqa4", g4, n, w, flush, dev)
        del g4
        torch.cuda.empty_cache()
        s1["context"] = ("the pages quote a paged kernel ~20-26% slower than a contiguous one "
                         "(attributed to the original paper, hardware not stated)")
        res["s1_placement"] = s1
        log("s1", s1)
        log("MFMA-loop ceiling")
        res["mfma_peak"] = mfma_peak(pkv, torch, dev)
        log("mfma", res["mfma_peak"])
        log("prefill leg: varlen_prefill")
        res["prefill"] = prefill_leg(pkv, torch, workloads, n, w, flush, dev,
                                     0 if args.no_cpu_baseline else 5.0)
        res["prefill"]["frac_of_measured_mfma"] = round(
            res["prefill"]["tflops"] / res["mfma_peak"]["tflops"], 4)
        log("prefill", res["prefill"])
        torch.cuda.empty_cache()
        log("paged prefill leg")
        res["paged_prefill"] = paged_prefill_leg(pkv, torch, workloads, n, w, flush, dev)
        res["paged_prefill"]["varlen_paged_frac_of_measured_mfma"] = round(
            res["paged_prefill"]["varlen_paged_tflops"] / res["mfma_peak"]["tflops"], 4)
        log("paged prefill", res["paged_prefill"])
        torch.cuda.empty_cache()
        log("mixed step leg: mixed_step")
        res["mixed_step"] = mixed_leg(pkv, torch, workloads, n, w, flush, dev)
        log("mixed", res["mixed_step"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
