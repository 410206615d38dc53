#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of paged decode over the batch of the chosen workload
(default: the long-context batch -- 256 sequences, 64 q / 8 kv heads,
head_dim 128, 16-token blocks, log-uniform 1k..32k cached tokens, 512-token
split-context partitions): the per-partition kernel (block-table gather,
QK^T, online softmax, P.V) then the (m, l) merge.  Inputs are resident in HBM
before timing starts.  W untimed steps, then exactly K timed steps between two
device synchronisations; `value` is KV bytes read per second (algorithmic:
every cached K and V element of each kv head counted once).

The same JSON line carries
  roofline      the per-partition kernel against the 8 TB/s HBM peak, its
                duration taken from HIP events recorded on the launch stream
                around each launch in the timed region;
  cpu_baseline  the fp64 oracle timed on the host on a bounded sample of the
                same workload (about --cpu-seconds of work);
  prefill       the 16-sequence varlen prefill batch: algorithmic TFLOP/s
                against the 2.5 PFLOP/s dense bf16 MFMA peak;
  paged_prefill the same batch as a paged step: cache write of the new rows,
                then varlen attention through the block table;
  mixed_step    the continuous-batching step: 512 decode sequences with the
                in-place append, then 8 x 1024 prefill tokens, on one stream.
Only one GPU is supported: --gpus above 1 exits with a message.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-decode KV read GB/s (% of HBM peak) + queries/s; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kv_bytes(case):
    """Algorithmic KV bytes of one decode pass: sum_i L'_i * 2 * Hkv * D * elt."""
    _, _, Hkv, D = case.k_cache.shape
    elt = case.k_cache.element_size()
    return int(case.attended.sum()) * 2 * Hkv * D * elt


# the per-partition kernel each decode workload runs: the persistent kernel,
# or the direct grid for few units (up to two grid slots per resident wave)
DECODE_KERNEL = {"decode_b64_gqa4": "decode_direct_kernel", "tiny_decode_fp32": "decode_direct_kernel"}


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


def time_decode(pkv, torch, case, steps, warmup, with_events=True):
    """Runs warmup + timed decode steps; returns wall ms/step and the mean
    event-timed durations (ms) of the per-partition and merge kernels."""
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

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pkv.decode_partials(*args, **kw)
        if ev is not None:
            ev[1].record()
        pkv.decode_merge(*args, **kw)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i] if with_events else None)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    part = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    merge = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    return wall_ms, part, merge, out


def time_varlen(pkv, torch, case, steps, warmup):
    out = torch.empty_like(case.q)
    args = (case.q, case.k, case.v, case.cu_seq_lens_q, case.cu_seq_lens_k, case.max_length_q,
            case.max_length_k)
    for _ in range(warmup):
        pkv.varlen(*args, softmax_scale=case.softmax_scale, out=out)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record()
        pkv.varlen(*args, softmax_scale=case.softmax_scale, out=out)
        evs[i][1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kern = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    return wall_ms, kern


def time_call(torch, fn, steps, warmup, flush=None):
    """Mean HIP-event time (ms) of fn() on the current stream.  With `flush`
    (a byte tensor larger than the 256 MB last-level cache) it is
    overwritten before every timed call, outside the timed interval, so that
    fn() starts from a cold cache."""
    for _ in range(warmup):
        fn()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        evs[i][0].record()
        fn()
        evs[i][1].record()
    torch.cuda.synchronize()
    return sum(e[0].elapsed_time(e[1]) for e in evs) / steps


def paged_prefill_leg(pkv, torch, workloads, steps, warmup, dev):
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

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    # reference: a plain device copy of the same rows (torch), same flush
    kd, vd = torch.empty_like(pc.k_new), torch.empty_like(pc.v_new)
    ck = time_call(torch, lambda: (kd.copy_(pc.k_new), vd.copy_(pc.v_new)), steps, warmup, flush)
    del kd, vd
    wk = time_call(torch, write, steps, warmup, flush)
    ak = time_call(torch, attend, steps, warmup, flush)
    sk = time_call(torch, lambda: (write(), attend()), steps, warmup, flush)
    del flush
    return {"workload": "paged_prefill (varlen_prefill lengths, 16-token blocks, permuted pool)",
            "cache_write_ms": round(wk, 4), "cache_write_bytes": write_bytes,
            "cache_write_gbs": round(write_bytes / (wk * 1e-3) / 1e9, 1),
            "cache_write_frac_of_hbm_peak": round(write_bytes / (wk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "same_bytes_torch_copy_ms": round(ck, 4),
            "same_bytes_torch_copy_gbs": round(write_bytes / (ck * 1e-3) / 1e9, 1),
            "varlen_paged_ms": round(ak, 4), "flops": fl,
            "varlen_paged_tflops": round(fl / (ak * 1e-3) / 1e12, 2),
            "varlen_paged_frac_of_mfma_peak": round(fl / (ak * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "step_ms": round(sk, 4), "timing": "HIP events, last-level cache flushed before each call"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_b256_long",
                    choices=["decode_b256_long", "decode_b64_gqa4", "tiny_decode_fp32", "mixed_step",
                             "varlen_prefill", "paged_prefill", "copy_1gib"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill and mixed-step legs")
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

    if args.workload == "varlen_prefill":
        case = workloads.make_config("varlen_prefill", device=dev)
        wall, kern = time_varlen(pkv, torch, case, K, W)
        fl = varlen_flops(case)
        tf = fl / (wall * 1e-3) / 1e12
        ach = fl / (kern * 1e-3) / 1e12
        print(json.dumps({
            "metric": METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": round(wall, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "varlen_prefill", "batch": 16, "num_heads": 32,
                       "num_kv_heads": 8, "head_dim": 128, "flops_per_step": fl},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": None}}))
        return

    if args.workload == "paged_prefill":
        r = paged_prefill_leg(pkv, torch, workloads, K, W, dev)
        print(json.dumps(r))
        return

    log("generating", args.workload)
    if args.workload == "mixed_step":
        case = workloads.make_config("mixed_step", device=dev, part="decode")
    else:
        case = workloads.make_config(args.workload, device=dev)
    torch.cuda.synchronize()
    B, _, Hq, D = case.q.shape
    NB, bs, Hkv, _ = case.k_cache.shape
    kvb = kv_bytes(case)
    log(f"timing {K} steps after {W} warmup; KV bytes/step {kvb / 1e9:.3f} GB")
    wall, part_ms, merge_ms, _ = time_decode(pkv, torch, case, K, W)
    gbs = kvb / (wall * 1e-3) / 1e9
    ach = kvb / (part_ms * 1e-3) / 1e9
    eff_pt = pkv.decode_partition_tokens(B, Hq, Hkv, D, bs, case.block_table.shape[1],
                                         case.partition_tokens)
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(wall, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": str(case.q.dtype).replace("torch.", "").replace("bfloat16", "bf16").replace("float32", "f32"),
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "num_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": bs, "partition_tokens": eff_pt,
                   "append": case.k_new is not None,
                   "cached_tokens": int(case.lengths.sum()), "kv_bytes_per_step": kvb},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "queries_per_s": round(B / (wall * 1e-3), 1),
        "kernels_ms": {"decode_partial": round(part_ms, 4), "decode_merge": round(merge_ms, 4)},
        "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL.get(args.workload, "decode_partial_kernel"),
                     "achieved": round(ach, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("decode.hip", args.workload)},
    }
    log(f"decode {gbs:.1f} GB/s wall, partial kernel {ach:.1f} GB/s ({part_ms:.3f} ms), merge {merge_ms:.3f} ms")

    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        res["cpu_baseline"] = cpu_baseline(torch, case, args.cpu_seconds)
        log("cpu baseline", res["cpu_baseline"]["value"], "GB/s on", res["cpu_baseline"]["cores"], "threads")
    else:
        res["cpu_baseline"] = None

    if not args.no_extra and args.workload == "decode_b256_long":
        del case
        torch.cuda.empty_cache()
        log("prefill leg: varlen_prefill")
        pcase = workloads.make_config("varlen_prefill", device=dev)
        pw, pk = time_varlen(pkv, torch, pcase, max(K // 2, 5), max(W // 2, 2))
        fl = varlen_flops(pcase)
        res["prefill"] = {"workload": "varlen_prefill", "flops_per_step": fl,
                          "ms_per_step": round(pw, 4), "tflops": round(fl / (pw * 1e-3) / 1e12, 2),
                          "kernel_tflops": round(fl / (pk * 1e-3) / 1e12, 2),
                          "frac_of_mfma_peak": round(fl / (pk * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        log("prefill", res["prefill"])
        del pcase
        torch.cuda.empty_cache()
        log("paged prefill leg")
        res["paged_prefill"] = paged_prefill_leg(pkv, torch, workloads, max(K // 2, 5),
                                                 max(W // 2, 2), dev)
        log("paged prefill", res["paged_prefill"])
        torch.cuda.empty_cache()
        log("mixed step leg: mixed_step")
        dcase, vcase = workloads.make_config("mixed_step", device=dev)
        dk = kv_bytes(dcase)
        vf = varlen_flops(vcase)
        n = max(K // 2, 5)
        dw, dpart, dmerge, _ = time_decode(pkv, torch, dcase, n, max(W // 2, 2))
        vw, vk = time_varlen(pkv, torch, vcase, n, max(W // 2, 2))
        # the whole step back to back: decode (append + attend) then prefill
        out_d = torch.empty_like(dcase.q)
        out_v = torch.empty_like(vcase.q)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            pkv.decode(dcase.q, dcase.k_cache, dcase.v_cache, dcase.block_table, dcase.cache_seqlens,
                       dcase.k_new, dcase.v_new, softmax_scale=dcase.softmax_scale,
                       partition_tokens=dcase.partition_tokens, out=out_d)
            pkv.varlen(vcase.q, vcase.k, vcase.v, vcase.cu_seq_lens_q, vcase.cu_seq_lens_k,
                       vcase.max_length_q, vcase.max_length_k, softmax_scale=vcase.softmax_scale,
                       out=out_v)
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) * 1e3 / n
        ideal_ms = dk / (HBM_PEAK_GBS * 1e9) * 1e3 + vf / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
        res["mixed_step"] = {"workload": "mixed_step", "ms_per_step": round(step_ms, 4),
                             "decode_kv_bytes": dk, "decode_gbs": round(dk / (dpart + dmerge) / 1e6, 2),
                             "decode_queries_per_s": round(dcase.q.shape[0] / (dpart + dmerge) * 1e3, 1),
                             "prefill_flops": vf, "prefill_tflops": round(vf / (vk * 1e-3) / 1e12, 2),
                             "roofline_ms": round(ideal_ms, 4),
                             "frac_of_summed_roofline": round(ideal_ms / step_ms, 4)}
        log("mixed", res["mixed_step"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
