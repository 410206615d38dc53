"""GPU checks of the host-side launch state: the per-kernel occupancy caches
and the stream the binding allocates its temporaries on.

- Every decode kernel instantiation queries its own occupancy: an fp32
  head_dim-128 call (one wave per SIMD) made first in a process must not
  change the run length the bf16 head_dim-128 plan picks (two waves per
  SIMD).  The plan kernel writes the run length R into the third control
  word of the workspace; it is read back and compared with the plan rule
  R = clamp(units / (3 x resident waves), 1, 8).
- A decode launched on a side stream keeps its workspace away from
  allocations made meanwhile on the default stream.
"""
import os
import subprocess
import sys
import textwrap

import pytest
import torch

import paged_kv_cache_296_amd as pkv
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_PLAN_SCRIPT = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import torch
    import paged_kv_cache_296_amd as pkv
    import workloads
    torch.cuda.set_device(0)
    if {fp32_first}:
        c = workloads.make_decode(seed=1, dtype="fp32", batch=4, num_heads=8, num_kv_heads=2,
                                  head_dim=128, block_size=16, lengths=[100, 200, 300, 400],
                                  num_blocks=200, append=False, device="cuda")
        pkv.decode(c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens)
        torch.cuda.synchronize()
    # 72 sequences x 512 tokens in 16-token partitions, 8 kv heads, GQA 4:
    # 72 * 32 * 8 = 18432 units
    c = workloads.make_decode(seed=2, dtype="bf16", batch=72, num_heads=32, num_kv_heads=8,
                              head_dim=128, block_size=16, lengths=[512] * 72,
                              num_blocks=72 * 32 + 8, append=False, partition_tokens=16,
                              device="cuda")
    out, ws = pkv.decode_partials(c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens,
                                  partition_tokens=16)
    torch.cuda.synchronize()
    print("R", int(ws[8:12].view(torch.int32).item()),
          torch.cuda.get_device_properties(0).multi_processor_count, flush=True)
""")


def _plan_run_length(fp32_first):
    script = _PLAN_SCRIPT.format(root=ROOT, fp32_first=fp32_first)
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [x for x in r.stdout.splitlines() if x.startswith("R ")][-1]
    _, R, cus = line.split()
    return int(R), int(cus)


def test_decode_plan_not_changed_by_an_earlier_fp32_call():
    R, cus = _plan_run_length(fp32_first=True)
    units = 72 * 32 * 8
    resident_waves = 2 * cus * 4           # bf16 head_dim 128: 2 workgroups of 4 waves per CU
    # the plan aims at about two units per resident wave, at most 8 partitions a run
    want = max(1, min(8, units // (2 * resident_waves)))
    assert R == want, (R, want, cus)
    R2, _ = _plan_run_length(fp32_first=False)
    assert R2 == R


def test_side_stream_workspace_survives_default_stream_allocations():
    case = workloads.make_decode(seed=8100, dtype="bf16", batch=64, num_heads=32, num_kv_heads=8,
                                 head_dim=128, block_size=16, lengths=("uniform", 2000, 4000),
                                 num_blocks=20000, append=False, partition_tokens=256,
                                 device=DEV)
    ref = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table, case.cache_seqlens,
                     partition_tokens=256)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        out = pkv.decode(case.q, case.k_cache, case.v_cache, case.block_table,
                         case.cache_seqlens, partition_tokens=256, stream=side)
        # the workspace was dropped when decode returned; allocations on the
        # default stream must not be handed its memory while the side stream
        # still uses it
        junk = [torch.full((1 << 20,), float("nan"), device=DEV) for _ in range(64)]
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        del junk
