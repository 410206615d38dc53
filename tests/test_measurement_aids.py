"""GPU checks of the measurement aids that bench.py sets the kernels against
(the streaming read, the plain copy and the matrix-core loop): they run
through the C ABI, the copy moves every byte exactly, the read and the MFMA
loop leave their sinks untouched (they store only on a pattern that does not
occur), and out-of-range arguments are refused before any launch."""
import pytest
import torch

import paged_kv_cache_296_amd as pkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_stream_copy_is_exact():
    g = torch.Generator(device=DEV).manual_seed(7)
    for nbytes in (16, 4096 + 48, (3 << 20) + 16 * 37):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
        dst = torch.zeros_like(src)
        for wgs in (1, 3, 8192):
            dst.zero_()
            pkv.stream_copy(src, dst, wgs)
            torch.cuda.synchronize()
            assert torch.equal(src, dst), (nbytes, wgs)


def test_stream_read_and_mfma_loop_leave_sinks_alone():
    buf = torch.randn(1 << 20, device=DEV)
    sink = torch.full((64 * 4096 // 4,), 3.25, device=DEV)
    pkv.stream_read(buf, sink, 64, True)
    pkv.stream_read(buf, sink, 64, False)
    flops = pkv.mfma_peak(sink, 64, 100)
    torch.cuda.synchronize()
    assert flops == 64 * 4 * 100 * 4 * 32768
    assert bool((sink == 3.25).all())


def test_bad_arguments_are_refused():
    lib = pkv._load()
    x = torch.empty(1024, dtype=torch.uint8, device=DEV)
    p = x.data_ptr()
    assert lib.pkv_stream_copy(p, p + 512, 24, 4, None) == pkv.EINVAL          # not a multiple of 16
    assert lib.pkv_stream_copy(p, p + 512, 1 << 31, 4, None) == pkv.EINVAL     # 2 GiB or more
    assert lib.pkv_stream_copy(p, p + 512, 512, 0, None) == pkv.EINVAL         # no workgroups
    assert lib.pkv_stream_copy(None, p, 512, 4, None) == pkv.EINVAL
    assert lib.pkv_stream_read(p, 24, p, 4, 1, None) == pkv.EINVAL
    assert lib.pkv_stream_read(p, 512, p, 4, 2, None) == pkv.EINVAL           # hint is 0 or 1
    assert lib.pkv_stream_read(p, 8 << 30, p, 1, 1, None) == pkv.EINVAL       # 2 GiB per wave
    assert lib.pkv_mfma_peak(p, 0, 10, None) == pkv.EINVAL
    assert lib.pkv_mfma_peak(p, 4, -1, None) == pkv.EINVAL
    assert lib.pkv_mfma_peak(None, 4, 10, None) == pkv.EINVAL
    assert lib.pkv_mfma_peak(p, 4, 0, None) == pkv.OK                        # nothing to run
