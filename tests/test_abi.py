"""The C ABI on the CPU: the library loads without a GPU, exports every
function include/pkv.h declares, and its host-only checks and launch plan
behave as documented.  No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_296_amd as p
    p._load()
    return p


def test_header_declares_the_calls():
    names = declared_functions()
    for must in ("pkv_decode", "pkv_varlen", "pkv_decode_workspace_bytes",
                 "pkv_check_decode_args", "pkv_check_varlen_args", "pkv_status_string",
                 "pkv_cache_write", "pkv_varlen_paged", "pkv_check_cache_write_args",
                 "pkv_check_varlen_paged_args"):
        assert must in names


def test_library_exports_every_declared_symbol(pkv):
    lib = ctypes.CDLL(pkv.lib_path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_status_strings(pkv):
    assert pkv.status_string(0) == "ok"
    for s in range(1, 5):
        assert pkv.status_string(s) not in ("ok", "unknown status")
    assert pkv.status_string(99) == "unknown status"
    assert pkv.abi_version() >= 1


@pytest.mark.parametrize("args,want", [
    # dtype, has_new, batch, Hq, Hkv, D, num_blocks, bs, max_blocks, partition
    ((1, 0, 64, 32, 8, 128, 20000, 16, 256, 0), 0),
    ((0, 1, 3, 4, 4, 64, 8, 32, 4, 0), 0),
    ((1, 0, 4, 6, 4, 128, 10, 16, 4, 0), 1),      # Hq % Hkv != 0
    ((1, 0, 4, 8, 4, 96, 10, 16, 4, 0), 2),       # head_dim 96 unsupported
    ((1, 0, 4, 8, 4, 128, 10, 8, 4, 0), 2),       # block_size 8 unsupported
    ((2, 0, 4, 8, 4, 128, 10, 16, 4, 0), 2),      # unknown dtype
    ((1, 0, -1, 8, 4, 128, 10, 16, 4, 0), 1),     # negative batch
    ((1, 0, 4, 8, 0, 128, 10, 16, 4, 0), 1),      # zero kv heads
    ((1, 0, 4, 8, 4, 128, 10, 16, 4, 24), 2),     # partition not a block multiple
    ((1, 0, 4, 8, 4, 128, 10, 16, 4, 16 * 257), 2),  # partition beyond 256 blocks
    ((1, 2, 4, 8, 4, 128, 10, 16, 4, 0), 1),      # has_new must be 0/1
])
def test_check_decode_args(pkv, args, want):
    assert pkv.check_decode_args(*args) == want


@pytest.mark.parametrize("args,want", [
    ((1, 16, 100, 200, 32, 8, 128, 50, 60), 0),
    ((0, 16, 100, 200, 32, 8, 128, 50, 60), 2),   # fp32 varlen not built
    ((1, 16, 100, 200, 32, 8, 80, 50, 60), 2),
    ((1, 16, 100, 200, 30, 8, 128, 50, 60), 1),
    ((1, -1, 100, 200, 32, 8, 128, 50, 60), 1),
])
def test_check_varlen_args(pkv, args, want):
    assert pkv.check_varlen_args(*args) == want


@pytest.mark.parametrize("args,want", [
    # dtype, batch, total, Hkv, D, num_blocks, bs, max_blocks
    ((1, 16, 16000, 8, 128, 2634, 16, 241), 0),
    ((0, 3, 3, 4, 64, 8, 32, 4), 0),              # fp32 rows are fine (a byte copy)
    ((1, 0, 0, 8, 128, 10, 16, 4), 0),            # nothing to write
    ((1, 0, 5, 8, 128, 10, 16, 4), 1),            # rows without a request
    ((1, 4, 10, 8, 96, 10, 16, 4), 2),            # head_dim 96
    ((1, 4, 10, 8, 128, 10, 8, 4), 2),            # block_size 8
    ((1, 4, -1, 8, 128, 10, 16, 4), 1),
    ((3, 4, 10, 8, 128, 10, 16, 4), 2),
])
def test_check_cache_write_args(pkv, args, want):
    assert pkv.check_cache_write_args(*args) == want


@pytest.mark.parametrize("args,want", [
    # dtype, batch, total_q, Hq, Hkv, D, num_blocks, bs, max_blocks, max_q, max_k
    ((1, 16, 16000, 32, 8, 128, 2634, 16, 241, 2048, 3848), 0),
    ((1, 1, 1, 8, 8, 64, 10, 32, 4, 1, 2048 * 32), 0),      # the most keys the LDS table holds
    ((1, 1, 1, 8, 8, 64, 10, 32, 4, 1, 2048 * 32 + 1), 2),
    ((0, 16, 100, 32, 8, 128, 50, 16, 8, 60, 60), 2),        # bf16 only
    ((1, 16, 100, 30, 8, 128, 50, 16, 8, 60, 60), 1),
    ((1, 16, 100, 32, 8, 128, 50, 8, 8, 60, 60), 2),         # block_size 8
    ((1, 16, 100, 32, 8, 80, 50, 16, 8, 60, 60), 2),
])
def test_check_varlen_paged_args(pkv, args, want):
    assert pkv.check_varlen_paged_args(*args) == want


def test_partition_plan_and_workspace(pkv):
    # explicit partition: 512 tokens over a 2048-block row -> 64 partitions
    assert pkv.decode_partition_tokens(256, 64, 8, 128, 16, 2048, 512) == 512
    ws = pkv.decode_workspace_bytes(256, 64, 8, 128, 16, 2048, 512)
    slots = 256 * 64 * 64
    assert ws >= slots * (128 + 2) * 4
    # the tiny example fits one pass: only the work list, no partial results
    p = pkv.decode_partition_tokens(3, 4, 4, 64, 32, 4, 0)
    assert p >= 4 * 32
    assert 0 < pkv.decode_workspace_bytes(3, 4, 4, 64, 32, 4, 0) <= 4096
    # library choice is a block multiple within the LDS slice
    for args in [(64, 32, 8, 128, 16, 256), (512, 32, 8, 128, 16, 513), (1, 8, 1, 128, 32, 4096)]:
        p = pkv.decode_partition_tokens(*args, 0)
        assert p > 0 and p % args[4] == 0 and p // args[4] <= 256
    # rejected arguments give -1 / 0
    assert pkv.decode_partition_tokens(4, 6, 4, 128, 16, 4, 0) == -1
    assert pkv.decode_workspace_bytes(4, 6, 4, 128, 16, 4, 0) == 0


def test_product_path_refuses_cpu_tensors(pkv):
    import torch
    q = torch.zeros(1, 1, 4, 64)
    kc = torch.zeros(2, 16, 4, 64)
    bt = torch.zeros(1, 2, dtype=torch.int32)
    sl = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        pkv.decode(q, kc, kc.clone(), bt, sl)
    with pytest.raises(ValueError, match="GPU"):
        pkv.varlen(torch.zeros(1, 4, 4, 64), torch.zeros(1, 4, 4, 64), torch.zeros(1, 4, 4, 64),
                   torch.tensor([0, 4], dtype=torch.int32), torch.tensor([0, 4], dtype=torch.int32), 4, 4)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        pkv.cache_write(torch.zeros(1, 4, 4, 64), torch.zeros(1, 4, 4, 64), cu, sl, kc, kc.clone(), bt)
    with pytest.raises(ValueError, match="GPU"):
        pkv.varlen_paged(torch.zeros(1, 4, 4, 64), kc, kc.clone(), bt, cu, sl, 4, 4)


def test_library_partition_rule(pkv):
    # 512 tokens when the batch then has about 1.75 units per resident wave
    # (2048 waves; rows assumed to average half their span) or more: the
    # long-context and mixed-step shapes, whatever the row span beyond it
    assert pkv.decode_partition_tokens(256, 64, 8, 128, 16, 2048, 0) == 512
    assert pkv.decode_partition_tokens(512, 32, 8, 128, 16, 513, 0) == 512
    assert pkv.decode_partition_tokens(128, 32, 8, 128, 16, 256, 0) == 512
    # fewer: the length that gives that many, rounded up to 64 tokens --
    # 64 GQA-4 sequences of up to 4096 tokens get 320, 48 of them 256, 32
    # of them 192
    assert pkv.decode_partition_tokens(64, 32, 8, 128, 16, 256, 0) == 320
    assert pkv.decode_partition_tokens(48, 32, 8, 128, 16, 256, 0) == 256
    assert pkv.decode_partition_tokens(32, 32, 8, 128, 16, 256, 0) == 192
    # a row shorter than the partition: one pass over the whole row when
    # that gives enough units
    assert pkv.decode_partition_tokens(1024, 32, 8, 128, 16, 20, 0) == 320
    # ... else split: 64 x 8 one-pass units become 128-token parts
    assert pkv.decode_partition_tokens(64, 32, 8, 128, 16, 20, 0) == 128
    # never below 128 tokens (one long sequence: 192 here)
    assert pkv.decode_partition_tokens(1, 8, 8, 128, 16, 8192, 0) == 192
    assert pkv.decode_partition_tokens(1, 8, 2, 128, 16, 512, 0) == 128
    assert pkv.decode_partition_tokens(1, 8, 1, 128, 32, 4096, 0) == 128
    # an explicit partition is kept as given
    assert pkv.decode_partition_tokens(64, 32, 8, 128, 16, 256, 1024) == 1024
