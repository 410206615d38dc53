"""Host-side physical block pool used to build block tables for the synthetic
workloads (the harness allocator, not part of the GPU path).

It follows the block manager sketched on the "Paged Attention" notes page
(section on block allocation): a list of free physical block ids, allocation
pops from the END of the list, freeing appends, and a request larger than
what is free raises an out-of-memory error.  The number of blocks a sequence
needs to grow from ``cur_len`` to ``cur_len + n_new`` tokens when it already
owns ``owned`` blocks is ceil((cur_len + n_new) / block_size) - owned (the
page's own growth formula is garbled; this is the plain count).
"""
from __future__ import annotations


class OutOfBlocks(MemoryError):
    pass


class BlockPool:
    def __init__(self, free_ids):
        self.free = [int(b) for b in free_ids]

    @classmethod
    def of_size(cls, num_blocks: int) -> "BlockPool":
        return cls(range(num_blocks))

    def pop(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free physical block")
        return self.free.pop()

    def allocate(self, n: int) -> list:
        if len(self.free) < n:
            raise OutOfBlocks(f"need {n} blocks, {len(self.free)} free")
        return [self.free.pop() for _ in range(n)]

    def release(self, ids) -> None:
        self.free.extend(int(b) for b in ids)


def blocks_to_grow(cur_len: int, n_new: int, block_size: int, owned: int) -> int:
    need = -(-(cur_len + n_new) // block_size)
    return max(0, need - owned)
