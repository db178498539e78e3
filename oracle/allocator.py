"""Block allocator of the paged KV cache, replayed in plain Python.

What the pages fix, and where:
  - the KV memory is cut once into fixed-size physical blocks and every request
    keeps a table from logical block number to physical block number
    (deepsonar "PagedAttention de vLLM …", §2.2; §VII step 1);
  - a new block is taken only when the previous one is full, so a request never
    wastes more than one block (§2.2; §VII step 2; deeplearn.tn "PagedAttention :
    comment optimiser la mémoire GPU …", worked allocation example);
  - shared blocks carry a reference count; a writer whose block is shared copies
    it first, then writes (copy-on-write: §2.3; §VII step 3);
  - free blocks sit in a queue: allocation takes the head, release appends at the
    tail (§2.4, free-block queue of the block pool).

Readings where the pages are silent (both the oracle and the library follow them):
  - the initial queue order is an input (a permutation of block ids);
  - a released sequence returns its blocks in logical order, block 0 first, each
    one when its count reaches zero;
  - copy-on-write copies the whole block (all slots, K and V, every KV head);
    the last sharer (count 1) writes in place;
  - an append that cannot get every block it needs changes nothing and fails;
  - sequence ids are handed out 0, 1, 2, ... in create/fork order.
"""
from collections import deque


class OutOfBlocks(RuntimeError):
    pass


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be >= 1")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.free = deque(order)
        self.refcount = [0] * self.num_blocks
        self.tables = {}     # seq id -> list of physical block ids, logical order
        self.lengths = {}    # seq id -> number of tokens written
        self.next_id = 0

    # -- sequences ---------------------------------------------------------
    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        """New sequence that shares every block of `parent` (counts go up by one)."""
        if parent not in self.tables:
            raise KeyError(parent)
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = list(self.tables[parent])
        self.lengths[sid] = self.lengths[parent]
        for b in self.tables[sid]:
            self.refcount[b] += 1
        return sid

    def blocks_needed(self, seq: int, n: int) -> int:
        """Fresh blocks an append of n tokens would take from the queue."""
        length, bs = self.lengths[seq], self.block_size
        fresh = sum(1 for p in range(length, length + n) if p % bs == 0)
        if n > 0 and length % bs != 0 and self.refcount[self.tables[seq][-1]] > 1:
            fresh += 1      # the shared, partly filled tail block gets copied first
        return fresh

    def append(self, seq: int, n: int):
        """Reserve slots for n new tokens of `seq`.

        Returns (slots, copies): the slot of each new token (physical block x
        block size + offset in the block) and the (source, destination) block
        pairs that must be copied before the new tokens are written.
        """
        if seq not in self.tables:
            raise KeyError(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        if self.blocks_needed(seq, n) > len(self.free):
            raise OutOfBlocks(f"sequence {seq} needs {self.blocks_needed(seq, n)} blocks, "
                              f"{len(self.free)} free")
        bs, table = self.block_size, self.tables[seq]
        slots, copies = [], []
        for _ in range(n):
            p = self.lengths[seq]
            if p % bs == 0:
                b = self.free.popleft()
                self.refcount[b] = 1
                table.append(b)
            elif self.refcount[table[-1]] > 1:
                src = table[-1]
                dst = self.free.popleft()
                self.refcount[src] -= 1
                self.refcount[dst] = 1
                table[-1] = dst
                copies.append((src, dst))
            slots.append(table[p // bs] * bs + p % bs)
            self.lengths[seq] = p + 1
        return slots, copies

    def release(self, seq: int):
        """Drop a sequence (finished, cancelled or preempted)."""
        table = self.tables.pop(seq)
        del self.lengths[seq]
        for b in table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)

    # -- views ---------------------------------------------------------------
    def block_table(self, seq: int):
        return list(self.tables[seq])

    def context_len(self, seq: int) -> int:
        return self.lengths[seq]

    def num_free(self) -> int:
        return len(self.free)

    def num_used(self) -> int:
        return self.num_blocks - len(self.free)

    def waste_slots(self) -> int:
        """Reserved-but-empty slots summed over sequences (block size x blocks - tokens)."""
        return sum(self.block_size * len(t) - self.lengths[s] for s, t in self.tables.items())
