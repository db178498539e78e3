"""Prefix caching on top of the block allocator, replayed in plain Python.

Test infrastructure: only tests, the smoke check and the bench's CPU baseline use it.

What the pages fix (deepsonar "PagedAttention de vLLM …", §2.4 block pool and hash
chain of V1, and §VII step 5):
  - a full block is identified by a chained hash: SHA-256 over the parent block's
    hash, the block's token ids and an extra key, so one differing token changes the
    hash of its block and of every later block;
  - a map from block hash to physical block finds cached blocks;
  - a new prompt is compared block by block along its hash chain; each matching block
    is taken over (its count goes up) and its prefill is skipped;
  - even when every prompt block matches, the last prompt token is computed again
    (its logits are needed), so at most the blocks inside the first len-1 tokens match;
  - the free queue is ordered by last use (released blocks go to the tail, allocation
    takes the head) and is the eviction order: a block taken from the head that still
    holds cached content leaves the map first.

Readings where the pages are silent (the library follows the same ones):
  - hash input bytes: the parent digest (32 zero bytes for a sequence's first block),
    then the block's token ids as little-endian int32, then the extra key as a
    little-endian int64;
  - only full blocks are hashed; a block gets its hash when its last slot is filled
    by an append that gives token ids;
  - if a full block's hash is already in the map (another block holds the same
    content), the map keeps the older block and the new one stays unregistered;
  - a matched block sitting in the free queue (count 0) leaves the queue;
  - released blocks keep their hash (that is what makes later hits possible);
  - a sequence created without a prompt, or appended to without token ids, never
    registers blocks.
"""
import hashlib
import struct

from .allocator import BlockAllocator, OutOfBlocks

ZERO_HASH = bytes(32)


def block_hash(parent: bytes, tokens, extra_key: int = 0) -> bytes:
    """Chained block hash (deepsonar §2.4): SHA-256(parent || tokens || extra key)."""
    if len(parent) != 32:
        raise ValueError("parent hash must be 32 bytes")
    body = struct.pack(f"<{len(tokens)}i", *[int(t) for t in tokens])
    return hashlib.sha256(parent + body + struct.pack("<q", int(extra_key))).digest()


class PrefixCachingAllocator(BlockAllocator):
    def __init__(self, num_blocks, block_size, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.hash_of = {}          # block -> digest, for cached (registered) blocks
        self.block_of = {}         # digest -> block
        self.tokens = {}           # seq -> token ids written so far, or None (untracked)
        self.last_hash = {}        # seq -> digest of its last full block
        self.extra = {}            # seq -> extra key
        self.hit_blocks = 0
        self.evictions = 0

    # -- queue ---------------------------------------------------------------
    def _take_free(self) -> int:
        b = self.free.popleft()
        if b in self.hash_of:          # cached content at the head: evict it first
            del self.block_of[self.hash_of.pop(b)]
            self.evictions += 1
        return b

    # -- sequences -----------------------------------------------------------
    def create(self) -> int:
        sid = super().create()
        self.tokens[sid] = None
        self.last_hash[sid] = ZERO_HASH
        self.extra[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        sid = super().fork(parent)
        t = self.tokens[parent]
        self.tokens[sid] = None if t is None else list(t)
        self.last_hash[sid] = self.last_hash[parent]
        self.extra[sid] = self.extra[parent]
        return sid

    def create_prefix(self, prompt, extra_key: int = 0):
        """New sequence for `prompt`: take over the cached blocks its hash chain matches.

        Returns (seq, n_cached): the sequence holds the first n_cached prompt tokens
        (a multiple of the block size, at most len(prompt) - 1); the caller appends
        the rest with append_tokens."""
        sid = super().create()
        bs = self.block_size
        self.tokens[sid] = []
        self.extra[sid] = int(extra_key)
        parent = ZERO_HASH
        for i in range((len(prompt) - 1) // bs if len(prompt) else 0):
            h = block_hash(parent, prompt[i * bs:(i + 1) * bs], extra_key)
            b = self.block_of.get(h)
            if b is None:
                break
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
            self.tables[sid].append(b)
            self.tokens[sid].extend(int(t) for t in prompt[i * bs:(i + 1) * bs])
            self.lengths[sid] += bs
            self.hit_blocks += 1
            parent = h
        self.last_hash[sid] = parent
        return sid, self.lengths[sid]

    def append(self, seq: int, n: int):
        """Append without token ids: the sequence stops registering blocks (once the
        append succeeded: a failed append changes nothing)."""
        out = self._append(seq, n)
        self.tokens[seq] = None
        return out

    def append_tokens(self, seq: int, tokens):
        """Append with token ids: every block this fills is hashed and registered."""
        toks = [int(t) for t in tokens]
        slots, copies = self._append(seq, len(toks), toks)
        return slots, copies

    def _append(self, seq, n, toks=None):
        if seq not in self.tables:
            raise KeyError(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        if self.blocks_needed(seq, n) > len(self.free):
            raise OutOfBlocks(f"sequence {seq} needs {self.blocks_needed(seq, n)} blocks, "
                              f"{len(self.free)} free")
        bs, table = self.block_size, self.tables[seq]
        slots, copies = [], []
        for i in range(n):
            p = self.lengths[seq]
            if p % bs == 0:
                b = self._take_free()
                self.refcount[b] = 1
                table.append(b)
            elif self.refcount[table[-1]] > 1:
                src = table[-1]
                dst = self._take_free()
                self.refcount[src] -= 1
                self.refcount[dst] = 1
                table[-1] = dst
                copies.append((src, dst))
            slots.append(table[p // bs] * bs + p % bs)
            self.lengths[seq] = p + 1
            if toks is not None and self.tokens[seq] is not None:
                self.tokens[seq].append(toks[i])
                if (p + 1) % bs == 0:                     # block just became full
                    h = block_hash(self.last_hash[seq], self.tokens[seq][p + 1 - bs:p + 1],
                                   self.extra[seq])
                    self.last_hash[seq] = h
                    b = table[p // bs]
                    if h not in self.block_of and b not in self.hash_of:
                        self.block_of[h] = b
                        self.hash_of[b] = h
        return slots, copies

    def release(self, seq: int):
        super().release(seq)
        del self.tokens[seq], self.last_hash[seq], self.extra[seq]

    def num_cached(self) -> int:
        return len(self.block_of)
