"""Pins of the prefix-cache oracle (deepsonar "PagedAttention de vLLM …", §2.4 block pool
and hash chain of V1, §VII step 5) against what the pages state, by brute force and
by scenarios the pages describe.  CPU only."""
import random

import pytest

from oracle import prefix_cache as pc
from oracle.allocator import OutOfBlocks

BS = 16


def chain(tokens, extra=0, bs=BS):
    """Hashes of every full block of `tokens`, built block by block."""
    out, parent = [], pc.ZERO_HASH
    for i in range(len(tokens) // bs):
        parent = pc.block_hash(parent, tokens[i * bs:(i + 1) * bs], extra)
        out.append(parent)
    return out


def test_one_changed_token_changes_its_block_and_every_later_hash():
    rng = random.Random(1)
    toks = [rng.randrange(50000) for _ in range(6 * BS)]
    base = chain(toks)
    assert len(base) == 6 and len(set(base)) == 6 and all(len(h) == 32 for h in base)
    for pos in range(len(toks)):
        t2 = list(toks)
        t2[pos] += 1
        h2 = chain(t2)
        k = pos // BS
        assert h2[:k] == base[:k]                         # earlier blocks untouched
        assert all(a != b for a, b in zip(h2[k:], base[k:]))   # this one and all later differ


def test_parent_and_extra_key_salt_the_hash():
    toks = list(range(BS))
    h0 = pc.block_hash(pc.ZERO_HASH, toks, 0)
    assert pc.block_hash(pc.ZERO_HASH, toks, 0) == h0               # deterministic
    assert pc.block_hash(pc.ZERO_HASH, toks, 1) != h0               # extra key
    assert pc.block_hash(h0, toks, 0) != h0                         # parent
    assert chain(toks * 3, extra=7)[2] != chain(toks * 3, extra=0)[2]


def _write(a, seq, tokens):
    slots, copies = a.append_tokens(seq, tokens)
    return slots


def test_same_prompt_takes_over_every_block_before_the_last_token():
    a = pc.PrefixCachingAllocator(32, BS, list(range(32)))
    prompt = list(range(100, 100 + 3 * BS + 5))          # 53 tokens: 3 full blocks + 5
    s1, n1 = a.create_prefix(prompt)
    assert n1 == 0
    _write(a, s1, prompt)
    t1 = a.block_table(s1)
    s2, n2 = a.create_prefix(prompt)
    assert n2 == 3 * BS and a.block_table(s2) == t1[:3]   # the same physical blocks
    assert [a.refcount[b] for b in t1[:3]] == [2, 2, 2]
    _write(a, s2, prompt[n2:])
    assert a.block_table(s2)[:3] == t1[:3] and a.block_table(s2)[3] != t1[3]
    assert a.context_len(s2) == len(prompt)


def test_full_hit_still_recomputes_the_last_token():
    a = pc.PrefixCachingAllocator(32, BS)
    prompt = list(range(3 * BS))                          # exactly 3 full blocks
    s1, _ = a.create_prefix(prompt)
    _write(a, s1, prompt)
    assert a.num_cached() == 3
    s2, n2 = a.create_prefix(prompt)
    assert n2 == 2 * BS                                   # block 2 holds the last token


def test_differing_token_stops_the_match_at_its_block():
    a = pc.PrefixCachingAllocator(32, BS)
    p1 = list(range(4 * BS + 1))
    s1, _ = a.create_prefix(p1)
    _write(a, s1, p1)
    p2 = list(p1)
    p2[BS + 3] = -5                                       # inside block 1
    _, n2 = a.create_prefix(p2)
    assert n2 == BS


def test_released_blocks_stay_cached_until_the_queue_head_reaches_them():
    nb = 8
    a = pc.PrefixCachingAllocator(nb, BS, list(range(nb)))
    prompt = list(range(3 * BS + 1))                      # 4 blocks: 0,1,2,3
    s1, _ = a.create_prefix(prompt)
    _write(a, s1, prompt)
    assert a.block_table(s1) == [0, 1, 2, 3]
    a.release(s1)                                         # tail of the queue, logical order
    assert list(a.free) == [4, 5, 6, 7, 0, 1, 2, 3] and a.num_cached() == 3
    # a hit takes blocks out of the free queue
    s2, n2 = a.create_prefix(prompt)
    assert n2 == 3 * BS and a.num_free() == 5 and list(a.free) == [4, 5, 6, 7, 3]
    a.release(s2)
    assert list(a.free) == [4, 5, 6, 7, 3, 0, 1, 2]
    # other work takes the head: blocks 4..7, then 3 (no hash: partial), then 0 is
    # evicted, which breaks the chain at its first block
    s3 = a.create()
    a.append(s3, 5 * BS + 1)
    assert a.block_table(s3) == [4, 5, 6, 7, 3, 0] and a.evictions == 1
    _, n4 = a.create_prefix(prompt)
    assert n4 == 0 and a.num_cached() == 2               # blocks 1, 2 still mapped, unreachable


def test_eviction_order_is_queue_order_not_insertion():
    a = pc.PrefixCachingAllocator(6, BS, list(range(6)))
    pa, pb = [1] * (BS + 1), [2] * (BS + 1)
    sa, _ = a.create_prefix(pa)
    _write(a, sa, pa)                                     # blocks 0, 1 (0 cached)
    sb, _ = a.create_prefix(pb)
    _write(a, sb, pb)                                     # blocks 2, 3 (2 cached)
    a.release(sb)                                         # queue: 4 5 2 3
    a.release(sa)                                         # queue: 4 5 2 3 0 1
    s = a.create()
    a.append(s, 3 * BS)                                   # takes 4, 5, 2 -> evicts b's block
    assert a.evictions == 1
    assert a.create_prefix(pb)[1] == 0 and a.create_prefix(pa)[1] == BS


def test_untracked_appends_register_nothing():
    a = pc.PrefixCachingAllocator(8, BS)
    s = a.create()
    a.append(s, 3 * BS)
    assert a.num_cached() == 0
    s2, n = a.create_prefix(list(range(3 * BS)))
    assert n == 0


def test_random_streams_keep_the_invariants_and_hits_hold_the_prompt():
    """Brute force: every hit block was filled with exactly the prompt tokens it stands
    for, registered hashes equal the chain recomputed from the writer's tokens, and the
    allocator's counts stay consistent."""
    rng = random.Random(7)
    for trial in range(30):
        nb = rng.randrange(6, 40)
        a = pc.PrefixCachingAllocator(nb, 4, rng.sample(range(nb), nb))
        written = {}                                      # block -> tokens it holds (full)
        live = []
        vocab = [rng.randrange(5) for _ in range(3)]
        for _ in range(120):
            op = rng.random()
            try:
                if op < 0.35 or not live:
                    base = rng.choice([[0, 1, 2, 3, 4, 5, 6, 7, 8], [0, 1, 2, 3, 9, 9, 9, 9], [vocab[0]] * 9])
                    prompt = base[:rng.randrange(1, len(base) + 1)] + [rng.randrange(3) for _ in range(rng.randrange(4))]
                    s, n = a.create_prefix(prompt, extra_key=rng.randrange(2))
                    live.append(s)
                    for j, b in enumerate(a.block_table(s)):
                        assert written[b] == prompt[4 * j:4 * j + 4]
                    a.append_tokens(s, prompt[n:])
                elif op < 0.6:
                    s = rng.choice(live)
                    a.append_tokens(s, [rng.randrange(3) for _ in range(rng.randrange(1, 6))])
                elif op < 0.7:
                    live.append(a.fork(rng.choice(live)))
                else:
                    s = live.pop(rng.randrange(len(live)))
                    a.release(s)
            except OutOfBlocks:
                pass
            # record what each full block of each tracked sequence holds
            for s in live:
                toks = a.tokens[s]
                if toks is None:
                    continue
                for j in range(len(toks) // 4):
                    written[a.tables[s][j]] = toks[4 * j:4 * j + 4]
                hs = chain(toks, a.extra[s], 4)
                for j, h in enumerate(hs):
                    b = a.tables[s][j]
                    if b in a.hash_of:
                        assert a.block_of[a.hash_of[b]] == b
                        assert a.hash_of[b] == h
            used = {b for s in live for b in a.tables[s]}
            assert len(a.free) + len(used) == nb
            assert sorted(set(a.free)) == sorted(a.free) and not (set(a.free) & used)
            assert sum(a.refcount) == sum(len(a.tables[s]) for s in live)
            assert all(a.block_of[h] == b for b, h in a.hash_of.items())


# -- planted mistakes: each one must break a pin above ---------------------------

def test_planted_unchained_hash_is_caught():
    orig = pc.block_hash
    pc.block_hash = lambda parent, tokens, extra=0: orig(pc.ZERO_HASH, tokens, extra)
    try:
        with pytest.raises(AssertionError):
            test_one_changed_token_changes_its_block_and_every_later_hash()
    finally:
        pc.block_hash = orig


def test_planted_full_prompt_match_is_caught(monkeypatch):
    def create_prefix(self, prompt, extra_key=0):
        sid = pc.BlockAllocator.create(self)
        self.tokens[sid], self.extra[sid], parent = [], extra_key, pc.ZERO_HASH
        for i in range(len(prompt) // self.block_size):          # no last-token rule
            h = pc.block_hash(parent, prompt[i * BS:(i + 1) * BS], extra_key)
            b = self.block_of.get(h)
            if b is None:
                break
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
            self.tables[sid].append(b)
            self.tokens[sid].extend(prompt[i * BS:(i + 1) * BS])
            self.lengths[sid] += BS
            parent = h
        self.last_hash[sid] = parent
        return sid, self.lengths[sid]
    monkeypatch.setattr(pc.PrefixCachingAllocator, "create_prefix", create_prefix)
    with pytest.raises(AssertionError):
        test_full_hit_still_recomputes_the_last_token()


def test_planted_eviction_from_the_tail_is_caught(monkeypatch):
    def take(self):
        b = self.free.pop()
        if b in self.hash_of:
            del self.block_of[self.hash_of.pop(b)]
            self.evictions += 1
        return b
    monkeypatch.setattr(pc.PrefixCachingAllocator, "_take_free", take)
    with pytest.raises(AssertionError):
        test_released_blocks_stay_cached_until_the_queue_head_reaches_them()
