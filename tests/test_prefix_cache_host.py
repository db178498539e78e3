"""Prefix caching through the C ABI (host only, no GPU): the library's chained SHA-256
and its allocator with the hash map and LRU eviction, bit-exact against the oracle
(deepsonar "PagedAttention de vLLM …", §2.4 block pool and hash chain of V1)."""
import random

import numpy as np
import pytest

from oracle import prefix_cache as pc
from oracle.allocator import OutOfBlocks
from paged_kv_cache_15_amd import binding as B


def _pool(nb, bs, order=None, prefix=True):
    flags = B.PAGED_KV_POOL_HOST_ONLY | (B.PAGED_KV_POOL_PREFIX_CACHE if prefix else 0)
    desc = B.make_desc(nb, bs, 1, 64, "bf16", flags)
    return B.paged_kv_pool_create(desc, None if order is None else np.asarray(order, np.int32))


def test_block_hash_equals_the_oracle_sha256():
    rng = random.Random(5)
    for n in [0, 1, 3, 13, 14, 15, 16, 17, 100, 1000]:
        for _ in range(5):
            toks = [rng.randrange(-2**31, 2**31) for _ in range(n)]
            parent = bytes(rng.randrange(256) for _ in range(32)) if rng.random() < 0.7 else None
            extra = rng.randrange(-2**63, 2**63)
            got = B.paged_kv_block_hash(parent, toks, extra)
            want = pc.block_hash(parent if parent is not None else pc.ZERO_HASH, toks, extra)
            assert got == want, (n, parent, extra)


def test_prefix_entry_points_need_the_flag():
    p = _pool(8, 16, prefix=False)
    with pytest.raises(RuntimeError):
        B.paged_kv_seq_create_prefix(p, list(range(40)))
    B.paged_kv_pool_destroy(p)


def _state(p, al, live):
    tables, lens = B.paged_kv_block_tables(p, [c for c, _ in live], None)
    for i, (c, o) in enumerate(live):
        n = len(al.tables[o])
        assert list(tables[i, :n]) == al.tables[o] and (tables[i, n:] == -1).all()
        assert lens[i] == al.lengths[o]
    free, used, waste = B.paged_kv_stats(p)
    assert free == al.num_free() and used == al.num_used() and waste == al.waste_slots()
    cached, hits, ev = B.paged_kv_prefix_stats(p)
    assert (cached, hits, ev) == (al.num_cached(), al.hit_blocks, al.evictions)
    for b in range(al.num_blocks):
        assert B.paged_kv_block_refcount(p, b) == al.refcount[b]


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_random_streams_bit_exact_with_oracle(bs):
    rng = random.Random(100 + bs)
    for trial in range(12):
        nb = rng.randrange(4, 60)
        order = rng.sample(range(nb), nb)
        p = _pool(nb, bs, order)
        al = pc.PrefixCachingAllocator(nb, bs, order)
        live = []        # (library id, oracle id)
        prompts = [[rng.randrange(4) for _ in range(rng.randrange(1, 4 * bs + 3))] for _ in range(4)]
        for step in range(150):
            op = rng.random()
            try_lib = try_orc = None
            if op < 0.3 or not live:
                base = rng.choice(prompts)
                prompt = base[:rng.randrange(1, len(base) + 1)] + [rng.randrange(4) for _ in range(rng.randrange(3))]
                extra = rng.choice([0, 0, 5])
                c, nc = B.paged_kv_seq_create_prefix(p, prompt, extra)
                o, no = al.create_prefix(prompt, extra)
                assert nc == no
                live.append((c, o))
                try:
                    s_o, cp_o = al.append_tokens(o, prompt[no:])
                except OutOfBlocks:
                    s_o = None
                try:
                    s_c, cp_c = B.paged_kv_seq_append_tokens(p, c, prompt[nc:])
                except RuntimeError:
                    s_c = None
                assert (s_o is None) == (s_c is None)
                if s_o is not None:
                    assert list(s_c) == list(s_o) and [tuple(x) for x in cp_c] == list(cp_o)
            elif op < 0.55:
                c, o = rng.choice(live)
                toks = [rng.randrange(4) for _ in range(rng.randrange(0, 2 * bs + 2))]
                try:
                    s_o, cp_o = al.append_tokens(o, toks)
                except OutOfBlocks:
                    s_o = None
                try:
                    s_c, cp_c = B.paged_kv_seq_append_tokens(p, c, toks)
                except RuntimeError:
                    s_c = None
                assert (s_o is None) == (s_c is None)
                if s_o is not None:
                    assert list(s_c) == list(s_o) and [tuple(x) for x in cp_c] == list(cp_o)
            elif op < 0.62:
                c, o = rng.choice(live)                  # plain append: no token ids
                n = rng.randrange(0, bs + 2)
                try:
                    s_o, _ = al.append(o, n)
                except OutOfBlocks:
                    s_o = None
                try:
                    s_c, _ = B.paged_kv_seq_append(p, c, n)
                except RuntimeError:
                    s_c = None
                assert (s_o is None) == (s_c is None)
                if s_o is not None:
                    assert list(s_c) == list(s_o)
            elif op < 0.72:
                c, o = rng.choice(live)
                live.append((B.paged_kv_seq_fork(p, c), al.fork(o)))
            else:
                c, o = live.pop(rng.randrange(len(live)))
                B.paged_kv_seq_free(p, c)
                al.release(o)
            _state(p, al, live)
        B.paged_kv_pool_destroy(p)


def test_hit_takes_blocks_out_of_the_queue_and_eviction_follows_it():
    nb, bs = 8, 16
    p = _pool(nb, bs, list(range(nb)))
    prompt = list(range(3 * bs + 1))
    s1, n1 = B.paged_kv_seq_create_prefix(p, prompt)
    B.paged_kv_seq_append_tokens(p, s1, prompt)
    B.paged_kv_seq_free(p, s1)
    s2, n2 = B.paged_kv_seq_create_prefix(p, prompt)
    assert n2 == 3 * bs and B.paged_kv_stats(p)[0] == nb - 3
    B.paged_kv_seq_free(p, s2)
    s3 = B.paged_kv_seq_create(p)
    B.paged_kv_seq_append(p, s3, 5 * bs + 1)             # reaches block 0 at the queue head
    assert B.paged_kv_prefix_stats(p)[2] == 1
    assert B.paged_kv_seq_create_prefix(p, prompt)[1] == 0
    B.paged_kv_pool_destroy(p)


def _groups_brute(tables, lens, bs, max_group, need):
    """The grouping rule written out: consecutive sequences join while the tokens shared
    by all members (common leading blocks x block size, capped at the shortest length)
    stay >= max(1, need)."""
    need = max(1, need)
    starts, shared, i, n = [], [], 0, len(tables)
    while i < n:
        j, common, mlen = i + 1, len(tables[i]), lens[i]
        while j < n and j - i < max_group:
            c = 0
            while c < min(common, len(tables[j])) and tables[j][c] == tables[i][c]:
                c += 1
            if min(c * bs, min(mlen, lens[j])) < need:
                break
            common, mlen = c, min(mlen, lens[j])
            j += 1
        starts.append(i)
        shared.append(min(common * bs, mlen) if j - i > 1 else 0)
        i = j
    return starts + [n], shared


def test_shared_prefix_groups_of_the_parallel_sampling_workload():
    """32 prompts x 8 samples (2056-token prompts): 32 groups of 8 sharing 128 blocks."""
    import workloads as W
    w = W.make_config(4, draw_values=False)
    p = _pool(w.num_blocks, w.block_size, w.free_order, prefix=False)
    for op in w.ops:
        if op[0] == "create":
            B.paged_kv_seq_create(p)
        elif op[0] == "fork":
            B.paged_kv_seq_fork(p, op[1])
        elif op[0] == "append":
            B.paged_kv_append_batch(p, op[1], op[2])
        elif op[0] == "attend":
            seqs = op[1]
    gs, sh, ms = B.paged_kv_shared_prefix_groups(p, seqs, 8, 16)
    assert list(gs) == list(range(0, 257, 8)) and list(sh) == [2048] * 32 and ms == 2048
    gs, sh, ms = B.paged_kv_shared_prefix_groups(p, seqs, 4, 16)       # groups cut at 4
    assert list(gs) == list(range(0, 257, 4)) and list(sh) == [2048] * 64
    gs, sh, ms = B.paged_kv_shared_prefix_groups(p, seqs, 8, 4096)     # more than is shared
    assert list(gs) == list(range(257)) and ms == 0
    B.paged_kv_pool_destroy(p)


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_shared_prefix_groups_match_the_rule_on_random_forests(bs):
    rng = random.Random(bs + 500)
    for trial in range(20):
        nb = 4000
        p = _pool(nb, bs, None, prefix=False)
        seqs = []
        for _ in range(rng.randrange(1, 6)):
            root = B.paged_kv_seq_create(p)
            B.paged_kv_seq_append(p, root, rng.randrange(0, 8 * bs + 5))
            fam = [root]
            for _ in range(rng.randrange(0, 6)):
                c = B.paged_kv_seq_fork(p, rng.choice(fam))
                B.paged_kv_seq_append(p, c, rng.randrange(0, 3 * bs))
                fam.append(c)
            for s in fam:
                if rng.random() < 0.5:
                    B.paged_kv_seq_append(p, s, rng.randrange(0, 2 * bs))
            seqs += fam
        rng.shuffle(seqs) if rng.random() < 0.3 else None
        seqs = [s for s in seqs if B.paged_kv_seq_info(p, s)[0] > 0] or [B.paged_kv_seq_create(p)]
        tables, lens = B.paged_kv_block_tables(p, seqs, None)
        rows = [[int(x) for x in t if x >= 0] for t in tables]
        for mg in (1, 2, 8):
            for need in (0, bs, 3 * bs):
                gs, sh, ms = B.paged_kv_shared_prefix_groups(p, seqs, mg, need)
                want_gs, want_sh = _groups_brute(rows, [int(x) for x in lens], bs, mg, need)
                assert list(gs) == want_gs and list(sh) == want_sh, (trial, mg, need)
                assert ms == max(want_sh)
                for g in range(len(sh)):           # the description the kernel relies on
                    members = range(gs[g], gs[g + 1])
                    nblk = -(-int(sh[g]) // bs)
                    assert all(rows[m][:nblk] == rows[gs[g]][:nblk] for m in members)
                    assert all(lens[m] >= sh[g] for m in members)
        B.paged_kv_pool_destroy(p)
