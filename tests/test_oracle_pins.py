"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against what the pages print, a closed form, an
invariant, brute force, or a library routine the problem reduces to in a
special case — never against a retyped copy of the oracle's own formula.
"""
import os
import random

import numpy as np
import pytest
import torch

from oracle import allocator as A
from oracle import attention as ATT
from oracle import kvbytes, lowp, pool as P, replay
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- KV bytes ----
def test_kv_bytes_printed_values():
    for ln in _golden_lines("kv_bytes_printed.txt"):
        layers, heads, dim, nbytes, tokens, reqs, expect = map(int, ln.split())
        assert kvbytes.kv_bytes(tokens * reqs, layers, heads, dim, nbytes) == expect


def test_kv_bytes_units_and_mha_ratio():
    per_tok = kvbytes.kv_bytes_per_token(80, 8, 128, 2)
    assert per_tok * 8192 == int(2.5 * 2**30)
    assert per_tok * 8192 * 100 == 250 * 2**30
    assert kvbytes.kv_bytes_per_token(80, 64, 128, 2) == 8 * per_tok
    assert abs(per_tok / 2**20 - 0.3125) < 1e-12       # "about 0.31 MB" on the page
    with pytest.raises(ValueError):
        kvbytes.kv_bytes_per_token(80, -1, 128, 2)


# ------------------------------------------------------------ low precision ----
def test_bf16_rounding_hand_cases():
    def bits(x):
        return int(lowp.f32_to_bf16_bits(np.array([x], dtype=np.float32))[0])
    assert bits(1.0) == 0x3F80
    assert bits(-2.0) == 0xC000
    assert bits(1.0 + 2.0**-8) == 0x3F80            # tie, kept pattern even -> down
    assert bits(1.0 + 3 * 2.0**-8) == 0x3F82        # tie, kept pattern odd -> up
    assert bits(1.0 + 2.0**-8 + 2.0**-20) == 0x3F81  # above the tie -> up
    assert bits(1.0 + 2.0**-9) == 0x3F80            # below the tie -> down
    assert bits(np.inf) == 0x7F80
    big = np.array([0x7F7FFFFF], dtype=np.uint32).view(np.float32)[0]
    assert bits(big) == 0x7F80                      # largest finite fp32 rounds to inf
    nan = lowp.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_bf16_upcast_exact():
    v = lowp.bf16_bits_to_f64(np.array([0x3F80, 0x4049, 0xC000, 0x0001], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == 3.140625 and v[2] == -2.0
    assert v[3] == 2.0**-133                          # smallest bf16 subnormal


def test_bf16_rounding_matches_library_cast():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200_000).astype(np.float32)
    # force exact ties and near-ties
    b = x.view(np.uint32).copy()
    b[:50_000] = (b[:50_000] & 0xFFFF0000) | 0x8000
    b[50_000:60_000] = (b[50_000:60_000] & 0xFFFF0000) | 0x7FFF
    b[60_000:70_000] = (b[60_000:70_000] & 0xFFFF0000) | 0x8001
    x = b.view(np.float32)
    ours = lowp.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_storage_round_trip_types():
    x = np.array([1.5, -0.25, 3.0e-3], dtype=np.float32)
    for dt in ("f32", "f16", "bf16"):
        back = lowp.storage_bits_to_f64(lowp.to_storage_bits(x, dt), dt)
        assert np.allclose(back, x, rtol=2**-8)
    assert np.array_equal(lowp.storage_bits_to_f64(lowp.to_storage_bits(x, "f32"), "f32"), x)
    f16 = lowp.to_storage_bits(np.array([1.0 + 2**-11], dtype=np.float32), "f16")
    assert int(f16[0]) == 0x3C00                      # fp16 tie rounds to even


# --------------------------------------------------------------- allocator ----
def _parse_worked_example():
    lines = _golden_lines("worked_example_bs4.txt")
    bs = int(lines[0].split()[1])
    head = [int(t) for t in lines[1].split()[1:]]
    steps = []
    for ln in lines[2:]:
        if "->" in ln:
            left, right = ln.split("->")
            n = int(left.split()[1])
            tab, slots = right.split(";")
            steps.append((n, [int(t) for t in tab.split()], [int(t) for t in slots.split()]))
    idle = int([ln for ln in lines if ln.startswith("idle_slots")][0].split()[1])
    return bs, head, steps, idle


def test_worked_example_block_size_4():
    bs, head, steps, idle = _parse_worked_example()
    order = head + [b for b in range(64) if b not in head]
    al = A.BlockAllocator(64, bs, order)
    s = al.create()
    for n, table, slots in steps:
        got_slots, copies = al.append(s, n)
        assert got_slots == slots and copies == []
        assert al.block_table(s) == table
    assert al.waste_slots() == idle
    assert al.context_len(s) == 6 and 100 - al.context_len(s) == 94
    # offsets inside the last block: "today" first slot, "!" second slot
    assert [x % bs for x in steps[-2][2] + steps[-1][2]] == [0, 1]


def test_logical_to_physical_example():
    lines = _golden_lines("logical_to_physical_64.txt")
    bs = int(lines[0].split()[1])
    n = int(lines[1].split()[1])
    table = [int(t) for t in lines[2].split()[1:]]
    checks = [tuple(map(int, ln.split()[1:])) for ln in lines[3:]]
    al = A.BlockAllocator(32, bs, table + [b for b in range(32) if b not in table])
    s = al.create()
    slots, _ = al.append(s, n)
    assert al.block_table(s) == table
    for pos, slot in checks:
        assert slots[pos] == slot


def test_reservation_waste_example():
    lines = _golden_lines("reservation_waste.txt")
    reserved, used, idle = (int(lines[0].split()[i]) for i in (1, 3, 5))
    bs, blocks, nslots, pidle = (int(lines[1].split()[i]) for i in (1, 3, 5, 7))
    assert reserved - used == idle
    al = A.BlockAllocator(64, bs)
    s = al.create()
    al.append(s, used)
    assert len(al.block_table(s)) == blocks
    assert bs * blocks == nslots and al.waste_slots() == pidle


def _random_ops(rng, al, steps, max_n=40):
    live = []
    for _ in range(steps):
        r = rng.random()
        if r < 0.15 or not live:
            live.append(al.create())
        elif r < 0.25:
            live.append(al.fork(rng.choice(live)))
        elif r < 0.35 and len(live) > 1:
            s = rng.choice(live)
            live.remove(s)
            al.release(s)
        else:
            s = rng.choice(live)
            n = rng.randint(0, max_n)
            if al.blocks_needed(s, n) <= al.num_free():
                yield s, al.append(s, n)
    return


def test_waste_below_one_block_and_block_count():
    rng = random.Random(1)
    for bs in (1, 4, 16):
        al = A.BlockAllocator(4000, bs, list(range(4000)))
        for _ in _random_ops(rng, al, 400):
            for s, t in al.tables.items():
                L = al.lengths[s]
                assert len(t) == -(-L // bs)
                assert 0 <= bs * len(t) - L <= bs - 1


def test_refcount_invariants_and_full_release():
    rng = random.Random(2)
    nb = 3000
    al = A.BlockAllocator(nb, 16, np.random.default_rng(0).permutation(nb))
    for _ in _random_ops(rng, al, 600):
        used = {b for t in al.tables.values() for b in t}
        assert sum(al.refcount) == sum(len(t) for t in al.tables.values())
        assert al.num_free() + len(used) == nb
        assert all(al.refcount[b] == 0 for b in al.free)
        assert len(set(al.free)) == len(al.free)
    for s in list(al.tables):
        al.release(s)
    assert al.num_free() == nb and sum(al.refcount) == 0


def test_reading_back_through_tables_gives_each_sequence_its_tokens():
    """Brute force: tag every written token, replay copy-on-write on a slot->tag
    map, and check that every live sequence reads back exactly its own history."""
    rng = random.Random(3)
    bs, nb = 4, 2000
    al = A.BlockAllocator(nb, bs, np.random.default_rng(1).permutation(nb))
    content = {}                      # slot -> tag
    history = {}                      # seq -> list of tags, logical order
    tag = 0
    live = []
    for _ in range(700):
        r = rng.random()
        if r < 0.1 or not live:
            s = al.create()
            history[s] = []
            live.append(s)
        elif r < 0.25:
            p = rng.choice(live)
            s = al.fork(p)
            history[s] = list(history[p])
            live.append(s)
        elif r < 0.3 and len(live) > 1:
            s = rng.choice(live)
            live.remove(s)
            al.release(s)
            del history[s]
        else:
            s = rng.choice(live)
            n = rng.randint(1, 9)
            if al.blocks_needed(s, n) > al.num_free():
                continue
            slots, copies = al.append(s, n)
            for src, dst in copies:
                for o in range(bs):
                    if src * bs + o in content:
                        content[dst * bs + o] = content[src * bs + o]
            for sl in slots:
                content[sl] = tag
                history[s].append(tag)
                tag += 1
        for q in live:
            t = al.block_table(q)
            got = [content.get(t[p // bs] * bs + p % bs) for p in range(al.context_len(q))]
            assert got == history[q]


def test_out_of_blocks_changes_nothing():
    al = A.BlockAllocator(3, 16, [2, 0, 1])
    s = al.create()
    al.append(s, 20)                   # blocks 2, 0; block 1 left
    snap = (list(al.free), list(al.refcount), al.block_table(s), al.context_len(s))
    with pytest.raises(A.OutOfBlocks):
        al.append(s, 40)               # would open 2 more blocks, 1 free
    assert snap == (list(al.free), list(al.refcount), al.block_table(s), al.context_len(s))
    t = al.fork(s)                     # tail block 0 now shared
    slots, copies = al.append(s, 12)   # s copies the shared tail into block 1
    assert copies == [(0, 1)] and al.block_table(s) == [2, 1] and al.num_free() == 0
    al.append(t, 1)                    # t is the last holder of block 0: writes in place
    snap = (list(al.free), list(al.refcount), al.block_table(t), al.context_len(t))
    with pytest.raises(A.OutOfBlocks):
        al.append(t, 12)               # reaches position 32: needs a block, none left
    assert snap == (list(al.free), list(al.refcount), al.block_table(t), al.context_len(t))


def test_free_queue_is_fifo():
    al = A.BlockAllocator(8, 2, [5, 3, 7, 1, 0, 2, 4, 6])
    a = al.create()
    al.append(a, 4)                    # blocks 5, 3
    b = al.create()
    al.append(b, 2)                    # block 7
    al.release(a)                      # 5 then 3 go to the tail
    c = al.create()
    al.append(c, 12)                   # 1, 0, 2, 4, 6, then the released 5
    assert al.block_table(c) == [1, 0, 2, 4, 6, 5]
    al.append(c, 2)
    assert al.block_table(c)[-1] == 3


def test_copy_on_write_counts_shared_prefix():
    for plen, expect in ((2056, 7), (2048, 0)):
        al = A.BlockAllocator(1000, 16)
        s0 = al.create()
        al.append(s0, plen)
        group = [s0] + [al.fork(s0) for _ in range(7)]
        assert all(al.refcount[b] == 8 for b in al.block_table(s0))
        pairs = []
        for s in group:
            pairs += al.append(s, 5)[1]
        assert len(pairs) == expect
        full = plen // 16
        assert all(al.refcount[b] == 8 for b in al.block_table(s0)[:full])
        tails = {al.block_table(s)[full] for s in group}
        assert len(tails) == 8


# ------------------------------------------------------------------- pool ----
@pytest.mark.parametrize("bs", [4, 1, 32])
def test_pool_layout_element_by_element(bs):
    """The ABI layout, element by element: a block of more than 16 tokens is 16-token
    sub-blocks one after the other, each laid out like a 16-token block."""
    rng = np.random.default_rng(4 + bs)
    tb = min(bs, 16)
    ns = bs // tb
    for dt, d in (("f32", 8), ("bf16", 16), ("f16", 32)):
        nb, hkv = (5 if bs > 1 else 12), 3
        x = P.chunk_elems(dt)
        kp, vp = P.new_pool(nb, hkv, bs, d, dt)
        T = 7
        slots = rng.choice(nb * bs, size=T, replace=False)
        kbits = lowp.to_storage_bits(rng.standard_normal((T, hkv, d)).astype(np.float32), dt)
        vbits = lowp.to_storage_bits(rng.standard_normal((T, hkv, d)).astype(np.float32), dt)
        P.reshape_and_cache(kp, vp, kbits, vbits, slots, bs)
        flat_k, flat_v = kp.reshape(-1), vp.reshape(-1)
        written_k, written_v = set(), set()
        for t in range(T):
            b, o = divmod(int(slots[t]), bs)
            sub, o = divmod(o, tb)
            for h in range(hkv):
                for e in range(d):
                    r = (b * hkv + h) * ns + sub
                    ik = ((r * (d // x) + e // x) * tb + o) * x + e % x
                    iv = (r * d + e) * tb + o
                    assert flat_k[ik] == kbits[t, h, e]
                    assert flat_v[iv] == vbits[t, h, e]
                    written_k.add(ik)
                    written_v.add(iv)
        poison = lowp.poison_bits(dt)
        rest_k = np.ones(flat_k.size, bool)
        rest_k[list(written_k)] = False
        rest_v = np.ones(flat_v.size, bool)
        rest_v[list(written_v)] = False
        assert np.all(flat_k[rest_k] == poison) and np.all(flat_v[rest_v] == poison)


def test_block_of_32_is_two_blocks_of_16_side_by_side():
    """Per KV head, a 32-token-block pool holds the bytes of a 16-token-block pool whose
    blocks 2b and 2b + 1 are block b's two halves: the same slot numbers land in the
    same places, and reading back through either table gives the same tokens."""
    rng = np.random.default_rng(12)
    nb, hkv, d, dt = 6, 2, 16, "bf16"
    k32, v32 = P.new_pool(nb, hkv, 32, d, dt)
    k16, v16 = P.new_pool(2 * nb, hkv, 16, d, dt)
    T = 90
    slots = rng.choice(nb * 32, size=T, replace=False)
    kbits = lowp.to_storage_bits(rng.standard_normal((T, hkv, d)).astype(np.float32), dt)
    vbits = lowp.to_storage_bits(rng.standard_normal((T, hkv, d)).astype(np.float32), dt)
    P.reshape_and_cache(k32, v32, kbits, vbits, slots, 32)
    P.reshape_and_cache(k16, v16, kbits, vbits, slots, 16)
    for h in range(hkv):
        assert np.array_equal(k32[:, h].reshape(-1), k16[:, h].reshape(nb, -1).reshape(-1))
        assert np.array_equal(v32[:, h].reshape(-1), v16[:, h].reshape(nb, -1).reshape(-1))
    full = np.arange(nb * 32)
    kall = lowp.to_storage_bits(rng.standard_normal((nb * 32, hkv, d)).astype(np.float32), dt)
    vall = lowp.to_storage_bits(rng.standard_normal((nb * 32, hkv, d)).astype(np.float32), dt)
    P.reshape_and_cache(k32, v32, kall, vall, full, 32)
    table32 = rng.permutation(nb)
    table16 = np.stack([2 * table32, 2 * table32 + 1], 1).reshape(-1)
    n = nb * 32 - 5
    ka, va = P.gather_sequence(k32, v32, table32, n, 32)
    order = (table32[np.arange(n) // 32] * 32 + np.arange(n) % 32)
    assert np.array_equal(ka, kall[order]) and np.array_equal(va, vall[order])
    P.reshape_and_cache(k16, v16, kall, vall, full, 16)
    kb, vb = P.gather_sequence(k16, v16, table16, n, 16)
    assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_padding_slot_is_skipped_and_copy_is_exact():
    kp, vp = P.new_pool(4, 2, 16, 64, "bf16")
    k = lowp.to_storage_bits(np.ones((2, 2, 64), np.float32), "bf16")
    P.reshape_and_cache(kp, vp, k, k, [-1, 17], 16)
    assert np.all(kp[0] == lowp.poison_bits("bf16"))
    P.copy_block(kp, vp, 1, 3)
    assert np.array_equal(kp[3], kp[1]) and np.array_equal(vp[3], vp[1])


# -------------------------------------------------------------- attention ----
def _dense_via_library(q, k, v, scale):
    """torch SDPA in float64 on the CPU, KV heads repeated for GQA, no block table."""
    hq, hkv = q.shape[0], k.shape[1]
    kk = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2)   # [Hq][L][d]
    vv = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q)[:, None, :]                                        # [Hq][1][d]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk.contiguous(), vv.contiguous(),
                                                         scale=float(scale))
    return o[:, 0, :].numpy()


def _fill(rng, dt, lens, hq, hkv, d, bs=16, nb=None, perm=None):
    nb = nb or sum(-(-L // bs) for L in lens) + 3
    order = perm if perm is not None else rng.permutation(nb)
    al = A.BlockAllocator(nb, bs, order)
    kp, vp = P.new_pool(nb, hkv, bs, d, dt)
    ks, vs = [], []
    for L in lens:
        s = al.create()
        slots, _ = al.append(s, L)
        kb = lowp.to_storage_bits(rng.standard_normal((L, hkv, d)).astype(np.float32), dt)
        vb = lowp.to_storage_bits(rng.standard_normal((L, hkv, d)).astype(np.float32), dt)
        P.reshape_and_cache(kp, vp, kb, vb, slots, bs)
        ks.append(lowp.storage_bits_to_f64(kb, dt))
        vs.append(lowp.storage_bits_to_f64(vb, dt))
    tables = replay.padded_tables(al, list(range(len(lens))))
    return al, kp, vp, tables, ks, vs


@pytest.mark.parametrize("dt,hq,hkv,d", [("f32", 4, 4, 64), ("bf16", 8, 2, 64), ("f16", 6, 3, 8),
                                          ("bf16", 4, 1, 8), ("f32", 2, 1, 4)])
def test_paged_matches_library_dense_attention(dt, hq, hkv, d):
    rng = np.random.default_rng(6)
    lens = [1, 7, 16, 17, 40]
    al, kp, vp, tables, ks, vs = _fill(rng, dt, lens, hq, hkv, d)
    q = rng.standard_normal((len(lens), hq, d))
    scale = np.float32(1 / np.sqrt(d))
    out = ATT.paged_decode(q, kp, vp, tables, lens, scale, dt, 16)
    for b in range(len(lens)):
        ref = _dense_via_library(q[b], ks[b], vs[b], scale)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(7)
    d, hkv = 8, 2
    # one token: the output is that token's value exactly
    k = rng.standard_normal((1, hkv, d)); v = rng.standard_normal((1, hkv, d))
    q = rng.standard_normal((4, d))
    out = ATT.dense_decode(q, k, v, 0.3)
    assert np.array_equal(out, np.repeat(v[0], 2, axis=0))
    # zero query or zero scale: the mean of the values
    k = rng.standard_normal((9, hkv, d)); v = rng.standard_normal((9, hkv, d))
    np.testing.assert_allclose(ATT.dense_decode(np.zeros((4, d)), k, v, 0.3),
                               np.repeat(v.mean(0), 2, axis=0), atol=1e-14)
    np.testing.assert_allclose(ATT.dense_decode(q, k, v, 0.0), np.repeat(v.mean(0), 2, axis=0),
                               atol=1e-14)
    # identical keys: the mean of the values
    kk = np.repeat(k[:1], 9, axis=0)
    np.testing.assert_allclose(ATT.dense_decode(q, kk, v, 0.3), np.repeat(v.mean(0), 2, axis=0),
                               atol=1e-14)
    # identical values: that value
    vv = np.repeat(v[:1], 9, axis=0)
    np.testing.assert_allclose(ATT.dense_decode(q, k, vv, 0.3), np.repeat(v[0], 2, axis=0),
                               atol=1e-14)
    # one score far above the rest: that token's value
    qd = np.zeros((4, d)); qd[:, 0] = 1.0
    kd = np.zeros((9, hkv, d)); kd[5, :, 0] = 1e4
    np.testing.assert_allclose(ATT.dense_decode(qd, kd, v, 1.0), np.repeat(v[5], 2, axis=0),
                               atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(8)
    d, hq, hkv, L = 16, 8, 2, 23
    k = rng.standard_normal((L, hkv, d)); v = rng.standard_normal((L, hkv, d))
    q = rng.standard_normal((hq, d))
    gqa = ATT.dense_decode(q, k, v, 0.25)
    mha = ATT.dense_decode(q, np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1),
                           0.25)
    assert np.array_equal(gqa, mha)
    # and each query head of group g attends over KV head g only
    for h in range(hq):
        single = ATT.dense_decode(q[h:h + 1], k[:, h // 4:h // 4 + 1], v[:, h // 4:h // 4 + 1], 0.25)
        assert np.array_equal(single[0], gqa[h])


def test_placement_invariance():
    lens = [5, 16, 33, 70]
    outs = []
    for seed in (0, 1, 2):
        rng = np.random.default_rng(9)                      # same values every time
        nb = 20
        perm = np.random.default_rng(100 + seed).permutation(nb)
        al, kp, vp, tables, _, _ = _fill(rng, "bf16", lens, 4, 2, 32, nb=nb, perm=perm)
        q = np.random.default_rng(10).standard_normal((len(lens), 4, 32))
        outs.append(ATT.paged_decode(q, kp, vp, tables, lens, np.float32(0.17), "bf16", 16))
        if seed:
            assert not np.array_equal(tables, prev_tables)
        prev_tables = tables
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_and_copied_prefix_give_identical_outputs():
    shared, copied = W.configs.make_shared_prefix_pair(small=True)
    rs = replay.run(shared, attend_rows=[0, 5, 8, 15])
    rc = replay.run(copied, attend_rows=[0, 5, 8, 15])
    assert sum(len(c) for c in rs.copies) == 2 * 7
    assert sum(len(c) for c in rc.copies) == 0
    a, b = rs.outputs[0], rc.outputs[0]
    rows = [0, 5, 8, 15]
    assert np.array_equal(a[rows], b[rows])
    assert rs.allocator.num_used() < rc.allocator.num_used()


def test_lse_merge_equals_one_shot():
    rng = np.random.default_rng(11)
    z = rng.standard_normal(1000) * 3
    v = rng.standard_normal((1000, 16))
    w = np.exp(z - z.max())
    one = (w @ v) / w.sum()
    for cuts in ([500], [16 * i for i in range(1, 62)], [1, 2, 999], list(range(1, 1000))):
        edges = [0] + cuts + [1000]
        states = [ATT.partial_state(z[a:b], v[a:b]) for a, b in zip(edges, edges[1:])]
        np.testing.assert_allclose(ATT.lse_merge(states), one, rtol=1e-12, atol=1e-13)


def test_context_len_zero_rejected():
    kp, vp = P.new_pool(2, 1, 16, 8, "f32")
    with pytest.raises(ValueError):
        ATT.paged_decode(np.zeros((1, 1, 8)), kp, vp, np.array([[0]]), [0], 1.0, "f32", 16)


# ------------------------------------------------------- planted mistakes ----
def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible oracle mistake is planted here, on the CPU, and one of the
    pins above must notice it."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((8, 16)); k = rng.standard_normal((11, 2, 16))
    v = rng.standard_normal((11, 2, 16))
    good = ATT.dense_decode(q, k, v, 0.25)

    def wrong_group(q, k, v, scale):   # query head h -> KV head h % Hkv
        out = np.empty_like(q)
        for h in range(q.shape[0]):
            g = h % k.shape[1]
            z = scale * (k[:, g] @ q[h]); w = np.exp(z - z.max())
            out[h] = (w @ v[:, g]) / w.sum()
        return out
    mha = ATT.dense_decode(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.25)
    assert not np.allclose(wrong_group(q, k, v, 0.25), mha)
    assert np.allclose(good, mha)

    def no_scale(q, k, v, scale):
        return ATT.dense_decode(q, k, v, 1.0)
    lib = _dense_via_library(q, k, v, 0.25)
    assert not np.allclose(no_scale(q, k, v, 0.25), lib)

    # V stored token-major instead of dim-major: the layout brute force fails
    kp, vp = P.new_pool(2, 1, 4, 8, "f32")
    vb = lowp.to_storage_bits(np.arange(8, dtype=np.float32).reshape(1, 1, 8), "f32")
    P.reshape_and_cache(kp, vp, vb, vb, [5], 4)
    wrong_flat = vp.reshape(-1)[((1 * 1 + 0) * 4 + 1) * 8 + np.arange(8)]
    right_flat = vp.reshape(-1)[((1 * 1 + 0) * 8 + np.arange(8)) * 4 + 1]
    assert np.array_equal(right_flat, vb[0, 0]) and not np.array_equal(wrong_flat, vb[0, 0])

    # released blocks pushed at the head instead of the tail: FIFO pin fails
    class HeadFree(A.BlockAllocator):
        def release(self, seq):
            for b in reversed(self.tables.pop(seq)):
                self.refcount[b] -= 1
                if self.refcount[b] == 0:
                    self.free.appendleft(b)
            del self.lengths[seq]
    al = HeadFree(8, 2, [5, 3, 7, 1, 0, 2, 4, 6])
    a = al.create(); al.append(a, 4); b = al.create(); al.append(b, 2); al.release(a)
    c = al.create(); al.append(c, 12)
    assert al.block_table(c) != [1, 0, 2, 4, 6, 5]

    # copy-on-write skipped: reading back through the tables fails
    class NoCow(A.BlockAllocator):
        def blocks_needed(self, seq, n):
            L = self.lengths[seq]
            return sum(1 for p in range(L, L + n) if p % self.block_size == 0)

        def append(self, seq, n):
            slots = []
            for _ in range(n):
                p = self.lengths[seq]
                if p % self.block_size == 0:
                    blk = self.free.popleft(); self.refcount[blk] = 1; self.tables[seq].append(blk)
                slots.append(self.tables[seq][p // self.block_size] * self.block_size
                             + p % self.block_size)
                self.lengths[seq] = p + 1
            return slots, []
    al = NoCow(10, 4)
    s = al.create(); al.append(s, 2); t = al.fork(s)
    s_slots, _ = al.append(s, 1); t_slots, _ = al.append(t, 1)
    assert s_slots == t_slots          # both wrote the same physical slot: history lost
