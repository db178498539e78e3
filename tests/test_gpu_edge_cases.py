"""Edge cases and invariances of the HIP path (GPU), checked against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as oreplay
from oracle import lowp
from gpu_common import (TOL, say, assert_pools_equal, assert_bookkeeping_equal, max_err, out_f64,
                        assert_close)

pytestmark = pytest.mark.gpu

BOUNDARY_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1024, 1025, 1100]

# (dtype, q heads, kv heads, head_dim): VALU path (group 1, and fp32) and MFMA path
SHAPES = [("f32", 4, 4, 64), ("f32", 8, 2, 128), ("f16", 4, 4, 128), ("bf16", 2, 2, 64),
          ("bf16", 16, 2, 128), ("f16", 8, 4, 128), ("bf16", 8, 2, 64), ("bf16", 32, 2, 128),
          ("f16", 12, 4, 64)]


def _run(w, out_dtype="f32", pt=None):
    from paged_kv_cache_15_amd.replay import run_workload
    g = run_workload(w, "cuda", out_dtype=out_dtype, partition_tokens=pt)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("pt", [0, 512], ids=["streamk", "pt512"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_boundary_lengths_every_path(shape, pt):
    dt, hq, hkv, d = shape
    w = W.make_custom(BOUNDARY_LENS, hq, hkv, d, dt, seed=hq * 7 + d)
    say(f"[edge] boundary lengths {shape} partition_tokens={pt}")
    for out_dtype in ("f32", dt):
        g = _run(w, out_dtype, pt)
        o = oreplay.run(w)
        assert_bookkeeping_equal(g, o)
        assert_pools_equal(g.cache, o, dt)
        err = assert_close(g.outputs[0], o.outputs[0], dt, out_dtype)
        say(f"   out={out_dtype} max|err| {err:.3e}")
        g.cache.close()


@pytest.mark.parametrize("shape", SHAPES[:6], ids=lambda s: "-".join(map(str, s)))
def test_single_token_returns_its_value_exactly(shape):
    dt, hq, hkv, d = shape
    w = W.make_custom([1, 1, 1], hq, hkv, d, dt, seed=3)
    g = _run(w, "f32")
    k, v = w.kv[-1]
    vb = lowp.storage_bits_to_f64(lowp.to_storage_bits(v, dt), dt)   # [3][hkv][d]
    expect = np.repeat(vb, hq // hkv, axis=1)
    assert np.array_equal(out_f64(g.outputs[0]), expect)
    g.cache.close()


@pytest.mark.parametrize("dt,hq,hkv", [("bf16", 64, 8), ("f16", 32, 32), ("f32", 4, 4)])
def test_partition_size_invariance(dt, hq, hkv):
    w = W.make_custom([5, 700, 1500, 2049], hq, hkv, 128 if dt != "f32" else 64, dt, seed=11)
    o = oreplay.run(w)
    outs = []
    for pt in (16, 48, 512, 4096, 0):
        g = _run(w, "f32", pt)
        err = max_err(g.outputs[0], o.outputs[0])
        say(f"[edge] partition {pt}: max|err| {err:.3e}")
        assert err <= TOL[dt]
        outs.append(out_f64(g.outputs[0]))
        g.cache.close()
    for x in outs[1:]:
        assert np.abs(x - outs[0]).max() <= TOL[dt]


@pytest.mark.parametrize("pt", [0, 512], ids=["streamk", "pt512"])
@pytest.mark.parametrize("dt,hq,hkv", [("bf16", 64, 8), ("f16", 32, 32), ("f32", 4, 4)])
def test_placement_invariance_bitwise(dt, hq, hkv, pt):
    d = 128 if dt != "f32" else 64
    base = W.make_custom([300, 1000, 17, 2500], hq, hkv, d, dt, seed=21)
    outs = []
    for perm_seed in (0, 1, 2):
        w = W.make_custom([300, 1000, 17, 2500], hq, hkv, d, dt, seed=21,
                          free_order=np.random.default_rng(50 + perm_seed).permutation(base.num_blocks))
        g = _run(w, "f32", pt)
        outs.append((out_f64(g.outputs[0]), g.tables[0]))
        g.cache.close()
    assert not np.array_equal(outs[0][1], outs[1][1])
    for o, _ in outs[1:]:
        assert np.array_equal(o, outs[0][0])


@pytest.mark.parametrize("pt", [0, 512], ids=["streamk", "pt512"])
def test_shared_and_copied_prefix_bitwise(pt):
    shared, copied = W.configs.make_shared_prefix_pair(small=True)
    gs = _run(shared, "f32", pt)
    gc = _run(copied, "f32", pt)
    assert sum(len(c) for c in gs.copies) == 2 * 7
    assert sum(len(c) for c in gc.copies) == 0
    assert np.array_equal(out_f64(gs.outputs[0]), out_f64(gc.outputs[0]))
    os_ = oreplay.run(shared)
    assert_pools_equal(gs.cache, os_, "bf16")
    assert max_err(gs.outputs[0], os_.outputs[0]) <= TOL["bf16"]
    fs, us, _ = gs.cache.stats()
    fc, uc, _ = gc.cache.stats()
    assert us < uc
    gs.cache.close()
    gc.cache.close()


def test_gqa_matches_replicated_mha():
    gqa = W.make_custom([40, 600, 1300], 16, 2, 128, "bf16", seed=31)
    mha = W.make_custom([40, 600, 1300], 16, 16, 128, "bf16", seed=31)
    # same draws, KV heads repeated 8x for the MHA twin
    mha.kv = [(np.repeat(k, 8, axis=1), np.repeat(v, 8, axis=1)) for k, v in gqa.kv]
    mha.q = gqa.q
    mha.num_blocks = gqa.num_blocks
    mha.free_order = gqa.free_order
    a = _run(gqa, "f32")
    b = _run(mha, "f32")
    assert np.abs(out_f64(a.outputs[0]) - out_f64(b.outputs[0])).max() <= TOL["bf16"]
    a.cache.close()
    b.cache.close()


def test_invalid_lengths_and_block_ids_give_nan_without_reading():
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.replay import run_workload
    for dt, hq, hkv, d in [("bf16", 16, 2, 128), ("f16", 4, 4, 128), ("f32", 4, 4, 64)]:
        w = W.make_custom([100, 700, 30, 1200], hq, hkv, d, dt, seed=41)
        g = run_workload(w, "cuda", out_dtype="f32")
        o = oreplay.run(w)
        c = g.cache
        tables = g.tables[0].copy()
        lens = g.context_lens[0].copy()
        tables[1, 3] = c.desc.num_blocks + 5       # past the pool
        tables[3, 0] = -7                          # negative id
        lens[2] = 0                                # empty context
        max_ctx = 1200
        mb = tables.shape[1]
        lens_d = torch.from_numpy(lens).cuda()
        tab_d = torch.from_numpy(tables).cuda()
        from paged_kv_cache_15_amd.cache import TORCH_DTYPES
        q = torch.from_numpy(w.q[0]).cuda().to(TORCH_DTYPES[dt])
        out = torch.zeros((4, hq, d), device="cuda")
        for pt in (512, 2048, 0):
            nb = B.paged_attention_workspace_bytes(c.desc, 4, hq, max_ctx, pt)
            ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
            B.paged_attention_decode(c.desc, out, "f32", q, c.k_pool, c.v_pool, tab_d, lens_d, hq,
                                     max_ctx, float(w.scale), pt, ws)
            torch.cuda.synchronize()
            r = out_f64(out)
            assert np.isnan(r[1]).all() and np.isnan(r[2]).all() and np.isnan(r[3]).all()
            assert np.abs(r[0] - o.outputs[0][0]).max() <= TOL[dt]
        # a context longer than max_context_len is rejected the same way
        lens2 = g.context_lens[0].copy()
        lens_d2 = torch.from_numpy(lens2).cuda()
        for pt in (512, 0):
            nb = B.paged_attention_workspace_bytes(c.desc, 4, hq, 1000, pt)
            ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
            B.paged_attention_decode(c.desc, out, "f32", q, c.k_pool, c.v_pool,
                                     torch.from_numpy(g.tables[0]).cuda(), lens_d2, hq, 1000,
                                     float(w.scale), pt, ws)
            torch.cuda.synchronize()
            r = out_f64(out)
            assert np.isnan(r[3]).all() and not np.isnan(r[:3]).any()
        c.close()


def test_padding_and_out_of_range_slots_are_not_written():
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache
    c = PagedKVCache(8, 2, 64, "bf16")
    key = torch.randn(4, 2, 64, device="cuda").to(torch.bfloat16)
    val = torch.randn(4, 2, 64, device="cuda").to(torch.bfloat16)
    slots = torch.tensor([-1, 5, 8 * 16, 17], dtype=torch.int32, device="cuda")
    B.reshape_and_cache(c.desc, key, val, c.k_pool, c.v_pool, slots)
    pairs = torch.tensor([[1, 3], [9, 2], [1, -1]], dtype=torch.int32, device="cuda")
    B.paged_kv_copy_blocks(c.desc, c.k_pool, c.v_pool, pairs, 3)
    torch.cuda.synchronize()
    kb = c.k_pool.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = c.v_pool.view(torch.int16).cpu().numpy().view(np.uint16)
    kk = key.view(torch.int16).cpu().numpy().view(np.uint16)
    vv = val.view(torch.int16).cpu().numpy().view(np.uint16)
    poison = np.uint16(0xFFFF)
    # slot 5 -> block 0 offset 5; slot 17 -> block 1 offset 1 (then copied to block 3)
    assert np.array_equal(kb[0, :, :, 5, :].reshape(2, 64), kk[1])
    assert np.array_equal(vb[0, :, :, 5], vv[1])
    assert np.array_equal(kb[1, :, :, 1, :].reshape(2, 64), kk[3])
    assert np.array_equal(kb[3], kb[1]) and np.array_equal(vb[3], vb[1])
    written = np.zeros(kb.shape[:1] + (kb.shape[3],), bool)
    written[0, 5] = written[1, 1] = written[3, 1] = True
    for b in range(8):
        for o in range(16):
            if not written[b, o]:
                assert np.all(kb[b, :, :, o, :] == poison) and np.all(vb[b, :, :, o] == poison)
    c.close()


def test_empty_batches_launch_nothing():
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache
    c = PagedKVCache(8, 2, 64, "f16")
    e = torch.empty((0, 2, 64), dtype=torch.float16, device="cuda")
    B.reshape_and_cache(c.desc, e, e, c.k_pool, c.v_pool, torch.empty(0, dtype=torch.int32, device="cuda"))
    B.paged_kv_copy_blocks(c.desc, c.k_pool, c.v_pool, torch.empty((0, 2), dtype=torch.int32, device="cuda"), 0)
    out = torch.empty((0, 4, 64), device="cuda")
    B.paged_attention_decode(c.desc, out, "f32", torch.empty((0, 4, 64), dtype=torch.float16, device="cuda"),
                             c.k_pool, c.v_pool, torch.empty((0, 1), dtype=torch.int32, device="cuda"),
                             torch.empty(0, dtype=torch.int32, device="cuda"), 4, 16, 0.1)
    torch.cuda.synchronize()
    assert np.all(c.k_pool.view(torch.int16).cpu().numpy() == -1)
    c.close()


def test_decode_steps_append_and_attend():
    """Config-5 shape in small: eight consecutive steps, each one token per sequence."""
    w = W.make_config(5, small=True)
    g = _run(w, "bf16")
    o = oreplay.run(w)
    assert len(g.outputs) == 8
    assert_bookkeeping_equal(g, o)
    assert_pools_equal(g.cache, o, "bf16")
    for go, oo in zip(g.outputs, o.outputs):
        assert_close(go, oo, "bf16", "bf16")
    g.cache.close()


@pytest.mark.parametrize("pt", [0, 512], ids=["streamk", "pt512"])
def test_preempt_and_readmit_bitwise(pt):
    """Preemption ([DS] §2.5): a sequence is released mid-decode, its blocks go back to
    the free queue and are handed out again, and on re-admission its whole history is
    written again (the prefill redone) into whatever blocks the queue gives.  The new
    table has the same shape, the pool holds the same K/V for it, and attention over the
    same batch is bit-identical to before the preemption (the result depends on logical
    positions only), and matches the oracle."""
    from paged_kv_cache_15_amd.cache import PagedKVCache
    from paged_kv_cache_15_amd.replay import to_device
    from oracle.attention import paged_decode
    from oracle.pool import new_pool, reshape_and_cache
    rng = np.random.default_rng(53)
    hq, hkv, d, dt, bs = 32, 8, 128, "bf16", 16
    lens = [700, 1300, 2100, 90]
    victim = 2
    nb = sum((n + 8) // bs + 2 for n in lens) + 200
    c = PagedKVCache(nb, hkv, d, dt, bs, rng.permutation(nb).astype(np.int32))
    seqs = [c.create() for _ in lens]
    rows = [rng.standard_normal((2, n, hkv, d)).astype(np.float32) for n in lens]
    kd = to_device(np.concatenate([r[0] for r in rows]), dt, "cuda")
    vd = to_device(np.concatenate([r[1] for r in rows]), dt, "cuda")
    c.append(seqs, lens, kd, vd)
    hist = [list(r) for r in rows]            # each sequence's K and V rows so far
    for step in range(3):                      # decode steps: one token per sequence
        new = rng.standard_normal((2, len(lens), hkv, d)).astype(np.float32)
        c.append(seqs, [1] * len(lens), to_device(new[0], dt, "cuda"), to_device(new[1], dt, "cuda"))
        for i in range(len(lens)):
            hist[i][0] = np.concatenate([hist[i][0], new[0][i:i + 1]])
            hist[i][1] = np.concatenate([hist[i][1], new[1][i:i + 1]])
    q = to_device(rng.standard_normal((len(lens), hq, d)).astype(np.float32), dt, "cuda")
    before, tab0, len0 = c.attend(seqs, q, 0.088, "f32", pt, out_fill=float("nan"))
    torch.cuda.synchronize()
    free0 = c.stats()[0]
    c.free(seqs[victim])                       # preempted: every block released
    assert c.stats()[0] == free0 + int((tab0[victim] >= 0).sum())
    other = c.create()                         # meanwhile another request takes blocks
    filler = rng.standard_normal((2, 300, hkv, d)).astype(np.float32)
    c.append([other], [300], to_device(filler[0], dt, "cuda"), to_device(filler[1], dt, "cuda"))
    again = c.create()                         # re-admitted: its history written again
    n_hist = hist[victim][0].shape[0]
    c.append([again], [n_hist], to_device(hist[victim][0], dt, "cuda"),
             to_device(hist[victim][1], dt, "cuda"))
    seqs2 = list(seqs)
    seqs2[victim] = again
    after, tab1, len1 = c.attend(seqs2, q, 0.088, "f32", pt, out_fill=float("nan"))
    torch.cuda.synchronize()
    assert np.array_equal(len0, len1)
    assert np.array_equal(tab0 >= 0, tab1 >= 0)          # same table shape
    assert not np.array_equal(tab0[victim], tab1[victim])  # other physical blocks
    assert torch.equal(before, after)
    # the oracle, from the re-admitted tables and a pool written from the host rows
    kpool, vpool = new_pool(nb, hkv, bs, d, dt)
    for i, sq in enumerate(seqs2):
        blocks = tab1[i][tab1[i] >= 0]
        slots = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)[:len1[i]]
        reshape_and_cache(kpool, vpool, lowp.to_storage_bits(hist[i][0], dt),
                          lowp.to_storage_bits(hist[i][1], dt), slots.tolist(), bs)
    qf = lowp.storage_bits_to_f64(lowp.to_storage_bits(q.float().cpu().numpy(), dt), dt)
    want = paged_decode(qf, kpool, vpool, tab1, len1, np.float32(0.088), dt, bs)
    assert max_err(after, want) <= TOL[dt]
    c.close()


@pytest.mark.parametrize("pt", [0, 512], ids=["streamk", "pt512"])
def test_workspace_reused_across_calls_bitwise(pt):
    """Stream-K merge counters sit at the start of the workspace and every call must
    leave them at zero (fixed partitions keep no state across calls): one zero-filled
    workspace reused across calls with different batches gives the same bits as a fresh
    zero-filled workspace per call, as long as no batch has more sequences than one
    before it since the last zero-fill (the documented rule; the shared workspace is
    zero-filled again before the second round, which starts with the largest batch)."""
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.replay import to_device
    lens = [300, 1000, 17, 2500, 64, 4000, 1]
    w = W.make_custom(lens, 64, 8, 128, "bf16", seed=31)
    g = _run(w, "f32", pt)
    cache = g.cache
    seqs, qidx = w.attend_ops()[-1][1], w.attend_ops()[-1][2]
    q_all = to_device(w.q[qidx], w.dtype, "cuda")
    batches = [list(range(len(lens))), [5, 4, 3, 2, 1, 0], [1, 3, 5], [2, 6], [0]]

    def args(rows):
        tables, blens = cache.block_tables([seqs[i] for i in rows])
        return (torch.from_numpy(tables).cuda(), torch.from_numpy(blens).cuda(),
                int(blens.max()), q_all[rows].contiguous())

    need = max(B.paged_attention_workspace_bytes(cache.desc, len(r), 64, args(r)[2], pt)
               for r in batches)
    shared = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    say(f"[edge] workspace reuse, partition_tokens={pt}, {need} bytes")
    for rep in range(2):
        if rep == 1:
            shared.zero_()
        for rows in batches:
            tab, bl, mx, q = args(rows)
            outs = []
            for ws in (shared, None):
                if ws is None:
                    nb = B.paged_attention_workspace_bytes(cache.desc, len(rows), 64, mx, pt)
                    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
                out = torch.empty((len(rows), 64, 128), dtype=torch.float32, device="cuda")
                B.paged_attention_decode(cache.desc, out, "f32", q, cache.k_pool, cache.v_pool,
                                         tab, bl, 64, mx, float(w.scale), pt, ws)
                outs.append(out)
            torch.cuda.synchronize()
            assert torch.equal(outs[0], outs[1]), (rep, rows)
            if rows == batches[0]:   # the replay's own call on the full batch
                assert torch.equal(outs[0], g.outputs[0])
    o = oreplay.run(w)
    assert_close(g.outputs[0], o.outputs[0], "bf16", "f32")
    cache.close()


def test_workspace_reused_across_schedules_bitwise():
    """Fixed-partition calls reserve the stream-K counter prefix and never write it, so
    one zero-filled workspace serves stream-K, then 512-token partitions, then stream-K
    again on batches with the same counter count, and every call gives the bits of a
    call on a fresh workspace (before the prefix was reserved, the fixed call's partition
    maxima landed on the counters and the third call merged with garbage counts)."""
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.replay import to_device
    lens = [3000, 900, 2600, 17, 4100, 1300, 700, 2200]
    w = W.make_custom(lens, 64, 8, 128, "bf16", seed=37)
    g = _run(w, "f32", 0)
    cache = g.cache
    seqs, qidx = w.attend_ops()[-1][1], w.attend_ops()[-1][2]
    q = to_device(w.q[qidx], w.dtype, "cuda")
    tables, blens = cache.block_tables(seqs)
    tab, bl, mx = torch.from_numpy(tables).cuda(), torch.from_numpy(blens).cuda(), int(blens.max())
    need = max(B.paged_attention_workspace_bytes(cache.desc, len(lens), 64, mx, pt) for pt in (0, 512))
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    say(f"[edge] workspace across schedules, {need} bytes")
    for pt in (0, 512, 0, 512, 0):
        outs = []
        for ws in (shared, None):
            if ws is None:
                nb = B.paged_attention_workspace_bytes(cache.desc, len(lens), 64, mx, pt)
                ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
            out = torch.full((len(lens), 64, 128), float("nan"), dtype=torch.float32, device="cuda")
            B.paged_attention_decode(cache.desc, out, "f32", q, cache.k_pool, cache.v_pool, tab,
                                     bl, 64, mx, float(w.scale), pt, ws)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), pt
    o = oreplay.run(w)
    assert_close(outs[0], o.outputs[0], "bf16", "f32")
    cache.close()


@pytest.mark.parametrize("keep_first", [True, False], ids=["shared", "from-free-queue"])
def test_prefix_cache_hit_gives_the_same_attention_bitwise(keep_first):
    """A prompt that takes over cached prefix blocks ([DS] §2.4 hash chain) attends to the
    same K/V as one that writes the prefix itself: outputs are bit-identical, and match
    the oracle."""
    from paged_kv_cache_15_amd.cache import PagedKVCache
    from paged_kv_cache_15_amd.replay import to_device
    rng = np.random.default_rng(41)
    hq, hkv, d, dt, bs = 32, 8, 128, "bf16", 16
    pa = rng.integers(0, 50000, 2056).tolist()
    pb = pa[:2048] + rng.integers(0, 50000, 100).tolist()
    kva = rng.standard_normal((2, 2056, hkv, d)).astype(np.float32)
    kvb = np.concatenate([kva[:, :2048], rng.standard_normal((2, 100, hkv, d)).astype(np.float32)], 1)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    qd = to_device(q, dt, "cuda")

    c = PagedKVCache(400, hkv, d, dt, bs, np.random.default_rng(2).permutation(400), prefix_cache=True)
    sa, na = c.create_prefix(pa)
    assert na == 0
    c.append_tokens([sa], [pa], to_device(kva[0], dt, "cuda"), to_device(kva[1], dt, "cuda"))
    if not keep_first:
        c.free(sa)
    sb, nb = c.create_prefix(pb)
    assert nb == 2048
    c.append_tokens([sb], [pb[nb:]], to_device(kvb[0, nb:], dt, "cuda"), to_device(kvb[1, nb:], dt, "cuda"))
    out_hit, tables_hit, _ = c.attend([sb], qd, scale, "f32")

    r = PagedKVCache(400, hkv, d, dt, bs, np.random.default_rng(3).permutation(400))
    sr = r.create()
    r.append([sr], [len(pb)], to_device(kvb[0], dt, "cuda"), to_device(kvb[1], dt, "cuda"))
    out_ref, _, _ = r.attend([sr], qd, scale, "f32")
    torch.cuda.synchronize()
    say(f"[edge] prefix hit {nb} tokens, keep_first={keep_first}")
    assert torch.equal(out_hit, out_ref)
    # the oracle on the dense K/V of prompt b
    kb = lowp.storage_bits_to_f64(lowp.to_storage_bits(kvb[0], dt), dt)
    vb = lowp.storage_bits_to_f64(lowp.to_storage_bits(kvb[1], dt), dt)
    qb = lowp.storage_bits_to_f64(lowp.to_storage_bits(q, dt), dt)[0]
    from oracle.attention import dense_decode
    want = dense_decode(qb, kb, vb, scale)
    assert np.abs(out_f64(out_hit)[0] - want).max() <= TOL[dt]
    c.close()
    r.close()


@pytest.mark.parametrize("shape", [("bf16", 16, 2, 128), ("f16", 4, 4, 64)],
                         ids=lambda s: "-".join(map(str, s)))
def test_stream_k_batch_limit_and_fallback(shape):
    """8192 sequences (the most the stream-K schedule takes: its per-sequence tile
    prefix fills 32 KiB of LDS) and 8193 (falls back to 512-token partitions), short
    ragged contexts: every row against the oracle."""
    dt, hq, hkv, d = shape
    rng = np.random.default_rng(8)
    for n in (8192, 8193):
        lens = rng.integers(1, 48, size=n)
        w = W.make_custom(lens, hq, hkv, d, dt, seed=n % 97)
        say(f"[edge] {n} sequences {shape}")
        g = _run(w, "f32", 0)
        o = oreplay.run(w)
        assert_bookkeeping_equal(g, o)
        err = assert_close(g.outputs[0], o.outputs[0], dt, "f32")
        say(f"   max|err| {err:.3e}")
        g.cache.close()


@pytest.mark.parametrize("nseq,ctx_hi,shape", [(1, 2000, ("bf16", 64, 8)), (8, 2000, ("bf16", 64, 8)),
                                              (40, 2000, ("bf16", 64, 8)), (80, 2000, ("bf16", 64, 8)),
                                              (8, 1500, ("f16", 16, 16)), (4, 900, ("f32", 8, 2))],
                         ids=["1seq", "8seq", "40seq", "80seq", "mha-f16-8seq", "f32-4seq"])
def test_automatic_schedule_is_the_schedule_it_names(nseq, ctx_hi, shape):
    """PARTITION_AUTO gives bit for bit the result of the partition_tokens value it
    resolves to (256/512-token partitions for small batches, stream-K for large ones),
    and that result matches the oracle."""
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache
    from paged_kv_cache_15_amd.replay import to_device
    from oracle.attention import dense_decode
    rng = np.random.default_rng(nseq)
    lens = rng.integers(1, ctx_hi + 1, nseq).tolist()
    dt, hq, hkv = shape
    d = 128
    c = PagedKVCache(sum((n + 15) // 16 for n in lens) + 8, hkv, d, dt, 16,
                     rng.permutation(sum((n + 15) // 16 for n in lens) + 8).astype(np.int32))
    seqs = [c.create() for _ in lens]
    kv = rng.standard_normal((2, sum(lens), hkv, d)).astype(np.float32)
    c.append(seqs, lens, to_device(kv[0], dt, "cuda"), to_device(kv[1], dt, "cuda"))
    q = rng.standard_normal((nseq, hq, d)).astype(np.float32)
    qd = to_device(q, dt, "cuda")
    pt = B.paged_attention_auto_partition_tokens(c.desc, nseq, hq, max(lens))
    say(f"[auto] {nseq} sequences up to {max(lens)} tokens -> partition_tokens {pt}")
    a, _, _ = c.attend(seqs, qd, 0.088, "f32", partition_tokens=B.PARTITION_AUTO)
    b, _, _ = c.attend(seqs, qd, 0.088, "f32", partition_tokens=pt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # the oracle's dense decode on the same rounded inputs (gathered by position, not
    # through the pool), for three sequences
    qb = lowp.storage_bits_to_f64(lowp.to_storage_bits(q, dt), dt)
    kb = lowp.storage_bits_to_f64(lowp.to_storage_bits(kv, dt), dt)
    starts = np.concatenate([[0], np.cumsum(lens)])
    for s in sorted({0, nseq - 1, int(np.argmax(lens))}):
        ref = dense_decode(qb[s], kb[0, starts[s]:starts[s + 1]], kb[1, starts[s]:starts[s + 1]], 0.088)
        assert np.abs(a[s].double().cpu().numpy() - ref).max() <= TOL[dt]
    c.close()

