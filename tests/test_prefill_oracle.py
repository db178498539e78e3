"""Pins of the prefill oracle (CPU): causal multi-query attention over the pool.

deepsonar "PagedAttention de vLLM …" §2.5 (a prompt, a chunk of one, and the rest of
one after a prefix-cache hit are the same step) and §2.6 (that attention reads the
blocks through the table too).  The oracle is pinned against PyTorch's own causal
attention in float64 (an independent implementation), against the decode oracle for
one query per sequence, against itself across chunk boundaries, and by the exact
value of the first position; planted mistakes (no causal mask, a position off by one,
a chunk placed at the start of the context) each fail one of these checks.
"""
import numpy as np
import pytest
import torch

from oracle import attention as ATT
from oracle import lowp, pool as P


def _pool(rng, lens, hkv, d, dt, bs):
    """Pool holding every sequence's tokens at scattered blocks; returns bits of K/V per
    sequence too (logical order)."""
    nblk = [(-(-L // bs)) for L in lens]
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    kp, vp = P.new_pool(nb, hkv, bs, d, dt)
    tables, kv, used = [], [], 0
    for L, n in zip(lens, nblk):
        table = perm[used:used + n]
        used += n
        kb = lowp.to_storage_bits(rng.standard_normal((L, hkv, d)).astype(np.float32), dt)
        vb = lowp.to_storage_bits(rng.standard_normal((L, hkv, d)).astype(np.float32), dt)
        slots = table[np.arange(L) // bs] * bs + np.arange(L) % bs
        P.reshape_and_cache(kp, vp, kb, vb, slots, bs)
        tables.append(table)
        kv.append((lowp.storage_bits_to_f64(kb, dt), lowp.storage_bits_to_f64(vb, dt)))
    width = max(nblk)
    tab = np.full((len(lens), width), -1, np.int64)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    return kp, vp, tab, kv


def _queries(rng, n_rows, hq, d, dt):
    return lowp.storage_bits_to_f64(
        lowp.to_storage_bits(rng.standard_normal((n_rows, hq, d)).astype(np.float32), dt), dt)


def _sdpa_causal(q, k, v, scale):
    """PyTorch's causal attention in float64 for one sequence whose queries are its
    last len(q) tokens: q [n][Hq][d], k/v [L][Hkv][d]."""
    n, hq, d = q.shape
    L, hkv = k.shape[0], k.shape[1]
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][n][d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    # query i (position L - n + i) may see key j iff j <= L - n + i
    mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def _check_against_torch(prefill, bs, dt):
    rng = np.random.default_rng(bs * 3 + len(dt))
    hq, hkv, d = 8, 2, 16
    lens = [1, 5, 16, 17, 40]
    kp, vp, tab, kv = _pool(rng, lens, hkv, d, dt, bs)
    nq = [1, 3, 16, 9, 40]                  # full prefill for 1 and 40, chunks otherwise
    q_start = np.concatenate([[0], np.cumsum(nq)])
    q = _queries(rng, q_start[-1], hq, d, dt)
    scale = 0.3
    got = prefill(q, kp, vp, tab, lens, q_start, scale, dt, bs)
    for s, L in enumerate(lens):
        r0, r1 = q_start[s], q_start[s + 1]
        want = _sdpa_causal(q[r0:r1], kv[s][0], kv[s][1], scale)
        assert np.allclose(got[r0:r1], want, rtol=0, atol=1e-12), s


def _check_chunks_agree(prefill, bs, dt):
    """A chunk's rows equal the same rows of one prefill over the whole context."""
    rng = np.random.default_rng(7 + bs)
    hq, hkv, d, L = 4, 4, 16, 37
    kp, vp, tab, _ = _pool(rng, [L], hkv, d, dt, bs)
    qa = _queries(rng, L, hq, d, dt)
    full = prefill(qa, kp, vp, tab, [L], np.array([0, L]), 0.25, dt, bs)
    for a in (1, 16, 20, 36):
        part = prefill(qa[a:], kp, vp, tab, [L], np.array([0, L - a]), 0.25, dt, bs)
        assert np.array_equal(part, full[a:]), a


def _check_one_query_is_decode(prefill, bs, dt):
    rng = np.random.default_rng(11 + bs)
    hq, hkv, d = 8, 2, 32
    lens = [3, 18, 33]
    kp, vp, tab, _ = _pool(rng, lens, hkv, d, dt, bs)
    q = _queries(rng, len(lens), hq, d, dt)
    got = prefill(q, kp, vp, tab, lens, np.arange(len(lens) + 1), 0.2, dt, bs)
    want = ATT.paged_decode(q, kp, vp, [t[t >= 0] for t in tab], lens, 0.2, dt, bs)
    assert np.array_equal(got, want)


def _check_first_position_returns_its_value(prefill, bs, dt):
    rng = np.random.default_rng(13 + bs)
    hq, hkv, d, L = 6, 3, 16, 12
    kp, vp, tab, kv = _pool(rng, [L], hkv, d, dt, bs)
    q = _queries(rng, L, hq, d, dt)
    got = prefill(q, kp, vp, tab, [L], np.array([0, L]), 1.0, dt, bs)
    assert np.array_equal(got[0], np.repeat(kv[0][1][0], hq // hkv, axis=0))


CHECKS = [_check_against_torch, _check_chunks_agree, _check_one_query_is_decode,
          _check_first_position_returns_its_value]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
@pytest.mark.parametrize("bs,dt", [(16, "bf16"), (4, "f16"), (32, "f32"), (1, "bf16")])
def test_prefill_oracle_pins(check, bs, dt):
    check(ATT.paged_prefill, bs, dt)


def _planted(kind):
    """The oracle with one mistake planted (a copy written here, not a patch)."""
    def prefill(q, k_pool, v_pool, tables, context_lens, q_start, scale, dtype, block_size):
        out = np.full(q.shape, np.nan)
        for b in range(len(context_lens)):
            L, r0, r1 = int(context_lens[b]), int(q_start[b]), int(q_start[b + 1])
            n = r1 - r0
            kb, vb = P.gather_sequence(k_pool, v_pool, tables[b], L, block_size)
            k, v = lowp.storage_bits_to_f64(kb, dtype), lowp.storage_bits_to_f64(vb, dtype)
            for i in range(n):
                p = L - n + i
                if kind == "no_mask":
                    hi = L
                elif kind == "off_by_one":
                    hi = p + 2 if p + 2 <= L else p + 1
                else:                       # chunk taken as the start of the context
                    hi = i + 1
                out[r0 + i] = ATT.dense_decode(q[r0 + i], k[:hi], v[:hi], scale)
        return out
    return prefill


@pytest.mark.parametrize("kind", ["no_mask", "off_by_one", "chunk_at_start"])
def test_pins_catch_planted_prefill_mistakes(kind):
    bad = _planted(kind)
    caught = 0
    for check in CHECKS:
        try:
            check(bad, 16, "bf16")
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


@pytest.mark.parametrize("dt,hq,hkv,d,bs", [("bf16", 8, 2, 64, 16), ("f16", 4, 4, 32, 1),
                                           ("bf16", 6, 3, 16, 32)])
def test_matrix_form_equals_row_by_row_and_sdpa(dt, hq, hkv, d, bs):
    """The matrix form (causal_rows / paged_prefill_rows) against the row-by-row oracle
    and against PyTorch's causal attention in float64, whole prompts and chunks."""
    rng = np.random.default_rng(hq * 13 + d + bs)
    lens = [1, 17, 40, 75]
    kp, vp, tab, kv = _pool(rng, lens, hkv, d, dt, bs)
    counts = [1, 9, 40, 30]                        # a whole prompt (40) and chunks
    starts = np.concatenate([[0], np.cumsum(counts)])
    q = _queries(rng, int(starts[-1]), hq, d, dt)
    scale = 1 / np.sqrt(d)
    a = ATT.paged_prefill(q, kp, vp, tab, lens, starts, scale, dt, bs)
    b = ATT.paged_prefill_rows(q, kp, vp, tab, lens, starts, scale, dt, bs, seqs=range(len(lens)))
    assert np.abs(a - b).max() <= 1e-12
    for i, (L, n) in enumerate(zip(lens, counts)):
        ref = _sdpa_causal(q[starts[i]:starts[i + 1]], kv[i][0], kv[i][1], scale)
        assert np.abs(b[starts[i]:starts[i + 1]] - ref).max() <= 1e-12


def test_matrix_form_catches_a_dropped_mask():
    """Planted mistake: without removing the keys past each row's position the matrix
    form no longer matches the row-by-row oracle."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((20, 2, 8))
    v = rng.standard_normal((20, 2, 8))
    q = rng.standard_normal((20, 4, 8))
    good = ATT.causal_rows(q, k, v, 0.3, 0)
    rows = np.stack([ATT.dense_decode(q[i], k[:i + 1], v[:i + 1], 0.3) for i in range(20)])
    assert np.abs(good - rows).max() <= 1e-12
    nomask = np.stack([ATT.dense_decode(q[i], k, v, 0.3) for i in range(20)])
    assert np.abs(good - nomask).max() > 1e-3

