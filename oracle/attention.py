"""Paged decode attention, as its plain definition, in float64.

Paging only changes where the keys and values live: the model still sees each
sequence as contiguous (chester-dev.com "vLLM transforme la mémoire GPU …",
section on PagedAttention and the logical/physical split; deeplearn.tn
"PagedAttention : comment optimiser la mémoire GPU …", block-table section), and
the kernel gathers the physical blocks through the table (deepsonar
"PagedAttention de vLLM …", §2.2 and §2.6).  So the oracle reassembles each
sequence's K and V in logical order and runs textbook softmax attention for its
one query per head.

Readings: query head h uses KV head h // (Hq / Hkv) (consecutive groups share a
KV head; §2.1 of the deepsonar page has 64 query heads sharing 8 KV heads);
scores are scale x (q . k) with no mask beyond the context length.
"""
import numpy as np

from .lowp import storage_bits_to_f64
from .pool import gather_sequence


def dense_decode(q, k, v, scale):
    """One sequence: q[Hq][d], k/v[ctx][Hkv][d] float64 -> out[Hq][d]."""
    hq, hkv = q.shape[0], k.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    out = np.empty_like(q, dtype=np.float64)
    for h in range(hq):
        g = h // group
        z = float(scale) * (k[:, g, :] @ q[h])
        w = np.exp(z - z.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def paged_decode(q, k_pool, v_pool, tables, context_lens, scale, dtype, block_size, seqs=None):
    """q: float64 [B][Hq][d] (already the values of the rounded storage type).

    tables[b] lists sequence b's physical blocks in logical order; context_lens[b]
    is its number of tokens.  Returns float64 [B][Hq][d]; with `seqs` given, only
    those batch rows are computed (the others are NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    out = np.full(q.shape, np.nan)
    rows = range(q.shape[0]) if seqs is None else seqs
    for b in rows:
        L = int(context_lens[b])
        if L < 1:
            raise ValueError("context length must be >= 1")
        kb, vb = gather_sequence(k_pool, v_pool, tables[b], L, block_size)
        k = storage_bits_to_f64(kb, dtype)
        v = storage_bits_to_f64(vb, dtype)
        out[b] = dense_decode(q[b], k, v, scale)
    return out


def paged_prefill(q, k_pool, v_pool, tables, context_lens, q_start, scale, dtype, block_size,
                  seqs=None):
    """Causal multi-query attention over the pool: prefill, and prefill in chunks.

    deepsonar "PagedAttention de vLLM …" §2.5: a request only tracks how many of its
    tokens are already computed, so a whole prompt, a chunk of a long prompt and the
    rest of a prompt after a prefix-cache hit are the same operation; §2.6: that
    attention too reads the blocks through the table.  Reading: the queries of
    sequence s are rows q_start[s] .. q_start[s+1] - 1 of q, its last
    n_s = q_start[s+1] - q_start[s] tokens (already written to the pool, whose
    context_lens[s] tokens include them); query i sits at position
    context_lens[s] - n_s + i and attends to keys 0 .. that position (causal).

    q: float64 [total][Hq][d].  Returns float64 [total][Hq][d]; with `seqs` given,
    only those sequences' rows are computed (the others are NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    out = np.full(q.shape, np.nan)
    rows = range(len(context_lens)) if seqs is None else seqs
    for b in rows:
        L, r0, r1 = int(context_lens[b]), int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n < 0 or n > L:
            raise ValueError("a sequence needs 0 <= query count <= context length")
        if n == 0:
            continue
        kb, vb = gather_sequence(k_pool, v_pool, tables[b], L, block_size)
        k = storage_bits_to_f64(kb, dtype)
        v = storage_bits_to_f64(vb, dtype)
        for i in range(n):
            p = L - n + i
            out[r0 + i] = dense_decode(q[r0 + i], k[:p + 1], v[:p + 1], scale)
    return out


def causal_rows(q, k, v, scale, first_pos):
    """Causal attention of one sequence's consecutive query rows, all rows at once.

    Query i sits at position first_pos + i and sees keys 0 .. first_pos + i (the same
    reading as paged_prefill).  Per query head h (KV head h // (Hq / Hkv)): the score
    matrix scale * Q K^T, the keys past each row's position removed, the softmax of each
    row (exp(z - row max) / row sum) and its product with V: dense_decode of every row,
    written as matrix products.  q: float64 [n][Hq][d]; k, v: float64 [>= first_pos + n]
    [Hkv][d].  Returns float64 [n][Hq][d].
    """
    q = np.asarray(q, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    L = int(first_pos) + n
    hidden = np.arange(L)[None, :] > (int(first_pos) + np.arange(n))[:, None]
    out = np.empty((n, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        kg = np.ascontiguousarray(k[:L, g, :])  # (contiguous operands keep the products on
        vg = np.ascontiguousarray(v[:L, g, :])  # BLAS; the steps below work in place)
        z = q[:, h, :] @ kg.T
        z *= float(scale)
        np.putmask(z, hidden, -np.inf)
        z -= z.max(axis=1, keepdims=True)
        np.exp(z, out=z)
        out[:, h, :] = (z @ vg) / z.sum(axis=1, keepdims=True)
    return out


def paged_prefill_rows(q, k_pool, v_pool, tables, context_lens, q_start, scale, dtype,
                       block_size, seqs):
    """paged_prefill for the listed sequences with each sequence's rows computed at once
    by causal_rows (same reading, same result up to rounding order); the other rows are
    NaN."""
    q = np.asarray(q, dtype=np.float64)
    out = np.full(q.shape, np.nan)
    for b in seqs:
        L, r0, r1 = int(context_lens[b]), int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n < 0 or n > L:
            raise ValueError("a sequence needs 0 <= query count <= context length")
        if n == 0:
            continue
        kb, vb = gather_sequence(k_pool, v_pool, tables[b], L, block_size)
        out[r0:r1] = causal_rows(q[r0:r1], storage_bits_to_f64(kb, dtype),
                                 storage_bits_to_f64(vb, dtype), scale, L - n)
    return out


def partial_state(z, v):
    """Softmax state of one slice of tokens: (max score, sum of weights, weighted V)."""
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ v


def lse_merge(states):
    """Combine slice states into the softmax-weighted mean over all their tokens.

    Each slice's weights are relative to its own maximum; rescaling every slice to
    the overall maximum makes them comparable, then the weighted sums add up
    (the incremental softmax of deeplearn.tn, PagedAttention vs. FlashAttention).
    """
    big_m = max(s[0] for s in states)
    num = sum(np.exp(m - big_m) * acc for m, _, acc in states)
    den = sum(np.exp(m - big_m) * l for m, l, _ in states)
    return num / den
