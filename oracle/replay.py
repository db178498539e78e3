"""Replay a workload script on the CPU: allocator, pool writes, attention.

Executes the operations in script order with plain sequential semantics: for
each sequence of an append, its copy-on-write copies happen, then its tokens are
written, before the next sequence is handled.
"""
from dataclasses import dataclass, field

import numpy as np

from .allocator import BlockAllocator
from .attention import paged_decode, paged_prefill
from .lowp import to_storage_bits, storage_bits_to_f64
from .pool import new_pool, reshape_and_cache, copy_block


@dataclass
class ReplayResult:
    k_pool: np.ndarray
    v_pool: np.ndarray
    slot_mappings: list = field(default_factory=list)   # int32 per append op
    copies: list = field(default_factory=list)          # int32 [n][2] per append op
    tables: list = field(default_factory=list)          # int32 [B][max_blocks] per attend op
    context_lens: list = field(default_factory=list)    # int32 [B] per attend op
    outputs: list = field(default_factory=list)         # float64 [B][Hq][d] per attend op
    allocator: BlockAllocator = None


def padded_tables(alloc, seqs, max_blocks=None):
    rows = [alloc.block_table(s) for s in seqs]
    width = max(1, max(len(r) for r in rows)) if max_blocks is None else max_blocks
    t = np.full((len(seqs), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        t[i, :len(r)] = r
    return t


def run(w, attend_rows=None, compute_attention=True, last_rows="same"):
    """Replay workload `w`.  attend_rows: batch rows (sequences of a prefill op) to compute
    per attention op (None = all); last_rows: the rows of the script's last attention op
    instead ("same": attend_rows, None: all).
    A workload built without values replays the allocator only (pools stay None)."""
    n_att = sum(1 for op in w.ops if op[0] in ("attend", "prefill"))
    seen = 0

    def rows_now():
        return last_rows if (last_rows != "same" and seen == n_att) else attend_rows
    alloc = BlockAllocator(w.num_blocks, w.block_size, w.free_order)
    has_values = any(x is not None for x in w.kv)
    k_pool, v_pool = (new_pool(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.dtype)
                      if has_values else (None, None))
    res = ReplayResult(k_pool=k_pool, v_pool=v_pool, allocator=alloc)
    for op in w.ops:
        kind = op[0]
        if kind == "create":
            alloc.create()
        elif kind == "fork":
            alloc.fork(op[1])
        elif kind == "free":
            alloc.release(op[1])
        elif kind == "append":
            seqs, counts, vidx = op[1], op[2], op[3]
            values = w.kv[vidx]          # None: allocator-only replay, no pool writes
            if values is not None:
                kbits = to_storage_bits(values[0], w.dtype)
                vbits = to_storage_bits(values[1], w.dtype)
            all_slots, all_copies, row = [], [], 0
            for s, n in zip(seqs, counts):
                slots, copies = alloc.append(s, n)
                if values is not None:
                    for src, dst in copies:
                        copy_block(k_pool, v_pool, src, dst)
                    reshape_and_cache(k_pool, v_pool, kbits[row:row + n], vbits[row:row + n],
                                      slots, w.block_size)
                row += n
                all_slots += slots
                all_copies += copies
            res.slot_mappings.append(np.asarray(all_slots, dtype=np.int32))
            res.copies.append(np.asarray(all_copies, dtype=np.int32).reshape(-1, 2))
        elif kind == "attend":
            seen += 1
            seqs, qidx = op[1], op[2]
            tables = padded_tables(alloc, seqs)
            lens = np.asarray([alloc.context_len(s) for s in seqs], dtype=np.int32)
            res.tables.append(tables)
            res.context_lens.append(lens)
            if compute_attention and w.q[qidx] is not None:
                q = storage_bits_to_f64(to_storage_bits(w.q[qidx], w.dtype), w.dtype)
                res.outputs.append(paged_decode(q, k_pool, v_pool, tables, lens, w.scale,
                                                w.dtype, w.block_size, seqs=rows_now()))
            else:
                res.outputs.append(None)
        elif kind == "prefill":
            # causal attention of each listed sequence's last counts[i] tokens
            seen += 1
            seqs, counts, qidx = op[1], op[2], op[3]
            tables = padded_tables(alloc, seqs)
            lens = np.asarray([alloc.context_len(s) for s in seqs], dtype=np.int32)
            q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
            res.tables.append(tables)
            res.context_lens.append(lens)
            if compute_attention and w.q[qidx] is not None:
                q = storage_bits_to_f64(to_storage_bits(w.q[qidx], w.dtype), w.dtype)
                res.outputs.append(paged_prefill(q, k_pool, v_pool, tables, lens, q_start, w.scale,
                                                 w.dtype, w.block_size, seqs=rows_now()))
            else:
                res.outputs.append(None)
        else:
            raise ValueError(f"unknown op {kind}")
    return res
