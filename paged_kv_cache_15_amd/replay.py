"""Run a workload script (create / fork / append / free / attend) on the GPU.

The script format is the one the seeded workload generators produce: ops in
order, float32 K/V rows per append and float32 queries per attend, cast here to
the pool's storage type on the device.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

from .cache import PagedKVCache, TORCH_DTYPES


@dataclass
class GpuReplay:
    cache: PagedKVCache
    slot_mappings: list = field(default_factory=list)
    copies: list = field(default_factory=list)
    tables: list = field(default_factory=list)
    context_lens: list = field(default_factory=list)
    outputs: list = field(default_factory=list)     # device tensors, one per attend op


def to_device(x, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device).to(TORCH_DTYPES[dtype])


def run_workload(w, device="cuda", out_dtype=None, partition_tokens=None, poison=True,
                 out_fill=None):
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, w.block_size,
                         w.free_order, device=device, poison=poison)
    res = GpuReplay(cache=cache)
    pt = w.partition_tokens if partition_tokens is None else partition_tokens
    for op in w.ops:
        kind = op[0]
        if kind == "create":
            cache.create()
        elif kind == "fork":
            cache.fork(op[1])
        elif kind == "free":
            cache.free(op[1])
        elif kind == "append":
            seqs, counts, vidx = op[1], op[2], op[3]
            k, v = w.kv[vidx]
            kd, vd = to_device(k, w.dtype, device), to_device(v, w.dtype, device)
            slots, copies = cache.append(seqs, counts, kd, vd)
            del kd, vd
            res.slot_mappings.append(slots)
            res.copies.append(copies)
        elif kind == "attend":
            seqs, qidx = op[1], op[2]
            q = to_device(w.q[qidx], w.dtype, device)
            out, tables, lens = cache.attend(seqs, q, float(w.scale), out_dtype, pt,
                                             out_fill=out_fill)
            res.outputs.append(out)
            res.tables.append(tables)
            res.context_lens.append(lens)
        elif kind == "prefill":
            seqs, counts, qidx = op[1], op[2], op[3]
            q = to_device(w.q[qidx], w.dtype, device)
            out, tables, lens = cache.attend_prefill(seqs, counts, q, float(w.scale), out_dtype,
                                                     out_fill=out_fill)
            res.outputs.append(out)
            res.tables.append(tables)
            res.context_lens.append(lens)
        else:
            raise ValueError(f"unknown op {kind}")
    return res
