"""A multi-layer decode step captured in a HIP graph.

Per layer a decode step writes the batch's new tokens into that layer's pool and runs
paged attention over it (deepsonar "PagedAttention de vLLM …", §2.6: the block table
handed to the kernel, and graph capture of the decode step).  All layers share one
allocator: a block id names the same slot range in every layer's K/V buffers, so the
slot mapping and block tables of a step are computed once on the host (the allocator
is host code and stays out of the graph) and copied into the graph's fixed device
buffers before each replay.  The graph holds only kernel launches from libpagedkv.so
(no memset or copy nodes): per layer one fused launch (cache write, attention and
merge: paged_attention_decode_append) where the schedule has one, else the cache write
and the attention's launches.

Copy-on-write copies, when an append makes any, are issued eagerly for every layer
before the replay.
"""
import numpy as np
import torch

from . import binding as B
from .cache import PagedKVCache, TORCH_DTYPES, BITS_DTYPES


class LayeredKV:
    """One allocator, `num_layers` K/V pool pairs of the same shape."""

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, dtype, block_size=16,
                 free_order=None, device="cuda", poison=True):
        self.cache = PagedKVCache(num_blocks, num_kv_heads, head_dim, dtype, block_size,
                                  free_order, device, poison)
        self.k, self.v = [self.cache.k_pool], [self.cache.v_pool]
        for _ in range(num_layers - 1):
            k, v = torch.empty_like(self.cache.k_pool), torch.empty_like(self.cache.v_pool)
            if poison:
                k.view(BITS_DTYPES[dtype]).fill_(-1)
                v.view(BITS_DTYPES[dtype]).fill_(-1)
            self.k.append(k)
            self.v.append(v)
        self.num_layers = num_layers
        self.desc = self.cache.desc
        self.dtype = dtype
        self.device = self.cache.device

    def close(self):
        self.cache.close()

    def append(self, seqs, counts, keys, values, stream=None):
        """Reserve slots (once, for all layers), copy shared tail blocks in every layer
        and write each layer's new rows (keys[l], values[l]: [sum(counts)][Hkv][d])."""
        slots, copies = B.paged_kv_append_batch(self.cache.pool, seqs, counts)
        self.copy_blocks(copies, stream)
        if len(slots):
            slot_d = torch.from_numpy(slots).to(self.device)
            for l in range(self.num_layers):
                B.reshape_and_cache(self.desc, keys[l], values[l], self.k[l], self.v[l], slot_d,
                                    stream=stream)
        return slots, copies

    def copy_blocks(self, copies, stream=None):
        if len(copies):
            pairs = torch.from_numpy(np.ascontiguousarray(copies, dtype=np.int32)).to(self.device)
            for l in range(self.num_layers):
                B.paged_kv_copy_blocks(self.desc, self.k[l], self.v[l], pairs, len(copies), stream)


class DecodeStep:
    """One decode step (one new token per sequence) over all layers, eager or replayed
    from a HIP graph.  Shapes are fixed at construction: num_seqs rows, block tables
    max_blocks wide, attention sized for max_context_len.  partition_tokens as for
    paged_attention_decode; by default the library picks the schedule for the shape."""

    def __init__(self, kv: LayeredKV, num_seqs, num_q_heads, max_blocks, max_context_len, scale,
                 partition_tokens=B.PARTITION_AUTO, out_dtype=None, fused=True):
        self.kv = kv
        self.fused = fused
        self.B, self.hq = num_seqs, num_q_heads
        self.max_blocks, self.max_ctx = max_blocks, max_context_len
        self.scale, self.pt = float(scale), partition_tokens
        self.out_dtype = out_dtype or kv.dtype
        d, hkv, L, dev = kv.desc.head_dim, kv.desc.num_kv_heads, kv.num_layers, kv.device
        tdt = TORCH_DTYPES[kv.dtype]
        self.tables = torch.full((num_seqs, max_blocks), -1, dtype=torch.int32, device=dev)
        self.lens = torch.zeros(num_seqs, dtype=torch.int32, device=dev)
        self.slots = torch.full((num_seqs,), -1, dtype=torch.int32, device=dev)
        self.new_k = torch.zeros((L, num_seqs, hkv, d), dtype=tdt, device=dev)
        self.new_v = torch.zeros((L, num_seqs, hkv, d), dtype=tdt, device=dev)
        self.q = torch.zeros((L, num_seqs, num_q_heads, d), dtype=tdt, device=dev)
        self.out = torch.zeros((L, num_seqs, num_q_heads, d), dtype=TORCH_DTYPES[self.out_dtype],
                               device=dev)
        nbytes = B.paged_attention_workspace_bytes(kv.desc, num_seqs, num_q_heads,
                                                   max_context_len, partition_tokens)
        # zero-filled once; every call leaves the stream-K counters at zero again, and the
        # layers' calls follow each other on one stream, so they share it
        self.ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
        self.graph = None

    def set_step(self, seqs, new_k, new_v, q):
        """Host part of the step: reserve one slot per sequence, copy shared tail blocks
        in every layer, and load slots, tables, lengths and the step's rows into the
        fixed buffers (new_k/new_v [L][B][Hkv][d], q [L][B][Hq][d] device tensors)."""
        if len(seqs) != self.B:
            raise ValueError(f"step built for {self.B} sequences, got {len(seqs)}")
        slots, copies = B.paged_kv_append_batch(self.kv.cache.pool, seqs, [1] * len(seqs))
        self.kv.copy_blocks(copies)
        tables, lens = B.paged_kv_block_tables(self.kv.cache.pool, seqs, self.max_blocks)
        if int(lens.max()) > self.max_ctx:
            raise ValueError(f"context {int(lens.max())} exceeds the step's {self.max_ctx}")
        self.slots.copy_(torch.from_numpy(slots))
        self.tables.copy_(torch.from_numpy(tables))
        self.lens.copy_(torch.from_numpy(lens))
        self.new_k.copy_(new_k)
        self.new_v.copy_(new_v)
        self.q.copy_(q)
        return slots, copies

    def launch(self):
        """All layers' kernels on the current stream."""
        kv = self.kv
        for l in range(kv.num_layers):
            if self.fused:
                B.paged_attention_decode_append(kv.desc, self.out[l], self.out_dtype, self.q[l],
                                                self.new_k[l], self.new_v[l], self.slots, kv.k[l],
                                                kv.v[l], self.tables, self.lens, self.hq,
                                                self.max_ctx, self.scale, self.pt, self.ws)
                continue
            B.reshape_and_cache(kv.desc, self.new_k[l], self.new_v[l], kv.k[l], kv.v[l], self.slots)
            B.paged_attention_decode(kv.desc, self.out[l], self.out_dtype, self.q[l], kv.k[l],
                                     kv.v[l], self.tables, self.lens, self.hq, self.max_ctx,
                                     self.scale, self.pt, self.ws)

    def capture(self):
        """Record launch() into a HIP graph (the buffers' current contents are written
        during capture's warm-up run, so call this after set_step of a real step or on
        buffers whose slots are all -1)."""
        side = torch.cuda.Stream(self.kv.device)
        side.wait_stream(torch.cuda.current_stream(self.kv.device))
        with torch.cuda.stream(side):
            self.launch()                         # warm-up outside capture
        torch.cuda.current_stream(self.kv.device).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.launch()
        return self.graph

    def replay(self):
        self.graph.replay()
