"""One decode step on the paged KV cache, driven from the host.

A step (deepsonar "PagedAttention de vLLM …" §2.2 and §2.6; deeplearn.tn
"PagedAttention : comment optimiser la mémoire GPU …", continuous batching) is:
  1. the host allocator reserves a slot for each new token (taking a block only when
     the previous one is full, copying a shared partial block first);
  2. copy-on-write copies and the cache write run on the GPU;
  3. the block tables go to the GPU and paged attention reads the pool through them.
Every arithmetic step runs in libpagedkv.so; this module only moves arguments.
The pool buffers are torch tensors owned by this object (PyTorch provides device
memory and streams; the library never allocates them).
"""
import numpy as np
import torch

from . import binding as B

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
BITS_DTYPES = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}


class PagedKVCache:
    def __init__(self, num_blocks, num_kv_heads, head_dim, dtype, block_size=16, free_order=None,
                 device="cuda", poison=True, prefix_cache=False):
        self.dtype = dtype
        self.device = torch.device(device)
        self.desc = B.make_desc(num_blocks, block_size, num_kv_heads, head_dim, dtype,
                                B.PAGED_KV_POOL_PREFIX_CACHE if prefix_cache else 0)
        x = 16 // torch.tensor([], dtype=TORCH_DTYPES[dtype]).element_size()
        tdt = TORCH_DTYPES[dtype]
        # a block of more than 16 tokens is stored as 16-token sub-blocks, one after the
        # other: [block][kv_head][sub-block * head_dim / X][16][X] (V: [.][.][sub * d][16])
        tb = min(block_size, 16)
        ns = block_size // tb
        self.k_pool = torch.empty((num_blocks, num_kv_heads, ns * head_dim // x, tb, x),
                                  dtype=tdt, device=self.device)
        self.v_pool = torch.empty((num_blocks, num_kv_heads, ns * head_dim, tb), dtype=tdt,
                                  device=self.device)
        if poison:   # all-ones bytes: NaN in every supported type
            self.k_pool.view(BITS_DTYPES[dtype]).fill_(-1)
            self.v_pool.view(BITS_DTYPES[dtype]).fill_(-1)
        self.pool = B.paged_kv_pool_create(self.desc, free_order, self.k_pool, self.v_pool)

    def close(self):
        if self.pool:
            B.paged_kv_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- allocator ---------------------------------------------------------
    def create(self):
        return B.paged_kv_seq_create(self.pool)

    def fork(self, parent):
        return B.paged_kv_seq_fork(self.pool, parent)

    def free(self, seq):
        B.paged_kv_seq_free(self.pool, seq)

    def stats(self):
        return B.paged_kv_stats(self.pool)

    # -- prefix caching (pool made with prefix_cache=True) ----------------------
    def create_prefix(self, prompt, extra_key=0):
        """New sequence for a prompt of token ids; returns (seq, tokens already cached)."""
        return B.paged_kv_seq_create_prefix(self.pool, prompt, extra_key)

    def append_tokens(self, seqs, token_lists, key, value, stream=None):
        """Like append, with the new tokens' ids (full blocks enter the hash map); key and
        value hold the rows of all sequences' new tokens in order."""
        slots, copies = [], []
        for sq, toks in zip(seqs, token_lists):
            s_, c_ = B.paged_kv_seq_append_tokens(self.pool, sq, toks)
            slots.append(s_)
            copies.extend(tuple(x) for x in c_)
        slots = np.concatenate(slots) if slots else np.empty(0, np.int32)
        if copies:
            pairs = torch.from_numpy(np.asarray(copies, dtype=np.int32)).to(self.device)
            B.paged_kv_copy_blocks(self.desc, self.k_pool, self.v_pool, pairs, len(copies), stream)
        if len(slots):
            slot_d = torch.from_numpy(slots).to(self.device)
            B.reshape_and_cache(self.desc, key, value, self.k_pool, self.v_pool, slot_d,
                                stream=stream)
        return slots, copies

    def block_tables(self, seqs, max_blocks=None):
        return B.paged_kv_block_tables(self.pool, seqs, max_blocks)

    # -- steps -------------------------------------------------------------
    def append(self, seqs, counts, key, value, stream=None):
        """Reserve slots for counts[i] new tokens of seqs[i], then copy shared tail
        blocks and write key/value ([sum(counts)][Hkv][d] device tensors) into them.
        Returns the host slot mapping and copy pairs."""
        slots, copies = B.paged_kv_append_batch(self.pool, seqs, counts)
        if len(copies):
            pairs = torch.from_numpy(np.ascontiguousarray(copies)).to(self.device)
            B.paged_kv_copy_blocks(self.desc, self.k_pool, self.v_pool, pairs, len(copies), stream)
        if len(slots):
            slot_d = torch.from_numpy(slots).to(self.device)
            B.reshape_and_cache(self.desc, key, value, self.k_pool, self.v_pool, slot_d,
                                stream=stream)
        return slots, copies

    def attend(self, seqs, q, scale, out_dtype=None, partition_tokens=0, stream=None,
               out_fill=None):
        """Decode attention of q ([len(seqs)][Hq][d] device tensor) over the sequences.
        out_fill: a value to fill the output with before the call (tests fill NaN, so a
        row the kernels never write cannot pass for a result)."""
        tables, lens = self.block_tables(seqs)
        out_dtype = out_dtype or self.dtype
        max_ctx = int(lens.max()) if len(lens) else 1
        tables_d = torch.from_numpy(tables).to(self.device)
        lens_d = torch.from_numpy(lens).to(self.device)
        hq, d = q.shape[1], q.shape[2]
        shape = (len(seqs), hq, d)
        out = (torch.empty(shape, dtype=TORCH_DTYPES[out_dtype], device=self.device)
               if out_fill is None else
               torch.full(shape, out_fill, dtype=TORCH_DTYPES[out_dtype], device=self.device))
        nbytes = B.paged_attention_workspace_bytes(self.desc, len(seqs), hq, max_ctx,
                                                   partition_tokens)
        # zero-filled: the stream-K schedule keeps per-unit counters in the workspace
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=self.device) if nbytes else None
        B.paged_attention_decode(self.desc, out, out_dtype, q, self.k_pool, self.v_pool, tables_d,
                                 lens_d, hq, max_ctx, scale, partition_tokens, ws, stream)
        return out, tables, lens

    def attend_shared(self, seqs, q, scale, out_dtype=None, max_group=8, min_shared_tokens=16,
                      partition_tokens=0, stream=None, out_fill=None):
        """Decode attention that reads each group's shared prompt blocks once ([DS] §2.3):
        the host allocator forms the groups (consecutive sequences of the batch whose
        tables start with the same blocks), then paged_attention_decode_shared_prefix.
        Returns (out, group info)."""
        tables, lens = self.block_tables(seqs)
        hq, d = q.shape[1], q.shape[2]
        max_group = max(1, min(int(max_group), 64 // (hq // self.desc.num_kv_heads)))
        gs, sh, max_shared = B.paged_kv_shared_prefix_groups(self.pool, seqs, max_group,
                                                             min_shared_tokens)
        out_dtype = out_dtype or self.dtype
        max_ctx = int(lens.max()) if len(lens) else 1
        shape = (len(seqs), hq, d)
        out = (torch.empty(shape, dtype=TORCH_DTYPES[out_dtype], device=self.device)
               if out_fill is None else
               torch.full(shape, out_fill, dtype=TORCH_DTYPES[out_dtype], device=self.device))
        nbytes = B.paged_attention_shared_prefix_workspace_bytes(
            self.desc, len(seqs), hq, max_ctx, len(sh), max_group, max_shared, partition_tokens)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        B.paged_attention_decode_shared_prefix(
            self.desc, out, out_dtype, q, self.k_pool, self.v_pool,
            torch.from_numpy(tables).to(self.device), torch.from_numpy(lens).to(self.device), hq,
            max_ctx, scale, torch.from_numpy(gs).to(self.device),
            torch.from_numpy(sh).to(self.device), len(sh), max_group, max_shared,
            partition_tokens, ws, stream)
        return out, {"group_start": gs, "shared_tokens": sh, "num_groups": len(sh),
                     "max_shared_tokens": max_shared, "max_group": max_group}

    def attend_prefill(self, seqs, q_counts, q, scale, out_dtype=None, stream=None,
                       out_fill=None):
        """Causal attention of each sequence's last q_counts[i] tokens (already appended and
        written) over its whole context: q is [sum(q_counts)][Hq][d] on the device, rows
        in sequence order."""
        tables, lens = self.block_tables(seqs)
        out_dtype = out_dtype or self.dtype
        counts = np.asarray(q_counts, dtype=np.int32)
        q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        max_ctx = int(lens.max()) if len(lens) else 1
        max_q = int(counts.max()) if len(counts) else 0
        hq, d = q.shape[1], q.shape[2]
        shape = (int(q_start[-1]), hq, d)
        out = (torch.empty(shape, dtype=TORCH_DTYPES[out_dtype], device=self.device)
               if out_fill is None else
               torch.full(shape, out_fill, dtype=TORCH_DTYPES[out_dtype], device=self.device))
        B.paged_attention_prefill(self.desc, out, out_dtype, q,
                                  torch.from_numpy(q_start).to(self.device), self.k_pool,
                                  self.v_pool, torch.from_numpy(tables).to(self.device),
                                  torch.from_numpy(lens).to(self.device), hq, max_q, max_ctx,
                                  scale, stream)
        return out, tables, lens
