"""The five synthetic decode workloads (and reduced variants of each).

Every workload is a script of pool operations plus the random values they
consume.  Operations, in the order they are to be executed:

  ("create",)                         new empty sequence; ids are handed out 0, 1, 2, ...
  ("fork", parent)                    new sequence sharing all of parent's blocks
  ("append", seqs, counts, vidx)      append counts[i] tokens to seqs[i]; the K/V rows are
                                      kv[vidx] = (k, v), each float32 [sum(counts)][Hkv][d],
                                      rows grouped by sequence in the order of `seqs`
  ("free", seq)                       release a sequence
  ("attend", seqs, qidx)              one decode attention over `seqs`, queries q[qidx]
                                      (float32 [len(seqs)][Hq][d])

Values are float32 N(0, 1).  Casting them to the workload's storage type is
left to each consumer.  Seeds: workload k draws from numpy
``SeedSequence(k).spawn(3)`` = (lengths, free-queue order, values); the values
sequence spawns one child per draw, in op order.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = {
    1: "tiny_fp32_mha_d64",
    2: "mha_7b_b64_fp16",
    3: "gqa_72b_b128_bf16",
    4: "shared_prefix_32x8_bf16",
    5: "long_ctx_splitk_b16_bf16",
}

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # storage / compute-input type: "f32", "f16", "bf16"
    num_blocks: int
    free_order: np.ndarray          # int32 [num_blocks]: initial free-queue order, head first
    ops: list
    kv: list = field(default_factory=list)   # [(k, v)] float32 arrays per append op
    q: list = field(default_factory=list)    # float32 [B][Hq][d] per attend op
    scale: np.float32 = np.float32(1.0)
    block_size: int = 16
    partition_tokens: int = 0       # 0: stream-K schedule; > 0: fixed split-K partitions

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def attend_ops(self):
        return [op for op in self.ops if op[0] == "attend"]

    def final_lengths(self) -> dict:
        """Token count per sequence after the whole script (bookkeeping only)."""
        lens, nxt = {}, 0
        for op in self.ops:
            if op[0] == "create":
                lens[nxt] = 0
                nxt += 1
            elif op[0] == "fork":
                lens[nxt] = lens[op[1]]
                nxt += 1
            elif op[0] == "append":
                for s, n in zip(op[1], op[2]):
                    lens[s] += n
            elif op[0] == "free":
                del lens[op[1]]
        return lens


_CHUNK = 1 << 22
_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def _normal(ss, shape):
    """float32 N(0, 1) of `shape` from SeedSequence `ss`: the flat array is cut into
    chunks of 2**22 values, chunk i drawn from ss.spawn(n)[i] (filled in parallel
    threads; the values do not depend on the thread count)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    seeds = ss.spawn(max(1, -(-n // _CHUNK)))

    def fill(i):
        np.random.default_rng(seeds[i]).standard_normal(
            out=out[i * _CHUNK:(i + 1) * _CHUNK], dtype=np.float32)
    list(_POOL.map(fill, range(len(seeds))))
    return out.reshape(shape)


def _blocks(n_tokens: int, bs: int) -> int:
    return -(-int(n_tokens) // bs)


class _Builder:
    """Collects ops; each draw (K, V of an append; q of an attend) takes the next
    child of the values SeedSequence, in op order."""

    def __init__(self, ss_val, hkv, hq, d, draw_values=True):
        self.ss, self.hkv, self.hq, self.d = ss_val, hkv, hq, d
        self.draw_values = draw_values
        self.ops, self.kv, self.q = [], [], []
        self.next_id = 0

    def create(self):
        self.ops.append(("create",))
        self.next_id += 1
        return self.next_id - 1

    def fork(self, parent):
        self.ops.append(("fork", parent))
        self.next_id += 1
        return self.next_id - 1

    def append(self, seqs, counts):
        seqs, counts = [int(s) for s in seqs], [int(c) for c in counts]
        total = sum(counts)
        if self.draw_values:
            k = _normal(self.ss.spawn(1)[0], (total, self.hkv, self.d))
            v = _normal(self.ss.spawn(1)[0], (total, self.hkv, self.d))
            self.kv.append((k, v))
        else:
            self.kv.append(None)
        self.ops.append(("append", seqs, counts, len(self.kv) - 1))

    def attend(self, seqs):
        self.q.append(_normal(self.ss.spawn(1)[0], (len(seqs), self.hq, self.d))
                      if self.draw_values else None)
        self.ops.append(("attend", [int(s) for s in seqs], len(self.q) - 1))

    def prefill(self, seqs, counts):
        """Causal attention of each sequence's last counts[i] tokens (one query row each)."""
        counts = [int(c) for c in counts]
        self.q.append(_normal(self.ss.spawn(1)[0], (sum(counts), self.hq, self.d))
                      if self.draw_values else None)
        self.ops.append(("prefill", [int(s) for s in seqs], counts, len(self.q) - 1))

    def free(self, seq):
        self.ops.append(("free", int(seq)))


def _prefill_then_decode(name, lens, hq, hkv, d, dtype, num_blocks, rng_pool, rng_val,
                         steps=1, prefill_excludes=1, draw_values=True):
    """Prefill every sequence, then `steps` decode steps of one token each.

    With steps == 1 the listed length is the attention length of the one decode
    step, so each sequence is prefilled with len - 1 tokens (prefill_excludes=1).
    """
    b = _Builder(rng_val, hkv, hq, d, draw_values)
    seqs = [b.create() for _ in lens]
    pre = [int(L) - prefill_excludes for L in lens]
    if sum(pre) > 0:
        nz = [(s, n) for s, n in zip(seqs, pre) if n > 0]
        b.append([s for s, _ in nz], [n for _, n in nz])
    for _ in range(steps):
        b.append(seqs, [1] * len(seqs))
        b.attend(seqs)
    free_order = rng_pool.permutation(num_blocks).astype(np.int32)
    return Workload(name=name, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                    num_blocks=num_blocks, free_order=free_order, ops=b.ops, kv=b.kv, q=b.q,
                    scale=np.float32(1.0 / math.sqrt(d)))


def _pool_size(logical_blocks: int) -> int:
    return int(math.ceil(1.25 * logical_blocks))


def make_config(k: int, small: bool = False, draw_values: bool = True, block_size: int = 16,
                head_dim: int = None) -> Workload:
    """Workload k in 1..5.  small=True keeps heads, head_dim, type and block size
    but shrinks batch and lengths so the oracle finishes in seconds (still several
    512-token partitions with ragged tails).  draw_values=False builds the script
    only (lengths, pool order and operations are the same; kv and q hold None).
    block_size / head_dim (workloads 2, 3 and 5) give the same lengths over a pool of
    another block size (sized 1.25x its own need) or heads of another size."""
    dv = draw_values
    ss = np.random.SeedSequence(k + (100 if small else 0)).spawn(3)
    rng_len, rng_pool = (np.random.default_rng(s) for s in ss[:2])
    rng_val = ss[2]           # values: SeedSequence, children spawned per draw
    name = CONFIG_NAMES[k] + ("_small" if small else "")
    bs = int(block_size)
    if (bs != 16 or head_dim is not None) and k not in (2, 3, 5):
        raise ValueError(f"workload {k} has no block-size or head-size variants")
    if bs != 16:
        name += f"_bs{bs}"
    if head_dim is not None:
        name += f"_d{int(head_dim)}"

    def variant(w):
        w.block_size = bs
        return w
    if k == 1:
        lens = [7, 16, 33, 100]
        return _prefill_then_decode(name, lens, 4, 4, 64, "f32", 64, rng_pool, rng_val,
                                    draw_values=dv)
    if k == 2:
        B, lo, hi = (4, 512, 1500) if small else (64, 512, 4096)
        lens = rng_len.integers(lo, hi, size=B, endpoint=True)
        nb = _pool_size(sum(_blocks(L, bs) for L in lens))
        return variant(_prefill_then_decode(name, lens, 32, 32, head_dim or 128, "f16", nb,
                                            rng_pool, rng_val, draw_values=dv))
    if k == 3:
        B, med, cap = (6, 600, 2048) if small else (128, 2048, 8192)
        raw = rng_len.lognormal(mean=math.log(med), sigma=0.6, size=B)
        lens = np.clip(np.rint(raw), 1, cap).astype(np.int64)
        nb = _pool_size(sum(_blocks(L, bs) for L in lens))
        return variant(_prefill_then_decode(name, lens, 64, 8, head_dim or 128, "bf16", nb,
                                            rng_pool, rng_val, draw_values=dv))
    if k == 4:
        prompts = 2 if small else 32
        w = _shared_prefix(name, prompts, 8, 2056, (64, 512), rng_len, rng_pool, rng_val,
                           draw_values=dv)
        # siblings that share prefix blocks are adjacent workgroups in the partition grid
        # (and land on one L2 when the KV-head count is a multiple of 8): measured faster
        # than the stream-K schedule, which reads each sibling's prefix at a different time
        w.partition_tokens = 512
        return w
    if k == 5:
        B, lo, hi = (2, 1500, 2500) if small else (16, 16384, 32768)
        L0 = rng_len.integers(lo, hi, size=B, endpoint=True)
        nb = _pool_size(sum(_blocks(L + 8, bs) for L in L0))
        w = variant(_prefill_then_decode(name, L0, 64, 8, head_dim or 128, "bf16", nb, rng_pool,
                                         rng_val, steps=8, prefill_excludes=0, draw_values=dv))
        w.partition_tokens = 512     # the long-context workload is defined with 512-token partitions
        return w
    raise ValueError(f"no workload {k}")


def _shared_prefix(name, prompts, samples, prompt_len, tail_range, rng_len, rng_pool, rng_val,
                   share=True, draw_values=True):
    """Parallel sampling: each prompt is written once and forked `samples - 1` times;
    every sample then grows its own tail.  The last tail token is the decode step's
    appended token.  With share=False every sample writes its own copy of the prompt
    (same values) instead of forking: the physically copied counterpart."""
    hq, hkv, d, bs = 32, 8, 128, 16
    b = _Builder(rng_val, hkv, hq, d, draw_values)
    tails = rng_len.integers(tail_range[0], tail_range[1], size=(prompts, samples), endpoint=True)
    all_seqs = []
    prompt_vals = []
    for p in range(prompts):
        if share:
            s0 = b.create()
            b.append([s0], [prompt_len])
            group = [s0] + [b.fork(s0) for _ in range(samples - 1)]
        else:
            group = [b.create() for _ in range(samples)]
            # one draw for the prompt, re-used by every sample of the group
            b.append([group[0]], [prompt_len])
            shared = b.kv[-1]
            for s in group[1:]:
                b.kv.append(shared)
                b.ops.append(("append", [s], [prompt_len], len(b.kv) - 1))
        prompt_vals.append(group)
        all_seqs += group
    counts = [int(t) - 1 for t in tails.reshape(-1)]
    b.append(all_seqs, counts)
    b.append(all_seqs, [1] * len(all_seqs))
    b.attend(all_seqs)
    full, part = divmod(prompt_len, bs)
    if share:
        unique = prompts * full + sum(_blocks(part + int(t), bs) for t in tails.reshape(-1))
    else:
        unique = sum(_blocks(prompt_len + int(t), bs) for t in tails.reshape(-1))
    nb = _pool_size(unique)
    free_order = rng_pool.permutation(nb).astype(np.int32)
    return Workload(name=name, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype="bf16",
                    num_blocks=nb, free_order=free_order, ops=b.ops, kv=b.kv, q=b.q,
                    scale=np.float32(1.0 / math.sqrt(d)))


def make_shared_prefix_pair(small: bool = True, prompt_len: int = 2056):
    """The same parallel-sampling draw twice: once with forked (refcounted) prefix
    blocks, once with every sample holding its own copy.  Both use identical values."""
    out = []
    for share in (True, False):
        ss = np.random.SeedSequence(4 + (100 if small else 0)).spawn(3)
        rng_len, rng_pool = (np.random.default_rng(s) for s in ss[:2])
        rng_val = ss[2]
        prompts = 2 if small else 32
        out.append(_shared_prefix(f"shared_prefix_share{int(share)}", prompts, 8, prompt_len,
                                  (64, 512), rng_len, rng_pool, rng_val, share=share))
    return out


def make_custom(lengths, num_q_heads, num_kv_heads, head_dim, dtype, seed=0, num_blocks=None,
                free_order=None, steps=1, block_size=16):
    """A prefill-then-decode workload with the given attention lengths (edge cases)."""
    ss = np.random.SeedSequence(1000 + seed).spawn(3)
    rng_pool, rng_val = np.random.default_rng(ss[1]), ss[2]
    lens = [int(x) for x in lengths]
    if num_blocks is None:
        num_blocks = max(1, _pool_size(sum(_blocks(L + steps - 1, block_size) for L in lens)))
    w = _prefill_then_decode(f"custom_{seed}", lens, num_q_heads, num_kv_heads, head_dim, dtype,
                             num_blocks, rng_pool, rng_val, steps=steps)
    w.block_size = block_size
    if free_order is not None:
        w.free_order = np.asarray(free_order, dtype=np.int32)
    return w


PREFILL_NAMES = {
    1: "prefill_gqa_b16_bf16",
    2: "chunked_prefill_gqa_b32_bf16",
}


def make_prefill(prefix_lens, chunk_rounds, num_q_heads, num_kv_heads, head_dim, dtype,
                 seed=0, block_size=16, name=None, draw_values=True):
    """Sequences that already hold prefix_lens[i] tokens, then for each round of
    chunk_rounds (a list of per-sequence token counts) an append of that many tokens and
    a prefill op over them (the sequences with a count > 0)."""
    ss = np.random.SeedSequence(2000 + seed).spawn(3)
    rng_pool, rng_val = np.random.default_rng(ss[1]), ss[2]
    b = _Builder(rng_val, num_kv_heads, num_q_heads, head_dim, draw_values)
    seqs = [b.create() for _ in prefix_lens]
    nz = [(s, int(n)) for s, n in zip(seqs, prefix_lens) if int(n) > 0]
    if nz:
        b.append([s for s, _ in nz], [n for _, n in nz])
    total = [int(n) for n in prefix_lens]
    for counts in chunk_rounds:
        live = [(s, int(c)) for s, c in zip(seqs, counts) if int(c) > 0]
        if not live:
            continue
        b.append([s for s, _ in live], [c for _, c in live])
        b.prefill([s for s, _ in live], [c for _, c in live])
        for i, c in enumerate(counts):
            total[i] += int(c)
    nb = max(1, _pool_size(sum(_blocks(t, block_size) for t in total)))
    w = Workload(name=name or f"prefill_{seed}", num_q_heads=num_q_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, dtype=dtype, num_blocks=nb,
                 free_order=rng_pool.permutation(nb).astype(np.int32), ops=b.ops, kv=b.kv,
                 q=b.q, scale=np.float32(1.0 / math.sqrt(head_dim)))
    w.block_size = block_size
    return w


def make_prefill_config(k: int, small: bool = False, draw_values: bool = True,
                        block_size: int = 16, head_dim: int = 128) -> Workload:
    """Prefill workloads on the GQA 72B shape (64 query heads over 8 KV heads, bf16):
    1: whole prompts, 16 sequences, lengths lognormal around 2048 (capped at 8192);
    2: chunked prefill, 32 sequences holding lognormal contexts around 2048 that each
       take a 512-token chunk.  small=True: 3 sequences around 300 tokens (chunk 96)."""
    ss = np.random.SeedSequence(3000 + k + (100 if small else 0)).spawn(1)[0]
    rng_len = np.random.default_rng(ss)
    name = PREFILL_NAMES[k] + ("_small" if small else "")
    if block_size != 16:
        name += f"_bs{block_size}"
    if head_dim != 128:
        name += f"_d{head_dim}"
    B, med, cap, chunk = (3, 300, 700, 96) if small else ((16, 2048, 8192, 512) if k == 1
                                                           else (32, 2048, 8192, 512))
    if k == 1:
        lens = np.clip(np.rint(rng_len.lognormal(math.log(med), 0.6, size=B)), 16, cap).astype(int)
        return make_prefill([0] * B, [list(lens)], 64, 8, head_dim, "bf16", seed=10 + k,
                            block_size=block_size, name=name, draw_values=draw_values)
    if k == 2:
        ctx = np.clip(np.rint(rng_len.lognormal(math.log(med), 0.6, size=B)), 0, cap).astype(int)
        return make_prefill(list(ctx), [[chunk] * B], 64, 8, head_dim, "bf16", seed=10 + k,
                            block_size=block_size, name=name, draw_values=draw_values)
    raise ValueError(f"no prefill workload {k}")
