"""Physical KV pool contents: layouts, cache writes and block copies.

Layouts (the pages leave memory layout open; these are the library's ABI and are
restated here from their definition, element by element):

  K pool  bits[num_blocks][kv_heads][head_dim / X][block_size][X]
          X = 16 bytes / element size (8 for fp16 and bf16, 4 for fp32): element
          d of the key of the token at offset o of block b, head h, sits at
          [b][h][d // X][o][d % X].
  V pool  bits[num_blocks][kv_heads][head_dim][block_size]: element d of the value
          of the token at offset o sits at [b][h][d][o].

A token's slot is physical block x block size + offset within the block (the
deeplearn.tn worked example places the fifth token in the first slot of the
second physical block).  Slot -1 marks a padding token that is not written.
"""
import numpy as np

from .lowp import BITS_DTYPE, poison_bits


def chunk_elems(dtype: str) -> int:
    return 16 // np.dtype(BITS_DTYPE[dtype]).itemsize


def new_pool(num_blocks, kv_heads, block_size, head_dim, dtype):
    """Both pools filled with the all-ones pattern (NaN), so a slot that was never
    written is recognisable and poisons any result that reads it."""
    x = chunk_elems(dtype)
    if head_dim % x:
        raise ValueError("head_dim must be a multiple of the 16-byte chunk")
    bits_t = BITS_DTYPE[dtype]
    k = np.full((num_blocks, kv_heads, head_dim // x, block_size, x), poison_bits(dtype), bits_t)
    v = np.full((num_blocks, kv_heads, head_dim, block_size), poison_bits(dtype), bits_t)
    return k, v


def reshape_and_cache(k_pool, v_pool, key_bits, value_bits, slot_mapping, block_size):
    """Write token t's key and value rows ([kv_heads][head_dim] each) at slot_mapping[t]."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    if slots.size == 0:
        return
    if np.unique(slots).size != slots.size:
        raise ValueError("two tokens map to one slot")
    blk, off = slots // block_size, slots % block_size
    kv_heads, d = key_bits.shape[1], key_bits.shape[2]
    x = k_pool.shape[-1]
    kb = np.asarray(key_bits)[keep].reshape(-1, kv_heads, d // x, x)
    vb = np.asarray(value_bits)[keep]
    # K: [b][h][d//X][o][d%X]  <-  key[t][h][d]
    k_pool[blk, :, :, off, :] = kb
    # V: [b][h][d][o]  <-  value[t][h][d]
    v_pool[blk, :, :, off] = vb


def copy_block(k_pool, v_pool, src, dst):
    """Copy-on-write: the destination block becomes an exact copy of the source."""
    k_pool[dst] = k_pool[src]
    v_pool[dst] = v_pool[src]


def gather_sequence(k_pool, v_pool, table, context_len, block_size):
    """Reassemble one sequence's keys and values in logical order through its table.

    Returns bits arrays K[context_len][kv_heads][head_dim], V[...] (same shape).
    """
    t = np.arange(int(context_len))
    tab = np.asarray(table, dtype=np.int64)
    blk = tab[t // block_size]
    off = t % block_size
    if np.any(blk < 0):
        raise ValueError("block table entry missing for a position below context_len")
    kv_heads, nchunk, x = k_pool.shape[1], k_pool.shape[2], k_pool.shape[4]
    k = k_pool[blk, :, :, off, :].reshape(len(t), kv_heads, nchunk * x)
    v = v_pool[blk, :, :, off]
    return k, v
