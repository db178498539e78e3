"""Physical KV pool contents: layouts, cache writes and block copies.

Layouts (the pages leave memory layout open; these are the library's ABI and are
restated here from their definition, element by element):

  A block of more than 16 tokens is stored as NS = block_size / 16 sub-blocks of
  TB = 16 tokens, one after the other (block_size must then be a multiple of 16);
  up to 16 tokens, NS = 1 and TB = block_size.  The token at offset o of a block is
  token o % TB of sub-block o // TB.

  K pool  bits[num_blocks][kv_heads][NS * head_dim / X][TB][X]
          X = 16 bytes / element size (8 for fp16 and bf16, 4 for fp32): element
          d of the key of the token at offset o of block b, head h, sits at
          [b][h][(o // TB) * head_dim / X + d // X][o % TB][d % X].
  V pool  bits[num_blocks][kv_heads][NS * head_dim][TB]: element d of the value
          of the token at offset o sits at [b][h][(o // TB) * head_dim + d][o % TB].

A token's slot is physical block x block size + offset within the block (the
deeplearn.tn worked example places the fifth token in the first slot of the
second physical block).  Slot -1 marks a padding token that is not written.
"""
import numpy as np

from .lowp import BITS_DTYPE, poison_bits


def chunk_elems(dtype: str) -> int:
    return 16 // np.dtype(BITS_DTYPE[dtype]).itemsize


def sub_blocks(block_size):
    """(NS, TB): sub-blocks per block and tokens per sub-block."""
    if block_size <= 16:
        return 1, block_size
    if block_size % 16:
        raise ValueError("a block of more than 16 tokens must hold a multiple of 16")
    return block_size // 16, 16


def new_pool(num_blocks, kv_heads, block_size, head_dim, dtype):
    """Both pools filled with the all-ones pattern (NaN), so a slot that was never
    written is recognisable and poisons any result that reads it."""
    x = chunk_elems(dtype)
    if head_dim % x:
        raise ValueError("head_dim must be a multiple of the 16-byte chunk")
    ns, tb = sub_blocks(block_size)
    bits_t = BITS_DTYPE[dtype]
    k = np.full((num_blocks, kv_heads, ns * head_dim // x, tb, x), poison_bits(dtype), bits_t)
    v = np.full((num_blocks, kv_heads, ns * head_dim, tb), poison_bits(dtype), bits_t)
    return k, v


def _positions(slots, block_size, head_dim, x):
    """Block, K chunk-row indices [n][head_dim / X], V row indices [n][head_dim] and
    in-sub-block offset of each slot."""
    ns, tb = sub_blocks(block_size)
    blk, off = slots // block_size, slots % block_size
    sub, o = off // tb, off % tb
    krow = sub[:, None] * (head_dim // x) + np.arange(head_dim // x)[None, :]
    vrow = sub[:, None] * head_dim + np.arange(head_dim)[None, :]
    return blk, krow, vrow, o


def reshape_and_cache(k_pool, v_pool, key_bits, value_bits, slot_mapping, block_size):
    """Write token t's key and value rows ([kv_heads][head_dim] each) at slot_mapping[t]."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    if slots.size == 0:
        return
    if np.unique(slots).size != slots.size:
        raise ValueError("two tokens map to one slot")
    kv_heads, d = key_bits.shape[1], key_bits.shape[2]
    x = k_pool.shape[-1]
    blk, krow, vrow, o = _positions(slots, block_size, d, x)
    kb = np.asarray(key_bits)[keep].reshape(-1, kv_heads, d // x, x)
    vb = np.asarray(value_bits)[keep]
    # (array indices split by a slice: their broadcast shape [t][row] comes first)
    # K: [b][h][sub*d/X + d//X][o][d%X]  <-  key[t][h][d]
    k_pool[blk[:, None], :, krow, o[:, None], :] = kb.transpose(0, 2, 1, 3)
    # V: [b][h][sub*d + d][o]  <-  value[t][h][d]
    v_pool[blk[:, None], :, vrow, o[:, None]] = vb.transpose(0, 2, 1)


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
    if np.any(tab[t // block_size] < 0):
        raise ValueError("block table entry missing for a position below context_len")
    ns, _ = sub_blocks(block_size)
    kv_heads, x = k_pool.shape[1], k_pool.shape[4]
    d = k_pool.shape[2] * x // ns
    slots = tab[t // block_size] * block_size + t % block_size
    blk, krow, vrow, o = _positions(slots, block_size, d, x)
    k = k_pool[blk[:, None], :, krow, o[:, None], :].transpose(0, 2, 1, 3).reshape(len(t), kv_heads, d)
    v = v_pool[blk[:, None], :, vrow, o[:, None]].transpose(0, 2, 1)
    return k, v
