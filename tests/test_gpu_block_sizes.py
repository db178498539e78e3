"""Block sizes 1, 16 and 32 with head_dim 64, 128 and 256 (GPU), against the oracle.

Pools, slot mappings, tables and copy pairs bit-exact; attention within the tolerance
of the input type, on both schedules (stream-K and 512-token partitions) and both
kernel families (MFMA: fp16/bf16 with several query heads per KV head; VALU: one query
head per KV head, or fp32).  The lengths straddle the 16-token tile and the 1-, 16-
and 32-token block boundaries, and the decode steps append across them.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as oreplay
from gpu_common import say, assert_pools_equal, assert_bookkeeping_equal, assert_close

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 100, 511, 512, 513, 1100]

# (dtype, q heads, kv heads, head_dim)
SHAPES = [("bf16", 16, 2, 128), ("f16", 4, 4, 128), ("f32", 4, 4, 64), ("bf16", 8, 2, 64),
          ("bf16", 8, 2, 256), ("f16", 4, 4, 256), ("f32", 2, 2, 256)]


def _run(w, out_dtype, pt):
    from paged_kv_cache_15_amd.replay import run_workload
    g = run_workload(w, "cuda", out_dtype=out_dtype, partition_tokens=pt)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("pt", [0, 512], ids=["streamk", "pt512"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
@pytest.mark.parametrize("bs", [1, 32, 16])
def test_block_size_parity(bs, shape, pt):
    dt, hq, hkv, d = shape
    w = W.make_custom(LENS, hq, hkv, d, dt, seed=hq * 5 + d + bs, steps=3, block_size=bs)
    say(f"[block-size] bs={bs} {shape} partition_tokens={pt}")
    out_dtype = "f32" if dt == "f32" else dt
    g = _run(w, out_dtype, pt)
    o = oreplay.run(w)
    assert_bookkeeping_equal(g, o)
    assert_pools_equal(g.cache, o, dt)
    for go, oo in zip(g.outputs, o.outputs):
        err = assert_close(go, oo, dt, out_dtype)
        say(f"   max|err| {err:.3e}")
    g.cache.close()


@pytest.mark.parametrize("bs", [1, 32])
def test_block_size_fork_and_copy_on_write(bs):
    """The shared-prefix workload (forks, copy-on-write of partial tail blocks) at
    another block size: the pool is resized to hold the same tokens.  With one token
    per block there is never a partial block, so no copy is ever made."""
    w = W.make_config(4, small=True)
    w.block_size = bs
    if bs < 16:
        w.num_blocks *= 16 // bs
        w.free_order = np.random.default_rng(77).permutation(w.num_blocks).astype(np.int32)
    say(f"[block-size] shared prefix bs={bs} blocks={w.num_blocks}")
    for pt in (0, 512):
        g = _run(w, "f32", pt)
        o = oreplay.run(w)
        assert_bookkeeping_equal(g, o)
        if bs > 1:
            assert any(len(c) for c in o.copies), "workload made no copy-on-write copies"
        else:   # a one-token block is always full: sharing never needs a copy
            assert not any(len(c) for c in o.copies)
        assert_pools_equal(g.cache, o, w.dtype)
        for go, oo in zip(g.outputs, o.outputs):
            err = assert_close(go, oo, w.dtype, "f32")
            say(f"   partition_tokens={pt} max|err| {err:.3e}")
        g.cache.close()
