"""Fixed partitions whose states come from the stream-K schedule (GPU).

Large batches of long contexts at a fixed partition size have each partition's (max,
sum, weighted values) state computed by the stream-K kernel: each wave streams a
contiguous run of tiles and cuts its state at every partition boundary, so a partition
that a slice boundary crosses arrives as two pieces, which the merge kernel folds in
order.  At 128-token partitions over 19 sequences of up to 4096 tokens most slices cut a
partition, and with 16 query heads per KV head the wave's LDS holds only three pieces,
so the direct stores past it run too.  Checked against the oracle for every pool type,
head size, block size and group width the mode serves.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as oreplay
from gpu_common import say, assert_close

pytestmark = pytest.mark.gpu

# (dtype, q heads, kv heads, head_dim, block size)
CASES = [("bf16", 64, 8, 128, 16), ("f16", 64, 8, 128, 16), ("bf16", 64, 8, 64, 32),
         ("bf16", 32, 8, 256, 16), ("bf16", 128, 8, 128, 16), ("f16", 16, 8, 128, 32)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_partition_states_on_the_stream_k_schedule(case):
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.replay import run_workload
    dt, hq, hkv, d, bs = case
    rng = np.random.default_rng(hq + d + bs)
    lens = [int(x) for x in rng.integers(1024, 4097, 16)] + [1, 129, 4096]
    w = W.make_custom(lens, hq, hkv, d, dt, seed=hq + d, block_size=bs)
    g = run_workload(w, "cuda", out_dtype="f32", partition_tokens=128, out_fill=float("nan"))
    torch.cuda.synchronize()
    # the mode is in use: its workspace holds two rows per partition
    max_ctx = max(lens)
    parts = -(-max_ctx // 128)
    rows = len(lens) * hq * parts
    nbytes = B.paged_attention_workspace_bytes(g.cache.desc, len(lens), hq, max_ctx, 128)
    assert nbytes >= 2 * rows * (d + 2) * 4
    o = oreplay.run(w)
    err = assert_close(g.outputs[0], o.outputs[0], dt, "f32")
    say(f"[partition states] {case} max|err| {err:.3e}")
    g.cache.close()
