"""Fixed-partition MFMA decode for every query-head group width (GPU), against the oracle.

The matrix kernel packs a KV head's group of query heads into the 16 columns of its
products; its four waves' states are folded row by row (each wave taking a quarter of
the value columns), and only the group's rows are written.  Widths 2, 3, 5, 8 and 16 at
head_dim 64 and 128, with one-partition sequences (normalised in the partition launch)
and many-partition ones (partial states merged by the merge launch), outputs pre-filled
with NaN so that a row left unwritten fails.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as oreplay
from gpu_common import say, assert_close

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 64, 65, 200, 511, 513, 1100]


@pytest.mark.parametrize("group", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("pt", [64, 512])
def test_group_width_fixed_partitions(group, d, pt):
    from paged_kv_cache_15_amd.replay import run_workload
    dt = "bf16" if group % 2 else "f16"
    hkv = 2
    w = W.make_custom(LENS, group * hkv, hkv, d, dt, seed=group * 100 + d + pt)
    g = run_workload(w, "cuda", out_dtype="f32", partition_tokens=pt, out_fill=float("nan"))
    torch.cuda.synchronize()
    o = oreplay.run(w)
    assert len(g.outputs) == len(o.outputs)
    worst = 0.0
    for got, want in zip(g.outputs, o.outputs):
        worst = max(worst, assert_close(got, want, dt, "f32"))
    say(f"[group width] group={group} d={d} pt={pt} {dt} max|err| {worst:.3e}")
    g.cache.close()
