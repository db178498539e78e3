"""paged_attention_decode_static (the entry point that allocates nothing) against
paged_attention_decode with a caller workspace: the same kernels and schedule, so the
outputs must be bit-identical; two calls in a row, the second on a smaller batch (the
static scratch keeps the first call's contents, and its counters must be back at zero);
and a request too large for the scratch is refused before anything is launched."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import replay as oreplay
from gpu_common import say, assert_close

pytestmark = pytest.mark.gpu

# (dtype, q heads, kv heads, head_dim, partition_tokens): MFMA stream-K, MFMA 512-token
# partitions, VALU stream-K (group 1), fp32
CASES = [("bf16", 64, 8, 128, 0), ("bf16", 64, 8, 128, 512), ("f16", 16, 16, 128, 0),
         ("f32", 8, 2, 64, 512)]


def _decode_both(B, cache, w, seqs, q, pt):
    tables, lens = cache.block_tables(seqs)
    tab = torch.from_numpy(tables).cuda()
    bl = torch.from_numpy(lens).cuda()
    mx = int(lens.max())
    hq, d = w.num_q_heads, w.head_dim
    nb = B.paged_attention_workspace_bytes(cache.desc, len(seqs), hq, mx, pt)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
    ref = torch.full((len(seqs), hq, d), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    B.paged_attention_decode(cache.desc, ref, "f32", q, cache.k_pool, cache.v_pool, tab, bl, hq,
                             mx, float(w.scale), pt, ws)
    B.paged_attention_decode_static(cache.desc, got, "f32", q, cache.k_pool, cache.v_pool, tab,
                                    bl, hq, mx, float(w.scale), pt)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_static_scratch_matches_workspace_call(case):
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.replay import run_workload, to_device
    dt, hq, hkv, d, pt = case
    lens = [2900, 17, 1500, 4100, 1, 640, 2048, 333, 3700, 1200, 90, 2500]
    w = W.make_custom(lens, hq, hkv, d, dt, seed=71 + hq)
    g = run_workload(w, "cuda", out_dtype="f32", partition_tokens=pt, out_fill=float("nan"))
    seqs, qidx = w.attend_ops()[-1][1], w.attend_ops()[-1][2]
    q_all = to_device(w.q[qidx], dt, "cuda")
    o = oreplay.run(w)
    for rows in (list(range(len(lens))), [3, 0, 7]):          # the second call is smaller
        say(f"[no-alloc] {case} batch of {len(rows)}")
        ref, got = _decode_both(B, g.cache, w, [seqs[i] for i in rows], q_all[rows].contiguous(), pt)
        assert torch.isfinite(got).all()
        assert torch.equal(ref, got)
        assert_close(got, o.outputs[0][rows], dt, "f32")
    g.cache.close()


def test_static_scratch_refuses_oversized_requests():
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache
    c = PagedKVCache(64, 8, 128, "bf16")
    n, hq, mx = 64, 64, 65536
    q = torch.zeros((n, hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((n, hq, 128), 7.0, dtype=torch.float32, device="cuda")
    tab = torch.zeros((n, mx // 16), dtype=torch.int32, device="cuda")
    lens = torch.ones(n, dtype=torch.int32, device="cuda")
    # 16-token partitions over 65536 tokens: far more partial results than the scratch holds
    with pytest.raises(B.PagedKVError) as e:
        B.paged_attention_decode_static(c.desc, out, "f32", q, c.k_pool, c.v_pool, tab, lens, hq,
                                        mx, 0.1, 16)
    assert e.value.status == B.PAGED_KV_ERR_BUFFER_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())          # nothing was launched
    c.close()
