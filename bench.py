#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

A step is one pass of the decode hot path over one batch already resident in HBM:
  reshape_and_cache  (write each sequence's new token into its slot)
  paged attention    (the partition launch: by default the stream-K schedule, which
                      also merges split (sequence, KV head) units in-kernel; with fixed
                      partitions, one workgroup per (sequence, head, partition))
  partition merge    (the reduce launch: log-sum-exp merge of fixed partitions; it only
                      validates its arguments under the stream-K schedule)
for, by default, the GQA workload of 128 sequences, 64 query heads over 8 KV heads, head_dim 128,
bf16 KV, 16-token blocks scattered through a pool 1.25x the need, context lengths
lognormal around 2048 (capped at 8192).  The host allocator's work for the step
(slot reservation) happens before timing; the step re-writes the same slots, so every
step is the same work.

Prints one JSON line: decode KV GB/s over the whole step (algorithmic bytes / step
time, over K steps with nothing else queued), seq-tokens/s, the partition kernel
against the HBM roofline (HIP events on the launch stream, over K more steps), the
kernel's measured HBM traffic when a committed counter summary under profiles/ matches
the current kernel sources, and the CPU oracle timed on the host cores as a baseline.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: GQA 72B shape)")
    ap.add_argument("--block-size", type=int, default=16,
                    help="tokens per block of the pool (1, 16 or 32; workloads 2, 3 and 5)")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="head size of the workload's heads (64, 128 or 256; workloads 2, 3, 5)")
    ap.add_argument("--prefill", type=int, default=0, metavar="K",
                    help="time paged prefill workload K (1: whole prompts, 2: chunked) instead "
                         "of the decode step, and print its line")
    ap.add_argument("--partition-tokens", type=int, default=None,
                    help="0: stream-K schedule; > 0: fixed partitions; -1: picked by batch shape "
                         "(default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's timed CPU work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the decode step (no prefill, graph-step and step-loop lines)")
    ap.add_argument("--decode-graph", action="store_true",
                    help="only time the graph-captured 32-layer decode step of 8 sequences and "
                         "print that line")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="only time the parallel-sampling workload (per-sample and shared-prefix "
                         "decode) and print that line")
    ap.add_argument("--shared-partition-tokens", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times) and exit: the "
                         "known-size reference for scaling HBM byte counters")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


# Sources that determine the attention kernels' code and launch shape; a counter summary
# records their digest, and its traffic figure is only reported while they match.
KERNEL_SOURCES = ("paged_kv_cache_15_amd/csrc/common.h",
                  "paged_kv_cache_15_amd/csrc/attention_common.h",
                  "paged_kv_cache_15_amd/csrc/attention_host.h",
                  "paged_kv_cache_15_amd/csrc/decode_attention.hip",
                  "paged_kv_cache_15_amd/csrc/decode_attention_streamk.hip")


def code_text(src: str) -> str:
    """A source's code without comments and blank space: what the compiler sees of it
    (a comment edit does not change the kernel the counters were taken on)."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).strip() for ln in src.splitlines())
    return "\n".join(" ".join(ln.split()) for ln in lines if ln)


def kernel_source_digest(read=None):
    """SHA-256 over the code text of the kernel sources (`read` maps a path to its text;
    default: the files in this tree)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(code_text(text).encode())
    return h.hexdigest()


def measured_traffic(workload, partition_tokens):
    """HBM bytes per launch of the partition kernel from a committed counter summary
    (profiles/*_hbm_bytes.txt: FETCH_SIZE and WRITE_SIZE scaled by a plain copy's
    readings) for this workload and schedule, or None if none matches the current
    kernel sources."""
    digest = kernel_source_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_bytes.txt"))):
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith((" ", "#", "|")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if (kv.get("workload") == workload and kv.get("partition_tokens") == str(partition_tokens)
                and kv.get("kernel_source_sha256") == digest and "traffic_bytes_per_launch" in kv):
            return int(kv["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    return None, None


def attention_bytes(lens, nblocks, w, out_elem):
    kv = int(lens.sum()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    q = len(lens) * w.num_q_heads * w.head_dim * w.elem_bytes
    out = len(lens) * w.num_q_heads * w.head_dim * out_elem
    return kv, kv + q + out + 4 * int(nblocks) + 4 * len(lens)


SCRUB_BYTES = 512 << 20     # written between timed launches: evicts L2 and the 256 MB MALL


class Scrubber:
    """A 512 MB buffer written (outside the timed region) before each timed launch, so
    no launch finds the previous one's data in the L2s or the Infinity Cache."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.int32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n)


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


def timed_launches(launch, stream, iters, scrub, before=None):
    """HIP events on `stream` around `launch()` for `iters` launches; before each one
    `scrub()` and then `before()` (untimed).  Returns the durations in ms."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        scrub()
        if before is not None:
            before()
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def read_bandwidth(dev, stream, iters=20, nbytes=2 << 30):
    """The streaming-read probe over a 2 GiB buffer: the measured second denominator."""
    import torch
    from paged_kv_cache_15_amd import binding as B
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    scrub = Scrubber(dev)
    B.paged_kv_read_bandwidth_probe(buf, sink, stream=stream)
    ms = timed_launches(lambda: B.paged_kv_read_bandwidth_probe(buf, sink, stream=stream), stream,
                        iters, scrub)
    st = percentiles(ms)
    del buf, scrub
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "launch_ms": st, "GB_per_s": round(nbytes / (st["median"] * 1e-3) / 1e9, 1)}


def cpu_baseline(w, seconds):
    """The oracle's attention on the same workload, timed on the host cores over a
    bounded prefix of the batch (pool build and input rounding are not timed)."""
    import numpy as np
    from oracle import replay as oreplay
    from oracle.attention import paged_decode
    from oracle.lowp import to_storage_bits, storage_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    log("[bench] cpu baseline: oracle replay (untimed)")
    r = oreplay.run(w, compute_attention=False)
    attends = w.attend_ops()
    qidx = attends[-1][2]
    tables, lens = r.tables[-1], r.context_lens[-1]
    q = storage_bits_to_f64(to_storage_bits(w.q[qidx], w.dtype), w.dtype)
    # sequences in batch order, wrapping round, until `seconds` of CPU work are spent
    done, kv_bytes, ctx_tokens = 0, 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        i = done % len(lens)
        paged_decode(q, r.k_pool, r.v_pool, tables, lens, w.scale, w.dtype, w.block_size,
                     seqs=[i])
        kv_bytes += int(lens[i]) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
        ctx_tokens += int(lens[i])
        done += 1
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {
        "value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
        "blas_threads": blas_threads, "kind": "oracle",
        "seq_tokens_per_s": round(done / dt, 3),
        "sample": f"fp64 NumPy oracle attention over {done} sequence decodes of the same step "
                  f"({done / len(lens):.2f} passes over its {len(lens)} sequences, "
                  f"{ctx_tokens} context tokens), {dt:.1f} s",
        "prefix_cache": prefix_cache_oracle(),
    }


def _prefix_requests():
    """The prefix-cache request stream: 32 prompts of 2056 token ids, each requested 8
    times, and the pool size that holds them."""
    import numpy as np
    rng = np.random.default_rng(4)
    prompts = [rng.integers(0, 50000, 2056).tolist() for _ in range(32)]
    order = [p for p in prompts for _ in range(8)]
    return prompts, order, 32 * 129 * 2, 16


def prefix_cache_host():
    """Host cost of prefix caching (deepsonar §2.4 hash chain) on the shared-prefix shape:
    a request matches its prompt against the cache, appends the uncached rest with token
    ids and is then released (library: C++ SHA-256 + allocator)."""
    from paged_kv_cache_15_amd import binding as B
    prompts, order, nb, bs = _prefix_requests()
    desc = B.make_desc(nb, bs, 8, 128, "bf16", B.PAGED_KV_POOL_HOST_ONLY | B.PAGED_KV_POOL_PREFIX_CACHE)
    pool = B.paged_kv_pool_create(desc)
    hit_tokens = 0
    t0 = time.perf_counter()
    for pr in order:
        s, n = B.paged_kv_seq_create_prefix(pool, pr)
        B.paged_kv_seq_append_tokens(pool, s, pr[n:])
        B.paged_kv_seq_free(pool, s)
        hit_tokens += n
    t_lib = time.perf_counter() - t0
    B.paged_kv_pool_destroy(pool)
    hashed = sum((len(p) - 1) // bs for p in order) + sum(len(p) // bs for p in prompts)
    return {"requests": len(order), "prompt_tokens": 2056, "hit_tokens": hit_tokens,
            "library_us_per_request": round(t_lib / len(order) * 1e6, 2),
            "library_block_hashes_per_s": round(hashed / t_lib, 1)}


def prefix_cache_oracle(seconds_cap=5.0):
    """The oracle's prefix-caching allocator (Python, hashlib) on the same request stream,
    timed as part of the CPU baseline."""
    from oracle import prefix_cache as opc
    prompts, order, nb, bs = _prefix_requests()
    al = opc.PrefixCachingAllocator(nb, bs)
    t0, done = time.perf_counter(), 0
    for pr in order:
        s, n = al.create_prefix(pr)
        al.append_tokens(s, pr[n:])
        al.release(s)
        done += 1
        if time.perf_counter() - t0 > seconds_cap:
            break
    return {"us_per_request": round((time.perf_counter() - t0) / done * 1e6, 2), "requests": done}


def decode_graph_timing(layers=32, reps=20, partition_tokens=None):
    """Launch cost of a small decode batch: one step of `layers` layers (cache write +
    paged attention each, fused into one launch per layer) over 8 sequences of the GQA
    shape (64 q / 8 kv heads, d 128, bf16, contexts 256..2048), launched eagerly vs
    replayed from a HIP graph.  The same step is re-run (idempotent), HIP events around
    `reps` repetitions."""
    import numpy as np
    import torch
    from paged_kv_cache_15_amd.graph import LayeredKV, DecodeStep
    from paged_kv_cache_15_amd.replay import to_device
    rng = np.random.default_rng(9)
    lens = rng.integers(256, 2049, 8).tolist()
    nb = sum((n + 16) // 16 + 1 for n in lens) + 8
    kv = LayeredKV(layers, nb, 8, 128, "bf16", 16, rng.permutation(nb), poison=False)
    seqs = [kv.cache.create() for _ in lens]
    keys = [to_device(rng.standard_normal((sum(lens), 8, 128)).astype(np.float32), "bf16", "cuda")] * layers
    kv.append(seqs, lens, keys, keys)
    mx = max(lens) + 1
    from paged_kv_cache_15_amd import binding as B
    pt = (B.paged_attention_auto_partition_tokens(kv.desc, len(lens), 64, mx)
          if partition_tokens is None else partition_tokens)
    st = DecodeStep(kv, len(lens), 64, (mx + 15) // 16, mx, 1 / np.sqrt(128.0),
                    B.PARTITION_AUTO if partition_tokens is None else partition_tokens, "bf16")
    nk = to_device(rng.standard_normal((layers, len(lens), 8, 128)).astype(np.float32), "bf16", "cuda")
    q = to_device(rng.standard_normal((layers, len(lens), 64, 128)).astype(np.float32), "bf16", "cuda")
    st.set_step(seqs, nk, nk, q)
    st.capture()
    res = {}
    for name, fn in (("eager", st.launch), ("graph", st.replay)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / reps
    kv.close()
    return {"layers": layers, "batch": len(lens), "partition_tokens": pt,
            # fused decode step: one launch per layer, except under stream-K (cache write
            # and attention)
            "launches_per_step": (2 if pt == 0 else 1) * layers,
            "eager_us_per_step": round(res["eager"], 1), "graph_us_per_step": round(res["graph"], 1)}


def long_context_step_loop(dev, iters=50):
    """The long-context workload's eight decode steps as a serving loop runs them (16
    sequences of 16k-32k tokens, 64 q / 8 kv heads, d 128, bf16, 512-token partitions
    merged by log-sum-exp).  Per step: the host allocator reserves one slot per sequence,
    the slot mapping, block tables and lengths are copied to the device, then the cache
    write and attention (partition + merge launches) run; the step ends with a device
    synchronisation.  Each part is timed (host parts by the wall clock, device parts by
    HIP events), and so is the whole step.  The new tokens' K/V and the queries are on the
    device before the loop (a model produces them there).  After the loop, the attention
    of the last step is timed on its own (median of `iters` scrubbed launches)."""
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache, TORCH_DTYPES
    from paged_kv_cache_15_amd.replay import to_device
    w = W.make_config(5)
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, w.block_size,
                         w.free_order, device=dev)
    stream = torch.cuda.current_stream(dev)
    ops = [op for op in w.ops]
    steps, pending = [], None
    for op in ops:
        if op[0] == "create":
            cache.create()
        elif op[0] == "append" and sum(op[2]) > len(op[1]):            # the prefill
            k, v = w.kv[op[3]]
            cache.append(op[1], op[2], to_device(k, w.dtype, dev), to_device(v, w.dtype, dev))
        elif op[0] == "append":
            k, v = w.kv[op[3]]
            pending = (op[1], op[2], to_device(k, w.dtype, dev), to_device(v, w.dtype, dev))
        elif op[0] == "attend":
            steps.append(pending + (to_device(w.q[op[2]], w.dtype, dev),))
    torch.cuda.synchronize()
    seqs = steps[0][0]
    hq, d, pt = w.num_q_heads, w.head_dim, w.partition_tokens
    final_lens = [L for L in w.final_lengths().values()]
    max_ctx = int(max(final_lens))
    max_blocks = (max_ctx + w.block_size - 1) // w.block_size
    nbytes = B.paged_attention_workspace_bytes(cache.desc, len(seqs), hq, max_ctx, pt)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((len(seqs), hq, d), dtype=TORCH_DTYPES[w.dtype], device=dev)

    def attend(tables_d, lens_d):
        B.paged_attention_partition(cache.desc, out, w.dtype, q, cache.k_pool, cache.v_pool,
                                    tables_d, lens_d, hq, max_ctx, float(w.scale), pt, ws, stream)
        B.paged_attention_reduce(cache.desc, out, w.dtype, lens_d, hq, max_ctx, pt, ws, stream)

    # warm-up: attention over the prefilled state (read-only)
    q = steps[0][4]
    t, L = cache.block_tables(seqs, max_blocks)
    attend(torch.from_numpy(t).to(dev), torch.from_numpy(L).to(dev))
    torch.cuda.synchronize()
    rows, total_bytes = [], 0
    t_loop = time.perf_counter()
    for sq, counts, kd, vd, q in steps:
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t0 = time.perf_counter()
        slots, copies = B.paged_kv_append_batch(cache.pool, sq, counts)
        tables, lens = cache.block_tables(sq, max_blocks)
        t1 = time.perf_counter()
        slot_d = torch.from_numpy(slots).to(dev)
        tables_d, lens_d = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
        pairs = torch.from_numpy(np.ascontiguousarray(copies)).to(dev) if len(copies) else None
        t2 = time.perf_counter()
        e[0].record(stream)
        if pairs is not None:
            B.paged_kv_copy_blocks(cache.desc, cache.k_pool, cache.v_pool, pairs, len(copies),
                                   stream)
        B.reshape_and_cache(cache.desc, kd, vd, cache.k_pool, cache.v_pool, slot_d, stream=stream)
        e[1].record(stream)
        attend(tables_d, lens_d)
        e[2].record(stream)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        kv, ab = attention_bytes(lens, int((tables >= 0).sum()), w, out.element_size())
        total_bytes += ab
        rows.append({"host_alloc_ms": round((t1 - t0) * 1e3, 4), "h2d_ms": round((t2 - t1) * 1e3, 4),
                     "cache_write_ms": round(e[0].elapsed_time(e[1]), 4),
                     "attention_ms": round(e[1].elapsed_time(e[2]), 4),
                     "step_ms": round((t3 - t0) * 1e3, 4), "copies": int(len(copies))})
    loop_s = time.perf_counter() - t_loop
    # the last step's attention alone, scrubbed launches (the kernel's roofline figure)
    scrub = Scrubber(dev)
    part_ms = timed_launches(lambda: B.paged_attention_partition(
        cache.desc, out, w.dtype, q, cache.k_pool, cache.v_pool, tables_d, lens_d, hq, max_ctx,
        float(w.scale), pt, ws, stream), stream, iters, scrub)
    red_ms = timed_launches(lambda: B.paged_attention_reduce(
        cache.desc, out, w.dtype, lens_d, hq, max_ctx, pt, ws, stream), stream, iters, scrub,
        before=lambda: B.paged_attention_partition(
            cache.desc, out, w.dtype, q, cache.k_pool, cache.v_pool, tables_d, lens_d, hq,
            max_ctx, float(w.scale), pt, ws, stream))
    kv, ab = attention_bytes(lens, int((tables >= 0).sum()), w, out.element_size())
    pst, rst = percentiles(part_ms), percentiles(red_ms)
    del scrub
    cache.close()
    torch.cuda.empty_cache()
    mean = {k: round(float(np.mean([r[k] for r in rows])), 4) for k in rows[0] if k != "copies"}
    return {
        "workload": w.name, "batch": len(seqs), "steps": len(rows), "partition_tokens": pt,
        "per_step": rows, "mean": mean,
        "loop_ms": round(loop_s * 1e3, 3),
        "loop_seq_tokens_per_s": round(len(seqs) * len(rows) / loop_s, 1),
        "loop_GB_per_s": round(total_bytes / loop_s / 1e9, 1),
        "last_step_partition_ms": pst, "last_step_reduce_ms": rst,
        "roofline": {"kernel": "paged_attention_partition (512-token partitions)", "bound": "hbm",
                     "achieved": round(ab / (pst["median"] * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ab / (pst["median"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": ab,
                     "frac_with_merge": round(ab / ((pst["median"] + rst["median"]) * 1e-3) / 1e9
                                              / HBM_PEAK_GBS, 4)},
    }


def shared_prefix_timing(dev, iters=50, partition_tokens=0, max_group=8):
    """The parallel-sampling workload (32 prompts x 8 samples, 2056-token prompts forked,
    tails of 64-512 tokens; 32 q / 8 kv heads, d 128, bf16): attention launched per
    sample (the standard decode at the workload's 512-token partitions) and with each
    prompt's shared blocks read once for its 8 samples (paged_attention_decode_shared_
    prefix).  Median of `iters` scrubbed launches each.  Fractions of the HBM peak are
    stated on the unique bytes: every distinct token's K/V once (a group's shared tokens
    once, each sample's own tokens once), plus queries, outputs, tables and lengths."""
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache, TORCH_DTYPES
    from paged_kv_cache_15_amd.replay import to_device
    w = W.make_config(4)
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, w.block_size,
                         w.free_order, device=dev)
    for op in w.ops:
        if op[0] == "create":
            cache.create()
        elif op[0] == "fork":
            cache.fork(op[1])
        elif op[0] == "append":
            k, v = w.kv[op[3]]
            cache.append(op[1], op[2], to_device(k, w.dtype, dev), to_device(v, w.dtype, dev))
        elif op[0] == "attend":
            seqs, q = op[1], to_device(w.q[op[2]], w.dtype, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    hq, d = w.num_q_heads, w.head_dim
    tables, lens = cache.block_tables(seqs)
    tables_d, lens_d = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    max_ctx = int(lens.max())
    out = torch.empty((len(seqs), hq, d), dtype=TORCH_DTYPES[w.dtype], device=dev)
    gs, sh, max_shared = B.paged_kv_shared_prefix_groups(cache.pool, seqs, max_group, 16)
    gs_d, sh_d = torch.from_numpy(gs).to(dev), torch.from_numpy(sh).to(dev)
    nb_sh = B.paged_attention_shared_prefix_workspace_bytes(cache.desc, len(seqs), hq, max_ctx,
                                                            len(sh), max_group, max_shared,
                                                            partition_tokens)
    ws_sh = torch.empty(nb_sh, dtype=torch.uint8, device=dev)
    pt = w.partition_tokens
    nb_std = B.paged_attention_workspace_bytes(cache.desc, len(seqs), hq, max_ctx, pt)
    ws_std = torch.zeros(max(nb_std, 16), dtype=torch.uint8, device=dev)
    scrub = Scrubber(dev)

    def shared():
        B.paged_attention_decode_shared_prefix(cache.desc, out, w.dtype, q, cache.k_pool,
                                               cache.v_pool, tables_d, lens_d, hq, max_ctx,
                                               float(w.scale), gs_d, sh_d, len(sh), max_group,
                                               max_shared, partition_tokens, ws_sh, stream)

    def standard():
        B.paged_attention_decode(cache.desc, out, w.dtype, q, cache.k_pool, cache.v_pool,
                                 tables_d, lens_d, hq, max_ctx, float(w.scale), pt, ws_std,
                                 stream)
    shared()
    standard()
    t_sh = percentiles(timed_launches(shared, stream, iters, scrub))
    t_std = percentiles(timed_launches(standard, stream, iters, scrub))
    grp = np.repeat(np.arange(len(sh)), np.diff(gs))
    unique_tokens = int(sh.sum()) + int((lens - sh[grp]).sum())
    per_tok = 2 * w.num_kv_heads * d * w.elem_bytes
    extra = 2 * len(seqs) * hq * d * w.elem_bytes + 4 * int((tables >= 0).sum()) + 4 * len(seqs)
    unique = unique_tokens * per_tok + extra
    logical = int(lens.sum()) * per_tok + extra
    distinct_blocks = len(np.unique(tables[tables >= 0]))
    del scrub
    cache.close()
    torch.cuda.empty_cache()

    def line(st):
        ach = unique / (st["median"] * 1e-3) / 1e9
        return {"launch_ms": st, "unique_GB_per_s": round(ach, 1),
                "frac_of_peak_on_unique_bytes": round(ach / HBM_PEAK_GBS, 4),
                "logical_GB_per_s": round(logical / (st["median"] * 1e-3) / 1e9, 1)}
    return {"workload": w.name, "batch": len(seqs), "groups": len(sh), "max_group": max_group,
            "shared_tokens_per_group": int(max_shared), "partition_tokens": partition_tokens,
            "unique_bytes": unique, "logical_bytes": logical,
            "distinct_blocks": distinct_blocks,
            "distinct_block_bytes": distinct_blocks * w.block_size * per_tok,
            "shared_prefix_decode": line(t_sh),
            "per_sample_decode_pt512": line(t_std),
            "roofline": {"kernel": "paged_attention_decode_shared_prefix (partition + merge)",
                         "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                         "achieved": line(t_sh)["unique_GB_per_s"],
                         "frac": line(t_sh)["frac_of_peak_on_unique_bytes"],
                         "algorithmic_bytes_per_launch": unique}}


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}


def prefill_flops(op, lens, w):
    """Algorithmic flops of causal attention for a prefill op: each query at position p
    meets p + 1 keys, 2*d flops for its score and 2*d for its share of the value sum,
    per query head."""
    counts = [int(c) for c in op[2]]
    pairs = 0
    for n, L in zip(counts, lens):
        first = int(L) - n + 1          # keys seen by the first query of the chunk
        pairs += n * first + n * (n - 1) // 2
    return pairs * w.num_q_heads * 4 * w.head_dim


def prefill_timing(k, steps, warmup, block_size=16, head_dim=128):
    """Paged prefill on prefill workload k at full size: a step writes the chunk's K/V
    (reshape_and_cache) and runs the causal attention over the pool; the attention
    launch is timed with HIP events on its stream."""
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache, TORCH_DTYPES
    from paged_kv_cache_15_amd.replay import to_device

    dev = torch.device("cuda:0")
    w = W.make_prefill_config(k, block_size=block_size, head_dim=head_dim)
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, w.block_size,
                         w.free_order, device=dev)
    last = None
    for op in w.ops:
        if op[0] == "create":
            cache.create()
        elif op[0] == "append":
            kv = w.kv[op[3]]
            kd, vd = to_device(kv[0], w.dtype, dev), to_device(kv[1], w.dtype, dev)
            slots, copies = B.paged_kv_append_batch(cache.pool, op[1], op[2])
            slot_d = torch.from_numpy(slots).to(dev)
            B.reshape_and_cache(cache.desc, kd, vd, cache.k_pool, cache.v_pool, slot_d)
            last = (kd, vd, slot_d)
        elif op[0] == "prefill":
            pre = op
    torch.cuda.synchronize()
    new_k, new_v, slot_d = last
    seqs, counts = pre[1], pre[2]
    tables, lens = cache.block_tables(seqs)
    q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    q = to_device(w.q[pre[3]], w.dtype, dev)
    out = torch.empty_like(q)
    tables_d, lens_d = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    q_start_d = torch.from_numpy(q_start).to(dev)
    max_q, max_ctx = int(max(counts)), int(lens.max())
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        B.reshape_and_cache(cache.desc, new_k, new_v, cache.k_pool, cache.v_pool, slot_d,
                            stream=stream)
        if ev is not None:
            ev[0].record(stream)
        B.paged_attention_prefill(cache.desc, out, w.dtype, q, q_start_d, cache.k_pool,
                                  cache.v_pool, tables_d, lens_d, w.num_q_heads, max_q, max_ctx,
                                  float(w.scale), stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_attn = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    flops = prefill_flops(pre, lens, w)
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    tf = flops / (ms_attn * 1e-3) / 1e12
    cache.close()
    return {
        "workload": w.name, "sequences": len(seqs), "query_tokens": int(q_start[-1]),
        "context_tokens": int(lens.sum()), "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim, "block_size": w.block_size, "dtype": w.dtype,
        "ms_per_step": round(ms_step, 4), "attention_ms": round(ms_attn, 4),
        "query_tokens_per_s": round(int(q_start[-1]) / (ms_step * 1e-3), 1),
        "roofline": {"kernel": "paged_attention_prefill", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tf / peak, 4), "algorithmic_flops_per_launch": flops},
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or KV head with no exchange; what is measured "
              "is one MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.decode_graph:
        res = decode_graph_timing(partition_tokens=args.partition_tokens)
        print(json.dumps({"metric": "graph-captured decode step us, 1 MI355X",
                          "value": res["graph_us_per_step"], "unit": "us",
                          "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": "gqa_decode_graph_b8_l32"},
                          **res}), flush=True)
        return
    if args.shared_prefix:
        import torch
        res = shared_prefix_timing(torch.device("cuda:0"), max(50, args.steps),
                                   args.shared_partition_tokens)
        print(json.dumps({"metric": "shared-prefix decode GB/s on unique bytes, 1 MI355X",
                          "value": res["shared_prefix_decode"]["unique_GB_per_s"],
                          "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                          "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": res["workload"]}, **res}), flush=True)
        return
    if args.prefill:
        res = prefill_timing(args.prefill, args.steps, args.warmup, args.block_size,
                             args.head_dim or 128)
        print(json.dumps({"metric": "paged prefill attention TFLOP/s, 1 MI355X",
                          "value": res["roofline"]["achieved"], "unit": "TFLOP/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": res["ms_per_step"], "higher_is_better": True,
                          "dtype": res["dtype"], "data": "synthetic",
                          "config": {"workload": res["workload"]}, **res}), flush=True)
        return
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_cache_15_amd import binding as B
    from paged_kv_cache_15_amd.cache import PagedKVCache, TORCH_DTYPES
    from paged_kv_cache_15_amd.replay import to_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] building workload {args.config}")
    w = W.make_config(args.config, block_size=args.block_size, head_dim=args.head_dim)
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.dtype, w.block_size,
                         w.free_order, device=dev)
    last_append = last_attend = None
    t_host = 0.0
    for op in w.ops:
        if op[0] == "create":
            cache.create()
        elif op[0] == "fork":
            cache.fork(op[1])
        elif op[0] == "free":
            cache.free(op[1])
        elif op[0] == "append":
            k, v = w.kv[op[3]]
            kd, vd = to_device(k, w.dtype, dev), to_device(v, w.dtype, dev)
            t0 = time.perf_counter()
            slots, copies = B.paged_kv_append_batch(cache.pool, op[1], op[2])
            t_host = time.perf_counter() - t0
            if len(copies):
                pairs = torch.from_numpy(np.ascontiguousarray(copies)).to(dev)
                B.paged_kv_copy_blocks(cache.desc, cache.k_pool, cache.v_pool, pairs, len(copies))
            slot_d = torch.from_numpy(slots).to(dev)
            B.reshape_and_cache(cache.desc, kd, vd, cache.k_pool, cache.v_pool, slot_d)
            last_append = (kd, vd, slot_d, len(op[1]))
        elif op[0] == "attend":
            last_attend = op
    torch.cuda.synchronize()
    new_k, new_v, slot_d, n_app = last_append
    seqs, qidx = last_attend[1], last_attend[2]
    tables, lens = cache.block_tables(seqs)
    nb_total = int((tables >= 0).sum())
    tables_d = torch.from_numpy(tables).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    q = to_device(w.q[qidx], w.dtype, dev)
    out_dtype = w.dtype
    out = torch.empty((len(seqs), w.num_q_heads, w.head_dim), dtype=TORCH_DTYPES[out_dtype], device=dev)
    max_ctx = int(lens.max())
    pt = w.partition_tokens if args.partition_tokens is None else args.partition_tokens
    ws_bytes = B.paged_attention_workspace_bytes(cache.desc, len(seqs), w.num_q_heads, max_ctx, pt)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)   # zero before first use
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        B.reshape_and_cache(cache.desc, new_k, new_v, cache.k_pool, cache.v_pool, slot_d,
                            stream=stream)
        if ev is not None:
            ev[0].record(stream)
        B.paged_attention_partition(cache.desc, out, out_dtype, q, cache.k_pool, cache.v_pool,
                                    tables_d, lens_d, w.num_q_heads, max_ctx, float(w.scale), pt,
                                    ws, stream)
        if ev is not None:
            ev[1].record(stream)
        B.paged_attention_reduce(cache.desc, out, out_dtype, lens_d, w.num_q_heads, max_ctx, pt,
                                 ws, stream)
        if ev is not None:
            ev[2].record(stream)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The step rate comes from steps with nothing else on the stream (a recorded event
    # costs the queue a few microseconds); a second pass with events around each launch
    # gives the per-kernel durations.
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # Per-kernel durations: at least 50 launches of each, HIP events on the launch stream
    # around each one, a 512 MB scrub write before each (outside the events).
    iters = max(50, args.steps)
    scrub = Scrubber(dev)
    log(f"[bench] per-kernel timing, {iters} launches each, scrubbed")
    rac = timed_launches(lambda: B.reshape_and_cache(cache.desc, new_k, new_v, cache.k_pool,
                                                     cache.v_pool, slot_d, stream=stream),
                         stream, iters, scrub)

    def partition():
        B.paged_attention_partition(cache.desc, out, out_dtype, q, cache.k_pool, cache.v_pool,
                                    tables_d, lens_d, w.num_q_heads, max_ctx, float(w.scale), pt,
                                    ws, stream)

    def reduce():
        B.paged_attention_reduce(cache.desc, out, out_dtype, lens_d, w.num_q_heads, max_ctx, pt,
                                 ws, stream)
    part = timed_launches(partition, stream, iters, scrub)
    streamk = pt == 0 or (pt == B.PARTITION_AUTO and B.paged_attention_auto_partition_tokens(
        cache.desc, len(seqs), w.num_q_heads, max_ctx) == 0)
    # under stream-K the merge happens inside the partition launch: nothing to time
    red = None if streamk else timed_launches(reduce, stream, iters, scrub, before=partition)
    part_st, rac_st = percentiles(part), percentiles(rac)
    red_st = None if red is None else percentiles(red)
    part_ms, rac_ms = part_st["median"], rac_st["median"]
    red_ms = None if red_st is None else red_st["median"]
    del scrub
    torch.cuda.empty_cache()
    log("[bench] streaming-read probe")
    probe = read_bandwidth(dev, stream)

    kv_bytes, attn_bytes = attention_bytes(lens, nb_total, w, out.element_size())
    write_bytes = 2 * 2 * n_app * w.num_kv_heads * w.head_dim * w.elem_bytes + 4 * n_app
    step_bytes = attn_bytes + write_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    traffic, traffic_src = measured_traffic(w.name, pt)
    achieved = attn_bytes / (part_ms * 1e-3) / 1e9
    res = {
        "metric": "decode KV GB/s (% of HBM peak) + seq-tokens/s, paged attention, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, seeded lengths and pool permutation)",
        "config": {
            "workload": w.name,
            "batch": len(seqs), "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": w.dtype,
            "context_tokens": int(lens.sum()), "max_context": max_ctx,
            "partition_tokens": pt, "pool_blocks": w.num_blocks, "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(len(seqs) / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "step_bytes": step_bytes,
        "kernel_ms": {"reshape_and_cache": round(rac_ms, 5), "paged_attention_partition": round(part_ms, 5),
                      "paged_attention_reduce": None if red_ms is None else round(red_ms, 5)},
        "kernel_ms_stats": {"reshape_and_cache": rac_st, "paged_attention_partition": part_st,
                            "paged_attention_reduce": red_st,
                            "protocol": f"median of {iters} launches each, HIP events on the "
                                        "launch stream, 512 MB scrub write before each launch "
                                        "outside the events"},
        "host_alloc_ms_per_step": round(t_host * 1e3, 4),
        "roofline": {
            "kernel": "paged_attention_partition",
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": attn_bytes,
            "traffic_source": traffic_src,
            "launch_ms": part_st,
            "measured_read_GB_per_s": probe["GB_per_s"],
            "frac_of_measured_read": round(achieved / probe["GB_per_s"], 4),
        },
        "read_probe": probe,
        "cpu_baseline": None,
    }
    del new_k, new_v
    res["prefix_cache_host"] = prefix_cache_host()
    if not args.no_extras:
        del out, q, tables_d, lens_d, ws
        cache.close()
        del cache
        torch.cuda.empty_cache()
        log("[bench] prefill")
        res["prefill"] = prefill_timing(1, 10, 2)
        log("[bench] decode graph")
        res["decode_graph"] = decode_graph_timing()
        log("[bench] long-context step loop")
        res["long_context_step_loop"] = long_context_step_loop(dev)
        log("[bench] shared-prefix decode")
        res["shared_prefix"] = shared_prefix_timing(dev)
    # The host baseline runs last: GPU timings taken after it came out slower (the
    # prefill launch at 0.368 of peak against 0.398 when run before it, in the same
    # bench), most likely from its BLAS worker threads still holding the host cores.
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
