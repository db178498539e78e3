"""Helpers shared by the GPU parity tests (compare the HIP path with the oracle)."""
import sys

import numpy as np
import torch

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
BITS = {"f32": (torch.int32, np.uint32), "f16": (torch.int16, np.uint16),
        "bf16": (torch.int16, np.uint16)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pool_bits(t, dtype):
    tbits, nbits = BITS[dtype]
    return t.view(tbits).cpu().numpy().view(nbits)


def out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_pools_equal(cache, oracle_res, dtype):
    gk, gv = pool_bits(cache.k_pool, dtype), pool_bits(cache.v_pool, dtype)
    assert gk.shape == oracle_res.k_pool.shape and gv.shape == oracle_res.v_pool.shape
    if not np.array_equal(gk, oracle_res.k_pool):
        bad = np.argwhere(gk != oracle_res.k_pool)
        raise AssertionError(f"K pool differs at {len(bad)} elements, first {bad[:3].tolist()}")
    if not np.array_equal(gv, oracle_res.v_pool):
        bad = np.argwhere(gv != oracle_res.v_pool)
        raise AssertionError(f"V pool differs at {len(bad)} elements, first {bad[:3].tolist()}")


def assert_bookkeeping_equal(gpu_res, oracle_res):
    assert len(gpu_res.slot_mappings) == len(oracle_res.slot_mappings)
    for a, b in zip(gpu_res.slot_mappings, oracle_res.slot_mappings):
        assert np.array_equal(a, b)
    for a, b in zip(gpu_res.copies, oracle_res.copies):
        assert np.array_equal(np.asarray(a).reshape(-1, 2), np.asarray(b).reshape(-1, 2))
    for a, b in zip(gpu_res.tables, oracle_res.tables):
        assert np.array_equal(a, b)
    for a, b in zip(gpu_res.context_lens, oracle_res.context_lens):
        assert np.array_equal(a, b)


MANT_BITS = {"bf16": 7, "f16": 10}
MIN_EXP = {"bf16": -126, "f16": -14}


def out_tolerance(ref, in_dtype, out_dtype):
    """Per-element bound: the attention tolerance of the input type, plus half an ulp
    of the output type when the result is stored in 16 bits (rounding the exact value
    to fp16/bf16 can move it by up to half an ulp on top of the arithmetic error)."""
    base = TOL[in_dtype]
    if out_dtype == "f32":
        return np.full(ref.shape, base)
    mag = np.abs(ref) + base
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** MIN_EXP[out_dtype])))
    return base + 0.5 * 2.0 ** (e - MANT_BITS[out_dtype])


def assert_close(gpu_out, ref, in_dtype, out_dtype, rows=None):
    g = out_f64(gpu_out)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert not np.isnan(g).any(), "NaN in output"
    err = np.abs(g - ref)
    tol = out_tolerance(ref, in_dtype, out_dtype)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"max excess at {worst}: |err| {err[worst]:.3e} > tol "
                                f"{tol[worst]:.3e} (ref {ref[worst]:.4f})")
    return float(err.max())


def max_err(gpu_out, ref, rows=None):
    g = out_f64(gpu_out)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert not np.isnan(g).any(), "NaN in output"
    return float(np.abs(g - ref).max())
