"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs, and compare against the CPU oracle.  Nothing here feeds a GPU
result into the oracle except routing indices for the attention comparison
(so that near-tie routing differences cannot leak into output comparisons)."""
from __future__ import annotations

import math

import numpy as np
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from hga_testlib import allclose_report, tie_band_ok

TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}
DEV = "cuda:0"


def shape_of(w: syn.Workload, **kw):
    base = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                head_dim=w.head_dim, q_len=w.q_len, kv_len=w.kv_len, top_k=w.top_k,
                top_g=w.top_g, dtype=w.dtype)
    base.update(kw)
    return hga.make_shape(**base)


def upload(x: dict, dtype: str) -> dict:
    return {k: syn.to_torch(v, dtype, DEV) for k, v in x.items()}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_forward(w: syn.Workload, x: dict | None = None):
    if x is None:
        x = syn.make_inputs(w)
    t = upload(x, w.dtype)
    s = shape_of(w)
    out = hga.forward(s, t["Q"], t["K"], t["V"])
    torch.cuda.synchronize()
    return s, x, t, out


def check_routing(oracle, w, Qf, cm_o, gm_o, ci_gpu, gi_gpu, rows=None, causal=False,
                  Qprev=None):
    """GPU routing vs the oracle under the near-tie rule (``causal``: the
    strictly causal variant, ``Qprev`` the 64 queries before the segment).
    Returns the number of rows where a near tie allowed a difference; the
    counts by stage are appended to TIE_LOG (chunk rows tolerated, group rows
    re-derived on the GPU's chunk set, group rows tolerated)."""
    rows = list(rows) if rows is not None else None
    ci_o, gi_o, cs, gs = oracle.route(Qf, cm_o, gm_o, w.kv_len, w.top_k, w.top_g,
                                      want_scores=True, causal=causal, Qprev=Qprev)
    tolerated = 0
    chunk_tol = 0
    B, Hq, nblk = ci_gpu.shape[:3]
    for idx in (rows if rows is not None else np.ndindex(B, Hq, nblk)):
        a, b = ci_gpu[idx], ci_o[idx]
        # format: ascending valid prefix, -1 padding
        v = a[a >= 0]
        assert np.all(np.diff(v) > 0) and np.all(a[len(v):] == -1), (idx, a)
        if not np.array_equal(a, b):
            ok, exact = tie_band_ok(a, b, cs[idx], w.top_k)
            assert ok, f"chunk routing differs beyond the tie band at {idx}: {a} vs {b}"
            tolerated += 1
    chunk_tol = tolerated
    # groups: against the oracle's choice given the GPU's chunk sets (the
    # oracle's forced-chunk branch, pinned on the CPU)
    forced_rows = 0
    if not np.array_equal(ci_gpu, ci_o):
        forced_rows = int(np.any(ci_gpu != ci_o, axis=-1).sum())
        _, gi_o, _, gs = oracle.route(Qf, cm_o, gm_o, w.kv_len, w.top_k, w.top_g,
                                      forced_chunk_idx=ci_gpu, want_scores=True, causal=causal,
                                      Qprev=Qprev)
    for idx in (rows if rows is not None else np.ndindex(B, Hq, nblk)):
        a, b = gi_gpu[idx], gi_o[idx]
        v = a[a >= 0]
        assert np.all(np.diff(v) > 0) and np.all(a[len(v):] == -1), (idx, a)
        if not np.array_equal(a, b):
            ok, exact = tie_band_ok(a, b, gs[idx], w.top_g)
            assert ok, f"group routing differs beyond the tie band at {idx}: {a} vs {b}"
            tolerated += 1
    nrows = int(np.prod(ci_gpu.shape[:3])) if rows is None else len(rows)
    TIE_LOG.append({"case": w.name, "rows": nrows, "chunk_rows_tolerated": chunk_tol,
                    "group_rows_on_gpu_chunk_set": forced_rows,
                    "group_rows_tolerated": tolerated - chunk_tol})
    return tolerated


# per-call counts of check_routing, for the tie-band summary a GPU run writes
# when HGA_TEST_REPORT_DIR names a directory (see conftest.py)
TIE_LOG = []


def assert_close(got, ref, dtype, what):
    atol, rtol = TOL[dtype]
    ok, maxerr, nbad = allclose_report(got, ref, atol, rtol)
    assert ok, f"{what}: {nbad} elements beyond atol={atol} rtol={rtol}; max abs err {maxerr:.3e}"
    return maxerr


def random_shapes(n, seed, backward=True):
    """n valid problems drawn from a seeded generator: bf16 and fp32, D 64 and
    128, 1 to 8 query heads per kv head, batch 1 or 2, 1 to 6 query blocks,
    kv histories of 0 to 12 extra chunks, top-k from 0 to 20 and top-g from 0
    to 8 groups past what the kept chunks hold (the rest is padding)."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        dtype = "bf16" if i % 2 == 0 else "fp32"
        D = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 4, 8]))
        q_len = 64 * int(rng.integers(1, 7))
        kv_len = q_len + 64 * int(rng.integers(0, 13))
        top_k = int(rng.integers(0, 21))
        top_g = int(rng.integers(0, 8 * top_k + 9))
        scale = 1 / math.sqrt(D) if dtype == "bf16" else 0.3
        name = f"rand{i}_{dtype}_d{D}_h{hkv * r}x{hkv}_q{q_len}_kv{kv_len}_k{top_k}_g{top_g}"
        out[name] = syn.Workload(name, int(rng.integers(1, 3)), hkv * r, hkv, D, q_len, kv_len,
                                 top_k, top_g, dtype, seed + i, scale, backward=backward)
    return out
