"""HIP path vs the CPU oracle, element by element (needs an MI355X).

Small cases compare every output; the full-size workloads compare summaries
and routing in full and the attention outputs and gradients on sampled heads
(the oracle run on the slice of one query head, or of one kv head with its
query heads for the backward).  Routing indices must match bit for bit except
inside the near-tie band; attention is always checked on the GPU's own
routing.  Tolerances: |gpu - oracle| <= atol + rtol |oracle| with (2e-2, 1e-2)
for bf16 and (1e-5, 1e-5) for fp32.
"""
import math

import numpy as np
import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from gpu_common import (DEV, assert_close, check_routing, f64, random_shapes, run_forward,
                        shape_of, upload)
from hga_testlib import (causal_mask, hand_example_inputs, hand_example_output_e1,
                         load_golden, sdpa_f64)

pytestmark = pytest.mark.gpu

W = syn.WORKLOADS
SMALL = {
    "tiny_fp32_1k": W["tiny_fp32_1k"],
    "bf16_r2_512": syn.Workload("bf16_r2_512", 1, 4, 2, 128, 512, 512, 3, 12, "bf16", 11,
                                1 / math.sqrt(128), backward=True),
    "bf16_seg_b2": syn.Workload("bf16_seg_b2", 2, 8, 2, 128, 256, 1024, 4, 20, "bf16", 12,
                                1 / math.sqrt(128), backward=True),
    "bf16_d64": syn.Workload("bf16_d64", 1, 2, 1, 64, 384, 384, 2, 7, "bf16", 13, 0.125,
                             backward=True),
    "fp32_d128": syn.Workload("fp32_d128", 1, 2, 2, 128, 128, 320, 3, 9, "fp32", 14, 0.3,
                              backward=True),
    "bf16_r8_allgroups": syn.Workload("bf16_r8_allgroups", 1, 8, 1, 128, 256, 640, 2, 40,
                                      "bf16", 15, 1 / math.sqrt(128), backward=True),
    "bf16_local_only_k0": syn.Workload("bf16_local_only_k0", 1, 2, 1, 128, 192, 192, 0, 8,
                                       "bf16", 16, 1 / math.sqrt(128), backward=True),
    "bf16_local_only_g0": syn.Workload("bf16_local_only_g0", 1, 2, 1, 128, 192, 192, 3, 0,
                                       "bf16", 17, 1 / math.sqrt(128), backward=True),
    "bf16_one_block": syn.Workload("bf16_one_block", 1, 2, 2, 128, 64, 64, 4, 16, "bf16", 18,
                                   1 / math.sqrt(128), backward=True),
}


def _oracle_inputs(w, x):
    return {k: syn.to_f64(v, w.dtype) for k, v in x.items()}


RANDOM = random_shapes(12, seed=97)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_case_full_parity(oracle, name):
    """Summaries, routing, O, lse, dQ, dK, dV against the oracle, every element."""
    _full_parity(oracle, SMALL[name])


@pytest.mark.parametrize("name", list(RANDOM))
def test_random_shapes_full_parity(oracle, name):
    """The same element-by-element comparison on seeded random valid shapes
    (ragged histories, grouped heads, budgets past what the history holds)."""
    _full_parity(oracle, RANDOM[name])


def _full_parity(oracle, w):
    print(f"[case] {w.name}", flush=True)
    s, x, t, out = run_forward(w)
    xf = _oracle_inputs(w, x)
    cm_o, gm_o = oracle.summaries(xf["K"])
    tol = (1e-5, 1e-5)
    np.testing.assert_allclose(f64(out["chunk_mean"]), cm_o, atol=tol[0], rtol=tol[1])
    np.testing.assert_allclose(f64(out["group_mean"]), gm_o, atol=tol[0], rtol=tol[1])
    ci = out["chunk_idx"].cpu().numpy()
    gi = out["group_idx"].cpu().numpy()
    check_routing(oracle, w, xf["Q"], cm_o, gm_o, ci, gi)
    O_o, lse_o = oracle.attend_fwd(xf["Q"], xf["K"], xf["V"], gi)
    assert_close(f64(out["O"]), O_o, w.dtype, "O")
    assert_close(f64(out["lse"]), lse_o, "fp32" if w.dtype == "fp32" else "bf16", "lse")
    if w.backward:
        if "dO" not in x:
            x.update(syn.make_inputs(w, with_grad_output=True))
        dO = syn.to_torch(x["dO"], w.dtype, DEV)
        dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], dO,
                                  out["group_idx"])
        torch.cuda.synchronize()
        dQ_o, dK_o, dV_o = oracle.attend_bwd(xf["Q"], xf["K"], xf["V"], gi,
                                             syn.to_f64(x["dO"], w.dtype))
        assert_close(f64(dQ), dQ_o, w.dtype, "dQ")
        assert_close(f64(dK), dK_o, w.dtype, "dK")
        assert_close(f64(dV), dV_o, w.dtype, "dV")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_hand_example_on_gpu(dtype):
    """The hand-derived routing case: indices bit-exact, output vs closed form."""
    gold = load_golden("hand_example.json")
    for variant, key in (("expected", 1.0), ("tie_variant", 1.5)):
        Q, K, V = hand_example_inputs(chunk0_key=key)
        tt = torch.bfloat16 if dtype == "bf16" else torch.float32
        Qt, Kt, Vt = (torch.tensor(a, dtype=tt, device=DEV) for a in (Q, K, V))
        s = hga.make_shape(1, 1, 1, 64, 192, 192, 1, 2, dtype=dtype)
        out = hga.forward(s, Qt, Kt, Vt)
        torch.cuda.synchronize()
        assert out["chunk_idx"][0, 0].tolist() == gold[variant]["chunk_idx"]
        assert out["group_idx"][0, 0].tolist() == gold[variant]["group_idx"]
        if variant == "expected":
            O = f64(out["O"])[0, 0]
            ref = np.array([hand_example_output_e1(p, key) for p in range(192)])
            atol, rtol = (2e-2, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)
            np.testing.assert_allclose(O[:, 1], ref, atol=atol, rtol=rtol)


def test_full_coverage_equals_dense_causal_on_gpu():
    """k and g covering all history: the GPU output equals dense causal
    attention computed by torch in float64 on the CPU."""
    w = syn.Workload("cover", 1, 4, 2, 128, 512, 768, 12, 96, "bf16", 21, 1 / math.sqrt(128))
    s, x, t, out = run_forward(w)
    xf = {k: syn.to_f64(v, "bf16") for k, v in x.items()}
    ref = sdpa_f64(xf["Q"], xf["K"], xf["V"], causal_mask(512, 768))
    assert_close(f64(out["O"]), ref, "bf16", "O vs dense causal")


def test_outputs_fully_written_and_deterministic():
    """Outputs poisoned with NaN are fully overwritten; two runs are bitwise equal."""
    w = SMALL["bf16_seg_b2"]
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, "bf16")
    s = shape_of(w)
    res = []
    for _ in range(2):
        o = hga.forward(s, t["Q"], t["K"], t["V"])
        for k in ("O", "lse", "chunk_mean", "group_mean"):
            o[k].fill_(float("nan"))
        o["chunk_idx"].fill_(-7)
        o["group_idx"].fill_(-7)
        hga.hga_build_summaries(s, t["K"], o["chunk_mean"], o["group_mean"])
        hga.hga_route(s, t["Q"], o["chunk_mean"], o["group_mean"], o["chunk_idx"], o["group_idx"])
        hga.hga_attend_fwd(s, t["Q"], t["K"], t["V"], o["group_idx"], o["O"], o["lse"])
        dQ = torch.full_like(t["Q"], float("nan"))
        dK = torch.full_like(t["K"], float("nan"))
        dV = torch.full_like(t["V"], float("nan"))
        ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=DEV)
        hga.hga_attend_bwd(s, t["Q"], t["K"], t["V"], o["O"], o["lse"], t["dO"], o["group_idx"],
                           dQ, dK, dV, ws)
        torch.cuda.synchronize()
        for name, v in (("O", o["O"]), ("lse", o["lse"]), ("cm", o["chunk_mean"]),
                        ("gm", o["group_mean"]), ("dQ", dQ), ("dK", dK), ("dV", dV)):
            assert not torch.isnan(v.float()).any(), name
        assert (o["chunk_idx"] != -7).all() and (o["group_idx"] != -7).all()
        res.append([v.clone() for v in (o["O"], o["lse"], o["group_idx"], dQ, dK, dV)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_split_backward_matches_combined():
    """hga_attend_bwd_dq then hga_attend_bwd_dkdv (sharing one workspace) give
    bit for bit what hga_attend_bwd gives."""
    w = SMALL["bf16_seg_b2"]
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, "bf16")
    s = shape_of(w)
    o = hga.forward(s, t["Q"], t["K"], t["V"])
    ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=DEV)
    a = [torch.empty_like(t["Q"]), torch.empty_like(t["K"]), torch.empty_like(t["V"])]
    hga.hga_attend_bwd(s, t["Q"], t["K"], t["V"], o["O"], o["lse"], t["dO"], o["group_idx"],
                       *a, ws)
    bq, bk, bv = (torch.empty_like(v) for v in a)
    ws.fill_(0xFF)
    hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], o["O"], o["lse"], t["dO"], o["group_idx"],
                          bq, ws)
    hga.hga_attend_bwd_dkdv(s, t["Q"], t["K"], t["V"], o["lse"], t["dO"], o["group_idx"], bk, bv,
                            ws)
    torch.cuda.synchronize()
    for x0, x1 in zip(a, (bq, bk, bv)):
        assert torch.equal(x0, x1)


def test_prep_then_side_by_side_backward_matches_combined():
    """hga_attend_bwd_prep, then a workspace-free hga_attend_bwd_dq on a second
    stream beside hga_attend_bwd_dkdv on the first (forked and joined by
    events), give bit for bit what hga_attend_bwd gives; also in sequence."""
    w = SMALL["bf16_seg_b2"]
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, "bf16")
    s = shape_of(w)
    o = hga.forward(s, t["Q"], t["K"], t["V"])
    ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=DEV)
    ref = [torch.empty_like(t["Q"]), torch.empty_like(t["K"]), torch.empty_like(t["V"])]
    hga.hga_attend_bwd(s, t["Q"], t["K"], t["V"], o["O"], o["lse"], t["dO"], o["group_idx"],
                       *ref, ws)
    torch.cuda.synchronize()
    for side_by_side in (False, True):
        got = [torch.full_like(v, float("nan")) for v in ref]
        ws.fill_(0xFF)
        main = torch.cuda.current_stream()
        hga.hga_attend_bwd_prep(s, o["O"], t["dO"], o["group_idx"], ws)
        side = torch.cuda.Stream()
        side.wait_stream(main)
        with torch.cuda.stream(side if side_by_side else main):
            hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], o["O"], o["lse"], t["dO"],
                                  o["group_idx"], got[0], None)
        hga.hga_attend_bwd_dkdv(s, t["Q"], t["K"], t["V"], o["lse"], t["dO"], o["group_idx"],
                                got[1], got[2], ws)
        main.wait_stream(side)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), (name, side_by_side)


def test_incremental_summaries_match_full_build():
    w = SMALL["bf16_seg_b2"]
    x = syn.make_inputs(w)
    t = upload(x, "bf16")
    s = shape_of(w)
    n = w.kv_len // 64
    full_c = torch.empty(w.batch, w.n_kv_heads, n, 128, device=DEV)
    full_g = torch.empty(w.batch, w.n_kv_heads, n * 8, 128, device=DEV)
    hga.hga_build_summaries(s, t["K"], full_c, full_g)
    inc_c = torch.full_like(full_c, float("nan"))
    inc_g = torch.full_like(full_g, float("nan"))
    for a, b in ((0, 3), (3, 4), (4, 11), (11, n)):
        hga.hga_build_summaries(s, t["K"], inc_c, inc_g, a, b)
    torch.cuda.synchronize()
    assert torch.equal(full_c, inc_c) and torch.equal(full_g, inc_g)


@pytest.mark.parametrize("name", ["bf16_seg_b2", "fp32_d128", "bf16_d64"])
def test_summaries_from_a_row_range_match_full_build(name):
    """hga_build_summaries_rows over a buffer holding a range of positions
    writes, for the chunks in that range, exactly what the full build writes,
    and nothing outside them."""
    w = SMALL[name]
    x = syn.make_inputs(w)
    t = upload(x, w.dtype)
    s = shape_of(w)
    n, D = w.kv_len // 64, w.head_dim
    full_c = torch.empty(w.batch, w.n_kv_heads, n, D, device=DEV)
    full_g = torch.empty(w.batch, w.n_kv_heads, n * 8, D, device=DEV)
    hga.hga_build_summaries(s, t["K"], full_c, full_g)
    row0, rows = 64 * (n // 3), 64 * (n - n // 3)
    part = t["K"][:, :, row0:row0 + rows].contiguous()
    inc_c = torch.full_like(full_c, float("nan"))
    inc_g = torch.full_like(full_g, float("nan"))
    c0, c1 = row0 // 64 + 1, n
    hga.hga_build_summaries_rows(s, part, row0, inc_c, inc_g, c0, c1)
    torch.cuda.synchronize()
    assert torch.equal(full_c[:, :, c0:c1], inc_c[:, :, c0:c1])
    assert torch.equal(full_g[:, :, 8 * c0:8 * c1], inc_g[:, :, 8 * c0:8 * c1])
    assert torch.isnan(inc_c[:, :, :c0]).all() and torch.isnan(inc_g[:, :, :8 * c0]).all()


# ------------------------------------------------------------------ full-size workloads

_cache = {}


def _full(name):
    if name not in _cache:
        w = W[name]
        x = syn.make_inputs(w)
        s, x, t, out = run_forward(w, x)
        _cache.clear()
        _cache[name] = (w, s, x, t, out)
    return _cache[name]


FULL = ["qwen3_8b_2k", "segment_2k_over_16k", "segment_2k_over_64k_ties", "fwd_bwd_b2_4k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_summaries_and_routing(oracle, name):
    print(f"[case] full {name}", flush=True)
    w, s, x, t, out = _full(name)
    Kf = syn.to_f64(x["K"], w.dtype)
    cm_o, gm_o = oracle.summaries(Kf)
    np.testing.assert_allclose(f64(out["chunk_mean"]), cm_o, atol=1e-5, rtol=1e-5)
    np.testing.assert_allclose(f64(out["group_mean"]), gm_o, atol=1e-5, rtol=1e-5)
    del Kf
    tolerated = check_routing(oracle, w, syn.to_f64(x["Q"], w.dtype), cm_o, gm_o,
                              out["chunk_idx"].cpu().numpy(), out["group_idx"].cpu().numpy())
    print(f"[routing] {name}: rows inside the near-tie band: {tolerated}", flush=True)


@pytest.mark.parametrize("name", FULL)
def test_full_size_forward_sampled_heads(oracle, name):
    w, s, x, t, out = _full(name)
    r = w.n_q_heads // w.n_kv_heads
    gi = out["group_idx"].cpu().numpy()
    O, lse = f64(out["O"]), f64(out["lse"])
    picks = [(0, 0), (w.batch - 1, w.n_q_heads - 1), (0, w.n_q_heads // 2 + 1)]
    for b, hq in picks:
        hkv = hq // r
        Qs = syn.to_f64(x["Q"][b:b + 1, hq:hq + 1], w.dtype)
        Ks = syn.to_f64(x["K"][b:b + 1, hkv:hkv + 1], w.dtype)
        Vs = syn.to_f64(x["V"][b:b + 1, hkv:hkv + 1], w.dtype)
        O_o, lse_o = oracle.attend_fwd(Qs, Ks, Vs, gi[b:b + 1, hq:hq + 1])
        assert_close(O[b:b + 1, hq:hq + 1], O_o, w.dtype, f"O[{b},{hq}]")
        assert_close(lse[b:b + 1, hq:hq + 1], lse_o, w.dtype, f"lse[{b},{hq}]")


@pytest.mark.parametrize("name,b,hkv", [("segment_2k_over_16k", 0, 0), ("fwd_bwd_b2_4k", 1, 7),
                                        ("segment_2k_over_64k_ties", 0, 5)])
def test_full_size_backward_sampled_kv_group(oracle, name, b, hkv):
    """dQ of the kv group's query heads and dK, dV of the kv head, at full size."""
    w, s, x, t, out = _full(name)
    xd = syn.make_inputs(w, with_grad_output=True)["dO"]
    dO = syn.to_torch(xd, w.dtype, DEV)
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], dO,
                              out["group_idx"])
    torch.cuda.synchronize()
    r = w.n_q_heads // w.n_kv_heads
    hs = slice(hkv * r, (hkv + 1) * r)
    gi = out["group_idx"].cpu().numpy()[b:b + 1, hs]
    Qs = syn.to_f64(x["Q"][b:b + 1, hs], w.dtype)
    Ks = syn.to_f64(x["K"][b:b + 1, hkv:hkv + 1], w.dtype)
    Vs = syn.to_f64(x["V"][b:b + 1, hkv:hkv + 1], w.dtype)
    dOs = syn.to_f64(xd[b:b + 1, hs], w.dtype)
    dQ_o, dK_o, dV_o = oracle.attend_bwd(Qs, Ks, Vs, gi, dOs)
    assert_close(f64(dQ)[b:b + 1, hs], dQ_o, w.dtype, "dQ")
    assert_close(f64(dK)[b:b + 1, hkv:hkv + 1], dK_o, w.dtype, "dK")
    assert_close(f64(dV)[b:b + 1, hkv:hkv + 1], dV_o, w.dtype, "dV")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_maximum_kv_length(oracle, dtype):
    """kv_len = HGA_MAX_KV_LEN (131072): 2047 candidate chunks for the last
    block (the widest routing select), a group-mask map of 2048 chunks per
    row, dK/dV over every chunk of the history.  Two 64-query blocks at the end
    of the history, full parity."""
    from gpu_common import assert_close
    w = syn.Workload("max_kv", 1, 2, 1, 64, 128, 131072, 12, 40, dtype, 71,
                     0.125 if dtype == "bf16" else 0.4, backward=True)
    print(f"[case] maximum kv_len {dtype}", flush=True)
    s, x, t, out = run_forward(w)
    xf = _oracle_inputs(w, x)
    cm_o, gm_o = oracle.summaries(xf["K"])
    np.testing.assert_allclose(f64(out["chunk_mean"]), cm_o, atol=1e-5, rtol=1e-5)
    ci, gi = out["chunk_idx"].cpu().numpy(), out["group_idx"].cpu().numpy()
    check_routing(oracle, w, xf["Q"], cm_o, gm_o, ci, gi)
    O_o, lse_o = oracle.attend_fwd(xf["Q"], xf["K"], xf["V"], gi)
    assert_close(f64(out["O"]), O_o, dtype, "O")
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], t["dO"],
                              out["group_idx"])
    torch.cuda.synchronize()
    dQ_o, dK_o, dV_o = oracle.attend_bwd(xf["Q"], xf["K"], xf["V"], gi, xf["dO"])
    assert_close(f64(dQ), dQ_o, dtype, "dQ")
    assert_close(f64(dK), dK_o, dtype, "dK")
    assert_close(f64(dV), dV_o, dtype, "dV")


# ------------------------------------------------------------------ boundary extremes

EXTREMES = {
    # block routing at the largest budgets: 64 chunks (the 8-slot group select),
    # 512 groups (routing-row slots 256..511, the second pass of the row load)
    # out of 66 and 67 candidate chunks
    "k64_g512_bf16": syn.Workload("k64_g512_bf16", 1, 2, 1, 64, 128, 4352, 64, 512, "bf16",
                                  81, 0.125, backward=True),
    "k64_g512_fp32": syn.Workload("k64_g512_fp32", 1, 2, 1, 64, 128, 4352, 64, 512, "fp32",
                                  82, 0.3, backward=True),
    # more than 1024 routing rows per kv head (8 query heads x 129 blocks = 1032):
    # the dK/dV entry list is built in two passes over the rows
    "rows1032_bf16": syn.Workload("rows1032_bf16", 1, 8, 1, 64, 8256, 8256, 2, 8, "bf16", 83,
                                  0.125, backward=True),
}


@pytest.mark.parametrize("name", list(EXTREMES))
def test_boundary_extremes_full_parity(oracle, name):
    """Element-by-element parity at the limits the boundary accepts."""
    _full_parity(oracle, EXTREMES[name])


def test_causal_16k_full_size(oracle):
    """The full 16384-token causal self-attention (32q/8kv, D128, k16 g64):
    summaries and routing of every row; the forward of three sampled query
    heads on their blocks 128..255; the backward of one kv head with its four
    query heads on blocks 224..255.  A query block attends only keys at or
    before its own chunk, so the oracle run on the rows of blocks >= c (a
    segment at the end of the same history) gives those rows' O, lse and dQ
    exactly, and the complete dK, dV of every key in chunks >= c."""
    w = W["causal_16k"]
    print(f"[case] full {w.name}", flush=True)
    x = syn.make_inputs(w, with_grad_output=True)
    s, x, t, out = run_forward(w, x)
    Kf = syn.to_f64(x["K"], w.dtype)
    cm_o, gm_o = oracle.summaries(Kf)
    np.testing.assert_allclose(f64(out["chunk_mean"]), cm_o, atol=1e-5, rtol=1e-5)
    np.testing.assert_allclose(f64(out["group_mean"]), gm_o, atol=1e-5, rtol=1e-5)
    tolerated = check_routing(oracle, w, syn.to_f64(x["Q"], w.dtype), cm_o, gm_o,
                              out["chunk_idx"].cpu().numpy(), out["group_idx"].cpu().numpy())
    print(f"[routing] {w.name}: rows inside the near-tie band: {tolerated}", flush=True)
    del Kf, cm_o, gm_o
    r = w.n_q_heads // w.n_kv_heads
    gi = out["group_idx"].cpu().numpy()
    O, lse = f64(out["O"]), f64(out["lse"])
    c = 128
    qs = slice(64 * c, w.q_len)
    for hq in (0, 13, 31):
        hkv = hq // r
        O_o, lse_o = oracle.attend_fwd(syn.to_f64(x["Q"][:, hq:hq + 1, qs], w.dtype),
                                       syn.to_f64(x["K"][:, hkv:hkv + 1], w.dtype),
                                       syn.to_f64(x["V"][:, hkv:hkv + 1], w.dtype),
                                       gi[:, hq:hq + 1, c:])
        assert_close(O[:, hq:hq + 1, qs], O_o, w.dtype, f"O[{hq}]")
        assert_close(lse[:, hq:hq + 1, qs], lse_o, w.dtype, f"lse[{hq}]")
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], t["dO"],
                              out["group_idx"])
    torch.cuda.synchronize()
    hkv, c = 3, 224
    hs, qs, ks = slice(hkv * r, (hkv + 1) * r), slice(64 * c, w.q_len), slice(64 * c, w.kv_len)
    dQ_o, dK_o, dV_o = oracle.attend_bwd(syn.to_f64(x["Q"][:, hs, qs], w.dtype),
                                         syn.to_f64(x["K"][:, hkv:hkv + 1], w.dtype),
                                         syn.to_f64(x["V"][:, hkv:hkv + 1], w.dtype),
                                         gi[:, hs, c:], syn.to_f64(x["dO"][:, hs, qs], w.dtype))
    assert_close(f64(dQ)[:, hs, qs], dQ_o, w.dtype, "dQ")
    assert_close(f64(dK)[:, hkv:hkv + 1, ks], dK_o[:, :, ks], w.dtype, "dK")
    assert_close(f64(dV)[:, hkv:hkv + 1, ks], dV_o[:, :, ks], w.dtype, "dV")
