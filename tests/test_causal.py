"""Strictly causal routing (hga_route_causal): HIP path vs the oracle's causal
routing, element by element, and the causality property on the GPU (needs an
MI355X, except the host-side checks at the end).

Block j is routed with the mean of the 64 queries before it; the attention and
the backward take the resulting indices unchanged, so they are compared
against the oracle on the GPU's own routing, as for the block method.
Tolerances: (2e-2, 1e-2) for bf16, (1e-5, 1e-5) for fp32.
"""
import ctypes
import math

import numpy as np
import pytest

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from gpu_common import random_shapes

CASES = {
    "bf16_seg_b2": syn.Workload("c1", 2, 8, 2, 128, 256, 1024, 4, 20, "bf16", 61,
                                1 / math.sqrt(128), backward=True),
    "bf16_self_512": syn.Workload("c2", 1, 4, 2, 128, 512, 512, 3, 12, "bf16", 62,
                                  1 / math.sqrt(128), backward=True),
    "fp32_d64_seg": syn.Workload("c3", 1, 2, 1, 64, 192, 448, 2, 9, "fp32", 63, 0.4,
                                 backward=True),
    "bf16_r8_k0": syn.Workload("c4", 1, 8, 1, 128, 128, 384, 0, 8, "bf16", 64,
                               1 / math.sqrt(128), backward=True),
}


RANDOM = random_shapes(8, seed=211)


def _run(w, x, causal=True):
    import torch
    from gpu_common import shape_of, upload
    t = upload(x, w.dtype)
    s = shape_of(w)
    out = hga.forward(s, t["Q"], t["K"], t["V"], causal=causal,
                      Q_prev=t.get("Qprev") if w.kv_len > w.q_len else None)
    torch.cuda.synchronize()
    return s, t, out


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_causal_small_case_full_parity(oracle, name):
    _causal_full_parity(oracle, CASES[name])


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(RANDOM))
def test_causal_random_shapes_full_parity(oracle, name):
    """The same comparison on seeded random valid shapes."""
    _causal_full_parity(oracle, RANDOM[name])


def _causal_full_parity(oracle, w):
    import torch
    from gpu_common import DEV, assert_close, check_routing, f64
    print(f"[case] causal {w.name}", flush=True)
    x = syn.make_inputs(w, with_qprev=True)
    s, t, out = _run(w, x)
    xf = {k: syn.to_f64(v, w.dtype) for k, v in x.items()}
    cm_o, gm_o = oracle.summaries(xf["K"])
    ci, gi = out["chunk_idx"].cpu().numpy(), out["group_idx"].cpu().numpy()
    check_routing(oracle, w, xf["Q"], cm_o, gm_o, ci, gi, causal=True,
                  Qprev=xf["Qprev"] if w.kv_len > w.q_len else None)
    O_o, lse_o = oracle.attend_fwd(xf["Q"], xf["K"], xf["V"], gi)
    assert_close(f64(out["O"]), O_o, w.dtype, "O")
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], t["dO"],
                              out["group_idx"])
    torch.cuda.synchronize()
    dQ_o, dK_o, dV_o = oracle.attend_bwd(xf["Q"], xf["K"], xf["V"], gi, xf["dO"])
    assert_close(f64(dQ), dQ_o, w.dtype, "dQ")
    assert_close(f64(dK), dK_o, w.dtype, "dK")
    assert_close(f64(dV), dV_o, w.dtype, "dV")


@pytest.mark.gpu
@pytest.mark.parametrize("t_cut", [64 * 3 + 17, 64 * 6])
def test_causal_outputs_do_not_see_the_future_on_gpu(t_cut):
    """Replacing every query, key and value from position t on leaves the GPU's
    outputs at earlier positions bit-identical (deterministic kernels)."""
    import torch
    w = CASES["bf16_self_512"]
    x = syn.make_inputs(w)
    _, _, a = _run(w, x)
    y = {k: v.copy() for k, v in x.items()}
    z = syn.make_inputs(syn.scaled_workload(w, seed=99))
    for k in ("Q", "K", "V"):
        y[k][:, :, t_cut:] = z[k][:, :, t_cut:]
    _, _, b = _run(w, y)
    assert torch.equal(a["O"][:, :, :t_cut], b["O"][:, :, :t_cut])
    assert torch.equal(a["lse"][:, :, :t_cut], b["lse"][:, :, :t_cut])


@pytest.mark.gpu
def test_causal_full_size_routing(oracle):
    """The benchmark workload (2048 queries over 16384 keys) with causal
    routing: summaries and routing in full against the oracle."""
    from gpu_common import check_routing
    w = syn.WORKLOADS["segment_2k_over_16k"]
    print("[case] causal full size", flush=True)
    x = syn.make_inputs(w, with_qprev=True)
    _, _, out = _run(w, x)
    Kf = syn.to_f64(x["K"], w.dtype)
    cm_o, gm_o = oracle.summaries(Kf)
    del Kf
    tol = check_routing(oracle, w, syn.to_f64(x["Q"], w.dtype), cm_o, gm_o,
                        out["chunk_idx"].cpu().numpy(), out["group_idx"].cpu().numpy(),
                        causal=True, Qprev=syn.to_f64(x["Qprev"], w.dtype))
    print(f"[routing] causal full size: rows inside the near-tie band: {tol}", flush=True)


@pytest.mark.gpu
def test_causal_segments_route_like_the_whole_sequence(oracle):
    """Segment-wise causal routing (the runner carries each segment's last 64
    queries to the next) equals the oracle's causal routing of the whole
    sequence, segment by segment."""
    import torch
    from gpu_common import check_routing
    from hierarchical_routed_sparse_amd.segments import SegmentRunner
    L, S = 1024, 256
    w = syn.Workload("cseg", 1, 4, 2, 128, L, L, 3, 12, "bf16", 65, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w)
    t = {k: syn.to_torch(v, "bf16", "cuda:0") for k, v in x.items()}
    run = SegmentRunner(1, 4, 2, 128, L, S, 3, 12, device="cuda:0", causal=True)
    run.k_history.copy_(t["K"])
    run.v_history.copy_(t["V"])
    Qf, Kf = syn.to_f64(x["Q"], "bf16"), syn.to_f64(x["K"], "bf16")
    cm_o, gm_o = oracle.summaries(Kf)
    for i in range(L // S):
        run.forward(i, t["Q"][:, :, i * S:(i + 1) * S].contiguous())
        torch.cuda.synchronize()
        ws = syn.scaled_workload(w, q_len=S, kv_len=(i + 1) * S)
        check_routing(oracle, ws, Qf[:, :, i * S:(i + 1) * S], cm_o[:, :, :(i + 1) * S // 64],
                      gm_o[:, :, :(i + 1) * S // 8], run.chunk_idx.cpu().numpy(),
                      run.group_idx.cpu().numpy(), causal=True,
                      Qprev=Qf[:, :, i * S - 64:i * S] if i > 0 else None)


def test_route_causal_argument_errors():
    """Host-side checks: nothing is launched on an error."""
    lib = ctypes.CDLL(hga.lib_path())
    lib.hga_route_causal.restype = ctypes.c_int
    lib.hga_route_causal.argtypes = [ctypes.POINTER(hga.HgaShape)] + [ctypes.c_void_p] * 7
    seg = hga.make_shape(1, 32, 8, 128, 2048, 16384, 16, 64)
    assert lib.hga_route_causal(ctypes.byref(seg), 16, None, 16, 16, 16, 16, None) == 1
    assert lib.hga_route_causal(ctypes.byref(seg), None, 16, 16, 16, 16, 16, None) == 1
    assert lib.hga_route_causal(ctypes.byref(seg), 16, 16, 16, 16, 16, None, None) == 1
    bad = hga.make_shape(1, 32, 8, 128, 2048, 1024, 16, 64)
    assert lib.hga_route_causal(ctypes.byref(bad), 16, 16, 16, 16, 16, 16, None) == 2
    dec = hga.make_shape(1, 32, 8, 128, 1, 1024, 16, 64)
    assert lib.hga_route_causal(ctypes.byref(dec), 16, 16, 16, 16, 16, 16, None) == 2


# ------------------------------------------------------------------ decode

@pytest.mark.gpu
@pytest.mark.parametrize("L0,k,g", [(16384 + 64 * 3, 16, 64), (640, 3, 11), (64, 2, 8)])
def test_causal_decode_routes_once_per_block(oracle, L0, k, g):
    """hga_decode_route_causal for block j = L0 / 64 equals the oracle's causal
    routing of a one-block segment whose preceding queries are block j - 1;
    every token of block j then attends with those groups exactly what the
    oracle's attention gives its row of the block."""
    import torch
    from gpu_common import DEV, check_routing
    j = L0 // 64
    w = syn.Workload("cdec", 2, 8, 2, 128, 64, L0 + 64, k, g, "bf16", 66, 1 / math.sqrt(128))
    x = syn.make_inputs(w, with_qprev=True)        # Q: block j, Qprev: block j - 1
    cap = L0 + 64
    K = syn.to_torch(x["K"], "bf16", DEV)
    V = syn.to_torch(x["V"], "bf16", DEV)
    cm = torch.full((2, 2, cap // 64, 128), float("nan"), device=DEV)
    gm = torch.full((2, 2, cap // 8, 128), float("nan"), device=DEV)
    s0 = hga.make_shape(2, 8, 2, 128, 1, L0 + 1, k, g, kv_capacity=cap)
    hga.hga_build_summaries(s0, K, cm, gm, 0, j)
    ci = torch.full((2, 8, k), -7, dtype=torch.int32, device=DEV)
    gi = torch.full((2, 8, g), -7, dtype=torch.int32, device=DEV)
    Qp = syn.to_torch(x["Qprev"], "bf16", DEV) if j > 0 else None
    hga.hga_decode_route_causal(s0, Qp, cm, gm, ci, gi)
    torch.cuda.synchronize()
    xf = {kk: syn.to_f64(v, "bf16") for kk, v in x.items()}
    # the oracle's layout spans the segment's own chunk j too (never a candidate)
    cm_o, gm_o = oracle.summaries(xf["K"][:, :, :64 * (j + 1)])
    wb = syn.scaled_workload(w, kv_len=64 * (j + 1))
    ci_n = ci.cpu().numpy()[:, :, None]
    gi_n = gi.cpu().numpy()[:, :, None]
    if j > 0:
        check_routing(oracle, wb, xf["Q"], cm_o, gm_o, ci_n, gi_n, causal=True, Qprev=xf["Qprev"])
    else:
        assert (ci_n == -1).all() and (gi_n == -1).all()
    # every token of the block, attended with the block's groups
    O_o, lse_o = oracle.attend_fwd(xf["Q"], xf["K"][:, :, :64 * (j + 1)],
                                   xf["V"][:, :, :64 * (j + 1)], gi_n)
    Qt = syn.to_torch(x["Q"], "bf16", DEV)
    for i in (0, 17, 63):
        s = hga.make_shape(2, 8, 2, 128, 1, 64 * j + i + 1, k, g, kv_capacity=cap)
        O = torch.empty(2, 8, 128, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(2, 8, device=DEV)
        hga.hga_decode_attend(s, Qt[:, :, i].contiguous(), K, V, gi, O, lse)
        torch.cuda.synchronize()
        got = O.float().cpu().numpy().astype(np.float64)
        ref = O_o[:, :, i]
        assert (np.abs(got - ref) <= 2e-2 + 1e-2 * np.abs(ref)).all(), i
        assert np.allclose(lse.cpu().numpy(), lse_o[:, :, i], atol=2e-2, rtol=1e-2), i


def test_decode_route_causal_argument_errors():
    lib = ctypes.CDLL(hga.lib_path())
    lib.hga_decode_route_causal.restype = ctypes.c_int
    lib.hga_decode_route_causal.argtypes = [ctypes.POINTER(hga.HgaShape)] + [ctypes.c_void_p] * 6
    s = hga.make_shape(4, 32, 8, 128, 1, 16424, 16, 64, kv_capacity=16448)
    assert lib.hga_decode_route_causal(ctypes.byref(s), None, 16, 16, 16, 16, None) == 1  # Q_prev
    assert lib.hga_decode_route_causal(ctypes.byref(s), 16, 16, 16, 16, None, None) == 1  # group_idx
    assert lib.hga_decode_route_causal(ctypes.byref(s), 16, None, 16, 16, 16, None) == 1  # summaries
    blk = hga.make_shape(4, 32, 8, 128, 64, 16384, 16, 64)
    assert lib.hga_decode_route_causal(ctypes.byref(blk), 16, 16, 16, 16, 16, None) == 2
