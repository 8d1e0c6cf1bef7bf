"""The entry points launch only kernels (no allocation, no memset), so a step
captured into a HIP graph replays the eager work: every replay, with eager work
and synchronisations between replays, must equal the eager result bit for bit
(needs an MI355X)."""
import math

import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outs, ref, n=3):
    for i in range(n):
        for o in outs:                       # eager work between replays
            o.fill_(float("nan") if o.is_floating_point() else -7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"replay {i}: output {k} differs from the eager step"


def test_forward_backward_step_replays_bit_exact():
    w = syn.Workload("graph", 2, 8, 2, 128, 256, 1024, 4, 20, "bf16", 51, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w)
    t = {k: syn.to_torch(v, "bf16", DEV) for k, v in x.items()}
    s = hga.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.q_len, w.kv_len,
                       w.top_k, w.top_g)
    sz = hga._sizes(s)
    cm = torch.empty(sz["cm"], device=DEV)
    gm = torch.empty(sz["gm"], device=DEV)
    ci = torch.empty(sz["ci"], dtype=torch.int32, device=DEV)
    gi = torch.empty(sz["gi"], dtype=torch.int32, device=DEV)
    O = torch.empty(sz["q"], dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(sz["lse"], device=DEV)
    dQ = torch.empty_like(O)
    dK = torch.empty(sz["kv"], dtype=torch.bfloat16, device=DEV)
    dV = torch.empty_like(dK)
    ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=DEV)

    def step():
        hga.hga_build_summaries(s, t["K"], cm, gm)
        hga.hga_route(s, t["Q"], cm, gm, ci, gi)
        hga.hga_attend_fwd(s, t["Q"], t["K"], t["V"], gi, O, lse)
        hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], O, lse, t["dO"], gi, dQ, ws)
        hga.hga_attend_bwd_dkdv(s, t["Q"], t["K"], t["V"], lse, t["dO"], gi, dK, dV, ws)

    outs = [cm, gm, ci, gi, O, lse, dQ, dK, dV]
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    _replays_match(_capture(step), outs, ref)


def test_decode_step_replays_bit_exact():
    w = syn.Workload("graph_dec", 4, 8, 2, 128, 1, 3000, 8, 40, "bf16", 52, 1 / math.sqrt(128))
    x = syn.make_inputs(w)
    cap = 3008
    s = hga.make_shape(4, 8, 2, 128, 1, 3000, 8, 40, kv_capacity=cap)
    K = torch.zeros(4, 2, cap, 128, dtype=torch.bfloat16, device=DEV)
    V = torch.zeros_like(K)
    K[:, :, :3000] = syn.to_torch(x["K"], "bf16", DEV)
    V[:, :, :3000] = syn.to_torch(x["V"], "bf16", DEV)
    Q = syn.to_torch(x["Q"], "bf16", DEV)[:, :, 0].contiguous()
    cm = torch.zeros(4, 2, cap // 64, 128, device=DEV)
    gm = torch.zeros(4, 2, cap // 8, 128, device=DEV)
    hga.hga_build_summaries(s, K, cm, gm, 0, 3000 // 64)
    ci = torch.empty(4, 8, 8, dtype=torch.int32, device=DEV)
    gi = torch.empty(4, 8, 40, dtype=torch.int32, device=DEV)
    O = torch.empty(4, 8, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(4, 8, device=DEV)

    def step():
        hga.hga_decode(s, Q, K, V, cm, gm, ci, gi, O, lse)

    outs = [ci, gi, O, lse]
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    _replays_match(_capture(step), outs, ref)
