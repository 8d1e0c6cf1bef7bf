"""Keys and values in pinned host memory (the RAM tier of segment-wise
training): the kernels fetch the rows they gather across the host link.  The
results must be bit for bit those of device-resident keys and values (same
kernels, same order of operations), and the forward must match the oracle."""
import math

import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from hierarchical_routed_sparse_amd.segments import SegmentRunner

pytestmark = pytest.mark.gpu


def test_host_kv_matches_device(oracle):
    from gpu_common import DEV, assert_close, f64, shape_of, upload
    w = syn.Workload("host_kv", 1, 4, 2, 128, 256, 1024, 4, 20, "bf16", 41, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, "bf16")
    s = shape_of(w)
    Kh = t["K"].cpu().pin_memory()
    Vh = t["V"].cpu().pin_memory()
    res = []
    for K, V in ((t["K"], t["V"]), (Kh, Vh)):
        o = hga.forward(s, t["Q"], K, V)
        dQ, dK, dV = hga.backward(s, t["Q"], K, V, o["O"], o["lse"], t["dO"], o["group_idx"])
        torch.cuda.synchronize()
        res.append([o["chunk_mean"], o["group_mean"], o["group_idx"], o["O"], o["lse"], dQ, dK, dV])
    for a, b in zip(*res):
        assert torch.equal(a, b)
    xf = {k: syn.to_f64(v, "bf16") for k, v in x.items()}
    O_o, _ = oracle.attend_fwd(xf["Q"], xf["K"], xf["V"], res[1][2].cpu().numpy())
    assert_close(f64(res[1][3]), O_o, "bf16", "O (host K/V)")


def test_segments_with_host_kv_match_device():
    from gpu_common import DEV
    w = syn.Workload("seg_host", 1, 4, 2, 128, 512, 512, 3, 12, "bf16", 42, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = {k: syn.to_torch(v, "bf16", DEV) for k, v in x.items()}
    S = 256
    outs = []
    for on_host in (False, True):
        run = SegmentRunner(1, 4, 2, 128, 512, S, 3, 12, device=DEV, kv_on_host=on_host)
        run.k_history.copy_(t["K"].cpu() if on_host else t["K"])
        run.v_history.copy_(t["V"].cpu() if on_host else t["V"])
        seg = []
        for i in range(2):
            rows = slice(i * S, (i + 1) * S)
            r = run.step(i, t["Q"][:, :, rows].contiguous(), t["dO"][:, :, rows].contiguous())
            torch.cuda.synchronize()
            seg.append([v.clone() for v in (r.O, r.lse, r.group_idx, r.dQ, r.dK, r.dV)])
        outs.append(seg)
    for a, b in zip(outs[0], outs[1]):
        for u, v in zip(a, b):
            assert torch.equal(u, v)


@pytest.mark.parametrize("name,L,S,k,g,on_host", [
    ("stage_dev", 1024, 256, 3, 12, False),
    ("stage_host", 1024, 256, 3, 12, True),
    # budgets that keep more groups than the history holds for early segments
    # and fewer than it for late ones: the union bounded both ways
    ("stage_host_wide", 2048, 256, 20, 150, True),
])
def test_staged_working_set_matches_unstaged(name, L, S, k, g, on_host):
    """Segment-wise training with each segment's routed working set staged
    into a compact device buffer gives, segment by segment, the unstaged
    results bit for bit (O, lse, routing, dQ, the segment's dK and dV)."""
    from gpu_common import DEV
    print(f"[case] {name}", flush=True)
    w = syn.Workload(name, 1, 4, 2, 128, L, L, k, g, "bf16", 43, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = {kk: syn.to_torch(v, "bf16", DEV) for kk, v in x.items()}
    outs = []
    for staged in (False, True):
        run = SegmentRunner(1, 4, 2, 128, L, S, k, g, device=DEV,
                            kv_on_host=on_host and staged, stage=staged)
        run.k_history.copy_(t["K"].cpu() if (on_host and staged) else t["K"])
        run.v_history.copy_(t["V"].cpu() if (on_host and staged) else t["V"])
        seg = []
        for i in range(L // S):
            rows = slice(i * S, (i + 1) * S)
            r = run.step(i, t["Q"][:, :, rows].contiguous(), t["dO"][:, :, rows].contiguous())
            torch.cuda.synchronize()
            seg.append([v.clone() for v in (r.O, r.lse, r.group_idx, r.dQ, r.dK, r.dV)])
        outs.append(seg)
    for i, (a, b) in enumerate(zip(outs[0], outs[1])):
        for nm, u, v in zip(("O", "lse", "group_idx", "dQ", "dK", "dV"), a, b):
            assert torch.equal(u, v), (i, nm)
