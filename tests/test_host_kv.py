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


@pytest.mark.parametrize("name,B,L,S,k,g,on_host,seg_dev,causal", [
    ("stage_dev", 1, 1024, 256, 3, 12, False, False, False),
    ("stage_host", 1, 1024, 256, 3, 12, True, False, False),
    # the active segment's keys and values also in device memory
    ("stage_host_segdev", 1, 1024, 256, 3, 12, True, True, False),
    # two sequences: every (b, kv head) has its own union and sources
    ("stage_host_segdev_b2", 2, 768, 256, 4, 20, True, True, False),
    # strictly causal routing (each segment's first block routed with the
    # previous segment's last 64 queries)
    ("stage_host_segdev_causal", 1, 1024, 256, 3, 12, True, True, True),
    # budgets that keep more groups than the history holds for early segments
    # and fewer than it for late ones: the union bounded both ways
    ("stage_host_wide", 1, 2048, 256, 20, 150, True, False, False),
])
def test_staged_working_set_matches_unstaged(name, B, L, S, k, g, on_host, seg_dev, causal):
    """Segment-wise training with each segment's routed working set staged
    into a compact device buffer (from the previous segment's staging where it
    holds a group) gives, segment by segment, the unstaged results bit for bit
    (O, lse, routing, dQ, the segment's dK and dV)."""
    from gpu_common import DEV
    print(f"[case] {name}", flush=True)
    w = syn.Workload(name, B, 4, 2, 128, L, L, k, g, "bf16", 43, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = {kk: syn.to_torch(v, "bf16", DEV) for kk, v in x.items()}
    outs = []
    for staged in (False, True):
        run = SegmentRunner(B, 4, 2, 128, L, S, k, g, device=DEV,
                            kv_on_host=on_host and staged, stage=staged, causal=causal)
        run.k_history.copy_(t["K"].cpu() if (on_host and staged) else t["K"])
        run.v_history.copy_(t["V"].cpu() if (on_host and staged) else t["V"])
        seg = []
        for i in range(L // S):
            rows = slice(i * S, (i + 1) * S)
            kv = {}
            if staged and seg_dev:
                kv = dict(K_seg=t["K"][:, :, rows].contiguous(), V_seg=t["V"][:, :, rows].contiguous())
            r = run.step(i, t["Q"][:, :, rows].contiguous(), t["dO"][:, :, rows].contiguous(), **kv)
            torch.cuda.synchronize()
            seg.append([v.clone() for v in (r.O, r.lse, r.group_idx, r.dQ, r.dK, r.dV)])
        outs.append(seg)
    for i, (a, b) in enumerate(zip(outs[0], outs[1])):
        for nm, u, v in zip(("O", "lse", "group_idx", "dQ", "dK", "dV"), a, b):
            assert torch.equal(u, v), (i, nm)


def test_stage_from_previous_writes_what_plain_staging_writes():
    """hga_stage_routed_from (previous staging and device segment rows as
    sources) writes the same staged rows, unions and rewritten routing rows
    as hga_stage_routed from the history alone, segment after segment; and
    from the second segment on most union groups are copied from the previous
    staging."""
    from gpu_common import DEV
    L, S, k, g = 2048, 256, 6, 40
    print("[case] stage_from L2048 S256", flush=True)
    w = syn.Workload("stage_from", 1, 4, 2, 128, L, L, k, g, "bf16", 44, 1 / math.sqrt(128),
                     backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = {kk: syn.to_torch(v, "bf16", DEV) for kk, v in x.items()}
    run = SegmentRunner(1, 4, 2, 128, L, S, k, g, device=DEV, kv_on_host=True, stage=True)
    run.k_history.copy_(t["K"].cpu())
    run.v_history.copy_(t["V"].cpu())
    kst = torch.empty_like(run.k_stages[0])
    vst = torch.empty_like(run.v_stages[0])
    gis = torch.empty_like(run.group_idx_staged)
    ws = torch.empty_like(run.stage_wss[0])
    nbh = 2
    for i in range(L // S):
        rows = slice(i * S, (i + 1) * S)
        run.forward(i, t["Q"][:, :, rows].contiguous(), K_seg=t["K"][:, :, rows].contiguous(),
                    V_seg=t["V"][:, :, rows].contiguous())
        s = run.shape(i)
        sg = run.stage_groups[i]
        hga.hga_stage_routed(s, run.group_idx, run.k_history, run.v_history, sg, kst, vst, gis, ws)
        torch.cuda.synchronize()
        assert torch.equal(gis, run.group_idx_staged), i
        lb = -(-(nbh * sg * 4) // 256) * 256
        cw = run.stage_wss[i % 2]
        cnt = cw[lb:lb + 4 * nbh].view(torch.int32).cpu()
        assert torch.equal(cnt, ws[lb:lb + 4 * nbh].view(torch.int32).cpu()), i
        ul_a = cw[:4 * nbh * sg].view(torch.int32).view(nbh, sg).cpu()
        ul_b = ws[:4 * nbh * sg].view(torch.int32).view(nbh, sg).cpu()
        src = cw[lb + 256:][:4 * nbh * sg].view(torch.int32).view(nbh, sg).cpu()
        from_prev = 0
        for h in range(nbh):
            n = int(cnt[h])
            assert torch.equal(ul_a[h, :n], ul_b[h, :n]), (i, h)
            written = list(range(8 * n)) + list(range(8 * sg, 8 * sg + S))
            assert torch.equal(run.k_stage[0, h, written], kst[0, h, written]), (i, h)
            assert torch.equal(run.v_stage[0, h, written], vst[0, h, written]), (i, h)
            from_prev += int((src[h, :n] >= 0).sum())
            if i == 0:
                assert int((src[h, :n] >= 0).sum()) == 0
        if i >= 2:
            # the previous staging held the previous segment and most of the
            # history before it
            assert from_prev > 0.5 * int(cnt.sum()), (i, from_prev, int(cnt.sum()))
