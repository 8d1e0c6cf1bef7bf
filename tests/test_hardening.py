"""The attention kernels on rows and workspaces that break the contract (needs
an MI355X).  Every case is in bounds by construction of the kernels' own
checks; the tests show the documented outcome:

- a routing row is read as its longest prefix of groups that lie before the
  block's own chunk and each exceed the entry before (page section "What HGA
  does differently": the kept groups of a block, in ascending order); the
  forward, the backward and decode on a malformed row equal the oracle on
  that prefix, so a group is never out of range or attended twice;
- a dK/dV call whose workspace holds no valid work order writes nothing.
"""
import math

import numpy as np
import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from gpu_common import DEV, assert_close, f64, shape_of, upload

pytestmark = pytest.mark.gpu


def _prefix_cut(gi, q0):
    """Host restatement of the prefix rule: each row cut at its first entry
    that is negative, at or past 8 * own chunk, or not above the one before."""
    out = np.full_like(gi, -1)
    B, H, nblk, g = gi.shape
    for b, h, blk in np.ndindex(B, H, nblk):
        lim = 8 * (q0 // 64 + blk)
        prev = -1
        for i in range(g):
            v = int(gi[b, h, blk, i])
            if v < 0 or v >= lim or v <= prev:
                break
            out[b, h, blk, i] = v
            prev = v
    return out


def _malformed(gi, q0, seed):
    """Routing rows spoiled in the ways a caller could: duplicates, a
    descending entry, an entry in the block's own chunk, a far out-of-range
    entry, a -1 hole followed by valid groups."""
    rng = np.random.default_rng(seed)
    bad = gi.copy()
    B, H, nblk, g = gi.shape
    kinds = ["dup", "desc", "own", "huge", "hole"]
    for n, (b, h, blk) in enumerate(np.ndindex(B, H, nblk)):
        row = bad[b, h, blk]
        k = int((row >= 0).sum())
        if k < 3:
            continue
        i = int(rng.integers(1, k))
        kind = kinds[n % len(kinds)]
        if kind == "dup":
            row[i] = row[i - 1]
        elif kind == "desc":
            row[i] = max(row[i - 1] - 5, 0)
        elif kind == "own":
            row[i] = 8 * (q0 // 64 + blk) + 3
        elif kind == "huge":
            row[i] = 1 << 30
        else:
            row[i] = -1
    return bad


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_malformed_rows_read_as_their_prefix(oracle, dtype):
    D = 128 if dtype == "bf16" else 64
    w = syn.Workload(f"malformed_{dtype}", 1, 4, 2, D, 256, 1024, 4, 24, dtype, 91,
                     1 / math.sqrt(D), backward=True)
    print(f"[case] {w.name}", flush=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, dtype)
    s = shape_of(w)
    out = hga.forward(s, t["Q"], t["K"], t["V"])
    torch.cuda.synchronize()
    q0 = w.kv_len - w.q_len
    bad = _malformed(out["group_idx"].cpu().numpy(), q0, 5)
    cut = _prefix_cut(bad, q0)
    assert not np.array_equal(cut, bad)
    gbad = torch.from_numpy(bad).to(DEV)
    O = torch.full_like(out["O"], float("nan"))
    lse = torch.full_like(out["lse"], float("nan"))
    hga.hga_attend_fwd(s, t["Q"], t["K"], t["V"], gbad, O, lse)
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], O, lse, t["dO"], gbad)
    torch.cuda.synchronize()
    xf = {k: syn.to_f64(v, dtype) for k, v in x.items()}
    O_o, lse_o = oracle.attend_fwd(xf["Q"], xf["K"], xf["V"], cut)
    assert_close(f64(O), O_o, dtype, "O")
    assert_close(f64(lse), lse_o, dtype, "lse")
    dQ_o, dK_o, dV_o = oracle.attend_bwd(xf["Q"], xf["K"], xf["V"], cut, xf["dO"])
    assert_close(f64(dQ), dQ_o, dtype, "dQ")
    assert_close(f64(dK), dK_o, dtype, "dK")
    assert_close(f64(dV), dV_o, dtype, "dV")


def test_malformed_decode_row_read_as_its_prefix(oracle):
    B, Hq, Hkv, D, L, k, g = 2, 4, 2, 128, 1000, 4, 20
    w = syn.Workload("malformed_decode", B, Hq, Hkv, D, 1, L, k, g, "bf16", 92,
                     1 / math.sqrt(D))
    s = hga.make_shape(B, Hq, Hkv, D, 1, L, k, g, dtype="bf16", kv_capacity=1024)
    x = syn.make_inputs(syn.scaled_workload(w, q_len=64, kv_len=1024))
    K = syn.to_torch(x["K"], "bf16", DEV)
    V = syn.to_torch(x["V"], "bf16", DEV)
    Q = syn.to_torch(x["Q"][:, :, 0], "bf16", DEV).contiguous()
    cm = torch.zeros(B, Hkv, 16, D, device=DEV)
    gm = torch.zeros(B, Hkv, 128, D, device=DEV)
    hga.hga_build_summaries(s, K, cm, gm, 0, L // 64)
    out = hga.decode(s, Q, K, V, cm, gm)
    torch.cuda.synchronize()
    gi = out["group_idx"].cpu().numpy()
    bad = gi.copy()
    cp = (L - 1) // 64
    bad[0, 0, 3] = bad[0, 0, 2]            # duplicate
    bad[0, 1, 5] = 8 * cp + 1              # inside the own chunk
    bad[1, 2, 1] = 1 << 30                 # out of range
    bad[1, 3, 4] = -1                      # hole
    gbad = torch.from_numpy(bad).to(DEV)
    O = torch.full_like(out["O"], float("nan"))
    lse = torch.full_like(out["lse"], float("nan"))
    hga.hga_decode_attend(s, Q, K, V, gbad, O, lse)
    torch.cuda.synchronize()
    # the oracle's attention over each row's prefix of kept groups + own chunk
    Kf = syn.to_f64(x["K"], "bf16")[:, :, :L]
    Vf = syn.to_f64(x["V"], "bf16")[:, :, :L]
    Qf = syn.to_f64(x["Q"][:, :, 0], "bf16")
    r = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            row, keep, prev = bad[b, h], [], -1
            for v in row[:min(g, 8 * min(k, cp))]:
                if v < 0 or v >= 8 * cp or v <= prev:
                    break
                keep.append(int(v))
                prev = v
            keys = np.concatenate([np.arange(8 * v, 8 * v + 8) for v in keep] +
                                  [np.arange(64 * cp, L)])
            lg = Kf[b, h // r, keys] @ Qf[b, h] / math.sqrt(D)
            m = lg.max()
            p = np.exp(lg - m)
            ref = (p[:, None] * Vf[b, h // r, keys]).sum(0) / p.sum()
            assert_close(f64(O)[b, h], ref, "bf16", f"decode O[{b},{h}]")
            assert_close(f64(lse)[b, h], m + math.log(p.sum()), "bf16", f"decode lse[{b},{h}]")


def test_dkdv_without_work_order_writes_nothing():
    """A dK/dV call whose workspace holds no valid work order (every entry -1,
    as if no dQ call had written it) writes no row of dK or dV, and nothing
    past them."""
    w = syn.Workload("no_order", 1, 4, 2, 128, 256, 1024, 4, 24, "bf16", 93,
                     1 / math.sqrt(128), backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, "bf16")
    s = shape_of(w)
    out = hga.forward(s, t["Q"], t["K"], t["V"])
    nbytes = hga.hga_attend_bwd_workspace(s)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    dQ = torch.empty_like(t["Q"])
    hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], t["dO"],
                          out["group_idx"], dQ, ws)
    # the work orders follow delta and the group-mask map (each part rounded to 256)
    r256 = lambda n: (n + 255) // 256 * 256
    off = r256(4 * 1 * 4 * 256) + r256(1 * 4 * 4 * 16)
    ws[off:].fill_(0xFF)
    n = t["K"].numel()
    big_k = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    big_v = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    dK = big_k[:n].view_as(t["K"])
    dV = big_v[:n].view_as(t["V"])
    hga.hga_attend_bwd_dkdv(s, t["Q"], t["K"], t["V"], out["lse"], t["dO"], out["group_idx"],
                            dK, dV, ws)
    torch.cuda.synchronize()
    assert torch.isnan(big_k.float()).all() and torch.isnan(big_v.float()).all()
