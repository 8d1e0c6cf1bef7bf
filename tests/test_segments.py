"""Segment-wise HGA (history detached) against the oracle, segment by segment.

For segment i of a sequence cut into S-token segments, the oracle runs on the
segment's queries over the keys/values of positions [0, (i+1) S): summaries,
routing (compared under the near-tie rule), attention forward on the GPU's
routing, and the backward; dQ is compared in full and dK, dV on the segment's
own rows, the only rows the segment-wise backward writes.  Rows of dK, dV
outside the segments processed so far must stay untouched.
"""
import math

import numpy as np
import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from hierarchical_routed_sparse_amd.segments import SegmentRunner


def _seq_workload(dtype="bf16"):
    # 4 segments of 256 tokens; 32 q / 8 kv heads would be slow in the oracle:
    # 4 q / 2 kv heads, D 128, k 3, g 12
    return syn.Workload("seg_1k", 1, 4, 2, 128, 1024, 1024, 3, 12, dtype, 31,
                        1 / math.sqrt(128), backward=True)


def test_segment_shapes_validate():
    r = SegmentRunner.__new__(SegmentRunner)
    r.B, r.Hq, r.Hkv, r.D, r.L, r.S, r.top_k, r.top_g = 1, 32, 8, 128, 16384, 2048, 16, 64
    r.dtype, r.scale, r.nseg = "bf16", 0.0, 8
    sizes = []
    for i in range(r.nseg):
        s = r.shape(i)
        assert hga.hga_validate_shape(s) == 0
        assert s.kv_len == (i + 1) * 2048 and s.kv_capacity == 16384
        sizes.append(hga.hga_attend_bwd_workspace(s))
    assert sizes == sorted(sizes)


@pytest.mark.gpu
def test_segments_match_oracle(oracle):
    from gpu_common import DEV, assert_close, check_routing, f64
    w = _seq_workload()
    x = syn.make_inputs(w, with_grad_output=True)
    S = 256
    run = SegmentRunner(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.kv_len, S, w.top_k,
                        w.top_g, dtype=w.dtype, device=DEV)
    t = {k: syn.to_torch(v, w.dtype, DEV) for k, v in x.items()}
    run.k_history.copy_(t["K"])
    run.v_history.copy_(t["V"])
    run.dK.fill_(float("nan"))
    run.dV.fill_(float("nan"))
    for i in range(w.kv_len // S):
        print(f"[case] segment {i}", flush=True)
        rows = slice(i * S, (i + 1) * S)
        Q = t["Q"][:, :, rows].contiguous()
        dO = t["dO"][:, :, rows].contiguous()
        res = run.step(i, Q, dO)
        torch.cuda.synchronize()
        # the oracle on the segment over its history
        ws = syn.Workload(f"seg{i}", w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, S,
                          (i + 1) * S, w.top_k, w.top_g, w.dtype, w.seed, w.qv_scale)
        Qf = syn.to_f64(x["Q"][:, :, rows], w.dtype)
        Kf = syn.to_f64(x["K"][:, :, :(i + 1) * S], w.dtype)
        Vf = syn.to_f64(x["V"][:, :, :(i + 1) * S], w.dtype)
        dOf = syn.to_f64(x["dO"][:, :, rows], w.dtype)
        cm, gm = oracle.summaries(Kf)
        n = (i + 1) * S // 64
        np.testing.assert_allclose(f64(run.chunk_mean[:, :, :n]), cm, atol=1e-5, rtol=1e-5)
        np.testing.assert_allclose(f64(run.group_mean[:, :, :8 * n]), gm, atol=1e-5, rtol=1e-5)
        gi = run.group_idx.cpu().numpy()
        check_routing(oracle, ws, Qf, cm, gm, run.chunk_idx.cpu().numpy(), gi)
        O_o, lse_o = oracle.attend_fwd(Qf, Kf, Vf, gi)
        assert_close(f64(res.O), O_o, w.dtype, f"O seg {i}")
        assert_close(f64(res.lse), lse_o, w.dtype, f"lse seg {i}")
        dQ_o, dK_o, dV_o = oracle.attend_bwd(Qf, Kf, Vf, gi, dOf)
        assert_close(f64(res.dQ), dQ_o, w.dtype, f"dQ seg {i}")
        assert_close(f64(res.dK), dK_o[:, :, rows], w.dtype, f"dK seg {i}")
        assert_close(f64(res.dV), dV_o[:, :, rows], w.dtype, f"dV seg {i}")
        # rows of later segments are still untouched
        later = slice((i + 1) * S, None)
        assert torch.isnan(run.dK[:, :, later].float()).all()
        assert torch.isnan(run.dV[:, :, later].float()).all()
