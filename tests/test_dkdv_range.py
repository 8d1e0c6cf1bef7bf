"""dK/dV over a chunk range (hga_attend_bwd_dkdv_range) against the full
backward on the same inputs and routing (needs an MI355X).

Each 64-key chunk's dK and dV rows are summed by one workgroup in a fixed
order whatever range it is launched in, so the rows of the range must equal
the full call's rows bit for bit; rows outside the range must be untouched.
Ranges that start and end off a multiple of 4 chunks take the byte-wise path
of the work-order kernel."""
import math

import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from gpu_common import DEV, run_forward

pytestmark = pytest.mark.gpu

CASES = {
    # B = 2, 16 chunks
    "bf16_b2_1k": (syn.Workload("bf16_b2_1k", 2, 8, 2, 128, 256, 1024, 4, 20, "bf16", 31,
                                1 / math.sqrt(128), backward=True),
                   [(0, 16), (3, 9), (0, 1), (15, 16), (5, 6), (4, 12)]),
    # 10 chunks (not a multiple of 4)
    "bf16_r8_640": (syn.Workload("bf16_r8_640", 1, 8, 1, 128, 256, 640, 2, 40, "bf16", 32,
                                 1 / math.sqrt(128), backward=True),
                    [(0, 10), (1, 10), (6, 7), (2, 5)]),
    "fp32_d64_512": (syn.Workload("fp32_d64_512", 1, 4, 2, 64, 192, 512, 3, 9, "fp32", 33, 0.2,
                                  backward=True),
                     [(0, 8), (1, 3), (7, 8)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_range_rows_equal_full_call(name):
    w, ranges = CASES[name]
    print(f"[case] dkdv range {name}", flush=True)
    s, x, t, out = run_forward(w)
    x.update(syn.make_inputs(w, with_grad_output=True))
    dO = syn.to_torch(x["dO"], w.dtype, DEV)
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], dO,
                              out["group_idx"])
    torch.cuda.synchronize()
    ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=DEV)
    dQ2 = torch.empty_like(dQ)
    hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], dO, out["group_idx"],
                          dQ2, ws)
    torch.cuda.synchronize()
    assert torch.equal(dQ2, dQ)
    for c0, c1 in ranges:
        dK2 = torch.full_like(dK, float("nan"))
        dV2 = torch.full_like(dV, float("nan"))
        hga.hga_attend_bwd_dkdv_range(s, t["Q"], t["K"], t["V"], out["lse"], dO,
                                      out["group_idx"], c0, c1, dK2, dV2, ws)
        torch.cuda.synchronize()
        k0, k1 = 64 * c0, 64 * c1
        assert torch.equal(dK2[:, :, k0:k1], dK[:, :, k0:k1]), (c0, c1)
        assert torch.equal(dV2[:, :, k0:k1], dV[:, :, k0:k1]), (c0, c1)
        assert torch.isnan(dK2[:, :, :k0]).all() and torch.isnan(dK2[:, :, k1:]).all()
        assert torch.isnan(dV2[:, :, :k0]).all() and torch.isnan(dV2[:, :, k1:]).all()


def test_range_call_leaves_the_full_range_order_intact():
    """The dQ call writes the whole range's dK/dV work order into the
    workspace; a chunk sub-range call orders its own range in a second
    buffer.  A full-range dK/dV call after a sub-range call on the same
    workspace must still equal the full backward bit for bit."""
    w, _ = CASES["bf16_b2_1k"]
    print("[case] dkdv full after range", flush=True)
    s, x, t, out = run_forward(w)
    x.update(syn.make_inputs(w, with_grad_output=True))
    dO = syn.to_torch(x["dO"], w.dtype, DEV)
    dQ, dK, dV = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], dO,
                              out["group_idx"])
    ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=DEV)
    dQ2 = torch.empty_like(dQ)
    hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], dO, out["group_idx"],
                          dQ2, ws)
    dK2 = torch.full_like(dK, float("nan"))
    dV2 = torch.full_like(dV, float("nan"))
    hga.hga_attend_bwd_dkdv_range(s, t["Q"], t["K"], t["V"], out["lse"], dO, out["group_idx"],
                                  3, 9, dK2, dV2, ws)
    hga.hga_attend_bwd_dkdv(s, t["Q"], t["K"], t["V"], out["lse"], dO, out["group_idx"],
                            dK2, dV2, ws)
    torch.cuda.synchronize()
    assert torch.equal(dK2, dK) and torch.equal(dV2, dV)
