"""hga_attend_bwd_noalloc (the backward with its workspace held by the library,
for callers that cannot allocate) against hga_attend_bwd with a caller
workspace, bit for bit, on two calls in a row, the second with a smaller
problem (needs an MI355X)."""
import math

import pytest
import torch

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from gpu_common import DEV, shape_of, upload

pytestmark = pytest.mark.gpu

CASES = [
    syn.Workload("noalloc_big", 2, 8, 2, 128, 512, 2048, 8, 32, "bf16", 101,
                 1 / math.sqrt(128), backward=True),
    syn.Workload("noalloc_small", 1, 4, 1, 64, 128, 512, 3, 10, "bf16", 102, 0.125,
                 backward=True),
]


def _both(w):
    x = syn.make_inputs(w, with_grad_output=True)
    t = upload(x, w.dtype)
    s = shape_of(w)
    out = hga.forward(s, t["Q"], t["K"], t["V"])
    ref = hga.backward(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], t["dO"],
                       out["group_idx"])
    got = [torch.full_like(v, float("nan")) for v in ref]
    hga.hga_attend_bwd_noalloc(s, t["Q"], t["K"], t["V"], out["O"], out["lse"], t["dO"],
                               out["group_idx"], *got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_backward_equals_workspace_backward_twice():
    for w in CASES:
        print(f"[case] noalloc {w.name}", flush=True)
        ref, got = _both(w)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(a, b), f"{w.name}: {name} differs from hga_attend_bwd"


def test_noalloc_rejects_oversize_workspace():
    # 128 query heads x 16384 queries: the row statistics alone exceed 16 MiB
    s = hga.make_shape(1, 128, 8, 128, 16384, 16384, 16, 64, dtype="bf16")
    need = hga.hga_attend_bwd_workspace(s)
    assert need > (16 << 20)
    lib = hga._load()
    rc = lib.hga_attend_bwd_noalloc(__import__("ctypes").byref(s), *([16] * 10), None)
    assert rc == 4
