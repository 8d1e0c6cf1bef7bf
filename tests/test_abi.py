"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad arguments before launching anything (host-only checks)."""
import ctypes
import os
import re

import pytest

import hierarchical_routed_sparse_amd as hga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "hga.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hga_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hga.lib_path()):
        from hierarchical_routed_sparse_amd import build_lib
        build_lib.build()
    return ctypes.CDLL(hga.lib_path())


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"hga_build_summaries", "hga_route", "hga_attend_fwd", "hga_attend_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert hga.hga_abi_version() == 11


def _ok_shape(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, q_len=2048, kv_len=16384,
                top_k=16, top_g=64, dtype="bf16")
    base.update(kw)
    return hga.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"dtype": "fp32", "head_dim": 64}, 0),
    ({"q_len": 16384}, 0),
    ({"top_k": 0, "top_g": 0}, 0),
    ({"batch": 0}, 2),
    ({"n_q_heads": 30}, 2),              # not a multiple of n_kv_heads
    ({"q_len": 100}, 2),                 # not a multiple of 64
    ({"q_len": 0}, 2),
    ({"kv_len": 1024}, 2),               # shorter than q_len
    ({"kv_len": 16400}, 2),              # not a multiple of 64
    ({"kv_len": 262144, "q_len": 2048}, 2),
    ({"top_k": 65}, 2),
    ({"top_k": -1}, 2),
    ({"top_g": 513}, 2),
    ({"head_dim": 96}, 3),
    ({"dtype": 7}, 3),
    ({"softmax_scale": float("nan")}, 2),
    ({"softmax_scale": float("inf")}, 2),
    ({"softmax_scale": -1.0}, 0),                 # <= 0 selects 1/sqrt(head_dim)
    ({"kv_capacity": 32768}, 0),                  # rows allocated beyond kv_len
    ({"kv_capacity": 16384}, 0),                  # equal to kv_len
    ({"kv_capacity": 8192}, 2),                   # smaller than kv_len
    ({"kv_capacity": 16400}, 2),                  # not a multiple of 64
    ({"kv_capacity": 262144}, 2),                 # beyond the maximum
])
def test_validate_shape(kw, status):
    assert hga.hga_validate_shape(_ok_shape(**kw)) == status


def test_null_and_workspace_errors_before_launch(lib):
    s = _ok_shape()
    SP = ctypes.POINTER(hga.HgaShape)
    lib.hga_build_summaries.argtypes = [SP] + [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 2 + [ctypes.c_void_p]
    assert lib.hga_build_summaries(ctypes.byref(s), None, None, None, 0, 256, None) == 1
    # a non-null but bogus pointer with a bad chunk range is still rejected before launch
    assert lib.hga_build_summaries(ctypes.byref(s), 16, 16, 16, 0, 257, None) == 2
    assert lib.hga_build_summaries(ctypes.byref(s), 16, 16, 16, 5, 4, None) == 2
    lib.hga_route.argtypes = [SP] + [ctypes.c_void_p] * 6
    assert lib.hga_route(ctypes.byref(s), 16, 16, None, None, None, None) == 1   # top_g>0 needs group_idx
    lib.hga_attend_fwd.argtypes = [SP] + [ctypes.c_void_p] * 7
    assert lib.hga_attend_fwd(ctypes.byref(s), 16, 16, 16, None, 16, None, None) == 1
    lib.hga_attend_bwd.argtypes = [SP] + [ctypes.c_void_p] * 11 + [ctypes.c_size_t, ctypes.c_void_p]
    need = hga.hga_attend_bwd_workspace(s)
    assert need >= 4 * 32 * 2048
    args = [16] * 11
    assert lib.hga_attend_bwd(ctypes.byref(s), *args[:10], None, need, None) == 4
    assert lib.hga_attend_bwd(ctypes.byref(s), *args, need - 1, None) == 4
    # the workspace holds delta, the one-byte-per-(routing row, chunk) group map
    # and two dK/dV work orders (one int per (b, kv head, chunk) each)
    nblk, nch = 2048 // 64, 16384 // 64
    assert need == 4 * 32 * 2048 + 32 * nblk * nch + 2 * 4 * 8 * nch
    lib.hga_attend_bwd_dkdv_range.argtypes = ([SP] + [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 2
                                              + [ctypes.c_void_p] * 3 + [ctypes.c_size_t,
                                                                         ctypes.c_void_p])
    rng = [16] * 6
    assert lib.hga_attend_bwd_dkdv_range(ctypes.byref(s), *rng, 5, 4, 16, 16, 16, need, None) == 2
    assert lib.hga_attend_bwd_dkdv_range(ctypes.byref(s), *rng, 0, nch + 1, 16, 16, 16, need,
                                         None) == 2
    assert lib.hga_attend_bwd_dkdv_range(ctypes.byref(s), *rng, 7, 7, 16, 16, 16, need, None) == 0
    assert lib.hga_validate_shape(None) == 1


def test_status_strings(lib):
    lib.hga_status_str.restype = ctypes.c_char_p
    for code in range(6):
        assert lib.hga_status_str(code)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hga, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(hga, "_libs", {})
    with pytest.raises(hga.HGAError):
        hga.hga_abi_version()


def _dec_shape(**kw):
    base = dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, q_len=1, kv_len=16424,
                top_k=16, top_g=64, dtype="bf16", kv_capacity=16448)
    base.update(kw)
    return hga.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"kv_len": 1, "kv_capacity": 64}, 0),           # the very first token
    ({"kv_len": 64, "kv_capacity": 0}, 0),           # capacity 0 = kv_len, a multiple of 64
    ({"kv_len": 100, "kv_capacity": 0}, 2),          # capacity must be a multiple of 64
    ({"kv_capacity": 16400}, 2),
    ({"kv_capacity": 16384}, 2),                     # below kv_len
    ({"kv_capacity": -64}, 2),
    ({"kv_len": 0}, 2),
    ({"q_len": 64}, 2),                              # a block shape is not a decode shape
    ({"kv_len": 131073, "kv_capacity": 131136}, 2),
    ({"top_g": 513}, 2),
    ({"n_q_heads": 30}, 2),
    ({"head_dim": 96}, 3),
    ({"dtype": 7}, 3),
    ({"softmax_scale": float("nan")}, 2),
])
def test_validate_decode_shape(kw, status):
    assert hga.hga_validate_decode_shape(_dec_shape(**kw)) == status


def test_block_and_decode_shapes_are_told_apart():
    assert hga.hga_validate_shape(_dec_shape()) == 2
    assert hga.hga_validate_decode_shape(_ok_shape()) == 2


def test_decode_argument_errors(lib):
    s = _dec_shape()
    lib.hga_decode.restype = ctypes.c_int
    lib.hga_decode.argtypes = [ctypes.POINTER(hga.HgaShape)] + [ctypes.c_void_p] * 10
    ok = [16] * 10    # dummy non-null addresses; nothing is launched on an error
    assert lib.hga_decode(None, *ok) == 1
    for i in (0, 1, 2, 7):             # Q, K, V, O
        args = list(ok)
        args[i] = None
        assert lib.hga_decode(ctypes.byref(s), *args) == 1
    args = list(ok)
    args[6] = None                      # group_idx with top_g > 0
    assert lib.hga_decode(ctypes.byref(s), *args) == 1
    args = list(ok)
    args[3] = None                      # chunk summaries when there are candidates
    assert lib.hga_decode(ctypes.byref(s), *args) == 1
    bad = _dec_shape(kv_capacity=16400)
    assert lib.hga_decode(ctypes.byref(bad), *ok) == 2
    assert lib.hga_decode(ctypes.byref(_ok_shape()), *ok) == 2


def test_build_summaries_accepts_decode_shapes_complete_chunks_only(lib):
    s = _dec_shape()      # kv_len 16424: 256 complete chunks
    lib.hga_build_summaries.restype = ctypes.c_int
    assert lib.hga_build_summaries(ctypes.byref(s), 16, 16, 16, 0, 257, None) == 2
    assert lib.hga_build_summaries(ctypes.byref(s), 16, 16, 16, 3, 3, None) == 0   # empty range


def test_decode_halves_argument_errors(lib):
    s = _dec_shape()
    sp = ctypes.POINTER(hga.HgaShape)
    lib.hga_decode_route.restype = ctypes.c_int
    lib.hga_decode_route.argtypes = [sp] + [ctypes.c_void_p] * 6
    lib.hga_decode_attend.restype = ctypes.c_int
    lib.hga_decode_attend.argtypes = [sp] + [ctypes.c_void_p] * 7
    assert lib.hga_decode_route(ctypes.byref(s), None, 16, 16, 16, 16, None) == 1     # Q
    assert lib.hga_decode_route(ctypes.byref(s), 16, None, 16, 16, 16, None) == 1     # summaries
    assert lib.hga_decode_route(ctypes.byref(s), 16, 16, 16, 16, None, None) == 1     # group_idx
    assert lib.hga_decode_route(ctypes.byref(_ok_shape()), 16, 16, 16, 16, 16, None) == 2
    # a first-chunk token has no candidates: nothing to route with budgets 0
    first = _dec_shape(kv_len=10, kv_capacity=64, top_k=0, top_g=0)
    assert lib.hga_decode_route(ctypes.byref(first), 16, None, None, None, None, None) == 0
    assert lib.hga_decode_attend(ctypes.byref(s), 16, 16, 16, None, 16, 16, None) == 1  # group_idx
    assert lib.hga_decode_attend(ctypes.byref(s), 16, None, 16, 16, 16, 16, None) == 1  # K
    assert lib.hga_decode_attend(ctypes.byref(s), 16, 16, 16, 16, None, 16, None) == 1  # O
    assert lib.hga_decode_attend(ctypes.byref(_ok_shape()), 16, 16, 16, 16, 16, 16, None) == 2


def test_zero_budget_routing_launches_nothing(lib):
    """top_k == top_g == 0: both index arrays have no entries, so the routing
    calls return before any launch.  In particular hga_route_causal with
    kv_len > q_len and Q_prev NULL does not read Q_prev (the pointers below
    are not device memory: a launch would have to touch them).  Host only."""
    s = _ok_shape(top_k=0, top_g=0)
    fake = ctypes.c_void_p(16)
    lib.hga_route_causal.argtypes = [ctypes.c_void_p] * 8
    lib.hga_route.argtypes = [ctypes.c_void_p] * 7
    assert lib.hga_route_causal(ctypes.byref(s), fake, None, fake, None, fake, fake, None) == 0
    assert lib.hga_route(ctypes.byref(s), fake, fake, None, fake, fake, None) == 0
    # with a budget, the missing Q_prev is still an argument error
    s = _ok_shape(top_k=4, top_g=0)
    assert lib.hga_route_causal(ctypes.byref(s), fake, None, fake, None, fake, None, None) == 1


def test_stage_argument_errors(lib):
    """Both staging calls reject bad arguments before launching anything
    (bogus non-null pointers are never dereferenced on these paths)."""
    s = _ok_shape()
    SP = ctypes.POINTER(hga.HgaShape)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.hga_stage_min_groups.argtypes = [SP]
    lib.hga_stage_workspace.argtypes = [SP, i32, ctypes.POINTER(sz)]
    lib.hga_stage_routed.argtypes = [SP, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.hga_stage_routed_from.argtypes = [SP, vp, vp, vp, vp, vp, ctypes.POINTER(hga.HgaStagePrev),
                                          i32, i32, vp, vp, vp, vp, sz, vp]
    sg = lib.hga_stage_min_groups(ctypes.byref(s))
    assert sg == 8 * 1792 // 8 and sg % 8 == 0   # every history group (14336 tokens)
    cap = -(-(8 * sg + s.q_len) // 64) * 64
    n = sz(0)
    assert lib.hga_stage_workspace(ctypes.byref(s), sg, ctypes.byref(n)) == 0
    r256 = lambda x: -(-x // 256) * 256
    assert n.value == 2 * r256(8 * sg * 4) + r256(8 * 4)   # unions, sizes, copy sources
    assert lib.hga_stage_workspace(ctypes.byref(s), sg + 4, ctypes.byref(n)) == 2
    assert lib.hga_stage_workspace(ctypes.byref(s), -8, ctypes.byref(n)) == 2
    assert lib.hga_stage_workspace(ctypes.byref(s), 131072 // 8, ctypes.byref(n)) == 0   # the bound
    assert lib.hga_stage_workspace(ctypes.byref(s), 131072 // 8 + 8, ctypes.byref(n)) == 2
    assert lib.hga_stage_workspace(ctypes.byref(s), sg, None) == 1
    assert lib.hga_stage_workspace(ctypes.byref(s), sg, ctypes.byref(n)) == 0
    need = n.value
    ok = [16, 16, 16]
    stage = lambda *a: lib.hga_stage_routed(ctypes.byref(s), *a)
    assert stage(16, None, 16, sg, cap, 16, 16, 16, 16, need, None) == 1
    assert stage(16, 16, 16, sg + 4, cap, 16, 16, 16, 16, need, None) == 2
    assert stage(16, 16, 16, sg - 8, cap, 16, 16, 16, 16, need, None) == 2
    assert stage(16, 16, 16, sg, cap - 64, 16, 16, 16, 16, need, None) == 2
    assert stage(16, 16, 16, sg, cap, 16, 16, 16, 16, need - 1, None) == 4
    assert stage(16, 16, 16, 1 << 28, cap, 16, 16, 16, 16, need, None) == 2   # 8x would overflow

    def frm(kseg, vseg, prev, ws=need):
        return lib.hga_stage_routed_from(ctypes.byref(s), *ok, kseg, vseg,
                                         ctypes.byref(prev) if prev else None, sg, cap,
                                         16, 16, 16, 16, ws, None)
    pneed = r256(8 * 8 * 1536 * 4) + r256(8 * 4)   # its unions and sizes
    good = dict(K_stage=16, V_stage=16, workspace=16, workspace_bytes=pneed,
                stage_groups=8 * 1536, q0=12288, q_len=2048,
                stage_capacity=8 * 8 * 1536 + 2048)
    P = lambda **kw: hga.HgaStagePrev(**{**good, **kw})
    assert frm(16, None, None) == 1                        # K_seg without V_seg
    assert frm(16, 16, P(), need - 1) == 4                 # otherwise valid: workspace short
    assert frm(None, None, P(workspace=None)) == 1
    assert frm(None, None, P(V_stage=None)) == 1
    assert frm(None, None, P(stage_groups=12)) == 2        # not a multiple of 8
    assert frm(None, None, P(q0=12288 + 64)) == 2          # its segment runs into this one
    assert frm(None, None, P(q0=100)) == 2                 # not chunk aligned
    assert frm(None, None, P(q_len=0)) == 2
    assert frm(None, None, P(stage_capacity=8 * 8 * 1536 + 2048 - 64)) == 2
    assert frm(None, None, P(workspace_bytes=pneed - 1)) == 4   # its unions would be overread
    assert frm(None, None, P(stage_groups=1 << 28)) == 2        # 8x would overflow


def test_summaries_rows_argument_errors(lib):
    """The row-range summaries call rejects ranges that the buffer does not
    hold, before launching anything."""
    s = _ok_shape()
    SP = ctypes.POINTER(hga.HgaShape)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    lib.hga_build_summaries_rows.argtypes = [SP, vp, i32, i32, vp, vp, i32, i32, vp]
    f = lambda *a: lib.hga_build_summaries_rows(ctypes.byref(s), *a)
    assert f(None, 14336, 2048, 16, 16, 224, 256, None) == 1
    assert f(16, 14336, 2048, None, 16, 224, 256, None) == 1
    assert f(16, 14300, 2048, 16, 16, 224, 256, None) == 2      # row0 not chunk aligned
    assert f(16, 14336, 2000, 16, 16, 224, 256, None) == 2      # rows not a multiple of 64
    assert f(16, 14336, 4096, 16, 16, 224, 256, None) == 2      # past kv_len
    assert f(16, 14336, 2048, 16, 16, 223, 256, None) == 2      # chunk before the buffer
    assert f(16, 14336, 2048, 16, 16, 224, 257, None) == 2      # chunk past the buffer
    assert f(16, 14336, 2048, 16, 16, 230, 229, None) == 2
    assert f(16, 14336, 2048, 16, 16, 230, 230, None) == 0      # empty range: nothing launched
