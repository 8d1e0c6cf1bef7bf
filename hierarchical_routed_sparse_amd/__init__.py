"""MI355X (gfx950) Hierarchical Global Attention: Python binding of libhga.so.

The functions below carry the names of the C ABI in ``include/hga.h`` and do
argument marshalling only (shape struct, device pointers, current HIP stream);
every step of the method runs in the library's HIP kernels.  Torch is used for
device memory and streams.  If ``libhga.so`` has not been built, the first call
raises ``HGAError``: there is no fallback implementation.

Tensors (block shapes): Q, O, dO, dQ [B,Hq,q_len,D]; K, V, dK, dV [B,Hkv,C,D] of the
shape's dtype (torch.bfloat16 or torch.float32), C = kv_capacity (kv_len when
0); chunk_mean [B,Hkv,C/64,D] and group_mean [B,Hkv,C/8,D] float32; chunk_idx
[B,Hq,q_len/64,top_k] and group_idx [B,Hq,q_len/64,top_g] int32; lse
[B,Hq,q_len] float32.  All contiguous, on the current GPU, except that K and
V may also be pinned host tensors (``pin_memory=True``): HIP maps pinned host
memory into the GPU's address space, and the kernels then fetch the rows they
gather (the kept groups) across the host link.  A decode shape (q_len == 1,
``hga_decode``) takes Q and O [B,Hq,D], chunk_idx [B,Hq,top_k], group_idx
[B,Hq,top_g] and lse [B,Hq].
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "HGAError", "HgaShape", "make_shape", "lib_path", "hga_abi_version", "hga_validate_shape",
    "hga_build_summaries", "hga_build_summaries_rows", "hga_route", "hga_route_causal", "hga_attend_fwd", "hga_attend_bwd_workspace",
    "hga_attend_bwd", "hga_attend_bwd_noalloc", "hga_attend_bwd_prep", "hga_attend_bwd_dq", "hga_attend_bwd_dkdv", "hga_attend_bwd_dkdv_range",
    "hga_validate_decode_shape", "hga_decode", "hga_decode_route", "hga_decode_attend",
    "hga_decode_route_causal", "hga_stage_min_groups", "hga_stage_workspace", "hga_stage_routed",
    "HgaStagePrev", "hga_stage_routed_from", "forward", "backward", "decode",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhga.so")

HGA_DTYPE_BF16, HGA_DTYPE_FP32 = 0, 1
CHUNK, GROUP, QBLOCK = 64, 8, 64


class HGAError(RuntimeError):
    pass


class HgaShape(ctypes.Structure):
    """Mirror of ``hga_shape`` in include/hga.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("top_g", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
    ]

    def __repr__(self):
        f = ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_)
        return f"HgaShape({f})"


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, q_len, kv_len, top_k, top_g,
               dtype="bf16", softmax_scale=0.0, kv_capacity=0) -> HgaShape:
    dt = {"bf16": HGA_DTYPE_BF16, "fp32": HGA_DTYPE_FP32}.get(dtype, dtype)
    return HgaShape(batch, n_q_heads, n_kv_heads, head_dim, q_len, kv_len, top_k, top_g,
                    float(softmax_scale), int(dt), int(kv_capacity))


_libs = {}
_vp = ctypes.c_void_p
_SP = ctypes.POINTER(HgaShape)


class HgaStagePrev(ctypes.Structure):
    """hga_stage_prev of include/hga.h: the previous staging of the same history."""
    _fields_ = [("K_stage", ctypes.c_void_p), ("V_stage", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stage_groups", ctypes.c_int32),
                ("stage_capacity", ctypes.c_int32), ("q0", ctypes.c_int32),
                ("q_len", ctypes.c_int32)]


def lib_path() -> str:
    return LIB_PATH


def _load(path: str = None):
    path = path or LIB_PATH
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        raise HGAError(f"{path} is not built; run python -m hierarchical_routed_sparse_amd.build_lib")
    lib = ctypes.CDLL(path)
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    lib.hga_abi_version.restype = ctypes.c_int
    lib.hga_status_str.restype = ctypes.c_char_p
    lib.hga_status_str.argtypes = [ctypes.c_int]
    lib.hga_validate_shape.argtypes = [_SP]
    lib.hga_build_summaries.argtypes = [_SP, _vp, _vp, _vp, i32, i32, _vp]
    lib.hga_route.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.hga_route_causal.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.hga_attend_fwd.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.hga_attend_bwd_workspace.argtypes = [_SP, ctypes.POINTER(sz)]
    lib.hga_attend_bwd.argtypes = [_SP] + [_vp] * 11 + [sz, _vp]
    lib.hga_attend_bwd_noalloc.argtypes = [_SP] + [_vp] * 11
    lib.hga_attend_bwd_prep.argtypes = [_SP] + [_vp] * 4 + [sz, _vp]
    lib.hga_attend_bwd_dq.argtypes = [_SP] + [_vp] * 9 + [sz, _vp]
    lib.hga_attend_bwd_dkdv.argtypes = [_SP] + [_vp] * 9 + [sz, _vp]
    lib.hga_attend_bwd_dkdv_range.argtypes = [_SP] + [_vp] * 6 + [i32, i32] + [_vp] * 3 + [sz, _vp]
    lib.hga_validate_decode_shape.argtypes = [_SP]
    lib.hga_decode.argtypes = [_SP] + [_vp] * 10
    lib.hga_decode_route.argtypes = [_SP] + [_vp] * 6
    lib.hga_decode_attend.argtypes = [_SP] + [_vp] * 7
    lib.hga_decode_route_causal.argtypes = [_SP] + [_vp] * 6
    lib.hga_build_summaries_rows.argtypes = [_SP, _vp, i32, i32, _vp, _vp, i32, i32, _vp]
    lib.hga_stage_min_groups.argtypes = [_SP]
    lib.hga_stage_min_groups.restype = ctypes.c_int32
    lib.hga_stage_workspace.argtypes = [_SP, i32, ctypes.POINTER(sz)]
    lib.hga_stage_routed.argtypes = [_SP, _vp, _vp, _vp, i32, i32, _vp, _vp, _vp, _vp, sz, _vp]
    lib.hga_stage_routed_from.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.POINTER(HgaStagePrev), i32, i32, _vp, _vp, _vp,
                                          _vp, sz, _vp]
    for name in ("hga_validate_shape", "hga_validate_decode_shape", "hga_decode", "hga_route_causal",
                 "hga_decode_route", "hga_decode_attend", "hga_decode_route_causal", "hga_build_summaries", "hga_route", "hga_attend_fwd",
                 "hga_attend_bwd_workspace", "hga_attend_bwd", "hga_attend_bwd_noalloc",
                 "hga_attend_bwd_prep",
                 "hga_attend_bwd_dq",
                 "hga_attend_bwd_dkdv", "hga_attend_bwd_dkdv_range", "hga_stage_workspace",
                 "hga_stage_routed", "hga_stage_routed_from", "hga_build_summaries_rows"):
        getattr(lib, name).restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise HGAError(f"{what}: {_load().hga_status_str(rc).decode()} (status {rc})")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _elt_dtype(shape: HgaShape):
    import torch
    return torch.bfloat16 if shape.dtype == HGA_DTYPE_BF16 else torch.float32


_hip = None


def _hip_runtime():
    """The HIP runtime torch has loaded (shared by soname with libhga.so)."""
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (loads the runtime)
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
    return _hip


def _host_device_address(t, name):
    """GPU address of a pinned host tensor; raises unless HIP maps it."""
    if not t.is_pinned():
        raise HGAError(f"{name} is a host tensor but not pinned (allocate it with pin_memory=True)")
    dp = ctypes.c_void_p()
    rc = _hip_runtime().hipHostGetDevicePointer(ctypes.byref(dp), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0 or not dp.value:
        raise HGAError(f"{name}: HIP does not map this pinned host memory (hipError {rc})")
    return dp.value


def _ptr(t, name, dtype=None, size=None, nullable=False, host_ok=False):
    """Device pointer of a contiguous tensor after checking dtype and shape.
    With host_ok, a pinned host tensor is accepted and its GPU address used."""
    if t is None:
        if nullable:
            return None
        raise HGAError(f"{name} is required")
    if isinstance(t, int):
        return t
    if not t.is_cuda and not host_ok:
        raise HGAError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise HGAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise HGAError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if size is not None and tuple(t.shape) != tuple(size):
        raise HGAError(f"{name} has shape {tuple(t.shape)}, expected {tuple(size)}")
    if not t.is_cuda:
        return _host_device_address(t, name)
    return t.data_ptr()


def capacity(s: HgaShape) -> int:
    """Key/value rows allocated per (b, kv head)."""
    return s.kv_capacity if s.kv_capacity > 0 else s.kv_len


def _sizes(s: HgaShape):
    cap = capacity(s)
    if s.q_len == 1:   # decode shape
        return dict(
            q=(s.batch, s.n_q_heads, s.head_dim),
            kv=(s.batch, s.n_kv_heads, cap, s.head_dim),
            cm=(s.batch, s.n_kv_heads, cap // CHUNK, s.head_dim),
            gm=(s.batch, s.n_kv_heads, cap // GROUP, s.head_dim),
            ci=(s.batch, s.n_q_heads, s.top_k),
            gi=(s.batch, s.n_q_heads, s.top_g),
            lse=(s.batch, s.n_q_heads),
        )
    nblk = s.q_len // QBLOCK
    return dict(
        q=(s.batch, s.n_q_heads, s.q_len, s.head_dim),
        kv=(s.batch, s.n_kv_heads, cap, s.head_dim),
        cm=(s.batch, s.n_kv_heads, cap // CHUNK, s.head_dim),
        gm=(s.batch, s.n_kv_heads, cap // GROUP, s.head_dim),
        ci=(s.batch, s.n_q_heads, nblk, s.top_k),
        gi=(s.batch, s.n_q_heads, nblk, s.top_g),
        lse=(s.batch, s.n_q_heads, s.q_len),
        qprev=(s.batch, s.n_q_heads, QBLOCK, s.head_dim),
    )


# ------------------------------------------------------------------ C ABI names

def hga_abi_version() -> int:
    return _load().hga_abi_version()


def hga_validate_shape(shape: HgaShape) -> int:
    """Returns the status code (0 = valid); host only."""
    return _load().hga_validate_shape(ctypes.byref(shape))


def hga_validate_decode_shape(shape: HgaShape) -> int:
    """Returns the status code (0 = valid) of a decode shape; host only."""
    return _load().hga_validate_decode_shape(ctypes.byref(shape))


def hga_build_summaries(shape, K, chunk_mean, group_mean, chunk_begin=0, chunk_end=None,
                        stream=None):
    import torch
    sz = _sizes(shape)
    if chunk_end is None:
        chunk_end = shape.kv_len // CHUNK
    _check(_load().hga_build_summaries(
        ctypes.byref(shape), _ptr(K, "K", _elt_dtype(shape), sz["kv"], host_ok=True),
        _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"]),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"]),
        int(chunk_begin), int(chunk_end), _stream(stream)), "hga_build_summaries")


def hga_route(shape, Q, chunk_mean, group_mean, chunk_idx, group_idx, stream=None):
    import torch
    sz = _sizes(shape)
    _check(_load().hga_route(
        ctypes.byref(shape), _ptr(Q, "Q", _elt_dtype(shape), sz["q"]),
        _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"]),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"], nullable=True),
        _ptr(chunk_idx, "chunk_idx", torch.int32, sz["ci"], nullable=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _stream(stream)), "hga_route")


def hga_route_causal(shape, Q, Q_prev, chunk_mean, group_mean, chunk_idx, group_idx,
                     stream=None):
    """Strictly causal routing: block j routed with the mean of the 64 queries
    before it; Q_prev [B,Hq,64,D] holds the 64 queries before the segment
    (None when kv_len == q_len)."""
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    _check(_load().hga_route_causal(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]),
        _ptr(Q_prev, "Q_prev", dt, sz["qprev"], nullable=True),
        _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"]),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"], nullable=True),
        _ptr(chunk_idx, "chunk_idx", torch.int32, sz["ci"], nullable=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _stream(stream)), "hga_route_causal")


def hga_attend_fwd(shape, Q, K, V, group_idx, O, lse=None, stream=None):
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    _check(_load().hga_attend_fwd(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(O, "O", dt, sz["q"]), _ptr(lse, "lse", torch.float32, sz["lse"], nullable=True),
        _stream(stream)), "hga_attend_fwd")


def hga_attend_bwd_workspace(shape) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().hga_attend_bwd_workspace(ctypes.byref(shape), ctypes.byref(n)),
           "hga_attend_bwd_workspace")
    return int(n.value)


def _ws(workspace):
    if isinstance(workspace, int):
        raise HGAError("pass the workspace as a tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def hga_attend_bwd(shape, Q, K, V, O, lse, dO, group_idx, dQ, dK, dV, workspace, stream=None):
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    wp, wb = _ws(workspace)
    _check(_load().hga_attend_bwd(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True), _ptr(O, "O", dt, sz["q"]),
        _ptr(lse, "lse", torch.float32, sz["lse"]), _ptr(dO, "dO", dt, sz["q"]),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(dQ, "dQ", dt, sz["q"]), _ptr(dK, "dK", dt, sz["kv"]), _ptr(dV, "dV", dt, sz["kv"]),
        wp, wb, _stream(stream)), "hga_attend_bwd")


def hga_attend_bwd_noalloc(shape, Q, K, V, O, lse, dO, group_idx, dQ, dK, dV, stream=None):
    """hga_attend_bwd with the workspace held by the library (for callers that
    cannot allocate); calls that overlap on one GPU race on it."""
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    _check(_load().hga_attend_bwd_noalloc(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True), _ptr(O, "O", dt, sz["q"]),
        _ptr(lse, "lse", torch.float32, sz["lse"]), _ptr(dO, "dO", dt, sz["q"]),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(dQ, "dQ", dt, sz["q"]), _ptr(dK, "dK", dt, sz["kv"]), _ptr(dV, "dV", dt, sz["kv"]),
        _stream(stream)), "hga_attend_bwd_noalloc")


def hga_attend_bwd_prep(shape, O, dO, group_idx, workspace, stream=None):
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    wp, wb = _ws(workspace)
    _check(_load().hga_attend_bwd_prep(
        ctypes.byref(shape), _ptr(O, "O", dt, sz["q"]), _ptr(dO, "dO", dt, sz["q"]),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True), wp, wb,
        _stream(stream)), "hga_attend_bwd_prep")


def hga_attend_bwd_dq(shape, Q, K, V, O, lse, dO, group_idx, dQ, workspace, stream=None):
    """``workspace`` None: dQ only (no workspace written)."""
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    wp, wb = _ws(workspace) if workspace is not None else (None, 0)
    _check(_load().hga_attend_bwd_dq(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True), _ptr(O, "O", dt, sz["q"]),
        _ptr(lse, "lse", torch.float32, sz["lse"]), _ptr(dO, "dO", dt, sz["q"]),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(dQ, "dQ", dt, sz["q"]), wp, wb, _stream(stream)), "hga_attend_bwd_dq")


def hga_attend_bwd_dkdv(shape, Q, K, V, lse, dO, group_idx, dK, dV, workspace, stream=None):
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    wp, wb = _ws(workspace)
    _check(_load().hga_attend_bwd_dkdv(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True), _ptr(lse, "lse", torch.float32, sz["lse"]),
        _ptr(dO, "dO", dt, sz["q"]),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(dK, "dK", dt, sz["kv"]), _ptr(dV, "dV", dt, sz["kv"]), wp, wb, _stream(stream)),
        "hga_attend_bwd_dkdv")


def hga_attend_bwd_dkdv_range(shape, Q, K, V, lse, dO, group_idx, chunk_begin, chunk_end, dK, dV,
                              workspace, stream=None):
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    wp, wb = _ws(workspace)
    _check(_load().hga_attend_bwd_dkdv_range(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True), _ptr(lse, "lse", torch.float32, sz["lse"]),
        _ptr(dO, "dO", dt, sz["q"]),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        int(chunk_begin), int(chunk_end),
        _ptr(dK, "dK", dt, sz["kv"]), _ptr(dV, "dV", dt, sz["kv"]), wp, wb, _stream(stream)),
        "hga_attend_bwd_dkdv_range")


def hga_decode(shape, Q, K, V, chunk_mean, group_mean, chunk_idx, group_idx, O, lse=None,
               stream=None):
    import torch
    sz, dt = _decode_sizes(shape)
    _check(_load().hga_decode(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True),
        _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"], nullable=True),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"], nullable=True),
        _ptr(chunk_idx, "chunk_idx", torch.int32, sz["ci"], nullable=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(O, "O", dt, sz["q"]), _ptr(lse, "lse", torch.float32, sz["lse"], nullable=True),
        _stream(stream)), "hga_decode")


def _decode_sizes(shape):
    if shape.q_len != 1:
        raise HGAError("decode calls take a decode shape (q_len == 1)")
    return _sizes(shape), _elt_dtype(shape)


def hga_decode_route(shape, Q, chunk_mean, group_mean, chunk_idx, group_idx, stream=None):
    import torch
    sz, dt = _decode_sizes(shape)
    _check(_load().hga_decode_route(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]),
        _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"], nullable=True),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"], nullable=True),
        _ptr(chunk_idx, "chunk_idx", torch.int32, sz["ci"], nullable=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _stream(stream)), "hga_decode_route")


def hga_decode_route_causal(shape, Q_prev, chunk_mean, group_mean, chunk_idx, group_idx,
                            stream=None):
    """Decode routing under strictly causal routing: once per block, from the
    previous block's 64 queries Q_prev [B,Hq,64,D] (None in the first block)."""
    import torch
    sz, dt = _decode_sizes(shape)
    _check(_load().hga_decode_route_causal(
        ctypes.byref(shape),
        _ptr(Q_prev, "Q_prev", dt, (shape.batch, shape.n_q_heads, QBLOCK, shape.head_dim),
             nullable=True),
        _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"], nullable=True),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"], nullable=True),
        _ptr(chunk_idx, "chunk_idx", torch.int32, sz["ci"], nullable=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _stream(stream)), "hga_decode_route_causal")


def hga_decode_attend(shape, Q, K, V, group_idx, O, lse=None, stream=None):
    import torch
    sz, dt = _decode_sizes(shape)
    _check(_load().hga_decode_attend(
        ctypes.byref(shape), _ptr(Q, "Q", dt, sz["q"]), _ptr(K, "K", dt, sz["kv"], host_ok=True),
        _ptr(V, "V", dt, sz["kv"], host_ok=True),
        _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(O, "O", dt, sz["q"]), _ptr(lse, "lse", torch.float32, sz["lse"], nullable=True),
        _stream(stream)), "hga_decode_attend")


def hga_build_summaries_rows(shape, K_rows, row0, chunk_mean, group_mean, chunk_begin,
                             chunk_end, stream=None):
    """Summaries of chunks [chunk_begin, chunk_end) from K_rows [B, Hkv, rows, D]
    holding positions row0 .. row0 + rows - 1 (see include/hga.h)."""
    import torch
    sz = _sizes(shape)
    rows = K_rows.shape[2]
    _check(_load().hga_build_summaries_rows(
        ctypes.byref(shape),
        _ptr(K_rows, "K_rows", _elt_dtype(shape), (shape.batch, shape.n_kv_heads, rows,
                                                   shape.head_dim), host_ok=True),
        int(row0), int(rows), _ptr(chunk_mean, "chunk_mean", torch.float32, sz["cm"]),
        _ptr(group_mean, "group_mean", torch.float32, sz["gm"]), int(chunk_begin),
        int(chunk_end), _stream(stream)), "hga_build_summaries_rows")


def hga_stage_min_groups(shape) -> int:
    return int(_load().hga_stage_min_groups(ctypes.byref(shape)))


def hga_stage_workspace(shape, stage_groups) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().hga_stage_workspace(ctypes.byref(shape), int(stage_groups), ctypes.byref(n)),
           "hga_stage_workspace")
    return int(n.value)


def hga_stage_routed(shape, group_idx, K, V, stage_groups, K_stage, V_stage, group_idx_staged,
                     workspace, stream=None):
    """Stages the routed working set (see include/hga.h); K_stage and V_stage
    [B, Hkv, stage_capacity, D] device tensors."""
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    cap = K_stage.shape[2]
    st = (shape.batch, shape.n_kv_heads, cap, shape.head_dim)
    wp, wb = _ws(workspace)
    _check(_load().hga_stage_routed(
        ctypes.byref(shape), _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(K, "K", dt, sz["kv"], host_ok=True), _ptr(V, "V", dt, sz["kv"], host_ok=True),
        int(stage_groups), int(cap), _ptr(K_stage, "K_stage", dt, st),
        _ptr(V_stage, "V_stage", dt, st),
        _ptr(group_idx_staged, "group_idx_staged", torch.int32, sz["gi"], nullable=True),
        wp, wb, _stream(stream)), "hga_stage_routed")


def hga_stage_routed_from(shape, group_idx, K, V, stage_groups, K_stage, V_stage,
                          group_idx_staged, workspace, K_seg=None, V_seg=None, prev=None,
                          stream=None):
    """hga_stage_routed with the previous staging and the segment's rows in
    device memory as copy sources (see include/hga.h).  ``prev`` is None or a
    dict with the previous call's K_stage, V_stage, workspace (tensors),
    stage_groups, q0 and q_len; K_seg and V_seg [B, Hkv, q_len, D] device
    tensors or None."""
    import torch
    sz, dt = _sizes(shape), _elt_dtype(shape)
    cap = K_stage.shape[2]
    st = (shape.batch, shape.n_kv_heads, cap, shape.head_dim)
    seg = (shape.batch, shape.n_kv_heads, shape.q_len, shape.head_dim)
    wp, wb = _ws(workspace)
    pp = None
    if prev is not None:
        pcap = prev["K_stage"].shape[2]
        pst = (shape.batch, shape.n_kv_heads, pcap, shape.head_dim)
        pw, pwb = _ws(prev["workspace"])
        pp = ctypes.byref(HgaStagePrev(
            _ptr(prev["K_stage"], "prev K_stage", dt, pst), _ptr(prev["V_stage"], "prev V_stage", dt, pst),
            pw, pwb, int(prev["stage_groups"]), int(pcap), int(prev["q0"]), int(prev["q_len"])))
    _check(_load().hga_stage_routed_from(
        ctypes.byref(shape), _ptr(group_idx, "group_idx", torch.int32, sz["gi"], nullable=True),
        _ptr(K, "K", dt, sz["kv"], host_ok=True), _ptr(V, "V", dt, sz["kv"], host_ok=True),
        _ptr(K_seg, "K_seg", dt, seg, nullable=True), _ptr(V_seg, "V_seg", dt, seg, nullable=True),
        pp, int(stage_groups), int(cap), _ptr(K_stage, "K_stage", dt, st),
        _ptr(V_stage, "V_stage", dt, st),
        _ptr(group_idx_staged, "group_idx_staged", torch.int32, sz["gi"], nullable=True),
        wp, wb, _stream(stream)), "hga_stage_routed_from")


# ------------------------------------------------------------------ compositions

def forward(shape, Q, K, V, stream=None, causal=False, Q_prev=None):
    """Summaries, routing and attention with freshly allocated outputs (with
    ``causal``: strictly causal routing, ``Q_prev`` the 64 queries before the
    segment).  Returns dict(chunk_mean, group_mean, chunk_idx, group_idx, O, lse)."""
    import torch
    sz = _sizes(shape)
    dev = Q.device
    out = dict(
        chunk_mean=torch.empty(sz["cm"], dtype=torch.float32, device=dev),
        group_mean=torch.empty(sz["gm"], dtype=torch.float32, device=dev),
        chunk_idx=torch.empty(sz["ci"], dtype=torch.int32, device=dev),
        group_idx=torch.empty(sz["gi"], dtype=torch.int32, device=dev),
        O=torch.empty(sz["q"], dtype=_elt_dtype(shape), device=dev),
        lse=torch.empty(sz["lse"], dtype=torch.float32, device=dev),
    )
    hga_build_summaries(shape, K, out["chunk_mean"], out["group_mean"], stream=stream)
    if causal:
        hga_route_causal(shape, Q, Q_prev, out["chunk_mean"], out["group_mean"],
                         out["chunk_idx"], out["group_idx"], stream=stream)
    else:
        hga_route(shape, Q, out["chunk_mean"], out["group_mean"], out["chunk_idx"],
                  out["group_idx"], stream=stream)
    hga_attend_fwd(shape, Q, K, V, out["group_idx"], out["O"], out["lse"], stream=stream)
    return out


def backward(shape, Q, K, V, O, lse, dO, group_idx, stream=None):
    """dQ, dK, dV with freshly allocated outputs and workspace."""
    import torch
    sz = _sizes(shape)
    dev = Q.device
    dQ = torch.empty(sz["q"], dtype=_elt_dtype(shape), device=dev)
    dK = torch.empty(sz["kv"], dtype=_elt_dtype(shape), device=dev)
    dV = torch.empty(sz["kv"], dtype=_elt_dtype(shape), device=dev)
    ws = torch.empty(hga_attend_bwd_workspace(shape), dtype=torch.uint8, device=dev)
    hga_attend_bwd(shape, Q, K, V, O, lse, dO, group_idx, dQ, dK, dV, ws, stream=stream)
    return dQ, dK, dV


def decode(shape, Q, K, V, chunk_mean, group_mean, stream=None):
    """One decode step with freshly allocated outputs (the summaries of every
    complete chunk before the token's own chunk already built).
    Returns dict(chunk_idx, group_idx, O, lse)."""
    import torch
    sz = _sizes(shape)
    dev = Q.device
    out = dict(
        chunk_idx=torch.empty(sz["ci"], dtype=torch.int32, device=dev),
        group_idx=torch.empty(sz["gi"], dtype=torch.int32, device=dev),
        O=torch.empty(sz["q"], dtype=_elt_dtype(shape), device=dev),
        lse=torch.empty(sz["lse"], dtype=torch.float32, device=dev),
    )
    hga_decode(shape, Q, K, V, chunk_mean, group_mean, out["chunk_idx"], out["group_idx"],
               out["O"], out["lse"], stream=stream)
    return out
