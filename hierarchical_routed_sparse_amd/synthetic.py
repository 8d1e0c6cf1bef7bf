"""Seeded synthetic inputs for the HGA workloads.

This module holds only random-number generation and tensor construction; none
of the attention method's arithmetic lives here, so both the HIP path and the
CPU oracle can be fed from it.

Generator (counter based, so any slice can be drawn independently):
  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): the i-th output (i = 1, 2, ...) of a stream with
    state s is mix(s + i * 0x9E3779B97F4A7C15).
  * each tensor draws from its own stream, keyed by (seed, tag) with
    s = mix(seed * 256 + tag + 0x9E3779B97F4A7C15);
  * uniforms are the top 53 bits of an output times 2**-53, in [0, 1);
  * normals come in Box-Muller pairs from consecutive uniforms (u1, u2):
    r = sqrt(-2 ln(1 - u1)), n0 = r cos(2 pi u2), n1 = r sin(2 pi u2),
    in row-major order of the tensor.

Workload recipe (shapes like a Qwen3-8B attention layer: 32 query heads, 8 KV
heads, head_dim 128):
  * keys are clustered per 64-token chunk: K[b,h,s] = centroid[b,h,s//64] +
    0.5 * noise, centroid and noise ~ N(0, I);
  * Q and V ~ N(0, 1), scaled by 1/sqrt(head_dim) for the bf16 workloads;
  * dO ~ N(0, 1);
  * optionally a fraction of chunks (5 % in the long-history stress case) are
    copies of an earlier chunk's 64 key rows: half exact copies, half with one
    element moved by one unit in the last place, to create exact and near ties;
  * values are drawn in float64 and rounded to float32 (round to nearest even),
    then, for bf16 workloads, to bfloat16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TAG_Q, TAG_K, TAG_V, TAG_DO, TAG_CENTROID, TAG_DUP, TAG_QPREV = 1, 2, 3, 4, 5, 6, 7

_BLOCK = 1 << 22  # draws per generation block (bounds temporary memory)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(state: int, first: int, count: int) -> np.ndarray:
    """Outputs number first+1 .. first+count of the SplitMix64 stream with the given state."""
    with np.errstate(over="ignore"):
        i = np.arange(first + 1, first + count + 1, dtype=np.uint64)
        return _mix(np.uint64(state & 0xFFFFFFFFFFFFFFFF) + i * GAMMA)


def stream_state(seed: int, tag: int) -> int:
    with np.errstate(over="ignore"):
        z = np.array([(seed * 256 + tag) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64) + GAMMA
        return int(_mix(z)[0])


def uniforms(state: int, first: int, count: int) -> np.ndarray:
    z = splitmix64(state, first, count)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def _normals_block(state: int, out: np.ndarray, pos: int, n: int) -> None:
    u = uniforms(state, pos, n)
    r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
    th = (2.0 * math.pi) * u[1::2]
    out[pos:pos + n:2] = r * np.cos(th)
    out[pos + 1:pos + n:2] = r * np.sin(th)


def normals(state: int, count: int) -> np.ndarray:
    """count standard normals (count rounded up to even internally).  Blocks of
    the stream are independent (counter based), so large draws are split over
    threads (numpy releases the GIL inside each block's array operations); the
    values do not depend on the thread count."""
    out = np.empty(count + (count & 1), dtype=np.float64)
    starts = list(range(0, out.size, _BLOCK))
    work = [(p, min(_BLOCK, out.size - p)) for p in starts]
    if len(work) <= 2:
        for p, n in work:
            _normals_block(state, out, p, n)
    else:
        import concurrent.futures as cf
        threads = max(1, min(16, os.cpu_count() or 1, len(work)))
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda pn: _normals_block(state, out, *pn), work))
    return out[:count]


def _bf16_block(src: np.ndarray, dst: np.ndarray) -> None:
    b = src.view(np.uint32).astype(np.uint64)
    b = b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    dst[...] = (b >> np.uint64(16)).astype(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even
    (elementwise; large arrays are converted in blocks over threads)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    flat = x32.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    spans = [(p, min(p + _BLOCK, flat.size)) for p in range(0, flat.size, _BLOCK)]
    if len(spans) <= 2:
        for a, b in spans:
            _bf16_block(flat[a:b], out[a:b])
    else:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(lambda ab: _bf16_block(flat[ab[0]:ab[1]], out[ab[0]:ab[1]]), spans))
    return out.reshape(x32.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One HGA problem: shapes, routing budget, input recipe."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q_len: int
    kv_len: int
    top_k: int
    top_g: int
    dtype: str            # "bf16" or "fp32"
    seed: int
    qv_scale: float       # Q and V are N(0,1) * qv_scale
    dup_fraction: float = 0.0
    backward: bool = False
    description: str = ""

    @property
    def n_blocks(self) -> int:
        return self.q_len // 64


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_1k", 1, 1, 1, 64, 1024, 1024, 4, 8, "fp32", 0, 1.0,
                 description="fp32 causal self-attention, 1 head, D64, 1K tokens, k4 g8"),
        Workload("qwen3_8b_2k", 1, 32, 8, 128, 2048, 2048, 8, 32, "bf16", 1, 1 / math.sqrt(128),
                 description="bf16 causal self-attention, 32q/8kv, D128, 2K tokens, k8 g32"),
        Workload("segment_2k_over_16k", 1, 32, 8, 128, 2048, 16384, 16, 64, "bf16", 2,
                 1 / math.sqrt(128), backward=True,
                 description="bf16 2048-query segment at the end of a 16384-token history, "
                             "32q/8kv, D128, k16 g64, forward + backward"),
        Workload("segment_2k_over_64k_ties", 1, 32, 8, 128, 2048, 65536, 32, 128, "bf16", 3,
                 1 / math.sqrt(128), dup_fraction=0.05,
                 description="bf16 2048-query segment over 65536-token history with 5% "
                             "duplicated chunks, 32q/8kv, D128, k32 g128"),
        Workload("fwd_bwd_b2_4k", 2, 32, 8, 128, 4096, 4096, 8, 32, "bf16", 4,
                 1 / math.sqrt(128), backward=True,
                 description="bf16 causal self-attention, batch 2, 32q/8kv, D128, 4K tokens, "
                             "k8 g32, forward + backward"),
        Workload("causal_16k", 1, 32, 8, 128, 16384, 16384, 16, 64, "bf16", 6,
                 1 / math.sqrt(128), backward=True,
                 description="bf16 causal self-attention over a whole 16384-token sequence, "
                             "32q/8kv, D128, k16 g64, forward + backward"),
        Workload("decode_b16_16k", 16, 32, 8, 128, 1, 16424, 16, 64, "bf16", 5,
                 1 / math.sqrt(128),
                 description="bf16 decode: one new token per sequence at position 16423 of "
                             "a 16424-token cache (40 tokens into its own chunk), batch 16, "
                             "32q/8kv, D128, k16 g64"),
    ]
}


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x.astype(np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _duplicate_chunks(Kr: np.ndarray, seed: int, fraction: float, dtype: str) -> None:
    """In place: copy the 64 key rows of an earlier chunk onto a seeded set of chunks."""
    B, H, S, D = Kr.shape
    nchunks = S // 64
    ndup = int(fraction * nchunks)
    if ndup <= 0 or nchunks < 2:
        return
    state = stream_state(seed, TAG_DUP)
    pos = 0
    for b in range(B):
        for h in range(H):
            # partial Fisher-Yates over chunks 1..nchunks-1
            pool = list(range(1, nchunks))
            u = uniforms(state, pos, ndup)
            pos += ndup
            for i in range(ndup):
                j = i + int(u[i] * (len(pool) - i))
                pool[i], pool[j] = pool[j], pool[i]
            chosen = sorted(pool[:ndup])
            u_src = uniforms(state, pos, ndup)
            pos += ndup
            u_elt = uniforms(state, pos, ndup)
            pos += ndup
            for n, c in enumerate(chosen):
                src = int(u_src[n] * c)
                Kr[b, h, c * 64:(c + 1) * 64] = Kr[b, h, src * 64:(src + 1) * 64]
                if n % 2 == 1:  # near tie: one element moved by one unit in the last place
                    e = int(u_elt[n] * 64 * D)
                    row, col = c * 64 + e // D, e % D
                    if dtype == "bf16":
                        Kr[b, h, row, col] = np.uint16(int(Kr[b, h, row, col]) ^ 1)
                    else:
                        Kr[b, h, row, col] = np.nextafter(Kr[b, h, row, col], np.float32(np.inf))


def make_inputs(w: Workload, with_grad_output: bool | None = None,
                with_qprev: bool = False) -> dict:
    """Rounded inputs for a workload as numpy arrays.

    bf16 tensors are returned as uint16 bit patterns, fp32 tensors as float32.
    Keys: Q [B,Hq,Sq,D], K and V [B,Hkv,Skv,D], dO [B,Hq,Sq,D] when a backward
    is wanted, and with ``with_qprev`` Qprev [B,Hq,64,D]: the 64 queries before
    the segment (strictly causal routing), drawn like Q from their own stream.
    """
    B, Hq, Hkv, D, Sq, Skv = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.q_len, w.kv_len
    out = {}
    nq = B * Hq * Sq * D
    out["Q"] = _round(normals(stream_state(w.seed, TAG_Q), nq) * w.qv_scale, w.dtype).reshape(
        B, Hq, Sq, D)
    nch = -(-Skv // 64)   # chunks, the last one possibly partial (a decode cache)
    cen = normals(stream_state(w.seed, TAG_CENTROID), B * Hkv * nch * D).reshape(
        B, Hkv, nch, 1, D)
    noise = normals(stream_state(w.seed, TAG_K), B * Hkv * Skv * D)
    if Skv % 64 == 0:
        K = (cen + 0.5 * noise.reshape(B, Hkv, nch, 64, D)).reshape(B, Hkv, Skv, D)
    else:
        K = np.repeat(cen[:, :, :, 0], 64, axis=2)[:, :, :Skv] + 0.5 * noise.reshape(
            B, Hkv, Skv, D)
    K = _round(K, w.dtype)
    del cen, noise
    if w.dup_fraction > 0:
        _duplicate_chunks(K, w.seed, w.dup_fraction, w.dtype)
    out["K"] = K
    out["V"] = _round(normals(stream_state(w.seed, TAG_V), B * Hkv * Skv * D) * w.qv_scale,
                      w.dtype).reshape(B, Hkv, Skv, D)
    if with_qprev:
        out["Qprev"] = _round(normals(stream_state(w.seed, TAG_QPREV), B * Hq * 64 * D) *
                              w.qv_scale, w.dtype).reshape(B, Hq, 64, D)
    if with_grad_output is None:
        with_grad_output = w.backward
    if with_grad_output:
        out["dO"] = _round(normals(stream_state(w.seed, TAG_DO), nq), w.dtype).reshape(
            B, Hq, Sq, D)
    return out


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of rounded inputs to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def to_torch(x: np.ndarray, dtype: str, device=None):
    """Rounded inputs as a torch tensor (bfloat16 or float32)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device) if device is not None else t


def scaled_workload(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)
