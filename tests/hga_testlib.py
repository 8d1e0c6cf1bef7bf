"""Shared test helpers: independent references and comparison rules.

Nothing here calls the HIP library.  The references below reduce HGA special
cases to library routines (torch's scaled_dot_product_attention in float64 on
the CPU) so that the oracle is pinned to something other than itself.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hga_mask(group_idx: np.ndarray, Sq: int, Skv: int, C: int = 64, G: int = 8) -> np.ndarray:
    """Boolean [B,Hq,Sq,Skv] mask of attended pairs: the tokens of each kept
    group for every query of the block, plus the block's own chunk causally."""
    B, Hq, nblk, top_g = group_idx.shape
    q0 = Skv - Sq
    m = np.zeros((B, Hq, Sq, Skv), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for blk in range(nblk):
                rows = slice(blk * C, (blk + 1) * C)
                for gam in group_idx[b, h, blk]:
                    if gam >= 0:
                        m[b, h, rows, gam * G:(gam + 1) * G] = True
                cb = q0 // C + blk
                for i in range(C):
                    p = q0 + blk * C + i
                    m[b, h, blk * C + i, cb * C:p + 1] = True
    return m


def causal_mask(Sq: int, Skv: int) -> np.ndarray:
    q0 = Skv - Sq
    return np.arange(Skv)[None, :] <= (q0 + np.arange(Sq))[:, None]


def sdpa_f64(Q, K, V, mask, scale=None, requires_grad=False):
    """torch scaled_dot_product_attention in float64 on the CPU with GQA expansion
    (query head h reads kv head h // (Hq / Hkv))."""
    Q = torch.as_tensor(np.asarray(Q, dtype=np.float64))
    K = torch.as_tensor(np.asarray(K, dtype=np.float64))
    V = torch.as_tensor(np.asarray(V, dtype=np.float64))
    if requires_grad:
        Q.requires_grad_(True)
        K.requires_grad_(True)
        V.requires_grad_(True)
    r = Q.shape[1] // K.shape[1]
    Ke = K.repeat_interleave(r, dim=1)
    Ve = V.repeat_interleave(r, dim=1)
    m = torch.as_tensor(np.ascontiguousarray(
        np.broadcast_to(mask, (Q.shape[0], Q.shape[1], Q.shape[2], K.shape[2]))))
    if scale is None:
        scale = 1.0 / math.sqrt(Q.shape[-1])
    O = torch.nn.functional.scaled_dot_product_attention(Q, Ke, Ve, attn_mask=m, scale=scale)
    return (O, Q, K, V) if requires_grad else O.numpy()


def hand_example_inputs(chunk0_key: float = 1.0):
    """The hand-built 3-chunk case described in golden/hand_example.json."""
    C, D, S = 64, 64, 192
    Q = np.zeros((1, 1, S, D))
    Q[..., 0] = 1.0
    K = np.zeros((1, 1, S, D))
    K[0, 0, 0:64, 0] = chunk0_key
    for t in range(8):
        K[0, 0, 64 + 8 * t:64 + 8 * t + 8, 0] = t - 2
    V = np.zeros((1, 1, S, D))
    V[0, 0, :, 1] = np.arange(S)
    return Q, K, V


def hand_example_output_e1(p: int, chunk0_key: float = 1.0) -> float:
    """Closed form of O_p[1] for the original hand example (scale 1/8), for the
    query at position p.  Block 2 (p >= 128) attends groups 14 (keys 4 e0,
    tokens 112..119) and 15 (keys 5 e0, tokens 120..127) and its own chunk
    128..p (keys 0).  Block 1 (64 <= p < 128) attends groups 0 and 1 (keys
    chunk0_key e0, tokens 0..15) and its own chunk 64..p, where token j has key
    ((j - 64) // 8 - 2) e0.  Block 0 attends 0..p (keys chunk0_key e0)."""
    if p >= 128:
        a, b = math.exp(0.5), math.exp(0.625)
        num = a * sum(range(112, 120)) + b * sum(range(120, 128)) + sum(range(128, p + 1))
        den = 8 * a + 8 * b + (p - 127)
        return num / den
    if p >= 64:
        w0 = math.exp(chunk0_key / 8)
        num = w0 * sum(range(0, 16))
        den = 16 * w0
        for j in range(64, p + 1):
            w = math.exp(((j - 64) // 8 - 2) / 8)
            num += w * j
            den += w
        return num / den
    return sum(range(0, p + 1)) / (p + 1)


def tie_band_ok(sel_test, sel_ref, scores, keep, rel=1e-5):
    """Selection comparison with the near-tie rule.

    scores: fp64 scores of every candidate (NaN for non-candidates), indexed by
    candidate id.  sel_*: kept ids (any order, -1 ignored).  Let s_k and s_k1 be
    the keep-th and (keep+1)-th best candidate scores and tau = rel * max |s|
    over candidates.  If s_k - s_k1 >= tau the sets must be identical;
    otherwise they may differ only in members whose score lies within tau of
    s_k.  Returns (ok, exact_required)."""
    cand = np.flatnonzero(~np.isnan(scores))
    a = set(int(x) for x in sel_test if x >= 0)
    b = set(int(x) for x in sel_ref if x >= 0)
    n = min(keep, cand.size)
    if len(a) != n or len(b) != n:
        return False, True
    if n == cand.size or n == 0:
        return a == b, True
    s = scores[cand]
    order = sorted(range(cand.size), key=lambda i: (-s[i], cand[i]))
    sk, sk1 = s[order[n - 1]], s[order[n]]
    tau = rel * np.max(np.abs(s))
    if sk - sk1 >= tau:
        return a == b, True
    diff = a ^ b
    ok = all(abs(scores[x] - sk) <= tau for x in diff) and all(x in set(cand.tolist()) for x in a)
    return ok, False


def allclose_report(got, ref, atol, rtol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    return (not bad.any(), float(err.max()) if err.size else 0.0, int(bad.sum()))
