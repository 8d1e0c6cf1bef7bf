"""Decode (one new token per sequence over a resident cache): HIP path vs the
CPU oracle's decode, element by element (needs an MI355X, except the first
test).

The cache is allocated at its capacity and the rows past kv_len, and the
summary rows never built, hold NaN: a kernel that reads them fails the test.
Routing indices must match bit for bit except inside the near-tie band; the
attention is always checked on the GPU's own routing.  Tolerances as for the
block path: |gpu - oracle| <= atol + rtol |oracle|, (2e-2, 1e-2) for bf16 and
(1e-5, 1e-5) for fp32.
"""
import math

import numpy as np
import pytest

import hierarchical_routed_sparse_amd as hga
from hierarchical_routed_sparse_amd import synthetic as syn
from hga_testlib import tie_band_ok

TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}


def _workload(name, B, Hq, Hkv, D, L, k, g, dtype, seed):
    return syn.Workload(name, B, Hq, Hkv, D, 1, L, k, g, dtype, seed,
                        1 / math.sqrt(D) if dtype == "bf16" else 0.4)


CASES = {
    "bf16_d128_L200_gqa4": _workload("a", 2, 8, 2, 128, 200, 2, 10, "bf16", 31),
    "bf16_d64_L1000": _workload("b", 1, 4, 1, 64, 1000, 4, 13, "bf16", 32),
    "fp32_d128_L777": _workload("c", 1, 2, 2, 128, 777, 3, 17, "fp32", 33),
    "fp32_d64_L129_one_own_token": _workload("d", 2, 2, 1, 64, 129, 2, 16, "fp32", 34),
    "bf16_first_token": _workload("e", 1, 4, 2, 128, 1, 4, 8, "bf16", 35),
    "bf16_L64_no_candidates": _workload("f", 1, 4, 2, 128, 64, 4, 8, "bf16", 36),
    "bf16_L65_one_candidate": _workload("g", 1, 8, 1, 128, 65, 1, 3, "bf16", 37),
    "bf16_k0_own_chunk_only": _workload("h", 1, 4, 2, 128, 300, 0, 8, "bf16", 38),
    "bf16_g0_own_chunk_only": _workload("i", 1, 4, 2, 128, 300, 3, 0, "bf16", 39),
    "bf16_max_budgets": _workload("j", 1, 4, 1, 128, 4113, 64, 512, "bf16", 40),
    "bf16_r8_two_route_sets": _workload("k", 1, 8, 1, 128, 2000, 5, 30, "bf16", 41),
}


def _random_cases(n, seed=131):
    """n valid decode problems from a seeded generator: bf16 and fp32, D 64 and
    128, 1 to 8 query heads per kv head, batch 1 to 3, cache lengths of 1 to
    3000 tokens (any length, so any position within its chunk), top-k 0 to 24
    and top-g up to 8 groups past what the kept chunks hold."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        dtype = "bf16" if i % 2 == 0 else "fp32"
        D = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 3))
        r = int(rng.choice([1, 2, 4, 8]))
        L = int(rng.integers(1, 3001))
        k = int(rng.integers(0, 25))
        g = int(rng.integers(0, 8 * k + 9))
        name = f"rand{i}_{dtype}_d{D}_h{hkv * r}x{hkv}_L{L}_k{k}_g{g}"
        out[name] = _workload(name, int(rng.integers(1, 4)), hkv * r, hkv, D, L, k, g, dtype,
                              500 + i)
    return out


RANDOM = _random_cases(10)


def _cap(L):
    return max(64, -(-L // 64) * 64)


def test_decode_inputs_extend_the_block_recipe():
    """A cache of L tokens, L not a multiple of 64, holds the first L rows of
    the recipe's keys and values at any longer length (one sequence, one kv
    head: the counter-based streams line up), so decode inputs follow the same
    clustered-key recipe as the block workloads."""
    w = _workload("x", 1, 1, 1, 64, 200, 2, 4, "fp32", 3)
    a = syn.make_inputs(w)
    for L in (192, 256):
        b = syn.make_inputs(syn.scaled_workload(w, kv_len=L))
        n = min(200, L)
        assert np.array_equal(a["K"][:, :, :n], b["K"][:, :, :n])
        assert np.array_equal(a["V"][:, :, :n], b["V"][:, :, :n])
    assert a["K"].shape == (1, 1, 200, 64) and a["Q"].shape == (1, 1, 1, 64)


# ------------------------------------------------------------------ GPU

def _run(w, x, kv_on_host=False, chunk_idx_out=True):
    import torch
    dev = "cuda:0"
    B, Hq, Hkv, D, L = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.kv_len
    cap = _cap(L)
    s = hga.make_shape(B, Hq, Hkv, D, 1, L, w.top_k, w.top_g, dtype=w.dtype, kv_capacity=cap)
    elt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    K = torch.full((B, Hkv, cap, D), float("nan"), dtype=elt, device=dev)
    V = torch.full((B, Hkv, cap, D), float("nan"), dtype=elt, device=dev)
    K[:, :, :L] = syn.to_torch(x["K"], w.dtype, dev)
    V[:, :, :L] = syn.to_torch(x["V"], w.dtype, dev)
    Q = syn.to_torch(x["Q"], w.dtype, dev)[:, :, 0].contiguous()
    cm = torch.full((B, Hkv, cap // 64, D), float("nan"), device=dev)
    gm = torch.full((B, Hkv, cap // 8, D), float("nan"), device=dev)
    hga.hga_build_summaries(s, K, cm, gm, 0, L // 64)
    if kv_on_host:
        torch.cuda.synchronize()
        Kh = torch.empty(K.shape, dtype=elt, pin_memory=True)
        Vh = torch.empty(V.shape, dtype=elt, pin_memory=True)
        Kh.copy_(K)
        Vh.copy_(V)
        K, V = Kh, Vh
    ci = torch.full((B, Hq, w.top_k), -7, dtype=torch.int32, device=dev)
    gi = torch.full((B, Hq, w.top_g), -7, dtype=torch.int32, device=dev)
    O = torch.full((B, Hq, D), float("nan"), dtype=elt, device=dev)
    lse = torch.full((B, Hq), float("nan"), device=dev)
    hga.hga_decode(s, Q, K, V, cm, gm, ci if chunk_idx_out else None, gi, O, lse)
    torch.cuda.synchronize()
    return dict(ci=ci.cpu().numpy(), gi=gi.cpu().numpy(),
                O=O.float().cpu().numpy().astype(np.float64),
                lse=lse.cpu().numpy().astype(np.float64), cm=cm, gm=gm)


def _attend_keys(q, K, V, keys, scale):
    """Softmax attention of one query over the listed key rows (fp64)."""
    s = scale * (K[keys] @ q)
    m = s.max()
    p = np.exp(s - m)
    return (p / p.sum()) @ V[keys], m + math.log(p.sum())


def _key_list(groups, L):
    p = L - 1
    own = np.arange(64 * (p // 64), p + 1)
    return np.concatenate([np.arange(8 * g, 8 * g + 8) for g in groups if g >= 0] + [own])


def _check(oracle, w, x, out, batches=None):
    """Routing (tie band) and O, lse of the GPU against the oracle; returns the
    number of rows where a near tie allowed a routing difference."""
    atol, rtol = TOL[w.dtype]
    L, r = w.kv_len, w.n_q_heads // w.n_kv_heads
    scale = 1 / math.sqrt(w.head_dim)
    tolerated = 0
    for b in (batches if batches is not None else range(w.batch)):
        Qf = syn.to_f64(x["Q"][b:b + 1, :, 0], w.dtype)
        Kf = syn.to_f64(x["K"][b:b + 1], w.dtype)
        Vf = syn.to_f64(x["V"][b:b + 1], w.dtype)
        nca = L // 64
        if nca:
            cm_o, gm_o = oracle.summaries(Kf[:, :, :64 * nca])
            # the GPU's summaries, every built row, against the oracle's
            np.testing.assert_allclose(out["cm"][b:b + 1, :, :nca].cpu().numpy(), cm_o,
                                       atol=1e-5, rtol=1e-5)
            np.testing.assert_allclose(out["gm"][b:b + 1, :, :8 * nca].cpu().numpy(), gm_o,
                                       atol=1e-5, rtol=1e-5)
        else:
            cm_o = np.zeros((1, w.n_kv_heads, 0, w.head_dim))
            gm_o = np.zeros((1, w.n_kv_heads, 0, w.head_dim))
        ci_g, gi_g = out["ci"][b:b + 1], out["gi"][b:b + 1]
        ci_o, gi_o, O_o, lse_o, cs, gs = oracle.decode(Qf, Kf, Vf, cm_o, gm_o, w.top_k,
                                                       w.top_g, want_scores=True)
        if not np.array_equal(ci_g, ci_o):
            for h in range(w.n_q_heads):
                a = ci_g[0, h]
                v = a[a >= 0]
                assert np.all(np.diff(v) > 0) and np.all(a[len(v):] == -1), (b, h, a)
                if not np.array_equal(a, ci_o[0, h]):
                    ok, _ = tie_band_ok(a, ci_o[0, h], cs[0, h], w.top_k)
                    assert ok, f"chunks differ beyond the tie band at ({b},{h}): {a} vs {ci_o[0, h]}"
                    tolerated += 1
            _, gi_o, O_o, lse_o, _, gs = oracle.decode(Qf, Kf, Vf, cm_o, gm_o, w.top_k, w.top_g,
                                                       forced_chunk_idx=ci_g, want_scores=True)
        for h in range(w.n_q_heads):
            a = gi_g[0, h]
            v = a[a >= 0]
            assert np.all(np.diff(v) > 0) and np.all(a[len(v):] == -1), (b, h, a)
            if not np.array_equal(a, gi_o[0, h]):
                ok, _ = tie_band_ok(a, gi_o[0, h], gs[0, h], w.top_g)
                assert ok, f"groups differ beyond the tie band at ({b},{h}): {a} vs {gi_o[0, h]}"
                tolerated += 1
                # attention on the GPU's own groups
                O_o[0, h], lse_o[0, h] = _attend_keys(Qf[0, h], Kf[0, h // r], Vf[0, h // r],
                                                      _key_list(a, L), scale)
        for name, got, ref in (("O", out["O"][b:b + 1], O_o), ("lse", out["lse"][b:b + 1], lse_o)):
            err = np.abs(got - ref)
            bad = err > atol + rtol * np.abs(ref)
            assert not bad.any(), f"{name}[{b}]: {int(bad.sum())} beyond tolerance, max {err.max():.3e}"
    return tolerated


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_decode_small_case_parity(oracle, name):
    w = CASES[name]
    print(f"[case] decode {name}", flush=True)
    x = syn.make_inputs(w)
    out = _run(w, x)
    _check(oracle, w, x, out)


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(RANDOM))
def test_decode_random_shapes_parity(oracle, name):
    """The same comparison on seeded random valid decode problems."""
    w = RANDOM[name]
    print(f"[case] decode {name}", flush=True)
    x = syn.make_inputs(w)
    out = _run(w, x)
    _check(oracle, w, x, out)


@pytest.mark.gpu
def test_decode_full_coverage_equals_dense():
    """Budgets covering every candidate: the token attends its whole history."""
    w = _workload("cover", 1, 4, 2, 128, 520, 8, 64, "bf16", 42)
    x = syn.make_inputs(w)
    out = _run(w, x)
    Qf, Kf, Vf = (syn.to_f64(x[k], "bf16") for k in ("Q", "K", "V"))
    for h in range(4):
        ref, _ = _attend_keys(Qf[0, h, 0], Kf[0, h // 2], Vf[0, h // 2], np.arange(520),
                              1 / math.sqrt(128))
        np.testing.assert_allclose(out["O"][0, h], ref, atol=2e-2, rtol=1e-2)


@pytest.mark.gpu
def test_decode_deterministic_and_chunk_idx_optional(oracle):
    w = CASES["bf16_d128_L200_gqa4"]
    x = syn.make_inputs(w)
    a = _run(w, x)
    b = _run(w, x, chunk_idx_out=False)
    assert np.array_equal(a["gi"], b["gi"])
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])


@pytest.mark.gpu
def test_decode_host_resident_cache_is_bit_exact():
    """K and V in pinned host memory give the same bits as in HBM."""
    w = CASES["bf16_r8_two_route_sets"]
    x = syn.make_inputs(w)
    a = _run(w, x)
    b = _run(w, x, kv_on_host=True)
    for k in ("ci", "gi", "O", "lse"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.gpu
def test_decode_loop_across_a_chunk_boundary(oracle):
    """Tokens at positions 120..140 decoded one by one over one growing cache;
    the summary of chunk 1 is appended once its 64th key (position 127) is in."""
    import torch
    dev = "cuda:0"
    B, Hq, Hkv, D, cap, k, g = 1, 4, 2, 128, 192, 2, 6
    full = _workload("loop", B, Hq, Hkv, D, 141, k, g, "bf16", 43)
    x = syn.make_inputs(full)
    Qbits = syn.f32_to_bf16_bits(
        (syn.normals(syn.stream_state(43, 99), 21 * B * Hq * D) / math.sqrt(D)).astype(
            np.float32)).reshape(21, B, Hq, 1, D)
    K = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=dev)
    V = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=dev)
    cm = torch.full((B, Hkv, cap // 64, D), float("nan"), device=dev)
    gm = torch.full((B, Hkv, cap // 8, D), float("nan"), device=dev)
    Kt, Vt = syn.to_torch(x["K"], "bf16", dev), syn.to_torch(x["V"], "bf16", dev)
    K[:, :, :120] = Kt[:, :, :120]
    V[:, :, :120] = Vt[:, :, :120]
    hga.hga_build_summaries(hga.make_shape(B, Hq, Hkv, D, 1, 120, k, g, kv_capacity=cap),
                            K, cm, gm, 0, 1)
    for i, L in enumerate(range(121, 142)):
        K[:, :, L - 1] = Kt[:, :, L - 1]          # append the new token's key and value
        V[:, :, L - 1] = Vt[:, :, L - 1]
        s = hga.make_shape(B, Hq, Hkv, D, 1, L, k, g, kv_capacity=cap)
        if L % 64 == 0:
            hga.hga_build_summaries(s, K, cm, gm, L // 64 - 1, L // 64)
        Q = syn.to_torch(Qbits[i][:, :, 0], "bf16", dev)
        o = hga.decode(s, Q, K, V, cm, gm)
        torch.cuda.synchronize()
        out = dict(ci=o["chunk_idx"].cpu().numpy(), gi=o["group_idx"].cpu().numpy(),
                   O=o["O"].float().cpu().numpy().astype(np.float64),
                   lse=o["lse"].cpu().numpy().astype(np.float64), cm=cm, gm=gm)
        xs = {"Q": Qbits[i], "K": x["K"][:, :, :L], "V": x["V"][:, :, :L]}
        _check(oracle, syn.scaled_workload(full, kv_len=L), xs, out)


@pytest.mark.gpu
def test_decode_full_size_sampled_sequences(oracle):
    """The 16,424-token cache at batch 16 (the benchmark's decode workload):
    summaries, routing and O, lse of every head of four sampled sequences."""
    w = syn.WORKLOADS["decode_b16_16k"]
    print("[case] decode full size", flush=True)
    x = syn.make_inputs(w)
    out = _run(w, x)
    tolerated = _check(oracle, w, x, out, batches=[0, 5, 10, 15])
    print(f"[routing] decode full size: rows inside the near-tie band: {tolerated}", flush=True)


@pytest.mark.gpu
def test_decode_maximum_cache(oracle):
    """A full 131072-token cache (the largest decode shape): 2047 candidate
    chunks, the widest decode routing select."""
    w = _workload("max", 1, 4, 1, 128, 131072, 16, 64, "bf16", 44)
    print("[case] decode maximum cache", flush=True)
    x = syn.make_inputs(w)
    out = _run(w, x)
    _check(oracle, w, x, out)
