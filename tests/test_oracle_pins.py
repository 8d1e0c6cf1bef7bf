"""Pins of the CPU oracle to things other than itself (runs without a GPU).

Each test fixes the oracle against a closed form, a library routine, an
independent brute force or a hand-derived case, chosen so that a dropped term,
a wrong sign or index, a wrong offset or a transposed operand fails one of them.
"""
import math

import numpy as np
import pytest
import torch

from hga_testlib import (allclose_report, causal_mask, hand_example_inputs,
                         hand_example_output_e1, hga_mask, load_golden, sdpa_f64)

rng = np.random.default_rng(12345)


def _rand(shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- summaries

def test_summaries_closed_form(oracle):
    """K[j, d] = j + d/1000: chunk c mean = 64c + 31.5 + d/1000, group mean = 8g + 3.5 + d/1000."""
    S, D = 256, 8
    K = (np.arange(S)[:, None] + np.arange(D)[None, :] / 1000.0)[None, None]
    cm, gm = oracle.summaries(K)
    for c in range(S // 64):
        np.testing.assert_allclose(cm[0, 0, c], 64 * c + 31.5 + np.arange(D) / 1000.0, rtol=0,
                                   atol=1e-12)
    for g in range(S // 8):
        np.testing.assert_allclose(gm[0, 0, g], 8 * g + 3.5 + np.arange(D) / 1000.0, rtol=0,
                                   atol=1e-12)


def test_summaries_match_numpy_mean_and_nest(oracle):
    K = _rand((2, 3, 512, 16))
    cm, gm = oracle.summaries(K)
    np.testing.assert_allclose(cm, K.reshape(2, 3, 8, 64, 16).mean(axis=3), atol=1e-13)
    np.testing.assert_allclose(gm, K.reshape(2, 3, 64, 8, 16).mean(axis=3), atol=1e-13)
    # a chunk mean is the mean of its eight group means
    np.testing.assert_allclose(cm, gm.reshape(2, 3, 8, 8, 16).mean(axis=3), atol=1e-13)


# ---------------------------------------------------------------- routing

def _route_case(B=1, Hq=4, Hkv=2, Sq=256, Skv=512, D=16, k=3, g=5):
    Q = _rand((B, Hq, Sq, D))
    K = _rand((B, Hkv, Skv, D))
    return Q, K, dict(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D, k=k, g=g)


def test_route_scores_are_block_means_of_dense_scores(oracle):
    """score(chunk c) = mean over the 64x64 block of the dense Q K^T matrix, and
    score(group) = mean over the 64x8 block; candidates are the chunks strictly
    before the block's own chunk, with the segment placed at the end."""
    Q, K, s = _route_case()
    cm, gm = oracle.summaries(K)
    ci, gi, cs, gs = oracle.route(Q, cm, gm, s["Skv"], s["k"], s["g"], want_scores=True)
    r = s["Hq"] // s["Hkv"]
    q0 = s["Skv"] - s["Sq"]
    for b in range(s["B"]):
        for h in range(s["Hq"]):
            dense = Q[b, h] @ K[b, h // r].T           # [Sq, Skv]
            for blk in range(s["Sq"] // 64):
                cb = q0 // 64 + blk
                blockrows = dense[blk * 64:(blk + 1) * 64]
                want = blockrows.reshape(64, -1, 64).mean(axis=(0, 2))
                got = cs[b, h, blk]
                assert np.all(np.isnan(got[cb:]))
                np.testing.assert_allclose(got[:cb], want[:cb], atol=1e-12)
                wantg = blockrows.reshape(64, -1, 8).mean(axis=(0, 2))
                kept = [c for c in ci[b, h, blk] if c >= 0]
                cand = sorted(8 * c + t for c in kept for t in range(8))
                gotg = gs[b, h, blk]
                assert sorted(np.flatnonzero(~np.isnan(gotg)).tolist()) == cand
                np.testing.assert_allclose(gotg[cand], wantg[cand], atol=1e-12)


def _expected_keep(scores, keep):
    cand = np.flatnonzero(~np.isnan(scores))
    order = sorted(cand.tolist(), key=lambda c: (-scores[c], c))
    kept = sorted(order[:min(keep, len(order))])
    return kept + [-1] * (keep - len(kept))


@pytest.mark.parametrize("k,g", [(3, 5), (1, 8), (4, 32), (0, 4), (2, 0), (16, 200)])
def test_topk_matches_full_sort(oracle, k, g):
    """Kept sets equal an independent Python full sort by (score desc, index asc),
    emitted ascending and padded with -1; fewer candidates than k keeps all."""
    Q, K, s = _route_case(k=k, g=g)
    cm, gm = oracle.summaries(K)
    ci, gi, cs, gs = oracle.route(Q, cm, gm, s["Skv"], k, g, want_scores=True)
    for idx in np.ndindex(ci.shape[:3]):
        assert ci[idx].tolist() == _expected_keep(cs[idx], k)
        assert gi[idx].tolist() == _expected_keep(gs[idx], g)


def test_topk_exact_ties_take_lower_index(oracle):
    """Exact duplicate chunks tie exactly; the lower chunk index is kept."""
    D = 8
    K = _rand((1, 1, 512, D))
    K[0, 0, 64 * 5:64 * 6] = K[0, 0, 64 * 2:64 * 3]      # chunk 5 == chunk 2
    K[0, 0, 64 * 6:64 * 7] = K[0, 0, 64 * 2:64 * 3]      # chunk 6 == chunk 2
    Q = _rand((1, 1, 64, D))
    cm, gm = oracle.summaries(K)
    # query block at the end: own chunk 7, candidates 0..6
    ci, gi, cs, _ = oracle.route(Q, cm, gm, 512, 7, 0, want_scores=True)
    assert cs[0, 0, 0, 2] == cs[0, 0, 0, 5] == cs[0, 0, 0, 6]
    # make chunk 2's triplet the best ones: pick q as +chunk-2 mean direction
    Q[:] = cm[0, 0, 2][None, None, None, :]
    ci, gi, cs, _ = oracle.route(Q, cm, gm, 512, 2, 0, want_scores=True)
    assert ci[0, 0, 0].tolist() == [2, 5]


def test_hand_example_routing_and_output(oracle):
    gold = load_golden("hand_example.json")
    for variant, key in (("expected", 1.0), ("tie_variant", 1.5)):
        Q, K, V = hand_example_inputs(chunk0_key=key)
        cm, gm = oracle.summaries(K)
        ci, gi = oracle.route(Q, cm, gm, 192, 1, 2)
        assert ci[0, 0].tolist() == gold[variant]["chunk_idx"]
        assert gi[0, 0].tolist() == gold[variant]["group_idx"]
        O, lse = oracle.attend_fwd(Q, K, V, gi, scale=0.125)
        for p in range(192):
            if variant == "tie_variant" and p >= 128:
                continue
            assert O[0, 0, p, 1] == pytest.approx(hand_example_output_e1(p, key), rel=1e-12)
        assert np.all(O[0, 0, :, 0] == 0) and np.all(O[0, 0, :, 2:] == 0)


# ---------------------------------------------------------------- attention forward

@pytest.mark.parametrize("Sq,Skv", [(256, 256), (128, 448)])
def test_full_coverage_equals_dense_causal(oracle, Sq, Skv):
    """With k and g covering the whole history, HGA is dense causal attention
    (the segment-at-end causal mask when Sq < Skv)."""
    B, Hq, Hkv, D = 1, 4, 2, 16
    Q, K, V = _rand((B, Hq, Sq, D)), _rand((B, Hkv, Skv, D)), _rand((B, Hkv, Skv, D))
    cm, gm = oracle.summaries(K)
    n = Skv // 64
    ci, gi = oracle.route(Q, cm, gm, Skv, n, 8 * n)
    O, lse = oracle.attend_fwd(Q, K, V, gi)
    ref = sdpa_f64(Q, K, V, causal_mask(Sq, Skv))
    np.testing.assert_allclose(O, ref, atol=1e-12)
    # lse against a direct logsumexp of the causal logits
    r = Hq // Hkv
    logits = np.einsum("bhqd,bhkd->bhqk", Q, np.repeat(K, r, axis=1)) / math.sqrt(D)
    logits = np.where(causal_mask(Sq, Skv), logits, -np.inf)
    ref_lse = torch.logsumexp(torch.as_tensor(logits), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


@pytest.mark.parametrize("k,g", [(0, 8), (3, 0)])
def test_local_only_is_block_diagonal_causal(oracle, k, g):
    B, Hq, Hkv, S, D = 1, 2, 1, 256, 16
    Q, K, V = _rand((B, Hq, S, D)), _rand((B, Hkv, S, D)), _rand((B, Hkv, S, D))
    cm, gm = oracle.summaries(K)
    ci, gi = oracle.route(Q, cm, gm, S, k, g)
    assert np.all(gi == -1)
    O, _ = oracle.attend_fwd(Q, K, V, gi)
    blockdiag = (np.arange(S)[:, None] // 64 == np.arange(S)[None, :] // 64) & causal_mask(S, S)
    np.testing.assert_allclose(O, sdpa_f64(Q, K, V, blockdiag), atol=1e-12)


def _random_routing(B, Hq, Sq, Skv, top_g, seed=0):
    r = np.random.default_rng(seed)
    nblk = Sq // 64
    q0 = Skv - Sq
    gi = np.full((B, Hq, nblk, top_g), -1, dtype=np.int32)
    for b, h, blk in np.ndindex(B, Hq, nblk):
        ncand = 8 * (q0 // 64 + blk)
        take = min(top_g, ncand, int(r.integers(0, top_g + 1)))
        if take:
            gi[b, h, blk, :take] = np.sort(r.choice(ncand, size=take, replace=False))
    return gi


def test_any_routing_equals_masked_dense(oracle):
    """For an arbitrary valid routing, HGA equals dense attention under the
    boolean mask of attended pairs (GQA: query head h reads kv head h//r)."""
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 192, 384, 16
    Q, K, V = _rand((B, Hq, Sq, D)), _rand((B, Hkv, Skv, D)), _rand((B, Hkv, Skv, D))
    gi = _random_routing(B, Hq, Sq, Skv, 12, seed=3)
    O, _ = oracle.attend_fwd(Q, K, V, gi, scale=0.3)
    ref = sdpa_f64(Q, K, V, hga_mask(gi, Sq, Skv), scale=0.3)
    np.testing.assert_allclose(O, ref, atol=1e-12)


def test_invalid_routing_rejected(oracle):
    B, Hq, Hkv, S, D = 1, 1, 1, 128, 8
    Q, K, V = _rand((B, Hq, S, D)), _rand((B, Hkv, S, D)), _rand((B, Hkv, S, D))
    gi = np.full((1, 1, 2, 2), -1, dtype=np.int32)
    gi[0, 0, 1] = [3, 8]        # group 8 lies in the block's own chunk
    with pytest.raises(ValueError):
        oracle.attend_fwd(Q, K, V, gi)
    gi[0, 0, 1] = [5, 3]        # not ascending
    with pytest.raises(ValueError):
        oracle.attend_fwd(Q, K, V, gi)


# ---------------------------------------------------------------- backward

def test_backward_matches_autograd_of_masked_dense(oracle):
    B, Hq, Hkv, Sq, Skv, D = 1, 4, 2, 128, 320, 16
    Q, K, V = _rand((B, Hq, Sq, D)), _rand((B, Hkv, Skv, D)), _rand((B, Hkv, Skv, D))
    dO = _rand((B, Hq, Sq, D))
    gi = _random_routing(B, Hq, Sq, Skv, 10, seed=7)
    dQ, dK, dV = oracle.attend_bwd(Q, K, V, gi, dO)
    O, tQ, tK, tV = sdpa_f64(Q, K, V, hga_mask(gi, Sq, Skv), requires_grad=True)
    O.backward(torch.as_tensor(dO))
    np.testing.assert_allclose(dQ, tQ.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dK, tK.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dV, tV.grad.numpy(), atol=1e-11)


def test_backward_central_differences(oracle):
    """d/dx sum(O * dO) by central differences (h = 1e-6) at sampled entries."""
    B, Hq, Hkv, S, D = 1, 2, 1, 192, 8
    Q, K, V = _rand((B, Hq, S, D)), _rand((B, Hkv, S, D)), _rand((B, Hkv, S, D))
    dO = _rand((B, Hq, S, D))
    cm, gm = oracle.summaries(K)
    ci, gi = oracle.route(Q, cm, gm, S, 1, 3)
    dQ, dK, dV = oracle.attend_bwd(Q, K, V, gi, dO)

    def loss(Qx, Kx, Vx):
        O, _ = oracle.attend_fwd(Qx, Kx, Vx, gi)
        return float((O * dO).sum())

    h = 1e-6
    pick = np.random.default_rng(5)
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for _ in range(6):
            idx = tuple(int(pick.integers(0, n)) for n in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = {"Q": (Xp, K, V), "K": (Q, Xp, V), "V": (Q, K, Xp)}[name]
            args_m = {"Q": (Xm, K, V), "K": (Q, Xm, V), "V": (Q, K, Xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert G[idx] == pytest.approx(fd, abs=1e-6), (name, idx)


def test_unattended_keys_get_zero_gradient(oracle):
    B, Hq, Hkv, S, D = 1, 1, 1, 256, 8
    Q, K, V, dO = (_rand((B, Hq, S, D)), _rand((B, Hkv, S, D)), _rand((B, Hkv, S, D)),
                   _rand((B, Hq, S, D)))
    gi = np.full((1, 1, 4, 1), -1, dtype=np.int32)
    gi[0, 0, 3, 0] = 2                      # block 3 reads group 2 only
    _, dK, dV = oracle.attend_bwd(Q, K, V, gi, dO)
    attended = hga_mask(gi, S, S).any(axis=2)[0, 0]
    assert np.all(dK[0, 0, ~attended] == 0) and np.all(dV[0, 0, ~attended] == 0)
    assert np.all(np.abs(dV[0, 0, attended]).sum(axis=-1) > 0)


# ---------------------------------------------------------------- work count

def test_attended_pairs_constant_per_block(oracle):
    """Attention work per query block is 64*8*g_sel + 64*65/2 pairs, independent of
    the history length once the budget is saturated."""
    for Skv in (1024, 4096):
        Q, K = _rand((1, 2, 256, 8)), _rand((1, 1, Skv, 8))
        cm, gm = oracle.summaries(K)
        _, gi = oracle.route(Q, cm, gm, Skv, 4, 16)
        nrows = 2 * 4
        assert oracle.attended_pairs(gi) == nrows * (64 * 8 * 16 + 64 * 65 // 2)
        assert oracle.attended_pairs(gi) == hga_mask(gi, 256, Skv).sum()


# ---------------------------------------------------------------- forced chunk sets

def _numpy_groups_on_chunks(qbar, K, chunks, top_g, G=8):
    """Independent joint top-g over the groups of a given chunk set: group means
    from a numpy reshape, scores q.mean, full sort on (-score, index), kept
    groups ascending, -1 padded."""
    cand = [8 * c + t for c in chunks if c >= 0 for t in range(8)]
    gmean = K.reshape(-1, G, K.shape[-1]).mean(axis=1)
    scored = sorted(((-float(qbar @ gmean[x]), x) for x in cand))
    kept = sorted(x for _, x in scored[:min(top_g, len(cand))])
    return kept + [-1] * (top_g - len(kept))


@pytest.mark.parametrize("causal", [False, True])
def test_route_forced_chunks_match_numpy(oracle, causal):
    """With forced chunk sets (here random sets, not the top-k), the oracle's
    group stage equals an independent numpy joint top-g over those chunks'
    groups, for the block routing query and for the strictly causal one (the
    mean of the 64 queries before the block).  This is the branch the GPU tests
    use when a near tie lets the GPU keep a different chunk set."""
    B, Hq, Hkv, Sq, Skv, D, k, g = 1, 4, 2, 256, 768, 16, 4, 13
    Q = _rand((B, Hq, Sq, D))
    K = _rand((B, Hkv, Skv, D))
    Qprev = _rand((B, Hq, 64, D)) if causal else None
    cm, gm = oracle.summaries(K)
    nblk, q0, r = Sq // 64, Skv - Sq, Hq // Hkv
    frng = np.random.default_rng(7)
    forced = np.full((B, Hq, nblk, k), -1, dtype=np.int32)
    for h in range(Hq):
        for blk in range(nblk):
            cb = q0 // 64 + blk
            n = int(frng.integers(0, k + 1))
            forced[0, h, blk, :n] = np.sort(frng.choice(cb, size=n, replace=False))
    ci, gi = oracle.route(Q, cm, gm, Skv, k, g, forced_chunk_idx=forced, causal=causal,
                          Qprev=Qprev)
    assert np.array_equal(ci, forced)
    for h in range(Hq):
        for blk in range(nblk):
            if not causal:
                src = Q[0, h, blk * 64:(blk + 1) * 64]
            elif blk > 0:
                src = Q[0, h, (blk - 1) * 64:blk * 64]
            else:
                src = Qprev[0, h]
            want = _numpy_groups_on_chunks(src.mean(axis=0), K[0, h // r], forced[0, h, blk], g)
            assert gi[0, h, blk].tolist() == want, (h, blk)


def test_route_forced_chunk_outside_candidates_rejected(oracle):
    Q, K = _rand((1, 1, 64, 8)), _rand((1, 1, 256, 8))
    cm, gm = oracle.summaries(K)
    forced = np.array([[[[1, 3]]]], dtype=np.int32)   # chunk 3 is the block's own chunk
    with pytest.raises(ValueError):
        oracle.route(Q, cm, gm, 256, 2, 4, forced_chunk_idx=forced)


def test_decode_forced_chunks_match_numpy(oracle):
    """The decode form with forced chunk sets: groups equal the numpy joint
    top-g over the forced chunks' groups, scored with the token's query."""
    B, Hq, Hkv, L, D, k, g = 2, 2, 1, 600, 16, 3, 11
    Q = _rand((B, Hq, D))
    K = _rand((B, Hkv, L, D))
    V = _rand((B, Hkv, L, D))
    cm, gm = oracle.summaries(K[:, :, :64 * (L // 64)])
    cp = (L - 1) // 64
    frng = np.random.default_rng(11)
    forced = np.full((B, Hq, k), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            n = int(frng.integers(0, k + 1))
            forced[b, h, :n] = np.sort(frng.choice(cp, size=n, replace=False))
    ci, gi, O, lse = oracle.decode(Q, K, V, cm, gm, k, g, forced_chunk_idx=forced)
    assert np.array_equal(ci, forced)
    for b in range(B):
        for h in range(Hq):
            want = _numpy_groups_on_chunks(Q[b, h], K[b, 0, :64 * cp], forced[b, h], g)
            assert gi[b, h].tolist() == want, (b, h)
