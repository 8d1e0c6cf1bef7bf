"""Pins of the oracle's strictly causal routing variant (runs without a GPU).

The variant routes block j with the mean of the 64 queries just before it
(block j-1 of the segment, or for the first block the 64 queries before the
segment), so that no position's key set depends on a later position.  Pinned
to an independent numpy routing, to the defining causality property (and to
the block method's leak, so the property test is shown to have power), to
dense causal attention under full coverage, and to the segment boundary.
"""
import numpy as np
import pytest

from hga_testlib import causal_mask, sdpa_f64

rng = np.random.default_rng(777)


def _inputs(B=1, Hq=4, Hkv=2, Sq=384, Skv=640, D=16, prev=True):
    Q = rng.standard_normal((B, Hq, Sq, D))
    K = rng.standard_normal((B, Hkv, Skv, D))
    V = rng.standard_normal((B, Hkv, Skv, D))
    Qp = rng.standard_normal((B, Hq, 64, D)) if prev else None
    return Q, K, V, Qp


def _numpy_route(qbar, cm, gm, cb, k, g):
    s = [(float(qbar @ cm[c]), c) for c in range(cb)]
    kept = sorted(c for _, c in sorted(s, key=lambda t: (-t[0], t[1]))[:k])
    gs = [(float(qbar @ gm[8 * c + t]), 8 * c + t) for c in kept for t in range(8)]
    groups = sorted(x for _, x in sorted(gs, key=lambda t: (-t[0], t[1]))[:g])
    return kept, groups


@pytest.mark.parametrize("Sq,Skv,k,g", [(384, 640, 3, 11), (256, 256, 2, 9), (128, 1024, 5, 40)])
def test_causal_routing_matches_numpy(oracle, Sq, Skv, k, g):
    Q, K, V, Qp = _inputs(Sq=Sq, Skv=Skv, prev=Skv > Sq)
    cm, gm = oracle.summaries(K)
    ci, gi = oracle.route(Q, cm, gm, Skv, k, g, causal=True, Qprev=Qp)
    q0c = (Skv - Sq) // 64
    for h in range(Q.shape[1]):
        for blk in range(Sq // 64):
            cb = q0c + blk
            src = Q[0, h, 64 * (blk - 1):64 * blk] if blk > 0 else (Qp[0, h] if Qp is not None else None)
            if cb == 0:
                assert np.all(ci[0, h, blk] == -1) and np.all(gi[0, h, blk] == -1)
                continue
            kept, groups = _numpy_route(src.mean(0), cm[0, h // 2], gm[0, h // 2], cb, k, g)
            assert list(ci[0, h, blk][:len(kept)]) == kept and np.all(ci[0, h, blk][len(kept):] == -1)
            assert list(gi[0, h, blk][:len(groups)]) == groups
            assert np.all(gi[0, h, blk][len(groups):] == -1)


def _forward(oracle, Q, K, V, Qp, k, g, causal):
    cm, gm = oracle.summaries(K)
    _, gi = oracle.route(Q, cm, gm, K.shape[2], k, g, causal=causal, Qprev=Qp)
    return oracle.attend_fwd(Q, K, V, gi)[0]


@pytest.mark.parametrize("t", [192 + 17, 64 * 5 + 1, 63])
def test_causal_variant_has_no_future_dependence(oracle, t):
    """O at positions < t is unchanged, bit for bit, when every query, key and
    value at positions >= t is replaced (self-attention, q0 = 0)."""
    Q, K, V, _ = _inputs(Sq=512, Skv=512, prev=False)
    O = _forward(oracle, Q, K, V, None, 3, 12, causal=True)
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    Q2[:, :, t:] = rng.standard_normal(Q2[:, :, t:].shape)
    K2[:, :, t:] = rng.standard_normal(K2[:, :, t:].shape)
    V2[:, :, t:] = rng.standard_normal(V2[:, :, t:].shape)
    O2 = _forward(oracle, Q2, K2, V2, None, 3, 12, causal=True)
    assert np.array_equal(O[:, :, :t], O2[:, :, :t])


def test_block_method_leaks_where_the_variant_does_not(oracle):
    """The block method's routing mixes the block's later queries into its
    earlier positions: replacing queries from the middle of a block on changes
    the outputs of the block's earlier positions (the page's caveat)."""
    Q, K, V, _ = _inputs(Sq=512, Skv=512, prev=False)
    t = 64 * 4 + 32
    Q2 = Q.copy()
    Q2[:, :, t:] = 3.0 * rng.standard_normal(Q2[:, :, t:].shape)
    leak = _forward(oracle, Q, K, V, None, 2, 6, causal=False)
    leak2 = _forward(oracle, Q2, K, V, None, 2, 6, causal=False)
    assert not np.array_equal(leak[:, :, 256:t], leak2[:, :, 256:t])
    ok = _forward(oracle, Q, K, V, None, 2, 6, causal=True)
    ok2 = _forward(oracle, Q2, K, V, None, 2, 6, causal=True)
    assert np.array_equal(ok[:, :, :t], ok2[:, :, :t])


def test_causal_full_coverage_is_dense_causal(oracle):
    Q, K, V, Qp = _inputs(Sq=256, Skv=512, prev=True)
    O = _forward(oracle, Q, K, V, Qp, 8, 64, causal=True)
    ref = sdpa_f64(Q, K, V, causal_mask(256, 512))
    np.testing.assert_allclose(O, ref, atol=1e-12, rtol=1e-12)


def test_segment_boundary_uses_the_previous_segments_last_block(oracle):
    """Routing the second half of a sequence as a segment, with the last 64
    queries of the first half as Qprev, equals routing the whole sequence."""
    Q, K, V, _ = _inputs(Sq=512, Skv=512, prev=False)
    cm, gm = oracle.summaries(K)
    ci_all, gi_all = oracle.route(Q, cm, gm, 512, 3, 10, causal=True)
    ci_seg, gi_seg = oracle.route(Q[:, :, 256:], cm, gm, 512, 3, 10, causal=True,
                                  Qprev=Q[:, :, 192:256])
    assert np.array_equal(ci_all[:, :, 4:], ci_seg) and np.array_equal(gi_all[:, :, 4:], gi_seg)


def test_missing_previous_queries_is_an_error(oracle):
    Q, K, V, _ = _inputs(Sq=128, Skv=256, prev=False)
    cm, gm = oracle.summaries(K)
    with pytest.raises(ValueError):
        oracle.route(Q, cm, gm, 256, 2, 4, causal=True, Qprev=None)
