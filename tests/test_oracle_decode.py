"""Pins of the decode oracle (one query per head at the last cache position)
to things other than itself: dense softmax over the whole cache when the
budgets cover every candidate, the own chunk alone when no chunk is kept, an
independent sort of the routing scores, the hand example's closed form, and
the block form of the method when every query of a block equals the decode
query."""
import math

import numpy as np
import pytest

from hga_testlib import hand_example_inputs, hand_example_output_e1

rng = np.random.default_rng(2024)


def _case(B=2, Hq=4, Hkv=2, L=200, D=16):
    Q = rng.standard_normal((B, Hq, D))
    K = rng.standard_normal((B, Hkv, L, D))
    V = rng.standard_normal((B, Hkv, L, D))
    return Q, K, V


def _summ(oracle, K):
    L = K.shape[2]
    return oracle.summaries(K[:, :, :(L // 64) * 64])


def _dense_last(Q, K, V, keys, scale):
    """Softmax attention of each query over the listed key positions."""
    B, Hq, D = Q.shape
    r = Hq // K.shape[1]
    O = np.empty((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            s = scale * K[b, h // r, keys] @ Q[b, h]
            p = np.exp(s - s.max())
            O[b, h] = (p / p.sum()) @ V[b, h // r, keys]
    return O


@pytest.mark.parametrize("L", [200, 193, 256, 130])
def test_decode_full_coverage_is_dense(oracle, L):
    Q, K, V = _case(L=L)
    cm, gm = _summ(oracle, K)
    cp = (L - 1) // 64
    _, _, O, _ = oracle.decode(Q, K, V, cm, gm, top_k=max(cp, 1), top_g=max(8 * cp, 1))
    ref = _dense_last(Q, K, V, np.arange(L), 1 / math.sqrt(Q.shape[-1]))
    np.testing.assert_allclose(O, ref, atol=1e-12, rtol=1e-12)


def test_decode_no_chunks_is_own_chunk(oracle):
    Q, K, V = _case(L=200)
    cm, gm = _summ(oracle, K)
    ci, gi, O, _ = oracle.decode(Q, K, V, cm, gm, top_k=0, top_g=0)
    ref = _dense_last(Q, K, V, np.arange(192, 200), 1 / math.sqrt(Q.shape[-1]))
    np.testing.assert_allclose(O, ref, atol=1e-12, rtol=1e-12)


def test_decode_routing_matches_sort(oracle):
    Q, K, V = _case(L=500, D=16)
    cm, gm = _summ(oracle, K)
    k, g = 3, 10
    ci, gi, O, _ = oracle.decode(Q, K, V, cm, gm, top_k=k, top_g=g)
    B, Hq, D = Q.shape
    r = Hq // K.shape[1]
    cp = 499 // 64
    for b in range(B):
        for h in range(Hq):
            s = [(float(Q[b, h] @ cm[b, h // r, c]), c) for c in range(cp)]
            kept = sorted(c for _, c in sorted(s, key=lambda t: (-t[0], t[1]))[:k])
            assert list(ci[b, h][:len(kept)]) == kept and all(ci[b, h][len(kept):] == -1)
            gs = [(float(Q[b, h] @ gm[b, h // r, 8 * c + t]), 8 * c + t) for c in kept
                  for t in range(8)]
            gk = sorted(x for _, x in sorted(gs, key=lambda t: (-t[0], t[1]))[:g])
            assert list(gi[b, h]) == gk
            keys = np.concatenate([np.arange(8 * x, 8 * x + 8) for x in gk] +
                                  [np.arange(64 * cp, 500)])
            ref = _dense_last(Q[b:b + 1, h:h + 1], K[b:b + 1, h // r:h // r + 1],
                              V[b:b + 1, h // r:h // r + 1], keys, 1 / math.sqrt(D))
            np.testing.assert_allclose(O[b, h], ref[0, 0], atol=1e-12, rtol=1e-12)


def test_decode_hand_example(oracle):
    """Query e0 at position 191 of the hand example: chunk 1, groups 14 and 15."""
    Qb, K, V = hand_example_inputs()
    cm, gm = oracle.summaries(K)
    Q = Qb[:, :, 191]
    ci, gi, O, _ = oracle.decode(Q, K, V, cm, gm, top_k=1, top_g=2, scale=1 / 8)
    assert ci.tolist() == [[[1]]] and gi.tolist() == [[[14, 15]]]
    assert abs(O[0, 0, 1] - hand_example_output_e1(191)) < 1e-9


def test_decode_equals_block_form_with_repeated_query(oracle):
    """When all 64 queries of a block equal q, the block's routing query is q,
    so the block form's last query (position p = end of the block) gets the
    decode result for q at p."""
    B, Hq, Hkv, D, L = 1, 2, 1, 16, 320
    q = rng.standard_normal((B, Hq, D))
    K = rng.standard_normal((B, Hkv, L, D))
    V = rng.standard_normal((B, Hkv, L, D))
    cm, gm = oracle.summaries(K)
    ci_d, gi_d, O_d, lse_d = oracle.decode(q, K, V, cm, gm, top_k=2, top_g=9)
    Qb = np.repeat(q[:, :, None, :], 64, axis=2)          # the last block, 64 copies of q
    ci_b, gi_b = oracle.route(Qb, cm, gm, L, 2, 9)
    O_b, lse_b = oracle.attend_fwd(Qb, K, V, gi_b)
    assert np.array_equal(ci_b[:, :, 0], ci_d) and np.array_equal(gi_b[:, :, 0], gi_d)
    np.testing.assert_allclose(O_b[:, :, 63], O_d, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse_b[:, :, 63], lse_d, atol=1e-12, rtol=1e-12)
