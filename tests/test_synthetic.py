"""The seeded input generator against its published definitions (no GPU)."""
import numpy as np

from hierarchical_routed_sparse_amd import synthetic as syn


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 from state 0 (Steele, Lea, Flood 2014; the
    # reference C implementation distributed with the xoshiro generators).
    got = [int(x) for x in syn.splitmix64(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_agree():
    whole = syn.splitmix64(1234, 0, 100)
    part = syn.splitmix64(1234, 40, 10)
    assert np.array_equal(whole[40:50], part)


def test_normals_moments():
    x = syn.normals(syn.stream_state(7, syn.TAG_Q), 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert abs(np.mean(x ** 4) - 3) < 0.05


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    b = syn.f32_to_bf16_bits(x)
    back = syn.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]


def test_workload_recipe_structure():
    w = syn.scaled_workload(syn.WORKLOADS["segment_2k_over_64k_ties"], kv_len=4096, q_len=512,
                            n_q_heads=4, n_kv_heads=2)
    x = syn.make_inputs(w)
    assert x["K"].dtype == np.uint16 and x["K"].shape == (1, 2, 4096, 128)
    K = syn.to_f64(x["K"], "bf16").reshape(1, 2, 64, 64, 128)
    # clustered keys: rows of a chunk sit around a shared centroid (noise sigma 0.5)
    within = K.std(axis=3).mean()
    assert 0.4 < within < 0.6
    # duplicated chunks: int(0.05 * 64) = 3 chunks per head copy an earlier chunk
    flat = K.reshape(1, 2, 64, -1)
    for h in range(2):
        exact = sum(any(np.array_equal(flat[0, h, c], flat[0, h, s]) for s in range(c))
                    for c in range(64))
        near = sum(any(np.count_nonzero(flat[0, h, c] != flat[0, h, s]) == 1 for s in range(c))
                   for c in range(64))
        assert exact >= 1 and near >= 1
    q = syn.to_f64(x["Q"], "bf16")
    assert abs(q.std() * np.sqrt(128) - 1) < 0.02
