"""bench.py on the CPU: the one-GPU guard and the algorithmic work figures the
roofline is computed from (each restated here from its per-unit definition)."""
import os
import subprocess
import sys

import numpy as np
import torch

import bench
from hierarchical_routed_sparse_amd import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_attended_pairs_sums_every_query_key_set():
    """Each query of a block attends 8 keys per kept group and the keys of its
    own chunk up to itself: query i of the block, i + 1 of them."""
    rng = np.random.default_rng(5)
    B, Hq, nblk, g = 2, 3, 4, 12
    gi = np.full((B, Hq, nblk, g), -1, dtype=np.int32)
    for idx in np.ndindex(B, Hq, nblk):
        n = rng.integers(0, g + 1)
        gi[idx][:n] = np.sort(rng.choice(500, size=n, replace=False))
    expect = 0
    for idx in np.ndindex(B, Hq, nblk):
        kept = int((gi[idx] >= 0).sum())
        for i in range(64):
            expect += 8 * kept + (i + 1)
    assert bench.attended_pairs(torch.from_numpy(gi)) == expect


def test_training_step_work_per_unit():
    w = syn.WORKLOADS["segment_2k_over_16k"]
    pairs = 35_684_352
    work = bench.algorithmic_work(w, pairs)
    # summaries: per 64-key chunk, 16 KB of bf16 keys read, one fp32 chunk mean
    # and eight fp32 group means written
    per_chunk = 64 * 128 * 2 + 128 * 4 + 8 * 128 * 4
    assert per_chunk == 20_992
    assert work["summaries"] == ("hbm", 8 * 256 * per_chunk)
    # routing: the block's 64 bf16 query rows, then once the means, then indices
    means = 8 * (256 + 2048) * 128 * 4
    assert work["route"] == ("hbm", 32 * 2048 * 128 * 2 + means + 32 * 32 * (16 + 64) * 4)
    # 2 flops per multiply-add, D = 128 per product and pair: the forward's two
    # products; the backward's five, three (Q.K^T, dO.V^T, dS.K) for dQ and
    # two (P^T.dO, dS^T.Q) for dK/dV, 10 D per pair in all
    assert work["attend_fwd"] == ("mfma", 2 * 2 * 128 * pairs)
    assert work["attend_bwd_dq"] == ("mfma", 3 * 2 * 128 * pairs)
    assert work["attend_bwd_dkdv"] == ("mfma", 2 * 2 * 128 * pairs)
    assert work["attend_bwd_dq"][1] + work["attend_bwd_dkdv"][1] == 10 * 128 * pairs
    assert work["attend_bwd_dkdv"][1] == 18_270_388_224


def test_executed_work_counts_tiles_and_slices():
    """Executed MFMA flops from the kernels' tiling, restated by brute force on
    a small routing: forward and dQ walk 2 own-chunk tiles plus one 32-key
    tile per 4 kept groups; dK/dV works on every 16-key slice (group pair)
    with a kept group, plus the 4 slices of the own chunk."""
    gi = np.full((1, 2, 2, 6), -1, dtype=np.int32)
    gi[0, 0, 0, :5] = [0, 1, 2, 9, 17]      # pairs {0, 1, 4, 8}; 2 group tiles
    gi[0, 1, 1, :2] = [3, 40]               # pairs {1, 20}; 1 group tile
    D = 64
    ex = bench.executed_work(gi, D)
    tiles = (2 + 2) + (2 + 0) + (2 + 0) + (2 + 1)
    assert ex["attend_fwd"] == tiles * 32 * 64 * 4 * D
    assert ex["attend_bwd_dq"] == tiles * 32 * 64 * 6 * D
    slices = (4 + 4) + 4 + 4 + (2 + 4)
    assert ex["attend_bwd_dkdv"] == slices * 16 * 64 * 8 * D


def test_decode_work_per_row():
    w = syn.WORKLOADS["decode_b16_16k"]     # position 16423: own chunk 256, 40 own keys
    kept = 32_768                             # 64 groups for each of the 512 rows
    work = bench.decode_work(w, kept)
    rows = 16 * 32
    route = (rows * 128 * 2                   # the queries
             + 16 * 8 * 256 * 128 * 4         # chunk means before the own chunk, per kv head
             + rows * 16 * 8 * 128 * 4        # group means of each row's 16 kept chunks
             + rows * (16 + 64) * 4)          # indices written
    attend = (rows * (128 * 2 + 128 * 2 + 4)  # query, output row, lse
              + kept * 4                      # group indices
              + (kept * 8 + rows * 40) * 128 * 2 * 2)   # key and value rows
    assert work["decode_route"] == route == 50_626_560
    assert work["decode_attend"] == attend == 145_098_752
