"""Pins of the paged-cache view in the oracle (CPU only): a hand-worked
block table, the identity table, and the round trip through the seeded
paged layout (written independently: a scatter there, a gather here)."""

import numpy as np

import oracle
import synth


def test_hand_example():
    # 2 sequences, 1 head, block size 2, 2 logical blocks each; pool of 5
    pool = np.arange(5 * 2, dtype=np.float32).reshape(5, 1, 2, 1)   # block p holds 2p, 2p+1
    table = np.array([[3, 0], [1, 4]], np.int32)
    k, v = oracle.paged_to_contiguous(pool, -pool, table)
    np.testing.assert_array_equal(k[0, 0, :, 0], [6, 7, 0, 1])
    np.testing.assert_array_equal(k[1, 0, :, 0], [2, 3, 8, 9])
    np.testing.assert_array_equal(v, -k)


def test_identity_table():
    rng = np.random.Generator(np.random.PCG64(80))
    B, H, S, D, bs = 3, 2, 256, 8, 64
    k = rng.standard_normal((B, H, S, D)).astype(np.float32)
    pool = k.reshape(B, H, S // bs, bs, D).transpose(0, 2, 1, 3, 4).reshape(-1, H, bs, D)
    table = np.arange(B * S // bs, dtype=np.int32).reshape(B, S // bs)
    k2, _ = oracle.paged_to_contiguous(pool, pool, table)
    np.testing.assert_array_equal(k2, k)


def test_round_trip_through_the_paged_layout():
    rng = np.random.Generator(np.random.PCG64(81))
    for dtype, bs in ((np.float32, 64), (np.uint16, 128), (np.uint16, 256)):
        B, H, S, D = 2, 3, 512, 16
        k = rng.integers(0, 1 << 15, (B, H, S, D)).astype(dtype)
        v = rng.integers(0, 1 << 15, (B, H, S, D)).astype(dtype)
        kp, vp, table = synth.to_paged(k, v, bs, rng, spare_blocks=2)
        assert kp.shape == (B * S // bs + 2, H, bs, D) and table.shape == (B, S // bs)
        assert np.unique(table).size == table.size
        k2, v2 = oracle.paged_to_contiguous(kp, vp, table)
        np.testing.assert_array_equal(k2, k)
        np.testing.assert_array_equal(v2, v)
        unused = np.setdiff1d(np.arange(kp.shape[0]), table)
        assert unused.size == 2
