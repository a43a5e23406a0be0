"""Pins for the oracle's greedy argmax (oracle_argmax_f32) against facts
outside it: hand-written rows (ties, signed zeros, subnormals, infinities,
NaN), numpy.argmax on random rows up to a full vocabulary, and the split
property the device kernel relies on (combining chunk winners with the
(value, lower index) rule gives the whole-row winner).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_argmax_hand_written_rows():
    d = json.load(open(os.path.join(GOLDEN, "argmax_rows.json")))
    for row in d["rows"]:
        x = np.array([float(v) for v in row["x"]], np.float32)
        assert oracle.argmax_f32(x[None, :])[0] == row["argmax"], row["why"]


@pytest.mark.parametrize("N", [1, 2, 7, 1000, 151936])
def test_argmax_matches_numpy_on_random_rows(N):
    rng = np.random.default_rng(N)
    x = rng.normal(0, 3, size=(4, N)).astype(np.float32)
    if N > 10:
        x[1, rng.integers(0, N, 3)] = x[1].max() + 1          # planted three-way tie
        x[2, rng.integers(0, N, 2)] = np.nan
    assert np.array_equal(oracle.argmax_f32(x), np.argmax(x, axis=1))


def test_argmax_of_quantized_logits_with_many_ties():
    # Values on a coarse grid make ties common everywhere in the row.
    rng = np.random.default_rng(5)
    x = rng.integers(-4, 5, size=(3, 5000)).astype(np.float32)
    assert np.array_equal(oracle.argmax_f32(x), np.argmax(x, axis=1))


def test_argmax_split_and_combine_gives_the_row_winner():
    # Winner of each chunk, then the best winner by (value, lower index):
    # the row winner for any split, which is what lets a device kernel split
    # a row across blocks and still return the same index.
    rng = np.random.default_rng(6)
    x = rng.integers(-3, 4, size=(8, 3001)).astype(np.float32)
    whole = oracle.argmax_f32(x)
    for trial in range(20):
        cuts = np.sort(rng.choice(np.arange(1, 3001), size=rng.integers(1, 30), replace=False))
        bounds = [0] + cuts.tolist() + [3001]
        for i in range(x.shape[0]):
            best = None
            for a, b in zip(bounds[:-1], bounds[1:]):
                j = a + int(oracle.argmax_f32(x[i:i + 1, a:b])[0])
                if best is None or x[i, j] > x[i, best] or (x[i, j] == x[i, best] and j < best):
                    best = j
            assert best == whole[i]


def test_argmax_accepts_bit_patterns():
    x = np.array([[0x3F800000, 0x40000000, 0xBF800000]], np.uint32)   # 1, 2, -1
    assert oracle.argmax_f32(x)[0] == 1
