"""Pins for the oracle's top-k selection (NVFP4 article section 3.3: block
level top-2048 with the newest block kept, position level top-512).

Checked against a Python ``sorted`` brute force and against the selection
invariants; ties are frequent on purpose (integer-valued scores)."""
import numpy as np
import pytest

from oracle import csa2_ref as ref


def _brute(scores, ids, k, forced):
    valid = [(s, i) for s, i in zip(scores, ids) if i >= 0 and not np.isnan(s) and s != -np.inf]
    rest = [(s, i) for s, i in valid if i != forced]
    have_forced = len(rest) != len(valid)
    rest.sort(key=lambda e: (-e[0], e[1]))
    pick = ([forced] if have_forced else []) + [i for _, i in rest]
    pick = sorted(pick[:k])
    return pick + [-1] * (k - len(pick))


@pytest.mark.parametrize("seed", range(6))
def test_random_rows_with_ties(seed):
    rng = np.random.default_rng(seed)
    R, n = 7, 300
    scores = rng.integers(0, 12, (R, n)).astype(np.float64) / 4
    scores[rng.random((R, n)) < 0.1] = -np.inf
    ids = np.tile(np.arange(n, dtype=np.int32) * 3 + 5, (R, 1))
    ids[rng.random((R, n)) < 0.05] = -1
    forced = rng.integers(-1, n, R).astype(np.int32) * 3 + 5
    forced[0] = -1
    for k in (1, 17, 64, 299, 400):
        out = ref.select(scores, k, ids=ids, forced=forced)
        for r in range(R):
            assert list(out[r]) == _brute(scores[r], ids[r], k, forced[r]), (seed, k, r)


def test_ids_default_to_columns_and_ties_prefer_small_ids():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 0.5]])
    assert list(ref.select(s, 2)[0]) == [1, 2]
    assert list(ref.select(s, 4)[0]) == [1, 2, 3, 4]


def test_forced_replaces_the_weakest_pick():
    s = np.array([[5.0, 4.0, 3.0, 2.0, 1.0, 0.0]])
    out = ref.select(s, 3, forced=np.array([5], np.int32))
    assert list(out[0]) == [0, 1, 5]
    # forced already among the top k: nothing changes
    out = ref.select(s, 3, forced=np.array([1], np.int32))
    assert list(out[0]) == [0, 1, 2]


def test_fewer_valid_than_k_keeps_all_and_pads():
    s = np.array([[-np.inf, 2.0, -np.inf, 1.0]])
    assert list(ref.select(s, 3)[0]) == [1, 3, -1]
    s = np.full((1, 4), -np.inf)
    assert list(ref.select(s, 2)[0]) == [-1, -1]


def test_invariants_large_row():
    rng = np.random.default_rng(99)
    n, k = 20000, 512
    s = rng.integers(0, 50, (1, n)).astype(np.float64)
    out = ref.select(s, k)[0]
    assert len(set(out)) == k and np.all(np.diff(out) > 0)
    chosen = set(out.tolist())
    worst = min((s[0, i], -i) for i in chosen)
    for i in range(n):
        if i not in chosen:
            assert (s[0, i], -i) < worst
