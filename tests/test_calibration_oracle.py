"""Pins of the fp64 calibration oracle (greedy outlier-aware block search,
DuQuant++ page sec. 3.2) against facts outside it."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import calibration as CAL

GROUP = 32


def givens_matrix(d, j, n=GROUP):
    """Explicit rotation for the row-vector product x G that maps
    (x_d, x_j) to (c x_d - s x_j, s x_d + c x_j), c = s = sqrt(1/2)."""
    c = s = math.sqrt(0.5)
    g = np.eye(n)
    g[d, d] = c
    g[j, d] = -s
    g[d, j] = s
    g[j, j] = c
    return g


def test_single_outlier_first_step_closed_form():
    x = np.zeros((4, GROUP))
    x[2, 5] = 8.0
    R, cur, hist, pairs = CAL.greedy_givens(x, steps=1)
    assert pairs == [(5, 0)]  # every candidate ties at 8/sqrt(2): lowest j
    assert hist[0] == 8.0
    assert abs(hist[1] - 8.0 / math.sqrt(2.0)) <= 1e-15 * 8.0
    assert np.array_equal(R, givens_matrix(5, 0))
    assert np.allclose(cur, x @ givens_matrix(5, 0), atol=1e-15)


def test_brute_force_candidate_choice():
    """One step chooses the candidate an explicit enumeration of all 31
    rotation matrices (dense NumPy products) finds best."""
    rng = np.random.default_rng(3)
    for trial in range(20):
        x = rng.standard_normal((7, GROUP)) * np.exp(rng.standard_normal(GROUP))
        d = int(np.argmax(np.abs(x).max(axis=0)))
        norms = [(np.abs(x @ givens_matrix(d, j)).max(), j) for j in range(GROUP) if j != d]
        best_norm, best_j = min(norms)
        R, cur, hist, pairs = CAL.greedy_givens(x, steps=1)
        if best_norm > np.abs(x).max():
            assert pairs == []
            continue
        assert pairs == [(d, best_j)], trial
        assert abs(hist[1] - best_norm) <= 1e-14 * best_norm


def test_invariants_over_a_full_search():
    rng = np.random.default_rng(5)
    x = rng.standard_t(3, size=(300, GROUP))
    x[rng.integers(0, 300, 6), 11] = rng.choice([-1, 1], 6) * rng.uniform(50, 100, 6)
    R, cur, hist, pairs = CAL.greedy_givens(x, steps=128)
    # orthogonal, and x R reproduces the transformed block (dense product)
    assert np.abs(R @ R.T - np.eye(GROUP)).max() < 1e-13
    assert np.abs(x @ R - cur).max() <= 1e-12 * np.abs(x).max()
    # the norm never increases, and is recorded per step taken
    assert np.all(np.diff(hist) <= 0)
    assert len(hist) == len(pairs) + 1
    assert abs(hist[-1] - np.abs(cur).max()) == 0
    # rows keep their length, so the maximum cannot fall below max ||x_t|| / sqrt(32)
    assert hist[-1] >= np.linalg.norm(x, axis=1).max() / math.sqrt(GROUP) * (1 - 1e-12)
    # the planted outlier dimension was spread: the norm dropped a lot
    assert hist[-1] < 0.5 * hist[0]
    assert pairs[0][0] == 11


def test_flat_block_stops_immediately():
    """Rows of a Hadamard block have all entries of equal size: every pi/4
    rotation of two columns doubles some entries' squares, so no step is taken."""
    h = W.sylvester_hadamard(GROUP) / math.sqrt(GROUP)
    R, cur, hist, pairs = CAL.greedy_givens(h, steps=128)
    assert pairs == [] and np.array_equal(R, np.eye(GROUP)) and len(hist) == 1


def test_zero_block_takes_no_step():
    R, cur, hist, pairs = CAL.greedy_givens(np.zeros((3, GROUP)), steps=10)
    assert pairs == [] and hist.tolist() == [0.0]


def test_worst_group_with_and_without_lambda():
    x = np.zeros((5, 128))
    x[1, 40] = 9.0     # group 1
    x[3, 100] = 6.0    # group 3
    g, linf, xw = CAL.worst_group(x)
    assert g == 1 and linf == 9.0 and xw.shape == (5, GROUP) and xw[1, 8] == 9.0
    lam = np.ones(128, np.float32)
    lam[40] = 4.0      # 9/4 < 6: group 3 wins after smoothing
    g, linf, xw = CAL.worst_group(x, lam)
    assert g == 3 and linf == 6.0
    x[2, 70] = 9.0     # tie with group 1 without lambda: lowest index
    g, _, _ = CAL.worst_group(x)
    assert g == 1


@pytest.mark.parametrize("n", [16, 64, 128])
def test_other_block_widths(n):
    """The search at the ablation's block widths (DuQuant++ page sec. 4.3):
    one step picks the candidate an explicit enumeration finds best, a flat
    Hadamard block takes no step, and the worst block is found at width n."""
    rng = np.random.default_rng(60 + n)
    x = rng.standard_normal((9, n)) * np.exp(rng.standard_normal(n))
    d = int(np.argmax(np.abs(x).max(axis=0)))
    norms = [(np.abs(x @ givens_matrix(d, j, n)).max(), j) for j in range(n) if j != d]
    best_norm, best_j = min(norms)
    R, cur, hist, pairs = CAL.greedy_givens(x, steps=1)
    assert R.shape == (n, n)
    if best_norm <= np.abs(x).max():
        assert pairs == [(d, best_j)]
    h = W.sylvester_hadamard(n) / math.sqrt(n)
    _, _, _, pairs = CAL.greedy_givens(h, steps=8)
    assert pairs == []
    big = np.zeros((3, 4 * n))
    big[1, 2 * n + 5] = 7.0
    g, linf, xw = CAL.worst_group(big, block=n)
    assert g == 2 and linf == 7.0 and xw.shape == (3, n)
