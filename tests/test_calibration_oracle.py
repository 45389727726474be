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


# ---- second reading: a per-candidate angle ----------------------------------

def givens_theta(d, j, theta, n=GROUP):
    """Dense rotation by theta in the (d, j) plane, from np.cos / np.sin:
    x G maps (x_d, x_j) to (cos x_d - sin x_j, sin x_d + cos x_j)."""
    c, s = math.cos(theta), math.sin(theta)
    g = np.eye(n)
    g[d, d] = c
    g[j, d] = -s
    g[d, j] = s
    g[j, j] = c
    return g


def grid_angles(grid):
    """The grid's angles from the half-angle tangent, by np.arctan."""
    return [math.pi / 4] + [2.0 * math.atan(k / grid) for k in range(1, grid)]


@pytest.mark.parametrize("grid", [2, 16, 64, 1024])
def test_angle_table_matches_trigonometry(grid):
    """The exact-integer ratios are cos and sin of the grid angles (the
    half-angle tangent substitution), to the last bit or two."""
    table = CAL.angle_table(grid)
    assert len(table) == grid
    for (c, s), th in zip(table, grid_angles(grid)):
        assert abs(c - math.cos(th)) <= 3e-16 and abs(s - math.sin(th)) <= 3e-16
        assert abs(c * c + s * s - 1.0) <= 4.5e-16
        assert 0.0 < th < math.pi / 2 and c > 0.0 and s > 0.0
    # the grid spans (0, pi/2) with no gap wider than 2 / grid
    th = np.sort(grid_angles(grid))
    gaps = np.diff(np.concatenate([[0.0], th, [math.pi / 2]]))
    assert gaps.max() <= 2.0 / grid + 1e-15
    with pytest.raises(ValueError):
        CAL.angle_table(0)
    with pytest.raises(ValueError):
        CAL.angle_table(CAL.MAX_ANGLE_GRID + 1)


def test_angle_brute_force_one_step():
    """One step of the second reading picks the (j, angle) that an explicit
    enumeration of every dense rotation matrix (built from np.cos / np.sin)
    finds best."""
    rng = np.random.default_rng(71)
    grid = 16
    th = grid_angles(grid)
    for trial in range(12):
        x = rng.standard_normal((6, GROUP)) * np.exp(rng.standard_normal(GROUP))
        d = int(np.argmax(np.abs(x).max(axis=0)))
        norms = sorted((np.abs(x @ givens_theta(d, j, t)).max(), j, a)
                       for j in range(GROUP) if j != d for a, t in enumerate(th))
        R, cur, hist, steps = CAL.greedy_givens_angle(x, steps=1, grid=grid)
        best = norms[0][0]
        assert steps, trial  # some small angle always lowers a unique maximum
        assert steps[0][0] == d
        assert abs(hist[1] - best) <= 1e-13 * best
        if norms[1][0] - best > 1e-12 * best:  # a clear winner: same candidate
            assert steps[0][1:] == norms[0][1:], trial
        # the step's rotation, rebuilt densely, reproduces the block and R
        G = givens_theta(d, steps[0][1], th[steps[0][2]])
        assert np.abs(R - G).max() <= 4e-16
        assert np.abs(cur - x @ G).max() <= 1e-14 * np.abs(x).max()


def test_angle_near_the_continuous_optimum():
    """Against a dense scan of theta over [0, pi/2) with trigonometry: the
    norm the second reading reaches in one step is never below the scan's
    minimum and at most r_max / M above it (the norm moves at most r_max per
    radian, r_max the largest length of a (x_d, x_j) pair; grid gaps are at
    most 2 / M), and well below the pi/4 reading's one-step norm on data
    whose best angle is far from pi/4."""
    rng = np.random.default_rng(72)
    grid = 64
    thetas = np.linspace(0.0, math.pi / 2, 20001)[:-1]
    c, s = np.cos(thetas)[:, None], np.sin(thetas)[:, None]
    for trial in range(6):
        x = rng.standard_normal((9, GROUP))
        x[:, 7] *= 6.0
        x[:, 20] = 0.3 * x[:, 7] + 0.2 * rng.standard_normal(9)  # correlated partner
        d = int(np.argmax(np.abs(x).max(axis=0)))
        colmax = np.abs(x).max(axis=0)
        scan_min, r_max = np.inf, 0.0
        for j in range(GROUP):
            if j == d:
                continue
            rest = np.delete(colmax, [d, j]).max()
            nd = np.abs(c * x[:, d] - s * x[:, j]).max(axis=1)
            nj = np.abs(s * x[:, d] + c * x[:, j]).max(axis=1)
            scan_min = min(scan_min, np.maximum(np.maximum(nd, nj), rest).min())
            r_max = max(r_max, np.hypot(x[:, d], x[:, j]).max())
        step_err = r_max * (math.pi / 2) / 20000
        _, _, hist, steps = CAL.greedy_givens_angle(x, steps=1, grid=grid)
        assert scan_min - step_err <= hist[1] <= scan_min + r_max / grid, trial
        _, _, hist_a, _ = CAL.greedy_givens(x, steps=1)
        assert hist[1] <= hist_a[1]


def test_angle_single_outlier_closed_form():
    """One nonzero entry v: a rotation by theta leaves max(|cos|, |sin|) v,
    smallest at pi/4 (v / sqrt 2), which is angle index 0 for every
    candidate; the lowest partner wins the tie."""
    x = np.zeros((3, GROUP))
    x[1, 9] = -5.0
    R, cur, hist, steps = CAL.greedy_givens_angle(x, steps=1, grid=64)
    assert steps == [(9, 0, 0)]
    assert abs(hist[1] - 5.0 / math.sqrt(2.0)) <= 1e-15 * 5.0


def test_angle_pair_closed_form():
    """A block of two columns and one token (31, 17): its length is 25 sqrt 2
    and a rotation leaves 25 sqrt 2 max(|cos(phi + theta)|, |sin(phi + theta)|),
    smallest (25) where the two magnitudes meet.  That angle has
    tan(theta / 2) = 1/7 (c = 24/25, s = 7/25 map (31, 17) to (25, 25)), so
    with M = 7 the grid's index 1 lands on it; with M = 8 it does not, and the
    best grid angle is within the r_max / M bound."""
    x = np.array([[31.0, 17.0]])
    R, cur, hist, steps = CAL.greedy_givens_angle(x, steps=1, grid=7)
    assert steps == [(0, 1, 1)]
    assert abs(hist[1] - 25.0) <= 4e-15 * 25.0
    assert np.abs(cur - 25.0).max() <= 4e-15 * 25.0
    R, cur, hist, steps = CAL.greedy_givens_angle(x, steps=1, grid=8)
    assert 25.0 < hist[1] <= 25.0 + 25.0 * math.sqrt(2.0) / 8
    dense = min(np.abs(x @ givens_theta(0, 1, t, n=2)).max() for t in grid_angles(8))
    assert abs(hist[1] - dense) <= 1e-14 * dense


def test_angle_ties_go_to_the_first_candidate():
    """When two other columns hold 9.9, no single step can go below 9.9:
    every candidate ties there for all angles that bring the (d, j) pair
    under it, and the rule takes the lowest j, then pi/4 (index 0)."""
    x = np.zeros((3, GROUP))
    x[0, 5], x[1, 10], x[2, 20] = 10.0, 9.9, -9.9
    R, cur, hist, steps = CAL.greedy_givens_angle(x, steps=1, grid=64)
    assert steps == [(5, 0, 0)] and hist[1] == 9.9


def test_angle_invariants_over_a_full_search():
    rng = np.random.default_rng(73)
    x = rng.standard_t(3, size=(200, GROUP))
    x[rng.integers(0, 200, 6), 11] = rng.choice([-1, 1], 6) * rng.uniform(50, 100, 6)
    R, cur, hist, steps = CAL.greedy_givens_angle(x, steps=128, grid=32)
    assert np.abs(R @ R.T - np.eye(GROUP)).max() < 1e-13
    assert np.abs(x @ R - cur).max() <= 1e-12 * np.abs(x).max()
    assert np.all(np.diff(hist) <= 0)
    assert len(hist) == len(steps) + 1 and hist[-1] == np.abs(cur).max()
    assert hist[-1] >= np.linalg.norm(x, axis=1).max() / math.sqrt(GROUP) * (1 - 1e-12)
    assert all(0 <= a < 32 for _, _, a in steps)
    # small angles keep lowering a unique maximum, so the search runs longer
    # than the pi/4 reading's (31 steps on this block); given the steps, the
    # coarse grid of M = 8 ends lower
    _, _, hist_a, pairs_a = CAL.greedy_givens(x, steps=128)
    assert len(steps) > len(pairs_a)
    _, _, hist8, steps8 = CAL.greedy_givens_angle(x, steps=512, grid=8)
    assert len(steps8) < 512 and hist8[-1] < hist_a[-1]


def test_angle_grid_one_is_the_first_reading():
    """With the grid cut to pi/4 alone the two readings coincide bit for bit
    (a consistency check of the two code paths, not an outside pin)."""
    rng = np.random.default_rng(74)
    x = rng.standard_t(4, size=(50, GROUP))
    R1, cur1, hist1, pairs1 = CAL.greedy_givens(x, steps=64)
    R2, cur2, hist2, steps2 = CAL.greedy_givens_angle(x, steps=64, grid=1)
    assert pairs1 == [(d, j) for d, j, _ in steps2] and all(a == 0 for _, _, a in steps2)
    assert np.array_equal(hist1, hist2) and np.array_equal(R1, R2) and np.array_equal(cur1, cur2)


def test_angle_flat_and_zero_blocks():
    h = W.sylvester_hadamard(GROUP) / math.sqrt(GROUP)
    # every column holds the maximum in every row: no rotation of two columns
    # can lower it, and pi/4 (the tie-order first) raises it the least; the
    # search still stops because all candidates raise the norm
    R, cur, hist, steps = CAL.greedy_givens_angle(h, steps=16, grid=64)
    assert steps == [] and np.array_equal(R, np.eye(GROUP))
    R, cur, hist, steps = CAL.greedy_givens_angle(np.zeros((3, GROUP)), steps=8)
    assert steps == [] and hist.tolist() == [0.0]
