"""fp64 reference of the offline calibration of the shared rotation block.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``).  Follows the greedy
search of the DuQuant++ page, sec. 3.2 ("constructing the outlier-aware
block-diagonal rotation"), in the page's order, with the page's advice to
search in double precision (sec. 3 pitfalls, item 3):

1. worst group: over all 32-channel groups of the (smoothed, sec. 5.1 item 3)
   calibration activations X' = X / Lambda, the group whose tokens x 32 slice
   has the largest absolute value; that slice is X_worst;
2. start from the 32x32 identity;
3. for at most ``steps`` steps (the page uses 128):
   a. d = the dimension (column of X_worst) holding the largest |value|;
   b. for every other dimension j, the Givens rotation mixing d and j;
   c. the L-infinity norm of X_worst times each candidate;
   d. keep the candidate with the smallest norm;
   e. R <- R * G;  f. X_worst <- X_worst * G.
4. R is then shared by every group (BlockDiag(R, ..., R)).

Readings where the page is silent (listed in the design notes too):
* a Givens rotation by theta maps, in the row-vector convention, (x_d, x_j)
  to (c x_d - s x_j, s x_d + c x_j) with c = cos theta, s = sin theta;
* the angle, first reading (``greedy_givens``): pi/4 for every candidate
  (equal mixing of the two dimensions, c = s = sqrt(1/2));
* the angle, second reading (``greedy_givens_angle``): each candidate j also
  picks, from a fixed grid, the angle that leaves the smallest L-infinity
  norm, so "the rotation that lowers the norm the most" ranges over pairs
  and angles.  The norm is periodic in theta with period pi/2 (a quarter
  turn only swaps the two columns' magnitudes), so the grid covers
  (0, pi/2): pi/4 first, then the angles with tan(theta / 2) = k / M,
  k = 1 .. M - 1.  Through the half-angle tangent t, c = (1 - t^2) / (1 + t^2)
  and s = 2 t / (1 + t^2), so c = (M^2 - k^2) / (M^2 + k^2) and
  s = 2 k M / (M^2 + k^2) are single correctly rounded divisions of exact
  integers: no trigonometric function is needed (the page's stability
  advice, sec. 3 pitfalls item 3, is met by building the matrix in fp64);
* ties: d is the lowest column holding the maximum, the chosen j the lowest
  index among equally good candidates (then the earliest angle of the grid),
  the worst group the lowest index;
* a step is taken while the best candidate does not raise the norm; the
  search stops early when every candidate would raise it, or when X_worst is
  all zero.

Every product, sum and difference is an fp64 operation written out in
NumPy (no fused multiply-add), in the order stated here.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 32
C = S = math.sqrt(0.5)


def smoothed(x, lam=None) -> np.ndarray:
    """X' = X / Lambda in fp64 (exact upcast of bf16/fp16/fp32 input)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    xs = np.asarray(x, dtype=np.float64)
    if lam is not None:
        xs = xs / np.asarray(lam, dtype=np.float64)[None, :]
    return xs


def worst_group(x, lam=None, block: int = GROUP):
    """(group index, its L-infinity norm, X_worst [T, block] fp64).  ``block``
    is the rotation block width (32 on the page's main path; 16, 64 and 128
    in its block-size ablation, sec. 4.3)."""
    xs = smoothed(x, lam)
    T, Cn = xs.shape
    per_group = np.abs(xs).reshape(T, Cn // block, block).max(axis=(0, 2))
    g = int(np.argmax(per_group))  # first index among ties
    return g, float(per_group[g]), np.ascontiguousarray(xs[:, g * block:(g + 1) * block])


def greedy_givens(x_worst, steps: int = 128):
    """Greedy outlier-aware search.  Returns (R [n, n], X_worst * R, norm
    history [steps_done + 1], chosen pairs [(d, j)]), n = X_worst's width."""
    cur = np.array(x_worst, dtype=np.float64, copy=True)
    n = cur.shape[1]
    R = np.eye(n)
    colmax = np.abs(cur).max(axis=0) if cur.shape[0] else np.zeros(n)
    linf = float(colmax.max())
    history = [linf]
    pairs = []
    for _ in range(steps):
        if linf == 0.0:
            break
        d = int(np.argmax(colmax))
        xd = cur[:, d]
        best = None
        for j in range(n):
            if j == d:
                continue
            xj = cur[:, j]
            new_d = C * xd - S * xj
            new_j = S * xd + C * xj
            m_d = float(np.abs(new_d).max())
            m_j = float(np.abs(new_j).max())
            rest = max([float(colmax[k]) for k in range(n) if k != d and k != j], default=0.0)
            norm = max(m_d, m_j, rest)
            if best is None or norm < best[0]:
                best = (norm, j, m_d, m_j, new_d, new_j)
        norm, j, m_d, m_j, new_d, new_j = best
        if norm > linf:
            break
        cur[:, d] = new_d
        cur[:, j] = new_j
        r_d = C * R[:, d] - S * R[:, j]
        r_j = S * R[:, d] + C * R[:, j]
        R[:, d] = r_d
        R[:, j] = r_j
        colmax[d] = m_d
        colmax[j] = m_j
        linf = float(colmax.max())
        history.append(linf)
        pairs.append((d, j))
    return R, cur, np.array(history), pairs


MAX_ANGLE_GRID = 1024


def angle_table(grid: int):
    """(c, s) of the second reading's candidate angles, in tie order: index 0
    is pi/4, index k (1 <= k < grid) the angle with tan(theta / 2) = k / grid.
    ``grid`` = 1 leaves pi/4 alone (the first reading's single angle)."""
    if not 1 <= grid <= MAX_ANGLE_GRID:
        raise ValueError("angle grid must be in [1, %d]" % MAX_ANGLE_GRID)
    table = [(C, S)]
    for k in range(1, grid):
        den = float(grid * grid + k * k)          # exact: below 2^53
        table.append((float(grid * grid - k * k) / den, float(2 * k * grid) / den))
    return table


def greedy_givens_angle(x_worst, steps: int = 128, grid: int = 64):
    """Greedy outlier-aware search, second reading: every candidate pair
    (d, j) also chooses its angle from ``angle_table(grid)``.  Returns
    (R [n, n], X_worst * R, norm history [steps_done + 1], chosen steps
    [(d, j, angle index)])."""
    table = angle_table(grid)
    cvec = np.array([c for c, _ in table])[:, None]
    svec = np.array([s for _, s in table])[:, None]
    cur = np.array(x_worst, dtype=np.float64, copy=True)
    n = cur.shape[1]
    R = np.eye(n)
    colmax = np.abs(cur).max(axis=0) if cur.shape[0] else np.zeros(n)
    linf = float(colmax.max())
    history = [linf]
    chosen = []
    for _ in range(steps):
        if linf == 0.0:
            break
        d = int(np.argmax(colmax))
        xd = cur[:, d][None, :]
        best = None
        for j in range(n):
            if j == d:
                continue
            xj = cur[:, j][None, :]
            # one row per candidate angle; each product and difference is a
            # separately rounded fp64 operation, as in the first reading
            new_d = cvec * xd - svec * xj
            new_j = svec * xd + cvec * xj
            m_d = np.abs(new_d).max(axis=1)
            m_j = np.abs(new_j).max(axis=1)
            rest = max([float(colmax[k]) for k in range(n) if k != d and k != j], default=0.0)
            norms = np.maximum(np.maximum(m_d, m_j), rest)
            a = int(np.argmin(norms))              # earliest angle among ties
            if best is None or norms[a] < best[0]:
                best = (float(norms[a]), j, a, float(m_d[a]), float(m_j[a]))
        norm, j, a, m_d, m_j = best
        if norm > linf:
            break
        c, s = table[a]
        xd1, xj1 = cur[:, d].copy(), cur[:, j].copy()
        cur[:, d] = c * xd1 - s * xj1
        cur[:, j] = s * xd1 + c * xj1
        r_d = c * R[:, d] - s * R[:, j]
        r_j = s * R[:, d] + c * R[:, j]
        R[:, d] = r_d
        R[:, j] = r_j
        colmax[d] = m_d
        colmax[j] = m_j
        linf = float(colmax.max())
        history.append(linf)
        chosen.append((d, j, a))
    return R, cur, np.array(history), chosen
