"""Comparison of the HIP path against the fp64 oracle.

Rules (the fused path computes the rotation in fp32 on the matrix cores, the
oracle in fp64, so an integer decision can differ only where the exact value
sits on a decision boundary):

* rotated values: |y_gpu - y*| <= 1e-5 * ||x'_g||_2 + 2^-149 for every
  element of group g (x' = x / lambda), an absolute bound per group because a
  purely relative bound fails on cancellation; 2^-149, fp32's smallest
  subnormal, is what an fp32 output cannot resolve (groups far below fp32's
  normal range);
* same-precision decisions: the oracle's encoder applied to the GPU's own
  fp32 rotated values reproduces the GPU's codes and scales bit for bit,
  except in groups with a scale byte below 61 (a rotated maximum below
  2^-64) that hold fp32 subnormal outputs: the kernel decides those groups on
  values 2^k times larger, of which the subnormal outputs are roundings;
* against the oracle's fp64 decisions: at most 1e-4 of the scales and 1e-4
  of the codes differ; a differing scale is one E8M0 step away and the
  oracle's group maximum lies within 1e-5 * ||x'_g|| of the power of two that
  separates the two exponents; a differing code (compared under the GPU's
  scale) is one step away on the signed E2M1 grid and the oracle's value lies
  within 1e-5 * ||x'_g|| of the midpoint between the two code values.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

GROUP = 32
TOL = 1e-5
MAX_RATE = 1e-4
FP32_FLOOR = 2.0 ** -149  # smallest fp32 subnormal
TINY_SCALE = 61           # scale byte of a group maximum 2^-64

# signed E2M1 grid in increasing order, with 0 and -0 as one point
_SIGNED = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _grid_index(codes):
    v = O.code_value(codes)
    return np.searchsorted(_SIGNED, v)


def smoothed_group_norms(x: torch.Tensor, lam) -> np.ndarray:
    """||x'_g||_2 in fp64 for every group, x' = x / lam, shape [T, C/32]."""
    xs = x.to(torch.float64).numpy()
    if lam is not None:
        xs = xs / np.asarray(lam, dtype=np.float64)[None, :]
    T, C = xs.shape
    return np.sqrt((xs.reshape(T, C // GROUP, GROUP) ** 2).sum(axis=2))


def check_rotated_values(y_gpu: np.ndarray, y_ref: np.ndarray, norms: np.ndarray):
    T, C = y_ref.shape
    err = np.abs(y_gpu.astype(np.float64) - y_ref).reshape(T, C // GROUP, GROUP).max(axis=2)
    bound = TOL * norms + FP32_FLOOR
    bad = err > bound
    worst = float(np.max(err / np.maximum(norms, 1e-300)))
    assert not bad.any(), f"{int(bad.sum())} groups exceed 1e-5*||x'_g||; worst ratio {worst:.3e}"
    return worst


def check_same_precision(y_gpu: np.ndarray, codes: np.ndarray, scales: np.ndarray, orc=None):
    orc = orc or O.default()
    T, C = y_gpu.shape
    yg = y_gpu.astype(np.float64).reshape(-1, GROUP)
    c_ref, s_ref = orc.encode_groups(yg)
    keep = ~((scales.reshape(-1) < TINY_SCALE) & ((yg != 0) & (np.abs(yg) < 2.0 ** -126)).any(axis=1))
    s_ref, s_got = s_ref.reshape(-1)[keep], scales.reshape(-1)[keep]
    c_ref, c_got = c_ref.reshape(-1, GROUP // 2)[keep], codes.reshape(-1, GROUP // 2)[keep]
    assert np.array_equal(s_ref, s_got), "scales differ from oracle(y_gpu)"
    assert np.array_equal(c_ref, c_got), "codes differ from oracle(y_gpu)"
    return int((~keep).sum())


def check_against_oracle(codes, scales, c_ref, s_ref, y_ref_rows, norms):
    """Tie-aware comparison.  ``y_ref_rows(rows)`` returns the oracle's fp64
    rotated values [len(rows), C] for the requested token rows (so large
    workloads only recompute rows that hold a mismatch)."""
    T, half = codes.shape
    C = half * 2
    G = T * (C // GROUP)
    stats = {"groups": G, "scale_mismatch": 0, "code_mismatch": 0}
    s_bad = np.argwhere(scales != s_ref)
    u = O.unpack_codes(codes).reshape(T, C // GROUP, GROUP)
    u_ref = O.unpack_codes(c_ref).reshape(T, C // GROUP, GROUP)
    same_scale = (scales == s_ref)[:, :, None]
    c_bad = np.argwhere((u != u_ref) & same_scale)
    rows = np.unique(np.concatenate([s_bad[:, 0], c_bad[:, 0]]).astype(np.int64))
    stats["scale_mismatch"] = int(len(s_bad))
    if rows.size == 0:
        return stats
    yr = y_ref_rows(rows)
    row_pos = {int(r): i for i, r in enumerate(rows)}
    n_code_bad = 0
    for t, g in s_bad:
        sg, so = int(scales[t, g]), int(s_ref[t, g])
        assert abs(sg - so) == 1, f"scale {sg} vs oracle {so} at ({t},{g})"
        ys = yr[row_pos[int(t)], g * GROUP:(g + 1) * GROUP]
        edge = np.ldexp(1.0, max(sg, so) - 127 + 2)
        amax = np.abs(ys).max()
        assert abs(amax - edge) <= TOL * norms[t, g], f"scale flip at ({t},{g}) not at a boundary"
        # codes of this group compared under the GPU's scale
        expect = O.brute_force_codes(np.ldexp(ys, -(sg - 127)))
        got = u[t, g]
        for n in np.nonzero(got != expect)[0]:
            _check_code_step(int(got[n]), int(expect[n]), ys[n], sg, norms[t, g], (t, g, n))
            n_code_bad += 1
    for t, g, n in c_bad:
        ys = yr[row_pos[int(t)], g * GROUP + n]
        _check_code_step(int(u[t, g, n]), int(u_ref[t, g, n]), ys, int(scales[t, g]), norms[t, g], (t, g, n))
        n_code_bad += 1
    stats["code_mismatch"] = n_code_bad
    assert stats["scale_mismatch"] <= MAX_RATE * G, stats
    assert stats["code_mismatch"] <= MAX_RATE * G * GROUP, stats
    return stats


def _check_code_step(cg, co, y, S, norm, where):
    ig, io = _grid_index(np.array([cg]))[0], _grid_index(np.array([co]))[0]
    assert abs(int(ig) - int(io)) == 1, f"code {cg:#x} vs oracle {co:#x} not adjacent at {where}"
    mid = 0.5 * (_SIGNED[ig] + _SIGNED[io])
    boundary = np.ldexp(mid, S - 127)
    assert abs(y - boundary) <= TOL * norm, f"code flip at {where} is {abs(y - boundary):.3e} from the boundary"
