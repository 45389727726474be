"""GPU calibration of the shared block (DuQuant++ page sec. 3.2) against the
fp64 oracle: every decision and every fp64 value bit for bit."""
import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq
import workloads as W
from oracle import calibration as CAL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    mxq.load()
    return torch.device("cuda:0")


def gpu_search(x, lam, steps, dev):
    xd = x.to(dev)
    lam_d = None if lam is None else torch.from_numpy(np.ascontiguousarray(lam, np.float32)).to(dev)
    xw, g, linf = mxq.calib_worst_group(xd, lam_d)
    xw0 = xw.clone()
    R, hist, done, pairs = mxq.calib_givens(xw, steps)
    torch.cuda.synchronize()
    n = int(done)
    return (int(g), float(linf), xw0.cpu().numpy(), R.cpu().numpy(), xw.cpu().numpy(),
            hist.cpu().numpy()[: n + 1], [tuple(p) for p in pairs.cpu().numpy()[:n].tolist()])


def check_against_oracle(x, lam, steps, dev):
    g, linf, xw0, R, cur, hist, pairs = gpu_search(x, lam, steps, dev)
    g_o, linf_o, xw_o = CAL.worst_group(x, lam)
    assert g == g_o and linf == linf_o
    assert np.array_equal(xw0, xw_o)
    R_o, cur_o, hist_o, pairs_o = CAL.greedy_givens(xw_o, steps)
    assert pairs == pairs_o
    assert np.array_equal(hist, hist_o)
    assert np.array_equal(R, R_o)
    assert np.array_equal(cur, cur_o)
    print(f"  group {g}, steps {len(pairs)}, L_inf {hist_o[0]:.4g} -> {hist_o[-1]:.4g}", flush=True)
    return R


def test_config3_calibration_slice(dev):
    wl = W.make_config(3)
    s = wl.meta["calib_start"]
    check_against_oracle(wl.x[s:s + 256].contiguous(), None, 128, dev)


def test_config5_calibration_slice_smoothed(dev):
    wl = W.make_config(5)
    s = wl.meta["calib_start"]
    check_against_oracle(wl.x[s:s + 512].contiguous(), wl.lam, 128, dev)


def test_large_calibration_set(dev):
    wl = W.make_config(3)
    check_against_oracle(wl.x[:4096].contiguous(), None, 128, dev)


def test_page_scale_block(dev):
    """128 sequences x 2048 tokens of one 32-channel group (the page's
    calibration size, sec. 3 pitfalls item 1), fed to the search directly."""
    xw = W.calibration_block()
    t = torch.from_numpy(xw).to(dev)
    R, hist, done, pairs = mxq.calib_givens(t, 128)
    torch.cuda.synchronize()
    R_o, cur_o, hist_o, pairs_o = CAL.greedy_givens(xw, 128)
    n = int(done)
    assert [tuple(p) for p in pairs.cpu().numpy()[:n].tolist()] == pairs_o
    assert np.array_equal(hist.cpu().numpy()[: n + 1], hist_o)
    assert np.array_equal(R.cpu().numpy(), R_o)
    assert np.array_equal(t.cpu().numpy(), cur_o)


@pytest.mark.parametrize("case", ["fp32_one_token", "zero", "fp16_ragged", "flat"])
def test_calibration_edge_cases(dev, case):
    rng = np.random.default_rng(13)
    if case == "fp32_one_token":
        x = torch.from_numpy(rng.standard_normal((1, 96)).astype(np.float32))
        check_against_oracle(x, None, 40, dev)
    elif case == "zero":
        R = check_against_oracle(torch.zeros((8, 64), dtype=torch.bfloat16), None, 16, dev)
        assert np.array_equal(R, np.eye(32))
    elif case == "fp16_ragged":
        x = torch.from_numpy((rng.standard_normal((37, 160)) * 3).astype(np.float16))
        lam = np.exp(0.3 * rng.standard_normal(160)).astype(np.float32)
        check_against_oracle(x, lam, 128, dev)
    else:
        h = torch.from_numpy(np.tile(W.sylvester_hadamard(32), (2, 1)).astype(np.float32))
        R = check_against_oracle(h, None, 8, dev)
        assert np.array_equal(R, np.eye(32))


# ---- second reading: a per-candidate angle from a grid ----------------------

def check_angles_against_oracle(xw_np, steps, grid, dev):
    t = torch.from_numpy(np.ascontiguousarray(xw_np)).to(dev)
    R, hist, done, pairs, angles = mxq.calib_givens_angles(t, steps, grid)
    torch.cuda.synchronize()
    n = int(done)
    R_o, cur_o, hist_o, steps_o = CAL.greedy_givens_angle(xw_np, steps, grid)
    got = [(int(p[0]), int(p[1]), int(a)) for p, a in zip(pairs.cpu().numpy()[:n], angles.cpu().numpy()[:n])]
    assert got == steps_o
    assert np.array_equal(hist.cpu().numpy()[: n + 1], hist_o)
    assert np.array_equal(R.cpu().numpy(), R_o)
    assert np.array_equal(t.cpu().numpy(), cur_o)
    print(f"  grid {grid}: steps {n}, L_inf {hist_o[0]:.4g} -> {hist_o[-1]:.4g}", flush=True)
    return R.cpu().numpy(), n


@pytest.mark.parametrize("grid", [1, 8, 64])
def test_angles_config3_slice(dev, grid):
    wl = W.make_config(3)
    s, n = wl.meta["calib_start"], wl.meta["calib_len"]
    _, _, xw = CAL.worst_group(wl.x[s:s + n], None)
    check_angles_against_oracle(xw, 128, grid, dev)


@pytest.mark.parametrize("grid", [8, 64, 1024])
def test_angles_config5_slice_smoothed(dev, grid):
    wl = W.make_config(5)
    s, n = wl.meta["calib_start"], wl.meta["calib_len"]
    _, _, xw = CAL.worst_group(wl.x[s:s + n], wl.lam)
    check_angles_against_oracle(xw, 128 if grid < 1024 else 16, grid, dev)


def test_angles_grid_one_is_the_pi4_search(dev):
    """M = 1 through the angle kernels gives what the pi/4 kernels give."""
    wl = W.make_config(3)
    xw = torch.from_numpy(np.ascontiguousarray(CAL.worst_group(wl.x[:2048], None)[2])).to(dev)
    a = xw.clone()
    R1, h1, d1, p1 = mxq.calib_givens(xw, 128)
    R2, h2, d2, p2, ang = mxq.calib_givens_angles(a, 128, 1)
    torch.cuda.synchronize()
    n = int(d1)
    assert n == int(d2) and torch.equal(R1, R2) and torch.equal(xw, a)
    assert torch.equal(h1[: n + 1], h2[: n + 1]) and torch.equal(p1[:n], p2[:n])
    assert int(ang[:n].abs().sum()) == 0


def test_angles_large_set(dev):
    wl = W.make_config(3)
    _, _, xw = CAL.worst_group(wl.x[:2048], None)
    check_angles_against_oracle(xw, 128, 64, dev)


def test_angles_page_scale_block(dev):
    """The 262,144-token block: the first two steps bit for bit against the
    oracle, then the full 128-step search checked by what holds at any size
    (orthogonal R, the block equal to x R, a never-increasing history whose
    last entry is the block's largest |value|)."""
    xw = W.calibration_block()
    check_angles_against_oracle(xw, 2, 16, dev)
    t = torch.from_numpy(xw).to(dev)
    R, hist, done, pairs, angles = mxq.calib_givens_angles(t, 128, 64)
    torch.cuda.synchronize()
    n = int(done)
    R, hist, cur = R.cpu().numpy(), hist.cpu().numpy()[: n + 1], t.cpu().numpy()
    assert np.abs(R @ R.T - np.eye(32)).max() < 1e-13
    assert np.abs(xw @ R - cur).max() <= 1e-12 * np.abs(xw).max()
    assert np.all(np.diff(hist) <= 0) and hist[-1] == np.abs(cur).max()
    a = angles.cpu().numpy()[:n]
    assert n > 0 and a.min() >= 0 and a.max() < 64
    print(f"  page scale, grid 64: steps {n}, L_inf {hist[0]:.4g} -> {hist[-1]:.4g}", flush=True)


@pytest.mark.parametrize("case", ["fp32_one_token", "zero", "fp16_ragged", "flat"])
def test_angles_edge_cases(dev, case):
    rng = np.random.default_rng(17)
    if case == "fp32_one_token":
        xw = CAL.worst_group(rng.standard_normal((1, 96)).astype(np.float32))[2]
        check_angles_against_oracle(xw, 40, 64, dev)
    elif case == "zero":
        R, n = check_angles_against_oracle(np.zeros((8, 32)), 16, 64, dev)
        assert n == 0 and np.array_equal(R, np.eye(32))
    elif case == "fp16_ragged":
        x = torch.from_numpy((rng.standard_normal((37, 160)) * 3).astype(np.float16))
        lam = np.exp(0.3 * rng.standard_normal(160)).astype(np.float32)
        check_angles_against_oracle(CAL.worst_group(x, lam)[2], 128, 33, dev)
    else:
        h = np.tile(W.sylvester_hadamard(32), (2, 1)).astype(np.float64)
        R, n = check_angles_against_oracle(h, 8, 64, dev)
        assert n == 0 and np.array_equal(R, np.eye(32))
