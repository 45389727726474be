"""Rotation block sizes 16 / 32 / 64 / 128 (DuQuant++ page sec. 4.3) on an
MI355X through the C ABI, against the fp64 oracle, and the quantization
error study across block sizes and block kinds.

The tolerance rule is the plain path's, with the norm of each element's
whole rotation block as the scale (an output of a B-block sums B products,
so its rounding error scales with the block's norm; for B = 16 the norm of
the 32-wide group, which holds two blocks)."""
import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq
import oracle as O
import workloads as W
from parity import check_against_oracle, check_rotated_values, check_same_precision

pytestmark = pytest.mark.gpu
GROUP = 32


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mxq.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return O.default()


def _lam_dev(lam, dev):
    return None if lam is None else torch.from_numpy(np.ascontiguousarray(lam, np.float32)).to(dev)


def run_block(x, lam, r, dev, want_y=True):
    y = torch.empty(x.shape, dtype=torch.float32, device=dev) if want_y else None
    codes, scales = mxq.rotate_quant_block(x.to(dev), r.contiguous().to(dev), _lam_dev(lam, dev), y_rot=y)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (y.cpu().numpy() if want_y else None)


def block_norms(y, B):
    """Per 32-wide group: the norm of the rotation block that produced it."""
    T, C = y.shape
    if B <= GROUP:
        return np.linalg.norm(y.reshape(T, C // GROUP, GROUP), axis=2)
    nb = np.linalg.norm(y.reshape(T, C // B, B), axis=2)
    return np.repeat(nb, B // GROUP, axis=1)


def full_check(x, lam, r, dev, orc):
    B = r.shape[0]
    codes, scales, y = run_block(x, lam, r, dev)
    c2, s2, _ = run_block(x, lam, r, dev, want_y=False)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    c_ref, s_ref, y_ref = orc.rotate_quant_block(x, lam, r, want_y=True)
    norms = block_norms(y_ref, B)
    worst = check_rotated_values(y, y_ref, norms)
    check_same_precision(y, codes, scales, orc)
    stats = check_against_oracle(codes, scales, c_ref, s_ref, lambda rows: y_ref[rows], norms)
    stats["worst_abs_err_over_norm"] = worst
    print(f"  B={B} {tuple(x.shape)} {x.dtype} lam={lam is not None}: {stats}", flush=True)
    return codes, scales


@pytest.mark.parametrize("B", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype,with_lam", [(torch.bfloat16, False), (torch.bfloat16, True),
                                            (torch.float16, False), (torch.float16, True)])
def test_block_against_oracle(dev, orc, B, dtype, with_lam):
    rng = np.random.default_rng(7000 + B + 10 * with_lam + (dtype == torch.float16))
    T, C = 130, 2048 + 4 * 128  # a full super-tile plus a ragged one
    x = W.random_activations(rng, T, C, dtype, scale=2.0)
    x[3, 5] = 300.0
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32) if with_lam else None
    r = W.bf16_matrix(W.qr_orthogonal(rng, B))
    full_check(x, lam, r, dev, orc)


@pytest.mark.parametrize("B", [16, 32, 64, 128])
def test_block_very_long_rows(dev, orc, B):
    """Rows of 2^20 + 640 channels (513 super-tile columns, the last one a
    partial 20 of 64 groups), fp16 with Λ, against the oracle."""
    rng = np.random.default_rng(7100 + B)
    T, C = 2, (1 << 20) + 640
    x = W.random_activations(rng, T, C, torch.float16, scale=2.0)
    x[1, C - 2] = 500.0
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    r = W.bf16_matrix(W.qr_orthogonal(rng, B))
    full_check(x, lam, r, dev, orc)


@pytest.mark.parametrize("dtype,with_lam", [(torch.bfloat16, False), (torch.bfloat16, True), (torch.float16, True)])
def test_block32_same_bits_as_main_kernel(dev, dtype, with_lam):
    rng = np.random.default_rng(7101)
    x = W.random_activations(rng, 100, 4096, dtype, scale=3.0)
    lam = _lam_dev(np.exp(0.5 * rng.standard_normal(4096)).astype(np.float32) if with_lam else None, dev)
    r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
    xd = x.to(dev)
    c1, s1 = mxq.rotate_quant_block(xd, r, lam)
    c2, s2 = mxq.rotate_quant(xd, r, lam)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def _block_diag(blocks):
    n = sum(b.shape[0] for b in blocks)
    out = torch.zeros((n, n), dtype=torch.bfloat16)
    o = 0
    for b in blocks:
        k = b.shape[0]
        out[o:o + k, o:o + k] = b
        o += k
    return out


def test_block_embeddings_same_bits(dev):
    """A B-block gives the same codes as the 2B-block holding it twice on
    its diagonal (the extra products are exact zeros)."""
    rng = np.random.default_rng(7102)
    x = W.random_activations(rng, 64, 1024, torch.bfloat16, scale=2.0).to(dev)
    for B in (16, 32, 64):
        rb = W.bf16_matrix(W.qr_orthogonal(rng, B))
        c1, s1 = mxq.rotate_quant_block(x, rb.to(dev))
        c2, s2 = mxq.rotate_quant_block(x, _block_diag([rb, rb]).to(dev))
        torch.cuda.synchronize()
        assert torch.equal(c1, c2) and torch.equal(s1, s2), B


def _greedy_block(wl, B, grid=0):
    from oracle import calibration as CAL
    s, n = wl.meta["calib_start"], wl.meta["calib_len"]
    _, _, xw = CAL.worst_group(wl.x[s:s + n], wl.lam, block=B)
    if grid:
        R, _, _, pairs = CAL.greedy_givens_angle(xw, 128, grid)
    else:
        R, _, _, pairs = CAL.greedy_givens(xw, 128)
    return W.bf16_matrix(R), len(pairs)


@pytest.mark.parametrize("cfg", [3, 5])
def test_error_study_block_sizes(dev, orc, cfg):
    """Figure 1's per-group normalized MXFP4 error (mean, p99) for the
    rotation block sizes of the page's ablation (sec. 4.3) and two block
    kinds at each size: a seeded random Hadamard block and the greedy
    outlier-aware block searched on the workload's calibration slice.  The
    page reports B = 32 as best but prints no values: the numbers are only
    reported; the GPU figures are cross-checked against the oracle on a row
    sample."""
    wl = W.make_config(cfg)
    xd = wl.x.to(dev)
    lam_d = _lam_dev(wl.lam, dev)
    rows = np.sort(np.random.default_rng(7103).choice(wl.tokens, 128, replace=False))
    xs = wl.x[torch.from_numpy(rows)].contiguous()
    report = {}
    for B in (16, 32, 64, 128):
        greedy, steps = _greedy_block(wl, B)
        greedy8, steps8 = _greedy_block(wl, B, 8)
        kinds = {"hadamard": W.bf16_matrix(W.random_hadamard(np.random.default_rng(2005 + B), B)),
                 f"greedy({steps})": greedy, f"greedy_grid8({steps8})": greedy8}
        for name, r in kinds.items():
            y = torch.empty(wl.x.shape, dtype=torch.float32, device=dev)
            codes, scales = mxq.rotate_quant_block(xd, r.to(dev), lam_d, y_rot=y)
            dq = mxq.dequant(codes, scales, torch.float32)
            yg = y.view(-1, GROUP).double()
            ny = yg.norm(dim=1)
            keep = ny > 0
            eps = (dq.view(-1, GROUP).double() - yg).norm(dim=1)
            eps = torch.where(keep, eps / torch.where(keep, ny, torch.ones_like(ny)), torch.zeros_like(ny))
            mean = float(eps[keep].mean())
            p99 = float(torch.quantile(eps[keep][::16].float(), 0.99))
            c_ref, s_ref, y_ref = orc.rotate_quant_block(xs, wl.lam, r, want_y=True)
            e_ref = O.group_error(y_ref, orc.dequant(c_ref, s_ref))
            e_gpu = eps.view(wl.tokens, -1)[torch.from_numpy(rows).to(dev)].cpu().numpy().reshape(-1)
            e_gpu = e_gpu[np.linalg.norm(y_ref.reshape(-1, GROUP), axis=1) > 0]
            assert abs(e_gpu.mean() - e_ref.mean()) <= 1e-3 * e_ref.mean() + 1e-6
            report[f"B{B} {name}"] = (round(mean, 5), round(p99, 5))
            del y, dq, codes, scales, eps
            torch.cuda.empty_cache()
    print(f"  block-size error study, config {cfg} (mean, p99): {report}", flush=True)
