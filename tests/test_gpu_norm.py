"""Norm + smooth + rotate + MXFP4 (DuQuant++ page sec. 5.2 item 1) on an
MI355X, through the C ABI, against the fp64 oracle under the tolerance rule
of the plain fused path.  The group norms of the rule are those of the
oracle's rotated values (the block is orthogonal up to its bf16 rounding)."""
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


def _f32(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


def run_gpu(x, r, gamma, beta, lam, norm, eps, dev, want_y=True):
    xd = x.to(dev)
    y = torch.empty(x.shape, dtype=torch.float32, device=dev) if want_y else None
    codes, scales = mxq.norm_rotate_quant(xd, r.to(dev), _f32(gamma, dev), _f32(beta, dev), _f32(lam, dev),
                                          norm=norm, eps=eps, y_rot=y)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (y.cpu().numpy() if want_y else None)


def group_norms(y):
    T, C = y.shape
    return np.linalg.norm(y.reshape(T, C // GROUP, GROUP), axis=2)


def full_check(x, r, gamma, beta, lam, norm, eps, dev, orc):
    codes, scales, y = run_gpu(x, r, gamma, beta, lam, norm, eps, dev)
    c2, s2, _ = run_gpu(x, r, gamma, beta, lam, norm, eps, dev, want_y=False)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # the kernel receives eps as fp32: the oracle gets that same value
    c_ref, s_ref, y_ref = orc.norm_rotate_quant(x, norm, gamma, beta, float(np.float32(eps)), lam, r, want_y=True)
    norms = group_norms(y_ref)
    worst = check_rotated_values(y, y_ref, norms)
    check_same_precision(y, codes, scales, orc)
    stats = check_against_oracle(codes, scales, c_ref, s_ref, lambda rows: y_ref[rows], norms)
    stats["worst_abs_err_over_norm"] = worst
    print(f"  norm={norm} {tuple(x.shape)} {x.dtype} beta={beta is not None} lam={lam is not None}: {stats}",
          flush=True)
    return stats


@pytest.mark.parametrize("norm", ["rms", "layer"])
@pytest.mark.parametrize("T,C,dtype", [(64, 256, torch.bfloat16), (300, 1056, torch.bfloat16),
                                       (256, 4096, torch.float16), (33, 8192, torch.bfloat16),
                                       (9, 16384, torch.bfloat16), (5, 32, torch.float16),
                                       (70, 2080, torch.bfloat16)])
def test_norm_against_oracle(dev, orc, norm, T, C, dtype):
    wl = W.norm_workload(T, C, seed=4100 + C + T, dtype=dtype, with_beta=(norm == "layer"))
    full_check(wl.x, wl.r_hat, wl.gamma, wl.beta, wl.lam, norm, wl.eps, dev, orc)


@pytest.mark.parametrize("norm,T,C,dtype", [("rms", 3000, 8192, torch.bfloat16), ("layer", 3000, 8192, torch.float16),
                                            ("rms", 2600, 16384, torch.bfloat16),
                                            ("layer", 2600, 16384, torch.float16)])
def test_norm_long_rows_several_per_wave(dev, orc, norm, T, C, dtype):
    """Rows longer than 4096 channels keep one row buffer, and the next row
    loads super-tile by super-tile while the current one is encoded.  With
    more rows than the grid's waves (about 2048 at these widths), waves take
    two rows, so prefetched super-tiles are checked against the oracle too."""
    wl = W.norm_workload(T, C, seed=4700 + C + T, dtype=dtype, with_beta=(norm == "layer"))
    full_check(wl.x, wl.r_hat, wl.gamma, wl.beta, wl.lam, norm, wl.eps, dev, orc)


def test_norm_without_lambda_identity_block(dev, orc):
    wl = W.norm_workload(128, 512, seed=4201)
    full_check(wl.x, W.identity_r(), wl.gamma, None, None, "rms", wl.eps, dev, orc)
    full_check(wl.x, W.identity_r(), wl.gamma, wl.gamma * 0.25, None, "layer", 0.0, dev, orc)


def test_norm_strided_rows(dev, orc):
    wl = W.norm_workload(40, 1024, seed=4202)
    big = torch.zeros((40, 1024 + 64), dtype=torch.bfloat16)
    big[:, :1024] = wl.x
    view = big.to(dev)[:, :1024]
    codes, scales = mxq.norm_rotate_quant(view, wl.r_hat.to(dev), _f32(wl.gamma, dev), None, _f32(wl.lam, dev),
                                          norm="rms", eps=wl.eps)
    c2, s2, _ = run_gpu(wl.x, wl.r_hat, wl.gamma, None, wl.lam, "rms", wl.eps, dev, want_y=False)
    assert np.array_equal(codes.cpu().numpy(), c2) and np.array_equal(scales.cpu().numpy(), s2)


def test_norm_zero_rows_and_empty(dev):
    x = torch.zeros((6, 256), dtype=torch.bfloat16)
    gamma = np.ones(256, np.float32)
    codes, scales, _ = run_gpu(x, W.identity_r(), gamma, None, None, "rms", 1e-5, dev)
    assert not codes.any() and not scales.any()
    e = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    c, s = mxq.norm_rotate_quant(e, W.identity_r().to(dev), _f32(gamma, dev))
    assert c.shape == (0, 128) and s.shape == (0, 8)


def test_norm_determinism(dev):
    wl = W.norm_workload(512, 4096, seed=4203)
    a = run_gpu(wl.x, wl.r_hat, wl.gamma, None, wl.lam, "rms", wl.eps, dev, want_y=False)
    b = run_gpu(wl.x, wl.r_hat, wl.gamma, None, wl.lam, "rms", wl.eps, dev, want_y=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_norm_bench_workload_sampled(dev, orc):
    """The bench's launch configuration (bf16 8192 x 4096, RMSNorm, lambda),
    checked on 256 sampled rows recomputed by the oracle."""
    wl = W.norm_workload()
    codes, scales, y = run_gpu(wl.x, wl.r_hat, wl.gamma, None, wl.lam, "rms", wl.eps, dev)
    rows = np.sort(np.random.default_rng(4204).choice(wl.x.shape[0], 256, replace=False))
    xs = wl.x[torch.from_numpy(rows)]
    c_ref, s_ref, y_ref = orc.norm_rotate_quant(xs, "rms", wl.gamma, None, float(np.float32(wl.eps)), wl.lam,
                                                wl.r_hat, want_y=True)
    norms = group_norms(y_ref)
    check_rotated_values(y[rows], y_ref, norms)
    stats = check_against_oracle(codes[rows], scales[rows], c_ref, s_ref, lambda rr: y_ref[rr], norms)
    print(f"  bench workload, 256 sampled rows: {stats}", flush=True)


@pytest.mark.parametrize("C,dtype,offset,sigma", [(4096, torch.bfloat16, 200.0, 8.0),
                                                   (16384, torch.bfloat16, 200.0, 8.0),
                                                   (4096, torch.float16, 1000.0, 1.0),
                                                   (16384, torch.float16, 1000.0, 1.0)])
def test_layernorm_large_mean_offset(dev, orc, C, dtype, offset, sigma):
    """LayerNorm rows whose mean is large against their spread (mean / sd up
    to 1000): the mean's absolute error scales with the mean, so this is the
    case that tests the precision of the row sums."""
    rng = np.random.default_rng(4206 + C)
    T = 48
    x = torch.from_numpy(offset + sigma * rng.standard_normal((T, C))).to(dtype)
    gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32)
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    stats = full_check(x, W.bf16_matrix(W.qr_orthogonal(rng)), gamma, beta, lam, "layer", 1e-5, dev, orc)
    # x' enters the matrix cores as two rounded bf16 terms (2^-18 |x'| each),
    # so the worst value sits near 4e-6 of the group norm; a mean rounded
    # once to fp32 and subtracted gave 3.5e-5 here
    assert stats["worst_abs_err_over_norm"] < 8e-6


@pytest.mark.parametrize("norm", ["rms", "layer"])
def test_norm_block_sizes_same_bits(dev, norm):
    """Long batches run in 16-wave blocks, short ones in 4-wave blocks: the
    rows come out the same either way."""
    wl = W.norm_workload(4608, 4096, seed=4205, with_beta=(norm == "layer"))
    full = run_gpu(wl.x, wl.r_hat, wl.gamma, wl.beta, wl.lam, norm, wl.eps, dev, want_y=False)
    part = run_gpu(wl.x[:300].contiguous(), wl.r_hat, wl.gamma, wl.beta, wl.lam, norm, wl.eps, dev, want_y=False)
    assert np.array_equal(full[0][:300], part[0]) and np.array_equal(full[1][:300], part[1])
