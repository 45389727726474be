"""Pins of the fp64 MXFP4 x MXFP4 product oracle."""
import numpy as np

import oracle as O

GROUP = 32


def _pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_triple_loop_on_a_tiny_case():
    rng = np.random.default_rng(1)
    M, N, K = 3, 4, 64
    ca = rng.integers(0, 16, (M, K)); cb = rng.integers(0, 16, (N, K))
    sa = rng.integers(120, 135, (M, K // GROUP)).astype(np.uint8)
    sb = rng.integers(120, 135, (N, K // GROUP)).astype(np.uint8)
    y, s = O.gemm_mxfp4(_pack(ca), sa, _pack(cb), sb)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            acc_abs = 0.0
            for k in range(K):
                va = O.code_value(ca[m, k]) * 2.0 ** (int(sa[m, k // GROUP]) - 127)
                vb = O.code_value(cb[n, k]) * 2.0 ** (int(sb[n, k // GROUP]) - 127)
                acc += va * vb
                acc_abs += abs(va * vb)
            assert y[m, n] == acc and s[m, n] == acc_abs


def test_one_hot_closed_form():
    K = 128
    ca = np.zeros((1, K), np.uint8); cb = np.zeros((1, K), np.uint8)
    ca[0, 70] = 7    # +6 in group 2
    cb[0, 70] = 13   # -3 in group 2
    sa = np.full((1, 4), 127, np.uint8); sb = np.full((1, 4), 127, np.uint8)
    sa[0, 2] = 130   # 2^3
    sb[0, 2] = 125   # 2^-2
    y, s = O.gemm_mxfp4(_pack(ca), sa, _pack(cb), sb)
    assert y[0, 0] == 6 * 8 * (-3) * 0.25 and s[0, 0] == 36.0


def test_scale_equivariance():
    rng = np.random.default_rng(2)
    ca = rng.integers(0, 16, (5, 96)); cb = rng.integers(0, 16, (6, 96))
    sa = rng.integers(110, 140, (5, 3)).astype(np.uint8); sb = rng.integers(110, 140, (6, 3)).astype(np.uint8)
    y0, _ = O.gemm_mxfp4(_pack(ca), sa, _pack(cb), sb)
    y1, _ = O.gemm_mxfp4(_pack(ca), (sa + 3).astype(np.uint8), _pack(cb), sb)
    assert np.array_equal(y1, y0 * 8.0)


def _block_diag(r, groups):
    out = np.zeros((groups * GROUP, groups * GROUP))
    for g in range(groups):
        out[g * GROUP:(g + 1) * GROUP, g * GROUP:(g + 1) * GROUP] = r
    return out


def test_absorption_identity_reproduces_xw():
    """(X Lambda^-1 R)(R^T Lambda W) = X W for an orthogonal, non-symmetric R
    (a transposed block, a dropped or inverted Lambda all break it)."""
    import workloads as W
    rng = np.random.default_rng(4)
    M, K, N = 6, 128, 5
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((K, N))
    lam = np.exp(rng.standard_normal(K)).astype(np.float32)
    r = W.qr_orthogonal(rng)
    assert np.abs(r - r.T).max() > 0.1
    rot = _block_diag(r, K // GROUP)
    x_rot = (x / lam.astype(np.float64)[None, :]) @ rot
    w_hat_t = O.absorb_weights(w.T, lam, r)
    ref = x @ w
    bound = (np.abs(x_rot) @ np.abs(w_hat_t).T) * (4 * K * np.finfo(np.float64).eps)
    assert np.all(np.abs(x_rot @ w_hat_t.T - ref) <= bound + 1e-14 * np.abs(ref))


def test_absorption_matches_dense_block_diag():
    rng = np.random.default_rng(6)
    N, K = 3, 96
    w = rng.standard_normal((N, K))
    lam = rng.uniform(0.5, 2.0, K).astype(np.float32)
    r = rng.standard_normal((GROUP, GROUP))
    dense = (w * lam.astype(np.float64)[None, :]) @ _block_diag(r, K // GROUP)
    assert np.abs(O.absorb_weights(w, lam, r) - dense).max() <= 1e-13 * np.abs(dense).max()


def test_absorb_quant_without_lambda_and_rotation_is_plain_quant():
    import torch
    rng = np.random.default_rng(8)
    w = torch.from_numpy(rng.standard_normal((7, 64)).astype(np.float32)).to(torch.bfloat16)
    codes, scales = O.absorb_quant(w, None, np.eye(GROUP))
    c2, s2 = O.default().quant(w)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
