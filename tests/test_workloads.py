"""Seeded input generators: block-builder identities and config recipes."""
import math

import numpy as np
import torch

import workloads as W


def test_sylvester_hadamard_is_exact():
    h = W.sylvester_hadamard(32)
    assert np.array_equal(h @ h.T, 32 * np.eye(32))
    r = W.random_hadamard(np.random.default_rng(1))
    assert np.allclose(r @ r.T, np.eye(32), atol=1e-15)


def test_householder_maps_outlier_dim_to_flat():
    for k in (0, 3, 17, 31):
        h = W.householder_to_flat(k)
        assert np.allclose(h @ h, np.eye(32), atol=1e-14)
        assert np.allclose(h, h.T)
        assert np.allclose(h[:, k], np.ones(32) / math.sqrt(32), atol=1e-15)
        r = W.householder_outlier(np.random.default_rng(k), k)
        assert np.allclose(r @ r.T, np.eye(32), atol=1e-14)
        e = np.zeros(32)
        e[k] = 1.0
        assert np.allclose(e @ r, np.ones(32) / math.sqrt(32), atol=1e-14)


def test_qr_orthogonal_sign_convention():
    rng = np.random.default_rng(3)
    g_state = rng.bit_generator.state
    q = W.qr_orthogonal(rng)
    assert np.allclose(q @ q.T, np.eye(32), atol=1e-14)
    rng2 = np.random.default_rng()
    rng2.bit_generator.state = g_state
    g = rng2.standard_normal((32, 32))
    r = q.T @ g  # the triangular factor
    assert np.allclose(np.tril(r, -1), 0, atol=1e-12)
    assert np.all(np.diag(r) > 0)


def test_outlier_dim_picks_block_local_channel():
    x = np.zeros((4, 96))
    x[2, 70] = -9.0
    x[1, 5] = 8.0
    assert W.outlier_dim(x) == 70 % 32


def test_config_recipes_are_seeded_and_shaped():
    a = W.make_config(1)
    b = W.make_config(1)
    assert torch.equal(a.x, b.x) and torch.equal(a.r_hat, b.r_hat)
    assert a.x.shape == (64, 256) and a.x.dtype == torch.bfloat16
    assert float(a.x[3, 35]) == 1024.0
    c2 = W.make_config(2)
    assert c2.x.shape == (2048, 4096) and len(c2.meta["outlier_channels"]) == 20
    assert c2.lam.dtype == np.float32 and np.all(c2.lam > 0)
    c4 = W.make_config(4)
    assert c4.x.shape == (256 * 16, 8192)


def test_bf16_block_is_nearly_orthogonal():
    r = W.make_config(1).r_hat.to(torch.float64).numpy()
    assert np.linalg.norm(r @ r.T - np.eye(32), 2) < 0.02
