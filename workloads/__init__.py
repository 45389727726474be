"""Seeded synthetic workloads (inputs only) for the rotate + MXFP4 path.

This module is shared by the tests, the bench and the smoke check, and it
feeds both the HIP library and the CPU oracle.  It holds no part of the
online path (no division by lambda, no rotation, no scale or element
encoding).  It builds the *inputs* the online path consumes: activations X,
the per-channel smoothing factors lambda and the shared 32x32 block R.
Building lambda and R is the offline calibration side of the DuQuant++ page
(sec. 3.1 SmoothQuant factors; sec. 3.2 block rotation).  The page's own
calibration data (WikiText-2 activations of LLaMA-3) is not available, so
every config below is synthetic, seeded and shaped like a LLaMA-3 layer
input, with the outlier structure the page describes in sec. 1 and 2.1:
regular outlier channels and massive outliers on a few tokens.

Generation recipe (one NumPy PCG64 generator per config, seed 1000 + id,
draws taken in the order written): fp64 draws, cast to fp32, then cast to
bf16/fp16 by torch (round-to-nearest-even).

Configs (1-based ids):
  1  bf16 64x256.  N(0,1); channels 7 and 100 x50; X[3,35] = 1024.  lambda = ones.
     R = Q of QR(seeded 32x32 N(0,1)), diag(R_qr) > 0, stored bf16.  Also R = I.
  2  bf16 2048x4096.  N(0,1); 0.5% of channels (20) x20.  lambda = exp(0.5 z_c)
     (lognormal(0, 0.5)).  R seeded QR-orthogonal.
  3  bf16 8192x14336.  Student-t(3)/sqrt(3); on 1% of tokens (82) channels
     {17, 4099, 9001, 14000} take +-U(500, 2000).  lambda = none.  R outlier-aware
     Householder (see householder_outlier) from a seeded 256-token slice.
  4  256 calls of bf16 16x8192.  N(0,1); 2 seeded channels x30.  lambda and R as 2.
  5  fp16 32768x8192.  N(0,1); 8 seeded channels x25; then 0.1% of entries
     replaced by +-U(100, 1000).  lambda = amax_c^0.5 over a seeded 512-token slice
     (SmoothQuant with alpha = 0.5 and no weight term).  R Householder with k
     taken from X / lambda on the same slice.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

GROUP = 32

SHAPES = {1: (64, 256), 2: (2048, 4096), 3: (8192, 14336), 4: (16, 8192), 5: (32768, 8192)}
DTYPES = {1: torch.bfloat16, 2: torch.bfloat16, 3: torch.bfloat16, 4: torch.bfloat16, 5: torch.float16}
CONFIG4_CALLS = 256
CONFIG3_OUTLIER_CHANNELS = (17, 4099, 9001, 14000)


def seed_for(config_id: int) -> int:
    return 1000 + int(config_id)


@dataclasses.dataclass
class Workload:
    """Inputs of one config.  ``x`` is a host tensor [tokens, channels]
    (config 4: [calls * 16, 8192], one call per 16-row slice)."""

    config_id: int
    x: torch.Tensor
    lam: np.ndarray | None  # fp32 [channels] or None
    r_hat: torch.Tensor  # bf16 [32, 32], row-major, y_n = sum_k x_k r[k][n]
    r_hat_f64: np.ndarray  # the fp64 matrix before bf16 rounding
    meta: dict

    @property
    def tokens(self) -> int:
        return self.x.shape[0]

    @property
    def channels(self) -> int:
        return self.x.shape[1]


# ---- conversions (input plumbing) -----------------------------------------

def to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp64 NumPy -> fp32 -> bf16/fp16 torch (RNE at each step)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def bf16_matrix(r: np.ndarray) -> torch.Tensor:
    return to_dtype(r, torch.bfloat16).contiguous()


# ---- 32x32 block builders --------------------------------------------------

def qr_orthogonal(rng: np.random.Generator, n: int = GROUP) -> np.ndarray:
    """Haar-distributed orthogonal matrix: Q of QR(N(0,1) n x n) with the
    signs fixed so that diag(R_qr) > 0."""
    g = rng.standard_normal((n, n))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def sylvester_hadamard(n: int = GROUP) -> np.ndarray:
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def random_hadamard(rng: np.random.Generator, n: int = GROUP) -> np.ndarray:
    """Random Hadamard block, the data-oblivious comparison rotation of the
    DuQuant++ page (sec. 2.2, 4.1): diag(s) H / sqrt(n), s seeded +-1."""
    s = rng.choice(np.array([-1.0, 1.0]), size=n)
    return s[:, None] * sylvester_hadamard(n) / math.sqrt(n)


def householder_to_flat(k: int, n: int = GROUP) -> np.ndarray:
    """H = I - 2 v v^T / v^T v with v = e_k - 1/sqrt(n): symmetric, orthogonal,
    and H e_k = 1/sqrt(n) (the outlier dim's energy spread evenly)."""
    v = -np.ones(n) / math.sqrt(n)
    v[k] += 1.0
    return np.eye(n) - 2.0 * np.outer(v, v) / (v @ v)


def householder_outlier(rng: np.random.Generator, k: int, n: int = GROUP) -> np.ndarray:
    """Outlier-aware block: R = Q_k H.  Q_k is a seeded Haar orthogonal on the
    span of {e_j : j != k} with row and column k equal to e_k, so in the
    row-vector product x R the outlier direction e_k still lands on the flat
    vector 1/sqrt(n) (e_k Q_k = e_k), while the other 31 directions are mixed."""
    sub = qr_orthogonal(rng, n - 1)
    idx = [j for j in range(n) if j != k]
    qk = np.zeros((n, n))
    qk[k, k] = 1.0
    qk[np.ix_(idx, idx)] = sub
    return qk @ householder_to_flat(k, n)


def outlier_dim(x_slice: np.ndarray) -> int:
    """Block-local channel of the largest |x| in a calibration slice
    (first occurrence in row-major order, i.e. lowest token then channel)."""
    flat = int(np.argmax(np.abs(x_slice)))
    channel = flat % x_slice.shape[1]
    return channel % GROUP


# ---- configs ------------------------------------------------------------------

def _config1(rng):
    T, C = SHAPES[1]
    x = rng.standard_normal((T, C))
    x[:, 7] *= 50.0
    x[:, 100] *= 50.0
    x[3, 35] = 1024.0
    r = qr_orthogonal(rng)
    return x, np.ones(C, np.float32), r, {}


def _config2(rng):
    T, C = SHAPES[2]
    x = rng.standard_normal((T, C))
    n_out = int(round(0.005 * C))
    ch = np.sort(rng.choice(C, size=n_out, replace=False))
    x[:, ch] *= 20.0
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    r = qr_orthogonal(rng)
    return x, lam, r, {"outlier_channels": ch.tolist()}


def _config3(rng):
    T, C = SHAPES[3]
    x = rng.standard_t(3, size=(T, C)) / math.sqrt(3.0)
    n_tok = int(round(0.01 * T))
    toks = np.sort(rng.choice(T, size=n_tok, replace=False))
    chans = np.array(CONFIG3_OUTLIER_CHANNELS)
    mag = rng.uniform(500.0, 2000.0, size=(n_tok, chans.size))
    sign = rng.choice(np.array([-1.0, 1.0]), size=(n_tok, chans.size))
    x[np.ix_(toks, chans)] = mag * sign
    start = int(rng.integers(0, T - 256 + 1))
    xs = to_dtype(x[start:start + 256], torch.bfloat16).to(torch.float64).numpy()
    k = outlier_dim(xs)
    r = householder_outlier(rng, k)
    meta = {"outlier_tokens": int(n_tok), "calib_start": start, "calib_len": 256, "k": k,
            "slice_has_outlier_token": bool(np.any((toks >= start) & (toks < start + 256)))}
    return x, None, r, meta


def _config4(rng):
    T, C = SHAPES[4]
    x = rng.standard_normal((CONFIG4_CALLS * T, C))
    ch = np.sort(rng.choice(C, size=2, replace=False))
    x[:, ch] *= 30.0
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    r = qr_orthogonal(rng)
    return x, lam, r, {"calls": CONFIG4_CALLS, "tokens_per_call": T, "outlier_channels": ch.tolist()}


def _config5(rng):
    T, C = SHAPES[5]
    x = rng.standard_normal((T, C))
    ch = np.sort(rng.choice(C, size=8, replace=False))
    x[:, ch] *= 25.0
    n_ent = int(round(0.001 * T * C))
    flat = rng.choice(T * C, size=n_ent, replace=False)
    vals = rng.uniform(100.0, 1000.0, size=n_ent) * rng.choice(np.array([-1.0, 1.0]), size=n_ent)
    x.reshape(-1)[flat] = vals
    start = int(rng.integers(0, T - 512 + 1))
    xs = to_dtype(x[start:start + 512], torch.float16).to(torch.float64).numpy()
    amax = np.abs(xs).max(axis=0)
    lam = np.sqrt(np.maximum(amax, np.finfo(np.float32).tiny)).astype(np.float32)
    k = outlier_dim(xs / lam.astype(np.float64)[None, :])
    r = householder_outlier(rng, k)
    meta = {"outlier_channels": ch.tolist(), "outlier_entries": n_ent, "calib_start": start,
            "calib_len": 512, "k": k}
    return x, lam, r, meta


_BUILDERS = {1: _config1, 2: _config2, 3: _config3, 4: _config4, 5: _config5}


def make_config(config_id: int, seed: int | None = None) -> Workload:
    """Seeded inputs of config ``config_id`` (1..5)."""
    rng = np.random.default_rng(seed_for(config_id) if seed is None else seed)
    x, lam, r, meta = _BUILDERS[config_id](rng)
    xt = to_dtype(x, DTYPES[config_id])
    del x
    meta = dict(meta, seed=seed_for(config_id) if seed is None else seed)
    return Workload(config_id, xt, lam, bf16_matrix(r), r, meta)


def identity_r() -> torch.Tensor:
    return torch.eye(GROUP, dtype=torch.bfloat16)


def random_activations(rng: np.random.Generator, tokens: int, channels: int,
                       dtype: torch.dtype = torch.bfloat16, scale: float = 1.0) -> torch.Tensor:
    """Small seeded N(0, scale^2) activation block for unit and parity tests."""
    return to_dtype(scale * rng.standard_normal((tokens, channels)), dtype)


CALIB_TOKENS = 128 * 2048  # the page's calibration set size: 128 sequences of 2048 tokens


def calibration_block(seed: int = 2011, tokens: int = CALIB_TOKENS) -> np.ndarray:
    """Seeded stand-in for X_worst at the page's calibration size (sec. 3
    pitfalls, item 1): Student-t(3) background over 32 channels, with
    massive +-U(200, 800) values on 2000 seeded tokens of channel 9."""
    rng = np.random.default_rng(seed)
    xw = rng.standard_t(3, size=(tokens, GROUP))
    n = min(2000, tokens)
    rows = rng.choice(tokens, n, replace=False)
    xw[rows, 9] = rng.choice(np.array([-1.0, 1.0]), n) * rng.uniform(200.0, 800.0, n)
    return xw


# ---- the consumer linear layer --------------------------------------------------

# LLaMA-3-8B down_proj: 14336 input features -> 4096 outputs.  Config 3's
# activations are that layer's input.
DOWN_PROJ_OUT = 4096


def linear_weights(out_features: int, in_features: int, seed: int = 3001,
                   dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Seeded stand-in for a trained linear layer's weights, [out, in] (the
    transpose of W in Y = X W): N(0, 1/in) entries, as at initialisation, so
    every output has unit-order variance for unit-variance inputs."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((out_features, in_features), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(in_features))
    return torch.from_numpy(w).to(dtype)


def random_mxfp4(rng: np.random.Generator, rows: int, k: int, scale_lo: int = 110,
                 scale_hi: int = 140) -> tuple[np.ndarray, np.ndarray]:
    """Uniformly random MXFP4 operand: every byte of codes [rows, k/2] drawn
    from 0..255 (all 16 codes in both nibbles, -0 included), every scale byte
    from [scale_lo, scale_hi]."""
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, size=(rows, k // GROUP), dtype=np.uint8)
    return codes, scales


# ---- the norm in front of the rotation ------------------------------------------

NORM_SHAPE = (8192, 4096)  # LLaMA-3-8B hidden size: the input of the QKV and gate/up norms


@dataclasses.dataclass
class NormWorkload:
    """Residual-stream rows h (the norm's input) and the norm's parameters."""

    x: torch.Tensor
    gamma: np.ndarray
    beta: np.ndarray | None
    lam: np.ndarray
    r_hat: torch.Tensor
    eps: float
    meta: dict


def norm_workload(tokens: int = NORM_SHAPE[0], channels: int = NORM_SHAPE[1], seed: int = 4001,
                  dtype: torch.dtype = torch.bfloat16, with_beta: bool = False) -> NormWorkload:
    """Seeded stand-in for a pre-norm residual stream: N(0, 1) rows whose 4
    seeded channels carry +-U(50, 200) on 0.5% of the tokens (the massive
    residual-stream activations of LLaMA-type models), gamma ~ U(0.5, 1.5),
    beta ~ N(0, 0.1) when asked for (LayerNorm), lambda lognormal(0, 0.5),
    seeded orthogonal block, eps 1e-5."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, channels))
    ch = np.sort(rng.choice(channels, size=min(4, channels), replace=False))
    n_tok = max(1, int(round(0.005 * tokens)))
    toks = np.sort(rng.choice(tokens, size=n_tok, replace=False))
    x[np.ix_(toks, ch)] = rng.uniform(50.0, 200.0, (n_tok, ch.size)) * rng.choice(np.array([-1.0, 1.0]),
                                                                                  (n_tok, ch.size))
    gamma = rng.uniform(0.5, 1.5, channels).astype(np.float32)
    beta = (0.1 * rng.standard_normal(channels)).astype(np.float32) if with_beta else None
    lam = np.exp(0.5 * rng.standard_normal(channels)).astype(np.float32)
    r = qr_orthogonal(rng)
    return NormWorkload(to_dtype(x, dtype), gamma, beta, lam, bf16_matrix(r), 1e-5,
                        {"seed": seed, "massive_channels": ch.tolist(), "massive_tokens": int(n_tok)})
