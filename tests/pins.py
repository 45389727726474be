"""Pins that tie the fp64 oracle to facts outside itself.

Each ``pin_*`` takes an :class:`oracle.Oracle` and raises ``AssertionError``
when the oracle disagrees with what the pages, the MX standard or plain
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GROUP = 32


def _rng(seed):
    return np.random.default_rng(seed)


def _unpack(codes):
    return O.unpack_codes(codes)


# ---------------------------------------------------------------------------
def pin_worked_example(orc):
    """DuQuant++ page sec. 2.1: 1024.0 sets the group scale and crushes 0.1-0.4."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    x = np.array([g["group"]], dtype=np.float32)
    codes, scales = orc.quant(x)
    assert int(scales[0, 0]) == g["scale_byte"], scales
    assert codes[0].tolist() == g["packed_codes"], codes
    dq = orc.dequant(codes, scales)
    assert dq[0].tolist() == g["dequant"], dq
    # the same group through the fused path with the identity block
    c2, s2 = orc.rotate_quant(torch.from_numpy(x), None, W.identity_r())
    assert c2.tolist() == codes.tolist() and s2.tolist() == scales.tolist()
    # group error of the crushed group, closed form
    y = np.array(g["group"], dtype=np.float64)
    err = O.group_error(y, dq[0])
    small = math.sqrt(0.1 ** 2 + 0.2 ** 2 + 0.3 ** 2 + 0.4 ** 2)
    expect = small / math.sqrt(small ** 2 + 1024.0 ** 2)
    assert abs(err[0] - expect) <= 1e-6 * expect, (err, expect)


def pin_config1_massive_value(orc):
    """Config 1 plants the worked example's 1024.0 at token 3, channel 35:
    group 1 of token 3 must carry scale 0x87, code 6 at local index 3 and zeros
    elsewhere (its other entries are N(0,1) draws, all below 64)."""
    wl = W.make_config(1)
    codes, scales = orc.rotate_quant(wl.x, None, W.identity_r())
    assert int(scales[3, 1]) == 0x87
    c = _unpack(codes)[3, 32:64]
    assert c[3] == 6 and np.count_nonzero(c) == 1, c


def _pilot_groups(values, e):
    """Groups of 32 whose element 0 is 4*2^e (so the shared exponent is e
    whenever every |value| < 8) followed by 31 test values times 2^e."""
    v = np.asarray(values, dtype=np.float64)
    pad = (-v.size) % 31
    v = np.concatenate([v, np.zeros(pad)]).reshape(-1, 31)
    g = np.concatenate([np.full((v.shape[0], 1), 4.0), v], axis=1)
    return np.ldexp(g, e), v


def _codec_values():
    # every finite non-negative bf16 magnitude below 8
    bits = np.arange(0, 0x4100, dtype=np.uint32) << 16
    mags = bits.view(np.float32).astype(np.float64)
    mags = mags[np.isfinite(mags) & (mags < 8.0)]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    near = np.concatenate([ties, np.nextafter(ties, 0), np.nextafter(ties, 9),
                           ties * (1 - 2.0 ** -24), ties * (1 + 2.0 ** -24)])
    sat = np.array([5.0 + 2.0 ** -40, 6.0, 6.5, 7.0, 7.99, np.nextafter(8.0, 0)])
    grid = O.E2M1_VALUES
    v = np.concatenate([mags, near, sat, grid])
    return np.concatenate([v, -v])


def pin_bruteforce_codec(orc):
    """Every code equals the exhaustive nearest-of-16 search (ties to even,
    +0 for zero, saturation at 6) for all bf16 magnitudes below 8, planted
    ties and their neighbours, across the whole exponent range."""
    vals = _codec_values()
    expect = O.brute_force_codes(vals)
    for e in (-127, -126, -100, -3, -1, 0, 1, 7, 100, 126, 127):
        groups, v = _pilot_groups(vals, e)
        codes, scales = orc.quant(groups)
        assert np.all(scales == e + 127), (e, np.unique(scales))
        got = _unpack(codes)[:, 1:].reshape(-1)[: vals.size]
        bad = np.nonzero(got != expect)[0]
        assert bad.size == 0, (e, vals[bad[:5]], got[bad[:5]], expect[bad[:5]])
        # pilot element: 4 -> code 6
        assert np.all(_unpack(codes)[:, 0] == 6)


def pin_scale_clamps(orc):
    """E8M0 range: exponent clamps to [-127, 127]; an all-zero group is S = 0
    with all codes +0; below the range the elements are encoded against 2^-127."""
    z = np.zeros((1, GROUP))
    c, s = orc.quant(z)
    assert s[0, 0] == 0 and not c.any()
    vals = np.array([1.0, -1.0, 0.75, 0.25, 1.5, 2.0, 0.5, -0.3])
    tiny = np.zeros((1, GROUP))
    tiny[0, : vals.size] = np.ldexp(vals, -127)
    c, s = orc.quant(tiny)
    assert s[0, 0] == 0
    assert _unpack(c)[0, : vals.size].tolist() == O.brute_force_codes(vals).tolist()
    tinier = np.ldexp(np.array([[0.9] + [0.0] * 31]), -140)
    c, s = orc.quant(tinier)
    assert s[0, 0] == 0 and not c.any()
    huge = np.zeros((1, GROUP))
    huge[0, :3] = [2.0 ** 135, -(2.0 ** 129), 2.0 ** 128]
    c, s = orc.quant(huge)
    assert s[0, 0] == 254
    assert _unpack(c)[0, :3].tolist() == [7, 14, 4]  # 256 -> sat 6; -4; 2


def pin_scale_window(orc):
    """Defining property of e = floor(log2 amax) - 2: amax / 2^e lies in [4, 8),
    so the group's largest element always encodes to 4 or 6."""
    rng = _rng(7)
    mags = np.ldexp(rng.uniform(0.5, 1.0, (4000, 1)), rng.integers(-120, 120, (4000, 1)))
    x = mags * rng.standard_normal((4000, GROUP))
    codes, scales = orc.quant(x)
    amax = np.abs(x).max(axis=1)
    e = scales[:, 0].astype(np.int64) - 127
    ratio = np.ldexp(amax, -e)
    assert np.all((ratio >= 4.0) & (ratio < 8.0)), ratio.min()
    c = _unpack(codes)
    top = c[np.arange(x.shape[0]), np.abs(x).argmax(axis=1)] & 7
    assert np.all((top == 6) | (top == 7))


def pin_identity_rotation(orc):
    """With R = I (and lambda = ones or absent) the fused path is plain MXFP4,
    which the brute-force pins fix."""
    rng = _rng(11)
    x = W.random_activations(rng, 48, 256, scale=3.0)
    x[5, 40] = 700.0
    c0, s0 = orc.quant(x)
    c1, s1 = orc.rotate_quant(x, None, W.identity_r())
    c2, s2 = orc.rotate_quant(x, np.ones(256, np.float32), W.identity_r())
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert np.array_equal(c0, c2) and np.array_equal(s0, s2)
    xf = x.to(torch.float64).numpy()
    groups = xf.reshape(-1, GROUP)
    e = s0.reshape(-1).astype(np.int64) - 127
    expect = O.brute_force_codes(np.ldexp(groups, -e[:, None]))
    assert np.array_equal(_unpack(c0).reshape(-1), expect)


def _nonsymmetric_r(seed=5):
    r = W.qr_orthogonal(_rng(seed))
    rb = W.bf16_matrix(r)
    rf = rb.to(torch.float64).numpy()
    assert np.abs(rf - rf.T).max() > 0.1
    return rb, rf


def pin_dense_blockdiag(orc):
    """y = (x / lambda) . BlockDiag(R, ..., R) computed as one dense NumPy
    product equals the oracle's per-group rotated values (row-vector form,
    X * Lambda^-1 * R of the DuQuant++ page sec. 3.3), and the codes are the
    brute-force encoding of those values."""
    rng = _rng(13)
    T, C = 24, 256
    x = W.random_activations(rng, T, C, scale=2.0)
    lam = np.exp(0.4 * rng.standard_normal(C)).astype(np.float32)
    rb, rf = _nonsymmetric_r()
    codes, scales, y = orc.rotate_quant(x, lam, rb, want_y=True)
    xs = x.to(torch.float64).numpy() / lam.astype(np.float64)[None, :]
    dense = np.kron(np.eye(C // GROUP), rf)
    y_ref = xs @ dense
    norms = np.linalg.norm(xs.reshape(T, -1, GROUP), axis=2).repeat(GROUP, axis=1)
    assert np.all(np.abs(y - y_ref) <= 1e-13 * norms + 1e-300)
    e = scales.reshape(-1).astype(np.int64) - 127
    expect = O.brute_force_codes(np.ldexp(y_ref.reshape(-1, GROUP), -e[:, None]))
    assert np.array_equal(_unpack(codes).reshape(-1), expect)


def pin_norm_preservation(orc):
    """R orthogonal makes the rotation lossless (DuQuant++ page sec. 3.3):
    | ||y_g||^2 - ||x'_g||^2 | <= delta ||x'_g||^2, delta = ||R R^T - I||_2 of
    the bf16-rounded block."""
    rng = _rng(17)
    x = W.random_activations(rng, 64, 512, scale=1.5)
    for r64 in (W.qr_orthogonal(rng), W.householder_outlier(rng, 9), W.random_hadamard(rng)):
        rb = W.bf16_matrix(r64)
        rf = rb.to(torch.float64).numpy()
        delta = np.linalg.norm(rf @ rf.T - np.eye(GROUP), 2)
        _, _, y = orc.rotate_quant(x, None, rb, want_y=True)
        xs = x.to(torch.float64).numpy()
        ny = (y.reshape(-1, GROUP) ** 2).sum(1)
        nx = (xs.reshape(-1, GROUP) ** 2).sum(1)
        # the bound is attained by a Hadamard block (R R^T = c I): allow fp64 rounding of the sums
        assert np.all(np.abs(ny - nx) <= (delta + 1e-13) * nx + 1e-300)


def pin_equivariance(orc):
    """Q(2^j x) keeps the codes and adds j to every scale; Q(-x) flips the sign
    bit of every nonzero code; permuting tokens or whole groups permutes the
    outputs (groups are independent, DuQuant++ page sec. 2.3)."""
    rng = _rng(19)
    x = rng.standard_normal((32, 128)) * np.exp(rng.standard_normal((32, 1)))
    c0, s0 = orc.quant(x)
    for j in (-5, 1, 9):
        c, s = orc.quant(np.ldexp(x, j))
        assert np.array_equal(c, c0) and np.array_equal(s.astype(int), s0.astype(int) + j)
    c, s = orc.quant(-x)
    u0, u = _unpack(c0), _unpack(c)
    assert np.array_equal(s, s0)
    assert np.array_equal(u, np.where(u0 & 7, u0 ^ 8, 0))
    perm = rng.permutation(32)
    c, s = orc.quant(np.ascontiguousarray(x[perm]))
    assert np.array_equal(c, c0[perm]) and np.array_equal(s, s0[perm])
    gperm = rng.permutation(4)
    xg = np.ascontiguousarray(x.reshape(32, 4, GROUP)[:, gperm].reshape(32, 128))
    c, s = orc.quant(xg)
    assert np.array_equal(c.reshape(32, 4, 16), c0.reshape(32, 4, 16)[:, gperm])
    assert np.array_equal(s, s0[:, gperm])


def pin_lambda_powers_of_two(orc):
    """lambda = 2^j_c divides channel c exactly: the smoothed fused path with
    R = I equals plain MXFP4 of x * 2^-j_c."""
    rng = _rng(23)
    x = W.random_activations(rng, 16, 256, scale=4.0)
    j = rng.integers(-6, 7, 256)
    lam = np.ldexp(np.ones(256), j).astype(np.float32)
    c1, s1 = orc.rotate_quant(x, lam, W.identity_r())
    xs = np.ldexp(x.to(torch.float64).numpy(), -j[None, :])
    c0, s0 = orc.quant(xs)
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


def pin_strided_input(orc):
    """A row stride larger than the channel count reads only the first
    `channels` entries of each row."""
    rng = _rng(29)
    big = rng.standard_normal((8, 96 + 40))
    view = big[:, :96]
    c1, s1 = orc.quant(view)
    c0, s0 = orc.quant(np.ascontiguousarray(view))
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
    bt = torch.from_numpy(big).to(torch.bfloat16)
    rb, _ = _nonsymmetric_r()
    c1, s1 = orc.rotate_quant(bt[:, :96], None, rb)
    c0, s0 = orc.rotate_quant(bt[:, :96].contiguous(), None, rb)
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


def pin_input_decoding(orc):
    """bf16 and fp16 inputs are upcast exactly: quantizing every finite fp16
    (or a sweep of bf16) pattern equals quantizing the same values given as
    fp64 by the NumPy / torch conversions."""
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    h = h[: h.size // GROUP * GROUP].reshape(-1, GROUP)
    c1, s1 = orc.quant(h)
    c0, s0 = orc.quant(h.astype(np.float64))
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
    b = torch.arange(0, 0x10000, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    b = b[torch.isfinite(b)]
    b = b[: b.numel() // GROUP * GROUP].reshape(-1, GROUP)
    c1, s1 = orc.quant(b)
    c0, s0 = orc.quant(b.to(torch.float64).numpy())
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
    # rotated path: fp16 input with an fp64 identity block
    hx = torch.from_numpy(np.ascontiguousarray(h[:64]))
    c1, s1 = orc.rotate_quant(hx, None, np.eye(GROUP))
    c0, s0 = orc.quant(h[:64].astype(np.float64))
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)


def pin_dequant(orc):
    """Dequant is the E2M1 value times 2^(S-127) for all 16 codes (OCP MX v1.0
    tables); S = 255 is NaN; and quantizing a dequantized tensor returns the
    same codes and scales (its max re-encodes to 4 or 6 under the same e)."""
    codes_all = np.arange(16, dtype=np.uint8)
    for S in (0, 1, 3, 100, 127, 128, 200, 254, 255):
        packed = (codes_all[0::2] | (codes_all[1::2] << 4)).astype(np.uint8)
        packed = np.tile(packed, 2)[None, :]  # 32 codes: 0..15, 0..15
        sc = np.array([[S]], np.uint8)
        out = orc.dequant(packed, sc)[0]
        expect = np.tile(O.code_value(codes_all), 2)
        if S == 255:
            assert np.all(np.isnan(out))
        else:
            exp_v = np.ldexp(expect, S - 127)
            assert np.array_equal(out, exp_v)
            assert np.array_equal(np.signbit(out), np.signbit(exp_v))
    rng = _rng(31)
    x = rng.standard_normal((40, 128)) * np.exp(2 * rng.standard_normal((40, 1)))
    c, s = orc.quant(x)
    dq = orc.dequant(c, s)
    c2, s2 = orc.quant(dq)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def pin_encode_groups_matches_quant(orc):
    """The exported group encoder is the same map as quantization of a row."""
    rng = _rng(37)
    y = rng.standard_normal((100, GROUP)) * 10
    c, s = orc.encode_groups(y)
    c0, s0 = orc.quant(y)
    assert np.array_equal(c.reshape(c0.shape), c0) and np.array_equal(s.reshape(s0.shape), s0)


# ---- norm + smooth + rotate + quantize (DuQuant++ page sec. 5.2 item 1) -----

def _unit_ms_rows(rng, T, C):
    """Rows with sum x^2 = C and sum x = 0 exactly: C/64 copies of
    {+-2 x 4, +-1.5 x 8, +-1 x 30, 0 x 22}, signs balanced, shuffled."""
    base = np.array([2.0] * 2 + [-2.0] * 2 + [1.5] * 4 + [-1.5] * 4 + [1.0] * 15 + [-1.0] * 15 + [0.0] * 22)
    x = np.array([rng.permutation(np.concatenate([base] * (C // 64))) for _ in range(T)])
    assert np.all((x ** 2).sum(axis=1) == C) and np.all(x.sum(axis=1) == 0)
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def pin_norm_alternating_closed_form(orc):
    """x = (a, -a, a, ...): mean 0, mean square a^2, every normalized value
    +-1; gamma = 1, R = I: scale 2^-2 (byte 125), codes +4 / -4 (0x6 / 0xE)."""
    C = 128
    for norm in ("rms", "layer"):
        for a in (3.0, 0.375, 96.0):
            x = torch.tensor([[a if c % 2 == 0 else -a for c in range(C)]], dtype=torch.bfloat16)
            codes, scales = orc.norm_rotate_quant(x, norm, np.ones(C, np.float32), None, 0.0, None,
                                                  W.identity_r())
            assert np.all(scales == 125), (norm, a)
            assert np.all(codes == 0xE6), (norm, a)


def pin_norm_reduces_to_rotate_quant(orc):
    """Rows of mean 0 and mean square 1 normalize to themselves (eps = 0);
    with power-of-two gamma, dyadic beta and lambda the result is exactly
    rotate_quant((x gamma + beta), lambda): smoothing after gamma and beta."""
    rng = _rng(41)
    T, C = 6, 128
    x = _unit_ms_rows(rng, T, C)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    lam = (np.exp2(rng.integers(-2, 3, C)) * rng.choice([1.0, 1.25, 0.75], C)).astype(np.float32)
    gamma = np.exp2(rng.integers(-1, 3, C)).astype(np.float32)
    beta = (rng.integers(-8, 9, C) / 4.0).astype(np.float32)
    for norm in ("rms", "layer"):
        for b in (None, beta):
            c1, s1, y1 = orc.norm_rotate_quant(x, norm, gamma, b, 0.0, lam, r, want_y=True)
            a = x.to(torch.float32) * _f32(gamma)[None, :]
            if b is not None:
                a = a + _f32(b)[None, :]
            c2, s2, y2 = orc.rotate_quant(a, lam, r, want_y=True)
            assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(y1, y2), norm


def pin_norm_eps_under_root(orc):
    """Mean square 1 with eps = 3: 1 / sqrt(1 + 3) halves every value."""
    rng = _rng(42)
    x = _unit_ms_rows(rng, 4, 64)
    gamma = np.ones(64, np.float32)
    for norm in ("rms", "layer"):
        c1, s1, y1 = orc.norm_rotate_quant(x, norm, gamma, None, 3.0, None, W.identity_r(), want_y=True)
        c2, s2, y2 = orc.rotate_quant(x.to(torch.float32) * 0.5, None, W.identity_r(), want_y=True)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(y1, y2), norm


def pin_norm_scale_invariance(orc):
    """norm(2^k x) = norm(x) for eps = 0."""
    rng = _rng(43)
    x = W.random_activations(rng, 8, 256, torch.bfloat16, scale=3.0)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    gamma = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    for norm in ("rms", "layer"):
        base = orc.norm_rotate_quant(x, norm, gamma, None, 0.0, None, r, want_y=True)
        for k in (-6, 5):
            got = orc.norm_rotate_quant(x * 2.0 ** k, norm, gamma, None, 0.0, None, r, want_y=True)
            assert all(np.array_equal(u, v) for u, v in zip(got, base)), (norm, k)


def pin_layernorm_shift_invariance(orc):
    """LayerNorm removes the row mean (x + 5 normalizes like x); RMSNorm does not."""
    rng = _rng(44)
    grid = np.clip(np.round(rng.standard_normal((8, 256)) * 8) / 8, -4, 4)  # 1/8 grid: x + 5 stays exact
    x = torch.from_numpy(grid.astype(np.float32)).to(torch.bfloat16)
    shifted = (x.to(torch.float32) + 5.0).to(torch.bfloat16)
    assert torch.equal(shifted.to(torch.float32) - 5.0, x.to(torch.float32))
    gamma = np.ones(256, np.float32)
    _, _, y0 = orc.norm_rotate_quant(x, "layer", gamma, None, 1e-6, None, W.identity_r(), want_y=True)
    _, _, y1 = orc.norm_rotate_quant(shifted, "layer", gamma, None, 1e-6, None, W.identity_r(), want_y=True)
    assert np.abs(y1 - y0).max() <= 1e-12 * np.abs(y0).max()
    _, _, z1 = orc.norm_rotate_quant(shifted, "rms", gamma, None, 1e-6, None, W.identity_r(), want_y=True)
    assert np.abs(z1 - y0).max() > 0.1


def pin_norm_gamma_lambda_refactoring(orc):
    """(gamma 2^k, lambda 2^k) smooths exactly like (gamma, lambda)."""
    rng = _rng(45)
    x = W.random_activations(rng, 4, 128, torch.float16)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    gamma = rng.uniform(0.5, 2.0, 128).astype(np.float32)
    lam = rng.uniform(0.5, 4.0, 128).astype(np.float32)
    a = orc.norm_rotate_quant(x, "rms", gamma, None, 1e-5, lam, r, want_y=True)
    b = orc.norm_rotate_quant(x, "rms", gamma * 8, None, 1e-5, lam * 8, r, want_y=True)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def pin_norm_zero_row(orc):
    """A zero row normalizes to zero: all codes 0 and scale byte 0, or the
    encoding of beta alone."""
    C = 64
    x = torch.zeros((2, C), dtype=torch.bfloat16)
    gamma = np.ones(C, np.float32)
    beta = np.linspace(-1, 1, C).astype(np.float32)
    for norm in ("rms", "layer"):
        codes, scales = orc.norm_rotate_quant(x, norm, gamma, None, 1e-6, None, W.identity_r())
        assert not codes.any() and not scales.any()
        c1, s1 = orc.norm_rotate_quant(x, norm, gamma, beta, 1e-6, None, W.identity_r())
        c2, s2 = orc.rotate_quant(_f32(np.tile(beta, (2, 1))), None, W.identity_r())
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# ---- rotation block sizes 16 / 64 / 128 (DuQuant++ page sec. 4.3) ----------

def _block_diag(blocks):
    n = sum(b.shape[0] for b in blocks)
    out = np.zeros((n, n))
    o = 0
    for b in blocks:
        k = b.shape[0]
        out[o:o + k, o:o + k] = b
        o += k
    return out


def pin_block32_is_rotate_quant(orc):
    """B = 32 through the block entry is exactly the 32-wide rotation."""
    rng = _rng(51)
    x = W.random_activations(rng, 7, 256, torch.bfloat16, scale=4.0)
    lam = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    a = orc.rotate_quant_block(x, lam, r, want_y=True)
    b = orc.rotate_quant(x, lam, r, want_y=True)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def pin_block_embeddings(orc):
    """A B-block equals the 2B-block that holds it twice on the diagonal
    (the zero entries add exact zeros): 16 in 32, 32 in 64, 64 in 128."""
    rng = _rng(52)
    x = W.random_activations(rng, 5, 512, torch.float16, scale=2.0)
    lam = rng.uniform(0.5, 2.0, 512).astype(np.float32)
    for B in (16, 32, 64):
        rb = W.qr_orthogonal(rng, B)
        small = orc.rotate_quant_block(x, lam, rb, want_y=True)
        big = orc.rotate_quant_block(x, lam, _block_diag([rb, rb]), want_y=True)
        assert all(np.array_equal(u, v) for u, v in zip(small, big)), B


def pin_block_dense_product(orc):
    """y = (x / lam) BlockDiag(R_B) as one dense fp64 product, for a
    non-symmetric R at every block size."""
    rng = _rng(53)
    x = W.random_activations(rng, 4, 256, torch.bfloat16, scale=3.0)
    lam = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    xs = x.to(torch.float64).numpy() / lam.astype(np.float64)[None, :]
    for B in (16, 32, 64, 128):
        rb = rng.standard_normal((B, B))
        _, _, y = orc.rotate_quant_block(x, lam, rb, want_y=True)
        dense = xs @ _block_diag([rb] * (256 // B))
        assert np.abs(y - dense).max() <= 1e-12 * np.abs(dense).max(), B


def pin_block_norm_preservation(orc):
    """An orthogonal B-block keeps the norm of every B-channel block."""
    rng = _rng(54)
    x = W.random_activations(rng, 6, 512, torch.bfloat16, scale=5.0)
    xs = x.to(torch.float64).numpy()
    for B in (16, 64, 128):
        rb = W.random_hadamard(rng, B)
        _, _, y = orc.rotate_quant_block(x, None, rb, want_y=True)
        ny = np.linalg.norm(y.reshape(6, -1, B), axis=2)
        nx = np.linalg.norm(xs.reshape(6, -1, B), axis=2)
        assert np.abs(ny - nx).max() <= 1e-12 * nx.max(), B


ALL_PINS = [
    pin_worked_example,
    pin_config1_massive_value,
    pin_bruteforce_codec,
    pin_scale_clamps,
    pin_scale_window,
    pin_identity_rotation,
    pin_dense_blockdiag,
    pin_norm_preservation,
    pin_equivariance,
    pin_lambda_powers_of_two,
    pin_strided_input,
    pin_input_decoding,
    pin_dequant,
    pin_encode_groups_matches_quant,
    pin_norm_alternating_closed_form,
    pin_norm_reduces_to_rotate_quant,
    pin_norm_eps_under_root,
    pin_norm_scale_invariance,
    pin_layernorm_shift_invariance,
    pin_norm_gamma_lambda_refactoring,
    pin_norm_zero_row,
    pin_block32_is_rotate_quant,
    pin_block_embeddings,
    pin_block_dense_product,
    pin_block_norm_preservation,
]
