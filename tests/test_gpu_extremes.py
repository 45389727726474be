"""Inputs at the ends of the contract's range, on an MI355X through the C ABI,
against the fp64 oracle.

The MXFP4 scale comes from each group's own maximum (DuQuant++ page sec. 2.1)
and the smoothing factor is any per-channel value (sec. 3.1), so a group can
sit anywhere in fp32's range: every finite bf16 and fp16 bit pattern, groups
of subnormal size, smoothing factors up to 2^126, and norm rows whose squares
leave fp32's range (sec. 5.2 item 1).  The fused path then recomputes groups
whose rotated maximum is below 2^-64 at a power-of-two shift, and the norm
path rescales bf16 rows whose sum of squares leaves [2^-80, 2^1000]; these
tests reach every such branch.

With a signed permutation block (every product exact) and power-of-two
smoothing (exact division), the kernel's result is the oracle's bit for bit;
with general blocks and factors the tie-aware tolerance rule applies."""
import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq
import oracle as O
import workloads as W
from parity import (check_against_oracle, check_rotated_values, check_same_precision,
                    smoothed_group_norms)

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


def every_pattern(dtype, shuffle_seed=None, width=256):
    """Every finite bit pattern of a 16-bit float type as rows of `width`
    (the tail that does not fill a row dropped), in bit order or shuffled."""
    bits = torch.arange(0, 0x10000, dtype=torch.int32).to(torch.int16)
    v = bits.view(dtype)
    v = v[torch.isfinite(v)]
    if shuffle_seed is not None:
        perm = np.random.default_rng(shuffle_seed).permutation(v.numel())
        v = v[torch.from_numpy(perm)]
    return v[: v.numel() // width * width].reshape(-1, width).contiguous()


def signed_permutation(seed):
    rng = np.random.default_rng(seed)
    p = np.zeros((GROUP, GROUP))
    p[np.arange(GROUP), rng.permutation(GROUP)] = rng.choice(np.array([-1.0, 1.0]), GROUP)
    return W.bf16_matrix(p)


def run_fused(x, lam, r, dev, want_y=True):
    y = torch.empty(x.shape, dtype=torch.float32, device=dev) if want_y else None
    codes, scales = mxq.rotate_quant(x.to(dev), r.contiguous().to(dev), _f32(lam, dev), y_rot=y)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (y.cpu().numpy() if want_y else None)


def rule_check(x, lam, r, dev, orc, label):
    """Every output against the oracle under the tolerance rule, and the
    product entry point bit-identical to the one that also stores y."""
    codes, scales, y = run_fused(x, lam, r, dev)
    c2, s2, _ = run_fused(x, lam, r, dev, want_y=False)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    c_ref, s_ref, y_ref = orc.rotate_quant(x, lam, r, want_y=True)
    norms = smoothed_group_norms(x, lam)
    worst = check_rotated_values(y, y_ref, norms)
    skipped = check_same_precision(y, codes, scales, orc)
    stats = check_against_oracle(codes, scales, c_ref, s_ref, lambda rows: y_ref[rows], norms)
    tiny = int((scales < 61).sum())
    print(f"  {label}: {stats}, worst {worst:.2e}, tiny groups {tiny}, subnormal-output groups {skipped}",
          flush=True)
    return codes, scales, tiny


# ---- every bit pattern ----------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shuffle", [None, 5])
def test_identity_block_every_pattern(dev, orc, dtype, shuffle):
    """R = I: the fused path is plain MXFP4 bit for bit, for every finite
    pattern (in bit order, groups of like magnitude including all-subnormal
    ones; shuffled, groups of mixed magnitude), with and without lambda = 1."""
    x = every_pattern(dtype, shuffle)
    c_q, s_q = mxq.quant(x.to(dev))
    c_ref, s_ref = orc.quant(x)
    assert np.array_equal(s_q.cpu().numpy(), s_ref) and np.array_equal(c_q.cpu().numpy(), c_ref)
    for lam in (None, np.ones(x.shape[1], np.float32)):
        codes, scales, _ = run_fused(x, lam, W.identity_r(), dev, want_y=False)
        assert np.array_equal(scales, s_ref), int((scales != s_ref).sum())
        assert np.array_equal(codes, c_ref), int((codes != c_ref).sum())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_signed_permutation_long_batch(dev, orc, dtype):
    """Every pattern in bit order (groups of like magnitude) repeated to
    about 35000 rows (each wave of the row-major smoothed instance takes 18
    batches of rows; the tests above, at 250 rows, run the short-batch
    instance), lambda = 2^120 (every group far below 2^-64, so every row goes
    through the pass that redoes rows), a signed permutation block: bit for
    bit."""
    x = torch.cat([every_pattern(dtype)] * 140).contiguous()
    C = x.shape[1]
    lam = np.full(C, np.ldexp(1.0, 120), np.float32)
    r = signed_permutation(15)
    codes, scales, y = run_fused(x, lam, r, dev)
    c_ref, s_ref, y_ref = orc.rotate_quant(x, lam, r, want_y=True)
    assert np.array_equal(scales, s_ref), int((scales != s_ref).sum())
    assert np.array_equal(codes, c_ref), int((codes != c_ref).sum())
    check_rotated_values(y, y_ref, smoothed_group_norms(x, lam))
    assert (scales < 61).sum() > 0
    print(f"  {dtype} long batch: tiny groups {int((scales < 61).sum())}", flush=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("lam_exp", [None, 60, 120, 126, -126, "mixed"])
def test_signed_permutation_every_pattern(dev, orc, dtype, lam_exp):
    """A signed permutation block and power-of-two lambda make every product
    and quotient exact, so codes and scales equal the oracle's bit for bit at
    every pattern, including lambda = 2^126 (smoothed values down to 2^-259)
    and per-channel exponents spread over [-126, 126]."""
    for shuffle in (None, 11):
        x = every_pattern(dtype, shuffle)
        C = x.shape[1]
        if lam_exp is None:
            lam = None
        elif lam_exp == "mixed":
            e = np.random.default_rng(12).integers(-126, 127, C)
            if dtype == torch.float16:
                e = np.maximum(e, -100)  # keep x / lambda below fp32's overflow for fp16's 65504
            lam = np.ldexp(1.0, e).astype(np.float32)
        else:
            lam = np.full(C, np.ldexp(1.0, lam_exp), np.float32)
        if lam is not None:
            # keep x / lambda finite in fp32 (bf16 values reach 2^128)
            big = torch.abs(x.to(torch.float64)).numpy() / lam.astype(np.float64)[None, :] >= 2.0 ** 127
            x = x.clone()
            x[torch.from_numpy(big)] = 0
        r = signed_permutation(13 + (shuffle or 0))
        codes, scales, y = run_fused(x, lam, r, dev)
        c_ref, s_ref, y_ref = orc.rotate_quant(x, lam, r, want_y=True)
        assert np.array_equal(scales, s_ref), int((scales != s_ref).sum())
        assert np.array_equal(codes, c_ref), int((codes != c_ref).sum())
        check_rotated_values(y, y_ref, smoothed_group_norms(x, lam))
        print(f"  {dtype} lambda={lam_exp} shuffle={shuffle}: tiny groups {int((scales < 61).sum())}", flush=True)


# ---- general blocks and factors ------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("lam_exp", [100, 115, 118, 120, 124, 126])
def test_large_lambda_general_block(dev, orc, dtype, lam_exp):
    """N(0,1) activations divided by lambda = 2^e * U(1/2, 1) (up to the
    contract's 2^126): at e >= 115 the smoothed groups are far below 2^-64 (a
    bf16 term split of them would lose 5e-5 of the group norm at e = 120); a
    seeded orthogonal block."""
    rng = np.random.default_rng(8000 + lam_exp + 7 * (dtype == torch.float16))
    T, C = 96, 2048 + 640
    x = W.random_activations(rng, T, C, dtype)
    lam = (np.ldexp(1.0, lam_exp) * rng.uniform(0.5, 1.0, C)).astype(np.float32)
    lam[rng.choice(C, 64, replace=False)] = rng.uniform(0.5, 2.0, 64)  # a few normal channels
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    _, _, tiny = rule_check(x, lam, r, dev, orc, f"{dtype} lambda 2^{lam_exp}")
    assert tiny > 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("T", [300, 12000])
def test_mixed_magnitudes_in_one_batch(dev, orc, dtype, T):
    """Rows of ordinary size, rows scaled into the subnormal range, and rows
    with single tiny groups, so the pass that redoes rows meets rows with
    both kinds of groups; with lambda of every size in [2^-60, 2^120].
    300 rows launch the short-batch instance (block-shared factors), 12000
    rows (18 batches of rows per wave) the row-major one."""
    rng = np.random.default_rng(8100 + (dtype == torch.float16) + 2 * (T > 300))
    C = 4096 + 1024
    x = rng.standard_normal((T, C))
    lam = np.ldexp(1.0, rng.integers(-60, 121, C)).astype(np.float32) * rng.uniform(1, 2, C).astype(np.float32)
    if dtype == torch.bfloat16:
        x[::7] *= 2.0 ** -128  # bf16 subnormal rows
    else:
        x[::7] *= 2.0 ** -20   # fp16 subnormal rows
    g = rng.choice(C // GROUP, 40)
    for t, gi in zip(rng.choice(T, 40), g):
        x[t, gi * GROUP:(gi + 1) * GROUP] *= 2.0 ** -60
    x = W.to_dtype(x, dtype)
    big = torch.abs(x.to(torch.float64)).numpy() / lam.astype(np.float64)[None, :] >= 2.0 ** 120
    x[torch.from_numpy(big)] = 0
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    _, _, tiny = rule_check(x, lam, r, dev, orc, f"{dtype} mixed magnitudes")
    assert tiny > 0


def test_bf16_subnormal_activations_without_lambda(dev, orc):
    """bf16 activations of subnormal size, no smoothing: one bf16 term, but
    products below fp32's normal range; redone at a shift of 2^64."""
    rng = np.random.default_rng(8200)
    x = rng.standard_normal((64, 1024)) * 2.0 ** -130
    x[:, :256] *= 2.0 ** 70  # some groups of ordinary tiny size (2^-60)
    x = W.to_dtype(x, torch.bfloat16)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    _, _, tiny = rule_check(x, None, r, dev, orc, "bf16 subnormal, no lambda")
    assert tiny > 0


def test_tiled_output_of_tiny_groups(dev):
    """The fragment-tiled quantizer redoes the same groups (the 16-row-unit
    store path at 4700 x 14336 and the per-row path at 40 rows): its bytes
    equal the repacked row-layout output."""
    rng = np.random.default_rng(8300)
    for T in (40, 4700):
        C = 14336
        x = rng.standard_normal((T, C)).astype(np.float32)
        x[rng.choice(T, 50)] *= 2.0 ** -100
        x = W.to_dtype(x, torch.bfloat16)
        lam = (np.ldexp(1.0, 30) * rng.uniform(1, 2, C)).astype(np.float32)
        r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
        xd, ld = x.to(dev), _f32(lam, dev)
        codes, scales = mxq.rotate_quant(xd, r, ld)
        tc, ts = mxq.rotate_quant_tiled(xd, r, ld)
        torch.cuda.synchronize()
        codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
        assert int((scales < 61).sum()) > 0
        uc, us = O.untile_mxfp4(tc.cpu().numpy(), ts.cpu().numpy(), T, C)
        assert np.array_equal(uc, codes) and np.array_equal(us, scales)


# ---- norm path -------------------------------------------------------------------

def run_norm(x, r, gamma, beta, lam, norm, eps, dev, want_y=True):
    y = torch.empty(x.shape, dtype=torch.float32, device=dev) if want_y else None
    codes, scales = mxq.norm_rotate_quant(x.to(dev), r.to(dev), _f32(gamma, dev), _f32(beta, dev), _f32(lam, dev),
                                          norm=norm, eps=eps, y_rot=y)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (y.cpu().numpy() if want_y else None)


def norm_check(x, r, gamma, beta, lam, norm, eps, dev, orc, label):
    codes, scales, y = run_norm(x, r, gamma, beta, lam, norm, eps, dev)
    c2, s2, _ = run_norm(x, r, gamma, beta, lam, norm, eps, dev, want_y=False)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    eps32 = float(np.float32(eps))  # the kernel receives eps as fp32
    c_ref, s_ref, y_ref = orc.norm_rotate_quant(x, norm, gamma, beta, eps32, lam, r, want_y=True)
    T, C = y_ref.shape
    norms = np.linalg.norm(y_ref.reshape(T, C // GROUP, GROUP), axis=2)
    worst = check_rotated_values(y, y_ref, norms)
    skipped = check_same_precision(y, codes, scales, orc)
    stats = check_against_oracle(codes, scales, c_ref, s_ref, lambda rows: y_ref[rows], norms)
    print(f"  {label}: {stats}, worst {worst:.2e}, tiny groups {int((scales < 61).sum())}, "
          f"subnormal-output groups {skipped}", flush=True)
    if C % 128 == 0:
        tc, ts = mxq.norm_rotate_quant_tiled(x.to(dev), r.to(dev), _f32(gamma, dev), _f32(beta, dev),
                                             _f32(lam, dev), norm=norm, eps=eps)
        torch.cuda.synchronize()
        uc, us = O.untile_mxfp4(tc.cpu().numpy(), ts.cpu().numpy(), T, C)
        assert np.array_equal(uc, codes) and np.array_equal(us, scales)
    return codes, scales


def extreme_rows(dtype, T, C, seed):
    """Rows of ordinary size mixed with rows at the ends of the 16-bit range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, C))
    kinds = []
    for t in range(T):
        k = t % 6
        if dtype == torch.bfloat16:
            scale = [1.0, 2.0 ** -80, 2.0 ** 70, 2.0 ** -128, 2.0 ** 100, 1.0][k]
        else:
            scale = [1.0, 2.0 ** -19, 2.0 ** 12, 2.0 ** -22, 1.0, 1.0][k]
        x[t] *= scale
        if k == 5:  # one massive outlier: the other groups normalize to tiny values
            x[t, rng.integers(C)] = 2.0 ** 90 if dtype == torch.bfloat16 else 60000.0
        kinds.append(k)
    return W.to_dtype(x, dtype)


@pytest.mark.parametrize("norm", ["rms", "layer"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("eps", [0.0, 1e-5])
@pytest.mark.parametrize("T,C", [(48, 1024), (40, 4096), (12, 16384)])
def test_norm_extreme_rows(dev, orc, norm, dtype, eps, T, C):
    """Rows at |h| ~ 2^-80, 2^70, 2^100 and bf16-subnormal size (fp16: its
    subnormal range and 2^12), with eps = 0 and 1e-5, RMS and LayerNorm, and
    bf16 rows with one 2^90 outlier (squares out of range) whose other groups
    normalize far below 2^-64."""
    x = extreme_rows(dtype, T, C, 8400 + C + T)
    rng = np.random.default_rng(8500 + C)
    gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32) if norm == "layer" else None
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    norm_check(x, r, gamma, beta, lam, norm, eps, dev, orc, f"norm={norm} {dtype} eps={eps} {T}x{C}")


@pytest.mark.parametrize("norm", ["rms", "layer"])
def test_norm_small_factors(dev, orc, norm):
    """gamma / lambda near 2^-64 (the factors' lower limit), on rows whose
    one large value leaves the other channels' normalized size near 2^-8,
    puts whole groups of the smoothed output below 2^-64, redone at a shift;
    half the channels keep ordinary factors."""
    rng = np.random.default_rng(8600)
    T, C = 64, 2048
    x = rng.standard_normal((T, C))
    x[np.arange(T), rng.integers(0, C, T)] = 2000.0
    x = W.to_dtype(x, torch.bfloat16)
    gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    lam[C // 2:] = (np.ldexp(1.0, 62) * rng.uniform(1.0, 1.9, C // 2)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32) if norm == "layer" else None
    if beta is not None:
        beta[C // 2:] = 0.0  # beta / lambda is 0 there (nonzero factors must reach 2^-64)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    _, scales = norm_check(x, r, gamma, beta, lam, norm, 1e-5, dev, orc, f"norm={norm} small factors")
    assert int((scales < 61).sum()) > 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("T,C", [(64, 4096), (4200, 2048)])
def test_norm_zero_rows_among_tiny_groups(dev, orc, dtype, T, C):
    """RMSNorm without beta: rows and groups of zeros skip the pass that
    redoes rare rows (their x' is exactly 0), while tiny nonzero groups
    next to them, in the same row or wave, are still redone.  Row kinds:
    all zero; extreme rows; half the groups zero and the rest tiny; all
    groups zero but one holding a large value next to tiny ones."""
    rng = np.random.default_rng(8900 + C + T)
    tiny = 2.0 ** -80 if dtype == torch.bfloat16 else 2.0 ** -22
    big = 2.0 ** 60 if dtype == torch.bfloat16 else 30000.0
    x = extreme_rows(dtype, T, C, 8950 + C).float().numpy().astype(np.float64)
    for t in range(T):
        k = t % 4
        if k == 0:
            x[t] = 0.0
        elif k == 2:
            x[t, : C // 2] = 0.0
            x[t, C // 2:] = tiny * rng.standard_normal(C - C // 2)
        elif k == 3:
            x[t] = 0.0
            g = int(rng.integers(C // 32))
            x[t, 32 * g: 32 * g + 32] = tiny * rng.standard_normal(32)
            x[t, 32 * g + int(rng.integers(32))] = big
    x = W.to_dtype(x, dtype)
    gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
    lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    codes, scales = norm_check(x, r, gamma, None, lam, "rms", 1e-5, dev, orc, f"zero rows {dtype} {T}x{C}")
    assert not codes[0::4].any() and not scales[0::4].any()


def test_norm_long_batch_staged_with_extreme_rows(dev, orc):
    """The staged tiled path (8- and 16-wave blocks) with rows to redo: the
    block's record stores complete before the rewrites."""
    for T, C in ((4200, 2048), (2100, 8192)):
        x = extreme_rows(torch.bfloat16, T, C, 8700 + C)
        rng = np.random.default_rng(8800 + C)
        gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
        lam = np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)
        r = W.bf16_matrix(W.qr_orthogonal(rng))
        norm_check(x, r, gamma, None, lam, "rms", 0.0, dev, orc, f"staged {T}x{C}")


# ---- block-size kernel -------------------------------------------------------------

@pytest.mark.parametrize("B", [16, 32, 64, 128])
@pytest.mark.parametrize("case", ["lambda", "subnormal"])
def test_block_sizes_tiny_blocks(dev, orc, B, case):
    """Rotation blocks whose inputs are all tiny (lambda ~ 2^120, or bf16
    subnormal activations): redone at a shift, against the oracle with each
    output's block norm as the scale."""
    rng = np.random.default_rng(8900 + B + (case == "subnormal"))
    T, C = 64, 2048 + 512
    x = rng.standard_normal((T, C))
    if case == "lambda":
        lam = (np.ldexp(1.0, 120) * rng.uniform(1, 2, C)).astype(np.float32)
        lam[: C // 4] = rng.uniform(0.5, 2, C // 4)
    else:
        x[:, C // 4:] *= 2.0 ** -129
        lam = None
    x = W.to_dtype(x, torch.bfloat16)
    r = W.bf16_matrix(W.qr_orthogonal(rng, B))
    y = torch.empty(x.shape, dtype=torch.float32, device=dev)
    codes, scales = mxq.rotate_quant_block(x.to(dev), r.to(dev), _f32(lam, dev), y_rot=y)
    torch.cuda.synchronize()
    codes, scales, y = codes.cpu().numpy(), scales.cpu().numpy(), y.cpu().numpy()
    c_ref, s_ref, y_ref = orc.rotate_quant_block(x, lam, r, want_y=True)
    if B <= GROUP:
        norms = np.linalg.norm(y_ref.reshape(T, C // GROUP, GROUP), axis=2)
    else:
        norms = np.repeat(np.linalg.norm(y_ref.reshape(T, C // B, B), axis=2), B // GROUP, axis=1)
    check_rotated_values(y, y_ref, norms)
    check_same_precision(y, codes, scales, orc)
    stats = check_against_oracle(codes, scales, c_ref, s_ref, lambda rows: y_ref[rows], norms)
    assert int((scales < 61).sum()) > 0
    print(f"  B={B} {case}: {stats}", flush=True)


# ---- the binding refuses host tensors before any launch ------------------------------

def test_binding_rejects_host_tensors(dev):
    """A host tensor's address must never reach a kernel: every tensor the
    binding hands to the library is checked for the call's device first."""
    wl = W.make_config(1)
    x = wl.x.to(dev)
    r = wl.r_hat.to(dev)
    T, C = x.shape
    with pytest.raises(ValueError):
        mxq.rotate_quant(x, r, y_rot=torch.empty((T, C), dtype=torch.float32))
    with pytest.raises(ValueError):
        mxq.rotate_quant_block(x, r, y_rot=torch.empty((T, C), dtype=torch.float32))
    g = torch.ones(C, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        mxq.norm_rotate_quant(x, r, g, y_rot=torch.empty((T, C), dtype=torch.float32))
    codes, scales = mxq.quant(x)
    with pytest.raises(ValueError):
        mxq.dequant(codes, scales, out=torch.empty((T, C), dtype=torch.float32))
    with pytest.raises(ValueError):
        mxq.dequant(codes, scales.cpu())
    with pytest.raises(ValueError):
        mxq.tile_mxfp4(codes, scales.cpu())
    with pytest.raises(ValueError):
        mxq.gemm_mxfp4(codes, scales, codes, scales, out=torch.empty((T, T), dtype=torch.float32))
    with pytest.raises(ValueError):
        mxq.gemm_mxfp4(codes, scales, codes.cpu(), scales)
    tc, ts = mxq.tile_mxfp4(codes, scales)
    with pytest.raises(ValueError):
        mxq.gemm_mxfp4_tiled(tc, ts, tc, ts, T, T, C, out=torch.empty((T, T), dtype=torch.float32))
    with pytest.raises(ValueError):
        mxq.calib_worst_group(x, torch.ones(C, dtype=torch.float32))
    torch.cuda.synchronize()
