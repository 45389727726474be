"""The MXFP4 consumer on an MI355X: absorbed-weight quantization and the
W4A4 product, through the C ABI, against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq
import oracle as O
import workloads as W
from parity import check_against_oracle, check_same_precision

pytestmark = pytest.mark.gpu
GROUP = 32
U = 2.0 ** -24


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mxq.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return O.default()


def _dev_u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gemm_gpu(ac, asc, bc, bsc, dev, out_dtype=torch.float32, out=None):
    y = mxq.gemm_mxfp4(_dev_u8(ac, dev), _dev_u8(asc, dev), _dev_u8(bc, dev), _dev_u8(bsc, dev),
                       out_dtype, out=out)
    torch.cuda.synchronize()
    return y


def check_product(y, ref, s_abs, K, where=""):
    """fp32 accumulation bound: |y - exact| <= 2 K 2^-24 sum |products|."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    bound = 2.0 * K * U * s_abs
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{where}: {len(bad)} outputs outside the bound, first {bad[:3].tolist()}"
    rel = err / np.maximum(s_abs, np.finfo(np.float64).tiny)
    return float(rel.max())


@pytest.mark.parametrize("M,N,K", [(16, 16, 256), (128, 128, 512), (1, 1, 256), (200, 130, 768),
                                   (300, 257, 1024), (129, 383, 2048), (64, 640, 4096), (33, 70, 128),
                                   (100, 300, 384), (513, 260, 1152), (700, 2300, 256), (1100, 1500, 384)])
def test_gemm_random_operands(dev, orc, M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    ac, asc = W.random_mxfp4(rng, M, K)
    bc, bsc = W.random_mxfp4(rng, N, K)
    print(f"  gemm M={M} N={N} K={K}", flush=True)
    ref, s_abs = O.gemm_mxfp4(ac, asc, bc, bsc, orc)
    y = gemm_gpu(ac, asc, bc, bsc, dev).cpu().numpy()
    worst = check_product(y, ref, s_abs, K, f"{M}x{N}x{K}")
    print(f"    worst |err| / sum|products| = {worst:.3g}", flush=True)
    # bf16 output: the round-to-nearest-even of the same fp32 sums
    yb = gemm_gpu(ac, asc, bc, bsc, dev, torch.bfloat16).cpu()
    assert torch.equal(yb.view(torch.int16), torch.from_numpy(y).to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(1, 4096, 14336), (7, 100, 128), (16, 4096, 4096), (17, 300, 1152),
                                   (40, 64, 2048), (64, 1000, 14336), (16, 16, 256), (65, 300, 1152),
                                   (128, 4096, 2048), (100, 1000, 1024), (97, 70, 14336)])
def test_gemm_decode_shapes(dev, orc, M, N, K):
    """Decode-shaped products (the path for M <= 64 splits K over the waves
    of a block and sums the partial tiles in a fixed order), and small
    batches of 65 to 128 rows, which run the same kernel with one block row
    per 64 rows (ragged last block row included)."""
    rng = np.random.default_rng(M * 131 + N * 17 + K + 5)
    ac, asc = W.random_mxfp4(rng, M, K)
    bc, bsc = W.random_mxfp4(rng, N, K)
    ref, s_abs = O.gemm_mxfp4(ac, asc, bc, bsc, orc)
    y = gemm_gpu(ac, asc, bc, bsc, dev).cpu().numpy()
    worst = check_product(y, ref, s_abs, K, f"{M}x{N}x{K}")
    print(f"  decode gemm M={M} N={N} K={K}: worst |err| / sum|products| = {worst:.3g}", flush=True)
    yb = gemm_gpu(ac, asc, bc, bsc, dev, torch.bfloat16).cpu()
    assert torch.equal(yb.view(torch.int16), torch.from_numpy(y).to(torch.bfloat16).view(torch.int16))
    y2 = gemm_gpu(ac, asc, bc, bsc, dev).cpu().numpy()
    assert np.array_equal(y, y2)  # fixed reduction order


def test_gemm_one_hot_products(dev, orc):
    """Each output picks exactly one product: codes one-hot along K with the
    extreme magnitudes and a wide spread of scales (exact results)."""
    M, N, K = 32, 48, 512
    rng = np.random.default_rng(11)
    ac = np.zeros((M, K // 2), np.uint8)
    bc = np.zeros((N, K // 2), np.uint8)
    ka = rng.integers(0, K, M)
    for m in range(M):
        code = int(rng.integers(1, 16)) or 1
        ac[m, ka[m] // 2] = code << (4 * (ka[m] % 2))
    for n in range(N):
        kb = ka[n % M]  # output (n % M, n) has one product, others have none
        code = int(rng.integers(1, 16)) or 1
        bc[n, kb // 2] = code << (4 * (kb % 2))
    asc = rng.integers(60, 190, (M, K // GROUP)).astype(np.uint8)
    bsc = rng.integers(60, 190, (N, K // GROUP)).astype(np.uint8)
    ref, _ = O.gemm_mxfp4(ac, asc, bc, bsc, orc)
    y = gemm_gpu(ac, asc, bc, bsc, dev).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


def test_gemm_strided_output_and_tails(dev, orc):
    M, N, K = 70, 90, 256
    rng = np.random.default_rng(12)
    ac, asc = W.random_mxfp4(rng, M, K)
    bc, bsc = W.random_mxfp4(rng, N, K)
    base = torch.full((M, 100), 7.25, dtype=torch.float32, device=dev)
    out = base[:, :N]
    gemm_gpu(ac, asc, bc, bsc, dev, out=out)
    ref, s_abs = O.gemm_mxfp4(ac, asc, bc, bsc, orc)
    full = base.cpu().numpy()
    check_product(full[:, :N], ref, s_abs, K, "strided")
    assert np.all(full[:, N:] == 7.25)  # columns past N untouched


def _sparse_operand(rng, rows, K, positions, per_row):
    """MXFP4 operand that is zero except per_row codes in each row, drawn from
    positions (nonzero magnitudes), with scales in 2^-2..2^2 so that every sum
    of a few products is exact in fp32."""
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = rng.integers(125, 130, size=(rows, K // 32), dtype=np.uint8)
    for i in range(rows):
        for p in rng.choice(positions, size=per_row, replace=False):
            c = int(rng.integers(1, 8)) | (8 if rng.integers(0, 2) else 0)
            codes[i, p // 2] |= np.uint8(c << (4 * (p % 2)))
    return codes, scales


@pytest.mark.parametrize("M", [3, 80])
def test_gemm_max_k_sparse_exact(dev, orc, M):
    """K = 2^24, the largest the header allows: record and byte offsets of
    every operand reach their maximum.  Nonzero codes sit at positions spread
    over all of K (first and last included); the expected values are the
    oracle's product over just the groups that hold them (zero codes add
    nothing), and every output is exact in fp32, so both layouts must match
    it exactly, on the decode-shaped kernel (M = 3) and the tiled one."""
    K, N = 1 << 24, 24
    rng = np.random.default_rng(4242 + M)
    pos = np.unique(np.concatenate([[0, K - 1, K // 2, K - 32, 31],
                                    rng.choice(K, size=40, replace=False)]))
    ac, asc = _sparse_operand(rng, M, K, pos, 4)
    bc, bsc = _sparse_operand(rng, N, K, pos, 8)
    groups = np.unique(pos // 32)
    cols = (groups[:, None] * 16 + np.arange(16)[None, :]).ravel()
    ref, _ = O.gemm_mxfp4(ac[:, cols], asc[:, groups], bc[:, cols], bsc[:, groups], orc)
    assert np.count_nonzero(ref) > 0
    print(f"  K=2^24 M={M} N={N}: {len(groups)} groups hold nonzeros, "
          f"{np.count_nonzero(ref)} nonzero outputs", flush=True)
    a = [_dev_u8(t, dev) for t in (ac, asc)]
    b = [_dev_u8(t, dev) for t in (bc, bsc)]
    y = mxq.gemm_mxfp4(*a, *b, torch.float32)
    yt = mxq.gemm_mxfp4_tiled(*mxq.tile_mxfp4(*a), *mxq.tile_mxfp4(*b), M, N, K, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(yt.cpu().numpy().astype(np.float64), ref)


def test_gemm_empty_and_zero_k(dev):
    z = torch.empty((0, 128), dtype=torch.uint8, device=dev)
    zs = torch.empty((0, 8), dtype=torch.uint8, device=dev)
    b = torch.zeros((5, 128), dtype=torch.uint8, device=dev)
    bs = torch.zeros((5, 8), dtype=torch.uint8, device=dev)
    assert mxq.gemm_mxfp4(z, zs, b, bs).shape == (0, 5)
    a0 = torch.empty((3, 0), dtype=torch.uint8, device=dev)
    b0 = torch.empty((4, 0), dtype=torch.uint8, device=dev)
    y = torch.full((3, 4), 5.0, device=dev)
    mxq.gemm_mxfp4(a0, a0, b0, b0, out=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_gemm_nan_scale(dev):
    """E8M0 0xFF is NaN (OCP MX v1.0): a row with a NaN scale gives NaN."""
    M, N, K = 16, 16, 256
    rng = np.random.default_rng(13)
    ac, asc = W.random_mxfp4(rng, M, K)
    bc, bsc = W.random_mxfp4(rng, N, K)
    asc[3, 2] = 0xFF
    y = gemm_gpu(ac, asc, bc, bsc, dev).cpu().numpy()
    assert np.all(np.isnan(y[3])) and not np.any(np.isnan(np.delete(y, 3, axis=0)))


# ---- weight absorption ------------------------------------------------------------

def _absorb_check(w, lam, r, dev, orc):
    lam_d = None if lam is None else torch.from_numpy(lam).to(dev)
    codes, scales = mxq.absorb_quant(w.to(dev), r.to(dev), lam_d)
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    c_ref, s_ref = O.absorb_quant(w, lam, r, orc)
    y_ref = O.absorb_weights(w, lam, r)
    wl = w.to(torch.float64).numpy()
    if lam is not None:
        wl = wl * lam.astype(np.float64)[None, :]
    norms = np.linalg.norm(wl.reshape(wl.shape[0], -1, GROUP), axis=2)
    return check_against_oracle(codes, scales, c_ref, s_ref, lambda rows: y_ref[rows], norms), codes, scales


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_absorb_quant_against_oracle(dev, orc, dtype):
    rng = np.random.default_rng(21)
    N, K = 384, 4096
    w = W.linear_weights(N, K, seed=22, dtype=dtype)
    lam = np.exp(0.5 * rng.standard_normal(K)).astype(np.float32)
    r = W.bf16_matrix(W.qr_orthogonal(rng))
    for lam_case in (lam, None):
        stats, _, _ = _absorb_check(w, lam_case, r, dev, orc)
        print(f"  absorb {dtype} lambda={'yes' if lam_case is not None else 'no'}: {stats}", flush=True)


def test_absorb_identity_is_plain_quant(dev):
    w = W.linear_weights(64, 512, seed=23)
    c1, s1 = mxq.absorb_quant(w.to(dev), W.identity_r().to(dev))
    c2, s2 = mxq.quant(w.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


# ---- the whole consumer: rotate + quantize X, absorb + quantize W, multiply ---------

def _pipeline(x, lam, r, w, dev):
    xd = x.to(dev)
    lam_d = None if lam is None else torch.from_numpy(lam).to(dev)
    rd = r.to(dev)
    ac, asc = mxq.rotate_quant(xd, rd, lam_d)
    bc, bsc = mxq.absorb_quant(w.to(dev), rd, lam_d)
    y = mxq.gemm_mxfp4(ac, asc, bc, bsc)
    torch.cuda.synchronize()
    return ac, asc, bc, bsc, y


def test_consumer_pipeline_config2(dev, orc):
    """Config-2 activations (2048 x 4096, lambda) through a 4096 -> 1024
    layer: the product stage against the oracle on the GPU's own operands,
    and the W4A4 result against the exact X W (a quantization-error report)."""
    wl = W.make_config(2)
    w = W.linear_weights(1024, wl.channels, seed=24)
    ac, asc, bc, bsc, y = _pipeline(wl.x, wl.lam, wl.r_hat, w, dev)
    ac, asc, bc, bsc = (t.cpu().numpy() for t in (ac, asc, bc, bsc))
    ref, s_abs = O.gemm_mxfp4(ac, asc, bc, bsc, orc)
    check_product(y.cpu().numpy(), ref, s_abs, wl.channels, "config 2 pipeline")
    exact = wl.x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
    rel = np.linalg.norm(y.cpu().numpy() - exact) / np.linalg.norm(exact)
    print(f"  W4A4 relative Frobenius error vs exact X W: {rel:.4f}", flush=True)
    assert rel < 0.5


def test_consumer_full_size_sampled(dev, orc):
    """The down_proj-shaped product the bench times (8192 x 14336 activations
    of config 3, 4096 outputs), checked on 512 sampled outputs."""
    wl = W.make_config(3)
    w = W.linear_weights(W.DOWN_PROJ_OUT, wl.channels)
    ac, asc, bc, bsc, y = _pipeline(wl.x, wl.lam, wl.r_hat, w, dev)
    rng = np.random.default_rng(25)
    ms = rng.integers(0, wl.tokens, 512)
    ns = rng.integers(0, W.DOWN_PROJ_OUT, 512)
    um, un = np.unique(ms), np.unique(ns)
    da = orc.dequant(ac[torch.from_numpy(um).to(dev)].cpu().numpy(), asc[torch.from_numpy(um).to(dev)].cpu().numpy())
    db = orc.dequant(bc[torch.from_numpy(un).to(dev)].cpu().numpy(), bsc[torch.from_numpy(un).to(dev)].cpu().numpy())
    ia = np.searchsorted(um, ms)
    ib = np.searchsorted(un, ns)
    ref = np.einsum("ik,ik->i", da[ia], db[ib])
    s_abs = np.einsum("ik,ik->i", np.abs(da[ia]), np.abs(db[ib]))
    got = y[torch.from_numpy(ms).to(dev), torch.from_numpy(ns).to(dev)].cpu().numpy()
    worst = check_product(got, ref, s_abs, wl.channels, "full size")
    print(f"  full-size sampled worst |err| / sum|products| = {worst:.3g}", flush=True)
    assert not torch.isnan(y).any().item()


@pytest.mark.parametrize("cfg,smooth", [(3, False), (5, True), (5, False)])
def test_consumer_error_by_block(dev, orc, cfg, smooth):
    """The layer output the rotation exists for (DuQuant++ page sec. 3.3:
    X W = (X Lambda^-1 R)(R^T Lambda W)): 2048 rows of the workload through a
    layer of 1024 outputs, X and the absorbed W both MXFP4 (W4A4), for each
    block kind of the error studies, with the workload's smoothing or none.
    Reported, not asserted beyond sanity (the page prints no values): the
    relative Frobenius error against the exact X W in fp64, of the W4A4
    product and of the product with only X quantized (the absorbed weights
    exact, from the oracle)."""
    from oracle import calibration as CAL
    wl = W.make_config(cfg)
    lam = wl.lam if smooth else None
    rows = np.sort(np.random.default_rng(2100 + cfg).choice(wl.tokens, 2048, replace=False))
    x = wl.x[torch.from_numpy(rows)].contiguous()
    w = W.linear_weights(1024, wl.channels, seed=2200 + cfg, dtype=wl.x.dtype)
    exact = x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
    s, n = wl.meta["calib_start"], wl.meta["calib_len"]
    _, _, xw = CAL.worst_group(wl.x[s:s + n], lam)
    blocks = {"identity": W.identity_r(),
              "random_hadamard": W.bf16_matrix(W.random_hadamard(np.random.default_rng(2005))),
              "householder": wl.r_hat,
              "greedy_pi4": W.bf16_matrix(CAL.greedy_givens(xw, 128)[0]),
              "greedy_grid8": W.bf16_matrix(CAL.greedy_givens_angle(xw, 128, 8)[0])}
    report = {}
    for name, r in blocks.items():
        ac, asc, _, _, y = _pipeline(x, lam, r, w, dev)
        y = y.cpu().numpy().astype(np.float64)
        assert np.isfinite(y).all()
        da = orc.dequant(ac.cpu().numpy(), asc.cpu().numpy())
        ya = da @ O.absorb_weights(w, lam, r).T
        e4 = float(np.linalg.norm(y - exact) / np.linalg.norm(exact))
        ea = float(np.linalg.norm(ya - exact) / np.linalg.norm(exact))
        report[name] = (round(e4, 4), round(ea, 4))
        assert e4 < 1.5 and ea < 1.5, name
    print(f"  layer-output error (W4A4, A4 only), config {cfg}, smoothing {smooth}: {report}", flush=True)
