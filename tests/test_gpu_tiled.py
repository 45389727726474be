"""Fragment-tiled MXFP4 operands on an MI355X through the C ABI: the repack
against the oracle's definition of the layout (bit-exact), the quantizer's
tiled output against the repacked row output (bit-exact), and the tiled
product against the row-layout product (bit-identical: same instruction
sequence on the same operand bytes) and the fp64 oracle."""
import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mxq.load()
    return torch.device("cuda:0")


def _u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("rows,K", [(1, 128), (16, 128), (37, 384), (200, 1152), (64, 14336)])
def test_tile_matches_oracle(dev, rows, K):
    rng = np.random.default_rng(9000 + rows + K)
    codes, scales = W.random_mxfp4(rng, rows, K)
    tc, ts = mxq.tile_mxfp4(_u8(codes, dev), _u8(scales, dev))
    torch.cuda.synchronize()
    rc, rs = O.tile_mxfp4(codes, scales)
    assert np.array_equal(tc.cpu().numpy(), rc) and np.array_equal(ts.cpu().numpy(), rs)


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (5, 40, 256), (16, 300, 1152), (17, 33, 384), (33, 70, 128),
                                   (64, 130, 512), (65, 257, 1024), (300, 260, 768), (513, 129, 1152)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiled_product_same_bits(dev, M, N, K, out_dtype):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    a = [_u8(t, dev) for t in W.random_mxfp4(rng, M, K)]
    b = [_u8(t, dev) for t in W.random_mxfp4(rng, N, K)]
    print(f"  tiled gemm M={M} N={N} K={K} {out_dtype}", flush=True)
    y_row = mxq.gemm_mxfp4(*a, *b, out_dtype)
    ta = mxq.tile_mxfp4(*a)
    tb = mxq.tile_mxfp4(*b)
    y_t = mxq.gemm_mxfp4_tiled(*ta, *tb, M, N, K, out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_row)
    if out_dtype == torch.float32 and M * N <= 40000:
        ref, s_abs = O.gemm_mxfp4(*[t.cpu().numpy() for t in a], *[t.cpu().numpy() for t in b])
        err = np.abs(y_t.cpu().numpy().astype(np.float64) - ref)
        assert (err <= 2.0 * K * U * s_abs).all()


@pytest.mark.parametrize("M,N", [(20, 37), (300, 90)])
def test_tiled_product_garbage_padding(dev, M, N):
    """Padding rows of the records only reach outputs that are not written."""
    rng = np.random.default_rng(9101 + M)
    K = 256
    a = [_u8(t, dev) for t in W.random_mxfp4(rng, M, K)]
    b = [_u8(t, dev) for t in W.random_mxfp4(rng, N, K)]
    ta = mxq.tile_mxfp4(*a)
    tb = mxq.tile_mxfp4(*b)
    y0 = mxq.gemm_mxfp4_tiled(*ta, *tb, M, N, K)
    # overwrite every padding slot with NaN scales and random codes
    for (tc, ts), rows in ((ta, M), (tb, N)):
        nk = K // 128
        rec = torch.arange(tc.numel() // 16, device=dev)
        row = 16 * (rec // 64 // nk) + rec % 16
        pad = row >= rows
        tc.view(-1, 16)[pad] = torch.randint(0, 256, (int(pad.sum()), 16), dtype=torch.uint8, device=dev)
        ts[pad] = 255
    y1 = mxq.gemm_mxfp4_tiled(*ta, *tb, M, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.isfinite(y1).all()


def test_tiled_product_empty_and_k0(dev):
    e = torch.empty(0, dtype=torch.uint8, device=dev)
    nc, ns = mxq.tiled_sizes(16, 128)
    bc = torch.zeros(nc, dtype=torch.uint8, device=dev)
    bs = torch.zeros(ns, dtype=torch.uint8, device=dev)
    y = mxq.gemm_mxfp4_tiled(e, e, bc, bs, 0, 16, 128)
    assert y.shape == (0, 16)
    y = torch.full((3, 5), 7.0, device=dev)
    mxq.gemm_mxfp4_tiled(e, e, e, e, 3, 5, 0, out=y)
    torch.cuda.synchronize()
    assert (y == 0).all()


@pytest.mark.parametrize("T,C", [(1, 128), (16, 4096), (30, 14336), (130, 2048 + 4 * 128)])
@pytest.mark.parametrize("dtype,with_lam", [(torch.bfloat16, False), (torch.bfloat16, True),
                                            (torch.float16, True)])
def test_rotate_quant_tiled_same_bytes(dev, T, C, dtype, with_lam):
    rng = np.random.default_rng(9200 + T + C // 128 + 7 * with_lam)
    x = W.random_activations(rng, T, C, dtype, scale=2.0).to(dev)
    lam = torch.from_numpy(np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)).to(dev) if with_lam else None
    r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
    codes, scales = mxq.rotate_quant(x, r, lam)
    ref = mxq.tile_mxfp4(codes, scales)
    nc, ns = mxq.tiled_sizes(T, C)
    tc = torch.zeros(nc, dtype=torch.uint8, device=dev)  # padding rows stay zero, as in the repack
    ts = torch.zeros(ns, dtype=torch.uint8, device=dev)
    mxq.rotate_quant_tiled(x, r, lam, tcodes=tc, tscales=ts)
    torch.cuda.synchronize()
    assert torch.equal(tc, ref[0]) and torch.equal(ts, ref[1])
    c2, s2 = O.untile_mxfp4(tc.cpu().numpy(), ts.cpu().numpy(), T, C)
    assert np.array_equal(c2, codes.cpu().numpy()) and np.array_equal(s2, scales.cpu().numpy())


def test_decode_pipeline_full_size(dev):
    """16 tokens of the headline batch, rotated and quantized straight into
    records, times the absorbed 4096 x 14336 weights in records: the same
    bits as the row-layout pipeline."""
    wl = W.make_config(3)
    w = W.linear_weights(W.DOWN_PROJ_OUT, wl.channels)
    r = wl.r_hat.to(dev)
    lam = torch.from_numpy(wl.lam).to(dev) if wl.lam is not None else None
    x16 = wl.x[:16].contiguous().to(dev)
    bc, bsc = mxq.absorb_quant(w.to(dev), r, lam)
    ac, asc = mxq.rotate_quant(x16, r, lam)
    y_row = mxq.gemm_mxfp4(ac, asc, bc, bsc, torch.bfloat16)
    ta = mxq.rotate_quant_tiled(x16, r, lam)
    tb = mxq.tile_mxfp4(bc, bsc)
    y_t = mxq.gemm_mxfp4_tiled(*ta, *tb, 16, W.DOWN_PROJ_OUT, wl.channels, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_row)


def test_large_product_full_size_same_bits(dev):
    """8192 x 4096 x 14336 (the down_proj product of the headline batch):
    tiled and row-layout products agree bit for bit."""
    M, N, K = 8192, 4096, 14336
    g = torch.Generator(device=dev)
    g.manual_seed(9300)
    a = (torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=g),
         torch.randint(115, 135, (M, K // 32), dtype=torch.uint8, device=dev, generator=g))
    b = (torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g),
         torch.randint(115, 135, (N, K // 32), dtype=torch.uint8, device=dev, generator=g))
    y_row = mxq.gemm_mxfp4(*a, *b, torch.bfloat16)
    y_t = mxq.gemm_mxfp4_tiled(*mxq.tile_mxfp4(*a), *mxq.tile_mxfp4(*b), M, N, K, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_row)


@pytest.mark.parametrize("M,N,K", [(257, 8000, 128), (2048, 4096, 1024), (3840, 4096, 256), (4096, 3840, 384),
                                   (4096, 4000, 128), (4100, 3900, 384), (3900, 4100, 256), (2048, 4096, 14336)])
def test_product_either_large_kernel_same_bits(dev, M, N, K):
    """Both sides of the switch between the 256 x 256 kernel (grids with at
    least one such tile per CU) and the two-blocks-per-CU 256 x 128 kernel
    (fewer tiles, with too many rows for the chunked decode kernel), ragged
    edges included: the tiled product equals the row-layout product (always
    the 256 x 256 kernel at these sizes) bit for bit."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    tiles = -(-M // 256) * -(-N // 256)
    g = torch.Generator(device=dev)
    g.manual_seed(M * 7 + N * 3 + K)
    a = (torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=g),
         torch.randint(115, 135, (M, K // 32), dtype=torch.uint8, device=dev, generator=g))
    b = (torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g),
         torch.randint(115, 135, (N, K // 32), dtype=torch.uint8, device=dev, generator=g))
    ta, tb = mxq.tile_mxfp4(*a), mxq.tile_mxfp4(*b)
    for out_dtype in (torch.float32, torch.bfloat16):
        print(f"  product M={M} N={N} K={K} {out_dtype}: {tiles} tiles of 256x256 on {cus} CUs", flush=True)
        y_row = mxq.gemm_mxfp4(*a, *b, out_dtype)
        y_t = mxq.gemm_mxfp4_tiled(*ta, *tb, M, N, K, out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(y_t, y_row)


@pytest.mark.parametrize("T,dtype,with_lam", [(5000, torch.bfloat16, False), (4700, torch.float16, True)])
def test_rotate_quant_tiled_prefill_sizes(dev, T, dtype, with_lam):
    """Batches long enough that the quantizer writes records a 16-row unit at
    a time through LDS (a partial last unit included): the same bytes as the
    repacked row-layout output."""
    C = 14336
    rng = np.random.default_rng(9400 + T)
    x = W.random_activations(rng, T, C, dtype, scale=2.0).to(dev)
    lam = torch.from_numpy(np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)).to(dev) if with_lam else None
    r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
    ref = mxq.tile_mxfp4(*mxq.rotate_quant(x, r, lam))
    nc, ns = mxq.tiled_sizes(T, C)
    tc = torch.zeros(nc, dtype=torch.uint8, device=dev)
    ts = torch.zeros(ns, dtype=torch.uint8, device=dev)
    mxq.rotate_quant_tiled(x, r, lam, tcodes=tc, tscales=ts)
    torch.cuda.synchronize()
    assert torch.equal(tc, ref[0]) and torch.equal(ts, ref[1])


@pytest.mark.parametrize("T,C", [(1, 128), (16, 4096), (37, 2432), (300, 4096),
                                 # long batches: 16-wave blocks stage a record row in LDS
                                 # (>= 4096 rows up to 4096 channels), 8-wave blocks half
                                 # of one (>= 2048 rows up to 8192 channels); ragged ends
                                 (4100, 4096), (4099, 2432), (2050, 8192), (2061, 5120),
                                 (64, 16384)])
@pytest.mark.parametrize("norm,dtype,with_beta,with_lam", [("rms", torch.bfloat16, False, True),
                                                           ("layer", torch.float16, True, True),
                                                           ("rms", torch.float16, False, False)])
def test_norm_rotate_quant_tiled_same_bytes(dev, T, C, norm, dtype, with_beta, with_lam):
    rng = np.random.default_rng(9500 + T + C // 128)
    x = W.random_activations(rng, T, C, dtype, scale=2.0).to(dev)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, C).astype(np.float32)).to(dev)
    beta = torch.from_numpy(rng.normal(0, 0.1, C).astype(np.float32)).to(dev) if with_beta else None
    lam = torch.from_numpy(np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)).to(dev) if with_lam else None
    r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
    ref = mxq.tile_mxfp4(*mxq.norm_rotate_quant(x, r, gamma, beta, lam, norm=norm))
    nc, ns = mxq.tiled_sizes(T, C)
    tc = torch.zeros(nc, dtype=torch.uint8, device=dev)
    ts = torch.zeros(ns, dtype=torch.uint8, device=dev)
    mxq.norm_rotate_quant_tiled(x, r, gamma, beta, lam, norm=norm, tcodes=tc, tscales=ts)
    torch.cuda.synchronize()
    assert torch.equal(tc, ref[0]) and torch.equal(ts, ref[1])


def test_decode_qkv_pipeline(dev):
    """RMSNorm + rotate + quantize 16 tokens straight into records, times
    absorbed 4096 x 4096 weights in records: the same bits as the row-layout
    pipeline."""
    nw = W.norm_workload()
    r = nw.r_hat.to(dev)
    lam = torch.from_numpy(nw.lam).to(dev)
    gamma = torch.from_numpy(nw.gamma).to(dev)
    x16 = nw.x[:16].contiguous().to(dev)
    C = nw.x.shape[1]
    w = W.linear_weights(4096, C)
    bc, bsc = mxq.absorb_quant(w.to(dev), r, lam)
    ac, asc = mxq.norm_rotate_quant(x16, r, gamma, None, lam, eps=nw.eps)
    y_row = mxq.gemm_mxfp4(ac, asc, bc, bsc, torch.bfloat16)
    ta = mxq.norm_rotate_quant_tiled(x16, r, gamma, None, lam, eps=nw.eps)
    y_t = mxq.gemm_mxfp4_tiled(*ta, *mxq.tile_mxfp4(bc, bsc), 16, 4096, C, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_row)


def test_tiled_outputs_from_strided_rows(dev):
    """Rows of x with a pitch larger than the row (a column slice of a wider
    tensor) give the same records as the contiguous copy."""
    rng = np.random.default_rng(9600)
    wide = W.random_activations(rng, 40, 3 * 1024, torch.bfloat16, scale=2.0).to(dev)
    x = wide[:, 512:512 + 2048]
    assert x.stride(0) == 3 * 1024
    r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, 2048).astype(np.float32)).to(dev)
    T, C = x.shape
    for fn in (lambda t: mxq.rotate_quant_tiled(t, r), lambda t: mxq.norm_rotate_quant_tiled(t, r, gamma)):
        a = fn(x)
        b = fn(x.contiguous())
        torch.cuda.synchronize()
        # the padding rows of the last record row are not written: compare the 40 real rows
        ua = O.untile_mxfp4(a[0].cpu().numpy(), a[1].cpu().numpy(), T, C)
        ub = O.untile_mxfp4(b[0].cpu().numpy(), b[1].cpu().numpy(), T, C)
        assert np.array_equal(ua[0], ub[0]) and np.array_equal(ua[1], ub[1])


def _random_shapes(seed, n, t_max, c_max):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, t_max + 1)), 128 * int(rng.integers(1, c_max // 128 + 1))) for _ in range(n)]


def _large_shapes(seed, n):
    # long batches over wide rows: units of 16 rows x super-tile columns reach the
    # grid's resident waves, so the tiled quantizer takes its 16-row-unit path
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(8192, 16001)), 128 * int(rng.integers(49, 113))) for _ in range(n)]


@pytest.mark.parametrize("T,C", _random_shapes(9700, 6, 6000, 8192) + _large_shapes(9703, 4))
def test_random_shapes_quantizer_tiled_same_bytes(dev, T, C):
    """Seeded random shapes on both sides of the 16-row-unit switch, with
    partial super-tile columns: the tiled output equals the repacked row
    output byte for byte (bf16 without Λ, fp16 with Λ)."""
    rng = np.random.default_rng(T * 7 + C)
    for dtype, with_lam in ((torch.bfloat16, False), (torch.float16, True)):
        x = W.random_activations(rng, T, C, dtype, scale=2.0).to(dev)
        lam = torch.from_numpy(np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)).to(dev) if with_lam else None
        r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
        print(f"  quantizer tiled T={T} C={C} {dtype} lam={with_lam}", flush=True)
        ref = mxq.tile_mxfp4(*mxq.rotate_quant(x, r, lam))
        nc, ns = mxq.tiled_sizes(T, C)
        tc = torch.zeros(nc, dtype=torch.uint8, device=dev)
        ts = torch.zeros(ns, dtype=torch.uint8, device=dev)
        mxq.rotate_quant_tiled(x, r, lam, tcodes=tc, tscales=ts)
        torch.cuda.synchronize()
        assert torch.equal(tc, ref[0]) and torch.equal(ts, ref[1])


@pytest.mark.parametrize("T,C", _random_shapes(9701, 10, 6000, 8192))
def test_random_shapes_norm_tiled_same_bytes(dev, T, C):
    """Seeded random shapes on both sides of the staged-store switch (record
    rows staged in LDS for long batches): the tiled norm output equals the
    repacked row output byte for byte (RMSNorm bf16, LayerNorm fp16 with β)."""
    rng = np.random.default_rng(T * 5 + C)
    for norm, dtype, with_beta in (("rms", torch.bfloat16, False), ("layer", torch.float16, True)):
        x = W.random_activations(rng, T, C, dtype, scale=2.0).to(dev)
        gamma = torch.from_numpy(rng.uniform(0.5, 1.5, C).astype(np.float32)).to(dev)
        beta = torch.from_numpy(rng.normal(0, 0.1, C).astype(np.float32)).to(dev) if with_beta else None
        lam = torch.from_numpy(np.exp(0.5 * rng.standard_normal(C)).astype(np.float32)).to(dev)
        r = W.bf16_matrix(W.qr_orthogonal(rng)).to(dev)
        print(f"  norm tiled T={T} C={C} {norm} {dtype}", flush=True)
        ref = mxq.tile_mxfp4(*mxq.norm_rotate_quant(x, r, gamma, beta, lam, norm=norm))
        nc, ns = mxq.tiled_sizes(T, C)
        tc = torch.zeros(nc, dtype=torch.uint8, device=dev)
        ts = torch.zeros(ns, dtype=torch.uint8, device=dev)
        mxq.norm_rotate_quant_tiled(x, r, gamma, beta, lam, norm=norm, tcodes=tc, tscales=ts)
        torch.cuda.synchronize()
        assert torch.equal(tc, ref[0]) and torch.equal(ts, ref[1])


def _random_products(seed, n):
    # every other M at most 64 (the split-K decode kernel), the rest above it
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 65) if i % 2 else rng.integers(65, 3000)), int(rng.integers(1, 3000)),
             128 * int(rng.integers(1, 33))) for i in range(n)]


@pytest.mark.parametrize("M,N,K", _random_products(9702, 12))
def test_random_shapes_product_same_bits(dev, M, N, K):
    """Seeded random products (decode and large kernels, ragged tiles, odd
    stage counts): the tiled product equals the row-layout product bit for
    bit, fp32 and bf16 out."""
    rng = np.random.default_rng(M * 3 + N * 11 + K)
    a = [_u8(t, dev) for t in W.random_mxfp4(rng, M, K)]
    b = [_u8(t, dev) for t in W.random_mxfp4(rng, N, K)]
    ta, tb = mxq.tile_mxfp4(*a), mxq.tile_mxfp4(*b)
    for out_dtype in (torch.float32, torch.bfloat16):
        print(f"  random product M={M} N={N} K={K} {out_dtype}", flush=True)
        y_row = mxq.gemm_mxfp4(*a, *b, out_dtype)
        y_t = mxq.gemm_mxfp4_tiled(*ta, *tb, M, N, K, out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(y_t, y_row)
