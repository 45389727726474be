"""Ragged channel counts, rows of zeros and the tiled norm output keep the
common path.

A row whose group count is not a multiple of a super-tile (64 groups) leaves
padding groups in the last super-tile: they load zeros, and their stores are
dropped.  Their rotated maximum is 0, below the 2^-64 bound under which a
group is recomputed exactly (the rare pass after each kernel's main loop).
Padding must not count there, or every wave of the last super-tile column
redoes all of its rows: the outputs stay the same, but such shapes ran 2.6
to 9 times slower than aligned ones of the same size (8192 x 5120: 56 us
against 22 us for 8192 x 6144).  The outputs are covered by the parity tests;
these check the time, against an aligned shape with at least as many bytes,
with margins far above the run-to-run spread (a few per cent).

Groups of zeros have rotated maximum 0 too, but their codes and scale are
exact already; the quantize kernel tells them from tiny groups by their input
(only in rows where some group fell below the bound).  Before, a batch with
every other row zero ran 3.6 times slower (8192 x 14336: 175 us against 48 us)
and 6.4 times with smoothing at 2048 x 4096.
"""
import numpy as np
import pytest
import torch

import mxfp4_activation_rotation_amd as mxq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mxq.load()
    return torch.device("cuda:0")


def _orthogonal(n, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.linalg.qr(torch.randn(n, n, generator=g, dtype=torch.float64))[0]
    return q.contiguous().to(torch.bfloat16).to(dev)


def _inputs(T, C, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = (torch.randn(T, C, generator=g) * 2).to(torch.bfloat16).to(dev)
    lam = (torch.rand(C, generator=g) + 0.5).to(dev)
    gamma = (torch.rand(C, generator=g) + 0.5).to(dev)
    return x, lam, gamma


def _time_us(fn, launches=30, repeats=3):
    """Best of `repeats` means over `launches` back-to-back calls."""
    best = float("inf")
    for _ in range(repeats):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(launches):
            fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / launches)
    return best


def _outputs(T, C, dev):
    return (torch.empty((T, C // 2), dtype=torch.uint8, device=dev),
            torch.empty((T, C // 32), dtype=torch.uint8, device=dev))


@pytest.mark.parametrize("smoothed", [False, True])
def test_rotate_quant_ragged_columns(dev, smoothed):
    # 5120 channels: 160 groups, the third super-tile column half padding;
    # 6144 channels: three full columns (20 % more bytes)
    r = _orthogonal(32, 1, dev)
    times = {}
    for C in (5120, 6144):
        x, lam, _ = _inputs(8192, C, 2, dev)
        codes, scales = _outputs(8192, C, dev)
        times[C] = _time_us(lambda: mxq.rotate_quant(x, r, lam if smoothed else None, codes=codes, scales=scales))
    print(f"  rotate_quant smoothed={smoothed}: 8192x5120 {times[5120]:.1f} us, 8192x6144 {times[6144]:.1f} us")
    assert times[5120] < 1.3 * times[6144]


def test_norm_ragged_super_tiles(dev):
    # 5120 channels run with 4 super-tiles of 64 groups (160 of 256 used);
    # 8192 channels fill the same 4 (60 % more bytes)
    r = _orthogonal(32, 3, dev)
    times = {}
    for C in (5120, 8192):
        x, lam, gamma = _inputs(8192, C, 4, dev)
        codes, scales = _outputs(8192, C, dev)
        times[C] = _time_us(lambda: mxq.norm_rotate_quant(x, r, gamma, None, lam, norm="rms", eps=1e-5,
                                                          codes=codes, scales=scales))
    print(f"  norm_rotate_quant: 8192x5120 {times[5120]:.1f} us, 8192x8192 {times[8192]:.1f} us")
    assert times[5120] < 1.2 * times[8192]


def test_block64_ragged_columns(dev):
    h = _orthogonal(64, 5, dev)
    times = {}
    for C in (5120, 6144):
        x, _, _ = _inputs(8192, C, 6, dev)
        codes, scales = _outputs(8192, C, dev)
        times[C] = _time_us(lambda: mxq.rotate_quant_block(x, h, None, codes=codes, scales=scales))
    print(f"  rotate_quant_block B=64: 8192x5120 {times[5120]:.1f} us, 8192x6144 {times[6144]:.1f} us")
    assert times[5120] < 1.3 * times[6144]


def test_ragged_rows_still_redo_tiny_groups(dev):
    """The exclusion covers padding only: a real group below 2^-64 in a ragged
    row still takes the exact pass (its codes then match those of the same
    group scaled by 2^100, with the scale byte lowered by 100)."""
    r = _orthogonal(32, 7, dev)
    T, C = 64, 5120
    g = torch.Generator(device="cpu").manual_seed(8)
    base = torch.randn(T, C, generator=g, dtype=torch.float64)
    big = (base * 2.0 ** 20).to(torch.float32)
    tiny = (base * 2.0 ** -80).to(torch.float32)
    # the last group of every row tiny (it sits in the ragged column), the rest ordinary
    x_big = big.clone()
    x = big.clone()
    x[:, C - 32:] = tiny[:, C - 32:]
    x_big[:, C - 32:] = (tiny[:, C - 32:].double() * 2.0 ** 100).float()
    xb = x.to(torch.bfloat16)
    xbb = x_big.to(torch.bfloat16)
    # scaling a bf16 value by 2^100 is exact while it stays normal
    assert torch.equal((xb[:, C - 32:].double() * 2.0 ** 100).to(torch.bfloat16), xbb[:, C - 32:])
    c1, s1 = mxq.rotate_quant(xb.to(dev), r, None)
    c2, s2 = mxq.rotate_quant(xbb.to(dev), r, None)
    torch.cuda.synchronize()
    c1, s1, c2, s2 = (t.cpu().numpy() for t in (c1, s1, c2, s2))
    assert np.array_equal(c1[:, -16:], c2[:, -16:])
    assert np.array_equal(s1[:, -1].astype(np.int64), s2[:, -1].astype(np.int64) - 100)
    assert (s1[:, -1] < 61).all()


@pytest.mark.parametrize("smoothed", [False, True])
def test_rotate_quant_rows_of_zeros(dev, smoothed):
    r = _orthogonal(32, 9, dev)
    x, lam, _ = _inputs(2048, 4096, 10, dev)
    xz = x.clone()
    xz[1::2] = 0
    codes, scales = _outputs(2048, 4096, dev)
    t = _time_us(lambda: mxq.rotate_quant(x, r, lam if smoothed else None, codes=codes, scales=scales))
    tz = _time_us(lambda: mxq.rotate_quant(xz, r, lam if smoothed else None, codes=codes, scales=scales))
    print(f"  rotate_quant smoothed={smoothed} 2048x4096: {t:.1f} us, every other row zero {tz:.1f} us")
    assert tz < 1.5 * t
    # the zero rows come out as zero codes with the scale byte of a zero maximum,
    # and the other rows as they do without the zero rows
    c1, s1 = mxq.rotate_quant(x, r, lam if smoothed else None)
    c2, s2 = mxq.rotate_quant(xz, r, lam if smoothed else None)
    torch.cuda.synchronize()
    c1, s1, c2, s2 = (a.cpu().numpy() for a in (c1, s1, c2, s2))
    assert np.array_equal(c1[0::2], c2[0::2]) and np.array_equal(s1[0::2], s2[0::2])
    assert not c2[1::2].any() and not s2[1::2].any()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_norm_rows_of_zeros(dev, dtype):
    """Padding rows (all zero) of an RMSNorm batch without beta have exact
    statistics and x' = 0: they must not send the wave through the pass that
    redoes rare rows, and they encode as zero codes and zero scale bytes."""
    r = _orthogonal(32, 11, dev)
    x, lam, gamma = _inputs(8192, 4096, 12, dev)
    x = x.to(dtype)
    xz = x.clone()
    xz[1::2] = 0
    codes, scales = _outputs(8192, 4096, dev)
    t = _time_us(lambda: mxq.norm_rotate_quant(x, r, gamma, None, lam, codes=codes, scales=scales))
    tz = _time_us(lambda: mxq.norm_rotate_quant(xz, r, gamma, None, lam, codes=codes, scales=scales))
    print(f"  norm {dtype} 8192x4096: {t:.1f} us, every other row zero {tz:.1f} us")
    assert tz < 1.3 * t
    c1, s1 = mxq.norm_rotate_quant(x, r, gamma, None, lam)
    c2, s2 = mxq.norm_rotate_quant(xz, r, gamma, None, lam)
    torch.cuda.synchronize()
    c1, s1, c2, s2 = (a.cpu().numpy() for a in (c1, s1, c2, s2))
    assert np.array_equal(c1[0::2], c2[0::2]) and np.array_equal(s1[0::2], s2[0::2])
    assert not c2[1::2].any() and not s2[1::2].any()


@pytest.mark.parametrize("B", [64, 128])
def test_block_rows_of_zeros(dev, B):
    """The same for the block-size kernel: blocks of zero inputs are exact."""
    rb = _orthogonal(B, 13, dev)
    x, _, _ = _inputs(4096, 14336, 14, dev)
    xz = x.clone()
    xz[1::2] = 0
    codes, scales = _outputs(4096, 14336, dev)
    t = _time_us(lambda: mxq.rotate_quant_block(x, rb, codes=codes, scales=scales))
    tz = _time_us(lambda: mxq.rotate_quant_block(xz, rb, codes=codes, scales=scales))
    print(f"  block {B} 4096x14336: {t:.1f} us, every other row zero {tz:.1f} us")
    assert tz < 1.3 * t
    c1, s1 = mxq.rotate_quant_block(x, rb)
    c2, s2 = mxq.rotate_quant_block(xz, rb)
    torch.cuda.synchronize()
    c1, s1, c2, s2 = (a.cpu().numpy() for a in (c1, s1, c2, s2))
    assert np.array_equal(c1[0::2], c2[0::2]) and np.array_equal(s1[0::2], s2[0::2])
    assert not c2[1::2].any() and not s2[1::2].any()


@pytest.mark.parametrize("T,C,bound", [(8192, 4096, 1.4), (2048, 5120, 1.6)])
def test_norm_tiled_output_keeps_pace(dev, T, C, bound):
    """The tiled output of long batches stages record rows in LDS and meets
    at one block barrier per step; it should cost about what the row layout
    does.  An agent-scope release fence before the rare pass (an L2
    write-back by every wave) once made it 3.4-3.6 times slower."""
    r = _orthogonal(32, 11, dev)
    x, lam, gamma = _inputs(T, C, 12, dev)
    codes, scales = _outputs(T, C, dev)
    tc, ts = mxq.norm_rotate_quant_tiled(x, r, gamma, None, lam, norm="rms", eps=1e-5)
    t_row = _time_us(lambda: mxq.norm_rotate_quant(x, r, gamma, None, lam, norm="rms", eps=1e-5,
                                                   codes=codes, scales=scales))
    t_tiled = _time_us(lambda: mxq.norm_rotate_quant_tiled(x, r, gamma, None, lam, norm="rms", eps=1e-5,
                                                           tcodes=tc, tscales=ts))
    print(f"  norm {T}x{C}: row layout {t_row:.1f} us, tiled {t_tiled:.1f} us")
    assert t_tiled < bound * t_row
