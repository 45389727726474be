"""C ABI checks that need no GPU: exports, argument validation, launch plan.

Every call below fails validation on the host, which by contract happens
before any HIP call, so nothing touches a device.
"""
import ctypes
import os
import re
import subprocess

import pytest

import mxfp4_activation_rotation_amd as mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")

OK, NULL, SHAPE, DTYPE, ALIGN, STRIDE = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p(0x10000)       # never dereferenced: validation rejects first
P_ODD = ctypes.c_void_p(0x10008)   # 8-byte but not 16-byte aligned


@pytest.fixture(scope="module")
def lib():
    return mxq.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


def test_header_is_plain_c():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER], check=True)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(mxq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", mxq.library_path()], capture_output=True, text=True,
                         check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), f"{n} not exported as text symbol"


def test_library_carries_gfx950_code():
    data = open(mxq.library_path(), "rb").read()
    assert b"gfx950" in data


def test_status_strings(lib):
    for s in range(7):
        assert lib.mxq_status_str(s).decode().startswith("MXQ_")
    assert lib.mxq_version() == 1


def rq(lib, x=P, dt=0, T=8, C=64, stride=64, lam=None, r=P, codes=P, scales=P):
    return lib.mxq_rotate_quant(x, dt, T, C, stride, lam, r, codes, scales, None)


def test_rotate_quant_validation(lib):
    assert rq(lib, dt=2) == DTYPE          # fp32 x is not a fused input
    assert rq(lib, dt=7) == DTYPE
    assert rq(lib, C=48, stride=48) == SHAPE
    assert rq(lib, T=-1) == SHAPE
    assert rq(lib, C=-32) == SHAPE
    assert rq(lib, T=0, x=None, r=None, codes=None, scales=None) == OK   # empty: no launch
    assert rq(lib, C=0, stride=0, x=None) == OK
    assert rq(lib, x=None) == NULL
    assert rq(lib, r=None) == NULL
    assert rq(lib, codes=None) == NULL
    assert rq(lib, scales=None) == NULL
    assert rq(lib, stride=32) == STRIDE
    assert rq(lib, x=P_ODD) == ALIGN
    assert rq(lib, codes=P_ODD) == ALIGN
    assert rq(lib, lam=P_ODD) == ALIGN
    assert rq(lib, stride=68) == ALIGN     # 136-byte rows are not 16-byte multiples
    assert rq(lib, T=1 << 31) == SHAPE
    assert lib.mxq_rotate_quant_ex(P, 0, 8, 64, 64, None, P, P, P, P_ODD, None) == ALIGN


def test_quant_and_dequant_validation(lib):
    q = lib.mxq_quant
    assert q(P, 3, 8, 64, 64, P, P, None) == DTYPE
    assert q(P, 2, 8, 64, 66, P, P, None) == ALIGN   # fp32 rows of 264 bytes
    assert q(P, 2, 8, 64, 60, P, P, None) == STRIDE
    assert q(None, 0, 8, 64, 64, P, P, None) == NULL
    assert q(P, 1, 8, 40, 40, P, P, None) == SHAPE
    assert q(None, 0, 0, 64, 64, None, None, None) == OK
    d = lib.mxq_dequant
    assert d(P, P, 8, 64, P, 1, None) == DTYPE       # fp16 output not offered
    assert d(P, P, 8, 40, P, 0, None) == SHAPE
    assert d(None, P, 8, 64, P, 0, None) == NULL
    assert d(P, P, 8, 64, P_ODD, 2, None) == ALIGN
    assert d(None, None, 0, 64, None, 2, None) == OK


@pytest.mark.parametrize("T,C,cu", [(8192, 14336, 256), (16, 8192, 256), (64, 256, 256), (37, 1440, 256),
                                    (1, 32, 256), (32768, 8192, 256), (3, 1 << 20, 4), (100000, 96, 80)])
def test_plan_covers_every_tile_once(T, C, cu):
    pl = mxq.plan(T, C, cu)
    tcols, rs, waves = pl["tile_columns"], pl["row_step"], pl["waves"]
    assert tcols == -(-(C // 32) // 64)
    assert waves == tcols * rs and 1 <= rs <= T
    assert pl["blocks"] * pl["waves_per_block"] >= waves > (pl["blocks"] - 1) * pl["waves_per_block"]
    seen = {}
    for w in range(waves):
        tc, r0 = w % tcols, w // tcols
        n_rows = len(range(r0, T, rs))
        seen[tc] = seen.get(tc, 0) + n_rows
    assert seen == {tc: T for tc in range(tcols)}


def test_plan_rejects_bad_shapes():
    for T, C in ((0, 64), (8, 0), (8, 33), (-1, 64)):
        with pytest.raises(mxq.MXQError):
            mxq.plan(T, C)


def test_calibration_validation(lib):
    ws = lib.mxq_calib_workspace_bytes(14336)
    assert ws >= lib.mxq_calib_workspace_bytes(0) > 0
    W16 = ctypes.c_void_p(0x20000)  # 256-byte aligned stand-in, never dereferenced
    w = lib.mxq_calib_worst_group
    assert w(P, 5, 8, 64, 64, None, P, P, P, W16, ws, None) == DTYPE
    assert w(P, 0, 0, 64, 64, None, P, P, P, W16, ws, None) == SHAPE
    assert w(P, 0, 8, 48, 48, None, P, P, P, W16, ws, None) == SHAPE
    assert w(None, 0, 8, 64, 64, None, P, P, P, W16, ws, None) == NULL
    assert w(P, 0, 8, 64, 32, None, P, P, P, W16, ws, None) == STRIDE
    assert w(P, 0, 8, 64, 64, None, P, P, P, W16, 16, None) == ALIGN
    assert w(P, 0, 8, 64, 64, None, P, P, P, ctypes.c_void_p(0x20010), ws, None) == ALIGN
    g = lib.mxq_calib_givens
    assert g(P, 0, 128, P, P, P, None, W16, ws, None) == SHAPE
    assert g(P, 8, -1, P, P, P, None, W16, ws, None) == SHAPE
    assert g(None, 8, 128, P, P, P, None, W16, ws, None) == NULL
    assert g(P, 8, 128, P, None, P, None, W16, ws, None) == NULL
    assert g(P, 8, 128, P, P, P, None, W16, 8, None) == ALIGN
    assert g(ctypes.c_void_p(0x10004), 8, 128, P, P, P, None, W16, ws, None) == ALIGN
    a = lib.mxq_calib_givens_angles
    assert a(P, 8, 128, 0, P, P, P, None, None, W16, ws, None) == SHAPE
    assert a(P, 8, 128, 1025, P, P, P, None, None, W16, ws, None) == SHAPE
    assert a(P, 0, 128, 64, P, P, P, None, None, W16, ws, None) == SHAPE
    assert a(P, 8, -1, 64, P, P, P, None, None, W16, ws, None) == SHAPE
    assert a(None, 8, 128, 64, P, P, P, None, None, W16, ws, None) == NULL
    assert a(P, 8, 128, 64, P, P, None, None, None, W16, ws, None) == NULL
    assert a(P, 8, 128, 64, P, P, P, None, None, W16, 8, None) == ALIGN
    assert a(P, 8, 128, 64, P, P, P, None, ctypes.c_void_p(0x10002), W16, ws, None) == ALIGN


def test_calibration_noalloc_validation(lib):
    """The allocation-free scan rejects bad arguments, and channels above its
    scratch limit (262144), on the host before any HIP call."""
    w = lib.mxq_calib_worst_group_noalloc
    assert w(P, 5, 8, 64, 64, None, P, P, P, None) == DTYPE
    assert w(P, 0, 0, 64, 64, None, P, P, P, None) == SHAPE
    assert w(P, 0, 8, 48, 48, None, P, P, P, None) == SHAPE
    assert w(P, 0, 1, 262144 + 32, 262144 + 32, None, P, P, P, None) == SHAPE
    assert w(P, 0, 1, 1 << 20, 1 << 20, None, P, P, P, None) == SHAPE
    assert w(None, 0, 8, 64, 64, None, P, P, P, None) == NULL
    assert w(P, 0, 8, 64, 64, None, P, None, P, None) == NULL
    assert w(P, 0, 8, 64, 32, None, P, P, P, None) == STRIDE
    assert w(P, 0, 8, 64, 64, None, ctypes.c_void_p(0x10004), P, P, None) == ALIGN
    assert b"SHAPE" in lib.mxq_status_str(SHAPE)


def aq(lib, w=P, dt=0, N=8, K=64, stride=64, lam=None, r=P, codes=P, scales=P):
    return lib.mxq_absorb_quant(w, dt, N, K, stride, lam, r, codes, scales, None)


def test_absorb_quant_validation(lib):
    assert aq(lib, dt=2) == DTYPE
    assert aq(lib, K=48, stride=48) == SHAPE
    assert aq(lib, N=-1) == SHAPE
    assert aq(lib, N=0, w=None, r=None, codes=None, scales=None) == OK
    assert aq(lib, w=None) == NULL
    assert aq(lib, r=None) == NULL
    assert aq(lib, codes=None) == NULL
    assert aq(lib, stride=32) == STRIDE
    assert aq(lib, w=P_ODD) == ALIGN
    assert aq(lib, lam=P_ODD) == ALIGN
    assert aq(lib, N=1 << 31) == SHAPE


def gm(lib, a=P, sa=P, b=P, sb=P, M=8, N=8, K=256, y=P, dt=2, ldy=8):
    return lib.mxq_gemm_mxfp4(a, sa, b, sb, M, N, K, y, dt, ldy, None)


def test_gemm_validation(lib):
    assert gm(lib, dt=1) == DTYPE          # fp16 output is not offered
    assert gm(lib, K=64) == SHAPE          # K must be a multiple of 128
    assert gm(lib, K=320) == SHAPE
    assert gm(lib, K=-256) == SHAPE
    assert gm(lib, M=-1) == SHAPE
    assert gm(lib, K=(1 << 24) + 128) == SHAPE
    assert gm(lib, M=1 << 31) == SHAPE
    assert gm(lib, M=0, a=None, sa=None, b=None, sb=None, y=None) == OK
    assert gm(lib, N=0, y=None) == OK
    assert gm(lib, y=None) == NULL
    assert gm(lib, a=None) == NULL
    assert gm(lib, sb=None) == NULL
    assert gm(lib, ldy=7) == STRIDE
    assert gm(lib, a=P_ODD) == ALIGN
    assert gm(lib, b=P_ODD) == ALIGN
    assert gm(lib, sa=ctypes.c_void_p(0x10001)) == ALIGN
    assert gm(lib, y=ctypes.c_void_p(0x10002)) == ALIGN            # fp32 output: 4-byte alignment


def nq(lib, x=P, dt=0, T=8, C=64, stride=64, kind=0, g=P, b=None, eps=1e-5, lam=None, r=P, codes=P, scales=P,
       y=None):
    return lib.mxq_norm_rotate_quant(x, dt, T, C, stride, kind, g, b, ctypes.c_float(eps), lam, r, codes, scales,
                                     y, None)


def test_norm_rotate_quant_validation(lib):
    assert nq(lib, dt=2) == DTYPE
    assert nq(lib, kind=2) == DTYPE
    assert nq(lib, kind=-1) == DTYPE
    assert nq(lib, C=48, stride=48) == SHAPE
    assert nq(lib, C=16384 + 32, stride=16384 + 32) == SHAPE   # rows live in registers: at most 16384
    assert nq(lib, T=-1) == SHAPE
    assert nq(lib, T=1 << 31) == SHAPE
    assert nq(lib, eps=-1.0) == SHAPE
    assert nq(lib, eps=float("nan")) == SHAPE
    assert nq(lib, T=0, x=None, g=None, r=None, codes=None, scales=None) == OK
    assert nq(lib, x=None) == NULL
    assert nq(lib, g=None) == NULL
    assert nq(lib, r=None) == NULL
    assert nq(lib, scales=None) == NULL
    assert nq(lib, stride=32) == STRIDE
    assert nq(lib, x=P_ODD) == ALIGN
    assert nq(lib, codes=P_ODD) == ALIGN
    assert nq(lib, y=P_ODD) == ALIGN
    assert nq(lib, g=ctypes.c_void_p(0x10002)) == ALIGN
    assert nq(lib, stride=68) == ALIGN


def bq(lib, x=P, dt=0, T=8, C=128, stride=128, lam=None, r=P, B=64, codes=P, scales=P, y=None):
    return lib.mxq_rotate_quant_block(x, dt, T, C, stride, lam, r, B, codes, scales, y, None)


def test_rotate_quant_block_validation(lib):
    assert bq(lib, dt=2) == DTYPE
    for B in (8, 48, 256, 0, -32):
        assert bq(lib, B=B) == SHAPE
    assert bq(lib, C=96, stride=96, B=64) == SHAPE      # channels not a multiple of the block
    assert bq(lib, C=48, stride=48, B=16) == SHAPE      # nor of the 32-wide group
    assert bq(lib, T=-1) == SHAPE
    assert bq(lib, T=0, x=None, r=None, codes=None, scales=None) == OK
    assert bq(lib, x=None) == NULL
    assert bq(lib, r=None) == NULL
    assert bq(lib, codes=None) == NULL
    assert bq(lib, stride=64) == STRIDE
    assert bq(lib, x=P_ODD) == ALIGN
    assert bq(lib, lam=P_ODD) == ALIGN
    assert bq(lib, y=P_ODD) == ALIGN


def gt(lib, a=P, sa=P, b=P, sb=P, M=8, N=8, K=256, y=P, dt=2, ldy=8):
    return lib.mxq_gemm_mxfp4_tiled(a, sa, b, sb, M, N, K, y, dt, ldy, None)


def test_tiled_entry_points_validation(lib):
    # tiled product: same rules as the row layout, scales 4-byte aligned
    assert gt(lib, dt=1) == DTYPE
    assert gt(lib, K=64) == SHAPE
    assert gt(lib, K=(1 << 24) + 128) == SHAPE
    assert gt(lib, N=-1) == SHAPE
    assert gt(lib, M=0, a=None, sa=None, b=None, sb=None, y=None) == OK
    assert gt(lib, y=None) == NULL
    assert gt(lib, sa=None) == NULL
    assert gt(lib, ldy=7) == STRIDE
    assert gt(lib, a=P_ODD) == ALIGN
    assert gt(lib, sb=ctypes.c_void_p(0x10002)) == ALIGN
    # repacking into records
    tile = lib.mxq_tile_mxfp4
    assert tile(P, P, 8, 192, P, P, None) == SHAPE
    assert tile(P, P, -1, 128, P, P, None) == SHAPE
    assert tile(P, P, 8, (1 << 24) + 128, P, P, None) == SHAPE
    assert tile(P, P, 1 << 31, 128, P, P, None) == SHAPE
    assert tile(None, None, 0, 128, None, None, None) == OK
    assert tile(P, P, 8, 0, P, P, None) == OK
    assert tile(P, None, 8, 128, P, P, None) == NULL
    assert tile(P, P, 8, 128, P, None, None) == NULL
    assert tile(P_ODD, P, 8, 128, P, P, None) == ALIGN
    assert tile(P, P, 8, 128, P_ODD, P, None) == ALIGN
    # quantizer with tiled output: channels must be a multiple of 128
    rqt = lib.mxq_rotate_quant_tiled
    assert rqt(P, 0, 8, 96, 96, None, P, P, P, None) == SHAPE
    assert rqt(P, 2, 8, 128, 128, None, P, P, P, None) == DTYPE
    assert rqt(P, 0, 8, 128, 128, None, None, P, P, None) == NULL
    assert rqt(P, 0, 8, 128, 64, None, P, P, P, None) == STRIDE
    assert rqt(P, 0, 8, 128, 128, None, P, P_ODD, P, None) == ALIGN
    assert rqt(P, 0, 8, 128, 128, None, P, P, ctypes.c_void_p(0x10004), None) == ALIGN
    assert rqt(None, 0, 0, 128, 128, None, None, None, None, None) == OK


def test_tiled_sizes():
    assert mxq.tiled_sizes(1, 128) == (16 * 64, 16 * 4)
    assert mxq.tiled_sizes(17, 256) == (32 * 128, 32 * 8)
    with pytest.raises(ValueError):
        mxq.tiled_sizes(4, 96)


def test_norm_tiled_validation(lib):
    def nqt(x=P, dt=0, T=8, C=128, stride=128, kind=0, g=P, b=None, eps=1e-5, lam=None, r=P, codes=P, scales=P):
        return lib.mxq_norm_rotate_quant_tiled(x, dt, T, C, stride, kind, g, b, ctypes.c_float(eps), lam, r, codes,
                                               scales, None)
    assert nqt(C=96, stride=96) == SHAPE      # tiled output needs channels % 128 == 0
    assert nqt(dt=2) == DTYPE
    assert nqt(kind=5) == DTYPE
    assert nqt(eps=-1.0) == SHAPE
    assert nqt(g=None) == NULL
    assert nqt(stride=64) == STRIDE
    assert nqt(codes=P_ODD) == ALIGN
    assert nqt(T=0, x=None, g=None, r=None, codes=None, scales=None) == OK
