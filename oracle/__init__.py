"""fp64 CPU oracle for smooth + block rotation + MXFP4 quantization.

TEST INFRASTRUCTURE ONLY: tests/, the package smoke check and the bench's
CPU-baseline leg may import this module; the HIP library never does, and
nothing here imports the HIP package.  The arithmetic lives in
``mxq_oracle.c`` (plain fp64 C, OpenMP over token rows); this file only
marshals arrays, plus two pure-NumPy checkers that pin the C code:

* :func:`brute_force_codes` -- nearest of all 16 E2M1 codes by exhaustive
  search (DuQuant++ page, sec. 2.1: "round to the nearest 4-bit float"),
  ties to the even code, zero emitted as +0.
* :func:`group_error` -- per-group normalised quantization error
  ||dq_g - y_g||_2 / ||y_g||_2, the quantity plotted in the DuQuant++ page's
  Figure 1 (sec. 4.1); the page prints no values for it, so its numbers are
  reported, never asserted ("parity unpinned" for the values themselves).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mxq_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

BF16, FP16, FP32, FP64 = 0, 1, 2, 3
GROUP = 32

# E2M1 element values by code, OCP MX v1.0 FP4 (E2M1) table; codes 8..15 negate.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def build_command(src: str = SOURCE, out: str = LIBRARY, extra=()) -> list[str]:
    return ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
            "-shared", "-fPIC", *extra, "-o", out, src, "-lm"]


def build(src: str = SOURCE, out: str = LIBRARY, extra=()) -> str:
    """Compile the C oracle with gcc (no GPU involved)."""
    subprocess.run(build_command(src, out, extra), check=True)
    return out


def _i64(v):
    return ctypes.c_int64(int(v))


class Oracle:
    """ctypes view of one compiled copy of ``mxq_oracle.c``."""

    def __init__(self, lib_path: str = LIBRARY):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        self.lib = ctypes.CDLL(lib_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        self.lib.oracle_quant.argtypes = [vp, i32, i64, i64, i64, vp, vp]
        self.lib.oracle_rotate_quant.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, vp, vp, vp]
        self.lib.oracle_encode_groups.argtypes = [vp, i64, vp, vp]
        self.lib.oracle_dequant.argtypes = [vp, vp, i64, i64, vp]
        self.lib.oracle_rotate_quant_block.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, i32, vp, vp, vp]
        self.lib.oracle_rotate_quant_block.restype = ctypes.c_int
        self.lib.oracle_norm_rotate_quant.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, ctypes.c_double,
                                                      vp, vp, i32, vp, vp, vp]
        for f in ("oracle_quant", "oracle_rotate_quant", "oracle_encode_groups",
                  "oracle_dequant", "oracle_num_threads", "oracle_norm_rotate_quant"):
            getattr(self.lib, f).restype = ctypes.c_int

    # -- input marshalling ------------------------------------------------
    @staticmethod
    def _raw(x):
        """(numpy view keeping memory alive, dtype code, tokens, channels, row stride)."""
        try:
            import torch
        except ImportError:  # pragma: no cover
            torch = None
        if torch is not None and isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise ValueError("oracle takes host tensors")
            if x.dim() != 2 or x.stride(1) != 1:
                raise ValueError("expected a 2-D tensor with unit column stride")
            code = {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32,
                    torch.float64: FP64}[x.dtype]
            if x.dtype in (torch.bfloat16, torch.float16):
                arr = x.view(torch.int16).numpy()
            else:
                arr = x.numpy()
            return arr, code, x.shape[0], x.shape[1], x.stride(0)
        arr = np.asarray(x)
        if arr.ndim != 2 or arr.strides[1] != arr.itemsize:
            raise ValueError("expected a 2-D array with unit column stride")
        code = {np.dtype(np.float16): FP16, np.dtype(np.float32): FP32,
                np.dtype(np.float64): FP64}.get(arr.dtype)
        if code is None:
            raise ValueError(f"unsupported numpy dtype {arr.dtype} (bf16 goes in as a torch tensor)")
        return arr, code, arr.shape[0], arr.shape[1], arr.strides[0] // arr.itemsize

    @staticmethod
    def _ptr(arr):
        return ctypes.c_void_p(arr.ctypes.data) if arr is not None else None

    @staticmethod
    def _r_hat(r):
        try:
            import torch
        except ImportError:  # pragma: no cover
            torch = None
        if torch is not None and isinstance(r, torch.Tensor):
            r = r.contiguous()
            if r.dtype == torch.bfloat16:
                return np.ascontiguousarray(r.view(torch.int16).numpy()), BF16
            return np.ascontiguousarray(r.to(torch.float64).numpy()), FP64
        r = np.asarray(r)
        if r.dtype == np.uint16 or r.dtype == np.int16:
            return np.ascontiguousarray(r), BF16
        return np.ascontiguousarray(r, dtype=np.float64), FP64

    @staticmethod
    def _lambda(lam, channels):
        if lam is None:
            return None
        try:
            import torch
            if isinstance(lam, torch.Tensor):
                lam = lam.detach().cpu().numpy()
        except ImportError:  # pragma: no cover
            pass
        lam = np.ascontiguousarray(lam, dtype=np.float32)
        if lam.shape != (channels,):
            raise ValueError("lambda must have one fp32 entry per channel")
        return lam

    # -- entry points -----------------------------------------------------
    def quant(self, x):
        arr, code, T, C, stride = self._raw(x)
        codes = np.zeros((T, C // 2), np.uint8)
        scales = np.zeros((T, C // GROUP), np.uint8)
        rc = self.lib.oracle_quant(self._ptr(arr), code, _i64(T), _i64(C), _i64(stride),
                                   self._ptr(codes), self._ptr(scales))
        if rc != 0:
            raise ValueError(f"oracle_quant rejected the shape (rc={rc})")
        return codes, scales

    def rotate_quant(self, x, lam, r_hat, want_y: bool = False):
        arr, code, T, C, stride = self._raw(x)
        lam = self._lambda(lam, C)
        r, r_code = self._r_hat(r_hat)
        if r.shape != (GROUP, GROUP):
            raise ValueError("r_hat must be 32x32")
        codes = np.zeros((T, C // 2), np.uint8)
        scales = np.zeros((T, C // GROUP), np.uint8)
        y = np.zeros((T, C), np.float64) if want_y else None
        rc = self.lib.oracle_rotate_quant(self._ptr(arr), code, _i64(T), _i64(C), _i64(stride),
                                          self._ptr(lam), self._ptr(r), r_code,
                                          self._ptr(codes), self._ptr(scales), self._ptr(y))
        if rc != 0:
            raise ValueError(f"oracle_rotate_quant rejected the shape (rc={rc})")
        return (codes, scales, y) if want_y else (codes, scales)

    def rotate_quant_block(self, x, lam, r_block, want_y: bool = False):
        """Rotation by a B x B block (B = 16, 32, 64, 128: the block sizes of
        the DuQuant++ page's ablation, sec. 4.3), then MXFP4 of every 32-wide
        group.  ``r_block`` is B x B (bf16 torch tensor or fp64 array)."""
        arr, code, T, C, stride = self._raw(x)
        lam = self._lambda(lam, C)
        r, r_code = self._r_hat(r_block)
        B = r.shape[0]
        if r.shape != (B, B):
            raise ValueError("r_block must be square")
        codes = np.zeros((T, C // 2), np.uint8)
        scales = np.zeros((T, C // GROUP), np.uint8)
        y = np.zeros((T, C), np.float64) if want_y else None
        rc = self.lib.oracle_rotate_quant_block(self._ptr(arr), code, _i64(T), _i64(C), _i64(stride),
                                                self._ptr(lam), self._ptr(r), r_code, B,
                                                self._ptr(codes), self._ptr(scales), self._ptr(y))
        if rc != 0:
            raise ValueError(f"oracle_rotate_quant_block rejected the arguments (rc={rc})")
        return (codes, scales, y) if want_y else (codes, scales)

    def norm_rotate_quant(self, x, norm: str, gamma, beta, eps: float, lam, r_hat, want_y: bool = False):
        """RMSNorm ("rms") or LayerNorm ("layer") of each row, times gamma plus
        beta, then x / lam, the block rotation and MXFP4 (sec. 5.2 item 1 of
        the DuQuant++ page: the smoothing folds into the norm's output)."""
        arr, code, T, C, stride = self._raw(x)
        kind = {"rms": 0, "layer": 1}[norm]
        gamma = self._lambda(gamma, C)
        beta = self._lambda(beta, C)
        lam = self._lambda(lam, C)
        r, r_code = self._r_hat(r_hat)
        if r.shape != (GROUP, GROUP):
            raise ValueError("r_hat must be 32x32")
        codes = np.zeros((T, C // 2), np.uint8)
        scales = np.zeros((T, C // GROUP), np.uint8)
        y = np.zeros((T, C), np.float64) if want_y else None
        rc = self.lib.oracle_norm_rotate_quant(self._ptr(arr), code, _i64(T), _i64(C), _i64(stride), kind,
                                               self._ptr(gamma), self._ptr(beta), ctypes.c_double(eps),
                                               self._ptr(lam), self._ptr(r), r_code,
                                               self._ptr(codes), self._ptr(scales), self._ptr(y))
        if rc != 0:
            raise ValueError(f"oracle_norm_rotate_quant rejected the arguments (rc={rc})")
        return (codes, scales, y) if want_y else (codes, scales)

    def encode_groups(self, y):
        y = np.ascontiguousarray(y, dtype=np.float64).reshape(-1, GROUP)
        G = y.shape[0]
        codes = np.zeros((G, GROUP // 2), np.uint8)
        scales = np.zeros((G,), np.uint8)
        rc = self.lib.oracle_encode_groups(self._ptr(y), _i64(G), self._ptr(codes), self._ptr(scales))
        if rc != 0:
            raise ValueError("oracle_encode_groups failed")
        return codes, scales

    def dequant(self, codes, scales):
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        T, half = codes.shape
        C = half * 2
        if scales.shape != (T, C // GROUP):
            raise ValueError("scales must be [tokens][channels/32]")
        out = np.zeros((T, C), np.float64)
        rc = self.lib.oracle_dequant(self._ptr(codes), self._ptr(scales), _i64(T), _i64(C),
                                     self._ptr(out))
        if rc != 0:
            raise ValueError("oracle_dequant rejected the shape")
        return out

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


# ---- pure-NumPy checkers ----------------------------------------------------

def code_value(codes):
    """Value of each 4-bit E2M1 code (0x8 is -0.0)."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = E2M1_VALUES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def brute_force_codes(v):
    """Nearest E2M1 code for each value of ``v`` (already divided by the scale).

    Exhaustive over all 16 codes: minimise |v - value(code)|; among equally
    near codes keep one whose magnitude code is even; a zero result is +0.
    Magnitudes above 8 are clipped to 8 first, which changes no decision (the
    nearest grid point of anything beyond 6 is 6) and keeps the fp64
    distances meaningful for huge inputs.
    """
    v = np.clip(np.asarray(v, dtype=np.float64), -8.0, 8.0).reshape(-1)
    all_codes = np.arange(16)
    vals = code_value(all_codes)
    dist = np.abs(v[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    tied = dist == best
    odd = (all_codes & 7) % 2
    pick = np.where(tied, odd[None, :] * 32 + all_codes[None, :], 1 << 20).argmin(axis=1)
    return np.where((pick & 7) == 0, 0, pick).astype(np.uint8)


def unpack_codes(packed):
    """[..., C/2] bytes -> [..., C] codes (low nibble is the even element)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def group_error(y, dq):
    """Per-group ||dq_g - y_g|| / ||y_g|| over 32-wide groups; zero groups dropped."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, GROUP)
    dq = np.asarray(dq, dtype=np.float64).reshape(-1, GROUP)
    ny = np.linalg.norm(y, axis=1)
    keep = ny > 0
    return np.linalg.norm(dq[keep] - y[keep], axis=1) / ny[keep]


# ---- MXFP4 x MXFP4 product (the consumer of the quantized activations) -----

def gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, orc: "Oracle | None" = None):
    """Y = dq(A) dq(B)^T in fp64, and S = |dq(A)| |dq(B)|^T (the sum of
    |products| per output, the scale of the fp32 accumulation error).

    A is [M, K] MXFP4 (codes [M, K/2], scales [M, K/32]); B is [N, K] (the
    weights, quantized along the reduction dimension K).  The DuQuant++ page
    (sec. 3.3, 5.4 item 3) feeds the rotated, quantized activations to an
    MXFP4 linear layer with pre-absorbed, pre-quantized weights; this is that
    product, exactly (dequantization is exact, the matmul is fp64)."""
    orc = orc or default()
    a = orc.dequant(a_codes, a_scales)
    b = orc.dequant(b_codes, b_scales)
    return a @ b.T, np.abs(a) @ np.abs(b).T


def _as_f64(a):
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def absorb_weights(w_lin, lam, r):
    """Rows of the absorbed weight matrix, in fp64.

    The DuQuant++ page (sec. 3.3, eq. for W-hat) folds the smoothing and the
    rotation into the weights: with Y = X W, W-hat = R^T Lambda W, so that
    (X Lambda^-1 R)(R^T Lambda W) = X W for orthogonal R.  ``w_lin`` holds W
    transposed, one row per output feature ([N, K], the usual linear-layer
    layout); row n of W-hat^T is (w_n * Lambda) BlockDiag(R, ..., R), i.e.
    each 32-channel group of w_n * Lambda times the shared 32x32 block.
    ``lam`` may be None (Lambda = I)."""
    w = _as_f64(w_lin)
    if lam is not None:
        w = w * _as_f64(lam)[None, :]
    N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    r = _as_f64(r)
    return (w.reshape(N, K // GROUP, GROUP) @ r).reshape(N, K)


def absorb_quant(w_lin, lam, r, orc: "Oracle | None" = None):
    """MXFP4 codes [N, K/2] and scales [N, K/32] of the absorbed weights
    (each row quantized along K, the reduction dimension of the product)."""
    orc = orc or default()
    w = absorb_weights(w_lin, lam, r)
    N, K = w.shape
    codes, scales = orc.encode_groups(w)
    return codes.reshape(N, K // 2), scales.reshape(N, K // GROUP)


# ---- fragment-tiled storage of MXFP4 operands --------------------------------
#
# A storage order, not arithmetic: the pages fix no memory layout.  An MXFP4
# operand of R rows and K reduction positions (codes [R, K/2], scales
# [R, K/32], K a multiple of 128) is cut into records of 16 rows x 128
# positions.  Record (t, s) -- rows 16 t .. 16 t + 15, positions 128 s ..
# 128 s + 127 -- has index t * (K / 128) + s and 64 slots; slot l belongs to
# row 16 t + l % 16 and group 4 s + l // 16 (32 positions).  The code record
# holds the slots' 16 code bytes one after another (1024 bytes), the scale
# record their scale bytes (64 bytes).  Rows past R in the last record row
# are padding, written as zero bytes here.  The slot order is the operand
# order of the 16 x 16 x 128 scaled matrix-core instruction (lane l: row
# l % 16, group l // 16), so a record is one contiguous operand fragment.

TILE_ROWS, TILE_K = 16, 128


def _tile_dims(rows, K):
    if K % TILE_K:
        raise ValueError("K must be a multiple of 128")
    return -(-rows // TILE_ROWS), K // TILE_K


def tile_mxfp4(codes, scales):
    """Row layout -> fragment-tiled layout; returns flat uint8 arrays of
    ceil(R/16) * (K/128) * 1024 code bytes and * 64 scale bytes."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    R, half = codes.shape
    K = 2 * half
    if scales.shape != (R, K // GROUP):
        raise ValueError("scales must be [rows, K/32]")
    rt, nk = _tile_dims(R, K)
    pc = np.zeros((rt * TILE_ROWS, half), np.uint8)
    pc[:R] = codes
    ps = np.zeros((rt * TILE_ROWS, K // GROUP), np.uint8)
    ps[:R] = scales
    # [t, row-in-tile, s, group-in-stage, byte] -> [t, s, group-in-stage, row-in-tile, byte]
    tc = pc.reshape(rt, TILE_ROWS, nk, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    ts = ps.reshape(rt, TILE_ROWS, nk, 4).transpose(0, 2, 3, 1).reshape(-1)
    return np.ascontiguousarray(tc), np.ascontiguousarray(ts)


def untile_mxfp4(tcodes, tscales, rows, K):
    """Inverse of :func:`tile_mxfp4` (padding rows dropped)."""
    rt, nk = _tile_dims(rows, K)
    tc = np.asarray(tcodes, np.uint8).reshape(rt, nk, 4, TILE_ROWS, 16)
    ts = np.asarray(tscales, np.uint8).reshape(rt, nk, 4, TILE_ROWS)
    codes = tc.transpose(0, 3, 1, 2, 4).reshape(rt * TILE_ROWS, K // 2)[:rows]
    scales = ts.transpose(0, 3, 1, 2).reshape(rt * TILE_ROWS, K // GROUP)[:rows]
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)
