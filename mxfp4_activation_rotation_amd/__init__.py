"""MI355X (gfx950) online smoothing + block rotation + MXFP4 quantization.

Thin ctypes binding over ``libmxq.so`` (C ABI in ``include/mxq.h``).  Every
step of the path runs in the library's HIP kernels; PyTorch only provides
device memory and the current stream.  There is no CPU fallback: importing
works without the library, but every call raises if it is not built.

Functions follow the online transform of the DuQuant++ page
(sec. 3.3: X * Lambda^-1 * R, R block diagonal with one shared 32x32 block)
and its MXFP4 encoding (sec. 2.1).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libmxq.so")

MXQ_BF16, MXQ_FP16, MXQ_FP32 = 0, 1, 2
STATUS = {0: "MXQ_OK", 1: "MXQ_ERR_NULL", 2: "MXQ_ERR_SHAPE", 3: "MXQ_ERR_DTYPE",
          4: "MXQ_ERR_ALIGN", 5: "MXQ_ERR_STRIDE", 6: "MXQ_ERR_HIP"}
EXPORTS = ("mxq_rotate_quant", "mxq_rotate_quant_ex", "mxq_quant", "mxq_dequant",
           "mxq_status_str", "mxq_plan", "mxq_version", "mxq_calib_workspace_bytes",
           "mxq_calib_worst_group", "mxq_calib_givens", "mxq_absorb_quant", "mxq_gemm_mxfp4",
           "mxq_norm_rotate_quant", "mxq_rotate_quant_block", "mxq_tile_mxfp4", "mxq_rotate_quant_tiled",
           "mxq_gemm_mxfp4_tiled", "mxq_norm_rotate_quant_tiled", "mxq_calib_worst_group_noalloc",
           "mxq_calib_givens_angles")

_lib = None


class MXQError(RuntimeError):
    def __init__(self, fn, status):
        self.status = int(status)
        super().__init__(f"{fn}: {STATUS.get(self.status, self.status)}")


def library_path() -> str:
    return LIBRARY


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmxq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() "
                           "or python -m mxfp4_activation_rotation_amd._build")
    lib = ctypes.CDLL(p)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mxq_rotate_quant.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.mxq_rotate_quant_ex.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.mxq_quant.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    lib.mxq_dequant.argtypes = [vp, vp, i64, i64, vp, i32, vp]
    lib.mxq_status_str.argtypes = [i32]
    lib.mxq_status_str.restype = ctypes.c_char_p
    lib.mxq_plan.argtypes = [i64, i64, i32, ctypes.POINTER(ctypes.c_int32)]
    sz = ctypes.c_size_t
    lib.mxq_calib_workspace_bytes.argtypes = [i64]
    lib.mxq_calib_workspace_bytes.restype = sz
    lib.mxq_calib_worst_group.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.mxq_calib_givens.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.mxq_calib_givens_angles.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mxq_calib_worst_group_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.mxq_absorb_quant.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.mxq_gemm_mxfp4.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp]
    lib.mxq_gemm_mxfp4_tiled.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp]
    lib.mxq_tile_mxfp4.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.mxq_rotate_quant_tiled.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.mxq_norm_rotate_quant_tiled.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, ctypes.c_float, vp, vp, vp,
                                                vp, vp]
    lib.mxq_rotate_quant_block.argtypes = [vp, i32, i64, i64, i64, vp, vp, i32, vp, vp, vp, vp]
    lib.mxq_norm_rotate_quant.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                          vp, vp]
    for f in ("mxq_rotate_quant", "mxq_rotate_quant_ex", "mxq_quant", "mxq_dequant", "mxq_plan",
              "mxq_version", "mxq_calib_worst_group", "mxq_calib_givens", "mxq_absorb_quant",
              "mxq_gemm_mxfp4", "mxq_norm_rotate_quant", "mxq_rotate_quant_block", "mxq_tile_mxfp4",
              "mxq_rotate_quant_tiled", "mxq_gemm_mxfp4_tiled", "mxq_norm_rotate_quant_tiled",
              "mxq_calib_worst_group_noalloc", "mxq_calib_givens_angles"):
        getattr(lib, f).restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


_DT = {torch.bfloat16: MXQ_BF16, torch.float16: MXQ_FP16, torch.float32: MXQ_FP32}
_HALF_TYPES = (torch.bfloat16, torch.float16)


try:  # raw current-stream handle without building a Stream object
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover
    _raw_stream = None


def _stream(t: torch.Tensor, stream, dev: int | None = None):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(t.get_device() if dev is None else dev)
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _on(name: str, t: torch.Tensor, device: torch.device):
    """Every tensor handed to the library must live on the GPU the call runs
    on: a host pointer would reach a kernel, which the C layer cannot detect."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")


def _check_x(x: torch.Tensor, allowed):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens, channels]")
    T, C = x.shape
    st = x.stride()
    if T > 0 and C > 0 and st[1] != 1:
        raise ValueError("x must have unit column stride")
    if x.dtype not in allowed:
        raise ValueError(f"unsupported x dtype {x.dtype}")
    return T, C, (st[0] if T > 1 else C)


# Per-call checks compare device indices (get_device(): -1 for host
# tensors) rather than torch.device objects, which cost several times more
# to build and compare; a decode-sized call spends most of its host time here.
def _outputs(x, T, C, codes, scales, dev: int | None = None):
    if dev is None:
        dev = x.get_device()
    if codes is None:
        codes = torch.empty((T, C // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T, C // 32), dtype=torch.uint8, device=x.device)
    if codes.dtype != torch.uint8 or codes.shape != (T, C // 2) or not codes.is_contiguous() \
            or codes.get_device() != dev:
        raise ValueError(f"codes must be a contiguous uint8 tensor of shape {(T, C // 2)} on {x.device}")
    if scales.dtype != torch.uint8 or scales.shape != (T, C // 32) or not scales.is_contiguous() \
            or scales.get_device() != dev:
        raise ValueError(f"scales must be a contiguous uint8 tensor of shape {(T, C // 32)} on {x.device}")
    return codes, scales


def rotate_quant(x: torch.Tensor, r_hat: torch.Tensor, lam: torch.Tensor | None = None, *,
                 codes=None, scales=None, y_rot=None, stream=None):
    """codes, scales = MXFP4(x / lam @ BlockDiag(r_hat)) (and y_rot if given).

    x: bf16/fp16 [tokens, channels] on the GPU; r_hat: bf16 [32, 32] with
    y_n = sum_k x_k r_hat[k, n]; lam: fp32 [channels] or None.  y_rot, if
    given, is a contiguous fp32 [tokens, channels] tensor that receives the
    rotated values (test and error-study use).
    """
    lib = _lib or load()
    T, C, stride = _check_x(x, _HALF_TYPES)
    dev = x.get_device()
    if r_hat.dtype != torch.bfloat16 or r_hat.shape != (32, 32) or not r_hat.is_contiguous() \
            or r_hat.get_device() != dev:
        raise ValueError("r_hat must be a contiguous bf16 [32, 32] tensor on x's device")
    if lam is not None and (lam.dtype != torch.float32 or lam.shape != (C,) or not lam.is_contiguous()
                            or lam.get_device() != dev):
        raise ValueError("lam must be a contiguous fp32 [channels] tensor on x's device")
    codes, scales = _outputs(x, T, C, codes, scales, dev)
    if y_rot is not None:
        if y_rot.dtype != torch.float32 or y_rot.shape != (T, C) or not y_rot.is_contiguous():
            raise ValueError("y_rot must be a contiguous fp32 [tokens, channels] tensor")
        _on("y_rot", y_rot, x.device)
        st = lib.mxq_rotate_quant_ex(_ptr(x), _DT[x.dtype], T, C, stride, _ptr(lam), _ptr(r_hat),
                                     _ptr(codes), _ptr(scales), _ptr(y_rot), _stream(x, stream))
        fn = "mxq_rotate_quant_ex"
    else:
        st = lib.mxq_rotate_quant(x.data_ptr(), _DT[x.dtype], T, C, stride, _ptr(lam), r_hat.data_ptr(),
                                  codes.data_ptr(), scales.data_ptr(), _stream(x, stream, dev))
        fn = "mxq_rotate_quant"
    if st != 0:
        raise MXQError(fn, st)
    return codes, scales


def quant(x: torch.Tensor, *, codes=None, scales=None, stream=None):
    """Plain MXFP4 quantization of bf16/fp16/fp32 x [tokens, channels]."""
    lib = load()
    T, C, stride = _check_x(x, (torch.bfloat16, torch.float16, torch.float32))
    codes, scales = _outputs(x, T, C, codes, scales)
    st = lib.mxq_quant(_ptr(x), _DT[x.dtype], T, C, stride, _ptr(codes), _ptr(scales), _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_quant", st)
    return codes, scales


def dequant(codes: torch.Tensor, scales: torch.Tensor, out_dtype=torch.float32, *, out=None, stream=None):
    """Decode MXFP4 codes/scales [tokens, channels/2], [tokens, channels/32] to bf16 or fp32."""
    lib = load()
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or codes.dim() != 2:
        raise ValueError("codes and scales must be uint8 2-D tensors")
    if not codes.is_cuda:
        raise ValueError("codes must be a device tensor")
    _on("scales", scales, codes.device)
    T, C = codes.shape[0], codes.shape[1] * 2
    if tuple(scales.shape) != (T, C // 32) or not codes.is_contiguous() or not scales.is_contiguous():
        raise ValueError("scales must be contiguous [tokens, channels/32]; codes contiguous")
    if out is None:
        out = torch.empty((T, C), dtype=out_dtype, device=codes.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or tuple(out.shape) != (T, C) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16/fp32 [tokens, channels] tensor")
    _on("out", out, codes.device)
    st = lib.mxq_dequant(_ptr(codes), _ptr(scales), T, C, _ptr(out), _DT[out.dtype], _stream(codes, stream))
    if st != 0:
        raise MXQError("mxq_dequant", st)
    return out


def absorb_quant(w: torch.Tensor, r_hat: torch.Tensor, lam: torch.Tensor | None = None, *,
                 codes=None, scales=None, stream=None):
    """Quantized absorbed weights: codes, scales = MXFP4((w * lam) @ BlockDiag(r_hat)).

    w: bf16/fp16 [N, K] on the GPU, one row per output feature (W^T of
    Y = X W); lam: fp32 [K] or None; r_hat as in :func:`rotate_quant`.  The
    result is the B operand of :func:`gemm_mxfp4`.
    """
    lib = load()
    N, K, stride = _check_x(w, (torch.bfloat16, torch.float16))
    if r_hat.dtype != torch.bfloat16 or r_hat.shape != (32, 32) or not r_hat.is_contiguous() \
            or r_hat.device != w.device:
        raise ValueError("r_hat must be a contiguous bf16 [32, 32] tensor on w's device")
    if lam is not None and (lam.dtype != torch.float32 or lam.shape != (K,) or not lam.is_contiguous()
                            or lam.device != w.device):
        raise ValueError("lam must be a contiguous fp32 [K] tensor on w's device")
    codes, scales = _outputs(w, N, K, codes, scales)
    st = lib.mxq_absorb_quant(_ptr(w), _DT[w.dtype], N, K, stride, _ptr(lam), _ptr(r_hat),
                              _ptr(codes), _ptr(scales), _stream(w, stream))
    if st != 0:
        raise MXQError("mxq_absorb_quant", st)
    return codes, scales


def gemm_mxfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
               out_dtype=torch.float32, *, out=None, stream=None):
    """y [M, N] = dq(A) @ dq(B)^T on the scaled matrix cores.

    A = (a_codes [M, K/2], a_scales [M, K/32]) from :func:`rotate_quant`,
    B = (b_codes [N, K/2], b_scales [N, K/32]) from :func:`absorb_quant`.
    out: optional fp32/bf16 [M, N] tensor with unit column stride.
    """
    lib = load()
    for t in (a_codes, a_scales, b_codes, b_scales):
        if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("codes and scales must be contiguous uint8 2-D device tensors")
        _on("operand", t, a_codes.device)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    if b_codes.shape[1] * 2 != K or tuple(a_scales.shape) != (M, K // 32) or tuple(b_scales.shape) != (N, K // 32):
        raise ValueError("operand shapes disagree: codes [rows, K/2], scales [rows, K/32]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or tuple(out.shape) != (M, N) or \
            (M > 0 and N > 0 and out.stride(1) != 1):
        raise ValueError("out must be a bf16/fp32 [M, N] tensor with unit column stride")
    _on("out", out, a_codes.device)
    ldy = out.stride(0) if M > 1 else N
    st = lib.mxq_gemm_mxfp4(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
                            _ptr(out), _DT[out.dtype], ldy, _stream(a_codes, stream))
    if st != 0:
        raise MXQError("mxq_gemm_mxfp4", st)
    return out


def rotate_quant_block(x: torch.Tensor, r_block: torch.Tensor, lam: torch.Tensor | None = None, *,
                       codes=None, scales=None, y_rot=None, stream=None):
    """MXFP4 of x / lam rotated block by block with a B x B bf16 matrix
    (B = 16, 32, 64, 128: the block sizes of the DuQuant++ page's ablation)."""
    lib = load()
    T, C, stride = _check_x(x, (torch.bfloat16, torch.float16))
    B = r_block.shape[0]
    if r_block.dtype != torch.bfloat16 or r_block.dim() != 2 or r_block.shape != (B, B) \
            or not r_block.is_contiguous() or r_block.device != x.device:
        raise ValueError("r_block must be a contiguous square bf16 tensor on x's device")
    if lam is not None and (lam.dtype != torch.float32 or lam.shape != (C,) or not lam.is_contiguous()
                            or lam.device != x.device):
        raise ValueError("lam must be a contiguous fp32 [channels] tensor on x's device")
    codes, scales = _outputs(x, T, C, codes, scales)
    if y_rot is not None and (y_rot.dtype != torch.float32 or y_rot.shape != (T, C) or not y_rot.is_contiguous()):
        raise ValueError("y_rot must be a contiguous fp32 [tokens, channels] tensor")
    if y_rot is not None:
        _on("y_rot", y_rot, x.device)
    st = lib.mxq_rotate_quant_block(_ptr(x), _DT[x.dtype], T, C, stride, _ptr(lam), _ptr(r_block), B,
                                    _ptr(codes), _ptr(scales), _ptr(y_rot), _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_rotate_quant_block", st)
    return codes, scales


NORM_KINDS = {"rms": 0, "layer": 1}


def _check_norm_args(x, r_hat, gamma, beta, lam, norm):
    T, C, stride = _check_x(x, (torch.bfloat16, torch.float16))
    if r_hat.dtype != torch.bfloat16 or r_hat.shape != (32, 32) or not r_hat.is_contiguous() \
            or r_hat.device != x.device:
        raise ValueError("r_hat must be a contiguous bf16 [32, 32] tensor on x's device")
    for name, t, required in (("gamma", gamma, True), ("beta", beta, False), ("lam", lam, False)):
        if t is None and not required:
            continue
        if t is None or t.dtype != torch.float32 or t.shape != (C,) or not t.is_contiguous() or t.device != x.device:
            raise ValueError(f"{name} must be a contiguous fp32 [channels] tensor on x's device")
    if norm not in NORM_KINDS:
        raise ValueError(f"norm must be one of {sorted(NORM_KINDS)}")
    return T, C, stride


def norm_rotate_quant(x: torch.Tensor, r_hat: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor | None = None,
                      lam: torch.Tensor | None = None, *, norm: str = "rms", eps: float = 1e-5, codes=None,
                      scales=None, y_rot=None, stream=None):
    """codes, scales = MXFP4(((norm(x) * gamma + beta) / lam) @ BlockDiag(r_hat)).

    norm is "rms" (RMSNorm) or "layer" (LayerNorm); x is the norm's bf16/fp16
    input [tokens, channels <= 16384]; gamma, beta, lam are contiguous fp32
    [channels] tensors on x's device (beta and lam may be None).
    """
    lib = load()
    T, C, stride = _check_norm_args(x, r_hat, gamma, beta, lam, norm)
    codes, scales = _outputs(x, T, C, codes, scales)
    if y_rot is not None and (y_rot.dtype != torch.float32 or y_rot.shape != (T, C) or not y_rot.is_contiguous()):
        raise ValueError("y_rot must be a contiguous fp32 [tokens, channels] tensor")
    if y_rot is not None:
        _on("y_rot", y_rot, x.device)
    st = lib.mxq_norm_rotate_quant(_ptr(x), _DT[x.dtype], T, C, stride, NORM_KINDS[norm], _ptr(gamma), _ptr(beta),
                                   ctypes.c_float(eps), _ptr(lam), _ptr(r_hat), _ptr(codes), _ptr(scales),
                                   _ptr(y_rot), _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_norm_rotate_quant", st)
    return codes, scales


def plan(tokens: int, channels: int, cu_count: int = 256):
    """Launch plan {blocks, waves, tile_columns, row_step, waves_per_block} (host only)."""
    lib = load()
    out = (ctypes.c_int32 * 5)()
    st = lib.mxq_plan(tokens, channels, cu_count, out)
    if st != 0:
        raise MXQError("mxq_plan", st)
    return dict(zip(("blocks", "waves", "tile_columns", "row_step", "waves_per_block"), list(out)))


# ---- offline calibration of the shared block (DuQuant++ page sec. 3.2) -----

def _workspace(channels: int, device):
    n = int(load().mxq_calib_workspace_bytes(channels))
    return torch.empty((n + 256,), dtype=torch.uint8, device=device), n


def _aligned256(buf):
    ptr = buf.data_ptr()
    return ptr + ((-ptr) % 256)


def calib_worst_group(x: torch.Tensor, lam: torch.Tensor | None = None, *, stream=None):
    """(x_worst [tokens, 32] fp64, group index tensor, its largest |value| tensor).

    x: bf16/fp16/fp32 calibration activations [tokens, channels] on the GPU;
    lam: fp32 [channels] or None.  The group and value stay on the device
    (0-d tensors) so the call does not synchronize."""
    lib = load()
    T, C, stride = _check_x(x, (torch.bfloat16, torch.float16, torch.float32))
    if lam is not None and (lam.dtype != torch.float32 or lam.shape != (C,) or not lam.is_contiguous()):
        raise ValueError("lam must be a contiguous fp32 [channels] tensor")
    if lam is not None:
        _on("lam", lam, x.device)
    xw = torch.empty((T, 32), dtype=torch.float64, device=x.device)
    group = torch.empty((), dtype=torch.int64, device=x.device)
    linf = torch.empty((), dtype=torch.float64, device=x.device)
    ws, n = _workspace(C, x.device)
    st = lib.mxq_calib_worst_group(_ptr(x), _DT[x.dtype], T, C, stride, _ptr(lam), _ptr(xw), _ptr(group),
                                   _ptr(linf), _aligned256(ws), n, _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_calib_worst_group", st)
    return xw, group, linf


def calib_worst_group_noalloc(x: torch.Tensor, lam: torch.Tensor | None = None, *, x_worst=None, group=None,
                              linf=None, stream=None):
    """:func:`calib_worst_group` through the entry point that allocates
    nothing (its scratch is a library-owned device array; channels <= 262144).
    The outputs may be passed in, so a caller that cannot allocate can make
    the whole call without allocating."""
    lib = load()
    T, C, stride = _check_x(x, (torch.bfloat16, torch.float16, torch.float32))
    if lam is not None and (lam.dtype != torch.float32 or lam.shape != (C,) or not lam.is_contiguous()):
        raise ValueError("lam must be a contiguous fp32 [channels] tensor")
    if lam is not None:
        _on("lam", lam, x.device)
    xw = torch.empty((T, 32), dtype=torch.float64, device=x.device) if x_worst is None else x_worst
    group = torch.empty((), dtype=torch.int64, device=x.device) if group is None else group
    linf = torch.empty((), dtype=torch.float64, device=x.device) if linf is None else linf
    for name, t, dt, shape in (("x_worst", xw, torch.float64, (T, 32)), ("group", group, torch.int64, ()),
                               ("linf", linf, torch.float64, ())):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape}")
        _on(name, t, x.device)
    st = lib.mxq_calib_worst_group_noalloc(_ptr(x), _DT[x.dtype], T, C, stride, _ptr(lam), _ptr(xw), _ptr(group),
                                           _ptr(linf), _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_calib_worst_group_noalloc", st)
    return xw, group, linf


def calib_givens(x_worst: torch.Tensor, max_steps: int = 128, *, stream=None):
    """Greedy Givens search on x_worst [tokens, 32] fp64 (overwritten with
    x_worst @ R).  Returns (R [32, 32] fp64, history [max_steps + 1] fp64,
    steps_done 0-d int32, pairs [max_steps, 2] int32), all on the device;
    entries of history and pairs past steps_done are unspecified."""
    lib = load()
    if x_worst.dtype != torch.float64 or x_worst.dim() != 2 or x_worst.shape[1] != 32 \
            or not x_worst.is_contiguous() or not x_worst.is_cuda:
        raise ValueError("x_worst must be a contiguous fp64 [tokens, 32] device tensor")
    dev = x_worst.device
    r = torch.empty((32, 32), dtype=torch.float64, device=dev)
    hist = torch.empty((max_steps + 1,), dtype=torch.float64, device=dev)
    done = torch.empty((), dtype=torch.int32, device=dev)
    pairs = torch.empty((max(max_steps, 1), 2), dtype=torch.int32, device=dev)
    ws, n = _workspace(0, dev)
    st = lib.mxq_calib_givens(_ptr(x_worst), x_worst.shape[0], max_steps, _ptr(r), _ptr(hist), _ptr(done),
                              _ptr(pairs), _aligned256(ws), n, _stream(x_worst, stream))
    if st != 0:
        raise MXQError("mxq_calib_givens", st)
    return r, hist, done, pairs


def calib_givens_angles(x_worst: torch.Tensor, max_steps: int = 128, angle_grid: int = 64, *, stream=None):
    """:func:`calib_givens` with a per-candidate angle from a grid of
    ``angle_grid`` angles (index 0 = pi/4, index k: tan(theta / 2) = k / M).
    Returns (R, history, steps_done, pairs, angles [max_steps] int32), all on
    the device; entries past steps_done are unspecified."""
    lib = load()
    if x_worst.dtype != torch.float64 or x_worst.dim() != 2 or x_worst.shape[1] != 32 \
            or not x_worst.is_contiguous() or not x_worst.is_cuda:
        raise ValueError("x_worst must be a contiguous fp64 [tokens, 32] device tensor")
    dev = x_worst.device
    r = torch.empty((32, 32), dtype=torch.float64, device=dev)
    hist = torch.empty((max_steps + 1,), dtype=torch.float64, device=dev)
    done = torch.empty((), dtype=torch.int32, device=dev)
    pairs = torch.empty((max(max_steps, 1), 2), dtype=torch.int32, device=dev)
    angles = torch.empty((max(max_steps, 1),), dtype=torch.int32, device=dev)
    ws, n = _workspace(0, dev)
    st = lib.mxq_calib_givens_angles(_ptr(x_worst), x_worst.shape[0], max_steps, angle_grid, _ptr(r), _ptr(hist),
                                     _ptr(done), _ptr(pairs), _ptr(angles), _aligned256(ws), n,
                                     _stream(x_worst, stream))
    if st != 0:
        raise MXQError("mxq_calib_givens_angles", st)
    return r, hist, done, pairs, angles


# ---- fragment-tiled operands (records of 16 rows x 128 positions in the
# operand order of the 16 x 16 x 128 scaled MFMA; layout in include/mxq.h) --

def tiled_sizes(rows: int, K: int):
    """Bytes of the tiled code and scale buffers of a rows x K operand."""
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    padded = (rows + 15) // 16 * 16
    return padded * K // 2, padded * K // 32


def _tiled_outputs(device, rows, K, tcodes, tscales):
    nc, ns = tiled_sizes(rows, K)
    if tcodes is None:
        tcodes = torch.empty((nc,), dtype=torch.uint8, device=device)
    if tscales is None:
        tscales = torch.empty((ns,), dtype=torch.uint8, device=device)
    for name, t, n in (("tcodes", tcodes, nc), ("tscales", tscales, ns)):
        if t.dtype != torch.uint8 or t.numel() != n or not t.is_contiguous() or t.device != device:
            raise ValueError(f"{name} must be a contiguous uint8 tensor of {n} bytes on {device}")
    return tcodes, tscales


def tile_mxfp4(codes: torch.Tensor, scales: torch.Tensor, *, tcodes=None, tscales=None, stream=None):
    """Row-layout MXFP4 (codes [rows, K/2], scales [rows, K/32]) to the
    fragment-tiled layout (flat uint8 tensors; padding rows zero)."""
    lib = load()
    if codes.dtype != torch.uint8 or codes.dim() != 2 or not codes.is_contiguous() or not codes.is_cuda:
        raise ValueError("codes must be a contiguous uint8 2-D device tensor")
    R, K = codes.shape[0], codes.shape[1] * 2
    if scales.dtype != torch.uint8 or tuple(scales.shape) != (R, K // 32) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous uint8 [rows, K/32] tensor")
    _on("scales", scales, codes.device)
    tcodes, tscales = _tiled_outputs(codes.device, R, K, tcodes, tscales)
    st = lib.mxq_tile_mxfp4(_ptr(codes), _ptr(scales), R, K, _ptr(tcodes), _ptr(tscales), _stream(codes, stream))
    if st != 0:
        raise MXQError("mxq_tile_mxfp4", st)
    return tcodes, tscales


def rotate_quant_tiled(x: torch.Tensor, r_hat: torch.Tensor, lam: torch.Tensor | None = None, *,
                       tcodes=None, tscales=None, stream=None):
    """:func:`rotate_quant` with its output in the fragment-tiled layout
    (channels % 128 == 0); the A operand of :func:`gemm_mxfp4_tiled`."""
    lib = load()
    T, C, stride = _check_x(x, (torch.bfloat16, torch.float16))
    if r_hat.dtype != torch.bfloat16 or r_hat.shape != (32, 32) or not r_hat.is_contiguous() \
            or r_hat.device != x.device:
        raise ValueError("r_hat must be a contiguous bf16 [32, 32] tensor on x's device")
    if lam is not None and (lam.dtype != torch.float32 or lam.shape != (C,) or not lam.is_contiguous()
                            or lam.device != x.device):
        raise ValueError("lam must be a contiguous fp32 [channels] tensor on x's device")
    tcodes, tscales = _tiled_outputs(x.device, T, C, tcodes, tscales)
    st = lib.mxq_rotate_quant_tiled(_ptr(x), _DT[x.dtype], T, C, stride, _ptr(lam), _ptr(r_hat),
                                    _ptr(tcodes), _ptr(tscales), _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_rotate_quant_tiled", st)
    return tcodes, tscales


def gemm_mxfp4_tiled(a_tcodes: torch.Tensor, a_tscales: torch.Tensor, b_tcodes: torch.Tensor,
                     b_tscales: torch.Tensor, M: int, N: int, K: int, out_dtype=torch.float32, *,
                     out=None, stream=None):
    """:func:`gemm_mxfp4` on fragment-tiled operands (A: M x K, B: N x K);
    bit-identical results."""
    lib = load()
    for name, rows, codes, scales in (("a", M, a_tcodes, a_tscales), ("b", N, b_tcodes, b_tscales)):
        nc, ns = tiled_sizes(rows, K)
        for t, n in ((codes, nc), (scales, ns)):
            if t.dtype != torch.uint8 or t.numel() != n or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} operand: tiled buffers must be contiguous uint8 device tensors "
                                 f"of {nc} and {ns} bytes")
            _on(f"{name} operand", t, a_tcodes.device)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_tcodes.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or tuple(out.shape) != (M, N) or \
            (M > 0 and N > 0 and out.stride(1) != 1):
        raise ValueError("out must be a bf16/fp32 [M, N] tensor with unit column stride")
    _on("out", out, a_tcodes.device)
    ldy = out.stride(0) if M > 1 else N
    st = lib.mxq_gemm_mxfp4_tiled(_ptr(a_tcodes), _ptr(a_tscales), _ptr(b_tcodes), _ptr(b_tscales), M, N, K,
                                  _ptr(out), _DT[out.dtype], ldy, _stream(a_tcodes, stream))
    if st != 0:
        raise MXQError("mxq_gemm_mxfp4_tiled", st)
    return out


def norm_rotate_quant_tiled(x: torch.Tensor, r_hat: torch.Tensor, gamma: torch.Tensor,
                            beta: torch.Tensor | None = None, lam: torch.Tensor | None = None, *,
                            norm: str = "rms", eps: float = 1e-5, tcodes=None, tscales=None, stream=None):
    """:func:`norm_rotate_quant` with its output in the fragment-tiled
    layout (channels % 128 == 0); the A operand of :func:`gemm_mxfp4_tiled`."""
    lib = load()
    T, C, stride = _check_norm_args(x, r_hat, gamma, beta, lam, norm)
    tcodes, tscales = _tiled_outputs(x.device, T, C, tcodes, tscales)
    st = lib.mxq_norm_rotate_quant_tiled(_ptr(x), _DT[x.dtype], T, C, stride, NORM_KINDS[norm], _ptr(gamma),
                                         _ptr(beta), ctypes.c_float(eps), _ptr(lam), _ptr(r_hat), _ptr(tcodes),
                                         _ptr(tscales), _stream(x, stream))
    if st != 0:
        raise MXQError("mxq_norm_rotate_quant_tiled", st)
    return tcodes, tscales
