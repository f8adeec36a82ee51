"""H-BitLinear forward (BitNet v2) on AMD Instinct MI355X.

A thin ctypes binding over ``libhbl.so`` (C ABI in ``include/hbl.h``).  It
marshals torch tensors (device memory) and the current HIP stream into the
library's raw pointers; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is not built, importing
this package raises.

The method (architecture write-up of "BitNet v2: Native 4-bit Activations
with Hadamard Transformation for 1-bit LLMs", §3.4): ternary absmean weights
(Eq. 1-2), an online per-token Hadamard rotation (Eq. 3-6), per-token INT8
absmax or INT4 absmean activation codes (Eq. 7-8), and the integer matmul
with one rescale (Eq. 9).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhbl.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_WORKSPACE, ERR_HIP = 1, 2, 3, 4, 5, 6
DTYPE_F32, DTYPE_BF16 = 0, 1
HADAMARD = 1
OUT_BF16, OUT_F32, OUT_I32 = 0, 1, 2
EPS = 1e-5
MAX_K = 16384

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python bit_quantization_amd/build.py` "
        "first")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_lib = ctypes.CDLL(LIB_PATH)
_SIGS = {
    "hbl_version": ([], _I),
    "hbl_status_string": ([_I], ctypes.c_char_p),
    "hbl_last_error": ([], ctypes.c_char_p),
    "hbl_device_cu_count": ([], _I),
    "hbl_ternarize_workspace_size": ([_I64, _I64], _SZ),
    "hbl_ternarize_weights": ([_P, _I, _I64, _I64, _P, _P, _P, _SZ, _P], _I),
    "hbl_hadamard_f32": ([_P, _I, _I64, _I64, _I64, _P, _P], _I),
    "hbl_hadamard_quant": ([_P, _I, _I64, _I64, _I64, _I, _I, _P, _P, _P, _P], _I),
    "hbl_ternary_gemm": ([_P, _I, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _P], _I),
    "hbl_forward_workspace_size": ([_I64, _I64, _I64, _I], _SZ),
    "hbl_forward": ([_P, _I, _I64, _I64, _I64, _I64, _I, _I, _P, _P, _P, _I64, _P, _SZ, _P], _I),
    "hbl_forward_noalloc": ([_P, _I, _I64, _I64, _I64, _I64, _I, _I, _P, _P, _P, _I64, _P], _I),
    "hbl_hadamard_backward_f32": ([_P, _I, _I64, _I64, _I64, _P, _P], _I),
    "hbl_norm_hadamard_quant": ([_P, _I, _I64, _I64, _I64, _P, _I, _I, _P, _P, _P, _P], _I),
    "hbl_norm_forward": ([_P, _I, _I64, _I64, _I64, _P, _I64, _I, _I, _P, _P, _P, _I64, _P, _SZ, _P], _I),
    "hbl_ternarize_rotated_workspace_size": ([_I64, _I64], _SZ),
    "hbl_ternarize_weights_rotated": ([_P, _I, _I64, _I64, _P, _P, _P, _SZ, _P], _I),
    "hbl_prepare_weights_mx": ([_P, _I64, _I64, _P, _P], _I),
    "hbl_hadamard_quant_mx": ([_P, _I, _I64, _I64, _I64, _I, _P, _P, _P], _I),
    "hbl_ternary_gemm_mx": ([_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _P], _I),
    "hbl_forward_mx_workspace_size": ([_I64, _I64, _I64], _SZ),
    "hbl_forward_mx": ([_P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _I64, _P, _SZ, _P], _I),
    "hbl_kv_quant": ([_P, _I, _I64, _I64, _I64, _I64, _I, _I, _P, _P, _P, _P, _P], _I),
    "hbl_mx_codes_bytes": ([_I64, _I64], _SZ),
    "hbl_mx_weights_bytes": ([_I64, _I64], _SZ),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def lib() -> ctypes.CDLL:
    """The loaded library (raw C entry points)."""
    return _lib


class HblError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = _lib.hbl_last_error().decode()
        text = _lib.hbl_status_string(status).decode()
        super().__init__(f"{what}: {text} ({detail})")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != OK:
        raise HblError(status, what)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libhbl must live in GPU memory")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return DTYPE_BF16
    if x.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"activations/weights must be bfloat16 or float32, got {x.dtype}")


def _rows(x: torch.Tensor) -> tuple[int, int, int]:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along its last dimension")
    return x.shape[0], x.shape[1], x.stride(0)


def version() -> int:
    return int(_lib.hbl_version())


def cu_count() -> int:
    return int(_lib.hbl_device_cu_count())


def ternarize_weights(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Absmean ternarisation (Eq. 1-2).  Returns (packed int32 [N][K/16]
    holding the uint32 words, alpha float32 [1])."""
    w = w.contiguous()
    N, K = w.shape
    packed = torch.empty((N, K // 16), dtype=torch.int32, device=w.device)
    alpha = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = torch.empty(max(1, _lib.hbl_ternarize_workspace_size(N, K)), dtype=torch.uint8, device=w.device)
    _check(_lib.hbl_ternarize_weights(_ptr(w), _x_dtype(w), N, K, _ptr(packed), _ptr(alpha), _ptr(ws),
                                      ws.numel(), _stream()), "hbl_ternarize_weights")
    return packed, alpha


def ternarize_weights_rotated(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Q_w(W H^T), the weight side of the weight-and-activation rotation
    variant (Table 5): rows of W rotated, then ternarised.  Returns (packed,
    alpha) as ternarize_weights."""
    w = w.contiguous()
    N, K = w.shape
    packed = torch.empty((N, K // 16), dtype=torch.int32, device=w.device)
    alpha = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = torch.empty(max(1, _lib.hbl_ternarize_rotated_workspace_size(N, K)), dtype=torch.uint8, device=w.device)
    _check(_lib.hbl_ternarize_weights_rotated(_ptr(w), _x_dtype(w), N, K, _ptr(packed), _ptr(alpha), _ptr(ws),
                                              ws.numel(), _stream()), "hbl_ternarize_weights_rotated")
    return packed, alpha


def hadamard_backward_f32(dy: torch.Tensor) -> torch.Tensor:
    """dL/dx = H^T dL/d(Hx) per row (Eq. 10), fp32 [M][K]."""
    M, K, ld = _rows(dy)
    dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    _check(_lib.hbl_hadamard_backward_f32(_ptr(dy), _x_dtype(dy), M, K, ld, _ptr(dx), _stream()),
           "hbl_hadamard_backward_f32")
    return dx


def _gain(gain: torch.Tensor | None, K: int) -> int | None:
    if gain is None:
        return None
    if gain.dtype != torch.float32 or gain.shape != (K,) or not gain.is_contiguous():
        raise ValueError("gain must be a contiguous float32 tensor of shape (K,)")
    return _ptr(gain)


def hadamard_f32(x: torch.Tensor) -> torch.Tensor:
    """Row-wise normalised Hadamard rotation (Eq. 3-6), fp32 [M][K]."""
    M, K, ldx = _rows(x)
    y = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _check(_lib.hbl_hadamard_f32(_ptr(x), _x_dtype(x), M, K, ldx, _ptr(y), _stream()), "hbl_hadamard_f32")
    return y


def codes_shape(M: int, K: int, bits: int) -> tuple[tuple[int, int], torch.dtype]:
    return ((M, K), torch.int8) if bits == 8 else ((M, K // 8), torch.int32)


def hadamard_quant(x: torch.Tensor, bits: int, hadamard: bool = True):
    """Per-token quantisation (Eq. 7 or 8), after the rotation when
    ``hadamard``.  Returns (codes, scales float32 [M], rowsum int32 [M]);
    codes are int8 [M][K] (bits 8) or int32 [M][K/8] holding the packed
    uint32 INT4 words (bits 4)."""
    M, K, ldx = _rows(x)
    shape, dt = codes_shape(M, K, bits)
    codes = torch.empty(shape, dtype=dt, device=x.device)
    scales = torch.empty(M, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(M, dtype=torch.int32, device=x.device)
    _check(_lib.hbl_hadamard_quant(_ptr(x), _x_dtype(x), M, K, ldx, HADAMARD if hadamard else 0, bits,
                                   _ptr(codes), _ptr(scales), _ptr(rowsum), _stream()),
           "hbl_hadamard_quant")
    return codes, scales, rowsum


def norm_hadamard_quant(x: torch.Tensor, bits: int, gain: torch.Tensor | None = None, hadamard: bool = True):
    """hadamard_quant after the RMSNorm layer of Eq. 9 (per-channel gain,
    None for one).  Same returns as hadamard_quant."""
    M, K, ldx = _rows(x)
    shape, dt = codes_shape(M, K, bits)
    codes = torch.empty(shape, dtype=dt, device=x.device)
    scales = torch.empty(M, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(M, dtype=torch.int32, device=x.device)
    _check(_lib.hbl_norm_hadamard_quant(_ptr(x), _x_dtype(x), M, K, ldx, _gain(gain, K),
                                        HADAMARD if hadamard else 0, bits, _ptr(codes), _ptr(scales),
                                        _ptr(rowsum), _stream()), "hbl_norm_hadamard_quant")
    return codes, scales, rowsum


_OUT_DT = {OUT_BF16: torch.bfloat16, OUT_F32: torch.float32, OUT_I32: torch.int32}


def ternary_gemm(codes: torch.Tensor, bits: int, scales: torch.Tensor, rowsum: torch.Tensor,
                 packed: torch.Tensor, alpha: torch.Tensor, K: int, out_dtype: int = OUT_BF16,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Integer matmul of the codes with the packed ternary weights and the
    rescale of Eq. 9 (``out_dtype`` OUT_I32 returns the raw int32 sums)."""
    M = codes.shape[0]
    N = packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=codes.device)
    _check(_lib.hbl_ternary_gemm(_ptr(codes), bits, _ptr(scales), _ptr(rowsum), _ptr(packed), _ptr(alpha),
                                 M, N, K, out_dtype, _ptr(out), out.stride(0), _stream()),
           "hbl_ternary_gemm")
    return out


def forward_workspace(M: int, N: int, K: int, bits: int, device) -> torch.Tensor:
    return torch.empty(max(1, _lib.hbl_forward_workspace_size(M, N, K, bits)), dtype=torch.uint8, device=device)


def forward(x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor, bits: int, hadamard: bool = True,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The whole H-BitLinear (or, with ``hadamard=False``, BitLinear)
    forward of Eq. 9: bf16 [M][N]."""
    M, K, ldx = _rows(x)
    N = packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = forward_workspace(M, N, K, bits, x.device)
    _check(_lib.hbl_forward(_ptr(x), _x_dtype(x), M, K, ldx, N, HADAMARD if hadamard else 0, bits,
                            _ptr(packed), _ptr(alpha), _ptr(out), out.stride(0), _ptr(workspace),
                            workspace.numel(), _stream()), "hbl_forward")
    return out


NOALLOC_WORKSPACE_BYTES = 64 * 1024 * 1024


def forward_noalloc(x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor, bits: int, hadamard: bool = True,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """forward() with the library's static workspace (hbl_forward_noalloc):
    the library allocates nothing; calls that overlap on one GPU race."""
    M, K, ldx = _rows(x)
    N = packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(_lib.hbl_forward_noalloc(_ptr(x), _x_dtype(x), M, K, ldx, N, HADAMARD if hadamard else 0, bits,
                                    _ptr(packed), _ptr(alpha), _ptr(out), out.stride(0), _stream()),
           "hbl_forward_noalloc")
    return out


def norm_forward(x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor, bits: int,
                 gain: torch.Tensor | None = None, hadamard: bool = True, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """forward with the RMSNorm layer of Eq. 9 in front: bf16 [M][N]."""
    M, K, ldx = _rows(x)
    N = packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = forward_workspace(M, N, K, bits, x.device)
    _check(_lib.hbl_norm_forward(_ptr(x), _x_dtype(x), M, K, ldx, _gain(gain, K), N,
                                 HADAMARD if hadamard else 0, bits, _ptr(packed), _ptr(alpha), _ptr(out),
                                 out.stride(0), _ptr(workspace), workspace.numel(), _stream()), "hbl_norm_forward")
    return out


# ---------------------------------------------------------------------------
# INT4 on the FP6 x FP4 matrix cores (MX6 codes, MX4 weights; include/hbl.h)

def prepare_weights_mx(packed: torch.Tensor, K: int) -> torch.Tensor:
    """Ternary layout -> MX4 layout: int32 [ceil(N/128)*128][K/16] holding the
    words in the tiled order of include/hbl.h (rows past N zero)."""
    N = packed.shape[0]
    wq = torch.empty(((N + 127) // 128 * 128, K // 16), dtype=torch.int32, device=packed.device)
    _check(_lib.hbl_prepare_weights_mx(_ptr(packed), N, K, _ptr(wq), _stream()), "hbl_prepare_weights_mx")
    return wq


def hadamard_quant_mx(x: torch.Tensor, hadamard: bool = True):
    """INT4 quantisation (Eq. 8) with MX6 codes: (codes uint8
    [ceil(M/256)*256][3K/4] in the tiled order of include/hbl.h, scales
    float32 [M])."""
    M, K, ldx = _rows(x)
    codes = torch.empty(((M + 255) // 256 * 256, K // 4 * 3), dtype=torch.uint8, device=x.device)
    scales = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(_lib.hbl_hadamard_quant_mx(_ptr(x), _x_dtype(x), M, K, ldx, HADAMARD if hadamard else 0, _ptr(codes),
                                      _ptr(scales), _stream()), "hbl_hadamard_quant_mx")
    return codes, scales


def ternary_gemm_mx(codes: torch.Tensor, scales: torch.Tensor, wq: torch.Tensor, alpha: torch.Tensor, K: int,
                    out_dtype: int = OUT_BF16, out: torch.Tensor | None = None, N: int | None = None) -> torch.Tensor:
    """The FP6 x FP4 matmul with the rescale of Eq. 9 (M = len(scales); N
    defaults to the rows of the prepared weights, which are padded to 128:
    pass the matrix's N, or an ``out`` of that width)."""
    M = scales.shape[0]
    N = out.shape[1] if out is not None else (N if N is not None else wq.shape[0])
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_DT[out_dtype], device=codes.device)
    _check(_lib.hbl_ternary_gemm_mx(_ptr(codes), _ptr(scales), _ptr(wq), _ptr(alpha), M, N, K, out_dtype, _ptr(out),
                                    out.stride(0), _stream()), "hbl_ternary_gemm_mx")
    return out


def forward_mx_workspace(M: int, N: int, K: int, device) -> torch.Tensor:
    return torch.empty(max(1, _lib.hbl_forward_mx_workspace_size(M, N, K)), dtype=torch.uint8, device=device)


def forward_mx(x: torch.Tensor, wq: torch.Tensor, alpha: torch.Tensor, hadamard: bool = True,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               N: int | None = None) -> torch.Tensor:
    """The INT4 layer of Eq. 9 on the FP6 x FP4 matrix cores: bf16 [M][N],
    the same values as forward(x, packed, alpha, 4, hadamard).  N defaults to
    the prepared weights' (128-padded) rows: pass the matrix's N, or an
    ``out`` of that width."""
    M, K, ldx = _rows(x)
    N = out.shape[1] if out is not None else (N if N is not None else wq.shape[0])
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = forward_mx_workspace(M, N, K, x.device)
    _check(_lib.hbl_forward_mx(_ptr(x), _x_dtype(x), M, K, ldx, N, HADAMARD if hadamard else 0, _ptr(wq), _ptr(alpha),
                               _ptr(out), out.stride(0), _ptr(workspace), workspace.numel(), _stream()),
           "hbl_forward_mx")
    return out


def kv_quant(x: torch.Tensor, bits: int, keep_bos8: bool = True):
    """Post-RoPE QKV / KV-cache quantiser on x [B][S][H][D] (contiguous).
    Returns (codes uint8 [B][S][H][D*bits/8], scales [B][S][H], bos_codes
    uint8 [B][H][D], bos_scales [B][H]); the BOS tensors are empty without
    keep_bos8."""
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B][S][H][D] tensor")
    B, S, H, D = x.shape
    codes = torch.empty((B, S, H, D * bits // 8), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, S, H), dtype=torch.float32, device=x.device)
    bos = torch.empty((B, H, D) if keep_bos8 else (0,), dtype=torch.uint8, device=x.device)
    bos_s = torch.empty((B, H) if keep_bos8 else (0,), dtype=torch.float32, device=x.device)
    _check(_lib.hbl_kv_quant(_ptr(x), _x_dtype(x), B, S, H, D, bits, int(keep_bos8), _ptr(codes), _ptr(scales),
                             _ptr(bos) if keep_bos8 else None, _ptr(bos_s) if keep_bos8 else None, _stream()),
           "hbl_kv_quant")
    return codes, scales, bos, bos_s
