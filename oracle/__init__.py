"""Plain CPU oracle for the H-BitLinear forward of BitNet v2.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports
this package, and this package never imports the product library.

The arithmetic lives in ``hbl_oracle.c`` (plain C, fp64 Hadamard transform,
fp32 quantiser decisions, exact integer matmul); this module only marshals
numpy arrays through ctypes.  Every formula is cited in the C file against the
architecture write-up of "BitNet v2: Native 4-bit Activations with Hadamard
Transformation for 1-bit LLMs", §3.4 (Eq. 1-2 weights, Eq. 3-6 Hadamard,
Eq. 7-8 activations, Eq. 9 the layer).

Parity pins: every function here is pinned by tests in
``tests/test_oracle_pins.py`` against closed forms, library routines,
brute-force enumeration and hand-worked cases (see that file's header).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hbl_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
EPS = np.float32(1e-5)


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fused multiply-adds, OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared",
            "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        _lib.hbo_fwht_f64.argtypes = [P, I64]
        _lib.hbo_fwht_f64.restype = I64
        _lib.hbo_hadamard.argtypes = [P, I, I64, I64, I64, P]
        _lib.hbo_quantize.argtypes = [P, I, I64, I64, I64, I, I, P, P, P, P]
        _lib.hbo_norm_quantize.argtypes = [P, I, I64, I64, I64, P, I, I, P, P, P, P]
        _lib.hbo_hadamard_backward.argtypes = [P, I, I64, I64, I64, P]
        _lib.hbo_ternarize_rotated.argtypes = [P, I, I64, I64, P, P, P, P]
        _lib.hbo_kv_quant.argtypes = [P, I, I64, I64, I64, I64, I, I, P, P, P, P]
        _lib.hbo_kv_dequant.argtypes = [P, P, I64, I64, I, P]
        _lib.hbo_ternarize.argtypes = [P, I, I64, I64, P, P, P]
        _lib.hbo_gemm_i32.argtypes = [P, I, P, I64, I64, I64, P]
        _lib.hbo_dequant_output.argtypes = [P, P, ctypes.c_float, I64, I64, P, P]
        _lib.hbo_forward.argtypes = [P, I, I64, I64, I64, I, I, P, ctypes.c_float, I64, P]
        _lib.hbo_pack_int4.argtypes = [P, I64, I64, P]
        _lib.hbo_unpack_int4.argtypes = [P, I64, I64, P]
        _lib.hbo_pack_ternary.argtypes = [P, I64, I64, P]
        _lib.hbo_unpack_ternary.argtypes = [P, I64, I64, P]
        _lib.hbo_unpack_ternary.restype = I64
        _lib.hbo_f32_to_bf16.argtypes = [ctypes.c_float]
        _lib.hbo_f32_to_bf16.restype = ctypes.c_uint16
        _lib.hbo_num_threads.restype = I
        _lib.hbo_set_num_threads.argtypes = [I]
        _lib.hbo_set_num_threads.restype = None
    return _lib


def _p(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError(f"oracle input must be float32 or bf16 bits (uint16), got {x.dtype}")


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def num_threads() -> int:
    return int(lib().hbo_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later parallel loops (OpenMP)."""
    lib().hbo_set_num_threads(int(n))


def fwht_unnormalized(v: np.ndarray) -> tuple[np.ndarray, int]:
    """Unnormalised Walsh-Hadamard transform of one fp64 vector; returns
    (H~ v, number of add/sub operations)."""
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    ops = lib().hbo_fwht_f64(_p(out), out.size)
    return out, int(ops)


def hadamard(x: np.ndarray) -> np.ndarray:
    """Row-wise normalised Hadamard transform, fp64 result [M][K]."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    y = np.empty((M, K), np.float64)
    _check(lib().hbo_hadamard(_p(x), _dtype_code(x), M, K, K, _p(y)), "hadamard")
    return y


def quantize(x: np.ndarray, bits: int, hadamard: bool = True, want_xr: bool = False):
    """Per-token quantisation (optionally after the Hadamard rotation).

    Returns (codes, scales, rowsum[, xr]); codes are int8 [M][K] for bits=8 and
    packed uint32 [M][K/8] for bits=4.
    """
    x = np.ascontiguousarray(x)
    M, K = x.shape
    if bits == 8:
        codes = np.empty((M, K), np.int8)
    else:
        codes = np.empty((M, K // 8), np.uint32)
    scales = np.empty(M, np.float32)
    rowsum = np.empty(M, np.int32)
    xr = np.empty((M, K), np.float32) if want_xr else None
    _check(lib().hbo_quantize(_p(x), _dtype_code(x), M, K, K, int(hadamard), bits,
                              _p(codes), _p(scales), _p(rowsum),
                              _p(xr) if want_xr else None), "quantize")
    return (codes, scales, rowsum, xr) if want_xr else (codes, scales, rowsum)


def norm_quantize(x: np.ndarray, bits: int, gain: np.ndarray | None = None,
                  hadamard: bool = True, want_xr: bool = False):
    """RMSNorm (per-channel gain, None = ones), then the optional rotation, then
    per-token quantisation: Eq. 9 with its normalisation layer.  Same returns
    as quantize()."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float32)
    if g is not None and g.shape != (K,):
        raise ValueError("gain must have shape (K,)")
    codes = np.empty((M, K), np.int8) if bits == 8 else np.empty((M, K // 8), np.uint32)
    scales = np.empty(M, np.float32)
    rowsum = np.empty(M, np.int32)
    xr = np.empty((M, K), np.float32) if want_xr else None
    _check(lib().hbo_norm_quantize(_p(x), _dtype_code(x), M, K, K, _p(g) if g is not None else None,
                                   int(hadamard), bits, _p(codes), _p(scales), _p(rowsum),
                                   _p(xr) if want_xr else None), "norm_quantize")
    return (codes, scales, rowsum, xr) if want_xr else (codes, scales, rowsum)


def hadamard_backward(dy: np.ndarray) -> np.ndarray:
    """dX = H^T dY per row by the explicit transposed product (O(K^2) per
    row), fp64 [M][K]."""
    dy = np.ascontiguousarray(dy)
    M, K = dy.shape
    dx = np.empty((M, K), np.float64)
    _check(lib().hbo_hadamard_backward(_p(dy), _dtype_code(dy), M, K, K, _p(dx)), "hadamard_backward")
    return dx


def ternarize_rotated(w: np.ndarray, want_wr: bool = False):
    """Q_w(W H^T): rows of W rotated, then ternarised.  Returns (packed, alpha,
    codes[, the rotated fp32 matrix])."""
    w = np.ascontiguousarray(w)
    N, K = w.shape
    packed = np.empty((N, K // 16), np.uint32)
    alpha = np.zeros(1, np.float32)
    q = np.empty((N, K), np.int8)
    wr = np.empty((N, K), np.float32) if want_wr else None
    _check(lib().hbo_ternarize_rotated(_p(w), _dtype_code(w), N, K, _p(packed), _p(alpha), _p(q),
                                       _p(wr) if want_wr else None), "ternarize_rotated")
    out = (packed, np.float32(alpha[0]), q)
    return out + (wr,) if want_wr else out


def ternarize(w: np.ndarray):
    """Per-tensor absmean ternarisation.  Returns (packed uint32 [N][K/16],
    alpha float32, codes int8 [N][K])."""
    w = np.ascontiguousarray(w)
    N, K = w.shape
    packed = np.empty((N, K // 16), np.uint32)
    alpha = np.zeros(1, np.float32)
    q = np.empty((N, K), np.int8)
    _check(lib().hbo_ternarize(_p(w), _dtype_code(w), N, K, _p(packed), _p(alpha), _p(q)),
           "ternarize")
    return packed, np.float32(alpha[0]), q


def gemm_i32(codes: np.ndarray, bits: int, packed: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    packed = np.ascontiguousarray(packed)
    M = codes.shape[0]
    N = packed.shape[0]
    acc = np.empty((M, N), np.int32)
    _check(lib().hbo_gemm_i32(_p(codes), bits, _p(packed), M, N, K, _p(acc)), "gemm")
    return acc


def gemm_exact(codes: np.ndarray, bits: int, packed: np.ndarray, K: int) -> np.ndarray:
    """acc[m][n] = sum_k q_x[m][k] q_w[n][k], the same integers as
    gemm_i32, with a library matmul as the step (numpy/BLAS in fp64) for
    the large parity cases the triple loop cannot finish in seconds.

    The codes and weights are unpacked by the oracle's own unpackers; every
    product and every partial sum is an integer of magnitude at most
    128 K <= 2^21 < 2^53, so the fp64 matmul is exact whatever its blocking
    and summation order.  Pinned against gemm_i32 and numpy's int64 matmul
    in tests/test_oracle_pins.py."""
    if K > (1 << 23):
        raise ValueError("gemm_exact: K too large for the exactness argument")
    q = codes_int8(np.ascontiguousarray(codes), bits, K).astype(np.float64)
    t, bad = unpack_ternary(packed, K)
    if bad:
        raise ValueError(f"gemm_exact: {bad} invalid 2-bit weight fields")
    acc = q @ t.astype(np.float64).T
    return acc.astype(np.int32)


def dequant_output(acc: np.ndarray, scales: np.ndarray, alpha) -> tuple[np.ndarray, np.ndarray]:
    """(y64 fp64, y as bf16 bits) from the int32 accumulator."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    M, N = acc.shape
    y64 = np.empty((M, N), np.float64)
    yb = np.empty((M, N), np.uint16)
    lib().hbo_dequant_output(_p(acc), _p(scales), float(alpha), M, N, _p(y64), _p(yb))
    return y64, yb


def forward(x: np.ndarray, packed: np.ndarray, alpha, bits: int, hadamard: bool = True):
    """Whole layer; returns y64 [M][N] (fp64)."""
    x = np.ascontiguousarray(x)
    packed = np.ascontiguousarray(packed)
    M, K = x.shape
    N = packed.shape[0]
    y = np.empty((M, N), np.float64)
    _check(lib().hbo_forward(_p(x), _dtype_code(x), M, K, K, int(hadamard), bits,
                             _p(packed), float(alpha), N, _p(y)), "forward")
    return y


def pack_int4(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = q.shape
    out = np.empty((M, K // 8), np.uint32)
    lib().hbo_pack_int4(_p(q), M, K, _p(out))
    return out


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    M = packed.shape[0]
    out = np.empty((M, K), np.int8)
    lib().hbo_unpack_int4(_p(packed), M, K, _p(out))
    return out


def pack_ternary(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    N, K = q.shape
    out = np.empty((N, K // 16), np.uint32)
    lib().hbo_pack_ternary(_p(q), N, K, _p(out))
    return out


def unpack_ternary(packed: np.ndarray, K: int) -> tuple[np.ndarray, int]:
    """Returns (codes int8 [N][K], number of invalid 2-bit fields)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    N = packed.shape[0]
    out = np.empty((N, K), np.int8)
    bad = lib().hbo_unpack_ternary(_p(packed), N, K, _p(out))
    return out, int(bad)


def codes_int8(codes: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Codes as int8 [M][K] whatever their storage."""
    return codes if bits == 8 else unpack_int4(codes, K)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits, element by element (slow)."""
    f = lib().hbo_f32_to_bf16
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    return np.array([f(float(v)) for v in flat], np.uint16).reshape(np.shape(a))


def kv_quant(x: np.ndarray, bits: int, keep_bos8: bool = True):
    """Post-RoPE QKV / KV-cache quantiser on x [B][S][H][D] (fp32 or bf16
    bits).  Returns (codes uint8 [B][S][H][D*bits/8], scales [B][S][H],
    bos_codes uint8 [B][H][D], bos_scales [B][H]); the BOS arrays are zero
    without keep_bos8."""
    x = np.ascontiguousarray(x)
    B, S, H, D = x.shape
    codes = np.zeros((B, S, H, D * bits // 8), np.uint8)
    scales = np.zeros((B, S, H), np.float32)
    bos = np.zeros((B, H, D), np.uint8)
    bos_s = np.zeros((B, H), np.float32)
    _check(lib().hbo_kv_quant(_p(x), _dtype_code(x), B, S, H, D, bits, int(keep_bos8), _p(codes), _p(scales),
                              _p(bos), _p(bos_s)), "kv_quant")
    return codes, scales, bos, bos_s


def kv_dequant(codes: np.ndarray, scales: np.ndarray, D: int, bits: int) -> np.ndarray:
    """(u - 2^(b-1)) * scale per group; codes [..][D*bits/8], scales [..]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, D * bits // 8)
    sc = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1)
    out = np.empty((c.shape[0], D), np.float64)
    _check(lib().hbo_kv_dequant(_p(c), _p(sc), c.shape[0], D, bits, _p(out)), "kv_dequant")
    return out.reshape(tuple(scales.shape) + (D,))
