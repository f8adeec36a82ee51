"""Parity metrics between the HIP path and the CPU oracle (test helpers).

Tolerances (the arithmetic behind them is in the design notes):
  rotated values   per row max|gpu - ref| / max|ref| <= 1e-5 (fp32 transform
                   against the oracle's fp64 one)
  codes            identical, except at most ceil(1e-4 * n) elements per
                   tensor that differ by exactly 1 and sit at a rounding tie
                   of the oracle's value (|frac(|x_r * factor|) - 1/2| < 1e-3)
  scales           relative difference <= 1e-6 (about 8 ulp: the fp32
                   statistic of rotated values that agree with the oracle's
                   to a few ulp, or an fp32 tree sum against an fp64 sum)
  integer matmul   bit-exact on the oracle's codes
  layer output     per row ||y_gpu - y_ref||_2 <= 1e-2 ||y_ref||_2; rows with
                   y_ref == 0 must be exactly 0
"""
from __future__ import annotations

import math

import numpy as np
import torch

HAD_TOL = 1e-5
CODE_FRAC = 1e-4
SCALE_TOL = 1e-6
OUT_TOL = 1e-2

# worst cases met in this process, written out by the test session when
# HBL_PARITY_REPORT names a file (tests/conftest.py)
WORST = {"hadamard_rel": 0.0, "scale_rel": 0.0, "output_rel_l2": 0.0, "code_tie_mismatches": 0,
         "code_tie_fraction": 0.0}


def to_device(x: np.ndarray) -> torch.Tensor:
    """float32 arrays as float32, uint16 arrays as bf16 bit patterns."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def codes_to_numpy(codes: torch.Tensor, bits: int) -> np.ndarray:
    a = codes.cpu().numpy()
    return a if bits == 8 else a.view(np.uint32)


def quant_factor(xr: np.ndarray, bits: int) -> np.ndarray:
    """Per-row factor Qmax/(stat + eps) of the oracle's values, used only to
    locate rounding ties among mismatching codes."""
    eps = np.float32(1e-5)
    if bits == 8:
        g = np.abs(xr).max(axis=1).astype(np.float32)
        return (np.float32(127.0) / (g + eps)).astype(np.float32)
    beta = (np.abs(xr.astype(np.float64)).sum(axis=1) / xr.shape[1]).astype(np.float32)
    return (np.float32(math.sqrt(7.0)) / (beta + eps)).astype(np.float32)


def check_codes(gpu_q: np.ndarray, ora_q: np.ndarray, xr: np.ndarray, bits: int, what: str) -> int:
    """gpu_q and ora_q are int8 [M][K] codes; xr the oracle's quantised
    values.  Returns the number of (allowed) tie mismatches."""
    d = gpu_q.astype(np.int32) - ora_q.astype(np.int32)
    idx = np.nonzero(d)
    nbad = idx[0].size
    if nbad == 0:
        return 0
    assert np.all(np.abs(d[idx]) == 1), f"{what}: codes differ by more than 1"
    limit = math.ceil(CODE_FRAC * d.size)
    assert nbad <= limit, f"{what}: {nbad} codes differ (limit {limit} of {d.size})"
    f = quant_factor(xr, bits)
    v = np.abs(xr[idx] * f[idx[0]]).astype(np.float64)
    frac = v - np.floor(v)
    assert np.all(np.abs(frac - 0.5) < 1e-3), f"{what}: a mismatch is not at a rounding tie: {frac}"
    WORST["code_tie_mismatches"] += nbad
    WORST["code_tie_fraction"] = max(WORST["code_tie_fraction"], nbad / d.size)
    return nbad


def check_scales(gpu_s: np.ndarray, ora_s: np.ndarray, what: str) -> None:
    den = np.maximum(np.abs(ora_s), np.float32(1e-30))
    rel = np.abs(gpu_s.astype(np.float64) - ora_s) / den
    zero = ora_s == 0
    assert np.all(gpu_s[zero] == 0), f"{what}: zero rows must have zero scale"
    if np.any(~zero):
        WORST["scale_rel"] = max(WORST["scale_rel"], float(rel[~zero].max()))
    assert np.all(rel[~zero] <= SCALE_TOL), f"{what}: scale rel err {rel[~zero].max():.3e}"


def check_hadamard(gpu_y: np.ndarray, ref: np.ndarray, what: str) -> float:
    den = np.abs(ref).max(axis=1)
    err = np.abs(gpu_y.astype(np.float64) - ref).max(axis=1)
    zero = den == 0
    assert np.all(err[zero] == 0), f"{what}: zero rows must map to zero"
    rel = err[~zero] / den[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    WORST["hadamard_rel"] = max(WORST["hadamard_rel"], worst)
    assert worst <= HAD_TOL, f"{what}: Hadamard max rel err {worst:.3e}"
    return worst


def check_output(gpu_y: np.ndarray, y64: np.ndarray, what: str) -> float:
    g = gpu_y.astype(np.float64)
    ref = np.linalg.norm(y64, axis=1)
    err = np.linalg.norm(g - y64, axis=1)
    zero = ref == 0
    assert np.all(np.abs(g[zero]) == 0), f"{what}: rows with zero reference must be exactly zero"
    rel = err[~zero] / ref[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    WORST["output_rel_l2"] = max(WORST["output_rel_l2"], worst)
    assert worst <= OUT_TOL, f"{what}: output rel L2 {worst:.3e}"
    return worst


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
