"""GPU parity of every entry point against the CPU oracle, through the C ABI.

Small cases span several tiles and ragged tails (the five workloads at their
full sizes are in test_gpu_full_size.py).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mx_util
import oracle
import workloads
from parity_util import (bf16_to_f64, check_codes, check_hadamard, check_output, check_scales,
                         codes_to_numpy, to_device)

pytestmark = pytest.mark.gpu

ALL_LOG2K = list(range(4, 15))


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("log2k", ALL_LOG2K)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hadamard_values(hbl, log2k, dtype):
    K = 1 << log2k
    M = 37
    x = workloads.random_rows(100 + log2k, M, K, "t3", as_bf16=(dtype == "bf16"))
    y = hbl.hadamard_f32(to_device(x)).cpu().numpy()
    check_hadamard(y, oracle.hadamard(x), f"K={K} {dtype}")


def test_hadamard_strided_rows(hbl):
    K, M, ld = 1024, 19, 1024 + 64
    big = workloads.random_rows(7, M, ld, "normal", as_bf16=True)
    x_dev = to_device(big)[:, :K]
    y = hbl.hadamard_f32(x_dev).cpu().numpy()
    check_hadamard(y, oracle.hadamard(np.ascontiguousarray(big[:, :K])), "strided")


@pytest.mark.parametrize("K", [1024, 4096, 16384])
@pytest.mark.parametrize("M", [37, 600])
@pytest.mark.parametrize("had", [False, True])
def test_quant_strided_rows(hbl, K, M, had):
    """Row-strided bf16 inputs (row stride K + 24 elements, 16-byte aligned
    rows): INT8 and INT4 codes, scales and row sums, and MX6 codes and scales,
    equal those of the same rows stored contiguously, bit for bit (the row
    loads of every path, the line-wise non-temporal ones included, follow the
    stride)."""
    big = to_device(workloads.random_rows(4400 + K + M, M, K + 24, "t3", as_bf16=True))
    xs, xc = big[:, :K], big[:, :K].contiguous()
    assert xs.stride(0) == K + 24
    for bits in (8, 4):
        for u, v in zip(hbl.hadamard_quant(xs, bits, hadamard=had), hbl.hadamard_quant(xc, bits, hadamard=had)):
            assert torch.equal(u, v), f"K={K} M={M} had={had} bits={bits}"
    # (the MX6 buffer holds whole 256-row blocks; rows past M are not written)
    (cs, ss), (cc, sc) = hbl.hadamard_quant_mx(xs, hadamard=had), hbl.hadamard_quant_mx(xc, hadamard=had)
    assert torch.equal(ss, sc), f"K={K} M={M} had={had} MX6 scales"
    assert np.array_equal(mx_util.decode_mx6(cs.cpu().numpy(), K, M), mx_util.decode_mx6(cc.cpu().numpy(), K, M)), \
        f"K={K} M={M} had={had} MX6 codes"


def test_hadamard_twice_is_identity(hbl):
    K, M = 4096, 8
    x = workloads.random_rows(5, M, K, "normal", as_bf16=False)
    y = hbl.hadamard_f32(to_device(x))
    z = hbl.hadamard_f32(y).cpu().numpy()
    assert np.abs(z - x).max() <= 1e-5 * np.abs(x).max()


# ------------------------------------------------------------ quantisation

def _quant_case(hbl, x, bits, had, what):
    q, s, rs = hbl.hadamard_quant(to_device(x), bits, hadamard=had)
    torch.cuda.synchronize()
    oq, os_, ors, xr = oracle.quantize(x, bits, hadamard=had, want_xr=True)
    K = x.shape[1]
    gq = oracle.codes_int8(codes_to_numpy(q, bits), bits, K)
    oq8 = oracle.codes_int8(oq, bits, K)
    nbad = check_codes(gq, oq8, xr, bits, what)
    check_scales(s.cpu().numpy(), os_, what)
    grs = rs.cpu().numpy()
    assert np.array_equal(grs, gq.astype(np.int64).sum(axis=1)), f"{what}: rowsum != sum of codes"
    assert np.abs(grs.astype(np.int64) - ors).sum() <= nbad
    return gq, nbad


@pytest.mark.parametrize("log2k", ALL_LOG2K)
@pytest.mark.parametrize("bits", [8, 4])
def test_quant_with_rotation(hbl, log2k, bits):
    K = 1 << log2k
    x = workloads.random_rows(200 + log2k, 37, K, "t3", as_bf16=True)
    _quant_case(hbl, x, bits, True, f"K={K} INT{bits}")


# Rotated bf16 rows take the one-row-per-block kernel up to 256 tokens at
# K = 16384 and 1024 below (INT8, INT4 and MX6 codes alike), the row-group
# kernel beyond: both sides of each boundary against the oracle
@pytest.mark.parametrize("M,K", [(1, 1024), (5, 2048), (65, 4096), (1024, 4096), (1025, 4096), (256, 8192),
                                 (200, 16384), (256, 16384), (257, 16384)])
@pytest.mark.parametrize("bits", [8, 4])
def test_quant_rotation_token_counts(hbl, M, K, bits):
    x = workloads.random_rows(400 + M + K // 1024, M, K, "t3", as_bf16=True)
    _quant_case(hbl, x, bits, True, f"M={M} K={K} INT{bits}")


@pytest.mark.parametrize("K", [64, 192, 960, 1024, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_plain(hbl, K, bits, dtype):
    x = workloads.random_rows(300 + K % 97, 21, K, "t3", as_bf16=(dtype == "bf16"))
    _quant_case(hbl, x, bits, False, f"plain K={K} INT{bits} {dtype}")


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_degenerate_rows(hbl, bits):
    K = 2048
    rows = [np.zeros(K, np.float32),                      # all zero
            np.full(K, 3.0, np.float32),                  # constant: rotates to a spike
            np.eye(1, K, 17, dtype=np.float32)[0] * 50,   # spike: rotates to a flat row
            np.full(K, 1e-30, np.float32),                # far below eps
            (np.arange(K) % 7 - 3).astype(np.float32) * 6e4]
    x = np.stack(rows)
    gq, _ = _quant_case(hbl, x, bits, True, f"degenerate INT{bits}")
    assert np.all(gq[0] == 0) and np.all(gq[3] == 0)


# -------------------------------------------------------------- ternarise

@pytest.mark.parametrize("N,K", [(256, 256), (64, 4096), (48, 272), (4096, 4096)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ternarize(hbl, N, K, dtype):
    w = workloads.gaussian_weights(9, N + K, N, K)
    if dtype == "bf16":
        w = workloads.bf16_bits(w)
    packed, alpha = hbl.ternarize_weights(to_device(w))
    o_packed, o_alpha, _ = oracle.ternarize(w)
    assert float(alpha.cpu()[0]) == float(o_alpha)
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), o_packed)


# ----------------------------------------------------- integer matmul

def _gemm_inputs(M, N, K, bits, seed):
    x = workloads.random_rows(seed, M, K, "t3", as_bf16=True)
    had = (K & (K - 1)) == 0
    codes, scales, rowsum = oracle.quantize(x, bits, hadamard=had)
    w = workloads.gaussian_weights(seed, 7, N, K)
    packed, alpha, _ = oracle.ternarize(w)
    return codes, scales, rowsum, packed, alpha


def _dev_codes(codes, bits):
    return torch.from_numpy(codes).cuda() if bits == 8 else torch.from_numpy(codes.view(np.int32)).cuda()


@pytest.mark.parametrize("M", [1, 2, 3, 4, 16, 17, 33, 100, 129, 256, 300])
@pytest.mark.parametrize("N,K", [(16, 64), (48, 192), (256, 256), (272, 1024), (64, 2048)])
@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_exact_on_oracle_codes(hbl, M, N, K, bits):
    codes, scales, rowsum, packed, alpha = _gemm_inputs(M, N, K, bits, 1000 + M + N + K)
    acc = hbl.ternary_gemm(_dev_codes(codes, bits), bits, torch.from_numpy(scales).cuda(),
                           torch.from_numpy(rowsum).cuda(), torch.from_numpy(packed.view(np.int32)).cuda(),
                           torch.tensor([alpha], dtype=torch.float32).cuda(), K, out_dtype=hbl.OUT_I32)
    ref = oracle.gemm_i32(codes, bits, packed, K)
    assert np.array_equal(acc.cpu().numpy(), ref)


# decode token counts with K past the dot-product kernel's range (a power
# of two up to 16384): K = 3072 and 5120 (multiples of 1024, not powers of
# two) and 32768 take the matrix-core weight streaming
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("N,K", [(32, 3072), (16, 5120), (16, 32768)])
@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_decode_widths_outside_dot_kernel(hbl, M, N, K, bits):
    codes, scales, rowsum, packed, alpha = _gemm_inputs(M, N, K, bits, 2000 + M + N + K)
    acc = hbl.ternary_gemm(_dev_codes(codes, bits), bits, torch.from_numpy(scales).cuda(),
                           torch.from_numpy(rowsum).cuda(), torch.from_numpy(packed.view(np.int32)).cuda(),
                           torch.tensor([alpha], dtype=torch.float32).cuda(), K, out_dtype=hbl.OUT_I32)
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(codes, bits, packed, K))


# every decode dispatch branch at the 7B widths: the dot-product kernel (M <=
# 2), its interleaved INT8 code loads (K <= 8192) and the matrix-core weight
# streaming (M = 3-4)
@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("K", [4096, 8192, 16384])
@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_decode_dispatch_exact(hbl, M, K, bits):
    N = 4096
    codes, scales, rowsum, packed, alpha = _gemm_inputs(M, N, K, bits, 3000 + M + K // 1024 + bits)
    acc = hbl.ternary_gemm(_dev_codes(codes, bits), bits, torch.from_numpy(scales).cuda(),
                           torch.from_numpy(rowsum).cuda(), torch.from_numpy(packed.view(np.int32)).cuda(),
                           torch.tensor([alpha], dtype=torch.float32).cuda(), K, out_dtype=hbl.OUT_I32)
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_exact(codes, bits, packed, K))


@pytest.mark.parametrize("M", [5, 130])
@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_rescaled_outputs(hbl, M, bits):
    N, K = 96, 512
    codes, scales, rowsum, packed, alpha = _gemm_inputs(M, N, K, bits, 77 + M)
    args = (_dev_codes(codes, bits), bits, torch.from_numpy(scales).cuda(), torch.from_numpy(rowsum).cuda(),
            torch.from_numpy(packed.view(np.int32)).cuda(), torch.tensor([alpha], dtype=torch.float32).cuda(), K)
    y32 = hbl.ternary_gemm(*args, out_dtype=hbl.OUT_F32).cpu().numpy().astype(np.float64)
    y16 = bf16_to_f64(hbl.ternary_gemm(*args, out_dtype=hbl.OUT_BF16))
    acc = oracle.gemm_i32(codes, bits, packed, K)
    y64, _ = oracle.dequant_output(acc, scales, alpha)
    # fp32: two roundings (scale*alpha, then the product); bf16: one more
    assert np.all(np.abs(y32 - y64) <= 2.5e-7 * np.abs(y64))
    assert np.all(np.abs(y16 - y64) <= (2.0 ** -8) * np.abs(y64))


def test_gemm_strided_output(hbl):
    M, N, K, bits = 40, 64, 256, 8
    codes, scales, rowsum, packed, alpha = _gemm_inputs(M, N, K, bits, 5)
    out = torch.full((M, N + 32), -7, dtype=torch.int32, device="cuda")
    hbl.ternary_gemm(_dev_codes(codes, bits), bits, torch.from_numpy(scales).cuda(),
                     torch.from_numpy(rowsum).cuda(), torch.from_numpy(packed.view(np.int32)).cuda(),
                     torch.tensor([alpha], dtype=torch.float32).cuda(), K, out_dtype=hbl.OUT_I32,
                     out=out[:, :N])
    o = out.cpu().numpy()
    assert np.array_equal(o[:, :N], oracle.gemm_i32(codes, bits, packed, K))
    assert np.all(o[:, N:] == -7), "wrote outside the output view"


@pytest.mark.parametrize("pad", [4, 8])
@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_strided_bf16_output(hbl, pad, bits):
    """bf16 outputs into a row-strided view (stride = N + pad elements), on
    the persistent matmul path, equal the contiguous result; the padding
    columns are untouched."""
    M, N, K = 300, 256, 1024
    codes, scales, rowsum, packed, alpha = _gemm_inputs(M, N, K, bits, 31 + pad)
    args = (_dev_codes(codes, bits), bits, torch.from_numpy(scales).cuda(), torch.from_numpy(rowsum).cuda(),
            torch.from_numpy(packed.view(np.int32)).cuda(), torch.tensor([alpha], dtype=torch.float32).cuda(), K)
    ref = hbl.ternary_gemm(*args, out_dtype=hbl.OUT_BF16)
    buf = torch.full((M, N + pad), -7.0, dtype=torch.bfloat16, device="cuda")
    hbl.ternary_gemm(*args, out_dtype=hbl.OUT_BF16, out=buf[:, :N])
    assert torch.equal(buf[:, :N].view(torch.int16), ref.view(torch.int16))
    assert torch.all(buf[:, N:] == -7.0), "wrote outside the output view"


# ---------------------------------------------------------- whole layer

def test_forward_tiny_workload(hbl):
    c = workloads.tiny()
    packed, alpha = hbl.ternarize_weights(to_device(c["w"]))
    y = hbl.forward(to_device(c["x"]), packed, alpha, c["bits"], hadamard=True)
    o_packed, o_alpha, _ = oracle.ternarize(c["w"])
    y64 = oracle.forward(c["x"], o_packed, o_alpha, c["bits"], hadamard=True)
    check_output(bf16_to_f64(y), y64, "tiny")


def test_forward_equals_the_two_steps(hbl):
    M, K, N, bits = 70, 1024, 128, 4
    x = to_device(workloads.random_rows(3, M, K, "t3"))
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(3, 3, N, K)))
    y = hbl.forward(x, packed, alpha, bits)
    q, s, rs = hbl.hadamard_quant(x, bits)
    y2 = hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K)
    assert torch.equal(y, y2)


def test_forward_deterministic(hbl):
    M, K, N, bits = 300, 4096, 512, 8
    x = to_device(workloads.random_rows(4, M, K, "t3"))
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(4, 4, N, K)))
    a = hbl.forward(x, packed, alpha, bits)
    b = hbl.forward(x, packed, alpha, bits)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_zero_tokens(hbl):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(1, 1, 32, 256)))
    assert hbl.forward(x, packed, alpha, 4).shape == (0, 32)
