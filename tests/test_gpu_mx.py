"""GPU parity of the INT4 path on the FP6 x FP4 matrix cores, through the C
ABI: MX4 weight preparation, MX6 codes, the matmul (bit-exact int32 on the
oracle's codes), and the whole layer against both the oracle and the int8
matrix-core path (whose bf16 outputs it must reproduce bit for bit, since
both compute the same exact integer sums and the same rescale)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mx_util
import oracle
import workloads
from parity_util import bf16_to_f64, check_codes, check_output, check_scales, to_device

pytestmark = pytest.mark.gpu


def _weights(hbl, N, K, seed):
    w = workloads.gaussian_weights(seed, N + K, N, K)
    packed, alpha = hbl.ternarize_weights(to_device(w))
    return w, packed, alpha, hbl.prepare_weights_mx(packed, K)


@pytest.mark.parametrize("N,K", [(16, 512), (272, 1024), (4096, 4096)])
def test_prepare_weights_mx(hbl, N, K):
    w, packed, alpha, wq = _weights(hbl, N, K, 1)
    _, _, q = oracle.ternarize(w)
    assert np.array_equal(wq.cpu().numpy().view(np.uint32), mx_util.encode_mx4(q))


@pytest.mark.parametrize("log2k", [10, 11, 12, 13, 14])
@pytest.mark.parametrize("had", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_mx_codes(hbl, log2k, had, dtype):
    K = 1 << log2k
    x = workloads.random_rows(800 + log2k, 37, K, "t3", as_bf16=(dtype == "bf16"))
    xd = to_device(x)
    cm, sm = hbl.hadamard_quant_mx(xd, hadamard=had)
    q4, s4, _ = hbl.hadamard_quant(xd, 4, hadamard=had)
    torch.cuda.synchronize()
    got = mx_util.decode_mx6(cm.cpu().numpy(), K, 37)
    # the same codes and scales as the INT4 layout, bit for bit
    assert np.array_equal(got, oracle.unpack_int4(q4.cpu().numpy().view(np.uint32), K).astype(np.float64))
    assert np.array_equal(sm.cpu().numpy(), s4.cpu().numpy())
    # and the oracle's, to the code rule
    oq, os_, _, xr = oracle.quantize(x, 4, hadamard=had, want_xr=True)
    check_codes(got.astype(np.int8), oracle.unpack_int4(oq, K), xr, 4, f"mx K={K} had={had} {dtype}")
    check_scales(sm.cpu().numpy(), os_, "mx scales")


@pytest.mark.parametrize("M,K", [(1, 1024), (3, 4096), (1024, 4096), (1025, 4096), (255, 16384), (256, 16384),
                                 (257, 16384)])
def test_quant_mx_codes_token_counts(hbl, M, K):
    """Rotated bf16 rows take the one-row-per-block kernel up to 256 tokens
    at K = 16384 and 1024 below, for the MX6 and the INT4 layouts alike:
    on both sides of each boundary the two layouts hold the same codes and
    scales bit for bit, and match the oracle to the code rule."""
    x = workloads.random_rows(900 + M + K // 1024, M, K, "t3", as_bf16=True)
    xd = to_device(x)
    cm, sm = hbl.hadamard_quant_mx(xd, hadamard=True)
    q4, s4, _ = hbl.hadamard_quant(xd, 4, hadamard=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(min(M, 40)), np.arange(max(0, M - 40), M)]))
    got = mx_util.decode_mx6(cm.cpu().numpy(), K, rows)
    q4n = q4.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.unpack_int4(q4n[rows], K).astype(np.float64))
    assert np.array_equal(sm.cpu().numpy(), s4.cpu().numpy())
    oq, os_, _, xr = oracle.quantize(np.ascontiguousarray(x[rows]), 4, hadamard=True, want_xr=True)
    check_codes(got.astype(np.int8), oracle.unpack_int4(oq, K), xr, 4, f"mx M={M} K={K}")
    check_scales(sm.cpu().numpy()[rows], os_, f"mx M={M} K={K} scales")


def test_quant_mx_codes_xcd_row_ranges(hbl):
    """K = 16384 rotated rows, at least 32 per block of the persistent grid,
    so that each XCD walks a contiguous range of rows: the MX6 codes equal
    the INT4 layout's (whose kernel walks the rows in the plain order) bit
    for bit on rows at the start, the middle, the ragged end and around
    each XCD's range boundary, every scale equals, and a few rows match the
    oracle to the code rule."""
    K, M = 16384, 16421
    x = workloads.random_rows(1603, M, K, "t3", as_bf16=True)
    xd = to_device(x)
    cm, sm = hbl.hadamard_quant_mx(xd, hadamard=True)
    q4, s4, _ = hbl.hadamard_quant(xd, 4, hadamard=True)
    torch.cuda.synchronize()
    assert np.array_equal(sm.cpu().numpy(), s4.cpu().numpy())
    bounds = (np.arange(1, 8) * ((M + 7) // 8))[:, None] + np.arange(-3, 3)
    rows = np.unique(np.concatenate([np.arange(0, 260), np.arange(8000, 8260), np.arange(M - 260, M),
                                     bounds.reshape(-1)]))
    got = mx_util.decode_mx6(cm.cpu().numpy(), K, rows)
    q4n = q4.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.unpack_int4(q4n[rows], K).astype(np.float64))
    few = np.array([0, 2052, 8191, M - 1])
    oq, os_, _, xr = oracle.quantize(x[few], 4, hadamard=True, want_xr=True)
    check_codes(oracle.unpack_int4(q4n[few], K), oracle.unpack_int4(oq, K), xr, 4, "mx K=16384 xcd ranges")
    check_scales(sm.cpu().numpy()[few], os_, "mx K=16384 xcd ranges scales")


# (unsplit: 128 x 256 tiles, whose rows are one half of a 256-row MX6 block;
# M = 129 and 383 end in the second half of a block and the first half of the
# next one, N = 16 and 272 leave part of a 256-column tile empty)
@pytest.mark.parametrize("M", [1, 5, 100, 129, 256, 300, 383])
@pytest.mark.parametrize("N,K", [(16, 512), (48, 1024), (272, 2048)])
def test_gemm_mx_exact_on_oracle_codes(hbl, M, N, K):
    x = workloads.random_rows(M + N + K, M, K, "t3", as_bf16=True)
    oq, os_, _ = oracle.quantize(x, 4, hadamard=False)
    q8 = oracle.unpack_int4(oq, K)
    w, packed, alpha, wq = _weights(hbl, N, K, 2)
    codes = torch.from_numpy(mx_util.encode_mx6(q8)).cuda()
    acc = hbl.ternary_gemm_mx(codes, torch.from_numpy(os_).cuda(), wq, alpha, K, out_dtype=hbl.OUT_I32, N=N)
    o_packed, _, _ = oracle.ternarize(w)
    assert np.array_equal(acc.cpu().numpy(), oracle.gemm_i32(oq, 4, o_packed, K))


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_gemm_mx_equals_int8_path(hbl, out_dtype):
    M, N, K = 300, 528, 4096
    x = to_device(workloads.random_rows(41, M, K, "t3"))
    _, packed, alpha, wq = _weights(hbl, N, K, 3)
    od = hbl.OUT_BF16 if out_dtype == "bf16" else hbl.OUT_F32
    cm, sm = hbl.hadamard_quant_mx(x)
    q4, s4, r4 = hbl.hadamard_quant(x, 4)
    a = hbl.ternary_gemm_mx(cm, sm, wq, alpha, K, out_dtype=od, N=N)
    b = hbl.ternary_gemm(q4, 4, s4, r4, packed, alpha, K, out_dtype=od)
    assert torch.equal(a.view(torch.int16) if od == hbl.OUT_BF16 else a.view(torch.int32),
                       b.view(torch.int16) if od == hbl.OUT_BF16 else b.view(torch.int32))


def test_gemm_mx_strided_output(hbl):
    M, N, K, pad = 261, 256, 1024, 8
    x = to_device(workloads.random_rows(43, M, K, "t3"))
    _, packed, alpha, wq = _weights(hbl, N, K, 4)
    cm, sm = hbl.hadamard_quant_mx(x)
    big = torch.full((M, N + pad), 7, dtype=torch.bfloat16, device="cuda")
    hbl.ternary_gemm_mx(cm, sm, wq, alpha, K, out=big[:, :N])
    ref = hbl.ternary_gemm_mx(cm, sm, wq, alpha, K, N=N)
    assert torch.equal(big[:, :N].contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.all(big[:, N:] == 7)


def test_forward_mx_small(hbl):
    M, N, K = 70, 128, 1024
    x_np = workloads.random_rows(45, M, K, "t3")
    w, packed, alpha, wq = _weights(hbl, N, K, 5)
    y = hbl.forward_mx(to_device(x_np), wq, alpha, N=N)
    y_int = hbl.forward(to_device(x_np), packed, alpha, 4)
    assert torch.equal(y.view(torch.int16), y_int.view(torch.int16))
    o_packed, o_alpha, _ = oracle.ternarize(w)
    check_output(bf16_to_f64(y), oracle.forward(x_np, o_packed, o_alpha, 4, hadamard=True), "forward_mx small")


def test_forward_mx_zero_tokens(hbl):
    _, packed, alpha, wq = _weights(hbl, 32, 1024, 6)
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    assert hbl.forward_mx(x, wq, alpha, N=32).shape == (0, 32)


def test_gemm_mx_full_tile_grid_exact(hbl):
    # 256 x 256 tiles (the grid fills the chip): int32 sums on sampled rows
    M, N, K = 4096, 4096, 4096
    x_np = workloads.random_rows(47, M, K, "t3")
    w, packed, alpha, wq = _weights(hbl, N, K, 7)
    cm, sm = hbl.hadamard_quant_mx(to_device(x_np))
    acc = hbl.ternary_gemm_mx(cm, sm, wq, alpha, K, out_dtype=hbl.OUT_I32, N=N)
    rows = np.array([0, 1, 255, 256, 2047, 4095])
    oq, _, _ = oracle.quantize(np.ascontiguousarray(x_np[rows]), 4, hadamard=True)
    gq = mx_util.decode_mx6(cm.cpu().numpy(), K, rows).astype(np.int8)
    o_packed, _, _ = oracle.ternarize(w)
    # on the GPU's own codes (identical to the oracle's up to ties)
    assert np.array_equal(acc.cpu().numpy()[rows], oracle.gemm_i32(oracle.pack_int4(gq), 4, o_packed, K))
    assert np.abs(gq.astype(int) - oracle.unpack_int4(oq, K).astype(int)).max() <= 1


# bf16 output of the 256 x 256 tiles (at least one tile per CU): 33 x 9 =
# 297 tiles, so some blocks run two (the second tile's first stages start
# while the first tile's stores drain); ragged M and N; contiguous rows,
# 16-byte aligned strided rows (pad 8) and 8-byte aligned ones (pad 4).
# Every element against the int8 path, which has its own oracle parity.
@pytest.mark.parametrize("pad", [0, 8, 4])
def test_gemm_mx_bf16_wide_tiles(hbl, pad):
    M, N, K = 33 * 256 - 179, 8 * 256 + 16, 1024
    assert ((M + 255) // 256) * ((N + 255) // 256) >= torch.cuda.get_device_properties(0).multi_processor_count
    x = to_device(workloads.random_rows(51, M, K, "t3"))
    _, packed, alpha, wq = _weights(hbl, N, K, 10)
    cm, sm = hbl.hadamard_quant_mx(x)
    q4, s4, r4 = hbl.hadamard_quant(x, 4)
    ref = hbl.ternary_gemm(q4, 4, s4, r4, packed, alpha, K)
    big = torch.full((M, N + pad), 5, dtype=torch.bfloat16, device="cuda")
    hbl.ternary_gemm_mx(cm, sm, wq, alpha, K, out=big[:, :N])
    assert torch.equal(big[:, :N].contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.all(big[:, N:] == 5)


# (M, N, K) -> slices: (1, 4096, 16384) 8, (100, 272, 4096) 4, (256, 4096,
# 16384) 8, (300, 528, 8192) 8, (768, 4096, 4096) 2 (int16 partial sums);
# (200, 4224, 16384) 4 (slices of 4096: fp32 partial sums)
@pytest.mark.parametrize("M,N,K", [(1, 4096, 16384), (100, 272, 4096), (256, 4096, 16384), (300, 528, 8192),
                                   (768, 4096, 4096), (200, 4224, 16384)])
def test_forward_mx_k_split(hbl, M, N, K):
    # fewer than 256 tiles: the layer splits K over the workspace's partial
    # sums; exact integer partials give the unsplit matmul's bits
    lib = hbl.lib()
    assert lib.hbl_forward_mx_workspace_size(M, N, K) > lib.hbl_mx_codes_bytes(M, K) + 4 * M + 512
    x_np = workloads.random_rows(M + 3 * N + K, M, K, "t3")
    w, packed, alpha, wq = _weights(hbl, N, K, 8)
    x = to_device(x_np)
    y = hbl.forward_mx(x, wq, alpha, N=N)
    cm, sm = hbl.hadamard_quant_mx(x)
    y1 = hbl.ternary_gemm_mx(cm, sm, wq, alpha, K, N=N)  # no workspace: unsplit
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
    y_int = hbl.forward(x, packed, alpha, 4)
    assert torch.equal(y.view(torch.int16), y_int.view(torch.int16))
    rows = np.unique(np.array([0, M // 2, M - 1]))
    o_packed, o_alpha, _ = oracle.ternarize(w)
    y64 = oracle.forward(np.ascontiguousarray(x_np[rows]), o_packed, o_alpha, 4, hadamard=True)
    check_output(bf16_to_f64(y[torch.from_numpy(rows).cuda()]), y64, f"k split M={M} N={N} K={K}")


def test_forward_mx_k_split_strided_output(hbl):
    M, N, K, pad = 77, 256, 8192, 24
    x = to_device(workloads.random_rows(49, M, K, "t3"))
    _, packed, alpha, wq = _weights(hbl, N, K, 9)
    big = torch.full((M, N + pad), 3, dtype=torch.bfloat16, device="cuda")
    hbl.forward_mx(x, wq, alpha, out=big[:, :N])
    ref = hbl.forward(x, packed, alpha, 4)
    assert torch.equal(big[:, :N].contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.all(big[:, N:] == 3)
