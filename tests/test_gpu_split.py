"""GPU parity of the K split of the int8 matrix-core layer (hbl_forward and
hbl_norm_forward with a workspace that holds the int32 partial sums):
bit-identical to the unsplit matmul (hbl_ternary_gemm, which has no
workspace) and within the output tolerance of the oracle on sampled rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import bf16_to_f64, check_output, to_device

pytestmark = pytest.mark.gpu

# (M, N, K) -> slices of the 128 x 256 tiles: (64, 4096, 16384) 8,
# (100, 272, 16384) 16, (256, 4096, 4096) 4, (200, 4224, 16384) 4 (a ragged
# last tile column), (768, 4096, 4096) 2
SHAPES = [(64, 4096, 16384), (100, 272, 16384), (256, 4096, 4096), (200, 4224, 16384), (768, 4096, 4096)]


def _split_active(hbl, M, N, K, bits):
    lib = hbl.lib()
    codes = M * K if bits == 8 else M * K // 2
    return lib.hbl_forward_workspace_size(M, N, K, bits) > codes + 2 * 4 * M + 1024


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forward_k_split(hbl, M, N, K, bits):
    assert _split_active(hbl, M, N, K, bits)
    x_np = workloads.random_rows(M + N + K + bits, M, K, "t3")
    w = workloads.gaussian_weights(bits, M, N, K)
    packed, alpha = hbl.ternarize_weights(to_device(w))
    x = to_device(x_np)
    y = hbl.forward(x, packed, alpha, bits)
    q, s, rs = hbl.hadamard_quant(x, bits)
    y1 = hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K)
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"split {M}x{N}x{K} bits={bits}"
    rows = np.unique(np.array([0, M // 3, M - 1]))
    o_packed, o_alpha, _ = oracle.ternarize(w)
    y64 = oracle.forward(np.ascontiguousarray(x_np[rows]), o_packed, o_alpha, bits, hadamard=True)
    check_output(bf16_to_f64(y[torch.from_numpy(rows).cuda()]), y64, f"split {M}x{N}x{K} bits={bits}")


@pytest.mark.parametrize("bits", [8, 4])
def test_norm_forward_k_split(hbl, bits):
    M, N, K = 64, 1024, 16384
    assert _split_active(hbl, M, N, K, bits)
    x = to_device(workloads.random_rows(51, M, K, "t3"))
    gain = torch.from_numpy(np.random.default_rng(5).uniform(0.5, 1.5, K).astype(np.float32)).cuda()
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(52, 5, N, K)))
    y = hbl.norm_forward(x, packed, alpha, bits, gain=gain)
    q, s, rs = hbl.norm_hadamard_quant(x, bits, gain=gain)
    y1 = hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K)
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


def test_forward_k_split_strided_output(hbl):
    M, N, K, pad, bits = 70, 512, 16384, 8, 8
    assert _split_active(hbl, M, N, K, bits)
    x = to_device(workloads.random_rows(53, M, K, "t3"))
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(54, 6, N, K)))
    big = torch.full((M, N + pad), 5, dtype=torch.bfloat16, device="cuda")
    hbl.forward(x, packed, alpha, bits, out=big[:, :N])
    q, s, rs = hbl.hadamard_quant(x, bits)
    ref = hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K)
    assert torch.equal(big[:, :N].contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.all(big[:, N:] == 5)
