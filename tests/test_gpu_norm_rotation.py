"""GPU parity of the entry points around the core path, through the C ABI:
the RMSNorm layer of Eq. 9 in front of the rotation and quantiser, the
backward of the rotation (Eq. 10), and the weight side of the weight-and-
activation rotation variant (Table 5), each against the CPU oracle.

Tolerances as for the core path: rotated values 1e-5 of the row maximum;
codes identical except at most 1e-4 of them, off by one at rounding ties;
scales 1e-6 relative; bf16 layer outputs 1e-2 per-row L2.  Ternary codes of
the rotated weights follow the code rule (the GPU rotates in fp32, the
oracle in fp64), and alpha agrees to 1e-5 relative.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import (bf16_to_f64, check_codes, check_hadamard, check_output, check_scales,
                         codes_to_numpy, to_device)

pytestmark = pytest.mark.gpu

ALL_LOG2K = list(range(4, 15))


def _gain(K, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(-2.0, 2.0, K).astype(np.float32)


def _norm_case(hbl, x, bits, had, gain, what):
    g_dev = torch.from_numpy(gain).cuda() if gain is not None else None
    q, s, rs = hbl.norm_hadamard_quant(to_device(x), bits, gain=g_dev, hadamard=had)
    torch.cuda.synchronize()
    oq, os_, ors, xr = oracle.norm_quantize(x, bits, gain=gain, hadamard=had, want_xr=True)
    K = x.shape[1]
    gq = oracle.codes_int8(codes_to_numpy(q, bits), bits, K)
    nbad = check_codes(gq, oracle.codes_int8(oq, bits, K), xr, bits, what)
    check_scales(s.cpu().numpy(), os_, what)
    grs = rs.cpu().numpy()
    assert np.array_equal(grs, gq.astype(np.int64).sum(axis=1)), f"{what}: rowsum != sum of codes"
    assert np.abs(grs.astype(np.int64) - ors).sum() <= nbad
    return gq


# ------------------------------------------------- RMSNorm layer (Eq. 9)

@pytest.mark.parametrize("log2k", ALL_LOG2K)
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("with_gain", [False, True])
def test_norm_quant_with_rotation(hbl, log2k, bits, with_gain):
    K = 1 << log2k
    x = workloads.random_rows(400 + log2k, 37, K, "t3", as_bf16=True)
    gain = _gain(K, log2k) if with_gain else None
    _norm_case(hbl, x, bits, True, gain, f"norm K={K} INT{bits} gain={with_gain}")


@pytest.mark.parametrize("K", [256, 4096, 16384])
@pytest.mark.parametrize("bits", [8, 4])
def test_norm_quant_f32_input(hbl, K, bits):
    x = workloads.random_rows(500 + K % 89, 21, K, "t3", as_bf16=False)
    _norm_case(hbl, x, bits, True, _gain(K, 7), f"norm f32 K={K} INT{bits}")


@pytest.mark.parametrize("K", [64, 192, 960, 4096])
@pytest.mark.parametrize("bits", [8, 4])
def test_norm_quant_plain(hbl, K, bits):
    # BitLinear inputs (no rotation) go through the same normalisation
    x = workloads.random_rows(600 + K % 83, 21, K, "t3", as_bf16=True)
    _norm_case(hbl, x, bits, False, _gain(K, 8), f"norm plain K={K} INT{bits}")


@pytest.mark.parametrize("bits", [8, 4])
def test_norm_quant_degenerate_rows(hbl, bits):
    K = 2048
    rows = [np.zeros(K, np.float32),                      # all zero: r = 1/sqrt(eps), codes 0
            np.full(K, 3.0, np.float32),                  # constant
            np.eye(1, K, 17, dtype=np.float32)[0] * 50,   # spike
            np.full(K, 1e-30, np.float32),                # squares underflow: eps dominates
            (np.arange(K) % 7 - 3).astype(np.float32) * 6e4]
    x = np.stack(rows)
    gq = _norm_case(hbl, x, bits, True, None, f"norm degenerate INT{bits}")
    assert np.all(gq[0] == 0) and np.all(gq[3] == 0)


def test_norm_rows_of_one_block_are_independent(hbl):
    # K = 1024 packs 16 rows into a block: scaling one row must not move the others
    K, M, bits = 1024, 32, 4
    x = workloads.random_rows(9, M, K, "t3", as_bf16=False)
    y = x.copy()
    y[5] *= np.float32(1000.0)
    qa, sa, _ = hbl.norm_hadamard_quant(to_device(x), bits)
    qb, sb, _ = hbl.norm_hadamard_quant(to_device(y), bits)
    keep = np.arange(M) != 5
    assert torch.equal(qa[torch.from_numpy(keep).cuda()], qb[torch.from_numpy(keep).cuda()])
    assert np.array_equal(sa.cpu().numpy()[keep], sb.cpu().numpy()[keep])


@pytest.mark.parametrize("bits", [8, 4])
def test_norm_forward(hbl, bits):
    M, K, N = 70, 1024, 128
    x = workloads.random_rows(13, M, K, "t3")
    w = workloads.gaussian_weights(13, 1, N, K)
    gain = _gain(K, 13)
    packed, alpha = hbl.ternarize_weights(to_device(w))
    g_dev = torch.from_numpy(gain).cuda()
    y = hbl.norm_forward(to_device(x), packed, alpha, bits, gain=g_dev)
    # the same as the two steps
    q, s, rs = hbl.norm_hadamard_quant(to_device(x), bits, gain=g_dev)
    assert torch.equal(y, hbl.ternary_gemm(q, bits, s, rs, packed, alpha, K))
    o_packed, o_alpha, _ = oracle.ternarize(w)
    oq, os_, _ = oracle.norm_quantize(x, bits, gain=gain, hadamard=True)
    y64, _ = oracle.dequant_output(oracle.gemm_i32(oq, bits, o_packed, K), os_, o_alpha)
    check_output(bf16_to_f64(y), y64, f"norm forward INT{bits}")


@pytest.mark.parametrize("name", ["wo_7b", "wdown_7b"])
def test_norm_full_size(hbl, name):
    c = getattr(workloads, name)()
    x_np, w_np, bits = c["x"], c["w"], c["bits"]
    M, K = x_np.shape
    gain = _gain(K, 21)
    packed, alpha = hbl.ternarize_weights(to_device(w_np))
    o_packed, o_alpha, _ = oracle.ternarize(w_np)
    x = to_device(x_np)
    g_dev = torch.from_numpy(gain).cuda()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(M, 14, replace=False)]))
    xs = np.ascontiguousarray(x_np[rows])
    q, s, _ = hbl.norm_hadamard_quant(x, bits, gain=g_dev)
    oq, os_, _, xr = oracle.norm_quantize(xs, bits, gain=gain, hadamard=True, want_xr=True)
    gq = oracle.codes_int8(codes_to_numpy(q, bits)[rows], bits, K)
    check_codes(gq, oracle.codes_int8(oq, bits, K), xr, bits, f"{name} norm")
    check_scales(s.cpu().numpy()[rows], os_, f"{name} norm")
    y = hbl.norm_forward(x, packed, alpha, bits, gain=g_dev)
    gr = rows[:6]
    oq6, os6, _ = oracle.norm_quantize(np.ascontiguousarray(x_np[gr]), bits, gain=gain, hadamard=True)
    y64, _ = oracle.dequant_output(oracle.gemm_i32(oq6, bits, o_packed, K), os6, o_alpha)
    check_output(bf16_to_f64(y[torch.from_numpy(gr).cuda()]), y64, f"{name} norm forward")


# ------------------------------------------- backward of the rotation (Eq. 10)

@pytest.mark.parametrize("log2k", ALL_LOG2K)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hadamard_backward_values(hbl, log2k, dtype):
    K = 1 << log2k
    M = 9 if log2k <= 12 else 3  # the oracle's transposed product is O(K^2) per row
    dy = workloads.random_rows(700 + log2k, M, K, "t3", as_bf16=(dtype == "bf16"))
    dx = hbl.hadamard_backward_f32(to_device(dy)).cpu().numpy()
    check_hadamard(dx, oracle.hadamard_backward(dy), f"backward K={K} {dtype}")


def test_hadamard_backward_inverts_forward(hbl):
    K, M = 16384, 6
    x = workloads.random_rows(71, M, K, "normal", as_bf16=False)
    z = hbl.hadamard_backward_f32(hbl.hadamard_f32(to_device(x))).cpu().numpy()
    assert np.abs(z - x).max() <= 1e-5 * np.abs(x).max()


# ------------------------------------ weight and activation rotation (Table 5)

def _check_ternary_codes(gpu_packed, ora_q, wr, alpha, what):
    K = wr.shape[1]
    gq, bad = oracle.unpack_ternary(gpu_packed, K)
    assert bad == 0, f"{what}: invalid 2-bit fields"
    d = gq.astype(np.int32) - ora_q.astype(np.int32)
    idx = np.nonzero(d)
    if idx[0].size:
        assert np.all(np.abs(d[idx]) == 1), f"{what}: codes differ by more than 1"
        assert idx[0].size <= math.ceil(1e-4 * d.size), f"{what}: {idx[0].size} codes differ"
        v = np.abs(wr[idx].astype(np.float64) / (float(alpha) + 1e-5))
        assert np.all(np.abs(v - 0.5) < 1e-4), f"{what}: a mismatch is not at the 1/2 boundary"


@pytest.mark.parametrize("N,K", [(256, 256), (64, 4096), (4096, 4096), (1024, 16384)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ternarize_rotated(hbl, N, K, dtype):
    w = workloads.gaussian_weights(19, N + K, N, K)
    if dtype == "bf16":
        w = workloads.bf16_bits(w)
    packed, alpha = hbl.ternarize_weights_rotated(to_device(w))
    o_packed, o_alpha, o_q, wr = oracle.ternarize_rotated(w, want_wr=True)
    a = float(alpha.cpu()[0])
    assert abs(a - float(o_alpha)) <= 1e-5 * float(o_alpha), f"alpha {a} vs {o_alpha}"
    _check_ternary_codes(packed.cpu().numpy().view(np.uint32), o_q, wr, o_alpha, f"rotated N={N} K={K} {dtype}")


@pytest.mark.parametrize("bits", [8, 4])
def test_rotation_variant_forward(hbl, bits):
    # Q_w(W H^T) . Q(H x): the rotated weights with the rotated activations
    M, K, N = 96, 4096, 256
    x = workloads.random_rows(23, M, K, "t3")
    w = workloads.gaussian_weights(23, 2, N, K)
    packed, alpha = hbl.ternarize_weights_rotated(to_device(w))
    y = hbl.forward(to_device(x), packed, alpha, bits, hadamard=True)
    gp = packed.cpu().numpy().view(np.uint32)
    y64 = oracle.forward(x, gp, float(alpha.cpu()[0]), bits, hadamard=True)
    check_output(bf16_to_f64(y), y64, f"rotation variant INT{bits}")
