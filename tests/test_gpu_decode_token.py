"""The few-token decode layer in one launch: hbl_forward with M bf16 tokens
(M <= 4 up to K = 2048, 2 up to 8192, else 1), INT8 or INT4 codes and the
rotation (BitNet v2 architecture write-up, §3.4 "H-BitLinear", Eq. 9 with
the INT8 quantiser of Eq. 7 or the INT4 one of Eq. 8) runs in one kernel
whose every block rotates and quantises the token rows itself.

Checked here:
  - INT8: the layer output bit for bit against the two-launch path
    (hbl_hadamard_quant, then hbl_ternary_gemm): the same rotation and
    rounding give the same codes, and the integer sums are exact;
  - the layer output against the oracle's fp64 layer value (per-row L2);
  - every supported (K, M), K = 1024 ... 16384, M up to those limits, and N = 16 (one
    matmul block of 16 features), 48 (three) and 4096; strided token rows and outputs; an all-zero token among others
    (its outputs exactly zero); the next M up, which takes two launches;
  - 100 consecutive calls on changing inputs, each checked;
  - a HIP graph of several calls replayed with new inputs between replays;
  - INT4 at every supported (K, M): against the oracle, and bit for bit
    against the two-launch path;
  - plain BitLinear (no rotation, INT8; up to four tokens at K <= 4096, two
    at 8192) at every supported (K, M): the same two checks, strided rows,
    an all-zero token and repeated calls.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import bf16_to_f64, check_output, to_device

pytestmark = pytest.mark.gpu


def _two_launch(hbl, x, packed, alpha):
    q, s, rs = hbl.hadamard_quant(x, 8)
    return hbl.ternary_gemm(q, 8, s, rs, packed, alpha, x.shape[1])


# rotated: up to 4 tokens in one launch up to K = 2048, 2 at 4096 and 8192
KM = [(K, M) for K, mmax in ((1024, 4), (2048, 4), (4096, 2), (8192, 2), (16384, 1)) for M in range(1, mmax + 2)]


@pytest.mark.parametrize("K,M", KM)
@pytest.mark.parametrize("N", [16, 48, 4096])
def test_decode_token_layer(hbl, K, M, N):
    print(f"[few-token decode] K={K} M={M} N={N}", flush=True)
    x_np = workloads.random_rows(K + 3 * N + M, M, K, "t3")
    w_np = workloads.gaussian_weights(9, K // 1024 + N, N, K)
    x = to_device(x_np)
    packed, alpha = hbl.ternarize_weights(to_device(w_np))
    y = hbl.forward(x, packed, alpha, 8)
    y2 = _two_launch(hbl, x, packed, alpha)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "one-launch and two-launch outputs differ"
    o_packed, o_alpha, _ = oracle.ternarize(w_np)
    y64 = oracle.forward(x_np, o_packed, o_alpha, 8, hadamard=True)
    check_output(bf16_to_f64(y), y64, f"few-token decode K={K} M={M} N={N}")


@pytest.mark.parametrize("K,M", [(4096, 1), (4096, 2), (4096, 3), (8192, 2), (16384, 1)])
def test_decode_token_strided_and_zero_row(hbl, K, M):
    N = 64
    zero = M - 1  # the last token is all zero
    xb = torch.zeros((M, K + 256), dtype=torch.bfloat16, device="cuda")
    if M > 1:
        xb[:zero, :K] = to_device(workloads.random_rows(33 + M, zero, K, "t3"))
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(10, 1, N, K)))
    yb = torch.full((M, N + 24), -7.0, dtype=torch.bfloat16, device="cuda")
    hbl.forward(xb[:, :K], packed, alpha, 8, out=yb[:, :N])
    y2 = _two_launch(hbl, xb[:, :K].contiguous(), packed, alpha)
    torch.cuda.synchronize()
    assert torch.equal(yb[:, :N].view(torch.int16), y2.view(torch.int16))
    assert torch.all(yb[:, N:] == -7.0), "wrote outside the output view"
    assert torch.all(yb[zero, :N].view(torch.int16) == 0), "an all-zero token must give exactly zero"


@pytest.mark.parametrize("K", [4096, 16384])
def test_decode_token_many_calls(hbl, K):
    N = 512
    xs = [to_device(workloads.random_rows(80 + i, 1, K, "t3")) for i in range(3)]
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(11, 2, N, K)))
    refs = [_two_launch(hbl, xi, packed, alpha) for xi in xs]
    x = torch.empty_like(xs[0])
    outs = torch.empty((100, 1, N), dtype=torch.bfloat16, device="cuda")
    for i in range(100):
        x.copy_(xs[i % 3])
        hbl.forward(x, packed, alpha, 8, out=outs[i])
    torch.cuda.synchronize()
    for i in range(100):
        assert torch.equal(outs[i].view(torch.int16), refs[i % 3].view(torch.int16)), f"call {i}"


def test_decode_token_graph_replays(hbl):
    """A graph of four calls (two matrices at each of two widths: two tokens
    at K = 4096, one at K = 16384), replayed four times with new token rows
    copied in eagerly before each replay."""
    mats = [(4096, hbl.ternarize_weights(to_device(workloads.gaussian_weights(12, j, 4096, 4096)))) for j in range(2)]
    mats += [(16384, hbl.ternarize_weights(to_device(workloads.gaussian_weights(12, 2 + j, 4096, 16384))))
             for j in range(2)]
    rows = {4096: 2, 16384: 1}
    xs = {K: torch.empty((rows[K], K), dtype=torch.bfloat16, device="cuda") for K in rows}
    outs = [torch.empty((rows[K], 4096), dtype=torch.bfloat16, device="cuda") for K, _ in mats]
    ws = [hbl.forward_workspace(rows[K], 4096, K, 8, "cuda") for K, _ in mats]

    def run():
        for c, (K, (p, a)) in enumerate(mats):
            hbl.forward(xs[K], p, a, 8, out=outs[c], workspace=ws[c])

    for K in xs:
        xs[K].copy_(to_device(workloads.random_rows(90 + K // 1024, rows[K], K, "t3")))
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(4):
        for K in xs:
            xs[K].copy_(to_device(workloads.random_rows(100 + 10 * r + K // 1024, rows[K], K, "t3")))
        refs = [_two_launch(hbl, xs[K], p, a) for K, (p, a) in mats]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c in range(len(mats)):
            assert torch.equal(outs[c].view(torch.int16), refs[c].view(torch.int16)), f"replay {r}, call {c}"


@pytest.mark.parametrize("K,M", KM)
@pytest.mark.parametrize("N", [16, 4096])
def test_decode_token_layer_int4(hbl, K, M, N):
    """INT4 absmean codes (Eq. 8): against the oracle (per-row L2), and bit
    for bit against the two-launch path, whose quantiser takes the same
    row function for these few tokens."""
    print(f"[few-token decode INT4] K={K} M={M} N={N}", flush=True)
    x_np = workloads.random_rows(2 * K + 3 * N + M, M, K, "t3")
    w_np = workloads.gaussian_weights(13, K // 1024 + N, N, K)
    x = to_device(x_np)
    packed, alpha = hbl.ternarize_weights(to_device(w_np))
    y = hbl.forward(x, packed, alpha, 4)
    q, s, rs = hbl.hadamard_quant(x, 4)
    y2 = hbl.ternary_gemm(q, 4, s, rs, packed, alpha, K)
    torch.cuda.synchronize()
    o_packed, o_alpha, _ = oracle.ternarize(w_np)
    y64 = oracle.forward(x_np, o_packed, o_alpha, 4, hadamard=True)
    check_output(bf16_to_f64(y), y64, f"few-token decode INT4 K={K} M={M} N={N}")
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "one-launch and two-launch outputs differ"


def _two_launch_plain(hbl, x, packed, alpha):
    q, s, rs = hbl.hadamard_quant(x, 8, hadamard=False)
    return hbl.ternary_gemm(q, 8, s, rs, packed, alpha, x.shape[1])


# plain INT8 takes up to 4 tokens in one launch up to K = 4096, 2 at 8192
KM_PLAIN = [(K, M) for K, mmax in ((1024, 4), (2048, 4), (4096, 4), (8192, 2), (16384, 1))
            for M in range(1, mmax + 2)]


@pytest.mark.parametrize("K,M", KM_PLAIN)
@pytest.mark.parametrize("N", [16, 4096])
def test_decode_plain_layer(hbl, K, M, N):
    """Plain BitLinear (Eq. 9 without the rotation), INT8 absmax codes of
    Eq. 7 on the raw token rows: one launch for up to four tokens (up to K =
    4096; two at 8192, one at 16384), bit for bit against the two-launch
    path (the same absmax, factor and rounding) and against the oracle's
    fp64 layer value; the next M up takes two launches."""
    print(f"[plain decode] K={K} M={M} N={N}", flush=True)
    x_np = workloads.random_rows(7 * K + N + M, M, K, "t3")
    w_np = workloads.gaussian_weights(13, K // 1024 + N, N, K)
    x = to_device(x_np)
    packed, alpha = hbl.ternarize_weights(to_device(w_np))
    y = hbl.forward(x, packed, alpha, 8, hadamard=False)
    y2 = _two_launch_plain(hbl, x, packed, alpha)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "one-launch and two-launch outputs differ"
    o_packed, o_alpha, _ = oracle.ternarize(w_np)
    y64 = oracle.forward(x_np, o_packed, o_alpha, 8, hadamard=False)
    check_output(bf16_to_f64(y), y64, f"plain decode K={K} M={M} N={N}")


@pytest.mark.parametrize("K,M", [(4096, 1), (4096, 2), (4096, 4), (8192, 2), (16384, 1)])
def test_decode_plain_strided_zero_row_and_repeats(hbl, K, M):
    """Strided token rows and outputs, an all-zero token (exactly zero
    outputs), and 20 consecutive calls on changing inputs, each equal to the
    two-launch result."""
    N = 64
    xb = torch.zeros((M, K + 256), dtype=torch.bfloat16, device="cuda")
    if M > 1:
        xb[:M - 1, :K] = to_device(workloads.random_rows(44 + M, M - 1, K, "t3"))
    packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(14, 1, N, K)))
    yb = torch.full((M, N + 24), -7.0, dtype=torch.bfloat16, device="cuda")
    hbl.forward(xb[:, :K], packed, alpha, 8, hadamard=False, out=yb[:, :N])
    y2 = _two_launch_plain(hbl, xb[:, :K].contiguous(), packed, alpha)
    torch.cuda.synchronize()
    assert torch.equal(yb[:, :N].view(torch.int16), y2.view(torch.int16))
    assert torch.all(yb[:, N:] == -7.0), "wrote outside the output view"
    assert torch.all(yb[M - 1, :N].view(torch.int16) == 0), "an all-zero token must give exactly zero"
    xs = [to_device(workloads.random_rows(120 + i, M, K, "t3")) for i in range(3)]
    refs = [_two_launch_plain(hbl, xi, packed, alpha) for xi in xs]
    x = torch.empty_like(xs[0])
    outs = torch.empty((20, M, N), dtype=torch.bfloat16, device="cuda")
    for i in range(20):
        x.copy_(xs[i % 3])
        hbl.forward(x, packed, alpha, 8, hadamard=False, out=outs[i])
    torch.cuda.synchronize()
    for i in range(20):
        assert torch.equal(outs[i].view(torch.int16), refs[i % 3].view(torch.int16)), f"call {i}"
