"""GPU parity at the five workloads' full sizes, through the C ABI, in the
launch configuration the benchmark times, against the CPU oracle.

Rows compared with the oracle:
  tiny (M = 8), wo_7b (M = 2048), wdown_7b (M = 4096) and the decode shapes
  (M = 1, 4, 16 at K = 4096 and 16384): every row;
  each of the seven linears of the 7B block (M = 65536), INT8 and INT4:
  4096 rows drawn with numpy's default_rng(BLOCK_SAMPLE_SEED) without
  replacement, plus the first and the last row.
What is compared on those rows (BitNet v2 architecture write-up, §3.4):
  the ternary codes and alpha of the whole weight matrix (Eq. 1-2), bit for
  bit; the activation codes, scales and row sums of the full-batch
  quantiser launch (Eq. 3-8) under the code and scale rules of
  parity_util; the int32 matmul (Eq. 9) of the full batch fed the oracle's
  codes, bit-exact against the oracle's integers; the bf16 layer output
  against the oracle's fp64 layer value, per-row relative L2.  INT4 layers
  whose width allows it also run the FP6 x FP4 path: its MX4 weights, its
  MX6 codes and scales, its int32 matmul on the oracle's codes, and its
  layer output (against the oracle, and bit for bit against the int8
  path's output on every row).
The oracle's matmul on these sizes is oracle.gemm_exact (the oracle's
unpacked codes through an exact fp64 library matmul, pinned against its
triple loop on the CPU).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import mx_util
import oracle
import workloads
from parity_util import bf16_to_f64, check_codes, check_output, check_scales, codes_to_numpy, to_device

pytestmark = pytest.mark.gpu

BLOCK_SAMPLE = 4096
BLOCK_SAMPLE_SEED = 2024


def block_rows(M: int) -> np.ndarray:
    rng = np.random.default_rng(BLOCK_SAMPLE_SEED)
    r = set(rng.choice(M, BLOCK_SAMPLE, replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(r))


@functools.lru_cache(maxsize=1)
def _block_input(name: str) -> np.ndarray:
    return workloads.block_input(name)


@functools.lru_cache(maxsize=2)
def _block_weights(layer: str) -> np.ndarray:
    return workloads.block_weights(layer)


def _dev_codes(codes: np.ndarray, bits: int) -> torch.Tensor:
    c = np.ascontiguousarray(codes)
    return torch.from_numpy(c if bits == 8 else c.view(np.int32)).cuda()


def _take(t: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    return t[torch.from_numpy(rows).cuda()]


def _layer_parity(hbl, x_np, w_np, bits, had, what, rows=None):
    M, K = x_np.shape
    N = w_np.shape[0]
    rows = np.arange(M) if rows is None else rows
    print(f"[parity] {what}: M={M} K={K} N={N} INT{bits} rotation={had} rows={rows.size}", flush=True)
    x = to_device(x_np)

    # weights (Eq. 1-2): the whole matrix, bit for bit
    packed, alpha = hbl.ternarize_weights(to_device(w_np))
    o_packed, o_alpha, o_tern = oracle.ternarize(w_np)
    assert float(alpha.cpu()[0]) == float(o_alpha), f"{what}: alpha"
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), o_packed), f"{what}: ternary codes"

    # quantiser over the full batch (the benchmark's launch), checked on rows
    q, s, rs = hbl.hadamard_quant(x, bits, hadamard=had)
    torch.cuda.synchronize()
    all_q, all_s, all_rs = oracle.quantize(x_np, bits, hadamard=had)
    xr_rows = np.ascontiguousarray(x_np[rows])
    oq, os_, ors, xr = oracle.quantize(xr_rows, bits, hadamard=had, want_xr=True)
    assert np.array_equal(oq, all_q[rows]) and np.array_equal(os_, all_s[rows])
    gq = oracle.codes_int8(codes_to_numpy(_take(q, rows), bits), bits, K)
    oq8 = oracle.codes_int8(oq, bits, K)
    nbad = check_codes(gq, oq8, xr, bits, what)
    check_scales(_take(s, rows).cpu().numpy(), os_, what)
    grs = _take(rs, rows).cpu().numpy().astype(np.int64)
    assert np.array_equal(grs, gq.astype(np.int64).sum(axis=1)), f"{what}: rowsum != sum of codes"
    assert np.abs(grs - ors).sum() <= nbad
    del q, s, rs

    # int32 matmul of the full batch on the oracle's codes
    acc = hbl.ternary_gemm(_dev_codes(all_q, bits), bits, torch.from_numpy(all_s).cuda(),
                           torch.from_numpy(all_rs).cuda(), packed, alpha, K, out_dtype=hbl.OUT_I32)
    ref = oracle.gemm_exact(oq, bits, o_packed, K)
    assert np.array_equal(_take(acc, rows).cpu().numpy(), ref), f"{what}: integer matmul"
    del acc

    # the whole layer
    y = hbl.forward(x, packed, alpha, bits, hadamard=had)
    y64, _ = oracle.dequant_output(ref, os_, o_alpha)
    worst = check_output(bf16_to_f64(_take(y, rows)), y64, what)

    mx = bits == 4 and K >= 1024 and (K & (K - 1)) == 0
    if mx:
        wq = hbl.prepare_weights_mx(packed, K)
        assert np.array_equal(wq.cpu().numpy().view(np.uint32), mx_util.encode_mx4(o_tern)), f"{what}: MX4 weights"
        cm, sm = hbl.hadamard_quant_mx(x, hadamard=had)
        torch.cuda.synchronize()
        gq6 = mx_util.decode_mx6(cm.cpu().numpy(), K, rows).astype(np.int8)
        check_codes(gq6, oq8, xr, 4, what + " MX6")
        check_scales(_take(sm, rows).cpu().numpy(), os_, what + " MX6")
        assert np.array_equal(gq6, gq), f"{what}: MX6 codes differ from the INT4 layout's"
        del cm, sm
        codes6 = torch.from_numpy(mx_util.encode_mx6(oq8)).cuda()
        acc6 = hbl.ternary_gemm_mx(codes6, torch.from_numpy(os_).cuda(), wq, alpha, K, out_dtype=hbl.OUT_I32, N=N)
        assert np.array_equal(acc6.cpu().numpy(), ref), f"{what}: FP6 x FP4 integer matmul"
        del codes6, acc6
        y6 = hbl.forward_mx(x, wq, alpha, hadamard=had, N=N)
        assert torch.equal(y6.view(torch.int16), y.view(torch.int16)), f"{what}: FP6 x FP4 and int8 outputs differ"
        check_output(bf16_to_f64(_take(y6, rows)), y64, what + " FP6 x FP4")
    print(f"[parity] {what}: ok, worst row rel-L2 {worst:.2e}", flush=True)


def test_full_tiny(hbl):
    c = workloads.tiny()
    _layer_parity(hbl, c["x"], c["w"], c["bits"], True, "tiny")


def test_full_wo_7b(hbl):
    c = workloads.wo_7b()
    _layer_parity(hbl, c["x"], c["w"], c["bits"], True, "wo_7b")


def test_full_wdown_7b(hbl):
    c = workloads.wdown_7b()
    _layer_parity(hbl, c["x"], c["w"], c["bits"], True, "wdown_7b")


@pytest.mark.parametrize("K,N", [(4096, 4096), (16384, 4096)])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_full_decode(hbl, K, N, M):
    x = workloads.decode_inputs(K, M)
    w = workloads.decode_weights(K, N, 0)
    _layer_parity(hbl, x, w, 8, True, f"decode M={M} K={K}")


# parameters ordered so that consecutive tests share an input (cached)
BLOCK_CASES = [(layer, bits) for layer in ("q", "k", "v", "o", "up", "gate", "down") for bits in (8, 4)]


@pytest.mark.parametrize("layer,bits", BLOCK_CASES)
def test_full_block_7b(hbl, layer, bits):
    names = [n for n, *_ in workloads.BLOCK_7B_LAYERS]
    _, K, N, had = workloads.BLOCK_7B_LAYERS[names.index(layer)]
    x = _block_input(workloads.BLOCK_7B_INPUT_OF[layer])
    w = _block_weights(layer)
    _layer_parity(hbl, x, w, bits, had, f"block_7b {layer} INT{bits}", rows=block_rows(x.shape[0]))
