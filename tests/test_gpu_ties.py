"""Exact rounding ties on the GPU, through the C ABI.

The rows of tests/golden/quant_ties.txt make the fp32 product each quantiser
rounds exactly k + 1/2 (BitNet v2 architecture write-up, §3.4 "Weight
Quantization", Eq. 2, read as round half to even; the construction is in
that file).  Zero padding leaves the INT8 and KV statistics (a maximum)
unchanged, and for the INT4 and ternary statistics (a mean) the rows keep
the fixture's length.  At an exact tie the kernel and the oracle must agree
bit for bit: no tie allowance applies here.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from parity_util import codes_to_numpy, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_ties.txt")


def _fixture():
    kv = {}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.split()
    return kv


def _row(kv, key, K):
    x = np.array([float.fromhex(v) for v in kv[f"{key}.x"]], np.float32)
    r = np.zeros(K, np.float32)
    r[:x.size] = x
    return r, x.size


# fp32 rows (the fixture's gamma has more significant bits than bf16 holds);
# K = 64 takes the small-row kernel (rint of the fp32 product), K = 1024 and
# 16384 the wide-row kernel (one FMA rounding the exact product)
@pytest.mark.parametrize("K", [64, 1024, 16384])
def test_int8_ties(hbl, K):
    kv = _fixture()
    r, n = _row(kv, "int8", K)
    x = np.stack([r, -r, np.roll(r, K // 2)])
    q, s, rs = hbl.hadamard_quant(to_device(x), 8, hadamard=False)
    got = codes_to_numpy(q, 8)
    oq, os_, ors = oracle.quantize(x, 8, hadamard=False)
    want = np.array([int(v) for v in kv["int8.codes"]], np.int8)
    assert np.array_equal(got[0, :n], want) and np.array_equal(got[1, :n], -want)
    assert np.array_equal(got, oq), "GPU and oracle codes differ at exact ties"
    assert np.array_equal(rs.cpu().numpy(), ors)
    assert np.array_equal(s.cpu().numpy(), os_)


def test_int4_ties(hbl):
    kv = _fixture()
    K = int(kv["int4.K"][0])
    r, n = _row(kv, "int4", K)
    x = np.stack([r, -r, r[::-1].copy()])
    q, s, rs = hbl.hadamard_quant(to_device(x), 4, hadamard=False)
    got = oracle.unpack_int4(codes_to_numpy(q, 4), K)
    oq, os_, ors = oracle.quantize(x, 4, hadamard=False)
    want = np.array([int(v) for v in kv["int4.codes"]], np.int8)
    assert np.array_equal(got[0, :n], want)
    assert np.array_equal(got, oracle.unpack_int4(oq, K)), "GPU and oracle codes differ at exact ties"
    assert np.array_equal(rs.cpu().numpy(), ors)
    assert np.array_equal(s.cpu().numpy(), os_)


@pytest.mark.parametrize("N", [1, 64])
def test_ternary_ties(hbl, N):
    kv = _fixture()
    K = int(kv["ternary.K"][0])
    r, n = _row(kv, "ternary", K)
    w = np.tile(r, (N, 1))  # copies keep the mean |W|
    packed, alpha = hbl.ternarize_weights(to_device(w))
    o_packed, o_alpha, o_q = oracle.ternarize(w)
    assert float(alpha.cpu()[0]) == float(o_alpha) == float.fromhex(kv["ternary.alpha"][0])
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), o_packed)
    assert o_q[0, :n].tolist() == [int(v) for v in kv["ternary.codes"]]


@pytest.mark.parametrize("bits", [3, 4])
def test_kv_ties(hbl, bits):
    kv = _fixture()
    D = 32
    r, n = _row(kv, f"kv{bits}", D)
    x = np.stack([r, -r]).reshape(1, 1, 2, D)  # one token, two heads
    codes, scales, _, _ = hbl.kv_quant(to_device(x), bits, keep_bos8=False)
    oc, os_, _, _ = oracle.kv_quant(x, bits, keep_bos8=False)
    assert np.array_equal(codes.cpu().numpy(), oc), "GPU and oracle codes differ at exact ties"
    assert np.array_equal(scales.cpu().numpy(), os_)
    half = 1 << (bits - 1)
    u = np.rint(oracle.kv_dequant(oc, os_, D, bits)[0, 0, 0] / os_[0, 0, 0]).astype(int) + half
    assert u[:n].tolist() == [int(v) for v in kv[f"kv{bits}.codes"]]
