"""GPU parity of the post-RoPE QKV / KV-cache quantiser against the CPU
oracle, through the C ABI.  Both sides form the per-head factor with an
IEEE divide and round the fp32 product, so codes and scales must agree bit
for bit (the maximum of a head is exact)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import to_device

pytestmark = pytest.mark.gpu


def _heads(seed, B, S, H, D, bf16):
    x = workloads.random_rows(seed, B * S * H, D, "t3", as_bf16=bf16)
    return x.reshape(B, S, H, D)


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("D", [32, 64, 128, 256, 2048])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_quant_matches_oracle(hbl, bits, D, dtype):
    B, S, H = 3, 5, 4
    x = _heads(900 + D + bits, B, S, H, D, dtype == "bf16")
    c, s, bc, bs = hbl.kv_quant(to_device(x), bits, keep_bos8=True)
    oc, os_, obc, obs = oracle.kv_quant(x, bits, keep_bos8=True)
    assert np.array_equal(c.cpu().numpy(), oc)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(bc.cpu().numpy(), obc)
    assert np.array_equal(bs.cpu().numpy(), obs)


def test_kv_quant_without_bos_and_degenerate_heads(hbl):
    B, S, H, D = 2, 3, 5, 128
    x = _heads(31, B, S, H, D, False)
    x[0, 1, 2] = 0.0                      # all-zero head
    x[1, 2, 4] = 1e-30                    # far below eps
    x[1, 0, 0, 7] = 3.0e4                 # one spike
    c, s, _, _ = hbl.kv_quant(to_device(x), 3, keep_bos8=False)
    oc, os_, _, _ = oracle.kv_quant(x, 3, keep_bos8=False)
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)


@pytest.mark.parametrize("bits", [3, 4])
def test_kv_quant_full_size(hbl, bits):
    # a 7B layer's K (or V) states, 1024 positions x 32 heads x 128, for 16
    # sequences (the benchmark's launch shape per sequence)
    B, S, H, D = 16, 1024, 32, 128
    x_np = workloads.random_rows(77, B * S * H, D, "t3", as_bf16=True).reshape(B, S, H, D)
    x = to_device(x_np.reshape(-1, D)).view(B, S, H, D)
    c, s, bc, bs = hbl.kv_quant(x, bits, keep_bos8=True)
    for b in (0, 1, B - 1):  # whole sequences, the oracle one by one
        oc, os_, obc, obs = oracle.kv_quant(np.ascontiguousarray(x_np[b:b + 1]), bits, keep_bos8=True)
        assert np.array_equal(c[b:b + 1].cpu().numpy(), oc)
        assert np.array_equal(s[b:b + 1].cpu().numpy(), os_)
        assert np.array_equal(bc[b:b + 1].cpu().numpy(), obc)
        assert np.array_equal(bs[b:b + 1].cpu().numpy(), obs)
