"""The allocation-free entry point hbl_forward_noalloc, through the C ABI:
its output equals hbl_forward's bit for bit (the same kernels on the same
inputs; the bar of the parity tests is a tolerance, equality is stricter),
on consecutive calls that share the library's static workspace, the later
ones smaller; and a shape whose workspace exceeds the static array is
rejected before anything is enqueued."""
from __future__ import annotations

import pytest
import torch

import workloads
from parity_util import to_device

pytestmark = pytest.mark.gpu


def _call(hbl, x, packed, alpha, bits, had):
    M, K = x.shape
    N = packed.shape[0]
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = hbl.lib().hbl_forward_noalloc(x.data_ptr(), hbl.DTYPE_BF16, M, K, K, N, hbl.HADAMARD if had else 0, bits,
                                       packed.data_ptr(), alpha.data_ptr(), y.data_ptr(), N, hbl._stream())
    assert rc == hbl.OK, hbl.lib().hbl_last_error()
    return y


# (M, K, N, bits, rotation): the first splits K over partial sums in the
# static workspace (256 tokens, fewer tiles than compute units); each later
# call is smaller than the one before and reuses the same array
CASES = [(256, 16384, 4096, 8, True), (130, 4096, 512, 4, True), (37, 1024, 256, 8, False), (3, 4096, 4096, 4, True)]


def test_forward_noalloc_equals_forward(hbl):
    lib = hbl.lib()
    for i, (M, K, N, bits, had) in enumerate(CASES):
        assert lib.hbl_forward_workspace_size(M, N, K, bits) <= hbl.NOALLOC_WORKSPACE_BYTES
        x = to_device(workloads.random_rows(500 + i, M, K, "t3"))
        packed, alpha = hbl.ternarize_weights(to_device(workloads.gaussian_weights(500 + i, 1, N, K)))
        ref = hbl.forward(x, packed, alpha, bits, hadamard=had)
        y = _call(hbl, x, packed, alpha, bits, had)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"case {i}: differs from hbl_forward"
        # a second call on the same inputs after the others (same bits)
        y2 = hbl.forward_noalloc(x, packed, alpha, bits, hadamard=had)
        assert torch.equal(y2.view(torch.int16), ref.view(torch.int16))


def test_forward_noalloc_rejects_oversized_workspace(hbl):
    lib = hbl.lib()
    M, K, N = 4096, 16384, 4096  # INT8 codes alone are 64 MiB
    assert lib.hbl_forward_workspace_size(M, N, K, 8) > hbl.NOALLOC_WORKSPACE_BYTES
    rc = lib.hbl_forward_noalloc(0x100000, hbl.DTYPE_BF16, M, K, K, N, hbl.HADAMARD, 8, 0x200000, 0x300000,
                                 0x400000, N, None)
    assert rc == hbl.ERR_WORKSPACE
    assert b"static workspace" in lib.hbl_last_error()
