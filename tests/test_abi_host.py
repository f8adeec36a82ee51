"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/hbl.h declares, and
reject invalid arguments with the documented status code before anything is
enqueued.  Pointers passed here are never dereferenced: every call below is
rejected by validation, or is a documented no-op (M == 0).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hbl.h")


@pytest.fixture(scope="module")
def hbl():
    import bit_quantization_amd
    return bit_quantization_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hbl_\w+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ["hbl_ternarize_weights", "hbl_hadamard_quant", "hbl_ternary_gemm", "hbl_forward"]:
        assert n in names


def test_library_exports_every_declared_symbol(hbl):
    lib = ctypes.CDLL(hbl.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_version_and_status_strings(hbl):
    lib = hbl.lib()
    assert lib.hbl_version() >= 100
    for s in range(7):
        assert lib.hbl_status_string(s)
    assert lib.hbl_status_string(99) == b"unknown status"


# fake, 256-byte aligned addresses: validation must fail before any use
A = 0x100000
B = 0x200000
C = 0x300000
D = 0x400000
E = 0x500000
F = 0x600000


def last(hbl):
    return hbl.lib().hbl_last_error().decode()


@pytest.mark.parametrize("K,flags,expect", [
    (100, 1, 2),      # not a power of two with the rotation
    (8, 1, 2),        # below 16
    (32768, 1, 2),    # above the maximum
    (96, 0, 2),       # not a multiple of 64 without the rotation
    (32768, 0, 2),
])
def test_quant_shape_errors(hbl, K, flags, expect):
    rc = hbl.lib().hbl_hadamard_quant(A, hbl.DTYPE_BF16, 4, K, K, flags, 8, B, C, D, None)
    assert rc == expect
    assert "K =" in last(hbl)


def test_quant_mode_errors(hbl):
    lib = hbl.lib()
    assert lib.hbl_hadamard_quant(A, 7, 4, 256, 256, 1, 8, B, C, D, None) == hbl.ERR_MODE
    assert lib.hbl_hadamard_quant(A, 1, 4, 256, 256, 1, 5, B, C, D, None) == hbl.ERR_MODE
    assert lib.hbl_hadamard_quant(A, 1, 4, 256, 256, 4, 8, B, C, D, None) == hbl.ERR_MODE


def test_quant_pointer_errors(hbl):
    lib = hbl.lib()
    assert lib.hbl_hadamard_quant(None, 1, 4, 256, 256, 1, 8, B, C, D, None) == hbl.ERR_NULL
    assert lib.hbl_hadamard_quant(A, 1, 4, 256, 256, 1, 8, None, C, D, None) == hbl.ERR_NULL
    assert lib.hbl_hadamard_quant(A + 8, 1, 4, 256, 256, 1, 8, B, C, D, None) == hbl.ERR_ALIGN
    assert lib.hbl_hadamard_quant(A, 1, 4, 256, 260, 1, 8, B, C, D, None) == hbl.ERR_ALIGN
    assert lib.hbl_hadamard_quant(A, 1, 4, 256, 128, 1, 8, B, C, D, None) == hbl.ERR_SHAPE
    assert lib.hbl_hadamard_quant(A, 1, -1, 256, 256, 1, 8, B, C, D, None) == hbl.ERR_SHAPE


def test_quant_zero_rows_is_a_noop(hbl):
    assert hbl.lib().hbl_hadamard_quant(A, 1, 0, 256, 256, 1, 4, B, C, D, None) == hbl.OK


def test_gemm_errors(hbl):
    lib = hbl.lib()
    g = lib.hbl_ternary_gemm
    assert g(A, 8, B, C, D, E, 4, 40, 256, 0, F, 40, None) == hbl.ERR_SHAPE    # N % 16
    assert g(A, 8, B, C, D, E, 4, 64, 100, 0, F, 64, None) == hbl.ERR_SHAPE    # K % 64
    assert g(A, 8, B, C, D, E, 4, 64, 256, 0, F, 32, None) == hbl.ERR_SHAPE    # ldo < N
    assert g(A, 8, B, C, D, E, 4, 64, 256, 0, F, 66, None) == hbl.ERR_ALIGN    # ldo % 4
    assert g(A, 3, B, C, D, E, 4, 64, 256, 0, F, 64, None) == hbl.ERR_MODE
    assert g(A, 8, B, C, D, E, 4, 64, 256, 9, F, 64, None) == hbl.ERR_MODE
    assert g(A, 8, B, None, D, E, 4, 64, 256, 0, F, 64, None) == hbl.ERR_NULL  # rowsum required
    assert g(A + 4, 8, B, C, D, E, 4, 64, 256, 0, F, 64, None) == hbl.ERR_ALIGN
    assert g(A, 8, B, C, D, E, 0, 64, 256, 0, F, 64, None) == hbl.OK         # M = 0


@pytest.mark.parametrize("K,expect", [((1 << 21), 0), ((1 << 21) + 64, 2), ((1 << 23), 2)])
def test_gemm_k_bound(hbl, K, expect):
    # K <= 2^21 (HBL_MAX_GEMM_K): the int32 sums and 32-bit tile offsets of
    # the int8 path and the fp32 sums of the FP6 x FP4 path stay exact;
    # checked with M = 0 so nothing is enqueued when the call is accepted
    lib = hbl.lib()
    assert lib.hbl_ternary_gemm(A, 8, B, C, D, E, 0, 64, K, 0, F, 64, None) == expect
    assert lib.hbl_ternary_gemm_mx(A, B, D, E, 0, 64, K, 0, F, 64, None) == expect
    if expect:
        assert "K =" in last(hbl)


@pytest.mark.parametrize("ldo,expect", [((1 << 27), 0), ((1 << 27) + 4, 2)])
def test_gemm_ldo_bound(hbl, ldo, expect):
    # ldo <= 2^27 (HBL_MAX_LDO): the tile kernels address the rows of one
    # store with 32-bit byte offsets; M = 0, so nothing is enqueued
    lib = hbl.lib()
    assert lib.hbl_ternary_gemm(A, 8, B, C, D, E, 0, 64, 256, 0, F, ldo, None) == expect
    assert lib.hbl_ternary_gemm_mx(A, B, D, E, 0, 64, 512, 0, F, ldo, None) == expect
    if expect:
        assert "ldo =" in last(hbl)


def test_forward_workspace(hbl):
    lib = hbl.lib()
    need = lib.hbl_forward_workspace_size(10, 64, 256, 4)
    assert need >= 10 * 128 + 2 * 40
    assert need % 256 == 0
    # room for int32 partial sums of a K split of the persistent matmul when
    # its tiles leave most CUs idle and M K >= 2^20: M = 64, N = 4096,
    # K = 16384 -> 16 tiles of 128 x 256, 8 slices; M = 32 streams the weights
    assert lib.hbl_forward_workspace_size(32, 4096, 16384, 8) == 32 * 16384 + 2 * 256
    assert lib.hbl_forward_workspace_size(64, 4096, 16384, 8) == 64 * 16384 + 2 * 256 + 8 * 16 * 128 * 256 * 4
    # 16 tokens stream the weights; 256 tiles need no split
    assert lib.hbl_forward_workspace_size(16, 4096, 16384, 8) == 16 * 16384 + 2 * 256
    assert lib.hbl_forward_workspace_size(2048, 4096, 4096, 4) == 2048 * 2048 + 2 * 8192
    rc = lib.hbl_forward(A, 1, 10, 256, 256, 64, 1, 4, B, C, D, 64, E, need - 1, None)
    assert rc == hbl.ERR_WORKSPACE
    rc = lib.hbl_forward(A, 1, 10, 256, 256, 64, 1, 4, B, C, D, 64, None, need, None)
    assert rc == hbl.ERR_WORKSPACE
    assert lib.hbl_forward(A, 1, 10, 256, 256, 60, 1, 4, B, C, D, 64, E, need, None) == hbl.ERR_SHAPE


@pytest.mark.parametrize("M,K,bits", [(1, 4096, 8), (2, 4096, 8), (1, 16384, 8), (1, 16384, 4)])
def test_forward_one_launch_shapes_still_validated(hbl, M, K, bits):
    """One or two bf16 tokens with the rotation run as one kernel that does
    not write the workspace; the arguments are validated all the same, and
    an invalid call enqueues nothing (no device is needed to reach these
    returns)."""
    lib = hbl.lib()
    N = 4096
    need = lib.hbl_forward_workspace_size(M, N, K, bits)
    assert need > 0
    f = lib.hbl_forward
    assert f(A, 1, M, K, K, N, 1, bits, B, C, D, N, E, need - 1, None) == hbl.ERR_WORKSPACE
    assert f(A, 1, M, K, K, N, 1, bits, B, C, D, N, None, need, None) == hbl.ERR_WORKSPACE
    assert f(A, 1, M, K, K, N, 1, bits, B, C, D, N - 4, E, need, None) == hbl.ERR_SHAPE  # ldy < N
    assert f(A, 1, M, K, K, N, 1, bits, None, C, D, N, E, need, None) == hbl.ERR_NULL
    assert f(A, 1, M, K, K, N, 1, bits, B, C, D + 2, N, E, need, None) == hbl.ERR_ALIGN


def test_ternarize_errors(hbl):
    lib = hbl.lib()
    need = lib.hbl_ternarize_workspace_size(64, 256)
    assert need >= 8
    t = lib.hbl_ternarize_weights
    assert t(A, 0, 64, 250, B, C, D, need, None) == hbl.ERR_SHAPE
    assert t(A, 0, 0, 256, B, C, D, need, None) == hbl.ERR_SHAPE
    assert t(A, 5, 64, 256, B, C, D, need, None) == hbl.ERR_MODE
    assert t(None, 0, 64, 256, B, C, D, need, None) == hbl.ERR_NULL
    assert t(A, 0, 64, 256, B, C, D, need - 1, None) == hbl.ERR_WORKSPACE
    assert t(A + 2, 0, 64, 256, B, C, D, need, None) == hbl.ERR_ALIGN


def test_hadamard_f32_errors(hbl):
    lib = hbl.lib()
    assert lib.hbl_hadamard_f32(A, 1, 4, 48, 48, B, None) == hbl.ERR_SHAPE
    assert lib.hbl_hadamard_f32(A, 1, 4, 256, 256, None, None) == hbl.ERR_NULL
    assert lib.hbl_hadamard_f32(A, 1, 0, 256, 256, B, None) == hbl.OK


def test_norm_quant_errors(hbl):
    lib = hbl.lib()
    q = lib.hbl_norm_hadamard_quant
    assert q(A, 1, 4, 256, 256, E + 4, 1, 8, B, C, D, None) == hbl.ERR_ALIGN           # gain alignment
    assert "gain" in last(hbl)
    assert q(A, 1, 4, 100, 100, E, 1, 8, B, C, D, None) == hbl.ERR_SHAPE
    assert q(A, 1, 4, 256, 256, E, 4, 8, B, C, D, None) == hbl.ERR_MODE
    assert q(A, 1, 4, 256, 256, None, 1, 3, B, C, D, None) == hbl.ERR_MODE
    assert q(A, 1, 4, 256, 256, None, 1, 8, None, C, D, None) == hbl.ERR_NULL
    assert q(A, 1, 0, 256, 256, None, 1, 4, B, C, D, None) == hbl.OK                   # M = 0


def test_norm_forward_errors(hbl):
    lib = hbl.lib()
    need = lib.hbl_forward_workspace_size(10, 64, 256, 4)
    f = lib.hbl_norm_forward
    assert f(A, 1, 10, 256, 256, F + 8, 64, 1, 4, B, C, D, 64, E, need, None) == hbl.ERR_ALIGN
    assert f(A, 1, 10, 256, 256, None, 64, 1, 4, B, C, D, 64, E, need - 1, None) == hbl.ERR_WORKSPACE
    assert f(A, 1, 10, 256, 256, None, 60, 1, 4, B, C, D, 64, E, need, None) == hbl.ERR_SHAPE
    assert f(A, 1, 0, 256, 256, None, 64, 1, 4, B, C, D, 64, E, need, None) == hbl.OK


def test_hadamard_backward_errors(hbl):
    lib = hbl.lib()
    b = lib.hbl_hadamard_backward_f32
    assert b(A, 1, 4, 48, 48, B, None) == hbl.ERR_SHAPE
    assert b(A, 1, 4, 256, 256, None, None) == hbl.ERR_NULL
    assert b(A, 2, 4, 256, 256, B, None) == hbl.ERR_MODE
    assert b(A, 1, 0, 256, 256, B, None) == hbl.OK


def test_ternarize_rotated_errors(hbl):
    lib = hbl.lib()
    need = lib.hbl_ternarize_rotated_workspace_size(64, 256)
    assert need >= 64 * 256 * 4 + lib.hbl_ternarize_workspace_size(64, 256)
    t = lib.hbl_ternarize_weights_rotated
    assert t(A, 0, 64, 192, B, C, D, need, None) == hbl.ERR_SHAPE      # not a power of two
    assert t(A, 0, 64, 32768, B, C, D, need, None) == hbl.ERR_SHAPE    # above the maximum
    assert t(A, 0, 0, 256, B, C, D, need, None) == hbl.ERR_SHAPE
    assert t(A, 5, 64, 256, B, C, D, need, None) == hbl.ERR_MODE
    assert t(None, 0, 64, 256, B, C, D, need, None) == hbl.ERR_NULL
    assert t(A, 0, 64, 256, B, C, D, need - 1, None) == hbl.ERR_WORKSPACE
    assert t(A + 2, 0, 64, 256, B, C, D, need, None) == hbl.ERR_ALIGN


def test_mx_entry_point_errors(hbl):
    lib = hbl.lib()
    q = lib.hbl_hadamard_quant_mx
    assert q(A, 1, 4, 512, 512, 1, B, C, None) == hbl.ERR_SHAPE          # K below 1024
    assert "FP6 x FP4" in last(hbl)
    assert q(A, 1, 4, 3072, 3072, 0, B, C, None) == hbl.ERR_SHAPE        # not a power of two
    assert q(A, 1, 4, 1024, 1024, 2, B, C, None) == hbl.ERR_MODE
    assert q(A, 1, 4, 1024, 1024, 1, None, C, None) == hbl.ERR_NULL
    assert q(A, 1, 0, 1024, 1024, 1, B, C, None) == hbl.OK
    g = lib.hbl_ternary_gemm_mx
    assert g(A, B, C, D, 4, 64, 768, 0, F, 64, None) == hbl.ERR_SHAPE     # K % 512
    assert g(A, B, C, D, 4, 40, 1024, 0, F, 40, None) == hbl.ERR_SHAPE    # N % 16
    assert g(A, B, C, D, 4, 64, 1024, 5, F, 64, None) == hbl.ERR_MODE
    assert g(A, B, None, D, 4, 64, 1024, 0, F, 64, None) == hbl.ERR_NULL
    assert g(A + 8, B, C, D, 4, 64, 1024, 0, F, 64, None) == hbl.ERR_ALIGN
    assert g(A, B, C, D, 0, 64, 1024, 0, F, 64, None) == hbl.OK
    # whole 256-row code blocks and 128-row weight blocks
    assert lib.hbl_mx_codes_bytes(10, 1024) == 256 * 768 and lib.hbl_mx_codes_bytes(257, 1024) == 512 * 768
    assert lib.hbl_mx_weights_bytes(130, 1024) == 256 * 256 and lib.hbl_mx_weights_bytes(128, 1024) == 128 * 256
    need = lib.hbl_forward_mx_workspace_size(10, 64, 1024)
    assert need >= 256 * 768 + 40 and need % 256 == 0
    # fewer than 256 tiles of 256 x 128: room for a split of K (one tile;
    # at least 8 stages of 128 per slice, so none at K = 1024; at K = 16384
    # 16 slices of 256 x 128 int16 partial sums, |sum| <= 8 * 1024)
    assert lib.hbl_forward_mx_workspace_size(10, 64, 16384) == 256 * 12288 + 256 + 16 * 256 * 128 * 2
    # M = 1024, N = K = 16384: 128 tiles, 2 slices of 8192 (fp32 partials)
    assert lib.hbl_forward_mx_workspace_size(1024, 4096, 16384) == 1024 * 12288 + 4096 + 2 * 1024 * 4096 * 4
    # 256 tiles already: no split
    big = lib.hbl_forward_mx_workspace_size(4096, 4096, 16384)
    assert big == 4096 * 12288 + 4096 * 4
    f = lib.hbl_forward_mx
    assert f(A, 1, 10, 1024, 1024, 64, 1, B, C, D, 64, E, need - 1, None) == hbl.ERR_WORKSPACE
    assert f(A, 1, 10, 2048, 2048, 64, 1, B, C, D, 64, E, need, None) == hbl.ERR_WORKSPACE
    assert f(A, 1, 10, 1024, 1024, 64, 1, None, C, D, 64, E, need, None) == hbl.ERR_NULL
    p = lib.hbl_prepare_weights_mx
    assert p(A, 64, 100, B, None) == hbl.ERR_SHAPE
    assert p(A, 64, 64, B, None) == hbl.ERR_SHAPE      # K % 128
    assert p(None, 64, 256, B, None) == hbl.ERR_NULL
    assert p(A, 64, 256, B + 4, None) == hbl.ERR_ALIGN


def test_kv_quant_errors(hbl):
    lib = hbl.lib()
    q = lib.hbl_kv_quant
    assert q(A, 1, 2, 4, 8, 128, 5, 1, B, C, D, E, None) == hbl.ERR_MODE      # bits
    assert q(A, 3, 2, 4, 8, 128, 4, 1, B, C, D, E, None) == hbl.ERR_MODE      # dtype
    assert q(A, 1, 2, 4, 8, 96, 4, 1, B, C, D, E, None) == hbl.ERR_SHAPE      # D not a power of two
    assert q(A, 1, 2, 4, 8, 4096, 4, 1, B, C, D, E, None) == hbl.ERR_SHAPE    # D above 2048
    assert q(A, 1, 2, 0, 8, 128, 4, 1, B, C, D, E, None) == hbl.ERR_SHAPE     # S
    assert q(A, 1, 2, 4, 8, 128, 4, 1, B, C, None, E, None) == hbl.ERR_NULL   # BOS buffers needed
    assert q(A + 8, 1, 2, 4, 8, 128, 4, 0, B, C, None, None, None) == hbl.ERR_ALIGN
    assert q(A, 1, 0, 4, 8, 128, 4, 1, B, C, D, E, None) == hbl.OK             # B = 0
