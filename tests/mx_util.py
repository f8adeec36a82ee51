"""Host-side encoders and decoders of the MX6 code and MX4 weight layouts of
the FP6 x FP4 path (include/hbl.h), for the tests.  They follow the layout
contract and the OCP MX element formats (E3M2: sign, 3 exponent bits with
bias 3, 2 mantissa bits; E2M1: sign, 2 exponent bits with bias 1, 1
mantissa bit) and share nothing with the library."""
from __future__ import annotations

import numpy as np


def e3m2_value(code: int) -> float:
    """The value of a 6-bit E3M2 code, from the format's definition."""
    s, e, m = (code >> 5) & 1, (code >> 2) & 7, code & 3
    mag = 2.0 ** (e - 3) * (1 + m / 4) if e > 0 else 2.0 ** (1 - 3) * (m / 4)
    return -mag if s else mag


def e2m1_value(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 2.0 ** (e - 1) * (1 + m / 2) if e > 0 else 2.0 ** (1 - 1) * (m / 2)
    return -mag if s else mag


# integer -> code tables, found by search over the formats (not typed in)
E3M2_OF = {int(e3m2_value(c)): c for c in range(64) if e3m2_value(c) == int(e3m2_value(c)) and -8 <= e3m2_value(c) <= 8
           and not (e3m2_value(c) == 0 and c != 0)}
E2M1_OF = {int(e2m1_value(c)): c for c in range(16) if e2m1_value(c) in (-1.0, 0.0, 1.0) and not (e2m1_value(c) == 0 and c != 0)}
E3M2_TABLE = np.array([e3m2_value(c) for c in range(64)])


def _mx6_offsets(M, K: int):
    """Byte offsets of the first 16 and the last 8 bytes of the 192-bit field
    of (row m, group g) in the tiled MX6 buffer, [rows][K/32] each, for rows
    0 .. M - 1 (M an int) or the given row indices."""
    m = (np.arange(M, dtype=np.int64) if np.isscalar(M) else np.asarray(M, np.int64))[:, None]
    g = np.arange(K // 32, dtype=np.int64)[None, :]
    tile = (m >> 8) * (K // 128) + (g >> 2)
    r, gi = m & 255, g & 3
    main = tile * 24576 + 16 * (4 * r + (gi ^ ((r >> 2) & 3)))
    tail = tile * 24576 + 16384 + 16 * (2 * r + ((gi >> 1) ^ ((r >> 3) & 1))) + 8 * (gi & 1)
    return main, tail


def encode_mx6(q: np.ndarray) -> np.ndarray:
    """int8 codes [M][K] in [-8, 7] (K % 128 == 0) -> the tiled MX6 buffer,
    uint8 [ceil(M/256)*256][3K/4] (padding rows zero)."""
    M, K = q.shape
    Mp = (M + 255) // 256 * 256
    lut = np.array([E3M2_OF[v] for v in range(-8, 8)], np.uint8)
    c6 = lut[q.astype(np.int64) + 8].reshape(M, K // 32, 32)   # 6-bit codes
    # the 192-bit field of each group, code e at bits 6 e .. 6 e + 5
    bits = ((c6[:, :, :, None] >> np.arange(6, dtype=np.uint8)) & 1).reshape(M, K // 32, 192)
    field = np.packbits(bits, axis=2, bitorder="little")        # [M][K/32][24]
    out = np.zeros(Mp * (K // 4 * 3), np.uint8)
    main, tail = _mx6_offsets(M, K)
    for j in range(16):
        out[main + j] = field[:, :, j]
    for j in range(8):
        out[tail + j] = field[:, :, 16 + j]
    return out.reshape(Mp, K // 4 * 3)


def decode_mx6(b: np.ndarray, K: int, M=None) -> np.ndarray:
    """The tiled MX6 buffer -> values [rows][K] (float64, from the E3M2
    definition) of rows 0 .. M - 1, or of the row indices M; M defaults to
    the buffer's (padded) rows."""
    flat = np.ascontiguousarray(b).reshape(-1)
    M = M if M is not None else flat.size // (K // 4 * 3)
    main, tail = _mx6_offsets(M, K)
    M = main.shape[0]
    field = np.concatenate([flat[main[:, :, None] + np.arange(16)], flat[tail[:, :, None] + np.arange(8)]], axis=2)
    bits = np.unpackbits(field, axis=2, bitorder="little").reshape(M, K // 32, 32, 6).astype(np.int64)
    code = (bits << np.arange(6)).sum(axis=3)
    return E3M2_TABLE[code].reshape(M, K)


def _ternary_words(q: np.ndarray) -> np.ndarray:
    """Ternary codes int8 [N][K] -> the 32-bit words [N][K/16] of the MX4
    encoding, before tiling."""
    N, K = q.shape
    g = q.reshape(N, K // 16, 16).astype(np.int64)
    nz = (g != 0).astype(np.uint32)
    neg = (g < 0).astype(np.uint32)
    w = np.zeros((N, K // 16), np.uint32)
    for n in range(8):
        w |= nz[:, :, n] << np.uint32(4 * n + 1)
        w |= neg[:, :, n] << np.uint32(4 * n + 3)
        w |= nz[:, :, 8 + n] << np.uint32(4 * n)
        w |= neg[:, :, 8 + n] << np.uint32(4 * n + 2)
    return w


def _mx4_word_index(N: int, K: int) -> np.ndarray:
    """Word index in the tiled MX4 buffer of (row n, word c): [N][K/16]."""
    n = np.arange(N, dtype=np.int64)[:, None]
    c = np.arange(K // 16, dtype=np.int64)[None, :]
    tile = (n >> 7) * (K // 128) + (c >> 3)
    r, u, wi = n & 127, (c >> 2) & 1, c & 3
    return tile * 1024 + 4 * (2 * r + (u ^ ((r >> 3) & 1))) + wi


def encode_mx4(q: np.ndarray) -> np.ndarray:
    """Ternary codes int8 [N][K] (K % 128 == 0) -> the tiled MX4 buffer,
    uint32 [ceil(N/128)*128][K/16] (rows past N zero)."""
    N, K = q.shape
    Np = (N + 127) // 128 * 128
    out = np.zeros(Np * (K // 16), np.uint32)
    out[_mx4_word_index(N, K)] = _ternary_words(q)
    return out.reshape(Np, K // 16)


def decode_mx4(w: np.ndarray, K: int, N: int | None = None) -> np.ndarray:
    """The tiled MX4 buffer -> ternary values [N][K] via the E2M1 codes of
    the two halves of each word; N defaults to the buffer's rows."""
    flat = np.ascontiguousarray(w).reshape(-1).view(np.uint32)
    N = N if N is not None else flat.size // (K // 16)
    words = flat[_mx4_word_index(N, K)]
    out = np.zeros((N, K // 16, 16))
    lo = words & np.uint32(0xAAAAAAAA)
    hi = (words << np.uint32(1)) & np.uint32(0xAAAAAAAA)
    tab = np.array([e2m1_value(c) for c in range(16)])
    for n in range(8):
        out[:, :, n] = tab[(lo >> np.uint32(4 * n)) & np.uint32(15)]
        out[:, :, 8 + n] = tab[(hi >> np.uint32(4 * n)) & np.uint32(15)]
    return out.reshape(N, K)
