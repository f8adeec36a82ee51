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


def encode_mx6(q: np.ndarray) -> np.ndarray:
    """int8 codes [M][K] in [-8, 7] (K % 128 == 0) -> MX6 bytes [M][3K/4]."""
    M, K = q.shape
    lut = np.array([E3M2_OF[v] for v in range(-8, 8)], np.uint64)
    c6 = lut[q.astype(np.int64) + 8]                      # [M][K] 6-bit codes
    g = c6.reshape(M, K // 32, 32)
    out = np.zeros((M, K // 128, 96), np.uint8)
    for gi in range(4):
        grp = g[:, gi::4, :]                               # group gi of each block
        # the 192-bit field as 24 bytes, code e at bits 6 e .. 6 e + 5
        bits = np.zeros((M, K // 128, 24), np.uint8)
        for e in range(32):
            v = grp[:, :, e].astype(np.uint64)
            pos = 6 * e
            for b in range(6):
                bit = ((v >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
                p = pos + b
                bits[:, :, p // 8] |= (bit << (p % 8)).astype(np.uint8)
        out[:, :, 16 * gi:16 * gi + 16] = bits[:, :, :16]
        out[:, :, 64 + 8 * gi:64 + 8 * gi + 8] = bits[:, :, 16:]
    return out.reshape(M, K // 4 * 3)


def decode_mx6(b: np.ndarray, K: int) -> np.ndarray:
    """MX6 bytes [M][3K/4] -> values [M][K] (float64, from the E3M2 definition)."""
    M = b.shape[0]
    blk = b.reshape(M, K // 128, 96)
    out = np.zeros((M, K // 128, 4, 32))
    for gi in range(4):
        field = np.concatenate([blk[:, :, 16 * gi:16 * gi + 16], blk[:, :, 64 + 8 * gi:64 + 8 * gi + 8]], axis=2)
        bits = np.unpackbits(field, axis=2, bitorder="little")  # [M][blocks][192]
        for e in range(32):
            code = np.zeros((M, K // 128), np.int64)
            for j in range(6):
                code |= bits[:, :, 6 * e + j].astype(np.int64) << j
            out[:, :, gi, e] = E3M2_TABLE[code]
    return out.reshape(M, K)


def encode_mx4(q: np.ndarray) -> np.ndarray:
    """Ternary codes int8 [N][K] (K % 16 == 0) -> MX4 words uint32 [N][K/16]."""
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


def decode_mx4(w: np.ndarray, K: int) -> np.ndarray:
    """MX4 words -> ternary values [N][K] via the E2M1 codes of the halves."""
    N = w.shape[0]
    out = np.zeros((N, K // 16, 16))
    lo = w & np.uint32(0xAAAAAAAA)
    hi = (w << np.uint32(1)) & np.uint32(0xAAAAAAAA)
    tab = np.array([e2m1_value(c) for c in range(16)])
    for n in range(8):
        out[:, :, n] = tab[(lo >> np.uint32(4 * n)) & np.uint32(15)]
        out[:, :, 8 + n] = tab[(hi >> np.uint32(4 * n)) & np.uint32(15)]
    return out.reshape(N, K)
