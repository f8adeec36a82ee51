"""Seeded synthetic inputs for the H-BitLinear forward (shared by tests,
bench.py and the smoke check).

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no transform, no quantiser, no matmul), so both the
oracle and the GPU path can take their inputs from it.

Shapes follow the model table of the BitNet v2 architecture write-up
(§3.4 "Training Recipe", Table 8: 7B hidden 4096, GLU 16384).  The pages
measure no throughput and use no public benchmark for this path; these inputs
are synthetic stand-ins with the distributions the five workloads name:

  tiny      M=8, K=N=256, fp32 N(0,1) with 4 outlier channels x50, INT4.
  wo_7b     M=2048, K=N=4096, bf16 Student-t(3), 1% channels x20, INT4.
  wdown_7b  M=4096, K=16384, N=4096, bf16 relu(a)^2*b, a,b ~ N(0,1), INT4.
  decode    M in {1,4,16}, (K,N) in {(4096,4096), (16384,4096)}, bf16
            Student-t(3), INT8, distinct weight matrices cycled.
  block_7b  M=65536 (64 x 1024), the seven linears of one 7B block, INT8 and
            INT4; Q/K/V/up/gate plain, Wo/Wdown with the rotation.
Weights are fp32 N(0, 0.02^2) (0.02 read as the standard deviation).

Generation: numpy PCG64.  Large arrays are drawn in chunks of 4096 rows, each
chunk from its own stream ``default_rng([seed, stream, chunk])`` so that chunks
can be drawn in parallel threads and any row can be regenerated alone.
Student-t(3) is drawn with ``standard_t(3)``.  bf16 inputs are the fp32 draws
rounded to nearest-even and stored as uint16 bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

CHUNK = 4096
W_STD = 0.02

SEEDS = {"tiny": 0, "wo_7b": 1, "wdown_7b": 2, "decode": 3, "block_7b": 4}

# (name, K, N, hadamard) for the seven linears of one 7B block
BLOCK_7B_LAYERS = [
    ("q", 4096, 4096, False),
    ("k", 4096, 4096, False),
    ("v", 4096, 4096, False),
    ("o", 4096, 4096, True),
    ("up", 4096, 16384, False),
    ("gate", 4096, 16384, False),
    ("down", 16384, 4096, True),
]
# the four distinct activation inputs of the block and which layers read them
BLOCK_7B_INPUTS = [("attn_in", 4096), ("o_in", 4096), ("ffn_in", 4096), ("down_in", 16384)]
BLOCK_7B_INPUT_OF = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
                     "up": "ffn_in", "gate": "ffn_in", "down": "down_in"}

CONFIGS = {
    "tiny": dict(M=8, K=256, N=256, bits=4, hadamard=True, x_dtype="f32"),
    "wo_7b": dict(M=2048, K=4096, N=4096, bits=4, hadamard=True, x_dtype="bf16"),
    "wdown_7b": dict(M=4096, K=16384, N=4096, bits=4, hadamard=True, x_dtype="bf16"),
    "decode": dict(Ms=(1, 4, 16), shapes=((4096, 4096), (16384, 4096)), bits=8,
                   hadamard=True, x_dtype="bf16", n_mats=10),
    "block_7b": dict(M=65536, layers=BLOCK_7B_LAYERS, bits=(8, 4), x_dtype="bf16"),
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rows_parallel(M: int, K: int, fill, dtype) -> np.ndarray:
    out = np.empty((M, K), dtype)
    chunks = [(c, c * CHUNK, min(M, (c + 1) * CHUNK)) for c in range((M + CHUNK - 1) // CHUNK)]

    def job(t):
        c, a, b = t
        out[a:b] = fill(c, b - a)

    if len(chunks) == 1:
        job(chunks[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, chunks))
    return out


def outlier_channels(seed: int, stream: int, K: int, n_out: int) -> np.ndarray:
    rng = np.random.default_rng([seed, stream, 1 << 20])
    return np.sort(rng.choice(K, n_out, replace=False))


def student_t_rows(seed: int, stream: int, M: int, K: int, out_frac: float | None,
                   factor: float, as_bf16: bool = True) -> np.ndarray:
    """Student-t(3) activations; ``round(out_frac*K)`` channels (the same
    columns for every token) multiplied by ``factor``."""
    cols = None
    if out_frac:
        cols = outlier_channels(seed, stream, K, int(round(out_frac * K)))

    def fill(c, rows):
        rng = np.random.default_rng([seed, stream, c])
        a = rng.standard_t(3, size=(rows, K)).astype(np.float32)
        if cols is not None:
            a[:, cols] *= np.float32(factor)
        return bf16_bits(a) if as_bf16 else a

    return _rows_parallel(M, K, fill, np.uint16 if as_bf16 else np.float32)


def relu2_gated_rows(seed: int, stream: int, M: int, K: int) -> np.ndarray:
    """bf16 relu(a)^2 * b with a, b ~ N(0,1) iid (squared-ReLU gating)."""

    def fill(c, rows):
        rng = np.random.default_rng([seed, stream, c])
        a = rng.standard_normal((rows, K), dtype=np.float32)
        b = rng.standard_normal((rows, K), dtype=np.float32)
        r = np.maximum(a, np.float32(0))
        return bf16_bits(r * r * b)

    return _rows_parallel(M, K, fill, np.uint16)


def gaussian_weights(seed: int, stream: int, N: int, K: int) -> np.ndarray:
    def fill(c, rows):
        rng = np.random.default_rng([seed, stream, c])
        return (rng.standard_normal((rows, K), dtype=np.float64) * W_STD).astype(np.float32)

    return _rows_parallel(N, K, fill, np.float32)


def tiny():
    """M=8, K=N=256: fp32 N(0,1) with 4 outlier channels x50; seed 0."""
    s = SEEDS["tiny"]
    cfg = CONFIGS["tiny"]
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    rng = np.random.default_rng(s)
    x = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, 4, replace=False)
    x[:, cols] *= np.float32(50.0)
    w = (rng.standard_normal((N, K)) * W_STD).astype(np.float32)
    return dict(cfg, x=x, w=w)


def wo_7b():
    s = SEEDS["wo_7b"]
    cfg = CONFIGS["wo_7b"]
    x = student_t_rows(s, 0, cfg["M"], cfg["K"], 0.01, 20.0)
    w = gaussian_weights(s, 1, cfg["N"], cfg["K"])
    return dict(cfg, x=x, w=w)


def wdown_7b():
    s = SEEDS["wdown_7b"]
    cfg = CONFIGS["wdown_7b"]
    x = relu2_gated_rows(s, 0, cfg["M"], cfg["K"])
    w = gaussian_weights(s, 1, cfg["N"], cfg["K"])
    return dict(cfg, x=x, w=w)


def decode_inputs(K: int, M: int) -> np.ndarray:
    """bf16 Student-t(3) decode activations (no outlier channels)."""
    return student_t_rows(SEEDS["decode"], 100 + K // 1024 + M, M, K, None, 1.0)


def decode_weights(K: int, N: int, index: int) -> np.ndarray:
    return gaussian_weights(SEEDS["decode"], 1000 + 64 * (K // 1024) + index, N, K)


def block_input(name: str, M: int | None = None) -> np.ndarray:
    """One of the four bf16 activation inputs of the 7B block (first M rows)."""
    K = dict(BLOCK_7B_INPUTS)[name]
    stream = [n for n, _ in BLOCK_7B_INPUTS].index(name)
    M = CONFIGS["block_7b"]["M"] if M is None else M
    return student_t_rows(SEEDS["block_7b"], stream, M, K, 0.01, 20.0)


def block_weights(layer: str) -> np.ndarray:
    names = [n for n, *_ in BLOCK_7B_LAYERS]
    _, K, N, _ = BLOCK_7B_LAYERS[names.index(layer)]
    return gaussian_weights(SEEDS["block_7b"], 10 + names.index(layer), N, K)


def random_rows(seed: int, M: int, K: int, kind: str = "t3", as_bf16: bool = True) -> np.ndarray:
    """Small ad-hoc inputs for edge-case tests."""
    rng = np.random.default_rng(seed)
    if kind == "t3":
        a = rng.standard_t(3, size=(M, K)).astype(np.float32)
    elif kind == "normal":
        a = rng.standard_normal((M, K)).astype(np.float32)
    else:
        raise ValueError(kind)
    return bf16_bits(a) if as_bf16 else a
