"""Readers for the hand-written fixtures under tests/golden/ (each file cites its source)."""
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32(token: str) -> float:
    """A decimal literal rounded to FP32, or an exact FP32 bit pattern written 'bits:0x...'."""
    if token.startswith("bits:"):
        return struct.unpack("<f", struct.pack("<I", int(token[5:], 16)))[0]
    return float(np.float32(float(token)))


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def rows(name: str):
    """Non-comment lines of a fixture, split on whitespace (trailing notes kept as extra tokens)."""
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def int_list(text: str):
    text = text.strip()
    return [int(v) for v in text.split(",")] if text else []


def layernorm_order_key():
    """The key, LayerNorm weights and biases of tests/golden/layernorm_order.txt (FP32 arrays
    holding BF16 values): x0 = 2^24, x8 = -2^24, ones at columns 1..7 and 9..15, zeros after;
    gamma 0.5 at columns 0 and 8, 1.34375 * 2^21 at columns 1..7 and 9..15, 1 elsewhere;
    beta 0."""
    x = np.zeros(128, np.float32)
    x[0], x[8] = 2.0 ** 24, -(2.0 ** 24)
    x[1:8] = 1.0
    x[9:16] = 1.0
    gamma = np.ones(128, np.float32)
    gamma[[0, 8]] = 0.5
    gamma[1:8] = 1.34375 * 2.0 ** 21
    gamma[9:16] = 1.34375 * 2.0 ** 21
    return x, gamma, np.zeros(128, np.float32)


def byte_list(text: str):
    """Comma-separated bytes; 'v*n' repeats v n times."""
    out = []
    for tok in text.split(","):
        v, _, n = tok.partition("*")
        out += [int(v, 0)] * (int(n) if n else 1)
    return out
