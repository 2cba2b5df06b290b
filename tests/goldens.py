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
