"""Independent NumPy decoders of the quantized formats, written from the bit fields
(not from lookup tables), used to pin byte layouts and the brute-force scores.

Layouts (page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index", module
text and insert_fp4_key; page "vllm.models.kimi_k3.amd.ops.fp4_indexer", cache_views):
  MXFP4 query row  [H x 64 B E2M1 | H x 4 B UE8M0]
  MXFP4 key section [64 tokens x 64 B E2M1 | 64 tokens x 4 B UE8M0]   (4352 B)
  FP8 key section   [64 tokens x 128 B E4M3 | 64 tokens x 4 B FP32]    (8448 B)
  FP8 mx section    [64 tokens x 128 B E4M3 | 64 tokens x 4 equal UE8M0 bytes]
Byte j of a 128-value vector holds column 2j in its low nibble, 2j+1 in its high nibble;
scale byte g covers columns [32g, 32g + 32).
"""
import numpy as np


def e2m1(nibbles) -> np.ndarray:
    n = np.asarray(nibbles, dtype=np.int64)
    sign = np.where(n & 8, -1.0, 1.0)
    e = (n >> 1) & 3
    m = n & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e4m3(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def unpack_nibbles(payload: np.ndarray) -> np.ndarray:
    """[..., 64] bytes -> [..., 128] nibbles, column 2j from the low nibble of byte j."""
    p = np.asarray(payload, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mxfp4_vector(payload64: np.ndarray, scales4: np.ndarray) -> np.ndarray:
    vals = e2m1(unpack_nibbles(payload64))
    sc = np.exp2(np.asarray(scales4, dtype=np.float64) - 127.0)
    return vals * np.repeat(sc, 32, axis=-1)


def mxfp4_query_rows(q_rows: np.ndarray, heads: int) -> np.ndarray:
    """uint8 [rows, >= 68 H] -> float64 [rows, H, 128]."""
    q = np.asarray(q_rows, dtype=np.uint8)
    rows = q.shape[0]
    payload = q[:, :heads * 64].reshape(rows, heads, 64)
    scales = q[:, heads * 64:heads * 68].reshape(rows, heads, 4)
    return mxfp4_vector(payload, scales)


def fp8_query_rows(q_rows: np.ndarray, heads: int) -> np.ndarray:
    q = np.asarray(q_rows, dtype=np.uint8)
    return e4m3(q[:, :heads * 128].reshape(q.shape[0], heads, 128))


def mxfp4_key(cache: np.ndarray, page: int, slot: int, page_stride: int, offset: int = 0):
    base = offset + page * page_stride
    payload = cache[base + slot * 64: base + slot * 64 + 64]
    scales = cache[base + 4096 + slot * 4: base + 4096 + slot * 4 + 4]
    return mxfp4_vector(payload, scales)


def fp8_key(cache: np.ndarray, page: int, slot: int, page_stride: int, offset: int = 0):
    base = offset + page * page_stride
    vals = e4m3(cache[base + slot * 128: base + slot * 128 + 128])
    scale = np.frombuffer(cache[base + 8192 + slot * 4: base + 8192 + slot * 4 + 4].tobytes(),
                          dtype="<f4")[0]
    return vals * float(scale), float(scale)


def fp8_mx_key(cache: np.ndarray, page: int, slot: int, page_stride: int, offset: int = 0):
    """FP8 key whose scale 2^e is stored as four UE8M0 bytes e + 127; returns (values,
    scale, the four bytes)."""
    base = offset + page * page_stride
    vals = e4m3(cache[base + slot * 128: base + slot * 128 + 128])
    sb = cache[base + 8192 + slot * 4: base + 8192 + slot * 4 + 4].astype(np.int64)
    scale = float(np.exp2(sb[0] - 127.0))
    return vals * scale, scale, sb


def bf16(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
