"""Exhaustive sweeps of the gfx950 conversions the quantizers rely on, through the C-ABI,
byte for byte against the oracle's table encoders.

- MXFP4 queries (E2M1 codes from the BF16 scaled conversion at scale 2^e): every finite BF16
  pattern at every UE8M0 exponent e in [-126, 126] for which the pattern can sit in a block
  of exponent e (|x| <= the block's largest magnitude), in blocks whose largest magnitude is
  set to fix e (page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index",
  mxfp4_scale, e2m1x2, quantize_fp4_query).
- FP8 queries (E4M3 codes of x * (1 / s)): every finite BF16 pattern at every power-of-two
  head scale s = 2^k a head can have, k in [-42, 120] (same page, DsaIndex.fp8_query).
- Keys (the FP32 E2M1 and E4M3 conversions after the LayerNorm): with gamma = 0 the
  LayerNorm output is beta itself, so beta drives the key quantizers directly: every finite
  BF16 value at a spread of block exponents (MXFP4) and key scales (FP8) (insert_key,
  insert_fp4_key).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_quant_amd as dsa
from gpu_util import bf16_dev, dev
from sparse_attention_indexer_quant_amd.workloads import bf16_to_f32

pytestmark = pytest.mark.gpu

MAX_BF16 = 0x7F7F  # largest finite BF16 (1.9921875 * 2^127)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def _bits(x: float) -> int:
    """BF16 bits of a value that BF16 holds exactly."""
    u = int(np.array([x], np.float32).view(np.uint32)[0])
    assert u & 0xFFFF == 0, x
    return u >> 16


def _blocks(values: np.ndarray, setter: int, size: int, rng) -> np.ndarray:
    """values (BF16 bits) packed size - 1 to a block with the setter (the block's largest
    magnitude) at a random place in each block; the last block padded with zeros."""
    per = size - 1
    n = -(-values.size // per)
    body = np.zeros(n * per, np.uint16)
    body[:values.size] = values
    blk = np.concatenate([body.reshape(n, per), np.full((n, 1), setter, np.uint16)], axis=1)
    return rng.permuted(blk, axis=1)


def _mxfp4_sweep_rows(heads=64):
    fin = _finite_bf16()
    mag = np.abs(bf16_to_f32(fin).astype(np.float64))
    rng = np.random.default_rng(71)
    blocks = []
    for e in range(-126, 127):
        # 6 * 2^e is the largest amax of exponent e; at e = 126 it is beyond FP32, and the
        # largest finite BF16 (M = 1.99 > 1.5, so e = 127 - 2 + 1) fixes e instead
        setter = _bits(6.0 * 2.0 ** e) if e <= 125 else MAX_BF16
        lim = float(bf16_to_f32(np.array([setter], np.uint16))[0])
        blocks.append(_blocks(fin[mag <= lim], setter, 32, rng))
    blk = np.concatenate(blocks)
    per_row = heads * 4
    rows = -(-blk.shape[0] // per_row)
    q = np.zeros((rows * per_row, 32), np.uint16)
    q[:blk.shape[0]] = blk
    return q.reshape(rows, heads, 128), int(sum(b.shape[0] for b in blocks))


def _fp8_sweep_rows(heads=64):
    fin = _finite_bf16()
    mag = np.abs(bf16_to_f32(fin).astype(np.float64))
    rng = np.random.default_rng(72)
    heads_ = []
    for k in range(-42, 121):
        # amax = 448 * 2^k gives s = 2^k exactly; k = 120 needs amax above 448 * 2^119, which
        # only the largest BF16 values reach
        setter = _bits(448.0 * 2.0 ** k) if k <= 119 else MAX_BF16
        lim = float(bf16_to_f32(np.array([setter], np.uint16))[0])
        heads_.append(_blocks(fin[mag <= lim], setter, 128, rng))
    hd = np.concatenate(heads_)
    rows = -(-hd.shape[0] // heads)
    q = np.zeros((rows * heads, 128), np.uint16)
    q[:hd.shape[0]] = hd
    return q.reshape(rows, heads, 128)


def test_mxfp4_query_every_bf16_at_every_exponent():
    q, nblocks = _mxfp4_sweep_rows()
    assert nblocks > 250_000  # ~8.4 M values: every reachable (pattern, exponent) pair
    wv = np.zeros(q.shape[:2], np.uint16)
    want, _ = oracle.quantize_queries(q, wv, "mxfp4")
    got, _ = dsa.quantize_queries(bf16_dev(q), bf16_dev(wv), "mxfp4")
    got = got.cpu().numpy()
    heads = q.shape[1]
    # every block's UE8M0 byte is the exponent its setter fixes
    scales = want[:, heads * 64:].reshape(-1)
    assert scales.min() == 1 and scales.max() == 253
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at rows {bad[0][:4]} cols {bad[1][:4]}"


def test_fp8_query_every_bf16_at_every_scale():
    q = _fp8_sweep_rows()
    wv = np.full(q.shape[:2], _bits(1.0), np.uint16)
    want, want_w = oracle.quantize_queries(q, wv, "fp8")
    got, got_w = dsa.quantize_queries(bf16_dev(q), bf16_dev(wv), "fp8")
    got = got.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} bytes differ, first at rows {bad[0][:4]} cols {bad[1][:4]}"
    gw = got_w.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gw, want_w)  # the weights carry every scale 2^-42 .. 2^120 folded


def _key_sweep_betas(fmt):
    """beta vectors (FP32 holding BF16 values) that, with gamma = 0, are the LayerNorm output:
    every finite BF16 value no larger than the block's (or key's) amax, at a spread of MXFP4
    block exponents or FP8 key scales."""
    fin = _finite_bf16()
    mag = np.abs(bf16_to_f32(fin).astype(np.float64))
    rng = np.random.default_rng(73)
    out = []
    if fmt == "mxfp4":
        for e in (-126, -100, -60, -2, 0, 1, 60, 125, 126):
            setter = _bits(6.0 * 2.0 ** e) if e <= 125 else MAX_BF16
            lim = float(bf16_to_f32(np.array([setter], np.uint16))[0])
            out.append(_blocks(fin[mag <= lim], setter, 32, rng))
        blk = np.concatenate(out)
        n = -(-blk.shape[0] // 4)
        b = np.zeros((n * 4, 32), np.uint16)
        b[:blk.shape[0]] = blk
        return bf16_to_f32(b.reshape(n, 128))
    for k in (-42, -9, 0, 7, 60, 119, 120):
        setter = _bits(448.0 * 2.0 ** k) if k <= 119 else MAX_BF16
        lim = float(bf16_to_f32(np.array([setter], np.uint16))[0])
        out.append(_blocks(fin[mag <= lim], setter, 128, rng))
    return bf16_to_f32(np.concatenate(out))


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_key_quantizers_every_bf16_value(fmt):
    betas = _key_sweep_betas(fmt)
    n = betas.shape[0]
    section = 4352 if fmt == "mxfp4" else 8448
    rng = np.random.default_rng(74)
    key = rng.standard_normal((2, 128)).astype(np.float32)
    key_bits = (key.view(np.uint32) >> 16).astype(np.uint16)  # BF16 by truncation: any values do
    gamma = np.zeros(128, np.float32)
    pages = -(-n // 64)
    slots = np.arange(n, dtype=np.int64)
    want = np.zeros(pages * section, np.uint8)
    got = torch.zeros(pages * section, dtype=torch.uint8, device="cuda")
    betas_dev = dev(betas)
    g_dev = dev(gamma)
    kd = bf16_dev(key_bits)
    # one key per call (beta is shared by a call's keys); odd calls take the one-wavefront
    # kernel through a key row that is not 16-byte aligned
    wide = torch.zeros((1, 130), dtype=torch.bfloat16, device="cuda")
    wide[0, 2:] = kd[1]
    slots_dev = dev(slots)
    for i in range(n):
        oracle.store_keys(key_bits[i % 2:i % 2 + 1], gamma, betas[i], 1e-6, slots[i:i + 1], want,
                          pages, section, 0, fmt)
        keys = kd[0:1] if i % 2 == 0 else wide[:, 2:]
        dsa.store_keys(keys, g_dev, betas_dev[i], 1e-6, slots_dev[i:i + 1], got, pages, section, fmt)
    got = got.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4]} (key {bad[:4] // section * 64})"
