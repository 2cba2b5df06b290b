"""Pins of the oracle's scalar formats against hand-worked values, exact rationals and
library conversions (torch CPU bfloat16 / float8_e4m3fn). No GPU needed."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from goldens import f32, f32_bits, rows


def test_e2m1_golden():
    # tests/golden/e2m1_encode.txt: grid, midpoints, saturation, signed zero.
    n = 0
    for line in rows("e2m1_encode.txt"):
        tok = line.split()
        assert oracle.e2m1_encode(f32(tok[0])) == int(tok[1]), line
        n += 1
    assert n >= 35


def test_e2m1_table_matches_field_definition():
    # E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0, subnormal at exponent 0.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = 0.5 * m if e == 0 else (1 + 0.5 * m) * 2.0 ** (e - 1)
        v = oracle.e2m1_value(c)
        assert v == (-mag if s else mag) and np.signbit(v) == bool(s)


def _e2m1_thresholds(x: float) -> int:
    # Same rounding stated as decision thresholds between neighbouring grid values, with the tie
    # at each midpoint going to the even code: an independent form of nearest-even + satfinite.
    m = abs(x)
    code = int(m > 0.25) + int(m >= 0.75) + int(m > 1.25) + int(m >= 1.75) + int(m > 2.5) \
        + int(m >= 3.5) + int(m > 5.0)
    return code | (8 if np.signbit(x) else 0)


def test_e2m1_exhaustive_bf16_sweep():
    # Every finite BF16 value (the inputs are BF16 or BF16-rounded).
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << np.uint32(16)).view(np.float32)
    fails = 0
    for v in vals[np.isfinite(vals)]:
        fails += oracle.e2m1_encode(float(v)) != _e2m1_thresholds(float(v))
    assert fails == 0


def test_e2m1_fp32_near_midpoints():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    for m in mids:
        b = f32_bits(m)
        for d in range(-40, 41):
            for sgn in (1.0, -1.0):
                x = sgn * f32(f"bits:0x{b + d:08X}")
                assert oracle.e2m1_encode(x) == _e2m1_thresholds(x), (x, d)


def test_ue8m0_golden():
    for line in rows("ue8m0.txt"):
        tok = line.split()
        assert oracle.ue8m0_byte(f32(tok[0])) == int(tok[1]), line


def test_ue8m0_powers_of_two():
    # amax = 2^k needs 6 * 2^e >= 2^k, i.e. e = k - 2 (1.5 * 2^k >= 2^k > 0.75 * 2^k), for every
    # k at which 2^k is at least the floor 6 * 2^-126 = 1.5 * 2^-124.
    for k in range(-123, 128):
        assert oracle.ue8m0_exponent(float(2.0 ** k)) == k - 2, k


def _ue8m0_exact(a: float) -> int:
    # Exact rationals: the e with 6 * 2^(e-1) < max(a, 6 * 2^-126) <= 6 * 2^e.
    t = max(Fraction(a), 6 * Fraction(2) ** -126)
    e = 0
    while 6 * Fraction(2) ** e < t:
        e += 1
    while 6 * Fraction(2) ** (e - 1) >= t:
        e -= 1
    return e


def test_ue8m0_random_vs_exact_rationals():
    rng = np.random.default_rng(11)
    mant = rng.uniform(1.0, 2.0, size=3000).astype(np.float32)
    expo = rng.integers(-130, 127, size=3000)
    vals = [float(np.float32(m) * np.float32(2.0) ** int(e)) if -126 <= e else float(np.ldexp(np.float32(m), int(e)))
            for m, e in zip(mant, expo)]
    for k in range(-120, 120, 7):  # neighbours of 6 * 2^k
        b = f32_bits(6.0 * 2.0 ** k)
        vals += [f32(f"bits:0x{b - 1:08X}"), f32(f"bits:0x{b:08X}"), f32(f"bits:0x{b + 1:08X}")]
    for v in vals:
        if np.isfinite(v):
            assert oracle.ue8m0_exponent(v) == _ue8m0_exact(v), v


def test_pow2_ceil_properties():
    rng = np.random.default_rng(12)
    xs = np.abs(rng.standard_normal(2000).astype(np.float32)) * np.float32(2.0) ** rng.integers(-60, 60, 2000)
    xs = [float(x) for x in xs if x > 0] + [1.0, 0.5, 2.0 ** -42, 1.0000001, 0.99999994]
    for x in xs:
        p = oracle.pow2_ceil(x)
        m, _ = np.frexp(p)
        assert m == 0.5 and Fraction(p) >= Fraction(x) and Fraction(p) / 2 < Fraction(x), x


def test_e4m3_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v)
        else:
            assert v == ref[c] and np.signbit(v) == np.signbit(ref[c]), c


def test_e4m3_encode_matches_torch_float8_below_464():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even; it returns NaN at 464 and above
    # instead of saturating, so the sweep stops below the 464 tie (saturation is pinned by golden).
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << np.uint32(16)).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 464)]
    ref = torch.from_numpy(vals.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref)
    # FP32 values around every E4M3 midpoint as well
    mids = []
    for c in range(0x7E):
        a, b = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mb = f32_bits((a + b) / 2)
        mids += [f32(f"bits:0x{mb + d:08X}") for d in (-2, -1, 0, 1, 2)]
    mids = np.array(mids + [-m for m in mids], dtype=np.float32)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in mids], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    ties = ((rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 17) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], -ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.bf16_round(float(v)) for v in x], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_head_weight_scale_golden_and_nearest():
    for line in rows("head_weight_scale.txt"):
        h, b = line.split()[:2]
        c = oracle.head_weight_scale(int(h))
        assert f32_bits(c) == int(b, 16), line
        # c is the FP32 value nearest to (128 H)^-1/2: the midpoints to its neighbours bracket it.
        n = 128 * int(h)
        lo = Fraction(f32(f"bits:0x{f32_bits(c) - 1:08X}"))
        hi = Fraction(f32(f"bits:0x{f32_bits(c) + 1:08X}"))
        cf = Fraction(c)
        assert ((lo + cf) / 2) ** 2 * n < 1 < ((cf + hi) / 2) ** 2 * n


@pytest.mark.parametrize("kind", ["scale", "e4m3", "fold"])
def test_fp8_query_golden(kind):
    # Scale and fold cases go through the oracle's FP8 quantize_queries on a crafted head:
    # one element carries the amax, w_out = BF16((wv * s) * c_32) with c_32 = 2^-6.
    for line in rows("fp8_query.txt"):
        tok = line.split()
        if tok[0] != kind:
            continue
        if kind == "e4m3":
            assert oracle.e4m3_encode(f32(tok[1])) == int(tok[2], 16), line
            continue
        if kind == "scale":
            amax, want_s, wv = f32(tok[1]), f32(tok[2]), 1.0
        else:
            wv, want_s, heads, want_w = f32(tok[1]), f32(tok[2]), int(tok[3]), f32(tok[4])
            amax = 448.0 * want_s
        q = np.zeros((1, 32, 128), dtype=np.float32)
        q[0, 5, 17] = amax
        qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert float(torch.from_numpy(q[0, 5, 17:18]).to(torch.bfloat16)) == amax
        wvb = torch.full((1, 32), wv, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        out, w_out = oracle.quantize_queries(qb, wvb, "fp8")
        s = float(torch.from_numpy(w_out.view(np.int16)).view(torch.bfloat16)[0, 5].float()) / wv * 64
        assert s == want_s, line
        if kind == "fold":
            got = float(torch.from_numpy(w_out.view(np.int16)).view(torch.bfloat16)[0, 5].float())
            assert got == want_w, line
        # the amax element is stored as 448 * amax / (448 s) = amax / s exactly when representable
        if amax > 0:
            assert out[0, 5 * 128 + 17] == oracle.e4m3_encode(amax / want_s)
