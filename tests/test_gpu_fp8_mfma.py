"""Why the FP8 scoring path widens E4M3 to BF16 for the matrix instruction: the scaled FP8
instruction rounds small terms away next to a large product of the same block, the BF16 one
(fed the same values, exactly representable in BF16) sums them exactly. Probe kernels in
tests/probes (one 16 x 16 tile over K = 128; every lane holds the same 32 values, so every
element is 4 times the pattern's dot product). Re-runnable evidence for that choice: if the FP8
instruction ever summed these cases exactly, the first test fails and says so."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_indexer_quant_amd.workloads import bf16_bits

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libmfma_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE)
    for f in (lib.probe_fp8_scaled_tile, lib.probe_bf16_tile):
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        f.restype = ctypes.c_int
    return lib


def _run(lib, p, q):
    """Both instructions on per-lane patterns p, q (32 values each, E4M3- and BF16-exact)."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    a8 = np.array([oracle.e4m3_encode(v) for v in p], np.uint8)
    b8 = np.array([oracle.e4m3_encode(v) for v in q], np.uint8)
    assert np.array_equal([oracle.e4m3_value(c) for c in a8], p), "pattern must be E4M3 values"
    assert np.array_equal([oracle.e4m3_value(c) for c in b8], q), "pattern must be E4M3 values"
    a16 = bf16_bits(p.astype(np.float32))
    b16 = bf16_bits(q.astype(np.float32))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(np.tile(x, 64))).cuda()
    out8 = torch.zeros(256, dtype=torch.float32, device="cuda")
    out16 = torch.zeros(256, dtype=torch.float32, device="cuda")
    A8, B8 = dev(a8), dev(b8)
    A16, B16 = dev(a16.view(np.int16)), dev(b16.view(np.int16))
    assert lib.probe_fp8_scaled_tile(A8.data_ptr(), B8.data_ptr(), out8.data_ptr()) == 0
    assert lib.probe_bf16_tile(A16.data_ptr(), B16.data_ptr(), out16.data_ptr()) == 0
    exact = 4.0 * float(np.dot(p, q))
    return out8.cpu().numpy().astype(np.float64), out16.cpu().numpy().astype(np.float64), exact


# patterns whose exact sums FP32 holds; each pairs a large product with small terms of one block
CASES = {
    "448^2 + 1": ([448.0, 1.0] + [0.0] * 30, [448.0, 1.0] + [0.0] * 30),
    "448^2 - 448^2 + 1": ([448.0, 448.0, 1.0] + [0.0] * 29, [448.0, -448.0, 1.0] + [0.0] * 29),
    "256^2 + 15 x 0.125^2": ([256.0] + [0.125] * 15 + [0.0] * 16, [256.0] + [0.125] * 15 + [0.0] * 16),
}


def test_fp8_instruction_drops_small_terms_bf16_keeps_them(probe):
    lost = []
    for name, (p, q) in CASES.items():
        r8, r16, exact = _run(probe, p, q)
        assert np.all(r16 == exact), f"{name}: BF16 instruction {r16[:2]} != exact {exact}"
        if not np.all(r8 == exact):
            lost.append((name, float(r8[0]), exact))
    assert lost, ("the scaled FP8 instruction summed every case exactly: the FP8 scoring path "
                  "could use it instead of widening to BF16")
    print("scaled FP8 instruction:", "; ".join(f"{n}: {g} vs exact {e}" for n, g, e in lost))


def test_bf16_instruction_within_fp32_summation_bound(probe):
    # random signed E4M3 patterns with one 448 outlier each: the BF16 instruction stays within
    # the worst-case bound of FP32 summation over its 128 terms, (n - 1) u sum|terms|
    rng = np.random.default_rng(41)
    for _ in range(20):
        codes = rng.integers(0, 0x7F, size=32) | (rng.integers(0, 2, size=32) << 7)
        vals = np.array([oracle.e4m3_value(int(c)) for c in codes])
        vals[rng.integers(0, 32)] = 448.0
        q = vals[rng.permutation(32)]
        _, r16, exact = _run(probe, vals, q)
        bound = 127 * 2.0 ** -24 * 4.0 * float(np.abs(vals * q).sum())
        assert np.all(np.abs(r16 - exact) <= bound), (codes, r16[0], exact, bound)
