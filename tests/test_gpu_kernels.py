"""GPU parity of each HIP kernel against the oracle on small seeded inputs that still span
several tiles and ragged tails, plus the edge cases: empty inputs, padding slots and rows,
bounds that are zero, below k, or not a multiple of 64, every head count, FP8, and the
placement invariances. Bit-exact on bytes, scales, weights and index sets; logits within
1e-5 * max |logit| per row."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_quant_amd as dsa
from gpu_util import (DeviceWorkload, assert_logits_close, assert_topk_sets, bf16_dev, bf16_host,
                      dev, oracle_cache)
from goldens import byte_list, layernorm_order_key, rows
from sparse_attention_indexer_quant_amd.workloads import bf16_bits, bf16_to_f32, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()  # fail loudly if the HIP library is missing


# ---- quantize_queries -----------------------------------------------------------------------

def _query_cases():
    rng = np.random.default_rng(100)
    cases = {}
    for heads in (16, 32, 64):
        cases[f"normal_h{heads}"] = rng.standard_normal((37, heads, 128)).astype(np.float32)
    q = rng.standard_normal((9, 32, 128)).astype(np.float32)
    q[0] = 0.0                                       # all-zero rows (scale floor)
    q[1, :, :] *= 1e-38                              # tiny values around the subnormal range
    q[2, :, ::3] *= 1e30                             # huge values
    q[3] = np.where(rng.random((32, 128)) < 0.01, q[3] * 20, q[3])   # outliers x20
    q[4, :, :] = -0.0                                # negative zeros
    q[5] = np.round(q[5] * 4) / 4                    # many exact E2M1 midpoints after scaling
    q[6] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], size=(32, 128)) * \
        rng.choice([-1, 1], size=(32, 128))          # midpoints with amax 6 -> scale 1
    cases["edges"] = q
    return cases


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "fp8_mx"])
@pytest.mark.parametrize("case", list(_query_cases().keys()))
def test_quantize_queries_bit_exact(fmt, case):
    q = _query_cases()[case]
    qb = bf16_bits(q)
    wvb = bf16_bits(np.random.default_rng(3).standard_normal(q.shape[:2]).astype(np.float32) * 3)
    want_q, want_w = oracle.quantize_queries(qb, wvb, fmt)
    got_q, got_w = dsa.quantize_queries(bf16_dev(qb), bf16_dev(wvb), fmt)
    assert np.array_equal(got_q.cpu().numpy(), want_q)
    assert np.array_equal(bf16_host(got_w), want_w)


def test_quantize_queries_strided_input_and_no_weights():
    rng = np.random.default_rng(5)
    full = bf16_bits(rng.standard_normal((6, 40, 136)).astype(np.float32))
    view = bf16_dev(full)[:, 2:34, 8:136]  # head stride 136, row stride 40*136
    want, _ = oracle.quantize_queries(full[:, 2:34, 8:136], None, "mxfp4")
    out = torch.full((6, 2304), 7, dtype=torch.uint8, device="cuda")
    got, w = dsa.quantize_queries(view, None, "mxfp4", out=out)
    assert w is None
    assert np.array_equal(got.cpu().numpy()[:, :2176], want)
    assert np.all(got.cpu().numpy()[:, 2176:] == 7)  # row padding untouched


def test_quantize_queries_empty():
    got, w = dsa.quantize_queries(torch.empty((0, 32, 128), dtype=torch.bfloat16, device="cuda"),
                                  torch.empty((0, 32), dtype=torch.bfloat16, device="cuda"))
    assert got.shape == (0, 2176)


# ---- store_keys -----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,stride,offset", [("mxfp4", 4352, 0), ("mxfp4", 8192, 3840),
                                               ("mxfp4", 8192, 0), ("fp8", 8448, 0),
                                               ("fp8", 12288, 1024), ("fp8_mx", 8448, 0),
                                               ("fp8_mx", 9216, 512)])
def test_store_keys_bit_exact(fmt, stride, offset):
    rng = np.random.default_rng(7)
    pages = 9
    wl = make_workload("st", fmt=fmt, heads=16, seq_lens=[64 * pages - 5], query_lens=[1], topk=4,
                       seed=8, page_stride=stride, section_offset=offset)
    keys = wl.key_bits.copy()
    keys[3] = bf16_bits(np.full(128, 2.5, np.float32))              # constant key -> beta
    keys[4] = bf16_bits(np.zeros(128, np.float32))
    keys[5] = bf16_bits(rng.standard_normal(128).astype(np.float32) * 1e4)
    keys[6] = bf16_bits(rng.standard_normal(128).astype(np.float32) * 1e-4)
    slots = wl.key_slots.copy()
    slots[10] = -1                                                   # padding
    slots[11] = -12345
    slots[12] = 64 * pages + 3                                       # beyond the cache
    slots[13] = 1 << 40
    want = np.full(wl.cache_bytes, 0xA5, np.uint8)
    oracle.store_keys(keys, wl.gamma, wl.beta, wl.eps, slots, want, wl.num_pages, stride, offset, fmt)
    got = torch.full((wl.cache_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    dsa.store_keys(bf16_dev(keys), dev(wl.gamma), dev(wl.beta), wl.eps, dev(slots), got, wl.num_pages,
                   stride, fmt, offset)
    got = got.cpu().numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "fp8_mx"])
def test_store_keys_bulk_layernorm_bit_exact(fmt):
    # 300k keys spanning 2^-20 .. 2^20 in scale and offset: every LayerNorm rounding step
    # (tree sums, correctly rounded sqrt and divide, BF16) must match; FP8's finer grid
    # exposes a one-ulp rstd difference far more often than E2M1 does.
    rng = np.random.default_rng(21)
    T = 300_000
    scale = np.exp2(rng.uniform(-20, 20, size=(T, 1))).astype(np.float32)
    shift = (rng.standard_normal((T, 1)) * np.exp2(rng.uniform(-20, 20, size=(T, 1)))).astype(np.float32)
    keys = bf16_bits(rng.standard_normal((T, 128)).astype(np.float32) * scale + shift)
    pages = (T + 63) // 64
    section = 4352 if fmt == "mxfp4" else 8448
    slots = rng.permutation(pages * 64)[:T].astype(np.int64)
    gamma = bf16_to_f32(bf16_bits(1 + 0.1 * rng.standard_normal(128).astype(np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128).astype(np.float32)))
    want = np.zeros(pages * section, np.uint8)
    oracle.store_keys(keys, gamma, beta, 1e-6, slots, want, pages, section, 0, fmt)
    got = torch.zeros(pages * section, dtype=torch.uint8, device="cuda")
    dsa.store_keys(bf16_dev(keys), dev(gamma), dev(beta), 1e-6, dev(slots), got, pages, section, fmt)
    got = got.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4]}"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "fp8_mx"])
@pytest.mark.parametrize("lead,width", [(2, 130), (8, 136), (0, 132)])
def test_store_keys_strided_rows_bit_exact(fmt, lead, width):
    # Key rows that are not 16-byte rows (a 4-byte-aligned start, a row stride that is not a
    # multiple of 8 elements) take the one-wavefront-per-key kernel; 16-byte rows with a
    # stride of 136 take the sixteen-lanes-per-key one. Both write the oracle's bytes.
    rng = np.random.default_rng(23)
    T = 3000
    wide = bf16_bits((rng.standard_normal((T, width)) * 3 + 0.5).astype(np.float32))
    keys = wide[:, lead:lead + 128]
    pages = (T + 63) // 64 + 1
    section = 4352 if fmt == "mxfp4" else 8448
    slots = rng.permutation(pages * 64)[:T].astype(np.int64)
    slots[::7] = -1
    gamma = bf16_to_f32(bf16_bits(1 + 0.1 * rng.standard_normal(128).astype(np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128).astype(np.float32)))
    want = np.full(pages * section, 0x3C, np.uint8)
    oracle.store_keys(np.ascontiguousarray(keys), gamma, beta, 1e-6, slots, want, pages, section, 0, fmt)
    got = torch.full((pages * section,), 0x3C, dtype=torch.uint8, device="cuda")
    kdev = bf16_dev(wide)[:, lead:lead + 128]
    dsa.store_keys(kdev, dev(gamma), dev(beta), 1e-6, dev(slots), got, pages, section, fmt)
    assert np.array_equal(got.cpu().numpy(), want)


def test_store_keys_empty_and_all_padding():
    cache = torch.full((4352,), 0x5A, dtype=torch.uint8, device="cuda")
    g = torch.ones(128, device="cuda")
    b = torch.zeros(128, device="cuda")
    dsa.store_keys(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), g, b, 1e-6,
                   torch.empty(0, dtype=torch.int64, device="cuda"), cache, 1, 4352)
    dsa.store_keys(torch.ones((5, 128), dtype=torch.bfloat16, device="cuda"), g, b, 1e-6,
                   torch.full((5,), -1, dtype=torch.int64, device="cuda"), cache, 1, 4352)
    assert torch.all(cache == 0x5A)


def _golden_order_bytes():
    gold = {}
    for line in rows("layernorm_order.txt"):
        kind, *vals = line.split()
        gold.setdefault(kind, []).append(vals)
    return (np.array(byte_list(gold["mxfp4_payload"][0][0]), np.uint8),
            np.array(byte_list(gold["mxfp4_scales"][0][0]), np.uint8))


def _assert_golden_entry(cache: np.ndarray, slot: int, stride: int, offset: int, what: str):
    payload, scales = _golden_order_bytes()
    sec = offset + (slot // 64) * stride
    off = slot % 64
    assert np.array_equal(cache[sec + off * 64:sec + off * 64 + 64], payload), f"{what}: payload"
    assert np.array_equal(cache[sec + 4096 + off * 4:sec + 4096 + off * 4 + 4], scales), f"{what}: scales"


@pytest.mark.parametrize("path", ["bulk", "one_wave", "index_inputs"])
def test_key_layernorm_summation_order_golden(path):
    # tests/golden/layernorm_order.txt: a key whose MXFP4 bytes depend on the LayerNorm's
    # summation order (page "...cutedsl.dsa.index", insert_key), worked by hand; every key
    # path writes those bytes, among random keys that go through the oracle as usual.
    x, gamma, beta = layernorm_order_key()
    rng = np.random.default_rng(61)
    T, pages = 40, 2
    keys = bf16_bits(rng.standard_normal((T, 128)).astype(np.float32))
    gold_at = [0, 13, 39]
    keys[gold_at] = bf16_bits(x)
    slots = rng.permutation(pages * 64)[:T].astype(np.int64)
    want = np.full(pages * 4352, 0xA5, np.uint8)
    oracle.store_keys(keys, gamma, beta, 1e-6, slots, want, pages, 4352, 0, "mxfp4")
    got = torch.full((pages * 4352,), 0xA5, dtype=torch.uint8, device="cuda")
    if path == "bulk":
        dsa.store_keys(bf16_dev(keys), dev(gamma), dev(beta), 1e-6, dev(slots), got, pages, 4352)
    elif path == "one_wave":  # rows that are not 16-byte rows take the one-wavefront kernel
        wide = np.zeros((T, 130), np.uint16)
        wide[:, 2:] = keys
        dsa.store_keys(bf16_dev(wide)[:, 2:], dev(gamma), dev(beta), 1e-6, dev(slots), got, pages, 4352)
    else:
        heads = 16
        proj = np.zeros((T, 128 + heads + 8), np.uint16)
        proj[:, 8:136] = keys
        q = bf16_bits(rng.standard_normal((T, heads, 128)).astype(np.float32))
        dsa.index_inputs(bf16_dev(proj), 8, 136, bf16_dev(q), dev(gamma), dev(beta), 1e-6,
                         dev(slots), got, pages, 4352)
    got = got.cpu().numpy()
    for t in gold_at:
        _assert_golden_entry(want, int(slots[t]), 4352, 0, "oracle")
        _assert_golden_entry(got, int(slots[t]), 4352, 0, path)
    assert np.array_equal(got, want)


# ---- index_inputs (fused per-token query quant + weights + key insert) ---------------------

@pytest.mark.parametrize("fmt,heads,stride,offset,key_col,weight_col",
                         [("mxfp4", 32, 4352, 0, 4096, 4224), ("mxfp4", 64, 8192, 3840, 0, 130),
                          ("mxfp4", 16, 4352, 0, 2, 1), ("fp8", 32, 8448, 0, 200, 4),
                          ("fp8_mx", 16, 8448, 0, 64, 300),
                          ("fp8", 64, 9216, 512, 8192, 0)])
def test_index_inputs_bit_exact(fmt, heads, stride, offset, key_col, weight_col):
    # queries with the same edge rows as the quantize tests, keys with extreme scales, padding
    # and out-of-range slots, and packed rows whose other columns hold NaN / Inf patterns
    rng = np.random.default_rng(30 + heads)
    pages = 7
    tokens = 45
    q = rng.standard_normal((tokens, heads, 128)).astype(np.float32)
    q[0] = 0.0
    q[1] *= 1e-38
    q[2, :, ::3] *= 1e30
    q[3] = -0.0
    keys = rng.standard_normal((tokens, 128)).astype(np.float32)
    keys[4] = 2.5
    keys[5] *= 1e4
    keys[6] *= 1e-4
    wv = (rng.standard_normal((tokens, heads)) * 3).astype(np.float32)
    cols = max(key_col + 128, weight_col + heads) + 6
    proj = rng.choice(np.array([0x7FC0, 0xFF80, 0x7F80, 0x3F80], np.uint16), size=(tokens, cols))
    proj[:, key_col:key_col + 128] = bf16_bits(keys)
    proj[:, weight_col:weight_col + heads] = bf16_bits(wv)
    slots = rng.permutation(pages * 64)[:tokens].astype(np.int64)
    slots[7] = -1
    slots[8] = 64 * pages + 1
    gamma = bf16_to_f32(bf16_bits(1 + 0.1 * rng.standard_normal(128).astype(np.float32)))
    beta = bf16_to_f32(bf16_bits(0.1 * rng.standard_normal(128).astype(np.float32)))
    section = 4352 if fmt == "mxfp4" else 8448
    nbytes = offset + (pages - 1) * stride + section
    want_cache = np.full(nbytes, 0xA5, np.uint8)
    want_q, want_w = oracle.index_inputs(proj, key_col, weight_col, bf16_bits(q), gamma, beta, 1e-6,
                                         slots, want_cache, pages, stride, offset, fmt)
    got_cache = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    proj_dev = bf16_dev(proj)
    got_q, got_w = dsa.index_inputs(proj_dev, key_col, weight_col, bf16_dev(bf16_bits(q)), dev(gamma),
                                    dev(beta), 1e-6, dev(slots), got_cache, pages, stride, fmt,
                                    offset)
    assert np.array_equal(got_q.cpu().numpy(), want_q)
    assert np.array_equal(bf16_host(got_w), want_w)
    assert np.array_equal(got_cache.cpu().numpy(), want_cache)


@pytest.mark.parametrize("dcp", [(0, 1, 1), (1, 4, 64)])
def test_index_inputs_layout_matches_separate_calls(dcp):
    # one launch: the fused inputs plus the row bounds, bit-identical to the two calls
    rng = np.random.default_rng(45)
    tokens, heads, pages = 10, 32, 30
    proj = bf16_bits(rng.standard_normal((tokens, 200)).astype(np.float32))
    q = bf16_bits(rng.standard_normal((tokens, heads, 128)).astype(np.float32))
    slots = rng.permutation(pages * 64)[:tokens].astype(np.int64)
    slots[3] = -1
    seq = rng.integers(1, 1500, size=7).astype(np.int32)
    ql = np.array([1, 2, 0, 3, 1, 1, 2], np.int32)
    g, b = dev(np.ones(128, np.float32)), dev(np.zeros(128, np.float32))
    c1 = torch.zeros(pages * 4352, dtype=torch.uint8, device="cuda")
    c2 = torch.zeros(pages * 4352, dtype=torch.uint8, device="cuda")
    pd = bf16_dev(proj)
    q1, w1, s1, e1 = dsa.index_inputs_layout(pd, 8, 140, bf16_dev(q), g, b, 1e-6, dev(slots), c1,
                                             pages, 4352, dev(seq), dev(ql), 13, "mxfp4", 0, *dcp)
    q2, w2 = dsa.index_inputs(pd, 8, 140, bf16_dev(q), g, b, 1e-6, dev(slots), c2, pages, 4352)
    s2, e2 = dsa.decode_layout(dev(seq), dev(ql), 13, *dcp)
    assert torch.equal(q1, q2) and torch.equal(w1, w2) and torch.equal(c1, c2)
    assert torch.equal(s1, s2) and torch.equal(e1, e2)
    os_, oe = oracle.decode_layout(seq, ql, 13, *dcp)
    assert np.array_equal(s1.cpu().numpy(), os_) and np.array_equal(e1.cpu().numpy(), oe)
    # no tokens: only the layout
    _, _, s3, e3 = dsa.index_inputs_layout(pd[:0], 8, 140, bf16_dev(q)[:0], g, b, 1e-6,
                                           dev(slots)[:0], c1, pages, 4352, dev(seq), dev(ql), 13,
                                           "mxfp4", 0, *dcp)
    assert torch.equal(s3, s2) and torch.equal(e3, e2)


def test_index_inputs_matches_separate_calls_and_empty():
    # one launch gives the same bytes as quantize_queries + store_keys on the extracted columns
    rng = np.random.default_rng(44)
    tokens, heads, pages = 20, 32, 3
    proj = bf16_bits(rng.standard_normal((tokens, 300)).astype(np.float32))
    q = bf16_bits(rng.standard_normal((tokens, heads, 128)).astype(np.float32))
    slots = rng.permutation(pages * 64)[:tokens].astype(np.int64)
    g, b = dev(np.ones(128, np.float32)), dev(np.zeros(128, np.float32))
    c1 = torch.zeros(pages * 4352, dtype=torch.uint8, device="cuda")
    c2 = torch.zeros(pages * 4352, dtype=torch.uint8, device="cuda")
    proj_dev = bf16_dev(proj)
    q1, w1 = dsa.index_inputs(proj_dev, 10, 160, bf16_dev(q), g, b, 1e-6, dev(slots), c1, pages, 4352)
    q2, w2 = dsa.quantize_queries(bf16_dev(q), proj_dev[:, 160:160 + heads].contiguous())
    dsa.store_keys(proj_dev[:, 10:138].contiguous(), g, b, 1e-6, dev(slots), c2, pages, 4352)
    assert torch.equal(q1, q2) and torch.equal(w1, w2) and torch.equal(c1, c2)
    # no tokens: nothing enqueued, nothing written
    c3 = torch.full((4352,), 0x5A, dtype=torch.uint8, device="cuda")
    dsa.index_inputs(proj_dev[:0], 10, 160, bf16_dev(q)[:0], g, b, 1e-6, dev(slots)[:0], c3, 1, 4352)
    assert torch.all(c3 == 0x5A)


# ---- decode_layout --------------------------------------------------------------------------

@pytest.mark.parametrize("seq,ql,rows,dcp", [
    ([10, 20, 5], [1, 3, 2], 8, (0, 1, 1)), ([1], [3], 3, (0, 1, 1)), ([], [], 4, (0, 1, 1)),
    ([7], [1], 0, (0, 1, 1)), ([100], [1], 1, (0, 4, 8)), ([100], [1], 1, (3, 4, 8)),
    ([45], [1], 1, (1, 2, 4)), ([9, 9], [2, 0], 3, (0, 1, 1))])
def test_decode_layout_small(seq, ql, rows, dcp):
    s_want, e_want = oracle.decode_layout(seq, ql, rows, *dcp)
    s, e = dsa.decode_layout(dev(np.array(seq, np.int32)), dev(np.array(ql, np.int32)), rows, *dcp)
    assert np.array_equal(s.cpu().numpy(), s_want) and np.array_equal(e.cpu().numpy(), e_want)


def test_decode_layout_large_random():
    rng = np.random.default_rng(9)
    for R, rows in [(3000, 9000), (128, 512), (1, 1)]:
        ql = rng.integers(0, 5, R).astype(np.int32)
        seq = (ql + rng.integers(0, 70000, R)).astype(np.int32)
        rows = max(rows, int(ql.sum()))
        for dcp in [(0, 1, 1), (2, 4, 16)]:
            s_want, e_want = oracle.decode_layout(seq, ql, rows, *dcp)
            s, e = dsa.decode_layout(dev(seq), dev(ql), rows, *dcp)
            assert np.array_equal(s.cpu().numpy(), s_want)
            assert np.array_equal(e.cpu().numpy(), e_want)


# ---- score_paged ----------------------------------------------------------------------------

SCORE_CASES = {
    # name: make_workload kwargs
    "fp4_h32_ragged": dict(fmt="mxfp4", heads=32, seq_lens=[1000, 64, 1, 777, 130], query_lens=[1, 1, 1, 1, 1]),
    "fp4_h16_verify": dict(fmt="mxfp4", heads=16, seq_lens=[300, 1200, 7, 64], query_lens=[4, 2, 3, 1],
                           num_rows=16),
    "fp4_h64_merged": dict(fmt="mxfp4", heads=64, seq_lens=[2100, 513], query_lens=[1, 3],
                           page_stride=8192, section_offset=3840),
    "fp4_h32_qlen16": dict(fmt="mxfp4", heads=32, seq_lens=[600, 40], query_lens=[16, 5], num_rows=24),
    "fp8_h32": dict(fmt="fp8", heads=32, seq_lens=[1500, 65, 300], query_lens=[1, 2, 1],
                    outlier_frac=0.01, outlier_gain=20.0),
    "fp8_h64_verify": dict(fmt="fp8", heads=64, seq_lens=[500, 129], query_lens=[3, 4], num_rows=9,
                           page_stride=9216, section_offset=512),
    "fp4_h32_scaled_heads": dict(fmt="mxfp4", heads=32, seq_lens=[900], query_lens=[2], head_log2_scale=4.0),
    "fp8mx_h32_verify": dict(fmt="fp8_mx", heads=32, seq_lens=[700, 130, 5], query_lens=[2, 1, 1],
                             num_rows=6, outlier_frac=0.01, outlier_gain=20.0),
}


def _run_score(name, seed=11):
    kw = dict(SCORE_CASES[name])
    wl = make_workload(name, topk=64, seed=seed, extra_pages=3, **kw)
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    ocache = oracle_cache(wl)
    assert np.array_equal(dw.cache.cpu().numpy(), ocache)
    q_rows, w = dw.quantize()
    oq, ow = oracle.quantize_queries(wl.q_bits, wl.wv_bits, wl.fmt)
    assert np.array_equal(q_rows.cpu().numpy(), oq) and np.array_equal(bf16_host(w), ow)
    starts, ends = dw.layout()
    os_, oe = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
    assert np.array_equal(starts.cpu().numpy(), os_) and np.array_equal(ends.cpu().numpy(), oe)
    logits = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    dsa.score_paged(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride, dw.block_table,
                    starts, ends, wl.max_query_len, wl.fmt, wl.section_offset, out=logits)
    ref = oracle.score_paged(oq, wl.heads, ow, ocache, wl.num_pages, wl.page_stride, wl.block_table,
                             os_, oe, wl.fmt, wl.section_offset)
    return wl, dw, logits.cpu().numpy(), ref, oe, (q_rows, w, starts, ends)


@pytest.mark.parametrize("name", list(SCORE_CASES))
def test_score_paged_matches_oracle(name):
    wl, _, got, ref, ends, _ = _run_score(name)
    # written exactly where the oracle writes (bounds respected, padding rows untouched)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert_logits_close(got, ref, ends, range(wl.num_rows), name)


@pytest.mark.parametrize("name", list(SCORE_CASES))
@pytest.mark.parametrize("k", [1, 64, 700])
def test_score_topk_matches_separate_calls(name, k):
    # the scorer writing the selection's histograms changes nothing: the same logits bit for
    # bit, and index sets equal to the oracle's top-k of those logits (workspace starts as
    # arbitrary bytes)
    wl, dw, got, ref, ends, (q_rows, w, starts, dends) = _run_score(name)
    logits = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    ws = torch.full((dsa.score_topk_workspace_bytes(wl.num_requests, wl.max_blocks, wl.num_rows),),
                    0x5C, dtype=torch.uint8, device="cuda")
    _, idx = dsa.score_topk(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride,
                            dw.block_table, starts, dends, wl.max_query_len, k, wl.fmt,
                            wl.section_offset, out=logits, workspace=ws)
    fused = logits.cpu().numpy()
    assert np.array_equal(fused.view(np.uint32), got.view(np.uint32))
    want = oracle.topk(np.nan_to_num(fused, nan=0.0), ends, k)
    assert_topk_sets(idx.cpu().numpy(), want, range(wl.num_rows), f"{name} k={k}")


# ---- bounded logits: row tiles (page "...amd.ops.fp4_indexer", decode_tile_size) -------------

TILED_CASES = {
    # verify rows (1..4 per request, tiles splitting requests) with graph padding rows
    "fp4_h32_verify": (dict(fmt="mxfp4", heads=32, seq_lens=[700, 129, 2000, 64, 1500, 5, 900],
                            query_lens=[3, 1, 4, 2, 4, 1, 2], num_rows=21), [1, 3, 5, 8, 32]),
    "fp4_h64_merged": (dict(fmt="mxfp4", heads=64, seq_lens=[600, 1300, 70], query_lens=[2, 1, 3],
                            page_stride=8192, section_offset=3840), [2, 4]),
    "fp8_h32_verify": (dict(fmt="fp8", heads=32, seq_lens=[500, 129, 1000], query_lens=[2, 1, 2],
                            num_rows=7, outlier_frac=0.01, outlier_gain=20.0), [3]),
}


@pytest.mark.parametrize("name", list(TILED_CASES))
@pytest.mark.parametrize("k", [64, 700])
def test_score_topk_tiled_matches_untiled_and_oracle(name, k):
    kw, tiles = TILED_CASES[name]
    wl = make_workload(name, topk=k, seed=29, extra_pages=2, **kw)
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    q_rows, w = dw.quantize()
    starts, ends = dw.layout()
    oe = ends.cpu().numpy()
    full = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    _, idx_full = dsa.score_topk(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride,
                                 dw.block_table, starts, ends, wl.max_query_len, k, wl.fmt,
                                 wl.section_offset, out=full)
    full_np = full.cpu().numpy()
    oq, ow = oracle.quantize_queries(wl.q_bits, wl.wv_bits, wl.fmt)
    os_, _ = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
    ref = oracle.score_paged(oq, wl.heads, ow, oracle_cache(wl), wl.num_pages, wl.page_stride,
                             wl.block_table, os_, oe, wl.fmt, wl.section_offset)
    assert_logits_close(full_np, ref, oe, range(wl.num_rows), name)
    want = oracle.topk(np.nan_to_num(full_np, nan=0.0), oe, k)
    for tile in tiles + [wl.num_rows + 5]:
        ws = torch.full((dsa.library().dsaidx_score_topk_tiled_workspace_bytes(
            wl.num_requests, wl.max_blocks, tile, wl.max_query_len),), 0xA7, dtype=torch.uint8,
            device="cuda")
        lt = torch.full((tile, wl.width), float("nan"), device="cuda")
        idx, lt = dsa.score_topk_tiled(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride,
                                       dw.block_table, starts, ends, wl.max_query_len, k, tile,
                                       wl.fmt, wl.section_offset, logits_tile=lt, workspace=ws)
        what = f"{name} k={k} tile={tile}"
        assert_topk_sets(idx.cpu().numpy(), idx_full.cpu().numpy(), range(wl.num_rows), what)
        assert_topk_sets(idx.cpu().numpy(), want, range(wl.num_rows), what)
        # the buffer holds the last tile's logits, bit for bit those of the untiled scorer
        last = (wl.num_rows - 1) // tile * tile
        got = lt.cpu().numpy()
        for r in range(last, wl.num_rows):
            n = min(int(oe[r]), wl.width)
            assert np.array_equal(got[r - last, :n].view(np.uint32), full_np[r, :n].view(np.uint32)), what


# ---- index_score_hist (step inputs made inside the scorer) ----------------------------------

FUSED_CASES = {
    "fp4_h32_ragged": SCORE_CASES["fp4_h32_ragged"],
    "fp4_h16_verify": SCORE_CASES["fp4_h16_verify"],
    "fp4_h64_merged": SCORE_CASES["fp4_h64_merged"],
    "fp4_h32_scaled_heads": SCORE_CASES["fp4_h32_scaled_heads"],
    # keys at the first positions, a request with no rows, keys that straddle a page boundary
    # and end a page, padding rows, and a row whose keys start past its request's first chunk
    "fp4_h64_edges": dict(fmt="mxfp4", heads=64, seq_lens=[2, 130, 4098, 64, 9000],
                          query_lens=[2, 0, 4, 1, 3], num_rows=13),
    # FP8 (at most 2 rows per request): outliers, the mx scale bytes, merged pages, keys at
    # position 0, straddling and ending pages, a request with no rows, padding rows
    "fp8_h32": SCORE_CASES["fp8_h32"],
    "fp8mx_h32_verify": SCORE_CASES["fp8mx_h32_verify"],
    "fp8_h64_merged": dict(fmt="fp8", heads=64, seq_lens=[500, 129, 64], query_lens=[2, 1, 2],
                           num_rows=7, page_stride=9216, section_offset=512),
    "fp8mx_h16_edges": dict(fmt="fp8_mx", heads=16, seq_lens=[2, 130, 65, 700], query_lens=[2, 0, 2, 1],
                            num_rows=8, outlier_frac=0.01, outlier_gain=20.0),
    # one-row groups whose first row is not the request's index (requests with no rows before
    # them), more requests than rows, and a padding row: the query each workgroup loads before
    # its row is known is the wrong one here and must be replaced
    "fp4_h32_one_row_gaps": dict(fmt="mxfp4", heads=32, seq_lens=[70, 5, 300, 64, 1, 130],
                                 query_lens=[1, 0, 1, 1, 0, 1], num_rows=5),
    "fp8_h16_one_row_gaps": dict(fmt="fp8", heads=16, seq_lens=[200, 9, 64, 65],
                                 query_lens=[0, 1, 1, 1], num_rows=3),
}


def _step_projection(wl, key_col, weight_col, cols, rng):
    """Packed projection rows of the step, one per query row: the row's new key and raw head
    weights at the given columns, other columns (and padding rows) NaN / Inf / junk bits."""
    proj = rng.choice(np.array([0x7FC0, 0xFF80, 0x7F80, 0x3F80], np.uint16), size=(wl.num_rows, cols))
    sk = wl.step_key_index()
    proj[:sk.size, key_col:key_col + 128] = wl.key_bits[sk]
    proj[:, weight_col:weight_col + wl.heads] = wl.wv_bits
    slots = np.full(wl.num_rows, -1, np.int64)
    slots[:sk.size] = wl.key_slots[sk]
    return proj, slots


def _cache_without_step_keys(wl):
    """A device cache holding every key but the step's (their slots keep the filler)."""
    keep = np.ones(wl.total_keys, bool)
    keep[wl.step_key_index()] = False
    dw = DeviceWorkload(wl)
    if keep.any():
        dsa.store_keys(bf16_dev(wl.key_bits[keep]), dw.gamma, dw.beta, wl.eps,
                       dev(wl.key_slots[keep]), dw.cache, wl.num_pages, wl.page_stride, wl.fmt,
                       wl.section_offset)
    return dw


@pytest.mark.parametrize("name", list(FUSED_CASES))
@pytest.mark.parametrize("k", [1, 700])
def test_index_score_matches_oracle_and_separate_calls(name, k):
    # the fused step against the oracle (cache bytes with the new keys, row layout, logits,
    # top-k sets), and bit for bit against index_inputs_layout + score_paged_hist + topk_scored
    wl = make_workload(name, topk=64, seed=17, extra_pages=3, **FUSED_CASES[name])
    rng = np.random.default_rng(5)
    key_col, weight_col, cols = 6, 140, 210
    proj, slots = _step_projection(wl, key_col, weight_col, cols, rng)
    ocache = oracle_cache(wl)
    oq, ow = oracle.quantize_queries(wl.q_bits, wl.wv_bits, wl.fmt)
    os_, oe = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
    ref = oracle.score_paged(oq, wl.heads, ow, ocache, wl.num_pages, wl.page_stride,
                             wl.block_table, os_, oe, wl.fmt, wl.section_offset)

    a = _cache_without_step_keys(wl)
    b = _cache_without_step_keys(wl)
    pd = bf16_dev(proj)
    la = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    wsa = torch.full((dsa.score_topk_workspace_bytes(wl.num_requests, wl.max_blocks, wl.num_rows),),
                     0x5C, dtype=torch.uint8, device="cuda")
    starts, ends, _, idx = dsa.index_score_topk(
        pd, key_col, weight_col, a.q, a.gamma, a.beta, wl.eps, a.seq_lens, a.query_lens,
        wl.num_rows, a.cache, wl.num_pages, wl.page_stride, a.block_table, wl.max_query_len, k,
        wl.fmt, wl.section_offset, out=la, workspace=wsa)
    assert np.array_equal(a.cache.cpu().numpy(), ocache), f"{name}: cache bytes"
    assert np.array_equal(starts.cpu().numpy(), os_) and np.array_equal(ends.cpu().numpy(), oe)
    got = la.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{name}: written entries"
    assert_logits_close(got, ref, oe, range(wl.num_rows), name)
    want = oracle.topk(np.nan_to_num(got, nan=0.0), oe, k)
    assert_topk_sets(idx.cpu().numpy(), want, range(wl.num_rows), f"{name} k={k}")

    qb, wb, sb, eb = dsa.index_inputs_layout(pd, key_col, weight_col, b.q, b.gamma, b.beta, wl.eps,
                                             dev(slots), b.cache, wl.num_pages, wl.page_stride,
                                             b.seq_lens, b.query_lens, wl.num_rows, wl.fmt,
                                             wl.section_offset)
    lb = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    _, idx_b = dsa.score_topk(qb, wl.heads, wb, b.cache, wl.num_pages, wl.page_stride,
                              b.block_table, sb, eb, wl.max_query_len, k, wl.fmt,
                              wl.section_offset, out=lb)
    assert torch.equal(a.cache, b.cache)
    assert np.array_equal(got.view(np.uint32), lb.cpu().numpy().view(np.uint32)), f"{name}: logits bits"
    assert_topk_sets(idx.cpu().numpy(), idx_b.cpu().numpy(), range(wl.num_rows), f"{name} k={k}")


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_index_score_layernorm_order_golden(fmt):
    # the fused step inserts the hand-worked key of tests/golden/layernorm_order.txt (as the
    # step key of two of its rows) with the bytes worked out there, and the rest as the oracle
    x, gamma, beta = layernorm_order_key()
    wl = make_workload("ln_gold", fmt=fmt, heads=32, seq_lens=[300, 129, 70], query_lens=[2, 1, 2],
                       topk=64, seed=19, extra_pages=2)
    wl.gamma, wl.beta = gamma, beta
    sk = wl.step_key_index()
    wl.key_bits[sk[[0, 3]]] = bf16_bits(x)
    rng = np.random.default_rng(6)
    key_col, weight_col, cols = 0, 130, 170
    proj, slots = _step_projection(wl, key_col, weight_col, cols, rng)
    ocache = oracle_cache(wl)
    a = _cache_without_step_keys(wl)
    la = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    dsa.index_score_topk(bf16_dev(proj), key_col, weight_col, a.q, a.gamma, a.beta, wl.eps,
                         a.seq_lens, a.query_lens, wl.num_rows, a.cache, wl.num_pages,
                         wl.page_stride, a.block_table, wl.max_query_len, 16, wl.fmt,
                         wl.section_offset, out=la)
    got = a.cache.cpu().numpy()
    if fmt == "mxfp4":
        for t in (0, 3):
            _assert_golden_entry(ocache, int(wl.key_slots[sk[t]]), wl.page_stride, 0, "oracle")
            _assert_golden_entry(got, int(wl.key_slots[sk[t]]), wl.page_stride, 0, "fused")
    assert np.array_equal(got, ocache)


LONG_ROW_CASES = {
    # one or two requests of 64K-131K keys: the scorer's segments number in the hundreds per
    # row, so the selection takes the separate threshold and collect kernels over sparse
    # histogram blocks (rows of more than 64 segments), and above 128 segments their
    # multi-block loops
    "fp4_one_64k": dict(fmt="mxfp4", heads=32, seq_lens=[65536], query_lens=[1]),
    "fp4_two_long_verify": dict(fmt="mxfp4", heads=32, seq_lens=[131072, 70001], query_lens=[3, 1]),
    "fp8_one_80k": dict(fmt="fp8", heads=32, seq_lens=[80000], query_lens=[2]),
}


@pytest.mark.parametrize("name", list(LONG_ROW_CASES))
@pytest.mark.parametrize("k", [2048, 7])
def test_score_topk_rows_of_many_segments(name, k):
    # score_topk and index_score_topk on rows spanning hundreds of scoring segments, with a
    # workspace of arbitrary bytes: logits bit for bit equal to score_paged's (and, fused, to
    # the separate calls), index sets equal to the oracle's top-k of the same logits
    wl = make_workload(name, topk=k, seed=23, extra_pages=1, **LONG_ROW_CASES[name])
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    q_rows, w = dw.quantize()
    starts, ends = dw.layout()
    oe = ends.cpu().numpy()
    plain = dw.score(q_rows, w, starts, ends)
    ws = torch.full((dsa.score_topk_workspace_bytes(wl.num_requests, wl.max_blocks, wl.num_rows),),
                    0xC3, dtype=torch.uint8, device="cuda")
    la = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    _, idx = dsa.score_topk(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride,
                            dw.block_table, starts, ends, wl.max_query_len, k, wl.fmt,
                            wl.section_offset, out=la, workspace=ws)
    cols = torch.arange(wl.width, device="cuda")
    valid = cols[None, :] < ends.to(torch.int64)[:, None]
    assert torch.equal(la.view(torch.int32)[valid], plain.view(torch.int32)[valid]), f"{name}: logits"
    got = la.cpu().numpy()
    want = oracle.topk(np.nan_to_num(got, nan=0.0), oe, k)
    assert_topk_sets(idx.cpu().numpy(), want, range(wl.num_rows), f"{name} k={k}")
    # the fused step from a cache without the step keys, on the same (reused) workspace
    rng = np.random.default_rng(8)
    proj, _ = _step_projection(wl, 0, 128, 128 + wl.heads, rng)
    b = _cache_without_step_keys(wl)
    lb = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    _, fe, _, fidx = dsa.index_score_topk(
        bf16_dev(proj), 0, 128, b.q, b.gamma, b.beta, wl.eps, b.seq_lens, b.query_lens,
        wl.num_rows, b.cache, wl.num_pages, wl.page_stride, b.block_table, wl.max_query_len, k,
        wl.fmt, wl.section_offset, out=lb, workspace=ws)
    assert torch.equal(b.cache, dw.cache), f"{name}: fused cache bytes"
    assert torch.equal(fe, ends)
    assert torch.equal(lb.view(torch.int32)[valid], plain.view(torch.int32)[valid]), f"{name}: fused logits"
    assert_topk_sets(fidx.cpu().numpy(), want, range(wl.num_rows), f"{name} fused k={k}")


# Rows of 8K-40K keys in at most 64 scoring segments (the selection's one-launch threshold and
# collect, then the select) whose threshold bin is not the usual few hundred keys: a segment of
# identical keys that align with the row's most weighted query head (a tie of 1024+ keys at the
# top, all in one segment), rows whose query is zero (every logit +0: one bin of every key, more
# than the candidate list holds, selected from the row itself), next to random rows, for decode,
# uneven and verify-shaped batches, FP8 and merged 64-head pages.
ADVERSARIAL_CASES = {
    "fp4_decode_32seg": dict(fmt="mxfp4", heads=32, seq_lens=[32768] * 8, query_lens=[1] * 8),
    "fp4_uneven_rows": dict(fmt="mxfp4", heads=32, seq_lens=[30000, 9000, 20000, 12000, 9100, 15000],
                            query_lens=[2, 0, 1, 3, 0, 0]),
    "fp8_decode": dict(fmt="fp8", heads=32, seq_lens=[20000, 17000, 9000, 20000, 3000, 15000],
                       query_lens=[1] * 6, outlier_frac=0.01, outlier_gain=20.0),
    "fp4_h64_merged": dict(fmt="mxfp4", heads=64, seq_lens=[40000, 23000, 8300, 40000],
                           query_lens=[1, 1, 1, 1], page_stride=8192, section_offset=3840),
    "fp4_verify_ragged": dict(fmt="mxfp4", heads=32, seq_lens=[30000, 9000, 4200, 20000, 12000, 65, 9100],
                              query_lens=[4, 1, 3, 2, 4, 1, 2], num_rows=20),
    # more (row, segment) items than the chip holds workgroups at once: 300 requests of 1-20000
    # keys, some without rows, rows of at most k keys, 40 padding rows
    "fp4_many_uneven": dict(fmt="mxfp4", heads=32,
                            seq_lens=np.random.default_rng(43).integers(1, 20001, size=300),
                            query_lens=(np.random.default_rng(44).random(300) < 0.93).astype(np.int32),
                            num_rows=int((np.random.default_rng(44).random(300) < 0.93).sum()) + 40),
}


def _hot_segment(wl, req, lo, hi):
    """Keys [lo, hi) of request `req` made equal to its first row's most weighted query head
    (pre-norm), so that they tie near the top of that row."""
    r0 = int(np.sum(wl.query_lens[:req]))
    h = int(np.argmax(bf16_to_f32(wl.wv_bits[r0])))
    off = int(wl.key_offsets[req])
    wl.key_bits[off + lo:off + hi] = wl.q_bits[r0, h]


@pytest.mark.parametrize("name", list(ADVERSARIAL_CASES))
@pytest.mark.parametrize("variant", ["random", "hot_segment", "zero_query"])
@pytest.mark.parametrize("k", [1, 64, 2048, 6000])
def test_score_topk_adversarial_rows(name, variant, k):
    # score_topk and index_score_topk: logits bit for bit equal to score_paged's and close to the
    # oracle's, index sets equal to the oracle's top-k of the same logits, on a workspace of
    # arbitrary bytes
    kw = ADVERSARIAL_CASES[name]
    wl = make_workload(name, topk=k, seed=31, extra_pages=1, **kw)
    seg = dsa.score_segment_keys(wl.num_requests, wl.max_blocks)
    assert wl.width > 8192 and -(-wl.width // seg) <= 64, "not the one-launch threshold and collect"
    if variant == "hot_segment":
        for q in range(wl.num_requests):
            n = int(wl.seq_lens[q])
            if n > 3 * seg and wl.query_lens[q] > 0:
                _hot_segment(wl, q, seg, seg + max(1024, seg))
    elif variant == "zero_query":
        wl.q_bits[::2] = 0
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    q_rows, w = dw.quantize()
    starts, ends = dw.layout()
    oe = ends.cpu().numpy()
    plain = dw.score(q_rows, w, starts, ends)
    ws = torch.full((dsa.score_topk_workspace_bytes(wl.num_requests, wl.max_blocks, wl.num_rows),),
                    0x3C, dtype=torch.uint8, device="cuda")
    la = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    _, idx = dsa.score_topk(q_rows, wl.heads, w, dw.cache, wl.num_pages, wl.page_stride,
                            dw.block_table, starts, ends, wl.max_query_len, k, wl.fmt,
                            wl.section_offset, out=la, workspace=ws)
    cols = torch.arange(wl.width, device="cuda")
    valid = cols[None, :] < ends.to(torch.int64)[:, None]
    assert torch.equal(la.view(torch.int32)[valid], plain.view(torch.int32)[valid]), f"{name}: logits"
    got = la.cpu().numpy()
    if k == 64:  # the logits do not depend on k: compared with the oracle's once per workload
        oq, ow = oracle.quantize_queries(wl.q_bits, wl.wv_bits, wl.fmt)
        os_, _ = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
        ref = oracle.score_paged(oq, wl.heads, ow, oracle_cache(wl), wl.num_pages, wl.page_stride,
                                 wl.block_table, os_, oe, wl.fmt, wl.section_offset)
        assert_logits_close(got, ref, oe, range(wl.num_rows), name)
    want = oracle.topk(np.nan_to_num(got, nan=0.0), oe, k)
    what = f"{name} {variant} k={k}"
    assert_topk_sets(idx.cpu().numpy(), want, range(wl.num_rows), what)
    # the fused step from a cache without the step keys, on the same (reused) workspace
    rng = np.random.default_rng(12)
    proj, _ = _step_projection(wl, 0, 128, 128 + wl.heads, rng)
    b = _cache_without_step_keys(wl)
    lb = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    _, fe, _, fidx = dsa.index_score_topk(
        bf16_dev(proj), 0, 128, b.q, b.gamma, b.beta, wl.eps, b.seq_lens, b.query_lens,
        wl.num_rows, b.cache, wl.num_pages, wl.page_stride, b.block_table, wl.max_query_len, k,
        wl.fmt, wl.section_offset, out=lb, workspace=ws)
    assert torch.equal(b.cache, dw.cache), f"{what}: fused cache bytes"
    assert torch.equal(fe, ends)
    assert torch.equal(lb.view(torch.int32)[valid], plain.view(torch.int32)[valid]), f"{what}: fused logits"
    assert_topk_sets(fidx.cpu().numpy(), want, range(wl.num_rows), f"{what} fused")


def _one_launch_case(name):
    """Batches whose requests each have at most one row, every row's keys in one scoring
    workgroup: index_score_topk selects inside the scoring launch."""
    rng = np.random.default_rng(41)
    if name == "fp4_tiny":
        return dict(fmt="mxfp4", heads=32, seq_lens=[256], query_lens=[1])
    if name == "fp4_h64_one_short_padded":  # a ragged last page and two padding rows
        return dict(fmt="mxfp4", heads=64, seq_lens=[200], query_lens=[1], num_rows=3)
    if name == "fp4_many_short":  # requests without rows, one-key rows, padding rows
        seq = rng.integers(1, 4097, size=300)
        seq[:3] = [1, 64, 65]
        ql = (rng.random(300) < 0.9).astype(np.int32)
        ql[:3] = 1
        return dict(fmt="mxfp4", heads=32, seq_lens=seq, query_lens=ql, num_rows=int(ql.sum()) + 5)
    if name == "fp8_many_short":
        return dict(fmt="fp8", heads=32, seq_lens=rng.integers(1, 4097, size=256),
                    query_lens=[1] * 256, outlier_frac=0.01, outlier_gain=20.0)
    if name == "fp8mx_h16_many_short":
        return dict(fmt="fp8_mx", heads=16, seq_lens=rng.integers(1, 2049, size=260),
                    query_lens=[1] * 260)
    if name == "fp4_h64_merged_many_short":
        return dict(fmt="mxfp4", heads=64, seq_lens=rng.integers(1, 3001, size=256),
                    query_lens=[1] * 256, page_stride=8192, section_offset=3840)
    raise KeyError(name)


ONE_LAUNCH_CASES = ["fp4_tiny", "fp4_h64_one_short_padded", "fp4_many_short", "fp8_many_short",
                    "fp8mx_h16_many_short", "fp4_h64_merged_many_short"]


@pytest.mark.parametrize("name", ONE_LAUNCH_CASES)
@pytest.mark.parametrize("variant", ["random", "hot_segment", "zero_query"])
@pytest.mark.parametrize("k", [1, 64, 2048])
def test_index_score_topk_one_launch(name, variant, k):
    # the step with its selection in the scoring launch: cache bytes and row layout as the
    # oracle's, logits bit for bit equal to score_paged's (and close to the oracle's), index
    # sets equal to the oracle's top-k of the same logits -- with rows of at most k keys, ties
    # of a thousand keys at the top of a row, and rows whose logits are all +0 (one bin of every
    # key: up to 64 candidates, up to the LDS list's 1024, and more), padding rows and rows of
    # requests without keys selecting none
    wl = make_workload(name, topk=k, seed=37, extra_pages=1, **_one_launch_case(name))
    assert dsa.score_segment_keys(wl.num_requests, wl.max_blocks) >= wl.width, "not one launch"
    if variant == "hot_segment":
        for q in range(wl.num_requests):
            n = int(wl.seq_lens[q])
            if n > 1200 and wl.query_lens[q] > 0:
                _hot_segment(wl, q, 64, 64 + 1024)
    elif variant == "zero_query":
        wl.q_bits[::2] = 0
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    q_rows, w = dw.quantize()
    starts, ends = dw.layout()
    oe = ends.cpu().numpy()
    plain = dw.score(q_rows, w, starts, ends)
    cols = torch.arange(wl.width, device="cuda")
    valid = cols[None, :] < ends.to(torch.int64)[:, None]
    what = f"{name} {variant} k={k}"

    rng = np.random.default_rng(14)
    proj, _ = _step_projection(wl, 2, 140, 140 + wl.heads, rng)
    b = _cache_without_step_keys(wl)
    lb = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    ws = torch.full((dsa.score_topk_workspace_bytes(wl.num_requests, wl.max_blocks, wl.num_rows),),
                    0x77, dtype=torch.uint8, device="cuda")
    idx = torch.full((wl.num_rows, k + 3), 0x3FFFFFFF, dtype=torch.int32, device="cuda")
    fs, fe, _, _ = dsa.index_score_topk(
        bf16_dev(proj), 2, 140, b.q, b.gamma, b.beta, wl.eps, b.seq_lens, b.query_lens,
        wl.num_rows, b.cache, wl.num_pages, wl.page_stride, b.block_table, wl.max_query_len, k,
        wl.fmt, wl.section_offset, out=lb, indices=idx[:, :k], workspace=ws)
    assert torch.equal(b.cache, dw.cache), f"{what}: cache bytes"
    assert torch.equal(fs, starts) and torch.equal(fe, ends), f"{what}: row layout"
    assert torch.equal(lb.view(torch.int32)[valid], plain.view(torch.int32)[valid]), f"{what}: logits"
    assert torch.all(ws == 0x77), f"{what}: the one-launch form touches no workspace"
    assert torch.all(idx[:, k:] == 0x3FFFFFFF), f"{what}: written past k"
    got = lb.cpu().numpy()
    if k == 64:  # the logits do not depend on k: compared with the oracle's once per workload
        oq, ow = oracle.quantize_queries(wl.q_bits, wl.wv_bits, wl.fmt)
        os_, _ = oracle.decode_layout(wl.seq_lens, wl.query_lens, wl.num_rows)
        ref = oracle.score_paged(oq, wl.heads, ow, oracle_cache(wl), wl.num_pages, wl.page_stride,
                                 wl.block_table, os_, oe, wl.fmt, wl.section_offset)
        assert_logits_close(got, ref, oe, range(wl.num_rows), name)
    want = oracle.topk(np.nan_to_num(got, nan=0.0), oe, k)
    assert_topk_sets(idx[:, :k].cpu().numpy(), want, range(wl.num_rows), what)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_index_score_topk_one_launch_only_padding_rows(fmt):
    # no request has a row: every row is graph padding, selects nothing (-1) and ends at 0,
    # and the cache is untouched
    wl = make_workload("pad_only", fmt=fmt, heads=32, seq_lens=[100, 50, 7], query_lens=[0, 0, 0],
                       num_rows=3, topk=16, seed=53)
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    before = dw.cache.clone()
    proj = np.zeros((3, 128 + 32), np.uint16)
    q = bf16_dev(bf16_bits(np.random.default_rng(1).standard_normal((3, 32, 128)).astype(np.float32)))
    assert dsa.score_segment_keys(wl.num_requests, wl.max_blocks) >= wl.width
    idx = torch.full((3, 20), 0x3FFFFFFF, dtype=torch.int32, device="cuda")
    starts, ends, _, _ = dsa.index_score_topk(
        bf16_dev(proj), 0, 128, q, dw.gamma, dw.beta, wl.eps, dw.seq_lens, dw.query_lens, 3,
        dw.cache, wl.num_pages, wl.page_stride, dw.block_table, 1, 16, fmt, indices=idx[:, :16])
    assert torch.equal(dw.cache, before)
    assert starts.cpu().tolist() == [0, 0, 0, 0] and ends.cpu().tolist() == [0, 0, 0]
    got = idx.cpu().numpy()
    assert np.all(got[:, :16] == -1) and np.all(got[:, 16:] == 0x3FFFFFFF)


@pytest.mark.parametrize("shape", ["one_launch", "row", "segmented"])
def test_selection_stays_in_bounds_when_pages_are_missing(shape):
    # Block-table entries outside [0, num_pages) inside rows' bounds break the caller contract:
    # the scorer skips those pages (their keys are neither scored nor counted), so a row's
    # counts fall short of its bound. Whatever the selection then returns, it writes nothing
    # at or past k in any row: the columns after k keep their sentinel, and every written
    # position is -1 or below the row's bound.
    cases = {"one_launch": dict(seq_lens=[256, 200, 130], k=64),      # one chunk per request
             "row": dict(seq_lens=[3000, 2500, 1500], k=700),         # rows of <= 8192 keys
             "segmented": dict(seq_lens=[30000, 20000, 9000], k=1500)}  # segments of 4096
    c = cases[shape]
    wl = make_workload("missing", fmt="mxfp4", heads=32, seq_lens=c["seq_lens"],
                       query_lens=[1] * len(c["seq_lens"]), topk=c["k"], seed=51)
    k = c["k"]
    bt = wl.block_table.copy()
    for q, n in enumerate(wl.seq_lens):
        nb = (int(n) + 63) // 64
        bt[q, nb // 2] = wl.num_pages + 7   # one page of each row is no page of the cache
        bt[q, 0] = -3
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    rng = np.random.default_rng(3)
    proj, _ = _step_projection(wl, 0, 128, 128 + wl.heads, rng)
    idx = torch.full((wl.num_rows, k + 64), 0x3FFFFFFF, dtype=torch.int32, device="cuda")
    lg = torch.full((wl.num_rows, wl.width), float("nan"), device="cuda")
    if shape == "one_launch":
        assert dsa.score_segment_keys(wl.num_requests, wl.max_blocks) >= wl.width
    _, ends, _, _ = dsa.index_score_topk(
        bf16_dev(proj), 0, 128, dw.q, dw.gamma, dw.beta, wl.eps, dw.seq_lens, dw.query_lens,
        wl.num_rows, dw.cache, wl.num_pages, wl.page_stride, dev(bt), wl.max_query_len, k,
        wl.fmt, out=lg, indices=idx[:, :k])
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert np.all(got[:, k:] == 0x3FFFFFFF), f"{shape}: written past k"
    e = ends.cpu().numpy()
    for r in range(wl.num_rows):
        row = got[r, :k]
        assert np.all((row == -1) | (row == 0x3FFFFFFF) | ((row >= 0) & (row < e[r]))), \
            f"{shape} row {r}: positions outside the row"


def test_index_score_degenerate_sizes():
    # no pages or no blocks: only the row layout is written; more than 4 rows per request
    # (MXFP4) or 2 (FP8) are refused
    rng = np.random.default_rng(9)
    seq = np.array([5, 70], np.int32)
    ql = np.array([1, 2], np.int32)
    q = bf16_dev(bf16_bits(rng.standard_normal((4, 16, 128)).astype(np.float32)))
    pd = bf16_dev(bf16_bits(rng.standard_normal((4, 200)).astype(np.float32)))
    g, b = dev(np.ones(128, np.float32)), dev(np.zeros(128, np.float32))
    cache = torch.full((4352,), 0x33, dtype=torch.uint8, device="cuda")
    bt = dev(np.zeros((2, 2), np.int32))
    os_, oe = oracle.decode_layout(seq, ql, 4)
    s, e, _, _ = dsa.index_score_topk(pd, 0, 130, q, g, b, 1e-6, dev(seq), dev(ql), 4, cache, 0,
                                      4352, bt, 2, 8)
    assert np.array_equal(s.cpu().numpy(), os_) and np.array_equal(e.cpu().numpy(), oe)
    assert torch.all(cache == 0x33)
    with pytest.raises(RuntimeError):
        dsa.index_score_topk(pd, 0, 130, q, g, b, 1e-6, dev(seq), dev(ql), 4, cache, 1, 4352, bt,
                             5, 8)
    with pytest.raises(RuntimeError):  # FP8 takes at most 2 rows per request
        dsa.index_score_topk(pd, 0, 130, q, g, b, 1e-6, dev(seq), dev(ql), 4, cache, 1, 8448, bt,
                             3, 8, "fp8")


def test_score_paged_placement_invariance_and_determinism():
    outs = []
    for permute, stride, offset in [(True, 4352, 0), (False, 4352, 0), (True, 8192, 3840)]:
        wl = make_workload("inv", fmt="mxfp4", heads=32, seq_lens=[700, 129], query_lens=[2, 1],
                           topk=8, seed=12, permute_pages=permute, page_stride=stride,
                           section_offset=offset, extra_pages=2)
        dw = DeviceWorkload(wl)
        dw.fill_cache()
        q_rows, w = dw.quantize()
        starts, ends = dw.layout()
        for _ in range(2):
            outs.append(dw.score(q_rows, w, starts, ends).cpu().numpy())
    e = ends.cpu().numpy()
    for r in range(3):
        for o in outs[1:]:
            assert np.array_equal(o[r, :e[r]], outs[0][r, :e[r]])


def test_score_paged_zero_bounds_write_nothing():
    wl = make_workload("zero", fmt="mxfp4", heads=32, seq_lens=[200, 64], query_lens=[1, 1], topk=8,
                       seed=13)
    dw = DeviceWorkload(wl)
    dw.fill_cache()
    q_rows, w = dw.quantize()
    starts, _ = dw.layout()
    ends = dev(np.array([0, 0], np.int32))
    out = torch.full((2, wl.width), 3.0, device="cuda")
    dsa.score_paged(q_rows, 32, w, dw.cache, wl.num_pages, wl.page_stride, dw.block_table, starts,
                    ends, 1, out=out)
    assert torch.all(out == 3.0)


# ---- topk -----------------------------------------------------------------------------------

def _topk_inputs(seed):
    rng = np.random.default_rng(seed)
    rows, width = 12, 5000
    lg = rng.standard_normal((rows, width)).astype(np.float32)
    lg[1] = 1.0                                        # all equal
    lg[2, :] = np.round(lg[2, :] * 2) / 2              # heavy ties
    lg[3, ::2] = -0.0
    lg[3, 1::2] = 0.0                                  # signed zeros are equal
    lg[4] = -np.abs(lg[4])                             # all negative
    lg[5, 100:] = lg[5, 99]                            # ties spanning the boundary
    lg[6] *= 1e30
    lg[7] = np.arange(width, dtype=np.float32)         # strictly increasing
    ends = np.array([5000, 5000, 4999, 5000, 3333, 5000, 64, 5000, 0, 1, 2047, 2049], np.int32)
    return lg, ends


@pytest.mark.parametrize("pad", [0, 4200])
@pytest.mark.parametrize("k", [1, 64, 2048, 4999, 6000])
def test_topk_sets_match_oracle(k, pad):
    # pad 0: rows of 5000 keys take the one-workgroup-per-row kernel; pad 4200: the same bounds
    # in rows 9200 wide take the segmented kernels (keys past the bounds are 1e38 decoys)
    lg, ends = _topk_inputs(14)
    wide = np.full((lg.shape[0], lg.shape[1] + pad), 1e38, np.float32)
    wide[:, :lg.shape[1]] = lg
    want = oracle.topk(lg, ends, k)
    got = dsa.topk(dev(wide), dev(ends), k).cpu().numpy()
    assert_topk_sets(got, want, range(lg.shape[0]), f"k={k} pad={pad}")


def test_topk_strided_rows():
    lg, ends = _topk_inputs(15)
    wide = np.full((lg.shape[0], lg.shape[1] + 120), 1e38, np.float32)
    wide[:, :lg.shape[1]] = lg
    want = oracle.topk(lg, ends, 100)
    got = dsa.topk(dev(wide), dev(ends), 100, width=lg.shape[1]).cpu().numpy()
    assert_topk_sets(got, want, range(lg.shape[0]))


def test_topk_candidate_overflow_and_workspace_reuse():
    # A threshold bin holding more keys than the candidate list keeps (20000 equal logits)
    # selects from the row itself; the workspace needs no initialisation (it starts as
    # arbitrary bytes here) and one workspace serves several calls in a row.
    rng = np.random.default_rng(16)
    lg = np.full((3, 20000), 0.5, np.float32)
    lg[0, 7777] = 2.0
    lg[1] = rng.standard_normal(20000).astype(np.float32)
    lg[2, ::3] = 0.25
    ends = np.array([20000, 20000, 19999], np.int32)
    ws = torch.full((dsa.topk_workspace_bytes(3, 20000, 100),), 0xA5, dtype=torch.uint8,
                    device="cuda")
    for k in (100, 5000, 1, 100, 2047):
        want = oracle.topk(lg, ends, k)
        got = dsa.topk(dev(lg), dev(ends), k, workspace=ws).cpu().numpy()
        assert_topk_sets(got, want, range(3), f"k={k}")


def test_topk_threshold_bin_sizes_in_the_last_workgroup():
    # Segmented rows (40000 keys) whose threshold bin holds a few candidates, 3000 equal keys
    # (ties go to the lower position) and 5000 distinct keys -- more than the row's last
    # workgroup keeps in LDS, fewer than the candidate list holds -- twice on one workspace.
    rng = np.random.default_rng(17)
    n = 40000
    lg = (0.1 * rng.random((3, n))).astype(np.float32)
    lg[0] = rng.standard_normal(n).astype(np.float32)
    lg[1, rng.choice(n, 3000, replace=False)] = 1.0
    hot = rng.choice(n, 5000, replace=False)
    lg[2, hot] = (1.0 + 0.12 * rng.random(5000)).astype(np.float32)  # one 12-bit bin: [1, 1.125)
    ends = np.array([n, n - 17, n], np.int32)
    ws = torch.full((dsa.topk_workspace_bytes(3, n, 2048),), 0x5A, dtype=torch.uint8, device="cuda")
    for k in (2048, 1000, 2048):
        want = oracle.topk(lg, ends, k)
        got = dsa.topk(dev(lg), dev(ends), k, workspace=ws).cpu().numpy()
        assert_topk_sets(got, want, range(3), f"k={k}")


@pytest.mark.parametrize("rows,width,k", [(1, 3_000_000, 2048), (40, 300_000, 2048), (3, 70_000, 1)])
def test_topk_wide_rows(rows, width, k):
    # hundreds of segments per row (733 for the 3M-key row); 40 rows double the segment
    # length to 8192 keys; a row whose top bin holds everything but the first few keys
    rng = np.random.default_rng(17)
    lg = rng.standard_normal((rows, width)).astype(np.float32)
    lg[-1, 5:] = 3.0
    ends = np.full(rows, width, np.int32)
    ends[0] = width - 1
    want = oracle.topk(lg, ends, k)
    got = dsa.topk(dev(lg), dev(ends), k).cpu().numpy()
    assert_topk_sets(got, want, range(rows), f"{rows}x{width}")
